// The C ABI (include/moe_cache.h), part 3: the look-ahead prefetch
// (llama.cpp fork PR #126, sections Consumer and Eviction guard) and its
// fork/join with the cache's prefetch stream.
#include "moe_api_internal.h"

using namespace moe;
using namespace moe::api;

namespace moe {
namespace api {

// Orders `s` after the copy of a pending prefetch.  A copy issued outside
// the capture that `s` is in cannot be waited for inside it (the graph would
// not order itself after it): that is refused, loudly, instead of racing.
moe_status_t join_prefetch(moe_cache *c, hipStream_t s) {
    if (!c->pf_pending) return MOE_OK;
    hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
    HIP_TRY(rec::is_capturing(s, &cs), "capture status");
    const bool capturing = cs != hipStreamCaptureStatusNone;
    if (capturing && !c->pf_captured)
        return fail(MOE_INVALID_ARG,
                    "a prefetch issued outside this capture is still pending: call moe_prefetch_join "
                    "before beginning the capture");
    if (!capturing && c->pf_captured) {
        // left pending by a capture that ended without joining (that capture
        // failed); its event belongs to no launched work
        c->pf_pending = 0;
        return MOE_OK;
    }
    HIP_TRY(rec::stream_wait(s, c->pf_done), "wait for the prefetch copy");
    c->pf_pending = 0;
    return MOE_OK;
}

}  // namespace api
}  // namespace moe

extern "C" {

moe_status_t moe_prefetch(moe_cache_t *c, int32_t layer, const int32_t *ids, int32_t n,
                          void *stream) {
    if (!c) return fail(MOE_INVALID_ARG, "NULL cache");
    if (layer < 0 || layer >= c->d.num_layers)
        return fail(MOE_INVALID_ARG, "layer %d outside [0, %d)", layer, c->d.num_layers);
    if (n < 0 || n > c->d.max_routes)
        return fail(MOE_INVALID_ARG, "n=%d outside [0, max_routes=%d]", n, c->d.max_routes);
    if (n == 0) return MOE_OK;   // width 0 leaves everything as it is
    if (!ids) return fail(MOE_INVALID_ARG, "NULL ids");
    if (!c->prefetch_ok)
        return fail(MOE_UNSUPPORTED, "prefetch needs %zu B of LDS (E=%d, S=%d, max_routes=%d)",
                    prefetch_lds_bytes(std::min(c->d.num_experts, c->d.max_routes), c->d.num_experts,
                                       c->d.num_slots),
                    c->d.num_experts, c->d.num_slots, c->d.max_routes);
    hipStream_t s = static_cast<hipStream_t>(stream);
    // the kernel rewrites the fill plan the pending copy reads
    moe_status_t js = join_prefetch(c, s);
    if (js != MOE_OK) return js;
    PrefetchParams p{};
    p.ids = ids;
    p.n = n;
    p.M = std::min(n, c->d.num_experts);
    p.layer = layer;
    p.E = c->d.num_experts;
    p.S = c->d.num_slots;
    p.pairs = admit_order_pairs(p.S) ? 1 : 0;
    p.res = c->res;
    p.own = c->own;
    p.stamp = c->stamp;
    p.order = c->order;
    p.clock = c->clock;
    p.stats = c->stats;
    p.freq = c->freq;
    p.dlast = c->dlast;
    p.fill_slot = c->fill_slot;
    p.fill_expert = c->fill_expert;
    p.n_fill = c->n_fill;
    HIP_TRY(launch_prefetch(p, s), "prefetch launch");
    if (c->nb == 0) return MOE_OK;
    // The copy forks off `s`: nothing on `s` waits for it until the next
    // demand admission or prefetch.
    HIP_TRY(rec::event_record(c->pf_ready, s), "record prefetch fork");
    HIP_TRY(rec::stream_wait(c->pf_side, c->pf_ready), "prefetch stream waits");
    HIP_TRY(launch_gather(gather_params(c, layer, c->n_fill, c->fill_slot, c->fill_expert),
                          c->gather_wg, c->pf_side),
            "prefetch copy launch");
    HIP_TRY(rec::event_record(c->pf_done, c->pf_side), "record prefetch done");
    hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
    HIP_TRY(rec::is_capturing(s, &cs), "capture status");
    c->pf_pending = 1;
    c->pf_captured = cs != hipStreamCaptureStatusNone;
    return MOE_OK;
}

moe_status_t moe_prefetch_join(moe_cache_t *c, void *stream) {
    if (!c) return fail(MOE_INVALID_ARG, "NULL cache");
    return join_prefetch(c, static_cast<hipStream_t>(stream));
}

}  // extern "C"
