// The C ABI (include/moe_cache.h), part 1: errors, the cache and its
// device state, admission, gather, the routed and shared experts alone, and
// inspection.  The layer step is in moe_layer.hip, the look-ahead prefetch
// in moe_prefetch.hip.  Every check happens on the host before any launch,
// so a failing call launches nothing; launching calls never synchronise
// and never allocate, so a whole token's layers capture into one hipGraph.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <numeric>
#include <string>
#include <functional>
#include <mutex>
#include <vector>

#include "moe_api_internal.h"

using namespace moe;
using namespace moe::api;

namespace moe {
namespace api {

thread_local std::string g_last_error;

moe_status_t fail(moe_status_t s, const char *fmt, ...) {
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof buf, fmt, ap);
    va_end(ap);
    g_last_error = buf;
    return s;
}

moe_status_t hip_fail(hipError_t e, const char *what) {
    return fail(MOE_HIP_ERROR, "%s: %s", what, hipGetErrorString(e));
}

constexpr size_t kAlign = 256;
size_t align_up(size_t v) { return (v + kAlign - 1) & ~(kAlign - 1); }

bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15) == 0; }

void row_bytes_of(int fmt, int H, int F, int64_t rb[MOE_MAX_BANKS], int *nb) {
    for (int b = 0; b < MOE_MAX_BANKS; ++b) rb[b] = bank_row_bytes(fmt, b, H, F);
    *nb = bank_count(fmt);
}

RoutedWs routed_ws(int H, int F, int T, int K) {
    RoutedWs w;
    const size_t n = (size_t)T * K;
    size_t off = 0;
    w.h = off;
    off += align_up(n * F * 2);
    w.d = off;
    off += align_up(std::max(n * H * 4, (size_t)T * 4));
    w.ngroups = off;
    off += align_up(4);
    w.grp_row = off;
    off += align_up(n * 4);
    w.grp_start = off;
    off += align_up(n * 4);
    w.grp_count = off;
    off += align_up(n * 4);
    w.grp_routes = off;
    off += align_up(n * 4);
    w.total = off;
    return w;
}

// The device image of the LRU order: slots by (stamp, slot) ascending, as
// (slot, owner) pairs when the admission keeps pairs.  No stamps: all 0.
std::vector<int32_t> order_image(int S, const uint32_t *stamp, const int32_t *own) {
    std::vector<int32_t> slots(S);
    std::iota(slots.begin(), slots.end(), 0);
    if (stamp)
        std::stable_sort(slots.begin(), slots.end(),
                         [&](int32_t a, int32_t b) { return stamp[a] < stamp[b]; });
    if (!admit_order_pairs(S)) return slots;
    std::vector<int32_t> img(2 * (size_t)S);
    for (int i = 0; i < S; ++i) {
        img[2 * i] = slots[i];
        img[2 * i + 1] = own ? own[slots[i]] : -1;
    }
    return img;
}

// Records a timing event on `s`.  Under stream capture the event becomes an
// event-record node of the graph being captured, appended after the
// stream's current capture dependencies, so every replay re-records it.
hipError_t record_timing(hipEvent_t ev, hipStream_t s) {
    hipStreamCaptureStatus st = hipStreamCaptureStatusNone;
    hipGraph_t graph = nullptr;
    const hipGraphNode_t *deps = nullptr;
    size_t ndeps = 0;
    hipError_t e = hipStreamGetCaptureInfo_v2(s, &st, nullptr, &graph, &deps, &ndeps);
    if (e != hipSuccess) return e;
    if (st != hipStreamCaptureStatusActive) return hipEventRecord(ev, s);
    hipGraphNode_t node = nullptr;
    e = hipGraphAddEventRecordNode(&node, graph, deps, ndeps, ev);
    if (e != hipSuccess) return e;
    return hipStreamUpdateCaptureDependencies(s, &node, 1, hipStreamSetCaptureDependencies);
}

}  // namespace api
}  // namespace moe


namespace moe {
namespace api {

PoolView slot_pool_view(const moe_cache *c) {
    PoolView pv{};
    pv.fmt = c->d.weight_format;
    pv.H = c->d.hidden;
    pv.F = c->d.ffn;
    pv.num_rows = c->d.num_slots;
    for (int b = 0; b < c->nb; ++b) {
        pv.bank[b] = static_cast<const uint8_t *>(c->d.slot_banks_dev[b]);
        pv.rb[b] = c->rb[b];
    }
    return pv;
}

moe_status_t pool_view_of(const moe_pool_t *pool, PoolView &pv) {
    if (!pool) return fail(MOE_INVALID_ARG, "pool is NULL");
    if (pool->weight_format != MOE_FMT_BF16 && pool->weight_format != MOE_FMT_E2M1 &&
        pool->weight_format != MOE_FMT_MXFP4)
        return fail(MOE_INVALID_ARG, "unknown weight format %d", pool->weight_format);
    if (pool->num_rows < 1) return fail(MOE_INVALID_ARG, "pool has %d rows", pool->num_rows);
    if (!expert_shape_supported(pool->weight_format, pool->hidden, pool->ffn))
        return fail(MOE_UNSUPPORTED, "hidden %d / ffn %d not supported for format %d", pool->hidden,
                    pool->ffn, pool->weight_format);
    int nb;
    pv = PoolView{};
    pv.fmt = pool->weight_format;
    pv.H = pool->hidden;
    pv.F = pool->ffn;
    pv.num_rows = pool->num_rows;
    row_bytes_of(pv.fmt, pv.H, pv.F, pv.rb, &nb);
    for (int b = 0; b < nb; ++b) {
        if (!pool->banks_dev[b]) return fail(MOE_INVALID_ARG, "pool bank %d is NULL", b);
        if (pv.rb[b] % 16 == 0 && !aligned16(pool->banks_dev[b]))
            return fail(MOE_INVALID_ARG, "pool bank %d is not 16-byte aligned", b);
        pv.bank[b] = static_cast<const uint8_t *>(pool->banks_dev[b]);
    }
    return MOE_OK;
}

// The routed experts and the combine on one stream (no argument checks).
hipError_t routed_sequence(const PoolView &pv, const uint16_t *x, const int32_t *idx,
                           const float *w, int T, int K, const float *addend, uint16_t *out,
                           uint8_t *ws, hipStream_t s, const BeforeAddend *before) {
    auto wait_join = [&]() { return before ? (*before)() : hipSuccess; };
    if (T == 0) return wait_join();
    const RoutedWs L = routed_ws(pv.H, pv.F, T, K);
    uint16_t *h = reinterpret_cast<uint16_t *>(ws + L.h);
    const int n = T * K;
    if (T == 1 && stage_supported(pv.fmt, pv.H, pv.F)) {
        // the decode schedule's two stage launches, with no gather and no
        // shared expert (identical arithmetic to the kernels below)
        hipError_t e = launch_stages(GatherParams{}, 0, nullptr, pv, idx, w, nullptr, K, x, h, nullptr,
                                     nullptr, nullptr, nullptr, addend, out, 1, s);
        hipError_t je = wait_join();
        if (e != hipSuccess) return e;
        if (je != hipSuccess) return je;
        return launch_stages(GatherParams{}, 0, nullptr, pv, idx, w, nullptr, K, x, h, nullptr, nullptr,
                             nullptr, nullptr, addend, out, 2, s);
    }
    if (T == 1) {
        Items it{};
        it.mode = ITEM_ROUTE;
        it.K = K;
        it.n = n;
        it.idx = idx;
        hipError_t e = launch_up(pv, it, n, x, h, nullptr, nullptr, s);
        hipError_t je = wait_join();
        if (e != hipSuccess) return e;
        if (je != hipSuccess) return je;
        return launch_down_fused(pv, idx, w, T, K, h, addend, nullptr, nullptr, out, s);
    }
    int32_t *ng = reinterpret_cast<int32_t *>(ws + L.ngroups);
    int32_t *grow = reinterpret_cast<int32_t *>(ws + L.grp_row);
    int32_t *gstart = reinterpret_cast<int32_t *>(ws + L.grp_start);
    int32_t *gcount = reinterpret_cast<int32_t *>(ws + L.grp_count);
    int32_t *groutes = reinterpret_cast<int32_t *>(ws + L.grp_routes);
    float *d = reinterpret_cast<float *>(ws + L.d);
    hipError_t e = group_count_supported(pv.num_rows, n)
                       ? launch_group_count(idx, n, pv.num_rows, ng, grow, gstart, gcount, groutes, s)
                       : launch_group_routes(idx, n, pv.num_rows, ng, grow, gstart, gcount, groutes, s);
    if (e != hipSuccess) {
        (void)wait_join();
        return e;
    }
    Items it{};
    it.mode = ITEM_GROUP;
    it.K = K;
    it.n = n;
    it.n_groups = ng;
    it.grp_row = grow;
    it.grp_start = gstart;
    it.grp_count = gcount;
    it.grp_routes = groutes;
    const int max_items = std::min(n, pv.num_rows);
    if (group_mfma_supported(pv.fmt, pv.H, pv.F)) {
        e = launch_up_mfma(pv, it, max_items, x, h, s);
        if (e == hipSuccess) e = launch_down_mfma(pv, it, max_items, h, d, s);
    } else {
        e = launch_up(pv, it, max_items, x, h, nullptr, nullptr, s);
        if (e == hipSuccess) e = launch_down_to_d(pv, it, max_items, h, d, nullptr, s);
    }
    hipError_t je = wait_join();
    if (e != hipSuccess) return e;
    if (je != hipSuccess) return je;
    return launch_combine(idx, w, T, K, pv.H, pv.num_rows, d, addend, out, s);
}

hipError_t shared_sequence(const moe_shared_t *sh, int H, int Fs, const uint16_t *x, int T,
                           float *addend, uint8_t *ws, hipStream_t s) {
    if (T == 0) return hipSuccess;
    PoolView pv{};
    pv.fmt = MOE_FMT_BF16;
    pv.H = H;
    pv.F = Fs;
    pv.num_rows = 1;
    pv.bank[0] = static_cast<const uint8_t *>(sh->w13_dev);
    pv.bank[1] = static_cast<const uint8_t *>(sh->w2_dev);
    pv.rb[0] = (int64_t)4 * Fs * H;
    pv.rb[1] = (int64_t)2 * H * Fs;
    const RoutedWs L = routed_ws(H, Fs, T, 1);
    uint16_t *h = reinterpret_cast<uint16_t *>(ws + L.h);
    float *gamma = reinterpret_cast<float *>(ws + L.d);
    Items it{};
    it.mode = ITEM_ALL;
    it.K = 1;
    it.n = T;
    hipError_t e = launch_up(pv, it, 1, x, h, static_cast<const uint16_t *>(sh->gate_dev), gamma, s);
    if (e != hipSuccess) return e;
    return launch_down_to_d(pv, it, 1, h, addend, gamma, s);
}

moe_status_t check_shared(const moe_shared_t *sh, int H, int F, int *Fs) {
    if (!sh->w13_dev || !sh->w2_dev || !sh->gate_dev)
        return fail(MOE_INVALID_ARG, "shared expert has a NULL weight");
    if (!aligned16(sh->w13_dev) || !aligned16(sh->w2_dev) || !aligned16(sh->gate_dev))
        return fail(MOE_INVALID_ARG, "shared expert weights must be 16-byte aligned");
    *Fs = sh->ffn > 0 ? sh->ffn : F;
    if (sh->ffn < 0) return fail(MOE_INVALID_ARG, "shared ffn %d", sh->ffn);
    if (!expert_shape_supported(MOE_FMT_BF16, H, *Fs))
        return fail(MOE_UNSUPPORTED, "shared expert hidden %d / ffn %d not supported", H, *Fs);
    return MOE_OK;
}


// With logits set, the admission computes the top-k of T rows itself
// (R = T * K) and writes the weights to w.
moe_status_t launch_admit_checked(moe_cache *c, int layer, int32_t *ids, int R, int max_fetch,
                                  hipStream_t s, int32_t *route_plan, const float *logits, int T,
                                  int K, float *w) {
    {
        moe_status_t js = join_prefetch(c, s);
        if (js != MOE_OK) return js;
    }
    AdmitParams p{};
    p.route_plan = route_plan;
    p.logits = logits;
    p.T = T;
    p.K = K;
    p.w_out = w;
    p.ids = ids;
    p.R = R;
    p.layer = layer;
    p.max_fetch = max_fetch;
    p.E = c->d.num_experts;
    p.S = c->d.num_slots;
    p.one_call = c->d.one_call_width;
    p.query_width = c->d.query_width;
    p.res = c->res;
    p.own = c->own;
    p.stamp = c->stamp;
    p.order = c->order;
    p.clock = c->clock;
    p.stats = c->stats;
    p.freq = c->freq;
    p.dlast = c->dlast;
    p.plan_slot = c->plan_slot;
    p.plan_expert = c->plan_expert;
    p.n_miss = c->n_miss;
    HIP_TRY(launch_admit(p, c->admit_lds, s), "admission launch");
    c->last_layer = layer;
    return MOE_OK;
}

// The gather of a plan of (slot, expert) rows of one layer.
GatherParams gather_params(const moe_cache *c, int layer, const int32_t *n, const int32_t *ps,
                           const int32_t *pe) {
    GatherParams g{};
    g.n_miss = n;
    g.plan_slot = ps;
    g.plan_expert = pe;
    g.nb = c->nb;
    const int unit = gather_unit_bytes();
    int units = 0;
    for (int b = 0; b < c->nb; ++b) {
        g.unit_start[b] = units;
        units += (int)((c->rb[b] + unit - 1) / unit);
        g.host[b] = c->host_dev[(size_t)layer * c->nb + b];
        g.slot[b] = static_cast<uint8_t *>(c->d.slot_banks_dev[b]);
        g.rb[b] = c->rb[b];
    }
    g.unit_start[c->nb] = units;
    g.units_per_entry = units;
    return g;
}

// The miss gather of the last demand admission.
GatherParams gather_params(const moe_cache *c) {
    return gather_params(c, c->last_layer, c->n_miss, c->plan_slot, c->plan_expert);
}

// The same plan for stage 1's gather role: with 4-bit weights the gate/up
// scale bank travels with the units of the codes it scales.
GatherParams gather_params_staged(const moe_cache *c) {
    GatherParams g = gather_params(c);
    if (c->d.weight_format == MOE_FMT_BF16 || c->nb < 2) return g;
    const int unit = gather_unit_bytes();
    int units = 0;
    for (int b = 0; b < c->nb; ++b) {
        g.unit_start[b] = units;
        if (b != 1) units += (int)((c->rb[b] + unit - 1) / unit);
    }
    g.unit_start[c->nb] = units;
    g.units_per_entry = units;
    g.carry_scales = c->d.weight_format == MOE_FMT_E2M1 ? 2 : 1;
    return g;
}

moe_status_t launch_gather_checked(moe_cache *c, hipStream_t s) {
    if (c->nb == 0) return MOE_OK;
    HIP_TRY(launch_gather(gather_params(c), c->gather_wg, s), "gather launch");
    return MOE_OK;
}

}  // namespace api
}  // namespace moe

// ====================================================================== ABI

extern "C" {

const char *moe_status_string(moe_status_t s) {
    switch (s) {
    case MOE_OK: return "ok";
    case MOE_INVALID_ARG: return "invalid argument";
    case MOE_UNSUPPORTED: return "unsupported";
    case MOE_HIP_ERROR: return "HIP error";
    case MOE_OUT_OF_MEMORY: return "out of memory";
    }
    return "unknown status";
}

const char *moe_last_error(void) { return g_last_error.c_str(); }

moe_status_t moe_bank_row_bytes(int32_t weight_format, int32_t hidden, int32_t ffn,
                                int64_t row_bytes_out[MOE_MAX_BANKS], int32_t *num_banks_out) {
    if (!row_bytes_out || !num_banks_out) return fail(MOE_INVALID_ARG, "NULL output");
    if (weight_format != MOE_FMT_BF16 && weight_format != MOE_FMT_E2M1 &&
        weight_format != MOE_FMT_MXFP4)
        return fail(MOE_INVALID_ARG, "unknown weight format %d", weight_format);
    if (hidden < 1 || ffn < 1) return fail(MOE_INVALID_ARG, "hidden/ffn must be >= 1");
    if (weight_format == MOE_FMT_E2M1 && (hidden % 16 || ffn % 16))
        return fail(MOE_INVALID_ARG, "4-bit rows need hidden and ffn multiples of 16");
    if (weight_format == MOE_FMT_MXFP4 && (hidden % 32 || ffn % 32))
        return fail(MOE_INVALID_ARG, "mxfp4 rows need hidden and ffn multiples of 32");
    int nb;
    row_bytes_of(weight_format, hidden, ffn, row_bytes_out, &nb);
    *num_banks_out = nb;
    return MOE_OK;
}

moe_status_t moe_query_widths(int32_t R, int32_t E, int32_t one_call_width, int32_t query_width,
                              int32_t *out_host, int32_t cap, int32_t *n_out) {
    if (!n_out || (cap > 0 && !out_host)) return fail(MOE_INVALID_ARG, "NULL output");
    if (R < 0 || E < 1 || one_call_width < 1 || query_width < 1)
        return fail(MOE_INVALID_ARG, "bad sizes R=%d E=%d widths %d/%d", R, E, one_call_width,
                    query_width);
    int n = 0;
    if (R > 0 && R <= one_call_width) {
        if (n < cap) out_host[n] = R;
        n = 1;
    } else if (R > 0) {
        const int len = std::min(R, E);
        for (int start = 0; start < len; start += query_width) {
            if (n < cap) out_host[n] = std::min(query_width, len - start);
            ++n;
        }
    }
    *n_out = n;
    return MOE_OK;
}

moe_status_t moe_cache_create(const moe_cache_desc_t *d, moe_cache_t **out) {
    if (!d || !out) return fail(MOE_INVALID_ARG, "NULL desc or out");
    *out = nullptr;
    if (d->num_layers < 1 || d->num_experts < 1 || d->num_slots < 1)
        return fail(MOE_INVALID_ARG, "layers/experts/slots must be >= 1");
    if (d->one_call_width < 1 || d->query_width < 1)
        return fail(MOE_INVALID_ARG, "one_call_width and query_width must be >= 1");
    if (d->max_routes < 1) return fail(MOE_INVALID_ARG, "max_routes must be >= 1");
    if (d->overlap < 0 || d->overlap > 3)
        return fail(MOE_INVALID_ARG, "overlap must be 0, 1, 2 or 3, got %d", d->overlap);
    if (d->max_tokens < 0 || d->max_top_k < 0)
        return fail(MOE_INVALID_ARG, "max_tokens/max_top_k must be >= 0");
    if (d->gather_workgroups < 0) return fail(MOE_INVALID_ARG, "gather_workgroups < 0");
    if ((int64_t)d->num_layers * d->num_experts > INT32_MAX)
        return fail(MOE_INVALID_ARG, "num_layers * num_experts overflows int32");

    moe_cache *c = new moe_cache();
    c->d = *d;
    c->d.host_banks_host = nullptr;
    c->gather_wg = d->gather_workgroups > 0 ? d->gather_workgroups : 16;
    auto bail = [&](moe_status_t s) {
        moe_cache_destroy(c);
        return s;
    };
    // a failed HIP call after this point also frees what was made
#define CREATE_TRY(call, what)                              \
    do {                                                    \
        hipError_t e_ = (call);                             \
        if (e_ != hipSuccess) return bail(hip_fail(e_, what)); \
    } while (0)
    CREATE_TRY(hipGetDevice(&c->device), "hipGetDevice");

    // Weights.
    if (d->num_banks != 0) {
        if (d->weight_format != MOE_FMT_BF16 && d->weight_format != MOE_FMT_E2M1 &&
            d->weight_format != MOE_FMT_MXFP4) {
            moe_status_t s = fail(MOE_INVALID_ARG, "unknown weight format %d", d->weight_format);
            return bail(s);
        }
        if (!expert_shape_supported(d->weight_format, d->hidden, d->ffn))
            return bail(fail(MOE_UNSUPPORTED, "hidden %d / ffn %d not supported for format %d",
                             d->hidden, d->ffn, d->weight_format));
        row_bytes_of(d->weight_format, d->hidden, d->ffn, c->rb, &c->nb);
        if (d->num_banks != c->nb)
            return bail(fail(MOE_INVALID_ARG, "format %d has %d banks, desc says %d",
                             d->weight_format, c->nb, d->num_banks));
        if (!d->host_banks_host) return bail(fail(MOE_INVALID_ARG, "host_banks_host is NULL"));
        for (int b = 0; b < c->nb; ++b) {
            if (!d->slot_banks_dev[b] || !aligned16(d->slot_banks_dev[b]))
                return bail(fail(MOE_INVALID_ARG, "slot bank %d is NULL or not 16-byte aligned", b));
        }
        c->host_dev.resize((size_t)d->num_layers * c->nb);
        c->host_rows.resize((size_t)d->num_layers * c->nb);
        for (int l = 0; l < d->num_layers; ++l)
            for (int b = 0; b < c->nb; ++b) {
                void *hp = const_cast<void *>(d->host_banks_host[(size_t)l * c->nb + b]);
                const size_t align = (c->rb[b] % 16 == 0) ? 16 : 4;
                if (!hp || (reinterpret_cast<uintptr_t>(hp) % align))
                    return bail(fail(MOE_INVALID_ARG, "host bank (layer %d, bank %d) is NULL or unaligned",
                                     l, b));
                void *dp = nullptr;
                hipError_t e = hipHostGetDevicePointer(&dp, hp, 0);
                if (e != hipSuccess || !dp) {
                    (void)hipGetLastError();
                    return bail(fail(MOE_INVALID_ARG,
                                     "host bank (layer %d, bank %d) is not pinned, device-mapped host memory",
                                     l, b));
                }
                c->host_dev[(size_t)l * c->nb + b] = static_cast<const uint8_t *>(dp);
                c->host_rows[(size_t)l * c->nb + b] = static_cast<const uint8_t *>(hp);
            }
    }

    // Admission state.
    int max_lds = 0;
    CREATE_TRY(hipDeviceGetAttribute(&max_lds, hipDeviceAttributeMaxSharedMemoryPerBlock, c->device),
            "device attribute");
    c->admit_lds = admit_lds_bytes(d->num_experts, d->num_slots, d->max_routes);
    if (c->admit_lds > (size_t)max_lds)
        return bail(fail(MOE_UNSUPPORTED, "admission needs %zu B of LDS (E=%d, S=%d, max_routes=%d); device has %d",
                         c->admit_lds, d->num_experts, d->num_slots, d->max_routes, max_lds));
    CREATE_TRY(admit_prepare(c->admit_lds), "admission LDS attribute");

    const size_t L = d->num_layers, E = d->num_experts, S = d->num_slots;
    c->plan_cap = (int)std::min<size_t>(E, (size_t)d->max_routes);
    size_t off = 0;
    const size_t o_res = off; off += align_up(L * E * 4);
    const size_t o_own = off; off += align_up(S * 4);
    const size_t o_stamp = off; off += align_up(S * 4);
    const size_t o_order = off; off += align_up(admit_order_bytes((int)S));
    const size_t o_clock = off; off += align_up(8);
    const size_t o_stats = off; off += align_up(L * MOE_NUM_STATS * 8);
    const size_t o_freq = off; off += align_up(L * E * 8);
    const size_t o_dlast = off; off += align_up(L * E * 4);
    const size_t o_fs = off; off += align_up(E * 4);
    const size_t o_fe = off; off += align_up(E * 4);
    const size_t o_nf = off; off += align_up(4);
    const size_t o_ps = off; off += align_up((size_t)c->plan_cap * 4);
    const size_t o_pe = off; off += align_up((size_t)c->plan_cap * 4);
    const size_t o_nm = off; off += align_up(4);
    {
        hipError_t e = hipMalloc(&c->state, off);
        if (e != hipSuccess) {
            (void)hipGetLastError();
            return bail(fail(MOE_OUT_OF_MEMORY, "cache state (%zu B): %s", off, hipGetErrorString(e)));
        }
    }
    uint8_t *base = static_cast<uint8_t *>(c->state);
    c->res = reinterpret_cast<int32_t *>(base + o_res);
    c->own = reinterpret_cast<int32_t *>(base + o_own);
    c->stamp = reinterpret_cast<uint32_t *>(base + o_stamp);
    c->order = reinterpret_cast<int32_t *>(base + o_order);
    c->clock = reinterpret_cast<uint32_t *>(base + o_clock);
    c->stats = reinterpret_cast<int64_t *>(base + o_stats);
    c->freq = reinterpret_cast<int64_t *>(base + o_freq);
    c->dlast = reinterpret_cast<uint32_t *>(base + o_dlast);
    c->fill_slot = reinterpret_cast<int32_t *>(base + o_fs);
    c->fill_expert = reinterpret_cast<int32_t *>(base + o_fe);
    c->n_fill = reinterpret_cast<int32_t *>(base + o_nf);
    c->plan_slot = reinterpret_cast<int32_t *>(base + o_ps);
    c->plan_expert = reinterpret_cast<int32_t *>(base + o_pe);
    c->n_miss = reinterpret_cast<int32_t *>(base + o_nm);
    {
        moe_status_t s = MOE_OK;
        hipError_t e = hipMemset(c->state, 0, off);
        if (e == hipSuccess) e = hipMemset(c->res, 0xff, L * E * 4);
        if (e == hipSuccess) e = hipMemset(c->own, 0xff, S * 4);
        const std::vector<int32_t> order = order_image(S, nullptr, nullptr);
        if (e == hipSuccess)
            e = hipMemcpy(c->order, order.data(), order.size() * 4, hipMemcpyHostToDevice);
        if (e != hipSuccess) s = hip_fail(e, "cache state init");
        if (s != MOE_OK) return bail(s);
    }

    // Layer workspace.
    if (d->max_tokens > 0) {
        if (d->max_top_k < 1 || d->max_top_k > kMaxTopK || d->max_top_k > d->num_experts)
            return bail(fail(MOE_INVALID_ARG, "max_top_k must be in [1, min(64, E)]"));
        if ((int64_t)d->max_tokens * d->max_top_k > kMaxRoutedRoutes)
            return bail(fail(MOE_UNSUPPORTED, "max_tokens * max_top_k > %d", kMaxRoutedRoutes));
        const size_t T = d->max_tokens, K = d->max_top_k, H = std::max(d->hidden, 1);
        const int F = std::max(d->ffn, 8);
        c->shared_ffn_cap = F;
        const RoutedWs rw = routed_ws((int)H, F, (int)T, (int)K);
        const RoutedWs sw = routed_ws((int)H, c->shared_ffn_cap, (int)T, 1);
        size_t o = 0;
        const size_t o_ids = o; o += align_up(T * K * 4);
        const size_t o_plan = o; o += align_up(T * K * 4);
        const size_t o_w = o; o += align_up(T * K * 4);
        const size_t o_add = o; o += align_up(T * H * 4);
        const size_t o_gu = o; o += align_up(K * 2 * (size_t)F * 4);
        const size_t o_r = o; o += rw.total;
        const size_t o_s = o; o += sw.total;
        hipError_t e = hipMalloc(&c->ws, o);
        if (e != hipSuccess) {
            (void)hipGetLastError();
            return bail(fail(MOE_OUT_OF_MEMORY, "layer workspace (%zu B): %s", o, hipGetErrorString(e)));
        }
        uint8_t *wb = static_cast<uint8_t *>(c->ws);
        c->ws_ids = reinterpret_cast<int32_t *>(wb + o_ids);
        c->ws_route_plan = reinterpret_cast<int32_t *>(wb + o_plan);
        c->ws_w = reinterpret_cast<float *>(wb + o_w);
        c->ws_addend = reinterpret_cast<float *>(wb + o_add);
        c->ws_gu = reinterpret_cast<float *>(wb + o_gu);
        c->ws_routed = wb + o_r;
        c->ws_routed_bytes = rw.total;
        c->ws_shared = wb + o_s;
        c->ws_shared_bytes = sw.total;
        const size_t glds = group_lds_bytes((int)(T * K));
        if (glds > (size_t)max_lds) return bail(fail(MOE_UNSUPPORTED, "route grouping LDS too large"));
        CREATE_TRY(group_prepare(glds), "grouping LDS attribute");
        CREATE_TRY(group_count_prepare(), "grouping LDS attribute");
        if ((int64_t)T * K > d->max_routes)
            return bail(fail(MOE_INVALID_ARG, "max_tokens * max_top_k > max_routes"));
    }

    // Side stream and the two events, made before any capture.
    CREATE_TRY(hipStreamCreateWithFlags(&c->side, hipStreamNonBlocking), "side stream");
    CREATE_TRY(hipEventCreateWithFlags(&c->ready, hipEventDisableTiming), "ready event");
    CREATE_TRY(hipEventCreateWithFlags(&c->done, hipEventDisableTiming), "done event");
    CREATE_TRY(hipStreamCreateWithFlags(&c->pf_side, hipStreamNonBlocking), "prefetch stream");
    CREATE_TRY(hipEventCreateWithFlags(&c->pf_ready, hipEventDisableTiming), "prefetch event");
    CREATE_TRY(hipEventCreateWithFlags(&c->pf_done, hipEventDisableTiming), "prefetch event");
    // the look-ahead prefetch of up to max_routes ids: usable only if its
    // kernel fits the LDS (checked again by moe_prefetch)
    {
        const size_t pl = prefetch_lds_bytes(std::min(d->num_experts, d->max_routes), d->num_experts,
                                             d->num_slots);
        c->prefetch_ok = pl <= (size_t)max_lds;
        if (c->prefetch_ok) CREATE_TRY(prefetch_prepare(pl), "prefetch LDS attribute");
    }
    c->tev.assign((size_t)d->num_layers * 6, nullptr);
    c->trecorded.assign(d->num_layers, 0);
    CREATE_TRY(hipDeviceSynchronize(), "create sync");
    *out = c;
    return MOE_OK;
#undef CREATE_TRY
}

moe_status_t moe_cache_set_schedule(moe_cache_t *c, int32_t overlap) {
    if (!c) return fail(MOE_INVALID_ARG, "NULL cache");
    if (overlap < 0 || overlap > 3)
        return fail(MOE_INVALID_ARG, "overlap must be 0, 1, 2 or 3, got %d", overlap);
    c->d.overlap = overlap;
    return MOE_OK;
}

void moe_cache_destroy(moe_cache_t *c) {
    if (!c) return;
    (void)hipDeviceSynchronize();
    if (c->cpu) cpu_experts_destroy(c->cpu);
    if (c->hyb_host) (void)hipHostFree(c->hyb_host);
    if (c->hyb_ready) (void)hipEventDestroy(c->hyb_ready);
    for (hipEvent_t e : c->tev)
        if (e) (void)hipEventDestroy(e);
    if (c->ready) (void)hipEventDestroy(c->ready);
    if (c->done) (void)hipEventDestroy(c->done);
    if (c->side) (void)hipStreamDestroy(c->side);
    if (c->pf_ready) (void)hipEventDestroy(c->pf_ready);
    if (c->pf_done) (void)hipEventDestroy(c->pf_done);
    if (c->pf_side) (void)hipStreamDestroy(c->pf_side);
    if (c->ws) (void)hipFree(c->ws);
    if (c->state) (void)hipFree(c->state);
    delete c;
}

moe_status_t moe_cache_pool(const moe_cache_t *c, moe_pool_t *pool) {
    if (!c || !pool) return fail(MOE_INVALID_ARG, "NULL cache or pool");
    if (c->nb == 0) return fail(MOE_INVALID_ARG, "cache has no weight banks");
    memset(pool, 0, sizeof *pool);
    pool->weight_format = c->d.weight_format;
    pool->hidden = c->d.hidden;
    pool->ffn = c->d.ffn;
    pool->num_rows = c->d.num_slots;
    for (int b = 0; b < c->nb; ++b) pool->banks_dev[b] = c->d.slot_banks_dev[b];
    return MOE_OK;
}

moe_status_t moe_topk(const float *logits, int32_t T, int32_t E, int32_t K, int32_t *ids, float *w,
                      void *stream) {
    if (T < 0 || E < 1 || K < 1 || K > E || K > kMaxTopK)
        return fail(MOE_INVALID_ARG, "bad top-k sizes T=%d E=%d K=%d", T, E, K);
    if (T > 0 && (!logits || !ids || !w)) return fail(MOE_INVALID_ARG, "NULL top-k buffer");
    HIP_TRY(launch_topk(logits, T, E, K, ids, w, static_cast<hipStream_t>(stream)), "top-k launch");
    return MOE_OK;
}

moe_status_t moe_admit(moe_cache_t *c, int32_t layer, int32_t *ids, int32_t R, int32_t max_fetch,
                       void *stream) {
    if (!c) return fail(MOE_INVALID_ARG, "NULL cache");
    if (layer < 0 || layer >= c->d.num_layers)
        return fail(MOE_INVALID_ARG, "layer %d outside [0, %d)", layer, c->d.num_layers);
    if (R < 0 || R > c->d.max_routes)
        return fail(MOE_INVALID_ARG, "R=%d outside [0, max_routes=%d]", R, c->d.max_routes);
    if (R > 0 && !ids) return fail(MOE_INVALID_ARG, "NULL ids");
    return launch_admit_checked(c, layer, ids, R, max_fetch, static_cast<hipStream_t>(stream));
}

moe_status_t moe_gather_misses(moe_cache_t *c, void *stream) {
    if (!c) return fail(MOE_INVALID_ARG, "NULL cache");
    if (c->last_layer < 0) return fail(MOE_INVALID_ARG, "no admission to gather for");
    return launch_gather_checked(c, static_cast<hipStream_t>(stream));
}

int64_t moe_routed_workspace_bytes(int32_t weight_format, int32_t hidden, int32_t ffn, int32_t T,
                                   int32_t K) {
    (void)weight_format;
    if (hidden < 1 || ffn < 1 || T < 0 || K < 1) return 0;
    return (int64_t)routed_ws(hidden, ffn, T, K).total;
}

}  // extern "C"

namespace {

// moe_routed_decode's body, for a workspace of ws_bytes at ws (caller
// memory, or the allocation-free entry point's scratch).
moe_status_t routed_decode_into(const moe_pool_t *pool, const void *x, const int32_t *idx,
                                const float *w, int32_t T, int32_t K, const float *addend, void *out,
                                void *ws, int64_t ws_bytes, void *stream) {
    PoolView pv;
    moe_status_t s = pool_view_of(pool, pv);
    if (s != MOE_OK) return s;
    if (T < 0 || K < 1 || K > kMaxTopK) return fail(MOE_INVALID_ARG, "bad T=%d K=%d", T, K);
    if ((int64_t)T * K > kMaxRoutedRoutes)
        return fail(MOE_UNSUPPORTED, "T*K=%lld > %d routes", (long long)T * K, kMaxRoutedRoutes);
    if (T == 0) return MOE_OK;
    if (!x || !idx || !w || !out || !ws) return fail(MOE_INVALID_ARG, "NULL routed buffer");
    if (!aligned16(x)) return fail(MOE_INVALID_ARG, "x must be 16-byte aligned");
    if (reinterpret_cast<uintptr_t>(ws) % kAlign) return fail(MOE_INVALID_ARG, "workspace must be 256-byte aligned");
    const RoutedWs L = routed_ws(pv.H, pv.F, T, K);
    if (ws_bytes < (int64_t)L.total)
        return fail(MOE_INVALID_ARG, "workspace %lld B < %zu B", (long long)ws_bytes, L.total);
    if (T > 1) {
        int max_lds = 0;
        int dev = 0;
        HIP_TRY(hipGetDevice(&dev), "hipGetDevice");
        HIP_TRY(hipDeviceGetAttribute(&max_lds, hipDeviceAttributeMaxSharedMemoryPerBlock, dev), "attr");
        const size_t glds = group_lds_bytes(T * K);
        if (glds > (size_t)max_lds) return fail(MOE_UNSUPPORTED, "too many routes to group");
        HIP_TRY(group_prepare(glds), "grouping LDS attribute");
        HIP_TRY(group_count_prepare(), "grouping LDS attribute");
    }
    HIP_TRY(routed_sequence(pv, static_cast<const uint16_t *>(x), idx, w, T, K, addend,
                            static_cast<uint16_t *>(out), static_cast<uint8_t *>(ws),
                            static_cast<hipStream_t>(stream)),
            "routed launch");
    return MOE_OK;
}

// The allocation-free entry point's workspace: a file-scope device array,
// one copy per GPU, held until the process ends.  Host code never uses the
// array's name as an address (on the host it is only a stand-in): each
// device's copy is looked up once with hipGetSymbolAddress, with that
// device current, and that address is what the kernels get.
constexpr int kScratchDevices = 64;
std::mutex g_scratch_mu;
void *g_scratch_dev[kScratchDevices] = {};

}  // namespace

static __device__ __align__(256) uint8_t scratch[MOE_NOALLOC_SCRATCH_BYTES];

namespace {

moe_status_t scratch_of_current_device(void **out) {
    int dev = 0;
    HIP_TRY(hipGetDevice(&dev), "hipGetDevice");
    if (dev < 0 || dev >= kScratchDevices)
        return fail(MOE_UNSUPPORTED, "device %d: the scratch table holds %d devices", dev, kScratchDevices);
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_dev[dev]) {
        void *p = nullptr;
        const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess || !p) {
            (void)hipGetLastError();
            return fail(MOE_HIP_ERROR, "hipGetSymbolAddress(scratch) on device %d: %s", dev,
                        hipGetErrorString(e));
        }
        g_scratch_dev[dev] = p;
    }
    *out = g_scratch_dev[dev];
    return MOE_OK;
}

}  // namespace

extern "C" {

moe_status_t moe_routed_decode(const moe_pool_t *pool, const void *x, const int32_t *idx,
                               const float *w, int32_t T, int32_t K, const float *addend, void *out,
                               void *ws, int64_t ws_bytes, void *stream) {
    return routed_decode_into(pool, x, idx, w, T, K, addend, out, ws, ws_bytes, stream);
}

moe_status_t moe_routed_decode_noalloc(const moe_pool_t *pool, const void *x, const int32_t *idx,
                                       const float *w, int32_t T, int32_t K, const float *addend,
                                       void *out, void *stream) {
    if (!pool) return fail(MOE_INVALID_ARG, "NULL pool");
    if (T < 0 || K < 1 || K > kMaxTopK) return fail(MOE_INVALID_ARG, "bad T=%d K=%d", T, K);
    if (T == 0) return MOE_OK;
    const size_t need = routed_ws(pool->hidden, pool->ffn, T, K).total;
    if (pool->hidden < 1 || pool->ffn < 1 || need > (size_t)MOE_NOALLOC_SCRATCH_BYTES)
        return fail(MOE_INVALID_ARG,
                    "T=%d K=%d at hidden %d, ffn %d needs %zu B of workspace, more than the %d B "
                    "the allocation-free entry point holds; use moe_routed_decode",
                    T, K, pool->hidden, pool->ffn, need, (int)MOE_NOALLOC_SCRATCH_BYTES);
    void *ws = nullptr;
    moe_status_t s = scratch_of_current_device(&ws);
    if (s != MOE_OK) return s;
    return routed_decode_into(pool, x, idx, w, T, K, addend, out, ws, (int64_t)MOE_NOALLOC_SCRATCH_BYTES,
                              stream);
}

moe_status_t moe_shared_expert(const moe_shared_t *sh, int32_t H, const void *x, int32_t T,
                               float *addend, void *ws, int64_t ws_bytes, void *stream) {
    if (!sh) return fail(MOE_INVALID_ARG, "NULL shared expert");
    int Fs;
    moe_status_t s = check_shared(sh, H, 0, &Fs);
    if (s != MOE_OK) return s;
    if (sh->ffn == 0) return fail(MOE_INVALID_ARG, "standalone shared expert needs ffn > 0");
    if (T < 0) return fail(MOE_INVALID_ARG, "T < 0");
    if (T == 0) return MOE_OK;
    if (!x || !addend || !ws) return fail(MOE_INVALID_ARG, "NULL shared buffer");
    if (!aligned16(x)) return fail(MOE_INVALID_ARG, "x must be 16-byte aligned");
    const RoutedWs L = routed_ws(H, Fs, T, 1);
    if (ws_bytes < (int64_t)L.total)
        return fail(MOE_INVALID_ARG, "workspace %lld B < %zu B", (long long)ws_bytes, L.total);
    HIP_TRY(shared_sequence(sh, H, Fs, static_cast<const uint16_t *>(x), T, addend,
                            static_cast<uint8_t *>(ws), static_cast<hipStream_t>(stream)),
            "shared launch");
    return MOE_OK;
}

moe_status_t moe_cache_stats(moe_cache_t *c, int32_t layer, int64_t *out, void *stream) {
    if (!c || !out) return fail(MOE_INVALID_ARG, "NULL cache or output");
    if (layer < -1 || layer >= c->d.num_layers) return fail(MOE_INVALID_ARG, "layer %d", layer);
    const int L = c->d.num_layers;
    std::vector<int64_t> all((size_t)L * MOE_NUM_STATS);
    hipStream_t s = static_cast<hipStream_t>(stream);
    HIP_TRY(hipMemcpyAsync(all.data(), c->stats, all.size() * 8, hipMemcpyDeviceToHost, s), "stats copy");
    HIP_TRY(hipStreamSynchronize(s), "stats sync");
    for (int k = 0; k < MOE_NUM_STATS; ++k) out[k] = 0;
    for (int l = 0; l < L; ++l)
        if (layer < 0 || l == layer)
            for (int k = 0; k < MOE_NUM_STATS; ++k) out[k] += all[(size_t)l * MOE_NUM_STATS + k];
    return MOE_OK;
}

moe_status_t moe_cache_read_state(moe_cache_t *c, int32_t *res, int32_t *own, uint32_t *stamp,
                                  uint32_t *clock, int64_t *stats, int64_t *freq, int32_t *order,
                                  uint32_t *dlast, uint32_t *last_demand) {
    if (!c) return fail(MOE_INVALID_ARG, "NULL cache");
    const size_t L = c->d.num_layers, E = c->d.num_experts, S = c->d.num_slots;
    HIP_TRY(hipDeviceSynchronize(), "sync");
    if (res) HIP_TRY(hipMemcpy(res, c->res, L * E * 4, hipMemcpyDeviceToHost), "copy res");
    if (own) HIP_TRY(hipMemcpy(own, c->own, S * 4, hipMemcpyDeviceToHost), "copy own");
    if (stamp) HIP_TRY(hipMemcpy(stamp, c->stamp, S * 4, hipMemcpyDeviceToHost), "copy stamp");
    if (clock) HIP_TRY(hipMemcpy(clock, c->clock, 4, hipMemcpyDeviceToHost), "copy clock");
    if (stats) HIP_TRY(hipMemcpy(stats, c->stats, L * MOE_NUM_STATS * 8, hipMemcpyDeviceToHost), "copy stats");
    if (freq) HIP_TRY(hipMemcpy(freq, c->freq, L * E * 8, hipMemcpyDeviceToHost), "copy freq");
    if (dlast) HIP_TRY(hipMemcpy(dlast, c->dlast, L * E * 4, hipMemcpyDeviceToHost), "copy dlast");
    if (last_demand)
        HIP_TRY(hipMemcpy(last_demand, c->clock + 1, 4, hipMemcpyDeviceToHost), "copy last demand");
    if (order) {
        std::vector<int32_t> img(admit_order_pairs((int)S) ? 2 * S : S);
        HIP_TRY(hipMemcpy(img.data(), c->order, img.size() * 4, hipMemcpyDeviceToHost), "copy order");
        const size_t stride = img.size() / S;
        for (size_t i = 0; i < S; ++i) order[i] = img[i * stride];
    }
    return MOE_OK;
}

moe_status_t moe_cache_write_state(moe_cache_t *c, const int32_t *res, const int32_t *own,
                                   const uint32_t *stamp, uint32_t clock, const int64_t *freq,
                                   const uint32_t *dlast, const uint32_t *last_demand) {
    if (!c || !res || !own || !stamp) return fail(MOE_INVALID_ARG, "NULL state");
    const size_t L = c->d.num_layers, E = c->d.num_experts, S = c->d.num_slots;
    for (size_t s = 0; s < S; ++s) {
        if (own[s] < -1 || own[s] >= (int64_t)(L * E)) return fail(MOE_INVALID_ARG, "own[%zu] out of range", s);
        if (own[s] >= 0 && res[own[s]] != (int32_t)s) return fail(MOE_INVALID_ARG, "res/own disagree at slot %zu", s);
        if (stamp[s] > clock) return fail(MOE_INVALID_ARG, "stamp[%zu] > clock", s);
    }
    for (size_t i = 0; i < L * E; ++i) {
        if (res[i] < -1 || res[i] >= (int32_t)S) return fail(MOE_INVALID_ARG, "res[%zu] out of range", i);
        if (res[i] >= 0 && own[res[i]] != (int32_t)i) return fail(MOE_INVALID_ARG, "res/own disagree at %zu", i);
        if (dlast && dlast[i] > clock) return fail(MOE_INVALID_ARG, "dlast[%zu] > clock", i);
        if (freq && freq[i] < 0) return fail(MOE_INVALID_ARG, "freq[%zu] < 0", i);
    }
    if (last_demand && *last_demand > clock) return fail(MOE_INVALID_ARG, "last_demand > clock");
    const std::vector<int32_t> order = order_image((int)S, stamp, own);
    HIP_TRY(hipDeviceSynchronize(), "sync");
    HIP_TRY(hipMemcpy(c->res, res, L * E * 4, hipMemcpyHostToDevice), "write res");
    HIP_TRY(hipMemcpy(c->own, own, S * 4, hipMemcpyHostToDevice), "write own");
    HIP_TRY(hipMemcpy(c->stamp, stamp, S * 4, hipMemcpyHostToDevice), "write stamp");
    HIP_TRY(hipMemcpy(c->clock, &clock, 4, hipMemcpyHostToDevice), "write clock");
    if (freq) HIP_TRY(hipMemcpy(c->freq, freq, L * E * 8, hipMemcpyHostToDevice), "write freq");
    if (dlast) HIP_TRY(hipMemcpy(c->dlast, dlast, L * E * 4, hipMemcpyHostToDevice), "write dlast");
    if (last_demand)
        HIP_TRY(hipMemcpy(c->clock + 1, last_demand, 4, hipMemcpyHostToDevice), "write last demand");
    HIP_TRY(hipMemcpy(c->order, order.data(), order.size() * 4, hipMemcpyHostToDevice), "write order");
    return MOE_OK;
}

moe_status_t moe_cache_read_plan(moe_cache_t *c, int32_t *ps, int32_t *pe, int32_t cap, int32_t *n) {
    if (!c || !n || (cap > 0 && (!ps || !pe))) return fail(MOE_INVALID_ARG, "NULL plan output");
    HIP_TRY(hipDeviceSynchronize(), "sync");
    int32_t nm = 0;
    HIP_TRY(hipMemcpy(&nm, c->n_miss, 4, hipMemcpyDeviceToHost), "copy n_miss");
    *n = nm;
    const int k = std::min(std::max(cap, 0), nm);
    if (k > 0) {
        HIP_TRY(hipMemcpy(ps, c->plan_slot, (size_t)k * 4, hipMemcpyDeviceToHost), "copy plan");
        HIP_TRY(hipMemcpy(pe, c->plan_expert, (size_t)k * 4, hipMemcpyDeviceToHost), "copy plan");
    }
    return MOE_OK;
}

moe_status_t moe_cache_read_fills(moe_cache_t *c, int32_t *ps, int32_t *pe, int32_t cap, int32_t *n) {
    if (!c || !n || (cap > 0 && (!ps || !pe))) return fail(MOE_INVALID_ARG, "NULL fill plan output");
    HIP_TRY(hipDeviceSynchronize(), "sync");
    int32_t nf = 0;
    HIP_TRY(hipMemcpy(&nf, c->n_fill, 4, hipMemcpyDeviceToHost), "copy n_fill");
    *n = nf;
    const int k = std::min(std::max(cap, 0), nf);
    if (k > 0) {
        HIP_TRY(hipMemcpy(ps, c->fill_slot, (size_t)k * 4, hipMemcpyDeviceToHost), "copy fills");
        HIP_TRY(hipMemcpy(pe, c->fill_expert, (size_t)k * 4, hipMemcpyDeviceToHost), "copy fills");
    }
    return MOE_OK;
}

moe_status_t moe_record_event(void *event, void *stream) {
    if (!event) return fail(MOE_INVALID_ARG, "NULL event");
    HIP_TRY(record_timing(static_cast<hipEvent_t>(event), static_cast<hipStream_t>(stream)),
            "event record");
    return MOE_OK;
}

moe_status_t moe_cache_set_timing(moe_cache_t *c, int32_t enable) {
    if (!c) return fail(MOE_INVALID_ARG, "NULL cache");
    if (enable != 0 && enable != 1) return fail(MOE_INVALID_ARG, "enable must be 0 or 1");
    // events are made here, outside any capture
    if (enable)
        for (hipEvent_t &e : c->tev)
            if (!e) HIP_TRY(hipEventCreate(&e), "timing event");
    c->timing = enable;
    return MOE_OK;
}

moe_status_t moe_cache_timing(moe_cache_t *c, float *ms, int32_t *layers_read) {
    if (!c || !ms || !layers_read) return fail(MOE_INVALID_ARG, "NULL timing output");
    int n = 0;
    for (int l = 0; l < c->d.num_layers; ++l) {
        ms[l * 3] = ms[l * 3 + 1] = ms[l * 3 + 2] = -1.f;
        if (!c->trecorded[l]) continue;
        hipEvent_t *ev = &c->tev[(size_t)l * 6];
        HIP_TRY(hipEventSynchronize(ev[5]), "timing sync");
        HIP_TRY(hipEventSynchronize(ev[3]), "timing sync");
        for (int k = 0; k < 3; ++k)
            HIP_TRY(hipEventElapsedTime(&ms[l * 3 + k], ev[2 * k], ev[2 * k + 1]), "elapsed");
        ++n;
    }
    *layers_read = n;
    return MOE_OK;
}

}  // extern "C"
