// Host-side internals shared by the C ABI's sources (moe_api.hip,
// moe_layer.hip, moe_prefetch.hip): error reporting, the cache object, and
// the launch sequences several entry points share.  Not part of the ABI.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>
#include <functional>
#include <string>
#include <vector>

#include "cpu_experts.h"
#include "moe_internal.h"

namespace moe {
namespace api {

// Sets the calling thread's last error message and returns s.
moe_status_t fail(moe_status_t s, const char *fmt, ...);
moe_status_t hip_fail(hipError_t e, const char *what);

#define HIP_TRY(call, what)                          \
    do {                                             \
        hipError_t e_ = (call);                      \
        if (e_ != hipSuccess) return hip_fail(e_, what); \
    } while (0)

size_t align_up(size_t v);
bool aligned16(const void *p);
void row_bytes_of(int fmt, int H, int F, int64_t rb[MOE_MAX_BANKS], int *nb);

// Workspace of the routed experts for n = T*K routes.
struct RoutedWs {
    size_t h, d, ngroups, grp_row, grp_start, grp_count, grp_routes, total;
};

RoutedWs routed_ws(int H, int F, int T, int K);

// The device image of the LRU order for these stamps and owners.
std::vector<int32_t> order_image(int S, const uint32_t *stamp, const int32_t *own);

constexpr int kMaxTopK = 64;
constexpr int kFusedTopkRows = 32;   // up to this many rows, top-k runs inside the admission
constexpr int kMaxRoutedRoutes = 8192;

// Records ev on s; under capture, as an event-record node of the graph.
hipError_t record_timing(hipEvent_t ev, hipStream_t s);

// Work issued right before the launch that adds the fp32 term: a wait for
// the stream producing it, or the hybrid step's CPU half.  Always called,
// also after a failed launch, so a fork it closes is always joined.
using BeforeAddend = std::function<hipError_t()>;

hipError_t routed_sequence(const PoolView &pv, const uint16_t *x, const int32_t *idx,
                           const float *w, int T, int K, const float *addend, uint16_t *out,
                           uint8_t *ws, hipStream_t s, const BeforeAddend *before = nullptr);
hipError_t shared_sequence(const moe_shared_t *sh, int H, int Fs, const uint16_t *x, int T,
                           float *addend, uint8_t *ws, hipStream_t s);
moe_status_t pool_view_of(const moe_pool_t *pool, PoolView &pv);
moe_status_t check_shared(const moe_shared_t *sh, int H, int F, int *Fs);

}  // namespace api
}  // namespace moe

struct moe_cache {
    moe_cache_desc_t d{};
    int device = 0;
    int nb = 0;
    int64_t rb[MOE_MAX_BANKS] = {};
    std::vector<const uint8_t *> host_dev;  // [L * nb] device-visible host rows
    std::vector<const uint8_t *> host_rows; // [L * nb] the same rows, host addresses
    // device state
    void *state = nullptr;
    int32_t *res = nullptr, *own = nullptr, *order = nullptr;
    int32_t *plan_slot = nullptr, *plan_expert = nullptr, *n_miss = nullptr;
    uint32_t *stamp = nullptr, *clock = nullptr, *dlast = nullptr;
    int64_t *stats = nullptr, *freq = nullptr;
    int32_t *fill_slot = nullptr, *fill_expert = nullptr, *n_fill = nullptr;
    int plan_cap = 0;
    size_t admit_lds = 0;
    // layer workspace
    void *ws = nullptr;
    int32_t *ws_ids = nullptr;
    int32_t *ws_route_plan = nullptr;
    float *ws_w = nullptr;
    float *ws_addend = nullptr;
    float *ws_gu = nullptr;          // [max_top_k][2F] fetched experts' gate/up dots
    uint8_t *ws_routed = nullptr;
    size_t ws_routed_bytes = 0;
    uint8_t *ws_shared = nullptr;
    size_t ws_shared_bytes = 0;
    int shared_ffn_cap = 0;
    // ordering
    hipStream_t side = nullptr;
    hipEvent_t ready = nullptr, done = nullptr;
    // look-ahead prefetch: its copy stream, fork/join events, and whether a
    // copy is still to be waited for
    hipStream_t pf_side = nullptr;
    hipEvent_t pf_ready = nullptr, pf_done = nullptr;
    int pf_pending = 0;
    bool pf_captured = false;   // the pending copy was issued under stream capture
    bool prefetch_ok = false;
    int last_layer = -1;
    int gather_wg = 64;
    // hybrid decode: the host-core expert pool and its pinned staging
    // (original expert ids, slot ids, weights, x, the CPU partial)
    moe::CpuExperts *cpu = nullptr;
    void *hyb_host = nullptr;
    int32_t *h_experts = nullptr, *h_slots = nullptr;
    float *h_w = nullptr, *h_partial = nullptr, *d_partial = nullptr;
    uint16_t *h_x = nullptr;
    std::vector<int32_t> cpu_ids;
    hipEvent_t hyb_ready = nullptr;
    // timing
    int timing = 0;
    std::vector<hipEvent_t> tev;     // [L * 6]: admission, gather, routed start/end
    std::vector<int> trecorded;      // [L]
};

namespace moe {
namespace api {

PoolView slot_pool_view(const moe_cache *c);
// Orders s after the copy of a pending look-ahead prefetch.
moe_status_t join_prefetch(moe_cache *c, hipStream_t s);
// The admission launch (after join_prefetch).  With logits set, the
// admission computes the top-k of T rows itself (R = T * K).
moe_status_t launch_admit_checked(moe_cache *c, int layer, int32_t *ids, int R, int max_fetch,
                                  hipStream_t s, int32_t *route_plan = nullptr,
                                  const float *logits = nullptr, int T = 0, int K = 0,
                                  float *w = nullptr);
// The gather of a plan of (slot, expert) rows of one layer, and of the
// last demand admission's miss plan.
GatherParams gather_params(const moe_cache *c, int layer, const int32_t *n, const int32_t *ps,
                           const int32_t *pe);
GatherParams gather_params(const moe_cache *c);
GatherParams gather_params_staged(const moe_cache *c);
moe_status_t launch_gather_checked(moe_cache *c, hipStream_t s);

}  // namespace api
}  // namespace moe
