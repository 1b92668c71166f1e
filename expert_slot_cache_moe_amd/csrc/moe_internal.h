// Internal declarations shared by the gfx950 kernels and the C ABI layer.
// Nothing here is part of the public interface (include/moe_cache.h).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "moe_cache.h"
#include "moe_record.h"

namespace moe {

constexpr int kWave = 64;

// 16-byte vector of four dwords (a native vector type, so the nontemporal
// builtins and the vector memory instructions accept it).
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// ------------------------------------------------------------------ formats

// bf16 <-> fp32.  bf16 is the upper half of an IEEE binary32.
__device__ __forceinline__ float bf16_lo(uint32_t packed) { return __uint_as_float(packed << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t packed) { return __uint_as_float(packed & 0xffff0000u); }
__device__ __forceinline__ float bf16_f(uint16_t b) { return __uint_as_float((uint32_t)b << 16); }

// Round to nearest, ties to even; NaN stays a (quiet) NaN.
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
    uint32_t u = __float_as_uint(f);
    if ((u & 0x7fffffffu) > 0x7f800000u) return (uint16_t)((u >> 16) | 0x40u);
    u += 0x7fffu + ((u >> 16) & 1u);
    return (uint16_t)(u >> 16);
}

// OCP E4M3 (fn): bias 7, exponent 0 subnormal, S.1111.111 NaN.
__device__ __forceinline__ float e4m3_f(uint32_t v) {
    uint32_t s = (v & 0x80u) << 24;
    uint32_t e = (v >> 3) & 0xFu;
    uint32_t m = v & 7u;
    float mag;
    if (e == 0) {
        mag = (float)m * 0.001953125f;  // m * 2^-9
    } else {
        mag = __uint_as_float(((e + 120u) << 23) | (m << 20));
    }
    if (e == 0xFu && m == 7u) mag = __uint_as_float(0x7fc00000u);
    return __uint_as_float(__float_as_uint(mag) | s);
}

// OCP MX E8M0 block scale: 2^(v - 127), v = 255 NaN (v = 0 is the
// subnormal float 2^-127).
__device__ __forceinline__ float e8m0_f(uint32_t v) {
    if (v == 0xFFu) return __uint_as_float(0x7fc00000u);
    return __uint_as_float(v ? (v << 23) : 0x00400000u);
}

// OCP E2M1: bias 1, exponent 0 subnormal (0 or 0.5).
__device__ __forceinline__ float e2m1_f(uint32_t n) {
    uint32_t e = (n >> 1) & 3u;
    uint32_t m = n & 1u;
    uint32_t bits = e ? (((e + 126u) << 23) | (m << 22)) : (m ? 0x3f000000u : 0u);
    return __uint_as_float(bits | ((n & 8u) << 28));
}

// ------------------------------------------------------------------ reductions

// Sum over aligned groups of `width` lanes (width a power of two <= 64).
template <int WIDTH>
__device__ __forceinline__ float group_sum(float v) {
#pragma unroll
    for (int off = WIDTH / 2; off > 0; off >>= 1) v += __shfl_xor(v, off, kWave);
    return v;
}

// ------------------------------------------------------------------ DPP lane operations

// DPP (data-parallel primitives) moves: a lane reads another lane's VGPR
// inside one VALU instruction.  Lanes whose source is out of range, or
// whose row is masked off, read 0.
template <int CTRL, int ROW_MASK = 0xf>
__device__ __forceinline__ uint32_t dpp_or_zero(uint32_t x) {
    return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, CTRL, ROW_MASK, 0xf, false);
}
constexpr int kDppRowShr1 = 0x111, kDppRowShr2 = 0x112, kDppRowShr4 = 0x114,
              kDppRowShr8 = 0x118, kDppRowBcast15 = 0x142, kDppRowBcast31 = 0x143;

// Inclusive prefix sum of x over the 64 lanes of a wave: shifts by 1, 2,
// 4, 8 within each 16-lane row, then the row totals carried forward with
// the two row broadcasts.
__device__ __forceinline__ int wave_inclusive_sum(int x) {
    uint32_t v = (uint32_t)x;
    v += dpp_or_zero<kDppRowShr1>(v);
    v += dpp_or_zero<kDppRowShr2>(v);
    v += dpp_or_zero<kDppRowShr4>(v);
    v += dpp_or_zero<kDppRowShr8>(v);
    v += dpp_or_zero<kDppRowBcast15, 0xa>(v);
    v += dpp_or_zero<kDppRowBcast31, 0xc>(v);
    return (int)v;
}

// Sum of v over each aligned group of WIDTH lanes (a power of two, at most
// the wave), valid in the group's last lane only.  The tree is pairwise,
// lanes paired by their low index bits first: row shifts by 1, 2, 4, 8,
// then the two row broadcasts.  The group's last lane reads only lanes of
// its own group, so groups may sit in divergent branches.
template <int WIDTH>
__device__ __forceinline__ float group_total(float v) {
    static_assert(WIDTH >= 1 && WIDTH <= kWave && (WIDTH & (WIDTH - 1)) == 0, "group width");
    uint32_t u = __float_as_uint(v);
#define MOE_ADD_STEP(CTRL, RM) u = __float_as_uint(__uint_as_float(u) + __uint_as_float(dpp_or_zero<CTRL, RM>(u)));
    if constexpr (WIDTH >= 2) MOE_ADD_STEP(kDppRowShr1, 0xf)
    if constexpr (WIDTH >= 4) MOE_ADD_STEP(kDppRowShr2, 0xf)
    if constexpr (WIDTH >= 8) MOE_ADD_STEP(kDppRowShr4, 0xf)
    if constexpr (WIDTH >= 16) MOE_ADD_STEP(kDppRowShr8, 0xf)
    if constexpr (WIDTH >= 32) MOE_ADD_STEP(kDppRowBcast15, 0xa)
    if constexpr (WIDTH >= 64) MOE_ADD_STEP(kDppRowBcast31, 0xc)
#undef MOE_ADD_STEP
    return __uint_as_float(u);
}

// Exclusive prefix count of `f` over a workgroup of THREADS threads;
// `total` gets the sum.  Every thread must call it: it holds two barriers.
// wsum: THREADS / 64 ints of LDS.
template <int THREADS>
__device__ __forceinline__ int block_scan_flags(bool f, int32_t *wsum, int &total) {
    constexpr int kW = THREADS / kWave;
    const int lane = threadIdx.x & (kWave - 1);
    const int wave = threadIdx.x / kWave;
    const uint64_t m = __ballot(f);
    const int pre = __builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32),
                                              __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0u));
    if (lane == 0) wsum[wave] = __popcll(m);
    __syncthreads();
    int off = 0, tot = 0;
#pragma unroll
    for (int w = 0; w < kW; ++w) {
        const int v = wsum[w];
        off += (w < wave) ? v : 0;
        tot += v;
    }
    __syncthreads();
    total = tot;
    return off + pre;
}

// Maximum of a 32-bit unsigned value over the wave, returned to every lane:
// a max-scan with the shift/broadcast pattern (lane 63 ends with the
// maximum), then read back from lane 63.
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
    v = max(v, dpp_or_zero<kDppRowShr1>(v));
    v = max(v, dpp_or_zero<kDppRowShr2>(v));
    v = max(v, dpp_or_zero<kDppRowShr4>(v));
    v = max(v, dpp_or_zero<kDppRowShr8>(v));
    v = max(v, dpp_or_zero<kDppRowBcast15, 0xa>(v));
    v = max(v, dpp_or_zero<kDppRowBcast31, 0xc>(v));
    return (uint32_t)__builtin_amdgcn_readlane((int)v, 63);
}

// Maximum of a 64-bit value over the wave, returned to every lane: the same
// shift/broadcast pattern as a max-scan (lane 63 ends with the maximum),
// then read back from lane 63.  Values must be >= 0 (0 fills the gaps).
__device__ __forceinline__ uint64_t wave_max_u64(uint64_t v) {
    uint32_t lo = (uint32_t)v, hi = (uint32_t)(v >> 32);
#define MOE_MAX_STEP(CTRL, RM)                                   \
    {                                                            \
        const uint32_t l2 = dpp_or_zero<CTRL, RM>(lo);           \
        const uint32_t h2 = dpp_or_zero<CTRL, RM>(hi);           \
        const bool gt = h2 > hi || (h2 == hi && l2 > lo);        \
        lo = gt ? l2 : lo;                                       \
        hi = gt ? h2 : hi;                                       \
    }
    MOE_MAX_STEP(kDppRowShr1, 0xf)
    MOE_MAX_STEP(kDppRowShr2, 0xf)
    MOE_MAX_STEP(kDppRowShr4, 0xf)
    MOE_MAX_STEP(kDppRowShr8, 0xf)
    MOE_MAX_STEP(kDppRowBcast15, 0xa)
    MOE_MAX_STEP(kDppRowBcast31, 0xc)
#undef MOE_MAX_STEP
    lo = (uint32_t)__builtin_amdgcn_readlane((int)lo, 63);
    hi = (uint32_t)__builtin_amdgcn_readlane((int)hi, 63);
    return ((uint64_t)hi << 32) | lo;
}

// ------------------------------------------------------------------ kernel parameters

struct AdmitParams {
    int32_t *ids;          // [R] in/out
    int32_t R;
    int32_t layer;
    int32_t max_fetch;
    int32_t E, S;
    int32_t one_call, query_width;
    int32_t *res;          // [L*E]
    int32_t *own;          // [S]
    uint32_t *stamp;       // [S]
    int32_t *order;        // LRU order, least recently used first: [S] slots, or, when
                           // admit_order_pairs(S), [S] (slot, owner) pairs
    uint32_t *clock;       // [2]: the clock, the clock value of the latest demand step
    int64_t *stats;        // [L*MOE_NUM_STATS]
    int64_t *freq;         // [L*E]
    uint32_t *dlast;       // [L*E] clock value of each expert's last demand step
    int32_t *plan_slot;    // [min(max_routes, E)]
    int32_t *plan_expert;
    int32_t *n_miss;       // [1]
    int32_t *route_plan;   // [R] or NULL: the plan entry filling the route's slot in this
                           // step, or -1 (the route's expert was already resident)
    // Optional fused top-k: with logits set, the step's expert ids are the
    // top-K of each of T rows of logits [T][E] (R = T*K), the weights go to
    // w_out [T][K], and ids is output only.
    const float *logits;
    int32_t T, K;
    float *w_out;
};

// One look-ahead prefetch: predicted ids of one layer, the admission state,
// and the fill plan it writes.
struct PrefetchParams {
    const int32_t *ids;    // [n]
    int32_t n;
    int32_t M;             // capacity of the per-prediction LDS arrays, >= min(n, E)
    int32_t layer;
    int32_t E, S;
    int32_t pairs;         // order holds (slot, owner) pairs
    int32_t *res, *own;
    uint32_t *stamp;
    int32_t *order;
    uint32_t *clock;       // [2]
    int64_t *stats;
    const int64_t *freq;
    const uint32_t *dlast;
    int32_t *fill_slot;    // [E]
    int32_t *fill_expert;  // [E]
    int32_t *n_fill;       // [1]
};

struct GatherParams {
    const int32_t *n_miss;
    const int32_t *plan_slot;
    const int32_t *plan_expert;
    int32_t nb;
    int32_t units_per_entry;               // copy units per plan entry, all banks
    int32_t unit_start[MOE_MAX_BANKS + 1]; // first unit of each bank
    const uint8_t *host[MOE_MAX_BANKS];    // layer's rows [E][rb], device-visible
    uint8_t *slot[MOE_MAX_BANKS];          // [S][rb]
    int64_t rb[MOE_MAX_BANKS];
    // Staged one-token step, 4-bit formats: bank 1 (the gate/up scales)
    // has no units of its own; each bank-0 unit copies the scales of its
    // chunks, carry_scales bytes per 16-byte chunk (2: E4M3 pair, 1: E8M0).
    // 0 everywhere else.
    int32_t carry_scales;
};

// Work items of the expert kernels.
enum ItemMode : int32_t {
    ITEM_ROUTE = 0,  // item g = route g: pool row idx[g] (skip < 0), token g / K
    ITEM_GROUP = 1,  // item g = group g of routes that share a pool row
    ITEM_ALL = 2,    // item 0 = routes 0..n-1 on pool row 0, token = route
};

struct Items {
    int32_t mode;
    const int32_t *route_plan;  // ITEM_ROUTE filter: NULL = every route, else routes whose
    int32_t want_fresh;         //   (route_plan[r] >= 0) == want_fresh
    int32_t K;                  // routes per token (ITEM_ROUTE)
    int32_t n;                  // routes (ITEM_ROUTE / ITEM_ALL)
    const int32_t *idx;         // [routes] pool rows (ITEM_ROUTE)
    const int32_t *n_groups;    // [1] (ITEM_GROUP)
    const int32_t *grp_row;     // [min(routes, rows)] pool row per group, -1 past the last
    const int32_t *grp_start;   // [groups]
    const int32_t *grp_count;   // [groups]
    const int32_t *grp_routes;  // [routes] route ids sorted by group
};

struct PoolView {
    int32_t fmt, H, F;
    int32_t num_rows;           // rows in the pool; rows outside [0, num_rows) are skipped
    const uint8_t *bank[MOE_MAX_BANKS];
    int64_t rb[MOE_MAX_BANKS];
};

// Bytes of one expert's row in bank b (0 past the format's last bank):
// bf16 [gate|up][H] and down [H][F]; E2M1 gate/up codes, their E4M3 scales
// (one per 16), the fp32 global scale, then the same three for down; MXFP4
// gate/up codes, their E8M0 scales (one per 32), then down's two.
constexpr int64_t bank_row_bytes(int fmt, int b, int H, int F) {
    const int64_t up = (int64_t)2 * F * H, dn = (int64_t)H * F;
    if (fmt == MOE_FMT_BF16) return b == 0 ? up * 2 : b == 1 ? dn * 2 : 0;
    if (fmt == MOE_FMT_MXFP4) return b == 0 ? up / 2 : b == 1 ? up / 32 : b == 2 ? dn / 2 : b == 3 ? dn / 32 : 0;
    return b == 0 ? up / 2 : b == 1 ? up / 16 : b == 2 ? 4 : b == 3 ? dn / 2 : b == 4 ? dn / 16 : b == 5 ? 4 : 0;
}
constexpr int bank_count(int fmt) { return fmt == MOE_FMT_BF16 ? 2 : fmt == MOE_FMT_MXFP4 ? 4 : 6; }

// ------------------------------------------------------------------ launchers

hipError_t launch_topk(const float *logits, int T, int E, int K, int32_t *ids, float *w,
                       hipStream_t s);
// Admission.  admit_lds_bytes sizes the launch for the largest step;
// admit_prepare raises the kernels' LDS limit once; launch_admit picks the
// register-resident kernel when the slot count allows it.
hipError_t launch_admit(const AdmitParams &p, size_t lds_bytes, hipStream_t s);
size_t admit_lds_bytes(int E, int S, int max_routes);
hipError_t admit_prepare(size_t lds_bytes);
bool admit_fused_topk_supported(int E, int S, int K);
// Bytes of the LRU order buffer for S slots (padded for whole-vector loads).
size_t admit_order_bytes(int S);
bool admit_order_pairs(int S);
// Hybrid step: addend[i] = (accumulate ? addend[i] : 0) + partial[i], the
// partial read from device-mapped host memory.
hipError_t launch_hybrid_add(float *addend, const float *partial, int n, int accumulate,
                             hipStream_t s);
size_t prefetch_lds_bytes(int M, int E, int S);
// Allows the prefetch kernel lds_bytes of dynamic LDS (needed above 64 KB).
hipError_t prefetch_prepare(size_t lds_bytes);
hipError_t launch_prefetch(const PrefetchParams &p, hipStream_t s);
hipError_t launch_gather(const GatherParams &p, int workgroups, hipStream_t s);
int gather_unit_bytes();

// Expert kernels.  h: bf16 [routes][F]; d: fp32 [routes][H].
size_t group_lds_bytes(int routes);
hipError_t group_prepare(size_t lds_bytes);
hipError_t launch_group_routes(const int32_t *idx, int routes, int num_rows, int32_t *n_groups,
                               int32_t *grp_row, int32_t *grp_start, int32_t *grp_count,
                               int32_t *grp_routes, hipStream_t s);
hipError_t launch_up(const PoolView &pool, const Items &items, int max_items, const uint16_t *x,
                     uint16_t *h, const uint16_t *gate_vec, float *gamma, hipStream_t s);
hipError_t launch_down_to_d(const PoolView &pool, const Items &items, int max_items,
                            const uint16_t *h, float *d, const float *gamma, hipStream_t s);
// d/route_plan optional (both or neither): routes with route_plan < 0 read
// their down projection from d instead of computing it.
hipError_t launch_down_fused(const PoolView &pool, const int32_t *idx, const float *w, int T,
                             int K, const uint16_t *h, const float *addend, const float *d,
                             const int32_t *route_plan, uint16_t *out, hipStream_t s);
hipError_t launch_combine(const int32_t *idx, const float *w, int T, int K, int H, int num_rows,
                          const float *d, const float *addend, uint16_t *out, hipStream_t s);

// The single-token layer step in two launches: stage 1 = miss gather
// (+ the fetched experts' gate/up dots into gu [plan][2F]) | shared gate/up
// | resident routes' gate/up; stage 2 = all down projections + combine.
bool stage_supported(int fmt, int H, int F);
hipError_t launch_stages(const GatherParams &g, int gather_blocks, float *gu, const PoolView &slots,
                         const int32_t *idx, const float *w, const int32_t *route_plan, int K,
                         const uint16_t *x, uint16_t *h, const PoolView *shared, uint16_t *hs,
                         const uint16_t *gate_vec, float *gamma, const float *addend, uint16_t *out,
                         int which, hipStream_t s);   // which: 1 stage 1, 2 stage 2, 3 both
// (route_plan NULL: no route was fetched in this step; gather_blocks 0: no
// gather; shared NULL: no shared expert; addend NULL: nothing added)

// Shape support of the expert kernels for one matrix width.
bool expert_shape_supported(int fmt, int H, int F);

// Wide steps (k_group.hip): counting-sort grouping and the MFMA group kernels.
constexpr int kGroupCountMaxLds = 4 * (32 + 32768);  // pools of up to 32768 rows
size_t group_count_lds_bytes(int num_rows);
bool group_count_supported(int num_rows, int routes);
hipError_t group_count_prepare();
hipError_t launch_group_count(const int32_t *idx, int routes, int num_rows, int32_t *n_groups,
                              int32_t *grp_row, int32_t *grp_start, int32_t *grp_count,
                              int32_t *grp_routes, hipStream_t s);
bool group_mfma_supported(int fmt, int H, int F);
hipError_t launch_up_mfma(const PoolView &pool, const Items &items, int max_items, const uint16_t *x,
                          uint16_t *h, hipStream_t s);
hipError_t launch_down_mfma(const PoolView &pool, const Items &items, int max_items, const uint16_t *h,
                            float *d, hipStream_t s);

}  // namespace moe
