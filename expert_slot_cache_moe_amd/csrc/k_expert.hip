// Routed and shared SwiGLU experts over pool rows (slot ids, or expert ids
// of a whole layer's pool), bf16 or 4-bit E2M1 weights.
//
// What is computed (FreeToken issue #753, sections "Problem in upstream
// today" and "What we changed"; FreeToken PR #491, section 5):
//   g = W1[r] x, u = W3[r] x (fp32 accumulation), h = bf16(silu(g) * u),
//   d = W2[r] h, out[t] = bf16(sum_k w[t][k] d[t][k] + addend[t]),
// summing k in ascending order and skipping -1 routes.  The arithmetic of
// a route depends only on the bytes of its pool row, never on the row's
// number, so a slot pool and a streamed layer pool give bit-identical
// results (FreeToken PR #680, section Tests).
//
// Layout and mapping on CDNA4:
//  - Weights are row-major [rows][cols], so one output element is a dot of
//    one contiguous weight row with the activation.  A row is read as
//    16-byte chunks; LPR lanes share a row (LPR = chunks per row, up to
//    64) so every lane issues full 16-byte loads and a wave reads whole
//    contiguous rows -- coalesced, no LDS round trip.  The activation
//    chunks a lane needs are the same for every row it touches and stay
//    in registers.  Partial sums are reduced across the LPR lanes with
//    xor shuffles in a fixed order.
//  - Routes are items: one route (decode, one token), or a group of
//    routes sharing a pool row (wide steps), so each expert's weights are
//    read from HBM once per step; the tokens of a group loop over the
//    weights held in registers.
//  - The path is HBM-bound at decode sizes (2 flops per weight byte for
//    bf16), so it runs on the vector ALUs; no GEMM reshaping.
#include "k_expert.inc"

namespace moe {

// Instantiated in k_expert_bf16.hip, k_expert_e2m1.hip and k_expert_mxfp4.hip.
namespace expert_detail {
#define MOE_EXTERN_FMT(FMT)                                                                        \
    extern template hipError_t launch_up_fmt<FMT>(const PoolView &, const Items &, int,            \
                                                  const uint16_t *, uint16_t *, const uint16_t *,  \
                                                  float *, hipStream_t);                           \
    extern template hipError_t launch_down_to_d_fmt<FMT>(const PoolView &, const Items &, int,     \
                                                         const uint16_t *, float *, const float *, \
                                                         hipStream_t);                             \
    extern template hipError_t launch_down_fused_fmt<FMT>(const PoolView &, const int32_t *,       \
                                                          const float *, int, int,                 \
                                                          const uint16_t *, const float *,         \
                                                          const float *, const int32_t *,          \
                                                          uint16_t *, hipStream_t);
MOE_EXTERN_FMT(MOE_FMT_BF16)
MOE_EXTERN_FMT(MOE_FMT_E2M1)
MOE_EXTERN_FMT(MOE_FMT_MXFP4)
#undef MOE_EXTERN_FMT
}  // namespace expert_detail

using expert_detail::kThreads;
using expert_detail::kWavesPerBlock;

namespace {

// The ordered combine of per-route down projections (wide steps).
__global__ __launch_bounds__(kThreads) void combine_kernel(const int32_t *__restrict__ idx,
                                                           const float *__restrict__ w, int K,
                                                           int H, int num_rows,
                                                           const float *__restrict__ d,
                                                           const float *__restrict__ addend,
                                                           uint16_t *__restrict__ out) {
    const int t = blockIdx.y;
    const int i = blockIdx.x * kThreads + threadIdx.x;
    if (i >= H) return;
    float acc = 0.f;
    for (int k = 0; k < K; ++k) {
        const int64_t r = (int64_t)t * K + k;
        const int s = idx[r];
        if (s < 0 || s >= num_rows) continue;
        acc = fmaf(w[r], d[r * H + i], acc);
    }
    const float v = addend != nullptr ? acc + addend[(int64_t)t * H + i] : acc;
    out[(int64_t)t * H + i] = f32_to_bf16(v);
}

// The same combine (the same fma chain per output), 8 consecutive outputs
// per thread, for 16-byte aligned outputs and addends: each batch of 4
// routes' ids, weights and partials is loaded before any is used (a
// partial is read whether or not its route counts), which took the e2m1
// wide step 39.4 -> 38.8 us and the MXFP4 one 32.3 -> 31.5 us on MI355X.
constexpr int kCombineVec = 8, kCombineBatch = 4;
__global__ __launch_bounds__(kThreads) void combine8_kernel(const int32_t *__restrict__ idx,
                                                            const float *__restrict__ w, int K,
                                                            int H, int num_rows,
                                                            const float *__restrict__ d,
                                                            const float *__restrict__ addend,
                                                            uint16_t *__restrict__ out) {
    const int t = blockIdx.y;
    const int i0 = (blockIdx.x * blockDim.x + threadIdx.x) * kCombineVec;
    if (i0 >= H) return;
    float acc[kCombineVec];
#pragma unroll
    for (int e = 0; e < kCombineVec; ++e) acc[e] = 0.f;
    for (int k0 = 0; k0 < K; k0 += kCombineBatch) {
        int s[kCombineBatch];
        float wk[kCombineBatch];
        float4 a[kCombineBatch], b[kCombineBatch];
#pragma unroll
        for (int q = 0; q < kCombineBatch; ++q) {
            const int64_t r = (int64_t)t * K + min(k0 + q, K - 1);
            s[q] = idx[r];
            wk[q] = w[r];
            a[q] = *reinterpret_cast<const float4 *>(d + r * H + i0);
            b[q] = *reinterpret_cast<const float4 *>(d + r * H + i0 + 4);
        }
#pragma unroll
        for (int q = 0; q < kCombineBatch; ++q) {
            if (k0 + q >= K || s[q] < 0 || s[q] >= num_rows) continue;
            acc[0] = fmaf(wk[q], a[q].x, acc[0]);
            acc[1] = fmaf(wk[q], a[q].y, acc[1]);
            acc[2] = fmaf(wk[q], a[q].z, acc[2]);
            acc[3] = fmaf(wk[q], a[q].w, acc[3]);
            acc[4] = fmaf(wk[q], b[q].x, acc[4]);
            acc[5] = fmaf(wk[q], b[q].y, acc[5]);
            acc[6] = fmaf(wk[q], b[q].z, acc[6]);
            acc[7] = fmaf(wk[q], b[q].w, acc[7]);
        }
    }
    if (addend != nullptr) {
        const float4 p = *reinterpret_cast<const float4 *>(addend + (int64_t)t * H + i0);
        const float4 q = *reinterpret_cast<const float4 *>(addend + (int64_t)t * H + i0 + 4);
        acc[0] = acc[0] + p.x; acc[1] = acc[1] + p.y; acc[2] = acc[2] + p.z; acc[3] = acc[3] + p.w;
        acc[4] = acc[4] + q.x; acc[5] = acc[5] + q.y; acc[6] = acc[6] + q.z; acc[7] = acc[7] + q.w;
    }
    u32x4 o;
#pragma unroll
    for (int e = 0; e < 4; ++e) o[e] = f32_to_bf16(acc[2 * e]) | (f32_to_bf16(acc[2 * e + 1]) << 16);
    *reinterpret_cast<u32x4 *>(out + (int64_t)t * H + i0) = o;
}

// Groups routes by pool row: one workgroup ranks the (row, route) pairs
// (row ascending, then route) in LDS and writes the group table.
constexpr int kGroupThreads = 1024;
constexpr int kGroupWaves = kGroupThreads / kWave;

__global__ __launch_bounds__(kGroupThreads) void group_kernel(const int32_t *__restrict__ idx,
                                                              int n, int num_rows,
                                                              int32_t *__restrict__ n_groups,
                                                              int32_t *__restrict__ grp_row,
                                                              int32_t *__restrict__ grp_start,
                                                              int32_t *__restrict__ grp_count,
                                                              int32_t *__restrict__ grp_routes) {
    extern __shared__ __align__(16) int32_t lds[];
    int32_t *wsum = lds;           // [32]
    int32_t *key = lds + 32;       // [n]
    int32_t *skey = key + n;       // [n] sorted keys
    int32_t *sroute = skey + n;    // [n] routes in sorted order
    int32_t *gstart = sroute + n;  // [n + 1]
    const int tid = threadIdx.x;
    const int lane = tid & (kWave - 1), wave = tid / kWave;
    constexpr int kInvalid = 0x7fffffff;

    for (int i = tid; i < n; i += kGroupThreads) {
        const int r = idx[i];
        key[i] = (r >= 0 && r < num_rows) ? r : kInvalid;
    }
    __syncthreads();
    for (int i = tid; i < n; i += kGroupThreads) {
        const int ki = key[i];
        int rank = 0;
        for (int j = 0; j < n; ++j) {
            const int kj = key[j];
            rank += (kj < ki) || (kj == ki && j < i);
        }
        skey[rank] = ki;
        sroute[rank] = i;
    }
    __syncthreads();

    int ng = 0, nvalid = 0;
    for (int base = 0; base < n; base += kGroupThreads) {
        const int i = base + tid;
        const bool valid = i < n && skey[i] != kInvalid;
        const bool head = valid && (i == 0 || skey[i - 1] != skey[i]);
        const uint64_t mh = __ballot(head), mv = __ballot(valid);
        const int pre = __builtin_amdgcn_mbcnt_hi((uint32_t)(mh >> 32),
                                                  __builtin_amdgcn_mbcnt_lo((uint32_t)mh, 0u));
        if (lane == 0) {
            wsum[wave] = __popcll(mh);
            wsum[16 + wave] = __popcll(mv);
        }
        __syncthreads();
        int off = 0, toth = 0, totv = 0;
        for (int w = 0; w < kGroupWaves; ++w) {
            off += (w < wave) ? wsum[w] : 0;
            toth += wsum[w];
            totv += wsum[16 + w];
        }
        __syncthreads();
        if (head) {
            gstart[ng + off + pre] = i;
            grp_row[ng + off + pre] = skey[i];
            grp_start[ng + off + pre] = i;
        }
        ng += toth;
        nvalid += totv;
    }
    __syncthreads();
    for (int g = tid; g < ng; g += kGroupThreads)
        grp_count[g] = (g + 1 < ng ? gstart[g + 1] : nvalid) - gstart[g];
    for (int i = tid; i < nvalid; i += kGroupThreads) grp_routes[i] = sroute[i];
    // group slots past the last group read as "no row"
    for (int g = ng + tid; g < min(n, num_rows); g += kGroupThreads) grp_row[g] = -1;
    if (tid == 0) *n_groups = ng;
}

bool chunks_ok(int chunks, int max_chunks) {
    switch (chunks) {
    case 2: case 4: case 8: case 16: case 32: case 64: case 128: case 256: case 512:
        return chunks <= max_chunks;
    default: return false;
    }
}

int epc(int fmt) { return fmt == MOE_FMT_BF16 ? 8 : 32; }
int max_chunks(int fmt) {
    return fmt == MOE_FMT_BF16 ? expert_detail::MaxChunks<MOE_FMT_BF16>::v
                               : expert_detail::MaxChunks<MOE_FMT_E2M1>::v;  // = the MXFP4 limit
}

}  // namespace

bool expert_shape_supported(int fmt, int H, int F) {
    if (fmt != MOE_FMT_BF16 && fmt != MOE_FMT_E2M1 && fmt != MOE_FMT_MXFP4) return false;
    if (H <= 0 || F <= 0 || H % epc(fmt) || F % epc(fmt)) return false;
    // the shared gate reads H in 8-element chunks
    if (H % 8) return false;
    return chunks_ok(H / epc(fmt), max_chunks(fmt)) && chunks_ok(F / epc(fmt), max_chunks(fmt));
}

size_t group_lds_bytes(int n) { return (32 + 4 * (size_t)n + 1) * 4; }

hipError_t group_prepare(size_t lds_bytes) {
    if (lds_bytes <= 65536) return hipSuccess;
    return hipFuncSetAttribute(reinterpret_cast<const void *>(&group_kernel),
                               hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds_bytes);
}

hipError_t launch_group_routes(const int32_t *idx, int routes, int num_rows, int32_t *n_groups,
                               int32_t *grp_row, int32_t *grp_start, int32_t *grp_count,
                               int32_t *grp_routes, hipStream_t s) {
    if (rec::on())
        return rec::launch("group_kernel", s,
                           {{idx, rec::kRead}, {n_groups, rec::kWrite}, {grp_row, rec::kWrite},
                            {grp_start, rec::kWrite}, {grp_count, rec::kWrite}, {grp_routes, rec::kWrite}});
    hipLaunchKernelGGL(group_kernel, dim3(1), dim3(kGroupThreads), group_lds_bytes(routes), s, idx,
                       routes, num_rows, n_groups, grp_row, grp_start, grp_count, grp_routes);
    return hipGetLastError();
}

hipError_t launch_up(const PoolView &pool, const Items &items, int max_items, const uint16_t *x,
                     uint16_t *h, const uint16_t *gate_vec, float *gamma, hipStream_t s) {
    if (max_items <= 0) return hipSuccess;
    if (rec::on())
        return rec::launch("up_kernel", s,
                           {{x, rec::kRead}, {pool.bank[0], rec::kRead, rec::items_part(items.route_plan, items.want_fresh)},
                            {items.idx, rec::kRead}, {items.route_plan, rec::kRead}, {items.n_groups, rec::kRead},
                            {items.grp_row, rec::kRead}, {gate_vec, rec::kRead}, {h, rec::kWrite},
                            {gamma, rec::kWrite}});
    using namespace expert_detail;
    if (pool.fmt == MOE_FMT_MXFP4)
        return launch_up_fmt<MOE_FMT_MXFP4>(pool, items, max_items, x, h, gate_vec, gamma, s);
    return pool.fmt == MOE_FMT_BF16
               ? launch_up_fmt<MOE_FMT_BF16>(pool, items, max_items, x, h, gate_vec, gamma, s)
               : launch_up_fmt<MOE_FMT_E2M1>(pool, items, max_items, x, h, gate_vec, gamma, s);
}

hipError_t launch_down_to_d(const PoolView &pool, const Items &items, int max_items,
                            const uint16_t *h, float *d, const float *gamma, hipStream_t s) {
    if (max_items <= 0) return hipSuccess;
    if (rec::on())
        return rec::launch("down_d_kernel", s,
                           {{h, rec::kRead}, {pool.bank[0], rec::kRead, rec::items_part(items.route_plan, items.want_fresh)},
                            {items.idx, rec::kRead}, {items.route_plan, rec::kRead}, {items.n_groups, rec::kRead},
                            {items.grp_row, rec::kRead}, {gamma, rec::kRead}, {d, rec::kWrite}});
    using namespace expert_detail;
    if (pool.fmt == MOE_FMT_MXFP4)
        return launch_down_to_d_fmt<MOE_FMT_MXFP4>(pool, items, max_items, h, d, gamma, s);
    return pool.fmt == MOE_FMT_BF16
               ? launch_down_to_d_fmt<MOE_FMT_BF16>(pool, items, max_items, h, d, gamma, s)
               : launch_down_to_d_fmt<MOE_FMT_E2M1>(pool, items, max_items, h, d, gamma, s);
}

hipError_t launch_down_fused(const PoolView &pool, const int32_t *idx, const float *w, int T,
                             int K, const uint16_t *h, const float *addend, const float *d,
                             const int32_t *route_plan, uint16_t *out, hipStream_t s) {
    if (T <= 0) return hipSuccess;
    if (rec::on())
        // with a route plan, routes not filled this step take their down
        // projection from d; only the fresh routes read their slots
        return rec::launch("down_fused_kernel", s,
                           {{h, rec::kRead}, {pool.bank[0], rec::kRead, rec::items_part(route_plan, 1)},
                            {idx, rec::kRead}, {w, rec::kRead}, {addend, rec::kRead}, {d, rec::kRead},
                            {route_plan, rec::kRead}, {out, rec::kWrite}});
    using namespace expert_detail;
    if (pool.fmt == MOE_FMT_MXFP4)
        return launch_down_fused_fmt<MOE_FMT_MXFP4>(pool, idx, w, T, K, h, addend, d, route_plan, out, s);
    return pool.fmt == MOE_FMT_BF16
               ? launch_down_fused_fmt<MOE_FMT_BF16>(pool, idx, w, T, K, h, addend, d, route_plan, out, s)
               : launch_down_fused_fmt<MOE_FMT_E2M1>(pool, idx, w, T, K, h, addend, d, route_plan, out,
                                                     s);
}

hipError_t launch_combine(const int32_t *idx, const float *w, int T, int K, int H, int num_rows,
                          const float *d, const float *addend, uint16_t *out, hipStream_t s) {
    if (T <= 0) return hipSuccess;
    if (rec::on())
        return rec::launch("combine_kernel", s,
                           {{idx, rec::kRead}, {w, rec::kRead}, {d, rec::kRead}, {addend, rec::kRead},
                            {out, rec::kWrite}});
    const bool vec = H % kCombineVec == 0 && (reinterpret_cast<uintptr_t>(out) & 15) == 0 &&
                     (addend == nullptr || (reinterpret_cast<uintptr_t>(addend) & 15) == 0);
    if (vec) {
        const int lanes = H / kCombineVec;
        const int bs = std::min(kThreads, (lanes + kWave - 1) / kWave * kWave);
        hipLaunchKernelGGL(combine8_kernel, dim3((lanes + bs - 1) / bs, T), dim3(bs), 0, s, idx, w, K, H,
                           num_rows, d, addend, out);
        return hipGetLastError();
    }
    dim3 grid((H + kThreads - 1) / kThreads, T);
    hipLaunchKernelGGL(combine_kernel, grid, dim3(kThreads), 0, s, idx, w, K, H, num_rows, d,
                       addend, out);
    return hipGetLastError();
}

}  // namespace moe
