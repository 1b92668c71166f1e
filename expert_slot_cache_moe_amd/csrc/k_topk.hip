// Top-k routing: one wavefront per token row.
//
// FreeToken issue #753 (section "What we changed") orders the layer as
// router -> fused top-k -> admission.  For each row: the K largest logits,
// largest first, equal logits lower expert id first, NaN treated as
// -infinity; the weights are the softmax over the K selected logits.
//
// Each selection round is a wave-wide argmax over the elements that come
// strictly after the previous pick in that total order, so no "taken"
// mask is needed.  Lane k keeps pick k; the softmax is a wave reduction.
#include "moe_internal.h"

namespace moe {
namespace {

constexpr int kRowsPerBlock = 4;

__device__ __forceinline__ float key_of(float v) { return v != v ? -INFINITY : v; }

// a comes before b in (value descending, index ascending) order
__device__ __forceinline__ bool before(float va, int ia, float vb, int ib) {
    return va > vb || (va == vb && ia < ib);
}

__global__ __launch_bounds__(kRowsPerBlock * kWave) void topk_kernel(const float *__restrict__ logits,
                                                                     int T, int E, int K,
                                                                     int32_t *__restrict__ ids,
                                                                     float *__restrict__ w) {
    const int lane = threadIdx.x & (kWave - 1);
    const int row = blockIdx.x * kRowsPerBlock + threadIdx.x / kWave;
    if (row >= T) return;
    const float *lr = logits + (int64_t)row * E;

    float prev_v = INFINITY;
    int prev_i = -1;
    float mine = -INFINITY;
    int mine_i = 0;
    for (int k = 0; k < K; ++k) {
        float bv = -INFINITY;
        int bi = 0x7fffffff;
        for (int e = lane; e < E; e += kWave) {
            const float v = key_of(lr[e]);
            if (before(prev_v, prev_i, v, e) && before(v, e, bv, bi)) {
                bv = v;
                bi = e;
            }
        }
#pragma unroll
        for (int off = kWave / 2; off > 0; off >>= 1) {
            const float ov = __shfl_xor(bv, off, kWave);
            const int oi = __shfl_xor(bi, off, kWave);
            if (before(ov, oi, bv, bi)) {
                bv = ov;
                bi = oi;
            }
        }
        if (lane == k) {
            mine = bv;
            mine_i = bi;
        }
        prev_v = bv;
        prev_i = bi;
    }

    const float m = __shfl(mine, 0, kWave);
    float ex = 0.f;
    if (lane < K) ex = (m == -INFINITY) ? 1.f : __expf(mine - m);
    // the same sum, in the same order, as the top-k fused into admission
    const float z = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(group_total<kWave>(ex)), kWave - 1));
    if (lane < K) {
        ids[(int64_t)row * K + lane] = mine_i;
        w[(int64_t)row * K + lane] = ex / z;
    }
}

}  // namespace

hipError_t launch_topk(const float *logits, int T, int E, int K, int32_t *ids, float *w,
                       hipStream_t s) {
    if (T == 0) return hipSuccess;
    if (rec::on())
        return rec::launch("topk_kernel", s, {{logits, rec::kRead}, {ids, rec::kWrite}, {w, rec::kWrite}});
    const int blocks = (T + kRowsPerBlock - 1) / kRowsPerBlock;
    hipLaunchKernelGGL(topk_kernel, dim3(blocks), dim3(kRowsPerBlock * kWave), 0, s, logits, T, E,
                       K, ids, w);
    return hipGetLastError();
}

}  // namespace moe
