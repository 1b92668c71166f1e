// Wide steps: routes grouped by pool row, each group's expert applied to
// all of its tokens with MFMA (gfx950 v_mfma_f32_16x16x32_bf16).
//
// What is computed is the routed expert of FreeToken issue #753 (section
// "What we changed") over pool rows, as in the single-token kernels:
//   g = W1[r] x, u = W3[r] x (fp32 accumulation), h = bf16(silu(g) * u),
//   d = W2[r] h (fp32), combined later as sum_k w[t][k] d[t][k].
// A group is the set of routes of one step that share a pool row (one
// expert), so its weights stream from HBM once per step and meet every
// token of the group in the matrix cores: weights are the MFMA A operand
// (16 rows x 32 contraction elements), tokens the B operand (16 columns).
//
// Tiling on CDNA4: a wave owns 16 output rows and sweeps the contraction
// dimension in slabs of 128 elements.  Lane l = 16 q + c loads 32
// consecutive elements [k0 + 32 q, k0 + 32 q + 32) of weight row c (64
// bytes of bf16, or 16 bytes of 4-bit codes and two scales) and the same
// element range of token column c, and feeds them to four MFMAs: the
// contraction index is permuted identically on both operands, which leaves
// the sum unchanged and makes every load a full 16-byte vector.
//
// 4-bit weights (OCP E2M1 with one E4M3 scale per 16 elements, FreeToken
// PR #491 section 5) are expanded to bf16 in registers: the product of an
// E2M1 value and an E4M3 scale has at most six significant bits, so it is
// exact in bf16, and the MFMA sees exactly the dequantized weights.
#include <algorithm>

#include "k_expert.inc"

namespace moe {
namespace mfma_detail {

using namespace expert_detail;

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));

constexpr int kTile = 16;                       // rows and tokens of one MFMA tile
constexpr int kSlab = 128;                      // contraction elements per sweep step
// One wave per workgroup: the waves of a group's row tiles share nothing
// (each loads its own weight rows and token columns), and single-wave
// workgroups let the dispatcher fill every free wave slot, which shortens
// the tail of a launch with few groups (measured: the wide decode steps
// run 7-10% faster than with four-wave workgroups).
constexpr int kMWaves = 1;
constexpr int kMThreads = kMWaves * kWave;

__device__ __forceinline__ f32x4 mfma(u32x4 a, u32x4 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                  __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}

// One lane's 32 weights of one row for one slab, as four MFMA operands.
template <int FMT> struct ASlab;

template <> struct ASlab<MOE_FMT_BF16> {
    u32x4 v[4];
    // m: 0 = gate/up matrix, 1 = down matrix; row r of pool row prow.
    __device__ __forceinline__ void load(const PoolView &p, int64_t prow, int m, int r, int e0) {
        const int ncols = m == 0 ? p.H : p.F;
        const u32x4 *src = reinterpret_cast<const u32x4 *>(p.bank[m] + prow * p.rb[m] +
                                                           ((int64_t)r * ncols + e0) * 2);
#pragma unroll
        for (int i = 0; i < 4; ++i) v[i] = src[i];
    }
    __device__ __forceinline__ void expand(u32x4 (&a)[4]) const {
#pragma unroll
        for (int i = 0; i < 4; ++i) a[i] = v[i];
    }
};

template <> struct ASlab<MOE_FMT_E2M1> {
    u32x4 codes;   // 32 nibbles, element 2b in the low nibble of byte b
    uint32_t sc;   // two E4M3 scales (elements 0-15, 16-31)
    __device__ __forceinline__ void load(const PoolView &p, int64_t prow, int m, int r, int e0) {
        const int ncols = m == 0 ? p.H : p.F;
        const int b = 3 * m;
        codes = *reinterpret_cast<const u32x4 *>(p.bank[b] + prow * p.rb[b] +
                                                 (int64_t)r * (ncols / 2) + e0 / 2);
        sc = *reinterpret_cast<const uint16_t *>(p.bank[b + 1] + prow * p.rb[b + 1] +
                                                 (int64_t)r * (ncols / 16) + e0 / 16);
    }
    // codes * scale as bf16 pairs (exact): the hardware converts two codes
    // to fp32, the scale multiplies in fp32, and the upper halves are kept.
    __device__ __forceinline__ void expand(u32x4 (&a)[4]) const {
        const float s0 = e4m3_f(sc & 0xffu), s1 = e4m3_f(sc >> 8);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const uint32_t word = codes[i];
            const float s = i < 2 ? s0 : s1;
            u32x4 o;
#define MOE_EXPAND_BYTE(B)                                                                \
    {                                                                                     \
        const f32x2 f = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(word, 1.0f, B);          \
        o[B] = __builtin_amdgcn_perm(__float_as_uint(f.y * s), __float_as_uint(f.x * s),  \
                                     0x07060302u);                                        \
    }
            MOE_EXPAND_BYTE(0)
            MOE_EXPAND_BYTE(1)
            MOE_EXPAND_BYTE(2)
            MOE_EXPAND_BYTE(3)
#undef MOE_EXPAND_BYTE
            a[i] = o;
        }
    }
};

// MXFP4: a lane's 32 elements of a slab are exactly one E8M0 scale block;
// gfx950 converts two codes to bf16 with the block's power-of-two scale in
// one instruction, exactly (E2M1 times a power of two fits bf16).
template <> struct ASlab<MOE_FMT_MXFP4> {
    u32x4 codes;
    uint32_t sc;
    __device__ __forceinline__ void load(const PoolView &p, int64_t prow, int m, int r, int e0) {
        const int ncols = m == 0 ? p.H : p.F;
        const int b = 2 * m;
        codes = *reinterpret_cast<const u32x4 *>(p.bank[b] + prow * p.rb[b] +
                                                 (int64_t)r * (ncols / 2) + e0 / 2);
        sc = p.bank[b + 1][prow * p.rb[b + 1] + (int64_t)r * (ncols / 32) + e0 / 32];
    }
    __device__ __forceinline__ void expand(u32x4 (&a)[4]) const {
        const float s = e8m0_f(sc);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const uint32_t word = codes[i];
            u32x4 o;
#define MOE_MX_BYTE(B) \
    o[B] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(word, s, B));
            MOE_MX_BYTE(0)
            MOE_MX_BYTE(1)
            MOE_MX_BYTE(2)
            MOE_MX_BYTE(3)
#undef MOE_MX_BYTE
            a[i] = o;
        }
    }
};

template <int FMT>
__device__ __forceinline__ float matrix_glob(const PoolView &p, int64_t prow, int m) {
    if constexpr (FMT == MOE_FMT_E2M1) {
        const int b = 3 * m + 2;
        return *reinterpret_cast<const float *>(p.bank[b] + prow * p.rb[b]);
    } else {
        return 1.f;
    }
}

// 32 bf16 activations of one token row for one slab.
__device__ __forceinline__ void load_b(const uint16_t *row, int e0, u32x4 (&b)[4]) {
    const u32x4 *src = reinterpret_cast<const u32x4 *>(row + e0);
#pragma unroll
    for (int i = 0; i < 4; ++i) b[i] = src[i];
}

// A gate/up wave takes UT row tiles (16 gate and 16 up rows each) that share
// the activation operand, and keeps NB slabs of them in flight: slab s lives
// in buffer s % NB; once it is consumed, the buffer is refilled with slab
// s + NB, so loads stay in flight while the matrix cores work.  A bf16 slab
// of one tile carries 8 KB, a 4-bit one 2.3 KB.  The launcher picks (UT, NB)
// per format and width: measured on MI355X, E2M1 runs best with one tile
// and three slabs ahead, MXFP4 with two tiles and two slabs, bf16 with one
// tile and two slabs, or two tiles at FFN widths of 1024 and more (3% on
// the prefill chunks, 4% slower at width 256).

// The group table entry gi (row -1 past the last group).
struct GroupEntry {
    int row = -1, count = 0, start = -1;
    __device__ __forceinline__ void load(const Items &items, int gi, int gmax) {
        if (gi < gmax) {
            row = items.grp_row[gi];
            count = items.grp_count[gi];
            start = items.grp_start[gi];
        } else {
            row = -1;
        }
    }
    __device__ __forceinline__ bool valid(int num_rows) const {
        return (row >= 0) & (row < num_rows) & (count > 0) & (start >= 0);
    }
};

// gate/up + SwiGLU, 16 * UT rows j per wave, for the groups blockIdx.y,
// blockIdx.y + gridDim.y, ...: h[route][j] = bf16(silu(g) * u) for every
// route of a group.  The grid holds about as many workgroups as the device
// keeps resident; the group table is a prefix of valid groups followed by
// row -1, so the first invalid entry ends the loop.  The next group's
// table entry is read while the current one is computed; a group's weights
// are requested before its route list and token rows (two dependent
// loads) are read.  Tokens go through the matrix cores 16 at a time; a
// group of more than 16 routes streams its rows once per 16.
template <int FMT, int UT, int NB>
__global__ __launch_bounds__(kMThreads, 2) void up_mfma_kernel(PoolView pool, Items items,
                                                               const uint16_t *__restrict__ x,
                                                               uint16_t *__restrict__ h) {
    const int H = pool.H, F = pool.F, K = items.K;
    const int wave = threadIdx.x / kWave, lane = threadIdx.x & (kWave - 1);
    const int c = lane & (kTile - 1), q = lane / kTile;
    const int j0 = (blockIdx.x * kMWaves + wave) * kTile * UT;
    if (j0 >= F) return;
    const int gmax = min(items.n, pool.num_rows);
    const int nslab = H / kSlab;
    GroupEntry cur;
    cur.load(items, blockIdx.y, gmax);
    for (int gi = blockIdx.y; gi < gmax && cur.valid(pool.num_rows); gi += gridDim.y) {
        GroupEntry nxt;
        nxt.load(items, gi + gridDim.y, gmax);
        const int64_t row = cur.row;
        const int32_t *list = items.grp_routes + cur.start;
        for (int base = 0; base < cur.count; base += kTile) {
            ASlab<FMT> wg[NB][UT], wu[NB][UT];
            u32x4 xb[NB][4];
            auto load_w = [&](int s, int bfr) {
                const int e0 = s * kSlab + 32 * q;
#pragma unroll
                for (int t = 0; t < UT; ++t) {
                    wg[bfr][t].load(pool, row, 0, j0 + kTile * t + c, e0);
                    wu[bfr][t].load(pool, row, 0, F + j0 + kTile * t + c, e0);
                }
            };
#pragma unroll
            for (int bfr = 0; bfr < NB; ++bfr)
                if (bfr < nslab) load_w(bfr, bfr);
            const float glob = matrix_glob<FMT>(pool, row, 0);
            const int n = min(base + c, cur.count - 1);
            const uint16_t *xr = x + (int64_t)(list[n] / K) * H;
#pragma unroll
            for (int bfr = 0; bfr < NB; ++bfr)
                if (bfr < nslab) load_b(xr, bfr * kSlab + 32 * q, xb[bfr]);
            f32x4 ag[UT], au[UT];
#pragma unroll
            for (int t = 0; t < UT; ++t) ag[t] = au[t] = f32x4{0.f, 0.f, 0.f, 0.f};
            for (int s0 = 0; s0 < nslab; s0 += NB) {
#pragma unroll
                for (int bfr = 0; bfr < NB; ++bfr) {
                    const int s = s0 + bfr;
                    if (s < nslab) {
#pragma unroll
                        for (int t = 0; t < UT; ++t) {
                            u32x4 ga[4], ua[4];
                            wg[bfr][t].expand(ga);
                            wu[bfr][t].expand(ua);
#pragma unroll
                            for (int i = 0; i < 4; ++i) {
                                ag[t] = mfma(ga[i], xb[bfr][i], ag[t]);
                                au[t] = mfma(ua[i], xb[bfr][i], au[t]);
                            }
                        }
                        if (s + NB < nslab) {
                            load_w(s + NB, bfr);
                            load_b(xr, (s + NB) * kSlab + 32 * q, xb[bfr]);
                        }
                    }
                }
            }
            // lane holds rows j0 + 16t + 4q + i (i < 4) of token column c
            if (base + c < cur.count) {
                const int64_t r = list[base + c];
#pragma unroll
                for (int t = 0; t < UT; ++t)
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        const float g = ag[t][i] * glob, u = au[t][i] * glob;
                        h[r * F + j0 + kTile * t + 4 * q + i] = f32_to_bf16(silu_mul(g, u));
                    }
            }
        }
        cur = nxt;
    }
}

// down projection, 16 * RT rows i per wave, for the groups blockIdx.y,
// blockIdx.y + gridDim.y, ... (as in up_mfma_kernel):
// d[route][i] = (W2 h[route])_i, fp32, NB slabs in flight.  Its contraction
// (F) is short, so a wave takes several row tiles to keep enough bytes in
// flight; the activation operand is shared by all of them.
template <int FMT, int RT, int NB>
__global__ __launch_bounds__(kMThreads, 2) void down_mfma_kernel(PoolView pool, Items items,
                                                              const uint16_t *__restrict__ h,
                                                              float *__restrict__ d) {
    const int H = pool.H, F = pool.F;
    const int wave = threadIdx.x / kWave, lane = threadIdx.x & (kWave - 1);
    const int c = lane & (kTile - 1), q = lane / kTile;
    const int i0 = (blockIdx.x * kMWaves + wave) * RT * kTile;
    if (i0 >= H) return;
    const int gmax = min(items.n, pool.num_rows);
    const int nslab = F / kSlab;
    GroupEntry cur;
    cur.load(items, blockIdx.y, gmax);
    for (int gi = blockIdx.y; gi < gmax && cur.valid(pool.num_rows); gi += gridDim.y) {
        GroupEntry nxt;
        nxt.load(items, gi + gridDim.y, gmax);
        const int64_t row = cur.row;
        const int32_t *list = items.grp_routes + cur.start;
        for (int base = 0; base < cur.count; base += kTile) {
            ASlab<FMT> w2[NB][RT];
            u32x4 hb[NB][4];
            auto load_w = [&](int s, int bfr) {
                const int e0 = s * kSlab + 32 * q;
#pragma unroll
                for (int rt = 0; rt < RT; ++rt)
                    w2[bfr][rt].load(pool, row, 1, min(i0 + rt * kTile, H - kTile) + c, e0);
            };
#pragma unroll
            for (int bfr = 0; bfr < NB; ++bfr)
                if (bfr < nslab) load_w(bfr, bfr);
            const float glob = matrix_glob<FMT>(pool, row, 1);
            const int n = min(base + c, cur.count - 1);
            const uint16_t *hr = h + (int64_t)list[n] * F;
#pragma unroll
            for (int bfr = 0; bfr < NB; ++bfr)
                if (bfr < nslab) load_b(hr, bfr * kSlab + 32 * q, hb[bfr]);
            f32x4 acc[RT];
#pragma unroll
            for (int rt = 0; rt < RT; ++rt) acc[rt] = f32x4{0.f, 0.f, 0.f, 0.f};
            for (int s0 = 0; s0 < nslab; s0 += NB) {
#pragma unroll
                for (int bfr = 0; bfr < NB; ++bfr) {
                    const int s = s0 + bfr;
                    if (s < nslab) {
#pragma unroll
                        for (int rt = 0; rt < RT; ++rt) {
                            u32x4 wa[4];
                            w2[bfr][rt].expand(wa);
#pragma unroll
                            for (int i = 0; i < 4; ++i) acc[rt] = mfma(wa[i], hb[bfr][i], acc[rt]);
                        }
                        if (s + NB < nslab) {
                            load_w(s + NB, bfr);
                            load_b(hr, (s + NB) * kSlab + 32 * q, hb[bfr]);
                        }
                    }
                }
            }
            if (base + c < cur.count) {
                const int64_t r = list[base + c];
#pragma unroll
                for (int rt = 0; rt < RT; ++rt) {
                    const int ib = i0 + rt * kTile;
                    if (ib < H) {
                        float4 v;
                        v.x = acc[rt][0] * glob;
                        v.y = acc[rt][1] * glob;
                        v.z = acc[rt][2] * glob;
                        v.w = acc[rt][3] * glob;
                        *reinterpret_cast<float4 *>(d + r * H + ib + 4 * q) = v;
                    }
                }
            }
        }
        cur = nxt;
    }
}

// ------------------------------------------------------------------ grouping

// Routes grouped by pool row with a counting sort in LDS: per-row counts
// (atomics), one prefix sum over the rows numbers the groups in ascending
// row order, and each route lands at its row's start plus its arrival
// rank.  The order of routes inside a group is therefore not fixed; every
// consumer computes each route independently of its position.
constexpr int kCountThreads = 1024;
constexpr int kCountWaves = kCountThreads / kWave;
constexpr int kCountRoutesPerThread = 8;   // up to 8192 routes

__global__ __launch_bounds__(kCountThreads) void group_count_kernel(
    const int32_t *__restrict__ idx, int n, int num_rows, int32_t *__restrict__ n_groups,
    int32_t *__restrict__ grp_row, int32_t *__restrict__ grp_start, int32_t *__restrict__ grp_count,
    int32_t *__restrict__ grp_routes) {
    extern __shared__ __align__(16) int32_t lds[];
    int32_t *wsum = lds;          // [kCountWaves]
    int32_t *cnt = lds + 32;      // [num_rows] counts, then starts
    const int tid = threadIdx.x;
    const int lane = tid & (kWave - 1), wave = tid / kWave;

    for (int r = tid; r < num_rows; r += kCountThreads) cnt[r] = 0;
    __syncthreads();
    int row[kCountRoutesPerThread], pos[kCountRoutesPerThread];
#pragma unroll
    for (int k = 0; k < kCountRoutesPerThread; ++k) {
        const int i = tid + k * kCountThreads;
        const int r = i < n ? idx[i] : -1;
        row[k] = (r >= 0 && r < num_rows) ? r : -1;
        pos[k] = row[k] >= 0 ? atomicAdd(&cnt[row[k]], 1) : 0;
    }
    __syncthreads();

    // Each thread owns a run of rows: counts and non-empty rows, then one
    // block prefix sum of both (packed: routes in the low 16 bits, groups
    // in the high 16; both are at most 8192).
    const int run = (num_rows + kCountThreads - 1) / kCountThreads;
    const int r0 = tid * run;
    int routes = 0, groups = 0;
    for (int k = 0; k < run; ++k) {
        const int r = r0 + k;
        if (r < num_rows) {
            const int v = cnt[r];
            routes += v;
            groups += v > 0;
        }
    }
    const int packed = routes | (groups << 16);
    const int incl = wave_inclusive_sum(packed);
    if (lane == kWave - 1) wsum[wave] = incl;
    __syncthreads();
    int woff = 0, tot = 0;
#pragma unroll
    for (int w = 0; w < kCountWaves; ++w) {
        const int v = wsum[w];
        woff += w < wave ? v : 0;
        tot += v;
    }
    int pre = woff + incl - packed;
    int start = pre & 0xffff, g = pre >> 16;
    for (int k = 0; k < run; ++k) {
        const int r = r0 + k;
        if (r < num_rows) {
            const int v = cnt[r];
            if (v > 0) {
                grp_row[g] = r;
                grp_start[g] = start;
                grp_count[g] = v;
                ++g;
            }
            cnt[r] = start;
            start += v;
        }
    }
    if (tid == 0) n_groups[0] = tot >> 16;
    // group slots past the last group read as "no row"
    for (int gg = (tot >> 16) + tid; gg < min(n, num_rows); gg += kCountThreads) grp_row[gg] = -1;
    __syncthreads();
#pragma unroll
    for (int k = 0; k < kCountRoutesPerThread; ++k) {
        const int i = tid + k * kCountThreads;
        if (row[k] >= 0) grp_routes[cnt[row[k]] + pos[k]] = i;
    }
}

}  // namespace mfma_detail

// ------------------------------------------------------------------ launchers

bool group_mfma_supported(int fmt, int H, int F) {
    (void)fmt;
    return H >= mfma_detail::kSlab && F >= mfma_detail::kSlab && H % mfma_detail::kSlab == 0 &&
           F % mfma_detail::kSlab == 0;
}

namespace {
// Workgroups of `kern` the device keeps resident at once (computed once per
// kernel and device; 0 if the runtime cannot tell).
template <typename KERN>
int resident(KERN kern, int *cache) {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 16) return 0;
    if (cache[dev] == 0) {
        int cus = 0, per_cu = 0;
        if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
            hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kern, mfma_detail::kMThreads, 0) !=
                hipSuccess)
            return 0;
        cache[dev] = std::max(1, cus * per_cu);
    }
    return cache[dev];
}

// Group rows of the grid: every group gets a workgroup row when the device
// holds them all at once, else as many rows as it holds.
int group_rows(int max_items, int cols, int resident_wgs) {
    if (resident_wgs <= 0) return max_items;
    return std::max(1, std::min(max_items, resident_wgs / std::max(cols, 1)));
}

// F is a multiple of kSlab (group_mfma_supported), so every wave's UT row
// tiles lie inside the FFN width.
template <int FMT, int UT, int NB>
hipError_t launch_up_shape(const PoolView &pool, const Items &items, int max_items, const uint16_t *x,
                           uint16_t *h, hipStream_t s) {
    using namespace mfma_detail;
    static_assert(kSlab % (kMWaves * kTile * UT) == 0, "row tiles of a workgroup divide a slab");
    static int res[16];
    const int rows = kMWaves * kTile * UT;
    const int cols = pool.F / rows;
    const dim3 grid(cols, group_rows(max_items, cols, resident(up_mfma_kernel<FMT, UT, NB>, res)));
    hipLaunchKernelGGL((up_mfma_kernel<FMT, UT, NB>), grid, dim3(kMThreads), 0, s, pool, items, x, h);
    return hipGetLastError();
}

template <int FMT, int RT, int NB>
hipError_t launch_down_shape(const PoolView &pool, const Items &items, int max_items, const uint16_t *h,
                             float *d, hipStream_t s) {
    using namespace mfma_detail;
    static int res[16];
    const int rows = kMWaves * kTile * RT;
    const int cols = (pool.H + rows - 1) / rows;
    const dim3 grid(cols, group_rows(max_items, cols, resident(down_mfma_kernel<FMT, RT, NB>, res)));
    hipLaunchKernelGGL((down_mfma_kernel<FMT, RT, NB>), grid, dim3(kMThreads), 0, s, pool, items, h, d);
    return hipGetLastError();
}
}  // namespace

hipError_t launch_up_mfma(const PoolView &pool, const Items &items, int max_items, const uint16_t *x,
                          uint16_t *h, hipStream_t s) {
    using namespace mfma_detail;
    if (max_items <= 0) return hipSuccess;
    if (rec::on())
        return rec::launch("up_mfma_kernel", s,
                           {{x, rec::kRead}, {pool.bank[0], rec::kRead, rec::items_part(items.route_plan, items.want_fresh)},
                            {items.idx, rec::kRead}, {items.n_groups, rec::kRead}, {items.grp_row, rec::kRead},
                            {h, rec::kWrite}});
    if (pool.fmt == MOE_FMT_MXFP4) return launch_up_shape<MOE_FMT_MXFP4, 2, 2>(pool, items, max_items, x, h, s);
    if (pool.fmt == MOE_FMT_E2M1) return launch_up_shape<MOE_FMT_E2M1, 1, 3>(pool, items, max_items, x, h, s);
    if (pool.F >= 1024) return launch_up_shape<MOE_FMT_BF16, 2, 2>(pool, items, max_items, x, h, s);
    return launch_up_shape<MOE_FMT_BF16, 1, 2>(pool, items, max_items, x, h, s);
}

hipError_t launch_down_mfma(const PoolView &pool, const Items &items, int max_items, const uint16_t *h,
                            float *d, hipStream_t s) {
    using namespace mfma_detail;
    if (max_items <= 0) return hipSuccess;
    if (rec::on())
        return rec::launch("down_mfma_kernel", s,
                           {{h, rec::kRead}, {pool.bank[0], rec::kRead, rec::items_part(items.route_plan, items.want_fresh)},
                            {items.idx, rec::kRead}, {items.n_groups, rec::kRead}, {items.grp_row, rec::kRead},
                            {d, rec::kWrite}});
    // One slab in flight: measured on MI355X, the smaller register demand
    // (152 VGPRs for the 4-bit formats against 221 with two) lets three
    // waves share a SIMD, which beats a second buffer (E2M1 wide step 3%,
    // bf16 and MXFP4 1%); other tile counts were slower.
    if (pool.fmt == MOE_FMT_MXFP4) return launch_down_shape<MOE_FMT_MXFP4, 4, 1>(pool, items, max_items, h, d, s);
    if (pool.fmt == MOE_FMT_E2M1) return launch_down_shape<MOE_FMT_E2M1, 4, 1>(pool, items, max_items, h, d, s);
    return launch_down_shape<MOE_FMT_BF16, 2, 1>(pool, items, max_items, h, d, s);
}

size_t group_count_lds_bytes(int num_rows) { return (32 + (size_t)num_rows) * 4; }

bool group_count_supported(int num_rows, int routes) {
    return routes <= mfma_detail::kCountThreads * mfma_detail::kCountRoutesPerThread &&
           group_count_lds_bytes(num_rows) <= (size_t)kGroupCountMaxLds;
}

hipError_t group_count_prepare() {
    return hipFuncSetAttribute(reinterpret_cast<const void *>(&mfma_detail::group_count_kernel),
                               hipFuncAttributeMaxDynamicSharedMemorySize, kGroupCountMaxLds);
}

hipError_t launch_group_count(const int32_t *idx, int routes, int num_rows, int32_t *n_groups,
                              int32_t *grp_row, int32_t *grp_start, int32_t *grp_count,
                              int32_t *grp_routes, hipStream_t s) {
    using namespace mfma_detail;
    if (rec::on())
        return rec::launch("group_count_kernel", s,
                           {{idx, rec::kRead}, {n_groups, rec::kWrite}, {grp_row, rec::kWrite},
                            {grp_start, rec::kWrite}, {grp_count, rec::kWrite}, {grp_routes, rec::kWrite}});
    hipLaunchKernelGGL(group_count_kernel, dim3(1), dim3(kCountThreads), group_count_lds_bytes(num_rows),
                       s, idx, routes, num_rows, n_groups, grp_row, grp_start, grp_count, grp_routes);
    return hipGetLastError();
}

}  // namespace moe
