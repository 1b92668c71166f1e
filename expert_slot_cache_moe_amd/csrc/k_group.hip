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

// A lane's codes of one 4-bit weight row for the LDS-staged kernels, from
// slab 0, so slab s is a constant offset away (one address per row instead
// of one per slab in flight).
struct QRow {
    const uint8_t *codes;
    __device__ __forceinline__ void at(const PoolView &p, int fmt, int64_t prow, int m, int r, int q) {
        const int ncols = m == 0 ? p.H : p.F;
        const int b = (fmt == MOE_FMT_E2M1 ? 3 : 2) * m;
        codes = p.bank[b] + prow * p.rb[b] + (int64_t)r * (ncols / 2) + 16 * q;
    }
    __device__ __forceinline__ u32x4 load(int s) const {
        return *reinterpret_cast<const u32x4 *>(codes + s * (kSlab / 2));
    }
};

// The scales of 4-bit weight rows pass through LDS.  A slab's scales for a
// lane are 2 bytes (E2M1) or 1 byte (MXFP4) of its row, a few bytes apart
// from the next lane's: loaded straight from HBM, every slab costs a load
// instruction that touches 16 rows for a few bytes each, and those small
// requests, not the bytes, bounded the kernels (measured on MI355X: the
// gate/up kernel's loads took 22.7 us with them, 13.3 us without).  Each
// row's scale bytes are instead loaded in 4-16 byte vectors, written to
// LDS rows of SB + 4 bytes (bank spread), and read back per slab.
template <int FMT, int COLS> struct QScales {
    static constexpr int SB = COLS / (FMT == MOE_FMT_E2M1 ? 16 : 32);   // scale bytes per row
    static constexpr int PITCH = SB + 4;
    // scale byte offset of lane q's elements of slab s within a row
    __device__ static constexpr int offset(int s, int q) {
        return FMT == MOE_FMT_E2M1 ? 8 * s + 2 * q : 4 * s + q;
    }
    __device__ static const uint8_t *row_ptr(const PoolView &p, int64_t prow, int m, int r) {
        const int b = (FMT == MOE_FMT_E2M1 ? 3 : 2) * m + 1;
        return p.bank[b] + prow * p.rb[b] + (int64_t)r * SB;
    }
    // N bytes (a multiple of 4, 4-byte aligned) of scales in registers:
    // loaded from HBM, later written to LDS (after the code loads issue).
    template <int N> struct Chunk {
        static_assert(N % 4 == 0, "whole dwords");
        uint32_t v[N / 4];
        __device__ void load(const uint8_t *src) {
            if constexpr (N % 16 == 0) {
#pragma unroll
                for (int i = 0; i < N / 16; ++i) {
                    const u32x4 t = reinterpret_cast<const u32x4 *>(src)[i];
                    v[4 * i] = t[0], v[4 * i + 1] = t[1], v[4 * i + 2] = t[2], v[4 * i + 3] = t[3];
                }
            } else if constexpr (N == 8) {
                const uint2 t = *reinterpret_cast<const uint2 *>(src);
                v[0] = t.x, v[1] = t.y;
            } else {
                v[0] = *reinterpret_cast<const uint32_t *>(src);
            }
        }
        __device__ void store(uint8_t *dst) const {
#pragma unroll
            for (int i = 0; i < N / 4; ++i) reinterpret_cast<uint32_t *>(dst)[i] = v[i];
        }
    };
    __device__ static uint32_t read(const uint8_t *lds_row, int s, int q) {
        if constexpr (FMT == MOE_FMT_E2M1)
            return *reinterpret_cast<const uint16_t *>(lds_row + offset(s, q));
        else
            return lds_row[offset(s, q)];
    }
};

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

// The grouped kernels take what their first request needs -- the group
// table and its bounds -- as leading scalar arguments, which gfx950
// preloads into scalar registers at wave launch: the first group entry is
// requested without waiting for an argument load.
#define MOE_GROUP_LEAD_PARAMS                                                                       \
    const int32_t *__restrict__ lead_row, const int32_t *__restrict__ lead_count,                \
        const int32_t *__restrict__ lead_start, int lead_n, int lead_rows
#define MOE_GROUP_LEAD_ARGS(pool, items) \
    (items).grp_row, (items).grp_count, (items).grp_start, (items).n, (pool).num_rows
#define MOE_GROUP_TAKE_LEAD()             \
    PoolView pool = pool_in;              \
    Items items = items_in;               \
    pool.num_rows = lead_rows;            \
    items.grp_row = lead_row;             \
    items.grp_count = lead_count;         \
    items.grp_start = lead_start;         \
    items.n = lead_n

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
__global__ __launch_bounds__(kMThreads, 2) void up_mfma_kernel(MOE_GROUP_LEAD_PARAMS, PoolView pool_in,
                                                               Items items_in, const uint16_t *__restrict__ x,
                                                               uint16_t *__restrict__ h) {
    MOE_GROUP_TAKE_LEAD();
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
            // lane holds rows j0 + 16t + 4q + i (i < 4) of token column c:
            // four consecutive h elements, one 8-byte store
            if (base + c < cur.count) {
                const int64_t r = list[base + c];
#pragma unroll
                for (int t = 0; t < UT; ++t) {
                    uint32_t hv[4];
#pragma unroll
                    for (int i = 0; i < 4; ++i) hv[i] = f32_to_bf16(silu_mul(ag[t][i] * glob, au[t][i] * glob));
                    *reinterpret_cast<uint2 *>(h + r * F + j0 + kTile * t + 4 * q) =
                        make_uint2(hv[0] | (hv[1] << 16), hv[2] | (hv[3] << 16));
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
__global__ __launch_bounds__(kMThreads, 2) void down_mfma_kernel(MOE_GROUP_LEAD_PARAMS, PoolView pool_in,
                                                              Items items_in, const uint16_t *__restrict__ h,
                                                              float *__restrict__ d) {
    MOE_GROUP_TAKE_LEAD();
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

// ------------------------------------------------------------------ 4-bit weights, activations in LDS

// For 4-bit weights the activations are the larger operand: a 16-token
// batch of bf16 rows is four times the codes of a 16-row weight tile.  The
// kernels above hold a wave's own copy of them in registers, which leaves
// room for few weight slabs in flight at two waves per SIMD.  The kernels
// below stage a batch's 16 activation rows once per workgroup of four
// waves in LDS, and the scales of every wave's rows too (QScales); a wave
// keeps kXAhead slabs of codes in flight and three or four waves share a
// SIMD.  Measured on MI355X at the wide E2M1 step (H 1024, F 256, 160
// groups): gate/up 23.6 -> 18.2 us, down 12.7 -> 12.6 us; MXFP4 19.3 ->
// 14.1 and 11.1 -> 9.7 us.  Slab order, contraction permutation and MFMA
// sequence are those of the kernels above (with one row tile per gate/up
// wave), so both compute the same values.
constexpr int kXWaves = 4;
constexpr int kXThreads = kXWaves * kWave;
constexpr int kXPad = 8;          // bf16 elements of padding per staged row (bank spread)
constexpr int kXAhead = 4;        // slabs a gate/up wave keeps in flight
constexpr int kXDownAhead = 8;    // (row tile, slab) pairs a down wave keeps in flight

__host__ __device__ constexpr size_t x_rows_lds_bytes(int cols) { return (size_t)kTile * (cols + kXPad) * 2; }

// LDS of the staged kernels: the batch's rows, then the scales of every
// wave's weight rows (`scale_rows` rows of `scale_pitch` bytes per wave).
__host__ __device__ constexpr size_t x_lds_bytes(int cols, int scale_rows, int scale_pitch) {
    return x_rows_lds_bytes(cols) + (size_t)kXWaves * scale_rows * scale_pitch;
}

// Stages the batch's 16 rows of COLS bf16 elements (row `src_row` for this
// thread's token column threadIdx.x / (THREADS / 16), chosen by the caller)
// into LDS rows of COLS + kXPad.  The THREADS / 16 threads of a row copy
// its 16-byte vectors round-robin, so each load instruction reads whole
// runs of a row.  All threads of the workgroup take part; the caller
// places the barriers.
template <int COLS, int THREADS = kXThreads>
__device__ __forceinline__ void stage_rows(const uint16_t *__restrict__ src_row, uint16_t *__restrict__ xs) {
    constexpr int TPR = THREADS / kTile;     // threads per row
    constexpr int NV = COLS / 8 / TPR;       // vectors per thread
    static_assert(NV * TPR * 8 == COLS, "whole vectors per thread");
    const int t = threadIdx.x / TPR, part = threadIdx.x % TPR;
    const u32x4 *src = reinterpret_cast<const u32x4 *>(src_row) + part;
    u32x4 *dst = reinterpret_cast<u32x4 *>(xs + t * (COLS + kXPad)) + part;
#pragma unroll
    for (int v0 = 0; v0 < NV; v0 += 8) {
        u32x4 v[8];
#pragma unroll
        for (int i = 0; i < 8; ++i)
            if (v0 + i < NV) v[i] = src[(v0 + i) * TPR];
#pragma unroll
        for (int i = 0; i < 8; ++i)
            if (v0 + i < NV) dst[(v0 + i) * TPR] = v[i];
    }
}

// gate/up + SwiGLU as up_mfma_kernel (one row tile per wave, 64 gate and 64
// up rows per workgroup), the batch's activations from LDS; the hidden
// width is NS slabs (pool.H == NS * kSlab, launcher).
template <int FMT, int NS>
__global__ __launch_bounds__(kXThreads, 3) void up_x_kernel(MOE_GROUP_LEAD_PARAMS, PoolView pool_in,
                                                            Items items_in, const uint16_t *__restrict__ x,
                                                            uint16_t *__restrict__ h) {
    extern __shared__ __align__(16) uint16_t xs[];   // [kTile][H + kXPad], then scales
    MOE_GROUP_TAKE_LEAD();
    constexpr int H = NS * kSlab, nslab = NS;
    constexpr int AHEAD = NS < kXAhead ? NS : kXAhead;
    using QS = QScales<FMT, H>;
    const int F = pool.F, K = items.K;
    const int wave = threadIdx.x / kWave, lane = threadIdx.x & (kWave - 1);
    const int c = lane & (kTile - 1), q = lane / kTile;
    const int j0 = (blockIdx.x * kXWaves + wave) * kTile;   // < F: F % 64 == 0 (launcher)
    const int gmax = min(items.n, pool.num_rows);
    const uint16_t *xc = xs + c * (H + kXPad) + 32 * q;
    // this wave's scale rows: gate rows 0-15, up rows 16-31
    uint8_t *qs = reinterpret_cast<uint8_t *>(xs + kTile * (H + kXPad)) + wave * 2 * kTile * QS::PITCH;
    GroupEntry cur;
    cur.load(items, blockIdx.y, gmax);
    for (int gi = blockIdx.y; gi < gmax && cur.valid(pool.num_rows); gi += gridDim.y) {
        GroupEntry nxt;
        nxt.load(items, gi + gridDim.y, gmax);
        const int64_t row = cur.row;
        const int32_t *list = items.grp_routes + cur.start;
        for (int base = 0; base < cur.count; base += kTile) {
            // scales first (lane (c, q) loads quarter q of row c's bytes)
            constexpr int QB = QS::SB / 4;
            typename QS::template Chunk<QB> sg, su;
            sg.load(QS::row_ptr(pool, row, 0, j0 + c) + q * QB);
            su.load(QS::row_ptr(pool, row, 0, F + j0 + c) + q * QB);
            ASlab<FMT> wg[AHEAD], wu[AHEAD];
            QRow rg, ru;
            rg.at(pool, FMT, row, 0, j0 + c, q);
            ru.at(pool, FMT, row, 0, F + j0 + c, q);
#pragma unroll
            for (int bfr = 0; bfr < AHEAD; ++bfr) {
                wg[bfr].codes = rg.load(bfr);
                wu[bfr].codes = ru.load(bfr);
            }
            const float glob = matrix_glob<FMT>(pool, row, 0);
            const int n = min(base + (int)threadIdx.x / kTile, cur.count - 1);
            const uint16_t *src = x + (int64_t)(list[n] / K) * H;
            sg.store(qs + c * QS::PITCH + q * QB);      // this wave's own rows: no barrier
            su.store(qs + (kTile + c) * QS::PITCH + q * QB);
            __syncthreads();   // the previous batch's rows are consumed
            stage_rows<H>(src, xs);
            __syncthreads();
            f32x4 ag = f32x4{0.f, 0.f, 0.f, 0.f}, au = ag;
#pragma unroll
            for (int s0 = 0; s0 < nslab; s0 += AHEAD) {
#pragma unroll
                for (int bfr = 0; bfr < AHEAD; ++bfr) {
                    const int s = s0 + bfr;
                    if (s < nslab) {
                        u32x4 ga[4], ua[4], xb[4];
                        const u32x4 *xp = reinterpret_cast<const u32x4 *>(xc + s * kSlab);
#pragma unroll
                        for (int i = 0; i < 4; ++i) xb[i] = xp[i];
                        wg[bfr].sc = QS::read(qs + c * QS::PITCH, s, q);
                        wu[bfr].sc = QS::read(qs + (kTile + c) * QS::PITCH, s, q);
                        wg[bfr].expand(ga);
                        wu[bfr].expand(ua);
#pragma unroll
                        for (int i = 0; i < 4; ++i) {
                            ag = mfma(ga[i], xb[i], ag);
                            au = mfma(ua[i], xb[i], au);
                        }
                        if (s + AHEAD < nslab) {
                            wg[bfr].codes = rg.load(s + AHEAD);
                            wu[bfr].codes = ru.load(s + AHEAD);
                        }
                    }
                    // one slab's LDS reads and expansion at a time (hoisting
                    // them all ahead would spill)
                    __builtin_amdgcn_sched_barrier(0);
                }
            }
            // lane holds rows j0 + 4q + i (i < 4) of token column c: four
            // consecutive h elements, one 8-byte store
            if (base + c < cur.count) {
                const int64_t r = list[base + c];
                uint32_t hv[4];
#pragma unroll
                for (int i = 0; i < 4; ++i) hv[i] = f32_to_bf16(silu_mul(ag[i] * glob, au[i] * glob));
                *reinterpret_cast<uint2 *>(h + r * F + j0 + 4 * q) = make_uint2(hv[0] | (hv[1] << 16),
                                                                                hv[2] | (hv[3] << 16));
            }
        }
        cur = nxt;
    }
}

// down projection as down_mfma_kernel (RT row tiles per wave, 64 RT rows
// per workgroup), the batch's activations h from LDS; the FFN width is NS
// slabs (pool.F == NS * kSlab, launcher).
template <int FMT, int RT, int NS>
__global__ __launch_bounds__(kXThreads, 3) void down_x_kernel(MOE_GROUP_LEAD_PARAMS, PoolView pool_in,
                                                              Items items_in, const uint16_t *__restrict__ h,
                                                              float *__restrict__ d) {
    extern __shared__ __align__(16) uint16_t hs[];   // [kTile][F + kXPad], then scales
    MOE_GROUP_TAKE_LEAD();
    constexpr int F = NS * kSlab, nslab = NS;
    constexpr int NB0 = kXDownAhead / RT > 0 ? kXDownAhead / RT : 1;
    constexpr int NB = NS < NB0 ? NS : NB0;
    using QS = QScales<FMT, F>;
    const int H = pool.H;
    const int wave = threadIdx.x / kWave, lane = threadIdx.x & (kWave - 1);
    const int c = lane & (kTile - 1), q = lane / kTile;
    const int i0 = (blockIdx.x * kXWaves + wave) * RT * kTile;   // may pass H: such a wave only stages
    const int gmax = min(items.n, pool.num_rows);
    const uint16_t *hc = hs + c * (F + kXPad) + 32 * q;
    // this wave's RT * 16 scale rows; lane l loads all of row l's bytes
    static_assert(RT * kTile == kWave, "one scale row per lane");
    uint8_t *qs = reinterpret_cast<uint8_t *>(hs + kTile * (F + kXPad)) + wave * RT * kTile * QS::PITCH;
    const int srow = min(i0 + (lane / kTile) * kTile, H - kTile) + c;
    GroupEntry cur;
    cur.load(items, blockIdx.y, gmax);
    for (int gi = blockIdx.y; gi < gmax && cur.valid(pool.num_rows); gi += gridDim.y) {
        GroupEntry nxt;
        nxt.load(items, gi + gridDim.y, gmax);
        const int64_t row = cur.row;
        const int32_t *list = items.grp_routes + cur.start;
        for (int base = 0; base < cur.count; base += kTile) {
            typename QS::template Chunk<QS::SB> sc2;
            sc2.load(QS::row_ptr(pool, row, 1, srow));
            ASlab<FMT> w2[NB][RT];
            QRow r2[RT];
#pragma unroll
            for (int rt = 0; rt < RT; ++rt) r2[rt].at(pool, FMT, row, 1, min(i0 + rt * kTile, H - kTile) + c, q);
#pragma unroll
            for (int bfr = 0; bfr < NB; ++bfr)
#pragma unroll
                for (int rt = 0; rt < RT; ++rt) w2[bfr][rt].codes = r2[rt].load(bfr);
            const float glob = matrix_glob<FMT>(pool, row, 1);
            const int n = min(base + (int)threadIdx.x / kTile, cur.count - 1);
            const uint16_t *src = h + (int64_t)list[n] * F;
            sc2.store(qs + lane * QS::PITCH);        // this wave's own rows: no barrier
            __syncthreads();
            stage_rows<F>(src, hs);
            __syncthreads();
            f32x4 acc[RT];
#pragma unroll
            for (int rt = 0; rt < RT; ++rt) acc[rt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int s0 = 0; s0 < nslab; s0 += NB) {
#pragma unroll
                for (int bfr = 0; bfr < NB; ++bfr) {
                    const int s = s0 + bfr;
                    if (s < nslab) {
                        u32x4 hb[4];
                        const u32x4 *hp = reinterpret_cast<const u32x4 *>(hc + s * kSlab);
#pragma unroll
                        for (int i = 0; i < 4; ++i) hb[i] = hp[i];
#pragma unroll
                        for (int rt = 0; rt < RT; ++rt) {
                            u32x4 wa[4];
                            w2[bfr][rt].sc = QS::read(qs + (rt * kTile + c) * QS::PITCH, s, q);
                            w2[bfr][rt].expand(wa);
#pragma unroll
                            for (int i = 0; i < 4; ++i) acc[rt] = mfma(wa[i], hb[i], acc[rt]);
                        }
                        if (s + NB < nslab) {
#pragma unroll
                            for (int rt = 0; rt < RT; ++rt) w2[bfr][rt].codes = r2[rt].load(s + NB);
                        }
                    }
                    __builtin_amdgcn_sched_barrier(0);
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

    // the routes' rows first (in flight while the counts are cleared)
    int row[kCountRoutesPerThread], pos[kCountRoutesPerThread];
#pragma unroll
    for (int k = 0; k < kCountRoutesPerThread; ++k) {
        const int i = tid + k * kCountThreads;
        row[k] = i < n ? idx[i] : -1;
    }
    for (int r = tid; r < num_rows; r += kCountThreads) cnt[r] = 0;
    __syncthreads();
#pragma unroll
    for (int k = 0; k < kCountRoutesPerThread; ++k) {
        const int r = row[k];
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
    hipLaunchKernelGGL((up_mfma_kernel<FMT, UT, NB>), grid, dim3(kMThreads), 0, s,
                       MOE_GROUP_LEAD_ARGS(pool, items), pool, items, x, h);
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
    hipLaunchKernelGGL((down_mfma_kernel<FMT, RT, NB>), grid, dim3(kMThreads), 0, s,
                       MOE_GROUP_LEAD_ARGS(pool, items), pool, items, h, d);
    return hipGetLastError();
}
}  // namespace

namespace {
// The LDS-staged 4-bit kernels are built for hidden widths of 4 and 8
// slabs (512, 1024) and FFN widths of 2, 4 and 8 slabs (256 .. 1024); other
// widths take the kernels above.  Their LDS: 16 activation rows of the
// width plus padding, and every wave's scale rows (at most 49 KB).
template <int FMT, int COLS> constexpr size_t up_x_lds() {
    using namespace mfma_detail;
    return x_lds_bytes(COLS, 2 * kTile, QScales<FMT, COLS>::PITCH);
}
template <int FMT, int COLS> constexpr size_t down_x_lds() {
    using namespace mfma_detail;
    return x_lds_bytes(COLS, kWave, QScales<FMT, COLS>::PITCH);
}
constexpr int kXMaxLds = 64 * 1024;
static_assert(up_x_lds<MOE_FMT_E2M1, 1024>() <= kXMaxLds && down_x_lds<MOE_FMT_E2M1, 1024>() <= kXMaxLds,
              "staged kernels' LDS");

bool x_up_fits(int fmt, int H) { return fmt != MOE_FMT_BF16 && (H == 512 || H == 1024); }
bool x_down_fits(int fmt, int F) { return fmt != MOE_FMT_BF16 && (F == 256 || F == 512 || F == 1024); }

// resident() for the LDS-staged kernels, one cache per instantiation.
template <typename KERN>
int resident_x(KERN kern, int *cache, size_t lds) {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 16) return 0;
    if (cache[dev] == 0) {
        int cus = 0, per_cu = 0;
        if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
            hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kern, mfma_detail::kXThreads, lds) !=
                hipSuccess)
            return 0;
        cache[dev] = std::max(1, cus * per_cu);
    }
    return cache[dev];
}

template <int FMT, int NS>
hipError_t launch_up_x(const PoolView &pool, const Items &items, int max_items, const uint16_t *x,
                       uint16_t *h, hipStream_t s) {
    using namespace mfma_detail;
    static int res[16];
    constexpr size_t lds = up_x_lds<FMT, NS * kSlab>();
    const int cols = pool.F / (kXWaves * kTile);
    const dim3 grid(cols, group_rows(max_items, cols, resident_x(up_x_kernel<FMT, NS>, res, lds)));
    hipLaunchKernelGGL((up_x_kernel<FMT, NS>), grid, dim3(kXThreads), lds, s, MOE_GROUP_LEAD_ARGS(pool, items),
                       pool, items, x, h);
    return hipGetLastError();
}

template <int FMT, int NS>
hipError_t launch_down_x(const PoolView &pool, const Items &items, int max_items, const uint16_t *h,
                         float *d, hipStream_t s) {
    using namespace mfma_detail;
    constexpr int RT = 4;
    static int res[16];
    constexpr size_t lds = down_x_lds<FMT, NS * kSlab>();
    const int rows = kXWaves * kTile * RT;
    const int cols = (pool.H + rows - 1) / rows;
    const dim3 grid(cols, group_rows(max_items, cols, resident_x(down_x_kernel<FMT, RT, NS>, res, lds)));
    hipLaunchKernelGGL((down_x_kernel<FMT, RT, NS>), grid, dim3(kXThreads), lds, s,
                       MOE_GROUP_LEAD_ARGS(pool, items), pool, items, h, d);
    return hipGetLastError();
}

template <int FMT>
hipError_t launch_up_x_width(const PoolView &pool, const Items &items, int max_items, const uint16_t *x,
                             uint16_t *h, hipStream_t s) {
    switch (pool.H) {
    case 512: return launch_up_x<FMT, 4>(pool, items, max_items, x, h, s);
    default: return launch_up_x<FMT, 8>(pool, items, max_items, x, h, s);
    }
}

template <int FMT>
hipError_t launch_down_x_width(const PoolView &pool, const Items &items, int max_items, const uint16_t *h,
                               float *d, hipStream_t s) {
    switch (pool.F) {
    case 256: return launch_down_x<FMT, 2>(pool, items, max_items, h, d, s);
    case 512: return launch_down_x<FMT, 4>(pool, items, max_items, h, d, s);
    default: return launch_down_x<FMT, 8>(pool, items, max_items, h, d, s);
    }
}

template <int FMT>
hipError_t x_kernels_prepare_fmt(int lds) {
    using namespace mfma_detail;
    const void *kernels[] = {
        reinterpret_cast<const void *>(&up_x_kernel<FMT, 4>),
        reinterpret_cast<const void *>(&up_x_kernel<FMT, 8>),
        reinterpret_cast<const void *>(&down_x_kernel<FMT, 4, 2>),
        reinterpret_cast<const void *>(&down_x_kernel<FMT, 4, 4>),
        reinterpret_cast<const void *>(&down_x_kernel<FMT, 4, 8>),
    };
    for (const void *k : kernels) {
        hipError_t e = hipFuncSetAttribute(k, hipFuncAttributeMaxDynamicSharedMemorySize, lds);
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
}

hipError_t x_kernels_prepare() {
    const int lds = kXMaxLds;
    hipError_t e = x_kernels_prepare_fmt<MOE_FMT_E2M1>(lds);
    return e == hipSuccess ? x_kernels_prepare_fmt<MOE_FMT_MXFP4>(lds) : e;
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
    if (x_up_fits(pool.fmt, pool.H))
        return pool.fmt == MOE_FMT_MXFP4 ? launch_up_x_width<MOE_FMT_MXFP4>(pool, items, max_items, x, h, s)
                                         : launch_up_x_width<MOE_FMT_E2M1>(pool, items, max_items, x, h, s);
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
    if (x_down_fits(pool.fmt, pool.F))
        return pool.fmt == MOE_FMT_MXFP4 ? launch_down_x_width<MOE_FMT_MXFP4>(pool, items, max_items, h, d, s)
                                         : launch_down_x_width<MOE_FMT_E2M1>(pool, items, max_items, h, d, s);
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
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void *>(&mfma_detail::group_count_kernel),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, kGroupCountMaxLds);
    return e == hipSuccess ? x_kernels_prepare() : e;
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
