// The single-token layer step in two launches on one stream (bf16, E2M1
// or MXFP4 routed experts; the shared expert is bf16).
//
// FreeToken issue #753 (section "What we changed") overlaps the miss
// gather with the shared expert by forking a side stream and joining it
// with two events.  Under hipGraph on MI355X each cross-stream edge costs
// more than the overlap buys, so the same overlap is taken inside one
// launch instead: stage 1's workgroups split into disjoint roles that
// touch disjoint memory --
//   [0, G)            the miss gather: pinned host rows -> their slots; while
//                     a fetched expert's gate/up rows stream through, the
//                     same workgroup also takes their dot products with x
//                     (the link, not the ALUs, bounds it);
//   [G, G + Ts)       the shared expert's gate/up + SwiGLU and its gate;
//   [G + Ts, ...)     gate/up + SwiGLU of the routes whose experts were
//                     already resident.
// Stage 2 (after stage 1, stream order) computes every down projection --
// routed experts, fetched ones from their gate/up dots -- and the combine
// in ascending k, then + the gated shared term, exactly as the serial path.
//
// Without a miss plan and a shared expert the same two launches are the
// single-token routed GEMV over slot ids (resident routes' gate/up, then
// down + combine + an optional fp32 addend).
//
// Bit-exactness with the serial path: resident routes and the shared expert
// run the same device code; a fetched expert's gate/up dot products are
// built from the same 16-byte chunk partials combined by the same trees
// (tree_sum over a lane's chunks, then the lane tree), so every float
// matches.  A 4-bit chunk's partial needs its scales: the gather unit that
// carries a run of gate/up codes also carries (and copies) the run of the
// scale bank that belongs to them, so nothing is read over the link twice.
#include "k_expert.inc"

namespace moe {
namespace stage_detail {

using namespace expert_detail;

struct Stage1Params {
    GatherParams g;            // the step's miss plan and banks
    int gather_blocks;
    float *gu;                 // [plan entries][2F] fetched experts' gate/up dots (no global scale)
    PoolView slots;            // routed pool
    const int32_t *idx;        // [K] slot ids
    const int32_t *route_plan; // [K] plan entry of a fetched route, or -1
    int K;
    int a_tiles;               // gate/up tiles per route
    const uint16_t *x;         // [H]
    uint16_t *h;               // [K][F]
    PoolView shared;           // one bf16 row; shared F == routed F
    int s_tiles;               // 0: no shared expert
    uint16_t *hs;              // [F]
    const uint16_t *gate_vec;  // [H]
    float *gamma;              // [1]
};

struct Stage2Params {
    PoolView slots;
    const int32_t *idx;
    const float *w;
    const int32_t *route_plan;
    int K;
    const uint16_t *h;
    const float *gu;
    PoolView shared;
    int has_shared;
    const uint16_t *hs;
    const float *gamma;
    const float *addend;       // [H] fp32 added to the routed sum, or NULL
    uint16_t *out;
};

constexpr int kGatherUnit = kThreads * 16 * 4;  // 16 KiB, as the gather kernel
constexpr int kMaxStageRoutes = 64;             // top-k of a single-token step (kMaxTopK)
constexpr int kUnitChunks = kGatherUnit / 16;   // 1024 chunks of 16 bytes

// gate/up rows jj and F + jj of one expert with x -> h[j] (bf16), the
// arithmetic of up_kernel for one route
template <int FMT, int LPR, int NCH>
__device__ __forceinline__ void up_rows(const PoolView &pool, int64_t prow, int j, int li,
                                        const uint16_t *x, uint16_t *h) {
    const int F = pool.F;
    const bool jok = j < F;
    const int jj = jok ? j : F - 1;
    WSeg<FMT, NCH> wg, wu;
    wg.load(pool, prow, 0, jj, li, LPR);
    wu.load(pool, prow, 0, F + jj, li, LPR);
    XSeg<FMT, NCH> xs;
    xs.load(x, li, LPR);
    __builtin_amdgcn_sched_barrier(0);  // all of the row pair's loads issue before any math
    const float glob = wg.glob(pool, prow, 0);
    const float g = group_total<LPR>(seg_dot(wg, xs)) * glob;
    const float u = group_total<LPR>(seg_dot(wu, xs)) * glob;
    if (jok && li == LPR - 1) h[j] = f32_to_bf16(silu_mul(g, u));
}

// The partial dot of one 16-byte gate/up chunk with x, as seg_dot takes it.
template <int FMT>
__device__ __forceinline__ float chunk_part(u32x4 codes, uint32_t sc, const uint16_t *x, int c);

template <>
__device__ __forceinline__ float chunk_part<MOE_FMT_BF16>(u32x4 w, uint32_t, const uint16_t *x, int c) {
    return chunk_dot_bf16(w, *reinterpret_cast<const u32x4 *>(x + 8 * c));
}
template <>
__device__ __forceinline__ float chunk_part<MOE_FMT_E2M1>(u32x4 w, uint32_t sc, const uint16_t *x, int c) {
    const u32x4 *xv = reinterpret_cast<const u32x4 *>(x + 32 * c);
    const u32x4 xs[4] = {xv[0], xv[1], xv[2], xv[3]};
    return chunk_dot_e2m1(w, sc, xs);
}
template <>
__device__ __forceinline__ float chunk_part<MOE_FMT_MXFP4>(u32x4 w, uint32_t sc, const uint16_t *x, int c) {
    const u32x4 *xv = reinterpret_cast<const u32x4 *>(x + 32 * c);
    const u32x4 xs[4] = {xv[0], xv[1], xv[2], xv[3]};
    return chunk_dot_mxfp4(w, sc, xs);
}

// A pool view whose widths and row sizes are the compile-time (H, F) of a
// stage kernel, so that row addresses need no kernel-argument loads.
template <int FMT, int H, int F>
__device__ __forceinline__ PoolView fixed_view(const PoolView &v, int num_rows) {
    PoolView r = v;
    r.H = H;
    r.F = F;
    r.num_rows = num_rows;
#pragma unroll
    for (int b = 0; b < MOE_MAX_BANKS; ++b) r.rb[b] = bank_row_bytes(FMT, b, H, F);
    return r;
}

// Stage 1.  FMT, LPRH x NCHH: the routed gate/up rows (16-byte chunks per
// row); SLPRH x SNCHH: the shared expert's bf16 gate/up rows.
//
// The arguments the routed workgroups need before their first weight
// request come first, as scalars: gfx950 preloads the leading kernel
// arguments into scalar registers at wave launch (the library builds with
// kernel-argument preloading), so those waves wait on one load (the slot
// id) before streaming.  Measured on MI355X for the single-token routed
// GEMV (8 bf16 experts, H 2048, F 512): 12.56 -> 12.18 us per call with both
// stage kernels so arranged.
template <int FMT, int SH, int SF, int LPRH, int NCHH, int SLPRH, int SNCHH>
__global__ __launch_bounds__(kThreads) void stage1_kernel(int gather_blocks, int s_tiles, const int32_t *idx,
                                                          const int32_t *route_plan, const uint8_t *codes,
                                                          const uint8_t *scales, const uint16_t *x,
                                                          int num_rows, Stage1Params p) {
    __shared__ float part[kUnitChunks];
    __shared__ __align__(16) uint8_t scl[kUnitChunks * 2];   // a 4-bit unit's scales
    const int tid = threadIdx.x;
    const int wave = tid / kWave, lane = tid & (kWave - 1);
    constexpr int H = SH, F = SF;
    constexpr int C = LPRH * NCHH;  // 16-byte chunks per gate/up row

    if ((int)blockIdx.x < gather_blocks) {
        const GatherParams &g = p.g;
        const int n = *g.n_miss;
        const int64_t total = (int64_t)n * g.units_per_entry;
        for (int64_t u = blockIdx.x; u < total; u += gather_blocks) {
            const int entry = (int)(u / g.units_per_entry);
            const int uu = (int)(u - (int64_t)entry * g.units_per_entry);
            int b = 0;
            while (b + 1 < g.nb && uu >= g.unit_start[b + 1]) ++b;
            const int64_t rb = g.rb[b];
            const int64_t off = (int64_t)(uu - g.unit_start[b]) * kGatherUnit;
            const int expert = g.plan_expert[entry], slot = g.plan_slot[entry];
            const uint8_t *src = g.host[b] + (int64_t)expert * rb + off;
            uint8_t *dst = g.slot[b] + (int64_t)slot * rb + off;
            const int64_t len = min((int64_t)kGatherUnit, rb - off);
            if (rb & 15) {
                // a bank of sub-16-byte rows (the fp32 global scale): 4 B per lane
                for (int64_t o = (int64_t)tid * 4; o < len; o += kThreads * 4)
                    *reinterpret_cast<uint32_t *>(dst + o) =
                        __builtin_nontemporal_load(reinterpret_cast<const uint32_t *>(src + o));
                continue;
            }
            const u32x4 *s4 = reinterpret_cast<const u32x4 *>(src);
            u32x4 *d4 = reinterpret_cast<u32x4 *>(dst);
            u32x4 v[4];
#pragma unroll
            for (int k = 0; k < 4; ++k)
                if ((int64_t)(tid + k * kThreads) * 16 < len)
                    v[k] = __builtin_nontemporal_load(s4 + tid + k * kThreads);
            // a 4-bit unit of gate/up codes carries their scales: one E4M3
            // pair (2 B) or E8M0 (1 B) per chunk, a contiguous run of the
            // scale bank at the unit's chunk index
            const int64_t chunk0 = off / 16;
            const int carry = (b == 0) ? g.carry_scales : 0;
            const int64_t sbytes = carry * (len / 16);
            u32x4 sv{};
            const bool sload = carry && (int64_t)tid * 16 < sbytes;
            if (sload)
                sv = __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(
                    g.host[1] + (int64_t)expert * g.rb[1] + carry * chunk0 + (int64_t)tid * 16));
#pragma unroll
            for (int k = 0; k < 4; ++k)
                if ((int64_t)(tid + k * kThreads) * 16 < len) d4[tid + k * kThreads] = v[k];
            if (b != 0) continue;
            if (carry) {
                if (sload) {
                    *reinterpret_cast<u32x4 *>(g.slot[1] + (int64_t)slot * g.rb[1] + carry * chunk0 +
                                               (int64_t)tid * 16) = sv;
                    *reinterpret_cast<u32x4 *>(scl + tid * 16) = sv;
                }
                __syncthreads();
            }
            // Gate/up rows of a fetched expert: chunk partials with x ...
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                const int f = tid + k * kThreads;
                float pv = 0.f;
                if ((int64_t)f * 16 < len) {
                    const int c = (int)((chunk0 + f) % C);
                    uint32_t sc = 0;
                    if constexpr (FMT == MOE_FMT_E2M1) sc = *reinterpret_cast<const uint16_t *>(scl + 2 * f);
                    if constexpr (FMT == MOE_FMT_MXFP4) sc = scl[f];
                    pv = chunk_part<FMT>(v[k], sc, x, c);
                }
                part[f] = pv;
            }
            __syncthreads();
            // ... combined per row by the up kernels' trees.
            const int rows = (int)(len / 16) / C;
            const int row0 = (int)(chunk0 / C);
            constexpr int RPW = kWave / LPRH;
            const int sub = lane / LPRH, li = lane % LPRH;
            for (int r0 = 0; r0 < rows; r0 += kWavesPerBlock * RPW) {
                const int r = r0 + wave * RPW + sub;
                float q[NCHH];
#pragma unroll
                for (int i = 0; i < NCHH; ++i) q[i] = r < rows ? part[r * C + li + LPRH * i] : 0.f;
                const float sum = group_total<LPRH>(tree_sum<NCHH>(q));
                if (r < rows && li == LPRH - 1) p.gu[(int64_t)entry * 2 * F + row0 + r] = sum;
            }
            __syncthreads();
        }
        return;
    }

    int b = blockIdx.x - gather_blocks;
    if (b < s_tiles) {
        constexpr int SJT = kWavesPerBlock * (kWave / SLPRH);
        const int sub = lane / SLPRH, li = lane % SLPRH;
        up_rows<MOE_FMT_BF16, SLPRH, SNCHH>(fixed_view<MOE_FMT_BF16, SH, SF>(p.shared, 1), 0,
                                            b * SJT + wave * (kWave / SLPRH) + sub, li, x, p.hs);
        if (b == 0 && wave == 0) {
            float z = 0.f;
            for (int c = lane; c < H / 8; c += kWave) {
                const u32x4 a = *reinterpret_cast<const u32x4 *>(x + 8 * c);
                const u32x4 gv = *reinterpret_cast<const u32x4 *>(p.gate_vec + 8 * c);
                z = dot8_bf16(gv, a, z);
            }
            z = group_total<kWave>(z);
            if (lane == kWave - 1) p.gamma[0] = 1.f / (1.f + __expf(-z));
        }
        return;
    }
    b -= s_tiles;
    constexpr int JT = kWavesPerBlock * (kWave / LPRH);
    constexpr int a_tiles = (F + JT - 1) / JT;
    const int sub = lane / LPRH, li = lane % LPRH;
    const int k = b / a_tiles;
    const int tile = b - k * a_tiles;
    // both scalar loads in one batch: the plan entry is read (from the slot
    // ids when there is no plan) without a branch
    const int s = idx[k];
    const int plan_v = (route_plan ? route_plan : idx)[k];
    const int plan = route_plan ? plan_v : -1;
    PoolView sv = fixed_view<FMT, SH, SF>(p.slots, num_rows);
    sv.bank[0] = codes;
    if constexpr (FMT != MOE_FMT_BF16) sv.bank[1] = scales;
    if ((s < 0) | (s >= num_rows) | (plan >= 0)) return;
    up_rows<FMT, LPRH, NCHH>(sv, s, tile * JT + wave * (kWave / LPRH) + sub, li, x, p.h + (int64_t)k * F);
}

// h chunks of a fetched route, from its gate/up dots and the w13 global
// scale (as up_rows scales them).
template <int FMT, int NCH>
__device__ __forceinline__ void h_from_gu(const float *gu, int F, int li, int lpr, float glob,
                                          XSeg<FMT, NCH> &hs) {
    constexpr int V = XSeg<FMT, NCH>::kVecs;
#pragma unroll
    for (int c = 0; c < NCH; ++c) {
#pragma unroll
        for (int vv = 0; vv < V; ++vv) {
            const int j0 = (li + c * lpr) * Epc<FMT>::v + 8 * vv;
            const u32x4 *g4 = reinterpret_cast<const u32x4 *>(gu + j0);
            const u32x4 *u4 = reinterpret_cast<const u32x4 *>(gu + F + j0);
            const u32x4 ga = g4[0], gb = g4[1], ua = u4[0], ub = u4[1];
            float gv[8], uv[8];
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                gv[q] = __uint_as_float(ga[q]) * glob;
                gv[4 + q] = __uint_as_float(gb[q]) * glob;
                uv[q] = __uint_as_float(ua[q]) * glob;
                uv[4 + q] = __uint_as_float(ub[q]) * glob;
            }
            u32x4 o;
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const uint32_t lo = f32_to_bf16(silu_mul(gv[2 * q], uv[2 * q]));
                const uint32_t hi = f32_to_bf16(silu_mul(gv[2 * q + 1], uv[2 * q + 1]));
                o[q] = lo | (hi << 16);
            }
            hs.x[c][vv] = o;
        }
    }
}

// Stage 2 of bf16 rows gives each wave its own row group and all of the
// step's routes (kDownBatch at a time, accumulated in registers).  4-bit
// rows are a quarter of the bytes and their wave's dequantisation needs
// more registers, so there the four waves of a workgroup share one row
// group and split the routes, two at a time, with the per-route values
// meeting in LDS (measured on MI355X at the 40 x 256 decode: the 4-bit
// decode 19.8K -> 21.2K layer-steps/s; the same split made the bf16
// single-token GEMV 5% slower).
template <int FMT> struct Stage2Split {
    static constexpr int ways = FMT == MOE_FMT_BF16 ? 1 : kWavesPerBlock;   // waves per row group
    static constexpr int batch = FMT == MOE_FMT_BF16 ? kDownBatch : 2;      // routes in flight per wave
};

// One batch of up to B of a wave's routes [k0, khi) of stage 2.  load()
// issues the routes' slot ids and plan entries (scalar loads, together),
// then every W2 row and activation chunk; routes that contribute nothing
// read row 0 and the last route as in-range stand-ins, so every load is
// unconditional and none waits for another.  reduce() then accumulates each
// route's down value of the lane group's row (acc = fma(w, v, acc),
// ascending k), or with TO_LDS stores it to vals[k][sub] and whether it
// counts to ok[k].
template <int FMT, int F, int LPRF, int NCHF, int B>
struct Stage2Batch {
    int k0, khi;
    int rows[B], pe[B];
    WSeg<FMT, NCHF> w2[B];
    XSeg<FMT, NCHF> hs[B];
    float g13[B], g2[B];   // global scales (1 unless E2M1)

    __device__ __forceinline__ void load(const Stage2Params &p, int k0_, int khi_, int ii, int li) {
        k0 = k0_;
        khi = khi_;
        int sl[B];
#pragma unroll
        for (int q = 0; q < B; ++q) {
            const int kk = min(k0 + q, khi - 1);
            sl[q] = p.idx[kk];
            pe[q] = p.route_plan ? p.route_plan[kk] : -1;
        }
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int q = 0; q < B; ++q) {
            const int k = k0 + q;
            const bool use = k < khi && sl[q] >= 0 && sl[q] < p.slots.num_rows;
            rows[q] = use ? sl[q] : -1;
            const int r = use ? sl[q] : 0;
            w2[q].load(p.slots, r, 1, ii, li, LPRF);
            hs[q].load(p.h + (int64_t)min(k, khi - 1) * F, li, LPRF);
            g13[q] = w2[q].glob(p.slots, r, 0);
            g2[q] = w2[q].glob(p.slots, r, 1);
        }
        __builtin_amdgcn_sched_barrier(0);
    }

    template <bool TO_LDS>
    __device__ __forceinline__ void reduce(const Stage2Params &p, int li, int sub, float &acc,
                                           float (*vals)[kWave / LPRF], int *ok) {
        const int lane = threadIdx.x & (kWave - 1);
#pragma unroll
        for (int q = 0; q < B; ++q) {
            const int k = k0 + q;
            if (k >= khi) continue;
            if constexpr (TO_LDS) {
                if (lane == 0) ok[k] = rows[q] >= 0;
            }
            if (rows[q] < 0) continue;
            if (pe[q] >= 0) h_from_gu<FMT, NCHF>(p.gu + (int64_t)pe[q] * 2 * F, F, li, LPRF, g13[q], hs[q]);
            const float v = group_total<LPRF>(seg_dot(w2[q], hs[q])) * g2[q];
            if constexpr (TO_LDS) {
                if (li == LPRF - 1) vals[k][sub] = v;
            } else {
                acc = fmaf(p.w[k], v, acc);
            }
        }
    }
};

// Stage 2.  The routed W2 rows take LPRF x NCHF chunks, the shared
// expert's bf16 rows SLPRF x SNCHF (SLPRF >= LPRF: a bf16 row has four
// times the chunks of a 4-bit one).  A row group is RPW = 64 / LPRF output
// rows (one lane group per row) and WAYS waves (Stage2Split): wave way w
// takes routes [w KW, (w + 1) KW), KW = ceil(K / WAYS), and the shared
// expert's passes of 64 / SLPRF rows numbered WAYS - 1 - w, 2 WAYS - 1 -
// w, ...  With one way the wave sums its routes itself; with several they
// meet in LDS and the row group's first wave sums them in ascending k with
// the same fma chain.  Either way the gated shared term is added last.
// As in stage 1, the arguments on the way to the first weight request
// lead, as scalars (the W2 codes and, for 4-bit rows, their scales), and
// the first batch of routes is requested before the shared expert's rows.
template <int FMT, int SH, int SF, int LPRF, int NCHF, int SLPRF, int SNCHF>
__global__ __launch_bounds__(kThreads) void stage2_kernel(const int32_t *idx, const int32_t *route_plan,
                                                          const uint8_t *codes, const uint8_t *scales,
                                                          const uint16_t *h, uint16_t *out, int K,
                                                          int num_rows, Stage2Params p_in) {
    constexpr int RPW = kWave / LPRF;
    constexpr int SRPW = kWave / SLPRF;
    constexpr int PASSES = SLPRF / LPRF;
    constexpr int WAYS = Stage2Split<FMT>::ways, BATCH = Stage2Split<FMT>::batch;
    constexpr int GROUPS = kWavesPerBlock / WAYS;       // row groups per workgroup
    constexpr bool SPLIT = WAYS > 1;
    constexpr int H = SH;
    // W2's banks: bf16 rows in 1; E2M1 codes, scales, global scale in 3-5;
    // MXFP4 codes and scales in 2-3
    constexpr int WB = FMT == MOE_FMT_BF16 ? 1 : FMT == MOE_FMT_E2M1 ? 3 : 2;
    static_assert(SLPRF >= LPRF && PASSES * SRPW == RPW, "shared and routed row mapping");
    __shared__ float vals[SPLIT ? GROUPS * kMaxStageRoutes : 1][RPW];
    __shared__ int ok[SPLIT ? GROUPS * kMaxStageRoutes : 1];
    __shared__ float svals[SPLIT ? GROUPS : 1][RPW];
    Stage2Params p = p_in;
    p.slots = fixed_view<FMT, SH, SF>(p_in.slots, num_rows);
    p.slots.bank[WB] = codes;
    if constexpr (FMT != MOE_FMT_BF16) p.slots.bank[WB + 1] = scales;
    p.shared = fixed_view<MOE_FMT_BF16, SH, SF>(p_in.shared, 1);
    p.idx = idx;
    p.route_plan = route_plan;
    p.h = h;
    p.K = K;
    const int wave = threadIdx.x / kWave, lane = threadIdx.x & (kWave - 1);
    const int grp = wave / WAYS, way = wave % WAYS;
    const int sub = lane / LPRF, li = lane % LPRF;
    const int row0 = (blockIdx.x * GROUPS + grp) * RPW;
    const int i = row0 + sub;
    const bool iok = i < H;
    const int ii = iok ? i : H - 1;
    const int kw = (K + WAYS - 1) / WAYS;
    const int klo = way * kw, khi = min(K, klo + kw);
    float(*gvals)[RPW] = vals + (SPLIT ? grp * kMaxStageRoutes : 0);
    int *gok = ok + (SPLIT ? grp * kMaxStageRoutes : 0);

    Stage2Batch<FMT, SF, LPRF, NCHF, BATCH> bt;
    if (klo < khi) bt.load(p, klo, khi, ii, li);
    // this wave's passes of the shared expert's rows, in flight with its
    // first batch of routes
    constexpr int MYP = (PASSES + WAYS - 1) / WAYS;
    WSeg<MOE_FMT_BF16, SNCHF> w2s[MYP];
    XSeg<MOE_FMT_BF16, SNCHF> hss;
    const int ssub = lane / SLPRF, sli = lane % SLPRF;
    const int p0 = WAYS - 1 - way;   // first pass of this wave
    if (p.has_shared) {
#pragma unroll
        for (int m = 0; m < MYP; ++m) {
            const int pp = p0 + m * WAYS;
            if (pp < PASSES) w2s[m].load(p.shared, 0, 1, min(row0 + pp * SRPW + ssub, H - 1), sli, SLPRF);
        }
        if (p0 < PASSES) hss.load(p.hs, sli, SLPRF);
    }
    float acc = 0.f;
    for (int k0 = klo; k0 < khi; k0 += BATCH) {
        if (k0 != klo) bt.load(p, k0, khi, ii, li);
        bt.template reduce<SPLIT>(p, li, sub, acc, gvals, gok);
    }
    float vs = 0.f;
    if (p.has_shared) {
#pragma unroll
        for (int m = 0; m < MYP; ++m) {
            const int pp = p0 + m * WAYS;
            if (pp < PASSES) {
                const float v = group_total<SLPRF>(seg_dot(w2s[m], hss));
                if constexpr (SPLIT) {
                    if (sli == SLPRF - 1) svals[grp][pp * SRPW + ssub] = v;
                } else if constexpr (PASSES == 1) {
                    vs = v;          // the same lane group holds the row
                } else {
                    // row sub lives in pass sub / SRPW, lane group sub % SRPW
                    const float moved = __shfl(v, (sub % SRPW) * SLPRF + SLPRF - 1, kWave);
                    if (sub / SRPW == pp) vs = moved;
                }
            }
        }
    }
    if constexpr (SPLIT) {
        __syncthreads();
        if (way != 0) return;
        for (int k = 0; k < K; ++k)
            if (gok[k]) acc = fmaf(p.w[k], gvals[k][sub], acc);
        if (p.has_shared) vs = svals[grp][sub];
    }
    float res = acc;
    if (p.addend) res = acc + p.addend[ii];
    // gamma * vs is rounded on its own (the library builds without fp
    // contraction), as the serial path rounds it when storing it
    if (p.has_shared) res = acc + p.gamma[0] * vs;
    if (iok && li == LPRF - 1) out[i] = f32_to_bf16(res);
}

// Whether a view's row sizes are those its format has at (H, F), which the
// stage kernels take as compile-time constants.
bool rows_as_fixed(const PoolView &v, int fmt) {
    for (int b = 0; b < bank_count(fmt); ++b)
        if (v.rb[b] != bank_row_bytes(fmt, b, v.H, v.F)) return false;
    return true;
}

template <int FMT, int SH, int SF, int LPRH, int NCHH, int SLPRH, int SNCHH, int LPRF, int NCHF, int SLPRF,
          int SNCHF>
hipError_t launch_shape(const Stage1Params &a, const Stage2Params &b, int which, hipStream_t s) {
    constexpr int JT = kWavesPerBlock * (kWave / LPRH);
    constexpr int SJT = kWavesPerBlock * (kWave / SLPRH);
    constexpr int IT = kWavesPerBlock / Stage2Split<FMT>::ways * (kWave / LPRF);   // stage 2 rows per workgroup
    constexpr int WB = FMT == MOE_FMT_BF16 ? 1 : FMT == MOE_FMT_E2M1 ? 3 : 2;     // W2's first bank
    if (!rows_as_fixed(a.slots, FMT) || (a.s_tiles && !rows_as_fixed(a.shared, MOE_FMT_BF16)))
        return hipErrorInvalidValue;
    Stage1Params p1 = a;
    p1.a_tiles = (SF + JT - 1) / JT;
    p1.s_tiles = p1.s_tiles ? (SF + SJT - 1) / SJT : 0;
    const int blocks1 = p1.gather_blocks + p1.s_tiles + p1.K * p1.a_tiles;
    if (which & 1) {
        hipLaunchKernelGGL((stage1_kernel<FMT, SH, SF, LPRH, NCHH, SLPRH, SNCHH>), dim3(blocks1), dim3(kThreads),
                           0, s, p1.gather_blocks, p1.s_tiles, p1.idx, p1.route_plan, p1.slots.bank[0],
                           p1.slots.bank[1], p1.x, p1.slots.num_rows, p1);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    if (which & 2) {
        hipLaunchKernelGGL((stage2_kernel<FMT, SH, SF, LPRF, NCHF, SLPRF, SNCHF>), dim3((SH + IT - 1) / IT),
                           dim3(kThreads), 0, s, b.idx, b.route_plan, b.slots.bank[WB],
                           b.slots.bank[FMT == MOE_FMT_BF16 ? WB : WB + 1], b.h, b.out, b.K, b.slots.num_rows, b);
        return hipGetLastError();
    }
    return hipSuccess;
}

}  // namespace stage_detail

// (H, F) with instantiated stage kernels, and the lanes per row (LPR) and
// chunks per lane (NCH) of each row kind: LPR = min(chunks, 64), as the
// serial kernels choose them (MOE_ROW_SWITCH), so that every dot product
// reduces through the same trees.  Columns: H, F, then for bf16 rows
// (16-byte chunks of 8 elements) gate/up (LPR, NCH) and down (LPR, NCH),
// then for 4-bit rows (chunks of 32 elements) the same.
#define MOE_STAGE_SHAPES(X)                           \
    X(64, 128, 8, 1, 16, 1, 2, 1, 4, 1)               \
    X(1024, 256, 64, 2, 32, 1, 32, 1, 8, 1)           \
    X(1024, 512, 64, 2, 64, 1, 32, 1, 16, 1)          \
    X(2048, 256, 64, 4, 32, 1, 64, 1, 8, 1)           \
    X(2048, 512, 64, 4, 64, 1, 64, 1, 16, 1)          \
    X(2048, 1024, 64, 4, 64, 2, 64, 1, 32, 1)         \
    X(4096, 512, 64, 8, 64, 1, 64, 2, 16, 1)          \
    X(4096, 1024, 64, 8, 64, 2, 64, 2, 32, 1)

bool stage_supported(int fmt, int H, int F) {
    if (fmt != MOE_FMT_BF16 && fmt != MOE_FMT_E2M1 && fmt != MOE_FMT_MXFP4) return false;
#define MOE_STAGE_HAS(SH, SF, A, B, C, D, E_, F_, G, H_) \
    if (H == SH && F == SF) return true;
    MOE_STAGE_SHAPES(MOE_STAGE_HAS)
#undef MOE_STAGE_HAS
    return false;
}

hipError_t launch_stages(const GatherParams &g, int gather_blocks, float *gu, const PoolView &slots,
                         const int32_t *idx, const float *w, const int32_t *route_plan, int K,
                         const uint16_t *x, uint16_t *h, const PoolView *shared, uint16_t *hs,
                         const uint16_t *gate_vec, float *gamma, const float *addend, uint16_t *out,
                         int which, hipStream_t s) {
    using namespace stage_detail;
    if (K > kMaxStageRoutes) return hipErrorInvalidValue;
    Stage1Params a{};
    a.g = g;
    a.gather_blocks = gather_blocks;
    a.gu = gu;
    a.slots = slots;
    a.idx = idx;
    a.route_plan = route_plan;
    a.K = K;
    a.x = x;
    a.h = h;
    if (shared) {
        a.shared = *shared;
        a.s_tiles = 1;  // sized in launch_shape
        a.hs = hs;
        a.gate_vec = gate_vec;
        a.gamma = gamma;
    }
    Stage2Params b{};
    b.slots = slots;
    b.idx = idx;
    b.w = w;
    b.route_plan = route_plan;
    b.K = K;
    b.h = h;
    b.gu = gu;
    if (shared) {
        b.shared = *shared;
        b.has_shared = 1;
        b.hs = hs;
        b.gamma = gamma;
    } else {
        // stage 2 loads the shared view unconditionally: point it at row 0
        // of the routed pool and at the routed activations (never used)
        b.shared = slots;
        b.hs = h;
    }
    b.addend = addend;
    b.out = out;
    if (rec::on()) {
        const bool gather = gather_blocks > 0;
        hipError_t e = hipSuccess;
        if (which & 1)
            // gather role: plan rows over the host link into fresh slots, the
            // fetched rows' gate/up dots into gu; resident routes' gate/up
            // from their slots (every route's when nothing is fetched); the
            // shared expert's gate/up and gate
            e = rec::launch("stage1_kernel", s,
                            {{x, rec::kRead}, {idx, rec::kRead}, {route_plan, rec::kRead},
                             {slots.bank[0], rec::kRead, route_plan ? rec::kResidentSlots : rec::kAllSlots},
                             {gather ? g.n_miss : nullptr, rec::kRead}, {gather ? g.host[0] : nullptr, rec::kRead},
                             {gather ? g.slot[0] : nullptr, rec::kWrite, rec::kFreshSlots},
                             {gather ? gu : nullptr, rec::kWrite}, {h, rec::kWrite},
                             {shared ? shared->bank[0] : nullptr, rec::kRead}, {gate_vec, rec::kRead},
                             {shared ? hs : nullptr, rec::kWrite}, {shared ? gamma : nullptr, rec::kWrite}});
        if (e == hipSuccess && (which & 2))
            // every route's down rows from its slot, the fetched routes'
            // activations from gu, the shared expert's down rows
            e = rec::launch("stage2_kernel", s,
                            {{h, rec::kRead}, {route_plan ? gu : nullptr, rec::kRead}, {idx, rec::kRead},
                             {w, rec::kRead}, {route_plan, rec::kRead}, {slots.bank[0], rec::kRead, rec::kAllSlots},
                             {shared ? shared->bank[0] : nullptr, rec::kRead}, {shared ? hs : nullptr, rec::kRead},
                             {shared ? gamma : nullptr, rec::kRead}, {addend, rec::kRead}, {out, rec::kWrite}});
        return e;
    }
    const int H = slots.H, F = slots.F;
#define MOE_STAGE_CALL(SH, SF, BLH, BNH, BLF, BNF, QLH, QNH, QLF, QNF)                                   \
    if (H == SH && F == SF) {                                                                        \
        if (slots.fmt == MOE_FMT_BF16)                                                               \
            return launch_shape<MOE_FMT_BF16, SH, SF, BLH, BNH, BLH, BNH, BLF, BNF, BLF, BNF>(a, b, which, s); \
        if (slots.fmt == MOE_FMT_E2M1)                                                               \
            return launch_shape<MOE_FMT_E2M1, SH, SF, QLH, QNH, BLH, BNH, QLF, QNF, BLF, BNF>(a, b, which, s); \
        if (slots.fmt == MOE_FMT_MXFP4)                                                              \
            return launch_shape<MOE_FMT_MXFP4, SH, SF, QLH, QNH, BLH, BNH, QLF, QNF, BLF, BNF>(a, b, which, s); \
    }
    MOE_STAGE_SHAPES(MOE_STAGE_CALL)
#undef MOE_STAGE_CALL
    return hipErrorNotSupported;
}

}  // namespace moe
