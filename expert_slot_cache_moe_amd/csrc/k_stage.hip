// The single-token layer step in two launches on one stream (bf16 experts).
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
// built from the same 8-element chunk partials combined by the same trees
// (tree_sum over a lane's chunks, then the xor tree over lanes), so every
// float matches.
#include "k_expert.inc"

namespace moe {
namespace stage_detail {

using namespace expert_detail;

struct Stage1Params {
    GatherParams g;            // the step's miss plan and banks
    int gather_blocks;
    float *gu;                 // [plan entries][2F] fetched experts' gate/up dots
    PoolView slots;            // routed pool (bf16)
    const int32_t *idx;        // [K] slot ids
    const int32_t *route_plan; // [K] plan entry of a fetched route, or -1
    int K;
    int a_tiles;               // gate/up tiles per route
    const uint16_t *x;         // [H]
    uint16_t *h;               // [K][F]
    PoolView shared;           // one row; shared F == routed F
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
constexpr int kUnitChunks = kGatherUnit / 16;   // 1024 chunks of 8 bf16

// gate/up rows jj and F + jj of one expert with x -> h[j] (bf16)
template <int LPR, int NCH>
__device__ __forceinline__ void up_rows(const PoolView &pool, int64_t prow, int j, int li,
                                        const uint16_t *x, uint16_t *h) {
    const int F = pool.F;
    const bool jok = j < F;
    const int jj = jok ? j : F - 1;
    WSeg<MOE_FMT_BF16, NCH> wg, wu;
    wg.load(pool, prow, 0, jj, li, LPR);
    wu.load(pool, prow, 0, F + jj, li, LPR);
    XSeg<MOE_FMT_BF16, NCH> xs;
    xs.load(x, li, LPR);
    __builtin_amdgcn_sched_barrier(0);  // all of the row pair's loads issue before any math
    const float g = group_total<LPR>(seg_dot(wg, xs)) * wg.glob(pool, prow, 0);
    const float u = group_total<LPR>(seg_dot(wu, xs)) * wg.glob(pool, prow, 0);
    if (jok && li == LPR - 1) h[j] = f32_to_bf16(silu_mul(g, u));
}

template <int LPRH, int NCHH>
__global__ __launch_bounds__(kThreads) void stage1_kernel(Stage1Params p) {
    __shared__ float part[kUnitChunks];
    const int tid = threadIdx.x;
    const int wave = tid / kWave, lane = tid & (kWave - 1);
    const int H = p.slots.H, F = p.slots.F;
    constexpr int C = LPRH * NCHH;  // 16-byte chunks per gate/up row

    if ((int)blockIdx.x < p.gather_blocks) {
        const GatherParams &g = p.g;
        const int n = *g.n_miss;
        const int64_t total = (int64_t)n * g.units_per_entry;
        for (int64_t u = blockIdx.x; u < total; u += p.gather_blocks) {
            const int entry = (int)(u / g.units_per_entry);
            const int uu = (int)(u - (int64_t)entry * g.units_per_entry);
            int b = 0;
            while (b + 1 < g.nb && uu >= g.unit_start[b + 1]) ++b;
            const int64_t rb = g.rb[b];
            const int64_t off = (int64_t)(uu - g.unit_start[b]) * kGatherUnit;
            const uint8_t *src = g.host[b] + (int64_t)g.plan_expert[entry] * rb + off;
            uint8_t *dst = g.slot[b] + (int64_t)g.plan_slot[entry] * rb + off;
            const int64_t len = min((int64_t)kGatherUnit, rb - off);
            const u32x4 *s4 = reinterpret_cast<const u32x4 *>(src);
            u32x4 *d4 = reinterpret_cast<u32x4 *>(dst);
            u32x4 v[4];
#pragma unroll
            for (int k = 0; k < 4; ++k)
                if ((int64_t)(tid + k * kThreads) * 16 < len)
                    v[k] = __builtin_nontemporal_load(s4 + tid + k * kThreads);
#pragma unroll
            for (int k = 0; k < 4; ++k)
                if ((int64_t)(tid + k * kThreads) * 16 < len) d4[tid + k * kThreads] = v[k];
            if (b != 0) continue;
            // Gate/up rows of a fetched expert: chunk partials with x ...
            const int64_t chunk0 = off / 16;
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                const int f = tid + k * kThreads;
                float pv = 0.f;
                if ((int64_t)f * 16 < len) {
                    const int c = (int)((chunk0 + f) % C);
                    pv = chunk_dot_bf16(v[k], *reinterpret_cast<const u32x4 *>(p.x + 8 * c));
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
                const float s = group_total<LPRH>(tree_sum<NCHH>(q));
                if (r < rows && li == LPRH - 1) p.gu[(int64_t)entry * 2 * F + row0 + r] = s;
            }
            __syncthreads();
        }
        return;
    }

    constexpr int JT = kWavesPerBlock * (kWave / LPRH);
    const int sub = lane / LPRH, li = lane % LPRH;
    int b = blockIdx.x - p.gather_blocks;
    if (b < p.s_tiles) {
        up_rows<LPRH, NCHH>(p.shared, 0, b * JT + wave * (kWave / LPRH) + sub, li, p.x, p.hs);
        if (b == 0 && wave == 0) {
            float z = 0.f;
            for (int c = lane; c < H / 8; c += kWave) {
                const u32x4 a = *reinterpret_cast<const u32x4 *>(p.x + 8 * c);
                const u32x4 gv = *reinterpret_cast<const u32x4 *>(p.gate_vec + 8 * c);
                z = dot8_bf16(gv, a, z);
            }
            z = group_total<kWave>(z);
            if (lane == kWave - 1) p.gamma[0] = 1.f / (1.f + __expf(-z));
        }
        return;
    }
    b -= p.s_tiles;
    const int k = b / p.a_tiles;
    const int tile = b - k * p.a_tiles;
    const int s = p.idx[k];
    const int plan = p.route_plan ? p.route_plan[k] : -1;
    if ((s < 0) | (s >= p.slots.num_rows) | (plan >= 0)) return;
    up_rows<LPRH, NCHH>(p.slots, s, tile * JT + wave * (kWave / LPRH) + sub, li, p.x,
                        p.h + (int64_t)k * F);
}

// h chunks of a fetched route, from its gate/up dots.
template <int NCH>
__device__ __forceinline__ void h_from_gu(const float *gu, int F, int li, int lpr,
                                          XSeg<MOE_FMT_BF16, NCH> &hs) {
#pragma unroll
    for (int c = 0; c < NCH; ++c) {
        const int j0 = (li + c * lpr) * 8;
        const u32x4 *g4 = reinterpret_cast<const u32x4 *>(gu + j0);
        const u32x4 *u4 = reinterpret_cast<const u32x4 *>(gu + F + j0);
        const u32x4 ga = g4[0], gb = g4[1], ua = u4[0], ub = u4[1];
        float gv[8], uv[8];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            gv[q] = __uint_as_float(ga[q]);
            gv[4 + q] = __uint_as_float(gb[q]);
            uv[q] = __uint_as_float(ua[q]);
            uv[4 + q] = __uint_as_float(ub[q]);
        }
        u32x4 v;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const uint32_t lo = f32_to_bf16(silu_mul(gv[2 * q], uv[2 * q]));
            const uint32_t hi = f32_to_bf16(silu_mul(gv[2 * q + 1], uv[2 * q + 1]));
            v[q] = lo | (hi << 16);
        }
        hs.x[c][0] = v;
    }
}

// One batch of up to kDownBatch routes of stage 2, loads first, math after:
// the routes' slot ids and plan entries (scalar loads, issued together),
// then every W2 row and activation chunk, and with the first batch the
// shared expert's.  Routes that contribute nothing read row 0 and route 0
// as in-range stand-ins, and without a shared expert the shared view points
// at valid memory too (set by the launcher), so every load is
// unconditional and none waits for another.
template <int LPRF, int NCHF, bool FIRST>
__device__ __forceinline__ void stage2_batch(const Stage2Params &p, int k0, int ii, int li,
                                             float &acc, float &vs) {
    const int F = p.slots.F;
    int sl[kDownBatch], pe[kDownBatch];
#pragma unroll
    for (int q = 0; q < kDownBatch; ++q) {
        const int kk = min(k0 + q, p.K - 1);
        sl[q] = p.idx[kk];
        pe[q] = p.route_plan ? p.route_plan[kk] : -1;
    }
    __builtin_amdgcn_sched_barrier(0);
    WSeg<MOE_FMT_BF16, NCHF> w2[kDownBatch];
    XSeg<MOE_FMT_BF16, NCHF> hs[kDownBatch];
    int rows[kDownBatch];
#pragma unroll
    for (int q = 0; q < kDownBatch; ++q) {
        const int k = k0 + q;
        const bool ok = k < p.K && sl[q] >= 0 && sl[q] < p.slots.num_rows;
        rows[q] = ok ? sl[q] : -1;
        w2[q].load(p.slots, ok ? sl[q] : 0, 1, ii, li, LPRF);
        hs[q].load(p.h + (int64_t)min(k, p.K - 1) * F, li, LPRF);
    }
    WSeg<MOE_FMT_BF16, NCHF> w2s;
    XSeg<MOE_FMT_BF16, NCHF> hss;
    if constexpr (FIRST) {
        w2s.load(p.shared, 0, 1, ii, li, LPRF);
        hss.load(p.hs, li, LPRF);
    }
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int q = 0; q < kDownBatch; ++q) {
        if (rows[q] < 0) continue;
        if (pe[q] >= 0) h_from_gu<NCHF>(p.gu + (int64_t)pe[q] * 2 * F, F, li, LPRF, hs[q]);
        const float v = group_total<LPRF>(seg_dot(w2[q], hs[q])) * w2[q].glob(p.slots, rows[q], 1);
        acc = fmaf(p.w[k0 + q], v, acc);
    }
    if constexpr (FIRST) vs = group_total<LPRF>(seg_dot(w2s, hss)) * w2s.glob(p.shared, 0, 1);
}

template <int LPRF, int NCHF>
__global__ __launch_bounds__(kThreads) void stage2_kernel(Stage2Params p) {
    constexpr int RPW = kWave / LPRF;
    constexpr int IT = kWavesPerBlock * RPW;
    const int H = p.slots.H;
    const int wave = threadIdx.x / kWave, lane = threadIdx.x & (kWave - 1);
    const int sub = lane / LPRF, li = lane % LPRF;
    const int i = blockIdx.x * IT + wave * RPW + sub;
    const bool iok = i < H;
    const int ii = iok ? i : H - 1;

    float acc = 0.f, vs = 0.f;
    stage2_batch<LPRF, NCHF, true>(p, 0, ii, li, acc, vs);
    for (int k0 = kDownBatch; k0 < p.K; k0 += kDownBatch)
        stage2_batch<LPRF, NCHF, false>(p, k0, ii, li, acc, vs);
    float res = acc;
    if (p.addend) res = acc + p.addend[ii];
    if (p.has_shared) {
        // gamma * vs is rounded on its own (the library builds without fp
        // contraction), as the serial path rounds it when storing it
        res = acc + p.gamma[0] * vs;
    }
    if (iok && li == LPRF - 1) p.out[i] = f32_to_bf16(res);
}

template <int LPRH, int NCHH, int LPRF, int NCHF>
hipError_t launch_shape(const Stage1Params &a, const Stage2Params &b, int which, hipStream_t s) {
    constexpr int JT = kWavesPerBlock * (kWave / LPRH);
    constexpr int IT = kWavesPerBlock * (kWave / LPRF);
    Stage1Params p1 = a;
    p1.a_tiles = (p1.slots.F + JT - 1) / JT;
    p1.s_tiles = p1.s_tiles ? (p1.slots.F + JT - 1) / JT : 0;
    const int blocks1 = p1.gather_blocks + p1.s_tiles + p1.K * p1.a_tiles;
    if (which & 1) {
        hipLaunchKernelGGL((stage1_kernel<LPRH, NCHH>), dim3(blocks1), dim3(kThreads), 0, s, p1);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    if (which & 2) {
        hipLaunchKernelGGL((stage2_kernel<LPRF, NCHF>), dim3((b.slots.H + IT - 1) / IT),
                           dim3(kThreads), 0, s, b);
        return hipGetLastError();
    }
    return hipSuccess;
}

}  // namespace stage_detail

// (H chunks, F chunks) with instantiated stage kernels.
#define MOE_STAGE_SHAPES(X)                                                                  \
    X(8, 8, 1, 16, 16, 1)       /* H 64,   F 128  */                                         \
    X(128, 64, 2, 32, 32, 1)    /* H 1024, F 256  */                                         \
    X(128, 64, 2, 64, 64, 1)    /* H 1024, F 512  */                                         \
    X(256, 64, 4, 32, 32, 1)    /* H 2048, F 256  */                                         \
    X(256, 64, 4, 64, 64, 1)    /* H 2048, F 512  */                                         \
    X(256, 64, 4, 128, 64, 2)   /* H 2048, F 1024 */                                         \
    X(512, 64, 8, 64, 64, 1)    /* H 4096, F 512  */                                         \
    X(512, 64, 8, 128, 64, 2)   /* H 4096, F 1024 */

bool stage_supported(int fmt, int H, int F) {
    if (fmt != MOE_FMT_BF16) return false;
    const int ch = H / 8, cf = F / 8;
#define MOE_STAGE_HAS(CH, LH, NH, CF, LF, NF) \
    if (ch == CH && cf == CF) return true;
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
    const int ch = slots.H / 8, cf = slots.F / 8;
#define MOE_STAGE_CALL(CH, LH, NH, CF, LF, NF) \
    if (ch == CH && cf == CF) return launch_shape<LH, NH, LF, NF>(a, b, which, s);
    MOE_STAGE_SHAPES(MOE_STAGE_CALL)
#undef MOE_STAGE_CALL
    return hipErrorNotSupported;
}

}  // namespace moe
