// Slot-cache admission for one layer step, as one gfx950 workgroup.
//
// Semantics: FreeToken PR #680 "fix(moe): admit a wide offloaded decode
// step's experts 128 at a time" (section Solution) and FreeToken PR #491
// "refactor(moe): extract hybrid decode orchestration" (sections 4-5):
//  - steps of at most one_call routes are one query over their routes;
//    wider steps are the ascending distinct experts, padded to the fixed
//    length min(R, E), admitted query_width at a time;
//  - a slot used earlier in the step is never a victim, so no query
//    evicts an earlier query's experts;
//  - routes are rewritten in place to a slot id or -1; the miss plan and
//    its length stay on the device (no host sync).
// Expert ids outside [0, E) are ignored (llama.cpp fork PR #126, section
// Consumer).
//
// Design for CDNA4 (not the pages' register-block dedup):
//  - dedup is a counting pass over the expert range in LDS (E counters),
//    so its cost is O(R + E) for any step width, with no [K, K] block;
//  - the LRU order is kept as a persistent array of slots sorted by
//    (last use, slot id).  Victims of a query are the first untouched
//    entries from a cursor, found with wave ballots; at the end of the
//    step the untouched entries are compacted and the used slots appended
//    in ascending slot order.  No per-step sort of S keys is needed;
//  - one workgroup is the single writer of the slot map for the step.
//  - for caches of up to 16384 slots the step runs register-resident: each
//    thread holds a contiguous run of the LRU order (and those slots'
//    owners) in registers, loaded once at the start, so every later pass is
//    one workgroup prefix sum over per-thread counts with no global round
//    trip; the layer's slot-map row sits in LDS.  The top-k of a few token
//    rows can be fused in front (one wave per row).
#include <algorithm>

#include "moe_internal.h"

namespace moe {
namespace {

constexpr int kThreads = 1024;
constexpr int kWaves = kThreads / kWave;

// Exclusive prefix count of `f` over the workgroup (two barriers).
__device__ __forceinline__ int block_scan(bool f, int32_t *wsum, int &total) {
    return block_scan_flags<kThreads>(f, wsum, total);
}

__global__ __launch_bounds__(kThreads) void admit_kernel(AdmitParams p) {
    extern __shared__ __align__(16) int32_t lds[];
    const int E = p.E, S = p.S, R = p.R;
    int32_t *wsum = lds;            // [32]
    int32_t *misc = lds + 32;       // [8]
    int32_t *cnt = misc + 8;        // [E] routes per expert
    int32_t *slotof = cnt + E;      // [E] slot of each expert of the step, or -1
    int32_t *dlist = slotof + E;    // [E] distinct valid experts, ascending
    int32_t *missl = dlist + E;     // [E] misses of the current query
    int32_t *vict = missl + E;      // [E] victims of the current query
    int32_t *ids_l = vict + E;      // [R] the step's ids
    uint8_t *touched = reinterpret_cast<uint8_t *>(ids_l + R);  // [S] used this step
    uint8_t *filled = touched + S;  // [E] expert installed by this step's plan

    const int tid = threadIdx.x;
    const int64_t lbase = (int64_t)p.layer * E;

    for (int i = tid; i < E; i += kThreads) cnt[i] = 0;
    for (int i = tid; i < S; i += kThreads) touched[i] = 0;
    for (int i = tid; i < E; i += kThreads) filled[i] = 0;
    if (tid == 0) misc[0] = 0;
    const uint32_t now = p.clock[0] + 1u;
    __syncthreads();

    // Histogram of the step's valid routes; invalid routes counted.
    int my_invalid = 0;
    for (int i = tid; i < R; i += kThreads) {
        const int e = p.ids[i];
        ids_l[i] = e;
        if (e >= 0 && e < E)
            atomicAdd(&cnt[e], 1);
        else
            ++my_invalid;
    }
    if (my_invalid) atomicAdd(&misc[0], my_invalid);
    __syncthreads();

    // Distinct valid experts, ascending.
    int nD = 0;
    for (int base = 0; base < E; base += kThreads) {
        const int e = base + tid;
        const bool f = e < E && cnt[e] > 0;
        int tot;
        const int r = block_scan(f, wsum, tot);
        if (f) dlist[nD + r] = e;
        nD += tot;
    }
    __syncthreads();
    for (int i = tid; i < nD; i += kThreads) {
        const int e = dlist[i];
        slotof[e] = p.res[lbase + e];
        p.freq[lbase + e] += cnt[e];
        p.dlast[lbase + e] = now;
    }
    __syncthreads();

    // Query geometry: one query over the step, or query_width pieces of the
    // distinct list (pieces past the distinct experts hold only padding).
    int qwid, nq;
    if (R <= p.one_call) {
        qwid = nD > 0 ? nD : 1;
        nq = nD > 0 ? 1 : 0;
    } else {
        qwid = p.query_width;
        nq = (nD + qwid - 1) / qwid;
    }

    int cursor = 0, fetched = 0, nplan = 0, nmissed = 0, noverflow = 0;
    for (int q = 0; q < nq; ++q) {
        const int qs = q * qwid;
        const int qe = min(qs + qwid, nD);

        // Hits are used now.
        for (int i = qs + tid; i < qe; i += kThreads) {
            const int s = slotof[dlist[i]];
            if (s >= 0) {
                touched[s] = 1;
                p.stamp[s] = now;
            }
        }
        // Misses, ascending.
        int nm = 0;
        for (int base = qs; base < qe; base += kThreads) {
            const int i = base + tid;
            const bool f = i < qe && slotof[dlist[i]] < 0;
            int tot;
            const int r = block_scan(f, wsum, tot);
            if (f) missl[nm + r] = dlist[i];
            nm += tot;
        }
        __syncthreads();
        nmissed += nm;

        int allowed = nm;
        if (p.max_fetch >= 0) allowed = min(nm, max(0, p.max_fetch - fetched));

        // Victims: the first slots of the LRU order not used in this step.
        // Entries before the cursor are all used, so the walk resumes there.
        int nv = 0;
        while (nv < allowed && cursor < S) {
            const int i = cursor + tid;
            int s = -1;
            bool f = false;
            if (i < S) {
                s = p.order[i];
                f = touched[s] == 0;
            }
            int tot;
            const int r = block_scan(f, wsum, tot);
            if (f && nv + r < allowed) vict[nv + r] = s;
            if (nv + tot >= allowed) {
                nv = allowed;
                break;
            }
            nv += tot;
            cursor += kThreads;
        }
        __syncthreads();

        // Install: the j-th miss takes the j-th victim.
        for (int j = tid; j < nv; j += kThreads) {
            const int e = missl[j];
            const int s = vict[j];
            const int old = p.own[s];
            if (old >= 0) {
                p.res[old] = -1;
                // An expert of this layer losing its slot may belong to a
                // later query of this step: it becomes a miss there.
                if (old >= lbase && old < lbase + E) slotof[old - lbase] = -1;
            }
            p.own[s] = (int32_t)(lbase + e);
            p.res[lbase + e] = s;
            p.stamp[s] = now;
            slotof[e] = s;
            touched[s] = 1;
            filled[e] = 1;
            cnt[e] = nplan + j;   // the histogram is written; cnt now maps expert -> plan entry
            p.plan_slot[nplan + j] = s;
            p.plan_expert[nplan + j] = e;
        }
        noverflow += nm - nv;
        nplan += nv;
        fetched += nv;
        __syncthreads();
    }

    // Rewrite the routes in place.
    for (int i = tid; i < R; i += kThreads) {
        const int e = ids_l[i];
        const bool valid = e >= 0 && e < E;
        p.ids[i] = valid ? slotof[e] : -1;
        if (p.route_plan) p.route_plan[i] = (valid && filled[e]) ? cnt[e] : -1;
    }

    // LRU order: slots not used keep their relative order; the used ones
    // follow, ascending (they share this step's stamp).
    if (nD > 0) {
        int w = 0;
        for (int base = 0; base < S; base += kThreads) {
            const int i = base + tid;
            const int s = i < S ? p.order[i] : -1;
            const bool f = i < S && touched[s] == 0;
            int tot;
            const int r = block_scan(f, wsum, tot);
            if (f) p.order[w + r] = s;
            w += tot;
        }
        for (int base = 0; base < S; base += kThreads) {
            const int s = base + tid;
            const bool f = s < S && touched[s] != 0;
            int tot;
            const int r = block_scan(f, wsum, tot);
            if (f) p.order[w + r] = s;
            w += tot;
        }
    }

    if (tid == 0) {
        int64_t *st = p.stats + (int64_t)p.layer * MOE_NUM_STATS;
        st[MOE_STAT_CALLS] += 1;
        st[MOE_STAT_MET] += nD;
        st[MOE_STAT_MISSED] += nmissed;
        st[MOE_STAT_OVERFLOW] += noverflow;
        st[MOE_STAT_INVALID] += misc[0];
        p.clock[0] = now;
        p.clock[1] = now;   // the latest demand step
        p.n_miss[0] = nplan;
    }
}


// ------------------------------------------------------------------ register-resident admission

constexpr int kFastMaxP = 16;       // slots per thread: S <= 16384
constexpr int kTopkMaxPerLane = 16; // fused top-k: E <= 1024

// Exclusive prefix sum of per-thread counts over the workgroup.
__device__ __forceinline__ int block_scan_count(int v, int32_t *wsum, int &total) {
    const int lane = threadIdx.x & (kWave - 1);
    const int wave = threadIdx.x / kWave;
    const int x = wave_inclusive_sum(v);
    if (lane == kWave - 1) wsum[wave] = x;
    __syncthreads();
    int woff = 0, tot = 0;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) {
        const int c = wsum[w];
        woff += (w < wave) ? c : 0;
        tot += c;
    }
    __syncthreads();
    total = tot;
    return woff + x - v;
}

// Order-preserving key of a logit: larger key = larger value; NaN sorts as
// -infinity and -0 as +0.
__device__ __forceinline__ uint32_t logit_key(float v) {
    uint32_t u = __float_as_uint(v);
    if ((u & 0x7fffffffu) > 0x7f800000u) u = 0xff800000u;
    if (u == 0x80000000u) u = 0u;
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}
__device__ __forceinline__ float key_logit(uint32_t k) {
    return __uint_as_float((k & 0x80000000u) ? (k & 0x7fffffffu) : ~k);
}

// Top-K of one row of E <= 1024 logits by one wave: K rounds of a wave
// maximum over 64-bit (value key, ~index) pairs strictly below the previous
// pick, i.e. largest first and lower expert id first among equals.  The
// weights are the softmax over the picks (1/K each if all are -infinity).
// Top-K of one row of E logits by one wave.  Each lane holds the keys of
// experts lane, lane + 64, ... (NC of them) and its best key not yet taken;
// a round takes the wave's maximum of those (two 32-bit DPP max passes:
// value, then id among the lanes holding that value), and only the lane
// that held it looks for its next best.
template <int NC>
__device__ __forceinline__ void wave_topk_nc(const float *__restrict__ row, int E, int K, int32_t *ids_lds,
                                             float *w_out) {
    const int lane = threadIdx.x & (kWave - 1);
    // the row's logits, all loads in flight together (clamped in-range
    // indices)
    float lv[NC];
#pragma unroll
    for (int c = 0; c < NC; ++c) lv[c] = row[min(lane + kWave * c, E - 1)];
    uint64_t keys[NC];
    uint64_t lb = 0ull;
#pragma unroll
    for (int c = 0; c < NC; ++c) {
        const int e = lane + kWave * c;
        keys[c] = e < E ? ((uint64_t)logit_key(lv[c]) << 32) | (uint64_t)(0xffffffffu - (uint32_t)e)
                        : 0ull;
        lb = keys[c] > lb ? keys[c] : lb;
    }
    uint64_t mine = 0ull;
    for (int k = 0; k < K; ++k) {
        const uint32_t mh = wave_max_u32((uint32_t)(lb >> 32));
        const uint32_t ml = wave_max_u32((uint32_t)(lb >> 32) == mh ? (uint32_t)lb : 0u);
        const uint64_t best = ((uint64_t)mh << 32) | ml;
        if (lane == k) mine = best;
        if (lb == best) {
            uint64_t nb = 0ull;
#pragma unroll
            for (int c = 0; c < NC; ++c)
                if (keys[c] < best && keys[c] > nb) nb = keys[c];
            lb = nb;
        }
    }
    const float v = key_logit((uint32_t)(mine >> 32));
    const float m = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 0));
    float ex = 0.f;
    if (lane < K) ex = (m == -INFINITY) ? 1.f : __expf(v - m);
    const float z = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(group_total<kWave>(ex)), kWave - 1));
    if (lane < K) {
        ids_lds[lane] = (int32_t)(0xffffffffu - (uint32_t)mine);
        w_out[lane] = ex / z;
    }
}

__device__ __forceinline__ void wave_topk(const float *__restrict__ row, int E, int K, int32_t *ids_lds,
                                          float *w_out) {
    const int nc = (E + kWave - 1) / kWave;
    if (nc <= 1) wave_topk_nc<1>(row, E, K, ids_lds, w_out);
    else if (nc <= 2) wave_topk_nc<2>(row, E, K, ids_lds, w_out);
    else if (nc <= 4) wave_topk_nc<4>(row, E, K, ids_lds, w_out);
    else if (nc <= 8) wave_topk_nc<8>(row, E, K, ids_lds, w_out);
    else wave_topk_nc<16>(row, E, K, ids_lds, w_out);
}

// Register-resident admission.  p.order holds (slot, owner) pairs here, so
// the owners of victim candidates arrive with the order itself.  Every
// write to the persistent state is deferred to the final phase: a barrier
// waits for a wave's outstanding memory operations, so stores issued
// between barriers would each cost a memory round trip.
constexpr int kNarrowWindow = 4 * kWave;

// The admission's statistics are the first five (calls, met, missed,
// overflow, invalid); stat_delta gives statistic k's increment of a step.
constexpr int kAdmitStats = 5;
static_assert(MOE_STAT_CALLS == 0 && MOE_STAT_MET == 1 && MOE_STAT_MISSED == 2 && MOE_STAT_OVERFLOW == 3 &&
                  MOE_STAT_INVALID == 4,
              "admission statistics are indices 0-4");
__device__ __forceinline__ int64_t stat_delta(int k, int met, int missed, int overflow, int invalid) {
    return k == MOE_STAT_CALLS ? 1 : k == MOE_STAT_MET ? met : k == MOE_STAT_MISSED ? missed
                                                     : k == MOE_STAT_OVERFLOW ? overflow : invalid;
}

// Orders LDS accesses of one wave: a compiler fence (a wave's LDS
// instructions execute in issue order).
__device__ __forceinline__ void wave_lds_fence() {
    __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
    __builtin_amdgcn_wave_barrier();
}

struct lds_view {
    int64_t *freq_l;
    int32_t *cnt, *resl, *dlist, *missl, *pslot, *pold, *pexp, *ids_l;
    uint16_t *slot_e;
    uint8_t *touched, *filled;
    int32_t *misc;
};

// The whole admission step of at most 64 routes by wave 0 (lane i = route
// i, then lane j = distinct expert j), with the same steps and results as
// the wide path: histogram, ascending distinct list, the queries (hits
// used, misses ascending, the j-th admitted miss takes the j-th unused
// entry of the LRU order), and every write of the step except the order
// itself.  The victims of a query are among the first
//   (slots used so far this step) + (misses) <= 2 * 64 + 64
// entries of the order, inside the 256-entry window the wave holds.
__device__ __forceinline__ void narrow_step(const AdmitParams &p, lds_view v, const int (&wslot)[4],
                                         const int (&wown)[4], uint32_t now, int64_t st_lane) {
    const int lane = threadIdx.x;
    const int E = p.E, R = p.R;
    const int64_t lbase = (int64_t)p.layer * E;

    const int e_i = lane < R ? v.ids_l[lane] : -1;
    const bool valid = lane < R && e_i >= 0 && e_i < E;
    if (valid) atomicAdd(&v.cnt[e_i], 1);
    const int ninvalid = __popcll(__ballot(lane < R && !valid));
    wave_lds_fence();

    // distinct valid experts, ascending: each lane scans a run of E
    const int run = (E + kWave - 1) / kWave;
    int c = 0;
    for (int q = 0; q < run; ++q) {
        const int e = lane * run + q;
        c += (e < E && v.cnt[e] > 0);
    }
    const int incl = wave_inclusive_sum(c);
    const int nD = __builtin_amdgcn_readlane(incl, kWave - 1);
    {
        int off = incl - c;
        for (int q = 0; q < run; ++q) {
            const int e = lane * run + q;
            if (e < E && v.cnt[e] > 0) v.dlist[off++] = e;
        }
    }
    wave_lds_fence();

    int qwid, nq;
    if (R <= p.one_call) {
        qwid = nD > 0 ? nD : 1;
        nq = nD > 0 ? 1 : 0;
    } else {
        qwid = p.query_width;
        nq = (nD + qwid - 1) / qwid;
    }
    int fetched = 0, nplan = 0, nmissed = 0, noverflow = 0;
    for (int q = 0; q < nq; ++q) {
        const int qs = q * qwid;
        const int qn = min(qs + qwid, nD) - qs;
        // hits are used now; misses ranked in ascending expert order
        const int e = lane < qn ? v.dlist[qs + lane] : -1;
        const int s = e >= 0 ? v.resl[e] : -1;
        if (e >= 0 && s >= 0) v.touched[s] = 1;
        const bool miss = e >= 0 && s < 0;
        const uint64_t mm = __ballot(miss);
        const int nm = __popcll(mm);
        if (miss)
            v.missl[__builtin_amdgcn_mbcnt_hi((uint32_t)(mm >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)mm, 0u))] = e;
        nmissed += nm;
        int allowed = nm;
        if (p.max_fetch >= 0) allowed = min(nm, max(0, p.max_fetch - fetched));
        wave_lds_fence();
        if (allowed > 0) {
            bool el[4];
            int ce = 0;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                el[i] = wslot[i] >= 0 && v.touched[wslot[i]] == 0;
                ce += el[i];
            }
            const int incl2 = wave_inclusive_sum(ce);
            const int elig = __builtin_amdgcn_readlane(incl2, kWave - 1);
            int r = incl2 - ce;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                if (el[i]) {
                    if (r < allowed) {
                        const int j = nplan + r;
                        const int em = v.missl[r];
                        v.pslot[j] = wslot[i];
                        v.pold[j] = wown[i];
                        v.pexp[j] = em;
                        v.resl[em] = wslot[i];
                        v.filled[em] = 1;
                        const int old = wown[i];
                        // an expert of this layer losing its slot may belong to a
                        // later query of this step: it becomes a miss there
                        if (old >= lbase && old < lbase + E) v.resl[old - lbase] = -1;
                    }
                    ++r;
                }
            }
            const int nv = min(allowed, elig);
            wave_lds_fence();
            for (int j = lane; j < nv; j += kWave) v.touched[v.pslot[nplan + j]] = 1;
            wave_lds_fence();
            noverflow += nm - nv;
            nplan += nv;
            fetched += nv;
        } else {
            noverflow += nm;
        }
    }

    // expert -> plan entry, for the routes' plan indices
    if (p.route_plan) {
        for (int j = lane; j < nplan; j += kWave) v.missl[v.pexp[j]] = j;
        wave_lds_fence();
    }
    if (lane < R) {
        p.ids[lane] = valid ? v.resl[e_i] : -1;
        if (p.route_plan) p.route_plan[lane] = (valid && v.filled[e_i]) ? v.missl[e_i] : -1;
    }
    for (int e = lane; e < E; e += kWave) p.res[lbase + e] = v.resl[e];
    for (int j = lane; j < nplan; j += kWave) {
        const int s = v.pslot[j], old = v.pold[j], em = v.pexp[j];
        if (old >= 0 && !(old >= lbase && old < lbase + E)) p.res[old] = -1;
        p.own[s] = (int32_t)(lbase + em);
        p.plan_slot[j] = s;
        p.plan_expert[j] = em;
    }
    for (int i = lane; i < nD; i += kWave) {
        const int e = v.dlist[i];
        const int s = v.resl[e];
        if (s >= 0) {
            p.stamp[s] = now;
            v.slot_e[s] = (uint16_t)e;
        }
        p.freq[lbase + e] = v.freq_l[e] + v.cnt[e];
        p.dlast[lbase + e] = now;
    }
    if (lane < kAdmitStats)
        p.stats[(int64_t)p.layer * MOE_NUM_STATS + lane] =
            st_lane + stat_delta(lane, nD, nmissed, noverflow, ninvalid);
    if (lane == 0) {
        p.clock[0] = now;
        p.clock[1] = now;
        p.n_miss[0] = nplan;
        v.misc[1] = nD;
    }
}

// The arguments the prologue's loads need lead, as scalars: gfx950 preloads
// the leading kernel arguments into scalar registers at wave launch, so the
// clock, order, slot map, histogram and logits requests go out without
// waiting for an argument load first.
template <int P>
__global__ __launch_bounds__(kThreads) void admit_fast_kernel(uint32_t *clock, int32_t *order, int32_t *res,
                                                              int64_t *freq, const float *logits, int layer,
                                                              int E_, int R_, int S_, AdmitParams p_in) {
    extern __shared__ __align__(16) int32_t lds[];
    AdmitParams p = p_in;
    p.clock = clock;
    p.order = order;
    p.res = res;
    p.freq = freq;
    p.logits = logits;
    p.layer = layer;
    p.E = E_;
    p.R = R_;
    p.S = S_;
    const int E = p.E, S = p.S, R = p.R;
    int32_t *wsum = lds;            // [32]
    int32_t *misc = lds + 32;       // [16]: 0 invalid routes
    int64_t *freq_l = reinterpret_cast<int64_t *>(misc + 16);  // [E] the layer's histogram row
    int32_t *cnt = misc + 16 + 2 * E;  // [E] routes per expert
    int32_t *resl = cnt + E;        // [E] the layer's slot map row, kept current
    int32_t *dlist = resl + E;      // [E] distinct valid experts, ascending
    int32_t *missl = dlist + E;     // [E] misses of the current query
    int32_t *pslot = missl + E;     // [E] the step's plan: slot,
    int32_t *pold = pslot + E;      // [E]   previous owner of that slot,
    int32_t *pexp = pold + E;       // [E]   expert installed
    int32_t *ids_l = pexp + E;      // [R]
    uint16_t *slot_e = reinterpret_cast<uint16_t *>(ids_l + R);  // [S] expert of a used slot
    uint8_t *touched = reinterpret_cast<uint8_t *>(slot_e + S);    // [S] slot used this step
    uint8_t *filled = touched + S;                                 // [E] installed this step
    const int tid = threadIdx.x;
    const int wave = tid / kWave;
    const int64_t lbase = (int64_t)p.layer * E;

    // Every load of the prologue is issued before any result is used: the
    // clock, the statistics, the LRU order (and, for a narrow step, its
    // head again as wave 0's victim window), the slot map and histogram
    // rows, and last the logits of the fused top-k, which runs as soon as
    // they land, while the rows still wait for LDS.  Measured on MI355X at
    // the 40 x 256 decode: with the clock read after the rows reached LDS
    // (a second round trip) and the preloaded logits kept in scratch (one
    // round trip per 64 of them), prologue and top-k took 6.7 us.  This
    // kernel is the only writer of the layer's statistics and histogram
    // during the step, so they are updated with plain stores of the values
    // read here.
    // The clock and the admission statistics (one per lane of the first
    // threads) are read with vector loads: as scalar loads they shared a
    // counter with the kernel arguments read later, and waiting for those
    // waited for them.  mbcnt_lo(0, 0) is 0 in every lane, but lane-varying
    // to the compiler.
    const uint32_t clk = p.clock[__builtin_amdgcn_mbcnt_lo(0u, 0u)];

    // This thread's run of the LRU order: (slot, owner) pairs.  The order
    // buffer holds kThreads * P pairs (admit_order_bytes), so the loads are
    // unconditional 16-byte ones, all in flight together; positions past S
    // are masked once the top-k is done.
    int4 ov[P / 2 > 0 ? P / 2 : 1];
    int2 ov1;
    if constexpr (P == 1) {
        ov1 = reinterpret_cast<const int2 *>(p.order)[tid];
    } else {
        const int4 *q4 = reinterpret_cast<const int4 *>(p.order) + tid * (P / 2);
#pragma unroll
        for (int q = 0; q < P / 2; ++q) ov[q] = q4[q];
    }
    // A narrow step (at most one route per lane of wave 0) is admitted by
    // wave 0 alone; its victims come from the head of the LRU order, of
    // which the wave holds the first kNarrowWindow entries (four per lane).
    const bool narrow = R <= kWave;
    const bool window = narrow && wave == 0;
    int4 wa, wb;   // read only where window holds (selected after the top-k, so no early wait)
    if (window) {
        const int4 *q4 = reinterpret_cast<const int4 *>(p.order) + tid * 2;
        wa = q4[0];
        wb = q4[1];
    }
    // The layer's slot map and histogram rows into LDS, 4 * kThreads
    // entries a batch (clamped in-range indices): the first batch's loads
    // are issued here, their LDS stores follow the top-k.
    auto load_rows = [&](int e0, int32_t (&v)[4], int64_t (&fv)[4]) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int64_t e = lbase + min(e0 + tid + j * kThreads, E - 1);
            v[j] = p.res[e];
            fv[j] = p.freq[e];
        }
    };
    auto store_rows = [&](int e0, const int32_t (&v)[4], const int64_t (&fv)[4]) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int e = e0 + tid + j * kThreads;
            if (e < E) {
                resl[e] = v[j];
                freq_l[e] = fv[j];
                cnt[e] = 0;
                filled[e] = 0;
            }
        }
    };
    int32_t rv[4];
    int64_t rfv[4];
    load_rows(0, rv, rfv);
    // (after the requests above: the statistics' address is a kernel
    // argument that is not preloaded)
    const int64_t st_lane = tid < kAdmitStats ? p.stats[(int64_t)p.layer * MOE_NUM_STATS + tid] : 0;

    if (p.logits != nullptr) {
        for (int t = wave; t < p.T; t += kWaves)
            wave_topk(p.logits + (int64_t)t * E, E, p.K, ids_l + t * p.K, p.w_out + (int64_t)t * p.K);
    } else {
        for (int i = tid; i < R; i += kThreads) ids_l[i] = p.ids[i];
    }

    int ord[P], owner[P];
    if constexpr (P == 1) {
        ord[0] = ov1.x;
        owner[0] = ov1.y;
    } else {
#pragma unroll
        for (int q = 0; q < P / 2; ++q) {
            ord[2 * q] = ov[q].x;
            owner[2 * q] = ov[q].y;
            ord[2 * q + 1] = ov[q].z;
            owner[2 * q + 1] = ov[q].w;
        }
    }
#pragma unroll
    for (int q = 0; q < P; ++q)
        if (tid * P + q >= S) ord[q] = owner[q] = -1;
    int wslot[4] = {-1, -1, -1, -1}, wown[4] = {-1, -1, -1, -1};
    if (window) {
        wslot[0] = wa.x; wown[0] = wa.y; wslot[1] = wa.z; wown[1] = wa.w;
        wslot[2] = wb.x; wown[2] = wb.y; wslot[3] = wb.z; wown[3] = wb.w;
#pragma unroll
        for (int i = 0; i < 4; ++i)
            if (tid * 4 + i >= S) wslot[i] = wown[i] = -1;
    }
    store_rows(0, rv, rfv);
    for (int e0 = 4 * kThreads; e0 < E; e0 += 4 * kThreads) {
        load_rows(e0, rv, rfv);
        store_rows(e0, rv, rfv);
    }
    for (int i = tid; i < S; i += kThreads) touched[i] = 0;
    if (tid < 16) misc[tid] = 0;
    const uint32_t now = clk + 1u;
    __syncthreads();

    int nD;
    if (narrow) {
        if (wave == 0) narrow_step(p, lds_view{freq_l, cnt, resl, dlist, missl, pslot, pold, pexp, ids_l,
                                                slot_e, touched, filled, misc},
                                   wslot, wown, now, st_lane);
        __syncthreads();
        nD = misc[1];
    } else {
    // Histogram of the valid routes; invalid routes counted.
    int my_invalid = 0;
    for (int i = tid; i < R; i += kThreads) {
        const int e = ids_l[i];
        if (e >= 0 && e < E)
            atomicAdd(&cnt[e], 1);
        else
            ++my_invalid;
    }
    if (my_invalid) atomicAdd(&misc[0], my_invalid);
    __syncthreads();

    // Distinct valid experts, ascending: each thread scans a run of E.
    const int erun = (E + kThreads - 1) / kThreads;
    {
        int c = 0;
        for (int q = 0; q < erun; ++q) {
            const int e = tid * erun + q;
            c += (e < E && cnt[e] > 0);
        }
        int off = block_scan_count(c, wsum, nD);
        for (int q = 0; q < erun; ++q) {
            const int e = tid * erun + q;
            if (e < E && cnt[e] > 0) dlist[off++] = e;
        }
    }
    __syncthreads();

    int qwid, nq;
    if (R <= p.one_call) {
        qwid = nD > 0 ? nD : 1;
        nq = nD > 0 ? 1 : 0;
    } else {
        qwid = p.query_width;
        nq = (nD + qwid - 1) / qwid;
    }

    int fetched = 0, nplan = 0, nmissed = 0, noverflow = 0;
    for (int q = 0; q < nq; ++q) {
        const int qs = q * qwid;
        const int qn = min(qs + qwid, nD) - qs;

        // Hits are used now; misses, ascending (each thread a run).
        for (int i = tid; i < qn; i += kThreads) {
            const int s = resl[dlist[qs + i]];
            if (s >= 0) touched[s] = 1;
        }
        int nm;
        {
            const int run = (qn + kThreads - 1) / kThreads;
            int c = 0;
            for (int k = 0; k < run; ++k) {
                const int i = tid * run + k;
                c += (i < qn && resl[dlist[qs + i]] < 0);
            }
            int off = block_scan_count(c, wsum, nm);
            for (int k = 0; k < run; ++k) {
                const int i = tid * run + k;
                if (i < qn && resl[dlist[qs + i]] < 0) missl[off++] = dlist[qs + i];
            }
        }
        nmissed += nm;
        int allowed = nm;
        if (p.max_fetch >= 0) allowed = min(nm, max(0, p.max_fetch - fetched));

        // Victims: the first entries of the LRU order not used in this step;
        // the j-th miss takes the j-th victim.
        if (allowed > 0) {
            int c = 0;
#pragma unroll
            for (int k = 0; k < P; ++k) c += (ord[k] >= 0 && touched[ord[k]] == 0);
            int elig;
            int r = block_scan_count(c, wsum, elig);
#pragma unroll
            for (int k = 0; k < P; ++k) {
                if (ord[k] >= 0 && touched[ord[k]] == 0) {
                    if (r < allowed) {
                        const int j = nplan + r;
                        const int e = missl[r];
                        pslot[j] = ord[k];
                        pold[j] = owner[k];
                        pexp[j] = e;
                        resl[e] = ord[k];
                        filled[e] = 1;
                        const int old = owner[k];
                        // an expert of this layer losing its slot may belong to a
                        // later query of this step: it becomes a miss there
                        if (old >= lbase && old < lbase + E) resl[old - lbase] = -1;
                    }
                    ++r;
                }
            }
            const int nv = min(allowed, elig);
            __syncthreads();
            for (int j = tid; j < nv; j += kThreads) touched[pslot[nplan + j]] = 1;
            noverflow += nm - nv;
            nplan += nv;
            fetched += nv;
        } else {
            noverflow += nm;
        }
        __syncthreads();
    }

    // expert -> plan entry, for the routes' plan indices
    if (p.route_plan) {
        for (int j = tid; j < nplan; j += kThreads) missl[pexp[j]] = j;
        __syncthreads();
    }

    // ---- final phase: every write to the persistent state.
    for (int i = tid; i < R; i += kThreads) {
        const int e = ids_l[i];
        const bool valid = e >= 0 && e < E;
        p.ids[i] = valid ? resl[e] : -1;
        if (p.route_plan) p.route_plan[i] = (valid && filled[e]) ? missl[e] : -1;
    }
    for (int e = tid; e < E; e += kThreads) p.res[lbase + e] = resl[e];
    for (int j = tid; j < nplan; j += kThreads) {
        const int s = pslot[j], old = pold[j], e = pexp[j];
        if (old >= 0 && !(old >= lbase && old < lbase + E)) p.res[old] = -1;
        p.own[s] = (int32_t)(lbase + e);
        p.plan_slot[j] = s;
        p.plan_expert[j] = e;
    }
    for (int i = tid; i < nD; i += kThreads) {
        const int e = dlist[i];
        const int s = resl[e];
        if (s >= 0) {
            p.stamp[s] = now;
            slot_e[s] = (uint16_t)e;
        }
        p.freq[lbase + e] = freq_l[e] + cnt[e];
        p.dlast[lbase + e] = now;
    }
    if (tid < kAdmitStats)
        p.stats[(int64_t)p.layer * MOE_NUM_STATS + tid] =
            st_lane + stat_delta(tid, nD, nmissed, noverflow, misc[0]);
    if (tid == 0) {
        p.clock[0] = now;
        p.clock[1] = now;
        p.n_miss[0] = nplan;
    }

    }  // wide step

    // LRU order: the unused entries keep their order; the used slots follow
    // in ascending slot order (they share this step's stamp), each owned by
    // its expert of this layer.  One prefix sum counts both parts.
    if (nD > 0) {
        __syncthreads();   // slot_e
        int cu = 0, ct = 0;
#pragma unroll
        for (int k = 0; k < P; ++k) cu += (ord[k] >= 0 && touched[ord[k]] == 0);
#pragma unroll
        for (int k = 0; k < P; ++k) {
            const int s = tid * P + k;
            ct += (s < S && touched[s] != 0);
        }
        int tot;
        const int pre = block_scan_count(cu | (ct << 16), wsum, tot);
        const int kept = tot & 0xffff;
        int ou = pre & 0xffff, ot = kept + (pre >> 16);
        int2 *out = reinterpret_cast<int2 *>(p.order);
#pragma unroll
        for (int k = 0; k < P; ++k)
            if (ord[k] >= 0 && touched[ord[k]] == 0) out[ou++] = make_int2(ord[k], owner[k]);
#pragma unroll
        for (int k = 0; k < P; ++k) {
            const int s = tid * P + k;
            if (s < S && touched[s] != 0) out[ot++] = make_int2(s, (int)(lbase + slot_e[s]));
        }
    }
}

#define MOE_ADMIT_LEAD(p) (p).clock, (p).order, (p).res, (p).freq, (p).logits, (p).layer, (p).E, (p).R, (p).S

int fast_p(int S) {
    int P = 1;
    while (P * kThreads < S) P *= 2;
    return P;
}

}  // namespace

bool admit_order_pairs(int S) { return fast_p(S) <= kFastMaxP; }

size_t admit_order_bytes(int S) {
    return admit_order_pairs(S) ? (size_t)kThreads * fast_p(S) * 8 : (size_t)S * 4;
}

bool admit_fused_topk_supported(int E, int S, int K) {
    return E <= kWave * kTopkMaxPerLane && K <= kWave && fast_p(S) <= kFastMaxP;
}

size_t admit_lds_bytes(int E, int S, int max_routes) {
    // the larger of the two kernels' layouts
    const size_t general = (32 + 8 + 5 * (size_t)E + (size_t)max_routes) * 4 + (size_t)S + (size_t)E;
    const size_t fast =
        (32 + 16 + 10 * (size_t)E + (size_t)max_routes) * 4 + 3 * (size_t)S + (size_t)E;
    return (std::max(general, fast) + 15) & ~(size_t)15;
}

hipError_t admit_prepare(size_t lds_bytes) {
    if (lds_bytes <= 65536) return hipSuccess;
    const void *kernels[] = {
        reinterpret_cast<const void *>(&admit_kernel),
        reinterpret_cast<const void *>(&admit_fast_kernel<1>),
        reinterpret_cast<const void *>(&admit_fast_kernel<2>),
        reinterpret_cast<const void *>(&admit_fast_kernel<4>),
        reinterpret_cast<const void *>(&admit_fast_kernel<8>),
        reinterpret_cast<const void *>(&admit_fast_kernel<16>),
    };
    for (const void *k : kernels) {
        hipError_t e = hipFuncSetAttribute(k, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds_bytes);
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
}

hipError_t launch_admit(const AdmitParams &p, size_t lds_bytes, hipStream_t s) {
    if (rec::on())
        // the state (slot map, owners, stamps, order, clock, statistics,
        // histogram, demand recency) is read and rewritten; the plan, the
        // route plan, the rewritten ids and (fused top-k) the weights written
        return rec::launch("admit_kernel", s,
                           {{p.logits, rec::kRead}, {p.ids, p.logits ? rec::kWrite : rec::kReadWrite},
                            {p.res, rec::kReadWrite}, {p.plan_slot, rec::kWrite},
                            {p.route_plan, rec::kWrite}, {p.w_out, rec::kWrite}});
    switch (fast_p(p.S)) {
    case 1: hipLaunchKernelGGL(admit_fast_kernel<1>, dim3(1), dim3(kThreads), lds_bytes, s, MOE_ADMIT_LEAD(p), p); break;
    case 2: hipLaunchKernelGGL(admit_fast_kernel<2>, dim3(1), dim3(kThreads), lds_bytes, s, MOE_ADMIT_LEAD(p), p); break;
    case 4: hipLaunchKernelGGL(admit_fast_kernel<4>, dim3(1), dim3(kThreads), lds_bytes, s, MOE_ADMIT_LEAD(p), p); break;
    case 8: hipLaunchKernelGGL(admit_fast_kernel<8>, dim3(1), dim3(kThreads), lds_bytes, s, MOE_ADMIT_LEAD(p), p); break;
    case 16: hipLaunchKernelGGL(admit_fast_kernel<16>, dim3(1), dim3(kThreads), lds_bytes, s, MOE_ADMIT_LEAD(p), p); break;
    default:
        if (p.logits != nullptr) return hipErrorInvalidValue;
        hipLaunchKernelGGL(admit_kernel, dim3(1), dim3(kThreads), lds_bytes, s, p);
    }
    return hipGetLastError();
}

}  // namespace moe
