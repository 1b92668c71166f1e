// The look-ahead prefetch kernel (llama.cpp fork PR #126, sections
// Consumer and Eviction guard): one workgroup on the stream of the demand
// admissions fills a layer's predicted experts through the persistent LRU
// order the admission kernels keep, under the LFRU guard.
#include <algorithm>

#include "moe_internal.h"

namespace moe {
namespace {

constexpr int kThreads = 1024;

__device__ __forceinline__ int block_scan(bool f, int32_t *wsum, int &total) {
    return block_scan_flags<kThreads>(f, wsum, total);
}

// LFRU score of an expert's demand heat (llama.cpp fork PR #126, section
// Eviction guard): demand routes in the high bits, a recency byte that is
// 255 right after a demand step and falls by one per clock tick to 0 (0 if
// never demanded) in the low byte.
__device__ __forceinline__ int64_t lfru_score(int64_t freq, uint32_t dlast, uint32_t now) {
    const uint32_t age = now - dlast;
    const int64_t rec = dlast == 0u ? 0 : 255 - (int64_t)min(age, 255u);
    return freq * 256 + rec;
}

// One look-ahead prefetch of a layer's predicted experts (llama.cpp fork PR
// #126, sections Consumer and Eviction guard), as one workgroup on the
// stream of the demand admissions, so the slot map keeps a single writer.
//  - The predicted ids in [0, E) are marked in LDS; resident ones are hits
//    (used now), the others are the missing predictions, ascending.
//  - Candidates are read off the persistent LRU order from its head:
//    entries used by this call or pinned (stamp at or after the latest
//    demand step) are skipped; at most one per missing prediction is kept.
//  - The guard decisions are sequential in principle (a drop leaves the
//    cursor where it is), but wave 0 takes them 64 predictions at a time:
//    against the current victim, one ballot finds the first prediction the
//    victim does not block; the ones before it are dropped.
//  - Every write to the persistent state comes last; the order is
//    compacted like a demand step's (untouched entries keep their order,
//    the slots used by this call follow in ascending slot order).
__global__ __launch_bounds__(kThreads) void prefetch_kernel(PrefetchParams p) {
    extern __shared__ __align__(16) int32_t lds[];
    // M >= the distinct valid predictions of the call (min(n, E)): the
    // per-prediction arrays hold at most that many entries
    const int E = p.E, S = p.S, M = p.M;
    int32_t *wsum = lds;                                          // [32]
    int32_t *misc = lds + 32;                                     // [16]
    int64_t *score_v = reinterpret_cast<int64_t *>(misc + 16);    // [M] candidate owner's score, -1: never protected
    int64_t *score_p = score_v + M;                               // [M] missing prediction's score
    int32_t *missl = reinterpret_cast<int32_t *>(score_p + M);    // [M] missing predictions, ascending
    int32_t *vslot = missl + M;                                   // [M] candidates, least recently used first,
    int32_t *vown = vslot + M;                                    // [M]   and their owners
    int32_t *fslot = vown + M;                                    // [M] fills: slot,
    int32_t *fold = fslot + M;                                    // [M]   previous owner,
    int32_t *fexp = fold + M;                                     // [M]   expert
    int32_t *tslot = fexp + M;                                    // [M] slots used by this call
    int32_t *town = tslot + M;                                    // [M]   and their owners
    uint8_t *want = reinterpret_cast<uint8_t *>(town + M);        // [E] predicted
    uint8_t *touched = want + E;                                  // [S] used by this call
    const int tid = threadIdx.x;
    const int lane = tid & (kWave - 1);
    const int wave = tid / kWave;
    const int64_t lbase = (int64_t)p.layer * E;

    // ---- every load the call can issue before any result is used, in one
    // round trip (then one more for what depends on the order's entries):
    // the clock (vector loads: mbcnt_lo(0, 0) is 0 but lane-varying to the
    // compiler, so they do not share a counter with later kernel-argument
    // loads), the first predictions, the layer's slot-map entries and demand
    // heat, this thread's entries of the LRU order, and for its first entry
    // the slot's stamp and the owner's heat.  Measured on MI355X in the
    // decode graph, the same work with each load issued where it is used
    // took about seven dependent round trips (11 us a call).
    const int z = (int)__builtin_amdgcn_mbcnt_lo(0u, 0u);
    const uint32_t now = p.clock[z] + 1u;
    const uint32_t latest_demand = p.clock[z + 1];
    const int id0 = tid < p.n ? p.ids[tid] : -1;
    const int e0 = min(tid, E - 1);
    const int res0 = p.res[lbase + e0];
    const int64_t freq0 = p.freq[lbase + e0];
    const uint32_t dlast0 = p.dlast[lbase + e0];
    constexpr int kHeld = 4;                 // order entries a thread holds (S <= 4096)
    // (slot, owner) pairs or bare slots: the same two dword loads either
    // way (a bare slot read twice), so no branch sits between the loads
    int ord[kHeld], oown[kHeld];
    const int step = p.pairs ? 2 : 1;
#pragma unroll
    for (int k = 0; k < kHeld; ++k) {
        const int i = min(tid + k * kThreads, S - 1);
        ord[k] = p.order[(int64_t)i * step];
        oown[k] = p.order[(int64_t)i * step + (step - 1)];
    }
#pragma unroll
    for (int k = 0; k < kHeld; ++k)
        if (!p.pairs) oown[k] = -1;
    const int s00 = ord[0] >= 0 && ord[0] < S ? ord[0] : 0;
    // the first entry's owner and its heat, then its slot's stamp: with
    // pairs the owner came with the order (so both are a second round
    // trip), else it comes from the owner map first
    int o00;
    int64_t ofreq0;
    uint32_t odlast0, stamp0;
    if (p.pairs) {
        o00 = oown[0];
        const int oi = o00 >= 0 ? o00 : 0;
        ofreq0 = p.freq[oi];
        odlast0 = p.dlast[oi];
        stamp0 = p.stamp[s00];
    } else {
        stamp0 = p.stamp[s00];
        o00 = p.own[s00];
        const int oi = o00 >= 0 ? o00 : 0;
        ofreq0 = p.freq[oi];
        odlast0 = p.dlast[oi];
    }
    // entry i of the order (held for i < kHeld * kThreads)
    auto order_at = [&](int base, int i, int &sl, int &ow) {
        const int k = base / kThreads;
        if (k < kHeld) {
            sl = k == 0 ? ord[0] : k == 1 ? ord[1] : k == 2 ? ord[2] : ord[3];
            ow = k == 0 ? oown[0] : k == 1 ? oown[1] : k == 2 ? oown[2] : oown[3];
        } else if (p.pairs) {
            const int2 v = reinterpret_cast<const int2 *>(p.order)[i];
            sl = v.x;
            ow = v.y;
        } else {
            sl = p.order[i];
            ow = -1;
        }
    };

    for (int e = tid; e < E; e += kThreads) want[e] = 0;
    for (int sl = tid; sl < S; sl += kThreads) touched[sl] = 0;
    __syncthreads();
    for (int i = tid; i < p.n; i += kThreads) {
        const int e = i == tid ? id0 : p.ids[i];
        if (e >= 0 && e < E) want[e] = 1;
    }
    __syncthreads();

    // Hits (used now) and missing predictions, both ascending, with the
    // missing predictions' scores.
    int nh = 0, nm = 0;
    for (int base = 0; base < E; base += kThreads) {
        const int e = base + tid;
        const bool w = e < E && want[e] != 0;
        const int sl = w ? (base == 0 ? res0 : p.res[lbase + e]) : -1;
        const bool hit = w && sl >= 0, miss = w && sl < 0;
        int th, tm;
        const int rh = block_scan(hit, wsum, th);
        const int rm = block_scan(miss, wsum, tm);
        if (hit) {
            touched[sl] = 1;
            tslot[nh + rh] = sl;
            town[nh + rh] = (int32_t)(lbase + e);
        }
        if (miss) {
            missl[nm + rm] = e;
            score_p[nm + rm] = base == 0 ? lfru_score(freq0, dlast0, now)
                                         : lfru_score(p.freq[lbase + e], p.dlast[lbase + e], now);
        }
        nh += th;
        nm += tm;
    }
    __syncthreads();

    // Candidates: the first nm entries of the LRU order that this call has
    // not used and that are not pinned, with their owners' scores (-1: the
    // owner is never protected).
    int nv = 0;
    for (int base = 0; nv < nm && base < S; base += kThreads) {
        const int i = base + tid;
        int sl = -1, o = -1;
        bool f = false;
        int64_t sc = -1;
        if (i < S) {
            order_at(base, i, sl, o);
            const uint32_t st = base == 0 ? stamp0 : p.stamp[sl];
            f = touched[sl] == 0 && !(st != 0u && st >= latest_demand);
            if (f) {
                if (base == 0) {
                    o = o00;
                    if (o >= 0 && ofreq0 >= 2) sc = lfru_score(ofreq0, odlast0, now);
                } else {
                    if (!p.pairs) o = p.own[sl];
                    if (o >= 0) {
                        const int64_t fq = p.freq[o];
                        if (fq >= 2) sc = lfru_score(fq, p.dlast[o], now);
                    }
                }
            }
        }
        int tot;
        const int r = block_scan(f, wsum, tot);
        if (f && nv + r < nm) {
            vslot[nv + r] = sl;
            vown[nv + r] = o;
            score_v[nv + r] = sc;
        }
        nv = min(nm, nv + tot);
    }
    __syncthreads();

    // Guard decisions: a prediction takes the current victim unless the
    // victim's owner is protected against it (at least 2 demand accesses
    // and 4 * score > 5 * prediction's score + 16, i.e. hotter by 25% + 4).
    if (wave == 0) {
        int cur = 0, k = 0, nf = 0;
        while (k < nm && cur < nv) {
            const int kk = k + lane;
            const int64_t sv = score_v[cur];
            const bool take = kk < nm && !(sv >= 0 && 4 * sv > 5 * score_p[kk] + 16);
            const uint64_t m = __ballot(take);
            if (m == 0ull) {
                k += kWave;
                continue;
            }
            const int first = __ffsll((unsigned long long)m) - 1;
            if (lane == 0) {
                fslot[nf] = vslot[cur];
                fold[nf] = vown[cur];
                fexp[nf] = missl[k + first];
            }
            ++nf;
            ++cur;
            k += first + 1;
        }
        if (lane == 0) misc[0] = nf;
    }
    __syncthreads();
    const int nf = misc[0];
    for (int j = tid; j < nf; j += kThreads) {
        touched[fslot[j]] = 1;
        tslot[nh + j] = fslot[j];
        town[nh + j] = (int32_t)(lbase + fexp[j]);
    }
    __syncthreads();

    // The used slots in ascending slot order (distinct slots: rank = number
    // of smaller ones), into the candidate arrays, which are free now.
    const int nt = nh + nf;
    for (int t = tid; t < nt; t += kThreads) {
        const int s = tslot[t];
        int rank = 0;
        for (int u = 0; u < nt; ++u) rank += tslot[u] < s;
        vslot[rank] = s;
        vown[rank] = town[t];
    }
    __syncthreads();

    // ---- final phase: every write to the persistent state.
    for (int t = tid; t < nh; t += kThreads) p.stamp[tslot[t]] = now;
    for (int j = tid; j < nf; j += kThreads) {
        const int s = fslot[j], o = fold[j], e = fexp[j];
        if (o >= 0) p.res[o] = -1;
        p.own[s] = (int32_t)(lbase + e);
        p.res[lbase + e] = s;
        p.stamp[s] = now;
        p.fill_slot[j] = s;
        p.fill_expert[j] = e;
    }
    if (nt > 0) {
        int w = 0;
        for (int base = 0; base < S; base += kThreads) {
            const int i = base + tid;
            int s = -1, o = -1;
            if (i < S) order_at(base, i, s, o);
            const bool f = i < S && touched[s] == 0;
            int tot;
            const int r = block_scan(f, wsum, tot);
            if (f) {
                if (p.pairs) reinterpret_cast<int2 *>(p.order)[w + r] = make_int2(s, o);
                else p.order[w + r] = s;
            }
            w += tot;
        }
        for (int t = tid; t < nt; t += kThreads) {
            if (p.pairs) reinterpret_cast<int2 *>(p.order)[w + t] = make_int2(vslot[t], vown[t]);
            else p.order[w + t] = vslot[t];
        }
    }
    if (tid == 0) {
        int64_t *st = p.stats + (int64_t)p.layer * MOE_NUM_STATS;
        st[MOE_STAT_PF_CALLS] += 1;
        st[MOE_STAT_PF_FILLED] += nf;
        st[MOE_STAT_PF_DROPPED] += nm - nf;
        p.clock[0] = now;
        p.n_fill[0] = nf;
    }
}

}  // namespace

size_t prefetch_lds_bytes(int M, int E, int S) {
    const size_t b = (32 + 16) * 4 + 16 * (size_t)M + 32 * (size_t)M + (size_t)E + (size_t)S;
    return (b + 15) & ~(size_t)15;
}

hipError_t prefetch_prepare(size_t lds_bytes) {
    if (lds_bytes <= 65536) return hipSuccess;
    return hipFuncSetAttribute(reinterpret_cast<const void *>(&prefetch_kernel),
                               hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds_bytes);
}

hipError_t launch_prefetch(const PrefetchParams &p, hipStream_t s) {
    if (p.M < std::min(p.n, p.E)) return hipErrorInvalidValue;
    if (rec::on())
        return rec::launch("prefetch_kernel", s,
                           {{p.ids, rec::kRead}, {p.res, rec::kReadWrite}, {p.fill_slot, rec::kWrite}});
    const size_t lds = prefetch_lds_bytes(p.M, p.E, p.S);
    hipLaunchKernelGGL(prefetch_kernel, dim3(1), dim3(kThreads), lds, s, p);
    return hipGetLastError();
}

}  // namespace moe
