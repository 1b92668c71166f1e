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
    const uint32_t now = p.clock[0] + 1u;
    const uint32_t latest_demand = p.clock[1];

    for (int e = tid; e < E; e += kThreads) want[e] = 0;
    for (int s = tid; s < S; s += kThreads) touched[s] = 0;
    __syncthreads();
    for (int i = tid; i < p.n; i += kThreads) {
        const int e = p.ids[i];
        if (e >= 0 && e < E) want[e] = 1;
    }
    __syncthreads();

    // Hits (used now) and missing predictions, both ascending.
    int nh = 0, nm = 0;
    for (int base = 0; base < E; base += kThreads) {
        const int e = base + tid;
        const bool w = e < E && want[e] != 0;
        const int s = w ? p.res[lbase + e] : -1;
        const bool hit = w && s >= 0, miss = w && s < 0;
        int th, tm;
        const int rh = block_scan(hit, wsum, th);
        const int rm = block_scan(miss, wsum, tm);
        if (hit) {
            touched[s] = 1;
            tslot[nh + rh] = s;
            town[nh + rh] = (int32_t)(lbase + e);
        }
        if (miss) missl[nm + rm] = e;
        nh += th;
        nm += tm;
    }
    __syncthreads();

    // Candidates: the first nm entries of the LRU order that this call has
    // not used and that are not pinned.
    int nv = 0;
    for (int base = 0; nv < nm && base < S; base += kThreads) {
        const int i = base + tid;
        int s = -1, o = -1;
        bool f = false;
        if (i < S) {
            if (p.pairs) {
                const int2 v = reinterpret_cast<const int2 *>(p.order)[i];
                s = v.x;
                o = v.y;
            } else {
                s = p.order[i];
            }
            const uint32_t st = p.stamp[s];
            f = touched[s] == 0 && !(st != 0u && st >= latest_demand);
            if (f && !p.pairs) o = p.own[s];
        }
        int tot;
        const int r = block_scan(f, wsum, tot);
        if (f && nv + r < nm) {
            vslot[nv + r] = s;
            vown[nv + r] = o;
        }
        nv = min(nm, nv + tot);
    }
    __syncthreads();

    // Heat of the candidates' owners and of the missing predictions.
    for (int j = tid; j < nv; j += kThreads) {
        const int o = vown[j];
        int64_t sc = -1;
        if (o >= 0) {
            const int64_t f = p.freq[o];
            if (f >= 2) sc = lfru_score(f, p.dlast[o], now);
        }
        score_v[j] = sc;
    }
    for (int k = tid; k < nm; k += kThreads) {
        const int64_t x = lbase + missl[k];
        score_p[k] = lfru_score(p.freq[x], p.dlast[x], now);
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
            if (i < S) {
                if (p.pairs) {
                    const int2 v = reinterpret_cast<const int2 *>(p.order)[i];
                    s = v.x;
                    o = v.y;
                } else {
                    s = p.order[i];
                }
            }
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
