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
#include "moe_internal.h"

namespace moe {
namespace {

constexpr int kThreads = 1024;
constexpr int kWaves = kThreads / kWave;

// Exclusive prefix count of `f` over the workgroup; `total` gets the sum.
// Every thread must call it: it holds two barriers.
__device__ __forceinline__ int block_scan(bool f, int32_t *wsum, int &total) {
    const int lane = threadIdx.x & (kWave - 1);
    const int wave = threadIdx.x / kWave;
    const uint64_t m = __ballot(f);
    const int pre = __builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32),
                                              __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0u));
    if (lane == 0) wsum[wave] = __popcll(m);
    __syncthreads();
    int off = 0, tot = 0;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) {
        const int v = wsum[w];
        off += (w < wave) ? v : 0;
        tot += v;
    }
    __syncthreads();
    total = tot;
    return off + pre;
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

    const int tid = threadIdx.x;
    const int64_t lbase = (int64_t)p.layer * E;

    for (int i = tid; i < E; i += kThreads) cnt[i] = 0;
    for (int i = tid; i < S; i += kThreads) touched[i] = 0;
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
        p.ids[i] = (e >= 0 && e < E) ? slotof[e] : -1;
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
        p.n_miss[0] = nplan;
    }
}

}  // namespace

size_t admit_lds_bytes(int E, int S, int max_routes) {
    size_t words = 32 + 8 + 5 * (size_t)E + (size_t)max_routes;
    return words * 4 + (((size_t)S + 15) & ~(size_t)15);
}

hipError_t admit_prepare(size_t lds_bytes) {
    if (lds_bytes <= 65536) return hipSuccess;
    return hipFuncSetAttribute(reinterpret_cast<const void *>(&admit_kernel),
                               hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds_bytes);
}

hipError_t launch_admit(const AdmitParams &p, size_t lds_bytes, hipStream_t s) {
    hipLaunchKernelGGL(admit_kernel, dim3(1), dim3(kThreads), lds_bytes, s, p);
    return hipGetLastError();
}

}  // namespace moe
