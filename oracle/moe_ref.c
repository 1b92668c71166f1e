/*
 * moe_ref.c -- the CPU oracle for one offloaded MoE decode layer step.
 *
 * TEST INFRASTRUCTURE ONLY.  This file is the slow, plain, obviously
 * correct reference that the HIP library is checked against.  Only the
 * tests, the smoke check and the CPU-baseline leg of the benchmark may
 * load it.  It shares no code, header, table or constant with the HIP
 * path and includes nothing from it.
 *
 * Sources (web pages; cited by title and section):
 *   [P1] FreeToken PR #491, "refactor(moe): extract hybrid decode
 *        orchestration": sections 4 (how decode works) and 5 (how routes
 *        are split) -- the slot-id-or-minus-one contract.
 *   [P2] FreeToken issue #753, "[Perf] Offloaded decode: overlap the
 *        expert-miss gather with the same layer's shared expert ...":
 *        sections "Problem in upstream today" and "What we changed" --
 *        router, shared expert with a sigmoid gate, routed experts,
 *        routed + shared; admission writes the miss plan, the gather
 *        copies slot bytes.
 *   [P3] FreeToken PR #680, "fix(moe): admit a wide offloaded decode
 *        step's experts 128 at a time": sections Solution and Tests --
 *        one-call width, sorted fixed-length distinct list in query-width
 *        chunks, statistics counted once per step, histogram per route.
 *   [P4] llama.cpp fork PR #126, "cuda : MoE look-ahead expert prefetch
 *        ...": sections Consumer and Eviction guard -- expert ids outside
 *        [0, n_experts) are ignored; speculative fills through the LRU
 *        victim order, pinned slots never chosen, and the LFRU guard.
 *
 * Precision: every floating-point result is computed in double.  Inputs
 * are the stored formats (bf16, e2m1 nibbles, e4m3 scales, fp32 logits
 * and globals) decoded exactly.  Nothing is rounded between the two
 * projections; the GPU's intermediate bf16 rounding is covered by the
 * parity tolerance.
 *
 * Build: gcc -O2 -std=c99 -shared -fPIC moe_ref.c -o libmoe_ref.so -lm
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

/* ------------------------------------------------------------------ */
/* Stored-format decoders (exact).                                     */
/* ------------------------------------------------------------------ */

/* bfloat16: the upper 16 bits of an IEEE binary32. */
double ref_bf16_to_double(uint16_t b)
{
    uint32_t u = ((uint32_t)b) << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return (double)f;
}

/* OCP FP8 E4M3 ("fn" variant): 1 sign, 4 exponent (bias 7), 3 mantissa
 * bits; exponent 0 is subnormal; S.1111.111 is NaN; no infinities. */
double ref_e4m3_to_double(uint8_t v)
{
    int sign = (v >> 7) & 1;
    int ex = (v >> 3) & 0xF;
    int man = v & 7;
    double mag;
    if (ex == 0xF && man == 7)
        return NAN;
    if (ex == 0)
        mag = ldexp((double)man / 8.0, -6);
    else
        mag = ldexp(1.0 + (double)man / 8.0, ex - 7);
    return sign ? -mag : mag;
}

/* OCP FP4 E2M1: 1 sign, 2 exponent (bias 1), 1 mantissa bit; exponent 0
 * is subnormal (0 or 0.5). */
double ref_e2m1_to_double(uint8_t nib)
{
    int sign = (nib >> 3) & 1;
    int ex = (nib >> 1) & 3;
    int man = nib & 1;
    double mag;
    if (ex == 0)
        mag = 0.5 * (double)man;
    else
        mag = ldexp(1.0 + 0.5 * (double)man, ex - 1);
    return sign ? -mag : mag;
}

/* OCP MX E8M0 scale (the MX formats' shared block scale): an unsigned
 * biased exponent, value 2^(v - 127); v = 255 is NaN; no sign, no
 * mantissa, no zero. */
double ref_e8m0_to_double(uint8_t v)
{
    if (v == 0xFF)
        return NAN;
    return ldexp(1.0, (int)v - 127);
}

/* ------------------------------------------------------------------ */
/* Expert weight access.                                               */
/*                                                                     */
/* One expert "row" of a weight pool is split over banks; each bank is */
/* an array of rows, and row r of bank b starts at banks[b] + r*rb[b]. */
/* Format 0 (bf16), two banks:                                         */
/*   bank0: w13 [2F][H] bf16  (rows 0..F-1 gate, rows F..2F-1 up)      */
/*   bank1: w2  [H][F]  bf16                                           */
/* Format 1 (e2m1 with e4m3 scales per 16 and an fp32 global), six     */
/* banks:                                                              */
/*   bank0: w13 codes  [2F][H/2]   element c in byte c/2, even c low   */
/*   bank1: w13 scales [2F][H/16]  e4m3, one per 16 consecutive c      */
/*   bank2: w13 global fp32                                            */
/*   bank3: w2 codes   [H][F/2]                                        */
/*   bank4: w2 scales  [H][F/16]                                       */
/*   bank5: w2 global  fp32                                            */
/* Format 2 (MXFP4: e2m1 with one e8m0 scale per 32 consecutive        */
/* elements of a row, the OCP MX block), four banks:                   */
/*   bank0: w13 codes  [2F][H/2]   element c in byte c/2, even c low   */
/*   bank1: w13 scales [2F][H/32]  e8m0, one per 32 consecutive c      */
/*   bank2: w2 codes   [H][F/2]                                        */
/*   bank3: w2 scales  [H][F/32]                                       */
/* ------------------------------------------------------------------ */

typedef struct {
    int fmt;                 /* 0 = bf16, 1 = e2m1/e4m3/fp32, 2 = mxfp4 */
    int H, F;
    const uint8_t *bank[6];
    int64_t rb[6];           /* bytes per row in each bank */
} ref_pool;

static double ref_fp32_at(const uint8_t *p)
{
    float f;
    memcpy(&f, p, sizeof f);
    return (double)f;
}

/* Element (r, c) of matrix m (0 = w13 [2F][H], 1 = w2 [H][F]) of the
 * expert stored at pool row `row`. */
static double ref_weight(const ref_pool *p, int64_t row, int m, int64_t r, int64_t c)
{
    int64_t ncol = (m == 0) ? p->H : p->F;
    if (p->fmt == 0) {
        const uint8_t *base = p->bank[m] + row * p->rb[m];
        uint16_t b;
        memcpy(&b, base + 2 * (r * ncol + c), 2);
        return ref_bf16_to_double(b);
    } else if (p->fmt == 2) {
        int b0 = 2 * m;
        const uint8_t *codes = p->bank[b0] + row * p->rb[b0];
        const uint8_t *scales = p->bank[b0 + 1] + row * p->rb[b0 + 1];
        uint8_t byte = codes[r * (ncol / 2) + c / 2];
        uint8_t nib = (c % 2 == 0) ? (byte & 0xF) : (byte >> 4);
        uint8_t sc = scales[r * (ncol / 32) + c / 32];
        return ref_e2m1_to_double(nib) * ref_e8m0_to_double(sc);
    } else {
        int b0 = 3 * m;
        const uint8_t *codes = p->bank[b0] + row * p->rb[b0];
        const uint8_t *scales = p->bank[b0 + 1] + row * p->rb[b0 + 1];
        const uint8_t *glob = p->bank[b0 + 2] + row * p->rb[b0 + 2];
        uint8_t byte = codes[r * (ncol / 2) + c / 2];
        uint8_t nib = (c % 2 == 0) ? (byte & 0xF) : (byte >> 4);
        uint8_t sc = scales[r * (ncol / 16) + c / 16];
        return ref_e2m1_to_double(nib) * ref_e4m3_to_double(sc) * ref_fp32_at(glob);
    }
}

static double ref_silu(double g) { return g / (1.0 + exp(-g)); }

/* One SwiGLU expert applied to one token ([P2] "Problem in upstream
 * today": the routed and shared experts are gated FFNs):
 *   g_j = sum_c W13[j][c] x_c,  u_j = sum_c W13[F+j][c] x_c,
 *   h_j = silu(g_j) * u_j,      d_i = sum_j W2[i][j] h_j. */
static void ref_expert(const ref_pool *p, int64_t row, const uint16_t *x, double *d)
{
    int H = p->H, F = p->F;
    double *h = (double *)malloc(sizeof(double) * (size_t)F);
    for (int j = 0; j < F; j++) {
        double g = 0.0, u = 0.0;
        for (int c = 0; c < H; c++) {
            double xc = ref_bf16_to_double(x[c]);
            g += ref_weight(p, row, 0, j, c) * xc;
            u += ref_weight(p, row, 0, F + j, c) * xc;
        }
        h[j] = ref_silu(g) * u;
    }
    for (int i = 0; i < H; i++) {
        double acc = 0.0;
        for (int j = 0; j < F; j++)
            acc += ref_weight(p, row, 1, i, j) * h[j];
        d[i] = acc;
    }
    free(h);
}

static void ref_pool_init(ref_pool *p, int fmt, int H, int F, const uint8_t *const *banks,
                          const int64_t *rb)
{
    int nb = fmt == 0 ? 2 : (fmt == 2 ? 4 : 6);
    memset(p, 0, sizeof *p);
    p->fmt = fmt;
    p->H = H;
    p->F = F;
    for (int b = 0; b < nb; b++) {
        p->bank[b] = banks[b];
        p->rb[b] = rb[b];
    }
}

/* Single expert, single token: d[H] = expert(row)(x). */
void ref_expert_ffn(int fmt, int H, int F, const uint8_t *const *banks, const int64_t *rb,
                    int64_t row, const uint16_t *x, double *d)
{
    ref_pool p;
    ref_pool_init(&p, fmt, H, F, banks, rb);
    ref_expert(&p, row, x, d);
}

/* Routed experts over pool rows ([P2] "What we changed": routed GEMM,
 * then routed + shared; [P1] section 5: a -1 route contributes nothing).
 *   out[t] = sum over k = 0..K-1 with idx[t][k] >= 0, in ascending k, of
 *            w[t][k] * expert(idx[t][k])(x[t])
 *          + addend[t]              (when addend is given)
 * idx holds pool rows: slot ids over a slot pool, or expert ids over a
 * whole layer's pool (the streamed layer). */
void ref_routed(int fmt, int H, int F, const uint8_t *const *banks, const int64_t *rb,
                int T, int K, const int32_t *idx, const double *w, const uint16_t *x,
                const double *addend, double *out)
{
    ref_pool p;
    double *d = (double *)malloc(sizeof(double) * (size_t)H);
    ref_pool_init(&p, fmt, H, F, banks, rb);
    for (int t = 0; t < T; t++) {
        double *o = out + (int64_t)t * H;
        for (int i = 0; i < H; i++)
            o[i] = 0.0;
        for (int k = 0; k < K; k++) {
            int32_t r = idx[(int64_t)t * K + k];
            if (r < 0)
                continue;
            ref_expert(&p, r, x + (int64_t)t * H, d);
            for (int i = 0; i < H; i++)
                o[i] += w[(int64_t)t * K + k] * d[i];
        }
        if (addend)
            for (int i = 0; i < H; i++)
                o[i] += addend[(int64_t)t * H + i];
    }
    free(d);
}

/* Gated shared expert ([P2] "Problem in upstream today": the shared
 * expert and its sigmoid gate run after the router):
 *   gamma[t] = sigmoid(sum_c x[t][c] * wg[c]),  out[t] = gamma[t] * shared(x[t]).
 * The shared expert is a bf16 SwiGLU with w13 [2F][H] and w2 [H][F]. */
void ref_shared(int H, int F, const uint8_t *w13, const uint8_t *w2, const uint16_t *wg,
                int T, const uint16_t *x, double *gamma, double *out)
{
    ref_pool p;
    const uint8_t *banks[2] = {w13, w2};
    int64_t rb[2] = {(int64_t)2 * F * H * 2, (int64_t)H * F * 2};
    ref_pool_init(&p, 0, H, F, banks, rb);
    for (int t = 0; t < T; t++) {
        const uint16_t *xt = x + (int64_t)t * H;
        double z = 0.0;
        for (int c = 0; c < H; c++)
            z += ref_bf16_to_double(xt[c]) * ref_bf16_to_double(wg[c]);
        double gm = 1.0 / (1.0 + exp(-z));
        ref_expert(&p, 0, xt, out + (int64_t)t * H);
        for (int i = 0; i < H; i++)
            out[(int64_t)t * H + i] *= gm;
        if (gamma)
            gamma[t] = gm;
    }
}

/* ------------------------------------------------------------------ */
/* Top-k routing ([P2] "What we changed": router, then fused top-k).   */
/* For each row: the K largest logits, largest first, equal logits     */
/* taken lower expert id first, NaN treated as -infinity.  Weights are */
/* the softmax over the K selected logits (softmax over all E, top-k,  */
/* then renormalising gives the same numbers: the common denominator   */
/* cancels).  If every selected logit is -infinity the K weights are   */
/* equal, 1/K (softmax of equal values).                               */
/* ------------------------------------------------------------------ */

static int ref_logit_before(float a, int ia, float b, int ib)
{
    double da = isnan(a) ? -INFINITY : (double)a;
    double db = isnan(b) ? -INFINITY : (double)b;
    if (da != db)
        return da > db;
    return ia < ib;
}

void ref_topk(int T, int E, int K, const float *logits, int32_t *ids, double *w)
{
    char *taken = (char *)malloc((size_t)E);
    double *sel = (double *)malloc(sizeof(double) * (size_t)K);
    for (int t = 0; t < T; t++) {
        const float *row = logits + (int64_t)t * E;
        memset(taken, 0, (size_t)E);
        for (int k = 0; k < K; k++) {
            int best = -1;
            for (int e = 0; e < E; e++) {
                if (taken[e])
                    continue;
                if (best < 0 || ref_logit_before(row[e], e, row[best], best))
                    best = e;
            }
            taken[best] = 1;
            ids[(int64_t)t * K + k] = best;
            sel[k] = isnan(row[best]) ? -INFINITY : (double)row[best];
        }
        double mx = sel[0];
        if (mx == -INFINITY) {
            for (int k = 0; k < K; k++)
                w[(int64_t)t * K + k] = 1.0 / K;
            continue;
        }
        double z = 0.0;
        for (int k = 0; k < K; k++)
            z += exp(sel[k] - mx);
        for (int k = 0; k < K; k++)
            w[(int64_t)t * K + k] = exp(sel[k] - mx) / z;
    }
    free(taken);
    free(sel);
}

/* ------------------------------------------------------------------ */
/* Slot-cache admission.                                               */
/*                                                                     */
/* State (all caller-owned arrays):                                    */
/*   res[L*E]   slot holding expert (l, e), or -1                      */
/*   own[S]     l*E + e held by the slot, or -1                        */
/*   stamp[S]   clock value of the slot's last use (0 = never)         */
/*   clock[1]   step counter, one tick per admission step              */
/*   stats[L*8] per layer: calls, met, missed, overflow, invalid,      */
/*              prefetch calls, prefetch fills, prefetch drops         */
/*   freq[L*E]  per layer, per expert: routes seen (demand only)       */
/*   dlast[L*E] clock value of the expert's last demand step (0 never) */
/*   last_demand[1] clock value of the latest demand step (0 none)     */
/*                                                                     */
/* One step admits the routes of one layer ([P3] Solution):            */
/*  - a step of at most one_call routes is one query over its routes;  */
/*  - a wider step is the ascending list of its distinct experts,      */
/*    padded to the fixed length min(R, E) with a sentinel, cut into   */
/*    queries of query_width; each query's victims are chosen before   */
/*    the next query runs, and slots used earlier in the step are not  */
/*    eligible, so no query evicts an earlier one's experts.           */
/* Within a query: hits are touched first; misses, ascending, take the */
/* least recently used eligible slots, ordered by (stamp, slot id).    */
/* A miss that finds no eligible slot, or comes after the step has     */
/* fetched max_fetch experts (max_fetch < 0: no cap), stays            */
/* non-resident.  Finally every route is rewritten in place to its     */
/* expert's slot, or -1 ([P1] sections 4-5).  Ids outside [0, E) are   */
/* invalid: they are ignored and rewritten to -1 ([P4] Consumer).      */
/* Statistics count a step once: its distinct valid experts (met),     */
/* the distinct experts each query found non-resident (missed), and    */
/* one call; the histogram counts every valid route ([P3] Solution).   */
/* The miss plan lists (slot, expert) in query order, ascending expert */
/* within a query; the gather copies exactly these rows.               */
/* ------------------------------------------------------------------ */

enum {
    REF_CALLS = 0, REF_MET = 1, REF_MISSED = 2, REF_OVERFLOW = 3, REF_INVALID = 4,
    REF_PF_CALLS = 5, REF_PF_FILLED = 6, REF_PF_DROPPED = 7, REF_NSTATS = 8
};

/* The widths of the queries a step of R routes over E experts is
 * admitted in.  Returns the number of queries written to out. */
int ref_query_widths(int R, int E, int one_call, int qw, int32_t *out)
{
    if (R <= 0)
        return 0;
    if (R <= one_call) {
        out[0] = R;
        return 1;
    }
    int len = R < E ? R : E;
    int n = 0;
    for (int start = 0; start < len; start += qw)
        out[n++] = (len - start < qw) ? (len - start) : qw;
    return n;
}

typedef struct {
    uint32_t stamp;
    int32_t slot;
} ref_victim;

static int ref_victim_cmp(const void *a, const void *b)
{
    const ref_victim *x = (const ref_victim *)a, *y = (const ref_victim *)b;
    if (x->stamp != y->stamp)
        return x->stamp < y->stamp ? -1 : 1;
    return x->slot < y->slot ? -1 : (x->slot > y->slot ? 1 : 0);
}

/* Returns 0 on success, -1 on a bad argument. */
int ref_admit(int L, int E, int S, int one_call, int qw, int32_t *res, int32_t *own,
              uint32_t *stamp, uint32_t *clock, int64_t *stats, int64_t *freq, uint32_t *dlast,
              uint32_t *last_demand, int layer, int32_t *ids, int R, int max_fetch,
              int32_t *plan_slot, int32_t *plan_expert, int32_t *n_miss)
{
    if (layer < 0 || layer >= L || R < 0 || E < 1 || S < 1 || one_call < 1 || qw < 1)
        return -1;
    int32_t *resl = res + (int64_t)layer * E;
    int64_t *st = stats + (int64_t)layer * REF_NSTATS;
    uint32_t now = ++(*clock);

    /* Histogram over every valid route; invalid routes counted.  The
     * step is a demand access of each of its valid experts. */
    for (int i = 0; i < R; i++) {
        if (ids[i] >= 0 && ids[i] < E) {
            freq[(int64_t)layer * E + ids[i]] += 1;
            dlast[(int64_t)layer * E + ids[i]] = now;
        } else {
            st[REF_INVALID] += 1;
        }
    }
    *last_demand = now;

    /* The queries, as lists of candidate ids (sentinel E = padding). */
    int nlist;
    int32_t *list;
    int32_t nq;
    int32_t *qlen = (int32_t *)malloc(sizeof(int32_t) * (size_t)(R + 1));
    if (R <= one_call) {
        nlist = R;
        list = (int32_t *)malloc(sizeof(int32_t) * (size_t)(R + 1));
        for (int i = 0; i < R; i++)
            list[i] = ids[i];
        nq = R > 0 ? 1 : 0;
        qlen[0] = R;
    } else {
        char *present = (char *)calloc((size_t)E, 1);
        for (int i = 0; i < R; i++)
            if (ids[i] >= 0 && ids[i] < E)
                present[ids[i]] = 1;
        nlist = R < E ? R : E;
        list = (int32_t *)malloc(sizeof(int32_t) * (size_t)nlist);
        int n = 0;
        for (int e = 0; e < E; e++)
            if (present[e])
                list[n++] = e;
        while (n < nlist)
            list[n++] = E; /* sentinel */
        free(present);
        nq = ref_query_widths(R, E, one_call, qw, qlen);
    }

    char *inq = (char *)malloc((size_t)E);
    int32_t *dq = (int32_t *)malloc(sizeof(int32_t) * (size_t)E);
    int32_t *miss = (int32_t *)malloc(sizeof(int32_t) * (size_t)E);
    ref_victim *vict = (ref_victim *)malloc(sizeof(ref_victim) * (size_t)S);
    int fetched = 0, nplan = 0, pos = 0;

    for (int q = 0; q < nq; q++) {
        /* Ascending distinct valid ids of this query. */
        memset(inq, 0, (size_t)E);
        for (int i = pos; i < pos + qlen[q]; i++)
            if (list[i] >= 0 && list[i] < E)
                inq[list[i]] = 1;
        pos += qlen[q];
        int nd = 0;
        for (int e = 0; e < E; e++)
            if (inq[e])
                dq[nd++] = e;
        st[REF_MET] += nd;

        /* Hits are used now. */
        int nm = 0;
        for (int i = 0; i < nd; i++) {
            int32_t s = resl[dq[i]];
            if (s >= 0)
                stamp[s] = now;
            else
                miss[nm++] = dq[i];
        }
        st[REF_MISSED] += nm;

        /* Eligible victims: every slot not used in this step, least
         * recently used first, lower slot id first among equals. */
        int nv = 0;
        for (int s = 0; s < S; s++)
            if (stamp[s] < now) {
                vict[nv].stamp = stamp[s];
                vict[nv].slot = s;
                nv++;
            }
        qsort(vict, (size_t)nv, sizeof(ref_victim), ref_victim_cmp);

        for (int j = 0; j < nm; j++) {
            int e = miss[j];
            if (j >= nv || (max_fetch >= 0 && fetched >= max_fetch)) {
                st[REF_OVERFLOW] += 1;
                continue;
            }
            int32_t s = vict[j].slot;
            if (own[s] >= 0)
                res[own[s]] = -1;
            own[s] = layer * E + e;
            resl[e] = s;
            stamp[s] = now;
            plan_slot[nplan] = s;
            plan_expert[nplan] = e;
            nplan++;
            fetched++;
        }
    }
    st[REF_CALLS] += 1;

    /* Rewrite in place: slot id, or -1. */
    for (int i = 0; i < R; i++) {
        int32_t e = ids[i];
        ids[i] = (e >= 0 && e < E) ? resl[e] : -1;
    }
    *n_miss = nplan;

    free(list);
    free(qlen);
    free(inq);
    free(dq);
    free(miss);
    free(vict);
    return 0;
}

/* ------------------------------------------------------------------ */
/* Look-ahead prefetch with the LFRU eviction guard ([P4] Consumer,    */
/* Eviction guard).  One call fills a layer's predicted experts ahead  */
/* of its demand step, through the same LRU victim order:              */
/*  - ids outside [0, E) are ignored; the rest are taken once each,    */
/*    ascending;                                                       */
/*  - a predicted expert already resident is used now (its slot's      */
/*    stamp takes this call's clock value), so no fill of the same     */
/*    call evicts it;                                                  */
/*  - victims are the slots not used in this call and not pinned,      */
/*    least recently used first, lower slot id first among equals.  A  */
/*    slot is pinned when it was used at or after the latest demand    */
/*    step (its readers may still run, and fills made since then are   */
/*    still being copied);                                             */
/*  - each missing prediction, ascending, looks at the next victim.    */
/*    The victim's owner is protected when it has at least 2 demand    */
/*    accesses and its score exceeds 1.25 x the prediction's score + 4 */
/*    (score = demand frequency x 256 + recency byte, the byte being   */
/*    255 - min(255, clock - last demand), 0 if never demanded).  A    */
/*    protected owner stays and the prediction is dropped (the next    */
/*    prediction looks at the same victim); otherwise the prediction   */
/*    takes the slot;                                                  */
/*  - heat (freq, dlast) counts demand accesses only: prefetch reads   */
/*    it and never writes it.                                          */
/* The fill plan lists (slot, expert) in ascending expert order.       */
/* ------------------------------------------------------------------ */

static int64_t ref_lfru_score(const int64_t *freq, const uint32_t *dlast, int64_t x, uint32_t now)
{
    int64_t rec = 0;
    if (dlast[x] != 0) {
        uint32_t age = now - dlast[x];
        rec = 255 - (age < 255 ? (int64_t)age : 255);
    }
    return freq[x] * 256 + rec;
}

/* Returns 0 on success, -1 on a bad argument. */
int ref_prefetch(int L, int E, int S, int32_t *res, int32_t *own, uint32_t *stamp,
                 uint32_t *clock, const uint32_t *last_demand, int64_t *stats,
                 const int64_t *freq, const uint32_t *dlast, int layer, const int32_t *ids, int n,
                 int32_t *plan_slot, int32_t *plan_expert, int32_t *n_fill)
{
    if (layer < 0 || layer >= L || n < 0 || E < 1 || S < 1)
        return -1;
    *n_fill = 0;
    if (n == 0)   /* width 0: nothing happens, not even a call */
        return 0;
    int64_t lbase = (int64_t)layer * E;
    int64_t *st = stats + (int64_t)layer * REF_NSTATS;
    uint32_t now = ++(*clock);
    uint32_t ld = *last_demand;

    char *want = (char *)calloc((size_t)E, 1);
    for (int i = 0; i < n; i++)
        if (ids[i] >= 0 && ids[i] < E)
            want[ids[i]] = 1;

    /* Predicted experts already resident are used now. */
    for (int e = 0; e < E; e++)
        if (want[e] && res[lbase + e] >= 0)
            stamp[res[lbase + e]] = now;

    ref_victim *vict = (ref_victim *)malloc(sizeof(ref_victim) * (size_t)S);
    int nv = 0;
    for (int s = 0; s < S; s++) {
        int pinned = stamp[s] != 0 && stamp[s] >= ld;
        if (stamp[s] < now && !pinned) {
            vict[nv].stamp = stamp[s];
            vict[nv].slot = s;
            nv++;
        }
    }
    qsort(vict, (size_t)nv, sizeof(ref_victim), ref_victim_cmp);

    int cursor = 0, nfill = 0;
    for (int e = 0; e < E; e++) {
        if (!want[e] || res[lbase + e] >= 0)
            continue;
        if (cursor >= nv) {
            st[REF_PF_DROPPED] += 1;
            continue;
        }
        int32_t s = vict[cursor].slot;
        int32_t o = own[s];
        if (o >= 0 && freq[o] >= 2) {
            int64_t so = ref_lfru_score(freq, dlast, o, now);
            int64_t sp = ref_lfru_score(freq, dlast, lbase + e, now);
            if (4 * so > 5 * sp + 16) {   /* so > 1.25 sp + 4 */
                st[REF_PF_DROPPED] += 1;
                continue;
            }
        }
        if (o >= 0)
            res[o] = -1;
        own[s] = (int32_t)(lbase + e);
        res[lbase + e] = s;
        stamp[s] = now;
        plan_slot[nfill] = s;
        plan_expert[nfill] = e;
        nfill++;
        cursor++;
    }
    st[REF_PF_FILLED] += nfill;
    st[REF_PF_CALLS] += 1;
    *n_fill = nfill;

    free(want);
    free(vict);
    return 0;
}

/* The miss gather ([P2] "What we changed": the side stream reads the
 * plan and writes slot bytes): for every plan entry, every bank's row of
 * (layer, expert) in the host store is copied to the bank's slot row.
 * host[b] points at the layer's rows [E][rb[b]]; slots[b] at [S][rb[b]]. */
void ref_gather(int nb, const int64_t *rb, const uint8_t *const *host, uint8_t *const *slots,
                const int32_t *plan_slot, const int32_t *plan_expert, int n_miss)
{
    for (int i = 0; i < n_miss; i++)
        for (int b = 0; b < nb; b++)
            memcpy(slots[b] + (int64_t)plan_slot[i] * rb[b],
                   host[b] + (int64_t)plan_expert[i] * rb[b], (size_t)rb[b]);
}
