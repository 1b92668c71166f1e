/*
 * moe_cache.h -- C ABI of the MI355X (gfx950) offloaded MoE decode step.
 *
 * One layer's decode step over an expert slot cache:
 *   (1) top-k routing, (2) LRU slot-cache admission, (3) the miss gather
 *   from pinned host memory into device slots, (4) the routed expert
 *   GEMV / grouped GEMM over slot ids, (5) the gated shared expert and the
 *   final combine.
 *
 * Sources (web pages, cited by title and section):
 *   [P1] FreeToken PR #491, "refactor(moe): extract hybrid decode
 *        orchestration", sections 4-5: routes rewritten in place to a GPU
 *        slot id or -1; a -1 route contributes nothing to the GPU part.
 *   [P2] FreeToken issue #753, "[Perf] Offloaded decode: overlap the
 *        expert-miss gather with the same layer's shared expert,
 *        event-ordered inside the CUDA graph", sections "Problem in
 *        upstream today" and "What we changed": router -> top-k ->
 *        admission -> record(ready) -> shared expert + gate -> wait(done)
 *        -> routed GEMM -> routed + shared on the compute stream; the side
 *        stream waits for ready, gathers the misses, records done; one
 *        writer of the slot map; side stream and events made at cache
 *        construction, before any capture; device-side miss counts.
 *   [P3] FreeToken PR #680, "fix(moe): admit a wide offloaded decode
 *        step's experts 128 at a time", section Solution: load_experts
 *        returns slot ids; one-call width 256; wider steps admitted as
 *        a sorted fixed-length distinct-expert list in 128-wide queries,
 *        no host sync; statistics once per step, histogram per route.
 *   [P4] llama.cpp fork PR #126, "cuda : MoE look-ahead expert prefetch
 *        (PR-A consumer) + LFRU eviction guard", sections Consumer and
 *        Eviction guard: expert ids outside [0, n_experts) are ignored;
 *        predicted experts are filled ahead of their layer through the
 *        same victim order, never into a pinned slot, without a compute
 *        stream wait; a warm resident is protected by the LFRU guard.
 *
 * Conventions for every entry point:
 *   - Pointers named *_dev are device pointers (hipMalloc / torch cuda
 *     tensors); pointers named *_host are host pointers.  `stream` is a
 *     hipStream_t passed as void*; NULL is the null stream.
 *   - Calls that launch work are asynchronous and capturable in a
 *     hipGraph: they check their arguments on the host only, never
 *     synchronise and never allocate.  Data conditions found on the
 *     device (invalid ids, misses with no slot) never fail a call.
 *   - Every call returns a moe_status_t; the message of the last failure
 *     on the calling thread is moe_last_error().  Nothing throws.
 *   - A cache has one writer: moe_admit and moe_layer_decode on one cache
 *     must be issued from one thread, on one compute stream.
 */
#ifndef MOE_CACHE_H
#define MOE_CACHE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    MOE_OK = 0,
    MOE_INVALID_ARG = 1,   /* a bad pointer, size, index or flag        */
    MOE_UNSUPPORTED = 2,   /* a shape or alignment the kernels lack     */
    MOE_HIP_ERROR = 3,     /* a HIP runtime call failed                 */
    MOE_OUT_OF_MEMORY = 4  /* the cache's own device state did not fit  */
} moe_status_t;

/* Expert weight formats.
 * MOE_FMT_BF16, two banks per expert row:
 *   bank 0: w13 [2F][H] bf16, rows 0..F-1 the gate projection, rows
 *           F..2F-1 the up projection;          row bytes 4*F*H
 *   bank 1: w2  [H][F]  bf16 (down projection); row bytes 2*H*F
 * MOE_FMT_E2M1, six banks per expert row (4-bit OCP E2M1 values, one OCP
 * E4M3 scale per 16 consecutive elements of a row, one fp32 global scale
 * per matrix; element c of a row sits in byte c/2, even c in the low
 * nibble):
 *   bank 0: w13 codes  [2F][H/2]    bank 3: w2 codes  [H][F/2]
 *   bank 1: w13 scales [2F][H/16]   bank 4: w2 scales [H][F/16]
 *   bank 2: w13 global fp32         bank 5: w2 global fp32
 * A weight is code * scale * global.
 * MOE_FMT_MXFP4, four banks per expert row (OCP MX FP4: E2M1 values with
 * one E8M0 scale, 2^(s - 127), per 32 consecutive elements of a row; code
 * layout as above):
 *   bank 0: w13 codes  [2F][H/2]    bank 2: w2 codes  [H][F/2]
 *   bank 1: w13 scales [2F][H/32]   bank 3: w2 scales [H][F/32]
 * A weight is code * 2^(s - 127). */
enum { MOE_FMT_BF16 = 0, MOE_FMT_E2M1 = 1, MOE_FMT_MXFP4 = 2 };
#define MOE_MAX_BANKS 6

/* Statistics slots, per layer (int64 each) [P3 Solution]. */
enum {
    MOE_STAT_CALLS = 0,    /* admission steps                                  */
    MOE_STAT_MET = 1,      /* distinct valid experts of each step              */
    MOE_STAT_MISSED = 2,   /* distinct experts a query found non-resident      */
    MOE_STAT_OVERFLOW = 3, /* misses left without a slot (cap or no victim)    */
    MOE_STAT_INVALID = 4,  /* routes whose id is outside [0, E)                */
    MOE_STAT_PF_CALLS = 5,   /* prefetch calls of width > 0 [P4]               */
    MOE_STAT_PF_FILLED = 6,  /* predicted experts filled by a prefetch         */
    MOE_STAT_PF_DROPPED = 7, /* predictions dropped (guard, or no victim)      */
    MOE_NUM_STATS = 8
};

typedef struct moe_cache moe_cache_t;

typedef struct {
    int32_t num_layers;       /* L >= 1                                         */
    int32_t num_experts;      /* E >= 1, routed experts per layer               */
    int32_t num_slots;        /* S >= 1, device slots shared by all layers      */
    int32_t hidden;           /* H                                              */
    int32_t ffn;              /* F, routed expert width                         */
    int32_t weight_format;    /* MOE_FMT_*                                      */
    int32_t one_call_width;   /* steps of <= this many routes are one query (256) */
    int32_t query_width;      /* wider steps: distinct experts this many at a time (128) */
    int32_t max_routes;       /* upper bound on routes per admission step       */
    int32_t max_tokens;       /* upper bound on T for moe_layer_decode (0: no layer calls) */
    int32_t max_top_k;        /* upper bound on K for moe_layer_decode          */
    int32_t overlap;          /* schedule of moe_layer_decode:
                                 0: serial on the compute stream [P2];
                                 1: gather on the library's side stream, forked
                                    and joined by events around the shared
                                    expert and the resident routes [P2];
                                 2: one stream, two launches: the gather, the
                                    shared expert and the resident routes run
                                    as disjoint workgroups of one kernel, the
                                    down projections and combine in a second
                                    (single-token steps of any format at the
                                    supported widths; other steps run as 0);
                                 3: the split of the #678 variant [P2 "What we
                                    changed", difference from #678]: the
                                    shared expert and its gate on the side
                                    stream, forked at the start of the step;
                                    the gather and every routed launch on the
                                    compute stream, joined before the launch
                                    that adds the shared term.
                                 Results are bit-identical in all four.
                                 Other values are an error. */
    int32_t num_banks;        /* 0 (admission only: no gather, no experts) or
                                 the format's bank count (2 or 6)                */
    int32_t gather_workgroups;/* workgroups of the gather kernel; 0 = default   */
    /* host_banks_host[l * num_banks + b]: pinned host pointer (hipHostMalloc /
       pinned torch tensor) to layer l's rows of bank b, [E][row bytes].  The
       array is copied at create; the memory stays caller-owned and must
       outlive the cache.  Layers may share memory. */
    const void *const *host_banks_host;
    /* slot_banks_dev[b]: device pointer to bank b of the slot pool,
       [S][row bytes], caller-owned, 16-byte aligned. */
    void *slot_banks_dev[MOE_MAX_BANKS];
} moe_cache_desc_t;

/* A weight pool the routed kernels read: slot banks of a cache, or a whole
 * layer's experts in device memory (the "streamed" layer). */
typedef struct {
    int32_t weight_format;
    int32_t hidden;
    int32_t ffn;
    int32_t num_rows;                        /* rows in each bank              */
    const void *banks_dev[MOE_MAX_BANKS];    /* [num_rows][row bytes] each     */
} moe_pool_t;

/* The gated shared expert of a layer [P2 "Problem in upstream today"]:
 * a bf16 SwiGLU expert plus a [H] -> 1 sigmoid gate. */
typedef struct {
    int32_t ffn;              /* shared expert width; 0 = the routed F          */
    const void *w13_dev;      /* bf16 [2*ffn][H], gate rows then up rows        */
    const void *w2_dev;       /* bf16 [H][ffn]                                  */
    const void *gate_dev;     /* bf16 [H]                                       */
} moe_shared_t;

/* ---------------------------------------------------------------- helpers */

const char *moe_status_string(moe_status_t s);
/* Message of the last failed call on this thread ("" if none). */
const char *moe_last_error(void);

/* Bytes per row of each bank of a format; *num_banks_out gets 2 or 6. */
moe_status_t moe_bank_row_bytes(int32_t weight_format, int32_t hidden, int32_t ffn,
                                int64_t row_bytes_out[MOE_MAX_BANKS], int32_t *num_banks_out);

/* The widths of the queries one admission step of R routes over E experts
 * is cut into [P3 Solution]: {R} if R <= one_call_width, else the fixed
 * length min(R, E) cut into query_width pieces.  Writes at most `cap`
 * widths to out_host; *n_out gets the count. */
moe_status_t moe_query_widths(int32_t R, int32_t E, int32_t one_call_width, int32_t query_width,
                              int32_t *out_host, int32_t cap, int32_t *n_out);

/* ---------------------------------------------------------------- cache */

/* Validates the description, allocates the cache's device state (slot map,
 * slot owners, stamps, LRU order, clock, miss plan, statistics, histogram,
 * demand recency, prefetch fill plan, layer workspace), creates its side
 * stream, its prefetch stream and their events -- before any capture --
 * and leaves every slot empty.  Uses the current device.  A cache whose
 * full-width prefetch kernel would not fit the LDS is still created (only
 * moe_prefetch refuses).  The cache is not thread-safe: one caller issues
 * its calls, on one compute stream.  Errors: MOE_INVALID_ARG (bad sizes, null or unaligned
 * pointers, overlap outside 0..3), MOE_UNSUPPORTED (shapes the kernels lack,
 * LDS overflow), MOE_OUT_OF_MEMORY, MOE_HIP_ERROR. */
moe_status_t moe_cache_create(const moe_cache_desc_t *desc, moe_cache_t **out);

/* Switches the schedule of later moe_layer_decode calls (the `overlap`
 * field of the description; graphs captured before keep theirs).  Errors:
 * MOE_INVALID_ARG (overlap outside 0..3). */
moe_status_t moe_cache_set_schedule(moe_cache_t *cache, int32_t overlap);

/* Synchronises the device, stops the cache's host threads, and frees what
 * create and moe_cache_set_cpu_threads allocated. */
void moe_cache_destroy(moe_cache_t *cache);

/* The cache's slot banks as a pool for moe_routed_decode. */
moe_status_t moe_cache_pool(const moe_cache_t *cache, moe_pool_t *pool_out);

/* ---------------------------------------------------------------- the step */

/* (1) Top-k routing [P2 "What we changed": router, fused top-k].
 * logits_dev: fp32 [T][E] row-major.  For each row, the K largest logits,
 * largest first, equal logits lower expert id first, NaN as -infinity;
 * weights = softmax over the K selected logits (1/K each if all are
 * -infinity).  ids_dev: int32 [T][K]; w_dev: fp32 [T][K].
 * Errors: MOE_INVALID_ARG (T < 0, K < 1, K > E, K > 32, null pointers). */
moe_status_t moe_topk(const float *logits_dev, int32_t T, int32_t E, int32_t K,
                      int32_t *ids_dev, float *w_dev, void *stream);

/* (2) Admission of one layer step [P3 Solution; P1 sections 4-5].
 * ids_dev: int32 [R], expert ids in, rewritten in place to the slot now
 * holding each route's expert, or -1 (invalid id, or a miss left without
 * a slot).  One clock tick per call.  Steps of R <= one_call_width routes
 * are one query; wider steps are admitted as the ascending distinct
 * experts, padded to min(R, E), query_width at a time, and no query
 * evicts a slot used earlier in the step.  Within a query hits are used
 * first; misses, ascending, take the least recently used eligible slots
 * (ties: lower slot id).  max_fetch >= 0 caps the experts fetched this
 * step (first in plan order); < 0 is no cap.  Writes the miss plan
 * (slot, expert) and its length on the device for moe_gather_misses, and
 * the layer's statistics and histogram.  R may be 0 (an empty step).
 * Errors: MOE_INVALID_ARG (layer outside [0, L), R < 0 or R > max_routes,
 * null ids).  Launches one kernel on `stream`. */
moe_status_t moe_admit(moe_cache_t *cache, int32_t layer, int32_t *ids_dev, int32_t R,
                       int32_t max_fetch, void *stream);

/* (3) The miss gather [P2 "What we changed"].  Copies every bank's host row
 * of each plan entry of the last moe_admit (layer, expert) into its slot
 * row, reading pinned host memory over the host link from a kernel; the
 * miss count is read on the device.  The caller orders it after that
 * moe_admit (same stream, or an event) and before any reader of the
 * slots.  A cache without banks makes this a no-op.  Errors:
 * MOE_INVALID_ARG (no admission yet). */
moe_status_t moe_gather_misses(moe_cache_t *cache, void *stream);

/* Bytes of device workspace moe_routed_decode needs for T tokens x K
 * routes over a pool in this format and these widths. */
int64_t moe_routed_workspace_bytes(int32_t weight_format, int32_t hidden, int32_t ffn,
                                   int32_t T, int32_t K);

/* (4) Routed experts over pool rows, plus the combine [P2 "What we
 * changed": routed GEMM, then routed + shared; P1 section 5: -1 routes
 * add nothing; P3 Tests: the GEMV over slots equals the one over the
 * streamed layer].  For each token t:
 *   out[t] = bf16( sum over k ascending with idx[t][k] >= 0 of
 *                  w[t][k] * W2[r] (silu(W1[r] x_t) * (W3[r] x_t))
 *                  + addend[t] ),    r = idx[t][k]
 * x_dev: bf16 [T][H]; idx_dev: int32 [T][K] pool rows (slot ids, or expert
 * ids over a layer pool), -1 = skip; w_dev: fp32 [T][K]; addend_dev: fp32
 * [T][H] or NULL; out_dev: bf16 [T][H].  The intermediate activation is
 * rounded to bf16; dot products accumulate in fp32.  The result for a
 * route depends only on its pool row's bytes, never on the row's number,
 * so a slot pool and a layer pool holding the same expert bytes give
 * bit-identical outputs.  workspace_dev: at least
 * moe_routed_workspace_bytes(...), 256-byte aligned.  Pool rows in idx
 * must be < pool->num_rows (checked on the device: larger rows are
 * skipped like -1).  Errors: MOE_INVALID_ARG, MOE_UNSUPPORTED (H or F
 * not a supported width for the format). */
moe_status_t moe_routed_decode(const moe_pool_t *pool, const void *x_dev, const int32_t *idx_dev,
                               const float *w_dev, int32_t T, int32_t K, const float *addend_dev,
                               void *out_dev, void *workspace_dev, int64_t workspace_bytes,
                               void *stream);

/* Workspace held by moe_routed_decode_noalloc on each GPU: 16 MiB. */
#define MOE_NOALLOC_SCRATCH_BYTES (16 << 20)

/* moe_routed_decode for callers that cannot allocate device memory or pass
 * a workspace: code under hipGraph capture that may not call hipMalloc,
 * tight serving loops, harnesses that forbid allocation.  Same arguments,
 * arithmetic, kernels and results as moe_routed_decode, bit for bit, but
 * the workspace is the library's own static device array of
 * MOE_NOALLOC_SCRATCH_BYTES (one per GPU, held until the process ends).
 * The call allocates nothing: the first call on a device only looks up
 * that device's array address (hipGetSymbolAddress).  Every call on one
 * GPU shares that array and leaves its contents behind; nothing in it
 * needs to start at zero.  Calls that overlap on one GPU -- on different
 * streams, or from different threads, without an order between them --
 * race on the array and give undefined results; order them (one stream,
 * or events).  Errors: as moe_routed_decode, and MOE_INVALID_ARG when
 * moe_routed_workspace_bytes(...) for T, K and the pool's widths exceeds
 * MOE_NOALLOC_SCRATCH_BYTES. */
moe_status_t moe_routed_decode_noalloc(const moe_pool_t *pool, const void *x_dev,
                                       const int32_t *idx_dev, const float *w_dev, int32_t T,
                                       int32_t K, const float *addend_dev, void *out_dev,
                                       void *stream);

/* (5) Gated shared expert alone [P2 "Problem in upstream today"]:
 * addend[t] = sigmoid(x_t . gate) * shared(x_t), fp32 [T][H], the term
 * moe_routed_decode adds.  workspace: moe_routed_workspace_bytes(BF16, H,
 * shared ffn, T, 1) bytes. */
moe_status_t moe_shared_expert(const moe_shared_t *shared, int32_t hidden, const void *x_dev,
                               int32_t T, float *addend_dev, void *workspace_dev,
                               int64_t workspace_bytes, void *stream);

/* The whole layer step, (1)-(5), ordered as on [P2 "What we changed"]:
 * compute stream: top-k -> admission -> record(ready) -> shared expert
 * and gate (+ routed experts already resident, single token) -> wait(done)
 * -> routed experts -> routed + shared; side stream (overlap = 1):
 * wait(ready) -> gather -> record(done).  overlap = 0 runs the gather on
 * the compute stream right after the admission; overlap = 2 runs the
 * gather, the shared expert and the resident routes inside one launch
 * after the admission, then the down projections and the combine.  With
 * a few token rows the top-k runs inside the admission kernel.  The node
 * set does not depend on the hit pattern, so the call captures into one
 * hipGraph and replays with device-side counts.
 * x_dev: bf16 [T][H]; logits_dev: fp32 [T][E]; shared: NULL for a layer
 * without a shared expert; out_dev: bf16 [T][H]; ids_out_dev: int32
 * [T][K] slot ids (or NULL); w_out_dev: fp32 [T][K] (or NULL).
 * Errors: MOE_INVALID_ARG (layer, T > max_tokens, K > max_top_k, T*K >
 * max_routes, a cache without banks), MOE_UNSUPPORTED. */
moe_status_t moe_layer_decode(moe_cache_t *cache, int32_t layer, const void *x_dev,
                              const float *logits_dev, int32_t T, int32_t K,
                              const moe_shared_t *shared, int32_t max_fetch, void *out_dev,
                              int32_t *ids_out_dev, float *w_out_dev, void *stream);

/* Starts (threads >= 1) or stops (0) the cache's pool of host threads for
 * moe_layer_decode_hybrid, and on first use allocates its pinned staging
 * (max_tokens x (3 max_top_k + hidden/2 + hidden) x 4 bytes).  The calling
 * thread of a hybrid step works too: threads - 1 workers are started.
 * Synchronises the device.  Errors: MOE_INVALID_ARG (threads outside
 * [0, 1024], a cache without banks or layer workspace), MOE_UNSUPPORTED
 * (hidden and ffn not multiples of 16, or of 32 for MXFP4),
 * MOE_OUT_OF_MEMORY. */
moe_status_t moe_cache_set_cpu_threads(moe_cache_t *cache, int32_t threads);

/* The CPU half of the hybrid step on its own, on host memory only (no
 * device call): partial[t] = sum over k ascending with experts[t][k] >= 0
 * of w[t][k] * W2[e] (bf16(silu(W1[e] x_t) * (W3[e] x_t))), e =
 * experts[t][k], in fp32 with the activation rounded to bf16.  experts:
 * int32 [T][K] expert ids or -1; w: fp32 [T][K]; x: bf16 [T][H];
 * banks_host: the layer's host rows of each weight bank of the format, in
 * bank order (moe_bank_row_bytes: 2 for bf16, 6 for E2M1, 4 for MXFP4),
 * each [E][row bytes]; 4-bit weights are expanded to fp32 as code times
 * its block's scale (E4M3 per 16, or E8M0 per 32) and the E2M1 global
 * scale multiplies each dot product; partial: fp32 [T][H] out.  Starts
 * threads - 1 workers for the call.  The result does not depend on the
 * thread count.  Errors: MOE_INVALID_ARG (unknown format, threads
 * outside [1, 1024], H or F not a multiple of the format's block -- 16,
 * or 32 for MXFP4 -- null pointers). */
moe_status_t moe_cpu_experts(int32_t threads, int32_t weight_format, int32_t T, int32_t K, int32_t H,
                             int32_t F, const int32_t *experts_host, const float *w_host, const void *x_host,
                             const void *const *banks_host, float *partial_host);

/* The hybrid layer step [P1 sections 4-5]: routes the cache leaves at -1
 * (misses beyond max_fetch, or with no victim) run on host cores over the
 * pinned host store, overlapped with the GPU's capped gather, shared
 * expert and cached routes, and the two partial results are added.
 * Order: top-k -> original ids, weights and x copied to pinned host memory
 * -> admission (max_fetch) -> rewritten ids copied -> gather -> shared
 * expert -> GPU routes' gate/up -> [host: wait for the copies, compute
 * the CPU routes (ascending k per token) into a pinned fp32 partial, fold
 * it into the shared term] -> down projections and combine.  With the
 * cache's schedule 0 the CPU half runs before the GPU work is issued (the
 * pages' serial debug mode); otherwise it overlaps it.  The result:
 *   out[t] = bf16( sum over GPU routes, ascending k, of w * expert(x_t)
 *                  + (shared term + sum over CPU routes of w * expert(x_t)) )
 * The call blocks the host until the admission has run (it needs the slot
 * ids) and returns once the combine is issued; it cannot be captured in a
 * graph (MOE_INVALID_ARG on a capturing stream).  Arguments as
 * moe_layer_decode; ids_out_dev holds the slot ids, -1 for CPU routes.
 * Errors: MOE_INVALID_ARG (also: no CPU threads started), as
 * moe_layer_decode otherwise. */
moe_status_t moe_layer_decode_hybrid(moe_cache_t *cache, int32_t layer, const void *x_dev,
                                     const float *logits_dev, int32_t T, int32_t K,
                                     const moe_shared_t *shared, int32_t max_fetch, void *out_dev,
                                     int32_t *ids_out_dev, float *w_out_dev, void *stream);

/* Look-ahead prefetch of a layer's predicted experts [P4 Consumer,
 * Eviction guard].  ids_dev: int32 [n] predicted expert ids of `layer`;
 * ids outside [0, E) are ignored, the rest taken once each, ascending.
 * One clock tick per call of n > 0; n = 0 does nothing at all.
 *  - A predicted expert already resident is used now (stamped), so no
 *    fill of the same call evicts it.
 *  - Victims are the least recently used slots (ties: lower slot id)
 *    that are not pinned: a slot used at or after the latest demand
 *    admission (its readers may still run; fills since then may still be
 *    in flight) is never chosen.
 *  - Each missing prediction, ascending, looks at the next victim.  Its
 *    owner is protected when it has at least 2 demand accesses and
 *    score(owner) > 1.25 score(prediction) + 4, score = demand routes x
 *    256 + (255 - min(255, clock - last demand step), 0 if never); then
 *    the prediction is dropped and the next one looks at the same
 *    victim.  Otherwise the prediction takes the slot.
 *  - Heat (histogram, last demand step) counts demand admissions only.
 * On `stream` (the stream of the demand admissions: one writer of the
 * slot map) one kernel updates the state and writes the fill plan; the
 * fills' rows are then copied from pinned host memory on the cache's own
 * prefetch stream, forked from `stream` by an event, so the copy overlaps
 * whatever `stream` runs next.  The next demand admission of any layer
 * (moe_admit, moe_layer_decode) first waits for that copy, on the device;
 * so does the next prefetch, whose kernel reuses the fill plan.  Under
 * graph capture, call moe_prefetch_join before ending a capture with a
 * prefetch still pending, and before beginning one after an eager
 * prefetch (a call that would wait inside a capture for a copy issued
 * outside it fails with MOE_INVALID_ARG).  A cache without banks updates
 * the state only.
 * Errors: MOE_INVALID_ARG (layer outside [0, L), n < 0 or n > max_routes,
 * null ids with n > 0), MOE_UNSUPPORTED (the prefetch kernel for
 * min(max_routes, E) predictions does not fit the device's LDS: about
 * 48 min(max_routes, E) + E + S bytes). */
moe_status_t moe_prefetch(moe_cache_t *cache, int32_t layer, const int32_t *ids_dev, int32_t n,
                          void *stream);

/* Makes `stream` wait, on the device, for the copy of the last prefetch,
 * if one is pending (no-op otherwise). */
moe_status_t moe_prefetch_join(moe_cache_t *cache, void *stream);

/* ---------------------------------------------------------------- inspection */

/* Copies the layer's statistics (layer = -1: sums over layers) into
 * stats_host[MOE_NUM_STATS].  Synchronises `stream`. */
moe_status_t moe_cache_stats(moe_cache_t *cache, int32_t layer, int64_t *stats_host, void *stream);

/* Debug snapshot of the admission state into host arrays (any may be
 * NULL): res [L*E], own [S], stamp [S], clock [1], stats
 * [L*MOE_NUM_STATS], freq [L*E] (demand routes), order [S] (slots from
 * least to most recently used), dlast [L*E] (clock of each expert's last
 * demand step, 0 = never), last_demand [1] (clock of the latest demand
 * step, 0 = none).  Synchronises the device. */
moe_status_t moe_cache_read_state(moe_cache_t *cache, int32_t *res_host, int32_t *own_host,
                                  uint32_t *stamp_host, uint32_t *clock_host, int64_t *stats_host,
                                  int64_t *freq_host, int32_t *order_host, uint32_t *dlast_host,
                                  uint32_t *last_demand_host);

/* Debug restore of res/own/stamp/clock, and of freq/dlast/last_demand when
 * given (NULL leaves them, and the statistics, as they are).  own must be
 * the inverse of res, and no stamp, dlast or last_demand may exceed
 * clock; the LRU order is rebuilt from the stamps.  Synchronises the
 * device.  Errors: MOE_INVALID_ARG if these do not hold. */
moe_status_t moe_cache_write_state(moe_cache_t *cache, const int32_t *res_host,
                                   const int32_t *own_host, const uint32_t *stamp_host,
                                   uint32_t clock, const int64_t *freq_host,
                                   const uint32_t *dlast_host, const uint32_t *last_demand_host);

/* The miss plan of the last admission: up to cap (slot, expert) pairs and
 * its length.  Synchronises the device. */
moe_status_t moe_cache_read_plan(moe_cache_t *cache, int32_t *plan_slot_host,
                                 int32_t *plan_expert_host, int32_t cap, int32_t *n_miss_host);

/* The fill plan of the last moe_prefetch of width > 0: up to cap (slot,
 * expert) pairs, ascending expert, and its length.  Synchronises the
 * device. */
moe_status_t moe_cache_read_fills(moe_cache_t *cache, int32_t *fill_slot_host,
                                  int32_t *fill_expert_host, int32_t cap, int32_t *n_fill_host);

/* Optional timing of the layer step's kernels with HIP events recorded on
 * the stream each kernel runs on (as external event nodes when the step is
 * captured into a graph).  enable = 1 makes later moe_layer_decode calls
 * record, for each layer, events around its admission kernel, its gather
 * and its routed-expert kernels.  moe_cache_timing waits for the most
 * recent recording of every layer and writes its elapsed times to
 * ms_host[layer * 3 + {0: admission, 1: gather, 2: routed}] (-1 for a
 * layer never recorded); *layers_read gets the count.  For measurement
 * runs only. */
moe_status_t moe_cache_set_timing(moe_cache_t *cache, int32_t enable);
moe_status_t moe_cache_timing(moe_cache_t *cache, float *ms_host, int32_t *layers_read);

/* Records the HIP event `event` (a hipEvent_t, created by the caller) on
 * `stream`.  While the stream is being captured into a graph the record
 * becomes an event-record node of that graph, so every replay records it
 * again (a plain hipEventRecord under capture would not be replayed);
 * otherwise it is hipEventRecord.  A measurement aid: events around a
 * sequence of launches inside one graph time them with nothing between. */
moe_status_t moe_record_event(void *event, void *stream);

/* ---------------------------------------------------------------- verification */

/* The stream operations of a run of layer steps, recorded on the host
 * instead of issued, with no device involved [P2 "Correctness evidence":
 * the fork/join is checked on the CPU with fake streams].  A cache shaped
 * by *desc (its host and slot banks ignored) lives on the host only, with
 * placeholder device addresses; `tokens` tokens of num_layers layer steps
 * (moe_layer_decode of T x K routes, with a shared expert if with_shared,
 * in desc->overlap's schedule) are run, each followed, when
 * prefetch_width > 0, by moe_prefetch of the next layer's prefetch_width
 * predictions; a final moe_prefetch_join ends the run.  Every kernel
 * launch, event record and stream wait is written as one text line to
 * out_host (NUL-terminated, at most cap - 1 bytes; *len_out gets the full
 * length):
 *   S <token> <layer>                 a layer step begins
 *   P <token> <layer>                 a prefetch of that layer begins
 *   J                                 the final join
 *   L <stream> <kernel> <reads> <writes>   a launch; buffer names joined
 *                                     by ',' or '-' for none; "slots:fresh"
 *                                     / "slots:resident" are the slots the
 *                                     step's plan fills / that already held
 *                                     their expert, "slots" all of them
 *   E <stream> <event>                hipEventRecord
 *   W <stream> <event>                hipStreamWaitEvent
 * Streams: compute, side, prefetch; events: ready, done, pf_ready,
 * pf_done.  Errors: MOE_INVALID_ARG, MOE_UNSUPPORTED, as
 * moe_layer_decode for T and K. */
moe_status_t moe_trace_layer_steps(const moe_cache_desc_t *desc, int32_t T, int32_t K,
                                   int32_t with_shared, int32_t prefetch_width, int32_t tokens,
                                   char *out_host, int64_t cap, int64_t *len_out);

#ifdef __cplusplus
}
#endif
#endif /* MOE_CACHE_H */
