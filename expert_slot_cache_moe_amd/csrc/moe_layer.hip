// The C ABI (include/moe_cache.h), part 2: the layer step in its four
// schedules, and the hybrid CPU/GPU step with its host-thread experts.
#include "moe_api_internal.h"

using namespace moe;
using namespace moe::api;

extern "C" {

moe_status_t moe_layer_decode(moe_cache_t *c, int32_t layer, const void *x, const float *logits,
                              int32_t T, int32_t K, const moe_shared_t *shared, int32_t max_fetch,
                              void *out, int32_t *ids_out, float *w_out, void *stream) {
    if (!c) return fail(MOE_INVALID_ARG, "NULL cache");
    if (c->nb == 0) return fail(MOE_INVALID_ARG, "cache has no weight banks");
    if (layer < 0 || layer >= c->d.num_layers)
        return fail(MOE_INVALID_ARG, "layer %d outside [0, %d)", layer, c->d.num_layers);
    if (T < 0 || T > c->d.max_tokens) return fail(MOE_INVALID_ARG, "T=%d outside [0, max_tokens=%d]", T, c->d.max_tokens);
    if (K < 1 || K > c->d.max_top_k || K > c->d.num_experts)
        return fail(MOE_INVALID_ARG, "K=%d outside [1, %d]", K, c->d.max_top_k);
    if ((int64_t)T * K > c->d.max_routes) return fail(MOE_INVALID_ARG, "T*K > max_routes");
    if (T > 0 && (!x || !logits || !out)) return fail(MOE_INVALID_ARG, "NULL layer buffer");
    if (T > 0 && !aligned16(x)) return fail(MOE_INVALID_ARG, "x must be 16-byte aligned");
    int Fs = 0;
    if (shared) {
        moe_status_t s = check_shared(shared, c->d.hidden, c->d.ffn, &Fs);
        if (s != MOE_OK) return s;
        if (Fs > c->shared_ffn_cap)
            return fail(MOE_UNSUPPORTED, "shared ffn %d > the cache's workspace width %d", Fs, c->shared_ffn_cap);
    }
    hipStream_t s = static_cast<hipStream_t>(stream);
    int32_t *ids = ids_out ? ids_out : c->ws_ids;
    float *w = w_out ? w_out : c->ws_w;
    const int R = T * K;
    const bool timing = c->timing != 0;
    hipEvent_t *tev = timing ? &c->tev[(size_t)layer * 6] : nullptr;

    // Few token rows: the top-k runs inside the admission kernel.
    const bool fused_topk =
        T <= kFusedTopkRows && admit_fused_topk_supported(c->d.num_experts, c->d.num_slots, K);
    if (c->d.overlap == 3 && shared && T > 0) {
        // The #678 split: the shared expert and its gate on the side stream,
        // forked here; top-k, admission, gather and the routed experts on the
        // compute stream, joined right before the launch that adds the shared
        // term.  Every exit after the fork joins, so no side work outlives
        // the step.
        const uint16_t *xb = static_cast<const uint16_t *>(x);
        HIP_TRY(rec::event_record(c->ready, s), "record ready");
        HIP_TRY(rec::stream_wait(c->side, c->ready), "side waits ready");
        hipError_t e = shared_sequence(shared, c->d.hidden, Fs, xb, T, c->ws_addend, c->ws_shared, c->side);
        const hipError_t re = rec::event_record(c->done, c->side);
        auto joined = [&](moe_status_t r) {
            (void)rec::stream_wait(s, c->done);
            return r;
        };
        if (e != hipSuccess || re != hipSuccess)
            return joined(hip_fail(e != hipSuccess ? e : re, "shared expert on the side stream"));
        auto mark = [&](int i) { return timing ? record_timing(tev[i], s) : hipSuccess; };
        if (!fused_topk && (e = launch_topk(logits, T, c->d.num_experts, K, ids, w, s)) != hipSuccess)
            return joined(hip_fail(e, "top-k launch"));
        if ((e = mark(0)) != hipSuccess) return joined(hip_fail(e, "timing"));
        moe_status_t st = fused_topk
                              ? launch_admit_checked(c, layer, ids, R, max_fetch, s, c->ws_route_plan,
                                                     logits, T, K, w)
                              : launch_admit_checked(c, layer, ids, R, max_fetch, s, c->ws_route_plan);
        if (st != MOE_OK) return joined(st);
        if ((e = mark(1)) != hipSuccess || (e = mark(2)) != hipSuccess) return joined(hip_fail(e, "timing"));
        if ((st = launch_gather_checked(c, s)) != MOE_OK) return joined(st);
        if ((e = mark(3)) != hipSuccess || (e = mark(4)) != hipSuccess) return joined(hip_fail(e, "timing"));
        const BeforeAddend join = [&]() { return rec::stream_wait(s, c->done); };
        e = routed_sequence(slot_pool_view(c), xb, ids, w, T, K, c->ws_addend,
                            static_cast<uint16_t *>(out), c->ws_routed, s, &join);
        if (e != hipSuccess) return hip_fail(e, "routed launch");   // joined inside
        if (timing) {
            HIP_TRY(record_timing(tev[5], s), "timing");
            c->trecorded[layer] = 1;
        }
        return MOE_OK;
    }
    if (!fused_topk) HIP_TRY(launch_topk(logits, T, c->d.num_experts, K, ids, w, s), "top-k launch");
    if (timing) HIP_TRY(record_timing(tev[0], s), "timing");
    moe_status_t st = fused_topk ? launch_admit_checked(c, layer, ids, R, max_fetch, s, c->ws_route_plan,
                                                        logits, T, K, w)
                                 : launch_admit_checked(c, layer, ids, R, max_fetch, s, c->ws_route_plan);
    if (st != MOE_OK) return st;
    if (timing) HIP_TRY(record_timing(tev[1], s), "timing");
    if (c->d.overlap == 2 && T == 1 && stage_supported(c->d.weight_format, c->d.hidden, c->d.ffn) &&
        (!shared || Fs == c->d.ffn)) {
        // One stream, two launches: the gather overlaps the shared expert and
        // the resident routes inside stage 1.
        const PoolView pv = slot_pool_view(c);
        const RoutedWs rw = routed_ws(pv.H, pv.F, T, K);
        PoolView spv{};
        uint16_t *hs = nullptr;
        float *gamma = nullptr;
        if (shared) {
            spv.fmt = MOE_FMT_BF16;
            spv.H = c->d.hidden;
            spv.F = Fs;
            spv.num_rows = 1;
            spv.bank[0] = static_cast<const uint8_t *>(shared->w13_dev);
            spv.bank[1] = static_cast<const uint8_t *>(shared->w2_dev);
            spv.rb[0] = (int64_t)4 * Fs * c->d.hidden;
            spv.rb[1] = (int64_t)2 * c->d.hidden * Fs;
            const RoutedWs sw = routed_ws(c->d.hidden, Fs, T, 1);
            hs = reinterpret_cast<uint16_t *>(c->ws_shared + sw.h);
            gamma = reinterpret_cast<float *>(c->ws_shared + sw.d);
        }
        for (int which = 1; which <= 2; ++which) {
            if (timing) HIP_TRY(record_timing(tev[2 * which], s), "timing");
            HIP_TRY(launch_stages(gather_params_staged(c), c->gather_wg, c->ws_gu, pv, ids, w,
                                  c->ws_route_plan, K, static_cast<const uint16_t *>(x),
                                  reinterpret_cast<uint16_t *>(c->ws_routed + rw.h),
                                  shared ? &spv : nullptr, hs,
                                  shared ? static_cast<const uint16_t *>(shared->gate_dev)
                                         : nullptr,
                                  gamma, nullptr, static_cast<uint16_t *>(out), which, s),
                    "stage launch");
            if (timing) HIP_TRY(record_timing(tev[2 * which + 1], s), "timing");
        }
        if (timing) c->trecorded[layer] = 1;
        return MOE_OK;
    }
    const bool two_streams = c->d.overlap == 1;
    hipStream_t gs = s;
    if (two_streams) {
        HIP_TRY(rec::event_record(c->ready, s), "record ready");
        HIP_TRY(rec::stream_wait(c->side, c->ready), "side waits ready");
        gs = c->side;
    }
    if (timing) HIP_TRY(record_timing(tev[2], gs), "timing");
    st = launch_gather_checked(c, gs);
    if (st != MOE_OK) return st;
    if (timing) HIP_TRY(record_timing(tev[3], gs), "timing");
    if (two_streams) HIP_TRY(rec::event_record(c->done, c->side), "record done");

    // Between fork and join, on the compute stream: the shared expert and
    // its gate, and (single token) the routed experts whose slots were
    // already resident -- none of these reads a slot the gather writes.
    const PoolView pv = slot_pool_view(c);
    const uint16_t *xb = static_cast<const uint16_t *>(x);
    const bool split = two_streams && T == 1;
    const RoutedWs rw = routed_ws(pv.H, pv.F, T, K);
    uint16_t *h = reinterpret_cast<uint16_t *>(c->ws_routed + rw.h);
    float *dr = reinterpret_cast<float *>(c->ws_routed + rw.d);
    hipError_t e = hipSuccess;
    if (shared) e = shared_sequence(shared, c->d.hidden, Fs, xb, T, c->ws_addend, c->ws_shared, s);
    Items it{};
    it.mode = ITEM_ROUTE;
    it.K = K;
    it.n = R;
    it.idx = ids;
    it.route_plan = c->ws_route_plan;
    if (split && e == hipSuccess) {
        it.want_fresh = 0;
        e = launch_up(pv, it, R, xb, h, nullptr, nullptr, s);
        if (e == hipSuccess) e = launch_down_to_d(pv, it, R, h, dr, nullptr, s);
    }
    // The join is issued even if a launch above failed, so the side stream
    // never outlives the step.
    if (two_streams) {
        hipError_t je = rec::stream_wait(s, c->done);
        if (e == hipSuccess) e = je;
    }
    if (e != hipSuccess) return hip_fail(e, "shared expert / resident routes / join");

    if (timing) HIP_TRY(record_timing(tev[4], s), "timing");
    const float *add = shared ? c->ws_addend : nullptr;
    if (split) {
        it.want_fresh = 1;
        HIP_TRY(launch_up(pv, it, R, xb, h, nullptr, nullptr, s), "routed launch");
        HIP_TRY(launch_down_fused(pv, ids, w, T, K, h, add, dr, c->ws_route_plan,
                                  static_cast<uint16_t *>(out), s),
                "routed launch");
    } else {
        HIP_TRY(routed_sequence(pv, xb, ids, w, T, K, add, static_cast<uint16_t *>(out),
                                c->ws_routed, s),
                "routed launch");
    }
    if (timing) {
        HIP_TRY(record_timing(tev[5], s), "timing");
        c->trecorded[layer] = 1;
    }
    return MOE_OK;
}

moe_status_t moe_cache_set_cpu_threads(moe_cache_t *c, int32_t threads) {
    if (!c) return fail(MOE_INVALID_ARG, "NULL cache");
    if (threads < 0 || threads > 1024) return fail(MOE_INVALID_ARG, "threads %d outside [0, 1024]", threads);
    if (threads > 0) {
        if (c->nb == 0 || c->d.max_tokens < 1)
            return fail(MOE_INVALID_ARG, "the hybrid step needs weight banks and max_tokens > 0");
        const int blk = c->d.weight_format == MOE_FMT_MXFP4 ? 32 : 16;
        if (c->d.hidden % blk || c->d.ffn % blk)
            return fail(MOE_UNSUPPORTED, "the CPU experts take hidden and ffn multiples of %d in this format", blk);
    }
    HIP_TRY(hipDeviceSynchronize(), "sync");
    if (c->cpu) {
        cpu_experts_destroy(c->cpu);
        c->cpu = nullptr;
    }
    if (threads == 0) return MOE_OK;
    if (!c->hyb_host) {
        const size_t TK = (size_t)c->d.max_tokens * c->d.max_top_k, TH = (size_t)c->d.max_tokens * c->d.hidden;
        const size_t o_e = 0, o_s = align_up(TK * 4), o_w = o_s + align_up(TK * 4), o_x = o_w + align_up(TK * 4),
                     o_p = o_x + align_up(TH * 2), total = o_p + align_up(TH * 4);
        void *hp = nullptr;
        hipError_t e = hipHostMalloc(&hp, total, hipHostMallocMapped);
        if (e != hipSuccess) {
            (void)hipGetLastError();
            return fail(MOE_OUT_OF_MEMORY, "hybrid staging (%zu B pinned): %s", total, hipGetErrorString(e));
        }
        c->hyb_host = hp;
        uint8_t *b = static_cast<uint8_t *>(hp);
        c->h_experts = reinterpret_cast<int32_t *>(b + o_e);
        c->h_slots = reinterpret_cast<int32_t *>(b + o_s);
        c->h_w = reinterpret_cast<float *>(b + o_w);
        c->h_x = reinterpret_cast<uint16_t *>(b + o_x);
        c->h_partial = reinterpret_cast<float *>(b + o_p);
        void *dp = nullptr;
        HIP_TRY(hipHostGetDevicePointer(&dp, c->h_partial, 0), "map the hybrid partial");
        c->d_partial = static_cast<float *>(dp);
        c->cpu_ids.resize(TK);
        HIP_TRY(hipEventCreateWithFlags(&c->hyb_ready, hipEventDisableTiming), "hybrid event");
    }
    c->cpu = cpu_experts_create(threads);
    return MOE_OK;
}

moe_status_t moe_cpu_experts(int32_t threads, int32_t weight_format, int32_t T, int32_t K, int32_t H,
                             int32_t F, const int32_t *experts, const float *w, const void *x,
                             const void *const *banks, float *partial) {
    if (weight_format != MOE_FMT_BF16 && weight_format != MOE_FMT_E2M1 && weight_format != MOE_FMT_MXFP4)
        return fail(MOE_INVALID_ARG, "weight_format %d", weight_format);
    const int blk = weight_format == MOE_FMT_MXFP4 ? 32 : 16;
    if (threads < 1 || threads > 1024 || T < 0 || K < 1 || H < blk || F < blk || H % blk || F % blk)
        return fail(MOE_INVALID_ARG, "bad CPU expert sizes (threads %d, T %d, K %d, H %d, F %d)", threads,
                    T, K, H, F);
    if (T == 0) return MOE_OK;
    if (!experts || !w || !x || !banks || !partial) return fail(MOE_INVALID_ARG, "NULL CPU expert buffer");
    CpuRoutes r{};
    int nb = 0;
    row_bytes_of(weight_format, H, F, r.rb, &nb);
    for (int b = 0; b < nb; ++b) {
        if (!banks[b]) return fail(MOE_INVALID_ARG, "NULL CPU expert bank %d", b);
        r.bank[b] = static_cast<const uint8_t *>(banks[b]);
    }
    r.T = T;
    r.K = K;
    r.H = H;
    r.F = F;
    r.fmt = weight_format;
    r.expert = experts;
    r.w = w;
    r.x = static_cast<const uint16_t *>(x);
    r.partial = partial;
    CpuExperts *p = cpu_experts_create(threads);
    cpu_experts_run(p, r);
    cpu_experts_destroy(p);
    return MOE_OK;
}

moe_status_t moe_layer_decode_hybrid(moe_cache_t *c, int32_t layer, const void *x, const float *logits,
                                     int32_t T, int32_t K, const moe_shared_t *shared, int32_t max_fetch,
                                     void *out, int32_t *ids_out, float *w_out, void *stream) {
    if (!c) return fail(MOE_INVALID_ARG, "NULL cache");
    if (!c->cpu) return fail(MOE_INVALID_ARG, "no CPU experts: call moe_cache_set_cpu_threads first");
    if (layer < 0 || layer >= c->d.num_layers)
        return fail(MOE_INVALID_ARG, "layer %d outside [0, %d)", layer, c->d.num_layers);
    if (T < 0 || T > c->d.max_tokens) return fail(MOE_INVALID_ARG, "T=%d outside [0, max_tokens=%d]", T, c->d.max_tokens);
    if (K < 1 || K > c->d.max_top_k || K > c->d.num_experts)
        return fail(MOE_INVALID_ARG, "K=%d outside [1, %d]", K, c->d.max_top_k);
    if (T > 0 && (!x || !logits || !out)) return fail(MOE_INVALID_ARG, "NULL layer buffer");
    if (T > 0 && !aligned16(x)) return fail(MOE_INVALID_ARG, "x must be 16-byte aligned");
    int Fs = 0;
    if (shared) {
        moe_status_t st = check_shared(shared, c->d.hidden, c->d.ffn, &Fs);
        if (st != MOE_OK) return st;
        if (Fs > c->shared_ffn_cap)
            return fail(MOE_UNSUPPORTED, "shared ffn %d > the cache's workspace width %d", Fs, c->shared_ffn_cap);
    }
    hipStream_t s = static_cast<hipStream_t>(stream);
    {
        hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
        HIP_TRY(hipStreamIsCapturing(s, &cs), "capture status");
        if (cs != hipStreamCaptureStatusNone)
            return fail(MOE_INVALID_ARG, "the hybrid step waits on the host and cannot be captured");
    }
    const int H = c->d.hidden, E = c->d.num_experts, R = T * K;
    int32_t *ids = ids_out ? ids_out : c->ws_ids;
    float *w = w_out ? w_out : c->ws_w;
    const uint16_t *xb = static_cast<const uint16_t *>(x);
    const size_t lb = (size_t)layer * c->nb;

    // Cache decision: top-k, the original ids and x to the host, admission
    // (capped fetch), the rewritten ids to the host.
    HIP_TRY(launch_topk(logits, T, E, K, ids, w, s), "top-k launch");
    HIP_TRY(hipMemcpyAsync(c->h_experts, ids, (size_t)R * 4, hipMemcpyDeviceToHost, s), "ids to host");
    HIP_TRY(hipMemcpyAsync(c->h_w, w, (size_t)R * 4, hipMemcpyDeviceToHost, s), "weights to host");
    HIP_TRY(hipMemcpyAsync(c->h_x, x, (size_t)T * H * 2, hipMemcpyDeviceToHost, s), "x to host");
    moe_status_t st = launch_admit_checked(c, layer, ids, R, max_fetch, s, c->ws_route_plan);
    if (st != MOE_OK) return st;
    HIP_TRY(hipMemcpyAsync(c->h_slots, ids, (size_t)R * 4, hipMemcpyDeviceToHost, s), "slots to host");
    HIP_TRY(hipEventRecord(c->hyb_ready, s), "record hybrid ready");

    // The CPU half: waits for the decision, then runs the -1 routes with a
    // valid expert id on host cores into the pinned partial.  Folding the
    // partial into the fp32 term is issued right before the combine.
    auto cpu_half = [&]() -> hipError_t {
        hipError_t e = hipEventSynchronize(c->hyb_ready);
        if (e != hipSuccess) return e;
        for (int i = 0; i < R; ++i) {
            const int ex = c->h_experts[i];
            c->cpu_ids[i] = (c->h_slots[i] < 0 && ex >= 0 && ex < E) ? ex : -1;
        }
        CpuRoutes r{};
        r.T = T;
        r.K = K;
        r.H = H;
        r.F = c->d.ffn;
        r.expert = c->cpu_ids.data();
        r.w = c->h_w;
        r.x = c->h_x;
        r.fmt = c->d.weight_format;
        for (int b = 0; b < c->nb; ++b) {
            r.bank[b] = c->host_rows[lb + b];
            r.rb[b] = c->rb[b];
        }
        r.partial = c->h_partial;
        cpu_experts_run(c->cpu, r);
        return hipSuccess;
    };
    auto fold = [&]() { return launch_hybrid_add(c->ws_addend, c->d_partial, T * H, shared ? 1 : 0, s); };
    const bool serial = c->d.overlap == 0;
    if (serial) {
        // the debug order: the CPU wait before the GPU work
        hipError_t e = cpu_half();
        if (e != hipSuccess) return hip_fail(e, "hybrid CPU half");
    }
    // GPU half: the capped gather, the shared term, the GPU routes; the CPU
    // partial joins the fp32 term right before the combine adds it.
    st = launch_gather_checked(c, s);
    if (st != MOE_OK) return st;
    if (shared) {
        hipError_t e = shared_sequence(shared, H, Fs, xb, T, c->ws_addend, c->ws_shared, s);
        if (e != hipSuccess) return hip_fail(e, "shared launch");
    }
    const BeforeAddend cpu_join = [&]() {
        hipError_t e = serial ? hipSuccess : cpu_half();
        return e != hipSuccess ? e : fold();
    };
    HIP_TRY(routed_sequence(slot_pool_view(c), xb, ids, w, T, K, c->ws_addend, static_cast<uint16_t *>(out),
                            c->ws_routed, s, &cpu_join),
            "hybrid routed launch");
    return MOE_OK;
}

}  // extern "C"
