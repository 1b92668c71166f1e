#!/usr/bin/env python3
"""Benchmark of the offloaded MoE decode step on one MI355X.

Workload (the configuration the layer-steps/s metric is quoted on): the
shared-expert decode stack -- 40 MoE layers x 256 experts, top-8 plus a
gated shared expert, hidden 2048, expert FFN 512, bf16 expert weights in
pinned host memory (64.4 GB), a 3164-slot device cache, batch 1, Zipf(1.05)
routing with per-token temporal locality (~28 misses per token).

A step is one token: the whole hot path (top-k, admission, miss gather,
shared expert, routed experts, combine) for all 40 layers, captured as one
hipGraph and replayed; `value` is layer-steps per second (40 per token)
with every input resident in HBM before the timed region.

Also reported:
  roofline       the dominant kernel (the miss gather, host-link bound):
                 algorithmic bytes per launch / its average duration,
                 measured with HIP events captured around it in the graph,
                 replaying the same tokens from the same cache state.
  roofline_gemv  the routed expert kernels (gate/up + down) against HBM.
  admission_us   admission-only benchmark: 48 per-layer caches of 512
                 experts pre-filled into 2100 slots, 48 admissions per
                 graph, 40 replays, microseconds per admission by routes;
                 admission_us_one_call_width_128 repeats 130, 160 and 240
                 routes with the one-call width at 128 (chunked queries).
  cpu_baseline   the oracle (plain C, one thread) on a bounded sample of
                 the same decode workload; its "admission" entry times the
                 oracle's admission alone on the admission-only workload.

Profile summaries: with --launch-log the run also writes which launches
the timed and instrumented passes made (and this line); the summaries in
profiles/ are made from a rocprofv3 trace (or counter run) of the same
command by --summarize-trace / --summarize-pmc, over exactly the launches
the line's figures average.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

L, E, K, H, F, S = 40, 256, 8, 2048, 512, 3164
ROW_BYTES = 6 * F * H            # one bf16 expert: w13 (4FH) + w2 (2FH) bytes
HBM_PEAK_GBS = 8000.0            # MI355X HBM3E
HOST_LINK_PEAK_GBS = 64.0        # PCIe 5.0 x16, one direction
GEMV_PASSES = 4                  # routed-GEMV phase: passes over the 40 layers per graph
GEMV_REPLAYS = 5                 # timed replays of that graph (after one untimed)
GEMV_HEAD_START_CYCLES = 100_000_000  # spin before the timed calls (tens of ms of shader clock)


def log(*a):
    print(*a, file=sys.stderr, flush=True)


# Untimed token replays before the timed ones, whatever --warmup asks for:
# the 3164-slot cache starts empty and needs this many tokens to reach its
# steady state of ~28 misses per token (the pages' figure is taken after a
# warm-up too).  --warmup only adds graph warm-up beyond it.
CACHE_WARM_TOKENS = 64


def token_plan(warmup: int, steps: int):
    """(untimed tokens, trace length, first timed token) for a run of
    `steps` timed tokens: the trace holds the cache warm-up, then exactly
    the timed tokens."""
    n_warm = max(int(warmup), CACHE_WARM_TOKENS)
    return n_warm, n_warm + int(steps), n_warm


def leg_tokens(first: int, n_tok: int, limit=None) -> range:
    """The tokens a replay leg runs again: the timed tokens [first, n_tok),
    at most `limit` of them; never an index past the trace."""
    n = max(0, n_tok - first)
    if limit is not None:
        n = min(n, int(limit))
    return range(first, first + n)


def run_leg(name, fn, *a, **kw):
    """A side leg of the bench: its result, or {"error": ...} if it raised,
    so that one leg's failure never loses the result line."""
    import traceback

    try:
        return fn(*a, **kw)
    except Exception as e:  # noqa: BLE001 - reported in the line
        log(f"[bench] leg {name} failed:")
        log(traceback.format_exc())
        return {"error": f"{type(e).__name__}: {e}"}


def kernel_sources_hash() -> str:
    """Hash of the device-code sources (kernels and the headers they
    include); the host-side C-ABI files do not change what a kernel moves."""
    import glob
    import hashlib

    csrc = os.path.join(ROOT, "expert_slot_cache_moe_amd", "csrc")
    files = sorted(glob.glob(os.path.join(csrc, "k_*.hip")) + glob.glob(os.path.join(csrc, "*.inc"))
                   + [os.path.join(csrc, "moe_internal.h")])
    h = hashlib.sha256()
    for f in files:
        h.update(os.path.basename(f).encode())
        h.update(open(f, "rb").read())
    return h.hexdigest()[:16]


def traffic_ratios():
    """Counter-measured traffic/algorithmic ratios, valid only while the
    kernels are the ones the counters were taken on."""
    path = os.path.join(ROOT, "profiles", "decode_40x256_traffic.txt")
    vals = {}
    if os.path.exists(path):
        for line in open(path):
            line = line.split("#", 1)[0].strip()
            if "=" in line:
                k, v = (x.strip() for x in line.split("=", 1))
                vals[k] = v
    if vals.get("kernel_sources_sha256_16") != kernel_sources_hash():
        return None
    return {k: float(v) for k, v in vals.items() if k.endswith("_ratio")}


_SHARED = {}


def shared_experts(W, seed=0):
    """The 40 layers' gated shared experts (bf16 N(0, 0.02)), drawn once."""
    if seed not in _SHARED:
        gs = W.rng(seed, "bench", "shared")
        _SHARED[seed] = [(W.normal_bf16(gs, 2 * F * H, 0.02), W.normal_bf16(gs, H * F, 0.02),
                          W.normal_bf16(gs, H, 0.02)) for _ in range(L)]
    return _SHARED[seed]


def host_store(torch, W, fmt=0, seed=0):
    """Pinned host rows of 40 x 256 experts in format fmt: every expert of
    every layer drawn afresh on the device (N(0, 0.02), stored as bf16 or
    quantized to 4 bits), then copied into the layer's pinned host rows."""
    t0 = time.time()
    host = []
    for l in range(L):
        dev = W.device_expert_rows(fmt, (seed, "bench", l) if fmt == 0 else (seed, "bench", fmt, l), E, H, F)
        host.append([W.pinned_copy(b) for b in dev])
        del dev
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    nbytes = sum(b.numel() for hl in host for b in hl)
    log(f"[bench] pinned host store, format {fmt}: {nbytes / 1e9:.1f} GB in {time.time() - t0:.1f}s")
    return host


def build_stack(torch, m, W, seed=0, gather_workgroups=0, overlap=1, fmt=0, host=None):
    """Pinned host store for 40 x 256 experts, shared experts, the cache."""
    from expert_slot_cache_moe_amd.layer import SlotCacheLayers

    if host is None:
        host = host_store(torch, W, fmt, seed)
    lay = SlotCacheLayers(layers=L, experts=E, slots=S, hidden=H, ffn=F, fmt=fmt, host_rows=host,
                          shared=shared_experts(W, seed), max_tokens=1, max_top_k=K, overlap=overlap,
                          gather_workgroups=gather_workgroups)
    return lay


def release_pinned(torch):
    """Hands torch's cached pinned host blocks back (a leg's store is freed)."""
    import gc

    gc.collect()
    torch.cuda.synchronize()
    if hasattr(torch._C, "_host_emptyCache"):
        torch._C._host_emptyCache()
    torch.cuda.empty_cache()


def make_trace(torch, W, n, seed=0):
    tr = W.DecodeTrace(seed, L, E, K)
    gx = W.rng(seed, "bench", "hidden")
    lg = np.empty((n, L, 1, E), np.float32)
    xs = np.empty((n, L, 1, H), np.uint16)
    for t in range(n):
        lg[t, :, 0, :] = tr.logits(tr.step_sets())
        xs[t] = W.normal_bf16(gx, (L, 1, H))
    return (torch.from_numpy(lg).cuda(), torch.from_numpy(xs.view(np.int16)).cuda())


def stage_inputs(torch, pairs, step):
    """Inside a capture: each (source [tokens, ...], staging [...]) pair's
    row `step` (a one-element device tensor) copied into the staging
    buffer, then the step advanced, so that a replay of the token graph
    needs no host-issued work: the device-side counter picks the token."""
    for src, dst in pairs:
        torch.index_select(src, 0, step, out=dst.unsqueeze(0))
    step.add_(1)


def capture(torch, lay, x_st, lg_st, out, inputs, ids=None, w=None, pairs=None):
    """The 40-layer token graph, starting with the token's inputs staged by
    the device-side step counter (inputs = (x_all, lg_all, step)); with
    `pairs` (two lists of L created events), each layer step is preceded
    by an empty event pair (two event-record nodes back to back)."""
    import expert_slot_cache_moe_amd as m

    x_all, lg_all, step = inputs
    stream = torch.cuda.Stream()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=stream):
        stage_inputs(torch, ((x_all, x_st), (lg_all, lg_st)), step)
        for l in range(L):
            if pairs is not None:
                m.moe_record_event(pairs[0][l], stream)
                m.moe_record_event(pairs[1][l], stream)
            lay.decode(l, x_st[l], lg_st[l], K, out[l], ids_out=None if ids is None else ids[l],
                       w_out=None if w is None else w[l])
    return graph


# Wide steps (their routed GEMV alone, moe_routed_decode over a pool):
# (name, format, H, F, token rows, top-k, experts, pool copies rotated over)
WIDE = (
    ("wide decode bf16: 150 rows x top-2 over 160 experts, H 1024, F 256", 0, 1024, 256, 150, 2, 160, 8),
    ("wide decode e2m1 (E4M3 per-16 scales): 600 rows x top-2 over 160 experts, H 1024, F 256",
     1, 1024, 256, 600, 2, 160, 8),
    ("wide decode mxfp4 (E8M0 per-32 scales): 600 rows x top-2 over 160 experts, H 1024, F 256",
     2, 1024, 256, 600, 2, 160, 8),
    ("prefill chunk bf16: 42 rows x top-6 over 256 experts, H 4096, F 1024", 0, 4096, 1024, 42, 6, 256, 1),
    ("prefill chunk bf16: 50 rows x top-6 over 640 experts, H 4096, F 1024", 0, 4096, 1024, 50, 6, 640, 1),
)
WIDE_SETS = 8            # routing sets per graph (one call each)
WIDE_REPLAYS = 3         # timed replays (after one untimed)


def wide_gemv_benchmark(torch, m, seed=0):
    """Routed GEMV of the wide-step shapes: one graph per shape holding a
    head-start spin, an event node, WIDE_SETS calls over different routings
    (each over its own copy of the pool where the shape allows, so that no
    call finds its rows in the last-level cache) and an event node."""
    res = []
    for name, fmt, Hw, Fw, T, Kw, Ew, copies in WIDE:
        rb = m.moe_bank_row_bytes(fmt, Hw, Fw)
        rows = Ew * copies
        gen = torch.Generator(device="cuda")
        gen.manual_seed(seed)
        if fmt == 0:
            banks = [torch.randn((rows, r // 2), device="cuda", generator=gen).mul_(0.02)
                     .to(torch.bfloat16).view(torch.uint8) for r in rb]
        else:
            banks = [torch.randint(0, 256, (rows, r), dtype=torch.uint8, device="cuda", generator=gen)
                     for r in rb]
            if fmt == 1:
                for b in (1, 4):
                    banks[b].fill_(0x30)                       # E4M3 scale 0.125
                for b in (2, 5):
                    banks[b].view(torch.float32).fill_(1.0)    # global scales
            else:
                for b in (1, 3):
                    banks[b].fill_(120)                        # E8M0 scale 2^-7
        pool = m.make_pool(fmt, Hw, Fw, rows, banks)
        g = np.random.default_rng(seed)
        sets = [np.stack([g.choice(Ew, Kw, replace=False) for _ in range(T)]) + (i % copies) * Ew
                for i in range(WIDE_SETS)]
        distinct = float(np.mean([len(np.unique(x)) for x in sets]))
        idx = [torch.from_numpy(x.astype(np.int32)).cuda() for x in sets]
        x = torch.randn((T, Hw), device="cuda", generator=gen).to(torch.bfloat16).view(torch.int16)
        w = torch.rand((T, Kw), device="cuda", generator=gen)
        out = torch.empty((T, Hw), dtype=torch.int16, device="cuda")
        ws = torch.empty(m.moe_routed_workspace_bytes(fmt, Hw, Fw, T, Kw), dtype=torch.uint8, device="cuda")
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
        st = torch.cuda.Stream()
        for e in ev:
            e.record(st)
        torch.cuda.synchronize()
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph, stream=st):
            torch.cuda._sleep(GEMV_HEAD_START_CYCLES)
            m.moe_record_event(ev[0], st)
            for i in range(WIDE_SETS):
                m.moe_routed_decode(pool, x, idx[i], w, out, ws, stream=st)
            m.moe_record_event(ev[1], st)
        per = []
        for r in range(1 + WIDE_REPLAYS):
            graph.replay()
            torch.cuda.synchronize()
            if r:
                per.append(ev[0].elapsed_time(ev[1]) * 1000.0 / WIDE_SETS)
        us = float(np.mean(per))
        nbytes = distinct * sum(rb) + 2 * T * Hw * 2 + T * Kw * 8
        res.append({"workload": name, "us_per_call": round(us, 2), "distinct_experts": round(distinct, 1),
                    "bytes_per_call": round(nbytes), "achieved_gbs": round(nbytes / (us * 1e-6) / 1e9, 1),
                    "frac_of_hbm_peak": round(nbytes / (us * 1e-6) / 1e9 / HBM_PEAK_GBS, 4)})
        del banks, pool, ws, graph
        torch.cuda.empty_cache()
    return res


# The one-call/chunked crossover re-measured: these batches (130, 160 and
# 240 routes) again with the one-call width lowered to 128, so that they
# are admitted in 128-expert chunks instead of one query.
ADMISSION_CHUNKED_BATCHES = (13, 16, 24)


def admission_benchmark(torch, m, W, replays=40, layers=48, one_call_width=256, batches=None):
    res = {}
    caches = [m.moe_cache_create(num_layers=1, num_experts=512, num_slots=2100, max_routes=1280,
                                 one_call_width=one_call_width)
              for _ in range(layers)]
    try:
        full = torch.arange(512, dtype=torch.int32, device="cuda")
        for c in caches:
            m.moe_admit(c, 0, full.clone())
        torch.cuda.synchronize()
        for req in (batches or W.ADMISSION_BATCHES):
            R = req * 10
            src = torch.from_numpy(np.stack([W.admission_ids(l, req) for l in range(layers)])).cuda()
            work = torch.empty_like(src)
            stream = torch.cuda.Stream()
            graph = torch.cuda.CUDAGraph()
            with torch.cuda.graph(graph, stream=stream):
                work.copy_(src)
                for l, c in enumerate(caches):
                    m.moe_admit(c, 0, work[l])
            for _ in range(3):
                graph.replay()
            torch.cuda.synchronize()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            for _ in range(replays):
                graph.replay()
            e1.record()
            torch.cuda.synchronize()
            res[str(R)] = round(e0.elapsed_time(e1) * 1000.0 / (replays * layers), 2)
            st = m.moe_cache_stats(caches[0], 0)
            assert st[2] == 512, "admission benchmark steps must be all hits"
    finally:
        for c in caches:
            m.moe_cache_destroy(c)
    return res


# Look-ahead prefetch: accuracies of the synthetic next-layer predictor.
LOOKAHEAD_ACCURACY = (1.0, 0.5)


def lookahead_benchmark(torch, m, lay, snap, x_all, lg_all, first, n_tok, seed=0):
    """The timed tokens again, from the cache state they started from, with
    each layer step followed by a look-ahead prefetch of the next layer's
    predicted experts: the true top-8 of that layer's logits, each replaced
    by a uniformly drawn expert with probability 1 - accuracy.  The whole
    token is one graph; the prefetch copies fork to the cache's prefetch
    stream and join at the next layer's admission."""
    stream = torch.cuda.Stream()
    x_st = torch.empty((L, 1, H), dtype=torch.int16, device="cuda")
    lg_st = torch.empty((L, 1, E), dtype=torch.float32, device="cuda")
    pr_st = torch.empty((L, K), dtype=torch.int32, device="cuda")
    pred = torch.empty((n_tok, L, K), dtype=torch.int32, device="cuda")
    step = torch.zeros(1, dtype=torch.int64, device="cuda")
    out = torch.empty((L, 1, H), dtype=torch.int16, device="cuda")
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=stream):
        stage_inputs(torch, ((x_all, x_st), (lg_all, lg_st), (pred, pr_st)), step)
        for l in range(L):
            lay.decode(l, x_st[l], lg_st[l], K, out[l], stream=stream)
            if l + 1 < L:
                m.moe_prefetch(lay.cache, l + 1, pr_st[l + 1], stream=stream)
        m.moe_prefetch_join(lay.cache, stream)
    true_ids = torch.topk(lg_all[:, :, 0, :], K, dim=-1).indices.to(torch.int32)
    res = []
    for acc in LOOKAHEAD_ACCURACY:
        rng = np.random.default_rng([seed, int(round(acc * 1000))])
        keep = torch.from_numpy(rng.random((n_tok, L, K)) < acc).cuda()
        rnd = torch.from_numpy(rng.integers(0, E, (n_tok, L, K)).astype(np.int32)).cuda()
        pred.copy_(torch.where(keep, true_ids, rnd))
        step.fill_(first)
        m.moe_cache_write_state(lay.cache, snap["res"], snap["own"], snap["stamp"], snap["clock"],
                                freq=snap["freq"], dlast=snap["dlast"],
                                last_demand=snap["last_demand"])
        st0 = m.moe_cache_stats(lay.cache)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        toks = leg_tokens(first, n_tok)
        for t in toks:
            graph.replay()
        torch.cuda.synchronize()
        dt = time.perf_counter() - t0
        d = m.moe_cache_stats(lay.cache) - st0
        n = len(toks)
        res.append({"predictor_accuracy": acc,
                    "value": round(L * n / dt, 1),
                    "ms_per_step": round(dt / n * 1000.0, 4),
                    "demand_fetches_per_token": round(float(d[m.MOE_STAT_MISSED] - d[m.MOE_STAT_OVERFLOW]) / n, 2),
                    "prefetch_fills_per_token": round(float(d[m.MOE_STAT_PF_FILLED]) / n, 2),
                    "prefetch_drops_per_token": round(float(d[m.MOE_STAT_PF_DROPPED]) / n, 2)})
        log(f"[bench] look-ahead, accuracy {acc}: {res[-1]}")
    return res


# The look-ahead where it is meant to pay: the pages' prefetch hides the
# next layer's copies behind the rest of the current layer (attention and
# the other layer work), which this workload does not have.  A kernel that
# holds the compute stream for about LOOKAHEAD_REST_US without touching
# memory stands in for that work before every layer step (an idealised
# stand-in: real attention would also use HBM and compute units).
LOOKAHEAD_REST_US = 150.0


def rest_cycles(torch, us):
    """Clock cycles of torch.cuda._sleep that take about `us` microseconds
    on this device, measured."""
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    probe = 1_000_000
    torch.cuda._sleep(probe)
    torch.cuda.synchronize()
    e0.record()
    torch.cuda._sleep(probe)
    e1.record()
    torch.cuda.synchronize()
    return max(1, int(probe * us / (e0.elapsed_time(e1) * 1000.0)))


def lookahead_rest_benchmark(torch, m, lay, snap, x_all, lg_all, first, n_tok, seed=0):
    """The timed tokens again with the stand-in for the rest of each layer
    before every layer step: without look-ahead, and with it at each
    predictor accuracy (as in lookahead_benchmark); the same cache state
    each time.  Also the stand-in alone (40 of them per token)."""
    cyc = rest_cycles(torch, LOOKAHEAD_REST_US)
    stream = torch.cuda.Stream()
    x_st = torch.empty((L, 1, H), dtype=torch.int16, device="cuda")
    lg_st = torch.empty((L, 1, E), dtype=torch.float32, device="cuda")
    pr_st = torch.empty((L, K), dtype=torch.int32, device="cuda")
    pred = torch.empty((n_tok, L, K), dtype=torch.int32, device="cuda")
    step = torch.zeros(1, dtype=torch.int64, device="cuda")
    out = torch.empty((L, 1, H), dtype=torch.int16, device="cuda")

    def capture(prefetch, layers=True):
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph, stream=stream):
            stage_inputs(torch, ((x_all, x_st), (lg_all, lg_st), (pred, pr_st)), step)
            for l in range(L):
                torch.cuda._sleep(cyc)
                if not layers:
                    continue
                lay.decode(l, x_st[l], lg_st[l], K, out[l], stream=stream)
                if prefetch and l + 1 < L:
                    m.moe_prefetch(lay.cache, l + 1, pr_st[l + 1], stream=stream)
            if prefetch:
                m.moe_prefetch_join(lay.cache, stream)
        return graph

    true_ids = torch.topk(lg_all[:, :, 0, :], K, dim=-1).indices.to(torch.int32)
    toks = leg_tokens(first, n_tok)
    n = len(toks)

    def run(graph):
        step.fill_(first)
        m.moe_cache_write_state(lay.cache, snap["res"], snap["own"], snap["stamp"], snap["clock"],
                                freq=snap["freq"], dlast=snap["dlast"], last_demand=snap["last_demand"])
        st0 = m.moe_cache_stats(lay.cache)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in toks:
            graph.replay()
        torch.cuda.synchronize()
        dt = time.perf_counter() - t0
        d = m.moe_cache_stats(lay.cache) - st0
        return {"value": round(L * n / dt, 1), "ms_per_step": round(dt / n * 1000.0, 4),
                "demand_fetches_per_token": round(float(d[m.MOE_STAT_MISSED] - d[m.MOE_STAT_OVERFLOW]) / n, 2),
                "prefetch_fills_per_token": round(float(d[m.MOE_STAT_PF_FILLED]) / n, 2)}

    g = capture(False, layers=False)
    rest = run(g)
    del g
    res = {"rest_us": LOOKAHEAD_REST_US, "rest_ms_per_token": rest["ms_per_step"], "tokens": n, "runs": []}
    g = capture(False)
    r = run(g)
    del g
    res["runs"].append({"prefetch": False, **r})
    log(f"[bench] rest of the layer ({LOOKAHEAD_REST_US} us stand-in), no look-ahead: {r}")
    g = capture(True)
    for acc in LOOKAHEAD_ACCURACY:
        rng = np.random.default_rng([seed, int(round(acc * 1000))])
        keep = torch.from_numpy(rng.random((n_tok, L, K)) < acc).cuda()
        rnd = torch.from_numpy(rng.integers(0, E, (n_tok, L, K)).astype(np.int32)).cuda()
        pred.copy_(torch.where(keep, true_ids, rnd))
        r = run(g)
        res["runs"].append({"prefetch": True, "predictor_accuracy": acc, **r})
        log(f"[bench] rest of the layer ({LOOKAHEAD_REST_US} us stand-in), look-ahead at accuracy {acc}: {r}")
    del g
    return res


# The layer-step schedules timed beside the default one (overlap = 2).
SCHEDULES = ((0, "serial: gather, shared expert and routed experts in order on one stream"),
             (1, "gather on the side stream, overlapping the shared expert and the resident routes"),
             (3, "shared expert on the side stream, gather and routed experts on the compute stream"))


def schedule_benchmark(torch, m, lay, snap, x_all, lg_all, first, n_tok):
    """The timed tokens again under each other schedule of the layer step,
    from the same cache state (the cached experts, and so the fetches, are
    the same in every schedule)."""
    res = []
    x_st = torch.empty((L, 1, H), dtype=torch.int16, device="cuda")
    lg_st = torch.empty((L, 1, E), dtype=torch.float32, device="cuda")
    out = torch.empty((L, 1, H), dtype=torch.int16, device="cuda")
    step = torch.zeros(1, dtype=torch.int64, device="cuda")
    for ov, what in SCHEDULES:
        m.moe_cache_set_schedule(lay.cache, ov)
        graph = capture(torch, lay, x_st, lg_st, out, (x_all, lg_all, step))
        step.fill_(first)
        m.moe_cache_write_state(lay.cache, snap["res"], snap["own"], snap["stamp"], snap["clock"],
                                freq=snap["freq"], dlast=snap["dlast"],
                                last_demand=snap["last_demand"])
        st0 = m.moe_cache_stats(lay.cache)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        toks = leg_tokens(first, n_tok)
        for t in toks:
            graph.replay()
        torch.cuda.synchronize()
        dt = time.perf_counter() - t0
        d = m.moe_cache_stats(lay.cache) - st0
        n = len(toks)
        res.append({"overlap": ov, "schedule": what, "value": round(L * n / dt, 1),
                    "ms_per_step": round(dt / n * 1000.0, 4),
                    "misses_per_token": round(float(d[m.MOE_STAT_MISSED] - d[m.MOE_STAT_OVERFLOW]) / n, 2)})
        log(f"[bench] schedule {ov}: {res[-1]['value']} layer-steps/s")
        del graph
    m.moe_cache_set_schedule(lay.cache, 2)
    return res


# Hybrid decode: host threads for the CPU routes, fetch caps timed, tokens.
HYBRID_THREADS = 16
HYBRID_CAPS = (0, 1, -1)
HYBRID_TOKENS = 32


def hybrid_benchmark(torch, m, lay, snap, x_all, lg_all, first, n_tok):
    """The first HYBRID_TOKENS timed tokens again (fewer if fewer were
    timed), eagerly, as hybrid steps:
    misses beyond the fetch cap run on HYBRID_THREADS host threads over the
    pinned host store while the GPU runs the rest.  Cap -1 fetches every
    miss (no CPU route): the cost of the hybrid step's host orchestration
    alone."""
    m.moe_cache_set_cpu_threads(lay.cache, HYBRID_THREADS)
    out = torch.empty((L, 1, H), dtype=torch.int16, device="cuda")
    ids = torch.empty((L, 1, K), dtype=torch.int32, device="cuda")
    res = []
    toks = leg_tokens(first, n_tok, HYBRID_TOKENS)
    n = len(toks)
    for cap in HYBRID_CAPS:
        m.moe_cache_write_state(lay.cache, snap["res"], snap["own"], snap["stamp"], snap["clock"],
                                freq=snap["freq"], dlast=snap["dlast"],
                                last_demand=snap["last_demand"])
        st0 = m.moe_cache_stats(lay.cache)
        cpu_routes = torch.zeros((), dtype=torch.int64, device="cuda")
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for t in toks:
            for l in range(L):
                lay.decode_hybrid(l, x_all[t, l], lg_all[t, l], K, out[l], ids_out=ids[l], max_fetch=cap)
            cpu_routes += (ids < 0).sum()
        torch.cuda.synchronize()
        dt = time.perf_counter() - t0
        d = m.moe_cache_stats(lay.cache) - st0
        res.append({"fetch_cap": cap, "value": round(L * n / dt, 1), "ms_per_step": round(dt / n * 1000.0, 4),
                    "fetches_per_token": round(float(d[m.MOE_STAT_MISSED] - d[m.MOE_STAT_OVERFLOW]) / n, 2),
                    "cpu_routes_per_token": round(float(cpu_routes.item()) / n, 2)})
        log(f"[bench] hybrid, fetch cap {cap}: {res[-1]}")
    m.moe_cache_set_cpu_threads(lay.cache, 0)
    return {"threads": HYBRID_THREADS, "tokens": n, "runs": res}


# The same decode trace over 4-bit experts: E2M1 codes with one E4M3 scale
# per 16 elements and an fp32 global per matrix (the pages' decode model is
# NVFP4): 1.77 MB per expert, an 18.1 GB pinned host store, 5.6 GB of slots.
DECODE_4BIT_SCHEDULES = (2, 0)


def decode_4bit_benchmark(torch, m, W, x_all, lg_all, n_warm, n_tok, fmt=1, seed=0):
    """The timed tokens of the trace (after the same cache warm-up) over a
    40 x 256 stack of 4-bit experts, each token one graph, under the staged
    schedule (2) and the serial one (0)."""
    host = host_store(torch, W, fmt, seed)
    rb = m.moe_bank_row_bytes(fmt, H, F)
    runs = []
    try:
        for ov in DECODE_4BIT_SCHEDULES:
            lay = build_stack(torch, m, W, seed, overlap=ov, fmt=fmt, host=host)
            try:
                x_st = torch.empty((L, 1, H), dtype=torch.int16, device="cuda")
                lg_st = torch.empty((L, 1, E), dtype=torch.float32, device="cuda")
                out = torch.empty((L, 1, H), dtype=torch.int16, device="cuda")
                tok = torch.zeros(1, dtype=torch.int64, device="cuda")
                graph = capture(torch, lay, x_st, lg_st, out, (x_all, lg_all, tok))
                for _ in range(n_warm):
                    graph.replay()
                torch.cuda.synchronize()
                st0 = m.moe_cache_stats(lay.cache)
                t0 = time.perf_counter()
                toks = leg_tokens(n_warm, n_tok)
                for _ in toks:
                    graph.replay()
                torch.cuda.synchronize()
                dt = time.perf_counter() - t0
                d = m.moe_cache_stats(lay.cache) - st0
                n = len(toks)
                fetched = float(d[m.MOE_STAT_MISSED] - d[m.MOE_STAT_OVERFLOW]) / n
                runs.append({"overlap": ov, "value": round(L * n / dt, 1), "ms_per_step": round(dt / n * 1000.0, 4),
                             "misses_per_token": round(fetched, 2),
                             "gathered_gb_per_s": round(fetched * sum(rb) / (dt / n) / 1e9, 2)})
                log(f"[bench] 4-bit decode, schedule {ov}: {runs[-1]}")
                del graph
            finally:
                lay.close()
        # the hybrid step over the same 4-bit experts: the cache warmed by
        # the same tokens (eager layer steps), then the timed tokens again
        # per fetch cap, the CPU routes on host threads
        try:
            lay = build_stack(torch, m, W, seed, overlap=2, fmt=fmt, host=host)
            try:
                out = torch.empty((1, H), dtype=torch.int16, device="cuda")
                for t in range(n_warm):
                    for l in range(L):
                        lay.decode(l, x_all[t, l], lg_all[t, l], K, out)
                torch.cuda.synchronize()
                snap = m.moe_cache_read_state(lay.cache)
                hyb = hybrid_benchmark(torch, m, lay, snap, x_all, lg_all, n_warm, n_tok)
            finally:
                lay.close()
        except Exception as e:   # the schedule runs above stand on their own
            hyb = {"error": f"{type(e).__name__}: {e}"}
            log(f"[bench] 4-bit hybrid: {hyb['error']}")
    finally:
        del host
        release_pinned(torch)
    return {"workload": "the shared-expert decode trace over E2M1 experts (E4M3 per-16 scales, fp32 "
                        "globals): 40 x 256, top-8 + bf16 gated shared expert, H 2048, F 512, 3164 slots",
            "expert_bytes": int(sum(rb)), "tokens": len(leg_tokens(n_warm, n_tok)), "runs": runs,
            "hybrid": hyb}


# The other configurations as whole layer steps (admission, miss gather
# from pinned host memory, routed experts, combine), each step captured as
# a graph: (name, format, layers, experts, slots, H, F, top-k, token rows,
# widths (one-call, query), shared expert, residents before each step).
CONFIG_STEPS = (
    ("tiny decode: 1 layer, 8 experts, top-2, H 64, F 128, 4 slots, 32 steps", 0, 8, 4, 64, 128, 2, 1,
     (256, 128), False, None),
    ("tiny decode + gated shared expert (F 128)", 0, 8, 4, 64, 128, 2, 1, (256, 128), True, None),
    ("wide decode bf16: 150 rows x top-2 over 160 experts, 7 resident, 160 slots, H 1024, F 256", 0, 160,
     160, 1024, 256, 2, 150, (256, 128), False, 7),
    ("wide decode e2m1: 600 rows x top-2 over 160 experts, cold 1100 slots, H 1024, F 256", 1, 160, 1100,
     1024, 256, 2, 600, (256, 128), False, 0),
    ("prefill chunk bf16: 42 rows x top-6 over 256 experts, cold 256 slots, H 4096, F 1024", 0, 256, 256,
     4096, 1024, 6, 42, (256, 128), False, 0),
    ("prefill chunk bf16: 50 rows x top-6 over 640 experts, cold 640 slots, H 4096, F 1024", 0, 640, 640,
     4096, 1024, 6, 50, (256, 128), False, 0),
)
CONFIG_REPLAYS = 3
TINY_STEPS = 32


def config_steps_benchmark(torch, m, W, seed=0):
    """Each configuration's layer step.  Tiny: 32 decode steps of the Tiny
    trace (Zipf(1.1) router logits) in one graph, replayed; layer-steps/s.
    Wide and prefill: the step from its stated cache state (restored before
    each replay), one graph per step, HIP events around it; microseconds
    per step and the rate of the miss gather inside it."""
    from expert_slot_cache_moe_amd.layer import SlotCacheLayers

    res = []
    for name, fmt, Ec, Sc, Hc, Fc, Kc, T, (one, qw), shared, residents in CONFIG_STEPS:
        g = W.rng(seed, "bench", "config", name)
        host = [[W.pinned_copy(b) for b in W.device_expert_rows(fmt, (seed, "config", name), Ec, Hc, Fc)]]
        sh = None
        if shared:
            sh = [(W.normal_bf16(g, 2 * Fc * Hc, 0.02), W.normal_bf16(g, Hc * Fc, 0.02),
                   W.normal_bf16(g, Hc, 0.02))]
        lay = SlotCacheLayers(layers=1, experts=Ec, slots=Sc, hidden=Hc, ffn=Fc, fmt=fmt, host_rows=host,
                              shared=sh, max_tokens=T, max_top_k=Kc, overlap=2, one_call_width=one,
                              query_width=qw, max_routes=max(T * Kc, 1))
        try:
            stream = torch.cuda.Stream()
            rb = m.moe_bank_row_bytes(fmt, Hc, Fc)
            if T == 1:
                lgs = torch.from_numpy(W.tiny_logits(seed, TINY_STEPS)).cuda()
                xs = torch.from_numpy(W.normal_bf16(g, (TINY_STEPS, 1, Hc)).view(np.int16)).cuda()
                out = torch.empty((TINY_STEPS, 1, Hc), dtype=torch.int16, device="cuda")
                graph = torch.cuda.CUDAGraph()
                with torch.cuda.graph(graph, stream=stream):
                    for t in range(TINY_STEPS):
                        lay.decode(0, xs[t], lgs[t], Kc, out[t])
                for _ in range(3):
                    graph.replay()
                torch.cuda.synchronize()
                st0 = m.moe_cache_stats(lay.cache)
                reps = 20
                t0 = time.perf_counter()
                for _ in range(reps):
                    graph.replay()
                torch.cuda.synchronize()
                dt = time.perf_counter() - t0
                d = m.moe_cache_stats(lay.cache) - st0
                n = reps * TINY_STEPS
                res.append({"workload": name, "value": round(n / dt, 1), "unit": "layer-steps/s",
                            "us_per_step": round(dt / n * 1e6, 2),
                            "misses_per_step": round(float(d[m.MOE_STAT_MISSED]) / n, 3)})
            else:
                if fmt == 0 and residents:
                    chosen = W.wide_bf16_routes(seed)
                else:
                    chosen = np.stack([g.choice(Ec, Kc, replace=False) for _ in range(T)])
                lg = torch.from_numpy(W.forced_logits(g, chosen, Ec)).cuda()
                x = torch.from_numpy(W.normal_bf16(g, (T, Hc)).view(np.int16)).cuda()
                out = torch.empty((T, Hc), dtype=torch.int16, device="cuda")
                if residents:
                    pre = torch.from_numpy(g.permutation(Ec)[:residents].astype(np.int32)).cuda()
                    m.moe_admit(lay.cache, 0, pre)
                    m.moe_gather_misses(lay.cache)
                torch.cuda.synchronize()
                snap = m.moe_cache_read_state(lay.cache)
                graph = torch.cuda.CUDAGraph()
                with torch.cuda.graph(graph, stream=stream):
                    lay.decode(0, x, lg, Kc, out, stream=stream)
                e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                us = []
                for r in range(1 + CONFIG_REPLAYS):
                    m.moe_cache_write_state(lay.cache, snap["res"], snap["own"], snap["stamp"], snap["clock"])
                    st0 = m.moe_cache_stats(lay.cache)
                    # the replay runs on the current stream: the events bracket it there
                    e0.record()
                    graph.replay()
                    e1.record()
                    torch.cuda.synchronize()
                    if r:
                        us.append(e0.elapsed_time(e1) * 1000.0)
                    fetched = int((m.moe_cache_stats(lay.cache) - st0)[m.MOE_STAT_MISSED])
                u = float(np.median(us))
                gathered = fetched * sum(rb)
                res.append({"workload": name, "us_per_step": round(u, 1), "value": round(1e6 / u, 2),
                            "unit": "layer-steps/s", "routes": T * Kc, "fetched_experts": fetched,
                            "gathered_bytes": gathered, "gather_inclusive_gb_per_s": round(gathered / u / 1e3, 2)})
            log(f"[bench] config step: {res[-1]}")
        finally:
            lay.close()
            del host
            release_pinned(torch)
    return res


# Oracle admission timing: the admission-only workload's one-layer cache
# (512 experts pre-filled into 2100 slots), single-threaded, µs per
# admission at these batches (10, 480 and 1280 routes).
CPU_ADMISSION_BATCHES = (1, 48, 128)


def cpu_admission_baseline(W, steps=200):
    """The oracle's admission alone (it is sequential), on the same ids the
    GPU admission-only benchmark uses: µs per admission by routes."""
    import oracle

    res = {}
    warm = oracle.OracleCache(1, 512, 2100)      # warm-up (library, caches, clocks), not timed
    warm.admit(0, np.arange(512, dtype=np.int32))
    for i in range(100):
        warm.admit(0, W.admission_ids(i, 48))
    for req in CPU_ADMISSION_BATCHES:
        oc = oracle.OracleCache(1, 512, 2100)
        oc.admit(0, np.arange(512, dtype=np.int32))
        ids = [W.admission_ids(i, req) for i in range(steps)]
        for r in ids[:10]:                       # warm-up, not timed
            oc.admit(0, r)
        t0 = time.perf_counter()
        for r in ids:
            oc.admit(0, r)
        res[str(req * 10)] = round((time.perf_counter() - t0) / steps * 1e6, 2)
    return {"value": res["480"], "unit": "µs/admission at 480 routes", "by_routes": res, "cores": 1,
            "kind": "oracle",
            "sample": f"{steps} admissions per batch size on one cache of 512 experts pre-filled into 2100 "
                      "slots (all hits), single-threaded C oracle"}


def cpu_baseline(W, warm_tokens, sample_tokens, seed=0):
    """The oracle, single-threaded, on tokens [warm, warm + sample) of the
    same trace after replaying the first `warm` tokens' admissions and
    gathers (no math) to reach the same cache state."""
    import oracle

    # the oracle's own host store (timing only): 64 distinct bf16 rows, expert
    # (l, e) holding row (l E + e) 7919 mod 64
    g = W.rng(seed, "bench", "experts")
    distinct = 64
    base = W.bf16_expert_rows(g, distinct, H, F)
    host_idx = lambda l: ((np.arange(l * E, (l + 1) * E) * 7919) % distinct)
    shared = shared_experts(W, seed)
    slots = [np.zeros((S, 4 * F * H), np.uint8), np.zeros((S, 2 * F * H), np.uint8)]
    tr = W.DecodeTrace(seed, L, E, K)
    gx = W.rng(seed, "bench", "hidden")
    oc = oracle.OracleCache(L, E, S)
    for t in range(warm_tokens):
        sets = tr.step_sets()
        lg = tr.logits(sets)
        W.normal_bf16(gx, (L, 1, H))
        for l in range(L):
            ids, _ = oracle.topk(lg[l:l + 1], K)
            oc.admit(l, ids.reshape(-1))
            for s, e in zip(oc.plan_slot, oc.plan_expert):
                r = host_idx(l)[e]
                slots[0][s] = base[0][r]
                slots[1][s] = base[1][r]
    pool = oracle.Pool(0, H, F, slots)
    n = 0
    steps = []
    t0 = time.perf_counter()
    for t in range(sample_tokens):
        sets = tr.step_sets()
        lg = tr.logits(sets)
        xs = W.normal_bf16(gx, (L, 1, H))
        for l in range(L):
            ids, w = oracle.topk(lg[l:l + 1], K)
            sl = oc.admit(l, ids.reshape(-1)).reshape(1, K)
            # the layer's host rows are base rows host_idx(l)[expert]
            oracle.gather(base, slots, oc.plan_slot, host_idx(l)[oc.plan_expert].astype(np.int32))
            _, add = oracle.shared(H, F, *shared[l], xs[l])
            oracle.routed(pool, sl, w, xs[l], addend=add)
            steps.append((l, lg[l:l + 1].copy(), xs[l].copy()))
            n += 1
    dt = time.perf_counter() - t0

    # The layer math of the same layer-steps (top-k, shared expert, routed
    # experts over the host store: the same bytes the slots hold) on every
    # host core: one layer-step per task, the oracle's calls release the
    # interpreter lock; each dot product stays sequential.
    from concurrent.futures import ThreadPoolExecutor

    hpool = oracle.Pool(0, H, F, base)

    def layer_math(st):
        l, lgl, x = st
        ids, w = oracle.topk(lgl, K)
        _, add = oracle.shared(H, F, *shared[l], x)
        return oracle.routed(hpool, host_idx(l)[ids].astype(np.int32), w, x, addend=add)

    cores = len(os.sched_getaffinity(0))
    t1 = time.perf_counter()
    with ThreadPoolExecutor(cores) as ex:
        list(ex.map(layer_math, steps))
    dt_all = time.perf_counter() - t1
    return {"value": round(n / dt, 3), "unit": "layer-steps/s", "cores": 1, "kind": "oracle",
            "sample": f"{n} layer-steps ({sample_tokens} tokens x {L} layers) of the shared-expert "
                      f"decode trace after {warm_tokens} tokens of admission+gather warm-up; "
                      f"single-threaded C oracle (double precision), {dt:.1f} s",
            "all_cores": {"value": round(n / dt_all, 3), "unit": "layer-steps/s", "cores": cores,
                          "kind": "oracle",
                          "sample": f"the layer math of the same {n} layer-steps (top-k, shared expert, "
                                    f"routed experts; no admission or gather), one layer-step per "
                                    f"thread task, {dt_all:.1f} s"},
            "host": host_description()}


def host_description() -> dict:
    """CPU model, logical CPUs (and those this process may use) and RAM of
    the machine the baseline ran on."""
    model = "unknown"
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                model = line.split(":", 1)[1].strip()
                break
    except OSError:
        pass
    mem = 0
    try:
        for line in open("/proc/meminfo"):
            if line.startswith("MemTotal"):
                mem = int(line.split()[1]) * 1024
                break
    except OSError:
        pass
    return {"cpu_model": model, "nproc": os.cpu_count(), "usable_cpus": len(os.sched_getaffinity(0)),
            "ram_gb": round(mem / 2 ** 30, 1)}


DECODE_KERNELS = ("admit_fast_kernel", "admit_kernel", "topk_kernel", "stage1_kernel", "stage2_kernel",
                  "gather_kernel", "up_kernel", "down_d_kernel", "down_fused_kernel",
                  "group_count_kernel", "up_mfma_kernel", "down_mfma_kernel", "up_x_kernel",
                  "down_x_kernel", "combine_kernel", "combine8_kernel", "prefetch_kernel")


def _short(name: str) -> str:
    for k in DECODE_KERNELS:
        if k in name:
            return k
    return ""


def _read_dispatches(path, value_col=None):
    import csv

    out = []
    with open(path) as f:
        for r in csv.DictReader(f):
            k = _short(r["Kernel_Name"])
            d = {"id": int(r["Dispatch_Id"]), "k": k, "name": r["Kernel_Name"]}
            if "Start_Timestamp" in r and r["Start_Timestamp"]:
                d["us"] = (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1000.0
            if value_col:
                if r.get("Counter_Name") != value_col:
                    continue
                d["v"] = float(r["Counter_Value"])
            out.append(d)
    out.sort(key=lambda d: d["id"])
    return out


def _split(log, moe):
    """The moe dispatches of a bench run, in submission order, cut into
    (timed layer steps, instrumented layer steps, routed-GEMV calls): a
    staged layer step is admission, stage 1, stage 2; a routed-GEMV call is
    stage 1, stage 2."""
    L, W_, K_ = log["layers"], log.get("warm_tokens", log["warmup"]), log["steps"]
    n_steps = (W_ + 2 * K_) * L
    dec = moe[:3 * n_steps]
    steps = [dec[i:i + 3] for i in range(0, len(dec), 3)]
    ok = len(steps) == n_steps and all(
        [d["k"] for d in st] == ["admit_fast_kernel", "stage1_kernel", "stage2_kernel"] for st in steps)
    if not ok:
        raise SystemExit("trace does not hold the staged decode launches the run made")
    g = moe[3 * n_steps:3 * n_steps + 2 * log["gemv_calls"]]
    calls = [g[i:i + 2] for i in range(0, len(g), 2)]
    if len(calls) != log["gemv_calls"] or any([d["k"] for d in c] != ["stage1_kernel", "stage2_kernel"]
                                              for c in calls):
        raise SystemExit("trace does not hold the routed-GEMV launches the run made")
    return steps[W_ * L:(W_ + K_) * L], steps[(W_ + K_) * L:], calls


def _wide_calls(log, moe):
    """Per wide shape, its timed calls' dispatches (grouping, gate/up, down,
    combine), following the decode and routed-GEMV phases."""
    L, W_, K_ = log["layers"], log.get("warm_tokens", log["warmup"]), log["steps"]
    pos = 3 * (W_ + 2 * K_) * L + 2 * log["gemv_calls"]
    out = []
    # grouping, gate/up (bf16, or the LDS-staged 4-bit kernel), down, combine
    # (one output per thread, or eight for aligned outputs)
    kinds = [("group_count_kernel",), ("up_mfma_kernel", "up_x_kernel"), ("down_mfma_kernel", "down_x_kernel"),
             ("combine_kernel", "combine8_kernel")]
    for wcfg in log.get("wide") or []:
        seq = moe[pos:pos + 4 * wcfg["calls"]]
        pos += 4 * wcfg["calls"]
        calls = [seq[i:i + 4] for i in range(0, len(seq), 4)]
        if len(calls) != wcfg["calls"] or any(not all(d["k"] in ks for d, ks in zip(c, kinds)) for c in calls):
            raise SystemExit("trace does not hold the wide-step launches the run made")
        out.append((wcfg["workload"], calls[-wcfg["timed_calls"]:]))
    return out


def stage1_expected_bytes(fetched):
    """Bytes a fetching stage-1 launch must move: each fetched expert's row
    read over the host link and written to its slot (its gate/up dots are
    taken from the stream), the gate/up rows of the other routes and of
    the shared expert read from HBM, and x."""
    fetched = np.asarray(fetched, np.float64)
    return 2 * fetched * ROW_BYTES + (K - fetched) * 4 * F * H + 4 * F * H + 2 * H


def summarize_trace(csv_path, log_path):
    log = json.load(open(log_path))
    disp = _read_dispatches(csv_path)
    timed, inst, calls = _split(log, [d for d in disp if d["k"]])
    fetched = np.asarray(log["fetched"])
    line = log.get("line", {})
    out = []
    p = out.append
    p(f"# Kernel durations: {log['workload']}\n")
    p("Command (repository root, MI355X):\n")
    p(f"    {log['trace_command']}\n")
    p("Summarised by `python3 bench.py --summarize-trace <kernel_trace.csv> --launch-log <log>`.")
    p(f"The run made {log['warmup']} warm-up tokens, {log['steps']} timed tokens (graph replays, no "
      f"events), an instrumented pass over the same {log['steps']} tokens from the same cache state "
      f"(HIP events captured around each layer's launches), {log['layers']} layer steps per token, "
      f"then the routed-GEMV phase ({log['gemv_calls']} moe_routed_decode calls over resident slots, "
      f"the last {log['gemv_timed_calls']} timed), the admission-only benchmark"
      + (", and the look-ahead runs (the timed tokens again per predictor accuracy)"
         if (line.get("lookahead") if (line := log.get("line", {})) else None) else "") + ".\n")
    stats = csv_path.replace("kernel_trace.csv", "kernel_stats.csv")
    if stats != csv_path and os.path.exists(stats):
        import csv

        p("## All launches: rocprofv3 --stats (kernel_stats.csv)\n")
        p("| kernel | calls | total ms | mean µs | min µs | max µs |")
        p("|---|---|---|---|---|---|")
        for r in csv.DictReader(open(stats)):
            nm = _short(r["Name"]) or r["Name"].split("(")[0].replace("void ", "")[:60]
            p(f"| {nm} | {r['Calls']} | {float(r['TotalDurationNs']) / 1e6:.2f} | "
              f"{float(r['AverageNs']) / 1e3:.2f} | {float(r['MinNs']) / 1e3:.2f} | "
              f"{float(r['MaxNs']) / 1e3:.2f} |")
        p("")

    def dur(steps, i):
        return np.asarray([st[i]["us"] for st in steps])

    hit, miss = fetched == 0, fetched > 0
    rl, rg = line.get("roofline", {}), line.get("roofline_gemv", {})
    tok = np.asarray([sum(d["us"] for st in timed[i:i + log["layers"]] for d in st)
                      for i in range(0, len(timed), log["layers"])])
    p("## The bench line's figures\n")
    p("| figure | launches | rocprofv3 mean µs | bench (HIP events) µs |")
    p("|---|---|---|---|")
    p(f"| stage1_kernel in layer steps that fetched, instrumented pass (roofline) | {int(miss.sum())} | "
      f"{dur(inst, 1)[miss].mean():.2f} | {rl.get('avg_launch_us')} |")
    gc = np.asarray([c[0]["us"] + c[1]["us"] for c in calls])[-log["gemv_timed_calls"]:]
    p(f"| stage1_kernel + stage2_kernel per moe_routed_decode call, routed-GEMV phase (roofline_gemv) | "
      f"{len(gc)} | {gc.mean():.2f} | {rg.get('avg_launch_us')} |")
    p(f"| decode kernels per timed token (ms) | {len(tok)} | {tok.mean() / 1000:.4f} | "
      f"{line.get('ms_per_step')} (ms_per_step) |")
    wl = {r["workload"]: r for r in (line.get("routed_gemv_wide") or [])}
    for name, wc in _wide_calls(log, [d for d in disp if d["k"]]):
        tot = np.asarray([sum(d["us"] for d in c) for c in wc])
        parts = " + ".join(f"{np.mean([c[i]['us'] for c in wc]):.2f}" for i in range(4))
        names = " + ".join(d["k"].replace("_kernel", "") for d in wc[0])
        p(f"| routed GEMV, {name}: {names} ({parts}) | {len(wc)} | "
          f"{tot.mean():.2f} | {wl.get(name, {}).get('us_per_call')} |")
    p("")
    pfd = [d for d in disp if d["k"] == "prefetch_kernel"]
    pf = [d["us"] for d in pfd]
    if pf:
        # each prefetch is followed by its copy; the other schedules' gathers come later
        lo, hi = pfd[0]["id"], pfd[-1]["id"]
        pg = [d["us"] for d in disp if d["k"] == "gather_kernel" and lo < d["id"] <= hi + 2]
        p("## Look-ahead runs (each layer step followed by a prefetch of the next layer)\n")
        p("| launch | launches | rocprofv3 mean µs | max µs |")
        p("|---|---|---|---|")
        p(f"| prefetch_kernel (victims, LFRU guard, fill plan) | {len(pf)} | {np.mean(pf):.2f} | "
          f"{np.max(pf):.2f} |")
        if pg:
            p(f"| gather_kernel on the prefetch stream (copies of the fills) | {len(pg)} | "
              f"{np.mean(pg):.2f} | {np.max(pg):.2f} |")
        for r in line.get("lookahead") or []:
            p(f"\nPredictor accuracy {r['predictor_accuracy']}: {r['value']} layer-steps/s "
              f"({r['ms_per_step']} ms per token), {r['demand_fetches_per_token']} demand fetches, "
              f"{r['prefetch_fills_per_token']} prefetch fills and {r['prefetch_drops_per_token']} "
              "drops per token.")
        p("")
    if line.get("hybrid"):
        hy = line["hybrid"]
        p(f"## Hybrid CPU/GPU steps (eager, {hy['threads']} host threads, the first {hy['tokens']} timed "
          "tokens again from the same cache state; wall time)\n")
        p("| fetch cap | layer-steps/s | ms per token | fetches per token | CPU routes per token |")
        p("|---|---|---|---|---|")
        for r in hy["runs"]:
            p(f"| {r['fetch_cap']} | {r['value']} | {r['ms_per_step']} | {r['fetches_per_token']} | "
              f"{r['cpu_routes_per_token']} |")
        p("")
    if line.get("schedules"):
        p("## Other layer-step schedules (the timed tokens again, same cache state; wall time)\n")
        p("| overlap | schedule | layer-steps/s | ms per token |")
        p("|---|---|---|---|")
        p(f"| 2 (default, the line's value) | gather, shared expert and resident routes as disjoint "
          f"workgroups of one launch; down projections and combine in a second | {line.get('value')} | "
          f"{line.get('ms_per_step')} |")
        for r in line["schedules"]:
            p(f"| {r['overlap']} | {r['schedule']} | {r['value']} | {r['ms_per_step']} |")
        p("")
    p("The roofline interval is read between event-record nodes captured around the launch in the "
      f"graph ({rl.get('avg_launch_us_events')} µs); the nodes add their own processing to it, "
      f"which an empty pair of nodes recorded before every layer step measures "
      f"({rl.get('empty_event_pair_us')} µs) and the bench takes off.  The routed-GEMV "
      "figure is one event pair inside the graph around its 160 calls, divided by the calls.  "
      "ms_per_step is wall time over the timed replays (it also holds the per-token input "
      "copies).\n")
    p("## The timed tokens by kind of layer step (graph replays, no events; rocprofv3 only)\n")
    p("The timed and instrumented passes replay the same tokens from the same cache state, so "
      "each layer step has the same fetch count in both.\n")
    p("| launch | launches | rocprofv3 mean µs |")
    p("|---|---|---|")
    p(f"| admit_fast_kernel (admission + fused top-k) | {len(timed)} | {dur(timed, 0).mean():.2f} |")
    p(f"| stage1_kernel, layer steps that fetched | {int(miss.sum())} | {dur(timed, 1)[miss].mean():.2f} |")
    p(f"| stage1_kernel, all-hit layer steps | {int(hit.sum())} | {dur(timed, 1)[hit].mean():.2f} |")
    p(f"| stage2_kernel, all layer steps | {len(timed)} | {dur(timed, 2).mean():.2f} |")
    p(f"| stage1 + stage2, all-hit layer steps (8 routed + shared expert) | {int(hit.sum())} | "
      f"{(dur(timed, 1) + dur(timed, 2))[hit].mean():.2f} |")
    p("")
    d4 = line.get("decode_4bit") if line else None
    if d4 and "runs" in d4:
        # the 4-bit leg runs schedule 2 first (warm-up tokens, then the timed
        # ones; its token graphs hold admission, stage 1 and stage 2 of the
        # E2M1 kernels), then schedule 0
        Lx = log["layers"]
        n = d4["tokens"] * Lx
        w0 = log.get("warm_tokens", log["warmup"]) * Lx
        st = {k: [d["us"] for d in disp if d["k"] == k and "<1," in d["name"]]
              for k in ("stage1_kernel", "stage2_kernel")}
        if len(st["stage1_kernel"]) >= w0 + n:
            s1 = np.asarray(st["stage1_kernel"][w0:w0 + n])
            s2 = np.asarray(st["stage2_kernel"][w0:w0 + n])
            fetch = s1 > 15.0
            p("## 4-bit decode (E2M1 experts, schedule 2), its timed tokens\n")
            p("| launch | launches | rocprofv3 mean µs |")
            p("|---|---|---|")
            p(f"| stage1_kernel<E2M1>, layer steps that fetched (above 15 µs) | {int(fetch.sum())} | "
              f"{s1[fetch].mean() if fetch.any() else 0:.2f} |")
            p(f"| stage1_kernel<E2M1>, all-hit layer steps | {int((~fetch).sum())} | "
              f"{s1[~fetch].mean() if (~fetch).any() else 0:.2f} |")
            p(f"| stage2_kernel<E2M1>, all layer steps | {len(s2)} | {s2.mean():.2f} |")
            p("")
    if line:
        p("## bench.py line of the same run\n")
        p("    " + json.dumps(line))
    print("\n".join(out))


def summarize_pmc(fetch_csv, write_csv, log_path):
    log = json.load(open(log_path))
    fetched = np.asarray(log["fetched"])
    res = {}
    copy = {}
    for cname, path in (("FETCH_SIZE", fetch_csv), ("WRITE_SIZE", write_csv)):
        disp = _read_dispatches(path, cname)
        copies = [d for d in disp if "copyBuffer" in d["name"]]
        copy[cname] = max(d["v"] for d in copies)    # the 256 MiB device copy is the run's largest
        _, inst, calls = _split(log, [d for d in disp if d["k"]])
        res[cname] = {"stage1_kernel": np.asarray([st[1]["v"] for st in inst]),
                      "admit_fast_kernel": np.asarray([st[0]["v"] for st in inst]),
                      "gemv": np.asarray([c[0]["v"] + c[1]["v"] for c in calls])[-log["gemv_timed_calls"]:]}
    mib = 262144.0                                  # KiB moved each way by the calibration copy
    fs, ws = mib / copy["FETCH_SIZE"], mib / copy["WRITE_SIZE"]
    if not (0.5 <= fs <= 4.0 and 0.5 <= ws <= 4.0):
        raise SystemExit(f"calibration copy not found (scales {fs:.3g}, {ws:.3g})")
    miss = fetched > 0
    f1, w1 = res["FETCH_SIZE"]["stage1_kernel"], res["WRITE_SIZE"]["stage1_kernel"]
    fg, wg = res["FETCH_SIZE"]["gemv"], res["WRITE_SIZE"]["gemv"]
    gather_kib = fetched[miss].mean() * ROW_BYTES / 1024.0
    stage1_kib = stage1_expected_bytes(fetched[miss]).mean() / 1024.0
    gemv_kib = (K * ROW_BYTES + 2 * H * 2 + K * 8) / 1024.0
    miss_traffic = (f1[miss] * fs + w1[miss] * ws).mean()
    gemv_traffic = (fg * fs + wg * ws).mean()
    print(f"""# HBM / host-link traffic of the decode-step kernels: {log['workload']}
#
# Commands (two passes, one counter each, from the repository root):
#   {log['pmc_command'].replace('<C>', 'FETCH_SIZE')}
#   {log['pmc_command'].replace('<C>', 'WRITE_SIZE')}
# Summarised by: python3 bench.py --summarize-pmc <FETCH csv> <WRITE csv> --launch-log <log>
#
# Calibration: the run makes one 256 MiB device-to-device copy, its largest
# (262144 KiB read and 262144 KiB written); its counters read
# FETCH_SIZE = {copy['FETCH_SIZE']:.1f} KiB and WRITE_SIZE = {copy['WRITE_SIZE']:.1f} KiB, so
# fetch_scale = {fs:.3f} and write_scale = {ws:.3f}.
#
# Instrumented pass ({int(miss.sum())} layer steps that fetched) and routed-GEMV phase, mean KiB per launch:
#   stage1_kernel, fetching steps:  FETCH {f1[miss].mean():10.1f}  WRITE {w1[miss].mean():10.1f}
#       gathered bytes (algorithmic): {gather_kib:10.1f} KiB read over the host link, same written
#       all bytes the launch must move: {stage1_kib:10.1f} KiB (gathered rows read and written, gate/up
#       rows of the resident routes and of the shared expert read, x read)
#   routed GEMV (moe_routed_decode, stage1 + stage2, {len(fg)} calls): FETCH {fg.mean():10.1f}  WRITE {wg.mean():10.1f}
#       expert bytes (algorithmic): {gemv_kib:10.1f} KiB (8 routed experts' rows, x, out, ids, weights)
#   admit_fast_kernel:              FETCH {res['FETCH_SIZE']['admit_fast_kernel'].mean():10.1f}  WRITE {res['WRITE_SIZE']['admit_fast_kernel'].mean():10.1f}
#
# Traffic / algorithmic ratios (scaled FETCH + WRITE over algorithmic bytes) used by bench.py:
kernel_sources_sha256_16 = {kernel_sources_hash()}
fetch_scale = {fs:.4f}
write_scale = {ws:.4f}
# fetching stage1 launches: measured over all the bytes the launch must move
gather_traffic_ratio = {miss_traffic / stage1_kib:.4f}
# routed GEMV call (stage1 + stage2)
routed_traffic_ratio = {gemv_traffic / gemv_kib:.4f}""")


def summarize_counters(csv_paths):
    """Mean value per dispatch of every counter of one or more rocprofv3
    --pmc runs, per kernel of the library (template arguments kept: weight
    format, row tiles, slabs ahead), then per wave of the grouped kernels:
    the share of wave cycles stalled on outstanding loads
    (SQ_WAIT_INST_ANY) and issuing VALU, VALU and MFMA instructions."""
    import csv
    import re

    acc = {}
    for path in csv_paths:
        for r in csv.DictReader(open(path)):
            name = r["Kernel_Name"]
            k = _short(name)
            if not k:
                continue
            m_ = re.search(r"<([0-9, ]+)>", name)
            key = k + (f"<{m_.group(1)}>" if m_ else "")
            acc.setdefault(key, {}).setdefault(r["Counter_Name"], []).append(float(r["Counter_Value"]))
    for key in sorted(acc):
        vals = "  ".join(f"{c}={np.mean(v):.4g}" for c, v in sorted(acc[key].items()))
        print(f"{key}  (dispatches {max(len(v) for v in acc[key].values())})  {vals}")
    need = ("SQ_WAVES", "SQ_WAVE_CYCLES", "SQ_WAIT_INST_ANY", "SQ_ACTIVE_INST_VALU", "SQ_INSTS_VALU",
            "SQ_INSTS_MFMA")
    rows = []
    for key in sorted(acc):
        c = {n: np.mean(v) for n, v in acc[key].items()}
        if ("mfma" not in key and "_x_kernel" not in key) or any(n not in c for n in need) or c["SQ_WAVES"] <= 0:
            continue
        rows.append(f"#   {key}: {c['SQ_WAVES']:.0f} waves a dispatch; stalled on outstanding loads "
                    f"{100 * c['SQ_WAIT_INST_ANY'] / c['SQ_WAVE_CYCLES']:.0f}% of wave cycles, VALU issuing "
                    f"{100 * c['SQ_ACTIVE_INST_VALU'] / c['SQ_WAVE_CYCLES']:.0f}%; "
                    f"{c['SQ_INSTS_VALU'] / c['SQ_WAVES']:.0f} VALU and {c['SQ_INSTS_MFMA'] / c['SQ_WAVES']:.0f} "
                    f"MFMA instructions per wave")
    if rows:
        print("#\n# Per wave of the grouped kernels:")
        print("\n".join(rows))


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=256)
    ap.add_argument("--warmup", type=int, default=64)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-admission", action="store_true")
    ap.add_argument("--no-wide", action="store_true", help="skip the wide-step routed GEMV shapes")
    ap.add_argument("--no-lookahead", action="store_true", help="skip the look-ahead prefetch runs")
    ap.add_argument("--no-schedules", action="store_true", help="skip the other layer-step schedules")
    ap.add_argument("--no-hybrid", action="store_true", help="skip the hybrid CPU/GPU runs")
    ap.add_argument("--no-4bit", action="store_true", help="skip the 4-bit decode runs")
    ap.add_argument("--no-configs", action="store_true", help="skip the other configurations' layer steps")
    ap.add_argument("--only-wide", action="store_true",
                    help="run only the wide-step routed GEMV shapes (one JSON line each)")
    ap.add_argument("--summarize-counters", nargs="+", default=None, metavar="COUNTER_CSV",
                    help="per-kernel means of every counter in rocprofv3 --pmc csv files")
    ap.add_argument("--cpu-sample-tokens", type=int, default=6)
    ap.add_argument("--overlap", type=int, default=2,
                    help="layer-step schedule passed to the cache (0 serial, 1 side-stream "
                         "fork/join, 2 two staged launches on one stream)")
    ap.add_argument("--gather-workgroups", type=int, default=0,
                    help="workgroups of the miss-gather kernel (0: the library default)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="end with one 256 MiB device-to-device copy (counter calibration)")
    ap.add_argument("--launch-log", default=None,
                    help="write the timed/instrumented launch layout and the result line here")
    ap.add_argument("--trace-command", default="", help="recorded in the launch log")
    ap.add_argument("--pmc-command", default="", help="recorded in the launch log")
    ap.add_argument("--summarize-trace", default=None, metavar="KERNEL_TRACE_CSV")
    ap.add_argument("--summarize-pmc", nargs=2, default=None, metavar=("FETCH_CSV", "WRITE_CSV"))
    args = ap.parse_args()
    if args.summarize_trace:
        return summarize_trace(args.summarize_trace, args.launch_log)
    if args.summarize_pmc:
        return summarize_pmc(*args.summarize_pmc, args.launch_log)
    if args.summarize_counters:
        return summarize_counters(args.summarize_counters)
    if args.gpus != 1:
        print(f"bench.py measures one GPU: the decode step is data-parallel and the library runs "
              f"on a single MI355X; --gpus {args.gpus} is not supported.", file=sys.stderr)
        sys.exit(2)

    import torch

    import expert_slot_cache_moe_amd as m
    from expert_slot_cache_moe_amd import workloads as W

    m.lib()
    torch.cuda.set_device(0)
    if args.only_wide:
        # the wide-step shapes alone (for counter passes over their kernels)
        for r in wide_gemv_benchmark(torch, m):
            print(json.dumps(r), flush=True)
        return None
    W_, K_ = args.warmup, args.steps
    if K_ < 1:
        raise SystemExit("--steps must be at least 1")
    n_warm, n_tok, first = token_plan(W_, K_)
    lay = build_stack(torch, m, W, gather_workgroups=args.gather_workgroups, overlap=args.overlap)
    t0 = time.time()
    lg_all, x_all = make_trace(torch, W, n_tok)
    log(f"[bench] trace of {n_tok} tokens in {time.time() - t0:.1f}s")
    x_st = torch.empty((L, 1, H), dtype=torch.int16, device="cuda")
    lg_st = torch.empty((L, 1, E), dtype=torch.float32, device="cuda")
    out = torch.empty((L, 1, H), dtype=torch.int16, device="cuda")
    tok = torch.zeros(1, dtype=torch.int64, device="cuda")   # the device-side step counter
    graph = capture(torch, lay, x_st, lg_st, out, (x_all, lg_all, tok))

    def step(t):
        graph.replay()                     # stages token t: the counter holds t

    for t in range(n_warm):                # cache warm-up (and graph warm-up): untimed
        step(t)
    torch.cuda.synchronize()
    log(f"[bench] cache warm-up: {n_warm} tokens")
    snap = m.moe_cache_read_state(lay.cache)
    st0 = m.moe_cache_stats(lay.cache)
    t0 = time.perf_counter()
    for t in range(first, n_tok):
        step(t)
    torch.cuda.synchronize()
    dt = time.perf_counter() - t0
    st1 = m.moe_cache_stats(lay.cache)
    fetched = int((st1[2] - st0[2]) - (st1[3] - st0[3]))
    log(f"[bench] timed {K_} tokens in {dt:.3f}s, {fetched / K_:.1f} misses/token")

    # Same tokens again from the same cache state, with HIP events captured
    # around each layer's launches (event-record nodes of the graph), and
    # each layer's fetch count read after every token, so that layer-steps
    # with misses (host-link bound) and all-hit layer-steps (HBM bound) are
    # told apart.  The nodes add their own processing to an interval (a few
    # microseconds): an empty pair before each layer step measures it, and
    # it is taken off; this pass times only the long launches, the ones
    # that fetch.
    m.moe_cache_write_state(lay.cache, snap["res"], snap["own"], snap["stamp"], snap["clock"])
    m.moe_cache_set_timing(lay.cache, True)
    ids_l = torch.empty((L, 1, K), dtype=torch.int32, device="cuda")
    w_l = torch.empty((L, 1, K), dtype=torch.float32, device="cuda")
    pairs = ([torch.cuda.Event(enable_timing=True) for _ in range(L)],
             [torch.cuda.Event(enable_timing=True) for _ in range(L)])
    for e in pairs[0] + pairs[1]:
        e.record()                              # creates the events before capture
    torch.cuda.synchronize()
    tgraph = capture(torch, lay, x_st, lg_st, out, (x_all, lg_all, tok), ids_l, w_l, pairs)
    tok.fill_(first)
    staged = args.overlap == 2
    k1_ms, pair_ms, fetch_l = [], [], []
    prev = m.moe_cache_read_state(lay.cache)["stats"]
    for t in range(first, n_tok):
        tgraph.replay()
        torch.cuda.synchronize()
        ms = m.moe_cache_timing(lay.cache).astype(np.float64)
        cur = m.moe_cache_read_state(lay.cache)["stats"]
        d = cur - prev
        prev = cur
        fetch_l.append(d[:, m.MOE_STAT_MISSED] - d[:, m.MOE_STAT_OVERFLOW])
        k1_ms.append(ms[:, 1])
        pair_ms.append([pairs[0][l].elapsed_time(pairs[1][l]) for l in range(L)])
    m.moe_cache_set_timing(lay.cache, False)
    log("[bench] instrumented pass done")
    fetch_l = np.concatenate(fetch_l)
    k1_raw = np.concatenate(k1_ms)
    pair_us = float(np.mean(pair_ms)) * 1000.0
    fl = fetch_l > 0
    miss_n = int(fl.sum())
    gat_raw_us = k1_raw[fl].mean() * 1000.0 if miss_n else 0.0
    gat_us = gat_raw_us - pair_us
    gather_bytes = fetch_l[fl].mean() * ROW_BYTES if miss_n else 0.0
    gather_gbs = gather_bytes / (gat_us * 1e-6) / 1e9 if miss_n else 0.0

    # The routed GEMV alone (moe_routed_decode: the same two stage launches
    # without a miss plan or a shared expert) over the last token's slots,
    # one call per layer, GEMV_PASSES passes over the 40 layers in one graph
    # with an event-record node before and after them: the calls between
    # the two nodes run back to back, and a call's 8 experts were last read
    # 39 calls (2 GB) earlier, so they come from HBM, not from the 256 MB
    # last-level cache.
    pool = m.moe_cache_pool(lay.cache)
    ws = torch.empty(m.moe_routed_workspace_bytes(0, H, F, 1, K), dtype=torch.uint8, device="cuda")
    gout = torch.empty((L, 1, H), dtype=torch.int16, device="cuda")
    xg = x_all[n_tok - 1].clone()
    gstream = torch.cuda.Stream()
    ggraph = torch.cuda.CUDAGraph()
    g0 = torch.cuda.Event(enable_timing=True)
    g1 = torch.cuda.Event(enable_timing=True)
    g0.record(gstream)
    g1.record(gstream)
    torch.cuda.synchronize()
    with torch.cuda.graph(ggraph, stream=gstream):
        # a few milliseconds of spin first: the host enqueues the graph's
        # nodes one by one, and the routed calls (~15 us each) are shorter
        # than that, so without a head start it would feed them with gaps
        torch.cuda._sleep(GEMV_HEAD_START_CYCLES)
        m.moe_record_event(g0, gstream)
        for _ in range(GEMV_PASSES):
            for l in range(L):
                m.moe_routed_decode(pool, xg[l], ids_l[l], w_l[l], gout[l], ws, stream=gstream)
        m.moe_record_event(g1, gstream)
    per_call = []
    for r in range(1 + GEMV_REPLAYS):
        ggraph.replay()
        torch.cuda.synchronize()
        if r > 0:
            per_call.append(g0.elapsed_time(g1) * 1000.0 / (GEMV_PASSES * L))
    rout_us = float(np.mean(per_call))
    log(f"[bench] routed-GEMV phase: {rout_us:.2f} us per call")
    assert (ids_l >= 0).all(), "the GEMV phase reads resident slots only"
    gemv_bytes = K * ROW_BYTES + 2 * H * 2 + K * 8     # 8 experts' rows, x and out, ids and weights
    gemv_gbs = gemv_bytes / (rout_us * 1e-6) / 1e9

    # host-link ceiling: a pinned hipMemcpyAsync of the same size
    nbytes = max(int(round(gather_bytes)), ROW_BYTES)
    src = torch.empty(nbytes, dtype=torch.uint8, pin_memory=True)
    dst = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    for _ in range(2):
        dst.copy_(src, non_blocking=True)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(5):
        dst.copy_(src, non_blocking=True)
    e1.record()
    torch.cuda.synchronize()
    h2d_gbs = 5 * nbytes / (e0.elapsed_time(e1) * 1e-3) / 1e9
    del src, dst

    # HBM ceiling at the routed step's size: a device-to-device copy that
    # reads and writes half of the expert bytes each
    half = gemv_bytes // 2
    a = torch.empty(half, dtype=torch.uint8, device="cuda")
    b = torch.empty_like(a)
    rot = [torch.empty(256 << 20, dtype=torch.uint8, device="cuda") for _ in range(2)]
    best = float("inf")
    for i in range(12):
        rot[i % 2].zero_()                         # evicts the previous copy from the caches
        e0.record()
        b.copy_(a)
        e1.record()
        torch.cuda.synchronize()
        if i >= 2:
            best = min(best, e0.elapsed_time(e1))
    d2d_gbs = 2 * half / (best * 1e-3) / 1e9
    del a, b, rot

    if args.copy_calibration:
        a = torch.empty(256 << 20, dtype=torch.uint8, device="cuda")
        b = torch.empty_like(a)
        torch.cuda.synchronize()
        b.copy_(a)
        torch.cuda.synchronize()
        del a, b
    # The headline, its roofline and the routed-GEMV figure are in hand;
    # every side leg below reports an error field instead of raising.
    wide = None if args.no_wide else run_leg("wide", wide_gemv_benchmark, torch, m)
    adm = None if args.no_admission else run_leg("admission", admission_benchmark, torch, m, W)
    adm_chunked = None if args.no_admission else run_leg(
        "admission chunked", admission_benchmark, torch, m, W, one_call_width=128,
        batches=ADMISSION_CHUNKED_BATCHES)
    look = None if args.no_lookahead else run_leg(
        "look-ahead", lookahead_benchmark, torch, m, lay, snap, x_all, lg_all, first, n_tok)
    look_rest = None if args.no_lookahead else run_leg(
        "look-ahead with the rest of the layer", lookahead_rest_benchmark, torch, m, lay, snap, x_all, lg_all,
        first, n_tok)
    sched = (None if args.no_schedules or args.overlap != 2
             else run_leg("schedules", schedule_benchmark, torch, m, lay, snap, x_all, lg_all, first, n_tok))
    hyb = None if args.no_hybrid else run_leg(
        "hybrid", hybrid_benchmark, torch, m, lay, snap, x_all, lg_all, first, n_tok)
    lay.close()
    del lay
    release_pinned(torch)
    dec4 = None if args.no_4bit else run_leg(
        "4-bit decode", decode_4bit_benchmark, torch, m, W, x_all, lg_all, n_warm, n_tok)
    steps_cfg = None if args.no_configs else run_leg("config steps", config_steps_benchmark, torch, m, W)
    cpu = None
    if not args.no_cpu_baseline:
        cpu = run_leg("cpu baseline", cpu_baseline, W, n_warm, args.cpu_sample_tokens)
        if "error" not in cpu:
            cpu["admission"] = run_leg("cpu admission baseline", cpu_admission_baseline, W)

    ratios = traffic_ratios()
    value = L * K_ / dt
    workload = ("shared-expert decode: 40 layers x 256 experts, top-8 + gated shared expert, hidden "
                "2048, expert FFN 512, bf16 weights in pinned host memory, 3164-slot cache, batch 1, "
                "Zipf(1.05) routing with temporal locality; one step = one token = 40 layer-steps in "
                "one hipGraph")
    line = {
        "metric": "decode MoE layer-steps/s; admission µs/layer; routed GEMV HBM GB/s vs peak",
        "value": round(value, 1),
        "unit": "layer-steps/s",
        "n_gpus": 1,
        "steps": K_,
        "warmup": W_,
        "ms_per_step": round(dt / K_ * 1000.0, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": workload,
                   "layers": L, "experts": E, "top_k": K, "hidden": H, "ffn": F, "slots": S,
                   "batch": 1, "cache_warm_tokens": n_warm, "misses_per_token": round(fetched / K_, 2)},
        "roofline": {"kernel": ("stage1_kernel (miss gather + gate/up), layer-steps with misses" if staged
                                else "gather_kernel (miss gather, pinned host -> device slots)"),
                     "bound": "host-link", "achieved": round(gather_gbs, 2),
                     "peak": HOST_LINK_PEAK_GBS, "unit": "GB/s",
                     "frac": round(gather_gbs / HOST_LINK_PEAK_GBS, 4),
                     "traffic": (round(stage1_expected_bytes(fetch_l[fl]).mean() * ratios["gather_traffic_ratio"])
                                 if ratios and miss_n else None),
                     "traffic_expected": round(stage1_expected_bytes(fetch_l[fl]).mean()) if miss_n else None,
                     "bytes_per_launch": round(gather_bytes), "avg_launch_us": round(gat_us, 2),
                     "launches": miss_n, "memcpy_h2d_same_size_gbs": round(h2d_gbs, 2),
                     "avg_launch_us_events": round(gat_raw_us, 2), "empty_event_pair_us": round(pair_us, 2)},
        "roofline_gemv": {"kernel": "stage1_kernel + stage2_kernel as moe_routed_decode: 8 resident routed "
                                    "experts of one token (gate/up, then down + combine)",
                          "bound": "hbm",
                          "achieved": round(gemv_gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                          "frac": round(gemv_gbs / HBM_PEAK_GBS, 4),
                          "traffic": round(gemv_bytes * ratios["routed_traffic_ratio"]) if ratios else None,
                          "bytes_per_launch": gemv_bytes, "avg_launch_us": round(rout_us, 2),
                          "launches": GEMV_REPLAYS * GEMV_PASSES * L,
                          "d2d_copy_same_bytes_gbs": round(d2d_gbs, 1)},
        "admission_us": adm,
        "admission_us_one_call_width_128": adm_chunked,
        "routed_gemv_wide": wide,
        "lookahead": look,
        "lookahead_with_rest": look_rest,
        "schedules": sched,
        "hybrid": hyb,
        "decode_4bit": dec4,
        "config_steps": steps_cfg,
        "cpu_baseline": cpu,
    }
    print(json.dumps(line), flush=True)
    if args.launch_log:
        with open(args.launch_log, "w") as f:
            json.dump({"workload": workload, "layers": L, "warmup": W_, "warm_tokens": n_warm, "steps": K_,
                       "overlap": args.overlap, "fetched": fetch_l.astype(int).tolist(),
                       "gemv_calls": (1 + GEMV_REPLAYS) * GEMV_PASSES * L,
                       "gemv_timed_calls": GEMV_REPLAYS * GEMV_PASSES * L,
                       "wide": None if wide is None else [
                           {"workload": r["workload"], "calls": (1 + WIDE_REPLAYS) * WIDE_SETS,
                            "timed_calls": WIDE_REPLAYS * WIDE_SETS} for r in wide],
                       "trace_command": args.trace_command, "pmc_command": args.pmc_command,
                       "line": line}, f)


if __name__ == "__main__":
    main()
