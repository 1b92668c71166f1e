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
                 graph, 40 replays, microseconds per admission by routes.
  cpu_baseline   the oracle (plain C, one thread) on a bounded sample of
                 the same decode workload.
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


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def kernel_sources_hash() -> str:
    import glob
    import hashlib

    h = hashlib.sha256()
    for f in sorted(glob.glob(os.path.join(ROOT, "expert_slot_cache_moe_amd", "csrc", "*"))):
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


def build_stack(torch, m, W, seed=0, gather_workgroups=0, overlap=1):
    """Pinned host store for 40 x 256 experts, shared experts, the cache."""
    from expert_slot_cache_moe_amd.layer import SlotCacheLayers

    t0 = time.time()
    g = W.rng(seed, "bench", "experts")
    distinct = 64
    base = [torch.from_numpy(b) for b in W.bf16_expert_rows(g, distinct, H, F)]
    rb = m.moe_bank_row_bytes(0, H, F)
    host = []
    for l in range(L):
        idx = (torch.arange(l * E, (l + 1) * E) * 7919) % distinct
        banks = []
        for b in range(2):
            t = torch.empty((E, rb[b]), dtype=torch.uint8, pin_memory=True)
            torch.index_select(base[b], 0, idx, out=t)
            banks.append(t)
        host.append(banks)
    log(f"[bench] pinned host store {L * E * ROW_BYTES / 1e9:.1f} GB in {time.time() - t0:.1f}s")
    gs = W.rng(seed, "bench", "shared")
    shared = [(W.normal_bf16(gs, 2 * F * H, 0.02), W.normal_bf16(gs, H * F, 0.02),
               W.normal_bf16(gs, H, 0.02)) for _ in range(L)]
    lay = SlotCacheLayers(layers=L, experts=E, slots=S, hidden=H, ffn=F, host_rows=host,
                          shared=shared, max_tokens=1, max_top_k=K, overlap=overlap,
                          gather_workgroups=gather_workgroups)
    return lay


def make_trace(torch, W, n, seed=0):
    tr = W.DecodeTrace(seed, L, E, K)
    gx = W.rng(seed, "bench", "hidden")
    lg = np.empty((n, L, 1, E), np.float32)
    xs = np.empty((n, L, 1, H), np.uint16)
    for t in range(n):
        lg[t, :, 0, :] = tr.logits(tr.step_sets())
        xs[t] = W.normal_bf16(gx, (L, 1, H))
    return (torch.from_numpy(lg).cuda(), torch.from_numpy(xs.view(np.int16)).cuda())


def capture(torch, lay, x_st, lg_st, out):
    stream = torch.cuda.Stream()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=stream):
        for l in range(L):
            lay.decode(l, x_st[l], lg_st[l], K, out[l])
    return graph


def admission_benchmark(torch, m, W, replays=40, layers=48):
    res = {}
    caches = [m.moe_cache_create(num_layers=1, num_experts=512, num_slots=2100, max_routes=1280)
              for _ in range(layers)]
    try:
        full = torch.arange(512, dtype=torch.int32, device="cuda")
        for c in caches:
            m.moe_admit(c, 0, full.clone())
        torch.cuda.synchronize()
        for req in W.ADMISSION_BATCHES:
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


def cpu_baseline(W, warm_tokens, sample_tokens, seed=0):
    """The oracle, single-threaded, on tokens [warm, warm + sample) of the
    same trace after replaying the first `warm` tokens' admissions and
    gathers (no math) to reach the same cache state."""
    import oracle

    g = W.rng(seed, "bench", "experts")
    distinct = 64
    base = W.bf16_expert_rows(g, distinct, H, F)
    host_idx = lambda l: ((np.arange(l * E, (l + 1) * E) * 7919) % distinct)
    gs = W.rng(seed, "bench", "shared")
    shared = [(W.normal_bf16(gs, 2 * F * H, 0.02), W.normal_bf16(gs, H * F, 0.02),
               W.normal_bf16(gs, H, 0.02)) for _ in range(L)]
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
            n += 1
    dt = time.perf_counter() - t0
    return {"value": round(n / dt, 3), "unit": "layer-steps/s", "cores": 1, "kind": "oracle",
            "sample": f"{n} layer-steps ({sample_tokens} tokens x {L} layers) of the shared-expert "
                      f"decode trace after {warm_tokens} tokens of admission+gather warm-up; "
                      f"single-threaded C oracle (double precision), {dt:.1f} s"}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=256)
    ap.add_argument("--warmup", type=int, default=64)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-admission", action="store_true")
    ap.add_argument("--cpu-sample-tokens", type=int, default=6)
    ap.add_argument("--overlap", type=int, default=2,
                    help="layer-step schedule passed to the cache (0 serial, 1 side-stream "
                         "fork/join, 2 two staged launches on one stream)")
    ap.add_argument("--gather-workgroups", type=int, default=0,
                    help="workgroups of the miss-gather kernel (0: the library default)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="end with one 256 MiB device-to-device copy (counter calibration)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU: the decode step is data-parallel and this build runs "
              f"on a single MI355X; --gpus {args.gpus} is not supported.", file=sys.stderr)
        sys.exit(2)

    import torch

    import expert_slot_cache_moe_amd as m
    from expert_slot_cache_moe_amd import workloads as W

    m.lib()
    torch.cuda.set_device(0)
    W_, K_ = args.warmup, args.steps
    lay = build_stack(torch, m, W, gather_workgroups=args.gather_workgroups, overlap=args.overlap)
    n_tok = W_ + K_
    t0 = time.time()
    lg_all, x_all = make_trace(torch, W, n_tok)
    log(f"[bench] trace of {n_tok} tokens in {time.time() - t0:.1f}s")
    x_st = torch.empty((L, 1, H), dtype=torch.int16, device="cuda")
    lg_st = torch.empty((L, 1, E), dtype=torch.float32, device="cuda")
    out = torch.empty((L, 1, H), dtype=torch.int16, device="cuda")
    graph = capture(torch, lay, x_st, lg_st, out)

    def step(t):
        x_st.copy_(x_all[t])
        lg_st.copy_(lg_all[t])
        graph.replay()

    for t in range(W_):
        step(t)
    torch.cuda.synchronize()
    snap = m.moe_cache_read_state(lay.cache)
    st0 = m.moe_cache_stats(lay.cache)
    t0 = time.perf_counter()
    for t in range(W_, n_tok):
        step(t)
    torch.cuda.synchronize()
    dt = time.perf_counter() - t0
    st1 = m.moe_cache_stats(lay.cache)
    fetched = int((st1[2] - st0[2]) - (st1[3] - st0[3]))
    log(f"[bench] timed {K_} tokens in {dt:.3f}s, {fetched / K_:.1f} misses/token")

    # Same tokens again from the same cache state, with HIP events captured
    # around each layer's kernels, and each layer's fetch count read after
    # every token, so that layer-steps with misses (host-link bound) and
    # all-hit layer-steps (HBM bound) are timed apart.
    m.moe_cache_write_state(lay.cache, snap["res"], snap["own"], snap["stamp"], snap["clock"])
    m.moe_cache_set_timing(lay.cache, True)
    tgraph = capture(torch, lay, x_st, lg_st, out)
    staged = args.overlap == 2
    adm_ms = 0.0
    miss_rows, miss_ms, miss_n = 0, 0.0, 0      # layer-steps that fetched
    hit_ms, hit_n = 0.0, 0                      # layer-steps that fetched nothing
    prev = m.moe_cache_read_state(lay.cache)["stats"]
    for t in range(W_, n_tok):
        x_st.copy_(x_all[t])
        lg_st.copy_(lg_all[t])
        tgraph.replay()
        torch.cuda.synchronize()
        ms = m.moe_cache_timing(lay.cache).astype(np.float64)
        cur = m.moe_cache_read_state(lay.cache)["stats"]
        d = cur - prev
        prev = cur
        fetched_l = d[:, m.MOE_STAT_MISSED] - d[:, m.MOE_STAT_OVERFLOW]
        adm_ms += ms[:, 0].sum()
        fl = fetched_l > 0
        miss_rows += int(fetched_l.sum())
        miss_ms += ms[fl, 1].sum()
        miss_n += int(fl.sum())
        hit_n += int((~fl).sum())
        # staged schedule: both stages carry routed work; otherwise only
        # the routed slot does (the gather launch is empty on a hit)
        hit_ms += (ms[~fl, 1] + ms[~fl, 2]).sum() if staged else ms[~fl, 2].sum()
    m.moe_cache_set_timing(lay.cache, False)
    launches = K_ * L
    adm_us = adm_ms / launches * 1000.0
    gat_us = miss_ms / max(miss_n, 1) * 1000.0
    gather_bytes = miss_rows * ROW_BYTES / max(miss_n, 1)
    gather_gbs = gather_bytes / (gat_us * 1e-6) / 1e9 if miss_n else 0.0
    rout_us = hit_ms / max(hit_n, 1) * 1000.0
    experts = K + 1 if staged else K                   # the shared expert rides in the stages
    gemv_bytes = experts * ROW_BYTES + 2 * H * 2 + (E * 4 + H * 4 if staged else H * 4)
    gemv_gbs = gemv_bytes / (rout_us * 1e-6) / 1e9 if hit_n else 0.0

    # host-link ceiling: a pinned hipMemcpyAsync of the same size
    nbytes = max(int(round(miss_rows / max(miss_n, 1))), 1) * ROW_BYTES
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

    if args.copy_calibration:
        a = torch.empty(256 << 20, dtype=torch.uint8, device="cuda")
        b = torch.empty_like(a)
        torch.cuda.synchronize()
        b.copy_(a)
        torch.cuda.synchronize()
        del a, b
    adm = None if args.no_admission else admission_benchmark(torch, m, W)
    lay.close()
    del lay
    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(W, W_, args.cpu_sample_tokens)

    ratios = traffic_ratios()
    value = L * K_ / dt
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
        "config": {"workload": "shared-expert decode: 40 layers x 256 experts, top-8 + gated shared "
                               "expert, hidden 2048, expert FFN 512, bf16 weights in pinned host "
                               "memory, 3164-slot cache, batch 1, Zipf(1.05) routing with temporal "
                               "locality; one step = one token = 40 layer-steps in one hipGraph",
                   "layers": L, "experts": E, "top_k": K, "hidden": H, "ffn": F, "slots": S,
                   "batch": 1, "misses_per_token": round(fetched / K_, 2)},
        "roofline": {"kernel": ("stage1_kernel (miss gather + gate/up), layer-steps with misses" if staged
                                else "gather_kernel (miss gather, pinned host -> device slots)"),
                     "bound": "host-link", "achieved": round(gather_gbs, 2),
                     "peak": HOST_LINK_PEAK_GBS, "unit": "GB/s",
                     "frac": round(gather_gbs / HOST_LINK_PEAK_GBS, 4),
                     "traffic": round(gather_bytes * ratios["gather_traffic_ratio"]) if ratios else None,
                     "bytes_per_launch": round(gather_bytes), "avg_launch_us": round(gat_us, 2),
                     "launches": miss_n, "memcpy_h2d_same_size_gbs": round(h2d_gbs, 2)},
        "roofline_gemv": {"kernel": ("stage1_kernel + stage2_kernel, all-hit layer-steps (8 routed + "
                                     "shared expert)" if staged
                                     else "routed experts (up_kernel + down_fused_kernel), all-hit layer-steps"),
                          "bound": "hbm",
                          "achieved": round(gemv_gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                          "frac": round(gemv_gbs / HBM_PEAK_GBS, 4),
                          "traffic": round(gemv_bytes * ratios["routed_traffic_ratio"]) if ratios else None,
                          "bytes_per_launch": gemv_bytes, "avg_launch_us": round(rout_us, 2),
                          "launches": hit_n},
        "admission_us_decode": round(adm_us, 2),
        "admission_us": adm,
        "cpu_baseline": cpu,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
