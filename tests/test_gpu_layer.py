"""GPU decode-step arithmetic vs the oracle.

Tolerance for floating-point outputs: max |gpu - oracle| <= 2e-2 *
max |oracle| per output tensor (bf16 operands, fp32 accumulation, bf16
output, against the oracle's double precision).  Integer results (top-k
ids, slot ids) must match exactly; cached and streamed layers must match
bit for bit."""
import numpy as np
import pytest
import torch

import expert_slot_cache_moe_amd as m
from expert_slot_cache_moe_amd import workloads as W
from expert_slot_cache_moe_amd.layer import SlotCacheLayers
import oracle
from parity import check_close, oracle_routed_rows

pytestmark = pytest.mark.gpu


def _bf16_to_f64(t):
    return t.view(torch.bfloat16).double().cpu().numpy()


def _close(got, ref, what=""):
    check_close(got, ref, what)


def _dev_u16(a):
    return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).cuda()


# ---------------------------------------------------------------- top-k

@pytest.mark.parametrize("T,E,K", [(1, 8, 2), (37, 256, 8), (50, 640, 6), (600, 160, 2), (3, 4, 4), (2, 64, 64)])
def test_topk_matches_oracle(T, E, K):
    g = W.rng(3, "topk", T, E)
    lg = W.zipf_logits(g, T, E, 1.05)
    ids = torch.empty((T, K), dtype=torch.int32, device="cuda")
    w = torch.empty((T, K), dtype=torch.float32, device="cuda")
    m.moe_topk(torch.from_numpy(lg).cuda(), K, ids, w)
    oi, ow = oracle.topk(lg, K)
    np.testing.assert_array_equal(ids.cpu().numpy(), oi)
    np.testing.assert_allclose(w.cpu().numpy(), ow, rtol=1e-5, atol=1e-7)


def test_topk_ties_nan_and_infinities():
    lg = np.array([[0.5, 2.0, 2.0, np.nan, 2.0, -1.0],
                   [np.nan, -np.inf, 1.0, np.nan, -np.inf, np.inf],
                   [-np.inf] * 6], np.float32)
    K = 4
    ids = torch.empty((3, K), dtype=torch.int32, device="cuda")
    w = torch.empty((3, K), dtype=torch.float32, device="cuda")
    m.moe_topk(torch.from_numpy(lg).cuda(), K, ids, w)
    oi, ow = oracle.topk(lg, K)
    np.testing.assert_array_equal(ids.cpu().numpy(), oi)
    np.testing.assert_allclose(w.cpu().numpy(), ow, rtol=1e-6, atol=0)


# ---------------------------------------------------------------- routed experts

def _pool_pair(fmt, rows, H, F, seed):
    banks = W.expert_rows(fmt, W.rng(seed, "pool", fmt, H, F), rows, H, F)
    dev = [torch.from_numpy(b).cuda() for b in banks]
    return banks, m.make_pool(fmt, H, F, rows, dev), oracle.Pool(fmt, H, F, banks)


def _routed_gpu(pool, x, idx, w, H, addend=None):
    T, K = idx.shape
    out = torch.empty((T, H), dtype=torch.int16, device="cuda")
    wsb = m.moe_routed_workspace_bytes(pool.weight_format, pool.hidden, pool.ffn, T, K)
    ws = torch.empty(wsb, dtype=torch.uint8, device="cuda")
    m.moe_routed_decode(pool, _dev_u16(x), torch.from_numpy(idx).cuda(),
                        torch.from_numpy(w.astype(np.float32)).cuda(), out, ws,
                        addend=None if addend is None else torch.from_numpy(addend.astype(np.float32)).cuda())
    torch.cuda.synchronize()
    return out


@pytest.mark.parametrize("fmt,H,F,rows,T,K", [
    (0, 64, 128, 8, 1, 2),          # tiny, decode path
    (0, 64, 128, 8, 5, 2),          # tiny, grouped path
    (0, 2048, 512, 12, 1, 8),       # shared-expert decode shape
    (0, 1024, 256, 40, 24, 2),      # wide bf16 shape, ragged T
    (1, 1024, 256, 40, 1, 2),       # e2m1, decode path
    (1, 1024, 256, 40, 33, 2),      # e2m1, grouped path
    (0, 4096, 1024, 10, 7, 6),      # prefill-chunk shape
    (0, 128, 1024, 3, 40, 2),       # FFN 1024 (two gate/up row tiles per wave), groups of 20+ routes
    (2, 256, 1024, 3, 40, 2),       # mxfp4 at FFN 1024, groups of 20+ routes
    (1, 64, 64, 6, 3, 3),           # e2m1, smallest rows
    (2, 1024, 256, 40, 1, 2),       # mxfp4, decode path
    (2, 2048, 512, 12, 1, 8),       # mxfp4, shared-expert decode shape
    (2, 1024, 256, 40, 33, 2),      # mxfp4, grouped path (matrix cores)
    (2, 64, 64, 6, 3, 3),           # mxfp4, smallest rows (vector path)
    (1, 512, 512, 6, 40, 2),        # e2m1 grouped at H 512 / F 512 (LDS-staged kernels), several batches a group
    (2, 512, 512, 6, 40, 2),        # the same as mxfp4
])
def test_routed_matches_oracle(fmt, H, F, rows, T, K):
    g = W.rng(4, "routed", fmt, H, T)
    _, pool, opool = _pool_pair(fmt, rows, H, F, 5)
    x = W.normal_bf16(g, (T, H))
    idx = np.stack([g.choice(rows, K, replace=False) for _ in range(T)]).astype(np.int32)
    idx[g.random((T, K)) < 0.15] = -1
    w = g.random((T, K))
    add = g.standard_normal((T, H)) * 0.01
    out = _routed_gpu(pool, x, idx, w, H, addend=add)
    ref = oracle.routed(opool, idx, w.astype(np.float32).astype(np.float64), x, addend=add.astype(np.float32).astype(np.float64))
    _close(_bf16_to_f64(out), ref, f"fmt{fmt} H{H} T{T}")


@pytest.mark.parametrize("fmt,rows", [(0, 6), (1, 6), (2, 6), (0, 2), (1, 2), (2, 2)])
def test_grouped_routes_do_not_depend_on_their_place_in_the_group(fmt, rows):
    """Wide steps put a group's routes in arrival order; a token's output
    must not depend on it.  Permuting the tokens permutes the output bit
    for bit -- with groups of about 13 routes (one MFMA token tile) and of
    about 40 (two passes of two tiles)."""
    H, F, T, K = 1024, 256, 40, 2
    g = W.rng(9, "place", fmt, rows)
    _, pool, opool = _pool_pair(fmt, rows, H, F, 10)
    x = W.normal_bf16(g, (T, H))
    idx = np.stack([g.choice(rows, K, replace=False) for _ in range(T)]).astype(np.int32)
    w = g.random((T, K))
    a = _routed_gpu(pool, x, idx, w, H)
    perm = g.permutation(T)
    b = _routed_gpu(pool, x[perm], idx[perm], w[perm], H)
    assert torch.equal(b, a[torch.from_numpy(perm).cuda()])
    ref = oracle.routed(opool, idx, w.astype(np.float32).astype(np.float64), x)
    _close(_bf16_to_f64(a), ref, f"fmt{fmt} rows{rows}")


@pytest.mark.parametrize("fmt,H,T,K", [(1, 1024, 33, 2), (0, 64, 5, 3)])
def test_wide_combine_takes_unaligned_outputs_and_addends(fmt, H, T, K):
    """The combine of a grouped step writes 8 outputs per thread when the
    output and the addend are 16-byte aligned, one otherwise: the same
    bytes either way, and within tolerance of the oracle."""
    F, rows = 256 if H > 64 else 128, 12
    g = W.rng(12, "unaligned", fmt, H)
    _, pool, opool = _pool_pair(fmt, rows, H, F, 13)
    x = W.normal_bf16(g, (T, H))
    idx = np.stack([g.choice(rows, K, replace=False) for _ in range(T)]).astype(np.int32)
    idx[g.random((T, K)) < 0.15] = -1
    wts = g.random((T, K)).astype(np.float32)
    add = (g.standard_normal((T, H)) * 0.01).astype(np.float32)
    ws = torch.empty(m.moe_routed_workspace_bytes(fmt, H, F, T, K), dtype=torch.uint8, device="cuda")
    args = (_dev_u16(x), torch.from_numpy(idx).cuda(), torch.from_numpy(wts).cuda())
    outs = []
    for shift in (0, 1):
        ob = torch.empty(T * H + 8, dtype=torch.int16, device="cuda")
        ab = torch.zeros(T * H + 4, dtype=torch.float32, device="cuda")
        out = ob[shift:shift + T * H].view(T, H)
        a = ab[shift:shift + T * H].view(T, H)
        a.copy_(torch.from_numpy(add))
        m.moe_routed_decode(pool, *args, out, ws, addend=a)
        torch.cuda.synchronize()
        outs.append(out.clone())
    assert torch.equal(outs[0], outs[1])
    ref = oracle.routed(opool, idx, wts.astype(np.float64), x, addend=add.astype(np.float64))
    _close(_bf16_to_f64(outs[0]), ref, f"fmt{fmt} H{H}")


STAGE_SHAPES = [(64, 128), (1024, 256), (1024, 512), (2048, 256), (2048, 512), (2048, 1024), (4096, 512),
                (4096, 1024)]


@pytest.mark.parametrize("fmt", [0, 1, 2])
@pytest.mark.parametrize("H,F", STAGE_SHAPES)
def test_single_token_routed_at_every_stage_shape(H, F, fmt):
    """Every (hidden, FFN) width the one-token stage kernels are built for,
    in every format, against the oracle (device-drawn experts, all
    distinct; a -1 route and a weight of zero included)."""
    rows, K = 6, 5
    banks = W.device_expert_rows(fmt, (20, fmt, H, F), rows, H, F)
    pool = m.make_pool(fmt, H, F, rows, banks)
    opool = oracle.Pool(fmt, H, F, [b.cpu().numpy() for b in banks])
    g = W.rng(20, "stage-shapes", fmt, H, F)
    x = W.normal_bf16(g, (1, H))
    idx = g.choice(rows, K, replace=False).astype(np.int32)[None, :]
    idx[0, 2] = -1
    w = g.random((1, K))
    w[0, 4] = 0.0
    add = g.standard_normal((1, H)) * 0.01
    out = _routed_gpu(pool, x, idx, w, H, addend=add)
    ref = oracle.routed(opool, idx, w.astype(np.float32).astype(np.float64), x,
                        addend=add.astype(np.float32).astype(np.float64))
    _close(_bf16_to_f64(out), ref, f"fmt{fmt} H{H} F{F}")


@pytest.mark.parametrize("fmt", [0, 1, 2])
@pytest.mark.parametrize("H,F", [(128, 256), (512, 256), (512, 1024), (1024, 512), (1024, 1024), (2048, 512),
                                 (4096, 1024)])
def test_grouped_routed_across_widths(H, F, fmt):
    """Grouped steps (T > 1) across the widths that pick different kernels:
    matrix-core gate/up and down (bf16 at every width, 4-bit outside the
    LDS-staged widths), the LDS-staged 4-bit kernels (hidden 512 / 1024,
    FFN 256 / 512 / 1024); against the oracle, device-drawn experts."""
    rows, T, K = 8, 24, 2
    banks = W.device_expert_rows(fmt, (21, fmt, H, F), rows, H, F)
    pool = m.make_pool(fmt, H, F, rows, banks)
    opool = oracle.Pool(fmt, H, F, [b.cpu().numpy() for b in banks])
    g = W.rng(21, "grouped-widths", fmt, H, F)
    x = W.normal_bf16(g, (T, H))
    idx = np.stack([g.choice(rows, K, replace=False) for _ in range(T)]).astype(np.int32)
    idx[g.random((T, K)) < 0.1] = -1
    w = g.random((T, K))
    out = _routed_gpu(pool, x, idx, w, H)
    ref = oracle.routed(opool, idx, w.astype(np.float32).astype(np.float64), x)
    _close(_bf16_to_f64(out), ref, f"fmt{fmt} H{H} F{F}")


@pytest.mark.parametrize("fmt,T,K", [(0, 50, 3), (2, 40, 2)])
def test_routed_over_a_pool_of_more_than_32768_rows(fmt, T, K):
    """Pools past 32768 rows group their routes with the rank-sort kernel
    instead of the counting one (whose LDS holds one count per row); rows
    on both sides of 32768, against the oracle over host copies of the rows
    the step reads."""
    H, F, rows = 64, 128, 40000
    banks = W.device_expert_rows(fmt, (18, fmt), rows, H, F)
    pool = m.make_pool(fmt, H, F, rows, banks)
    g = W.rng(18, "big-pool", fmt)
    x = W.normal_bf16(g, (T, H))
    idx = np.stack([g.choice(rows, K, replace=False) for _ in range(T)]).astype(np.int32)
    idx[:4, 0] = [0, 32767, 32768, rows - 1]
    idx[g.random((T, K)) < 0.1] = -1
    w = g.random((T, K))
    out = _routed_gpu(pool, x, idx, w, H)
    used = np.unique(idx[idx >= 0])
    sel = torch.from_numpy(used.astype(np.int64)).cuda()
    opool = oracle.Pool(fmt, H, F, [b.index_select(0, sel).cpu().numpy() for b in banks])
    local = np.where(idx >= 0, np.searchsorted(used, idx), -1).astype(np.int32)
    ref = oracle.routed(opool, local, w.astype(np.float32).astype(np.float64), x)
    _close(_bf16_to_f64(out), ref, f"fmt{fmt} rows{rows}")


@pytest.mark.parametrize("fmt", [0, 1, 2])
def test_routed_at_the_route_limits(fmt):
    """The largest steps the routed call takes: one token with top-64 (the
    stage kernels' route limit) and 8192 routes (the counting grouping's
    limit, 8 per thread)."""
    H, F, rows = 64, 128, 300
    _, pool, opool = _pool_pair(fmt, rows, H, F, 19)
    g = W.rng(19, "limits", fmt)
    for T, K in ((1, 64), (4096, 2)):
        x = W.normal_bf16(g, (T, H))
        idx = np.stack([g.choice(rows, K, replace=False) for _ in range(T)]).astype(np.int32)
        idx[g.random((T, K)) < 0.05] = -1
        w = g.random((T, K))
        out = _routed_gpu(pool, x, idx, w, H)
        ref = oracle.routed(opool, idx, w.astype(np.float32).astype(np.float64), x)
        _close(_bf16_to_f64(out), ref, f"fmt{fmt} T{T} K{K}")


def test_routed_skips_minus_one_and_rows_outside_the_pool():
    """[P1 section 5] a -1 route adds nothing; rows >= num_rows are treated
    the same way."""
    _, pool, opool = _pool_pair(0, 4, 64, 128, 6)
    g = W.rng(4, "skip")
    x = W.normal_bf16(g, (1, 64))
    w = np.array([[0.7, 0.3, 0.5]])
    a = _routed_gpu(pool, x, np.array([[3, -1, 99]], np.int32), w, 64)
    b = _routed_gpu(pool, x, np.array([[3, -1, -1]], np.int32), w, 64)
    c = _routed_gpu(pool, x, np.array([[3, 0, 0]], np.int32), np.array([[0.7, 0.0, 0.0]]), 64)
    assert torch.equal(a, b) and torch.equal(a, c)
    ref = oracle.routed(opool, np.array([[3, -1, -1]], np.int32), np.float32(w).astype(np.float64), x)
    _close(_bf16_to_f64(a), ref)


def test_routed_empty_batch_is_a_noop():
    _, pool, _ = _pool_pair(0, 4, 64, 128, 6)
    out = torch.full((1, 64), 7, dtype=torch.int16, device="cuda")
    ws = torch.empty(1 << 16, dtype=torch.uint8, device="cuda")
    x = torch.zeros((0, 64), dtype=torch.int16, device="cuda")
    m.moe_routed_decode(pool, x, torch.zeros((0, 2), dtype=torch.int32, device="cuda"),
                        torch.zeros((0, 2), device="cuda"), out, ws)
    torch.cuda.synchronize()
    assert (out == 7).all()


# ---------------------------------------------------------------- shared expert

def test_shared_expert_matches_oracle():
    H, F, T = 2048, 512, 3
    g = W.rng(6, "shared")
    w13 = W.normal_bf16(g, 2 * F * H, 0.02)
    w2 = W.normal_bf16(g, H * F, 0.02)
    gate = W.normal_bf16(g, H, 0.02)
    x = W.normal_bf16(g, (T, H))
    sh = m.make_shared(_dev_u16(w13), _dev_u16(w2), _dev_u16(gate), ffn=F)
    add = torch.empty((T, H), dtype=torch.float32, device="cuda")
    ws = torch.empty(m.moe_routed_workspace_bytes(0, H, F, T, 1), dtype=torch.uint8, device="cuda")
    m.moe_shared_expert(sh, H, _dev_u16(x), add, ws)
    torch.cuda.synchronize()
    _, ref = oracle.shared(H, F, w13, w2, gate, x)
    _close(add.cpu().numpy(), ref, "shared")


# ---------------------------------------------------------------- gather, layers

def _tiny_layers(overlap, shared, seed=0, one=256, qw=128, fmt=0, L=1, E=8, S=4, H=64, F=128, T=1, K=2):
    g = W.rng(seed, "layers", fmt, L, E, H)
    host = [W.expert_rows(fmt, g, E, H, F) for _ in range(L)]
    sh = None
    if shared:
        sh = [(W.normal_bf16(g, 2 * F * H, 0.02), W.normal_bf16(g, H * F, 0.02), W.normal_bf16(g, H, 0.02))
              for _ in range(L)]
    lay = SlotCacheLayers(layers=L, experts=E, slots=S, hidden=H, ffn=F, fmt=fmt, host_rows=host,
                          shared=sh, max_tokens=T, max_top_k=K, overlap=overlap,
                          one_call_width=one, query_width=qw)
    return lay, host, sh


def _oracle_layer(oc, host, sh, layer, x, lg, K, fmt, H, F, max_fetch=-1):
    ids_e, w = oracle.topk(lg, K)
    T = lg.shape[0]
    slots = oc.admit(layer, ids_e.reshape(-1), max_fetch).reshape(T, K)
    add = None
    if sh is not None:
        _, add = oracle.shared(H, F, sh[layer][0], sh[layer][1], sh[layer][2], x)
    idx = np.where(slots >= 0, ids_e, -1)
    ref = oracle.routed(oracle.Pool(fmt, H, F, host[layer]), idx, w, x, addend=add)
    return ref, slots, w


@pytest.mark.parametrize("fmt", [1, 2])
def test_tiny_layer_decode_4bit_formats(fmt):
    """The layer step with 4-bit experts (E4M3-scaled E2M1 and MXFP4): slot
    ids exact, outputs within tolerance of the oracle, gathered slots hold
    their experts' bytes."""
    lay, host, sh = _tiny_layers(2, True, seed=31, fmt=fmt, E=16, S=6, H=64, F=128, K=2)
    oc = oracle.OracleCache(1, 16, 6)
    g = W.rng(31, "tiny-4bit", fmt)
    out = torch.empty((1, 64), dtype=torch.int16, device="cuda")
    ids = torch.empty((1, 2), dtype=torch.int32, device="cuda")
    try:
        for t in range(16):
            x = W.normal_bf16(g, (1, 64))
            lg = W.zipf_logits(g, 1, 16, 0.8)
            lay.decode(0, _dev_u16(x), torch.from_numpy(lg).cuda(), 2, out, ids_out=ids)
            torch.cuda.synchronize()
            ref, slots, _ = _oracle_layer(oc, host, sh, 0, x, lg, 2, fmt, 64, 128)
            np.testing.assert_array_equal(ids.cpu().numpy(), slots, err_msg=f"step {t}")
            _close(_bf16_to_f64(out), ref, f"fmt {fmt} step {t}")
        for b in range(len(lay.slot_banks)):
            sb = lay.slot_banks[b].cpu().numpy()
            for s_ in range(6):
                e = oc.own[s_]
                if e >= 0:
                    np.testing.assert_array_equal(sb[s_], host[0][b][e])
        assert m.moe_cache_stats(lay.cache)[2] > 5
    finally:
        lay.close()


@pytest.mark.parametrize("overlap", [0, 1, 2])
@pytest.mark.parametrize("shared", [False, True])
def test_tiny_layer_decode_32_steps(overlap, shared):
    lay, host, sh = _tiny_layers(overlap, shared)
    oc = oracle.OracleCache(1, 8, 4)
    lgs = W.tiny_logits(0, 32)
    g = W.rng(0, "tiny", "x")
    out = torch.empty((1, 64), dtype=torch.int16, device="cuda")
    ids = torch.empty((1, 2), dtype=torch.int32, device="cuda")
    w = torch.empty((1, 2), dtype=torch.float32, device="cuda")
    try:
        for t in range(32):
            x = W.normal_bf16(g, (1, 64))
            lay.decode(0, _dev_u16(x), torch.from_numpy(lgs[t]).cuda(), 2, out, ids_out=ids, w_out=w)
            torch.cuda.synchronize()
            ref, slots, ow = _oracle_layer(oc, host, sh, 0, x, lgs[t], 2, 0, 64, 128)
            np.testing.assert_array_equal(ids.cpu().numpy(), slots, err_msg=f"step {t}")
            np.testing.assert_allclose(w.cpu().numpy(), ow, rtol=1e-5)
            _close(_bf16_to_f64(out), ref, f"step {t}")
            # after the gather every route's slot holds its expert's rows
            for b in range(2):
                sb = lay.slot_banks[b].cpu().numpy()
                for s in slots.reshape(-1):
                    e = oc.own[s]
                    np.testing.assert_array_equal(sb[s], host[0][b][e])
    finally:
        lay.close()


def _covering_rows(chosen, E):
    """Token rows that between them route to every expert of the step
    (greedy): one checked route per group of the grouped kernels."""
    need, rows = set(chosen.reshape(-1).tolist()), []
    for t in np.argsort([-len(set(r)) for r in chosen.tolist()], kind="stable"):
        if need & set(chosen[t].tolist()):
            rows.append(int(t))
            need -= set(chosen[t].tolist())
        if not need:
            break
    return np.sort(np.asarray(rows))


@pytest.mark.parametrize("fmt,H,F,E,S,T,K,one,qw,rows", [
    (0, 1024, 256, 160, 160, 150, 2, 256, 128, "all"),      # wide bf16 step
    (1, 1024, 256, 160, 1100, 600, 2, 256, 128, "cover"),   # wide e2m1 step over 1100 slots
    (1, 1024, 256, 160, 160, 600, 2, 3, 3, "cover"),        # ... one layer's experts, 3 per query
    (2, 1024, 256, 160, 1100, 600, 2, 256, 128, "cover"),   # the wide 4-bit step as MXFP4
    (0, 4096, 1024, 256, 256, 42, 6, 3, 3, "all"),          # prefill chunk, 3 per query
    (0, 4096, 1024, 640, 640, 50, 6, 256, 128, "all"),      # prefill chunk over 640 experts
])
def test_wide_step_cached_equals_streamed_bit_for_bit(fmt, H, F, E, S, T, K, one, qw, rows):
    """[P3 Tests] the GEMV over the slots equals the one over the streamed
    layer exactly; token rows match the oracle (every row, or rows that
    between them route to every expert of the step).  Every expert's bytes
    are drawn afresh, so a read of the wrong slot cannot pass."""
    g = W.rng(7, "wide", fmt, E, T)
    print(f"wide step fmt {fmt} H {H} F {F} E {E} S {S} T {T} K {K} widths ({one}, {qw})", flush=True)
    host = [[W.pinned_copy(b) for b in W.device_expert_rows(fmt, (7, "wide", E, T), E, H, F)]]
    lay = SlotCacheLayers(layers=1, experts=E, slots=S, hidden=H, ffn=F, fmt=fmt, host_rows=host,
                          max_tokens=T, max_top_k=K, one_call_width=one, query_width=qw)
    try:
        chosen = np.stack([g.choice(E, K, replace=False) for _ in range(T)])
        lg = W.forced_logits(g, chosen, E)
        x = W.normal_bf16(g, (T, H))
        out = torch.empty((T, H), dtype=torch.int16, device="cuda")
        ids = torch.empty((T, K), dtype=torch.int32, device="cuda")
        w = torch.empty((T, K), dtype=torch.float32, device="cuda")
        lay.decode(0, _dev_u16(x), torch.from_numpy(lg).cuda(), K, out, ids_out=ids, w_out=w)
        torch.cuda.synchronize()
        st = m.moe_cache_stats(lay.cache, 0)
        assert st[0] == 1 and st[1] == len(set(chosen.reshape(-1).tolist()))
        own = m.moe_cache_read_state(lay.cache)["own"]
        slot_ids = ids.cpu().numpy()
        assert (slot_ids >= 0).all()
        experts = own[slot_ids].astype(np.int32)
        assert (np.sort(experts, 1) == np.sort(chosen, 1)).all()
        # streamed: the same kernels over the layer's experts, rows = expert ids
        out2 = torch.empty_like(out)
        ws = torch.empty(m.moe_routed_workspace_bytes(fmt, H, F, T, K), dtype=torch.uint8, device="cuda")
        m.moe_routed_decode(lay.streamed_pool(0), _dev_u16(x), torch.from_numpy(experts).cuda(), w, out2, ws)
        torch.cuda.synchronize()
        assert torch.equal(out, out2)
        sel = np.arange(T) if rows == "all" else _covering_rows(experts, E)
        assert len(set(experts[sel].reshape(-1).tolist())) == st[1]      # every group checked
        ref = oracle_routed_rows(oracle.Pool(fmt, H, F, [b.numpy() for b in host[0]]), experts[sel],
                                 w.cpu().numpy()[sel].astype(np.float64), x[sel])
        _close(_bf16_to_f64(out)[sel], ref, "wide")
    finally:
        lay.close()


@pytest.mark.parametrize("overlap,fmt", [(1, 0), (2, 0), (3, 0), (2, 1), (2, 2), (3, 1)])
def test_graph_replay_matches_eager_over_changing_routes(overlap, fmt):
    """A whole token (3 layers) captured as one graph and replayed over 40
    steps with changing routes equals the same steps run eagerly (bf16 and
    the 4-bit formats)."""
    L, E, S, H, F, K = 3, 16, 10, 64, 128, 2
    mk = lambda: _tiny_layers(overlap, True, seed=3, fmt=fmt, L=L, E=E, S=S)[0]
    graph_l, eager_l = mk(), mk()
    g = W.rng(3, "graph")
    steps = 40
    xs = [W.normal_bf16(g, (L, 1, H)) for _ in range(steps)]
    lgs = [W.zipf_logits(g, L, E, 1.1).reshape(L, 1, E) for _ in range(steps)]
    x_st = torch.empty((L, 1, H), dtype=torch.int16, device="cuda")
    lg_st = torch.empty((L, 1, E), dtype=torch.float32, device="cuda")
    out_g = torch.empty((L, 1, H), dtype=torch.int16, device="cuda")
    out_e = torch.empty_like(out_g)
    try:
        s = torch.cuda.Stream()
        x_st.copy_(torch.from_numpy(xs[0].view(np.int16)))
        lg_st.copy_(torch.from_numpy(lgs[0]))
        torch.cuda.synchronize()
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph, stream=s):
            for l in range(L):
                graph_l.decode(l, x_st[l], lg_st[l], K, out_g[l])
        for t in range(steps):
            x_st.copy_(torch.from_numpy(xs[t].view(np.int16)))
            lg_st.copy_(torch.from_numpy(lgs[t]))
            graph.replay()
            for l in range(L):
                eager_l.decode(l, x_st[l], lg_st[l], K, out_e[l])
            torch.cuda.synchronize()
            assert torch.equal(out_g, out_e), f"step {t}"
        a = m.moe_cache_read_state(graph_l.cache)
        b = m.moe_cache_read_state(eager_l.cache)
        for k in ("res", "own", "stamp", "stats", "freq", "order"):
            np.testing.assert_array_equal(a[k], b[k], err_msg=k)
        # capture never ran the step: the graph cache saw exactly `steps` tokens
        assert a["stats"][:, 0].tolist() == [steps] * L
    finally:
        graph_l.close()
        eager_l.close()


@pytest.mark.parametrize("overlap", [1, 2])
def test_kernel_timing_events_eager_and_captured(overlap):
    """The optional timing events work in eager mode and as event-record
    nodes of a captured graph."""
    L = 2
    lay, _, _ = _tiny_layers(overlap, True, seed=5, L=L, E=16, S=10)
    try:
        m.moe_cache_set_timing(lay.cache, True)
        g = W.rng(5, "timing")
        x = _dev_u16(W.normal_bf16(g, (L, 1, 64)))
        lg = torch.from_numpy(W.zipf_logits(g, L, 16, 1.1).reshape(L, 1, 16)).cuda()
        out = torch.empty((L, 1, 64), dtype=torch.int16, device="cuda")
        for l in range(L):
            lay.decode(l, x[l], lg[l], 2, out[l])
        ms = m.moe_cache_timing(lay.cache)
        assert ms.shape == (L, 3) and (ms >= 0).all()
        s = torch.cuda.Stream()
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph, stream=s):
            for l in range(L):
                lay.decode(l, x[l], lg[l], 2, out[l])
        for _ in range(3):
            graph.replay()
            torch.cuda.synchronize()
            ms = m.moe_cache_timing(lay.cache)
            assert (ms >= 0).all() and (ms < 1000).all()
        m.moe_cache_set_timing(lay.cache, False)
    finally:
        lay.close()


def test_timed_staged_steps_match_untimed_ones():
    """Timing the staged schedule eagerly (events attached to the launches)
    changes neither the output bytes nor the cache state, misses included."""
    L, E, S, H = 2, 32, 6, 64
    lays = [_tiny_layers(2, True, seed=21, L=L, E=E, S=S)[0] for _ in range(2)]
    g = W.rng(21, "timing-eager")
    outs = [torch.empty((1, H), dtype=torch.int16, device="cuda") for _ in lays]
    try:
        m.moe_cache_set_timing(lays[1].cache, True)
        for t in range(12):
            for l in range(L):
                x = _dev_u16(W.normal_bf16(g, (1, H)))
                lg = torch.from_numpy(W.zipf_logits(g, 1, E, 0.5)).cuda()
                for lay, o in zip(lays, outs):
                    lay.decode(l, x, lg, 2, o)
                torch.cuda.synchronize()
                assert torch.equal(outs[0], outs[1]), (t, l)
            ms = m.moe_cache_timing(lays[1].cache)
            assert (ms > 0).all() and (ms < 1000).all()
        a, b = (m.moe_cache_read_state(lay.cache) for lay in lays)
        for k in ("res", "own", "stamp", "stats", "freq"):
            np.testing.assert_array_equal(a[k], b[k], err_msg=k)
        assert m.moe_cache_stats(lays[0].cache)[2] > 10      # the trace does miss
    finally:
        for lay in lays:
            lay.close()


def test_all_schedules_are_bit_identical():
    """Serial, two-stream, single-stream staged and shared-on-the-side-stream
    steps give the same bytes at every step (the staged one rebuilds fetched
    experts' gate/up dots inside the gather with the same reduction trees)."""
    L, E, S, H = 2, 32, 12, 64
    lays = [_tiny_layers(ov, True, seed=9, L=L, E=E, S=S)[0] for ov in (0, 1, 2, 3)]
    g = W.rng(9, "serial")
    outs = [torch.empty((1, H), dtype=torch.int16, device="cuda") for _ in lays]
    try:
        for t in range(30):
            for l in range(L):
                x = _dev_u16(W.normal_bf16(g, (1, H)))
                lg = torch.from_numpy(W.zipf_logits(g, 1, E, 0.5)).cuda()
                for lay, o in zip(lays, outs):
                    lay.decode(l, x, lg, 2, o)
                torch.cuda.synchronize()
                assert all(torch.equal(outs[0], o) for o in outs[1:]), (t, l)
        assert m.moe_cache_stats(lays[0].cache)[2] > 20      # the trace does miss
    finally:
        for lay in lays:
            lay.close()


@pytest.mark.parametrize("fmt,K", [(1, 1), (1, 3), (1, 6), (2, 5), (2, 7), (0, 3)])
def test_staged_steps_split_any_top_k_like_the_serial_path(fmt, K):
    """Stage 2 of 4-bit rows splits a step's routes over four waves (the
    last ones may get none): any top-k gives the serial schedule's bytes
    and the oracle's values."""
    L, E, S, H, F = 2, 32, 12, 1024, 256
    lays = [_tiny_layers(ov, True, seed=41, fmt=fmt, L=L, E=E, S=S, H=H, F=F, K=K) for ov in (0, 2)]
    g = W.rng(41, "split", fmt, K)
    outs = [torch.empty((1, H), dtype=torch.int16, device="cuda") for _ in lays]
    host, sh = lays[0][1], lays[0][2]
    oc = oracle.OracleCache(L, E, S)
    try:
        for t in range(6):
            for l in range(L):
                xn = W.normal_bf16(g, (1, H))
                lg = W.zipf_logits(g, 1, E, 0.5)
                for (lay, _, _), o in zip(lays, outs):
                    lay.decode(l, _dev_u16(xn), torch.from_numpy(lg).cuda(), K, o)
                torch.cuda.synchronize()
                assert torch.equal(outs[0], outs[1]), (t, l)
                ref, _, _ = _oracle_layer(oc, host, sh, l, xn, lg, K, fmt, H, F)
                _close(_bf16_to_f64(outs[1]), ref, f"fmt{fmt} K{K} t{t} l{l}")
        assert m.moe_cache_stats(lays[1][0].cache)[2] > 0
    finally:
        for lay, _, _ in lays:
            lay.close()


@pytest.mark.parametrize("fmt,E,S,K", [(0, 128, 100, 64), (1, 128, 90, 64), (2, 1500, 40, 8), (0, 1025, 30, 6),
                                     (1, 1024, 30, 6)])
def test_single_token_layer_steps_at_the_top_k_and_expert_limits(fmt, E, S, K):
    """Top-64 (the largest a single-token step takes: the admission's fused
    top-k and the stage kernels' route limit), 1024 experts (the most the
    fused top-k takes) and more (a separate top-k launch first), with the
    shared expert and misses every step: slot ids exact, staged == serial
    bit for bit, outputs within tolerance of the oracle."""
    L, H, F = 2, 64, 128
    lays = [_tiny_layers(ov, True, seed=43, fmt=fmt, L=L, E=E, S=S, H=H, F=F, K=K) for ov in (2, 0)]
    host, sh = lays[0][1], lays[0][2]
    oc = oracle.OracleCache(L, E, S)
    g = W.rng(43, "limits", fmt, E, K)
    outs = [torch.empty((1, H), dtype=torch.int16, device="cuda") for _ in lays]
    ids = [torch.empty((1, K), dtype=torch.int32, device="cuda") for _ in lays]
    try:
        for t in range(5):
            for l in range(L):
                x = W.normal_bf16(g, (1, H))
                lg = W.zipf_logits(g, 1, E, 0.5)
                for (lay, _, _), o, i in zip(lays, outs, ids):
                    lay.decode(l, _dev_u16(x), torch.from_numpy(lg).cuda(), K, o, ids_out=i)
                torch.cuda.synchronize()
                assert torch.equal(outs[0], outs[1]) and torch.equal(ids[0], ids[1]), (t, l)
                ref, slots, _ = _oracle_layer(oc, host, sh, l, x, lg, K, fmt, H, F)
                np.testing.assert_array_equal(ids[0].cpu().numpy(), slots, err_msg=f"token {t} layer {l}")
                _close(_bf16_to_f64(outs[0]), ref, f"fmt{fmt} E{E} K{K} t{t} l{l}")
        assert m.moe_cache_stats(lays[0][0].cache)[2] > 0
    finally:
        for lay, _, _ in lays:
            lay.close()


def test_shared_expert_decode_shape_staged():
    """H 2048, F 512, top-8 of 256 + gated shared expert, 2 layers over a
    small cache (many misses): the staged schedule equals the serial one bit
    for bit and the oracle within tolerance."""
    L, E, S, H, F, K = 2, 256, 24, 2048, 512, 8
    g = W.rng(15, "c3-shape")
    host = [[W.pinned_copy(b) for b in W.device_expert_rows(0, (15, l), E, H, F)] for l in range(L)]
    sh = [(W.normal_bf16(g, 2 * F * H, 0.02), W.normal_bf16(g, H * F, 0.02), W.normal_bf16(g, H, 0.02))
          for _ in range(L)]
    lays = [SlotCacheLayers(layers=L, experts=E, slots=S, hidden=H, ffn=F, host_rows=host, shared=sh,
                            max_tokens=1, max_top_k=K, overlap=ov) for ov in (2, 0, 3)]
    oc = oracle.OracleCache(L, E, S)
    tr = W.DecodeTrace(15, L, E, K, stay=0.5)
    outs = [torch.empty((1, H), dtype=torch.int16, device="cuda") for _ in lays]
    try:
        for t in range(10):
            sets = tr.step_sets()
            lgs = tr.logits(sets)
            for l in range(L):
                x = W.normal_bf16(g, (1, H))
                for lay, o in zip(lays, outs):
                    lay.decode(l, _dev_u16(x), torch.from_numpy(lgs[l:l + 1]).cuda(), K, o)
                torch.cuda.synchronize()
                assert all(torch.equal(outs[0], o) for o in outs[1:]), (t, l)
                ref, _, _ = _oracle_layer(oc, [[b.numpy() for b in hl] for hl in host], sh, l, x,
                                          lgs[l:l + 1], K, 0, H, F)
                _close(_bf16_to_f64(outs[0]), ref, f"token {t} layer {l}")
        assert m.moe_cache_stats(lays[0].cache)[2] > 40
    finally:
        for lay in lays:
            lay.close()


@pytest.mark.parametrize("T", [5, 32, 33])
def test_fused_topk_in_the_layer_step_handles_ties_and_nan(T):
    """Up to 32 rows the layer step's top-k runs inside the admission
    kernel (33: a separate top-k launch); equal logits take the lower
    expert, NaN counts as -infinity."""
    E, S, H, K = 64, 40, 64, 4
    g = W.rng(14, "fused-topk")
    host = [W.bf16_expert_rows(g, E, H, 128)]
    lay = SlotCacheLayers(layers=1, experts=E, slots=S, hidden=H, ffn=128, host_rows=host,
                          max_tokens=T, max_top_k=K)
    oc = oracle.OracleCache(1, E, S)
    try:
        for step in range(6):
            lg = np.round(g.standard_normal((T, E)), 1).astype(np.float32)   # many ties
            lg[0, 3] = np.nan
            lg[1, :] = 0.0
            lg[2, 5] = -0.0
            x = W.normal_bf16(g, (T, H))
            out = torch.empty((T, H), dtype=torch.int16, device="cuda")
            ids = torch.empty((T, K), dtype=torch.int32, device="cuda")
            w = torch.empty((T, K), dtype=torch.float32, device="cuda")
            lay.decode(0, _dev_u16(x), torch.from_numpy(lg).cuda(), K, out, ids_out=ids, w_out=w)
            torch.cuda.synchronize()
            ref, slots, ow = _oracle_layer(oc, host, None, 0, x, lg, K, 0, H, 128)
            np.testing.assert_array_equal(ids.cpu().numpy(), slots)
            np.testing.assert_allclose(w.cpu().numpy(), ow, rtol=1e-5)
            _close(_bf16_to_f64(out), ref, f"step {step}")
    finally:
        lay.close()


@pytest.mark.parametrize("T,K,fmt", [(1, 2, 0), (5, 2, 0), (24, 2, 0), (3, 3, 1)])
def test_shared_on_the_side_stream_equals_serial(T, K, fmt):
    """The #678 split (shared expert on the side stream, gather and routed
    experts on the compute stream, joined before the shared term is added)
    equals the serial schedule bit for bit at one token, small batches
    (grouped path) and 4-bit weights; switching a cache's schedule with
    moe_cache_set_schedule gives the same bytes as creating it so."""
    L, E, S, H, F = 2, 32, 12, 64, 128
    lays = [_tiny_layers(ov, True, seed=19, fmt=fmt, L=L, E=E, S=S, H=H, F=F, T=T, K=K)[0]
            for ov in (0, 3, 0)]
    m.moe_cache_set_schedule(lays[2].cache, 3)
    g = W.rng(19, "split678", T, fmt)
    outs = [torch.empty((T, H), dtype=torch.int16, device="cuda") for _ in lays]
    try:
        for t in range(12):
            for l in range(L):
                x = _dev_u16(W.normal_bf16(g, (T, H)))
                lg = torch.from_numpy(W.zipf_logits(g, T, E, 0.5)).cuda()
                for lay, o in zip(lays, outs):
                    lay.decode(l, x, lg, K, o)
                torch.cuda.synchronize()
                assert all(torch.equal(outs[0], o) for o in outs[1:]), (t, l)
        a, b = (m.moe_cache_read_state(lay.cache) for lay in lays[:2])
        for k in ("res", "own", "stamp", "stats", "freq", "order"):
            np.testing.assert_array_equal(a[k], b[k], err_msg=k)
        assert m.moe_cache_stats(lays[0].cache)[2] > 10
        with pytest.raises(m.MoeError):
            m.moe_cache_set_schedule(lays[0].cache, 4)
    finally:
        for lay in lays:
            lay.close()


@pytest.mark.parametrize("overlap", [0, 1, 2, 3])
def test_empty_layer_step_ticks_the_clock_in_every_schedule(overlap):
    """T = 0 through moe_layer_decode (and the hybrid step): one admission
    of no routes (a clock tick and a call), nothing written to the output."""
    lay, host, sh = _tiny_layers(overlap, True, seed=23, E=8, S=4, T=2, K=2)
    oc = oracle.OracleCache(1, 8, 4)
    out = torch.full((2, 64), 7, dtype=torch.int16, device="cuda")
    x = torch.zeros((2, 64), dtype=torch.int16, device="cuda")
    lg = torch.zeros((2, 8), dtype=torch.float32, device="cuda")
    try:
        lay.decode(0, x[:0], lg[:0], 2, out[:0])
        oc.admit(0, [])
        m.moe_cache_set_cpu_threads(lay.cache, 2)
        lay.decode_hybrid(0, x[:0], lg[:0], 2, out[:0])
        oc.admit(0, [])
        torch.cuda.synchronize()
        st = m.moe_cache_read_state(lay.cache)
        assert st["clock"] == oc.state()["clock"] == 2
        np.testing.assert_array_equal(st["stats"], oc.state()["stats"])
        assert (out == 7).all()
    finally:
        lay.close()


def test_layer_step_rejects_bad_arguments_before_launching():
    lay, host, sh = _tiny_layers(2, True, seed=24, E=8, S=4, T=2, K=2)
    x = torch.zeros((4, 64), dtype=torch.int16, device="cuda")
    lg = torch.zeros((4, 8), dtype=torch.float32, device="cuda")
    out = torch.empty((4, 64), dtype=torch.int16, device="cuda")
    try:
        with pytest.raises(m.MoeError):
            lay.decode(0, x[:2], lg[:2], 3, out[:2])         # K > max_top_k
        with pytest.raises(m.MoeError):
            lay.decode(0, x, lg, 2, out)                     # T > max_tokens
        with pytest.raises(m.MoeError):
            lay.decode(1, x[:1], lg[:1], 2, out[:1])         # layer outside [0, L)
        xb = torch.zeros(2 * 64 + 1, dtype=torch.int16, device="cuda")[1:].view(2, 64)
        with pytest.raises(m.MoeError):
            lay.decode(0, xb, lg[:2], 2, out[:2])            # x not 16-byte aligned
        with pytest.raises(m.MoeError):
            m.moe_cache_set_schedule(lay.cache, -1)
        assert m.moe_cache_read_state(lay.cache)["clock"] == 0
    finally:
        lay.close()
