"""Pins for the oracle's layer arithmetic (CPU only).

The oracle's scalar C loops are checked against library routines and
closed forms: torch's float8_e4m3fn and bfloat16 conversions, the OCP
FP4 E2M1 value table, numpy's stable argsort and float64 matmul, scipy's
softmax and expit, and the limits of the sigmoid gate.
"""
import numpy as np
import pytest
import scipy.special as sps
import torch

import oracle
from expert_slot_cache_moe_amd import workloads as W

# OCP Microscaling Formats spec, FP4 E2M1 value table (codes 0..7; the
# sign bit gives codes 8..15).
E2M1_TABLE = [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]


def _bf16(a):
    """float32 array -> bf16 bit patterns (torch's round-to-nearest-even)."""
    t = torch.from_numpy(np.ascontiguousarray(a, np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16)


def _bf16_value(bits):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).double().numpy()


def test_e4m3_decode_matches_torch_for_every_code():
    ref = torch.arange(256, dtype=torch.uint8).view(torch.float8_e4m3fn).double().numpy()
    got = np.array([oracle.e4m3_to_f64(v) for v in range(256)])
    nan = np.isnan(ref)
    assert nan.sum() == 2 and (np.isnan(got) == nan).all()
    np.testing.assert_array_equal(got[~nan], ref[~nan])


def test_e8m0_decode_matches_torch_for_every_code():
    """The OCP MX shared scale: 2^(v - 127), 255 = NaN (torch float8_e8m0fnu)."""
    ref = torch.arange(256, dtype=torch.uint8).view(torch.float8_e8m0fnu).double().numpy()
    got = np.array([oracle.e8m0_to_f64(v) for v in range(256)])
    assert np.isnan(got[255]) and np.isnan(ref[255]) and not np.isnan(got[:255]).any()
    np.testing.assert_array_equal(got[:255], ref[:255])
    assert got[127] == 1.0 and got[0] == 2.0 ** -127 and got[254] == 2.0 ** 127


def test_e2m1_decode_matches_the_ocp_table():
    got = [oracle.e2m1_to_f64(v) for v in range(16)]
    assert got[:8] == E2M1_TABLE
    assert got[8:] == [-v for v in E2M1_TABLE]
    assert np.signbit(got[8])


def test_bf16_decode_matches_torch():
    rng = np.random.default_rng(0)
    bits = rng.integers(0, 1 << 16, 4000).astype(np.uint16)
    ref = _bf16_value(bits)
    got = np.array([oracle.bf16_to_f64(int(b)) for b in bits])
    nan = np.isnan(ref)
    assert (np.isnan(got) == nan).all()
    np.testing.assert_array_equal(got[~nan], ref[~nan])


# ---------------------------------------------------------------- top-k

def _numpy_topk(logits, K):
    key = np.where(np.isnan(logits), -np.inf, logits.astype(np.float64))
    order = np.argsort(-key, axis=1, kind="stable")[:, :K]
    sel = np.take_along_axis(key, order, axis=1)
    return order.astype(np.int32), sel


@pytest.mark.parametrize("T,E,K", [(1, 8, 2), (5, 256, 8), (3, 640, 6), (7, 160, 2), (2, 4, 4)])
def test_topk_matches_stable_sort_and_softmax(T, E, K):
    rng = np.random.default_rng(T * 1000 + E)
    logits = rng.standard_normal((T, E)).astype(np.float32)
    ids, w = oracle.topk(logits, K)
    ref_ids, sel = _numpy_topk(logits, K)
    np.testing.assert_array_equal(ids, ref_ids)
    np.testing.assert_allclose(w, sps.softmax(sel, axis=1), rtol=1e-14, atol=0)
    # softmax over all E, keep the top K, renormalise: the same weights
    full = sps.softmax(logits.astype(np.float64), axis=1)
    kept = np.take_along_axis(full, ref_ids, axis=1)
    np.testing.assert_allclose(w, kept / kept.sum(1, keepdims=True), rtol=1e-12)


def test_topk_ties_take_the_lower_expert_and_nan_is_minus_infinity():
    logits = np.array([[0.5, 2.0, 2.0, np.nan, 2.0, -1.0]], np.float32)
    ids, w = oracle.topk(logits, 4)
    assert ids.tolist() == [[1, 2, 4, 0]]
    e = np.exp([0.0, 0.0, 0.0, -1.5])
    np.testing.assert_allclose(w[0], e / e.sum(), rtol=1e-15)
    ids, w = oracle.topk(np.array([[np.nan, -np.inf, 1.0]], np.float32), 3)
    assert ids.tolist() == [[2, 0, 1]]
    np.testing.assert_array_equal(w, [[1.0, 0.0, 0.0]])
    ids, w = oracle.topk(np.full((1, 3), -np.inf, np.float32), 2)
    assert ids.tolist() == [[0, 1]]
    np.testing.assert_array_equal(w, [[0.5, 0.5]])


# ---------------------------------------------------------------- experts

def _bf16_pool(rng, rows, H, F):
    w13 = _bf16(rng.normal(0, 0.02, (rows, 2 * F, H)))
    w2 = _bf16(rng.normal(0, 0.02, (rows, H, F)))
    return w13, w2, oracle.Pool(0, H, F, [w13.reshape(rows, -1).view(np.uint8), w2.reshape(rows, -1).view(np.uint8)])


def _numpy_swiglu(W13, W2, x):
    F = W2.shape[1]
    gu = W13 @ x
    g, u = gu[:F], gu[F:]
    return W2 @ (g * sps.expit(g) * u)


def test_bf16_expert_matches_numpy_swiglu():
    rng = np.random.default_rng(7)
    H, F, rows = 64, 128, 3
    w13, w2, pool = _bf16_pool(rng, rows, H, F)
    x = _bf16(rng.standard_normal(H))
    for r in range(rows):
        got = oracle.expert_ffn(pool, r, x)
        ref = _numpy_swiglu(_bf16_value(w13[r]), _bf16_value(w2[r]), _bf16_value(x))
        np.testing.assert_allclose(got, ref, rtol=1e-10, atol=1e-15)


def _e2m1_pool(rng, rows, H, F, glob13=1.0, glob2=1.0):
    def mat(nr, nc, glob):
        codes = rng.integers(0, 256, (rows, nr, nc // 2), dtype=np.uint8)
        # scales: finite e4m3 codes 0x00..0x7E, random sign bit excluded
        scales = rng.integers(0, 0x7F, (rows, nr, nc // 16), dtype=np.uint8)
        g = np.full((rows, 1), glob, np.float32)
        return codes, scales, g

    c13, s13, g13 = mat(2 * F, H, glob13)
    c2, s2, g2 = mat(H, F, glob2)
    banks = [c13.reshape(rows, -1), s13.reshape(rows, -1), g13.view(np.uint8),
             c2.reshape(rows, -1), s2.reshape(rows, -1), g2.view(np.uint8)]
    return (c13, s13, g13, c2, s2, g2), oracle.Pool(1, H, F, banks)


def _numpy_dequant(codes, scales, glob):
    """codes [nr, nc/2] (element 2i low nibble, 2i+1 high), scales
    [nr, nc/16] e4m3 via torch, one fp32 global."""
    table = np.array(E2M1_TABLE + [-v for v in E2M1_TABLE])
    lo, hi = codes & 0xF, codes >> 4
    q = np.stack([table[lo], table[hi]], axis=-1).reshape(codes.shape[0], -1)
    s = torch.from_numpy(scales.copy()).view(torch.float8_e4m3fn).double().numpy()
    return q * np.repeat(s, 16, axis=1) * float(glob)


@pytest.mark.parametrize("g13,g2", [(1.0, 1.0), (0.75, -2.5)])
def test_e2m1_expert_matches_numpy_dequant_swiglu(g13, g2):
    rng = np.random.default_rng(8)
    H, F, rows = 64, 32, 2
    (c13, s13, _, c2, s2, _), pool = _e2m1_pool(rng, rows, H, F, g13, g2)
    x = _bf16(rng.standard_normal(H) * 0.05)
    for r in range(rows):
        W13 = _numpy_dequant(c13[r], s13[r], g13)
        W2 = _numpy_dequant(c2[r], s2[r], g2)
        ref = _numpy_swiglu(W13, W2, _bf16_value(x))
        np.testing.assert_allclose(oracle.expert_ffn(pool, r, x), ref, rtol=1e-9, atol=1e-12)


def _mxfp4_pool(rng, rows, H, F):
    def mat(nr, nc):
        codes = rng.integers(0, 256, (rows, nr, nc // 2), dtype=np.uint8)
        scales = rng.integers(110, 140, (rows, nr, nc // 32), dtype=np.uint8)
        return codes, scales

    c13, s13 = mat(2 * F, H)
    c2, s2 = mat(H, F)
    banks = [c13.reshape(rows, -1), s13.reshape(rows, -1), c2.reshape(rows, -1), s2.reshape(rows, -1)]
    return (c13, s13, c2, s2), oracle.Pool(2, H, F, banks)


def _numpy_dequant_mx(codes, scales):
    """codes [nr, nc/2] (element 2i low nibble), scales [nr, nc/32] e8m0 via torch."""
    table = np.array(E2M1_TABLE + [-v for v in E2M1_TABLE])
    lo, hi = codes & 0xF, codes >> 4
    q = np.stack([table[lo], table[hi]], axis=-1).reshape(codes.shape[0], -1)
    s = torch.from_numpy(scales.copy()).view(torch.float8_e8m0fnu).double().numpy()
    return q * np.repeat(s, 32, axis=1)


def test_mxfp4_expert_matches_numpy_dequant_swiglu():
    """MXFP4 (OCP MX: E2M1 elements, one E8M0 scale per 32) against an
    independent dequantisation and numpy matmuls."""
    rng = np.random.default_rng(18)
    H, F, rows = 64, 64, 3
    (c13, s13, c2, s2), pool = _mxfp4_pool(rng, rows, H, F)
    x = _bf16(rng.standard_normal(H) * 0.05)
    for r in range(rows):
        ref = _numpy_swiglu(_numpy_dequant_mx(c13[r], s13[r]), _numpy_dequant_mx(c2[r], s2[r]),
                            _bf16_value(x))
        np.testing.assert_allclose(oracle.expert_ffn(pool, r, x), ref, rtol=1e-9, atol=1e-12)


def test_mxfp4_quantized_rows_round_trip_within_half_a_step():
    """The generator's MXFP4 rows decode (oracle) to within half an E2M1
    step of the drawn weights, |w - q| <= scale * 1 (the widest gap, 4 -> 6,
    halved), except that magnitudes past 6 * scale (the OCP MX scale
    2^(floor(log2 amax) - 2) leaves amax / scale in [4, 8)) saturate to
    6 * scale; signs are kept."""
    g = W.rng(3, "mx-roundtrip")
    H, F = 64, 32
    banks = W.mxfp4_expert_rows(g, 1, H, F)
    pool = oracle.Pool(2, H, F, banks)
    g = W.rng(3, "mx-roundtrip")
    w13 = g.standard_normal((2 * F, H), dtype=np.float32) * np.float32(0.02)
    q = _numpy_dequant_mx(banks[0][0].reshape(2 * F, H // 2), banks[1][0].reshape(2 * F, H // 32))
    scale = np.repeat(torch.from_numpy(banks[1][0].reshape(2 * F, H // 32).copy())
                      .view(torch.float8_e8m0fnu).double().numpy(), 32, axis=1)
    sat = np.abs(w13) > 6 * scale
    assert (np.abs(w13 - q)[~sat] <= scale[~sat] * 1.0 + 1e-12).all()
    np.testing.assert_array_equal(np.abs(q[sat]), 6 * scale[sat])
    assert sat.any() and (~sat).any()
    assert ((np.sign(q) == np.sign(w13)) | (q == 0)).all()
    # the oracle reads the same rows: one unit activation picks column 0
    x = np.zeros(H, np.uint16)
    x[0] = 0x3F80                                    # bf16 1.0
    ref = _numpy_swiglu(q, _numpy_dequant_mx(banks[2][0].reshape(H, F // 2), banks[3][0].reshape(H, F // 32)),
                        _bf16_value(x))
    np.testing.assert_allclose(oracle.expert_ffn(pool, 0, x), ref, rtol=1e-9, atol=1e-15)


def test_routed_sums_weighted_experts_and_skips_minus_one():
    rng = np.random.default_rng(9)
    H, F, rows = 64, 128, 5
    w13, w2, pool = _bf16_pool(rng, rows, H, F)
    T, K = 3, 3
    x = _bf16(rng.standard_normal((T, H)))
    idx = np.array([[4, -1, 0], [2, 2, 3], [-1, -1, -1]], np.int32)
    w = rng.random((T, K)).astype(np.float32)
    add = rng.standard_normal((T, H))
    got = oracle.routed(pool, idx, w, x, add)
    for t in range(T):
        ref = add[t].copy()
        for k in range(K):
            if idx[t, k] >= 0:
                ref += float(w[t, k]) * _numpy_swiglu(_bf16_value(w13[idx[t, k]]), _bf16_value(w2[idx[t, k]]), _bf16_value(x[t]))
        np.testing.assert_allclose(got[t], ref, rtol=1e-10, atol=1e-14)
    # top-1 with weight 1 and no addend is the plain expert
    one = oracle.routed(pool, np.array([[3]], np.int32), np.ones((1, 1), np.float32), x[:1])
    np.testing.assert_array_equal(one[0], oracle.expert_ffn(pool, 3, x[0]))


def test_worked_split_example_gpu_part():
    """[3, -1] with weights [0.7, 0.3] is route 0 alone; the same as slot 0
    with weight 0.0 when slot 0 holds finite weights."""
    rng = np.random.default_rng(10)
    H, F = 64, 128
    _, _, pool = _bf16_pool(rng, 4, H, F)
    x = _bf16(rng.standard_normal((1, H)))
    a = oracle.routed(pool, np.array([[3, -1]], np.int32), np.array([[0.7, 0.3]]), x)
    b = oracle.routed(pool, np.array([[3, 0]], np.int32), np.array([[0.7, 0.0]]), x)
    c = 0.7 * oracle.expert_ffn(pool, 3, x[0])
    np.testing.assert_array_equal(a, b)
    np.testing.assert_allclose(a[0], c, rtol=1e-15)


def test_shared_expert_gate_closed_form_and_limits():
    rng = np.random.default_rng(11)
    H, F, T = 64, 128, 3
    w13, w2, _ = _bf16_pool(rng, 1, H, F)
    wg = _bf16(rng.normal(0, 0.02, H))
    x = _bf16(rng.standard_normal((T, H)))
    gamma, out = oracle.shared(H, F, w13[0], w2[0], wg, x)
    for t in range(T):
        z = _bf16_value(x[t]) @ _bf16_value(wg)
        np.testing.assert_allclose(gamma[t], sps.expit(z), rtol=1e-14)
        ref = sps.expit(z) * _numpy_swiglu(_bf16_value(w13[0]), _bf16_value(w2[0]), _bf16_value(x[t]))
        np.testing.assert_allclose(out[t], ref, rtol=1e-10, atol=1e-15)
    # gate logit -> -inf: the shared term vanishes; -> +inf: the plain expert
    big = _bf16(np.full(H, 3.0e4))
    xs = _bf16(np.ones((1, H)))
    g0, o0 = oracle.shared(H, F, w13[0], w2[0], _bf16(-_bf16_value(big)), xs)
    assert g0[0] == 0.0 and not o0.any()
    g1, o1 = oracle.shared(H, F, w13[0], w2[0], big, xs)
    assert g1[0] == 1.0
    ref = _numpy_swiglu(_bf16_value(w13[0]), _bf16_value(w2[0]), _bf16_value(xs[0]))
    np.testing.assert_allclose(o1[0], ref, rtol=1e-10, atol=1e-15)


def test_gather_copies_plan_rows_byte_for_byte():
    rng = np.random.default_rng(12)
    E, S = 9, 5
    host = [rng.integers(0, 256, (E, 48), dtype=np.uint8), rng.integers(0, 256, (E, 16), dtype=np.uint8)]
    slots = [np.zeros((S, 48), np.uint8), np.zeros((S, 16), np.uint8)]
    untouched = [s.copy() for s in slots]
    ps, pe = np.array([4, 0, 2], np.int32), np.array([8, 3, 5], np.int32)
    oracle.gather(host, slots, ps, pe)
    for b in range(2):
        for s, e in zip(ps, pe):
            np.testing.assert_array_equal(slots[b][s], host[b][e])
        for s in (1, 3):
            np.testing.assert_array_equal(slots[b][s], untouched[b][s])
