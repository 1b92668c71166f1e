"""ctypes marshalling for the oracle in ``moe_ref.c``.

TEST INFRASTRUCTURE ONLY (see the package docstring).  No arithmetic of
the method is done here: every function forwards numpy buffers to the C
oracle and returns its results.
"""
from __future__ import annotations

import ctypes as C
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "moe_ref.c")
_LIB = os.path.join(_HERE, "libmoe_ref.so")

_lib = None


def build(force: bool = True) -> str:
    """Compile moe_ref.c into oracle/libmoe_ref.so with gcc."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp%d" % os.getpid()
        subprocess.check_call(
            ["gcc", "-O2", "-std=c99", "-shared", "-fPIC", "-Wall", _SRC, "-o", tmp, "-lm"]
        )
        os.replace(tmp, _LIB)
    return _LIB


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB):
            build(force=False)
        L = C.CDLL(_LIB)
        P = C.c_void_p
        i32, i64, u8, u16 = C.c_int32, C.c_int64, C.c_uint8, C.c_uint16
        L.ref_bf16_to_double.argtypes = [u16]
        L.ref_bf16_to_double.restype = C.c_double
        L.ref_e4m3_to_double.argtypes = [u8]
        L.ref_e4m3_to_double.restype = C.c_double
        L.ref_e2m1_to_double.argtypes = [u8]
        L.ref_e2m1_to_double.restype = C.c_double
        L.ref_e8m0_to_double.argtypes = [u8]
        L.ref_e8m0_to_double.restype = C.c_double
        L.ref_query_widths.argtypes = [i32, i32, i32, i32, P]
        L.ref_query_widths.restype = i32
        L.ref_admit.argtypes = [i32, i32, i32, i32, i32, P, P, P, P, P, P, P, P, i32, P, i32, i32, P, P, P]
        L.ref_admit.restype = i32
        L.ref_prefetch.argtypes = [i32, i32, i32, P, P, P, P, P, P, P, P, i32, P, i32, P, P, P]
        L.ref_prefetch.restype = i32
        L.ref_topk.argtypes = [i32, i32, i32, P, P, P]
        L.ref_topk.restype = None
        L.ref_expert_ffn.argtypes = [i32, i32, i32, P, P, i64, P, P]
        L.ref_expert_ffn.restype = None
        L.ref_routed.argtypes = [i32, i32, i32, P, P, i32, i32, P, P, P, P, P]
        L.ref_routed.restype = None
        L.ref_shared.argtypes = [i32, i32, P, P, P, i32, P, P, P]
        L.ref_shared.restype = None
        L.ref_gather.argtypes = [i32, P, P, P, P, P, i32]
        L.ref_gather.restype = None
        _lib = L
    return _lib


def _p(a: np.ndarray):
    assert a.flags["C_CONTIGUOUS"], "oracle buffers must be C-contiguous"
    return a.ctypes.data_as(C.c_void_p)


def bf16_to_f64(b: int) -> float:
    return lib().ref_bf16_to_double(int(b))


def e4m3_to_f64(v: int) -> float:
    return lib().ref_e4m3_to_double(int(v))


def e2m1_to_f64(v: int) -> float:
    return lib().ref_e2m1_to_double(int(v))


def e8m0_to_f64(v: int) -> float:
    return lib().ref_e8m0_to_double(int(v))


def query_widths(R: int, E: int, one_call: int = 256, qw: int = 128) -> list:
    out = np.zeros(max(R, 1) + 1, np.int32)
    n = lib().ref_query_widths(R, E, one_call, qw, _p(out))
    return [int(v) for v in out[:n]]


class OracleCache:
    """Admission state of one slot cache, advanced by the C oracle."""

    def __init__(self, L: int, E: int, S: int, one_call: int = 256, query_width: int = 128):
        self.L, self.E, self.S = L, E, S
        self.one_call, self.query_width = one_call, query_width
        self.res = np.full(L * E, -1, np.int32)
        self.own = np.full(S, -1, np.int32)
        self.stamp = np.zeros(S, np.uint32)
        self.clock = np.zeros(1, np.uint32)
        self.stats = np.zeros((L, 8), np.int64)
        self.freq = np.zeros(L * E, np.int64)
        self.dlast = np.zeros(L * E, np.uint32)
        self.last_demand = np.zeros(1, np.uint32)
        self.plan_slot = np.zeros(0, np.int32)
        self.plan_expert = np.zeros(0, np.int32)
        self.fill_slot = np.zeros(0, np.int32)
        self.fill_expert = np.zeros(0, np.int32)

    def admit(self, layer: int, ids, max_fetch: int = -1) -> np.ndarray:
        """One admission step; returns the rewritten ids (slot or -1)."""
        ids = np.ascontiguousarray(np.asarray(ids, np.int32).copy())
        R = ids.size
        cap = max(min(R, self.E), 1)
        ps = np.zeros(cap, np.int32)
        pe = np.zeros(cap, np.int32)
        nm = np.zeros(1, np.int32)
        rc = lib().ref_admit(
            self.L, self.E, self.S, self.one_call, self.query_width,
            _p(self.res), _p(self.own), _p(self.stamp), _p(self.clock),
            _p(self.stats), _p(self.freq), _p(self.dlast), _p(self.last_demand),
            layer, _p(ids), R, max_fetch, _p(ps), _p(pe), _p(nm),
        )
        if rc != 0:
            raise ValueError("oracle admission rejected its arguments")
        self.plan_slot = ps[: nm[0]].copy()
        self.plan_expert = pe[: nm[0]].copy()
        return ids

    def prefetch(self, layer: int, ids):
        """One look-ahead prefetch of a layer's predicted experts; the fill
        plan lands in fill_slot / fill_expert."""
        ids = np.ascontiguousarray(np.asarray(ids, np.int32).copy())
        cap = max(self.E, 1)
        ps = np.zeros(cap, np.int32)
        pe = np.zeros(cap, np.int32)
        nf = np.zeros(1, np.int32)
        rc = lib().ref_prefetch(
            self.L, self.E, self.S, _p(self.res), _p(self.own), _p(self.stamp), _p(self.clock),
            _p(self.last_demand), _p(self.stats), _p(self.freq), _p(self.dlast),
            layer, _p(ids), ids.size, _p(ps), _p(pe), _p(nf),
        )
        if rc != 0:
            raise ValueError("oracle prefetch rejected its arguments")
        self.fill_slot = ps[: nf[0]].copy()
        self.fill_expert = pe[: nf[0]].copy()

    def state(self) -> dict:
        return dict(
            res=self.res.copy(), own=self.own.copy(), stamp=self.stamp.copy(),
            clock=int(self.clock[0]), stats=self.stats.copy(), freq=self.freq.copy(),
            dlast=self.dlast.copy(), last_demand=int(self.last_demand[0]),
        )


def topk(logits: np.ndarray, K: int):
    """Returns (ids int32 [T,K], weights float64 [T,K])."""
    logits = np.ascontiguousarray(logits, np.float32)
    T, E = logits.shape
    ids = np.zeros((T, K), np.int32)
    w = np.zeros((T, K), np.float64)
    lib().ref_topk(T, E, K, _p(logits), _p(ids), _p(w))
    return ids, w


class Pool:
    """Weight banks of a pool (slot pool or a layer's full expert set), as
    numpy uint8 arrays of shape [rows, row_bytes]."""

    def __init__(self, fmt: int, H: int, F: int, banks):
        self.fmt, self.H, self.F = fmt, H, F
        self.banks = [np.ascontiguousarray(b, np.uint8) for b in banks]
        nb = {0: 2, 1: 6, 2: 4}[fmt]
        assert len(self.banks) == nb
        self._ptrs = (C.c_void_p * 6)(*([b.ctypes.data for b in self.banks] + [0] * (6 - nb)))
        self._rb = (C.c_int64 * 6)(*([b.shape[1] for b in self.banks] + [0] * (6 - nb)))


def expert_ffn(pool: Pool, row: int, x_bf16: np.ndarray) -> np.ndarray:
    x = np.ascontiguousarray(x_bf16, np.uint16)
    d = np.zeros(pool.H, np.float64)
    lib().ref_expert_ffn(pool.fmt, pool.H, pool.F, pool._ptrs, pool._rb, row, _p(x), _p(d))
    return d


def routed(pool: Pool, idx: np.ndarray, w: np.ndarray, x_bf16: np.ndarray, addend=None) -> np.ndarray:
    idx = np.ascontiguousarray(idx, np.int32)
    w = np.ascontiguousarray(w, np.float64)
    x = np.ascontiguousarray(x_bf16, np.uint16)
    T, K = idx.shape
    out = np.zeros((T, pool.H), np.float64)
    add = None
    if addend is not None:
        add = np.ascontiguousarray(addend, np.float64)
    lib().ref_routed(
        pool.fmt, pool.H, pool.F, pool._ptrs, pool._rb, T, K, _p(idx), _p(w), _p(x),
        _p(add) if add is not None else None, _p(out),
    )
    return out


def shared(H: int, F: int, w13: np.ndarray, w2: np.ndarray, wg: np.ndarray, x_bf16: np.ndarray):
    """Returns (gamma [T], gamma * shared(x) [T,H]) in float64."""
    w13 = np.ascontiguousarray(w13).view(np.uint8)
    w2 = np.ascontiguousarray(w2).view(np.uint8)
    wg = np.ascontiguousarray(wg, np.uint16)
    x = np.ascontiguousarray(x_bf16, np.uint16)
    T = x.shape[0]
    gamma = np.zeros(T, np.float64)
    out = np.zeros((T, H), np.float64)
    lib().ref_shared(H, F, _p(w13), _p(w2), _p(wg), T, _p(x), _p(gamma), _p(out))
    return gamma, out


def gather(host_banks, slot_banks, plan_slot, plan_expert) -> None:
    """Copies plan rows from the layer's host banks into the slot banks
    (numpy uint8 arrays [rows, row_bytes]; slot banks are written)."""
    nb = len(host_banks)
    rb = (C.c_int64 * nb)(*[h.shape[1] for h in host_banks])
    hp = (C.c_void_p * nb)(*[h.ctypes.data for h in host_banks])
    sp = (C.c_void_p * nb)(*[s.ctypes.data for s in slot_banks])
    ps = np.ascontiguousarray(plan_slot, np.int32)
    pe = np.ascontiguousarray(plan_expert, np.int32)
    lib().ref_gather(nb, rb, hp, sp, _p(ps), _p(pe), int(ps.size))
