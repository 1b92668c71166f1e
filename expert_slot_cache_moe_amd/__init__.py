"""Python binding of the gfx950 offloaded-MoE decode-step library.

A thin ctypes layer over include/moe_cache.h: each function has the C
name, converts torch tensors to raw pointers (torch allocates device and
pinned host memory and supplies streams) and raises MoeError on a failed
status.  All computation happens in the HIP kernels of libmoe_cache.so;
there is no fallback: if the library is missing, every call raises.
"""
from __future__ import annotations

import ctypes as C
import os

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libmoe_cache.so")

MOE_OK, MOE_INVALID_ARG, MOE_UNSUPPORTED, MOE_HIP_ERROR, MOE_OUT_OF_MEMORY = range(5)
MOE_FMT_BF16, MOE_FMT_E2M1, MOE_FMT_MXFP4 = 0, 1, 2
MOE_MAX_BANKS = 6
MOE_NUM_STATS = 8
STAT_NAMES = ("calls", "met", "missed", "overflow", "invalid", "pf_calls", "pf_filled",
              "pf_dropped")
(MOE_STAT_CALLS, MOE_STAT_MET, MOE_STAT_MISSED, MOE_STAT_OVERFLOW, MOE_STAT_INVALID,
 MOE_STAT_PF_CALLS, MOE_STAT_PF_FILLED, MOE_STAT_PF_DROPPED) = range(8)


class MoeError(RuntimeError):
    def __init__(self, status, msg):
        super().__init__(f"{msg} (status {status})")
        self.status = status


class moe_cache_desc_t(C.Structure):
    _fields_ = [
        ("num_layers", C.c_int32), ("num_experts", C.c_int32), ("num_slots", C.c_int32),
        ("hidden", C.c_int32), ("ffn", C.c_int32), ("weight_format", C.c_int32),
        ("one_call_width", C.c_int32), ("query_width", C.c_int32), ("max_routes", C.c_int32),
        ("max_tokens", C.c_int32), ("max_top_k", C.c_int32), ("overlap", C.c_int32),
        ("num_banks", C.c_int32), ("gather_workgroups", C.c_int32),
        ("host_banks_host", C.POINTER(C.c_void_p)),
        ("slot_banks_dev", C.c_void_p * MOE_MAX_BANKS),
    ]


class moe_pool_t(C.Structure):
    _fields_ = [
        ("weight_format", C.c_int32), ("hidden", C.c_int32), ("ffn", C.c_int32),
        ("num_rows", C.c_int32), ("banks_dev", C.c_void_p * MOE_MAX_BANKS),
    ]


class moe_shared_t(C.Structure):
    _fields_ = [
        ("ffn", C.c_int32), ("w13_dev", C.c_void_p), ("w2_dev", C.c_void_p),
        ("gate_dev", C.c_void_p),
    ]


_lib = None


def lib():
    """The loaded HIP library; raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(
                f"{LIB_PATH} is missing: build the HIP library first "
                "(python -m expert_slot_cache_moe_amd.build)")
        L = C.CDLL(LIB_PATH)
        P, i32, i64 = C.c_void_p, C.c_int32, C.c_int64
        st = C.c_int
        sig = {
            "moe_status_string": (C.c_char_p, [st]),
            "moe_last_error": (C.c_char_p, []),
            "moe_bank_row_bytes": (st, [i32, i32, i32, P, P]),
            "moe_query_widths": (st, [i32, i32, i32, i32, P, i32, P]),
            "moe_cache_create": (st, [P, P]),
            "moe_cache_destroy": (None, [P]),
            "moe_cache_pool": (st, [P, P]),
            "moe_cache_set_schedule": (st, [P, i32]),
            "moe_topk": (st, [P, i32, i32, i32, P, P, P]),
            "moe_admit": (st, [P, i32, P, i32, i32, P]),
            "moe_gather_misses": (st, [P, P]),
            "moe_routed_workspace_bytes": (i64, [i32, i32, i32, i32, i32]),
            "moe_routed_decode": (st, [P, P, P, P, i32, i32, P, P, P, i64, P]),
            "moe_routed_decode_noalloc": (st, [P, P, P, P, i32, i32, P, P, P]),
            "moe_trace_layer_steps": (st, [P, i32, i32, i32, i32, i32, P, i64, P]),
            "moe_shared_expert": (st, [P, i32, P, i32, P, P, i64, P]),
            "moe_layer_decode": (st, [P, i32, P, P, i32, i32, P, i32, P, P, P, P]),
            "moe_cache_stats": (st, [P, i32, P, P]),
            "moe_prefetch": (st, [P, i32, P, i32, P]),
            "moe_cache_set_cpu_threads": (st, [P, i32]),
            "moe_cpu_experts": (st, [i32, i32, i32, i32, i32, i32, P, P, P, P, P]),
            "moe_layer_decode_hybrid": (st, [P, i32, P, P, i32, i32, P, i32, P, P, P, P]),
            "moe_prefetch_join": (st, [P, P]),
            "moe_cache_read_state": (st, [P, P, P, P, P, P, P, P, P, P]),
            "moe_cache_write_state": (st, [P, P, P, P, C.c_uint32, P, P, P]),
            "moe_cache_read_plan": (st, [P, P, P, i32, P]),
            "moe_cache_read_fills": (st, [P, P, P, i32, P]),
            "moe_cache_set_timing": (st, [P, i32]),
            "moe_cache_timing": (st, [P, P, P]),
            "moe_record_event": (st, [P, P]),
        }
        for name, (res, args) in sig.items():
            f = getattr(L, name)
            f.restype = res
            f.argtypes = args
        _lib = L
    return _lib


def exported_symbols():
    return [n for n in dir(lib()) if n.startswith("moe_")]


def _check(status):
    if status != MOE_OK:
        msg = lib().moe_last_error().decode()
        raise MoeError(status, msg)


def _ptr(t):
    """Raw pointer of a torch tensor (contiguous), an int, or None -> NULL."""
    if t is None:
        return None
    if isinstance(t, int):
        return t
    if not t.is_contiguous():
        raise ValueError("tensors passed to the library must be contiguous")
    return t.data_ptr()


def _dev_ptr(t):
    if t is not None and not isinstance(t, int) and not t.is_cuda:
        raise ValueError("expected a device tensor")
    return _ptr(t)


def _stream(stream):
    if stream is None:
        import torch

        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def _np_ptr(a):
    return None if a is None else a.ctypes.data_as(C.c_void_p)


# ---------------------------------------------------------------- helpers

def moe_status_string(status: int) -> str:
    return lib().moe_status_string(status).decode()


def moe_last_error() -> str:
    return lib().moe_last_error().decode()


def moe_bank_row_bytes(weight_format: int, hidden: int, ffn: int):
    rb = np.zeros(MOE_MAX_BANKS, np.int64)
    nb = np.zeros(1, np.int32)
    _check(lib().moe_bank_row_bytes(weight_format, hidden, ffn, _np_ptr(rb), _np_ptr(nb)))
    return [int(v) for v in rb[: nb[0]]]


def moe_query_widths(R: int, E: int, one_call_width: int = 256, query_width: int = 128):
    cap = max(R, 1) + 1
    out = np.zeros(cap, np.int32)
    n = np.zeros(1, np.int32)
    _check(lib().moe_query_widths(R, E, one_call_width, query_width, _np_ptr(out), cap, _np_ptr(n)))
    return [int(v) for v in out[: n[0]]]


# ---------------------------------------------------------------- cache

class Cache:
    """A created slot cache: the C handle plus references to the caller's
    buffers, which must stay alive while the cache exists."""

    def __init__(self, handle, desc, keep):
        self.handle = handle
        self.desc = desc
        self._keep = keep

    @property
    def L(self):
        return self.desc.num_layers

    @property
    def E(self):
        return self.desc.num_experts

    @property
    def S(self):
        return self.desc.num_slots

    def __enter__(self):
        return self

    def __exit__(self, *a):
        moe_cache_destroy(self)


def moe_cache_create(*, num_layers, num_experts, num_slots, hidden=0, ffn=0,
                     weight_format=MOE_FMT_BF16, one_call_width=256, query_width=128,
                     max_routes=2048, max_tokens=0, max_top_k=0, overlap=1,
                     gather_workgroups=0, host_banks=None, slot_banks=None) -> Cache:
    """host_banks: list over layers of lists over banks of pinned host
    tensors (or raw pointers); slot_banks: list over banks of device
    tensors.  Omit both for an admission-only cache."""
    d = moe_cache_desc_t()
    d.num_layers, d.num_experts, d.num_slots = num_layers, num_experts, num_slots
    d.hidden, d.ffn, d.weight_format = hidden, ffn, weight_format
    d.one_call_width, d.query_width, d.max_routes = one_call_width, query_width, max_routes
    d.max_tokens, d.max_top_k, d.overlap = max_tokens, max_top_k, overlap
    d.gather_workgroups = gather_workgroups
    keep = [host_banks, slot_banks]
    nb = 0
    if slot_banks is not None:
        nb = len(slot_banks)
        flat = (C.c_void_p * (num_layers * nb))()
        for l in range(num_layers):
            for b in range(nb):
                flat[l * nb + b] = _ptr(host_banks[l][b])
        d.host_banks_host = C.cast(flat, C.POINTER(C.c_void_p))
        keep.append(flat)
        for b in range(nb):
            d.slot_banks_dev[b] = _dev_ptr(slot_banks[b])
    d.num_banks = nb
    h = C.c_void_p()
    _check(lib().moe_cache_create(C.byref(d), C.byref(h)))
    return Cache(h, d, keep)


def moe_cache_destroy(cache: Cache) -> None:
    if cache.handle:
        lib().moe_cache_destroy(cache.handle)
        cache.handle = None


def moe_cache_set_schedule(cache: Cache, overlap: int) -> None:
    _check(lib().moe_cache_set_schedule(cache.handle, overlap))


def moe_cache_pool(cache: Cache) -> moe_pool_t:
    p = moe_pool_t()
    _check(lib().moe_cache_pool(cache.handle, C.byref(p)))
    return p


def make_pool(weight_format: int, hidden: int, ffn: int, num_rows: int, banks) -> moe_pool_t:
    """A pool over caller device tensors ([num_rows, row_bytes] each)."""
    p = moe_pool_t()
    p.weight_format, p.hidden, p.ffn, p.num_rows = weight_format, hidden, ffn, num_rows
    for b, t in enumerate(banks):
        p.banks_dev[b] = _dev_ptr(t)
    p._keep = list(banks)
    return p


def make_shared(w13, w2, gate, ffn: int = 0) -> moe_shared_t:
    s = moe_shared_t()
    s.ffn = ffn
    s.w13_dev, s.w2_dev, s.gate_dev = _dev_ptr(w13), _dev_ptr(w2), _dev_ptr(gate)
    s._keep = [w13, w2, gate]
    return s


# ---------------------------------------------------------------- the step

def moe_topk(logits, K: int, ids, w, stream=None) -> None:
    T, E = logits.shape
    _check(lib().moe_topk(_dev_ptr(logits), T, E, K, _dev_ptr(ids), _dev_ptr(w), _stream(stream)))


def moe_admit(cache: Cache, layer: int, ids, max_fetch: int = -1, stream=None, R=None) -> None:
    R = ids.numel() if R is None else R
    _check(lib().moe_admit(cache.handle, layer, _dev_ptr(ids), R, max_fetch, _stream(stream)))


def moe_gather_misses(cache: Cache, stream=None) -> None:
    _check(lib().moe_gather_misses(cache.handle, _stream(stream)))


def moe_routed_workspace_bytes(weight_format: int, hidden: int, ffn: int, T: int, K: int) -> int:
    return int(lib().moe_routed_workspace_bytes(weight_format, hidden, ffn, T, K))


def moe_routed_decode(pool: moe_pool_t, x, idx, w, out, workspace, addend=None, stream=None) -> None:
    T, K = idx.shape
    _check(lib().moe_routed_decode(
        C.byref(pool), _dev_ptr(x), _dev_ptr(idx), _dev_ptr(w), T, K, _dev_ptr(addend),
        _dev_ptr(out), _dev_ptr(workspace), workspace.numel() * workspace.element_size(),
        _stream(stream)))


def moe_routed_decode_noalloc(pool: moe_pool_t, x, idx, w, out, addend=None, stream=None) -> None:
    """moe_routed_decode on the library's own per-GPU scratch (no workspace
    argument, no allocation); calls on one GPU must not overlap."""
    T, K = idx.shape
    _check(lib().moe_routed_decode_noalloc(
        C.byref(pool), _dev_ptr(x), _dev_ptr(idx), _dev_ptr(w), T, K, _dev_ptr(addend),
        _dev_ptr(out), _stream(stream)))


MOE_NOALLOC_SCRATCH_BYTES = 16 << 20


def moe_trace_layer_steps(*, num_layers, num_experts, num_slots, hidden, ffn, T, K, overlap,
                          weight_format=MOE_FMT_BF16, with_shared=True, prefetch_width=0, tokens=2,
                          one_call_width=256, query_width=128, max_routes=None) -> list:
    """The stream operations of a run of layer steps, recorded on the host
    with no device (see include/moe_cache.h): a list of op lines."""
    d = moe_cache_desc_t()
    d.num_layers, d.num_experts, d.num_slots = num_layers, num_experts, num_slots
    d.hidden, d.ffn, d.weight_format = hidden, ffn, weight_format
    d.one_call_width, d.query_width = one_call_width, query_width
    d.max_routes = max_routes if max_routes is not None else max(T * K, prefetch_width, 1)
    d.max_tokens, d.max_top_k, d.overlap = max(T, 1), K, overlap
    n = C.c_int64(0)
    _check(lib().moe_trace_layer_steps(C.byref(d), T, K, int(with_shared), prefetch_width, tokens,
                                       None, 0, C.byref(n)))
    buf = C.create_string_buffer(n.value + 1)
    _check(lib().moe_trace_layer_steps(C.byref(d), T, K, int(with_shared), prefetch_width, tokens,
                                       buf, n.value + 1, C.byref(n)))
    return buf.value.decode().splitlines()


def moe_shared_expert(shared: moe_shared_t, hidden: int, x, addend, workspace, stream=None) -> None:
    T = x.shape[0]
    _check(lib().moe_shared_expert(
        C.byref(shared), hidden, _dev_ptr(x), T, _dev_ptr(addend), _dev_ptr(workspace),
        workspace.numel() * workspace.element_size(), _stream(stream)))


def moe_layer_decode(cache: Cache, layer: int, x, logits, K: int, out, shared=None,
                     max_fetch: int = -1, ids_out=None, w_out=None, stream=None) -> None:
    T = x.shape[0]
    _check(lib().moe_layer_decode(
        cache.handle, layer, _dev_ptr(x), _dev_ptr(logits), T, K,
        C.byref(shared) if shared is not None else None, max_fetch, _dev_ptr(out),
        _dev_ptr(ids_out), _dev_ptr(w_out), _stream(stream)))


def moe_cpu_experts(threads: int, experts, w, x, banks, H: int, F: int, fmt: int = MOE_FMT_BF16) -> np.ndarray:
    """The hybrid step's CPU half on host arrays: experts int32 [T,K] (-1 =
    not a CPU route), w fp32 [T,K], x bf16 bits uint16 [T,H], banks the
    layer's banks of the format in bank order, each uint8 [E, bytes].
    Returns fp32 [T,H]."""
    experts = np.ascontiguousarray(experts, np.int32)
    w = np.ascontiguousarray(w, np.float32)
    x = np.ascontiguousarray(x, np.uint16)
    banks = [np.ascontiguousarray(b, np.uint8) for b in banks]
    T, K = experts.shape
    out = np.zeros((T, H), np.float32)
    ptrs = (C.c_void_p * len(banks))(*[b.ctypes.data for b in banks])
    _check(lib().moe_cpu_experts(threads, fmt, T, K, H, F, _np_ptr(experts), _np_ptr(w), _np_ptr(x),
                                 ptrs, _np_ptr(out)))
    return out


def moe_cache_set_cpu_threads(cache: Cache, threads: int) -> None:
    _check(lib().moe_cache_set_cpu_threads(cache.handle, threads))


def moe_layer_decode_hybrid(cache: Cache, layer: int, x, logits, K: int, out, shared=None,
                            max_fetch: int = -1, ids_out=None, w_out=None, stream=None) -> None:
    T = x.shape[0]
    _check(lib().moe_layer_decode_hybrid(
        cache.handle, layer, _dev_ptr(x), _dev_ptr(logits), T, K,
        C.byref(shared) if shared is not None else None, max_fetch, _dev_ptr(out),
        _dev_ptr(ids_out), _dev_ptr(w_out), _stream(stream)))


def moe_prefetch(cache: Cache, layer: int, ids, n=None, stream=None) -> None:
    n = ids.numel() if n is None else n
    _check(lib().moe_prefetch(cache.handle, layer, _dev_ptr(ids), n, _stream(stream)))


def moe_prefetch_join(cache: Cache, stream=None) -> None:
    _check(lib().moe_prefetch_join(cache.handle, _stream(stream)))


# ---------------------------------------------------------------- inspection

def moe_cache_stats(cache: Cache, layer: int = -1, stream=None) -> np.ndarray:
    out = np.zeros(MOE_NUM_STATS, np.int64)
    _check(lib().moe_cache_stats(cache.handle, layer, _np_ptr(out), _stream(stream)))
    return out


def moe_cache_read_state(cache: Cache) -> dict:
    L, E, S = cache.L, cache.E, cache.S
    res = np.zeros(L * E, np.int32)
    own = np.zeros(S, np.int32)
    stamp = np.zeros(S, np.uint32)
    clock = np.zeros(1, np.uint32)
    stats = np.zeros((L, MOE_NUM_STATS), np.int64)
    freq = np.zeros(L * E, np.int64)
    order = np.zeros(S, np.int32)
    dlast = np.zeros(L * E, np.uint32)
    last_demand = np.zeros(1, np.uint32)
    _check(lib().moe_cache_read_state(cache.handle, _np_ptr(res), _np_ptr(own), _np_ptr(stamp),
                                      _np_ptr(clock), _np_ptr(stats), _np_ptr(freq), _np_ptr(order),
                                      _np_ptr(dlast), _np_ptr(last_demand)))
    return dict(res=res, own=own, stamp=stamp, clock=int(clock[0]), stats=stats, freq=freq,
                order=order, dlast=dlast, last_demand=int(last_demand[0]))


def moe_cache_write_state(cache: Cache, res, own, stamp, clock: int, freq=None, dlast=None,
                          last_demand=None) -> None:
    res = np.ascontiguousarray(res, np.int32)
    own = np.ascontiguousarray(own, np.int32)
    stamp = np.ascontiguousarray(stamp, np.uint32)
    fq = None if freq is None else np.ascontiguousarray(freq, np.int64)
    dl = None if dlast is None else np.ascontiguousarray(dlast, np.uint32)
    ld = None if last_demand is None else np.array([last_demand], np.uint32)
    _check(lib().moe_cache_write_state(cache.handle, _np_ptr(res), _np_ptr(own), _np_ptr(stamp),
                                       clock, _np_ptr(fq), _np_ptr(dl), _np_ptr(ld)))


def moe_cache_read_plan(cache: Cache):
    cap = cache.E
    ps = np.zeros(cap, np.int32)
    pe = np.zeros(cap, np.int32)
    n = np.zeros(1, np.int32)
    _check(lib().moe_cache_read_plan(cache.handle, _np_ptr(ps), _np_ptr(pe), cap, _np_ptr(n)))
    k = min(int(n[0]), cap)
    return ps[:k].copy(), pe[:k].copy()


def moe_cache_read_fills(cache: Cache):
    """The fill plan of the last prefetch: (slots, experts)."""
    cap = cache.E
    ps = np.zeros(cap, np.int32)
    pe = np.zeros(cap, np.int32)
    n = np.zeros(1, np.int32)
    _check(lib().moe_cache_read_fills(cache.handle, _np_ptr(ps), _np_ptr(pe), cap, _np_ptr(n)))
    k = min(int(n[0]), cap)
    return ps[:k].copy(), pe[:k].copy()


def moe_cache_set_timing(cache: Cache, enable: bool) -> None:
    _check(lib().moe_cache_set_timing(cache.handle, 1 if enable else 0))


def moe_cache_timing(cache: Cache) -> np.ndarray:
    """[L, 3] elapsed ms of each layer's last recorded admission, gather
    and routed-expert kernels (-1 where never recorded)."""
    ms = np.zeros(cache.L * 3, np.float32)
    n = np.zeros(1, np.int32)
    _check(lib().moe_cache_timing(cache.handle, _np_ptr(ms), _np_ptr(n)))
    return ms.reshape(cache.L, 3)


def moe_record_event(event, stream=None) -> None:
    """Records a torch.cuda.Event (already created: recorded once) on the
    stream; under graph capture it becomes an event-record node."""
    handle = event.cuda_event
    if not handle:
        raise ValueError("record the event once before capture so that it exists")
    _check(lib().moe_record_event(C.c_void_p(handle), _stream(stream)))
