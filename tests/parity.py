"""The floating-point parity bar shared by the tests, and the record of
what each test reached.

Bar: max |gpu - oracle| <= 2e-2 * max |oracle| per output tensor (bf16
operands, fp32 accumulation, bf16 output, against the oracle's double
precision).  Every check records its achieved ratio, and the terminal
summary prints the largest per test, so a drift toward the bound shows
before it fails."""
import os

import numpy as np

TOL = 2e-2
ERRORS: dict = {}


def record_error(ratio: float) -> None:
    test = os.environ.get("PYTEST_CURRENT_TEST", "?").rsplit(" ", 1)[0]
    ERRORS[test] = max(ERRORS.get(test, 0.0), float(ratio))


def check_close(got, ref, what="") -> float:
    """Asserts the bar; returns and records max |got - ref| / max |ref|."""
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    scale = np.abs(ref).max()
    err = np.abs(got - ref).max()
    ratio = err / scale if scale > 0 else (0.0 if err == 0 else np.inf)
    record_error(ratio)
    assert err <= TOL * scale, f"{what}: max err {err:.3e} > {TOL} * {scale:.3e}"
    return ratio


def oracle_routed_rows(pool, idx, w, x, addend=None, threads=8):
    """oracle.routed over token rows split across host threads (the C
    oracle releases the interpreter lock in its calls; each row's
    arithmetic is the same whichever thread runs it)."""
    from concurrent.futures import ThreadPoolExecutor

    import oracle

    T = idx.shape[0]
    parts = [p for p in np.array_split(np.arange(T), max(1, min(threads, T))) if p.size]
    with ThreadPoolExecutor(len(parts)) as ex:
        outs = list(ex.map(lambda p: oracle.routed(
            pool, np.ascontiguousarray(idx[p]), np.ascontiguousarray(w[p]), np.ascontiguousarray(x[p]),
            addend=None if addend is None else np.ascontiguousarray(addend[p])), parts))
    return np.concatenate(outs, 0)
