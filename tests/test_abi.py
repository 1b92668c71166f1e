"""The C ABI library loads and exports every entry point the header
declares; host-only argument checks (no GPU needed)."""
import ctypes as C
import os
import re

import pytest

import expert_slot_cache_moe_amd as m

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "moe_cache.h")


def _declared():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(moe_[a-z_]+)\s*\(", text)))


def test_header_declares_the_five_step_calls():
    names = _declared()
    for n in ("moe_cache_create", "moe_admit", "moe_gather_misses", "moe_routed_decode",
              "moe_layer_decode"):
        assert n in names


def test_library_exports_every_declared_symbol():
    lib = C.CDLL(m.LIB_PATH)
    missing = [n for n in _declared() if not hasattr(lib, n)]
    assert not missing, missing
    # the binding wires a Python function of the same name to each symbol
    for n in _declared():
        assert callable(getattr(m, n)), n


def test_query_widths_match_the_pages():
    assert m.moe_query_widths(300, 640) == [128, 128, 44]
    assert m.moe_query_widths(300, 160) == [128, 32]
    assert m.moe_query_widths(8, 160) == [8]
    assert m.moe_query_widths(256, 512) == [256]
    assert m.moe_query_widths(480, 512) == [128, 128, 128, 96]
    assert m.moe_query_widths(0, 512) == []


def test_bank_row_bytes():
    assert m.moe_bank_row_bytes(m.MOE_FMT_BF16, 2048, 512) == [4 * 512 * 2048, 2 * 2048 * 512]
    assert m.moe_bank_row_bytes(m.MOE_FMT_E2M1, 1024, 256) == [262144, 32768, 4, 131072, 16384, 4]
    # MXFP4: gate/up codes, one E8M0 per 32 of them, then down's two
    assert m.moe_bank_row_bytes(m.MOE_FMT_MXFP4, 1024, 256) == [262144, 16384, 131072, 8192]
    with pytest.raises(m.MoeError):
        m.moe_bank_row_bytes(7, 64, 64)


@pytest.mark.parametrize("bad", [dict(overlap=4), dict(overlap=-1), dict(num_slots=0), dict(query_width=0),
                                 dict(max_routes=0), dict(num_layers=0)])
def test_create_rejects_bad_descriptions_before_touching_the_gpu(bad):
    kw = dict(num_layers=1, num_experts=8, num_slots=4, overlap=1, query_width=128, max_routes=8)
    kw.update(bad)
    with pytest.raises(m.MoeError) as e:
        m.moe_cache_create(**kw)
    assert e.value.status == m.MOE_INVALID_ARG
    assert m.moe_last_error()


def test_status_strings():
    assert m.moe_status_string(m.MOE_OK) == "ok"
    assert m.moe_status_string(m.MOE_UNSUPPORTED) == "unsupported"
