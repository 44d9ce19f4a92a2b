"""C ABI tests that need no GPU: the library loads, exports every function the
header declares, validates arguments, and plans work that matches the
oracle's visible-pair counts.  attn_fwd is only called with arguments that are
rejected on the host before any launch."""
import ctypes
import os
import re

import numpy as np
import pytest

import oracle
import transformer_attention_attn_amd as attn
from tests.conftest import ROOT

HEADER = os.path.join(ROOT, "include", "attn.h")


def header_functions():
    txt = open(HEADER, encoding="utf-8").read()
    txt = re.sub(r"/\*.*?\*/", "", txt, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\**\s+\**(attn_\w+)\s*\(", txt, flags=re.M)))


def test_library_loads_and_exports_header_symbols():
    lib = attn.load()
    names = header_functions()
    assert names == sorted(attn.EXPORTS)
    for n in names:
        assert hasattr(lib, n), n
    assert attn.version() == 200


def test_status_strings():
    for code, name in attn.STATUS.items():
        assert attn.status_string(code) == name
    assert attn.status_string(99) == "ATTN_ERR_UNKNOWN"


BAD = [
    # (B, Hq, Hkv, S, D, mask, window, globals, dtype) -> status
    ((0, 4, 4, 16, 64, 1, 0, None, 1), 2),
    ((1, 4, 4, 0, 64, 1, 0, None, 1), 2),
    ((1, 4, 4, 16, 64, 1, 0, None, 7), 4),
    ((1, 4, 4, 16, 96, 1, 0, None, 1), 4),
    ((1, 4, 4, 16, 64, 9, 0, None, 1), 4),
    ((1, 4, 3, 16, 64, 1, 0, None, 1), 3),
    ((1, 4, 4, 16, 64, 2, 0, None, 1), 5),
    ((1, 4, 4, 16, 64, 3, -1, None, 1), 5),
    ((1, 4, 4, 16, 64, 3, 2, [16], 1), 6),
    ((1, 4, 4, 16, 64, 3, 2, [-1], 1), 6),
    ((1, 4, 4, 16, 64, 1, 0, [3], 1), 6),
    ((1, 4, 4, 100, 64, 3, 2, list(range(65)), 1), 6),
    ((1, 4, 4, (1 << 30) + 1, 64, 1, 0, None, 1), 2),
]


@pytest.mark.parametrize("args,status", BAD)
def test_plan_rejects(args, status):
    assert attn.plan_status(*args) == status


@pytest.mark.parametrize("args,status", BAD)
def test_fwd_rejects_before_launch(args, status):
    B, Hq, Hkv, S, D, mask, window, g, dt = args
    fake = 1 << 20  # aligned, never dereferenced: rejected on the host
    assert attn.fwd_raw(fake, fake * 2, fake * 3, fake * 4, B, Hq, Hkv, S, D, mask, window, g,
                        0.125, dt, 0) == status


def test_fwd_rejects_null_alignment_alias_scale():
    a = 1 << 24
    args = (1, 4, 4, 16, 64, 1, 0, None)
    n = 4 * 16 * 64 * 2
    assert attn.fwd_raw(0, a, a + n, a + 2 * n, *args, 0.1, 1, 0) == 1
    assert attn.fwd_raw(a + 8, a + n, a + 2 * n, a + 3 * n, *args, 0.1, 1, 0) == 7
    assert attn.fwd_raw(a, a + n, a + 2 * n, a + 16, *args, 0.1, 1, 0) == 9
    assert attn.fwd_raw(a, a + n, a + 2 * n, a + 3 * n, *args, float("nan"), 1, 0) == 10
    assert attn.fwd_raw(a, a + n, a + 2 * n, a + 3 * n, *args, float("inf"), 1, 0) == 10


CASES = [
    (1, 4, 4, 256, 64, "causal", 0, None, "fp32"),
    (4, 32, 32, 2048, 128, "causal", 0, None, "bf16"),
    (1, 32, 8, 8192, 128, "causal", 0, None, "bf16"),
    (1, 32, 8, 16384, 128, "causal_window", 4096, None, "bf16"),
    (1, 12, 12, 8192, 64, "local_global", 512, [0, 1000, 3000, 6000], "bf16"),
    (2, 6, 3, 1000, 128, "full", 0, None, "bf16"),
    (1, 8, 1, 129, 64, "causal_window", 65, None, "fp32"),
    (1, 2, 2, 77, 64, "local_global", 5, [76, 3, 3, 40], "fp32"),
    (1, 4, 2, 300, 128, "local_global", 0, [], "bf16"),
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: f"{c[5]}-S{c[3]}-{c[8]}")
def test_plan_matches_oracle_counts(case):
    B, Hq, Hkv, S, D, mask, w, g, dt = case
    info = attn.plan(B, Hq, Hkv, S, D, mask, w, g, dt)
    pairs = oracle.visible_pair_count(S, mask, w, g or ())
    assert info["visible_pairs"] == pairs
    assert info["effective_flops"] == pytest.approx(4.0 * D * pairs * B * Hq, rel=1e-15)
    # every visible pair lies in a visited tile: visited keys x rows >= visible pairs
    rows = info["rows_per_item"]
    assert info["tile_visits"] * info["keys_per_tile"] * rows * info["heads_per_item"] >= pairs * B * Hq
    if dt == "bf16":
        G = Hq // Hkv
        assert info["heads_per_item"] == (8 if G % 8 == 0 else 4 if G % 4 == 0 else
                                          2 if G % 2 == 0 else 1)
        assert rows * info["heads_per_item"] == 256
    else:
        assert (rows, info["heads_per_item"], info["keys_per_tile"]) == (16, 1, 32)


def test_plan_skips_masked_tiles():
    dense = attn.plan(1, 32, 8, 16384, 128, "full")
    causal = attn.plan(1, 32, 8, 16384, 128, "causal")
    window = attn.plan(1, 32, 8, 16384, 128, "causal_window", 4096)
    assert causal["tile_visits"] < 0.51 * dense["tile_visits"]
    assert window["tile_visits"] < 0.27 * dense["tile_visits"]
    lg = attn.plan(1, 12, 12, 8192, 64, "local_global", 512, [0, 1000, 3000, 6000])
    lgd = attn.plan(1, 12, 12, 8192, 64, "full")
    assert lg["tile_visits"] < 0.2 * lgd["tile_visits"]
    # only partial tiles need the element mask
    assert causal["partial_tiles"] <= 2 * causal["work_items"]


def test_plan_window_ge_s_same_work_as_causal():
    a = attn.plan(1, 8, 2, 1000, 128, "causal")
    b = attn.plan(1, 8, 2, 1000, 128, "causal_window", 5000)
    assert a["tile_visits"] == b["tile_visits"]
    assert a["visible_pairs"] == b["visible_pairs"]


def test_plan_global_dedup():
    a = attn.plan(1, 2, 2, 500, 64, "local_global", 7, [3, 3, 499, 100, 3])
    b = attn.plan(1, 2, 2, 500, 64, "local_global", 7, [3, 100, 499])
    assert a == b
