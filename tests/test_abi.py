"""Host-side checks of the C-ABI library (no GPU needed).

The library must load, export every entry point that include/bkv.h declares,
and reject invalid arguments before touching a device.  Its host-built RoPE
table must equal the oracle's bit for bit (both follow the same formula,
written independently).
"""
from __future__ import annotations

import ctypes as C
import os
import re

import numpy as np
import pytest

from long_reasoning_decode_amd import lib as L
from long_reasoning_decode_amd.configs import EVICT_CONFIGS, QWEN3_4B, TINY

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def so():
    if not os.path.exists(L.LIB_PATH):
        from long_reasoning_decode_amd import build
        build.build()
    return L.load()


def header_functions():
    txt = open(os.path.join(ROOT, "include", "bkv.h")).read()
    txt = re.sub(r"/\*.*?\*/", "", txt, flags=re.S)
    return sorted(set(re.findall(r"\b(bkv_[a-z_0-9]+)\s*\(", txt)))


def test_exports_every_declared_symbol(so):
    names = header_functions()
    assert set(names) == set(L.EXPORTS), names
    for n in names:
        assert hasattr(so, n), n


def test_version_and_strerror(so):
    assert L.version() == 5
    for code in (0, -1, -2, -3, -4):
        assert len(L.strerror(code)) > 0
    assert L.strerror(-99) == "unknown error"


def test_shape_struct_layout():
    # 12 int32 fields and two uint32, no padding
    assert C.sizeof(L.Shape) == 14 * 4


def test_rope_table_matches_oracle(so):
    import oracle as O
    for theta, d in ((1e4, 64), (1e6, 128), (1e4, 128)):
        ours = L.rope_table(theta, d, 0, 2000)
        ref = O.rope_table(theta, d, 0, 2000)
        assert ours.dtype == np.float32 and np.array_equal(ours.view(np.uint32), ref.view(np.uint32))
        assert np.array_equal(L.rope_table(theta, d, 30000, 30100).view(np.uint32),
                              O.rope_table(theta, d, 30000, 30100).view(np.uint32))


def test_rope_table_rejects_bad_args(so):
    buf = np.zeros(64, np.float32)
    p = buf.ctypes.data_as(C.c_void_p)
    assert so.bkv_rope_table(1e4, 63, 0, 1, p) == -1
    assert so.bkv_rope_table(1e4, 64, 5, 5, p) == -1
    assert so.bkv_rope_table(1e4, 64, -1, 1, p) == -1
    assert so.bkv_rope_table(1e4, 64, 0, 1, None) == -1


def _shape(**kw):
    s = L.shape_of(TINY)
    for k, v in kw.items():
        setattr(s, k, v)
    return s


FAKE = C.c_void_p(0x10000)       # 16-byte aligned, never dereferenced: validation fails first
MISALIGNED = C.c_void_p(0x10002)


@pytest.mark.parametrize("field,value,code", [
    ("head_dim", 96, -2), ("n_q_heads", 5, -1), ("n_kv_heads", 0, -1), ("n_q_heads", 18, -2),
    ("n_beacon", 20, -2), ("qcap", 16, -1), ("flags", 32, -1), ("flags", 12, -1), ("flags", 20, -1),
    ("flags", 24, -1), ("cap", 0, -1),
    ("n_beacon", -1, -1),
])
def test_shape_validation(so, field, value, code):
    s = _shape(**{field: value})
    assert so.bkv_fps_update(C.byref(s), FAKE, FAKE, FAKE, None, None) == code
    assert so.bkv_evict(C.byref(s), FAKE, FAKE, 100, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 10,
                        None, None, None, None) == code


def test_pointer_and_range_validation(so):
    s = _shape()
    # null / misaligned pointers
    assert so.bkv_fps_update(C.byref(s), None, FAKE, FAKE, None, None) == -1
    assert so.bkv_fps_update(C.byref(s), MISALIGNED, FAKE, FAKE, None, None) == -1
    assert so.bkv_compact(C.byref(s), FAKE, None, 100, FAKE, None) == -1
    # n_len beyond cap, non-positive, beyond the supported maximum
    assert so.bkv_compact(C.byref(s), FAKE, FAKE, s.cap + 1, FAKE, None) == -3
    assert so.bkv_select(C.byref(s), FAKE, 0, FAKE, None) == -3
    big = _shape(cap=9000)
    assert so.bkv_select(C.byref(big), FAKE, 9000, FAKE, None) == -2
    # budget below the forced keeps when an eviction is due
    tight = _shape(budget=10, n_prefix=8, n_recent_kv=16)
    assert so.bkv_select(C.byref(tight), FAKE, 100, FAKE, None) == -3
    # score: table rows must be positive; recent queries need their arrays
    assert so.bkv_score(C.byref(s), FAKE, 100, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 0, FAKE, None) == -3
    assert so.bkv_score(C.byref(s), FAKE, 100, FAKE, FAKE, None, FAKE, FAKE, FAKE, 10, FAKE, None) == -1
    # evict: missing V, misaligned optional outputs, keep set larger than the budget allows
    assert so.bkv_evict(C.byref(s), FAKE, None, 100, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 10,
                        None, None, None, None) == -1
    assert so.bkv_evict(C.byref(s), FAKE, FAKE, 100, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 10,
                        MISALIGNED, None, None, None) == -1
    assert so.bkv_evict(C.byref(tight), FAKE, FAKE, 100, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 10,
                        None, None, None, None) == -3


def test_prefill_validation(so):
    s = _shape()
    assert so.bkv_fps_prefill(C.byref(s), FAKE, -1, FAKE, FAKE, None, None) == -1
    assert so.bkv_fps_prefill(C.byref(s), FAKE, 8193, FAKE, FAKE, None, None) == -2
    assert so.bkv_fps_prefill(C.byref(s), None, 10, FAKE, FAKE, None, None) == -1
    assert so.bkv_fps_prefill(C.byref(s), MISALIGNED, 10, FAKE, FAKE, None, None) == -1
    assert so.bkv_fps_prefill(C.byref(s), FAKE, 10, None, FAKE, None, None) == -1
    assert so.bkv_fps_prefill(C.byref(s), FAKE, 10, FAKE, FAKE, MISALIGNED, None) == -1
    assert so.bkv_fps_prefill(C.byref(_shape(n_beacon=20)), FAKE, 10, FAKE, FAKE, None, None) == -2


def test_history_compress_and_workspace_validation(so):
    s = _shape()
    # bkv_fps_history: rows within [0, hcap], at most the longest prompt, its pointers
    assert so.bkv_fps_history(C.byref(s), FAKE, 100, 101, FAKE, FAKE, None, None) == -1
    assert so.bkv_fps_history(C.byref(s), FAKE, 100, -1, FAKE, FAKE, None, None) == -1
    assert so.bkv_fps_history(C.byref(s), FAKE, -1, 0, FAKE, FAKE, None, None) == -1
    assert so.bkv_fps_history(C.byref(s), FAKE, 9000, 8193, FAKE, FAKE, None, None) == -2
    assert so.bkv_fps_history(C.byref(s), None, 100, 10, FAKE, FAKE, None, None) == -1
    assert so.bkv_fps_history(C.byref(s), MISALIGNED, 100, 10, FAKE, FAKE, None, None) == -1
    assert so.bkv_fps_history(C.byref(s), FAKE, 100, 10, FAKE, FAKE, MISALIGNED, None) == -1
    # bkv_history_append and bkv_fps_compress: pointers and capacity
    assert so.bkv_history_append(C.byref(s), FAKE, -1, FAKE, FAKE, None) == -1
    assert so.bkv_history_append(C.byref(s), None, 10, FAKE, FAKE, None) == -1
    assert so.bkv_history_append(C.byref(s), FAKE, 10, FAKE, MISALIGNED, None) == -1
    assert so.bkv_fps_compress(C.byref(s), None, FAKE, None, None) == -1
    assert so.bkv_fps_compress(C.byref(s), MISALIGNED, FAKE, None, None) == -1
    assert so.bkv_fps_compress(C.byref(_shape(head_dim=96)), FAKE, FAKE, None, None) == -2
    # no call needs a workspace
    for cfg in EVICT_CONFIGS.values():
        assert L.workspace_bytes(L.shape_of(cfg), cfg.n_len) == 0


def test_attention_and_append_validation(so):
    s = _shape()
    args = lambda n: (C.byref(s), FAKE, FAKE, n, FAKE, FAKE, FAKE, 10, FAKE, None)
    assert so.bkv_decode_attention(*args(0)) == -3
    assert so.bkv_decode_attention(*args(s.cap + 1)) == -3
    assert so.bkv_decode_attention(C.byref(s), FAKE, FAKE, 10, FAKE, FAKE, FAKE, 0, FAKE, None) == -3
    assert so.bkv_decode_attention(C.byref(s), FAKE, None, 10, FAKE, FAKE, FAKE, 10, FAKE, None) == -1
    assert so.bkv_decode_attention(C.byref(s), FAKE, FAKE, 10, MISALIGNED, FAKE, FAKE, 10, FAKE, None) == -1
    assert so.bkv_append_kv(C.byref(s), FAKE, FAKE, -1, FAKE, FAKE, FAKE, FAKE, 10, None) == -3
    assert so.bkv_append_kv(C.byref(s), FAKE, FAKE, s.cap, FAKE, FAKE, FAKE, FAKE, 10, None) == -3
    assert so.bkv_append_kv(C.byref(s), FAKE, FAKE, 3, None, FAKE, FAKE, FAKE, 10, None) == -1


def test_all_configs_are_supported_shapes():
    for cfg in EVICT_CONFIGS.values():
        assert cfg.d in (64, 128) and cfg.hq % cfg.hkv == 0 and cfg.G <= 8
        assert cfg.n_beacon + cfg.n_recent_q <= 32 <= cfg.qcap
        assert cfg.n_len <= 8192 and cfg.budget >= cfg.n_prefix + cfg.n_recent_kv


def test_binding_refuses_to_run_without_the_library():
    """No fallback: with libbkv.so absent, loading and every call through the binding raise instead of
    computing anything on the host (checked in a fresh interpreter, so this process's loaded library is
    untouched)."""
    import subprocess
    import sys
    code = ("import torch\n"
            "from long_reasoning_decode_amd import lib as L\n"
            "from long_reasoning_decode_amd import synth\n"
            "from long_reasoning_decode_amd.configs import TINY\n"
            "L.LIB_PATH = '/nonexistent/libbkv.so'\n"
            "i = synth.make_evict_inputs(TINY)\n"
            "rope = torch.zeros(TINY.rope_rows, TINY.d)\n"
            "ev = lambda: L.evict(L.shape_of(TINY), i['K'], i['V'], TINY.n_len, i['qbuf'], i['qcount'],\n"
            "                     i['q_recent'], i['pos_recent'], i['t'], rope)\n"
            "for name, call in (('load', L.load), ('rope_table', lambda: L.rope_table(1e4, 64, 0, 8)),\n"
            "                   ('evict', ev)):\n"
            "    try:\n"
            "        call()\n"
            "        print(name, 'ran')\n"
            "    except ImportError as e:\n"
            "        print(name, 'refused:', e)\n")
    r = subprocess.run([sys.executable, "-c", code], cwd=ROOT, capture_output=True, text=True, timeout=300)
    lines = r.stdout.strip().splitlines()
    assert len(lines) == 3 and all("refused:" in ln and "missing" in ln for ln in lines), (r.stdout, r.stderr)
