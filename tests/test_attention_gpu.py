"""Decode attention over the cache (bkv_decode_attention) and the key/value
append (bkv_append_kv) against the oracle.

Tolerance of the attention output, derived from its arithmetic: the logits
are exact bf16 products summed in fp32 (relative error ~1e-7 of |q||k|), the
weights are fp32 exponentials, and each output element is an fp32 sum of
weight x value over up to a few thousand keys per wave.  Every error term is
relative to the element's natural magnitude s = sum_j w_j |v_j| (which the
oracle returns with the output), so the bar is |gpu - oracle| <= 1e-4 s +
1e-6, some 50x the errors seen; the append is bit-exact.
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle as O
from long_reasoning_decode_amd import lib as L
from long_reasoning_decode_amd import synth
from long_reasoning_decode_amd.configs import QWEN3_4B, R1_QWEN_7B, TINY

import _helpers as H

pytestmark = pytest.mark.gpu

ATOL = 1e-6
RTOL_SCALE = 1e-4


def _flush(msg: str) -> None:
    print(msg, flush=True)


def _check_attention(cfg, inp, n_len, units=None, where="", chunk: int = 1024):
    shape = L.shape_of(cfg, cap=inp["K"].shape[-2])
    rope = H.rope_dev(cfg)
    q = inp["q_recent"][..., 0, :].contiguous()           # one query per head: [L, B, Hq, d]
    out = torch.full((cfg.qbufs, cfg.d), float("nan"), dtype=torch.float32, device="cuda")
    L.decode_attention(shape, inp["K"], inp["V"], n_len, q, inp["t"], rope, out)
    torch.cuda.synchronize()
    U, G, D = cfg.units, cfg.G, cfg.d
    units = list(range(U)) if units is None else list(units)
    oc = H.ocfg(cfg, n_len=inp["K"].shape[-2])
    qn_all = synth.to_u16(q).reshape(U, G, D)
    g_all = out.reshape(U, G, D).cpu().numpy()
    worst = 0.0
    for c0 in range(0, len(units), chunk):   # a chunk of units at a time bounds the host copies
        us = units[c0:c0 + chunk]
        v = synth.oracle_views(cfg, inp, us)
        qn = np.ascontiguousarray(qn_all[us])
        o = np.empty((len(us), G, D))
        scale = np.empty_like(o)

        def one(sl):
            o[sl], scale[sl] = O.decode_attention(oc, v["K"][sl], v["V"][sl], qn[sl], v["t"][sl], n_len)

        H.on_threads(one, len(us))
        g = g_all[us].astype(np.float64)
        err = np.abs(g - o)
        lim = RTOL_SCALE * scale + ATOL
        bad = err > lim
        assert not bad.any(), f"{where}: {bad.sum()} outputs out of tolerance, worst {float((err / lim).max()):.3g}x"
        worst = max(worst, float((err / (scale + 1e-30)).max()))
    return worst


CASES = [
    (TINY, [1, 5, 31, 32, 33, 97, 160]),
    (TINY.scaled(hq=2, hkv=2, name="g1d64"), [1, 40, 160]),
    (TINY.scaled(hq=8, hkv=1, name="g8d64"), [7, 160]),
    (QWEN3_4B.scaled(n_layers=1, batch=2), [1, 100, 2176]),
    (R1_QWEN_7B.scaled(n_layers=1, batch=2), [64, 1152]),
    (TINY.scaled(d=128, hq=3, hkv=3, name="g1d128"), [160]),
    (TINY.scaled(d=128, hq=5, hkv=1, budget=8064, n_new=128, n_prefix=4, name="n8192"), [8192, 4097]),
]


@pytest.mark.parametrize("cfg,lens", CASES, ids=[c.name for c, _ in CASES])
def test_decode_attention_matches_oracle(cfg, lens):
    inp = synth.make_evict_inputs(cfg, device="cuda")
    for n in lens:
        _flush(f"attention {cfg.name} n_len={n}")
        rel = _check_attention(cfg, inp, n, where=f"{cfg.name} n_len={n}")
        _flush(f"  worst error / magnitude {rel:.2e}")


def test_decode_attention_full_size_all_units():
    """The qwen3-4b cache at full size (every unit, the cache length of an eviction); the oracle checks
    every output."""
    cfg = QWEN3_4B
    _flush(f"attention full size {cfg.name}: {cfg.units} units")
    inp = synth.make_evict_inputs(cfg, device="cuda")
    rel = _check_attention(cfg, inp, cfg.n_len, where="full size")
    _flush(f"  {cfg.units} units checked, worst error / magnitude {rel:.2e}")
    del inp
    torch.cuda.empty_cache()


@pytest.mark.parametrize("cfg", [TINY, QWEN3_4B.scaled(n_layers=2, batch=3)], ids=lambda c: c.name)
def test_append_kv_matches_oracle(cfg):
    inp = synth.make_evict_inputs(cfg, device="cuda")
    K, V = inp["K"].clone(), inp["V"].clone()
    g = torch.Generator(device="cuda").manual_seed(9)
    k_new = torch.randn(cfg.units, cfg.d, generator=g, device="cuda").to(torch.bfloat16)
    v_new = torch.randn(cfg.units, cfg.d, generator=g, device="cuda").to(torch.bfloat16)
    rope = H.rope_dev(cfg)
    row = cfg.n_len - 5
    L.append_kv(L.shape_of(cfg), K, V, row, k_new, v_new, inp["t"], rope)
    torch.cuda.synchronize()
    Kh, Vh = synth.to_u16(K).reshape(cfg.units, -1, cfg.d), synth.to_u16(V).reshape(cfg.units, -1, cfg.d)
    K0, V0 = synth.to_u16(inp["K"]).reshape(cfg.units, -1, cfg.d), synth.to_u16(inp["V"]).reshape(cfg.units, -1, cfg.d)
    kn, vn = synth.to_u16(k_new), synth.to_u16(v_new)
    t = inp["t"].cpu().numpy()
    for u in range(cfg.units):
        b = (u // cfg.hkv) % cfg.batch
        assert np.array_equal(Kh[u, row], O.rope_row(kn[u], cfg.theta, int(t[b]))), u
        assert np.array_equal(Vh[u, row], vn[u]), u
        others = np.arange(Kh.shape[1]) != row
        assert np.array_equal(Kh[u, others], K0[u, others]) and np.array_equal(Vh[u, others], V0[u, others])


def test_attention_rejects_bad_lengths():
    import ctypes as C
    cfg = TINY
    inp = synth.make_evict_inputs(cfg, device="cuda")
    shape = L.shape_of(cfg)
    so = L.load()
    ptr = lambda t: C.c_void_p(t.data_ptr())
    rope = H.rope_dev(cfg)
    out = torch.empty((cfg.qbufs, cfg.d), device="cuda")
    q = torch.zeros((cfg.qbufs, cfg.d), dtype=torch.bfloat16, device="cuda")
    for n in (0, cfg.n_len + 1):
        assert so.bkv_decode_attention(C.byref(shape), ptr(inp["K"]), ptr(inp["V"]), n, ptr(q), ptr(inp["t"]),
                                       ptr(rope), rope.shape[0], ptr(out), None) == -3
    for row in (-1, cfg.n_len):
        assert so.bkv_append_kv(C.byref(shape), ptr(inp["K"]), ptr(inp["V"]), row, ptr(q), ptr(q), ptr(inp["t"]),
                                ptr(rope), rope.shape[0], None) == -3


@pytest.mark.parametrize("mode", ["beacon", "full"])
def test_decode_loop_tiny(mode):
    """The synthetic decode loop on a tiny shape: the step count, the evictions, and the last step's attention
    output against the oracle on the cache the loop left."""
    from dataclasses import replace
    from long_reasoning_decode_amd.decode import DecodeConfig, DecodeRun
    dc = DecodeConfig(f"decode-tiny-{mode}", replace(TINY, batch=2, seed=20261202 + 620), mode, 70, gen_len=400)
    run = DecodeRun(dc, block=16)
    r = run.run()
    b = dc.base
    if mode == "beacon":
        assert r["evictions"] == 2 and run.L == b.budget + 70 - 2 * b.n_new
    else:
        assert r["evictions"] == 0 and run.L == dc.n0 + 70
    q, pos, n = run.last
    U, G, D = b.units, b.G, b.d
    cap = run.K.shape[-2]
    Kh = synth.to_u16(run.K).reshape(U, cap, D)
    Vh = synth.to_u16(run.V).reshape(U, cap, D)
    p_u = pos.cpu().numpy()[[(u // b.hkv) % b.batch for u in range(U)]].astype(np.int32)
    o, scale = O.decode_attention(H.ocfg(b, n_len=cap), Kh, Vh, synth.to_u16(q).reshape(U, G, D), p_u, n)
    g = run.out.reshape(U, G, D).cpu().numpy().astype(np.float64)
    assert np.all(np.abs(g - o) <= RTOL_SCALE * scale + ATOL)
