"""Prefill initialisation of the query buffers (bkv_fps_prefill) against the oracle.

Every buffer's selection order, count and buffer rows must equal the oracle's
bit for bit (the sampling decides integers from fp32 arithmetic that both
sides carry out in the same order).  The cases cover both head sizes, prompts
shorter than the buffer, prompts held in registers, in LDS and re-read from
memory, the longest prompt taken, and inputs full of ties (duplicate rows,
zero rows, rows that differ by a power of two).
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle as O
from long_reasoning_decode_amd import lib as L
from long_reasoning_decode_amd import synth
from long_reasoning_decode_amd.configs import PREFILL, TINY

pytestmark = pytest.mark.gpu

SMALL = TINY.scaled(name="prefill-small", n_layers=1, batch=2, hq=4, hkv=2)


def _flush(msg: str) -> None:
    print(msg, flush=True)


def _run(cfg, q: torch.Tensor, P: int):
    """bkv_fps_prefill on q [L, B, Hq, P, d]; returns (qbuf, qcount, sel) on the host."""
    shape = L.shape_of(cfg)
    qbuf = torch.full((cfg.qbufs, cfg.qcap, cfg.d), 0x7F7F, dtype=torch.int16, device="cuda").view(torch.bfloat16)
    qc = torch.full((cfg.qbufs,), -5, dtype=torch.int32, device="cuda")
    sel = torch.full((cfg.qbufs, cfg.n_beacon), -7, dtype=torch.int32, device="cuda")
    L.fps_prefill(shape, q, P, qbuf, qc, sel)
    torch.cuda.synchronize()
    return synth.to_u16(qbuf), qc.cpu().numpy(), sel.cpu().numpy()


def _check(cfg, q: torch.Tensor, P: int, bufs=None, where=""):
    g_buf, g_qc, g_sel = _run(cfg, q, P)
    qn = synth.to_u16(q).reshape(cfg.qbufs, P, cfg.d)
    bufs = range(cfg.qbufs) if bufs is None else bufs
    for b in bufs:
        ob = np.zeros((1, cfg.qcap, cfg.d), np.uint16)
        oc = np.zeros(1, np.int32)
        osel = O.prefill(qn[b:b + 1], ob, oc, cfg.n_beacon)
        w = f"{where} buffer {b}"
        assert g_qc[b] == oc[0], w
        assert np.array_equal(g_sel[b], osel[0]), f"{w}: selection {g_sel[b]} vs {osel[0]}"
        n = int(oc[0])
        assert np.array_equal(g_buf[b, :n], ob[0, :n]), f"{w}: buffer rows"
        assert np.all(g_buf[b, n:] == 0x7F7F), f"{w}: rows past the count were written"


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("P", [0, 1, 2, 5, 16, 17, 100, 511, 512, 513, 1024, 1025, 1500, 2049, 4100])
def test_prefill_matches_oracle(d, P):
    cfg = SMALL.scaled(d=d)
    _flush(f"prefill d={d} P={P}")
    q = synth.make_prompt_queries(cfg, P, device="cuda", seed=1000 + P + d)
    _check(cfg, q, P, where=f"d={d} P={P}")


@pytest.mark.parametrize("d", [64, 128])
def test_prefill_longest_prompt(d):
    cfg = SMALL.scaled(d=d, batch=1)
    P = L.BKV_PREFILL_MAX
    _flush(f"prefill d={d} P={P}")
    q = synth.make_prompt_queries(cfg, P, device="cuda", seed=77 + d)
    _check(cfg, q, P, where=f"d={d} P={P}")


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("P", [40, 700, 1300])
def test_prefill_ties(d, P):
    """Duplicated rows, zero rows and rows scaled by powers of two: many exactly equal cosines, so the
    lowest-index rule decides."""
    cfg = SMALL.scaled(d=d)
    _flush(f"prefill ties d={d} P={P}")
    g = torch.Generator(device="cpu").manual_seed(5 + P)
    base = torch.randn(cfg.qbufs, 12, d, generator=g)
    pick = torch.randint(0, 12, (cfg.qbufs, P), generator=g)
    x = torch.gather(base, 1, pick.unsqueeze(-1).expand(-1, -1, d))
    x = x * (2.0 ** torch.randint(-3, 4, (cfg.qbufs, P, 1), generator=g)).float()
    x[:, ::7] = 0.0
    q = x.to(torch.bfloat16).reshape(cfg.n_layers, cfg.batch, cfg.hq, P, d).cuda()
    _check(cfg, q, P, where=f"ties d={d} P={P}")


@pytest.mark.parametrize("src", ["initial", "random"])
@pytest.mark.parametrize("P", [0, 9, 16, 300, 5000])
def test_prefill_other_sources(src, P):
    cfg = SMALL.scaled(d=128, beacon=src, seed=31 + P)
    _flush(f"prefill {src} P={P}")
    q = synth.make_prompt_queries(cfg, P, device="cuda", seed=500 + P)
    g_buf, g_qc, g_sel = _run(cfg, q, P)
    qn = synth.to_u16(q).reshape(cfg.qbufs, P, cfg.d)
    ob = np.full((cfg.qbufs, cfg.qcap, cfg.d), 0x7F7F, np.uint16)
    oc = np.zeros(cfg.qbufs, np.int32)
    osel = O.prefill(qn, ob, oc, cfg.n_beacon, src={"initial": O.SRC_INITIAL, "random": O.SRC_RANDOM}[src],
                     seed=cfg.seed)
    assert np.array_equal(g_qc, oc)
    assert np.array_equal(g_sel, osel)
    assert np.array_equal(g_buf, ob)


def test_prefill_full_size_sampled_buffers():
    """The benchmark's workload (every query head of the Qwen3-4B-shaped batch, 1024-query prompts), same
    launch; the oracle checks a sample of buffers."""
    cfg, P = PREFILL.base, PREFILL.n_prompt
    _flush(f"prefill full size: {cfg.qbufs} buffers, P={P}")
    q = synth.make_prompt_queries(cfg, P, device="cuda")
    rng = np.random.default_rng(3)
    bufs = sorted(set([0, cfg.qbufs - 1] + rng.choice(cfg.qbufs, 22, replace=False).tolist()))
    _check(cfg, q, P, bufs=bufs, where="full size")
    del q
    torch.cuda.empty_cache()


def test_prefill_rejects_bad_lengths():
    """The C entry point refuses a negative or too long prompt before launching; the binding refuses a
    prompt tensor smaller than the length says."""
    import ctypes as C
    cfg = SMALL
    shape = L.shape_of(cfg)
    q = torch.zeros((cfg.qbufs, 4, cfg.d), dtype=torch.bfloat16, device="cuda")
    qbuf = torch.zeros((cfg.qbufs, cfg.qcap, cfg.d), dtype=torch.bfloat16, device="cuda")
    qc = torch.zeros((cfg.qbufs,), dtype=torch.int32, device="cuda")
    so = L.load()
    ptr = lambda t: C.c_void_p(t.data_ptr())
    assert so.bkv_fps_prefill(C.byref(shape), ptr(q), -1, ptr(qbuf), ptr(qc), None, None) == -1
    assert so.bkv_fps_prefill(C.byref(shape), ptr(q), L.BKV_PREFILL_MAX + 1, ptr(qbuf), ptr(qc), None, None) == -2
    assert so.bkv_fps_prefill(C.byref(shape), None, 4, ptr(qbuf), ptr(qc), None, None) == -1
    with pytest.raises(ValueError):
        L.fps_prefill(shape, q, 5, qbuf, qc)
