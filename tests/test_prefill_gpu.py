"""Prefill initialisation of the query buffers (bkv_fps_prefill) against the oracle.

Every buffer's selection order, count and buffer rows must equal the oracle's
bit for bit (the sampling decides integers from fp32 arithmetic that both
sides carry out in the same order).  The cases cover both head sizes, prompts
shorter than the buffer, prompts held in registers, in LDS and re-read from
memory, the longest prompt taken, and inputs full of ties (duplicate rows,
zero rows, rows that differ by a power of two).
"""
from __future__ import annotations

import time

import numpy as np
import pytest
import torch

import oracle as O
from long_reasoning_decode_amd import lib as L
from long_reasoning_decode_amd import synth
from long_reasoning_decode_amd.configs import PREFILL, TINY

import _helpers as H

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


def _oracle_prefill(qn: np.ndarray, cfg, nthreads: int | None = None):
    """The oracle's prefill of every buffer of qn [nbuf, P, d], slices of buffers on host threads (the C
    oracle releases the interpreter lock).  Returns (qbuf, qcount, sel) like _run."""
    nbuf = qn.shape[0]
    ob = np.zeros((nbuf, cfg.qcap, cfg.d), np.uint16)
    oc = np.zeros(nbuf, np.int32)
    osel = np.zeros((nbuf, cfg.n_beacon), np.int32)

    def one(sl):
        osel[sl] = O.prefill(qn[sl], ob[sl], oc[sl], cfg.n_beacon)

    H.on_threads(one, nbuf, nthreads)
    return ob, oc, osel


def _check(cfg, q: torch.Tensor, P: int, bufs=None, where=""):
    g_buf, g_qc, g_sel = _run(cfg, q, P)
    qn = synth.to_u16(q).reshape(cfg.qbufs, P, cfg.d)
    bufs = np.arange(cfg.qbufs) if bufs is None else np.asarray(bufs)
    t0 = time.perf_counter()
    ob, oc, osel = _oracle_prefill(np.ascontiguousarray(qn[bufs]), cfg)
    t_oracle = time.perf_counter() - t0
    g_buf, g_qc, g_sel = g_buf[bufs], g_qc[bufs], g_sel[bufs]
    for k, b in enumerate(bufs):
        w = f"{where} buffer {b}"
        assert g_qc[k] == oc[k], w
        assert np.array_equal(g_sel[k], osel[k]), f"{w}: selection {g_sel[k]} vs {osel[k]}"
        n = int(oc[k])
        assert np.array_equal(g_buf[k, :n], ob[k, :n]), f"{w}: buffer rows"
        assert np.all(g_buf[k, n:] == 0x7F7F), f"{w}: rows past the count were written"
    return t_oracle


# Across the kernel's layouts: every row in registers (up to 512 or 1024 rows at d = 128 or 64 on the fp32
# path, up to 1024 or 2048 on the packed path), one row per thread in LDS (fp32 path), several LDS rows,
# and rows re-read from memory; each boundary from both sides.
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("P", [0, 1, 2, 5, 16, 17, 100, 511, 512, 513, 1024, 1025, 1500, 1536, 1537, 1600, 2048,
                               2049, 4100])
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


@pytest.mark.parametrize("P", [PREFILL.n_prompt, 4096])
def test_prefill_full_size_all_buffers(P):
    """The benchmark's workloads (every query head of the Qwen3-4B-shaped batch, 1024- and 4096-query
    prompts), same launch; the oracle checks every buffer."""
    cfg = PREFILL.base
    _flush(f"prefill full size: {cfg.qbufs} buffers, P={P}")
    q = synth.make_prompt_queries(cfg, P, device="cuda")
    t = _check(cfg, q, P, where="full size")
    _flush(f"  {cfg.qbufs} buffers checked, oracle {t:.1f} s")
    del q
    torch.cuda.empty_cache()


def _check_plain(cfg, q: torch.Tensor, P: int, bufs, where=""):
    """Every pick of the GPU's sampling, replayed through the plain fp64 definition (the mean cosine summed
    over all n rows, then the greedy steps): its regret, the fp64 value of the row taken minus the best
    value at that step, must be within H.fps_band, which bounds what fp32 rounding can change.  Returns
    (picks, picks that differ from the fp64 optimum, steps whose fp64 margin lies inside the band)."""
    _, g_qc, g_sel = _run(cfg, q, P)
    bufs = list(bufs)
    qn = synth.to_u16(q.reshape(cfg.qbufs, P, cfg.d).index_select(0, torch.tensor(bufs, device=q.device)))
    m = min(P, cfg.n_beacon)
    band = H.fps_band(cfg.d, P)
    reg = np.zeros((len(bufs), m))
    mar = np.zeros((len(bufs), m))

    def one(sl):
        for k in range(sl.start, sl.stop):
            b = bufs[k]
            sel, reg[k], mar[k] = O.fps_plain(np.ascontiguousarray(qn[k]), cfg.n_beacon, forced=g_sel[b, :m])
            assert sel == g_sel[b, :m].tolist()

    H.on_threads(one, len(bufs))
    for k, b in enumerate(bufs):
        assert g_qc[b] == m, f"{where} buffer {b}: count"
        assert (reg[k] <= band).all(), (f"{where} buffer {b}: step {int(np.argmax(reg[k]))} regret "
                                        f"{reg[k].max():.3g} beyond the fp32 band {band:.3g}")
    return reg.size, int((reg > 0).sum()), int((mar < band).sum())


PLAIN_CASES = [("small", 64, 700), ("small", 128, 1500), ("full", 128, 1024), ("full", 128, 4096),
               ("longest", 128, 8192)]


@pytest.mark.parametrize("kind,d,P", PLAIN_CASES, ids=[f"{k}-d{d}-P{P}" for k, d, P in PLAIN_CASES])
def test_prefill_against_plain_definition(kind, d, P):
    """The prefill sampling against the page's definition in fp64, independent of the canonical fp32 order
    the kernel and bkvo_fps_long share: the full-size workloads (sampled buffers, the launch the benchmark
    times), small ones (every buffer) and the longest prompt."""
    if kind == "full":
        cfg = PREFILL.base
        bufs = np.random.default_rng(P).choice(cfg.qbufs, 96 if P <= 1024 else 24, replace=False).tolist()
        q = synth.make_prompt_queries(cfg, P, device="cuda")
    else:
        cfg = SMALL.scaled(d=d, batch=1) if kind == "longest" else SMALL.scaled(d=d)
        bufs = range(cfg.qbufs)
        q = synth.make_prompt_queries(cfg, P, device="cuda", seed=4000 + P + d)
    _flush(f"prefill vs plain definition {kind} d={d} P={P}: {len(bufs)} buffers")
    picks, off, near = _check_plain(cfg, q, P, bufs, where=f"{kind} d={d} P={P}")
    _flush(f"  {picks} picks within the band; {off} differ from the fp64 optimum; {near} fp64 margins inside "
           f"the band {H.fps_band(cfg.d, P):.2e}")
    del q
    torch.cuda.empty_cache()


def test_prefill_ties_against_plain_definition():
    """Exact ties (duplicated and power-of-two scaled rows): every pick is optimal for the definition."""
    cfg = SMALL.scaled(d=128)
    P = 700
    g = torch.Generator(device="cpu").manual_seed(55)
    base = torch.randn(cfg.qbufs, 12, cfg.d, generator=g)
    pick = torch.randint(0, 12, (cfg.qbufs, P), generator=g)
    x = torch.gather(base, 1, pick.unsqueeze(-1).expand(-1, -1, cfg.d))
    x = x * (2.0 ** torch.randint(-3, 4, (cfg.qbufs, P, 1), generator=g)).float()
    q = x.to(torch.bfloat16).reshape(cfg.n_layers, cfg.batch, cfg.hq, P, cfg.d).cuda()
    picks, off, near = _check_plain(cfg, q, P, range(cfg.qbufs), where="ties")
    _flush(f"ties: {picks} picks within the band; {off} differ from the fp64 optimum")


@pytest.mark.parametrize("d,hcap,n_rows", [(128, 700, 500), (64, 300, 300), (128, 2100, 17), (128, 64, 0),
                                           (128, 5000, 4100)])
def test_fps_history_matches_prefill(d, hcap, n_rows):
    """Beacons from the first n_rows of each buffer's history (rows hcap apart): the prefill sampling of those
    rows, bit-exact against the oracle, and every pick within the fp32 band of the plain definition; the
    history's later rows are never read (they hold NaNs)."""
    cfg = SMALL.scaled(d=d)
    _flush(f"fps_history d={d} hcap={hcap} n_rows={n_rows}")
    q = synth.make_prompt_queries(cfg, hcap, device="cuda", seed=900 + hcap + n_rows).reshape(cfg.qbufs, hcap, d)
    q[:, n_rows:] = float("nan")
    shape = L.shape_of(cfg)
    qbuf = torch.full((cfg.qbufs, cfg.qcap, d), 0x7F7F, dtype=torch.int16, device="cuda").view(torch.bfloat16)
    qc = torch.full((cfg.qbufs,), -5, dtype=torch.int32, device="cuda")
    sel = torch.full((cfg.qbufs, cfg.n_beacon), -7, dtype=torch.int32, device="cuda")
    L.fps_history(shape, q, hcap, n_rows, qbuf, qc, sel)
    torch.cuda.synchronize()
    g_buf, g_qc, g_sel = synth.to_u16(qbuf), qc.cpu().numpy(), sel.cpu().numpy()
    qn = np.ascontiguousarray(synth.to_u16(q)[:, :n_rows])
    ob, oc, osel = _oracle_prefill(qn, cfg)
    assert np.array_equal(g_qc, oc) and np.array_equal(g_sel, osel)
    for b in range(cfg.qbufs):
        n = int(oc[b])
        assert np.array_equal(g_buf[b, :n], ob[b, :n]), b
    m = min(n_rows, cfg.n_beacon)
    if n_rows > cfg.n_beacon:
        for b in range(cfg.qbufs):
            _, reg, _ = O.fps_plain(qn[b], cfg.n_beacon, forced=g_sel[b, :m])
            assert (reg <= H.fps_band(d, n_rows)).all(), b


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
