"""GPU parity: the HIP library (through its C ABI) against the CPU oracle on the
same seeded inputs.

Bars: FPS selections and merged buffers bit-exact; kept-index sets exact
except for keys tied with the k-th score (|s - s_k| <= 1e-6 and <= 2e-4 s_k);
scores within 1e-4 relative (+1e-30); compacted K/V rows byte-identical to the
gather of the original rows by the kept indices.
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle as O
from long_reasoning_decode_amd import lib as L
from long_reasoning_decode_amd import synth
from long_reasoning_decode_amd.configs import (QWEN3_4B, QWEN3_4B_MEAN, QWEN3_14B_1K, QWEN3_14B_4K, R1_QWEN_7B,
                                               TINY, EvictConfig)

import _helpers as H

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    L.load()
    yield


def _flush(msg: str) -> None:
    print(msg, flush=True)


# ---------------------------------------------------------------------------
# Continual FPS update and merge.

def _adversarial_buffers(nbuf: int, d: int, qcap: int, rng: np.random.Generator) -> np.ndarray:
    X = rng.standard_normal((nbuf, qcap, d)).astype(np.float32)
    for b in range(nbuf):
        kind = b % 6
        if kind == 1:    # duplicated rows
            X[b, 5] = X[b, 9]
            X[b, 20] = X[b, 9]
        elif kind == 2:  # +- basis vectors: exact cosine ties
            X[b, :8] = 0
            for i in range(8):
                X[b, i, i // 2] = 1.0 if i % 2 == 0 else -1.0
        elif kind == 3:  # power-of-two scaled rows
            X[b] *= 2.0 ** rng.integers(-8, 9, size=(qcap, 1))
        elif kind == 4:  # a zero row (cosine defined as 0)
            X[b, 3] = 0
        elif kind == 5:  # tight clusters: many near-ties
            c = rng.standard_normal((3, d))
            X[b] = c[rng.integers(0, 3, qcap)] * 10 + 0.01 * rng.standard_normal((qcap, d))
    return X


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("fill", [31, 30, 0, 17])
def test_fps_update_matches_oracle(d, fill):
    rng = np.random.default_rng(100 + d + fill)
    cfg = TINY.scaled(d=d, n_layers=3, batch=5, hq=8, hkv=2)
    nbuf, qcap = cfg.qbufs, cfg.qcap
    X = _adversarial_buffers(nbuf, d, qcap, rng)
    qb = torch.from_numpy(X).to(torch.bfloat16)
    qn = torch.from_numpy(rng.standard_normal((nbuf, d)).astype(np.float32)).to(torch.bfloat16)
    qc = np.full(nbuf, fill, np.int32)
    qc[::7] = rng.integers(0, 31, size=len(qc[::7]))
    qbuf_h = synth.to_u16(qb).copy()
    qc_h = qc.copy()
    sel_o = O.fps_update(qbuf_h, qc_h, synth.to_u16(qn), cfg.n_beacon, cfg.n_recent_q)
    qbuf_d = qb.cuda()
    qc_d = torch.from_numpy(qc).cuda()
    sel_d = torch.full((nbuf, cfg.n_beacon), -7, dtype=torch.int32, device="cuda")
    L.fps_update(L.shape_of(cfg), qbuf_d, qc_d, qn.cuda(), sel_d)
    torch.cuda.synchronize()
    assert np.array_equal(qc_d.cpu().numpy(), qc_h)
    assert np.array_equal(sel_d.cpu().numpy(), sel_o)
    g = synth.to_u16(qbuf_d)
    for b in range(nbuf):
        n = qc_h[b]
        assert np.array_equal(g[b, :n], qbuf_h[b, :n]), b


def test_fps_update_out_of_range_counts():
    """Counts outside [0, B_Q^max - 1] are clamped on entry (negative ones read as 0, large ones as a full
    buffer), as the oracle does."""
    rng = np.random.default_rng(321)
    cfg = TINY.scaled(d=128, n_layers=2, batch=3, hq=8, hkv=2)
    nbuf, qcap, d = cfg.qbufs, cfg.qcap, cfg.d
    X = _adversarial_buffers(nbuf, d, qcap, rng)
    qb = torch.from_numpy(X).to(torch.bfloat16)
    qn = torch.from_numpy(rng.standard_normal((nbuf, d)).astype(np.float32)).to(torch.bfloat16)
    vals = np.array([-5, -1, 0, 30, 31, 32, 33, 100, 1 << 30, -(1 << 30)], np.int32)
    qc = vals[np.arange(nbuf) % len(vals)].astype(np.int32)
    qbuf_h = synth.to_u16(qb).copy()
    qc_h = qc.copy()
    sel_o = O.fps_update(qbuf_h, qc_h, synth.to_u16(qn), cfg.n_beacon, cfg.n_recent_q)
    qbuf_d = qb.cuda()
    qc_d = torch.from_numpy(qc).cuda()
    sel_d = torch.full((nbuf, cfg.n_beacon), -7, dtype=torch.int32, device="cuda")
    L.fps_update(L.shape_of(cfg), qbuf_d, qc_d, qn.cuda(), sel_d)
    torch.cuda.synchronize()
    assert np.array_equal(qc_d.cpu().numpy(), qc_h)
    assert np.array_equal(sel_d.cpu().numpy(), sel_o)
    g = synth.to_u16(qbuf_d)
    live = np.arange(qcap)[None, :, None] < qc_h[:, None, None]
    assert np.array_equal(np.where(live, g, 0), np.where(live, qbuf_h, 0))


@pytest.mark.parametrize("nb,nrq", [(16, 16), (31, 1), (1, 31), (0, 20), (20, 0)])
def test_fps_compress_matches_oracle(nb, nrq):
    """Freeze-point compression: buffers holding more than n_beacon rows (counts of every value, out of range
    ones included) are sampled to n_beacon, the others left alone; bit-exact against the oracle."""
    rng = np.random.default_rng(700 + nb)
    cfg = TINY.scaled(d=128, n_layers=3, batch=5, hq=8, hkv=2, n_beacon=nb, n_recent_q=nrq)
    nbuf, qcap, d = cfg.qbufs, cfg.qcap, cfg.d
    X = _adversarial_buffers(nbuf, d, qcap, rng)
    qb = torch.from_numpy(X).to(torch.bfloat16)
    qc = rng.integers(-3, nb + nrq + 4, nbuf).astype(np.int32)
    qbuf_h = synth.to_u16(qb).copy()
    qc_h = qc.copy()
    sel_o = O.fps_compress(qbuf_h, qc_h, nb, nrq)
    qbuf_d = qb.cuda()
    qc_d = torch.from_numpy(qc).cuda()
    sel_d = torch.full((nbuf, max(nb, 1)), -7, dtype=torch.int32, device="cuda")
    L.fps_compress(L.shape_of(cfg), qbuf_d, qc_d, sel_d if nb > 0 else None)
    torch.cuda.synchronize()
    assert np.array_equal(qc_d.cpu().numpy(), qc_h)
    if nb > 0:
        assert np.array_equal(sel_d.cpu().numpy(), sel_o)
    g = synth.to_u16(qbuf_d)
    for b in range(nbuf):
        n = max(int(qc_h[b]), 0)
        assert np.array_equal(g[b, :n], qbuf_h[b, :n]), b
    if nb > 0 and nrq > 1:   # counts up to B_Q^max - 1 > n_beacon occur: some buffers were sampled
        assert (sel_o[:, 0] >= 0).any()


@pytest.mark.parametrize("nb,nrq", [(32, 0), (0, 32), (31, 1), (1, 31), (4, 28), (28, 4),
                                    (1, 0), (2, 3), (8, 8), (15, 2)])
def test_fps_update_splits(nb, nrq):
    """Every split of the 32-row buffer, the degenerate ones included: n_recent_q = 0 (a full buffer keeps
    all its rows) and n_beacon = 0 (a full buffer keeps none); and buffers whose B_Q^max is below 32, down
    to a single row."""
    rng = np.random.default_rng(500 + nb)
    cfg = TINY.scaled(d=128, n_layers=3, batch=5, hq=8, hkv=2, n_beacon=nb, n_recent_q=nrq)
    nbuf, qcap, d = cfg.qbufs, cfg.qcap, cfg.d
    X = _adversarial_buffers(nbuf, d, qcap, rng)
    qb = torch.from_numpy(X).to(torch.bfloat16)
    qn = torch.from_numpy(rng.standard_normal((nbuf, d)).astype(np.float32)).to(torch.bfloat16)
    bqmax = nb + nrq
    qc = np.where(rng.random(nbuf) < 0.5, bqmax - 1, rng.integers(0, bqmax, nbuf)).astype(np.int32)
    qbuf_h = synth.to_u16(qb).copy()
    qc_h = qc.copy()
    sel_o = O.fps_update(qbuf_h, qc_h, synth.to_u16(qn), nb, nrq)
    qbuf_d = qb.cuda()
    qc_d = torch.from_numpy(qc).cuda()
    sel_d = torch.full((nbuf, nb), -7, dtype=torch.int32, device="cuda")
    L.fps_update(L.shape_of(cfg), qbuf_d, qc_d, qn.cuda(), sel_d if nb > 0 else None)
    torch.cuda.synchronize()
    assert np.array_equal(qc_d.cpu().numpy(), qc_h)
    if nb > 0:
        assert np.array_equal(sel_d.cpu().numpy(), sel_o)
    g = synth.to_u16(qbuf_d)
    live = np.arange(qcap)[None, :, None] < qc_h[:, None, None]
    assert np.array_equal(np.where(live, g, 0), np.where(live, qbuf_h, 0))


@pytest.mark.parametrize("d,nbuf,nb", [(64, 100_000, 16), (128, 30_000, 16), (128, 30_000, 31)])
def test_fps_update_several_buffers_per_wave(d, nbuf, nb):
    """More buffers than the chip holds waves at once, so each wave updates a run of them (one or more
    passes of up to 32, whose full buffers are sampled four at a time): full and non-full buffers mixed
    within a run, so that the groups of four are ragged, adversarial contents in the first few hundred."""
    rng = np.random.default_rng(300 + d + nb)
    cfg = TINY.scaled(d=d, n_layers=1, batch=nbuf // 8, hq=8, hkv=2, n_beacon=nb, n_recent_q=32 - nb)
    assert cfg.qbufs == nbuf
    X = rng.standard_normal((nbuf, cfg.qcap, d), dtype=np.float32)
    X[:600] = _adversarial_buffers(600, d, cfg.qcap, rng)
    qb = torch.from_numpy(X).to(torch.bfloat16)
    del X
    qn = torch.randn(nbuf, d, generator=torch.Generator().manual_seed(301 + d)).to(torch.bfloat16)
    qc = np.where(rng.random(nbuf) < 0.6, 31, rng.integers(0, 31, nbuf)).astype(np.int32)
    qbuf_h = synth.to_u16(qb).copy()
    qc_h = qc.copy()
    _flush(f"fps update d={d} nbuf={nbuf} n_beacon={nb}: oracle")
    sel_o = O.fps_update(qbuf_h, qc_h, synth.to_u16(qn), cfg.n_beacon, cfg.n_recent_q)
    qbuf_d = qb.cuda()
    qc_d = torch.from_numpy(qc).cuda()
    sel_d = torch.full((nbuf, cfg.n_beacon), -7, dtype=torch.int32, device="cuda")
    _flush("  device")
    L.fps_update(L.shape_of(cfg), qbuf_d, qc_d, qn.cuda(), sel_d)
    torch.cuda.synchronize()
    assert np.array_equal(qc_d.cpu().numpy(), qc_h)
    assert np.array_equal(sel_d.cpu().numpy(), sel_o)
    g = synth.to_u16(qbuf_d)
    n = qc_h[:, None, None]
    live = np.arange(cfg.qcap)[None, :, None] < n
    assert np.array_equal(np.where(live, g, 0), np.where(live, qbuf_h, 0))


@pytest.mark.parametrize("cfg", [TINY, QWEN3_4B.scaled(n_layers=2, batch=3), R1_QWEN_7B.scaled(n_layers=1, batch=2)],
                         ids=lambda c: c.name)
def test_fps_update_many_random_buffers(cfg):
    """Full buffers of the workload's query mixture: one sampling round each."""
    cfgx = cfg.scaled(batch=max(cfg.batch, 64)) if cfg.name == "tiny" else cfg
    q = synth.make_query_buffers(cfgx, device="cuda")
    nbuf = cfgx.qbufs
    qbuf_h = synth.to_u16(q["qbuf"]).reshape(nbuf, cfgx.qcap, cfgx.d).copy()
    qc_h = q["qcount"].cpu().numpy().reshape(nbuf).copy()
    sel_o = O.fps_update(qbuf_h, qc_h, synth.to_u16(q["q_new"]).reshape(nbuf, cfgx.d),
                         cfgx.n_beacon, cfgx.n_recent_q)
    sel_d = torch.full((nbuf, cfgx.n_beacon), -7, dtype=torch.int32, device="cuda")
    L.fps_update(L.shape_of(cfgx), q["qbuf"], q["qcount"], q["q_new"], sel_d)
    torch.cuda.synchronize()
    assert np.array_equal(sel_d.cpu().numpy(), sel_o)
    assert np.array_equal(q["qcount"].cpu().numpy().reshape(-1), qc_h)
    g = synth.to_u16(q["qbuf"]).reshape(nbuf, cfgx.qcap, cfgx.d)
    assert np.array_equal(g[:, :cfgx.n_beacon], qbuf_h[:, :cfgx.n_beacon])


@pytest.mark.parametrize("src", ["initial", "random"])
@pytest.mark.parametrize("d", [64, 128])
def test_source_update_matches_oracle(src, d):
    """Initial and random-history beacons: three successive per-step updates from mixed counts."""
    rng = np.random.default_rng(300 + d + len(src))
    cfg = TINY.scaled(d=d, n_layers=3, batch=5, hq=8, hkv=2, beacon=src, seed=4242 + d)
    nbuf, qcap = cfg.qbufs, cfg.qcap
    oc = H.ocfg(cfg)
    qbuf_h = synth.to_u16(torch.from_numpy(rng.standard_normal((nbuf, qcap, d)).astype(np.float32))
                          .to(torch.bfloat16)).copy()
    qc_h = rng.integers(-2, 40, size=nbuf).astype(np.int32)
    qc_h[::9] = 1000 + rng.integers(0, 5000, size=len(qc_h[::9]))
    qbuf_d = torch.from_numpy(qbuf_h.view(np.int16)).cuda().view(torch.bfloat16)
    qc_d = torch.from_numpy(qc_h.copy()).cuda()
    shape = L.shape_of(cfg)
    for step in range(3):
        qn = torch.from_numpy(rng.standard_normal((nbuf, d)).astype(np.float32)).to(torch.bfloat16)
        sel_o = O.beacon_update(oc, qbuf_h, qc_h, synth.to_u16(qn))
        sel_d = torch.full((nbuf, cfg.n_beacon), -7, dtype=torch.int32, device="cuda")
        L.fps_update(shape, qbuf_d, qc_d, qn.cuda(), sel_d)
        torch.cuda.synchronize()
        assert np.array_equal(qc_d.cpu().numpy(), qc_h), step
        assert np.array_equal(sel_d.cpu().numpy(), sel_o), step
        assert np.array_equal(synth.to_u16(qbuf_d), qbuf_h), step


def test_random_source_update_many_buffers():
    """The random history at the stream's buffer count (221,184 buffers): two updates, every buffer
    compared (the draws are keyed by each buffer's global index)."""
    rng = np.random.default_rng(311)
    cfg = TINY.scaled(d=128, n_layers=36, batch=192, hq=32, hkv=8, beacon="random", seed=777)
    nbuf, qcap, d = cfg.qbufs, cfg.qcap, cfg.d
    assert nbuf == 221184
    oc = H.ocfg(cfg)
    qbuf_h = (rng.integers(0, 1 << 16, size=(nbuf, qcap, d), dtype=np.uint16) & 0xBFFF).astype(np.uint16)
    qc_h = rng.integers(0, 3000, size=nbuf).astype(np.int32)
    qbuf_d = torch.from_numpy(qbuf_h.view(np.int16)).cuda().view(torch.bfloat16)
    qc_d = torch.from_numpy(qc_h.copy()).cuda()
    shape = L.shape_of(cfg)
    for step in range(2):
        qn = (rng.integers(0, 1 << 16, size=(nbuf, d), dtype=np.uint16) & 0xBFFF).astype(np.uint16)
        O.beacon_update(oc, qbuf_h, qc_h, qn)
        L.fps_update(shape, qbuf_d, qc_d, torch.from_numpy(qn.view(np.int16)).cuda().view(torch.bfloat16), None)
        torch.cuda.synchronize()
        assert np.array_equal(qc_d.cpu().numpy(), qc_h), step
        assert np.array_equal(synth.to_u16(qbuf_d), qbuf_h), step


@pytest.mark.parametrize("src", ["initial", "random"])
def test_source_merge_matches_oracle(src):
    cfg = QWEN3_4B.scaled(n_layers=2, batch=3, beacon=src, seed=777)
    inp = synth.make_evict_inputs(cfg, device="cuda")
    qc = inp["qcount"].clone()
    qc.view(-1)[::5] = 3
    qc.view(-1)[1::7] = 5000
    v = synth.oracle_views(cfg, {**inp, "qcount": qc})
    sel_o = O.merge(H.ocfg(cfg), v["qbuf"], v["qcount"], v["q_recent"])
    qbuf = inp["qbuf"].clone()
    sel_d = torch.full((cfg.qbufs, cfg.n_beacon), -7, dtype=torch.int32, device="cuda")
    L.fps_merge(L.shape_of(cfg), qbuf, qc, inp["q_recent"], sel_d)
    torch.cuda.synchronize()
    G = cfg.G
    assert np.array_equal(sel_d.cpu().numpy().reshape(cfg.units, G, -1), sel_o)
    assert np.array_equal(qc.cpu().numpy().reshape(cfg.units, G), v["qcount"])
    assert np.array_equal(synth.to_u16(qbuf).reshape(cfg.units, G, cfg.qcap, cfg.d), v["qbuf"])


@pytest.mark.parametrize("qcount", [16, 9, 0, 20])
def test_fps_merge_matches_oracle(qcount):
    cfg = QWEN3_4B.scaled(n_layers=2, batch=3)
    inp = synth.make_evict_inputs(cfg, device="cuda", qcount=qcount)
    qc = inp["qcount"].clone()
    qc.view(-1)[::5] = 3
    v = synth.oracle_views(cfg, {**inp, "qcount": qc})
    sel_o = O.merge(H.ocfg(cfg), v["qbuf"], v["qcount"], v["q_recent"])
    qbuf = inp["qbuf"].clone()
    sel_d = torch.full((cfg.qbufs, cfg.n_beacon), -7, dtype=torch.int32, device="cuda")
    L.fps_merge(L.shape_of(cfg), qbuf, qc, inp["q_recent"], sel_d)
    torch.cuda.synchronize()
    G = cfg.G
    assert np.array_equal(sel_d.cpu().numpy().reshape(cfg.units, G, -1), sel_o)
    assert np.array_equal(qc.cpu().numpy().reshape(cfg.units, G), v["qcount"])
    g = synth.to_u16(qbuf).reshape(cfg.units, G, cfg.qcap, cfg.d)
    for u in range(cfg.units):
        for h in range(G):
            n = v["qcount"][u, h]
            assert np.array_equal(g[u, h, :n], v["qbuf"][u, h, :n])


@pytest.mark.parametrize("d,nb,batch,nrq", [(64, 16, 3, 16), (128, 16, 1001, 16), (128, 31, 333, 1),
                                             (64, 4, 5, 28), (128, 2, 7, 3), (128, 8, 9, 8), (64, 1, 3, 1)])
def test_fps_merge_adversarial_odd_counts(d, nb, batch, nrq):
    """Merge over an odd number of buffers (the last wave has one), with adversarial contents and counts
    from 0 to n_beacon (and some outside that range, clamped), so pairs mix sampling and non-sampling
    buffers; B_Q^max = 32 and smaller."""
    rng = np.random.default_rng(400 + d + nb + batch)
    cfg = TINY.scaled(d=d, n_layers=1, batch=batch, hq=3, hkv=1, n_beacon=nb, n_recent_q=nrq)
    nbuf, G = cfg.qbufs, cfg.G
    assert nbuf % 2 == 1
    X = _adversarial_buffers(nbuf, d, cfg.qcap, rng)
    R = _adversarial_buffers(nbuf, d, cfg.n_recent_q, rng) if cfg.n_recent_q >= 21 else \
        rng.standard_normal((nbuf, cfg.n_recent_q, d)).astype(np.float32)
    qb = torch.from_numpy(X).to(torch.bfloat16)
    qr = torch.from_numpy(R).to(torch.bfloat16)
    qc = rng.integers(0, nb + 1, nbuf).astype(np.int32)
    qc[::11] = -3                 # out of range: read as 0 beacons
    qc[5::13] = nb + 7            # out of range: read as n_beacon beacons
    qbuf_h = synth.to_u16(qb).reshape(cfg.units, G, cfg.qcap, d).copy()
    qc_h = qc.reshape(cfg.units, G).copy()
    sel_o = O.merge(H.ocfg(cfg), qbuf_h, qc_h, synth.to_u16(qr).reshape(cfg.units, G, cfg.n_recent_q, d))
    qbuf_d = qb.cuda()
    qc_d = torch.from_numpy(qc).cuda()
    sel_d = torch.full((nbuf, nb), -7, dtype=torch.int32, device="cuda")
    L.fps_merge(L.shape_of(cfg), qbuf_d, qc_d, qr.cuda(), sel_d)
    torch.cuda.synchronize()
    assert np.array_equal(sel_d.cpu().numpy().reshape(cfg.units, G, -1), sel_o)
    assert np.array_equal(qc_d.cpu().numpy().reshape(cfg.units, G), qc_h)
    g = synth.to_u16(qbuf_d).reshape(cfg.units, G, cfg.qcap, d)
    live = np.arange(cfg.qcap)[None, None, :, None] < qc_h[:, :, None, None]
    assert np.array_equal(np.where(live, g, 0), np.where(live, qbuf_h, 0))


# ---------------------------------------------------------------------------
# Scores.

SCORE_CASES = [
    (TINY, None, 1),
    (TINY, 97, 1),
    (TINY, 160, 0),
    (QWEN3_4B.scaled(n_layers=2, batch=2), None, 1),
    (QWEN3_4B.scaled(n_layers=1, batch=2), 1000, 1),
    (R1_QWEN_7B.scaled(n_layers=1, batch=2), None, 1),
    (QWEN3_14B_1K.scaled(n_layers=1, batch=2), None, 1),
    (QWEN3_14B_4K.scaled(n_layers=1, batch=1), None, 1),
    (TINY.scaled(hq=8, hkv=1, name="g8"), 150, 1),
    (TINY.scaled(hq=3, hkv=3, name="g1"), 33, 1),
    (TINY.scaled(hq=6, hkv=2, name="g3"), 159, 1),
    (TINY.scaled(hq=6, hkv=1, name="g6"), 140, 1),
    (TINY.scaled(d=128, hq=5, hkv=1, name="g5d128"), 160, 1),
    (TINY.scaled(n_recent_q=0, name="nrq0"), 160, 1),
    (TINY.scaled(n_beacon=0, name="nb0"), 160, 1),
    (TINY.scaled(d=128, budget=8064, n_new=128, n_prefix=4, name="n8192"), 8192, 1),
    (TINY, 10, 1),                  # fewer keys than recent queries: recent rows 0-5 see nothing
    (TINY, 1, 1),                   # a single key: only the beacons and the last recent row see it
    # mean pooling (flags 3: causal + mean, 2: mean alone) on every workgroup layout
    (TINY, None, 3),
    (TINY, 10, 3),
    (TINY, 160, 2),
    (QWEN3_4B.scaled(n_layers=2, batch=2), None, 3),
    (R1_QWEN_7B.scaled(n_layers=1, batch=2), None, 3),
    (TINY.scaled(hq=3, hkv=3, name="g1"), 33, 3),
    (TINY.scaled(hq=6, hkv=2, name="g3"), 159, 3),
    (TINY.scaled(hq=8, hkv=1, name="g8"), 150, 2),
    (TINY.scaled(d=128, hq=5, hkv=1, name="g5d128"), 160, 3),
    (TINY.scaled(n_recent_q=0, name="nrq0"), 160, 3),
    (TINY.scaled(n_beacon=0, name="nb0"), 160, 3),
    (TINY.scaled(d=128, budget=8064, n_new=128, n_prefix=4, name="n8192"), 8192, 3),
]


@pytest.mark.parametrize("cfg,n_len,flags", SCORE_CASES,
                         ids=[f"{c.name}-{n}-{z}" for c, n, z in SCORE_CASES])
def test_score_matches_oracle(cfg, n_len, flags):
    N = cfg.n_len if n_len is None else n_len
    _flush(f"score {cfg.name} N={N} flags={flags}")
    inp = synth.make_evict_inputs(cfg, device="cuda")
    qc = inp["qcount"]
    qc.view(-1)[::3] = 5     # some buffers hold fewer beacons
    qc.view(-1)[1::7] = 0
    shape = L.shape_of(cfg, cap=cfg.n_len, flags=flags)
    scores = torch.empty((cfg.units, N), dtype=torch.float32, device="cuda")
    L.score(shape, inp["K"], N, inp["qbuf"], qc, inp["q_recent"], inp["pos_recent"], inp["t"],
            H.rope_dev(cfg), scores)
    torch.cuda.synchronize()
    v = synth.oracle_views(cfg, inp)
    o = O.score(H.ocfg(cfg, n_len=cfg.n_len, flags=flags), v["K"], v["qbuf"], v["qcount"], v["q_recent"],
                v["pos_recent"], v["t"], n_len=N)
    H.check_scores(scores.cpu().numpy(), o, f"{cfg.name} N={N}")


# ---------------------------------------------------------------------------
# Keep set.

@pytest.mark.parametrize("n_len,budget,npf,nr", [(2176, 2048, 4, 16), (160, 128, 8, 16), (1000, 1000, 4, 16),
                                                  (4224, 4096, 4, 16), (33, 20, 0, 0), (8192, 100, 50, 50),
                                                  (300, 20, 4, 16),
                                                  (2049, 2048, 4, 16),     # exactly one row evicted
                                                  (100, 150, 4, 16)])      # budget above n_len: -1 padding
def test_select_matches_oracle(n_len, budget, npf, nr):
    rng = np.random.default_rng(n_len + budget)
    U = 24
    s = (rng.random((U, n_len)) ** 4).astype(np.float32)
    s[1] = np.round(s[1] * 20) / 20          # many exact ties
    s[2] = 0.5                               # all equal
    s[3, :] = 0.0                            # zeros
    s[4] = rng.integers(0, 3, n_len) * np.float32(1e-30)
    cfg = QWEN3_4B.scaled(n_layers=1, batch=U, hkv=1, hq=1, budget=budget, n_new=n_len - budget,
                          n_prefix=npf, n_recent_kv=nr)
    shape = L.shape_of(cfg, cap=n_len)
    idx = torch.full((U, budget), -7, dtype=torch.int32, device="cuda")
    L.select(shape, torch.from_numpy(s).cuda(), n_len, idx)
    torch.cuda.synchronize()
    g = idx.cpu().numpy()
    for u in range(U):
        ref, _ = O.select(s[u].astype(np.float64), budget, npf, nr)
        assert np.array_equal(g[u], ref), u


# ---------------------------------------------------------------------------
# Compaction.

def _index_lists(U, n_len, budget, rng):
    lists = []
    for u in range(U):
        kind = u % 6
        if kind == 0:
            sel = np.arange(budget)                                       # identity
        elif kind == 1:
            sel = np.arange(1, budget + 1)                                # single hole at 0
        elif kind == 2:
            sel = np.arange(n_len - budget, n_len)                        # keep only the tail
        elif kind == 3:
            sel = np.sort(rng.choice(n_len, budget, replace=False))
        elif kind == 4:
            sel = np.concatenate([np.arange(budget - 1), [n_len - 1]])    # last row only moves
        else:
            sel = np.sort(np.concatenate([np.arange(0, n_len, 2)[: budget // 2],
                                          np.arange(1, n_len, 2)[-(budget - budget // 2):]]))
        lists.append(sel[:budget])
    return np.stack(lists).astype(np.int32)


@pytest.mark.parametrize("d,n_len,budget", [(128, 2176, 2048), (64, 160, 128), (128, 300, 37), (128, 4224, 4096)])
def test_compact_matches_oracle(d, n_len, budget):
    rng = np.random.default_rng(d + n_len)
    U = 30
    cfg = TINY.scaled(d=d, n_layers=1, batch=U, hq=1, hkv=1, budget=budget, n_new=n_len - budget)
    idx = _index_lists(U, n_len, budget, rng)
    K = torch.from_numpy(rng.standard_normal((U, n_len, d)).astype(np.float32)).to(torch.bfloat16)
    V = torch.from_numpy(rng.standard_normal((U, n_len, d)).astype(np.float32)).to(torch.bfloat16)
    Kh, Vh = synth.to_u16(K).copy(), synth.to_u16(V).copy()
    O.compact(H.ocfg(cfg), Kh, Vh, idx, n_len=n_len)
    Kd, Vd = K.cuda(), V.cuda()
    L.compact(L.shape_of(cfg, cap=n_len), Kd, Vd, n_len, torch.from_numpy(idx).cuda())
    torch.cuda.synchronize()
    assert np.array_equal(synth.to_u16(Kd), Kh)
    assert np.array_equal(synth.to_u16(Vd), Vh)


# ---------------------------------------------------------------------------
# The whole eviction.

EVICT_CASES = [
    (TINY, None, 1),
    (TINY, 159, 1),
    (TINY, 128, 1),                 # nothing to evict
    (TINY, 129, 1),                 # exactly one row evicted
    (QWEN3_4B.scaled(n_layers=1, batch=2), 2049, 1),
    (TINY, 150, 0),
    (QWEN3_4B.scaled(n_layers=2, batch=2), None, 1),
    (R1_QWEN_7B.scaled(n_layers=1, batch=2), None, 1),
    (QWEN3_14B_1K.scaled(n_layers=1, batch=2), None, 1),
    (QWEN3_14B_4K.scaled(n_layers=1, batch=1), None, 1),
    (TINY.scaled(hq=8, hkv=1, name="g8"), 150, 1),
    # every workgroup layout of the fused kernel (query heads per unit 1, 2, 3-4, 5-8) and both head sizes
    (TINY.scaled(hq=3, hkv=3, name="g1"), 160, 1),
    (TINY.scaled(hq=3, hkv=3, name="g1"), 33, 1),          # one partial stage, nothing to evict
    (TINY.scaled(hq=6, hkv=2, name="g3"), 159, 1),
    (TINY.scaled(hq=6, hkv=1, name="g6"), 140, 0),
    (TINY.scaled(d=128, hq=5, hkv=1, name="g5d128"), 160, 1),
    (TINY.scaled(d=128, hq=2, hkv=2, name="g1d128"), 97, 1),
    # no recent queries; no beacons
    (TINY.scaled(n_recent_q=0, name="nrq0"), 160, 1),
    (TINY.scaled(n_beacon=0, name="nb0"), 160, 1),
    # the longest cache the kernels take (8192 keys)
    (TINY.scaled(d=128, budget=8064, n_new=128, n_prefix=4, name="n8192"), 8192, 1),
    # initial / random-history beacons (flags 5: causal + initial, 9: causal + random)
    (TINY.scaled(seed=91), None, 5),
    (TINY.scaled(seed=92), None, 9),
    (QWEN3_4B.scaled(n_layers=2, batch=2), None, 9),
    # mean pooling (flags 3: causal + mean, 2: mean alone)
    (TINY, None, 3),
    (TINY, 150, 2),
    (QWEN3_4B.scaled(n_layers=2, batch=2), None, 3),
    (R1_QWEN_7B.scaled(n_layers=1, batch=2), None, 3),
    (QWEN3_14B_1K.scaled(n_layers=1, batch=2), None, 3),
    (TINY.scaled(hq=3, hkv=3, name="g1"), 160, 3),
    (TINY.scaled(hq=6, hkv=2, name="g3"), 159, 3),
    (TINY.scaled(hq=6, hkv=1, name="g6"), 140, 2),
    (TINY.scaled(d=128, hq=5, hkv=1, name="g5d128"), 160, 3),
    (TINY.scaled(n_beacon=0, name="nb0"), 160, 3),
    (TINY.scaled(d=128, budget=8064, n_new=128, n_prefix=4, name="n8192"), 8192, 3),
]


@pytest.mark.parametrize("cfg,n_len,flags", EVICT_CASES, ids=[f"{c.name}-{n}-{z}" for c, n, z in EVICT_CASES])
def test_evict_matches_oracle(cfg, n_len, flags):
    N = cfg.n_len if n_len is None else n_len
    _flush(f"evict {cfg.name} N={N} flags={flags}")
    inp = synth.make_evict_inputs(cfg, device="cuda")
    inp["qcount"].view(-1)[::5] = 7
    out = H.run_evict_gpu(cfg, inp, N, flags=flags)
    r = H.compare_evict(cfg, inp, out, N, flags=flags, where=f"{cfg.name} N={N}")
    _flush(f"  tie-band differences: {r['n_tie_diff']}")


# Full workload size, the launch the benchmark times, every unit checked against the oracle.  The oracle runs
# chunk by chunk over the units (host threads over units); the qwen3-14b-b4096 workload is split into two tests
# so that each stays well inside a test's time limit.
FULL = [(QWEN3_4B, 0, 1), (R1_QWEN_7B, 0, 1), (QWEN3_14B_1K, 0, 1), (QWEN3_14B_4K, 0, 2), (QWEN3_14B_4K, 1, 2),
        (QWEN3_4B_MEAN, 0, 1)]


def _part(cfg: EvictConfig, part: int, parts: int) -> list:
    lo, hi = part * cfg.units // parts, (part + 1) * cfg.units // parts
    return list(range(lo, hi))


@pytest.mark.parametrize("flags", [L.BKV_CAUSAL_RECENT | L.BKV_BEACON_INITIAL, L.BKV_CAUSAL_RECENT | L.BKV_BEACON_RANDOM],
                         ids=["initial", "random"])
def test_evict_full_size_beacon_sources(flags):
    """Full qwen3-4b size with the other beacon sources (the merge offers the recents to the reservoir, keyed
    by the global buffer index), every unit checked."""
    cfg = QWEN3_4B
    _flush(f"full-size evict {cfg.name} flags {flags}: {cfg.units} units")
    inp = synth.make_evict_inputs(cfg, device="cuda")
    out = H.run_evict_gpu(cfg, inp, cfg.n_len, flags=flags)
    r = H.compare_evict_all(cfg, inp, out, cfg.n_len, flags=flags, where=f"{cfg.name} flags {flags}")
    assert r["units"] == cfg.units
    _flush(f"  {r['units']} units checked, oracle {r['oracle_s']:.1f} s, tie-band differences: {r['n_tie_diff']}")
    del inp, out
    torch.cuda.empty_cache()


@pytest.mark.parametrize("cfg,part,parts", FULL, ids=[f"{c.name}-{p}of{n}" for c, p, n in FULL])
def test_evict_full_size_all_units(cfg, part, parts):
    """Full workload size, the same launch as the benchmark; the oracle checks every unit (of this part of
    the workload): scores, keep sets, compacted rows and merged buffers."""
    units = _part(cfg, part, parts)
    _flush(f"full-size evict {cfg.name}: units [{units[0]}, {units[-1] + 1}) of {cfg.units}, N={cfg.n_len}")
    inp = synth.make_evict_inputs(cfg, device="cuda")
    out = H.run_evict_gpu(cfg, inp, cfg.n_len)
    r = H.compare_evict_all(cfg, inp, out, cfg.n_len, units=units, where=cfg.name)
    assert r["units"] == len(units)
    _flush(f"  {r['units']} units checked, oracle {r['oracle_s']:.1f} s, tie-band differences: {r['n_tie_diff']}")
    del inp, out
    torch.cuda.empty_cache()


def test_evict_rejects_bad_shapes_without_launching():
    cfg = TINY
    inp = synth.make_evict_inputs(cfg, device="cuda")
    shape = L.shape_of(cfg)
    with pytest.raises(L.BkvError) as e:
        L.evict(shape, inp["K"], inp["V"], cfg.n_len + 1, inp["qbuf"], inp["qcount"], inp["q_recent"],
                inp["pos_recent"], inp["t"], H.rope_dev(cfg), idx_out=torch.empty((2, 128), dtype=torch.int32,
                                                                                   device="cuda"),
                scores_out=torch.empty((2, 161), device="cuda"))
    assert e.value.code == -3


def test_positions_outside_the_table_are_clamped():
    """Positions below 0 or past the RoPE table read its first or last row: the eviction (beacons at t, recents
    at their own positions), the key append and decode attention give bit for bit what they give with the
    positions clamped into the table."""
    cfg = TINY.scaled(name="clamp", n_layers=2, batch=3)
    rope = H.rope_dev(cfg)
    R = rope.shape[0]
    inp = synth.make_evict_inputs(cfg, device="cuda")
    bad = {k: v.clone() for k, v in inp.items()}
    bad["t"] = torch.tensor([-7, R + 100, 5], dtype=torch.int32, device="cuda")
    pr = bad["pos_recent"].clone()
    pr[0, :5] = torch.arange(-5, 0, dtype=torch.int32, device="cuda")
    pr[1, -3:] = R + torch.arange(3, dtype=torch.int32, device="cuda")
    pr[2, 0] = -(1 << 30)
    pr[2, 1] = (1 << 31) - 1
    bad["pos_recent"] = pr
    good = {k: v.clone() for k, v in inp.items()}
    good["t"] = bad["t"].clamp(0, R - 1)
    good["pos_recent"] = bad["pos_recent"].clamp(0, R - 1)
    ob = H.run_evict_gpu(cfg, bad, cfg.n_len, rope=rope)
    og = H.run_evict_gpu(cfg, good, cfg.n_len, rope=rope)
    for k in ("scores", "idx", "fps_sel", "K", "V", "qbuf", "qcount"):
        assert torch.equal(ob[k].view(torch.uint8), og[k].view(torch.uint8)), k
    shape = L.shape_of(cfg)
    g = torch.Generator(device="cuda").manual_seed(3)
    kn = torch.randn(cfg.units, cfg.d, generator=g, device="cuda").to(torch.bfloat16)
    vn = torch.randn(cfg.units, cfg.d, generator=g, device="cuda").to(torch.bfloat16)
    Kb, Vb, Kg, Vg = inp["K"].clone(), inp["V"].clone(), inp["K"].clone(), inp["V"].clone()
    L.append_kv(shape, Kb, Vb, cfg.n_len - 2, kn, vn, bad["t"], rope)
    L.append_kv(shape, Kg, Vg, cfg.n_len - 2, kn, vn, good["t"], rope)
    q = inp["q_recent"][..., 0, :].contiguous()
    ab = torch.empty((cfg.qbufs, cfg.d), dtype=torch.float32, device="cuda")
    ag = torch.empty_like(ab)
    L.decode_attention(shape, inp["K"], inp["V"], cfg.n_len, q, bad["t"], rope, ab)
    L.decode_attention(shape, inp["K"], inp["V"], cfg.n_len, q, good["t"], rope, ag)
    torch.cuda.synchronize()
    assert torch.equal(Kb.view(torch.uint8), Kg.view(torch.uint8)) and torch.equal(Vb, Vg)
    assert torch.equal(ab.view(torch.uint8), ag.view(torch.uint8))


@pytest.mark.parametrize("cfg", [TINY, QWEN3_4B.scaled(n_layers=2, batch=2), R1_QWEN_7B.scaled(n_layers=1, batch=2),
                                 QWEN3_4B_MEAN.scaled(n_layers=2, batch=2), TINY.scaled(name="tiny-mean", pool="mean")],
                         ids=lambda c: c.name)
def test_evict_equals_the_separate_calls(cfg):
    """bkv_evict (one fused kernel per unit, then the merge) gives bit for bit what bkv_score, bkv_select,
    bkv_compact and bkv_fps_merge give one after the other, with or without its optional outputs."""
    N = cfg.n_len
    _flush(f"evict vs separate calls {cfg.name}")
    inp = synth.make_evict_inputs(cfg, device="cuda")
    inp["qcount"].view(-1)[::5] = 7
    rope = H.rope_dev(cfg)
    shape = L.shape_of(cfg, cap=N)
    fused = H.run_evict_gpu(cfg, inp, N, rope=rope)

    sep = {k: v.clone() for k, v in inp.items()}
    scores = torch.empty((cfg.units, N), dtype=torch.float32, device="cuda")
    idx = torch.empty((cfg.units, cfg.budget), dtype=torch.int32, device="cuda")
    sel = torch.empty((cfg.qbufs, cfg.n_beacon), dtype=torch.int32, device="cuda")
    L.score(shape, sep["K"], N, sep["qbuf"], sep["qcount"], sep["q_recent"], sep["pos_recent"], sep["t"], rope, scores)
    L.select(shape, scores, N, idx)
    L.compact(shape, sep["K"], sep["V"], N, idx)
    L.fps_merge(shape, sep["qbuf"], sep["qcount"], sep["q_recent"], sel)

    bare = {k: v.clone() for k, v in inp.items()}
    L.evict(shape, bare["K"], bare["V"], N, bare["qbuf"], bare["qcount"], bare["q_recent"], bare["pos_recent"],
            bare["t"], rope)
    torch.cuda.synchronize()
    assert torch.equal(fused["scores"], scores)
    assert torch.equal(fused["idx"], idx)
    assert torch.equal(fused["fps_sel"], sel)
    for k in ("K", "V", "qbuf", "qcount"):
        assert torch.equal(fused[k], sep[k]), k
        assert torch.equal(bare[k], sep[k]), k
