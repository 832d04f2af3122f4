"""GPU parity over seeded random shapes: every field of bkv_shape drawn within
the library's limits (head size, query heads per KV head 1..8, every split of
the query buffer, buffer strides qcap above B_Q^max, forced keeps from 0,
budgets below and above the cache length, causal or not, max or mean pooling,
each beacon source), with query counts that include out-of-range values.
Bars as in the other parity tests: selections, keep sets (up to the tie band)
and buffers exact, scores within 1e-4 relative, compacted rows byte-identical.
"""
from __future__ import annotations

import os

import numpy as np
import pytest
import torch

import oracle as O
from long_reasoning_decode_amd import lib as L
from long_reasoning_decode_amd import synth
from long_reasoning_decode_amd.configs import TINY

import _helpers as H
from _stream_helpers import check_run

pytestmark = pytest.mark.gpu

# The draws are fixed; BKV_RANDOM_SHAPES_SEED (default 0) offsets every generator's seed, for further sweeps.
_OFF = int(os.environ.get("BKV_RANDOM_SHAPES_SEED", "0"))

_SRC = {"fps": 0, "initial": L.BKV_BEACON_INITIAL, "random": L.BKV_BEACON_RANDOM}


def _split(rng: np.random.Generator) -> tuple:
    """(n_beacon, n_recent_q) with 1 <= n_beacon + n_recent_q <= 32; the edges (no beacons, no recents, a full
    32) drawn often."""
    k = rng.integers(0, 5)
    if k == 0:
        return 0, int(rng.integers(1, 33))
    if k == 1:
        return int(rng.integers(1, 33)), 0
    if k == 2:
        nb = int(rng.integers(1, 32))
        return nb, 32 - nb
    nb = int(rng.integers(0, 32))
    return nb, int(rng.integers(1 if nb == 0 else 0, 33 - nb))


def _evict_cases(n: int, seed: int) -> list:
    rng = np.random.default_rng(seed)
    out = []
    for i in range(n):
        d = int(rng.choice([64, 128]))
        hkv = int(rng.integers(1, 4))
        G = int(rng.integers(1, 9))
        nb, nrq = _split(rng)
        qcap = nb + nrq + int(rng.choice([0, 0, 1, 3, 9]))
        npf = int(rng.choice([0, 1, 4, 8, 16]))
        nrk = int(rng.choice([0, 1, 16, 32]))
        budget = npf + nrk + int(rng.integers(1, 700))
        n_new = int(rng.integers(1, 300))
        cap = budget + n_new
        kind = rng.integers(0, 6)
        N = {0: cap, 1: budget + 1, 2: max(1, budget), 3: max(1, budget - int(rng.integers(0, 40)))}.get(
            int(kind), int(rng.integers(budget + 1, cap + 1)))
        N = min(N, cap)
        flags = (L.BKV_CAUSAL_RECENT if rng.random() < 0.7 else 0) | (L.BKV_POOL_MEAN if rng.random() < 0.3 else 0)
        src = str(rng.choice(["fps", "fps", "initial", "random"]))
        flags |= _SRC[src]
        t_lo = int(rng.integers(40, 9000))
        t_hi = t_lo + int(rng.integers(0, 24000))
        cfg = TINY.scaled(name=f"r{i}", d=d, hq=hkv * G, hkv=hkv, n_layers=int(rng.integers(1, 3)),
                          batch=int(rng.integers(1, 4)), theta=float(rng.choice([1e4, 1e6])), budget=budget,
                          n_new=n_new, n_prefix=npf, n_recent_kv=nrk, n_beacon=nb, n_recent_q=nrq, qcap=qcap,
                          t_lo=t_lo, t_hi=t_hi, mix=str(rng.choice(["clusters8", "tight3"])),
                          seed=int(rng.integers(1, 1 << 31)), beacon=src)
        out.append((cfg, N, flags))
    # two long caches, one workgroup each
    for i, (d, G) in enumerate([(128, 5), (64, 8)]):
        nb, nrq = _split(rng)
        cfg = TINY.scaled(name=f"long{i}", d=d, hq=G, hkv=1, budget=int(rng.integers(4000, 8000)), n_new=0,
                          n_prefix=4, n_recent_kv=16, n_beacon=nb, n_recent_q=nrq, qcap=nb + nrq + 2,
                          t_lo=9000, t_hi=30000, mix="clusters8", seed=int(rng.integers(1, 1 << 31)))
        cfg = cfg.scaled(n_new=8192 - cfg.budget)
        out.append((cfg, 8192, L.BKV_CAUSAL_RECENT))
    return out


EVICT = _evict_cases(40, 20261202 + _OFF)


def _id(c) -> str:
    cfg, N, flags = c
    return (f"{cfg.name}-d{cfg.d}-g{cfg.G}x{cfg.hkv}-q{cfg.n_beacon}+{cfg.n_recent_q}/{cfg.qcap}"
            f"-k{cfg.n_prefix}+{cfg.n_recent_kv}-b{cfg.budget}-n{N}-f{flags}")


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    L.load()
    yield


@pytest.mark.parametrize("case", EVICT, ids=[_id(c) for c in EVICT])
def test_evict_random_shape(case):
    cfg, N, flags = case
    print(f"evict {_id(case)}", flush=True)
    inp = synth.make_evict_inputs(cfg, device="cuda")
    rng = np.random.default_rng(cfg.seed)
    qc = rng.integers(-2, cfg.qcap + 3, inp["qcount"].shape).astype(np.int32)
    inp["qcount"] = torch.from_numpy(qc).cuda()
    out = H.run_evict_gpu(cfg, inp, N, flags=flags)
    H.compare_evict(cfg, inp, out, N, flags=flags, where=_id(case))


def _buffer_cases(n: int, seed: int) -> list:
    rng = np.random.default_rng(seed)
    out = []
    for i in range(n):
        nb, nrq = _split(rng)
        out.append((int(rng.choice([64, 128])), nb, nrq, nb + nrq + int(rng.choice([0, 1, 5])),
                    int(rng.integers(1, 300)), int(rng.integers(1, 1 << 31))))
    return out


BUFFERS = _buffer_cases(16, 4242 + _OFF)


def _bid(c) -> str:
    d, nb, nrq, qcap, nbuf, _ = c
    return f"d{d}-q{nb}+{nrq}/{qcap}-x{nbuf}"


def _rows(rng, n, r, d):
    return torch.from_numpy(rng.standard_normal((n, r, d)).astype(np.float32)).to(torch.bfloat16)


@pytest.mark.parametrize("case", BUFFERS, ids=[_bid(c) for c in BUFFERS])
def test_fps_update_random_shape(case):
    """One decode step's buffer update over buffers of a random stride and split, counts from below 0 to
    past the stride (clamped on entry)."""
    d, nb, nrq, qcap, nbuf, seed = case
    print(f"fps_update {_bid(case)}", flush=True)
    rng = np.random.default_rng(seed)
    cfg = TINY.scaled(d=d, n_layers=1, batch=nbuf, hq=1, hkv=1, n_beacon=nb, n_recent_q=nrq, qcap=qcap)
    qb, qn = _rows(rng, nbuf, qcap, d), _rows(rng, nbuf, 1, d)[:, 0]
    bqmax = nb + nrq
    qc = np.where(rng.random(nbuf) < 0.5, bqmax - 1, rng.integers(-2, qcap + 3, nbuf)).astype(np.int32)
    qbuf_h, qc_h = synth.to_u16(qb).copy(), qc.copy()
    sel_o = O.fps_update(qbuf_h, qc_h, synth.to_u16(qn), nb, nrq)
    qbuf_d, qc_d = qb.cuda(), torch.from_numpy(qc).cuda()
    sel_d = torch.full((nbuf, max(nb, 1)), -7, dtype=torch.int32, device="cuda")
    L.fps_update(L.shape_of(cfg), qbuf_d, qc_d, qn.cuda(), sel_d if nb > 0 else None)
    torch.cuda.synchronize()
    assert np.array_equal(qc_d.cpu().numpy(), qc_h)
    if nb > 0:
        assert np.array_equal(sel_d.cpu().numpy(), sel_o)
    g = synth.to_u16(qbuf_d)
    live = np.arange(qcap)[None, :, None] < qc_h[:, None, None]
    assert np.array_equal(np.where(live, g, 0), np.where(live, qbuf_h, 0))


@pytest.mark.parametrize("case", BUFFERS, ids=[_bid(c) for c in BUFFERS])
def test_fps_merge_random_shape(case):
    """The end-of-cycle merge over buffers of a random stride and split, beacon counts out of range
    included."""
    d, nb, nrq, qcap, nbuf, seed = case
    print(f"fps_merge {_bid(case)}", flush=True)
    rng = np.random.default_rng(seed + 1)
    cfg = TINY.scaled(d=d, n_layers=1, batch=nbuf, hq=1, hkv=1, n_beacon=nb, n_recent_q=nrq, qcap=qcap)
    qb, qr = _rows(rng, nbuf, qcap, d), _rows(rng, nbuf, nrq, d)
    qc = rng.integers(-2, qcap + 3, nbuf).astype(np.int32)
    qbuf_h = synth.to_u16(qb).reshape(nbuf, 1, qcap, d).copy()
    qc_h = qc.reshape(nbuf, 1).copy()
    sel_o = O.merge(H.ocfg(cfg), qbuf_h, qc_h, synth.to_u16(qr).reshape(nbuf, 1, nrq, d))
    qbuf_d, qc_d = qb.cuda(), torch.from_numpy(qc).cuda()
    sel_d = torch.full((nbuf, max(nb, 1)), -7, dtype=torch.int32, device="cuda")
    L.fps_merge(L.shape_of(cfg), qbuf_d, qc_d, qr.cuda() if nrq > 0 else None, sel_d if nb > 0 else None)
    torch.cuda.synchronize()
    if nb > 0:
        assert np.array_equal(sel_d.cpu().numpy().reshape(nbuf, 1, -1), sel_o)
    assert np.array_equal(qc_d.cpu().numpy().reshape(nbuf, 1), qc_h)
    g = synth.to_u16(qbuf_d).reshape(nbuf, 1, qcap, d)
    live = np.arange(qcap)[None, None, :, None] < qc_h[:, :, None, None]
    assert np.array_equal(np.where(live, g, 0), np.where(live, qbuf_h, 0))


def _stream_cases(n: int, seed: int) -> list:
    """Short decode streams of random shape: every source (naive full history included), both poolings,
    strides above B_Q^max, at least three evictions each."""
    from dataclasses import replace
    from long_reasoning_decode_amd.configs import TINY_STREAM
    rng = np.random.default_rng(seed)
    out = []
    for i in range(n):
        d = int(rng.choice([64, 128]))
        hkv = int(rng.integers(1, 3))
        G = int(rng.integers(1, 9))
        nb, nrq = _split(rng)
        npf = int(rng.choice([0, 2, 8]))
        nrk = int(rng.choice([0, 1, 16]))
        budget = npf + nrk + int(rng.integers(1, 160))
        n_new = nrq + int(rng.integers(1, 60))
        src = str(rng.choice(["fps", "fps", "initial", "random", "naive"]))
        base = replace(TINY, name=f"s{i}", d=d, hq=hkv * G, hkv=hkv, batch=int(rng.integers(1, 3)),
                       budget=budget, n_new=n_new, n_prefix=npf, n_recent_kv=nrk, n_beacon=nb, n_recent_q=nrq,
                       qcap=nb + nrq + int(rng.choice([0, 2, 7])), pool=str(rng.choice(["max", "mean"])),
                       beacon=src, mix=str(rng.choice(["clusters8", "tight3"])), seed=int(rng.integers(1, 1 << 31)))
        steps = base.cap + 3 * n_new + int(rng.integers(0, n_new))
        out.append(replace(TINY_STREAM, name=f"stream-s{i}", base=base, steps=steps, drift_every=64,
                           p0_max=int(rng.integers(1, 5000))))
    return out


STREAMS = _stream_cases(14, 777 + _OFF)


def _sid(s) -> str:
    b = s.base
    return (f"{s.name}-d{b.d}-g{b.G}x{b.hkv}-q{b.n_beacon}+{b.n_recent_q}/{b.qcap}-k{b.n_prefix}+{b.n_recent_kv}"
            f"-b{b.budget}+{b.n_new}-{b.beacon}-{b.pool}")


@pytest.mark.parametrize("scfg", STREAMS, ids=[_sid(s) for s in STREAMS])
def test_stream_random_shape(scfg):
    """Decode steps and evictions from an empty cache, every unit recorded, against the oracle's replay."""
    from long_reasoning_decode_amd.stream import StreamRun
    print(f"stream {_sid(scfg)} steps {scfg.steps}", flush=True)
    units = range(scfg.base.units)
    run = StreamRun(scfg, record_units=units, block=40)
    r = run.run()
    assert r["evictions"] == scfg.evictions() >= 3
    check_run(scfg, run, units, _sid(scfg))


def _prefill_cases(n: int, seed: int) -> list:
    """Prompt sampling of random shape: every split (n_beacon 0 to 32), strides above B_Q^max, prompt lengths
    from empty to the longest taken, each source; and the same sampling from a history of random stride."""
    rng = np.random.default_rng(seed)
    out = []
    for i in range(n):
        d = int(rng.choice([64, 128]))
        nb, nrq = _split(rng)
        k = int(rng.integers(0, 7))
        P = [0, 1, nb, nb + 1, int(rng.integers(2, 600)), int(rng.integers(600, 2200)),
             int(rng.integers(2200, L.BKV_PREFILL_MAX + 1))][k]
        hkv = int(rng.integers(1, 3))
        cfg = TINY.scaled(name=f"p{i}", d=d, n_layers=1, batch=int(rng.integers(1, 3)), hq=hkv * int(rng.integers(1, 3)),
                          hkv=hkv, n_beacon=nb, n_recent_q=nrq, qcap=nb + nrq + int(rng.choice([0, 3])),
                          beacon=str(rng.choice(["fps", "fps", "initial", "random"])),
                          seed=int(rng.integers(1, 1 << 31)))
        hcap = P + int(rng.choice([0, 1, 37]))
        out.append((cfg, P, hcap))
    return out


PREFILLS = _prefill_cases(24, 99 + _OFF)


def _pid(c) -> str:
    cfg, P, hcap = c
    return f"{cfg.name}-d{cfg.d}-x{cfg.qbufs}-q{cfg.n_beacon}+{cfg.n_recent_q}/{cfg.qcap}-P{P}-h{hcap}-{cfg.beacon}"


def _oracle_sample(cfg, qn: np.ndarray) -> tuple:
    """The oracle's prompt sampling of every buffer of qn [nbuf, P, d] under the workload's source."""
    nbuf = qn.shape[0]
    ob = np.full((nbuf, cfg.qcap, cfg.d), 0x7F7F, np.uint16)
    oc = np.zeros(nbuf, np.int32)
    src = {"fps": O.SRC_FPS, "initial": O.SRC_INITIAL, "random": O.SRC_RANDOM}[cfg.beacon]
    osel = O.prefill(qn, ob, oc, cfg.n_beacon, src=src, seed=cfg.seed)
    return ob, oc, osel


def _check_sampled(cfg, qbuf, qc, sel, ob, oc, osel, where) -> None:
    g_buf, g_qc = synth.to_u16(qbuf), qc.cpu().numpy()
    assert np.array_equal(g_qc, oc), where
    if cfg.n_beacon > 0:
        assert np.array_equal(sel.cpu().numpy(), osel), where
    for b in range(cfg.qbufs):
        n = int(oc[b])
        assert np.array_equal(g_buf[b, :n], ob[b, :n]), f"{where} buffer {b}: rows"
        assert np.all(g_buf[b, n:] == 0x7F7F), f"{where} buffer {b}: rows past the count were written"


def _outputs(cfg):
    qbuf = torch.full((cfg.qbufs, cfg.qcap, cfg.d), 0x7F7F, dtype=torch.int16, device="cuda").view(torch.bfloat16)
    qc = torch.full((cfg.qbufs,), -5, dtype=torch.int32, device="cuda")
    sel = torch.full((cfg.qbufs, max(cfg.n_beacon, 1)), -7, dtype=torch.int32, device="cuda")
    return qbuf, qc, sel


@pytest.mark.parametrize("case", PREFILLS, ids=[_pid(c) for c in PREFILLS])
def test_prefill_random_shape(case):
    cfg, P, _ = case
    print(f"prefill {_pid(case)}", flush=True)
    q = synth.make_prompt_queries(cfg, P, device="cuda", seed=cfg.seed)
    qbuf, qc, sel = _outputs(cfg)
    L.fps_prefill(L.shape_of(cfg), q, P, qbuf, qc, sel if cfg.n_beacon > 0 else None)
    torch.cuda.synchronize()
    ob, oc, osel = _oracle_sample(cfg, synth.to_u16(q).reshape(cfg.qbufs, P, cfg.d))
    _check_sampled(cfg, qbuf, qc, sel, ob, oc, osel, _pid(case))


@pytest.mark.parametrize("case", [c for c in PREFILLS if c[0].beacon == "fps"],
                         ids=[_pid(c) for c in PREFILLS if c[0].beacon == "fps"])
def test_fps_history_random_shape(case):
    """The naive source's sampling of the first n_rows of a history of stride hcap (the later rows hold
    NaNs and must not be read)."""
    cfg, n_rows, hcap = case
    print(f"fps_history {_pid(case)}", flush=True)
    q = synth.make_prompt_queries(cfg, hcap, device="cuda", seed=cfg.seed + 1).reshape(cfg.qbufs, hcap, cfg.d)
    q[:, n_rows:] = float("nan")
    qbuf, qc, sel = _outputs(cfg)
    L.fps_history(L.shape_of(cfg), q, hcap, n_rows, qbuf, qc, sel if cfg.n_beacon > 0 else None)
    torch.cuda.synchronize()
    ob, oc, osel = _oracle_sample(cfg, np.ascontiguousarray(synth.to_u16(q)[:, :n_rows]))
    _check_sampled(cfg, qbuf, qc, sel, ob, oc, osel, _pid(case))


SEPARATE = EVICT[::2]


@pytest.mark.parametrize("case", SEPARATE, ids=[_id(c) for c in SEPARATE])
def test_separate_calls_random_shape(case):
    """bkv_score against the oracle, bkv_select on those scores against the oracle's ranking of the same
    fp32 values, bkv_compact against the gather, bkv_fps_merge after them; and bkv_evict equal to the four
    calls bit for bit."""
    cfg, N, flags = case
    print(f"separate calls {_id(case)}", flush=True)
    inp = synth.make_evict_inputs(cfg, device="cuda")
    rng = np.random.default_rng(cfg.seed + 3)
    inp["qcount"] = torch.from_numpy(rng.integers(-2, cfg.qcap + 3, inp["qcount"].shape).astype(np.int32)).cuda()
    rope = H.rope_dev(cfg)
    shape = L.shape_of(cfg, cap=inp["K"].shape[-2], flags=flags)
    sep = {k: v.clone() for k, v in inp.items()}
    U, B = cfg.units, cfg.budget
    scores = torch.empty((U, N), dtype=torch.float32, device="cuda")
    idx = torch.full((U, B), -7, dtype=torch.int32, device="cuda")
    sel = torch.full((cfg.qbufs, max(cfg.n_beacon, 1)), -7, dtype=torch.int32, device="cuda")
    L.score(shape, sep["K"], N, sep["qbuf"], sep["qcount"], sep["q_recent"], sep["pos_recent"], sep["t"], rope, scores)
    L.select(shape, scores, N, idx)
    L.compact(shape, sep["K"], sep["V"], N, idx)
    L.fps_merge(shape, sep["qbuf"], sep["qcount"], sep["q_recent"] if cfg.n_recent_q > 0 else None,
                sel if cfg.n_beacon > 0 else None)
    fused = H.run_evict_gpu(cfg, inp, N, flags=flags, rope=rope)
    torch.cuda.synchronize()
    v = synth.oracle_views(cfg, inp)
    o = O.score(H.ocfg(cfg, n_len=inp["K"].shape[-2], flags=flags), v["K"], v["qbuf"], v["qcount"], v["q_recent"],
                v["pos_recent"], v["t"], n_len=N)
    g_s = scores.cpu().numpy()
    H.check_scores(g_s, o, _id(case))
    g_idx = idx.cpu().numpy()
    for u in range(U):
        ref, _ = O.select(g_s[u].astype(np.float64), B, cfg.n_prefix, cfg.n_recent_kv)
        assert np.array_equal(g_idx[u], ref), f"{_id(case)} unit {u}: keep set"
    m = min(N, B)
    K0 = synth.to_u16(inp["K"]).reshape(U, -1, cfg.d)
    V0 = synth.to_u16(inp["V"]).reshape(U, -1, cfg.d)
    gi = g_idx[:, :m]
    assert np.array_equal(synth.to_u16(sep["K"]).reshape(U, -1, cfg.d)[:, :m], np.take_along_axis(K0, gi[:, :, None], 1))
    assert np.array_equal(synth.to_u16(sep["V"]).reshape(U, -1, cfg.d)[:, :m], np.take_along_axis(V0, gi[:, :, None], 1))
    assert torch.equal(fused["scores"], scores) and torch.equal(fused["idx"], idx)
    if cfg.n_beacon > 0:
        assert torch.equal(fused["fps_sel"], sel)
    for k in ("K", "V", "qbuf", "qcount"):
        assert torch.equal(fused[k], sep[k]), k


@pytest.mark.parametrize("case", SEPARATE, ids=[_id(c) for c in SEPARATE])
def test_decode_attention_random_shape(case):
    """Decode attention of one query per head over the first n_len rows, at three cache lengths, against the
    oracle (|gpu - oracle| <= 1e-4 sum_j w_j |v_j| + 1e-6, the bar of the attention tests)."""
    cfg, N, _ = case
    inp = synth.make_evict_inputs(cfg, device="cuda")
    rng = np.random.default_rng(cfg.seed + 5)
    shape = L.shape_of(cfg, cap=inp["K"].shape[-2])
    rope = H.rope_dev(cfg)
    q = inp["q_recent"][..., 0, :].contiguous() if cfg.n_recent_q > 0 else inp["qbuf"][..., 0, :].contiguous()
    U, G, D = cfg.units, cfg.G, cfg.d
    oc = H.ocfg(cfg, n_len=inp["K"].shape[-2])
    v = synth.oracle_views(cfg, inp)
    qn = synth.to_u16(q).reshape(U, G, D)
    for n in sorted({1, N, int(rng.integers(1, cfg.n_len + 1))}):
        print(f"attention {_id(case)} n_len={n}", flush=True)
        out = torch.full((cfg.qbufs, D), float("nan"), dtype=torch.float32, device="cuda")
        L.decode_attention(shape, inp["K"], inp["V"], n, q, inp["t"], rope, out)
        torch.cuda.synchronize()
        o, scale = O.decode_attention(oc, v["K"], v["V"], np.ascontiguousarray(qn), v["t"], n)
        err = np.abs(out.reshape(U, G, D).cpu().numpy().astype(np.float64) - o)
        assert (err <= 1e-4 * scale + 1e-6).all(), f"{_id(case)} n_len={n}"
