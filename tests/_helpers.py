"""Shared helpers of the GPU parity tests: run the HIP path, run the oracle on
the same seeded inputs, and compare element by element."""
from __future__ import annotations

import math
import time

import numpy as np
import torch

import oracle as O
from long_reasoning_decode_amd import lib as L
from long_reasoning_decode_amd import synth
from long_reasoning_decode_amd.configs import EvictConfig

SCORE_RTOL = 1e-4        # relative score tolerance
SCORE_ATOL = 1e-30       # floor for scores that underflow
TIE_BAND_ABS = 1e-6      # keys within this of the k-th score may swap
TIE_BAND_REL = 2e-4      # ... and only if within twice the score tolerance


def fps_band(d: int, n: int) -> float:
    """Largest fp64 regret a pick of the fp32 FPS may show against the plain definition.

    With u = 2^-24 and gamma_k ~= k u, the fp32 cosine dot_ij / (nrm_i nrm_j) of bf16 rows (exact products,
    a d-term fma chain, two square roots, a product and a division) is within 2 gamma_d + 4u of the real
    cosine; the mean cosine of the prefill seed, u_i . (pairwise sum of the unit rows) / n, is within
    2 gamma_d + gamma_ceil(log2 n) + 7u of its real value (each bound uses |u_i . u_j| <= 1).  A greedy
    value S_j is a maximum of cosines, so it carries the cosine bound.  When the fp32 pick r and the real
    optimum r* differ, S32[r] <= S32[r*] gives S[r] - S[r*] <= twice the bound.  The band is that, with
    three u to spare for the fp64 reference's own rounding."""
    lg = max(1, math.ceil(math.log2(max(n, 2))))
    return 2.0 * (2 * d + lg + 10) * 2.0 ** -24


def on_threads(fn, n: int, nthreads: int | None = None) -> None:
    """fn(slice) over [0, n) cut into contiguous slices, one per host thread (for oracle calls, which release
    the interpreter lock)."""
    from concurrent.futures import ThreadPoolExecutor
    nt = max(1, min(n, nthreads or O.default_threads()))
    cuts = [i * n // nt for i in range(nt + 1)]
    with ThreadPoolExecutor(nt) as ex:
        list(ex.map(fn, [slice(a, b) for a, b in zip(cuts[:-1], cuts[1:]) if b > a]))


def ocfg(cfg: EvictConfig, n_len: int | None = None, flags: int | None = None) -> O.OracleCfg:
    """Oracle configuration of a workload; flags as in bkv.h (default: the workload's own)."""
    N = cfg.n_len if n_len is None else n_len
    flags = L.flags_of(cfg) if flags is None else flags
    return O.OracleCfg(hq=cfg.hq, hkv=cfg.hkv, d=cfg.d, cap=N, budget=cfg.budget,
                       n_prefix=cfg.n_prefix, n_recent_kv=cfg.n_recent_kv, n_beacon=cfg.n_beacon,
                       n_recent_q=cfg.n_recent_q, theta=cfg.theta, qcap=cfg.qcap,
                       causal=int(bool(flags & L.BKV_CAUSAL_RECENT)), pool_mean=int(bool(flags & L.BKV_POOL_MEAN)),
                       beacon_src=src_of(flags), seed=cfg.seed & 0xFFFFFFFF,
                       n_layers=cfg.n_layers, batch=cfg.batch)


def src_of(flags: int) -> int:
    """The oracle's beacon source for library flags."""
    if flags & L.BKV_BEACON_INITIAL:
        return O.SRC_INITIAL
    if flags & L.BKV_BEACON_RANDOM:
        return O.SRC_RANDOM
    return O.SRC_FPS


def rope_dev(cfg: EvictConfig) -> torch.Tensor:
    return torch.from_numpy(L.rope_table(cfg.theta, cfg.d, 0, cfg.rope_rows)).cuda()


def check_scores(gpu: np.ndarray, orc: np.ndarray, where: str = "") -> None:
    err = np.abs(gpu.astype(np.float64) - orc)
    lim = SCORE_RTOL * np.abs(orc) + SCORE_ATOL
    bad = err > lim
    if bad.any():
        i = np.argwhere(bad)[0]
        raise AssertionError(f"{where}: {bad.sum()} scores out of tolerance; first at {tuple(i)}: "
                             f"gpu {gpu[tuple(i)]!r} oracle {orc[tuple(i)]!r}")


def check_keep(idx_gpu: np.ndarray, idx_orc: np.ndarray, s_orc: np.ndarray, n_len: int, budget: int,
               n_prefix: int, n_recent_kv: int, where: str = "") -> int:
    """Kept sets equal except for keys tied (within the band) with the k-th
    oracle score; the GPU set must itself be a valid keep set.  Returns the
    number of keys that differ."""
    g = idx_gpu[idx_gpu >= 0]
    o = idx_orc[idx_orc >= 0]
    assert len(g) == len(o) == min(n_len, budget), where
    assert np.all(np.diff(g) > 0), f"{where}: GPU idx not strictly ascending"
    assert g.min() >= 0 and g.max() < n_len
    if n_len <= budget:
        assert np.array_equal(g, np.arange(n_len)), where
        return 0
    forced = np.zeros(n_len, bool)
    forced[:min(n_prefix, n_len)] = True
    forced[max(0, n_len - n_recent_kv):] = True
    gm = np.zeros(n_len, bool)
    gm[g] = True
    om = np.zeros(n_len, bool)
    om[o] = True
    assert gm[forced].all(), f"{where}: forced keeps missing"
    chosen = om & ~forced
    if not chosen.any():
        assert np.array_equal(gm, om), where
        return 0
    sk = s_orc[chosen].min()
    diff = np.flatnonzero(gm ^ om)
    dj = np.abs(s_orc[diff] - sk)
    bad = (dj > TIE_BAND_ABS) | (dj > TIE_BAND_REL * sk + SCORE_ATOL)
    if bad.any():
        j = diff[np.argmax(bad)]
        raise AssertionError(f"{where}: key {j} kept differently with score {s_orc[j]!r} vs k-th {sk!r}")
    return len(diff) // 2


def run_evict_gpu(cfg: EvictConfig, inp: dict, n_len: int, flags: int | None = None,
                  rope: torch.Tensor | None = None) -> dict:
    """bkv_evict on device copies of inp; returns the outputs (device tensors)."""
    d = {k: v.clone() for k, v in inp.items()}
    shape = L.shape_of(cfg, cap=inp["K"].shape[-2], flags=flags)
    U = cfg.units
    idx = torch.full((U, cfg.budget), -7, dtype=torch.int32, device="cuda")
    scores = torch.empty((U, n_len), dtype=torch.float32, device="cuda")
    fps_sel = torch.full((cfg.qbufs, cfg.n_beacon), -7, dtype=torch.int32, device="cuda")
    rope = rope_dev(cfg) if rope is None else rope
    L.evict(shape, d["K"], d["V"], n_len, d["qbuf"], d["qcount"], d["q_recent"], d["pos_recent"],
            d["t"], rope, idx_out=idx, scores_out=scores, fps_sel_out=fps_sel)
    torch.cuda.synchronize()
    d.update(idx=idx, scores=scores, fps_sel=fps_sel)
    return d


def compare_evict(cfg: EvictConfig, inp: dict, out: dict, n_len: int, units=None, flags: int | None = None,
                  where: str = "") -> dict:
    """Oracle on the listed units (default all) vs the GPU outputs."""
    U = cfg.units
    units = list(range(U)) if units is None else list(units)
    v = synth.oracle_views(cfg, inp, units)
    oc = ocfg(cfg, n_len=inp["K"].shape[-2], flags=flags)
    oc.unit_ids = units   # the random history's draws are keyed by the global buffer index
    K0, V0 = v["K"].copy(), v["V"].copy()
    t0 = time.perf_counter()
    o = O.evict(oc, v["K"], v["V"], v["qbuf"], v["qcount"], v["q_recent"], v["pos_recent"], v["t"],
                n_len=n_len)
    t_oracle = time.perf_counter() - t0
    ut = torch.tensor(units, dtype=torch.long, device="cuda")
    G, D = cfg.G, cfg.d
    g_scores = out["scores"].index_select(0, ut).cpu().numpy()
    g_idx = out["idx"].index_select(0, ut).cpu().numpy()
    g_K = synth.to_u16(out["K"].reshape(U, -1, D).index_select(0, ut))
    g_V = synth.to_u16(out["V"].reshape(U, -1, D).index_select(0, ut))
    g_qbuf = synth.to_u16(out["qbuf"].reshape(U, G, cfg.qcap, D).index_select(0, ut))
    g_qc = out["qcount"].reshape(U, G).index_select(0, ut).cpu().numpy()
    g_sel = out["fps_sel"].reshape(U, G, cfg.n_beacon).index_select(0, ut).cpu().numpy()
    check_scores(g_scores, o["scores"], where)
    n_diff = 0
    B = min(cfg.budget, n_len)
    for k, u in enumerate(units):
        n_diff += check_keep(g_idx[k], o["idx"][k], o["scores"][k], n_len, cfg.budget, cfg.n_prefix,
                             cfg.n_recent_kv, f"{where} unit {u}")
    # compacted rows: byte-identical to the gather of the original rows by the GPU's own keep set, which
    # equals the oracle's compaction wherever the two keep sets agree
    gi = g_idx[:, :B]
    _first_bad(g_K[:, :B] == np.take_along_axis(K0, gi[:, :, None], axis=1), units, f"{where}: K rows differ "
               "from the gather")
    _first_bad(g_V[:, :B] == np.take_along_axis(V0, gi[:, :, None], axis=1), units, f"{where}: V rows differ "
               "from the gather")
    same = (gi == o["idx"][:, :B]).all(axis=1)
    _first_bad((g_K[same, :B] == v["K"][same, :B]), [u for u, s_ in zip(units, same) if s_], f"{where}: K vs oracle")
    _first_bad((g_V[same, :B] == v["V"][same, :B]), [u for u, s_ in zip(units, same) if s_], f"{where}: V vs oracle")
    # merged buffers: counts, selections and the live rows bit-exact
    _first_bad(g_qc == v["qcount"], units, f"{where}: qcount")
    _first_bad(g_sel == o["fps_sel"], units, f"{where}: merge FPS selection")
    live = np.arange(cfg.qcap)[None, None, :, None] < v["qcount"][:, :, None, None]
    _first_bad(np.where(live, g_qbuf, 0) == np.where(live, v["qbuf"], 0), units, f"{where}: merged buffer")
    return {"n_tie_diff": n_diff, "oracle": o, "oracle_s": t_oracle, "units": len(units)}


def _first_bad(eq: np.ndarray, units, what: str) -> None:
    """Raise naming the first unit whose entries of eq (unit-major) are not all true."""
    if eq.shape[0] == 0:
        return
    ok = eq.reshape(eq.shape[0], -1).all(axis=1) if eq.ndim > 1 else eq
    if not ok.all():
        k = int(np.argmin(ok))
        raise AssertionError(f"{what} (unit {units[k]}; {int((~ok).sum())} units differ)")


def compare_evict_all(cfg: EvictConfig, inp: dict, out: dict, n_len: int, units=None, flags: int | None = None,
                      where: str = "", chunk: int = 512) -> dict:
    """compare_evict over every listed unit (default: all of the workload's), a chunk of units at a time so
    that the host copies stay bounded.  Returns the totals: tie-band differences, units, oracle seconds."""
    units = list(range(cfg.units)) if units is None else list(units)
    tot = {"n_tie_diff": 0, "units": 0, "oracle_s": 0.0}
    for c0 in range(0, len(units), chunk):
        r = compare_evict(cfg, inp, out, n_len, units=units[c0:c0 + chunk], flags=flags, where=where)
        for k in tot:
            tot[k] += r[k]
    return tot
