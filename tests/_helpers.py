"""Shared helpers of the GPU parity tests: run the HIP path, run the oracle on
the same seeded inputs, and compare element by element."""
from __future__ import annotations

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
    forced = set(range(min(n_prefix, n_len))) | set(range(max(0, n_len - n_recent_kv), n_len))
    gs, os_ = set(g.tolist()), set(o.tolist())
    assert forced <= gs, f"{where}: forced keeps missing"
    chosen = [j for j in os_ if j not in forced]
    if not chosen:
        assert gs == os_, where
        return 0
    sk = min(s_orc[j] for j in chosen)
    diff = gs ^ os_
    for j in diff:
        dj = abs(s_orc[j] - sk)
        assert dj <= TIE_BAND_ABS and dj <= TIE_BAND_REL * sk + SCORE_ATOL, \
            f"{where}: key {j} kept differently with score {s_orc[j]!r} vs k-th {sk!r}"
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
    o = O.evict(oc, v["K"], v["V"], v["qbuf"], v["qcount"], v["q_recent"], v["pos_recent"], v["t"],
                n_len=n_len)
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
        w = f"{where} unit {u}"
        n_diff += check_keep(g_idx[k], o["idx"][k], o["scores"][k], n_len, cfg.budget, cfg.n_prefix,
                             cfg.n_recent_kv, w)
        gi = g_idx[k][:B]
        assert np.array_equal(g_K[k, :B], K0[k][gi]), f"{w}: K rows differ from the gather"
        assert np.array_equal(g_V[k, :B], V0[k][gi]), f"{w}: V rows differ from the gather"
        if np.array_equal(gi, o["idx"][k][:B]):
            assert np.array_equal(g_K[k, :B], v["K"][k, :B]) and np.array_equal(g_V[k, :B], v["V"][k, :B])
        assert np.array_equal(g_qc[k], v["qcount"][k]), f"{w}: qcount"
        assert np.array_equal(g_sel[k], o["fps_sel"][k]), f"{w}: merge FPS selection"
        for h in range(G):
            n = int(v["qcount"][k, h])
            assert np.array_equal(g_qbuf[k, h, :n], v["qbuf"][k, h, :n]), f"{w} head {h}: merged buffer"
    return {"n_tie_diff": n_diff, "oracle": o}
