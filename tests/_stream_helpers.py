"""Helpers of the streaming-decode tests: oracle replay of recorded units and
comparison with the GPU stream."""
from __future__ import annotations

import numpy as np
import torch

import oracle as O
from long_reasoning_decode_amd import synth
from long_reasoning_decode_amd.configs import StreamConfig

from _helpers import check_keep, check_scores


def stream_ocfg(scfg: StreamConfig, units=None) -> O.OracleCfg:
    """Oracle configuration of a stream workload; units: the global indices of the units replayed, when
    they are a sample of the workload's (the random-history draws are keyed by the global buffer index)."""
    b = scfg.base
    return O.OracleCfg(hq=b.hq, hkv=b.hkv, d=b.d, cap=b.cap, budget=b.budget, n_prefix=b.n_prefix,
                       n_recent_kv=b.n_recent_kv, n_beacon=b.n_beacon, n_recent_q=b.n_recent_q, theta=b.theta,
                       qcap=b.qcap, pool_mean=int(b.pool == "mean"),
                       beacon_src={"fps": O.SRC_FPS, "initial": O.SRC_INITIAL, "random": O.SRC_RANDOM,
                                   "naive": O.SRC_NAIVE}[b.beacon],
                       seed=b.seed & 0xFFFFFFFF, n_layers=b.n_layers, batch=b.batch,
                       unit_ids=None if units is None else list(units))


def empty_state(scfg: StreamConfig, U: int, hcap: int = 0) -> dict:
    b = scfg.base
    G, d = b.G, b.d
    st = {"K": np.zeros((U, b.cap, d), np.uint16), "V": np.zeros((U, b.cap, d), np.uint16),
          "qbuf": np.zeros((U, G, b.qcap, d), np.uint16), "qcount": np.zeros((U, G), np.int32),
          "q_recent": np.zeros((U, G, b.n_recent_q, d), np.uint16),
          "pos_recent": np.zeros((U, b.n_recent_q), np.int32)}
    if b.beacon == "naive":   # the whole query history of every head
        st["hist"] = np.zeros((U, G, hcap, d), np.uint16)
        st["hcount"] = np.zeros((U, G), np.int32)
    return st


def replay(scfg: StreamConfig, k_new, v_new, q_new, pos, max_ev: int, nthreads=None, units=None) -> dict:
    """Oracle stream from an empty state over step-major inputs of U units (units: their global indices,
    when they are a sample of the workload's)."""
    st = empty_state(scfg, pos.shape[1], hcap=pos.shape[0])
    o = O.stream(stream_ocfg(scfg, units), k_new, v_new, q_new, pos, st["K"], st["V"], 0, st["qbuf"], st["qcount"],
                 st["q_recent"], st["pos_recent"], max_ev=max_ev, nthreads=nthreads, hist=st.get("hist"),
                 hcount=st.get("hcount"))
    o.update(st)
    return o


def compare_stream(scfg: StreamConfig, o: dict, g_idx, g_scores, g_state: dict, where: str = "") -> dict:
    """Per unit: every eviction's kept set and scores, then the final state.

    Keep sets must equal the oracle's or differ only within the tie band; after
    such a (correct) difference the unit's cache legitimately differs from the
    oracle's, so later evictions and its final K/V are not compared.  The
    query-buffer state does not depend on the cache and is always compared."""
    b = scfg.base
    E, U = o["idx"].shape[:2]
    assert g_idx.shape[:2] == (E, U), (g_idx.shape, E, U)
    diverged = {}
    for k in range(U):
        for e in range(E):
            w = f"{where} unit {k} eviction {e}"
            check_scores(g_scores[e, k], o["scores"][e, k], w)
            if np.array_equal(g_idx[e, k], o["idx"][e, k]):
                continue
            check_keep(g_idx[e, k], o["idx"][e, k], o["scores"][e, k], b.cap, b.budget, b.n_prefix,
                       b.n_recent_kv, w)
            diverged[k] = e
            break
    L = o["L"]
    for k in range(U):
        w = f"{where} unit {k}"
        if k not in diverged:
            assert np.array_equal(g_state["K"][k, :L], o["K"][k, :L]), f"{w}: K rows"
            assert np.array_equal(g_state["V"][k, :L], o["V"][k, :L]), f"{w}: V rows"
        assert np.array_equal(g_state["qcount"][k], o["qcount"][k]), f"{w}: qcount"
        for h in range(b.G):
            n = int(o["qcount"][k, h])
            assert np.array_equal(g_state["qbuf"][k, h, :n], o["qbuf"][k, h, :n]), f"{w} head {h}: buffer"
        assert np.array_equal(g_state["q_recent"][k], o["q_recent"][k]), f"{w}: recent ring"
        assert np.array_equal(g_state["pos_recent"][k], o["pos_recent"][k]), f"{w}: ring positions"
    return {"diverged": diverged}


def gpu_state(run, units) -> dict:
    """Host copies of the listed units' cache, buffers and ring (unit-major)."""
    b = run.base
    U, G, d = b.units, b.G, b.d
    ut = torch.tensor(list(units), dtype=torch.long, device="cuda")
    bt = (ut // b.hkv) % b.batch
    return {"K": synth.to_u16(run.K.reshape(U, b.cap, d).index_select(0, ut)),
            "V": synth.to_u16(run.V.reshape(U, b.cap, d).index_select(0, ut)),
            "qbuf": synth.to_u16(run.qbuf.reshape(U, G, b.qcap, d).index_select(0, ut)),
            "qcount": run.qcount.reshape(U, G).index_select(0, ut).cpu().numpy(),
            "q_recent": synth.to_u16(run.q_recent.reshape(U, G, b.n_recent_q, d).index_select(0, ut)),
            "pos_recent": run.pos_recent.index_select(0, bt).cpu().numpy()}


def check_run(scfg, run, units, where, nthreads=None):
    """The recorded units of a GPU stream (a StreamRun) against the oracle's replay of the same inputs."""
    h = run.history()
    u16 = lambda t: t.contiguous().view(torch.int16).numpy().view(np.uint16)
    o = replay(scfg, u16(h["k_new"]), u16(h["v_new"]), u16(h["q_new"]), h["pos"].numpy().astype(np.int32),
               max_ev=run.n_ev, nthreads=nthreads, units=units)
    assert o["n_ev"] == run.n_ev and o["L"] == run.L
    res = compare_stream(scfg, o, h["idx"].numpy(), h["scores"].numpy(), gpu_state(run, units), where)
    print(f"{where}: {run.n_ev} evictions, L={run.L}, tie-band divergences {res['diverged']}", flush=True)
    return res
