"""CPU oracle for the BeaconKV eviction step -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this package.  It wraps ``liboracle.so`` (plain C, see
``bkv_oracle.c``) with ctypes and takes/returns numpy arrays; bf16 data is
passed as ``uint16`` bit patterns.  It shares no code with the HIP library.

Array layouts (unit-major; a unit is one (layer, batch, KV head), its G query
heads follow it):
    K, V        [U, cap, d]            uint16 (bf16), K holds post-RoPE keys
    qbuf        [U, G, qcap, d]        uint16, pre-RoPE query buffers
    qcount      [U, G]                 int32
    q_recent    [U, G, n_recent_q, d]  uint16, pre-RoPE recent queries
    pos_recent  [U, n_recent_q]        int32
    t           [U]                    int32
"""
from __future__ import annotations

import ctypes as C
import os
from dataclasses import dataclass

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "liboracle.so")
_lib = None

SRC_FPS, SRC_INITIAL, SRC_RANDOM, SRC_NAIVE = 0, 1, 2, 3


class _Cfg(C.Structure):
    _fields_ = [(n, C.c_int) for n in (
        "n_layers", "batch", "hq", "hkv", "d", "cap", "budget", "n_prefix",
        "n_recent_kv", "n_beacon", "n_recent_q", "causal", "qcap", "pool_mean", "beacon_src")] + [
        ("seed", C.c_uint), ("theta", C.c_double), ("unit_ids", C.c_void_p)]


@dataclass
class OracleCfg:
    hq: int
    hkv: int
    d: int
    cap: int
    budget: int
    n_prefix: int
    n_recent_kv: int
    n_beacon: int
    n_recent_q: int
    theta: float
    qcap: int = 32
    causal: int = 1
    pool_mean: int = 0
    beacon_src: int = 0   # SRC_FPS, SRC_INITIAL, SRC_RANDOM or SRC_NAIVE
    seed: int = 0
    n_layers: int = 1
    batch: int = 1
    unit_ids: object = None   # global unit index of each unit passed (a sample of the workload's units)

    def check_units(self, U: int) -> None:
        assert self.unit_ids is None or len(self.unit_ids) == U, "one global unit index per unit passed"

    def c(self) -> _Cfg:
        ids = None
        if self.unit_ids is not None:
            self._ids = np.ascontiguousarray(self.unit_ids, dtype=np.int64)   # kept alive with the config
            ids = self._ids.ctypes.data
        return _Cfg(self.n_layers, self.batch, self.hq, self.hkv, self.d, self.cap,
                    self.budget, self.n_prefix, self.n_recent_kv, self.n_beacon,
                    self.n_recent_q, self.causal, self.qcap, self.pool_mean, self.beacon_src,
                    self.seed & 0xFFFFFFFF, float(self.theta), ids)

    @property
    def G(self) -> int:
        return self.hq // self.hkv


def lib():
    """Load liboracle.so, building it with gcc if it is not there yet."""
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            from . import build as _b
            _b.build()
        L = C.CDLL(_LIB_PATH)
        P = C.c_void_p
        i32 = C.c_int
        L.bkvo_f32_to_bf16.argtypes = [C.c_float]
        L.bkvo_f32_to_bf16.restype = C.c_uint16
        L.bkvo_rope_table.argtypes = [C.c_double, i32, i32, i32, P]
        L.bkvo_rope_row.argtypes = [P, i32, C.c_double, i32, P]
        L.bkvo_fps.argtypes = [P, i32, i32, i32, P]
        L.bkvo_fps.restype = i32
        L.bkvo_fps_f64.argtypes = [P, i32, i32, i32, P, P]
        L.bkvo_fps_f64.restype = i32
        L.bkvo_fps_update.argtypes = [i32, i32, i32, i32, i32, P, P, P, P]
        L.bkvo_fps_plain.argtypes = [P, i32, i32, i32, P, P, P, P]
        L.bkvo_fps_plain.restype = i32
        L.bkvo_fps_long.argtypes = [P, i32, i32, i32, P]
        L.bkvo_fps_long.restype = i32
        L.bkvo_pairwise_sum.argtypes = [P, i32]
        L.bkvo_pairwise_sum.restype = C.c_float
        L.bkvo_prefill.argtypes = [i32, i32, i32, i32, i32, i32, C.c_uint, C.c_longlong, P, P, P, P]
        L.bkvo_philox4x32_10.argtypes = [P, P, P]
        L.bkvo_reservoir_slot.argtypes = [C.c_uint, C.c_longlong, i32, i32]
        L.bkvo_reservoir_slot.restype = i32
        L.bkvo_beacon_update.argtypes = [P, i32, C.c_longlong, P, P, P, P]
        L.bkvo_decode_attention.argtypes = [P, i32, i32, P, P, P, P, P, P]
        L.bkvo_row_weights.argtypes = [P, P, i32, i32, i32, P]
        L.bkvo_row_weights.restype = C.c_double
        L.bkvo_select.argtypes = [P, i32, i32, i32, i32, P]
        L.bkvo_select.restype = i32
        L.bkvo_score.argtypes = [P, i32, i32, P, P, P, P, P, P, P, i32]
        L.bkvo_evict.argtypes = [P, i32, i32, P, P, P, P, P, P, P, P, P, P, P, i32]
        L.bkvo_merge.argtypes = [P, i32, P, P, P, P]
        L.bkvo_compact.argtypes = [P, i32, i32, P, P, P]
        L.bkvo_stream.argtypes = [P, i32, i32, P, P, P, P, P, P, P, P, P, P, P, P, P, i32, P, P, i32, i32]
        L.bkvo_fps_compress.argtypes = [i32, i32, i32, i32, i32, P, P, P]
        L.bkvo_stream.restype = i32
        L.bkvo_cfg_size.restype = i32
        assert L.bkvo_cfg_size() == C.sizeof(_Cfg), "oracle cfg struct mismatch"
        _lib = L
    return _lib


def _p(a: np.ndarray | None):
    if a is None:
        return None
    assert a.flags["C_CONTIGUOUS"], "oracle arrays must be C-contiguous"
    return a.ctypes.data_as(C.c_void_p)


def _u16(a) -> np.ndarray:
    a = np.ascontiguousarray(a)
    assert a.dtype == np.uint16, a.dtype
    return a


def _i32(a) -> np.ndarray:
    return np.ascontiguousarray(a, dtype=np.int32)


def default_threads() -> int:
    try:
        return len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        return os.cpu_count() or 1


# --------------------------------------------------------------------------
def f32_to_bf16(x) -> np.ndarray:
    """Round fp32 values to bf16 codes (nearest, ties to even)."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    f = lib().bkvo_f32_to_bf16
    out = np.fromiter((f(float(v)) for v in x.ravel()), dtype=np.uint16, count=x.size)
    return out.reshape(x.shape)


def bf16_to_f32(x) -> np.ndarray:
    x = _u16(x)
    return (x.astype(np.uint32) << 16).view(np.float32)


def rope_table(theta: float, d: int, p0: int, p1: int) -> np.ndarray:
    out = np.empty((p1 - p0, d // 2, 2), dtype=np.float32)
    lib().bkvo_rope_table(float(theta), d, p0, p1, _p(out))
    return out


def rope_row(x, theta: float, p: int) -> np.ndarray:
    x = _u16(x)
    y = np.empty_like(x)
    lib().bkvo_rope_row(_p(x), x.shape[-1], float(theta), int(p), _p(y))
    return y


def fps(X, m: int) -> list[int]:
    X = _u16(X)
    n, d = X.shape
    sel = np.empty(max(n, 1), dtype=np.int32)
    got = lib().bkvo_fps(_p(X), n, d, m, _p(sel))
    return sel[:got].tolist()


def fps_f64(X, m: int):
    X = _u16(X)
    n, d = X.shape
    sel = np.empty(max(n, 1), dtype=np.int32)
    mar = np.empty(max(n, 1), dtype=np.float64)
    got = lib().bkvo_fps_f64(_p(X), n, d, m, _p(sel), _p(mar))
    return sel[:got].tolist(), mar[:got].copy()


def fps_long(X, m: int) -> list[int]:
    """FPS of many rows with the O(n d) seed (the prefill variant)."""
    X = _u16(X)
    n, d = X.shape
    sel = np.empty(max(n, 1), dtype=np.int32)
    got = lib().bkvo_fps_long(_p(X), n, d, m, _p(sel))
    return sel[:got].tolist()


def fps_plain(X, m: int, forced=None):
    """FPS by the page's definition in fp64 (O(n^2 d) seed), optionally replaying the picks `forced`.
    Returns (sel, regret, margin): the rows taken, and per step the fp64 value of the row taken minus the
    best value (0 when optimal, inf for an invalid forced pick) and the gap between the two best values."""
    X = _u16(X)
    n, d = X.shape
    k = max(1, min(n, m))
    sel = np.empty(k, dtype=np.int32)
    reg = np.empty(k, dtype=np.float64)
    mar = np.empty(k, dtype=np.float64)
    f = None
    if forced is not None:
        f = np.full(k, -1, dtype=np.int32)
        fr = np.asarray(forced, dtype=np.int32)[:k]
        f[:len(fr)] = fr
    got = lib().bkvo_fps_plain(_p(X), n, d, m, _p(f), _p(sel), _p(reg), _p(mar))
    return sel[:got].tolist(), reg[:got].copy(), mar[:got].copy()


def pairwise_sum(x) -> float:
    x = np.ascontiguousarray(x, dtype=np.float32)
    return float(np.float32(lib().bkvo_pairwise_sum(_p(x), x.size)))


def philox4x32_10(ctr, key) -> list[int]:
    c = np.ascontiguousarray(ctr, dtype=np.uint32)
    k = np.ascontiguousarray(key, dtype=np.uint32)
    out = np.empty(4, dtype=np.uint32)
    lib().bkvo_philox4x32_10(_p(c), _p(k), _p(out))
    return [int(v) for v in out]


def reservoir_slot(seed: int, uq: int, n: int, n_beacon: int) -> int:
    return lib().bkvo_reservoir_slot(seed & 0xFFFFFFFF, uq, n, n_beacon)


def beacon_update(cfg: OracleCfg, qbuf, qcount, q_new, buf0: int = 0) -> np.ndarray:
    """The per-step buffer update under cfg.beacon_src, in place on qbuf [nbuf, qcap, d], qcount [nbuf]."""
    assert qbuf.dtype == np.uint16 and qbuf.flags["C_CONTIGUOUS"]
    assert qcount.dtype == np.int32 and qcount.flags["C_CONTIGUOUS"]
    nbuf = qbuf.shape[0]
    q_new = _u16(q_new).reshape(nbuf, cfg.d)
    sel = np.empty((nbuf, cfg.n_beacon), dtype=np.int32)
    cc = cfg.c()
    lib().bkvo_beacon_update(C.byref(cc), nbuf, buf0, _p(qbuf), _p(qcount), _p(q_new), _p(sel))
    return sel


def prefill(q_prompt, qbuf, qcount, n_beacon: int, src: int = SRC_FPS, seed: int = 0, buf0: int = 0) -> np.ndarray:
    """Prefill initialisation, in place on qbuf [nbuf, qcap, d] and qcount [nbuf] from q_prompt [nbuf, P, d];
    returns the selection order (FPS) or the prompt row of each slot [nbuf, n_beacon] (-1 past the last)."""
    assert qbuf.dtype == np.uint16 and qbuf.flags["C_CONTIGUOUS"]
    assert qcount.dtype == np.int32 and qcount.flags["C_CONTIGUOUS"]
    q_prompt = _u16(q_prompt)
    nbuf, P, d = q_prompt.shape
    assert qbuf.shape[0] == nbuf and qbuf.shape[2] == d and qcount.shape == (nbuf,)
    sel = np.empty((nbuf, n_beacon), dtype=np.int32)
    lib().bkvo_prefill(nbuf, P, d, n_beacon, qbuf.shape[1], src, seed & 0xFFFFFFFF, buf0, _p(q_prompt), _p(qbuf),
                       _p(qcount), _p(sel))
    return sel


def fps_update(qbuf, qcount, q_new, n_beacon: int, n_recent_q: int) -> np.ndarray:
    """In place on qbuf [nbuf, qcap, d] and qcount [nbuf]; returns sel [nbuf, n_beacon]."""
    assert qbuf.dtype == np.uint16 and qbuf.flags["C_CONTIGUOUS"]
    assert qcount.dtype == np.int32 and qcount.flags["C_CONTIGUOUS"]
    nbuf, qcap, d = qbuf.shape
    q_new = _u16(q_new).reshape(nbuf, d)
    sel = np.empty((nbuf, n_beacon), dtype=np.int32)
    lib().bkvo_fps_update(nbuf, qcap, d, n_beacon, n_recent_q, _p(qbuf), _p(qcount), _p(q_new), _p(sel))
    return sel


def fps_compress(qbuf, qcount, n_beacon: int, n_recent_q: int) -> np.ndarray:
    """Freeze-point compression, in place on qbuf [nbuf, qcap, d] and qcount [nbuf]; returns sel [nbuf, n_beacon]."""
    assert qbuf.dtype == np.uint16 and qbuf.flags["C_CONTIGUOUS"]
    assert qcount.dtype == np.int32 and qcount.flags["C_CONTIGUOUS"]
    nbuf, qcap, d = qbuf.shape
    sel = np.empty((nbuf, max(n_beacon, 1)), dtype=np.int32)
    lib().bkvo_fps_compress(nbuf, qcap, d, n_beacon, n_recent_q, _p(qbuf), _p(qcount), _p(sel))
    return sel[:, :n_beacon]


def row_weights(q, K, vis: int | None = None):
    """Softmax weights of one (already rotated) query row over K [N, d]."""
    q = _u16(q)
    K = _u16(K)
    N, d = K.shape
    w = np.empty(N, dtype=np.float64)
    c = lib().bkvo_row_weights(_p(q), _p(K), N, d, N - 1 if vis is None else vis, _p(w))
    return w, c


def select(score, budget: int, n_prefix: int, n_recent_kv: int):
    s = np.ascontiguousarray(score, dtype=np.float64)
    idx = np.empty(budget, dtype=np.int32)
    moved = lib().bkvo_select(_p(s), s.shape[0], budget, n_prefix, n_recent_kv, _p(idx))
    return idx, moved


def score(cfg: OracleCfg, K, qbuf, qcount, q_recent, pos_recent, t, n_len: int | None = None,
          nthreads: int | None = None) -> np.ndarray:
    K = _u16(K)
    U = K.shape[0]
    N = cfg.cap if n_len is None else n_len
    out = np.empty((U, N), dtype=np.float64)
    cc = cfg.c()
    lib().bkvo_score(C.byref(cc), U, N, _p(K), _p(_u16(qbuf)), _p(_i32(qcount)), _p(_u16(q_recent)),
                     _p(_i32(pos_recent)), _p(_i32(t)), _p(out), nthreads or default_threads())
    return out


def evict(cfg: OracleCfg, K, V, qbuf, qcount, q_recent, pos_recent, t, n_len: int | None = None,
          nthreads: int | None = None) -> dict:
    """Full eviction, in place on K, V, qbuf, qcount (numpy arrays, C-contiguous)."""
    for a, dt in ((K, np.uint16), (V, np.uint16), (qbuf, np.uint16), (qcount, np.int32)):
        assert a.dtype == dt and a.flags["C_CONTIGUOUS"]
    U = K.shape[0]
    cfg.check_units(U)
    N = cfg.cap if n_len is None else n_len
    idx = np.empty((U, cfg.budget), dtype=np.int32)
    scores = np.empty((U, N), dtype=np.float64)
    moved = np.empty(U, dtype=np.int32)
    fps_sel = np.empty((U, cfg.G, cfg.n_beacon), dtype=np.int32)
    cc = cfg.c()
    lib().bkvo_evict(C.byref(cc), U, N, _p(K), _p(V), _p(qbuf), _p(qcount), _p(_u16(q_recent)),
                     _p(_i32(pos_recent)), _p(_i32(t)), _p(idx), _p(scores), _p(moved), _p(fps_sel),
                     nthreads or default_threads())
    return {"idx": idx, "scores": scores, "moved": moved, "fps_sel": fps_sel}


def merge(cfg: OracleCfg, qbuf, qcount, q_recent) -> np.ndarray:
    assert qbuf.dtype == np.uint16 and qbuf.flags["C_CONTIGUOUS"]
    assert qcount.dtype == np.int32 and qcount.flags["C_CONTIGUOUS"]
    U = qbuf.shape[0]
    cfg.check_units(U)
    fps_sel = np.empty((U, cfg.G, cfg.n_beacon), dtype=np.int32)
    cc = cfg.c()
    lib().bkvo_merge(C.byref(cc), U, _p(qbuf), _p(qcount), _p(_u16(q_recent)), _p(fps_sel))
    return fps_sel


def compact(cfg: OracleCfg, K, V, idx, n_len: int | None = None) -> None:
    U = K.shape[0]
    N = cfg.cap if n_len is None else n_len
    cc = cfg.c()
    lib().bkvo_compact(C.byref(cc), U, N, _p(K), _p(V), _p(_i32(idx)))


def decode_attention(cfg: OracleCfg, K, V, q, pos, n_len: int):
    """One decode step's attention: K, V [U, cap, d] (uint16 bf16, K post-RoPE), q [U, G, d] pre-RoPE, pos [U]
    (the position q is rotated to).  Returns (out, scale) [U, G, d] fp64."""
    K, V, q = _u16(K), _u16(V), _u16(q)
    U = K.shape[0]
    out = np.empty((U, cfg.G, cfg.d), dtype=np.float64)
    scale = np.empty_like(out)
    cc = cfg.c()
    lib().bkvo_decode_attention(C.byref(cc), U, n_len, _p(K), _p(V), _p(q), _p(_i32(pos)), _p(out), _p(scale))
    return out, scale


def stream(cfg: OracleCfg, k_new, v_new, q_new, pos, K, V, L: int, qbuf, qcount, q_recent, pos_recent,
           max_ev: int = 0, nthreads: int | None = None, hist=None, hcount=None) -> dict:
    """Decode steps of the eviction cycle for U units in lockstep, in place on the state (K, V, qbuf,
    qcount, q_recent, pos_recent: unit-major numpy arrays; under SRC_NAIVE also the query history
    hist [U, G, hcap, d] and its counts hcount [U, G]).  Step inputs are step-major:
    k_new, v_new [S, U, d] (k_new pre-RoPE), q_new [S, U, G, d], pos [S, U].
    Returns the final cache length, the number of evictions and the first max_ev evictions'
    keep sets [max_ev, U, budget] and scores [max_ev, U, cap]."""
    for a, dt in ((K, np.uint16), (V, np.uint16), (qbuf, np.uint16), (qcount, np.int32),
                  (q_recent, np.uint16), (pos_recent, np.int32)):
        assert a.dtype == dt and a.flags["C_CONTIGUOUS"]
    k_new, v_new, q_new, pos = _u16(k_new), _u16(v_new), _u16(q_new), _i32(pos)
    S, U = pos.shape
    cfg.check_units(U)
    assert k_new.shape == (S, U, cfg.d) and v_new.shape == (S, U, cfg.d)
    assert q_new.shape == (S, U, cfg.G, cfg.d)
    hcap = 0
    if cfg.beacon_src == SRC_NAIVE:
        assert hist is not None and hcount is not None
        assert hist.dtype == np.uint16 and hist.flags["C_CONTIGUOUS"] and hist.shape[:2] == (U, cfg.G)
        assert hcount.dtype == np.int32 and hcount.flags["C_CONTIGUOUS"] and hcount.shape == (U, cfg.G)
        hcap = hist.shape[2]
    idx = np.full((max_ev, U, cfg.budget), -1, dtype=np.int32) if max_ev > 0 else None
    sc = np.zeros((max_ev, U, cfg.cap), dtype=np.float64) if max_ev > 0 else None
    Lb = C.c_int32(int(L))
    cc = cfg.c()
    n_ev = lib().bkvo_stream(C.byref(cc), U, S, _p(k_new), _p(v_new), _p(q_new), _p(pos), _p(K), _p(V),
                             C.byref(Lb), _p(qbuf), _p(qcount), _p(q_recent), _p(pos_recent), _p(idx), _p(sc),
                             max_ev, _p(hist) if hcap else None, _p(hcount) if hcap else None, hcap,
                             nthreads or default_threads())
    return {"L": Lb.value, "n_ev": n_ev, "idx": idx, "scores": sc}
