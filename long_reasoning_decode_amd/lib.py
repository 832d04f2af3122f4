"""Thin Python binding of libbkv.so (include/bkv.h): argument marshalling only.

Every function takes torch tensors that already live on the GPU, checks dtype,
device and contiguity, and passes raw pointers and the current HIP stream to
the C entry point of the same name.  All computation happens in the library's
HIP kernels; there is no fallback.  If the library has not been built, the
first call raises ``ImportError``.
"""
from __future__ import annotations

import ctypes as C
import os
from typing import Optional

import numpy as np
import torch

from .configs import EvictConfig

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libbkv.so")

BKV_CAUSAL_RECENT = 1
BKV_POOL_MEAN = 2
BKV_BEACON_INITIAL = 4
BKV_BEACON_RANDOM = 8
BKV_BEACON_NAIVE = 16
ERRORS = {0: "BKV_OK", -1: "BKV_EINVAL", -2: "BKV_EUNSUPPORTED", -3: "BKV_ERANGE", -4: "BKV_EHIP"}

EXPORTS = ("bkv_version", "bkv_strerror", "bkv_rope_table", "bkv_workspace_bytes", "bkv_fps_update",
           "bkv_fps_merge", "bkv_fps_prefill", "bkv_score", "bkv_select", "bkv_compact", "bkv_evict",
           "bkv_decode_step", "bkv_append_kv", "bkv_decode_attention", "bkv_fps_compress", "bkv_history_append",
           "bkv_fps_history")


class Shape(C.Structure):
    _fields_ = [(n, C.c_int32) for n in (
        "n_layers", "batch", "n_q_heads", "n_kv_heads", "head_dim", "cap", "budget", "n_prefix",
        "n_recent_kv", "n_beacon", "n_recent_q", "qcap")] + [("flags", C.c_uint32), ("seed", C.c_uint32)]


class BkvError(RuntimeError):
    def __init__(self, code: int, where: str):
        self.code = code
        super().__init__(f"{where}: {ERRORS.get(code, code)} ({strerror(code)})")


_lib = None


def load():
    """Load libbkv.so (built in-tree by build.py)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is missing: build it with "
                              "`python -m long_reasoning_decode_amd.build`")
        L = C.CDLL(LIB_PATH)
        P, i32, st = C.c_void_p, C.c_int32, C.c_void_p
        SP = C.POINTER(Shape)
        L.bkv_version.restype = C.c_int
        L.bkv_strerror.argtypes = [C.c_int]
        L.bkv_strerror.restype = C.c_char_p
        L.bkv_rope_table.argtypes = [C.c_double, i32, i32, i32, P]
        L.bkv_fps_update.argtypes = [SP, P, P, P, P, st]
        L.bkv_fps_merge.argtypes = [SP, P, P, P, P, st]
        L.bkv_fps_prefill.argtypes = [SP, P, i32, P, P, P, st]
        L.bkv_score.argtypes = [SP, P, i32, P, P, P, P, P, P, i32, P, st]
        L.bkv_select.argtypes = [SP, P, i32, P, st]
        L.bkv_compact.argtypes = [SP, P, P, i32, P, st]
        L.bkv_evict.argtypes = [SP, P, P, i32, P, P, P, P, P, P, i32, P, P, P, st]
        L.bkv_decode_step.argtypes = [SP, P, P, i32, P, P, P, P, P, P, P, P, P, i32, P, st]
        L.bkv_append_kv.argtypes = [SP, P, P, i32, P, P, P, P, i32, st]
        L.bkv_decode_attention.argtypes = [SP, P, P, i32, P, P, P, i32, P, st]
        L.bkv_fps_compress.argtypes = [SP, P, P, P, st]
        L.bkv_history_append.argtypes = [SP, P, i32, P, P, st]
        L.bkv_fps_history.argtypes = [SP, P, i32, i32, P, P, P, st]
        for f in EXPORTS[4:]:
            getattr(L, f).restype = C.c_int
        L.bkv_workspace_bytes.argtypes = [SP, i32]
        L.bkv_workspace_bytes.restype = C.c_size_t
        _lib = L
    return _lib


def strerror(code: int) -> str:
    return load().bkv_strerror(int(code)).decode()


def version() -> int:
    return load().bkv_version()


def flags_of(cfg: EvictConfig) -> int:
    """Default flags of a workload: causal recent rows, and the pooling and beacon source it names."""
    src = {"fps": 0, "initial": BKV_BEACON_INITIAL, "random": BKV_BEACON_RANDOM, "naive": BKV_BEACON_NAIVE}[cfg.beacon]
    return BKV_CAUSAL_RECENT | (BKV_POOL_MEAN if cfg.pool == "mean" else 0) | src


def shape_of(cfg: EvictConfig, cap: Optional[int] = None, flags: Optional[int] = None) -> Shape:
    flags = flags_of(cfg) if flags is None else flags
    return Shape(cfg.n_layers, cfg.batch, cfg.hq, cfg.hkv, cfg.d, cfg.cap if cap is None else cap,
                 cfg.budget, cfg.n_prefix, cfg.n_recent_kv, cfg.n_beacon, cfg.n_recent_q, cfg.qcap, flags,
                 cfg.seed & 0xFFFFFFFF)


def _ptr(t: Optional[torch.Tensor], dtype, name: str):
    if t is None:
        return None
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name}: expected a torch.Tensor")
    if t.dtype != dtype:
        raise TypeError(f"{name}: dtype {t.dtype}, expected {dtype}")
    if not t.is_cuda:
        raise ValueError(f"{name}: must be a GPU tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name}: must be contiguous")
    return C.c_void_p(t.data_ptr())


def _stream(stream) -> C.c_void_p:
    if stream is None:
        stream = torch.cuda.current_stream()
    return C.c_void_p(stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream))


def _check(code: int, where: str) -> None:
    if code != 0:
        raise BkvError(code, where)


bf16, i32, f32 = torch.bfloat16, torch.int32, torch.float32

BKV_PREFILL_MAX = 8192


def _need(shape: Shape, **req) -> None:
    """Reject tensors smaller than the layout of include/bkv.h needs for this shape, before anything
    reaches the device.  Each keyword maps a name to (tensor or None, element count)."""
    for name, (t, n) in req.items():
        if t is not None and isinstance(t, torch.Tensor) and t.numel() < max(int(n), 0):
            raise ValueError(f"{name}: {t.numel()} elements, the shape needs {int(n)}")


def _counts(shape: Shape):
    units = shape.n_layers * shape.batch * shape.n_kv_heads
    qbufs = shape.n_layers * shape.batch * shape.n_q_heads
    return units, qbufs, shape.head_dim


def rope_table(theta: float, head_dim: int, p0: int, p1: int) -> np.ndarray:
    """Host-built {cos, sin} table [p1 - p0, head_dim/2, 2] (float32)."""
    out = np.empty((p1 - p0, head_dim // 2, 2), dtype=np.float32)
    _check(load().bkv_rope_table(float(theta), head_dim, p0, p1, out.ctypes.data_as(C.c_void_p)),
           "bkv_rope_table")
    return out


def fps_update(shape: Shape, qbuf, qcount, q_new, fps_sel=None, stream=None) -> None:
    U, Qb, d = _counts(shape)
    _need(shape, qbuf=(qbuf, Qb * shape.qcap * d), qcount=(qcount, Qb), q_new=(q_new, Qb * d),
          fps_sel=(fps_sel, Qb * shape.n_beacon))
    _check(load().bkv_fps_update(C.byref(shape), _ptr(qbuf, bf16, "qbuf"), _ptr(qcount, i32, "qcount"),
                                 _ptr(q_new, bf16, "q_new"), _ptr(fps_sel, i32, "fps_sel"), _stream(stream)),
           "bkv_fps_update")


def fps_merge(shape: Shape, qbuf, qcount, q_recent, fps_sel=None, stream=None) -> None:
    U, Qb, d = _counts(shape)
    _need(shape, qbuf=(qbuf, Qb * shape.qcap * d), qcount=(qcount, Qb),
          q_recent=(q_recent, Qb * shape.n_recent_q * d), fps_sel=(fps_sel, Qb * shape.n_beacon))
    _check(load().bkv_fps_merge(C.byref(shape), _ptr(qbuf, bf16, "qbuf"), _ptr(qcount, i32, "qcount"),
                                _ptr(q_recent, bf16, "q_recent"), _ptr(fps_sel, i32, "fps_sel"), _stream(stream)),
           "bkv_fps_merge")


def fps_prefill(shape: Shape, q_prompt, n_prompt: int, qbuf, qcount, fps_sel=None, stream=None) -> None:
    U, Qb, d = _counts(shape)
    _need(shape, q_prompt=(q_prompt, Qb * n_prompt * d), qbuf=(qbuf, Qb * shape.qcap * d), qcount=(qcount, Qb),
          fps_sel=(fps_sel, Qb * shape.n_beacon))
    _check(load().bkv_fps_prefill(C.byref(shape), _ptr(q_prompt, bf16, "q_prompt"), int(n_prompt),
                                  _ptr(qbuf, bf16, "qbuf"), _ptr(qcount, i32, "qcount"), _ptr(fps_sel, i32, "fps_sel"),
                                  _stream(stream)), "bkv_fps_prefill")


def workspace_bytes(shape: Shape, n_len: int) -> int:
    return int(load().bkv_workspace_bytes(C.byref(shape), int(n_len)))


def fps_compress(shape: Shape, qbuf, qcount, fps_sel=None, stream=None) -> None:
    U, Qb, d = _counts(shape)
    _need(shape, qbuf=(qbuf, Qb * shape.qcap * d), qcount=(qcount, Qb), fps_sel=(fps_sel, Qb * shape.n_beacon))
    _check(load().bkv_fps_compress(C.byref(shape), _ptr(qbuf, bf16, "qbuf"), _ptr(qcount, i32, "qcount"),
                                   _ptr(fps_sel, i32, "fps_sel"), _stream(stream)), "bkv_fps_compress")


def history_append(shape: Shape, hist, hcap: int, hcount, q_new, stream=None) -> None:
    U, Qb, d = _counts(shape)
    _need(shape, hist=(hist, Qb * hcap * d), hcount=(hcount, Qb), q_new=(q_new, Qb * d))
    _check(load().bkv_history_append(C.byref(shape), _ptr(hist, bf16, "hist"), int(hcap), _ptr(hcount, i32, "hcount"),
                                     _ptr(q_new, bf16, "q_new"), _stream(stream)), "bkv_history_append")


def fps_history(shape: Shape, hist, hcap: int, n_rows: int, qbuf, qcount, fps_sel=None, stream=None) -> None:
    U, Qb, d = _counts(shape)
    _need(shape, hist=(hist, Qb * hcap * d), qbuf=(qbuf, Qb * shape.qcap * d), qcount=(qcount, Qb),
          fps_sel=(fps_sel, Qb * shape.n_beacon))
    _check(load().bkv_fps_history(C.byref(shape), _ptr(hist, bf16, "hist"), int(hcap), int(n_rows),
                                  _ptr(qbuf, bf16, "qbuf"), _ptr(qcount, i32, "qcount"), _ptr(fps_sel, i32, "fps_sel"),
                                  _stream(stream)), "bkv_fps_history")


def score(shape: Shape, K, n_len: int, qbuf, qcount, q_recent, pos_recent, t, rope_cs, scores,
          stream=None) -> None:
    U, Qb, d = _counts(shape)
    _need(shape, K=(K, U * shape.cap * d), qbuf=(qbuf, Qb * shape.qcap * d), qcount=(qcount, Qb),
          q_recent=(q_recent, Qb * shape.n_recent_q * d), pos_recent=(pos_recent, shape.batch * shape.n_recent_q),
          t=(t, shape.batch), rope_cs=(rope_cs, rope_cs.shape[0] * d), scores=(scores, U * n_len))
    _check(load().bkv_score(C.byref(shape), _ptr(K, bf16, "K"), int(n_len), _ptr(qbuf, bf16, "qbuf"),
                            _ptr(qcount, i32, "qcount"), _ptr(q_recent, bf16, "q_recent"),
                            _ptr(pos_recent, i32, "pos_recent"), _ptr(t, i32, "t"),
                            _ptr(rope_cs, f32, "rope_cs"), int(rope_cs.shape[0]), _ptr(scores, f32, "scores"),
                            _stream(stream)), "bkv_score")


def select(shape: Shape, scores, n_len: int, idx, stream=None) -> None:
    U, Qb, d = _counts(shape)
    _need(shape, scores=(scores, U * n_len), idx=(idx, U * shape.budget))
    _check(load().bkv_select(C.byref(shape), _ptr(scores, f32, "scores"), int(n_len), _ptr(idx, i32, "idx"),
                             _stream(stream)), "bkv_select")


def compact(shape: Shape, K, V, n_len: int, idx, stream=None) -> None:
    U, Qb, d = _counts(shape)
    _need(shape, K=(K, U * shape.cap * d), V=(V, U * shape.cap * d), idx=(idx, U * shape.budget))
    _check(load().bkv_compact(C.byref(shape), _ptr(K, bf16, "K"), _ptr(V, bf16, "V"), int(n_len),
                              _ptr(idx, i32, "idx"), _stream(stream)), "bkv_compact")


def evict(shape: Shape, K, V, n_len: int, qbuf, qcount, q_recent, pos_recent, t, rope_cs,
          idx_out=None, scores_out=None, fps_sel_out=None, stream=None) -> None:
    U, Qb, d = _counts(shape)
    _need(shape, K=(K, U * shape.cap * d), V=(V, U * shape.cap * d), qbuf=(qbuf, Qb * shape.qcap * d),
          qcount=(qcount, Qb), q_recent=(q_recent, Qb * shape.n_recent_q * d),
          pos_recent=(pos_recent, shape.batch * shape.n_recent_q), t=(t, shape.batch),
          rope_cs=(rope_cs, rope_cs.shape[0] * d), idx_out=(idx_out, U * shape.budget),
          scores_out=(scores_out, U * n_len), fps_sel_out=(fps_sel_out, Qb * shape.n_beacon))
    _check(load().bkv_evict(C.byref(shape), _ptr(K, bf16, "K"), _ptr(V, bf16, "V"), int(n_len),
                            _ptr(qbuf, bf16, "qbuf"), _ptr(qcount, i32, "qcount"), _ptr(q_recent, bf16, "q_recent"),
                            _ptr(pos_recent, i32, "pos_recent"), _ptr(t, i32, "t"), _ptr(rope_cs, f32, "rope_cs"),
                            int(rope_cs.shape[0]), _ptr(idx_out, i32, "idx_out"), _ptr(scores_out, f32, "scores_out"),
                            _ptr(fps_sel_out, i32, "fps_sel_out"), _stream(stream)), "bkv_evict")


def decode_step(shape: Shape, K, V, L: int, k_new, v_new, pos, qbuf, qcount, q_new, q_recent, pos_recent,
                rope_cs, fps_sel=None, stream=None) -> None:
    U, Qb, d = _counts(shape)
    _need(shape, K=(K, U * shape.cap * d), V=(V, U * shape.cap * d), k_new=(k_new, U * d), v_new=(v_new, U * d),
          pos=(pos, shape.batch), qbuf=(qbuf, Qb * shape.qcap * d), qcount=(qcount, Qb), q_new=(q_new, Qb * d),
          q_recent=(q_recent, Qb * shape.n_recent_q * d), pos_recent=(pos_recent, shape.batch * shape.n_recent_q),
          rope_cs=(rope_cs, rope_cs.shape[0] * d), fps_sel=(fps_sel, Qb * shape.n_beacon))
    _check(load().bkv_decode_step(C.byref(shape), _ptr(K, bf16, "K"), _ptr(V, bf16, "V"), int(L),
                                  _ptr(k_new, bf16, "k_new"), _ptr(v_new, bf16, "v_new"), _ptr(pos, i32, "pos"),
                                  _ptr(qbuf, bf16, "qbuf"), _ptr(qcount, i32, "qcount"), _ptr(q_new, bf16, "q_new"),
                                  _ptr(q_recent, bf16, "q_recent"), _ptr(pos_recent, i32, "pos_recent"),
                                  _ptr(rope_cs, f32, "rope_cs"), int(rope_cs.shape[0]),
                                  _ptr(fps_sel, i32, "fps_sel"), _stream(stream)), "bkv_decode_step")


def append_kv(shape: Shape, K, V, L: int, k_new, v_new, pos, rope_cs, stream=None) -> None:
    U, Qb, d = _counts(shape)
    _need(shape, K=(K, U * shape.cap * d), V=(V, U * shape.cap * d), k_new=(k_new, U * d), v_new=(v_new, U * d),
          pos=(pos, shape.batch), rope_cs=(rope_cs, rope_cs.shape[0] * d))
    _check(load().bkv_append_kv(C.byref(shape), _ptr(K, bf16, "K"), _ptr(V, bf16, "V"), int(L),
                                _ptr(k_new, bf16, "k_new"), _ptr(v_new, bf16, "v_new"), _ptr(pos, i32, "pos"),
                                _ptr(rope_cs, f32, "rope_cs"), int(rope_cs.shape[0]), _stream(stream)), "bkv_append_kv")


def decode_attention(shape: Shape, K, V, n_len: int, q, pos, rope_cs, out, stream=None) -> None:
    U, Qb, d = _counts(shape)
    _need(shape, K=(K, U * shape.cap * d), V=(V, U * shape.cap * d), q=(q, Qb * d), pos=(pos, shape.batch),
          rope_cs=(rope_cs, rope_cs.shape[0] * d), out=(out, Qb * d))
    _check(load().bkv_decode_attention(C.byref(shape), _ptr(K, bf16, "K"), _ptr(V, bf16, "V"), int(n_len),
                                       _ptr(q, bf16, "q"), _ptr(pos, i32, "pos"), _ptr(rope_cs, f32, "rope_cs"),
                                       int(rope_cs.shape[0]), _ptr(out, f32, "out"), _stream(stream)),
           "bkv_decode_attention")
