"""Synthetic decode-attention loop: the attention side of a decode step over
the cache, with and without BeaconKV (the framing of Notes §3.5 Table 4:
tokens/s and memory at a full cache against a 2K-budget cache).

There are no model weights here.  A step is, per sequence, the new token's
key/value append and its attention over the cache for every layer and query
head; with BeaconKV the step also runs the eviction manager
(``bkv_decode_step``) and evicts when the cache is full.  The projections,
MLP and sampling of a real model are not simulated.

Each run starts at a steady state rather than from an empty cache:
  * beacon: the cache holds budget rows (just after an eviction) and the
    buffers n_beacon rows, so the window of steps covers whole eviction
    cycles;
  * full: the cache holds n0 rows, with n0 chosen so the window is centred on
    half the generation length, where the cost of a step linear in the cache
    length equals its mean over the whole generation.
Every step's inputs come from ``synth.StreamGen``; a block's inputs are drawn
before its timed region.
"""
from __future__ import annotations

import math
import time
from dataclasses import dataclass, replace

import torch

from . import lib, synth
from .configs import QWEN3_4B, EvictConfig, StreamConfig


@dataclass(frozen=True)
class DecodeConfig:
    name: str
    base: EvictConfig        # model shape and batch; for "beacon" also the budget and cache size
    mode: str                # "beacon" or "full"
    steps: int               # decode steps timed
    gen_len: int = 32768     # generation length the full-cache window stands for

    @property
    def cap(self) -> int:
        return self.base.cap if self.mode == "beacon" else self.gen_len

    @property
    def n0(self) -> int:
        """Cache rows at the start of the window."""
        return self.base.budget if self.mode == "beacon" else self.gen_len // 2 - self.steps // 2


# Notes §3.5 Table 4: Qwen3-4B, 32K generation; the full cache at batch 14 against a 2K budget at batch 192
DECODE_FULL = DecodeConfig("decode-qwen3-4b-full", replace(QWEN3_4B, batch=14, seed=20261202 + 600), "full", 256)
DECODE_BEACON = DecodeConfig("decode-qwen3-4b-beacon", replace(QWEN3_4B, batch=192, seed=20261202 + 610), "beacon",
                             512)
DECODE_CONFIGS = {c.name: c for c in (DECODE_FULL, DECODE_BEACON)}


def cache_bytes(dc: DecodeConfig, rows: int) -> int:
    b = dc.base
    return b.units * rows * b.d * 2 * 2


class DecodeRun:
    def __init__(self, dc: DecodeConfig, device="cuda", block: int = 64):
        self.dc = dc
        b = dc.base
        dev = torch.device(device)
        self.shape = lib.shape_of(b, cap=dc.cap)
        L, B, Hq, Hkv, d = b.n_layers, b.batch, b.hq, b.hkv, b.d
        g = torch.Generator(device=dev)
        g.manual_seed(b.seed + 1)
        self.K = torch.empty(L, B, Hkv, dc.cap, d, dtype=torch.bfloat16, device=dev)
        self.V = torch.empty_like(self.K)
        n0 = dc.n0
        for l in range(L):   # rows [0, n0): keys (post-RoPE) and values of the workload's distributions
            self.K[l, :, :, :n0] = synth.key_rows(g, (B, Hkv), n0, d, dev).to(torch.bfloat16)
            self.V[l, :, :, :n0] = torch.randn(B, Hkv, n0, d, generator=g, device=dev).to(torch.bfloat16)
        self.L = n0
        self.out = torch.empty(b.qbufs, d, dtype=torch.float32, device=dev)
        scfg = StreamConfig(name=dc.name, base=b, steps=dc.steps, drift_every=2048, p0_max=4096)
        self.gen = synth.StreamGen(scfg, dev)
        self.rope = torch.from_numpy(lib.rope_table(b.theta, d, 0, scfg.p0_max + dc.steps + 1)).to(dev)
        self.block = block
        self.pool = self.gen.alloc(block)
        if dc.mode == "beacon":
            q = synth.make_query_buffers(b, device=dev, fill=b.n_beacon)
            self.qbuf, self.qcount = q["qbuf"], q["qcount"]
            self.q_recent = torch.zeros(L, B, Hq, b.n_recent_q, d, dtype=torch.bfloat16, device=dev)
            self.pos_recent = torch.zeros(B, b.n_recent_q, dtype=torch.int32, device=dev)
        self.n_ev = 0

    def state_bytes(self) -> int:
        ts = [self.K, self.V]
        if self.dc.mode == "beacon":
            ts += [self.qbuf, self.qcount, self.q_recent, self.pos_recent]
        return sum(t.numel() * t.element_size() for t in ts)

    def run(self, stream=None) -> dict:
        """Time dc.steps decode steps; returns the summed GPU time and the cache rows attended to."""
        dc, b = self.dc, self.dc.base
        stream = torch.cuda.current_stream() if stream is None else stream
        gpu_ms, rows, done = 0.0, 0, 0
        t0 = time.perf_counter()
        while done < dc.steps:
            n = min(self.block, dc.steps - done)
            blk = self.gen.block(n, self.pool)
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            for i in range(n):
                if dc.mode == "beacon":
                    lib.decode_step(self.shape, self.K, self.V, self.L, blk["k_new"][i], blk["v_new"][i],
                                    blk["pos"][i], self.qbuf, self.qcount, blk["q_new"][i], self.q_recent,
                                    self.pos_recent, self.rope, stream=stream)
                else:
                    lib.append_kv(self.shape, self.K, self.V, self.L, blk["k_new"][i], blk["v_new"][i],
                                  blk["pos"][i], self.rope, stream=stream)
                self.L += 1
                lib.decode_attention(self.shape, self.K, self.V, self.L, blk["q_new"][i], blk["pos"][i], self.rope,
                                     self.out, stream=stream)
                rows += self.L
                self.last = (blk["q_new"][i], blk["pos"][i], self.L)
                if dc.mode == "beacon" and self.L == dc.cap:
                    lib.evict(self.shape, self.K, self.V, dc.cap, self.qbuf, self.qcount, self.q_recent,
                              self.pos_recent, blk["pos"][i], self.rope, stream=stream)
                    self.L = b.budget
                    self.n_ev += 1
            e1.record(stream)
            e1.synchronize()
            gpu_ms += e0.elapsed_time(e1)
            done += n
        return {"gpu_ms": gpu_ms, "rows": rows, "evictions": self.n_ev, "wall_s": time.perf_counter() - t0}

    def time_attention(self, n_len: int, reps: int = 10, stream=None) -> float:
        """Mean duration (ms) of bkv_decode_attention alone over n_len cached rows."""
        stream = torch.cuda.current_stream() if stream is None else stream
        blk = self.gen.block(1, self.pool)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        lib.decode_attention(self.shape, self.K, self.V, n_len, blk["q_new"][0], blk["pos"][0], self.rope, self.out,
                             stream=stream)
        e0.record(stream)
        for _ in range(reps):
            lib.decode_attention(self.shape, self.K, self.V, n_len, blk["q_new"][0], blk["pos"][0], self.rope,
                                 self.out, stream=stream)
        e1.record(stream)
        e1.synchronize()
        return e0.elapsed_time(e1) / reps


def mean_rows(dc: DecodeConfig) -> float:
    """Mean cache rows attended per step over the window (the new token included)."""
    if dc.mode == "full":
        return dc.n0 + (dc.steps + 1) / 2
    b = dc.base
    period = b.cap - b.budget
    return b.budget + (period + 1) / 2 if dc.steps % period == 0 else math.nan
