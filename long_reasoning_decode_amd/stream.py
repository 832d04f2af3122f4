"""Simulated decode loop around the eviction manager.

This is the caller's side of ``bkv_decode_step`` and ``bkv_evict``: a stand-in
for the model's decode loop (Notes §2.2, App. Alg. 2; Summary, pseudocode).
It draws every step's pre-RoPE q/k/v with ``synth.StreamGen``, hands them to
the library one decode step at a time, and evicts whenever the cache is full.
The library does all of the method's work; this loop only keeps the cache
length and passes pointers.  Under the naive full-history source (Notes §3.2
Fig. 7) it also hands every query to the library's history and, before each
eviction, has the library sample the beacons from the whole history.

Inputs are drawn a block of steps at a time, before the block's library calls,
so that timing a block (``timed=True``) measures the eviction manager alone.
"""
from __future__ import annotations

import time

import torch

from . import lib, synth
from .configs import StreamConfig


class StreamRun:
    """State of one simulated decode stream on the GPU.

    record_units: optional unit indices u = (l * batch + b) * Hkv + g whose
    step inputs and eviction results are kept (for checking against the
    oracle): ``hist`` holds q_new [S, Us, G, d], k_new / v_new [S, Us, d],
    pos [S, Us], and per eviction idx [E, Us, budget], scores [E, Us, cap]."""

    def __init__(self, scfg: StreamConfig, device="cuda", seed=None, record_units=None, block: int = 128):
        b = scfg.base
        self.scfg, self.base = scfg, b
        self.device = torch.device(device)
        self.shape = lib.shape_of(b)
        dev = self.device
        L, B, Hq, Hkv, d = b.n_layers, b.batch, b.hq, b.hkv, b.d
        self.K = torch.zeros(L, B, Hkv, b.cap, d, dtype=torch.bfloat16, device=dev)
        self.V = torch.zeros_like(self.K)
        self.qbuf = torch.zeros(L, B, Hq, b.qcap, d, dtype=torch.bfloat16, device=dev)
        self.qcount = torch.zeros(L, B, Hq, dtype=torch.int32, device=dev)
        self.q_recent = torch.zeros(L, B, Hq, b.n_recent_q, d, dtype=torch.bfloat16, device=dev)
        self.pos_recent = torch.zeros(B, b.n_recent_q, dtype=torch.int32, device=dev)
        self.rope = torch.from_numpy(lib.rope_table(b.theta, d, 0, scfg.rope_rows)).to(dev)
        self.naive = b.beacon == "naive"
        # naive full-history beacons: every past query of every head, up to the longest history the library
        # samples (a full history takes no more rows)
        self.hcap = lib.BKV_PREFILL_MAX if self.naive else 0
        self.hist = torch.zeros(L, B, Hq, self.hcap, d, dtype=torch.bfloat16, device=dev) if self.naive else None
        self.hcount = torch.zeros(L, B, Hq, dtype=torch.int32, device=dev) if self.naive else None
        self.h_rows = 0   # rows every history holds (the streams run in lockstep)
        self.idx = torch.empty(b.units, b.budget, dtype=torch.int32, device=dev)
        self.scores = torch.empty(b.units, b.cap, dtype=torch.float32, device=dev)
        self.gen = synth.StreamGen(scfg, dev, seed)
        self.block_steps = block
        self.pool = self.gen.alloc(block)
        self.L = 0
        self.n_ev = 0
        self.steps_done = 0
        self.rec = None
        if record_units is not None:
            self.rec_units = torch.tensor(list(record_units), dtype=torch.long, device=dev)
            self.rec_b = (self.rec_units // Hkv) % B
            self.rec = {k: [] for k in ("q_new", "k_new", "v_new", "pos", "idx", "scores")}

    @property
    def _STATE(self):
        return ("K", "V", "qbuf", "qcount", "q_recent", "pos_recent") + (("hist", "hcount") if self.naive else ())

    def state_dict(self) -> dict:
        """Everything needed to resume the stream: the eviction manager's tensors, the cache length and
        counters, and the input generator's state."""
        st = {k: getattr(self, k).clone() for k in self._STATE}
        st.update(L=self.L, n_ev=self.n_ev, steps_done=self.steps_done, h_rows=self.h_rows,
                  gen=self.gen.state_dict())
        return st

    def load_state_dict(self, st: dict) -> None:
        for k in self._STATE:
            getattr(self, k).copy_(st[k])
        self.L, self.n_ev, self.steps_done = int(st["L"]), int(st["n_ev"]), int(st["steps_done"])
        self.h_rows = int(st.get("h_rows", 0))
        self.gen.load_state_dict(st["gen"])

    def state_bytes(self) -> int:
        """HBM held by the eviction manager's own state (cache, buffers, ring, table, keep-set and score copies,
        and the query history under the naive source)."""
        ts = (self.K, self.V, self.qbuf, self.qcount, self.q_recent, self.pos_recent, self.rope, self.idx,
              self.scores) + ((self.hist, self.hcount) if self.naive else ())
        return sum(t.numel() * t.element_size() for t in ts)

    def beacon_state_bytes(self) -> dict:
        """HBM of the beacon state: the query buffers (and the history, under the naive source) -- the memory
        axis of the continual-against-naive FPS comparison (Notes §3.2 Fig. 7)."""
        buf = self.qbuf.numel() * self.qbuf.element_size() + self.qcount.numel() * 4
        hist = self.hist.numel() * self.hist.element_size() + self.hcount.numel() * 4 if self.naive else 0
        return {"buffers": buf, "history": hist, "total": buf + hist}

    def _record_inputs(self, blk: dict, n: int) -> None:
        b = self.base
        U, G, d = b.units, b.G, b.d
        r, u = self.rec, self.rec_units
        r["q_new"].append(blk["q_new"][:n].reshape(n, U, G, d).index_select(1, u))
        r["k_new"].append(blk["k_new"][:n].reshape(n, U, d).index_select(1, u))
        r["v_new"].append(blk["v_new"][:n].reshape(n, U, d).index_select(1, u))
        r["pos"].append(blk["pos"][:n].index_select(1, self.rec_b))

    def run(self, steps: int | None = None, timed: bool = False, stream=None, progress=None,
            detail_blocks=(), keep_idx: bool = False) -> dict:
        """Run `steps` decode steps (default: the config's).  Returns the step count, evictions and,
        when timed, the summed GPU time of the library calls (generation excluded), each eviction's
        latency, and the latency of every decode step in the blocks listed in `detail_blocks` (block
        indices counted from this call's first block).  keep_idx: every eviction also writes its keep
        sets to self.idx, and the counts it started from go to self.last_qcount."""
        b = self.base
        steps = self.scfg.steps if steps is None else steps
        stream = torch.cuda.current_stream() if stream is None else stream
        gpu_ms = 0.0
        evict_ms, step_ms = [], []
        t0 = time.perf_counter()
        done = 0
        blk_no = 0
        ev = lambda: torch.cuda.Event(enable_timing=True)
        while done < steps:
            n = min(self.block_steps, steps - done)
            blk = self.gen.block(n, self.pool)
            if self.rec is not None:
                self._record_inputs(blk, n)
            detail = timed and blk_no in detail_blocks
            evs, step_evs = [], []
            if timed:
                e0, e1 = ev(), ev()
                e0.record(stream)
            for i in range(n):
                if detail:
                    step_evs.append(ev())
                    step_evs[-1].record(stream)
                lib.decode_step(self.shape, self.K, self.V, self.L, blk["k_new"][i], blk["v_new"][i], blk["pos"][i],
                                self.qbuf, self.qcount, blk["q_new"][i], self.q_recent, self.pos_recent, self.rope,
                                stream=stream)
                if self.naive:
                    lib.history_append(self.shape, self.hist, self.hcap, self.hcount, blk["q_new"][i], stream=stream)
                    self.h_rows = min(self.h_rows + 1, self.hcap)
                self.L += 1
                if detail:
                    step_evs.append(ev())
                    step_evs[-1].record(stream)
                if self.L == b.cap:
                    rec = self.rec is not None
                    if keep_idx:
                        self.last_qcount = self.qcount.clone()
                    if timed:
                        evs.append((ev(), ev()))
                        evs[-1][0].record(stream)
                    if self.naive:   # beacons: FPS over each head's history, less the cycle's recent queries
                        lib.fps_history(self.shape, self.hist, self.hcap, max(0, self.h_rows - b.n_recent_q),
                                        self.qbuf, self.qcount, stream=stream)
                    lib.evict(self.shape, self.K, self.V, b.cap, self.qbuf, self.qcount, self.q_recent,
                              self.pos_recent, blk["pos"][i], self.rope,
                              idx_out=self.idx if rec or keep_idx else None,
                              scores_out=self.scores if rec else None, stream=stream)
                    if timed:
                        evs[-1][1].record(stream)
                    if rec:
                        self.rec["idx"].append(self.idx.index_select(0, self.rec_units))
                        self.rec["scores"].append(self.scores.index_select(0, self.rec_units))
                    self.n_ev += 1
                    self.L = b.budget
            if timed:
                e1.record(stream)
                e1.synchronize()
                gpu_ms += e0.elapsed_time(e1)
                evict_ms += [a.elapsed_time(z) for a, z in evs]
                step_ms += [step_evs[k].elapsed_time(step_evs[k + 1]) for k in range(0, len(step_evs), 2)]
            done += n
            blk_no += 1
            self.steps_done += n
            if progress is not None:
                progress(self)
        torch.cuda.synchronize()
        return {"steps": steps, "evictions": self.n_ev, "L": self.L, "gpu_ms": gpu_ms if timed else None,
                "evict_ms": evict_ms, "step_ms": step_ms, "wall_s": time.perf_counter() - t0}

    def fps_rounds_per_buffer(self, steps: int | None = None) -> int:
        """Sampling rounds each query buffer goes through in `steps` decode steps from an empty state
        (the count evolves the same way in every buffer).  Only continual FPS samples; the other beacon
        sources never do."""
        b = self.base
        steps = self.scfg.steps if steps is None else steps
        if b.beacon != "fps":
            return 0
        bqmax, ring0 = b.n_beacon + b.n_recent_q, b.cap - b.n_recent_q
        L = qc = rounds = 0
        for _ in range(steps):
            if L < ring0:
                qc += 1
                if qc >= bqmax:
                    rounds += 1
                    qc = b.n_beacon
            elif L == ring0 and qc > b.n_beacon:   # compressed at the freeze point
                rounds += 1
                qc = b.n_beacon
            L += 1
            if L == b.cap:
                qc = min(min(qc, b.n_beacon) + b.n_recent_q, b.n_beacon)
                L = b.budget
        return rounds

    def history(self) -> dict:
        """Recorded inputs and eviction results as host tensors (see the class docstring)."""
        out = {}
        for k, v in self.rec.items():
            out[k] = torch.cat(v, 0).cpu() if v else None
        if out["idx"] is not None:
            E = len(self.rec["idx"])
            out["idx"] = out["idx"].reshape(E, -1, self.base.budget)
            out["scores"] = out["scores"].reshape(E, -1, self.base.cap)
        return out
