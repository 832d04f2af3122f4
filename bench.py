"""Benchmark of the BeaconKV eviction step on one MI355X.

One step = one bkv_evict call over every (layer, batch, KV head) unit of the
Qwen3-4B-shaped cache: 36 layers x batch 16 x 8 KV heads = 4608 units, cache
length 2176 -> budget 2048, head_dim 128, 32 query heads (G = 4), 16 beacons
+ 16 recent queries per query head.  Two timings, both reported:
  * pristine (the default for `value`): before each step, outside its timed
    region, the original cache and buffers are restored from device copies and
    a 512 MB scratch buffer is touched to flush the MALL; each step is timed on
    its own between two synchronisations;
  * back-to-back: the steps run in place on one stream, each evicting 128 rows
    from the cache the previous step left (rows [budget, n_len) still hold the
    earlier tail rows), so every step does a full eviction's work.

Prints one JSON line (see the keys below); `value` is eviction steps/s with
all inputs resident in HBM.  `roofline` is for the dominant kernel (the fused
per-unit eviction kernel), `step_hbm` for the whole step, both from algorithmic bytes and
HIP-event durations measured here.  `cpu_baseline` times the CPU oracle on a
bounded sample of the same units.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np
import torch

from long_reasoning_decode_amd import lib as L
from long_reasoning_decode_amd import synth
from long_reasoning_decode_amd.configs import (EVICT_CONFIGS, PREFILL, PREFILL_CONFIGS, QWEN3_4B, STREAM,
                                               STREAM_CONFIGS)

HERE = os.path.dirname(os.path.abspath(__file__))
HBM_PEAK_GBS = 8000.0  # MI355X HBM3E, GB/s
# fp32 multiply-add issue rate without packed math: 256 CUs x 4 SIMDs x 16 lanes x 2 flop x 2.4 GHz.  The
# packed-math figure (157.3 TFLOP/s) needs v_pk_fma_f32, which these kernels are built without.
FP32_VALU_PEAK_TFS = 256 * 4 * 16 * 2 * 2.4e9 / 1e12
METRIC = "eviction steps/s (all layers x KV heads) at Qwen3-4B shape; % of HBM peak"
# kernel -> the .hip file it is compiled from; its stored counters hold only while that file, everything it
# includes and the build flags are unchanged
KERNEL_SOURCE = {"evict_kernel": "bkv_evict.hip", "compact_kernel": "bkv_compact.hip", "score_kernel": "bkv_score.hip",
                 "select_kernel": "bkv_select.hip", "fps_kernel": "bkv_fps.hip", "attn_kernel": "bkv_attention.hip",
                 "append_kernel": "bkv_stream.hip"}
TRAFFIC_FILE = os.path.join(HERE, "profiles", "hbm_traffic_qwen3-4b.txt")


def traffic_file(config: str) -> str:
    """The counter summary of an eviction workload (the headline one is TRAFFIC_FILE)."""
    return TRAFFIC_FILE if config == QWEN3_4B.name else os.path.join(HERE, "profiles", f"hbm_traffic_{config}.txt")


def kernel_sources_sha256(kernel: str) -> str:
    """sha256 over the kernel's .hip file, the local headers it includes (transitively) and the compile
    flags."""
    import hashlib
    import re
    dirs = [os.path.join(HERE, "long_reasoning_decode_amd", "csrc"), os.path.join(HERE, "include")]
    seen, todo, h = [], [KERNEL_SOURCE[kernel]], hashlib.sha256()
    while todo:
        f = todo.pop(0)
        if f in seen:
            continue
        seen.append(f)
        path = next(os.path.join(d, f) for d in dirs if os.path.exists(os.path.join(d, f)))
        text = open(path, "rb").read()
        h.update(f.encode() + b"\0" + text)
        todo += re.findall(r'#include "([^"]+)"', text.decode())
    from long_reasoning_decode_amd import build as lib_build
    h.update(" ".join(lib_build.device_flags()).encode())
    return h.hexdigest()


def stored_traffic(kernel: str, path: str | None = None):
    """HBM bytes per launch of `kernel` from a committed counter summary (default: the eviction step's),
    or None when there is none or the kernel's sources changed since the counters were taken."""
    path = TRAFFIC_FILE if path is None else path
    if not os.path.exists(path):
        return None
    for line in open(path):
        if line.startswith("#"):
            continue
        f = dict(kv.split("=", 1) for kv in line.split() if "=" in kv)
        if f.get("kernel") == kernel:
            if f.get("sources_sha256") != kernel_sources_sha256(kernel):
                return None
            return float(f["bytes_per_dispatch"])
    return None


def summarize_counters(fetch_dir: str, write_dir: str, calib_bytes: int) -> str:
    """Per-kernel HBM bytes from two rocprofv3 counter passes (CSV output): FETCH_SIZE in one,
    WRITE_SIZE in the other, KiB per dispatch.  Each counter is scaled by what it reads for the run's
    calibration copy (the longest copy dispatch, of calib_bytes read and calib_bytes written)."""
    import csv
    import glob

    def load(d, counter):
        per = {}   # dispatch id -> [kernel name, duration ns, value]
        for fn in glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True):
            for r in csv.DictReader(open(fn)):
                if r["Counter_Name"] != counter:
                    continue
                e = per.setdefault(r["Dispatch_Id"], [r["Kernel_Name"],
                                                      int(r["End_Timestamp"]) - int(r["Start_Timestamp"]), 0.0])
                e[2] += float(r["Counter_Value"])
        if not per:
            raise SystemExit(f"no {counter} rows under {d}")
        return per

    lines = []
    stats = {}
    for counter, d in (("FETCH_SIZE", fetch_dir), ("WRITE_SIZE", write_dir)):
        per = load(d, counter)
        copies = [e for e in per.values() if "copyBuffer" in e[0]]
        cal = max(copies, key=lambda e: e[1])
        factor = calib_bytes / (cal[2] * 1024.0)
        lines.append(f"# calibration {counter}: copy of {calib_bytes} bytes ({cal[1] / 1e3:.0f} us) reads "
                     f"{cal[2]:.0f} KiB -> factor {factor:.4f}")
        for k in KERNEL_SOURCE:
            vals = [e[2] for e in per.values() if k in e[0] and "bkv" in e[0]]
            if vals:
                stats.setdefault(k, {})[counter] = (float(np.mean(vals)), len(vals), factor)
    for k, st in stats.items():
        if len(st) != 2:
            continue
        (fk, nf, ff), (wk, nw, fw) = st["FETCH_SIZE"], st["WRITE_SIZE"]
        b = fk * 1024 * ff + wk * 1024 * fw
        lines.append(f"kernel={k} dispatches={nf},{nw} fetch_kib={fk:.0f} write_kib={wk:.0f} "
                     f"fetch_bytes={fk * 1024 * ff:.4g} write_bytes={wk * 1024 * fw:.4g} bytes_per_dispatch={b:.6g} "
                     f"sources_sha256={kernel_sources_sha256(k)}")
    return "\n".join(lines) + "\n"


def alg_bytes(cfg, qcount: np.ndarray, idx: np.ndarray, n_len: int) -> dict:
    """Algorithmic bytes of one eviction: K read once for scoring, the
    observation rows read, moved K and V rows read and written, the new
    buffers written.  qcount [units, G] before the call; idx [units, budget].

    The gather K^ = K[:, I_final, :] (Notes §2.3 Eq. 8) reads the moved key rows
    that the scoring has already read; "strict" counts them once (a moved key row
    is written, a moved value row read and written), the lower bound of any
    implementation that reads every key at most once."""
    d2 = cfg.d * 2
    B = min(cfg.budget, n_len)
    moved = (idx[:, :B] != np.arange(B)[None, :]).sum(axis=1).astype(np.int64)
    rows = (np.minimum(qcount, cfg.n_beacon) + cfg.n_recent_q).sum(axis=1).astype(np.int64)
    k_read = cfg.units * n_len * d2
    q_read = int(rows.sum()) * d2
    compact = int(4 * moved.sum()) * d2
    buf = cfg.qbufs * cfg.n_beacon * d2
    strict = k_read + q_read + int(3 * moved.sum()) * d2 + buf
    return {"k_read": k_read, "q_read": q_read, "compact": compact, "buffers": buf,
            "total": k_read + q_read + compact + buf, "total_strict": strict, "moved_rows": int(moved.sum())}


BF16_MFMA_PEAK_TFS = 2500.0   # MI355X dense bf16 matrix rate


def qkt_mfma(cfg, n_len: int, evict_ms: float, score_ms: float) -> dict:
    """Matrix-core rate of the scoring's Q K^T.  Algorithmic: one product of the R observation rows with
    the N keys per unit (R N d multiply-adds).  Issued: what the kernels run, two passes over the keys with
    each query head's rows padded to 32 and the keys to whole 32-key tiles."""
    R = cfg.G * (cfg.n_beacon + cfg.n_recent_q)
    alg = 2.0 * R * n_len * cfg.d * cfg.units
    tiles = (n_len + 31) // 32
    issued = 2 * (2.0 * cfg.G * 32 * tiles * 32 * cfg.d * cfg.units)
    tf = lambda f, ms: f / (ms * 1e-3) / 1e12
    return {"alg_flops": alg, "issued_flops": issued, "peak_TFs": BF16_MFMA_PEAK_TFS,
            "evict_kernel": {"alg_TFs": tf(alg, evict_ms), "issued_TFs": tf(issued, evict_ms),
                             "frac_issued": tf(issued, evict_ms) / BF16_MFMA_PEAK_TFS},
            "score_kernel": {"alg_TFs": tf(alg, score_ms), "issued_TFs": tf(issued, score_ms),
                             "frac_issued": tf(issued, score_ms) / BF16_MFMA_PEAK_TFS}}


def copy_reference(stream, nbytes: int = 1 << 30, reps: int = 5) -> dict:
    """A plain device-to-device copy of nbytes (torch's copy_, the runtime's copy kernel), timed with HIP
    events on `stream`: the read + write rate that a copy reaches on this GPU, as context for the
    eviction's rate (whose traffic is mostly such a copy)."""
    src = torch.empty(nbytes, dtype=torch.uint8, device="cuda").fill_(1)
    dst = torch.empty_like(src)
    with torch.cuda.stream(stream):
        dst.copy_(src)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(reps):
            dst.copy_(src)
        e1.record(stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / reps
    gbs = 2 * nbytes / (ms * 1e-3) / 1e9
    del src, dst
    return {"bytes_moved": 2 * nbytes, "ms": ms, "GBs": gbs, "frac": gbs / HBM_PEAK_GBS}


def cpu_baseline(cfg, inp, target_s: float = 10.0) -> dict:
    """The CPU oracle (as it stands) on a bounded sample of units, spread over the workload."""
    import oracle as O
    threads = O.default_threads()
    oc = O.OracleCfg(hq=cfg.hq, hkv=cfg.hkv, d=cfg.d, cap=cfg.n_len, budget=cfg.budget, n_prefix=cfg.n_prefix,
                     n_recent_kv=cfg.n_recent_kv, n_beacon=cfg.n_beacon, n_recent_q=cfg.n_recent_q,
                     theta=cfg.theta, qcap=cfg.qcap, pool_mean=int(cfg.pool == "mean"))

    def one(ns):
        v = synth.oracle_views(cfg, inp, _spread(ns, cfg.units).tolist())
        t0 = time.perf_counter()
        O.evict(oc, v["K"], v["V"], v["qbuf"], v["qcount"], v["q_recent"], v["pos_recent"], v["t"],
                nthreads=threads)
        return len(v["units"]), time.perf_counter() - t0

    n, dt = _grow_sample(one, max(threads, 8), cfg.units, target_s)
    units_per_s = n / dt
    return {"value": units_per_s / cfg.units, "unit": "eviction steps/s", "cores": threads, "kind": "oracle",
            "sample": f"{n} of {cfg.units} units of the same workload, one eviction each, {dt:.1f} s wall "
                      f"on {threads} threads; scaled to whole steps"}


def _grow_sample(run_sample, n0: int, n_max: int, target_s: float):
    """Calls run_sample(n) -> (items sampled, seconds) with a growing sample size n until one call takes
    about target_s (or n reaches n_max); returns the last call's (items, seconds)."""
    n = min(n0, n_max)
    while True:
        got, dt = run_sample(n)
        if dt >= target_s or n >= n_max:
            return got, dt
        n = min(n_max, max(n + n0, int(n * target_s / max(dt, 1e-3) * 1.05)))


def _spread(n: int, total: int) -> np.ndarray:
    """n distinct indices spread evenly over [0, total)."""
    return np.unique(np.linspace(0, total - 1, n).round().astype(np.int64))


def _in_threads(fn, n: int, threads: int) -> None:
    """fn(lo, hi) over `threads` contiguous slices of range(n), concurrently (the oracle's C calls
    release the GIL)."""
    from concurrent.futures import ThreadPoolExecutor
    cuts = [n * i // threads for i in range(threads + 1)]
    with ThreadPoolExecutor(threads) as ex:
        list(ex.map(lambda i: fn(cuts[i], cuts[i + 1]), [i for i in range(threads) if cuts[i] < cuts[i + 1]]))


def stream_cpu_baseline(run, target_s: float = 10.0) -> dict:
    """The CPU oracle (as it stands) replaying one eviction cycle of a bounded sample of units: from the
    state the GPU stream holds right after an eviction, the next n_new decode steps, the last of which
    evicts.  Scaled to tokens/s of the whole batch in that steady state."""
    import oracle as O
    b = run.base
    if run.L != b.budget:                 # advance the GPU stream to the start of a cycle
        run.run(b.cap - run.L)
    n = b.n_new
    blk = run.gen.block(n, run.pool)
    U, G, d, cap = b.units, b.G, b.d, b.cap
    dev = run.K.device
    threads = O.default_threads()
    K, V = run.K.reshape(U, cap, d), run.V.reshape(U, cap, d)
    qbuf, qcount = run.qbuf.reshape(U, G, b.qcap, d), run.qcount.reshape(U, G)
    q_recent = run.q_recent.reshape(U, G, b.n_recent_q, d)
    k_new, v_new = blk["k_new"][:n].reshape(n, U, d), blk["v_new"][:n].reshape(n, U, d)
    q_new = blk["q_new"][:n].reshape(n, U, G, d)
    i32 = lambda t: np.ascontiguousarray(t.cpu().numpy().astype(np.int32))

    def one(ns):
        units = _spread(ns, U)
        ut = torch.from_numpy(units).to(dev)
        bt = (ut // b.hkv) % b.batch
        st = [synth.to_u16(K.index_select(0, ut)), synth.to_u16(V.index_select(0, ut)),
              synth.to_u16(qbuf.index_select(0, ut)), i32(qcount.index_select(0, ut)),
              synth.to_u16(q_recent.index_select(0, ut)), i32(run.pos_recent.index_select(0, bt))]
        ins = [synth.to_u16(k_new.index_select(1, ut)), synth.to_u16(v_new.index_select(1, ut)),
               synth.to_u16(q_new.index_select(1, ut)), i32(blk["pos"][:n].index_select(1, bt))]
        oc = O.OracleCfg(hq=b.hq, hkv=b.hkv, d=d, cap=cap, budget=b.budget, n_prefix=b.n_prefix,
                         n_recent_kv=b.n_recent_kv, n_beacon=b.n_beacon, n_recent_q=b.n_recent_q, theta=b.theta,
                         qcap=b.qcap, pool_mean=int(b.pool == "mean"),
                         beacon_src={"fps": O.SRC_FPS, "initial": O.SRC_INITIAL, "random": O.SRC_RANDOM,
                                     "naive": O.SRC_NAIVE}[b.beacon],
                         seed=b.seed & 0xFFFFFFFF, n_layers=b.n_layers, batch=b.batch, unit_ids=units.tolist())
        hist = {}
        if getattr(run, "naive", False):   # the sampled units' query histories
            hist = {"hist": synth.to_u16(run.hist.reshape(U, G, run.hcap, d).index_select(0, ut)),
                    "hcount": i32(run.hcount.reshape(U, G).index_select(0, ut))}
        t0 = time.perf_counter()
        o = O.stream(oc, *ins, st[0], st[1], b.budget, *st[2:], nthreads=threads, **hist)
        dt = time.perf_counter() - t0
        assert o["n_ev"] == 1 and o["L"] == b.budget, o
        return len(units), dt

    ns, dt = _grow_sample(one, 4 * threads, min(U, 4096), target_s)
    return {"value": b.batch * n / (dt * U / ns), "unit": "tokens/s", "cores": threads, "kind": "oracle",
            "sample": f"{ns} of {U} units, one eviction cycle ({n} decode steps, the last evicting) from the "
                      f"GPU stream's state, {dt:.1f} s wall on {threads} threads; scaled to the whole batch"}


def stream_evict_roofline(run, evict_ms: float) -> dict:
    """HBM roofline of the stream's evictions, its dominant cost: the algorithmic bytes of one steady-state
    eviction (from one more, untimed cycle whose eviction reports its keep sets) over the timed run's mean
    eviction time (bkv_evict: evict_kernel and the buffer merge; under the naive source the timed eviction
    also holds the FPS over every history, which these bytes do not count)."""
    b = run.base
    if run.L != b.budget:                 # advance to the start of a cycle
        run.run(b.cap - run.L)
    run.run(b.n_new, keep_idx=True)
    ab = alg_bytes(b, run.last_qcount.reshape(b.units, b.G).cpu().numpy(), run.idx.cpu().numpy(), b.cap)
    ach = ab["total"] / (evict_ms * 1e-3) / 1e9
    kern = ("bkv_fps_history + bkv_evict (history FPS, evict_kernel)" if getattr(run, "naive", False)
            else "bkv_evict (evict_kernel + merge)")
    return {"bound": "hbm", "kernel": kern, "achieved": ach, "peak": HBM_PEAK_GBS,
            "unit": "GB/s", "frac": ach / HBM_PEAK_GBS, "traffic": None, "alg_bytes_per_launch": ab["total"],
            "moved_rows_per_unit": ab["moved_rows"] / b.units}


def stream_bench(args) -> int:
    """Streaming decode: tokens/s of the eviction manager (library calls only; each block's inputs are
    drawn before its timed region) and its HBM footprint."""
    from long_reasoning_decode_amd.stream import StreamRun
    scfg = STREAM_CONFIGS[args.stream_config]
    b = scfg.base
    steps = args.stream_steps or scfg.steps
    torch.cuda.set_device(0)
    L.load()
    print(f"# stream {scfg.name}: batch {b.batch}, {steps} steps, {b.units} units", file=sys.stderr, flush=True)
    run = StreamRun(scfg)
    torch.cuda.reset_peak_memory_stats()
    prog = lambda r: (r.steps_done % 4096 == 0) and print(f"# step {r.steps_done}, evictions {r.n_ev}",
                                                            file=sys.stderr, flush=True)
    n_blocks = (steps + run.block_steps - 1) // run.block_steps
    detail = sorted({n_blocks // 4, n_blocks // 2, (3 * n_blocks) // 4})
    r = run.run(steps, timed=True, progress=prog, detail_blocks=detail)
    tokens = b.batch * steps
    pct = lambda v, q: float(np.percentile(v, q)) if len(v) else None
    rounds = run.fps_rounds_per_buffer(steps)
    out = {
        "metric": "streaming decode: tokens/s through the eviction manager (decode-step bookkeeping + evictions)",
        "value": tokens / (r["gpu_ms"] * 1e-3), "unit": "tokens/s", "n_gpus": 1, "steps": steps,
        "higher_is_better": True, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": f"{scfg.name}: {b.n_layers} layers x batch {b.batch} x {b.hkv} KV heads "
                               f"({b.units} units), {b.hq} query heads, head_dim {b.d}, cache {b.cap} -> "
                               f"budget {b.budget}, evict every {b.n_new} steps",
                   "evictions": r["evictions"]},
        "gpu_s": r["gpu_ms"] * 1e-3, "wall_s_with_generation": r["wall_s"],
        "eviction_ms": {"mean": float(np.mean(r["evict_ms"])) if r["evict_ms"] else None,
                        "p50": pct(r["evict_ms"], 50), "p99": pct(r["evict_ms"], 99),
                        "max": max(r["evict_ms"]) if r["evict_ms"] else None},
        "decode_step_us": {"sampled_steps": len(r["step_ms"]), "mean": float(np.mean(r["step_ms"])) * 1e3,
                           "p50": pct(r["step_ms"], 50) * 1e3, "p99": pct(r["step_ms"], 99) * 1e3,
                           "max": max(r["step_ms"]) * 1e3},
        "fps_rounds": {"per_buffer": rounds, "total": rounds * b.qbufs},
        "state_bytes": run.state_bytes(), "peak_allocated_bytes": torch.cuda.max_memory_allocated(),
        "beacon_state_bytes": run.beacon_state_bytes(),
    }
    if r["evict_ms"]:
        out["roofline"] = stream_evict_roofline(run, out["eviction_ms"]["mean"])
    if b.beacon == "fps" and b.n_recent_q > 0 and b.n_beacon > 0:
        out["fps_round"] = fps_round_bench(b, run.shape, run.qbuf, run.gen.block(1, run.pool)["q_new"][0],
                                           name=scfg.name)
    if not args.no_cpu_baseline:
        print("# cpu baseline (oracle)", file=sys.stderr, flush=True)
        out["cpu_baseline"] = stream_cpu_baseline(run, args.cpu_seconds)
    print(json.dumps(out), flush=True)
    return 0


FP32_MFMA_PEAK_TFS = 157.3   # MI355X dense fp32 matrix rate


def fps_round_bench(b, shape, qbuf_src, q_new, reps: int = 10, name: str = "", timing: str = "pristine") -> dict:
    """One sampling round of every buffer: bkv_fps_update with every count at B_Q^max - 1, on a copy of
    the given buffers, timed alone with HIP events (the counts are reset between the timed calls).
    timing "pristine": before each round (untimed) a 512 MB scratch buffer is read, as the eviction bench
    does before each step, so that each round starts after memory-bound work, as in a decode stream, where
    fifteen decode steps separate two rounds; "back-to-back": the rounds follow each other (the chip's clock
    then drops under the sustained fp32 matrix load).
    Roofline: the Gram matrices are the matrix-core work, 2 n^2 d flops per buffer (all n^2 dot products,
    as the definition takes them; n = B_Q^max), against the dense fp32 MFMA rate."""
    n = b.n_beacon + b.n_recent_q
    qbuf = qbuf_src.clone()
    qc = torch.empty(b.qbufs, dtype=torch.int32, device=qbuf.device)
    stream = torch.cuda.current_stream()
    scratch = torch.ones(512 << 18, dtype=torch.int32, device=qbuf.device) if timing == "pristine" else None
    flush_sum = torch.zeros((), dtype=torch.int64, device=qbuf.device)
    ms = []
    for i in range(reps + 2):
        qc.fill_(n - 1)
        if scratch is not None:
            flush_sum.copy_(scratch.sum(dtype=torch.int64))   # reads all 512 MB
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        L.fps_update(shape, qbuf, qc, q_new, None, stream=stream)
        e1.record(stream)
        e1.synchronize()
        if i >= 2:
            ms.append(e0.elapsed_time(e1))
    t = float(np.mean(ms))
    flops = 2.0 * n * n * b.d * b.qbufs
    achieved = flops / (t * 1e-3) / 1e12
    if scratch is not None:
        assert int(flush_sum) == scratch.numel()
    del qbuf, qc, scratch
    return {"buffers": b.qbufs, "rows": n, "timing": timing, "ms": t, "ms_min": float(min(ms)),
            "roofline": {"bound": "mfma", "kernel": "fps_kernel (update, every buffer sampling)",
                         "achieved": achieved, "peak": FP32_MFMA_PEAK_TFS, "unit": "TFLOP/s",
                         "frac": achieved / FP32_MFMA_PEAK_TFS, "flops_per_launch": flops,
                         "traffic": stored_traffic("fps_kernel", os.path.join(HERE, "profiles",
                                                                              f"hbm_traffic_fps-round-{name}.txt"))
                         if name else None}}


def fps_round_cpu_baseline(b, q: dict, target_s: float = 10.0) -> dict:
    """The CPU oracle's buffer update (as it stands) on a bounded sample of the same full buffers, each
    sampling once; the oracle's call is one thread, run on slices of the sample in parallel."""
    import oracle as O
    threads = O.default_threads()
    nb, n = b.qbufs, b.n_beacon + b.n_recent_q
    qb, qn = q["qbuf"].reshape(nb, b.qcap, b.d), q["q_new"].reshape(nb, b.d)
    dev = qb.device

    def one(ns):
        t = torch.from_numpy(_spread(ns, nb)).to(dev)
        qbh, qnh = synth.to_u16(qb.index_select(0, t)), synth.to_u16(qn.index_select(0, t))
        qc = np.full(len(t), n - 1, np.int32)
        t0 = time.perf_counter()
        _in_threads(lambda lo, hi: O.fps_update(qbh[lo:hi], qc[lo:hi], qnh[lo:hi], b.n_beacon, b.n_recent_q),
                    len(t), threads)
        dt = time.perf_counter() - t0
        assert (qc == b.n_beacon).all()
        return len(t), dt

    ns, dt = _grow_sample(one, 64 * threads, nb, target_s)
    return {"value": ns / dt / nb, "unit": "rounds/s", "cores": threads, "kind": "oracle",
            "sample": f"{ns} of {nb} buffers, one sampling round each, {dt:.1f} s wall on {threads} threads; "
                      f"scaled to a round of every buffer"}


def fps_round_main(args) -> int:
    """Only the FPS sampling round, on buffers of a stream workload's shape filled with its query mixture."""
    scfg = STREAM_CONFIGS[args.stream_config]
    b = scfg.base
    torch.cuda.set_device(0)
    L.load()
    print(f"# fps round {scfg.name}: {b.qbufs} buffers", file=sys.stderr, flush=True)
    q = synth.make_query_buffers(b, device="cuda")
    r = fps_round_bench(b, L.shape_of(b), q["qbuf"], q["q_new"], reps=args.steps, name=scfg.name,
                        timing=args.timing)
    out = {"metric": "FPS sampling round of every query buffer (bkv_fps_update, every buffer full)",
           "value": 1000.0 / r["ms"], "unit": "rounds/s", "n_gpus": 1, "steps": args.steps,
           "higher_is_better": True, "dtype": "f32 (bf16 rows)", "data": "synthetic",
           "config": {"workload": f"{scfg.name} buffers: {b.n_layers} layers x batch {b.batch} x {b.hq} query "
                                  f"heads ({b.qbufs} buffers of {b.qcap} x {b.d}), {b.n_beacon} beacons + "
                                  f"{b.n_recent_q} recent queries"},
           **r}
    if args.copy_calibration_mib > 0:   # a copy of known size for counter passes (see the eviction bench)
        src = torch.empty(args.copy_calibration_mib << 20, dtype=torch.uint8, device="cuda").fill_(1)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
    if not args.no_cpu_baseline:
        print("# cpu baseline (oracle)", file=sys.stderr, flush=True)
        out["cpu_baseline"] = fps_round_cpu_baseline(b, q, args.cpu_seconds)
    print(json.dumps(out), flush=True)
    return 0


def prefill_flops_per_row(d: int, m: int) -> int:
    """Algorithmic fp32 flops per prompt row of the prefill sampling: norm (d multiply-adds), unit row (d
    products), column sum (d adds), mean cosine (d multiply-adds), and m - 1 cosine updates (d multiply-adds
    each), a multiply-add counting 2."""
    return (2 + 1 + 1 + 2 + 2 * (m - 1)) * d


def prefill_cpu_baseline(cfg, q: torch.Tensor, target_s: float) -> dict:
    """The CPU oracle's prefill sampling (as it stands) on a bounded sample of buffers; the oracle's call is
    one thread, run on slices of the sample in parallel."""
    import oracle as O
    b, P = cfg.base, cfg.n_prompt
    threads = O.default_threads()
    qn = q.reshape(b.qbufs, P, b.d)

    def one(ns):
        t = torch.from_numpy(_spread(ns, b.qbufs)).to(qn.device)
        x = synth.to_u16(qn.index_select(0, t))
        qbuf = np.zeros((len(t), b.qcap, b.d), np.uint16)
        qc = np.zeros(len(t), np.int32)
        t0 = time.perf_counter()
        _in_threads(lambda lo, hi: O.prefill(x[lo:hi], qbuf[lo:hi], qc[lo:hi], b.n_beacon), len(t), threads)
        dt = time.perf_counter() - t0
        assert (qc == min(P, b.n_beacon)).all()
        return len(t), dt

    ns, dt = _grow_sample(one, threads, b.qbufs, target_s)
    return {"value": ns / dt / b.qbufs, "unit": "prefill initialisations/s", "cores": threads, "kind": "oracle",
            "sample": f"{ns} of {b.qbufs} buffers of the same workload, {dt:.1f} s wall on {threads} threads; "
                      f"scaled to whole initialisations"}


def prefill_bench(args) -> int:
    """Prefill initialisation of every query buffer (bkv_fps_prefill) on the model-shaped batch."""
    pc = PREFILL_CONFIGS[args.prefill_config]
    b, P = pc.base, pc.n_prompt
    torch.cuda.set_device(0)
    L.load()
    print(f"# prefill {pc.name}: {b.qbufs} buffers x {P} prompt queries", file=sys.stderr, flush=True)
    q = synth.make_prompt_queries(b, P, device="cuda")
    shape = L.shape_of(b)
    qbuf = torch.empty((b.qbufs, b.qcap, b.d), dtype=torch.bfloat16, device="cuda")
    qc = torch.empty((b.qbufs,), dtype=torch.int32, device="cuda")
    stream = torch.cuda.current_stream()
    for _ in range(args.warmup):
        L.fps_prefill(shape, q, P, qbuf, qc, None, stream)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(args.steps):
        L.fps_prefill(shape, q, P, qbuf, qc, None, stream)
    e1.record(stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / args.steps
    flops = float(b.qbufs) * P * prefill_flops_per_row(b.d, b.n_beacon)
    q_bytes = float(b.qbufs) * P * b.d * 2
    ach = flops / (ms * 1e-3) / 1e12
    out = {
        "metric": "prefill initialisations/s (FPS of every query head's prompt queries to its beacons)",
        "value": 1000.0 / ms, "unit": "prefill initialisations/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": ms, "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "f32", "data": "synthetic",
        "config": {"workload": f"{pc.name}: {b.n_layers} layers x batch {b.batch} x {b.hq} query heads "
                               f"({b.qbufs} buffers), {P} prompt queries each, head_dim {b.d}, "
                               f"{b.n_beacon} beacons kept", "buffers": b.qbufs, "n_prompt": P},
        "roofline": {"bound": "alu", "kernel": "prefill_kernel", "achieved": ach, "peak": FP32_VALU_PEAK_TFS,
                     "unit": "TFLOP/s", "frac": ach / FP32_VALU_PEAK_TFS, "traffic": None,
                     "alg_flops_per_launch": flops},
        "hbm": {"query_bytes": q_bytes, "achieved_GBs": q_bytes / (ms * 1e-3) / 1e9,
                "frac": q_bytes / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS},
        "prompt_rows_per_s": float(b.qbufs) * P / (ms * 1e-3),
    }
    if not args.no_cpu_baseline:
        print("# cpu baseline (oracle)", file=sys.stderr, flush=True)
        out["cpu_baseline"] = prefill_cpu_baseline(pc, q, args.cpu_seconds)
    print(json.dumps(out), flush=True)
    return 0


def decode_cpu_baseline(run, n_len: int, target_s: float = 10.0) -> dict:
    """The CPU oracle's decode attention (as it stands) over n_len cached rows for one decode step, on a
    bounded sample of units (at most about 2 GB of their keys and values); the oracle's call is one thread,
    run on slices of the sample in parallel.  Scaled to tokens/s of the attention for the whole batch."""
    import oracle as O
    dc, b = run.dc, run.dc.base
    threads = O.default_threads()
    U, G, d = b.units, b.G, b.d
    K, V = run.K.reshape(U, dc.cap, d)[:, :n_len], run.V.reshape(U, dc.cap, d)[:, :n_len]
    blk = run.gen.block(1, run.pool)
    q, pos = blk["q_new"][0].reshape(U, G, d), blk["pos"][0]
    oc = O.OracleCfg(hq=b.hq, hkv=b.hkv, d=d, cap=n_len, budget=b.budget, n_prefix=b.n_prefix,
                     n_recent_kv=b.n_recent_kv, n_beacon=b.n_beacon, n_recent_q=b.n_recent_q, theta=b.theta,
                     qcap=b.qcap, n_layers=b.n_layers, batch=b.batch)

    def one(ns):
        ut = torch.from_numpy(_spread(ns, U)).to(K.device)
        Kh, Vh = synth.to_u16(K.index_select(0, ut)), synth.to_u16(V.index_select(0, ut))
        qh = synth.to_u16(q.index_select(0, ut))
        ph = np.ascontiguousarray(pos.index_select(0, (ut // b.hkv) % b.batch).cpu().numpy().astype(np.int32))
        t0 = time.perf_counter()
        _in_threads(lambda lo, hi: O.decode_attention(oc, Kh[lo:hi], Vh[lo:hi], qh[lo:hi], ph[lo:hi], n_len),
                    len(ut), threads)
        dt = time.perf_counter() - t0
        return len(ut), dt

    n_max = min(U, max(threads, int(2e9 // (n_len * d * 4))))
    ns, dt = _grow_sample(one, threads, n_max, target_s)
    return {"value": b.batch / (dt * U / ns), "unit": "tokens/s", "cores": threads, "kind": "oracle",
            "sample": f"attention only: {ns} of {U} units over {n_len} cached rows, one decode step, "
                      f"{dt:.1f} s wall on {threads} threads; scaled to the whole batch"}


def decode_bench(args) -> int:
    """The synthetic decode-attention loop: tokens/s of the attention side of decoding, full cache against
    BeaconKV (the framing of the pages' Table 4), and the attention kernel's HBM roofline."""
    from long_reasoning_decode_amd.decode import DECODE_CONFIGS, DecodeRun, cache_bytes, mean_rows
    torch.cuda.set_device(0)
    L.load()
    lines = []
    for name in args.decode_configs.split(","):
        dc = DECODE_CONFIGS[name]
        b = dc.base
        print(f"# decode {dc.name}: batch {b.batch}, cache {dc.n0} rows of {dc.cap}, {dc.steps} steps",
              file=sys.stderr, flush=True)
        torch.cuda.reset_peak_memory_stats()
        run = DecodeRun(dc)
        r = run.run()
        rows = r["rows"] / dc.steps
        att_ms = run.time_attention(int(round(rows)))
        att_bytes = cache_bytes(dc, int(round(rows)))
        ach = att_bytes / (att_ms * 1e-3) / 1e9
        ms = r["gpu_ms"] / dc.steps
        lines.append({
            "metric": "decode tokens/s, attention side (append + attention over the cache + eviction manager; "
                      "no weights)",
            "value": b.batch / (ms * 1e-3), "unit": "tokens/s", "n_gpus": 1, "steps": dc.steps, "warmup": 0,
            "ms_per_step": ms, "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
            "data": "synthetic",
            "config": {"workload": f"{dc.name}: {b.n_layers} layers x batch {b.batch} x {b.hkv} KV heads "
                                   f"({b.units} units), {b.hq} query heads, head_dim {b.d}, "
                                   + (f"budget {b.budget} (cache {b.budget}..{b.cap} rows), evict every "
                                      f"{b.n_new} steps" if dc.mode == "beacon" else
                                      f"full cache, {dc.n0}..{dc.n0 + dc.steps} rows (the middle of a "
                                      f"{dc.gen_len}-token generation)"),
                       "mode": dc.mode, "mean_rows": rows, "expected_mean_rows": mean_rows(dc),
                       "evictions": r["evictions"]},
            "roofline": {"bound": "hbm", "kernel": "attn_kernel", "achieved": ach, "peak": HBM_PEAK_GBS,
                         "unit": "GB/s", "frac": ach / HBM_PEAK_GBS,
                         "traffic": stored_traffic("attn_kernel", os.path.join(HERE, "profiles",
                                                                               f"hbm_traffic_{dc.name}.txt")),
                         "alg_bytes_per_launch": att_bytes, "attention_ms": att_ms},
            "cache_bytes_peak": cache_bytes(dc, dc.cap),
            "state_bytes": run.state_bytes(), "peak_allocated_bytes": torch.cuda.max_memory_allocated(),
        })
        if not args.no_cpu_baseline:
            print("# cpu baseline (oracle)", file=sys.stderr, flush=True)
            lines[-1]["cpu_baseline"] = decode_cpu_baseline(run, int(round(rows)), args.cpu_seconds)
        print(json.dumps(lines[-1]), flush=True)
        del run
        torch.cuda.empty_cache()
    if args.copy_calibration_mib > 0:   # a copy of known size for counter passes (see the eviction bench)
        src = torch.empty(args.copy_calibration_mib << 20, dtype=torch.uint8, device="cuda").fill_(1)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
    return 0


def main() -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--config", default=QWEN3_4B.name, choices=sorted(EVICT_CONFIGS))
    ap.add_argument("--timing", default="pristine", choices=["pristine", "back-to-back"],
                    help="which timing gives value and roofline: pristine (each step on the original cache, the "
                         "MALL flushed before it) or back-to-back (steps in place on the cache the previous one "
                         "left); both are measured and reported.  With --fps-round: pristine (a 512 MB read before "
                         "each round) or back-to-back rounds, only the one asked for")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    ap.add_argument("--copy-calibration-mib", type=int, default=0,
                    help="after the run, copy this many MiB device-to-device once (a plain copy kernel of "
                         "known size, for scaling hardware byte counters)")
    ap.add_argument("--stream", action="store_true",
                    help="instead of the eviction-step benchmark, run the streaming decode simulation "
                         "(bkv_decode_step every step, bkv_evict when the cache is full) and print its own line")
    ap.add_argument("--stream-config", default=STREAM.name, choices=sorted(STREAM_CONFIGS))
    ap.add_argument("--stream-steps", type=int, default=0, help="decode steps (default: the config's)")
    ap.add_argument("--fps-round", action="store_true",
                    help="time only the FPS sampling round of every buffer at --stream-config's shape")
    ap.add_argument("--prefill", action="store_true",
                    help="instead of the eviction-step benchmark, time the prefill initialisation of every query "
                         "buffer (bkv_fps_prefill) and print its own line")
    ap.add_argument("--prefill-config", default=PREFILL.name, choices=sorted(PREFILL_CONFIGS))
    ap.add_argument("--decode", action="store_true",
                    help="instead of the eviction-step benchmark, run the synthetic decode-attention loop (full "
                         "cache and BeaconKV) and print one line per config")
    ap.add_argument("--decode-configs", default="decode-qwen3-4b-full,decode-qwen3-4b-beacon")
    ap.add_argument("--summarize-counters", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"),
                    help="no benchmark: print per-kernel HBM bytes from two rocprofv3 --pmc runs of this script "
                         "(FETCH_SIZE, then WRITE_SIZE, --output-format csv) made with --copy-calibration-mib")
    args = ap.parse_args()
    if args.summarize_counters:
        if args.copy_calibration_mib <= 0:
            ap.error("--summarize-counters needs the --copy-calibration-mib the runs used")
        print(summarize_counters(*args.summarize_counters, args.copy_calibration_mib << 20), end="")
        return 0
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py: runs on one GPU only; every (layer, batch, KV head) unit is independent, so "
              "a multi-GPU step would shard units by batch or KV head with no exchange; --gpus must be 1",
              file=sys.stderr)
        return 2
    if not torch.cuda.is_available():
        print("bench.py: no GPU visible", file=sys.stderr)
        return 2
    if args.stream:
        return stream_bench(args)
    if args.fps_round:
        return fps_round_main(args)
    if args.prefill:
        return prefill_bench(args)
    if args.decode:
        return decode_bench(args)
    cfg = EVICT_CONFIGS[args.config]
    torch.cuda.set_device(0)
    L.load()
    N = cfg.n_len
    print(f"# generating {cfg.name}: {cfg.units} units, N={N}", file=sys.stderr, flush=True)
    inp = synth.make_evict_inputs(cfg, device="cuda")
    rope = torch.from_numpy(L.rope_table(cfg.theta, cfg.d, 0, cfg.rope_rows)).cuda()
    shape = L.shape_of(cfg)
    K, V, qbuf, qcount = inp["K"].clone(), inp["V"].clone(), inp["qbuf"].clone(), inp["qcount"].clone()
    stream = torch.cuda.current_stream()
    total_steps = args.warmup + args.steps
    idx_steps = [torch.empty((cfg.units, cfg.budget), dtype=torch.int32, device="cuda") for _ in range(total_steps)]

    def step(i):
        L.evict(shape, K, V, N, qbuf, qcount, inp["q_recent"], inp["pos_recent"], inp["t"], rope,
                idx_out=idx_steps[i], stream=stream)

    # back to back: the steps run in place, each on the cache the previous one left
    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    print(f"# timing {args.steps} steps back to back", file=sys.stderr, flush=True)
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    ev0.record(stream)
    for i in range(args.warmup, total_steps):
        step(i)
    ev1.record(stream)
    torch.cuda.synchronize()
    wall_b2b = time.perf_counter() - t0
    ms_b2b = ev0.elapsed_time(ev1) / args.steps
    qc0 = np.full((cfg.units, cfg.G), cfg.n_beacon, np.int64)   # qcount is n_beacon before every step
    ab_b2b = [alg_bytes(cfg, qc0, idx_steps[i].cpu().numpy(), N) for i in range(args.warmup, total_steps)]

    # pristine: before each step (untimed) the original cache and buffers are restored from their device
    # copies and a 512 MB scratch buffer is read, which evicts the keys from the 256 MB MALL and leaves it
    # holding clean lines (no write-back of the restore's writes falls into the timed step); each step is
    # timed alone, between two synchronisations
    print(f"# timing {args.steps} pristine steps", file=sys.stderr, flush=True)
    scratch = torch.ones(512 << 18, dtype=torch.int32, device="cuda")
    flush_sum = torch.zeros((), dtype=torch.int64, device="cuda")
    ms_pr = []
    t_pr = 0.0
    for i in range(total_steps):
        K.copy_(inp["K"])
        V.copy_(inp["V"])
        qbuf.copy_(inp["qbuf"])
        qcount.copy_(inp["qcount"])
        flush_sum.copy_(scratch.sum(dtype=torch.int64))   # reads all 512 MB
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        t1 = time.perf_counter()
        torch.cuda._sleep(1 << 20)   # the GPU waits here while the host enqueues the step, so no gap is timed
        e0.record(stream)
        step(i)
        e1.record(stream)
        torch.cuda.synchronize()
        if i >= args.warmup:
            t_pr += time.perf_counter() - t1
            ms_pr.append(e0.elapsed_time(e1))
    assert int(flush_sum) == scratch.numel()
    del scratch
    ab_pr = alg_bytes(cfg, inp["qcount"].reshape(cfg.units, cfg.G).cpu().numpy(),
                      idx_steps[total_steps - 1].cpu().numpy(), N)
    ms_pristine = float(np.mean(ms_pr))

    pristine = args.timing == "pristine"
    ms_step = ms_pristine if pristine else ms_b2b
    wall = t_pr if pristine else wall_b2b
    ab = [ab_pr] if pristine else ab_b2b
    step_bytes = float(np.mean([a["total"] for a in ab]))
    compact_bytes = float(np.mean([a["compact"] for a in ab]))

    # per-kernel breakdown.  bkv_evict is two launches: the fused per-unit kernel (scores, keep set,
    # compaction) and the buffer merge.  The merge alone is timed back to back over the same number of
    # launches; the fused kernel's duration is the timed step's minus the merge's.
    print("# per-kernel breakdown", file=sys.stderr, flush=True)
    m0, m1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    m0.record(stream)
    for s in range(args.steps):
        L.fps_merge(shape, qbuf, qcount, inp["q_recent"], None, stream)
    m1.record(stream)
    torch.cuda.synchronize()
    merge_ms = m0.elapsed_time(m1) / args.steps
    kern_ms = {"evict_kernel": ms_step - merge_ms, "fps_merge": merge_ms}
    buf_bytes = float(np.mean([x["buffers"] for x in ab]))
    evict_bytes = step_bytes - buf_bytes
    evict_ach = evict_bytes / (kern_ms["evict_kernel"] * 1e-3) / 1e9
    strict_bytes = float(np.mean([a["total_strict"] for a in ab])) - buf_bytes
    strict_ach = strict_bytes / (kern_ms["evict_kernel"] * 1e-3) / 1e9
    idx_b = torch.empty((cfg.units, cfg.budget), dtype=torch.int32, device="cuda")

    # the separate entry points, for reference
    scores = torch.empty((cfg.units, N), dtype=torch.float32, device="cuda")
    sep = {"score": [], "select": [], "compact": []}
    for s in range(min(args.steps, 5)):
        e = [torch.cuda.Event(enable_timing=True) for _ in range(4)]
        e[0].record(stream)
        L.score(shape, K, N, qbuf, qcount, inp["q_recent"], inp["pos_recent"], inp["t"], rope, scores,
                stream=stream)
        e[1].record(stream)
        L.select(shape, scores, N, idx_b, stream)
        e[2].record(stream)
        L.compact(shape, K, V, N, idx_b, stream)
        e[3].record(stream)
        torch.cuda.synchronize()
        for i, n in enumerate(("score", "select", "compact")):
            sep[n].append(e[i].elapsed_time(e[i + 1]))
    sep_ms = {n: float(np.mean(v)) for n, v in sep.items()}

    out = {
        "metric": METRIC,
        "value": 1000.0 / ms_step,
        "unit": "eviction steps/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": f"{cfg.name} eviction step: {cfg.n_layers} layers x batch {cfg.batch} x "
                               f"{cfg.hkv} KV heads ({cfg.units} units), {cfg.hq} query heads, head_dim {cfg.d}, "
                               f"cache {N} -> budget {cfg.budget}, prefix {cfg.n_prefix}, recent window "
                               f"{cfg.n_recent_kv}, {cfg.n_beacon} beacons + {cfg.n_recent_q} recent queries",
                   "units": cfg.units, "n_len": N, "budget": cfg.budget},
        "roofline": {"bound": "hbm", "kernel": "evict_kernel", "achieved": evict_ach, "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": evict_ach / HBM_PEAK_GBS,
                     "traffic": stored_traffic("evict_kernel", traffic_file(cfg.name)),
                     "alg_bytes_per_launch": evict_bytes,
                     "strict": {"alg_bytes_per_launch": strict_bytes, "achieved": strict_ach,
                                "frac": strict_ach / HBM_PEAK_GBS,
                                "counts": "every key read once: moved key rows written, moved value rows read "
                                          "and written"}},
        "step_hbm": {"alg_bytes": step_bytes, "achieved_GBs": step_bytes / (ms_step * 1e-3) / 1e9,
                     "frac": step_bytes / (ms_step * 1e-3) / 1e9 / HBM_PEAK_GBS,
                     "compact_alg_bytes": compact_bytes,
                     "strict_frac": (strict_bytes + buf_bytes) / (ms_step * 1e-3) / 1e9 / HBM_PEAK_GBS},
        "timing": args.timing,
        "pristine": {"ms_mean": ms_pristine, "ms_median": float(np.median(ms_pr)), "ms_min": float(min(ms_pr)),
                     "steps_per_s": 1000.0 / ms_pristine, "moved_rows_per_unit": ab_pr["moved_rows"] / cfg.units,
                     "step_frac": ab_pr["total"] / (ms_pristine * 1e-3) / 1e9 / HBM_PEAK_GBS},
        "back_to_back": {"ms_per_step": ms_b2b, "steps_per_s": 1000.0 / ms_b2b,
                         "moved_rows_per_unit": float(np.mean([a["moved_rows"] for a in ab_b2b])) / cfg.units,
                         "step_frac": float(np.mean([a["total"] for a in ab_b2b])) / (ms_b2b * 1e-3) / 1e9
                         / HBM_PEAK_GBS},
        "kernels_ms": kern_ms,
        "separate_calls_ms": sep_ms,
        "mfma_qkt": qkt_mfma(cfg, N, kern_ms["evict_kernel"], sep_ms["score"]),
        "wall_s": wall,
    }
    if args.copy_calibration_mib <= 0:   # (a counter pass takes its calibration from the longest copy)
        out["copy_reference"] = copy_reference(stream)
    if args.copy_calibration_mib > 0:
        # one device-to-device copy of known size, larger than any other copy in the run, so that a
        # counter pass can find it as the longest copy dispatch
        src = torch.empty(args.copy_calibration_mib << 20, dtype=torch.uint8, device="cuda").fill_(1)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        out["copy_calibration_bytes"] = src.numel()
        del src, dst
    if not args.no_cpu_baseline:
        print("# cpu baseline (oracle)", file=sys.stderr, flush=True)
        out["cpu_baseline"] = cpu_baseline(cfg, inp, args.cpu_seconds)
    print(json.dumps(out), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
