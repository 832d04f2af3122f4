"""Host-side logic of bench.py and decode.py (no GPU): the algorithmic byte and flop counts the roofline
fields are built on, the committed counter summary's lookup and its source hash, and the refusal of more
than one GPU."""
from __future__ import annotations

import os
import shutil
import subprocess
import sys
from dataclasses import replace

import numpy as np
import pytest

import bench
from long_reasoning_decode_amd import decode
from long_reasoning_decode_amd.configs import QWEN3_4B, TINY

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_alg_bytes_hand_example():
    cfg = TINY.scaled(n_layers=1, batch=1, hq=4, hkv=2, d=64, budget=8, n_prefix=2, n_recent_kv=2)
    assert (cfg.units, cfg.G, cfg.qbufs) == (2, 2, 4)
    idx = np.array([[0, 1, 2, 3, 4, 5, 6, 7],      # nothing moves
                    [0, 1, 2, 4, 5, 6, 8, 9]])     # slots 3..7 take rows 4, 5, 6, 8, 9: five moves
    qcount = np.array([[16, 3], [0, 20]])         # beacons min(qcount, 16): 16, 3, 0, 16
    a = bench.alg_bytes(cfg, qcount, idx, n_len=10)
    row = 64 * 2
    assert a["moved_rows"] == 5
    assert a["k_read"] == 2 * 10 * row
    assert a["q_read"] == (16 + 3 + 0 + 16 + 4 * cfg.n_recent_q) * row
    assert a["compact"] == 4 * 5 * row              # K and V, each read and written
    assert a["buffers"] == 4 * cfg.n_beacon * row
    assert a["total"] == a["k_read"] + a["q_read"] + a["compact"] + a["buffers"]
    # every key read once: the moved key rows are not read a second time
    assert a["total_strict"] == a["k_read"] + a["q_read"] + 3 * 5 * row + a["buffers"]


def test_qkt_flops_match_the_counted_mfmas():
    """At the qwen3-4b step the issued flops are the 20,054,016 bf16 MFMA 32x32x16 instructions that the
    counters record per eviction step (profiles/mfma_qwen3-4b.md), 32,768 flops each."""
    m = bench.qkt_mfma(QWEN3_4B, 2176, evict_ms=1.0, score_ms=1.0)
    assert m["issued_flops"] == 20_054_016 * 32 * 32 * 16 * 2
    assert m["alg_flops"] == 2 * QWEN3_4B.G * 32 * 2176 * 128 * QWEN3_4B.units
    assert m["evict_kernel"]["issued_TFs"] == pytest.approx(m["issued_flops"] / 1e9)


def test_prefill_flops_per_row():
    # norm (d fma) + unit row (d mul) + column sum (d add) + mean cosine (d fma) + (m - 1) cosines (d fma each)
    assert bench.prefill_flops_per_row(128, 16) == 128 * (2 + 1 + 1 + 2 + 2 * 15)


def _tree_copy(tmp_path):
    dst = tmp_path / "r"
    shutil.copytree(os.path.join(ROOT, "long_reasoning_decode_amd", "csrc"),
                    dst / "long_reasoning_decode_amd" / "csrc")
    shutil.copytree(os.path.join(ROOT, "include"), dst / "include")
    shutil.copy(os.path.join(ROOT, "long_reasoning_decode_amd", "build.py"), dst / "long_reasoning_decode_amd")
    return dst


def test_source_hash_follows_includes(tmp_path, monkeypatch):
    """The hash that validates a stored traffic figure changes with any header the kernel includes,
    directly or not, and with the compile flags; it ignores files the kernel does not include."""
    dst = _tree_copy(tmp_path)
    monkeypatch.setattr(bench, "HERE", str(dst))
    h0 = bench.kernel_sources_sha256("evict_kernel")
    assert h0 == bench.kernel_sources_sha256("evict_kernel")
    (dst / "long_reasoning_decode_amd" / "csrc" / "bkv_attention.hip").write_text("// not included\n")
    assert bench.kernel_sources_sha256("evict_kernel") == h0
    for rel in ("long_reasoning_decode_amd/csrc/bkv_device.hpp", "include/bkv.h"):
        p = dst / rel
        text = p.read_text()
        p.write_text(text + "\n// changed\n")
        assert bench.kernel_sources_sha256("evict_kernel") != h0, rel
        p.write_text(text)
    assert bench.kernel_sources_sha256("evict_kernel") == h0
    from long_reasoning_decode_amd import build as lib_build
    flags = lib_build.device_flags()
    monkeypatch.setattr(lib_build, "device_flags", lambda arch="gfx950": flags + ["-O2"])
    assert bench.kernel_sources_sha256("evict_kernel") != h0


def test_stored_traffic_lookup(tmp_path, monkeypatch):
    f = tmp_path / "traffic.txt"
    h = bench.kernel_sources_sha256("evict_kernel")
    f.write_text("# header\n"
                 f"kernel=evict_kernel dispatches=3,3 bytes_per_dispatch=1.5e+10 sources_sha256={h}\n"
                 "kernel=score_kernel dispatches=3,3 bytes_per_dispatch=5e+09 sources_sha256=0000\n")
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(f))
    assert bench.stored_traffic("evict_kernel") == 1.5e10
    assert bench.stored_traffic("score_kernel") is None      # sources changed since
    assert bench.stored_traffic("select_kernel") is None     # never measured
    assert bench.stored_traffic("evict_kernel", str(tmp_path / "none.txt")) is None
    assert bench.stored_traffic("evict_kernel", str(f)) == 1.5e10


@pytest.mark.parametrize("dc", list(decode.DECODE_CONFIGS.values()), ids=lambda c: c.name)
def test_decode_mean_rows_by_stepping(dc):
    """mean_rows against the decode loop's own cache-length rule stepped one token at a time."""
    b = dc.base
    L, total = dc.n0, 0
    for _ in range(dc.steps):
        L += 1              # the new token's row
        total += L
        if dc.mode == "beacon" and L == dc.cap:
            L = b.budget
    assert decode.mean_rows(dc) == pytest.approx(total / dc.steps)


def test_bench_refuses_more_than_one_gpu():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, cwd=ROOT, timeout=300)
    assert r.returncode == 2
    assert "one GPU" in r.stderr and r.stdout == ""


# ---------------------------------------------------------------------------
# The CPU-baseline legs of the stream, FPS-round and decode benches, on CPU tensors standing in for the GPU
# state (the functions only read the state and draw inputs; the oracle does the timed work).

class _State:
    pass


def _bf16(g, *shape):
    import torch
    return torch.randn(*shape, generator=g).to(torch.bfloat16)


def test_stream_cpu_baseline_replays_one_cycle():
    import torch
    from long_reasoning_decode_amd import synth
    from long_reasoning_decode_amd.configs import TINY_STREAM
    b = TINY_STREAM.base
    g = torch.Generator().manual_seed(5)
    run = _State()
    run.base, run.L = b, b.budget
    run.K = _bf16(g, b.n_layers, b.batch, b.hkv, b.cap, b.d)
    run.V = _bf16(g, b.n_layers, b.batch, b.hkv, b.cap, b.d)
    run.qbuf = _bf16(g, b.n_layers, b.batch, b.hq, b.qcap, b.d)
    run.qcount = torch.full((b.n_layers, b.batch, b.hq), b.n_beacon, dtype=torch.int32)
    run.q_recent = _bf16(g, b.n_layers, b.batch, b.hq, b.n_recent_q, b.d)
    run.pos_recent = torch.arange(b.batch * b.n_recent_q, dtype=torch.int32).reshape(b.batch, b.n_recent_q)
    run.gen = synth.StreamGen(TINY_STREAM, "cpu")
    run.pool = run.gen.alloc(b.n_new)
    r = bench.stream_cpu_baseline(run, target_s=0.0)   # one sample; the function asserts one eviction
    assert r["kind"] == "oracle" and r["unit"] == "tokens/s" and r["value"] > 0
    assert f"of {b.units} units" in r["sample"] and f"{b.n_new} decode steps" in r["sample"]


def test_fps_round_cpu_baseline_samples_every_buffer_once():
    from long_reasoning_decode_amd import synth
    b = TINY.scaled(n_layers=2, batch=3)
    q = synth.make_query_buffers(b, device="cpu")
    r = bench.fps_round_cpu_baseline(b, q, target_s=0.0)
    assert r["unit"] == "rounds/s" and r["value"] > 0 and f"of {b.qbufs} buffers" in r["sample"]


def test_decode_cpu_baseline_on_a_sample():
    import torch
    from long_reasoning_decode_amd import synth
    from long_reasoning_decode_amd.configs import StreamConfig
    dc = decode.DecodeConfig("decode-tiny-full", replace(TINY, batch=2), "full", 40, gen_len=200)
    b = dc.base
    g = torch.Generator().manual_seed(6)
    run = _State()
    run.dc = dc
    run.K = _bf16(g, b.n_layers, b.batch, b.hkv, dc.cap, b.d)
    run.V = _bf16(g, b.n_layers, b.batch, b.hkv, dc.cap, b.d)
    run.gen = synth.StreamGen(StreamConfig(name=dc.name, base=b, steps=dc.steps, drift_every=2048, p0_max=64), "cpu")
    run.pool = run.gen.alloc(1)
    r = bench.decode_cpu_baseline(run, dc.cap - 3, target_s=0.0)
    assert r["unit"] == "tokens/s" and r["value"] > 0 and f"over {dc.cap - 3} cached rows" in r["sample"]


def test_prefill_cpu_baseline_on_a_sample():
    from long_reasoning_decode_amd import synth
    from long_reasoning_decode_amd.configs import PrefillConfig
    pc = PrefillConfig("prefill-tiny", TINY.scaled(n_layers=2, batch=2), 40)
    q = synth.make_prompt_queries(pc.base, pc.n_prompt, device="cpu")
    r = bench.prefill_cpu_baseline(pc, q, target_s=0.0)
    assert r["unit"] == "prefill initialisations/s" and r["value"] > 0 and f"of {pc.base.qbufs} buffers" in r["sample"]


def test_eviction_cpu_baseline_sample_stays_within_the_units():
    """A workload with fewer units than host threads: the sample is every unit, never an index past them."""
    from long_reasoning_decode_amd import synth
    inp = synth.make_evict_inputs(TINY, device="cpu")
    r = bench.cpu_baseline(TINY, inp, target_s=0.0)
    assert r["value"] > 0 and f"{TINY.units} of {TINY.units} units" in r["sample"]
    with pytest.raises(IndexError):
        synth.oracle_views(TINY, inp, [0, TINY.units])
