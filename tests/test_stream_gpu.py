"""Streaming decode on the GPU (bkv_decode_step every step, bkv_evict when the
cache is full) against the oracle's replay of the same per-step inputs."""
from __future__ import annotations

from dataclasses import replace

import pytest
import torch

from long_reasoning_decode_amd import lib as L

from long_reasoning_decode_amd.configs import (STREAM, STREAM_NAIVE, STREAM_SOURCES, STREAM_SPLITS, TINY_STREAM,
                                               TINY_STREAM_MEAN, TINY_STREAM_NAIVE, TINY_STREAM_SOURCES,
                                               TINY_STREAM_SPLITS)
from long_reasoning_decode_amd.stream import StreamRun

from _stream_helpers import check_run as _check

pytestmark = pytest.mark.gpu


def test_stream_tiny_all_units():
    scfg = TINY_STREAM
    units = range(scfg.base.units)
    run = StreamRun(scfg, record_units=units, block=48)
    r = run.run()
    assert r["evictions"] == scfg.evictions() == 14
    res = _check(scfg, run, units, "stream-tiny")
    assert len(res["diverged"]) <= 1


def test_stream_tiny_resumes_across_calls():
    """Running the steps in several calls (blocks ending mid-cycle) gives the
    same stream as one call."""
    scfg = TINY_STREAM
    units = range(scfg.base.units)
    run = StreamRun(scfg, record_units=units, block=37)
    for n in (100, 61, 200, 239):
        run.run(n)
    assert run.steps_done == scfg.steps
    _check(scfg, run, units, "stream-tiny resumed")


@pytest.mark.parametrize("scfg", TINY_STREAM_SPLITS, ids=lambda c: c.name)
def test_stream_tiny_recent_beacon_splits(scfg):
    """The recent/beacon splits of the 32 observation queries; with 1 recent query a sampling round follows
    every collection step, with none (all recent) the buffers keep no beacons."""
    units = range(scfg.base.units)
    run = StreamRun(scfg, record_units=units, block=64)
    run.run()
    if scfg.base.n_recent_q == 1:
        assert run.fps_rounds_per_buffer() > 0.8 * scfg.steps   # nearly every step samples
    _check(scfg, run, units, scfg.name)


@pytest.mark.parametrize("scfg", TINY_STREAM_SOURCES, ids=lambda c: c.name)
def test_stream_tiny_beacon_sources(scfg):
    """The whole cycle with the initial queries or a random sample of the history as beacons."""
    units = range(scfg.base.units)
    run = StreamRun(scfg, record_units=units, block=64)
    run.run()
    _check(scfg, run, units, scfg.name)


def test_stream_tiny_mean_pooling():
    """The whole cycle with mean pooling of the weights."""
    scfg = TINY_STREAM_MEAN
    units = range(scfg.base.units)
    run = StreamRun(scfg, record_units=units, block=64)
    run.run()
    _check(scfg, run, units, "stream-tiny mean")


def test_stream_tiny_naive_history():
    """Naive full-history beacons: every query of every head kept, the beacons sampled from the whole history
    at each eviction, against the oracle's replay (which samples them with the prefill FPS)."""
    scfg = TINY_STREAM_NAIVE
    units = range(scfg.base.units)
    run = StreamRun(scfg, record_units=units, block=64)
    run.run()
    assert run.h_rows == scfg.steps and int(run.hcount.min()) == int(run.hcount.max()) == scfg.steps
    _check(scfg, run, units, "stream-tiny naive")


@pytest.mark.parametrize("n_new", [40, 23])
def test_stream_tiny_collection_not_a_multiple(n_new):
    """Cycles whose collection phase (n_new - n_recent_q steps) is not a multiple of n_recent_q: at the freeze
    point the buffers hold more than n_beacon rows and are compressed, so no collected query is dropped; the
    oracle's replay does the same."""
    scfg = replace(TINY_STREAM, name=f"stream-tiny-new{n_new}", steps=500,
                   base=replace(TINY_STREAM.base, n_new=n_new, seed=20261202 + 600 + n_new))
    b = scfg.base
    assert (b.n_new - b.n_recent_q) % b.n_recent_q != 0
    units = range(b.units)
    run = StreamRun(scfg, record_units=units, block=64)
    run.run()
    _check(scfg, run, units, scfg.name)


def test_stream_naive_qwen3_4b_sampled_units():
    """The naive full-history stream at its benchmark shape (Qwen3-4B, batch 16) for the first three
    evictions, checked on units spread over layers, batch elements and KV heads."""
    scfg = STREAM_NAIVE
    b = scfg.base
    steps = b.cap + 2 * b.n_new
    units = [0, b.units - 1, 9 * b.batch * b.hkv + 5 * b.hkv + 2, 31 * b.batch * b.hkv + 12 * b.hkv + 7]
    run = StreamRun(scfg, record_units=units)
    r = run.run(steps)
    assert r["evictions"] == scfg.evictions(steps) == 3
    res = _check(scfg, run, units, "stream-qwen3-4b-naive b16", nthreads=len(units))
    assert len(res["diverged"]) <= 2


def test_stream_checkpoint_resume(tmp_path):
    """Stopping at a step, saving the state to a file and resuming in a fresh stream object gives the
    same stream, bit for bit, as running straight through."""
    scfg = TINY_STREAM
    a = StreamRun(scfg, block=50)
    a.run(600)
    b = StreamRun(scfg, block=50)
    b.run(265)                      # mid-cycle, inside a collection phase
    torch.save(b.state_dict(), tmp_path / "stream.pt")
    c = StreamRun(scfg, block=50)
    c.load_state_dict(torch.load(tmp_path / "stream.pt", weights_only=True))
    c.run(335)
    assert (c.L, c.n_ev, c.steps_done) == (a.L, a.n_ev, a.steps_done)
    for k in a._STATE:
        assert torch.equal(getattr(c, k), getattr(a, k)), k


def test_decode_step_rejects_bad_length():
    scfg = TINY_STREAM
    run = StreamRun(scfg, block=4)
    blk = run.gen.block(1, run.pool)
    for bad in (-1, scfg.base.cap):
        with pytest.raises(L.BkvError) as e:
            L.decode_step(run.shape, run.K, run.V, bad, blk["k_new"][0], blk["v_new"][0], blk["pos"][0], run.qbuf,
                          run.qcount, blk["q_new"][0], run.q_recent, run.pos_recent, run.rope)
        assert e.value.code == -3


def test_stream_full_size_sampled_units():
    """The streaming workload at full size: Qwen3-4B shape, batch 192, 32768
    decode steps (240 evictions), checked on units spread over layers, batch
    elements and KV heads."""
    scfg = STREAM
    b = scfg.base
    units = [0, b.units - 1, 7 * b.batch * b.hkv + 93 * b.hkv + 3, 20 * b.batch * b.hkv + 150 * b.hkv + 6,
             35 * b.batch * b.hkv + 11 * b.hkv + 1, 13 * b.batch * b.hkv + 64 * b.hkv + 4]
    run = StreamRun(scfg, record_units=units)
    prog = lambda r: (r.steps_done % 4096 == 0) and print(f"  step {r.steps_done}, evictions {r.n_ev}", flush=True)
    r = run.run(progress=prog)
    assert r["evictions"] == scfg.evictions() == 240
    res = _check(scfg, run, units, "stream-qwen3-4b b192", nthreads=len(units))
    assert len(res["diverged"]) <= 2


@pytest.mark.parametrize("src", ["initial", "random"])
def test_stream_full_size_beacon_sources(src):
    """Batch 192 with the beacons drawn from the initial queries or by reservoir sampling of the history
    (one offer per buffer and step, the merge offering the cycle's recents): the first three evictions,
    checked on units spread over layers, batch elements and KV heads."""
    scfg = next(c for c in STREAM_SOURCES if c.base.beacon == src)
    b = scfg.base
    steps = b.cap + 2 * b.n_new
    units = [5, b.units - 2, 11 * b.batch * b.hkv + 77 * b.hkv + 1, 27 * b.batch * b.hkv + 140 * b.hkv + 7]
    run = StreamRun(scfg, record_units=units)
    r = run.run(steps)
    assert r["evictions"] == scfg.evictions(steps) == 3
    res = _check(scfg, run, units, f"{scfg.name} b192", nthreads=len(units))
    assert len(res["diverged"]) <= 2


def test_stream_full_size_fps_every_step():
    """Batch 192 with 31 beacons + 1 recent query, so every collection step samples all 221,184 buffers
    (the update kernel's runs of full buffers, two per wave): the first three evictions, checked on units
    spread over layers, batch elements and KV heads."""
    scfg = next(c for c in STREAM_SPLITS if c.name == "stream-qwen3-4b-r1b31")
    b = scfg.base
    steps = b.cap + 2 * b.n_new
    units = [0, b.units - 1, 3 * b.batch * b.hkv + 17 * b.hkv + 5, 30 * b.batch * b.hkv + 191 * b.hkv + 2]
    run = StreamRun(scfg, record_units=units)
    r = run.run(steps)
    assert r["evictions"] == scfg.evictions(steps) == 3
    assert run.fps_rounds_per_buffer(steps) > 2000
    res = _check(scfg, run, units, "stream-qwen3-4b-r1b31 b192", nthreads=len(units))
    assert len(res["diverged"]) <= 2

