"""The library's calls under HIP graph capture.

One eviction cycle of a small stream (the decode steps with their attention, then the eviction) is
captured once and replayed several times, each replay from the same restored state, with eager work
and synchronisations in between; every replay must give the eagerly run cycle's state bit for bit.
The library only enqueues kernels (no allocation, no memset, no host synchronisation), which is what
makes a serving loop able to capture it.
"""
from __future__ import annotations

import pytest
import torch

from long_reasoning_decode_amd import lib as L
from long_reasoning_decode_amd.configs import QWEN3_4B, TINY_STREAM, StreamConfig
from long_reasoning_decode_amd.stream import StreamRun

pytestmark = pytest.mark.gpu

_STATE = ("K", "V", "qbuf", "qcount", "q_recent", "pos_recent")


def _bits(t: torch.Tensor) -> torch.Tensor:
    return t.view(torch.int16) if t.dtype == torch.bfloat16 else t


@pytest.mark.parametrize("scfg", [TINY_STREAM,
                                  StreamConfig(name="stream-qwen3-4b-small", base=QWEN3_4B.scaled(n_layers=2, batch=3),
                                               steps=3000, drift_every=2048, p0_max=4096)],
                         ids=lambda c: c.name)
def test_captured_cycle_replays_match_eager(scfg):
    b = scfg.base
    print(f"graph capture {scfg.name}", flush=True)
    run = StreamRun(scfg)
    run.run(b.cap + 7)                     # past the first eviction, then to the start of a cycle
    run.run(b.cap - run.L)
    assert run.L == b.budget
    n = b.cap - b.budget
    blk = {k: v.clone() for k, v in run.gen.block(n).items()}
    out = torch.zeros(b.qbufs, b.d, dtype=torch.float32, device="cuda")
    idx = torch.full((b.units, b.budget), -7, dtype=torch.int32, device="cuda")
    s0 = {k: getattr(run, k).clone() for k in _STATE}

    def cycle():
        for i in range(n):
            L.decode_step(run.shape, run.K, run.V, b.budget + i, blk["k_new"][i], blk["v_new"][i], blk["pos"][i],
                          run.qbuf, run.qcount, blk["q_new"][i], run.q_recent, run.pos_recent, run.rope)
            L.decode_attention(run.shape, run.K, run.V, b.budget + i + 1, blk["q_new"][i], blk["pos"][i], run.rope, out)
        L.evict(run.shape, run.K, run.V, b.cap, run.qbuf, run.qcount, run.q_recent, run.pos_recent,
                blk["pos"][n - 1], run.rope, idx_out=idx)

    def restore():
        for k in _STATE:
            getattr(run, k).copy_(s0[k])
        out.zero_()
        idx.fill_(-7)

    cycle()                                # eager reference
    torch.cuda.synchronize()
    ref = {k: getattr(run, k).clone() for k in _STATE}
    ref_out, ref_idx = out.clone(), idx.clone()

    restore()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        cycle()                            # captured, not run
    torch.cuda.synchronize()
    for rep in range(3):
        restore()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for k in _STATE:
            assert torch.equal(_bits(getattr(run, k)), _bits(ref[k])), f"replay {rep}: {k} differs"
        assert torch.equal(out, ref_out), f"replay {rep}: attention output differs"
        assert torch.equal(idx, ref_idx), f"replay {rep}: keep sets differ"
        print(f"  replay {rep} matches the eager cycle", flush=True)
