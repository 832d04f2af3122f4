"""Calls on several streams at once.  The library keeps nothing between calls
(no scratch memory, no shared buffers; each call touches only the memory it
is given), so independent chains of calls enqueued on three non-default
streams and in flight together give bit for bit what the same chains give one
after another on one stream."""
from __future__ import annotations

import pytest
import torch

from long_reasoning_decode_amd import lib as L
from long_reasoning_decode_amd import synth
from long_reasoning_decode_amd.configs import QWEN3_4B, R1_QWEN_7B, TINY

import _helpers as H

pytestmark = pytest.mark.gpu

CFGS = [QWEN3_4B.scaled(n_layers=2, batch=3), R1_QWEN_7B.scaled(n_layers=1, batch=2),
        TINY.scaled(name="tiny-mean-random", batch=3, pool="mean", beacon="random")]


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    L.load()
    yield


def _prepare(cfg, k: int) -> dict:
    """One chain's inputs and output buffers, all allocated on the default stream."""
    inp = synth.make_evict_inputs(cfg, device="cuda", seed=cfg.seed + k)
    inp["qcount"].view(-1)[::4] = 9
    upd = synth.make_query_buffers(cfg, device="cuda", seed=cfg.seed + k)
    P = 700
    return {"inp": inp, "upd": upd, "rope": H.rope_dev(cfg), "P": P,
            "prompt": synth.make_prompt_queries(cfg, P, device="cuda", seed=cfg.seed + k),
            "idx": torch.full((cfg.units, cfg.budget), -7, dtype=torch.int32, device="cuda"),
            "scores": torch.full((cfg.units, cfg.n_len), -7.0, dtype=torch.float32, device="cuda"),
            "msel": torch.full((cfg.qbufs, cfg.n_beacon), -7, dtype=torch.int32, device="cuda"),
            "usel": torch.full((cfg.qbufs, cfg.n_beacon), -7, dtype=torch.int32, device="cuda"),
            "pbuf": torch.zeros((cfg.qbufs, cfg.qcap, cfg.d), dtype=torch.bfloat16, device="cuda"),
            "pcount": torch.zeros((cfg.qbufs,), dtype=torch.int32, device="cuda"),
            "att": torch.full((cfg.qbufs, cfg.d), float("nan"), dtype=torch.float32, device="cuda"),
            "q1": inp["q_recent"][..., 0, :].contiguous()}


def _chain(cfg, w: dict, stream) -> None:
    """Eviction, then decode attention over the compacted cache, a buffer update and a prompt sampling.  Only
    library calls: anything torch enqueued here would go to the current stream, not to `stream`."""
    inp, upd = w["inp"], w["upd"]
    shape = L.shape_of(cfg)
    L.evict(shape, inp["K"], inp["V"], cfg.n_len, inp["qbuf"], inp["qcount"], inp["q_recent"], inp["pos_recent"],
            inp["t"], w["rope"], idx_out=w["idx"], scores_out=w["scores"], fps_sel_out=w["msel"], stream=stream)
    L.decode_attention(shape, inp["K"], inp["V"], cfg.budget, w["q1"], inp["t"], w["rope"], w["att"], stream=stream)
    L.fps_update(shape, upd["qbuf"], upd["qcount"], upd["q_new"], w["usel"], stream=stream)
    L.fps_prefill(shape, w["prompt"], w["P"], w["pbuf"], w["pcount"], stream=stream)


def _flat(w: dict) -> dict:
    out = {k: v for k, v in w.items() if isinstance(v, torch.Tensor)}
    out.update({"inp." + k: v for k, v in w["inp"].items()})
    out.update({"upd." + k: v for k, v in w["upd"].items()})
    return out


def test_three_streams_match_one():
    seq = [_prepare(c, 1) for c in CFGS]
    par = [_prepare(c, 1) for c in CFGS]
    torch.cuda.synchronize()
    for c, w in zip(CFGS, seq):
        _chain(c, w, torch.cuda.current_stream())
    torch.cuda.synchronize()
    main = torch.cuda.current_stream()
    streams = [torch.cuda.Stream() for _ in CFGS]   # default priority
    for s in streams:
        s.wait_stream(main)
    for c, w, s in zip(CFGS, par, streams):
        _chain(c, w, s)
    for s in streams:
        main.wait_stream(s)
    torch.cuda.synchronize()
    for c, a, b in zip(CFGS, seq, par):
        fa, fb = _flat(a), _flat(b)
        for k in fa:   # bit patterns (NaN-safe)
            assert torch.equal(fa[k].contiguous().view(torch.uint8), fb[k].contiguous().view(torch.uint8)), \
                f"{c.name}: {k}"
