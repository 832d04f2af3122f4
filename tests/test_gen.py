"""The seeded input generator: shapes, determinism and the stated distributions."""
from __future__ import annotations

import math

import torch

from long_reasoning_decode_amd import synth
from long_reasoning_decode_amd.configs import QWEN3_4B, TINY


def test_shapes_and_determinism():
    cfg = TINY
    a = synth.make_evict_inputs(cfg)
    b = synth.make_evict_inputs(cfg)
    assert a["K"].shape == (1, 1, 2, cfg.n_len, 64) and a["K"].dtype == torch.bfloat16
    assert a["qbuf"].shape == (1, 1, 4, cfg.qcap, 64)
    assert a["q_recent"].shape == (1, 1, 4, cfg.n_recent_q, 64)
    assert a["qcount"].dtype == torch.int32 and bool((a["qcount"] == cfg.n_beacon).all())
    for k in a:
        assert torch.equal(a[k], b[k]), k
    c = synth.make_evict_inputs(cfg, seed=cfg.seed + 1)
    assert not torch.equal(a["K"], c["K"])


def test_positions():
    cfg = QWEN3_4B.scaled(n_layers=1, batch=64)
    a = synth.make_evict_inputs(cfg)
    t = a["t"].long()
    assert int(t.min()) >= cfg.t_lo and int(t.max()) <= cfg.t_hi
    pos = a["pos_recent"].long()
    assert torch.equal(pos[:, -1], t)
    assert torch.equal(pos[:, 1:] - pos[:, :-1], torch.ones_like(pos[:, 1:]))
    tiny = synth.make_evict_inputs(TINY)
    assert int(tiny["t"][0]) == 1000


def test_query_mixture_fractions():
    g = torch.Generator().manual_seed(5)
    d = 128
    cen = synth._unit_rows(g, (4, 8), d, "cpu")
    q = synth.query_rows(g, cen, 5000, "clusters8")
    qn = q / q.norm(dim=-1, keepdim=True)
    best = (qn @ cen.transpose(-1, -2)).max(dim=-1).values
    frac = (best > 0.99).float().mean().item()
    assert abs(frac - 0.3) < 0.02
    # cluster rows have norm s * sqrt(d) with s ~ N(1, 0.2)
    norms = q.norm(dim=-1)[best > 0.99] / math.sqrt(d)
    assert abs(norms.mean().item() - 1.0) < 0.02 and abs(norms.std().item() - 0.2) < 0.02
    q3 = synth.query_rows(g, cen[:, :3], 5000, "tight3")
    qn3 = q3 / q3.norm(dim=-1, keepdim=True)
    best3 = (qn3 @ cen[:, :3].transpose(-1, -2)).max(dim=-1).values
    assert abs((best3 > 0.98).float().mean().item() - 0.25) < 0.02


def test_key_outliers():
    g = torch.Generator().manual_seed(6)
    k = synth.key_rows(g, (8,), 4000, 128, "cpu")
    big = (k.norm(dim=-1) > 4 * math.sqrt(128)).float().mean().item()
    assert abs(big - 0.01) < 0.004


def test_oracle_views_unit_major():
    cfg = TINY.scaled(batch=3, n_layers=2)
    a = synth.make_evict_inputs(cfg)
    v = synth.oracle_views(cfg, a, units=[5, 0])
    # unit 5 = (l * batch + b) * Hkv + g with batch 3, Hkv 2: layer 0, batch 2, kv head 1
    assert (v["K"][0] == synth.to_u16(a["K"][0, 2, 1])).all()
    assert (v["qbuf"][0] == synth.to_u16(a["qbuf"][0, 2, 2:4])).all()
    assert int(v["t"][0]) == int(a["t"][2])
    assert (v["K"][1] == synth.to_u16(a["K"][0, 0, 0])).all()


def test_stream_inputs_do_not_depend_on_block_sizes_and_resume():
    """The streaming generator gives the same step sequence however the run is split into blocks, and
    continues exactly from a saved state."""
    from long_reasoning_decode_amd.configs import TINY_STREAM
    whole = synth.StreamGen(TINY_STREAM).block(300)
    g = synth.StreamGen(TINY_STREAM)
    parts = [g.block(n) for n in (7, 30, 13, 50, 200)]
    for k in whole:
        assert torch.equal(whole[k], torch.cat([p[k] for p in parts])), k
    g3 = synth.StreamGen(TINY_STREAM)
    g3.block(37)
    g4 = synth.StreamGen(TINY_STREAM, seed=1)
    g4.load_state_dict(g3.state_dict())
    rest = g4.block(263)
    for k in whole:
        assert torch.equal(whole[k][37:], rest[k]), k
    # cluster centres drift at the stated cadence: step 256 starts a new drift period
    assert g4._last_drift == 256
