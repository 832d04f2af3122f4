"""Workload shapes for the BeaconKV eviction step.

Each workload is one eviction over every (layer, batch, KV head) unit of a
model-shaped KV cache that has grown to ``n_len = budget + n_new`` rows.  The
hyper-parameters follow the BeaconKV reading notes (liuzhao09.github.io,
"BeaconKV：用历史查询代表保护长推理的远程回看"): 16 recent + 16 beacon queries
(§2.2 Eq. 9, §3.3 Table 1), a query buffer that grows to 32 and is sampled back
to 16 (§2.2), periodic eviction of a fixed-size block of new rows (§2.1,
Fig. 5).  The model shapes are those of the evaluated models (§3.1).
"""
from __future__ import annotations

from dataclasses import dataclass, replace


@dataclass(frozen=True)
class EvictConfig:
    name: str
    n_layers: int
    batch: int
    hq: int
    hkv: int
    d: int
    theta: float
    budget: int            # B_KV^min: rows kept
    n_new: int             # rows added since the previous eviction
    n_prefix: int          # forced prefix keep
    n_recent_kv: int       # forced recent-window keep
    n_beacon: int = 16     # B_Q^min
    n_recent_q: int = 16   # recent queries; B_Q^max = n_beacon + n_recent_q
    t_lo: int = 4096       # current step t per batch element ~ U[t_lo, t_hi]
    t_hi: int = 32768
    mix: str = "clusters8"  # query distribution, see synth.py
    seed: int = 20261202
    qcap: int = 32         # rows allocated per query buffer
    pool: str = "max"      # pooling of the weights: "max" (§2.3 Eq. 7) or "mean" (§2.1 Eq. 6, §3.3 Table 2)
    beacon: str = "fps"    # source of the beacons: "fps" (§2.2), "initial" (§3.4 Table 3), "random" (§3.2 Fig. 6),
    #                        "naive" (FPS over the whole query history at each eviction, §3.2 Fig. 7)

    @property
    def n_len(self) -> int:
        return self.budget + self.n_new

    @property
    def cap(self) -> int:
        return self.n_len

    @property
    def G(self) -> int:
        return self.hq // self.hkv

    @property
    def units(self) -> int:
        return self.n_layers * self.batch * self.hkv

    @property
    def qbufs(self) -> int:
        return self.n_layers * self.batch * self.hq

    @property
    def rope_rows(self) -> int:
        return self.t_hi + 1

    def scaled(self, **kw) -> "EvictConfig":
        return replace(self, **kw)


TINY = EvictConfig(
    name="tiny", n_layers=1, batch=1, hq=4, hkv=2, d=64, theta=1e4,
    budget=128, n_new=32, n_prefix=8, n_recent_kv=16,
    t_lo=1000, t_hi=1000, mix="tight3", seed=20261202 + 100)

QWEN3_4B = EvictConfig(
    name="qwen3-4b", n_layers=36, batch=16, hq=32, hkv=8, d=128, theta=1e6,
    budget=2048, n_new=128, n_prefix=4, n_recent_kv=16,
    t_lo=4096, t_hi=32768, seed=20261202 + 200)

R1_QWEN_7B = EvictConfig(
    name="r1-distill-qwen-7b", n_layers=28, batch=64, hq=28, hkv=4, d=128, theta=1e4,
    budget=1024, n_new=128, n_prefix=4, n_recent_kv=16,
    t_lo=2048, t_hi=32768, seed=20261202 + 300)

QWEN3_14B_1K = EvictConfig(
    name="qwen3-14b-b1024", n_layers=40, batch=32, hq=40, hkv=8, d=128, theta=1e6,
    budget=1024, n_new=128, n_prefix=4, n_recent_kv=16,
    t_lo=4096, t_hi=32768, seed=20261202 + 400)

QWEN3_14B_4K = EvictConfig(
    name="qwen3-14b-b4096", n_layers=40, batch=32, hq=40, hkv=8, d=128, theta=1e6,
    budget=4096, n_new=128, n_prefix=4, n_recent_kv=16,
    t_lo=4223, t_hi=32768, seed=20261202 + 410)

# the Max/Mean ablation (§3.3 Table 2): the same eviction with mean pooling over queries and heads
QWEN3_4B_MEAN = replace(QWEN3_4B, name="qwen3-4b-mean", pool="mean")

EVICT_CONFIGS = {c.name: c for c in (TINY, QWEN3_4B, R1_QWEN_7B, QWEN3_14B_1K, QWEN3_14B_4K, QWEN3_4B_MEAN)}


@dataclass(frozen=True)
class PrefillConfig:
    """Prefill initialisation of every query buffer of a model-shaped batch: FPS of each query head's
    n_prompt pre-RoPE prompt queries down to n_beacon representatives (§2.2)."""
    name: str
    base: EvictConfig
    n_prompt: int


# a 1024-token prompt (the tasks' problem statements are a few hundred to about a thousand tokens)
PREFILL = PrefillConfig("prefill-qwen3-4b", QWEN3_4B, 1024)
# a 4096-token prompt: rows beyond the registers and LDS of a CU are re-read from memory
PREFILL_4K = PrefillConfig("prefill-qwen3-4b-p4096", QWEN3_4B, 4096)
PREFILL_CONFIGS = {c.name: c for c in (PREFILL, PREFILL_4K)}


@dataclass(frozen=True)
class StreamConfig:
    """Streaming decode from an empty cache: every step appends one token per
    sequence and routes its queries (buffer update or recent ring); the cache
    is evicted from cap = budget + n_new rows to budget, i.e. every n_new
    steps once it is full.  Token s of sequence b sits at position p0_b + s,
    p0_b ~ U[0, p0_max); query cluster centres drift every drift_every steps."""
    name: str = "stream-qwen3-4b"
    base: EvictConfig = replace(QWEN3_4B, batch=192, seed=20261202 + 500)
    steps: int = 32768
    drift_every: int = 2048
    p0_max: int = 4096

    @property
    def rope_rows(self) -> int:
        return self.p0_max + self.steps

    def evictions(self, steps: int | None = None) -> int:
        s = self.steps if steps is None else steps
        c, n = self.base.cap, self.base.n_new
        return 0 if s < c else 1 + (s - c) // n


STREAM = StreamConfig()
TINY_STREAM = StreamConfig(name="stream-tiny", base=replace(TINY, batch=2, seed=20261202 + 510),
                           steps=600, drift_every=256, p0_max=1000)
# The recent/beacon splits of the 32 observation queries in the ablation of §3.3 Table 1: all recent (no
# beacons), 31 + 1, 16 + 16 (the default), 4 + 28 and 1 + 31.  With 1 recent query the buffer is full after
# every step, so every collection step runs a sampling round.
def _split(base_cfg: StreamConfig, nrq: int, nb: int, seed: int) -> StreamConfig:
    stem = base_cfg.name
    return replace(base_cfg, name=f"{stem}-r{nrq}b{nb}",
                   base=replace(base_cfg.base, n_recent_q=nrq, n_beacon=nb, seed=seed))


SPLITS = ((32, 0), (31, 1), (4, 28), (1, 31))
STREAM_SPLITS = tuple(_split(STREAM, nrq, nb, 20261202 + 520 + i) for i, (nrq, nb) in enumerate(SPLITS))
TINY_STREAM_SPLITS = tuple(replace(_split(TINY_STREAM, nrq, nb, 20261202 + 530 + i), steps=400)
                           for i, (nrq, nb) in enumerate(SPLITS))
TINY_STREAM_MEAN = StreamConfig(name="stream-tiny-mean", base=replace(TINY, batch=2, pool="mean", seed=20261202 + 540),
                                steps=600, drift_every=256, p0_max=1000)
# Other sources of beacons: the first queries (Initial+Recent, §3.4 Table 3) and a uniform random sample of
# the history (§3.2 Fig. 6), with the 16 + 16 split.
STREAM_SOURCES = tuple(replace(STREAM, name=f"stream-qwen3-4b-{src}", base=replace(STREAM.base, beacon=src,
                                                                                 seed=20261202 + 560 + i))
                       for i, src in enumerate(("initial", "random")))
TINY_STREAM_SOURCES = tuple(replace(TINY_STREAM, name=f"stream-tiny-{src}", base=replace(TINY_STREAM.base, beacon=src,
                                                                                        seed=20261202 + 570 + i))
                            for i, src in enumerate(("initial", "random")))
# Naive full-history FPS against continual FPS (§3.2 Fig. 7): every past query of every head is kept and
# sampled at each eviction.  At batch 192 and 32K steps that history would be 1.86 TB, so the comparison runs
# at batch 16 over 7936 decode steps (histories of up to 8192 queries, 38.7 GB, the longest the library
# samples), beside continual FPS at the same shape.
STREAM_NAIVE = replace(STREAM, name="stream-qwen3-4b-naive", steps=7936,
                       base=replace(STREAM.base, batch=16, beacon="naive", seed=20261202 + 580))
STREAM_B16 = replace(STREAM, name="stream-qwen3-4b-b16", steps=7936, base=replace(STREAM.base, batch=16,
                                                                                 seed=20261202 + 580))
TINY_STREAM_NAIVE = replace(TINY_STREAM, name="stream-tiny-naive", base=replace(TINY_STREAM.base, beacon="naive",
                                                                               seed=20261202 + 590))
STREAM_CONFIGS = {c.name: c for c in (TINY_STREAM, STREAM, TINY_STREAM_MEAN) + STREAM_SPLITS + TINY_STREAM_SPLITS
                  + STREAM_SOURCES + TINY_STREAM_SOURCES + (STREAM_NAIVE, STREAM_B16, TINY_STREAM_NAIVE)}
