"""Pins of the CPU oracle against things other than itself.

Each test checks one oracle function against a hand-derived value (the
fixtures under tests/golden/), a closed form, a library routine on a special
case, an invariant, or brute force on tiny inputs.  A plausible mistake in the
oracle (a dropped term, a wrong sign or index, a transposed operand, a wrong
tie rule) fails at least one of them.
"""
from __future__ import annotations

import math
import os

import numpy as np
import pytest
import scipy.special
import torch

import oracle as O

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def bf16(x) -> np.ndarray:
    """fp32 -> bf16 codes with torch's conversion (round to nearest even)."""
    t = torch.tensor(np.asarray(x, dtype=np.float32))
    return t.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def f32(u) -> np.ndarray:
    return O.bf16_to_f32(u)


def rows(coords, d):
    out = np.zeros((len(coords), d), dtype=np.float32)
    for i, c in enumerate(coords):
        out[i, :len(c)] = c
    return bf16(out)


# --------------------------------------------------------------------------
# bf16 rounding: equals torch's round-to-nearest-even conversion.

def test_bf16_rounding_matches_torch():
    rng = np.random.default_rng(1)
    x = np.concatenate([
        rng.standard_normal(20000).astype(np.float32) * np.float32(3.0),
        np.array([0.0, -0.0, 1.0, -1.0, np.inf, -np.inf, 3.4028235e38, -3.4028235e38,
                  1e-40, -1e-40, 1e-45, 3.3895314e38], dtype=np.float32),
        # halfway cases: below-even stays, below-odd rounds up
        np.array([0x3F808000, 0x3F818000, 0xBF808000, 0xBF818000, 0x3F80FFFF,
                  0x3F807FFF, 0x7F7F8000, 0x00008000, 0x00018000], dtype=np.uint32).view(np.float32),
    ])
    ours = O.f32_to_bf16(x)
    ref = bf16(x)
    assert np.array_equal(ours, ref)
    nan = O.f32_to_bf16(np.array([np.nan], dtype=np.float32))[0]
    assert (nan & 0x7F80) == 0x7F80 and (nan & 0x7F) != 0


# --------------------------------------------------------------------------
# RoPE.

def test_rope_table_closed_forms():
    # p = 0 is the identity rotation
    t0 = O.rope_table(1e6, 128, 0, 1)
    assert np.all(t0[0, :, 0] == 1.0) and np.all(t0[0, :, 1] == 0.0)
    # pair 0 has frequency 1: the angle is p itself (libm cos/sin, rounded to fp32)
    t = O.rope_table(1e4, 64, 0, 50)
    for p in range(50):
        assert t[p, 0, 0] == np.float32(math.cos(p))
        assert t[p, 0, 1] == np.float32(math.sin(p))
    # d = 8, theta = 1e4: frequencies 1e4^(-2i/8) = 1, 0.1, 0.01, 0.001
    t1 = O.rope_table(1e4, 8, 1, 2)[0]
    ang = np.arctan2(t1[:, 1].astype(np.float64), t1[:, 0].astype(np.float64))
    assert np.allclose(ang, [1.0, 0.1, 0.01, 0.001], rtol=1e-6, atol=1e-7)
    # a table starting at p0 equals the tail of one starting at 0
    assert np.array_equal(O.rope_table(1e6, 128, 100, 110), O.rope_table(1e6, 128, 0, 110)[100:])


def test_rope_rotation_is_complex_multiplication():
    """The half-split convention: (x_i + i x_{i+d/2}) * e^{i p f_i}, f_i = theta^(-2i/d)."""
    rng = np.random.default_rng(2)
    d, theta = 128, 1e6
    n_exact = n_tot = 0
    for p in [1, 7, 1000, 4097, 32768]:
        x = bf16(rng.standard_normal((16, d)))
        xf = f32(x).astype(np.float64)
        f = theta ** (-2.0 * np.arange(d // 2) / d)
        z = (xf[:, :d // 2] + 1j * xf[:, d // 2:]) * np.exp(1j * p * f)
        ref = bf16(np.concatenate([z.real, z.imag], axis=1))
        got = np.stack([O.rope_row(r, theta, p) for r in x])
        diff = np.abs(f32(got).astype(np.float64) - f32(ref).astype(np.float64))
        ulp = np.abs(f32(ref).astype(np.float64)) * 2.0 ** -7 + 1e-30
        assert np.all(diff <= ulp * 1.01)          # at most one bf16 step apart
        n_exact += int(np.sum(got == ref))
        n_tot += got.size
    assert n_exact >= 0.995 * n_tot                 # and almost always identical


def test_rope_identity_norm_and_relative_position():
    rng = np.random.default_rng(3)
    d, theta = 64, 1e4
    x = bf16(rng.standard_normal(d))
    y = bf16(rng.standard_normal(d))
    assert np.array_equal(O.rope_row(x, theta, 0), x)           # p = 0: identity
    nx = np.linalg.norm(f32(x))
    for p in (5, 999, 30000):
        r = f32(O.rope_row(x, theta, p))
        assert abs(np.linalg.norm(r) - nx) <= 2 ** -7 * nx       # norm kept to bf16 accuracy
    # q(p1).k(p2) depends only on p1 - p2
    def dot(p1, p2):
        return float(np.dot(f32(O.rope_row(x, theta, p1)).astype(np.float64),
                            f32(O.rope_row(y, theta, p2)).astype(np.float64)))
    ref = dot(1000, 990)
    scale = float(np.linalg.norm(f32(x)) * np.linalg.norm(f32(y)))
    for delta in (1, 17, 5000):
        assert abs(dot(1000 + delta, 990 + delta) - ref) <= 0.02 * scale
    # and it does depend on p1 - p2: a row against itself is |x|^2 only at distance 0
    xx = lambda p1, p2: float(np.dot(f32(O.rope_row(x, theta, p1)).astype(np.float64),
                                     f32(O.rope_row(x, theta, p2)).astype(np.float64)))
    assert abs(xx(1000, 1000) - nx * nx) <= 0.02 * nx * nx
    assert xx(1000, 700) < 0.8 * nx * nx


# --------------------------------------------------------------------------
# FPS.

def _read_fps_cases():
    cases, cur = [], None
    for line in open(os.path.join(GOLD, "fps_hand.txt")):
        line = line.split("#")[0].strip()
        if not line:
            continue
        key, *vals = line.split()
        if key == "case":
            cur = {"name": vals[0], "rows": []}
            cases.append(cur)
        elif key == "m":
            cur["m"] = int(vals[0])
        elif key == "row":
            cur["rows"].append([float(v) for v in vals])
        elif key == "order":
            cur["order"] = [int(v) for v in vals]
    return cases


@pytest.mark.parametrize("case", _read_fps_cases(), ids=lambda c: c["name"])
@pytest.mark.parametrize("d", [4, 64, 128])
def test_fps_hand_cases(case, d):
    X = rows(case["rows"], d)
    assert O.fps(X, case["m"]) == case["order"]
    sel64, _ = O.fps_f64(X, case["m"])
    assert sel64 == case["order"]


def _fps_brute(X: np.ndarray, m: int):
    """FPS recomputed from scratch at every step in fp64 with numpy: the seed
    minimises the mean cosine; each next point minimises its largest cosine to
    the points already taken.  Also returns the smallest decision margin."""
    x = f32(X).astype(np.float64)
    n = x.shape[0]
    nr = np.linalg.norm(x, axis=1)
    cs = (x @ x.T) / np.outer(nr, nr)
    a = cs.mean(axis=1)
    order = [int(np.argmin(a))]
    srt = np.sort(a)
    margin = srt[1] - srt[0]
    while len(order) < min(m, n):
        rest = [j for j in range(n) if j not in order]
        worst = np.array([max(cs[j, i] for i in order) for j in rest])
        k = int(np.argmin(worst))
        s = np.sort(worst)
        if len(s) > 1:
            margin = min(margin, s[1] - s[0])
        order.append(rest[k])
    return order, margin


def test_fps_brute_force_tiny():
    rng = np.random.default_rng(4)
    checked = 0
    for trial in range(300):
        n = int(rng.integers(5, 33))
        d = int(rng.choice([4, 8, 64, 128]))
        m = int(rng.integers(1, n))
        X = bf16(rng.standard_normal((n, d)) * rng.uniform(0.1, 10))
        ref, margin = _fps_brute(X, m)
        if margin < 1e-5:
            continue  # a near-tie that rounding may legitimately decide
        assert O.fps(X, m) == ref, (trial, n, d, m)
        assert O.fps_f64(X, m)[0] == ref
        checked += 1
    assert checked > 250


def test_fps_power_of_two_scaling_and_duplicates():
    rng = np.random.default_rng(5)
    for trial in range(50):
        n, d, m = 32, 128, 16
        X = bf16(rng.standard_normal((n, d)))
        sel = O.fps(X, m)
        sc = 2.0 ** rng.integers(-6, 7, size=(n, 1))
        Xs = bf16(f32(X) * sc)                  # exact: bf16 * power of two
        assert O.fps(Xs, m) == sel               # cosines are bit-identical
        # a duplicated row is never picked twice while distinct rows remain
        Xd = X.copy()
        Xd[5] = Xd[17]
        s2 = O.fps(Xd, m)
        assert not (5 in s2 and 17 in s2)
        assert len(set(s2)) == m


def test_fps_picks_one_per_cluster():
    """Three tight, mutually orthogonal clusters: three picks cover all three."""
    rng = np.random.default_rng(6)
    d = 64
    cen = np.eye(d)[:3]
    lab = rng.integers(0, 3, size=30)
    X = bf16(cen[lab] * 8 + 0.05 * rng.standard_normal((30, d)))
    sel = O.fps(X, 3)
    assert sorted(lab[sel].tolist()) == [0, 1, 2]


def test_fps_small_n_returns_all():
    X = bf16(np.random.default_rng(7).standard_normal((5, 16)))
    assert O.fps(X, 5) == [0, 1, 2, 3, 4]
    assert O.fps(X, 9) == [0, 1, 2, 3, 4]


# --------------------------------------------------------------------------
# FPS over a long query set (prefill initialisation, Notes §2.2).

def test_pairwise_sum_order_and_bounds():
    # hand-derived: pairwise ((1 + 2^-24) + (2^-24 + 2^-24)); 1 + 2^-24 is a tie that rounds to even (1),
    # 2^-24 + 2^-24 = 2^-23 exactly, 1 + 2^-23 is representable.  Left to right gives 1.
    x = np.array([1.0, 2.0 ** -24, 2.0 ** -24, 2.0 ** -24], np.float32)
    assert O.pairwise_sum(x) == 1.0 + 2.0 ** -23
    assert np.float32(np.float32(np.float32(x[0] + x[1]) + x[2]) + x[3]) == 1.0
    rng = np.random.default_rng(30)
    for n in (1, 2, 3, 7, 64, 100, 513, 4096):
        ints = rng.integers(-1000, 1000, size=n).astype(np.float32)
        assert O.pairwise_sum(ints) == float(ints.astype(np.int64).sum())    # exact on small integers
        v = (rng.standard_normal(n) * 10.0 ** rng.uniform(-3, 3, size=n)).astype(np.float32)
        exact = math.fsum(v.astype(np.float64))
        bound = max(1, math.ceil(math.log2(n))) * 2.0 ** -24 * float(np.abs(v).astype(np.float64).sum())
        assert abs(O.pairwise_sum(v) - exact) <= bound * 1.0001
        # padding with zeros to any length leaves the sum bit-identical
        assert O.pairwise_sum(np.concatenate([v, np.zeros(n + 5, np.float32)])) == O.pairwise_sum(v)


@pytest.mark.parametrize("case", _read_fps_cases(), ids=lambda c: c["name"])
@pytest.mark.parametrize("d", [4, 64, 128])
def test_fps_long_hand_cases(case, d):
    assert O.fps_long(rows(case["rows"], d), case["m"]) == case["order"]


def test_fps_long_brute_force():
    """The O(n d) seed gives the FPS of the definition (fp64 brute force) away from near-ties."""
    rng = np.random.default_rng(31)
    checked = 0
    for trial in range(60):
        n = int(rng.integers(33, 400))
        d = int(rng.choice([8, 64, 128]))
        m = int(rng.integers(1, 20))
        X = bf16(rng.standard_normal((n, d)) * rng.uniform(0.1, 10))
        ref, margin = _fps_brute(X, m)
        if margin < 1e-5:
            continue
        assert O.fps_long(X, m) == ref, (trial, n, d, m)
        checked += 1
    assert checked > 30


def test_fps_long_equals_buffer_fps_away_from_ties():
    rng = np.random.default_rng(32)
    checked = 0
    for trial in range(200):
        n = int(rng.integers(5, 33))
        d = int(rng.choice([8, 64, 128]))
        m = int(rng.integers(1, n))
        X = bf16(rng.standard_normal((n, d)))
        _, margins = O.fps_f64(X, m)
        if margins.min() < 1e-5:
            continue
        assert O.fps_long(X, m) == O.fps(X, m)
        checked += 1
    assert checked > 150


@pytest.mark.parametrize("case", _read_fps_cases(), ids=lambda c: c["name"])
@pytest.mark.parametrize("d", [4, 64, 128])
def test_fps_plain_hand_cases(case, d):
    sel, regret, _ = O.fps_plain(rows(case["rows"], d), case["m"])
    assert sel == case["order"] and not regret.any()


def test_fps_plain_equals_brute_force():
    """The plain fp64 FPS is the definition: a from-scratch numpy recomputation at every step picks the
    same rows (margins below 1e-9 aside, where fp64 rounding decides), and its reported margins agree.  With
    no more rows than picks nothing is sampled: the selection is every row in order."""
    rng = np.random.default_rng(34)
    X = bf16(rng.standard_normal((9, 16)))
    for m in (9, 12):
        sel, regret, mar = O.fps_plain(X, m)
        assert sel == list(range(9)) and not regret.any() and np.isinf(mar).all()
    checked = 0
    for trial in range(120):
        n = int(rng.integers(2, 90))
        d = int(rng.choice([4, 8, 64, 128]))
        m = int(rng.integers(1, n))
        X = bf16(rng.standard_normal((n, d)) * rng.uniform(0.1, 10))
        ref, margin = _fps_brute(X, m)
        sel, regret, mar = O.fps_plain(X, m)
        assert not regret.any()
        if margin < 1e-9:
            continue
        assert sel == ref, (trial, n, d, m)
        assert abs(mar.min() - margin) <= 1e-9 * max(1.0, abs(margin))
        checked += 1
    assert checked > 100


def test_fps_plain_replay_regret():
    """Replaying picks: its own picks have zero regret; a wrong pick's regret is its value minus the best
    value, both recomputed here from the definition; taken or out-of-range picks read as infinite."""
    rng = np.random.default_rng(35)
    n, d, m = 40, 64, 10
    X = bf16(rng.standard_normal((n, d)))
    sel, _, _ = O.fps_plain(X, m)
    s2, reg, _ = O.fps_plain(X, m, forced=sel)
    assert s2 == sel and not reg.any()
    x = f32(X).astype(np.float64)
    nr = np.linalg.norm(x, axis=1)
    cs = (x @ x.T) / np.outer(nr, nr)
    for step in (0, 1, 5):
        forced = list(sel)
        taken = sel[:step]
        if step == 0:
            vals = cs.mean(axis=1)
        else:
            vals = np.array([cs[j, taken].max() for j in range(n)])
        cand = [j for j in range(n) if j not in taken]
        alt = max(cand, key=lambda j: vals[j])      # the worst row to take
        forced[step] = alt
        _, reg, _ = O.fps_plain(X, m, forced=forced)
        assert not reg[:step].any()
        assert abs(reg[step] - (vals[alt] - min(vals[j] for j in cand))) <= 1e-12
        assert reg[step] > 0
    bad = list(sel)
    bad[3] = sel[1]
    assert np.isinf(O.fps_plain(X, m, forced=bad)[1][3])
    bad[3] = n
    assert np.isinf(O.fps_plain(X, m, forced=bad)[1][3])


def test_fps_long_within_band_of_plain_definition():
    """The fp32 prefill FPS (the canonical order the kernel follows) against the plain fp64 definition on
    prompts of hundreds to thousands of rows: replayed step by step, every pick's regret is within the band
    derived from fp32 rounding, and most picks are the optimum itself."""
    from _helpers import fps_band
    rng = np.random.default_rng(36)
    steps = optimal = 0
    for trial in range(10):
        n = int(rng.choice([100, 300, 1024, 2000]))
        d = int(rng.choice([64, 128]))
        m = 16
        c = rng.standard_normal((8, d))
        X = rng.standard_normal((n, d))
        clus = rng.random(n) < 0.3
        X[clus] = c[rng.integers(0, 8, clus.sum())] * np.sqrt(d) / np.linalg.norm(c, axis=1).mean()
        X = bf16(X)
        sel = O.fps_long(X, m)
        _, reg, mar = O.fps_plain(X, m, forced=sel)
        band = fps_band(d, n)
        assert (reg <= band).all(), (trial, n, d, reg.max(), band)
        steps += len(reg)
        optimal += int((reg == 0).sum())
    assert optimal >= 0.95 * steps


def test_fps_long_scaling_clusters_and_duplicates():
    rng = np.random.default_rng(33)
    n, d, m = 700, 128, 16
    X = bf16(rng.standard_normal((n, d)))
    sel = O.fps_long(X, m)
    sc = 2.0 ** rng.integers(-6, 7, size=(n, 1))
    assert O.fps_long(bf16(f32(X) * sc), m) == sel      # unit rows and cosines are bit-identical
    Xd = X.copy()
    Xd[sel[3]] = Xd[sel[5]]
    assert len(set(O.fps_long(Xd, m))) == m
    # eight tight clusters along orthogonal axes: the first eight picks cover all of them
    lab = rng.integers(0, 8, size=n)
    Xc = bf16(np.eye(d)[lab] * 8 + 0.05 * rng.standard_normal((n, d)))
    assert sorted(lab[O.fps_long(Xc, 8)].tolist()) == list(range(8))


def test_prefill_buffers():
    rng = np.random.default_rng(34)
    nb, d, qcap = 16, 64, 32
    for P in (0, 5, 16, 17, 300):
        q = bf16(rng.standard_normal((3, P, d)))
        qbuf = np.zeros((3, qcap, d), np.uint16)
        qc = np.full(3, 99, np.int32)
        sel = O.prefill(q, qbuf, qc, nb)
        for b in range(3):
            ref = O.fps_long(q[b], nb) if P else []
            assert sel[b, :len(ref)].tolist() == ref and np.all(sel[b, len(ref):] == -1)
            assert qc[b] == min(P, nb)
            assert np.array_equal(qbuf[b, :qc[b]], q[b][sorted(ref)])
            if P <= nb:
                assert ref == list(range(P))


# --------------------------------------------------------------------------
# Other sources of beacons (Notes §3.2 Fig. 6 random history, §3.4 Table 3 Initial+Recent).

def test_philox_known_answers():
    """Philox4x32-10 known-answer values published with the generator (Salmon, Moraes, Dror, Shaw,
    "Parallel random numbers: as easy as 1, 2, 3", SC 2011; counter, key -> output)."""
    cases = [
        ((0, 0, 0, 0), (0, 0), (0x6627E8D5, 0xE169C58D, 0xBC57AC4C, 0x9B00DBD8)),
        ((0xFFFFFFFF,) * 4, (0xFFFFFFFF,) * 2, (0x408F276D, 0x41C83B0E, 0xA20BC7C6, 0x6D5451FD)),
        ((0x243F6A88, 0x85A308D3, 0x13198A2E, 0x03707344), (0xA4093822, 0x299F31D0),
         (0xD16CFE09, 0x94FDCCEB, 0x5001E420, 0x24126EA1)),
    ]
    for ctr, key, want in cases:
        assert O.philox4x32_10(ctr, key) == list(want)


def test_reservoir_slot_fill_and_inclusion_rate():
    nb = 16
    for n in range(nb):
        assert O.reservoir_slot(5, 3, n, nb) == n
    # Algorithm R: the n-th offer (n >= nb) is kept with probability nb / (n + 1), into a uniform slot
    rng = np.random.default_rng(40)
    for n in (16, 40, 1000):
        trials = 20000
        js = np.array([O.reservoir_slot(int(rng.integers(0, 2**32)), int(u), n, nb) for u in range(trials)])
        p = nb / (n + 1)
        kept = (js >= 0).mean()
        assert abs(kept - p) < 5 * math.sqrt(p * (1 - p) / trials)
        counts = np.bincount(js[js >= 0], minlength=nb)
        assert counts.min() > 0 and js.max() < nb
        exp = (js >= 0).sum() / nb
        assert ((counts - exp) ** 2 / exp).sum() < 60          # chi-square, 15 dof, far tail


def _src_cfg(src, **kw):
    base = dict(hq=2, hkv=1, d=16, cap=40, budget=30, n_prefix=2, n_recent_kv=3, n_beacon=4, n_recent_q=3,
                theta=1e4, qcap=8, beacon_src=src, seed=1234)
    base.update(kw)
    return O.OracleCfg(**base)


def test_initial_source_keeps_the_first_queries():
    cfg = _src_cfg(O.SRC_INITIAL)
    rng = np.random.default_rng(41)
    qbuf = np.zeros((2, cfg.qcap, cfg.d), np.uint16)
    qc = np.zeros(2, np.int32)
    qs = bf16(rng.standard_normal((20, 2, cfg.d)))
    for s in range(20):
        sel = O.beacon_update(cfg, qbuf, qc, qs[s])
        assert np.all(sel == -1)
        assert qc.tolist() == [min(s + 1, cfg.n_beacon)] * 2
    for b in range(2):
        assert np.array_equal(qbuf[b, :cfg.n_beacon], qs[:cfg.n_beacon, b])


def test_random_source_is_a_reservoir_of_the_offers():
    """Every kept row is one of the offered queries, each offer at most once; the count is the number of
    offers; and over many buffers each offer is kept with probability n_beacon / offers."""
    cfg = _src_cfg(O.SRC_RANDOM)
    nbuf, S = 400, 50
    rng = np.random.default_rng(42)
    # offer s of buffer b is the row whose first element encodes s (distinct, exactly representable)
    qs = np.zeros((S, nbuf, cfg.d), np.float32)
    qs[:, :, 0] = np.arange(1, S + 1)[:, None]
    qs[:, :, 1:] = rng.standard_normal((S, nbuf, cfg.d - 1))
    qs = bf16(qs)
    qbuf = np.zeros((nbuf, cfg.qcap, cfg.d), np.uint16)
    qc = np.zeros(nbuf, np.int32)
    for s in range(S):
        O.beacon_update(cfg, qbuf, qc, qs[s])
    assert np.all(qc == S)
    ids = f32(qbuf[:, :cfg.n_beacon, 0]).astype(int) - 1
    hits = np.zeros(S)
    for b in range(nbuf):
        assert len(set(ids[b].tolist())) == cfg.n_beacon and ids[b].min() >= 0
        for k, i in enumerate(ids[b]):
            assert np.array_equal(qbuf[b, k], qs[i, b])
        hits[ids[b]] += 1
    p = cfg.n_beacon / S
    assert np.all(np.abs(hits / nbuf - p) < 5 * math.sqrt(p * (1 - p) / nbuf))


def test_merge_under_other_sources():
    rng = np.random.default_rng(43)
    for src in (O.SRC_INITIAL, O.SRC_RANDOM):
        cfg = _src_cfg(src)
        qbuf = np.ascontiguousarray(bf16(rng.standard_normal((1, cfg.G, cfg.qcap, cfg.d))))
        qc = np.full((1, cfg.G), 6 if src == O.SRC_RANDOM else 4, np.int32)
        qr = bf16(rng.standard_normal((1, cfg.G, cfg.n_recent_q, cfg.d)))
        want_buf, want_qc = qbuf.copy(), qc.copy()
        if src == O.SRC_RANDOM:   # the recents are offered in ring order
            for i in range(cfg.n_recent_q):
                O.beacon_update(cfg, want_buf[0], want_qc[0], qr[0, :, i])
        sel = O.merge(cfg, qbuf, qc, qr)
        assert np.all(sel == -1)
        assert np.array_equal(qbuf, want_buf) and np.array_equal(qc, want_qc)


def test_prefill_other_sources():
    rng = np.random.default_rng(44)
    nb, d = 16, 32
    for P in (0, 7, 300):
        q = bf16(rng.standard_normal((3, P, d)))
        qbuf = np.zeros((3, 32, d), np.uint16)
        qc = np.zeros(3, np.int32)
        sel = O.prefill(q, qbuf, qc, nb, src=O.SRC_INITIAL)
        m = min(P, nb)
        assert np.all(qc == m) and np.array_equal(qbuf[:, :m], q[:, :m])
        assert np.all(sel[:, :m] == np.arange(m)) and np.all(sel[:, m:] == -1)
        # random: the same as offering the prompt rows one by one
        cfg = _src_cfg(O.SRC_RANDOM, d=d, n_beacon=nb, qcap=32, seed=77)
        qbuf2, qc2 = np.zeros((3, 32, d), np.uint16), np.zeros(3, np.int32)
        sel = O.prefill(q, qbuf2, qc2, nb, src=O.SRC_RANDOM, seed=77)
        wb, wc = np.zeros((3, 32, d), np.uint16), np.zeros(3, np.int32)
        for n in range(P):
            O.beacon_update(cfg, wb, wc, q[:, n])
        assert np.array_equal(qc2, wc) and np.array_equal(qbuf2[:, :m], wb[:, :m])
        for b in range(3):
            for k in range(m):
                assert np.array_equal(qbuf2[b, k], q[b, sel[b, k]])


def test_fps_update_continual_buffer():
    """Eq. 9: append; at B_Q^max rows the buffer becomes FPS(buffer, n_beacon)
    in ascending slot order with count n_beacon; below it, only the append."""
    rng = np.random.default_rng(8)
    nb, nrq, d, qcap = 16, 16, 64, 32
    qbuf = bf16(rng.standard_normal((3, qcap, d)))
    qbuf = np.ascontiguousarray(qbuf)
    qnew = bf16(rng.standard_normal((3, d)))
    qcount = np.array([31, 10, 0], dtype=np.int32)
    before = qbuf.copy()
    sel = O.fps_update(qbuf, qcount, qnew, nb, nrq)
    # buffer 0: 31 + 1 = 32 -> sampled
    full = np.concatenate([before[0, :31], qnew[0:1]])
    ref = O.fps(full, nb)
    assert sel[0].tolist() == ref
    assert qcount[0] == nb
    assert np.array_equal(qbuf[0, :nb], full[sorted(ref)])
    # buffer 1: append only
    assert qcount[1] == 11 and np.array_equal(qbuf[1, 10], qnew[1])
    assert np.array_equal(qbuf[1, :10], before[1, :10]) and np.all(sel[1] == -1)
    assert qcount[2] == 1 and np.array_equal(qbuf[2, 0], qnew[2])


# --------------------------------------------------------------------------
# Attention weights and max pooling.

def _read_kv(name):
    out = {}
    for line in open(os.path.join(GOLD, name)):
        line = line.split("#")[0].strip()
        if not line:
            continue
        key, *vals = line.split()
        out.setdefault(key, []).append(vals)
    return out


def test_softmax_hand_row():
    g = _read_kv("softmax_row.txt")
    d = int(g["d"][0][0])
    q = np.zeros(d, np.float32)
    q[0] = float(g["q0"][0][0])
    keys = [float(v) for v in g["keys"][0]]
    K = np.zeros((len(keys), d), np.float32)
    K[:, 0] = keys
    w, c = O.row_weights(bf16(q), bf16(K))
    assert np.allclose(w, [float(v) for v in g["w"][0]], rtol=1e-14, atol=0)
    assert abs(c - math.log(1 + math.e + math.e ** 2)) < 1e-14


def test_row_weights_sum_to_one_and_match_scipy():
    rng = np.random.default_rng(9)
    for d in (64, 128):
        K = bf16(rng.standard_normal((300, d)) * np.where(rng.random((300, 1)) < 0.01, 8, 1))
        q = bf16(rng.standard_normal(d))
        w, _ = O.row_weights(q, K)
        z = f32(K).astype(np.float64) @ f32(q).astype(np.float64) / math.sqrt(d)
        assert abs(w.sum() - 1) < 1e-12
        assert np.allclose(w, scipy.special.softmax(z), rtol=1e-12, atol=1e-300)
        w5, _ = O.row_weights(q, K, vis=150)
        assert np.all(w5[151:] == 0) and abs(w5.sum() - 1) < 1e-12
        assert np.allclose(w5[:151], scipy.special.softmax(z[:151]), rtol=1e-12, atol=1e-300)


def _cfg(**kw):
    base = dict(hq=4, hkv=2, d=64, cap=40, budget=30, n_prefix=2, n_recent_kv=3,
                n_beacon=3, n_recent_q=4, theta=1e4, qcap=8)
    base.update(kw)
    return O.OracleCfg(**base)


def _random_unit_inputs(cfg, U, rng, qcount=None):
    G, d = cfg.G, cfg.d
    K = bf16(rng.standard_normal((U, cfg.cap, d)) * np.where(rng.random((U, cfg.cap, 1)) < 0.05, 6, 1))
    V = bf16(rng.standard_normal((U, cfg.cap, d)))
    qbuf = bf16(rng.standard_normal((U, G, cfg.qcap, d)) * 1.5)
    qc = np.full((U, G), cfg.n_beacon if qcount is None else qcount, np.int32)
    qr = bf16(rng.standard_normal((U, G, cfg.n_recent_q, d)) * 1.5)
    t = rng.integers(500, 3000, size=U).astype(np.int32)
    pos = (t[:, None] - cfg.n_recent_q + 1 + np.arange(cfg.n_recent_q)[None, :]).astype(np.int32)
    return dict(K=K, V=V, qbuf=qbuf, qcount=qc, q_recent=qr, pos_recent=pos, t=t)


def _brute_scores(cfg, inp, N, mean=False):
    """Max (or mean) over the group's heads and rows of scipy softmax rows (brute force)."""
    U = inp["K"].shape[0]
    out = np.zeros((U, N))
    for u in range(U):
        Kf = f32(inp["K"][u, :N]).astype(np.float64)
        stack = []
        for h in range(cfg.G):
            nb = min(int(inp["qcount"][u, h]), cfg.n_beacon)
            obs = [(O.rope_row(inp["qbuf"][u, h, s], cfg.theta, int(inp["t"][u])), N - 1) for s in range(nb)]
            for i in range(cfg.n_recent_q):
                vis = N - cfg.n_recent_q + i if cfg.causal else N - 1
                obs.append((O.rope_row(inp["q_recent"][u, h, i], cfg.theta, int(inp["pos_recent"][u, i])), vis))
            for q, vis in obs:
                w = np.zeros(N)
                if vis >= 0:
                    z = Kf[:vis + 1] @ f32(q).astype(np.float64) / math.sqrt(cfg.d)
                    w[:vis + 1] = scipy.special.softmax(z)
                stack.append(w)
        if stack:
            out[u] = np.mean(stack, axis=0) if mean else np.max(stack, axis=0)
    return out


@pytest.mark.parametrize("causal", [1, 0])
@pytest.mark.parametrize("qcount", [3, 1, 0, 6])
def test_score_is_max_over_heads_and_rows(causal, qcount):
    rng = np.random.default_rng(10 + qcount + 10 * causal)
    cfg = _cfg(causal=causal)
    inp = _random_unit_inputs(cfg, 3, rng, qcount=qcount)
    N = 37
    s = O.score(cfg, inp["K"], inp["qbuf"], inp["qcount"], inp["q_recent"], inp["pos_recent"], inp["t"], n_len=N)
    ref = _brute_scores(cfg, inp, N)
    assert np.allclose(s, ref, rtol=1e-12, atol=1e-300)


@pytest.mark.parametrize("causal", [1, 0])
@pytest.mark.parametrize("qcount", [3, 1, 0, 6, (5, 1)])
@pytest.mark.parametrize("N", [37, 2])
def test_mean_score_is_mean_over_heads_and_rows(causal, qcount, N):
    """Mean pooling (Notes §2.1 Eq. 6, over queries and heads as in §3.3 Table 2)."""
    rng = np.random.default_rng(20 + N + 10 * causal + (qcount if isinstance(qcount, int) else 7))
    cfg = _cfg(causal=causal, pool_mean=1)
    inp = _random_unit_inputs(cfg, 3, rng, qcount=0)
    inp["qcount"][:] = qcount
    s = O.score(cfg, inp["K"], inp["qbuf"], inp["qcount"], inp["q_recent"], inp["pos_recent"], inp["t"], n_len=N)
    assert np.allclose(s, _brute_scores(cfg, inp, N, mean=True), rtol=1e-12, atol=1e-300)
    # every row that sees a key has weights summing to 1, so the scores sum to
    # (rows that see a key) / (all rows); at N = 2 causal recent rows 0 and 1 see nothing
    nb = np.minimum(inp["qcount"][0], cfg.n_beacon).sum()
    rows = nb + cfg.G * cfg.n_recent_q
    seen = nb + cfg.G * sum(1 for i in range(cfg.n_recent_q)
                            if (N - cfg.n_recent_q + i if causal else N - 1) >= 0)
    assert np.allclose(s.sum(axis=1), seen / rows, rtol=1e-12)
    # the mean lies between max / rows and the max
    smax = O.score(_cfg(causal=causal), inp["K"], inp["qbuf"], inp["qcount"], inp["q_recent"],
                   inp["pos_recent"], inp["t"], n_len=N)
    assert np.all(s <= smax * (1 + 1e-12)) and np.all(s >= smax / rows * (1 - 1e-12))


def test_mean_of_identical_rows_is_one_softmax():
    """Every observation row the same query at the same position, no causal mask: the mean equals the
    max equals that row's softmax."""
    rng = np.random.default_rng(21)
    cfg = _cfg(causal=0, pool_mean=1)
    inp = _random_unit_inputs(cfg, 2, rng, qcount=3)
    q = inp["qbuf"][:, :1, :1]
    inp["qbuf"][:] = q
    inp["q_recent"][:] = q
    inp["pos_recent"][:] = inp["t"][:, None]
    s = O.score(cfg, inp["K"], inp["qbuf"], inp["qcount"], inp["q_recent"], inp["pos_recent"], inp["t"])
    for u in range(2):
        qr = O.rope_row(q[u, 0, 0], cfg.theta, int(inp["t"][u]))
        z = f32(inp["K"][u]).astype(np.float64) @ f32(qr).astype(np.float64) / math.sqrt(cfg.d)
        assert np.allclose(s[u], scipy.special.softmax(z), rtol=1e-12)


def test_score_single_row_equals_softmax():
    """G = 1, one beacon, no recent queries, t = 0: Score is one softmax row."""
    rng = np.random.default_rng(11)
    cfg = _cfg(hq=1, hkv=1, n_beacon=1, n_recent_q=0, cap=50)
    inp = _random_unit_inputs(cfg, 1, rng, qcount=1)
    inp["t"][:] = 0
    s = O.score(cfg, inp["K"], inp["qbuf"], inp["qcount"], inp["q_recent"], inp["pos_recent"], inp["t"])
    z = f32(inp["K"][0]).astype(np.float64) @ f32(inp["qbuf"][0, 0, 0]).astype(np.float64) / 8.0
    assert np.allclose(s[0], scipy.special.softmax(z), rtol=1e-12)


def test_no_beacons_reduces_to_recent_only():
    """qcount = 0: only the recent rows score (the all-recent split of Table 1)."""
    rng = np.random.default_rng(12)
    cfg = _cfg()
    inp = _random_unit_inputs(cfg, 2, rng, qcount=0)
    s0 = O.score(cfg, inp["K"], inp["qbuf"], inp["qcount"], inp["q_recent"], inp["pos_recent"], inp["t"])
    cfg_r = _cfg(n_beacon=0)
    s1 = O.score(cfg_r, inp["K"], inp["qbuf"], inp["qcount"], inp["q_recent"], inp["pos_recent"], inp["t"])
    assert np.array_equal(s0, s1)


# --------------------------------------------------------------------------
# Decode attention over the cache (Notes §2.1, the second formula).

def _attn_inputs(rng, U, G, N, d, cap=None):
    cap = N if cap is None else cap
    K = bf16(rng.standard_normal((U, cap, d)) * np.where(rng.random((U, cap, 1)) < 0.05, 6, 1))
    V = bf16(rng.standard_normal((U, cap, d)))
    q = bf16(rng.standard_normal((U, G, d)) * 1.5)
    pos = rng.integers(0, 5000, size=U).astype(np.int32)
    return K, V, q, pos


def test_decode_attention_is_softmax_times_values():
    rng = np.random.default_rng(50)
    cfg = _cfg(hq=6, hkv=2, cap=70)
    K, V, q, pos = _attn_inputs(rng, 3, cfg.G, 70, cfg.d)
    for N in (70, 33, 1):
        out, scale = O.decode_attention(cfg, K, V, q, pos, N)
        for u in range(3):
            Kf, Vf = f32(K[u, :N]).astype(np.float64), f32(V[u, :N]).astype(np.float64)
            for h in range(cfg.G):
                qr = f32(O.rope_row(q[u, h], cfg.theta, int(pos[u]))).astype(np.float64)
                w = scipy.special.softmax(Kf @ qr / math.sqrt(cfg.d))
                assert np.allclose(out[u, h], w @ Vf, rtol=1e-12, atol=1e-14)
                assert np.allclose(scale[u, h], w @ np.abs(Vf), rtol=1e-12, atol=1e-14)
        if N == 1:   # one row: its value, whatever the query
            assert np.array_equal(out, np.repeat(f32(V[:, :1]).astype(np.float64), cfg.G, axis=1))


def test_decode_attention_special_cases():
    rng = np.random.default_rng(51)
    cfg = _cfg(hq=2, hkv=1, cap=40)
    K, V, q, pos = _attn_inputs(rng, 2, cfg.G, 40, cfg.d)
    # identical keys: uniform weights, the mean of the values
    Ks = np.repeat(K[:, :1], 40, axis=1)
    out, _ = O.decode_attention(cfg, np.ascontiguousarray(Ks), V, q, pos, 40)
    assert np.allclose(out, f32(V).astype(np.float64).mean(axis=1)[:, None, :], rtol=1e-12, atol=1e-14)
    # a zero query: uniform weights too
    out0, _ = O.decode_attention(cfg, K, V, np.zeros_like(q), pos, 25)
    assert np.allclose(out0, f32(V[:, :25]).astype(np.float64).mean(axis=1)[:, None, :], rtol=1e-12, atol=1e-14)


# --------------------------------------------------------------------------
# Keep set.

def _select_ref(s, B, npf, nr):
    N = len(s)
    if N <= B:
        return np.array(list(range(N)) + [-1] * (B - N))
    forced = set(range(min(npf, N))) | set(range(max(0, N - nr), N))
    cand = np.array([j for j in range(N) if j not in forced])
    order = cand[np.argsort(-s[cand], kind="stable")]
    keep = sorted(forced | set(order[:B - len(forced)].tolist()))
    return np.array(keep)


def test_select_matches_stable_argsort():
    rng = np.random.default_rng(13)
    for trial in range(200):
        N = int(rng.integers(1, 400))
        B = int(rng.integers(0, 420))
        npf = int(rng.integers(0, 10))
        nr = int(rng.integers(0, 20))
        if N > B and B < npf + nr:
            continue  # not a valid configuration (budget below the forced keeps)
        if trial % 2:
            s = rng.random(N)
        else:
            s = rng.integers(0, 5, N).astype(np.float64)  # many exact ties
        idx, moved = O.select(s, B, npf, nr)
        ref = _select_ref(s, B, npf, nr)
        assert np.array_equal(idx, ref), trial
        assert moved == int(np.sum(ref[ref >= 0] != np.arange(len(ref))[ref >= 0]))


def test_select_invariants():
    rng = np.random.default_rng(14)
    for trial in range(50):
        N, B, npf, nr = 2176, 2048, 4, 16
        s = rng.random(N) ** 3
        idx, _ = O.select(s, B, npf, nr)
        assert len(idx) == B and np.all(np.diff(idx) > 0)
        assert set(range(npf)) <= set(idx.tolist())
        assert set(range(N - nr, N)) <= set(idx.tolist())
        kept = set(idx.tolist())
        cand = [j for j in range(npf, N - nr)]
        chosen = [s[j] for j in cand if j in kept]
        evicted = [s[j] for j in cand if j not in kept]
        assert min(chosen) >= max(evicted)


def test_compact_is_fancy_indexing():
    rng = np.random.default_rng(15)
    cfg = _cfg(cap=60, budget=40)
    K = bf16(rng.standard_normal((3, 60, 64)))
    V = bf16(rng.standard_normal((3, 60, 64)))
    idx = np.stack([np.sort(rng.choice(55, 40, replace=False)) for _ in range(3)]).astype(np.int32)
    K2, V2 = K.copy(), V.copy()
    O.compact(cfg, K2, V2, idx, n_len=55)
    for u in range(3):
        assert np.array_equal(K2[u, :40], K[u][idx[u]])
        assert np.array_equal(V2[u, :40], V[u][idx[u]])
        assert np.array_equal(K2[u, 40:], K[u, 40:])


# --------------------------------------------------------------------------
# The whole eviction.

def _hand_case(causal):
    g = _read_kv("evict_hand.txt")
    d = int(g["d"][0][0])
    N = int(g["n_len"][0][0])
    cfg = O.OracleCfg(hq=1, hkv=1, d=d, cap=N, budget=int(g["budget"][0][0]),
                      n_prefix=int(g["n_prefix"][0][0]), n_recent_kv=int(g["n_recent_kv"][0][0]),
                      n_beacon=len(g["beacon"]), n_recent_q=len(g["recent"]), theta=1e4,
                      qcap=4, causal=causal)
    K = bf16([[float(v) for v in r] for r in g["key"]]).reshape(1, N, d)
    V = bf16(np.arange(N * d, dtype=np.float32).reshape(1, N, d))
    qbuf = np.zeros((1, 1, 4, d), np.uint16)
    qbuf[0, 0, :len(g["beacon"])] = bf16([[float(v) for v in r] for r in g["beacon"]])
    qc = np.array([[len(g["beacon"])]], np.int32)
    qr = bf16([[float(v) for v in r] for r in g["recent"]]).reshape(1, 1, -1, d)
    pos = np.zeros((1, len(g["recent"])), np.int32)
    t = np.zeros(1, np.int32)
    return g, cfg, K, V, qbuf, qc, qr, pos, t


def test_evict_hand_example():
    g, cfg, K, V, qbuf, qc, qr, pos, t = _hand_case(1)
    K0, V0, qb0 = K.copy(), V.copy(), qbuf.copy()
    out = O.evict(cfg, K, V, qbuf, qc, qr, pos, t)
    want = [float(v) for v in g["scores_causal"][0]]
    assert np.allclose(out["scores"][0], want, atol=5e-7)
    idx = [int(v) for v in g["idx_causal"][0]]
    assert out["idx"][0].tolist() == idx
    assert np.array_equal(K[0, :4], K0[0][idx]) and np.array_equal(V[0, :4], V0[0][idx])
    assert out["moved"][0] == 2
    # merge: FPS over [beacon, r0, r1] keeps one row
    assert out["fps_sel"][0, 0].tolist() == [int(v) for v in g["merge_sel"][0]]
    assert qc[0, 0] == 1 and np.array_equal(qbuf[0, 0, 0], qb0[0, 0, 0])
    # without the causal mask the kept set changes as derived by hand
    g, cfg, K, V, qbuf, qc, qr, pos, t = _hand_case(0)
    out = O.evict(cfg, K, V, qbuf, qc, qr, pos, t)
    assert out["idx"][0].tolist() == [int(v) for v in g["idx_nocausal"][0]]


def test_evict_is_score_select_compact_merge():
    rng = np.random.default_rng(16)
    cfg = _cfg()
    inp = _random_unit_inputs(cfg, 4, rng)
    a = {k: v.copy() for k, v in inp.items()}
    out = O.evict(cfg, a["K"], a["V"], a["qbuf"], a["qcount"], a["q_recent"], a["pos_recent"], a["t"], nthreads=3)
    s = _brute_scores(cfg, inp, cfg.cap)
    assert np.allclose(out["scores"], s, rtol=1e-12, atol=1e-300)
    for u in range(4):
        ref = _select_ref(out["scores"][u], cfg.budget, cfg.n_prefix, cfg.n_recent_kv)
        assert np.array_equal(out["idx"][u], ref)
        assert np.array_equal(a["K"][u, :cfg.budget], inp["K"][u][ref])
        assert np.array_equal(a["V"][u, :cfg.budget], inp["V"][u][ref])
        for h in range(cfg.G):
            X = np.concatenate([inp["qbuf"][u, h, :cfg.n_beacon], inp["q_recent"][u, h]])
            sel = O.fps(X, cfg.n_beacon)
            assert out["fps_sel"][u, h].tolist() == sel
            assert np.array_equal(a["qbuf"][u, h, :cfg.n_beacon], X[sorted(sel)])
            assert a["qcount"][u, h] == cfg.n_beacon


def test_merge_hand_case():
    """Beacons [e0, e1], recents [-e0, -e1], n_beacon 2: FPS picks e0 then -e0."""
    d = 8
    cfg = _cfg(hq=1, hkv=1, d=d, n_beacon=2, n_recent_q=2, qcap=4)
    qbuf = np.zeros((1, 1, 4, d), np.uint16)
    qbuf[0, 0, :2] = rows([[1, 0], [0, 1]], d)
    qr = rows([[-1, 0], [0, -1]], d).reshape(1, 1, 2, d)
    qc = np.array([[2]], np.int32)
    sel = O.merge(cfg, qbuf, qc, qr)
    assert sel[0, 0].tolist() == [0, 2]
    assert np.array_equal(qbuf[0, 0, :2], rows([[1, 0], [-1, 0]], d)) and qc[0, 0] == 2


def test_evict_no_op_when_cache_not_full():
    rng = np.random.default_rng(17)
    cfg = _cfg(cap=40, budget=40)
    inp = _random_unit_inputs(cfg, 2, rng)
    K, V = inp["K"].copy(), inp["V"].copy()
    out = O.evict(cfg, K, V, inp["qbuf"].copy(), inp["qcount"].copy(), inp["q_recent"], inp["pos_recent"],
                  inp["t"], n_len=33)
    assert out["idx"][0].tolist() == list(range(33)) + [-1] * 7
    assert np.array_equal(K, inp["K"]) and np.all(out["moved"] == 0)
