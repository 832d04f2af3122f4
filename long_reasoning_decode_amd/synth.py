"""Seeded synthetic inputs for the eviction step.

This module only draws random numbers and rounds them to bf16; it holds none
of the method's arithmetic.  The same tensors feed the HIP library and the CPU
oracle.  Generation runs on the device the tensors are made for (a CPU
``torch.Generator`` for small cases, a GPU one for full-size workloads); each
is deterministic for a given seed, device and torch version.

Recipe (stand-in for the reasoning traces of AIME24 / MATH-500 /
LiveCodeBench / GPQA-Diamond that the pages evaluate on, which are not
available here):
  * queries (pre-RoPE; buffer rows, recent rows):
      - "clusters8": each row is, with probability 0.3, a cluster row
        s * sqrt(d) * u_c with c uniform over 8 random unit centres of its
        (layer, batch, query head) and s ~ N(1, 0.2); otherwise N(0, I_d).
        Cluster rows mimic the recurring "global" query directions, the
        isotropic rows the local ones.
      - "tight3": with probability 0.25, sqrt(d) * (u_c + 0.1 g), c uniform
        over 3 centres, g ~ N(0, I_d / d); otherwise N(0, I_d).
  * keys: N(0, I_d); each row independently, with probability 0.01, is an
    outlier row scaled by 8.  Keys are drawn directly in their post-RoPE form:
    a rotation maps an isotropic Gaussian row to an isotropic Gaussian row
    and keeps a row's norm, so this is the same distribution as rotating
    N(0, I_d) pre-RoPE keys at their positions.
  * values: N(0, I_d).
  * current step t_b ~ U[t_lo, t_hi] per batch element; the recent queries of
    batch element b sit at positions t_b - n_recent_q + 1 .. t_b.
  * every buffer holds n_beacon rows from the last sampling (qcount =
    n_beacon); its slots beyond that are filled with further query rows,
    which an eviction must ignore.
All bf16 values are fp32 draws rounded to nearest even (torch's conversion).
"""
from __future__ import annotations

import math

import torch

from .configs import EvictConfig


def _gen(device, seed: int) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(int(seed))
    return g


def _unit_rows(g, shape, d, device) -> torch.Tensor:
    x = torch.randn(*shape, d, generator=g, device=device, dtype=torch.float32)
    return x / x.norm(dim=-1, keepdim=True)


def query_rows(g: torch.Generator, centres: torch.Tensor, n_rows: int, mix: str) -> torch.Tensor:
    """Rows of the query mixture, fp32.  centres: [..., C, d] unit vectors.

    Returns [..., n_rows, d]."""
    lead = centres.shape[:-2]
    C, d = centres.shape[-2:]
    dev = centres.device
    iso = torch.randn(*lead, n_rows, d, generator=g, device=dev)
    pick = torch.randint(0, C, (*lead, n_rows), generator=g, device=dev)
    u = torch.rand(*lead, n_rows, generator=g, device=dev)
    cen = torch.gather(centres, -2, pick.unsqueeze(-1).expand(*lead, n_rows, d))
    if mix == "clusters8":
        s = 1.0 + 0.2 * torch.randn(*lead, n_rows, 1, generator=g, device=dev)
        clus = s * math.sqrt(d) * cen
        frac = 0.3
    elif mix == "tight3":
        noise = torch.randn(*lead, n_rows, d, generator=g, device=dev) / math.sqrt(d)
        clus = math.sqrt(d) * (cen + 0.1 * noise)
        frac = 0.25
    else:
        raise ValueError(f"unknown query mix {mix!r}")
    return torch.where((u < frac).unsqueeze(-1), clus, iso)


def n_centres(mix: str) -> int:
    return {"clusters8": 8, "tight3": 3}[mix]


def key_rows(g: torch.Generator, lead: tuple, n_rows: int, d: int, device) -> torch.Tensor:
    k = torch.randn(*lead, n_rows, d, generator=g, device=device)
    out = torch.rand(*lead, n_rows, 1, generator=g, device=device) < 0.01
    return torch.where(out, 8.0 * k, k)


def make_evict_inputs(cfg: EvictConfig, device="cpu", seed: int | None = None,
                      n_len: int | None = None, qcount: int | None = None) -> dict:
    """All inputs of one eviction, laid out as the library expects:

    K, V        bf16  [L, B, Hkv, cap, d]   (cap = n_len)
    qbuf        bf16  [L, B, Hq, qcap, d]
    qcount      int32 [L, B, Hq]
    q_recent    bf16  [L, B, Hq, n_recent_q, d]
    pos_recent  int32 [B, n_recent_q]
    t           int32 [B]
    """
    device = torch.device(device)
    g = _gen(device, cfg.seed if seed is None else seed)
    N = cfg.n_len if n_len is None else n_len
    L, B, Hq, Hkv, d = cfg.n_layers, cfg.batch, cfg.hq, cfg.hkv, cfg.d
    nrq = cfg.n_recent_q
    t = torch.randint(cfg.t_lo, cfg.t_hi + 1, (B,), generator=g, device=device, dtype=torch.int64)
    pos = t.unsqueeze(1) - nrq + 1 + torch.arange(nrq, device=device).unsqueeze(0)
    K = torch.empty(L, B, Hkv, N, d, dtype=torch.bfloat16, device=device)
    V = torch.empty_like(K)
    qbuf = torch.empty(L, B, Hq, cfg.qcap, d, dtype=torch.bfloat16, device=device)
    q_recent = torch.empty(L, B, Hq, nrq, d, dtype=torch.bfloat16, device=device)
    C = n_centres(cfg.mix)
    for l in range(L):  # one layer at a time bounds the fp32 temporaries
        K[l] = key_rows(g, (B, Hkv), N, d, device).to(torch.bfloat16)
        V[l] = torch.randn(B, Hkv, N, d, generator=g, device=device).to(torch.bfloat16)
        cen = _unit_rows(g, (B, Hq, C), d, device)
        qbuf[l] = query_rows(g, cen, cfg.qcap, cfg.mix).to(torch.bfloat16)
        q_recent[l] = query_rows(g, cen, nrq, cfg.mix).to(torch.bfloat16)
    qc = cfg.n_beacon if qcount is None else qcount
    return {
        "K": K, "V": V, "qbuf": qbuf,
        "qcount": torch.full((L, B, Hq), qc, dtype=torch.int32, device=device),
        "q_recent": q_recent,
        "pos_recent": pos.to(torch.int32), "t": t.to(torch.int32),
    }


def make_query_buffers(cfg: EvictConfig, device="cpu", seed: int | None = None,
                       fill: int | None = None) -> dict:
    """Query buffers for the per-step update: qbuf [L, B, Hq, qcap, d] with
    ``fill`` valid rows (default B_Q^max - 1, so the next append triggers a
    sampling round), and one new query row per buffer, q_new [L, B, Hq, d]."""
    device = torch.device(device)
    g = _gen(device, (cfg.seed if seed is None else seed) + 7)
    L, B, Hq, d = cfg.n_layers, cfg.batch, cfg.hq, cfg.d
    C = n_centres(cfg.mix)
    fill = cfg.n_beacon + cfg.n_recent_q - 1 if fill is None else fill
    qbuf = torch.empty(L, B, Hq, cfg.qcap, d, dtype=torch.bfloat16, device=device)
    q_new = torch.empty(L, B, Hq, d, dtype=torch.bfloat16, device=device)
    for l in range(L):
        cen = _unit_rows(g, (B, Hq, C), d, device)
        qbuf[l] = query_rows(g, cen, cfg.qcap, cfg.mix).to(torch.bfloat16)
        q_new[l] = query_rows(g, cen, 1, cfg.mix)[..., 0, :].to(torch.bfloat16)
    return {"qbuf": qbuf, "qcount": torch.full((L, B, Hq), fill, dtype=torch.int32, device=device),
            "q_new": q_new}


def make_prompt_queries(cfg: EvictConfig, n_prompt: int, device="cpu", seed: int | None = None) -> torch.Tensor:
    """Pre-RoPE prompt queries for the prefill sampling, bf16 [L, B, Hq, n_prompt, d], drawn from the
    workload's query mixture with centres of their own per (layer, batch, query head)."""
    device = torch.device(device)
    g = _gen(device, (cfg.seed if seed is None else seed) + 11)
    L, B, Hq, d = cfg.n_layers, cfg.batch, cfg.hq, cfg.d
    C = n_centres(cfg.mix)
    q = torch.empty(L, B, Hq, n_prompt, d, dtype=torch.bfloat16, device=device)
    for l in range(L):
        cen = _unit_rows(g, (B, Hq, C), d, device)
        q[l] = query_rows(g, cen, n_prompt, cfg.mix).to(torch.bfloat16)
    return q


# ---------------------------------------------------------------------------
# Streaming decode inputs.

class StreamGen:
    """Per-step inputs of the streaming decode simulation, drawn on the
    generator's device:
      q_new [n, L, B, Hq, d]   bf16, pre-RoPE, the query mixture of the base
                               config around per-(layer, batch, q-head) centres
      k_new [n, L, B, Hkv, d]  bf16, pre-RoPE keys (N(0, I), 1% rows x 8)
      v_new [n, L, B, Hkv, d]  bf16, N(0, I)
      pos   [n, B]             int32, p0_b + s for global step s
    Every drift_every steps (before step s = k * drift_every, k >= 1) each
    centre becomes normalize(u_c + 0.5 g), g ~ N(0, I_d / d).  Draws happen in
    whole chunks of `chunk` steps at fixed step boundaries, and steps a call
    does not use wait for the next one, so the sequence does not depend on how
    the caller splits the run into blocks (and resumes exactly from
    state_dict())."""

    def __init__(self, scfg, device="cpu", seed: int | None = None, chunk: int = 16):
        base = scfg.base
        if scfg.drift_every % chunk:
            raise ValueError("drift_every must be a multiple of the chunk size")
        self.scfg, self.base, self.chunk = scfg, base, chunk
        self.device = torch.device(device)
        self.g = _gen(self.device, base.seed if seed is None else seed)
        L, B, Hq, d = base.n_layers, base.batch, base.hq, base.d
        self.centres = _unit_rows(self.g, (L, B, Hq, n_centres(base.mix)), d, self.device)
        self.p0 = torch.randint(0, scfg.p0_max, (B,), generator=self.g, device=self.device, dtype=torch.int64)
        self.step = 0           # steps handed out
        self._last_drift = 0
        self._buf = None        # the current chunk
        self._cpos = 0          # steps of it handed out

    def state_dict(self) -> dict:
        st = {"rng": self.g.get_state(), "centres": self.centres.clone(), "p0": self.p0.clone(),
              "step": self.step, "last_drift": self._last_drift, "cpos": self._cpos}
        if self._buf is not None:
            st.update({"buf_" + k: v.clone() for k, v in self._buf.items()})
        return st

    def load_state_dict(self, st: dict) -> None:
        self.g.set_state(st["rng"])
        self.centres = st["centres"].to(self.device).clone()
        self.p0 = st["p0"].to(self.device).clone()
        self.step, self._last_drift, self._cpos = int(st["step"]), int(st["last_drift"]), int(st["cpos"])
        keys = [k[4:] for k in st if k.startswith("buf_")]
        self._buf = {k: st["buf_" + k].to(self.device).clone() for k in keys} if keys else None

    def _drift(self) -> None:
        d = self.base.d
        g = torch.randn(self.centres.shape, generator=self.g, device=self.device) / math.sqrt(d)
        c = self.centres + 0.5 * g
        self.centres = c / c.norm(dim=-1, keepdim=True)

    def _draw_chunk(self) -> None:
        """Draw the chunk that starts at step self.step (a multiple of the chunk size)."""
        b = self.base
        L, B, Hq, Hkv, d = b.n_layers, b.batch, b.hq, b.hkv, b.d
        s0, n = self.step, self.chunk
        if s0 % self.scfg.drift_every == 0 and s0 != self._last_drift:
            self._drift()
            self._last_drift = s0
        out = self.alloc(n) if self._buf is None else self._buf
        q = query_rows(self.g, self.centres, n, b.mix)                  # [L, B, Hq, n, d]
        out["q_new"].copy_(q.permute(3, 0, 1, 2, 4))
        del q
        out["k_new"].copy_(key_rows(self.g, (n, L, B, Hkv), 1, d, self.device)[..., 0, :])
        out["v_new"].copy_(torch.randn(n, L, B, Hkv, d, generator=self.g, device=self.device))
        s = torch.arange(s0, s0 + n, device=self.device, dtype=torch.int64)
        out["pos"].copy_(self.p0.unsqueeze(0) + s.unsqueeze(1))
        self._buf, self._cpos = out, 0

    def alloc(self, n: int) -> dict:
        b = self.base
        L, B, Hq, Hkv, d = b.n_layers, b.batch, b.hq, b.hkv, b.d
        dev = self.device
        return {"q_new": torch.empty(n, L, B, Hq, d, dtype=torch.bfloat16, device=dev),
                "k_new": torch.empty(n, L, B, Hkv, d, dtype=torch.bfloat16, device=dev),
                "v_new": torch.empty(n, L, B, Hkv, d, dtype=torch.bfloat16, device=dev),
                "pos": torch.empty(n, B, dtype=torch.int32, device=dev)}

    def block(self, n: int, out: dict | None = None) -> dict:
        """The next n steps' inputs (into `out` when given, a dict from alloc(>= n))."""
        out = self.alloc(n) if out is None else out
        at = 0
        while at < n:
            if self._buf is None or self._cpos >= self.chunk:
                self._draw_chunk()
            k = min(self.chunk - self._cpos, n - at)
            for key, t in out.items():
                t[at:at + k] = self._buf[key][self._cpos:self._cpos + k]
            self._cpos += k
            self.step += k
            at += k
        return out


# ---------------------------------------------------------------------------
# Views for the oracle (numpy, unit-major).

def to_u16(x: torch.Tensor):
    """bf16 tensor -> numpy uint16 bit patterns (host copy)."""
    return x.detach().contiguous().view(torch.int16).cpu().numpy().view("uint16")


def oracle_views(cfg: EvictConfig, inp: dict, units=None) -> dict:
    """Unit-major numpy copies of the inputs for the oracle, optionally only
    for the listed units u = (l * B + b) * Hkv + g."""
    L, B, Hq, Hkv, d = cfg.n_layers, cfg.batch, cfg.hq, cfg.hkv, cfg.d
    G = cfg.G
    U = L * B * Hkv
    units = list(range(U)) if units is None else list(units)
    bad = [u for u in units if not 0 <= u < U]
    if bad:   # checked here, before any device gather reads with them
        raise IndexError(f"unit indices outside [0, {U}): {bad[:5]}")
    ut = torch.tensor(units, dtype=torch.long, device=inp["K"].device)
    K = inp["K"].reshape(U, -1, d).index_select(0, ut)
    V = inp["V"].reshape(U, -1, d).index_select(0, ut)
    qbuf = inp["qbuf"].reshape(U, G, cfg.qcap, d).index_select(0, ut)
    qcount = inp["qcount"].reshape(U, G).index_select(0, ut)
    q_recent = inp["q_recent"].reshape(U, G, cfg.n_recent_q, d).index_select(0, ut)
    b_of = [(u // Hkv) % B for u in units]
    bt = torch.tensor(b_of, dtype=torch.long, device=inp["t"].device)
    return {
        "K": to_u16(K), "V": to_u16(V), "qbuf": to_u16(qbuf),
        "qcount": qcount.cpu().numpy().astype("int32").copy(),
        "q_recent": to_u16(q_recent),
        "pos_recent": inp["pos_recent"].index_select(0, bt).cpu().numpy().astype("int32").copy(),
        "t": inp["t"].index_select(0, bt).cpu().numpy().astype("int32").copy(),
        "units": units,
    }
