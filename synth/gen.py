"""Seeded synthetic Q/K/V for the five layer shapes.

Input creation only: this module holds none of the method's arithmetic (no
rotary embedding, no softmax, no selection).  Both the HIP path and the fp64
oracle consume exactly the tensors made here.

Recipe (all magnitudes are stated as the logit excess E over the background,
whose standard deviation is 1 at the 1/sqrt(D) scale):

* noise: V iid N(0, 1); Q and K iid N(0, 1) under the planted components
  (the config's qk_noise scales it: 0.5 for the refinement-stress layer,
  whose recall calibration needs flatter far-field logits); bf16 configs are
  rounded to bf16 (torch's round-to-nearest-even), the tiny config stays fp32
  (the library rounds it on entry);
* "sinks_band" / "sinks_every" (7B/14B-shaped layers): per KV head a unit
  sink direction u in the four lowest-frequency rotary planes (planes
  D/2-4 .. D/2-1, both halves), added with amplitude sqrt(E_sink sqrt(D)) to
  the sink keys and, scaled by a per-query-head factor, to every query; and a
  band component b_t with equal weight in rotary planes 10..47, added to
  query and key t of the KV head (amplitude sqrt(E_band sqrt(D)), per-head
  factor on the query side).  In plane p, b_t has the phase phi_{t,p}, a
  Gaussian random walk along t (step variance 2 / BAND_DRIFT) from a random
  start: slowly drifting shared content.  After rotation, q_i.k_j of the band
  is a sum over planes of cos((i - j) theta_p + phi_{i,p} - phi_{j,p}): it
  peaks on the main diagonal and fades both as the planes decohere with
  distance and as the content drifts (mean factor exp(-|i - j| / BAND_DRIFT)),
  a local band of slash lines with no coherent far-range ripple.  Sinks sit
  at columns 0..15, or at multiples of `sink_every`;
* "far_sinks_stripes" (refinement stress): 64 sinks per KV head at seeded
  uniform positions (sink direction spread over the eight lowest-frequency
  planes, which halves the bf16 rounding error of the large sink logits),
  plus periodic diagonal stripes: a harmonic code
  c(a) = (cos(2 pi k a / P), sin(2 pi k a / P))_{k=1..8} / sqrt(8) in rotary
  planes 48..55 added to key j with a = j mod P and to query i with
  a = i mod P, so q.k peaks where i - j is a multiple of P.  The period P
  cycles over (64, 96, 128, 192, 256, 512, 1024, 2048) by KV head; the
  per-query-head stripe factor varies, so some heads are well covered by the
  base budget and some are not.  Sink excess 9 (the config's
  far_sink_excess), stripe excess 4, Q/K noise 0.5: about a quarter of the
  heads reach a recall of 0.9 at the base budget and the rest fall below it
  (measured on the last chunk, 128 rows); weaker sinks leave every head far
  below 0.9, much stronger ones lift almost every head above it;
* "none" (tiny): noise only.
"""

import math

import numpy as np
import torch

E_SINK = 3.0
E_BAND = 4.0
BAND_DRIFT = 32768.0
E_STRIPE = 4.0
BAND_PLANES = (10, 48)
SINK_PLANES = 4
FAR_SINK_PLANES = 8
STRIPE_PLANES = (48, 56)
STRIPE_PERIODS = (64, 96, 128, 192, 256, 512, 1024, 2048)
N_FAR_SINKS = 64


def _rng(cfg, *tags):
    return np.random.default_rng([cfg.seed] + [int(t) for t in tags])


def _torch_seed(cfg, *tags):
    return int(np.random.SeedSequence([cfg.seed] + [int(t) for t in tags])
               .generate_state(1, dtype=np.uint64)[0] & 0x7FFFFFFFFFFFFFFF)


def _plane_dims(d, planes):
    half = d // 2
    lo, hi = planes
    return np.arange(lo, hi), np.arange(lo, hi) + half


def _band_component(cfg, g, n, device):
    """Unit-norm band vector of every token, [n, D] fp32 on `device`."""
    d = cfg.head_dim
    a, b = _plane_dims(d, BAND_PLANES)
    rng = _rng(cfg, 101, g)
    start = torch.tensor(rng.uniform(0, 2 * math.pi, a.size), dtype=torch.float64,
                         device=device)
    steps = _noise((n, a.size), _torch_seed(cfg, 105, g), device).double()
    steps *= math.sqrt(2.0 / BAND_DRIFT)
    phase = start + torch.cumsum(steps, dim=0)
    comp = torch.zeros((n, d), dtype=torch.float32, device=device)
    comp[:, a] = (torch.cos(phase) / math.sqrt(a.size)).float()
    comp[:, b] = (torch.sin(phase) / math.sqrt(a.size)).float()
    return comp


def _sink_direction(cfg, g):
    d = cfg.head_dim
    rng = _rng(cfg, 102, g)
    n_planes = FAR_SINK_PLANES if cfg.planting == "far_sinks_stripes" else SINK_PLANES
    a, b = _plane_dims(d, (d // 2 - n_planes, d // 2))
    u = np.zeros(d)
    u[a] = rng.normal(size=a.size)
    u[b] = rng.normal(size=b.size)
    return u / np.linalg.norm(u)


def _stripe_codes(cfg, g, positions):
    """Harmonic stripe code for each position, [n, D] (float64)."""
    d = cfg.head_dim
    period = STRIPE_PERIODS[g % len(STRIPE_PERIODS)]
    a, b = _plane_dims(d, STRIPE_PLANES)
    k = np.arange(1, a.size + 1)
    ph = 2 * math.pi * np.outer(np.asarray(positions) % period, k) / period
    code = np.zeros((len(positions), d))
    code[:, a] = np.cos(ph)
    code[:, b] = np.sin(ph)
    return code / math.sqrt(a.size)


def sink_positions(cfg, g):
    """Key columns planted as sinks for KV head g."""
    n = cfg.seq_len
    if cfg.planting == "sinks_band":
        return np.arange(min(16, n))
    if cfg.planting == "sinks_every":
        return np.arange(0, n, cfg.sink_every)[:16]
    if cfg.planting == "far_sinks_stripes":
        rng = _rng(cfg, 103, g)
        return np.sort(rng.choice(n, size=min(N_FAR_SINKS, n), replace=False))
    return np.zeros(0, dtype=np.int64)


def head_factors(cfg):
    """Per-query-head multipliers of the planted excess, [H] each."""
    rng = _rng(cfg, 104)
    return {"band": rng.uniform(0.6, 1.2, cfg.n_heads),
            "sink": rng.uniform(0.8, 1.2, cfg.n_heads),
            "stripe": rng.uniform(0.0, 1.2, cfg.n_heads)}


def _amp(excess, d):
    return math.sqrt(excess * math.sqrt(d))


def _noise(shape, seed, device):
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    return torch.randn(shape, generator=g, device=device, dtype=torch.float32)


def generate(cfg, device="cpu", n_tokens=None):
    """Q [H, N, D], K [H_kv, N, D], V [H_kv, N, D] on `device`.

    fp32 for the tiny config (made with numpy, identical on every device),
    bf16 otherwise (made with torch's seeded generator on `device`).
    n_tokens < seq_len keeps the recipe of the full layer but stops early.
    """
    n = cfg.seq_len if n_tokens is None else int(n_tokens)
    H, G, D = cfg.n_heads, cfg.n_kv_heads, cfg.head_dim
    if cfg.in_dtype == "fp32":
        rng = _rng(cfg, 1)
        q = rng.standard_normal((H, n, D), dtype=np.float32)
        k = rng.standard_normal((G, n, D), dtype=np.float32)
        v = rng.standard_normal((G, n, D), dtype=np.float32)
        if cfg.planting != "none":
            raise ValueError("planting is defined for bf16 layers only")
        return (torch.from_numpy(q).to(device), torch.from_numpy(k).to(device),
                torch.from_numpy(v).to(device))

    fac = head_factors(cfg)
    out_q = torch.empty((H, n, D), dtype=torch.bfloat16, device=device)
    out_k = torch.empty((G, n, D), dtype=torch.bfloat16, device=device)
    out_v = torch.empty((G, n, D), dtype=torch.bfloat16, device=device)
    group = H // G
    for g in range(G):
        k = _noise((n, D), _torch_seed(cfg, 2, g), device) * cfg.qk_noise
        per_head_q = []
        band = None
        if cfg.planting in ("sinks_band", "sinks_every"):
            band = _band_component(cfg, g, n, device)
            u = torch.tensor(_sink_direction(cfg, g), dtype=torch.float32,
                             device=device)
            k += _amp(E_BAND, D) * band
            sp = sink_positions(cfg, g)
            sinks = torch.as_tensor(sp[sp < n], device=device)
            k[sinks] += _amp(E_SINK, D) * u
            for hh in range(group):
                h = g * group + hh
                per_head_q.append(_amp(E_SINK, D) * float(fac["sink"][h]) * u)
        elif cfg.planting == "far_sinks_stripes":
            u = torch.tensor(_sink_direction(cfg, g), dtype=torch.float32,
                             device=device)
            sp = sink_positions(cfg, g)
            sinks = torch.as_tensor(sp[sp < n], device=device)
            # the sink keys carry exactly the planted amplitude along u
            ks = k[sinks]
            k[sinks] = ks - (ks @ u)[:, None] * u + _amp(cfg.far_sink_excess, D) * u
            period = STRIPE_PERIODS[g % len(STRIPE_PERIODS)]
            codes = torch.tensor(_stripe_codes(cfg, g, np.arange(period)),
                                 dtype=torch.float32, device=device)
            idx = torch.arange(n, device=device) % period
            k += _amp(E_STRIPE, D) * codes[idx]
            for hh in range(group):
                h = g * group + hh
                per_head_q.append(_amp(cfg.far_sink_excess, D) * float(fac["sink"][h]) * u)
        out_k[g] = k.to(torch.bfloat16)
        del k
        out_v[g] = _noise((n, D), _torch_seed(cfg, 3, g), device).to(
            torch.bfloat16)
        for hh in range(group):
            h = g * group + hh
            q = _noise((n, D), _torch_seed(cfg, 1, h), device) * cfg.qk_noise
            if per_head_q:
                q += per_head_q[hh]
            if band is not None:
                q += (_amp(E_BAND, D) * float(fac["band"][h])) * band
            if cfg.planting == "far_sinks_stripes":
                q += (_amp(E_STRIPE, D) * float(fac["stripe"][h])) * codes[idx]
            out_q[h] = q.to(torch.bfloat16)
            del q
        del band
    return out_q, out_k, out_v
