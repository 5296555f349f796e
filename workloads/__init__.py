"""Seeded synthetic inputs for the MALA operator (forward, backward, split-KV decode).

This module only draws random numbers and arranges them into tensors. It holds
none of the operator's arithmetic, so both the CPU oracle and the GPU library's
tests and benchmark can take their inputs from it.

Recipe (the same on every device; the numbers differ between a CPU and a GPU
generator, so a test always hands the oracle the exact tensors the GPU saw):

* one ``torch.Generator`` per drawn tensor, seeded with ``seed * 64 + tag``
  (tags: Q=1, K=2, V=3, dO=4, temperature=5, planting=6, Rademacher probe=7), seed defaulting to
  ``20260000 + config id``; decode sequence ``b`` adds ``1000 * b`` to the seed;
* Q, K, V, dO ~ N(0, 1), layout [B, H, N, d] with d contiguous, drawn in fp32;
* a per-query-head temperature T_h ~ U(lo, hi) is folded into Q before rounding
  (Q'_h = T_h * Q_h); the tiny fp32 config instead multiplies Q by a fixed
  factor so that the logits have standard deviation about 3;
* planted high-affinity keys: for every query head h, ``planted`` pairs
  (k, q') with k ~ U{0..L-2} and q' ~ U{k+1..L-1}; key row k of h's KV head is
  overwritten with 4 * Q'[h, q'] / ||Q'[h, q']|| (unit-norm reading of
  "normalised"), heads in order and pairs in draw order, later writes winning;
* bf16 configs round Q', K, V, dO to bf16 (round to nearest even) after
  planting; both sides read the rounded values.
"""
from __future__ import annotations

import dataclasses
import math
from typing import Optional, Sequence

import torch

TAG_Q, TAG_K, TAG_V, TAG_DO, TAG_T, TAG_PLANT, TAG_PROBE = 1, 2, 3, 4, 5, 6, 7


@dataclasses.dataclass(frozen=True)
class PrefillConfig:
    cid: int
    name: str
    batch: int
    hq: int
    hkv: int
    n: int
    d: int
    dtype: str                      # "f32" or "bf16"
    planted: int
    taus: Sequence[float]
    q_mult: Optional[float] = None  # fixed multiplier on Q (fp32 tiny config)
    temp: Optional[tuple] = None    # (lo, hi) of the per-head temperature


@dataclasses.dataclass(frozen=True)
class DecodeConfig:
    cid: int
    name: str
    batch: int
    hq: int
    hkv: int
    cache: int       # positions in the cache before the first decode step
    steps: int       # decode steps; step t has n_k = cache + t + 1
    d: int
    dtype: str
    planted: int
    chunk: int
    tau: float
    temp: tuple = (1.0, 4.0)


CONFIGS = {
    1: PrefillConfig(1, "tiny_causal_fp32_L256", 1, 2, 2, 256, 64, "f32", 8,
                     (1e-4, 0.0, 1.0, 2.0, 10.0, 1e3), q_mult=3.0),
    2: PrefillConfig(2, "prefill_8k_bf16_h16", 1, 16, 16, 8192, 128, "bf16", 64,
                     (1e-4,), temp=(1.0, 4.0)),
    3: PrefillConfig(3, "prefill_32k_bf16_gqa32x8", 1, 32, 8, 32768, 128, "bf16", 256,
                     (0.0, 1e-5, 1e-4, 1e-3), temp=(1.0, 4.0)),
    4: PrefillConfig(4, "prefill_128k_bf16_gqa8x1", 1, 8, 1, 131072, 128, "bf16", 1024,
                     (1e-4,), temp=(1.0, 4.0)),
    5: DecodeConfig(5, "decode_128k_bf16_b8_gqa8x1", 8, 8, 1, 131072, 64, 128, "bf16",
                    1024, 256, 1e-4),
}


def default_seed(cid: int) -> int:
    return 20260000 + cid


def _gen(device, seed: int, tag: int) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(seed * 64 + tag)
    return g


def _randn(shape, device, seed, tag):
    return torch.randn(shape, generator=_gen(device, seed, tag), device=device,
                       dtype=torch.float32)


def planting_pairs(n: int, count: int, device, seed: int, head: int):
    """(k, q') pairs for one query head: k ~ U{0..n-2}, q' ~ U{k+1..n-1}.

    Draws 2*count uniforms in fp64 from the planting stream (the stream is
    shared by all heads; head h uses draws [2*count*h, 2*count*(h+1))).
    Returned as CPU int64 tensors in draw order.
    """
    if count == 0 or n < 2:
        z = torch.zeros(0, dtype=torch.int64)
        return z, z
    g = _gen("cpu", seed, TAG_PLANT)
    u = torch.rand((head + 1) * 2 * count, generator=g, dtype=torch.float64)[-2 * count:]
    u1, u2 = u[:count], u[count:]
    k = torch.clamp((u1 * (n - 1)).floor().to(torch.int64), max=n - 2)
    span = (n - 1 - k).to(torch.float64)
    qp = k + 1 + torch.minimum((u2 * span).floor().to(torch.int64), (n - 2 - k))
    return k, qp


def _plant(q: torch.Tensor, k: torch.Tensor, count: int, seed: int):
    """Overwrite planted key rows in place. q: [B, Hq, N, d] fp32 (after the
    temperature fold), k: [B, Hkv, N, d] fp32."""
    b_, hq, n, d = q.shape
    hkv = k.shape[1]
    group = hq // hkv
    for b in range(b_):
        for h in range(hq):
            ks, qs = planting_pairs(n, count, "cpu", seed, h)
            if ks.numel() == 0:
                continue
            # later writes win: keep the last occurrence of every key row
            last = {}
            for idx, kk in enumerate(ks.tolist()):
                last[kk] = idx
            order = sorted(last.values())
            ksel = ks[order].to(q.device)
            qsel = qs[order].to(q.device)
            rows = q[b, h].index_select(0, qsel)
            rows = 4.0 * rows / rows.norm(dim=-1, keepdim=True)
            k[b, h // group].index_copy_(0, ksel, rows)


def _cast(x: torch.Tensor, dtype: str) -> torch.Tensor:
    if dtype == "bf16":
        return x.to(torch.bfloat16)
    return x.contiguous()


def make_prefill(cfg: PrefillConfig, *, seed: Optional[int] = None, device="cpu",
                 n: Optional[int] = None, hq: Optional[int] = None,
                 hkv: Optional[int] = None, d: Optional[int] = None,
                 batch: Optional[int] = None, planted: Optional[int] = None,
                 with_do: bool = True) -> dict:
    """Inputs of one prefill/training problem. Overrides shrink a config for
    tests while keeping its value distribution and structure."""
    seed = default_seed(cfg.cid) if seed is None else seed
    n = cfg.n if n is None else n
    hq = cfg.hq if hq is None else hq
    hkv = cfg.hkv if hkv is None else hkv
    d = cfg.d if d is None else d
    batch = cfg.batch if batch is None else batch
    planted = cfg.planted if planted is None else planted
    q = _randn((batch, hq, n, d), device, seed, TAG_Q)
    k = _randn((batch, hkv, n, d), device, seed, TAG_K)
    v = _randn((batch, hkv, n, d), device, seed, TAG_V)
    do = _randn((batch, hq, n, d), device, seed, TAG_DO) if with_do else None
    temps = None
    if cfg.temp is not None:
        lo, hi = cfg.temp
        temps = lo + (hi - lo) * torch.rand(hq, generator=_gen("cpu", seed, TAG_T),
                                            dtype=torch.float32)
        q = q * temps.to(device).view(1, hq, 1, 1)
    elif cfg.q_mult is not None:
        q = q * cfg.q_mult
    _plant(q, k, planted, seed)
    out = dict(q=_cast(q, cfg.dtype), k=_cast(k, cfg.dtype), v=_cast(v, cfg.dtype),
               do=_cast(do, cfg.dtype) if do is not None else None,
               scale=1.0 / math.sqrt(d), temps=temps, dtype=cfg.dtype)
    return out


def rademacher(shape, *, seed: int, device="cpu", dtype: str = "bf16") -> torch.Tensor:
    """A deterministic Rademacher probe: entries -1 or +1 with probability 1/2
    each, from their own stream (tag 7). It is the dO direction of the
    gradient-fidelity measurements (App. C.3 uses such a probe)."""
    u = torch.rand(shape, generator=_gen(device, seed, TAG_PROBE), device=device,
                   dtype=torch.float32)
    return _cast(torch.where(u < 0.5, -1.0, 1.0), dtype)


def make_decode(cfg: DecodeConfig, *, seed: Optional[int] = None, device="cpu",
                cache: Optional[int] = None, steps: Optional[int] = None,
                batch: Optional[int] = None, hq: Optional[int] = None,
                hkv: Optional[int] = None, planted: Optional[int] = None) -> dict:
    """KV caches and decode queries. Sequence b is generated like a prefill
    problem of length cache+steps with seed + 1000*b; its K/V rows fill cache
    slot b and its last ``steps`` query rows are the decode queries."""
    seed = default_seed(cfg.cid) if seed is None else seed
    cache = cfg.cache if cache is None else cache
    steps = cfg.steps if steps is None else steps
    batch = cfg.batch if batch is None else batch
    hq = cfg.hq if hq is None else hq
    hkv = cfg.hkv if hkv is None else hkv
    planted = cfg.planted if planted is None else planted
    total = cache + steps
    pre = PrefillConfig(cfg.cid, cfg.name, 1, hq, hkv, total, cfg.d, cfg.dtype,
                        planted, (cfg.tau,), temp=cfg.temp)
    ks, vs, qs = [], [], []
    for b in range(batch):
        x = make_prefill(pre, seed=seed + 1000 * b, device=device, with_do=False)
        ks.append(x["k"][0])
        vs.append(x["v"][0])
        qs.append(x["q"][0, :, cache:].contiguous())  # [Hq, steps, d]
        del x
    k = torch.stack(ks)                       # [B, Hkv, total, d]
    v = torch.stack(vs)
    q = torch.stack(qs).permute(2, 0, 1, 3).contiguous()   # [steps, B, Hq, d]
    return dict(k_cache=k, v_cache=v, q_steps=q, cache=cache, steps=steps,
                scale=1.0 / math.sqrt(cfg.d), dtype=cfg.dtype, chunk=cfg.chunk)


def make_structured(n: int, hq: int = 2, hkv: int = 1, d: int = 128, *, seed: int = 20269001,
                    device="cpu", dtype: str = "bf16", freqs: int = 48, peak: float = 25.0,
                    window: int = 128, n_sink: int = 4, sink_logit: float = 18.0,
                    retrieval: int = 16, retrieval_logit: float = 22.0,
                    noise: float = 0.3, batch: int = 1, with_do: bool = True) -> dict:
    """Structured-logit inputs whose attention mass concentrates the way the
    paper describes real attention (sink tokens, a local band and sparse
    retrieval keys), so that the tolerance actually skips tiles.

    Logit of query t and key s (scale 1/sqrt(d) included):
      peak/F * sum_f cos(w_f (t - s))    local band: F = ``freqs`` rotary pairs,
                                         periods log-uniform in [4, 64] x window
      + sink_logit                       for s < n_sink
      + retrieval_logit                  for ``retrieval`` planted (s, t) pairs
                                         per query head
      + noise                            N(0, noise^2) in the remaining dims
    """
    assert 2 * freqs + 8 <= d
    g = _gen(device, seed, TAG_Q)
    scale = 1.0 / math.sqrt(d)
    pos = torch.arange(n, device=device, dtype=torch.float64)
    periods = window * torch.exp(torch.linspace(math.log(4.0), math.log(64.0), freqs,
                                                dtype=torch.float64, device=device))
    w = 2 * math.pi / periods
    ang = pos[:, None] * w[None, :]                     # [n, F]
    rot = torch.stack([torch.cos(ang), torch.sin(ang)], -1).reshape(n, 2 * freqs)
    # every logit term is split evenly between Q and K (each carries the
    # square root), so neither side holds outsized components
    amp = math.sqrt(peak / freqs / scale)
    q = torch.zeros((batch, hq, n, d), dtype=torch.float64, device=device)
    k = torch.zeros((batch, hkv, n, d), dtype=torch.float64, device=device)
    q[..., : 2 * freqs] = amp * rot
    k[..., : 2 * freqs] = amp * rot
    # sinks: one shared direction
    sdim = 2 * freqs
    q[..., sdim] = math.sqrt(sink_logit / scale)
    k[:, :, :n_sink, sdim] = math.sqrt(sink_logit / scale)
    # noise in the remaining dims
    rest = d - (sdim + 1)
    qn = torch.randn((batch, hq, n, rest), generator=g, device=device, dtype=torch.float32)
    kn = torch.randn((batch, hkv, n, rest), generator=_gen(device, seed, TAG_K), device=device,
                     dtype=torch.float32)
    nscale = math.sqrt(noise / math.sqrt(rest) / scale)
    q[..., sdim + 1:] = qn.double() * nscale
    k[..., sdim + 1:] = kn.double() * nscale
    # retrieval keys: key s gets a random unit direction u in the noise dims,
    # its target query t > s gets the same direction, each scaled so that the
    # pair adds retrieval_logit
    group = hq // hkv
    gp = _gen("cpu", seed, TAG_PLANT)
    ramp = math.sqrt(retrieval_logit / scale)
    for b in range(batch):
        for h in range(hq):
            if n < 2 or retrieval == 0:
                continue
            u = torch.rand((retrieval, 2), generator=gp, dtype=torch.float64)
            ss = (u[:, 0] * (n - 1)).floor().long().clamp(max=n - 2)
            tt = ss + 1 + (u[:, 1] * (n - 1 - ss).double()).floor().long()
            tt = torch.minimum(tt, torch.full_like(tt, n - 1))
            dirs = torch.randn((retrieval, rest), generator=gp, dtype=torch.float64)
            dirs = dirs / dirs.norm(dim=-1, keepdim=True)
            for r in range(retrieval):
                k[b, h // group, ss[r], sdim + 1:] += dirs[r].to(device) * ramp
                q[b, h, tt[r], sdim + 1:] += dirs[r].to(device) * ramp
    v = torch.randn((batch, hkv, n, d), generator=_gen(device, seed, TAG_V), device=device,
                    dtype=torch.float32)
    do = (torch.randn((batch, hq, n, d), generator=_gen(device, seed, TAG_DO), device=device,
                      dtype=torch.float32) if with_do else None)
    out = dict(q=_cast(q.float(), dtype), k=_cast(k.float(), dtype), v=_cast(v, dtype),
               do=_cast(do, dtype) if do is not None else None, scale=scale, dtype=dtype)
    return out


# Named parameter sets of make_structured. "sparse" (the defaults) keeps
# about 250 forward key slots per query at 32K and tau = 1: its mass sits
# harder on few keys than the paper's measurements. "calibrated" widens the
# local band (window 1088) so that tau = 1 keeps about 1,050 forward slots
# per query at 32K (about 900 at 8K and 540 at 1K), the operating point the
# paper reports for its trained model (1,010-1,066 slots per query beyond
# 8K; Sec. 3 "Operator Fidelity Across Context Lengths", App. C.5).
STRUCTURED_PRESETS = {
    "sparse": {},
    "calibrated": {"window": 1088},
}


def make_structured_preset(preset: str, n: int, **kw) -> dict:
    """make_structured with the named parameter set (keyword arguments
    override it)."""
    args = dict(STRUCTURED_PRESETS[preset])
    args.update(kw)
    return make_structured(n, **args)
