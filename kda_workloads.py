"""Seeded synthetic inputs for KDA prefill and decode.

Shared by the tests, the smoke check and the bench.  This module only draws
random inputs of the right shapes and value distributions; it holds none of
the method's arithmetic.  Everything is generated on the CPU with a seeded
``torch.Generator``, so the GPU path and the CPU oracle receive exactly the
same numbers (the caller copies them to the device).

Value recipes (the pool-mode test of sglang PR 30169's digest fixes the style:
q, k normalised in fp32 then cast, beta = sigmoid(N(0,1)), initial states
0.05 * N(0,1), random slots in a larger pool):

* q, k ~ N(0,1), L2-normalised over K in fp32, then cast to the io dtype.
* v ~ N(0,1) in the io dtype.
* beta = sigmoid(N(0,1)), fp32.
* per-channel log-gate  g = -exp(a_c) * softplus(x + dt_bias_c), with a_c and
  dt_bias_c fixed per (value head, channel) and x ~ N(0,1) per
  (token, value head, channel).  "moderate" gates: a_c ~ U(-1, 1),
  dt_bias_c = 0.  "realistic" gates: a_c ~ U(-1, 2.7),
  dt_c = exp(U(ln 1e-3, ln 64)), dt_bias_c = dt_c + ln(-expm1(-dt_c)) (the
  inverse softplus of dt_c), which drives in-chunk cumulative log-decays to
  the 1e3..6e4 range.
* scalar (GDN) gates: the same recipe with one value per (token, value head).

Raw gate inputs for the fused-gate entry points (the GDN pool-mode test of
sglang PR 30169's digest draws them this way: raw a, b in bf16, per-head
A_log and dt_bias in fp32): ``gx`` = x and ``bx`` = the N(0,1) draw behind
beta, both cast to the io dtype; ``A_log`` = a_c and ``dt_bias`` =
dt_bias_c in fp32.  They come from the same draws as g and beta (no extra
random numbers), but a kernel fed with them sees x and b rounded to the io
dtype, so its expected values are computed from these raw tensors, not from
g and beta.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field
from typing import Optional

import torch

DTYPES = {"bf16": torch.bfloat16, "f32": torch.float32}


def _gen(seed: int) -> torch.Generator:
    return torch.Generator().manual_seed(int(seed))


def unit_rows(gen, shape, dtype):
    """N(0,1) rows L2-normalised over the last axis in fp32, then cast."""
    x = torch.randn(*shape, generator=gen, dtype=torch.float32)
    x = x / x.norm(dim=-1, keepdim=True).clamp_min(1e-12)
    return x.to(dtype)


def gate_params(gen, hv, dk, kind):
    """Per-(value head, channel) gate parameters (a_c, dt_bias_c)."""
    if kind == "moderate":
        a = torch.rand(hv, dk, generator=gen) * 2.0 - 1.0
        dt_bias = torch.zeros(hv, dk)
    elif kind == "realistic":
        a = torch.rand(hv, dk, generator=gen) * 3.7 - 1.0
        lo, hi = math.log(1e-3), math.log(64.0)
        dt = torch.exp(torch.rand(hv, dk, generator=gen, dtype=torch.float64) * (hi - lo) + lo)
        dt_bias = (dt + torch.log(-torch.expm1(-dt))).float()
    else:
        raise ValueError(kind)
    return a, dt_bias


def log_gates(gen, T, hv, dk, kind="moderate", scalar=False):
    """g <= 0: [T, hv, dk] per channel, or [T, hv] for the scalar gate, and the
    raw draws it is made of: (g, x, a, dt_bias) with x [T, hv, dk] / [T, hv]
    and a, dt_bias [hv, dk] / [hv]."""
    width = 1 if scalar else dk
    a, dt_bias = gate_params(gen, hv, width, kind)
    x = torch.randn(T, hv, width, generator=gen)
    g = -torch.exp(a)[None] * torch.nn.functional.softplus(x + dt_bias[None])
    if scalar:
        return g[..., 0].contiguous(), x[..., 0].contiguous(), a[:, 0].contiguous(), \
            dt_bias[:, 0].contiguous()
    return g.contiguous(), x.contiguous(), a.contiguous(), dt_bias.contiguous()


def seq_lengths(gen, n, lo, hi):
    """n lengths uniform on the integers lo..hi inclusive."""
    return torch.randint(lo, hi + 1, (n,), generator=gen, dtype=torch.int32)


def cu_from_lengths(lengths):
    cu = torch.zeros(len(lengths) + 1, dtype=torch.int32)
    cu[1:] = torch.as_tensor(lengths, dtype=torch.int32).cumsum(0)
    return cu


@dataclass
class Prefill:
    q: torch.Tensor
    k: torch.Tensor
    v: torch.Tensor
    g: torch.Tensor
    beta: torch.Tensor
    cu_seqlens: torch.Tensor
    h0: Optional[torch.Tensor] = None          # dense [N, Hv, V, K]
    pool: Optional[torch.Tensor] = None        # [S, Hv, V, K]
    indices: Optional[torch.Tensor] = None     # [N] int32, -1 = padding
    scale: float = 1.0
    meta: dict = field(default_factory=dict)
    gx: Optional[torch.Tensor] = None          # raw gate input, io dtype, shape of g
    A_log: Optional[torch.Tensor] = None       # [Hv, K] or [Hv] fp32
    dt_bias: Optional[torch.Tensor] = None     # [Hv, K] or [Hv] fp32
    bx: Optional[torch.Tensor] = None          # raw beta input [T, Hv], io dtype

    @property
    def num_seqs(self):
        return self.cu_seqlens.numel() - 1


def make_prefill(seed, lengths, hk, hv, dk, dv, io="bf16", gate="moderate",
                 scalar_gate=False, h0=None, pool_slots=0, state_dtype="f32",
                 pad_one=False, scale=1.0):
    """Generic seeded prefill input.  ``lengths`` is a list of ints, or a tuple
    (n, lo, hi) for n lengths drawn uniformly from lo..hi.  ``h0`` is None
    (zeros), "random" (0.05*N(0,1)).  ``pool_slots`` > 0 builds a pool of that
    many random rows and per-sequence slot indices drawn without replacement
    from [0, pool_slots - 1); with ``pad_one`` the last index is -1."""
    gen = _gen(seed)
    dt = DTYPES[io]
    if isinstance(lengths, tuple):
        n, lo, hi = lengths
        lens = seq_lengths(gen, n, lo, hi)
    else:
        lens = torch.as_tensor(lengths, dtype=torch.int32)
    cu = cu_from_lengths(lens)
    T = int(cu[-1])
    n = len(lens)
    q = unit_rows(gen, (T, hk, dk), dt)
    k = unit_rows(gen, (T, hk, dk), dt)
    v = torch.randn(T, hv, dv, generator=gen).to(dt)
    b = torch.randn(T, hv, generator=gen)
    beta = torch.sigmoid(b)
    g, x, a, dt_bias = log_gates(gen, T, hv, dk, gate, scalar_gate)
    sd = DTYPES[state_dtype]
    inp = Prefill(q, k, v, g, beta, cu, scale=scale,
                  meta=dict(seed=seed, hk=hk, hv=hv, dk=dk, dv=dv, io=io, gate=gate,
                            scalar_gate=scalar_gate, state_dtype=state_dtype, T=T),
                  gx=x.to(dt), A_log=a.float(), dt_bias=dt_bias.float(), bx=b.to(dt))
    if h0 == "random":
        inp.h0 = (torch.randn(n, hv, dv, dk, generator=gen) * 0.05).to(sd)
    if pool_slots:
        inp.pool = (torch.randn(pool_slots, hv, dv, dk, generator=gen) * 0.05).to(sd)
        idx = torch.randperm(pool_slots - 1, generator=gen)[:n].to(torch.int32)
        if pad_one:
            idx[-1] = -1
        inp.indices = idx
    return inp


def single_seq_t128(seed=1):
    """One sequence of 128 tokens (two chunks), Hk=Hv=1, K=V=32, fp32 io,
    moderate per-channel gates, zero initial state."""
    return make_prefill(seed, [128], 1, 1, 32, 32, io="f32")


def varlen_gqa5(seed=2):
    """Five sequences, lengths U{1..130}, Hk=4, Hv=8, K=V=128, bf16 io,
    moderate gates, random fp32 initial states."""
    return make_prefill(seed, (5, 1, 130), 4, 8, 128, 128, h0="random")


def varlen_pool64(seed=11, state_dtype="f32"):
    """The shapes of varlen_gqa5 in pool mode: 64-slot pool, slots drawn without
    replacement from [0, 63), the last sequence's index set to -1 (sentinel
    slot 63)."""
    return make_prefill(seed, (5, 1, 130), 4, 8, 128, 128, pool_slots=64,
                        state_dtype=state_dtype, pad_one=True)


def kimi_prefill_16seq(seed=4):
    """Kimi-Linear-shaped prefill: 16 sequences, lengths U{512..4096},
    Hk=Hv=32, K=V=128, bf16 io, realistic gates, fp32 pool of 32 slots."""
    return make_prefill(seed, (16, 512, 4096), 32, 32, 128, 128, gate="realistic",
                        pool_slots=32)


def long_prompt_32k(seed=12):
    """One long prompt: a single sequence of 32,768 tokens, Hk=Hv=32,
    K=V=128, bf16 io, realistic gates, fp32 pool of 2 slots (32 chains, each
    512 chunks long)."""
    return make_prefill(seed, [32768], 32, 32, 128, 128, gate="realistic", pool_slots=2)


def gdn_pool_page(seed=11, state_dtype="f32", pad_one=False):
    """The GDN pool-mode test recipe of the sglang PR 30169 digest (key-code
    test): 5 sequences of randint(1, 130) tokens, Hk = 4, Hv = 8, K = V = 128,
    bf16 q, k (N(0,1) rounded to bf16, L2-normalised in fp32, rounded again)
    and v; raw a, b ~ N(0,1) in bf16 per (token, value head); A ~ U(0, 16),
    A_log = log A; dt log-uniform on [1e-3, 0.1] clamped at 1e-4, dt_bias its
    inverse softplus; the scalar gate g = -exp(A_log) softplus(a + dt_bias)
    and beta = sigmoid(b) in fp32; dense initial states 0.05 N(0,1) in the
    state dtype, scattered into a 64-slot pool of 0.05 N(0,1) rows at
    randperm(64)[:5].  The draws follow the page's order from one seeded CPU
    generator (the page draws on the GPU, whose stream differs).  With
    pad_one, the last sequence's index becomes -1 (the sentinel, last slot),
    whose row then holds that sequence's initial state."""
    gen = _gen(seed)
    n, hk, hv, d = 5, 4, 8, 128
    lens = torch.randint(1, 130, (n,), generator=gen, dtype=torch.int32)
    cu = cu_from_lengths(lens)
    T = int(cu[-1])
    bf = torch.bfloat16
    q = torch.randn(T, hk, d, generator=gen).to(bf)
    k = torch.randn(T, hk, d, generator=gen).to(bf)
    v = torch.randn(T, hv, d, generator=gen).to(bf)
    q = torch.nn.functional.normalize(q.float(), p=2, dim=-1).to(bf)
    k = torch.nn.functional.normalize(k.float(), p=2, dim=-1).to(bf)
    a = torch.randn(T, hv, generator=gen).to(bf)
    b = torch.randn(T, hv, generator=gen).to(bf)
    A = torch.rand(hv, generator=gen) * 16.0
    A_log = torch.log(A)
    lo, hi = math.log(1e-3), math.log(0.1)
    dt = torch.exp(torch.rand(hv, generator=gen) * (hi - lo) + lo).clamp_min(1e-4)
    dt_bias = dt + torch.log(-torch.expm1(-dt))
    g = -A_log.exp()[None] * torch.nn.functional.softplus(a.float() + dt_bias[None])
    beta = torch.sigmoid(b.float())
    sd = DTYPES[state_dtype]
    h0 = (torch.randn(n, hv, d, d, generator=gen) * 0.05).to(sd)
    num_slots = 64
    pool = (torch.randn(num_slots, hv, d, d, generator=gen) * 0.05).to(sd)
    slots = torch.randperm(num_slots, generator=gen)[:n].to(torch.int32)
    if pad_one:
        slots[-1] = -1
    rows = torch.where(slots < 0, torch.full_like(slots, num_slots - 1), slots).long()
    pool[rows] = h0
    return Prefill(q, k, v, g.contiguous(), beta.contiguous(), cu, h0=h0, pool=pool, indices=slots,
                   meta=dict(seed=seed, hk=hk, hv=hv, dk=d, dv=d, io="bf16", gate="gdn-page",
                             scalar_gate=True, state_dtype=state_dtype, T=T),
                   gx=a, A_log=A_log.float(), dt_bias=dt_bias.float(), bx=b)


@dataclass
class Decode:
    q: torch.Tensor
    k: torch.Tensor
    v: torch.Tensor
    g: torch.Tensor
    beta: torch.Tensor
    pool: torch.Tensor
    indices: torch.Tensor
    scale: float = 1.0
    meta: dict = field(default_factory=dict)
    gx: Optional[torch.Tensor] = None          # raw gate input, io dtype, shape of g
    A_log: Optional[torch.Tensor] = None       # [Hv, K] or [Hv] fp32
    dt_bias: Optional[torch.Tensor] = None     # [Hv, K] or [Hv] fp32
    bx: Optional[torch.Tensor] = None          # raw beta input [B, Hv], io dtype


def make_decode(seed, batch, hk, hv, dk, dv, num_slots, io="bf16", gate="realistic",
                scalar_gate=False, state_dtype="f32", pad=0, scale=1.0):
    """``batch`` one-token requests over a pool of ``num_slots`` rows; slot
    indices are a random permutation of [0, num_slots - 1) cut to ``batch``
    (the sentinel slot num_slots-1 is never drawn); the last ``pad`` indices
    are set to -1."""
    gen = _gen(seed)
    dt = DTYPES[io]
    q = unit_rows(gen, (batch, hk, dk), dt)
    k = unit_rows(gen, (batch, hk, dk), dt)
    v = torch.randn(batch, hv, dv, generator=gen).to(dt)
    braw = torch.randn(batch, hv, generator=gen)
    beta = torch.sigmoid(braw)
    g, x, a, dt_bias = log_gates(gen, batch, hv, dk, gate, scalar_gate)
    assert batch <= num_slots - 1
    idx = torch.randperm(num_slots - 1, generator=gen)[:batch].to(torch.int32)
    if pad:
        idx[batch - pad:] = -1
    pool = torch.empty(num_slots, hv, dv, dk, dtype=DTYPES[state_dtype])
    # draw the pool row by row so a 8.7 GB pool never needs a second fp32 copy
    for s in range(num_slots):
        pool[s] = torch.randn(hv, dv, dk, generator=gen) * 0.05
    return Decode(q, k, v, g, beta, pool, idx, scale,
                  meta=dict(seed=seed, batch=batch, hk=hk, hv=hv, dk=dk, dv=dv, io=io,
                            state_dtype=state_dtype, num_slots=num_slots),
                  gx=x.to(dt), A_log=a.float(), dt_bias=dt_bias.float(), bx=braw.to(dt))


def decode_b4096(seed=5, batch=4096, num_slots=4160):
    """Recurrent decode: 4096 one-token requests, Hk=Hv=32, K=V=128, bf16 io,
    realistic gates, fp32 pool of 4160 slots."""
    return make_decode(seed, batch, 32, 32, 128, 128, num_slots)


@dataclass
class MultiDecode:
    """Multi-token decode: request n owns tokens [cu[n], cu[n+1]) of the packed
    token arrays (``tok``, a Prefill without states) and pool row indices[n]."""
    tok: Prefill
    pool: torch.Tensor
    indices: torch.Tensor
    cache_pitch: int
    meta: dict = field(default_factory=dict)


def make_multi_decode(seed, lengths, hk, hv, dk, dv, num_slots, cache_pitch, io="bf16",
                      gate="realistic", scalar_gate=False, state_dtype="f32", pad=0, scale=1.0):
    """Draft/verify batch: ``lengths`` tokens per request (list, or (n, lo, hi)),
    a pool of ``num_slots`` random rows, slot indices drawn without replacement
    from [0, num_slots - 1) with the last ``pad`` set to -1, and the step pitch
    of the intermediate-state cache."""
    tok = make_prefill(seed, lengths, hk, hv, dk, dv, io=io, gate=gate, scalar_gate=scalar_gate,
                       scale=scale)
    gen = _gen(seed + 7919)
    n = tok.num_seqs
    assert n <= num_slots - 1
    idx = torch.randperm(num_slots - 1, generator=gen)[:n].to(torch.int32)
    if pad:
        idx[n - pad:] = -1
    pool = torch.empty(num_slots, hv, dv, dk, dtype=DTYPES[state_dtype])
    for s in range(num_slots):
        pool[s] = torch.randn(hv, dv, dk, generator=gen) * 0.05
    return MultiDecode(tok, pool, idx, cache_pitch,
                       meta=dict(seed=seed, batch=n, hk=hk, hv=hv, dk=dk, dv=dv, io=io,
                                 state_dtype=state_dtype, num_slots=num_slots, pitch=cache_pitch))


def spec_decode_b1024(seed=6, batch=1024, draft=4, num_slots=1088, cache_pitch=8):
    """Speculative verify step: 1024 requests of 4 tokens (the last accepted
    token plus 3 drafts), Hk=Hv=32, K=V=128, bf16 io, realistic gates, fp32
    pool of 1088 slots, intermediate-state cache pitch 8 steps."""
    return make_multi_decode(seed, [draft] * batch, 32, 32, 128, 128, num_slots, cache_pitch)
