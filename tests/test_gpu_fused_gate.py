"""GPU parity of the fused-gate entry points (kda_chunk_prefill_fused_gate,
kda_recurrent_decode_fused_gate) against the fp64 oracle, through the C ABI.

The kernels receive the raw projections x, b (io dtype) and fp32 A_log,
dt_bias and compute g = -exp(A_log) softplus(x + dt_bias), beta = sigmoid(b)
themselves; the oracle computes the same activation in fp64 from the same
raw tensors (oracle.gate_activation, oracle.sigmoid) and runs its recurrence.
"""
import math

import numpy as np
import pytest
import torch

import kda_workloads as W
from gpu_util import O_MAXABS, check_states, compare_decode_streamed, dev, host, max_abs, say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def K():
    import gated_delta_rule_51_amd as kda
    kda.lib()
    return kda


def raw(inp):
    return dev(inp.gx), dev(inp.A_log), dev(inp.dt_bias), dev(inp.bx)


def run_fused(K, inp, h0=None, pool=None, indices=None):
    init = dev(h0) if pool is None else pool
    o, ht = K.chunk_prefill_fused_gate(dev(inp.q), dev(inp.k), dev(inp.v), *raw(inp), dev(inp.cu_seqlens),
                                       initial_state=init, state_indices=indices, scale=inp.scale)
    torch.cuda.synchronize()
    return o, ht


def oracle_fused(oracle, inp, h0):
    return oracle.prefill_fused_gate(inp.q, inp.k, inp.v, inp.gx, inp.A_log, inp.dt_bias, inp.bx,
                                     inp.cu_seqlens, h0=h0, scale=inp.scale)


def check(name, o, ht, o_ref, ht_ref, state_bf16=False):
    og, hg = host(o), host(ht)
    assert np.isfinite(og).all() and np.isfinite(hg).all(), name
    e_o = max_abs(og, o_ref)
    say("%s: o max-abs %.3e" % (name, e_o))
    assert e_o <= O_MAXABS, name
    check_states(name, hg, ht_ref, bf16=state_bf16)


def test_fused_prefill_varlen_gqa(K, oracle):
    inp = W.make_prefill(201, (5, 1, 130), 4, 8, 128, 128, gate="realistic", h0="random")
    o, ht = run_fused(K, inp, h0=inp.h0)
    check("fused varlen gqa", o, ht, *oracle_fused(oracle, inp, inp.h0))


def page_head_params(seed, hv):
    """Per-head parameters drawn as in the GDN pool-mode test of the sglang
    PR 30169 digest: A ~ U(0, 16), A_log = log A, dt log-uniform on
    [1e-3, 1e-1] clamped at 1e-4, dt_bias = dt + log(-expm1(-dt))."""
    gen = torch.Generator().manual_seed(seed)
    A = torch.rand(hv, generator=gen) * 16.0
    lo, hi = math.log(1e-3), math.log(1e-1)
    dt = torch.exp(torch.rand(hv, generator=gen) * (hi - lo) + lo).clamp_min(1e-4)
    return torch.log(A), dt + torch.log(-torch.expm1(-dt))


def test_fused_prefill_scalar_gate_page_recipe(K, oracle):
    """GDN's scalar gate with the pages' per-head parameters: 5 sequences of
    1..129 tokens, Hk = 4, Hv = 8, K = V = 128, bf16 raw a and b."""
    inp = W.make_prefill(202, (5, 1, 129), 4, 8, 128, 128, scalar_gate=True, h0="random")
    inp.A_log, inp.dt_bias = page_head_params(11, 8)
    o, ht = run_fused(K, inp, h0=inp.h0)
    check("fused scalar page recipe", o, ht, *oracle_fused(oracle, inp, inp.h0))


@pytest.mark.parametrize("dk,dv,io", [(32, 32, "f32"), (64, 128, "bf16"), (128, 64, "f32"), (32, 128, "bf16")])
def test_fused_prefill_head_dims(K, oracle, dk, dv, io):
    inp = W.make_prefill(203 + dk + dv, [150, 64, 7], 1, 2, dk, dv, io=io, gate="realistic",
                         h0="random", scale=dk ** -0.5)
    o, ht = run_fused(K, inp, h0=inp.h0)
    check("fused dk=%d dv=%d %s" % (dk, dv, io), o, ht, *oracle_fused(oracle, inp, inp.h0))


def test_fused_prefill_saturated_inputs(K, oracle):
    """Raw inputs at +-40: softplus in its linear and exponentially small
    limits (decay to zero, no decay), beta at 0 and 1; nothing overflows."""
    inp = W.make_prefill(204, [100, 40], 2, 4, 128, 128, gate="moderate", h0="random")
    gen = torch.Generator().manual_seed(5)
    pick = torch.randint(0, 3, inp.gx.shape, generator=gen)
    inp.gx = torch.where(pick == 0, torch.full_like(inp.gx, 40.0),
                         torch.where(pick == 1, torch.full_like(inp.gx, -40.0), inp.gx))
    pb = torch.randint(0, 3, inp.bx.shape, generator=gen)
    inp.bx = torch.where(pb == 0, torch.full_like(inp.bx, 40.0),
                         torch.where(pb == 1, torch.full_like(inp.bx, -40.0), inp.bx))
    o, ht = run_fused(K, inp, h0=inp.h0)
    check("fused saturated", o, ht, *oracle_fused(oracle, inp, inp.h0))


def test_fused_pool_matches_dense_bitwise(K, oracle):
    inp = W.varlen_pool64()
    S = inp.pool.shape[0]
    slots = oracle.map_slot(inp.indices.numpy(), S)
    pool_before = inp.pool.clone()
    h0_dense = pool_before[torch.as_tensor(slots)]
    o_d, ht_d = run_fused(K, inp, h0=h0_dense)
    pool = dev(inp.pool)
    o_p, _ = run_fused(K, inp, pool=pool, indices=dev(inp.indices))
    assert torch.equal(o_p, o_d)
    sl = torch.as_tensor(slots).cuda()
    assert torch.equal(pool[sl], ht_d)
    untouched = torch.ones(S, dtype=torch.bool)
    untouched[torch.as_tensor(slots)] = False
    assert torch.equal(pool.cpu()[untouched], pool_before[untouched])
    check("fused pool", o_p, pool[sl], *oracle_fused(oracle, inp, h0_dense))


def test_fused_kimi_shaped_full(K, oracle):
    """The Kimi-shaped prefill (16 sequences of 512..4096 tokens, 32 heads,
    K = V = 128, realistic gates, fp32 pool) from raw gate inputs; every
    output and written row compared."""
    say("generating prefill workload (16 seqs, 512..4096 tokens, 32 heads)")
    inp = W.kimi_prefill_16seq()
    S = inp.pool.shape[0]
    slots = oracle.map_slot(inp.indices.numpy(), S)
    pool_before = inp.pool.clone()
    pool = dev(inp.pool)
    o, _ = run_fused(K, inp, pool=pool, indices=dev(inp.indices))
    o_ref, ht_ref = oracle_fused(oracle, inp, pool_before[torch.as_tensor(slots)])
    check("fused kimi_prefill_16seq", o, pool[torch.as_tensor(slots).cuda()], o_ref, ht_ref)


# ---------------------------------------------------------------------------
# decode
# ---------------------------------------------------------------------------

def check_decode(K, oracle, d, scale=1.0):
    """Every request against the oracle (activation in fp64 from the same raw
    inputs), streamed; every row that is not indexed bitwise."""
    S = d.pool.shape[0]
    slots = oracle.map_slot(d.indices.numpy(), S)
    pool_before = d.pool.clone()
    pool = dev(d.pool)
    o = K.recurrent_decode_fused_gate(dev(d.q), dev(d.k), dev(d.v), dev(d.gx), dev(d.A_log),
                                      dev(d.dt_bias), dev(d.bx), pool, dev(d.indices), scale=scale)
    torch.cuda.synchronize()
    compare_decode_streamed(oracle, d, o, pool, pool_before, slots,
                            lambda r: oracle.gate_activation(d.gx[r], d.A_log, d.dt_bias),
                            lambda r: oracle.sigmoid(d.bx[r]), scale, "fused decode")
    untouched = torch.as_tensor(np.setdiff1d(np.arange(S), slots))
    assert torch.equal(pool[untouched.cuda()].cpu(), pool_before[untouched])


@pytest.mark.parametrize("dk,dv,io,state", [(128, 128, "bf16", "f32"), (64, 64, "f32", "f32"),
                                            (32, 128, "bf16", "bf16"), (128, 32, "f32", "bf16")])
def test_fused_decode_small(K, oracle, dk, dv, io, state):
    d = W.make_decode(300 + dk + dv, 37, 2, 4, dk, dv, num_slots=50, io=io, state_dtype=state, pad=1)
    check_decode(K, oracle, d, scale=dk ** -0.5)


def test_fused_decode_scalar_gate_page_recipe(K, oracle):
    d = W.make_decode(310, 24, 4, 8, 128, 128, num_slots=30, scalar_gate=True)
    d.A_log, d.dt_bias = page_head_params(12, 8)
    check_decode(K, oracle, d)


def test_fused_decode_full_size_all_requests(K, oracle):
    """B = 4096 requests, Hv = 32, K = V = 128, fp32 pool of 4160 slots; every
    request checked against the oracle (streamed), untouched rows bitwise."""
    say("generating decode workload B=4096 Hv=32 pool 4160 slots")
    d = W.decode_b4096()
    check_decode(K, oracle, d)
