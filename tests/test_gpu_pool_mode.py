"""Pool mode against dense mode, bit for bit, through the C ABI:

* the GDN pool-mode test of the sglang PR 30169 digest (key-code test
  ``test_gdn_chunk_cutedsl_pool_mode_matches_dense``), ported: seed 11, five
  sequences, GDN's scalar gate from the page's A / dt recipe, bf16 and fp32
  pools; the same o, the final states at the indexed rows, every other row
  untouched, and ``final_state is pool``;
* the same recipe with one index set to -1 (the sentinel, last slot);
* the same recipe through the fused-gate entry point (raw a and b);
* more than 256 (sequence, head) chains of sequences longer than 1024 tokens
  on average, where the state kernel runs both column parts of a chain in one
  sixteen-wave workgroup, with a bf16 pool and with fp32 io;
* 65 to 256 chains, and more than 256 chains of shorter sequences, where each
  column part is a workgroup of its own, with the same two variants (the
  four-part form for at most 64 chains is covered by the five-sequence
  recipes above).

Each pool-mode result is also held to the oracle's tolerances.
"""
import numpy as np
import pytest
import torch

import kda_workloads as W
from gpu_util import O_MAXABS, check_states, dev, host, max_abs, say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def K():
    import gated_delta_rule_51_amd as kda
    kda.lib()
    return kda


def pool_vs_dense(K, oracle, inp, name, fused=False):
    """Dense call from the indexed rows, then the pool call in place; both
    checked bitwise against each other and against the oracle."""
    S = inp.pool.shape[0]
    slots = oracle.map_slot(inp.indices.numpy(), S)
    sl = torch.as_tensor(slots)
    pool_before = inp.pool.clone()
    h0_dense = pool_before[sl].clone()
    args = (dev(inp.q), dev(inp.k), dev(inp.v))
    if fused:
        fn = K.chunk_prefill_fused_gate
        gate = (dev(inp.gx), dev(inp.A_log), dev(inp.dt_bias), dev(inp.bx))
    else:
        fn = K.chunk_prefill
        gate = (dev(inp.g), dev(inp.beta))
    o_d, ht_d = fn(*args, *gate, dev(inp.cu_seqlens), initial_state=dev(h0_dense), scale=inp.scale)
    pool = dev(inp.pool)
    o_p, ht_p = fn(*args, *gate, dev(inp.cu_seqlens), initial_state=pool, state_indices=dev(inp.indices),
                   scale=inp.scale)
    torch.cuda.synchronize()
    assert ht_p is pool, name
    assert torch.equal(o_p, o_d), name
    assert torch.equal(pool[sl.cuda()], ht_d), name
    untouched = torch.ones(S, dtype=torch.bool)
    untouched[sl] = False
    assert torch.equal(pool.cpu()[untouched], pool_before[untouched]), name
    if fused:
        o_ref, ht_ref = oracle.prefill_fused_gate(inp.q, inp.k, inp.v, inp.gx, inp.A_log, inp.dt_bias, inp.bx,
                                                  inp.cu_seqlens, h0=h0_dense, scale=inp.scale)
    else:
        o_ref, ht_ref = oracle.prefill(inp.q, inp.k, inp.v, inp.g, inp.beta, inp.cu_seqlens, h0=h0_dense,
                                       scale=inp.scale)
    og = host(o_p)
    assert np.isfinite(og).all(), name
    e_o = max_abs(og, o_ref)
    say("%s: pool == dense bitwise (%d rows written, %d untouched); o max-abs %.3e"
        % (name, len(set(slots.tolist())), int(untouched.sum()), e_o))
    assert e_o <= O_MAXABS, name
    check_states(name, host(pool[sl.cuda()]), ht_ref, bf16=inp.pool.dtype == torch.bfloat16)


@pytest.mark.parametrize("state_dtype", ["bf16", "f32"])
def test_gdn_pool_mode_matches_dense_page_recipe(K, oracle, state_dtype):
    inp = W.gdn_pool_page(11, state_dtype)
    pool_vs_dense(K, oracle, inp, "gdn page recipe %s pool" % state_dtype)


@pytest.mark.parametrize("state_dtype", ["bf16", "f32"])
def test_gdn_pool_mode_padding_index(K, oracle, state_dtype):
    inp = W.gdn_pool_page(11, state_dtype, pad_one=True)
    assert int(inp.indices[-1]) == -1
    pool_vs_dense(K, oracle, inp, "gdn page recipe %s pool, index -1" % state_dtype)


def test_gdn_pool_mode_fused_gate(K, oracle):
    inp = W.gdn_pool_page(11, "f32", pad_one=True)
    pool_vs_dense(K, oracle, inp, "gdn page recipe, fused gate", fused=True)


def test_many_chains_bf16_pool(K, oracle):
    """40 sequences of 1100..1500 tokens x 8 heads = 320 chains with V = 128
    (sixteen-wave state workgroups: more than 256 chains, sequences longer
    than 1024 tokens on average), bf16 pool of 48 slots with one -1 index."""
    inp = W.make_prefill(81, (40, 1100, 1500), 4, 8, 128, 128, gate="realistic", pool_slots=48,
                         state_dtype="bf16", pad_one=True)
    pool_vs_dense(K, oracle, inp, "320 chains, bf16 pool")


def test_many_chains_fp32_io(K, oracle):
    """The same shape with fp32 q, k, v and o and an fp32 pool."""
    inp = W.make_prefill(82, (40, 1100, 1500), 4, 8, 128, 128, io="f32", gate="realistic", pool_slots=48,
                         pad_one=True, scale=128 ** -0.5)
    pool_vs_dense(K, oracle, inp, "320 chains, fp32 io")


@pytest.mark.parametrize("io,state", [("bf16", "bf16"), ("f32", "f32")])
def test_many_short_chains(K, oracle, io, state):
    """40 sequences of 1..300 tokens x 8 heads = 320 chains with V = 128: with
    short sequences a workgroup per 64-column part, as for few chains."""
    inp = W.make_prefill(84, (40, 1, 300), 4, 8, 128, 128, io=io, gate="realistic", pool_slots=48,
                         state_dtype=state, pad_one=True, scale=128 ** -0.5)
    pool_vs_dense(K, oracle, inp, "320 short chains, %s io, %s pool" % (io, state))


@pytest.mark.parametrize("io,state", [("bf16", "bf16"), ("f32", "f32")])
def test_mid_chain_count_forms(K, oracle, io, state):
    """20 sequences x 8 heads = 160 chains with V = 128: one state workgroup
    per 64-column part; bf16 io with a bf16 pool, fp32 io with an fp32 pool."""
    inp = W.make_prefill(83, (20, 1, 300), 4, 8, 128, 128, io=io, gate="realistic", pool_slots=24,
                         state_dtype=state, pad_one=True, scale=128 ** -0.5)
    pool_vs_dense(K, oracle, inp, "160 chains, %s io, %s pool" % (io, state))
