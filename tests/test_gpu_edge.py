"""GPU parity of the chunked prefill on degenerate and boundary inputs, each
against the fp64 oracle through the C ABI:

* beta = 0: no write, the state only decays and o reads the decayed state;
* g = 0: no decay (every gate factor is exactly 1);
* very strong decay: every in-chunk factor underflows and only the current
  token's own contribution survives;
* wide GQA (one key head for eight value heads);
* many short sequences, including more than the meta kernel ranks by length
  (the natural order is kept beyond that count) and more than one scan block;
* 1200 (sequence, head) chains with 128 value columns (2400 column parts of
  the state kernel), many of them empty;
* a host tensor mixed into GPU arguments is refused before any launch.
"""
import numpy as np
import pytest
import torch

import kda_workloads as W
from gpu_util import O_MAXABS, STATE_REL_F32, check_states, dev, host, max_abs, rel_l2, say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def K():
    import gated_delta_rule_51_amd as kda
    kda.lib()
    return kda


def run_and_check(K, oracle, inp, name):
    o, ht = K.chunk_prefill(dev(inp.q), dev(inp.k), dev(inp.v), dev(inp.g), dev(inp.beta),
                            dev(inp.cu_seqlens), initial_state=dev(inp.h0), scale=inp.scale)
    torch.cuda.synchronize()
    o_ref, ht_ref = oracle.prefill(inp.q, inp.k, inp.v, inp.g, inp.beta, inp.cu_seqlens, h0=inp.h0,
                                   scale=inp.scale)
    og, hg = host(o), host(ht)
    assert np.isfinite(og).all() and np.isfinite(hg).all(), name
    e_o = max_abs(og, o_ref)
    say("%s: o max-abs %.3e" % (name, e_o))
    assert e_o <= O_MAXABS, name
    check_states(name, hg, ht_ref)
    return og, hg, o_ref, ht_ref


def test_beta_zero(K, oracle):
    inp = W.make_prefill(71, [150, 64, 3], 2, 4, 128, 128, gate="realistic", h0="random")
    inp.beta.zero_()
    run_and_check(K, oracle, inp, "beta=0")


def test_no_decay(K, oracle):
    inp = W.make_prefill(72, [200, 17], 2, 2, 128, 128, h0="random")
    inp.g.zero_()
    run_and_check(K, oracle, inp, "g=0")


def test_strong_decay_underflow(K, oracle):
    """log-decay -60 per token: exp(-60) ~ 9e-27 underflows fp16 and every
    cross-token factor is 0; the state after a token is k (beta (v - 0))^T."""
    inp = W.make_prefill(73, [130, 64, 1], 1, 2, 128, 128, h0="random")
    inp.g.fill_(-60.0)
    run_and_check(K, oracle, inp, "g=-60")


def test_wide_gqa(K, oracle):
    inp = W.make_prefill(74, [100, 33, 70], 1, 8, 128, 128, gate="realistic", h0="random")
    run_and_check(K, oracle, inp, "gqa 1:8")


@pytest.mark.parametrize("n", [300, 4096, 4200])
def test_many_short_sequences(K, oracle, n):
    g = torch.Generator().manual_seed(75 + n)
    lens = torch.randint(0, 5, (n,), generator=g).tolist()
    lens[n // 2] = 70   # one sequence with two chunks
    inp = W.make_prefill(75 + n, lens, 1, 2, 64, 64, h0="random", scale=64 ** -0.5)
    run_and_check(K, oracle, inp, "N=%d short" % n)


def test_many_state_chains(K, oracle):
    """600 sequences (lengths 0..79) x 2 heads = 1200 chains with V = 128,
    each split over two column parts: 2400 state workgroups, more than are
    resident at once, with empty and one-chunk chains among them."""
    g = torch.Generator().manual_seed(76)
    lens = torch.randint(0, 80, (600,), generator=g).tolist()
    inp = W.make_prefill(76, lens, 1, 2, 128, 128, gate="realistic", h0="random")
    run_and_check(K, oracle, inp, "1200 chains, V=128")


def test_many_short_sequences_full_heads(K, oracle):
    """1024 sequences of 32 tokens x 32 heads, K = V = 128, pool mode: 32,768
    chains of one half-filled chunk each (a workgroup per column part, as for
    short sequences; every length ties, so the order is the index order).
    The whole call runs; two heads of every sequence are compared with the
    oracle, and the unindexed pool row stays untouched."""
    inp = W.make_prefill(78, [32] * 1024, 32, 32, 128, 128, gate="realistic", pool_slots=1026)
    S = inp.pool.shape[0]
    slots = oracle.map_slot(inp.indices.numpy(), S)
    sl = torch.as_tensor(slots)
    pool_before = inp.pool.clone()
    pool = dev(inp.pool)
    o, _ = K.chunk_prefill(dev(inp.q), dev(inp.k), dev(inp.v), dev(inp.g), dev(inp.beta), dev(inp.cu_seqlens),
                           initial_state=pool, state_indices=dev(inp.indices))
    torch.cuda.synchronize()
    heads = [5, 26]
    sel = lambda x: x[:, heads].contiguous()
    o_ref, ht_ref = oracle.prefill(sel(inp.q), sel(inp.k), sel(inp.v), sel(inp.g), sel(inp.beta),
                                   inp.cu_seqlens, h0=sel(pool_before[sl]))
    og = host(o[:, heads])
    assert np.isfinite(og).all()
    e_o = max_abs(og, o_ref)
    say("1024 x 32 tokens, heads %s: o max-abs %.3e" % (heads, e_o))
    assert e_o <= O_MAXABS
    check_states("1024 x 32 tokens", host(pool[sl.cuda()][:, heads]), ht_ref)
    untouched = np.setdiff1d(np.arange(S), slots)
    assert torch.equal(pool[torch.as_tensor(untouched).cuda()].cpu(), pool_before[torch.as_tensor(untouched)])


def test_large_token_count(K, oracle):
    """131,072 tokens (one sequence of 100,000) x 32 heads, K = V = 128: input
    tensors of 1 GB and a 4.5 GB workspace, so every byte offset past 2^32 is
    exercised.  Two heads of every sequence are checked against the oracle
    (the heads do not interact; with Hk = Hv the head slice is exact)."""
    say("generating 131072-token prefill, 32 heads")
    inp = W.make_prefill(77, [100000, 20000, 11072], 32, 32, 128, 128, gate="realistic", h0="random")
    o, ht = K.chunk_prefill(dev(inp.q), dev(inp.k), dev(inp.v), dev(inp.g), dev(inp.beta),
                            dev(inp.cu_seqlens), initial_state=dev(inp.h0), scale=inp.scale)
    torch.cuda.synchronize()
    heads = [0, 17]
    og = host(o[:, heads])
    hg = host(ht[:, heads])
    del o, ht
    sel = lambda x: x[:, heads].contiguous()
    o_ref, ht_ref = oracle.prefill(sel(inp.q), sel(inp.k), sel(inp.v), sel(inp.g), sel(inp.beta),
                                   inp.cu_seqlens, h0=sel(inp.h0), scale=inp.scale)
    assert np.isfinite(og).all() and np.isfinite(hg).all()
    e_o = max_abs(og, o_ref)
    say("T=131072 heads %s: o max-abs %.3e" % (heads, e_o))
    assert e_o <= O_MAXABS
    check_states("T=131072", hg, ht_ref)


def test_mixed_device_arguments_refused(K):
    """A host tensor among GPU arguments is refused by the binding (its
    pointer would be dereferenced on the GPU); nothing is launched."""
    inp = W.make_prefill(3, [40], 2, 2, 32, 32, h0="random")
    args = [dev(x) for x in (inp.q, inp.k, inp.v, inp.g, inp.beta, inp.cu_seqlens)]
    for i in range(len(args)):
        bad = list(args)
        bad[i] = bad[i].cpu()
        with pytest.raises(ValueError, match="GPU tensors|must be on"):
            K.chunk_prefill(*bad)
    with pytest.raises(ValueError, match="must be on"):
        K.chunk_prefill(*args, initial_state=dev(inp.h0).cpu())


def test_decode_equals_one_token_prefill(K, oracle):
    """A one-token decode of B requests equals a prefill of B one-token
    sequences from the same states (within the prefill's tolerances: the
    prefill's matrix-core operands are fp16, the decode is fp32); both are
    held to the oracle too."""
    d = W.make_decode(78, 24, 2, 4, 128, 128, num_slots=30)
    S = d.pool.shape[0]
    slots = oracle.map_slot(d.indices.numpy(), S)
    pool = dev(d.pool)
    od = K.recurrent_decode(dev(d.q), dev(d.k), dev(d.v), dev(d.g), dev(d.beta), pool, dev(d.indices))
    cu = torch.arange(0, 25, dtype=torch.int32)
    op, hp = K.chunk_prefill(dev(d.q), dev(d.k), dev(d.v), dev(d.g), dev(d.beta), dev(cu),
                             initial_state=dev(d.pool[torch.as_tensor(slots)]))
    torch.cuda.synchronize()
    hd = host(pool[torch.as_tensor(slots).cuda()])
    e_o, e_s = max_abs(host(od), host(op)), rel_l2(host(hp), hd)
    say("decode vs one-token prefill: o max-abs %.3e  state rel-L2 %.3e" % (e_o, e_s))
    assert e_o <= O_MAXABS and e_s <= STATE_REL_F32
    o_ref, ht_ref = oracle.decode(d.q, d.k, d.v, d.g, d.beta, d.pool[torch.as_tensor(slots)])
    assert max_abs(host(od), o_ref) <= O_MAXABS and max_abs(host(op), o_ref) <= O_MAXABS
    check_states("decode", hd, ht_ref)
    check_states("one-token prefill", host(hp), ht_ref)


def test_empty_calls(K):
    """N = 0 sequences (prefill) and B = 0 requests (decode) are accepted and
    launch nothing; the outputs are empty."""
    q = torch.zeros(0, 2, 64, dtype=torch.bfloat16, device="cuda")
    v = torch.zeros(0, 4, 64, dtype=torch.bfloat16, device="cuda")
    g = torch.zeros(0, 4, 64, device="cuda")
    beta = torch.zeros(0, 4, device="cuda")
    cu = torch.zeros(1, dtype=torch.int32, device="cuda")
    o, ht = K.chunk_prefill(q, q, v, g, beta, cu)
    pool = torch.randn(3, 4, 64, 64, device="cuda")
    before = pool.clone()
    od = K.recurrent_decode(q, q, v, g, beta, pool, torch.zeros(0, dtype=torch.int32, device="cuda"))
    torch.cuda.synchronize()
    assert o.shape == (0, 4, 64) and ht.shape == (0, 4, 64, 64) and od.shape == (0, 4, 64)
    assert torch.equal(pool, before)
