"""GPU parity of the one-token decode (kda_recurrent_decode) against the fp64
oracle, through the C ABI."""
import numpy as np
import pytest
import torch

import kda_workloads as W
from gpu_util import (O_MAXABS, STATE_REL_F32, compare_decode_streamed, dev, host, max_abs, rel_l2, say)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def K():
    import gated_delta_rule_51_amd as kda
    kda.lib()
    return kda


def check_decode(K, oracle, d, scale=1.0, batch=256):
    """Run the decode in place on a device copy of the pool; compare every
    request with the oracle and every row that is not indexed bitwise."""
    S = d.pool.shape[0]
    slots = oracle.map_slot(d.indices.numpy(), S)
    pool_before = d.pool.clone()
    pool = dev(d.pool)
    o = K.recurrent_decode(dev(d.q), dev(d.k), dev(d.v), dev(d.g), dev(d.beta), pool,
                           dev(d.indices), scale=scale)
    torch.cuda.synchronize()
    compare_decode_streamed(oracle, d, o, pool, pool_before, slots, lambda r: d.g[r], lambda r: d.beta[r],
                            scale, "decode", batch=batch)
    # rows that are not indexed are untouched (bitwise)
    untouched = np.setdiff1d(np.arange(S), slots)
    ut = torch.as_tensor(untouched)
    assert torch.equal(pool[ut.cuda()].cpu(), pool_before[ut])
    return pool, pool_before


@pytest.mark.parametrize("dk,dv", [(128, 128), (64, 64), (32, 32), (128, 64), (32, 128)])
@pytest.mark.parametrize("io,state", [("bf16", "f32"), ("f32", "f32"), ("bf16", "bf16")])
def test_decode_small(K, oracle, dk, dv, io, state):
    d = W.make_decode(100 + dk + dv, 37, 2, 4, dk, dv, num_slots=50, io=io, state_dtype=state, pad=1)
    check_decode(K, oracle, d, scale=dk ** -0.5)


@pytest.mark.parametrize("gate", ["moderate", "realistic"])
def test_decode_scalar_gate(K, oracle, gate):
    d = W.make_decode(7, 20, 4, 8, 128, 128, num_slots=24, gate=gate, scalar_gate=True)
    check_decode(K, oracle, d)


def test_decode_equals_one_token_prefill_oracle_chain(K, oracle):
    """Two decode steps in a row continue from the written state."""
    d = W.make_decode(8, 16, 2, 2, 64, 64, num_slots=20)
    slots = oracle.map_slot(d.indices.numpy(), 20)
    pool0 = d.pool.clone()
    pool = dev(d.pool)
    o1 = K.recurrent_decode(dev(d.q), dev(d.k), dev(d.v), dev(d.g), dev(d.beta), pool, dev(d.indices))
    d2 = W.make_decode(9, 16, 2, 2, 64, 64, num_slots=20)
    o2 = K.recurrent_decode(dev(d2.q), dev(d2.k), dev(d2.v), dev(d2.g), dev(d2.beta), pool,
                            dev(d.indices))
    torch.cuda.synchronize()
    # oracle: two tokens per request as one sequence
    q = torch.stack([d.q, d2.q], 1).reshape(-1, 2, 64)
    k = torch.stack([d.k, d2.k], 1).reshape(-1, 2, 64)
    v = torch.stack([d.v, d2.v], 1).reshape(-1, 2, 64)
    g = torch.stack([d.g, d2.g], 1).reshape(-1, 2, 64)
    b = torch.stack([d.beta, d2.beta], 1).reshape(-1, 2)
    cu = np.arange(0, 33, 2, dtype=np.int32)
    o_ref, ht_ref = oracle.prefill(q, k, v, g, b, cu, h0=pool0[slots])
    assert max_abs(host(o1), o_ref[0::2]) <= O_MAXABS
    assert max_abs(host(o2), o_ref[1::2]) <= O_MAXABS
    assert rel_l2(host(pool[torch.as_tensor(slots).cuda()]), ht_ref) <= STATE_REL_F32


def test_decode_deterministic(K):
    d = W.make_decode(10, 64, 4, 8, 128, 128, num_slots=80)
    outs = []
    for _ in range(2):
        pool = dev(d.pool)
        o = K.recurrent_decode(dev(d.q), dev(d.k), dev(d.v), dev(d.g), dev(d.beta), pool, dev(d.indices))
        outs.append((o.cpu(), pool.cpu()))
    assert torch.equal(outs[0][0], outs[1][0]) and torch.equal(outs[0][1], outs[1][1])


def test_decode_full_size_all_requests(K, oracle):
    """The bench workload: B = 4096 requests, Hv = 32 (B * Hv = 131072 exceeds
    65535, so batch and head must sit on separate grid axes), K = V = 128, fp32
    pool of 4160 slots.  Every request's o and state row is checked against
    the oracle (streamed 256 requests at a time), every other row bitwise."""
    say("generating decode workload B=4096 Hv=32 pool 4160 slots")
    d = W.decode_b4096()
    check_decode(K, oracle, d)


def test_decode_batch_beyond_65535(K, oracle):
    """B = 70,000 requests of one head (K = V = 32): the batch sits on grid x,
    whose limit is 2^31 - 1, so a batch beyond the 65,535 of the other axes
    launches (sglang PR 37317 digest, 风险与影响 item 5, names the per-axis
    limit left after the split).  Every request checked."""
    d = W.make_decode(111, 70000, 1, 1, 32, 32, num_slots=70016, pad=1)
    check_decode(K, oracle, d, scale=32 ** -0.5, batch=8192)
