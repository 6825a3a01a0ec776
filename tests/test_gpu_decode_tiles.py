"""The decodes' value-row tile follows the size of the call: 32-row tiles
for small batches (more, shorter workgroups, for latency), the whole head
once the batch fills the chip.  A row's arithmetic does not depend on its
tile, so the same requests give bit-identical outputs, states and cached
steps on both sides of the switch.  Each test runs a batch just above the
switch (whole-head tiles) and its first requests alone, just at it (32-row
tiles), on copies of one pool, through the C ABI.  The one-token decode's
32-row tile result is also compared with the oracle here; both tile forms
are held to it elsewhere too (small batches in the decode and verify suites,
the full-size workloads there).
"""
import pytest
import torch

import kda_workloads as W
from gpu_util import O_MAXABS, check_states, dev, host, max_abs, say

pytestmark = pytest.mark.gpu

# state rows (batch x value heads x V) up to which the 32-row tiles are used
SMALL_ROWS_DECODE = 256 * 32 * 128
SMALL_ROWS_VERIFY = 32 * 32 * 128
HV = 32


@pytest.fixture(scope="module")
def K():
    import gated_delta_rule_51_amd as kda
    kda.lib()
    return kda


@pytest.mark.parametrize("dk,dv", [(128, 128), (64, 64), (128, 64)])
def test_decode_tile_switch(K, oracle, dk, dv):
    b_small = SMALL_ROWS_DECODE // (HV * dv)
    B = b_small + 8
    d = W.make_decode(800 + dk + dv, B, 8, HV, dk, dv, num_slots=B + 2, scale=dk ** -0.5)
    say("decode tile switch: K=%d V=%d, %d requests against the first %d" % (dk, dv, B, b_small))
    q, k, v, g, beta, idx = (dev(t) for t in (d.q, d.k, d.v, d.g, d.beta, d.indices))
    pool_all = dev(d.pool)
    pool_few = pool_all.clone()
    o_all = K.recurrent_decode(q, k, v, g, beta, pool_all, idx, scale=d.scale)
    o_few = K.recurrent_decode(q[:b_small], k[:b_small], v[:b_small], g[:b_small], beta[:b_small], pool_few,
                               idx[:b_small], scale=d.scale)
    torch.cuda.synchronize()
    rows = idx[:b_small].long()
    assert torch.equal(o_few, o_all[:b_small])
    assert torch.equal(pool_few[rows], pool_all[rows])
    # the 32-row tile result against the oracle as well
    o_ref, ht_ref = oracle.decode(d.q[:b_small], d.k[:b_small], d.v[:b_small], d.g[:b_small], d.beta[:b_small],
                                  d.pool[d.indices[:b_small].long()], scale=d.scale)
    e_o = max_abs(host(o_few), o_ref)
    say("decode tile switch: o max-abs %.3e" % e_o)
    assert e_o <= O_MAXABS
    check_states("decode tile switch", host(pool_few[rows]), ht_ref)


@pytest.mark.parametrize("dk,dv", [(128, 128), (64, 64)])
def test_verify_tile_switch(K, dk, dv):
    n_small = SMALL_ROWS_VERIFY // (HV * dv)
    N = n_small + 8
    lens = [(3 * i) % 6 for i in range(N)]   # 0 to 5 tokens, some requests empty
    m = W.make_multi_decode(820 + dk + dv, lens, 8, HV, dk, dv, num_slots=N + 2, cache_pitch=4,
                            scale=dk ** -0.5)
    t = m.tok
    say("verify tile switch: K=%d V=%d, %d requests against the first %d" % (dk, dv, N, n_small))
    q, k, v, g, beta, cu = (dev(x) for x in (t.q, t.k, t.v, t.g, t.beta, t.cu_seqlens))
    idx = dev(m.indices)
    T_small = int(t.cu_seqlens[n_small])
    pool_all = dev(m.pool)
    pool_few = pool_all.clone()
    cache_all = torch.zeros(N, 4, HV, dv, dk, dtype=pool_all.dtype, device="cuda")
    cache_few = torch.zeros(n_small, 4, HV, dv, dk, dtype=pool_all.dtype, device="cuda")
    o_all = K.recurrent_decode_multi(q, k, v, g, beta, cu, pool_all, idx, intermediate_states=cache_all,
                                     update_pool=True, scale=t.scale)
    o_few = K.recurrent_decode_multi(q[:T_small], k[:T_small], v[:T_small], g[:T_small], beta[:T_small],
                                     cu[:n_small + 1], pool_few, idx[:n_small], intermediate_states=cache_few,
                                     update_pool=True, scale=t.scale)
    torch.cuda.synchronize()
    rows = idx[:n_small].long()
    assert torch.equal(o_few, o_all[:T_small])
    assert torch.equal(cache_few, cache_all[:n_small])
    assert torch.equal(pool_few[rows], pool_all[rows])
