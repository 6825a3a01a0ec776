"""GPU test of the allocation-free prefill, kda_chunk_prefill_noalloc, through
the C ABI: its outputs equal those of kda_chunk_prefill (the entry point with
a caller-owned workspace) bit for bit, on consecutive calls that reuse the
library's one per-GPU workspace, the second with a smaller input; the first
call is also held to the oracle's tolerances.  A call whose workspace would
exceed the array is refused before any launch."""
import numpy as np
import pytest
import torch

import kda_workloads as W
from gpu_util import O_MAXABS, STATE_REL_F32, dev, host, max_abs, rel_l2, say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def K():
    import gated_delta_rule_51_amd as kda
    kda.lib()
    return kda


def both(K, inp, pool=None, indices=None):
    """(o, final) from kda_chunk_prefill_noalloc and from kda_chunk_prefill."""
    outs = []
    for fn in (K.chunk_prefill_noalloc, K.chunk_prefill):
        init = dev(inp.h0) if pool is None else pool.clone()
        o, ht = fn(dev(inp.q), dev(inp.k), dev(inp.v), dev(inp.g), dev(inp.beta), dev(inp.cu_seqlens),
                   initial_state=init, state_indices=indices, scale=inp.scale)
        torch.cuda.synchronize()
        outs.append((o, ht))
    return outs


def test_noalloc_matches_workspace_entry_two_calls(K, oracle):
    # call 1: near the array's capacity (one 8000-token sequence, 32 heads)
    say("noalloc call 1: 8000 tokens x 32 heads, K = V = 128")
    big = W.make_prefill(501, [8000], 32, 32, 128, 128, gate="realistic", h0="random")
    desc = K.prefill_desc(big.q, big.v, big.g, 1, torch.float32, 1.0)
    assert K.workspace_size(desc) <= K.SCRATCH_BYTES
    (o_n, h_n), (o_w, h_w) = both(K, big)
    assert torch.equal(o_n, o_w) and torch.equal(h_n, h_w)
    heads = [0, 21]   # heads are independent: two of them against the oracle
    sel = lambda x: x[:, heads].contiguous()
    o_ref, h_ref = oracle.prefill(sel(big.q), sel(big.k), sel(big.v), sel(big.g), sel(big.beta),
                                  big.cu_seqlens, h0=sel(big.h0))
    e_o, e_s = max_abs(host(o_n[:, heads]), o_ref), rel_l2(host(h_n[:, heads]), h_ref)
    say("noalloc call 1: bitwise equal; heads %s o max-abs %.3e state rel-L2 %.3e" % (heads, e_o, e_s))
    assert e_o <= O_MAXABS and e_s <= STATE_REL_F32
    del o_n, h_n, o_w, h_w

    # call 2: smaller, ragged, pool mode with a -1 index, reusing the array
    say("noalloc call 2: 4 sequences, pool mode")
    small = W.make_prefill(502, [90, 5, 64, 0], 2, 4, 128, 128, gate="realistic", h0="random")
    S = 9
    pool = torch.randn(S, 4, 128, 128, generator=torch.Generator().manual_seed(503)) * 0.05
    idx = torch.tensor([3, -1, 0, 5], dtype=torch.int32)
    (o_n, p_n), (o_w, p_w) = both(K, small, pool=dev(pool), indices=dev(idx))
    assert torch.equal(o_n, o_w) and torch.equal(p_n, p_w)
    slots = oracle.map_slot(idx.numpy(), S)
    o_ref, h_ref = oracle.prefill(small.q, small.k, small.v, small.g, small.beta, small.cu_seqlens,
                                  h0=pool[torch.as_tensor(slots)])
    e_o = max_abs(host(o_n), o_ref)
    e_s = rel_l2(host(p_n[torch.as_tensor(slots).cuda()]), h_ref)
    say("noalloc call 2: bitwise equal; o max-abs %.3e state rel-L2 %.3e" % (e_o, e_s))
    assert e_o <= O_MAXABS and e_s <= STATE_REL_F32
    untouched = torch.as_tensor(np.setdiff1d(np.arange(S), slots))
    assert torch.equal(p_n[untouched.cuda()].cpu(), pool[untouched])


def test_noalloc_refuses_oversize(K):
    """A workspace beyond the array is refused with KDA_ERR_WORKSPACE before
    any launch."""
    inp = W.make_prefill(504, [9000], 32, 32, 128, 128)
    desc = K.prefill_desc(inp.q, inp.v, inp.g, 1, torch.float32, 1.0)
    assert K.workspace_size(desc) > K.SCRATCH_BYTES
    with pytest.raises(K.KdaError, match="workspace"):
        K.chunk_prefill_noalloc(dev(inp.q), dev(inp.k), dev(inp.v), dev(inp.g), dev(inp.beta),
                                dev(inp.cu_seqlens))
