"""Calls on two streams at once, through the C ABI.

The binding keeps one prefill workspace per (device, stream), and the
library keeps no other state between calls, so work enqueued on different
streams may run at the same time.  Two different workloads, each a prefill
into its own state pool followed by a one-token decode on that pool, are
enqueued alternately on two streams, three times each, with nothing ordering
one stream against the other.  Every output and every pool must equal, bit
for bit, the same calls made alone on the current stream; those are held to
the oracle as well.  The two workloads use different head shapes, dtypes and
state-kernel forms (at most 64 chains, and more than 256).
"""
import numpy as np
import pytest
import torch

import kda_workloads as W
from gpu_util import O_MAXABS, check_states, dev, host, max_abs, say

pytestmark = pytest.mark.gpu

REPS = 3


@pytest.fixture(scope="module")
def K():
    import gated_delta_rule_51_amd as kda
    kda.lib()
    return kda


def workloads():
    a = W.make_prefill(601, (6, 1, 700), 4, 8, 128, 128, gate="realistic", pool_slots=10, pad_one=True)
    b = W.make_prefill(602, (40, 1, 300), 4, 8, 64, 128, io="f32", pool_slots=44, state_dtype="bf16",
                       pad_one=True, scale=64 ** -0.5)
    da = W.make_decode(611, a.num_seqs, 4, 8, 128, 128, num_slots=11)
    db = W.make_decode(612, b.num_seqs, 4, 8, 64, 128, num_slots=45, io="f32", scale=64 ** -0.5)
    return [(a, da), (b, db)]


def run(K, inp, d, pool):
    """Prefill into pool at the workload's indices, then one decode token for
    each of those rows.  Returns (prefill o, decode o); pool is updated."""
    idx = dev(inp.indices)
    o_p, _ = K.chunk_prefill(dev(inp.q), dev(inp.k), dev(inp.v), dev(inp.g), dev(inp.beta), dev(inp.cu_seqlens),
                             initial_state=pool, state_indices=idx, scale=inp.scale)
    o_d = K.recurrent_decode(dev(d.q), dev(d.k), dev(d.v), dev(d.g), dev(d.beta), pool, idx, scale=d.scale)
    return o_p, o_d


def test_two_streams_match_one(K, oracle):
    wl = workloads()
    # alone, on the current stream
    ref = []
    for i, (inp, d) in enumerate(wl):
        pool = dev(inp.pool)
        o_p, o_d = run(K, inp, d, pool)
        torch.cuda.synchronize()
        ref.append((o_p.clone(), o_d.clone(), pool.clone()))
        # the lone run against the oracle (prefill, then decode from its states)
        slots = oracle.map_slot(inp.indices.numpy(), inp.pool.shape[0])
        h0 = inp.pool[torch.as_tensor(slots)]
        o_ref, ht_ref = oracle.prefill(inp.q, inp.k, inp.v, inp.g, inp.beta, inp.cu_seqlens, h0=h0,
                                       scale=inp.scale)
        e = max_abs(host(o_p), o_ref)
        say("workload %d alone: prefill o max-abs %.3e" % (i, e))
        assert e <= O_MAXABS
        bf = inp.pool.dtype == torch.bfloat16
        ht_after_prefill = torch.as_tensor(ht_ref).to(inp.pool.dtype)
        od_ref, hd_ref = oracle.decode(d.q, d.k, d.v, d.g, d.beta, ht_after_prefill, scale=d.scale)
        e = max_abs(host(o_d), od_ref)
        say("workload %d alone: decode o max-abs %.3e" % (i, e))
        assert e <= O_MAXABS
        check_states("workload %d alone, after decode" % i, host(pool[torch.as_tensor(slots).cuda()]), hd_ref,
                     bf16=bf)

    # both, alternately on two streams, REPS times each
    pools = [[dev(inp.pool) for _ in range(REPS)] for inp, _ in wl]
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    for s in streams:
        s.wait_stream(torch.cuda.current_stream())
    outs = [[None] * REPS for _ in wl]
    for r in range(REPS):
        for i, (inp, d) in enumerate(wl):
            with torch.cuda.stream(streams[i]):
                outs[i][r] = run(K, inp, d, pools[i][r])
    for s in streams:
        torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    for i in range(len(wl)):
        for r in range(REPS):
            o_p, o_d = outs[i][r]
            assert torch.equal(o_p, ref[i][0]), "workload %d rep %d: prefill o" % (i, r)
            assert torch.equal(o_d, ref[i][1]), "workload %d rep %d: decode o" % (i, r)
            assert torch.equal(pools[i][r], ref[i][2]), "workload %d rep %d: pool" % (i, r)
    say("two streams: %d calls each, bitwise equal to the lone calls" % (2 * REPS))
