"""The library under HIP graph capture: a prefill and a decode call captured
into one graph (torch.cuda.CUDAGraph on ROCm) replay bit-identically to the
eager calls.  The library enqueues only kernels (no memset, copy or
allocation of its own), so capture records three prefill kernels and one
decode kernel.  Each replay is preceded by eager work of the program (input
restore, an unrelated kernel, a synchronisation) and checked against the
eager result."""
import pytest
import torch

import kda_workloads as W
from gpu_util import dev, say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def K():
    import gated_delta_rule_51_amd as kda
    kda.lib()
    return kda


def test_graph_replay_matches_eager(K):
    inp = W.make_prefill(601, [150, 64, 3, 200], 2, 4, 128, 128, gate="realistic", h0="random")
    d = W.make_decode(602, 64, 2, 4, 128, 128, num_slots=80)
    P = {n: dev(getattr(inp, n)) for n in ("q", "k", "v", "g", "beta", "cu_seqlens", "h0")}
    D = {n: dev(getattr(d, n)) for n in ("q", "k", "v", "g", "beta", "indices")}
    pool0 = dev(d.pool)
    pool = pool0.clone()

    def work():
        o, ht = K.chunk_prefill(P["q"], P["k"], P["v"], P["g"], P["beta"], P["cu_seqlens"],
                                initial_state=P["h0"])
        od = K.recurrent_decode(D["q"], D["k"], D["v"], D["g"], D["beta"], pool, D["indices"])
        return o, ht, od

    o_e, ht_e, od_e = (x.clone() for x in work())     # eager reference (also warms the workspace)
    pool_e = pool.clone()
    torch.cuda.synchronize()

    pool.copy_(pool0)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        work()                                          # warm-up on the capture stream
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    pool.copy_(pool0)
    torch.cuda.synchronize()
    with torch.cuda.graph(g):
        o_g, ht_g, od_g = work()
    for r in range(3):
        pool.copy_(pool0)                               # eager work between replays
        junk = torch.randn(1 << 20, device="cuda").sum()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        ok = (torch.equal(o_g, o_e) and torch.equal(ht_g, ht_e) and torch.equal(od_g, od_e)
              and torch.equal(pool, pool_e))
        say("graph replay %d: bit-identical %s (junk %.3f)" % (r, ok, float(junk)))
        assert ok, r
