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


def test_graph_replay_verify_decode(K):
    """The multi-token (verify) decode under capture: plain and fused-gate
    calls with a per-step state cache, one updating its pool, replayed three
    times with eager work between, each bit-identical to the eager calls."""
    m = W.make_multi_decode(603, [4, 0, 3, 5, 1], 2, 4, 128, 128, num_slots=8, cache_pitch=4)
    t = m.tok
    T = {n: dev(getattr(t, n)) for n in ("q", "k", "v", "g", "beta", "cu_seqlens", "gx", "A_log", "dt_bias", "bx")}
    idx = dev(m.indices)
    pool0 = dev(m.pool)
    pool = pool0.clone()
    N = t.num_seqs
    cache = torch.zeros(N, 4, 4, 128, 128, device="cuda")
    cache_f = torch.zeros_like(cache)

    def work():
        o = K.recurrent_decode_multi(T["q"], T["k"], T["v"], T["g"], T["beta"], T["cu_seqlens"], pool, idx,
                                     intermediate_states=cache, update_pool=True)
        of = K.recurrent_decode_multi_fused_gate(T["q"], T["k"], T["v"], T["gx"], T["A_log"], T["dt_bias"],
                                                 T["bx"], T["cu_seqlens"], pool0, idx,
                                                 intermediate_states=cache_f, update_pool=False)
        return o, of

    o_e, of_e = (x.clone() for x in work())
    pool_e, cache_e, cache_fe = pool.clone(), cache.clone(), cache_f.clone()
    torch.cuda.synchronize()

    pool.copy_(pool0)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        work()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    pool.copy_(pool0)
    torch.cuda.synchronize()
    with torch.cuda.graph(g):
        o_g, of_g = work()
    for r in range(3):
        pool.copy_(pool0)
        cache.zero_()
        cache_f.zero_()
        junk = torch.randn(1 << 20, device="cuda").sum()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        ok = (torch.equal(o_g, o_e) and torch.equal(of_g, of_e) and torch.equal(pool, pool_e)
              and torch.equal(cache, cache_e) and torch.equal(cache_f, cache_fe))
        say("verify graph replay %d: bit-identical %s (junk %.3f)" % (r, ok, float(junk)))
        assert ok, r


def test_graph_survives_workspace_growth(K):
    """A prefill captured on a stream keeps working after a larger eager
    prefill on that stream has replaced the stream's workspace: the replaced
    buffer stays alive, so a tensor allocated afterwards is not overwritten
    by the replay, and the replay still matches the eager result."""
    small = W.make_prefill(603, [100, 30], 2, 4, 128, 128, gate="realistic", h0="random")
    big = W.make_prefill(604, [3000, 2000], 2, 4, 128, 128, gate="realistic", h0="random")
    P = {n: dev(getattr(small, n)) for n in ("q", "k", "v", "g", "beta", "cu_seqlens", "h0")}

    def work():
        return K.chunk_prefill(P["q"], P["k"], P["v"], P["g"], P["beta"], P["cu_seqlens"],
                               initial_state=P["h0"])

    o_e, ht_e = (x.clone() for x in work())
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        work()                                          # the stream's first (small) workspace
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        o_g, ht_g = work()
    torch.cuda.synchronize()
    old_bytes = K._WS[(torch.cuda.current_device(), s.cuda_stream)].numel()
    with torch.cuda.stream(s):                          # grows the stream's workspace
        K.chunk_prefill(*(dev(getattr(big, n)) for n in ("q", "k", "v", "g", "beta", "cu_seqlens")),
                        initial_state=dev(big.h0))
    torch.cuda.synchronize()
    assert K._WS[(torch.cuda.current_device(), s.cuda_stream)].numel() > old_bytes
    # tensors the size of the replaced workspace: the allocator would hand
    # them its memory first if it had been freed
    sentinels = [torch.full((old_bytes // 4,), 7.0, device="cuda") for _ in range(4)]
    for r in range(2):
        g.replay()
        torch.cuda.synchronize()
        ok = torch.equal(o_g, o_e) and torch.equal(ht_g, ht_e)
        clean = all(bool((t == 7.0).all()) for t in sentinels)
        say("graph replay %d after workspace growth: bit-identical %s, sentinels intact %s" % (r, ok, clean))
        assert ok and clean, r
