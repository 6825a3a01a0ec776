"""GPU parity of the chunked prefill (kda_chunk_prefill) against the fp64
oracle, through the C ABI, plus pool-vs-dense bit identity and edge cases."""
import numpy as np
import pytest
import torch

import kda_workloads as W
from gpu_util import (O_MAXABS, STATE_REL_BF16, STATE_REL_F32, check_states, dev, host, max_abs, rel_l2,
                      say)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def K():
    import gated_delta_rule_51_amd as kda
    kda.lib()
    return kda


def run_dense(K, inp, h0=None, state_dtype=None):
    h0 = inp.h0 if h0 is None else h0
    o, ht = K.chunk_prefill(dev(inp.q), dev(inp.k), dev(inp.v), dev(inp.g), dev(inp.beta),
                            dev(inp.cu_seqlens), initial_state=dev(h0), scale=inp.scale,
                            state_dtype=state_dtype)
    torch.cuda.synchronize()
    return o, ht


def check(name, o, ht, o_ref, ht_ref, state_bf16=False):
    """o max-abs against the oracle; final states by whole-tensor and
    worst-(sequence, head) relative L2."""
    og, hg = host(o), host(ht)
    assert np.isfinite(og).all() and np.isfinite(hg).all()
    e_o = max_abs(og, o_ref)
    say("%s: o max-abs %.3e (|o| max %.2f)"
        % (name, e_o, float(np.abs(o_ref).max()) if o_ref.size else 0.0))
    assert e_o <= O_MAXABS, name
    check_states(name, hg, ht_ref, bf16=state_bf16)


def test_single_sequence_fp32(K, oracle):
    inp = W.single_seq_t128()
    o, ht = run_dense(K, inp)
    o_ref, ht_ref = oracle.prefill(inp.q, inp.k, inp.v, inp.g, inp.beta, inp.cu_seqlens)
    check("single_seq_t128", o, ht, o_ref, ht_ref)
    say("single_seq_t128 o rel-L2 %.3e" % rel_l2(host(o), o_ref))


def test_varlen_gqa(K, oracle):
    inp = W.varlen_gqa5()
    o, ht = run_dense(K, inp)
    o_ref, ht_ref = oracle.prefill(inp.q, inp.k, inp.v, inp.g, inp.beta, inp.cu_seqlens, h0=inp.h0)
    check("varlen_gqa5", o, ht, o_ref, ht_ref)


@pytest.mark.parametrize("state_dtype", ["f32", "bf16"])
def test_pool_matches_dense_bitwise(K, oracle, state_dtype):
    """Pool mode reproduces dense mode bit for bit: same o, the final states
    land in the indexed rows (the -1 index in the sentinel row), and every
    other row is untouched."""
    inp = W.varlen_pool64(state_dtype=state_dtype)
    S = inp.pool.shape[0]
    slots = oracle.map_slot(inp.indices.numpy(), S)
    pool_before = inp.pool.clone()
    h0_dense = pool_before[torch.as_tensor(slots)]
    o_d, ht_d = run_dense(K, inp, h0=h0_dense)
    pool = dev(inp.pool)
    o_p, ht_p = K.chunk_prefill(dev(inp.q), dev(inp.k), dev(inp.v), dev(inp.g), dev(inp.beta),
                                dev(inp.cu_seqlens), initial_state=pool, state_indices=dev(inp.indices))
    torch.cuda.synchronize()
    assert ht_p is pool
    assert torch.equal(o_p, o_d)
    sl = torch.as_tensor(slots).cuda()
    assert torch.equal(pool[sl], ht_d)
    untouched = torch.ones(S, dtype=torch.bool)
    untouched[torch.as_tensor(slots)] = False
    assert torch.equal(pool.cpu()[untouched], pool_before[untouched])
    o_ref, ht_ref = oracle.prefill(inp.q, inp.k, inp.v, inp.g, inp.beta, inp.cu_seqlens, h0=h0_dense)
    check("varlen_pool64-%s" % state_dtype, o_p, pool[sl], o_ref, ht_ref, state_bf16=state_dtype == "bf16")


def test_kimi_shaped_realistic_gates_full(K, oracle):
    """The bench workload: 16 sequences of 512..4096 tokens, Hk = Hv = 32,
    K = V = 128, realistic gates (in-chunk cumulative log-decay up to ~1e4),
    fp32 pool of 32 slots.  Every output and every written row is compared
    with the oracle, and the pool-mode call with a dense-mode twin bit for
    bit (512 chains: the state kernel's sixteen-wave form)."""
    say("generating prefill workload (16 seqs, 512..4096 tokens, 32 heads)")
    inp = W.kimi_prefill_16seq()
    S = inp.pool.shape[0]
    slots = oracle.map_slot(inp.indices.numpy(), S)
    sl = torch.as_tensor(slots)
    pool_before = inp.pool.clone()
    pool = dev(inp.pool)
    o, _ = K.chunk_prefill(dev(inp.q), dev(inp.k), dev(inp.v), dev(inp.g), dev(inp.beta),
                           dev(inp.cu_seqlens), initial_state=pool, state_indices=dev(inp.indices))
    torch.cuda.synchronize()
    o_d, ht_d = run_dense(K, inp, h0=pool_before[sl])
    assert torch.equal(o, o_d)
    assert torch.equal(pool[sl.cuda()], ht_d)
    del o_d, ht_d
    o_ref, ht_ref = oracle.prefill(inp.q, inp.k, inp.v, inp.g, inp.beta, inp.cu_seqlens,
                                   h0=pool_before[sl])
    check("kimi_prefill_16seq", o, pool[sl.cuda()], o_ref, ht_ref)
    untouched = np.setdiff1d(np.arange(S), slots)
    assert torch.equal(pool[torch.as_tensor(untouched).cuda()].cpu(), pool_before[torch.as_tensor(untouched)])


def test_long_prompt_full_call(K, oracle):
    """The long-prompt workload: one sequence of 32,768 tokens, 32 heads,
    K = V = 128, realistic gates, in pool mode as the bench calls it (32
    chains of 512 chunk steps: the state kernel's four-part form).  The whole
    call runs; every output of four heads and their final states are compared
    with the oracle (heads do not interact), and the other pool row stays
    untouched."""
    say("generating long-prompt workload (1 x 32768 tokens, 32 heads)")
    inp = W.long_prompt_32k()
    S = inp.pool.shape[0]
    slots = oracle.map_slot(inp.indices.numpy(), S)
    sl = torch.as_tensor(slots)
    pool_before = inp.pool.clone()
    pool = dev(inp.pool)
    o, _ = K.chunk_prefill(dev(inp.q), dev(inp.k), dev(inp.v), dev(inp.g), dev(inp.beta),
                           dev(inp.cu_seqlens), initial_state=pool, state_indices=dev(inp.indices))
    torch.cuda.synchronize()
    heads = [0, 9, 22, 31]
    sel = lambda x: x[:, heads].contiguous()
    o_ref, ht_ref = oracle.prefill(sel(inp.q), sel(inp.k), sel(inp.v), sel(inp.g), sel(inp.beta),
                                   inp.cu_seqlens, h0=sel(pool_before[sl]))
    check("long prompt, heads %s" % heads, o[:, heads], pool[sl.cuda()][:, heads], o_ref, ht_ref)
    untouched = np.setdiff1d(np.arange(S), slots)
    assert torch.equal(pool[torch.as_tensor(untouched).cuda()].cpu(), pool_before[torch.as_tensor(untouched)])


@pytest.mark.parametrize("gate", ["moderate", "realistic"])
def test_scalar_gate_gdn(K, oracle, gate):
    inp = W.make_prefill(61, [200, 64, 1, 77], 2, 4, 128, 128, gate=gate, scalar_gate=True, h0="random")
    o, ht = run_dense(K, inp)
    o_ref, ht_ref = oracle.prefill(inp.q, inp.k, inp.v, inp.g, inp.beta, inp.cu_seqlens, h0=inp.h0)
    check("gdn-%s" % gate, o, ht, o_ref, ht_ref)


@pytest.mark.parametrize("dk,dv,io", [(64, 64, "bf16"), (32, 32, "bf16"), (128, 64, "bf16"), (64, 128, "bf16"),
                                      (32, 128, "bf16"), (128, 32, "bf16"), (128, 128, "f32")])
def test_head_dims(K, oracle, dk, dv, io):
    """Every compiled (K, V) pairing the kernels specialise on, with K = 128
    (the per-wave gate levels) against V = 32 (two of four waves stage v) and
    fp32 io at K = V = 128 (two staging units per thread, fp32 output rows)."""
    inp = W.make_prefill(62 + dk + dv, [130, 5, 64], 1, 2, dk, dv, io=io, h0="random", scale=dk ** -0.5)
    o, ht = run_dense(K, inp)
    o_ref, ht_ref = oracle.prefill(inp.q, inp.k, inp.v, inp.g, inp.beta, inp.cu_seqlens, h0=inp.h0,
                                   scale=inp.scale)
    check("dims-%d-%d-%s" % (dk, dv, io), o, ht, o_ref, ht_ref)


def test_ragged_and_empty_sequences(K, oracle):
    """Lengths at and around chunk boundaries, and empty sequences (their final
    state equals the initial state)."""
    lens = [0, 1, 63, 64, 65, 0, 127, 128, 129, 2]
    inp = W.make_prefill(63, lens, 2, 2, 128, 128, h0="random")
    o, ht = run_dense(K, inp)
    o_ref, ht_ref = oracle.prefill(inp.q, inp.k, inp.v, inp.g, inp.beta, inp.cu_seqlens, h0=inp.h0)
    check("ragged", o, ht, o_ref, ht_ref)
    assert torch.equal(ht[0].cpu(), inp.h0[0]) and torch.equal(ht[5].cpu(), inp.h0[5])


def test_zero_initial_state_and_no_final(K, oracle):
    inp = W.make_prefill(64, [90, 40], 1, 1, 128, 128)
    o, _ = K.chunk_prefill(dev(inp.q), dev(inp.k), dev(inp.v), dev(inp.g), dev(inp.beta),
                           dev(inp.cu_seqlens), output_final_state=False)
    torch.cuda.synchronize()
    o_ref, _ = oracle.prefill(inp.q, inp.k, inp.v, inp.g, inp.beta, inp.cu_seqlens)
    assert max_abs(host(o), o_ref) <= O_MAXABS


def test_split_continuation(K, oracle):
    """prefill(x[:a]) then prefill(x[a:]) from the carried state equals
    prefill(x), for split points inside and at chunk boundaries."""
    inp = W.make_prefill(65, [300], 2, 4, 128, 128, h0="random")
    o_full, ht_full = run_dense(K, inp)
    for a in (64, 100):
        sa, sb = slice(0, a), slice(a, 300)
        cu_a = torch.tensor([0, a], dtype=torch.int32)
        cu_b = torch.tensor([0, 300 - a], dtype=torch.int32)
        oa, ha = K.chunk_prefill(dev(inp.q[sa]).contiguous(), dev(inp.k[sa]).contiguous(),
                                 dev(inp.v[sa]).contiguous(), dev(inp.g[sa]).contiguous(),
                                 dev(inp.beta[sa]).contiguous(), dev(cu_a), initial_state=dev(inp.h0))
        ob, hb = K.chunk_prefill(dev(inp.q[sb]).contiguous(), dev(inp.k[sb]).contiguous(),
                                 dev(inp.v[sb]).contiguous(), dev(inp.g[sb]).contiguous(),
                                 dev(inp.beta[sb]).contiguous(), dev(cu_b), initial_state=ha)
        torch.cuda.synchronize()
        assert max_abs(host(torch.cat([oa, ob])), host(o_full)) <= O_MAXABS
        assert rel_l2(host(hb), host(ht_full)) <= STATE_REL_F32


def test_prefill_then_decode(K, oracle):
    """A decode step after a prefill continues the same recurrence."""
    inp = W.make_prefill(66, [70, 129], 2, 4, 128, 128, h0="random")
    T = inp.q.shape[0]
    o, ht = run_dense(K, inp)
    nxt = W.make_decode(67, 2, 2, 4, 128, 128, num_slots=3)
    pool = ht.clone()
    idx = torch.tensor([0, 1], dtype=torch.int32).cuda()
    od = K.recurrent_decode(dev(nxt.q), dev(nxt.k), dev(nxt.v), dev(nxt.g), dev(nxt.beta), pool, idx)
    torch.cuda.synchronize()
    # oracle: append the decode token to each sequence
    cu = inp.cu_seqlens.numpy()
    parts = {n: [] for n in ("q", "k", "v", "g", "beta")}
    for s in range(2):
        for name in parts:
            src = getattr(inp, name)[cu[s]:cu[s + 1]]
            parts[name].append(torch.cat([src, getattr(nxt, name)[s:s + 1]]))
    cat = {n: torch.cat(p) for n, p in parts.items()}
    cu2 = torch.tensor([0, 71, 201], dtype=torch.int32)
    o_ref, ht_ref = oracle.prefill(cat["q"], cat["k"], cat["v"], cat["g"], cat["beta"], cu2, h0=inp.h0)
    assert max_abs(host(od), o_ref[[70, 200]]) <= O_MAXABS
    assert rel_l2(host(pool), ht_ref) <= STATE_REL_F32


def test_deterministic(K):
    inp = W.make_prefill(68, [200, 33, 128], 2, 4, 128, 128, h0="random")
    a = run_dense(K, inp)
    b = run_dense(K, inp)
    assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1])


def test_dense_in_place(K, oracle):
    """Dense mode with final_state == initial_state (the in-place form the
    header allows): the final states overwrite the initial ones."""
    import ctypes
    inp = W.make_prefill(69, [150, 7, 64], 2, 4, 128, 128, gate="realistic", h0="random")
    q, k, v, g, beta, cu = (dev(x) for x in (inp.q, inp.k, inp.v, inp.g, inp.beta, inp.cu_seqlens))
    h = dev(inp.h0)
    T, hv, dv = v.shape
    o = torch.empty(T, hv, dv, dtype=q.dtype, device="cuda")
    desc = K.prefill_desc(q, v, g, 3, torch.float32, 1.0)
    ws = torch.empty(K.workspace_size(desc), dtype=torch.uint8, device="cuda")
    stream = torch.cuda.current_stream().cuda_stream
    st = K.lib().kda_chunk_prefill(ctypes.byref(desc), q.data_ptr(), k.data_ptr(), v.data_ptr(), g.data_ptr(),
                                   beta.data_ptr(), cu.data_ptr(), h.data_ptr(), None, h.data_ptr(),
                                   o.data_ptr(), ws.data_ptr(), ws.numel(), stream)
    torch.cuda.synchronize()
    assert st == 0
    o_ref, ht_ref = oracle.prefill(inp.q, inp.k, inp.v, inp.g, inp.beta, inp.cu_seqlens, h0=inp.h0)
    check("dense in place", o, h, o_ref, ht_ref)
    o2, ht2 = run_dense(K, inp)   # out of place: bitwise the same
    assert torch.equal(o, o2) and torch.equal(h, ht2)


@pytest.mark.parametrize("s", [64.0, 1.0 / 64.0, 1000.0])
def test_value_and_state_magnitudes(K, oracle, s):
    """The prefill's matrix-core operands are fp16: relative errors do not
    depend on the magnitude of v and the states while it stays inside fp16's
    normal range (2^-14 .. 65504).  v and h0 scaled by s: the same state
    bounds, o max-abs bound scaled by s."""
    inp = W.varlen_gqa5()
    inp.v = (inp.v.float() * s).to(inp.v.dtype)
    inp.h0 = inp.h0 * s
    o, ht = run_dense(K, inp)
    o_ref, ht_ref = oracle.prefill(inp.q, inp.k, inp.v, inp.g, inp.beta, inp.cu_seqlens, h0=inp.h0)
    og = host(o)
    assert np.isfinite(og).all()
    e_o = max_abs(og, o_ref)
    say("v, h0 x %g: o max-abs %.3e (bound %.3e), |state| max %.1f" % (s, e_o, O_MAXABS * s,
                                                                      float(np.abs(ht_ref).max())))
    assert e_o <= O_MAXABS * s
    check_states("v, h0 x %g" % s, host(ht), ht_ref)
