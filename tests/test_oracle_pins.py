"""Pins for the CPU oracle (no GPU).

The oracle is the fp64 token-by-token recurrence of the KDA gated delta rule
(decay by exp(g), residual u = beta*(v - S'^T k), rank-1 write, read-out after
the write).  These tests tie it to things other than itself: hand-worked
values, closed forms, invariants, a brute-force transition-matrix form, and
the chunk-parallel (UT transform) form with an explicit triangular solve.
Each is chosen so a plausible slip (decay on the wrong axis, update order,
beta placement, read-out before the write, a transposed state, a wrong head
map) fails at least one of them.
"""
import json
import os

import numpy as np
import pytest

import kda_workloads as W

HERE = os.path.dirname(os.path.abspath(__file__))


def rand_case(seed, lengths, hk, hv, dk, dv, gate="moderate", scalar=False, h0=True):
    inp = W.make_prefill(seed, lengths, hk, hv, dk, dv, io="f32", gate=gate,
                         scalar_gate=scalar, h0="random" if h0 else None)
    return inp


def run(O, inp, **kw):
    return O.prefill(inp.q, inp.k, inp.v, inp.g, inp.beta, inp.cu_seqlens,
                     h0=kw.pop("h0", inp.h0), scale=kw.pop("scale", inp.scale), **kw)


def test_golden_handworked(oracle):
    """Dyadic examples worked out by hand (tests/golden/kda_handworked.json)."""
    with open(os.path.join(HERE, "golden", "kda_handworked.json")) as f:
        cases = json.load(f)["cases"]
    for c in cases:
        q = np.array(c["q"], np.float32)
        k = np.array(c["k"], np.float32)
        v = np.array(c["v"], np.float32)
        g = (np.log(2.0) * np.array(c["g_log_base2"], np.float64)).astype(np.float32)
        beta = np.array(c["beta"], np.float32)
        h0 = None if c["h0"] is None else np.array(c["h0"], np.float32)
        cu = np.array([0, q.shape[0]], np.int32)
        o, ht = oracle.prefill(q, k, v, g, beta, cu, h0=h0, scale=c["scale"])
        np.testing.assert_allclose(o, np.array(c["o"]), rtol=0, atol=1e-7, err_msg=c["name"])
        np.testing.assert_allclose(ht, np.array(c["ht"]), rtol=0, atol=1e-7, err_msg=c["name"])


def test_single_token_zero_state_closed_form(oracle):
    """S0 = 0, one token: S1 = beta k v^T, so o = scale * beta (q.k) v and the
    stored state is ht[j, c] = beta v_j k_c (K != V exposes a transpose)."""
    inp = rand_case(21, [1, 1, 1], 1, 2, 5, 3, h0=False)
    o, ht = run(oracle, inp, scale=0.7)
    q, k, v, b = (x.double().numpy() for x in (inp.q, inp.k, inp.v, inp.beta))
    for t in range(3):
        for h in range(2):
            want_o = 0.7 * b[t, h] * (q[t, 0] @ k[t, 0]) * v[t, h]
            np.testing.assert_allclose(o[t, h], want_o, rtol=1e-13, atol=1e-15)
            np.testing.assert_allclose(ht[t, h], b[t, h] * np.outer(v[t, h], k[t, 0]),
                                       rtol=1e-13, atol=1e-15)


def test_beta_zero_is_pure_per_channel_decay(oracle):
    """beta = 0: S_t = diag(exp(G_t)) S0 with G_t the running sum of g per key
    channel.  Decay acts along K (the contiguous axis of the stored state)."""
    inp = rand_case(22, [7, 12], 2, 4, 6, 5)
    inp.beta.zero_()
    o, ht = run(oracle, inp, scale=1.3)
    g, q, h0 = inp.g.double().numpy(), inp.q.double().numpy(), inp.h0.double().numpy()
    cu = inp.cu_seqlens.numpy()
    for n in range(2):
        for h in range(4):
            G = np.zeros(6)
            for t in range(cu[n], cu[n + 1]):
                G = G + g[t, h]
                St = h0[n, h] * np.exp(G)[None, :]          # [V, K]
                np.testing.assert_allclose(o[t, h], 1.3 * St @ q[t, h // 2], rtol=1e-12, atol=1e-14)
            np.testing.assert_allclose(ht[n, h], h0[n, h] * np.exp(G)[None, :], rtol=1e-12, atol=1e-14)


def test_zero_gate_zero_beta_is_identity(oracle):
    """g = 0 and beta = 0: the state passes through unchanged (bitwise in fp64)
    and every output is scale * S0^T q."""
    inp = rand_case(23, [9], 1, 3, 8, 4)
    inp.beta.zero_()
    inp.g.zero_()
    o, ht = run(oracle, inp, scale=0.5)
    h0 = inp.h0.double().numpy()
    assert np.array_equal(ht, h0)
    q = inp.q.double().numpy()
    for t in range(9):
        for h in range(3):
            np.testing.assert_allclose(o[t, h], 0.5 * h0[0, h] @ q[t, 0], rtol=1e-13, atol=1e-15)


@pytest.mark.parametrize("gate", ["moderate", "realistic"])
def test_delta_write_invariant(oracle, gate):
    """beta = 1 and a unit key: after the write S_t^T k_t = v_t exactly,
    whatever the gate and the incoming state.  Reading out with q_t = k_t
    therefore returns v_t.  Decaying after the write, or predicting from the
    undecayed state, breaks it."""
    inp = rand_case(24, [20, 33], 2, 2, 16, 8, gate=gate)
    inp.beta.fill_(1.0)
    # keys of exactly unit norm in float32: four entries of +-1/2
    rng = np.random.default_rng(24)
    k = np.zeros(inp.k.shape, np.float32)
    for t in range(k.shape[0]):
        for h in range(k.shape[1]):
            k[t, h, rng.choice(16, 4, replace=False)] = rng.choice([-0.5, 0.5], 4)
    inp.k.copy_(__import__("torch").from_numpy(k))
    inp.q.copy_(inp.k)
    o, _ = run(oracle, inp, scale=1.0)
    np.testing.assert_allclose(o, inp.v.double().numpy(), rtol=0, atol=1e-12)


def test_orthonormal_keys_decouple_channels(oracle):
    """k_t = e_{c(t)}: only row c(t) of the math state is written, every row
    decays by its own channel gate, and row c follows the scalar recurrence
    s <- (1 - beta) a s + beta v.  Computed here with scalar loops."""
    K, V, T, Hv = 4, 3, 11, 2
    rng = np.random.default_rng(5)
    chan = rng.integers(0, K, size=T)
    k = np.zeros((T, 1, K), np.float32)
    k[np.arange(T), 0, chan] = 1.0
    q = rng.standard_normal((T, 1, K)).astype(np.float32)
    v = rng.standard_normal((T, Hv, V)).astype(np.float32)
    g = (-rng.uniform(0.0, 1.5, (T, Hv, K))).astype(np.float32)
    beta = rng.uniform(0.1, 0.9, (T, Hv)).astype(np.float32)
    h0 = rng.standard_normal((1, Hv, V, K)).astype(np.float32)
    o, ht = oracle.prefill(q, k, v, g, beta, np.array([0, T], np.int32), h0=h0, scale=1.0)
    for h in range(Hv):
        s = [[float(h0[0, h, j, c]) for j in range(V)] for c in range(K)]
        for t in range(T):
            for c in range(K):
                a = float(np.exp(np.float64(g[t, h, c])))
                for j in range(V):
                    s[c][j] *= a
            c = int(chan[t])
            for j in range(V):
                s[c][j] = (1.0 - float(beta[t, h])) * s[c][j] + float(beta[t, h]) * float(v[t, h, j])
            for j in range(V):
                want = sum(float(q[t, 0, cc]) * s[cc][j] for cc in range(K))
                assert abs(o[t, h, j] - want) < 1e-12
        for c in range(K):
            for j in range(V):
                assert abs(ht[0, h, j, c] - s[c][j]) < 1e-12


@pytest.mark.parametrize("seed,lengths,hk,hv,dk,dv,scalar", [
    (31, [5], 1, 1, 4, 3, False),
    (32, [17, 3, 9], 1, 2, 8, 8, False),
    (33, [12], 2, 4, 6, 5, True),
])
def test_transition_matrix_brute_force(oracle, seed, lengths, hk, hv, dk, dv, scalar):
    """S_t = (I - b k k^T) diag(exp g) S_{t-1} + b k v^T with explicit K x K
    matrices, one sequence at a time."""
    inp = rand_case(seed, lengths, hk, hv, dk, dv, scalar=scalar)
    o, ht = run(oracle, inp, scale=0.9)
    cu = inp.cu_seqlens.numpy()
    for n in range(len(lengths)):
        sl = slice(cu[n], cu[n + 1])
        g = inp.g[sl]
        o2, ht2 = oracle.transition_np(inp.q[sl], inp.k[sl], inp.v[sl], g, inp.beta[sl],
                                       h0=inp.h0[n], scale=0.9)
        np.testing.assert_allclose(o[sl], o2, rtol=1e-11, atol=1e-13)
        np.testing.assert_allclose(ht[n], ht2, rtol=1e-11, atol=1e-13)


@pytest.mark.parametrize("chunk", [4, 16, 64])
@pytest.mark.parametrize("gate", ["moderate", "realistic"])
def test_chunked_equals_recurrent(oracle, chunk, gate):
    """The chunk-parallel UT-transform form (explicit triangular solve, pairwise
    exp of later-minus-earlier cumsum differences) reproduces the recurrence in
    fp64: this pins the algebra the GPU kernels implement, at ragged chunk
    boundaries, with GQA and several sequences."""
    inp = rand_case(40 + chunk, [1, chunk - 1, chunk, chunk + 1, 3 * chunk - 2], 2, 4, 8, 4, gate=gate)
    o, ht = run(oracle, inp, scale=0.8)
    o2, ht2 = oracle.chunked_np(inp.q, inp.k, inp.v, inp.g, inp.beta, inp.cu_seqlens.numpy(),
                                h0=inp.h0, scale=0.8, chunk=chunk)
    np.testing.assert_allclose(o2, o, rtol=1e-10, atol=1e-12)
    np.testing.assert_allclose(ht2, ht, rtol=1e-10, atol=1e-12)


def test_chunked_scalar_gate(oracle):
    inp = rand_case(47, [70, 5], 1, 2, 8, 8, scalar=True)
    o, ht = run(oracle, inp)
    o2, ht2 = oracle.chunked_np(inp.q, inp.k, inp.v, inp.g, inp.beta, inp.cu_seqlens.numpy(),
                                h0=inp.h0, chunk=16)
    np.testing.assert_allclose(o2, o, rtol=1e-10, atol=1e-12)
    np.testing.assert_allclose(ht2, ht, rtol=1e-10, atol=1e-12)


def test_split_continuation(oracle):
    """Running tokens [0, a) and then [a, T) from the carried state equals one
    run over [0, T), for split points inside and at chunk boundaries."""
    inp = rand_case(50, [150], 1, 2, 8, 8)
    o, ht = run(oracle, inp)
    for a in (1, 63, 64, 100):
        sa, sb = slice(0, a), slice(a, 150)
        oa, ha = oracle.prefill(inp.q[sa], inp.k[sa], inp.v[sa], inp.g[sa], inp.beta[sa],
                                np.array([0, a], np.int32), h0=inp.h0)
        ob, hb = oracle.prefill(inp.q[sb], inp.k[sb], inp.v[sb], inp.g[sb], inp.beta[sb],
                                np.array([0, 150 - a], np.int32), h0=ha.astype(np.float32))
        # the carried state passes through float32 here, so compare loosely
        np.testing.assert_allclose(np.concatenate([oa, ob]), o, rtol=0, atol=1e-6)
        np.testing.assert_allclose(hb, ht, rtol=0, atol=1e-6)


def test_varlen_isolation(oracle):
    """A packed batch equals each sequence run on its own (cu_seqlens handling),
    including an empty sequence, which leaves its state unchanged."""
    lengths = [13, 0, 64, 1, 70]
    inp = rand_case(51, lengths, 2, 2, 8, 4)
    o, ht = run(oracle, inp)
    cu = inp.cu_seqlens.numpy()
    for n, L in enumerate(lengths):
        sl = slice(cu[n], cu[n + 1])
        on, hn = oracle.prefill(inp.q[sl], inp.k[sl], inp.v[sl], inp.g[sl], inp.beta[sl],
                                np.array([0, L], np.int32), h0=inp.h0[n:n + 1])
        assert np.array_equal(on, o[sl])
        assert np.array_equal(hn[0], ht[n])
    assert np.array_equal(ht[1], inp.h0[1].double().numpy())


def test_gqa_head_map(oracle):
    """Value head h reads key head h // (Hv / Hk): the GQA run equals a run
    with Hk = Hv and q, k duplicated for consecutive value heads."""
    inp = rand_case(52, [20, 9], 2, 6, 8, 4)
    o, ht = run(oracle, inp)
    qd = inp.q.repeat_interleave(3, dim=1)
    kd = inp.k.repeat_interleave(3, dim=1)
    o2, ht2 = oracle.prefill(qd, kd, inp.v, inp.g, inp.beta, inp.cu_seqlens, h0=inp.h0)
    assert np.array_equal(o, o2) and np.array_equal(ht, ht2)


def test_scalar_gate_is_broadcast_channel_gate(oracle):
    """GDN's scalar gate equals a per-channel gate with equal channels."""
    inp = rand_case(53, [30, 7], 1, 2, 8, 4, scalar=True)
    o, ht = run(oracle, inp)
    gb = inp.g[:, :, None].expand(-1, -1, 8).contiguous()
    o2, ht2 = oracle.prefill(inp.q, inp.k, inp.v, gb, inp.beta, inp.cu_seqlens, h0=inp.h0)
    assert np.array_equal(o, o2) and np.array_equal(ht, ht2)


def test_linear_in_values_and_state(oracle):
    """For fixed q, k, g, beta the map (v, S0) -> (o, S_T) is linear."""
    a = rand_case(54, [25], 1, 2, 8, 4)
    b = rand_case(55, [25], 1, 2, 8, 4)
    # values on a 2^-12 grid so the float32 input a + 2b is formed exactly
    for x in (a.v, b.v, a.h0, b.h0):
        x.copy_(__import__("torch").round(x * 4096.0) / 4096.0)
    oa, ha = oracle.prefill(a.q, a.k, a.v, a.g, a.beta, a.cu_seqlens, h0=a.h0)
    ob, hb = oracle.prefill(a.q, a.k, b.v, a.g, a.beta, a.cu_seqlens, h0=b.h0)
    oc, hc = oracle.prefill(a.q, a.k, a.v + 2.0 * b.v, a.g, a.beta, a.cu_seqlens,
                            h0=a.h0 + 2.0 * b.h0)
    np.testing.assert_allclose(oc, oa + 2.0 * ob, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(hc, ha + 2.0 * hb, rtol=1e-12, atol=1e-12)


def test_numpy_recurrence_matches_c(oracle):
    """The numpy and C recurrences agree (guards against implementation slips
    in either; it pins nothing about the method by itself)."""
    inp = rand_case(56, [40, 3], 2, 4, 16, 8, gate="realistic")
    o, ht = run(oracle, inp)
    o2, ht2 = oracle.recurrent_np(inp.q, inp.k, inp.v, inp.g, inp.beta, inp.cu_seqlens.numpy(), inp.h0)
    np.testing.assert_allclose(o2, o, rtol=1e-13, atol=1e-14)
    np.testing.assert_allclose(ht2, ht, rtol=1e-13, atol=1e-14)


def test_pool_mode_bookkeeping(oracle):
    """Pool mode: indexed rows are the initial states, final states land in the
    same rows, a -1 index selects the last (sentinel) slot, and rows that are
    not indexed are untouched."""
    inp = W.make_prefill(57, [10, 3, 8], 1, 2, 8, 4, io="f32", pool_slots=9, pad_one=True)
    idx = inp.indices.numpy()
    assert idx[-1] == -1
    o, newpool = oracle.prefill_pool(inp.q, inp.k, inp.v, inp.g, inp.beta, inp.cu_seqlens,
                                     inp.pool, inp.indices)
    slots = [int(i) for i in idx[:-1]] + [8]
    h0 = inp.pool[slots]
    o2, ht2 = oracle.prefill(inp.q, inp.k, inp.v, inp.g, inp.beta, inp.cu_seqlens, h0=h0)
    assert np.array_equal(o, o2)
    for n, s in enumerate(slots):
        assert np.array_equal(newpool[s], ht2[n])
    untouched = [s for s in range(9) if s not in slots]
    assert np.array_equal(newpool[untouched], inp.pool[untouched].double().numpy())


def test_decode_is_one_token_prefill(oracle):
    """Decode over B requests equals B one-token sequences."""
    d = W.make_decode(58, 6, 2, 4, 8, 4, num_slots=10, pad=1)
    slots = oracle.map_slot(d.indices.numpy(), 10)
    h0 = d.pool[slots]
    o, ht = oracle.decode(d.q, d.k, d.v, d.g, d.beta, h0)
    for b in range(6):
        ob, hb = oracle.prefill(d.q[b:b + 1], d.k[b:b + 1], d.v[b:b + 1], d.g[b:b + 1],
                                d.beta[b:b + 1], np.array([0, 1], np.int32), h0=h0[b:b + 1])
        assert np.array_equal(ob[0], o[b]) and np.array_equal(hb[0], ht[b])


def test_decode_steps_transition_form(oracle):
    """The per-step states of the multi-token decode equal the transition-matrix
    form applied one token at a time, S_t = (I - b k k^T) D_t S_{t-1} + b k v^T
    (math orientation K x V), and o_t = scale S_t^T q_t; requests of 1..5
    tokens (one request empty) with GQA."""
    inp = W.make_prefill(59, [3, 1, 5, 0, 2], 1, 2, 6, 4, io="f32", gate="realistic", h0="random")
    o, st = oracle.decode_steps(inp.q, inp.k, inp.v, inp.g, inp.beta, inp.cu_seqlens, inp.h0, scale=0.8)
    q, k, v, g, b = (x.double().numpy() for x in (inp.q, inp.k, inp.v, inp.g, inp.beta))
    cu = inp.cu_seqlens.numpy()
    for n in range(5):
        for h in range(2):
            S = inp.h0[n, h].double().numpy().T
            for t in range(cu[n], cu[n + 1]):
                kt = k[t, 0]
                S = (np.eye(6) - b[t, h] * np.outer(kt, kt)) @ (np.exp(g[t, h])[:, None] * S) \
                    + b[t, h] * np.outer(kt, v[t, h])
                np.testing.assert_allclose(st[t, h], S.T, rtol=1e-12, atol=1e-13)
                np.testing.assert_allclose(o[t, h], 0.8 * S.T @ q[t, 0], rtol=1e-12, atol=1e-13)


def test_decode_steps_last_state_is_prefill_final(oracle):
    """The state after each request's last token is the prefill final state,
    and one token per request reduces to the one-token decode."""
    inp = W.make_prefill(60, [4, 2, 7], 2, 4, 8, 8, io="f32", gate="realistic", h0="random")
    o, st = oracle.decode_steps(inp.q, inp.k, inp.v, inp.g, inp.beta, inp.cu_seqlens, inp.h0)
    o2, ht = oracle.prefill(inp.q, inp.k, inp.v, inp.g, inp.beta, inp.cu_seqlens, h0=inp.h0)
    np.testing.assert_allclose(o, o2, rtol=1e-12, atol=1e-13)
    ends = inp.cu_seqlens.numpy()[1:] - 1
    np.testing.assert_allclose(st[ends], ht, rtol=1e-12, atol=1e-13)
    d = W.make_decode(61, 5, 2, 4, 8, 8, num_slots=6)
    h0 = d.pool[:5]
    o1, s1 = oracle.decode_steps(d.q, d.k, d.v, d.g, d.beta, np.arange(6, dtype=np.int32), h0)
    o3, s3 = oracle.decode(d.q, d.k, d.v, d.g, d.beta, h0)
    assert np.array_equal(o1, o3) and np.array_equal(s1, s3)
