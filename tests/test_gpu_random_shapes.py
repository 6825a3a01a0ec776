"""Seeded random configurations of the prefill and the one-token decode
against the fp64 oracle, through the C ABI.

Each case draws, from its own seed: the key and value head dims (32, 64 or
128 each), the key-head count and the GQA ratio, one to six sequences whose
lengths mix single tokens, chunk-size multiples and their neighbours with
free draws, the io and state dtypes, the gate kind (per-channel or scalar,
moderate or realistic decays, activated on the host or from raw inputs in
the kernels), and dense or pool mode (with a -1 index).  The prefill's final
states then seed a decode step of the same heads.  Every output is compared
with the oracle at the suite's tolerances; pool rows that are not indexed
must stay bit-identical.  Further cases draw multi-token (verify) decodes.
The drawn configuration is printed before the GPU calls.
"""
import numpy as np
import pytest
import torch

import kda_workloads as W
from gpu_util import O_MAXABS, check_states, dev, host, max_abs, say

pytestmark = pytest.mark.gpu

N_CASES = 24


@pytest.fixture(scope="module")
def K():
    import gated_delta_rule_51_amd as kda
    kda.lib()
    return kda


def draw(case):
    rng = np.random.default_rng(7000 + case)
    c = {}
    c["dk"] = int(rng.choice([32, 64, 128]))
    c["dv"] = int(rng.choice([32, 64, 128]))
    c["hk"] = int(rng.choice([1, 2, 4]))
    c["hv"] = c["hk"] * int(rng.choice([1, 2]))
    n = int(rng.integers(1, 7))
    c["lens"] = [int(rng.choice([1, 63, 64, 65, 128, int(rng.integers(2, 300))])) for _ in range(n)]
    c["io"] = str(rng.choice(["bf16", "f32"]))
    c["state"] = str(rng.choice(["f32", "bf16"]))
    c["gate"] = str(rng.choice(["moderate", "realistic"]))
    c["scalar"] = bool(rng.random() < 0.3)
    c["fused"] = bool(rng.random() < 0.3)
    c["pool"] = bool(rng.random() < 0.5)
    return c


def prefill_case(K, oracle, case, c):
    name = "case %d" % case
    inp = W.make_prefill(7000 + case, c["lens"], c["hk"], c["hv"], c["dk"], c["dv"], io=c["io"], gate=c["gate"],
                         scalar_gate=c["scalar"], h0=None if c["pool"] else "random",
                         pool_slots=len(c["lens"]) + 3 if c["pool"] else 0, state_dtype=c["state"],
                         pad_one=c["pool"], scale=c["dk"] ** -0.5)
    if c["fused"]:
        fn = K.chunk_prefill_fused_gate
        gate = (dev(inp.gx), dev(inp.A_log), dev(inp.dt_bias), dev(inp.bx))
    else:
        fn = K.chunk_prefill
        gate = (dev(inp.g), dev(inp.beta))
    if c["pool"]:
        S = inp.pool.shape[0]
        slots = oracle.map_slot(inp.indices.numpy(), S)
        pool_before = inp.pool.clone()
        h0 = pool_before[torch.as_tensor(slots)]
        pool = dev(inp.pool)
        o, _ = fn(dev(inp.q), dev(inp.k), dev(inp.v), *gate, dev(inp.cu_seqlens), initial_state=pool,
                  state_indices=dev(inp.indices), scale=inp.scale)
        torch.cuda.synchronize()
        ht = pool[torch.as_tensor(slots).cuda()]
        untouched = np.setdiff1d(np.arange(S), slots)
        assert torch.equal(pool.cpu()[torch.as_tensor(untouched)], pool_before[torch.as_tensor(untouched)]), name
    else:
        h0 = inp.h0
        o, ht = fn(dev(inp.q), dev(inp.k), dev(inp.v), *gate, dev(inp.cu_seqlens), initial_state=dev(h0),
                   scale=inp.scale)
        torch.cuda.synchronize()
    if c["fused"]:
        o_ref, ht_ref = oracle.prefill_fused_gate(inp.q, inp.k, inp.v, inp.gx, inp.A_log, inp.dt_bias, inp.bx,
                                                  inp.cu_seqlens, h0=h0, scale=inp.scale)
    else:
        o_ref, ht_ref = oracle.prefill(inp.q, inp.k, inp.v, inp.g, inp.beta, inp.cu_seqlens, h0=h0,
                                       scale=inp.scale)
    og = host(o)
    assert np.isfinite(og).all(), name
    e_o = max_abs(og, o_ref)
    say("%s prefill: o max-abs %.3e" % (name, e_o))
    assert e_o <= O_MAXABS, name
    check_states(name + " prefill", host(ht), ht_ref, bf16=c["state"] == "bf16")
    return ht


def decode_case(K, oracle, case, c, states):
    """One decode token per (sequence, head) state the prefill left, in a pool
    that holds those states in its first rows (request n at row n, the last
    request at -1 when the pool has a spare sentinel row)."""
    name = "case %d" % case
    N = states.shape[0]
    d = W.make_decode(8000 + case, N, c["hk"], c["hv"], c["dk"], c["dv"], num_slots=N + 1, io=c["io"],
                      gate=c["gate"], scalar_gate=c["scalar"], state_dtype=c["state"], scale=c["dk"] ** -0.5)
    pool = torch.zeros(N + 1, *states.shape[1:], dtype=states.dtype, device="cuda")
    pool[:N] = states
    idx = torch.arange(N, dtype=torch.int32)
    if N > 1:
        pool[N] = states[N - 1]   # the sentinel row carries the last request's state
        idx[N - 1] = -1
    pool_before = pool.cpu()
    if c["fused"]:
        o = K.recurrent_decode_fused_gate(dev(d.q), dev(d.k), dev(d.v), dev(d.gx), dev(d.A_log), dev(d.dt_bias),
                                          dev(d.bx), pool, dev(idx), scale=d.scale)
        g = oracle.gate_activation(d.gx, d.A_log, d.dt_bias)
        beta = oracle.sigmoid(d.bx)
    else:
        o = K.recurrent_decode(dev(d.q), dev(d.k), dev(d.v), dev(d.g), dev(d.beta), pool, dev(idx), scale=d.scale)
        g, beta = d.g, d.beta
    torch.cuda.synchronize()
    slots = oracle.map_slot(idx.numpy(), N + 1)
    o_ref, ht_ref = oracle.decode(d.q, d.k, d.v, g, beta, pool_before[torch.as_tensor(slots)], scale=d.scale)
    og = host(o)
    assert np.isfinite(og).all(), name
    e_o = max_abs(og, o_ref)
    say("%s decode: o max-abs %.3e" % (name, e_o))
    assert e_o <= O_MAXABS, name
    check_states(name + " decode", host(pool[torch.as_tensor(slots).cuda()]), ht_ref, bf16=c["state"] == "bf16")
    untouched = np.setdiff1d(np.arange(N + 1), slots)
    if len(untouched):
        assert torch.equal(pool.cpu()[torch.as_tensor(untouched)], pool_before[torch.as_tensor(untouched)]), name


@pytest.mark.parametrize("case", range(N_CASES))
def test_random_configuration(K, oracle, case):
    c = draw(case)
    say("case %d: %s" % (case, c))
    states = prefill_case(K, oracle, case, c)
    decode_case(K, oracle, case, c, states)


N_VERIFY = 12


def draw_verify(case):
    rng = np.random.default_rng(9000 + case)
    c = {}
    c["dk"] = int(rng.choice([32, 64, 128]))
    c["dv"] = int(rng.choice([32, 64, 128]))
    c["hk"] = int(rng.choice([1, 2, 4]))
    c["hv"] = c["hk"] * int(rng.choice([1, 2]))
    n = int(rng.integers(1, 9))
    c["lens"] = [int(rng.integers(0, 11)) for _ in range(n)]
    c["pitch"] = int(rng.integers(1, 9))
    c["io"] = str(rng.choice(["bf16", "f32"]))
    c["state"] = str(rng.choice(["f32", "bf16"]))
    c["scalar"] = bool(rng.random() < 0.3)
    c["fused"] = bool(rng.random() < 0.4)
    c["update_pool"] = bool(rng.random() < 0.6)
    c["pad"] = int(n > 1 and rng.random() < 0.5)
    return c


@pytest.mark.parametrize("case", range(N_VERIFY))
def test_random_verify_configuration(K, oracle, case):
    """Multi-token (verify) decode: requests of 0 to 10 tokens, a random
    cache pitch (steps at or beyond it are not cached), read-only or updated
    pool, an optional -1 index; checked by the verify suite's comparison
    (every token's o, every cached step, the pool row, and every cache entry
    and pool row the call must not write)."""
    from test_gpu_multi_decode import check as check_multi
    c = draw_verify(case)
    say("verify case %d: %s" % (case, c))
    m = W.make_multi_decode(9000 + case, c["lens"], c["hk"], c["hv"], c["dk"], c["dv"],
                            num_slots=len(c["lens"]) + 3, cache_pitch=c["pitch"], io=c["io"],
                            scalar_gate=c["scalar"], state_dtype=c["state"], pad=c["pad"],
                            scale=c["dk"] ** -0.5)
    check_multi(K, oracle, m, "verify case %d" % case, fused=c["fused"], update_pool=c["update_pool"])
