"""GPU parity of the multi-token (speculative verify) decode,
kda_recurrent_decode_multi[_fused_gate], against the fp64 oracle through the
C ABI: o for every token, the cached state after every step (within the
cache pitch), the pool row after the last step (or an untouched pool), and
every cache entry and pool row the call must not write."""
import numpy as np
import pytest
import torch

import kda_workloads as W
from gpu_util import (O_MAXABS, STATE_REL_BF16, STATE_REL_BF16_UNIT, STATE_REL_F32, STATE_REL_F32_UNIT, dev,
                      host, max_abs, say, unit_rel_l2)

pytestmark = pytest.mark.gpu

SENTINEL = 7.0   # cache fill: any entry the kernel must not write keeps it


@pytest.fixture(scope="module")
def K():
    import gated_delta_rule_51_amd as kda
    kda.lib()
    return kda


def run(K, m, fused=False, update_pool=True, alloc_steps=None):
    """Run one multi-token decode on the GPU; return what the checks need."""
    t = m.tok
    N = t.num_seqs
    hv, dv, dk = t.v.shape[1], t.v.shape[2], t.q.shape[2]
    steps = alloc_steps or m.cache_pitch
    full = torch.full((N, steps, hv, dv, dk), SENTINEL, dtype=m.pool.dtype, device="cuda")
    cache = full[:, :m.cache_pitch] if steps != m.cache_pitch else full
    pool_before = m.pool.clone()
    pool = dev(m.pool)
    if fused:
        o = K.recurrent_decode_multi_fused_gate(dev(t.q), dev(t.k), dev(t.v), dev(t.gx), dev(t.A_log),
                                                dev(t.dt_bias), dev(t.bx), dev(t.cu_seqlens), pool,
                                                dev(m.indices), intermediate_states=cache,
                                                update_pool=update_pool, scale=t.scale)
    else:
        o = K.recurrent_decode_multi(dev(t.q), dev(t.k), dev(t.v), dev(t.g), dev(t.beta), dev(t.cu_seqlens),
                                     pool, dev(m.indices), intermediate_states=cache,
                                     update_pool=update_pool, scale=t.scale)
    torch.cuda.synchronize()
    return o, pool, full, pool_before


def check(K, oracle, m, name, fused=False, update_pool=True, alloc_steps=None, batch=64):
    """Run once, then compare every request with the oracle, ``batch``
    requests at a time (their fp64 per-step states stay near 1 GB)."""
    t = m.tok
    o, pool, full, pool_before = run(K, m, fused, update_pool, alloc_steps)
    S = m.pool.shape[0]
    N = t.num_seqs
    slots = oracle.map_slot(m.indices.numpy(), S)
    cu = t.cu_seqlens.numpy()
    pitch = m.cache_pitch
    tol = STATE_REL_BF16 if m.pool.dtype == torch.bfloat16 else STATE_REL_F32
    tol_u = STATE_REL_BF16_UNIT if m.pool.dtype == torch.bfloat16 else STATE_REL_F32_UNIT
    e_o, worst_c, worst_p = 0.0, 0.0, 0.0
    sq = {"c": [0.0, 0.0], "p": [0.0, 0.0]}   # squared error, squared reference
    n_steps = 0
    for b0 in range(0, N, batch):
        reqs = np.arange(b0, min(N, b0 + batch))
        tok_idx = np.concatenate([np.arange(cu[n], cu[n + 1]) for n in reqs])
        sub_cu = np.concatenate([[0], np.cumsum([cu[n + 1] - cu[n] for n in reqs])]).astype(np.int32)
        if len(tok_idx) == 0:
            continue
        if fused:
            g = oracle.gate_activation(t.gx[tok_idx], t.A_log, t.dt_bias)
            beta = oracle.sigmoid(t.bx[tok_idx])
        else:
            g, beta = t.g[tok_idx], t.beta[tok_idx]
        o_ref, st_ref = oracle.decode_steps(t.q[tok_idx], t.k[tok_idx], t.v[tok_idx], g, beta, sub_cu,
                                            pool_before[slots[reqs]], scale=t.scale)
        og = host(o[torch.as_tensor(tok_idx).cuda()])
        assert np.isfinite(og).all(), name
        e_o = max(e_o, max_abs(og, o_ref))
        fullh = full[torch.as_tensor(reqs).cuda()].float().cpu().numpy()
        got, ref, last_got, last_ref = [], [], [], []
        for i, n in enumerate(reqs):
            L = cu[n + 1] - cu[n]
            for j in range(min(L, pitch)):
                got.append(fullh[i, j])
                ref.append(st_ref[sub_cu[i] + j])
            # cache entries the call must not write keep the sentinel
            assert (fullh[i, min(L, pitch):] == SENTINEL).all(), (name, n)
            if L > 0 and update_pool:
                last_got.append(host(pool[int(slots[n])]))
                last_ref.append(st_ref[sub_cu[i] + L - 1])
        for key, gg, rr in (("c", got, ref), ("p", last_got, last_ref)):
            if gg and (key == "c" or update_pool):
                gg, rr = np.stack(gg).astype(np.float64), np.stack(rr)
                sq[key][0] += float(np.sum((gg - rr) ** 2))
                sq[key][1] += float(np.sum(rr ** 2))
                w = unit_rel_l2(gg, rr)
                if key == "c":
                    worst_c = max(worst_c, w)
                    n_steps += len(gg)
                else:
                    worst_p = max(worst_p, w)
    e_c = (sq["c"][0] / sq["c"][1]) ** 0.5 if sq["c"][1] > 0 else 0.0
    say("%s: %d requests, o max-abs %.3e  cached-state rel-L2 %.3e (worst unit %.3e, %d steps)"
        % (name, N, e_o, e_c, worst_c, n_steps))
    assert e_o <= O_MAXABS, name
    assert e_c <= tol and worst_c <= tol_u, name
    lens = cu[1:] - cu[:-1]
    if update_pool and sq["p"][1] > 0:
        e_p = (sq["p"][0] / sq["p"][1]) ** 0.5
        say("%s: pool rows rel-L2 %.3e (worst unit %.3e)" % (name, e_p, worst_p))
        assert e_p <= tol and worst_p <= tol_u, name
        untouched = np.setdiff1d(np.arange(S), slots[lens > 0])
    else:
        untouched = np.arange(S)
    ut = torch.as_tensor(untouched)
    assert torch.equal(pool[ut.cuda()].cpu(), pool_before[ut]), name


def test_multi_varlen(K, oracle):
    """Requests of 1..6 tokens and one empty request, pitch 8, K = V = 128."""
    m = W.make_multi_decode(401, [3, 1, 6, 0, 5, 2, 4], 2, 4, 128, 128, num_slots=12, cache_pitch=8)
    check(K, oracle, m, "multi varlen")


def test_multi_pitch_shorter_than_drafts(K, oracle):
    """Steps at or beyond the pitch are not cached; the last state still
    reaches the pool."""
    m = W.make_multi_decode(402, [5, 2, 4, 1], 2, 4, 64, 64, num_slots=6, cache_pitch=2, pad=1)
    check(K, oracle, m, "multi pitch 2")


def test_multi_view_of_larger_cache(K, oracle):
    """A cache allocated for 8 steps and passed as a 3-step view: the pitch
    comes from stride(0), so request n's steps land at n * 8 + j."""
    m = W.make_multi_decode(403, [3, 3, 2, 3], 1, 2, 128, 128, num_slots=6, cache_pitch=3)
    check(K, oracle, m, "multi view pitch 8", alloc_steps=8)


@pytest.mark.parametrize("fused,state", [(False, "f32"), (True, "bf16")])
def test_multi_long_requests(K, oracle, fused, state):
    """Requests longer than the kernel's batch of tokens staged in LDS (8):
    9, 17 and 12 tokens run in two or three batches; steps at or beyond the
    pitch of 10 are not cached."""
    m = W.make_multi_decode(410, [9, 17, 3, 8, 12, 1], 2, 4, 128, 128, num_slots=8, cache_pitch=10,
                            state_dtype=state)
    check(K, oracle, m, "multi long requests%s %s" % (" fused" if fused else "", state), fused=fused)


def test_multi_read_only_pool(K, oracle):
    m = W.make_multi_decode(404, [4, 4, 4], 2, 4, 128, 128, num_slots=5, cache_pitch=4)
    check(K, oracle, m, "multi read-only pool", update_pool=False)


@pytest.mark.parametrize("dk,dv,io,state", [(32, 32, "f32", "f32"), (128, 64, "bf16", "bf16"),
                                            (64, 128, "f32", "bf16")])
def test_multi_head_dims(K, oracle, dk, dv, io, state):
    m = W.make_multi_decode(405 + dk + dv, [2, 5, 3], 2, 4, dk, dv, num_slots=8, cache_pitch=6, io=io,
                            state_dtype=state, scale=dk ** -0.5)
    check(K, oracle, m, "multi dk=%d dv=%d %s/%s" % (dk, dv, io, state))


def test_multi_scalar_gate(K, oracle):
    m = W.make_multi_decode(406, [4, 2, 3], 4, 8, 128, 128, num_slots=6, cache_pitch=4, scalar_gate=True)
    check(K, oracle, m, "multi scalar gate")


@pytest.mark.parametrize("scalar", [False, True])
def test_multi_fused_gate(K, oracle, scalar):
    m = W.make_multi_decode(407, [4, 1, 3, 5], 2, 4, 128, 128, num_slots=8, cache_pitch=5,
                            scalar_gate=scalar)
    check(K, oracle, m, "multi fused gate%s" % (" scalar" if scalar else ""), fused=True)


def test_multi_full_size_all_requests(K, oracle):
    """The verify workload: 1024 requests x 4 tokens, Hv = 32, K = V = 128,
    fp32 pool of 1088 slots, cache pitch 8 (16 GiB); every request's outputs
    and cached states checked against the oracle (streamed 64 requests at a
    time), every untouched pool row bitwise."""
    say("generating verify workload: 1024 requests x 4 tokens, Hv=32, pool 1088 slots")
    m = W.spec_decode_b1024()
    check(K, oracle, m, "multi B=1024x4", fused=True, update_pool=False)


def test_multi_batch_beyond_65535(K, oracle):
    """70,000 requests of 1..2 tokens, one head, K = V = 32: the request axis
    is grid x (limit 2^31 - 1).  Every request and cached step checked."""
    m = W.make_multi_decode(409, (70000, 1, 2), 1, 1, 32, 32, num_slots=70016, cache_pitch=2)
    check(K, oracle, m, "multi N=70000", batch=8192)
