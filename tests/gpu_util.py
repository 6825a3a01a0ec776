"""Helpers for the GPU parity tests (comparison metrics and device copies)."""
import sys

import numpy as np
import torch

# Tolerances (o: max-abs on the io dtype output; states: relative L2 over the
# whole written-state tensor).  bf16 state storage alone costs ~1.7e-3 rel-L2,
# so bf16 states are held to 5e-3 against the oracle fed the same bf16 input.
O_MAXABS = 2e-2
STATE_REL_F32 = 1e-3
STATE_REL_BF16 = 5e-3
# The same bounds held by every (sequence or request, head) state on its own,
# so that one bad chain cannot hide in the whole-tensor figure.
STATE_REL_F32_UNIT = 1e-3
STATE_REL_BF16_UNIT = 5e-3


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def dev(x):
    return None if x is None else x.cuda()


def rel_l2(got, ref):
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    den = np.linalg.norm(ref)
    return float(np.linalg.norm(got - ref) / (den if den > 0 else 1.0))


def max_abs(got, ref):
    if np.asarray(ref).size == 0:
        return 0.0
    return float(np.max(np.abs(np.asarray(got, np.float64) - np.asarray(ref, np.float64))))


def host(t):
    return t.detach().float().cpu().numpy()


def unit_rel_l2(got, ref):
    """Worst relative L2 error over the [V, K] states of a [..., V, K] array
    (states whose reference is all zero are skipped)."""
    got = np.asarray(got, np.float64).reshape(-1, *np.shape(ref)[-2:])
    ref = np.asarray(ref, np.float64).reshape(got.shape)
    num = np.linalg.norm((got - ref).reshape(len(ref), -1), axis=1)
    den = np.linalg.norm(ref.reshape(len(ref), -1), axis=1)
    keep = den > 0
    return float((num[keep] / den[keep]).max()) if keep.any() else 0.0


def check_states(name, got, ref, bf16=False):
    """Whole-tensor and worst-unit relative L2 of final states, asserted."""
    e, w = rel_l2(got, ref), unit_rel_l2(got, ref)
    say("%s: state rel-L2 %.3e (worst unit %.3e)" % (name, e, w))
    assert e <= (STATE_REL_BF16 if bf16 else STATE_REL_F32), name
    assert w <= (STATE_REL_BF16_UNIT if bf16 else STATE_REL_F32_UNIT), name
    return e, w


def compare_decode_streamed(oracle, d, o, pool, pool_before, slots, g, beta, scale, name, batch=256):
    """Every request against the oracle, a batch of requests at a time (the
    fp64 copies of a batch's states stay near 1 GB).  g, beta: callables
    giving the activated gate inputs of a request index array."""
    B = d.q.shape[0]
    e_o, num, den, worst = 0.0, 0.0, 0.0, 0.0
    for b0 in range(0, B, batch):
        reqs = np.arange(b0, min(B, b0 + batch))
        o_ref, ht_ref = oracle.decode(d.q[reqs], d.k[reqs], d.v[reqs], g(reqs), beta(reqs),
                                      pool_before[slots[reqs]], scale=scale)
        o_got = host(o[torch.as_tensor(reqs).cuda()])
        ht_got = host(pool[torch.as_tensor(slots[reqs]).cuda()])
        assert np.isfinite(o_got).all() and np.isfinite(ht_got).all(), name
        e_o = max(e_o, max_abs(o_got, o_ref))
        num += float(np.sum((ht_got.astype(np.float64) - ht_ref) ** 2))
        den += float(np.sum(ht_ref ** 2))
        worst = max(worst, unit_rel_l2(ht_got, ht_ref))
    e_s = (num / den) ** 0.5 if den > 0 else 0.0
    bf = d.pool.dtype == torch.bfloat16
    say("%s %s: %d requests, o max-abs %.3e  state rel-L2 %.3e (worst unit %.3e)"
        % (name, d.meta, B, e_o, e_s, worst))
    assert e_o <= O_MAXABS, name
    assert e_s <= (STATE_REL_BF16 if bf else STATE_REL_F32), name
    assert worst <= (STATE_REL_BF16_UNIT if bf else STATE_REL_F32_UNIT), name
