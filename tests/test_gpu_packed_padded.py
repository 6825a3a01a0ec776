"""Packed-qkv decode and padded batches, on the GPU through the C ABI.

* kda_recurrent_decode_packed[_fused_gate] reads q, k, v from one
  [q | k | v] row per request; it must give bit-for-bit the result of the
  unpacked call on the same values (the same kernel, other addresses), and
  match the oracle.
* Arrays longer than the described batch (a batch padded to a captured size)
  are read only up to the described count: rows of NaN past the end change
  nothing.
"""
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


def pack(d):
    B = d.q.shape[0]
    return torch.cat([d.q.reshape(B, -1), d.k.reshape(B, -1), d.v.reshape(B, -1)], dim=1).contiguous()


@pytest.mark.parametrize("fused", [False, True])
@pytest.mark.parametrize("hk,hv,dk,dv,io", [(2, 4, 128, 128, "bf16"), (4, 8, 64, 32, "f32")])
def test_packed_decode_bitwise_and_oracle(K, oracle, fused, hk, hv, dk, dv, io):
    d = W.make_decode(501 + dk, 40, hk, hv, dk, dv, num_slots=48, io=io, pad=1)   # one -1: the sentinel row has one writer
    qkv = dev(pack(d))
    p1, p2 = dev(d.pool.clone()), dev(d.pool.clone())
    idx = dev(d.indices)
    if fused:
        gate = (dev(d.gx), dev(d.A_log), dev(d.dt_bias), dev(d.bx))
        o1 = K.recurrent_decode_fused_gate(dev(d.q), dev(d.k), dev(d.v), *gate, p1, idx)
        o2 = K.recurrent_decode_packed_fused_gate(qkv, *gate, p2, idx, hk=hk, hv=hv, dk=dk, dv=dv)
        g, beta = oracle.gate_activation(d.gx, d.A_log, d.dt_bias), oracle.sigmoid(d.bx)
    else:
        o1 = K.recurrent_decode(dev(d.q), dev(d.k), dev(d.v), dev(d.g), dev(d.beta), p1, idx)
        o2 = K.recurrent_decode_packed(qkv, dev(d.g), dev(d.beta), p2, idx, hk=hk, hv=hv, dk=dk, dv=dv)
        g, beta = d.g, d.beta
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(p1, p2)
    slots = oracle.map_slot(d.indices.numpy(), 48)
    o_ref, ht_ref = oracle.decode(d.q, d.k, d.v, g, beta, d.pool[slots])
    e_o, e_s = max_abs(host(o2), o_ref), rel_l2(host(p2[torch.as_tensor(slots).cuda()]), ht_ref)
    say("packed decode fused=%s: o max-abs %.3e  state rel-L2 %.3e" % (fused, e_o, e_s))
    assert e_o <= O_MAXABS and e_s <= STATE_REL_F32


def nan_padded(t, extra):
    pad = torch.full((extra,) + tuple(t.shape[1:]), float("nan"), dtype=t.dtype)
    return torch.cat([t, pad]).contiguous()


def test_padded_prefill_arrays(K):
    """q, k, v, g, beta with 37 NaN rows past T: o and the final states are
    bitwise those of the unpadded call, and o has exactly T rows."""
    inp = W.make_prefill(510, [70, 3, 129], 2, 4, 128, 128, gate="realistic", h0="random")
    T = inp.q.shape[0]
    o1, h1 = K.chunk_prefill(dev(inp.q), dev(inp.k), dev(inp.v), dev(inp.g), dev(inp.beta),
                             dev(inp.cu_seqlens), initial_state=dev(inp.h0))
    qp, kp, vp, gp, bp = (dev(nan_padded(x, 37)) for x in (inp.q, inp.k, inp.v, inp.g, inp.beta))
    # the binding sizes the call from q, so pass views of the first T rows
    o2, h2 = K.chunk_prefill(qp[:T], kp[:T], vp[:T], gp[:T], bp[:T], dev(inp.cu_seqlens),
                             initial_state=dev(inp.h0))
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(h1, h2)
    assert torch.isfinite(o2).all()


def test_padded_decode_arrays(K):
    d = W.make_decode(511, 30, 2, 4, 128, 128, num_slots=40)
    B = 30
    p1, p2 = dev(d.pool.clone()), dev(d.pool.clone())
    o1 = K.recurrent_decode(dev(d.q), dev(d.k), dev(d.v), dev(d.g), dev(d.beta), p1, dev(d.indices))
    pads = [dev(nan_padded(x, 9)) for x in (d.q, d.k, d.v, d.g, d.beta)]
    idx = dev(torch.cat([d.indices, torch.full((9,), 5, dtype=torch.int32)]))
    o2 = K.recurrent_decode(*(x[:B] for x in pads), p2, idx[:B])
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(p1, p2)
