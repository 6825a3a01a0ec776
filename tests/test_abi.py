"""C-ABI checks that need no GPU: the library loads, exports every entry point
that include/kda.h declares, and rejects bad arguments before any HIP call.

Fake (host, never dereferenced) 16-byte-aligned pointer values are used; every
call here returns from host-side validation, so no kernel is launched."""
import ctypes
import os
import re

import pytest

import gated_delta_rule_51_amd as kda

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "kda.h")

OK, NULL, SHAPE, UNSUP, WS, ALIAS, HIP, ALIGN = range(8)


@pytest.fixture(scope="module")
def L():
    if not os.path.exists(kda.library_path()):
        from gated_delta_rule_51_amd import build
        build.build()
    return kda.lib()


def declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(kda_[a-z_0-9]+)\s*\(", src)))


def test_exports_every_declared_symbol(L):
    names = declared_functions()
    assert {"kda_chunk_prefill", "kda_chunk_prefill_workspace_size", "kda_recurrent_decode",
            "kda_status_string"} <= set(names)
    for n in names:
        assert hasattr(L, n), n


def test_status_strings(L):
    for s in range(8):
        assert L.kda_status_string(s).decode()
    assert L.kda_version() >= 100


def desc(**kw):
    d = dict(num_seqs=2, total_tokens=100, hk=2, hv=4, dk=128, dv=128, io_dtype=1, state_dtype=0,
             gate=0, scale=1.0, num_slots=0)
    d.update(kw)
    return kda.PrefillDesc(**d)


# distinct, far-apart, 16-byte aligned fake addresses
BASE = 1 << 40
def fake(i, off=0):
    return BASE + i * (1 << 32) + off


def prefill(L, d, **over):
    args = dict(q=fake(1), k=fake(2), v=fake(3), g=fake(4), beta=fake(5), cu=fake(6), state=None,
                idx=None, final=fake(7), o=fake(8), ws=fake(9), wsb=1 << 40)
    args.update(over)
    return L.kda_chunk_prefill(ctypes.byref(d), args["q"], args["k"], args["v"], args["g"], args["beta"],
                               args["cu"], args["state"], args["idx"], args["final"], args["o"],
                               args["ws"], args["wsb"], None)


def test_prefill_descriptor_errors(L):
    assert L.kda_chunk_prefill(None, *([None] * 11), 0, None) == NULL
    assert prefill(L, desc(hv=3)) == SHAPE            # hv % hk != 0
    assert prefill(L, desc(hk=0)) == SHAPE
    assert prefill(L, desc(num_seqs=-1)) == SHAPE
    assert prefill(L, desc(dk=96)) == UNSUP
    assert prefill(L, desc(dv=256)) == UNSUP
    assert prefill(L, desc(io_dtype=7)) == UNSUP
    assert prefill(L, desc(gate=5)) == UNSUP


def test_prefill_pointer_errors(L):
    d = desc()
    assert prefill(L, d, q=None) == NULL
    assert prefill(L, d, cu=None) == NULL
    assert prefill(L, d, o=None) == NULL
    assert prefill(L, d, q=fake(1, 4)) == ALIGN
    assert prefill(L, d, ws=None) == WS
    assert prefill(L, d, wsb=16) == WS
    # pool mode: pool required, final_state must be NULL or the pool
    dp = desc(num_slots=8)
    assert prefill(L, dp, idx=fake(10), state=None) == NULL
    assert prefill(L, dp, idx=fake(10), state=fake(11), final=fake(7)) == ALIAS
    assert prefill(L, desc(num_slots=0), idx=fake(10), state=fake(11), final=None) == SHAPE


def test_prefill_alias_errors(L):
    d = desc()
    assert prefill(L, d, o=fake(1)) == ALIAS                 # o is q
    assert prefill(L, d, o=fake(3, 256)) == ALIAS            # o overlaps v
    assert prefill(L, d, final=fake(2)) == ALIAS             # dense ht over k


def test_workspace_size(L):
    assert L.kda_chunk_prefill_workspace_size(None) == 0
    assert L.kda_chunk_prefill_workspace_size(ctypes.byref(desc(dk=48))) == 0
    a = L.kda_chunk_prefill_workspace_size(ctypes.byref(desc(total_tokens=1000)))
    b = L.kda_chunk_prefill_workspace_size(ctypes.byref(desc(total_tokens=5000)))
    assert b >= a


def test_noalloc_limits(L):
    """kda_chunk_prefill_noalloc: descriptor errors and a workspace beyond the
    library's array are refused from host values alone, before the array's
    device address is looked up (so these return without any HIP call)."""
    assert L.kda_chunk_prefill_noalloc(None, *([None] * 11)) == NULL
    assert L.kda_chunk_prefill_noalloc(ctypes.byref(desc(dk=48)), *([None] * 11)) == UNSUP
    big = desc(num_seqs=1, total_tokens=9000, hk=32, hv=32)
    assert L.kda_chunk_prefill_workspace_size(ctypes.byref(big)) > kda.SCRATCH_BYTES
    args = [fake(i) for i in range(1, 12)]
    assert L.kda_chunk_prefill_noalloc(ctypes.byref(big), *args) == WS
    fits = desc(num_seqs=1, total_tokens=8000, hk=32, hv=32)
    assert L.kda_chunk_prefill_workspace_size(ctypes.byref(fits)) <= kda.SCRATCH_BYTES
    hdr = open(HEADER).read()
    assert "#define KDA_SCRATCH_BYTES ((size_t)256 << 20)" in hdr
    assert kda.SCRATCH_BYTES == 256 << 20


def ddesc(**kw):
    d = dict(batch=4, hk=2, hv=4, dk=128, dv=128, io_dtype=1, state_dtype=0, gate=0, scale=1.0,
             num_slots=16)
    d.update(kw)
    return kda.DecodeDesc(**d)


def decode(L, d, **over):
    args = dict(q=fake(1), k=fake(2), v=fake(3), g=fake(4), beta=fake(5), pool=fake(6), idx=fake(7),
                o=fake(8))
    args.update(over)
    return L.kda_recurrent_decode(ctypes.byref(d), args["q"], args["k"], args["v"], args["g"],
                                  args["beta"], args["pool"], args["idx"], args["o"], None)


def test_decode_errors(L):
    assert L.kda_recurrent_decode(None, *([None] * 9)) == NULL
    assert decode(L, ddesc(hv=3)) == SHAPE
    assert decode(L, ddesc(num_slots=0)) == SHAPE
    assert decode(L, ddesc(dk=16)) == UNSUP
    assert decode(L, ddesc(state_dtype=3)) == UNSUP
    assert decode(L, ddesc(), pool=None) == NULL
    assert decode(L, ddesc(), idx=None) == NULL
    assert decode(L, ddesc(), o=fake(8, 8)) == ALIGN
    assert decode(L, ddesc(), o=fake(6, 1024)) == ALIAS     # o inside the pool
    assert decode(L, ddesc(batch=0), q=None) == OK          # nothing to do


def prefill_fused(L, d, **over):
    args = dict(q=fake(1), k=fake(2), v=fake(3), x=fake(4), A_log=fake(12), dt_bias=fake(13),
                b=fake(5), cu=fake(6), state=None, idx=None, final=fake(7), o=fake(8), ws=fake(9),
                wsb=1 << 40)
    args.update(over)
    return L.kda_chunk_prefill_fused_gate(ctypes.byref(d), args["q"], args["k"], args["v"], args["x"],
                                          args["A_log"], args["dt_bias"], args["b"], args["cu"],
                                          args["state"], args["idx"], args["final"], args["o"],
                                          args["ws"], args["wsb"], None)


def test_prefill_fused_gate_errors(L):
    assert L.kda_chunk_prefill_fused_gate(None, *([None] * 13), 0, None) == NULL
    d = desc()
    assert prefill_fused(L, desc(dk=96)) == UNSUP
    assert prefill_fused(L, d, x=None) == NULL
    assert prefill_fused(L, d, A_log=None) == NULL
    assert prefill_fused(L, d, dt_bias=None) == NULL
    assert prefill_fused(L, d, b=None) == NULL
    assert prefill_fused(L, d, A_log=fake(12, 8)) == ALIGN
    assert prefill_fused(L, d, o=fake(12)) == ALIAS          # o is A_log
    assert prefill_fused(L, d, o=fake(4, 512)) == ALIAS      # o inside the raw gate input
    assert prefill_fused(L, d, ws=None) == WS


def decode_fused(L, d, **over):
    args = dict(q=fake(1), k=fake(2), v=fake(3), x=fake(4), A_log=fake(12), dt_bias=fake(13),
                b=fake(5), pool=fake(6), idx=fake(7), o=fake(8))
    args.update(over)
    return L.kda_recurrent_decode_fused_gate(ctypes.byref(d), args["q"], args["k"], args["v"], args["x"],
                                             args["A_log"], args["dt_bias"], args["b"], args["pool"],
                                             args["idx"], args["o"], None)


def test_decode_fused_gate_errors(L):
    assert L.kda_recurrent_decode_fused_gate(None, *([None] * 11)) == NULL
    assert decode_fused(L, ddesc(hv=3)) == SHAPE
    assert decode_fused(L, ddesc(), A_log=None) == NULL
    assert decode_fused(L, ddesc(), dt_bias=None) == NULL
    assert decode_fused(L, ddesc(), dt_bias=fake(13, 4)) == ALIGN
    assert decode_fused(L, ddesc(), o=fake(13)) == ALIAS     # o is dt_bias
    assert decode_fused(L, ddesc(batch=0), x=None) == OK


def mdesc(**kw):
    d = dict(batch=4, total_tokens=12, hk=2, hv=4, dk=128, dv=128, io_dtype=1, state_dtype=0, gate=0,
             scale=1.0, num_slots=16, cache_pitch=4, update_pool=1)
    d.update(kw)
    return kda.MultiDecodeDesc(**d)


def multi(L, d, **over):
    args = dict(q=fake(1), k=fake(2), v=fake(3), g=fake(4), beta=fake(5), cu=fake(9), pool=fake(6),
                idx=fake(7), cache=fake(10), o=fake(8))
    args.update(over)
    return L.kda_recurrent_decode_multi(ctypes.byref(d), args["q"], args["k"], args["v"], args["g"],
                                        args["beta"], args["cu"], args["pool"], args["idx"], args["cache"],
                                        args["o"], None)


def test_multi_decode_errors(L):
    assert L.kda_recurrent_decode_multi(None, *([None] * 11)) == NULL
    assert L.kda_recurrent_decode_multi_fused_gate(None, *([None] * 13)) == NULL
    assert multi(L, mdesc(hv=3)) == SHAPE
    assert multi(L, mdesc(cache_pitch=-1)) == SHAPE
    assert multi(L, mdesc(total_tokens=-1)) == SHAPE
    assert multi(L, mdesc(dk=48)) == UNSUP
    assert multi(L, mdesc(), cu=None) == NULL
    assert multi(L, mdesc(), cache=None) == NULL                 # pitch > 0 needs a cache
    assert multi(L, mdesc(), cache=fake(10, 4)) == ALIGN
    assert multi(L, mdesc(), cache=fake(6, 1 << 20)) == ALIAS    # cache inside the pool
    assert multi(L, mdesc(), o=fake(10, 4096)) == ALIAS          # o inside the cache
    assert multi(L, mdesc(batch=0), q=None) == OK
    assert multi(L, mdesc(total_tokens=0), q=None, o=None, cache=fake(10)) == OK


def test_packed_decode_errors(L):
    assert L.kda_recurrent_decode_packed(None, *([None] * 7)) == NULL
    assert L.kda_recurrent_decode_packed_fused_gate(None, *([None] * 9)) == NULL
    d = ddesc()
    args = [fake(1), fake(4), fake(5), fake(6), fake(7), fake(8), None]
    bad = list(args); bad[0] = None
    assert L.kda_recurrent_decode_packed(ctypes.byref(d), *bad) == NULL
    bad = list(args); bad[5] = fake(1, 4096)                      # o inside the packed rows
    assert L.kda_recurrent_decode_packed(ctypes.byref(d), *bad) == ALIAS
    bad = list(args); bad[0] = fake(1, 8)
    assert L.kda_recurrent_decode_packed(ctypes.byref(d), *bad) == ALIGN


def test_binding_rejects_host_tensors():
    """The Python binding refuses tensors that are not on a GPU before it
    reaches the library: the kernels would dereference their host pointers."""
    import torch
    T, N, B, H, D = 8, 1, 2, 2, 32
    q = torch.zeros(T, H, D, dtype=torch.bfloat16)
    g = torch.zeros(T, H, D)
    beta = torch.zeros(T, H)
    cu = torch.tensor([0, T], dtype=torch.int32)
    with pytest.raises(ValueError, match="GPU tensors"):
        kda.chunk_prefill(q, q, q, g, beta, cu)
    pool = torch.zeros(4, H, D, D)
    idx = torch.zeros(B, dtype=torch.int32)
    qb, gb, bb = q[:B].contiguous(), g[:B].contiguous(), beta[:B].contiguous()
    with pytest.raises(ValueError, match="GPU tensors"):
        kda.recurrent_decode(qb, qb, qb, gb, bb, pool, idx)
    with pytest.raises(ValueError, match="GPU tensors"):
        kda.recurrent_decode_multi(q, q, q, g, beta, cu, pool, idx[:N].contiguous())
    qkv = torch.zeros(B, 3 * H * D, dtype=torch.bfloat16)
    with pytest.raises(ValueError, match="GPU tensors"):
        kda.recurrent_decode_packed(qkv, gb, bb, pool, idx, hk=H, hv=H, dk=D, dv=D)


def test_binding_rejects_bad_shapes():
    """Shape mismatches are refused by the binding before any device check or
    library call: each would otherwise reach the kernels as raw pointers and
    read or write past a tensor's end.  Extra (padding) rows are allowed."""
    import torch
    T, N, hk, hv, K, V = 10, 2, 2, 4, 32, 64
    bf = torch.bfloat16
    q = torch.zeros(T, hk, K, dtype=bf)
    v = torch.zeros(T, hv, V, dtype=bf)
    g = torch.zeros(T, hv, K)
    beta = torch.zeros(T, hv)
    cu = torch.tensor([0, 4, T], dtype=torch.int32)
    h0 = torch.zeros(N, hv, V, K)
    pool = torch.zeros(6, hv, V, K)
    idx = torch.zeros(N, dtype=torch.int32)
    pf = kda.chunk_prefill
    bad = [
        (lambda: pf(q, q[:, :1].contiguous(), v, g, beta, cu), "k must have shape"),
        (lambda: pf(q, q, v[:T - 1].contiguous(), g, beta, cu), "v must have shape"),
        (lambda: pf(q, q, v[:, :3].contiguous(), g, beta, cu), "multiple of key heads"),
        (lambda: pf(q, q, v, g[:, :, :16].contiguous(), beta, cu), "g must have shape"),
        (lambda: pf(q, q, v, g[:T - 2].contiguous(), beta, cu), "g must have shape"),
        (lambda: pf(q, q, v, g, beta[:T - 1].contiguous(), cu), "beta must have shape"),
        (lambda: pf(q, q, v, g, beta, cu, initial_state=h0[:1].contiguous()), "initial_state must have shape"),
        (lambda: pf(q, q, v, g, beta, cu, initial_state=h0.transpose(2, 3).contiguous()),
         "initial_state must have shape"),
        (lambda: pf(q, q, v, g, beta, cu, initial_state=pool.transpose(2, 3).contiguous(), state_indices=idx),
         "state pool must have shape"),
        (lambda: pf(q, q, v, g, beta, cu, initial_state=pool, state_indices=idx[:1].contiguous()),
         "state_indices must have shape"),
        (lambda: kda.chunk_prefill_fused_gate(q, q, v, g.to(bf), torch.zeros(hv, K), torch.zeros(hv, K),
                                              beta[:3].to(bf).contiguous(), cu), "beta_x must have shape"),
    ]
    for call, msg in bad:
        with pytest.raises(ValueError, match=msg):
            call()
    # padding rows past T are accepted (refused only for being host tensors)
    with pytest.raises(ValueError, match="GPU tensors"):
        pf(q, torch.zeros(T + 3, hk, K, dtype=bf), torch.zeros(T + 3, hv, V, dtype=bf), torch.zeros(T + 3, hv, K),
           torch.zeros(T + 3, hv), cu, initial_state=torch.zeros(N + 1, hv, V, K))
    # decode
    B = 3
    qd, vd = q[:B].contiguous(), v[:B].contiguous()
    gd, bd = g[:B].contiguous(), beta[:B].contiguous()
    dec = kda.recurrent_decode
    bad = [
        (lambda: dec(qd, qd, vd, gd, bd, pool.transpose(2, 3).contiguous(), idx[:1].repeat(B)),
         "state_pool must have shape"),
        (lambda: dec(qd, qd, vd, gd, bd, pool, idx[:2].contiguous()), "state_indices must have shape"),
        (lambda: dec(qd, qd, vd[:2].contiguous(), gd, bd, pool, idx.repeat(2)), "v must have shape"),
        (lambda: dec(qd, qd, vd, gd[:, :2].contiguous(), bd, pool, idx.repeat(2)), "g must have shape"),
        (lambda: kda.recurrent_decode_multi(qd, qd, vd, gd, bd, torch.tensor([0, 1, B], dtype=torch.int32),
                                            pool, idx[:1].contiguous()), "state_indices must have shape"),
        (lambda: kda.recurrent_decode_packed(torch.zeros(B, 2 * hk * K + hv * V, dtype=bf), gd, bd,
                                             pool, idx[:2].contiguous(), hk=hk, hv=hv, dk=K, dv=V),
         "state_indices must have shape"),
    ]
    for call, msg in bad:
        with pytest.raises(ValueError, match=msg):
            call()
