"""Python binding of libkda (KDA gated delta rule on MI355X / gfx950).

Argument marshalling only: every step of the computation runs in the HIP
kernels of ``libkda.so``.  PyTorch supplies device memory and the current
stream.  The library must have been built (``python -m
gated_delta_rule_51_amd.build``); importing the binding never falls back to
anything else.

    o, final_state = chunk_prefill(q, k, v, g, beta, cu_seqlens,
                                   initial_state=None, state_indices=None,
                                   scale=1.0, output_final_state=True)
    o = recurrent_decode(q, k, v, g, beta, state_pool, state_indices, scale=1.0)

    # gate activation fused into the kernels: g = -exp(A_log) softplus(x + dt_bias),
    # beta = sigmoid(b), from raw x, b in the io dtype
    o, final_state = chunk_prefill_fused_gate(q, k, v, x, A_log, dt_bias, b, cu_seqlens, ...)
    o = recurrent_decode_fused_gate(q, k, v, x, A_log, dt_bias, b, state_pool, state_indices)

    # decode from one packed [q | k | v] row per request
    o = recurrent_decode_packed(qkv, g, beta, state_pool, state_indices, hk=..., hv=..., dk=..., dv=...)

    # multi-token (speculative verify) decode with a per-step state cache
    o = recurrent_decode_multi(q, k, v, g, beta, cu_seqlens, state_pool, state_indices,
                               intermediate_states=cache, update_pool=False)

Layouts (contiguous): q, k [T, Hk, K]; v [T, Hv, V]; g [T, Hv, K] (per-channel
gate) or [T, Hv] (scalar gate); beta [T, Hv] fp32; states [.., Hv, V, K];
raw x shaped like g and b like beta, both in the io dtype; A_log, dt_bias
[Hv, K] (per channel) or [Hv] (scalar) fp32.
"""
from __future__ import annotations

import ctypes
import os

import torch

__all__ = ["chunk_prefill", "chunk_prefill_noalloc", "recurrent_decode", "chunk_prefill_fused_gate",
           "recurrent_decode_fused_gate", "recurrent_decode_multi", "recurrent_decode_multi_fused_gate",
           "recurrent_decode_packed", "recurrent_decode_packed_fused_gate",
           "workspace_size", "release_workspaces", "library_path", "KdaError"]

_PKG = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_PKG, "libkda.so")

F32, BF16 = 0, 1
SCRATCH_BYTES = 256 << 20   # KDA_SCRATCH_BYTES of include/kda.h
GATE_CHANNEL, GATE_SCALAR = 0, 1
_DT = {torch.float32: F32, torch.bfloat16: BF16}


class KdaError(RuntimeError):
    pass


class PrefillDesc(ctypes.Structure):
    _fields_ = [("num_seqs", ctypes.c_int32), ("total_tokens", ctypes.c_int32),
                ("hk", ctypes.c_int32), ("hv", ctypes.c_int32),
                ("dk", ctypes.c_int32), ("dv", ctypes.c_int32),
                ("io_dtype", ctypes.c_int32), ("state_dtype", ctypes.c_int32),
                ("gate", ctypes.c_int32), ("scale", ctypes.c_float),
                ("num_slots", ctypes.c_int32)]


class MultiDecodeDesc(ctypes.Structure):
    _fields_ = [("batch", ctypes.c_int32), ("total_tokens", ctypes.c_int32),
                ("hk", ctypes.c_int32), ("hv", ctypes.c_int32),
                ("dk", ctypes.c_int32), ("dv", ctypes.c_int32),
                ("io_dtype", ctypes.c_int32), ("state_dtype", ctypes.c_int32),
                ("gate", ctypes.c_int32), ("scale", ctypes.c_float),
                ("num_slots", ctypes.c_int32), ("cache_pitch", ctypes.c_int32),
                ("update_pool", ctypes.c_int32)]


class DecodeDesc(ctypes.Structure):
    _fields_ = [("batch", ctypes.c_int32), ("hk", ctypes.c_int32), ("hv", ctypes.c_int32),
                ("dk", ctypes.c_int32), ("dv", ctypes.c_int32),
                ("io_dtype", ctypes.c_int32), ("state_dtype", ctypes.c_int32),
                ("gate", ctypes.c_int32), ("scale", ctypes.c_float),
                ("num_slots", ctypes.c_int32)]


_lib = None
_P = ctypes.c_void_p


def library_path() -> str:
    return _LIB_PATH


def lib():
    """The loaded libkda (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            raise KdaError("libkda.so is not built; run `python -m gated_delta_rule_51_amd.build`")
        L = ctypes.CDLL(_LIB_PATH)
        L.kda_chunk_prefill_workspace_size.restype = ctypes.c_size_t
        L.kda_chunk_prefill_workspace_size.argtypes = [ctypes.POINTER(PrefillDesc)]
        L.kda_chunk_prefill.restype = ctypes.c_int
        L.kda_chunk_prefill.argtypes = [ctypes.POINTER(PrefillDesc)] + [_P] * 11 + [ctypes.c_size_t, _P]
        L.kda_chunk_prefill_noalloc.restype = ctypes.c_int
        L.kda_chunk_prefill_noalloc.argtypes = [ctypes.POINTER(PrefillDesc)] + [_P] * 11
        L.kda_recurrent_decode.restype = ctypes.c_int
        L.kda_recurrent_decode.argtypes = [ctypes.POINTER(DecodeDesc)] + [_P] * 9
        L.kda_chunk_prefill_fused_gate.restype = ctypes.c_int
        L.kda_chunk_prefill_fused_gate.argtypes = [ctypes.POINTER(PrefillDesc)] + [_P] * 13 + [ctypes.c_size_t, _P]
        L.kda_recurrent_decode_fused_gate.restype = ctypes.c_int
        L.kda_recurrent_decode_fused_gate.argtypes = [ctypes.POINTER(DecodeDesc)] + [_P] * 11
        L.kda_recurrent_decode_packed.restype = ctypes.c_int
        L.kda_recurrent_decode_packed.argtypes = [ctypes.POINTER(DecodeDesc)] + [_P] * 7
        L.kda_recurrent_decode_packed_fused_gate.restype = ctypes.c_int
        L.kda_recurrent_decode_packed_fused_gate.argtypes = [ctypes.POINTER(DecodeDesc)] + [_P] * 9
        L.kda_recurrent_decode_multi.restype = ctypes.c_int
        L.kda_recurrent_decode_multi.argtypes = [ctypes.POINTER(MultiDecodeDesc)] + [_P] * 11
        L.kda_recurrent_decode_multi_fused_gate.restype = ctypes.c_int
        L.kda_recurrent_decode_multi_fused_gate.argtypes = [ctypes.POINTER(MultiDecodeDesc)] + [_P] * 13
        L.kda_status_string.restype = ctypes.c_char_p
        L.kda_status_string.argtypes = [ctypes.c_int]
        L.kda_version.restype = ctypes.c_int32
        _lib = L
    return _lib


def _check(status: int):
    if status != 0:
        raise KdaError("libkda: %s (status %d)" % (lib().kda_status_string(status).decode(), status))


def _ptr(t):
    return None if t is None else t.data_ptr()


def _stream(device):
    return torch.cuda.current_stream(device).cuda_stream


def _need(t, name, dtype=None, ndim=None):
    if t is None:
        return
    if not t.is_contiguous():
        raise ValueError("%s must be contiguous" % name)
    if dtype is not None and t.dtype != dtype:
        raise ValueError("%s must be %s, got %s" % (name, dtype, t.dtype))
    if ndim is not None and t.dim() != ndim:
        raise ValueError("%s must have %d dims" % (name, ndim))


def _rows(t, name, n, tail):
    """t must be [>= n, *tail]: rows past n (a padded batch) are allowed and
    never read; every other size must match exactly."""
    if t is None:
        return
    if t.dim() != 1 + len(tail) or t.shape[0] < n or tuple(t.shape[1:]) != tuple(tail):
        raise ValueError("%s must have shape [>= %d, %s], got %s"
                         % (name, n, ", ".join(str(x) for x in tail), tuple(t.shape)))


def _gate_shapes(gate, raw, n, hv, dk):
    """g or raw x [>= n, hv, dk] (per-channel gate) or [>= n, hv] (scalar
    gate); beta or raw b [>= n, hv]; A_log, dt_bias [hv, dk] or [hv]."""
    g = gate[0]
    if g.dim() not in (2, 3):
        raise ValueError("%s must be [T, Hv, K] or [T, Hv]" % ("gate_x" if raw else "g"))
    tail = (hv, dk) if g.dim() == 3 else (hv,)
    _rows(g, "gate_x" if raw else "g", n, tail)
    b = gate[3] if raw else gate[1]
    _rows(b, "beta_x" if raw else "beta", n, (hv,))
    if raw:
        for t, name in ((gate[1], "A_log"), (gate[2], "dt_bias")):
            if tuple(t.shape) != tail:
                raise ValueError("%s must have shape %s, got %s" % (name, tail, tuple(t.shape)))


def _head_shapes(q, k, v):
    """q, k [n, hk, dk] (k may hold padding rows), v [>= n, hv, dv] with hv a
    multiple of hk.  Returns (n, hk, dk, hv, dv)."""
    n, hk, dk = q.shape
    _rows(k, "k", n, (hk, dk))
    if v.dim() != 3:
        raise ValueError("v must be [T, Hv, V]")
    hv, dv = v.shape[1], v.shape[2]
    _rows(v, "v", n, (hv, dv))
    if hk <= 0 or hv % hk != 0:
        raise ValueError("value heads (%d) must be a multiple of key heads (%d)" % (hv, hk))
    return n, hk, dk, hv, dv


def _on_device(ref, tensors):
    """Every tensor must be a GPU tensor on ref's device: the kernels take raw
    device pointers, and a host or foreign-device pointer would be
    dereferenced on the GPU.  Returns the device."""
    dev = ref.device
    if dev.type != "cuda":
        raise ValueError("inputs must be GPU tensors, got a tensor on %s" % dev)
    for t in tensors:
        if t is not None and t.device != dev:
            raise ValueError("all tensors must be on %s, got one on %s" % (dev, t.device))
    return dev


def _io_dtype(q):
    if q.dtype not in _DT:
        raise ValueError("q/k/v must be float32 or bfloat16")
    return _DT[q.dtype]


def prefill_desc(q, v, g, num_seqs, state_dtype, scale, num_slots=0):
    T, hk, dk = q.shape
    hv, dv = v.shape[1], v.shape[2]
    return PrefillDesc(num_seqs, T, hk, hv, dk, dv, _io_dtype(q), _DT[state_dtype],
                       GATE_SCALAR if g.dim() == 2 else GATE_CHANNEL, float(scale), num_slots)


def workspace_size(desc: PrefillDesc) -> int:
    return int(lib().kda_chunk_prefill_workspace_size(ctypes.byref(desc)))


# One workspace per (device, stream); calls ordered on one stream may share it.
_WS = {}
# Workspaces replaced by a larger one.  They are kept alive: a HIP graph
# captured earlier on that stream still writes to the address it recorded,
# and freeing the buffer would hand that memory to other tensors.  Growth is
# at least twofold, so they hold at most as many bytes as the live ones.
_WS_RETIRED = []


def _workspace(device, stream, nbytes):
    key = (device.index, stream)
    ws = _WS.get(key)
    if ws is None or ws.numel() < nbytes:
        size = max(nbytes, 256)
        if ws is not None:
            _WS_RETIRED.append(ws)
            size = max(size, 2 * ws.numel())
        ws = torch.empty(size, dtype=torch.uint8, device=device)
        _WS[key] = ws
    return ws


def release_workspaces():
    """Free every prefill workspace the binding holds (the current ones and
    those kept for captured graphs).  Only safe once no captured graph that
    contains a prefill will be replayed again."""
    _WS.clear()
    _WS_RETIRED.clear()


def _gate_args(q, g, beta, raw):
    """Check the gate inputs: (g, beta) fp32, or raw (x, A_log, dt_bias, b)."""
    if raw is None:
        _need(g, "g", torch.float32)
        _need(beta, "beta", torch.float32, 2)
        return (g, beta)
    x, A_log, dt_bias, b = raw
    _need(x, "gate_x", q.dtype)
    _need(b, "beta_x", q.dtype, 2)
    _need(A_log, "A_log", torch.float32, x.dim() - 1)
    _need(dt_bias, "dt_bias", torch.float32, x.dim() - 1)
    if A_log.shape != x.shape[1:] or dt_bias.shape != x.shape[1:]:
        raise ValueError("A_log and dt_bias must have shape %s" % (tuple(x.shape[1:]),))
    return raw


def _prefill(q, k, v, gate, cu_seqlens, initial_state, state_indices, scale, output_final_state,
             state_dtype, raw, noalloc=False):
    for t, n in ((q, "q"), (k, "k"), (v, "v")):
        _need(t, n, q.dtype, 3)
    _need(cu_seqlens, "cu_seqlens", torch.int32, 1)
    _need(initial_state, "initial_state", None, 4)
    _need(state_indices, "state_indices", torch.int32, 1)
    T, hk, dk, hv, dv = _head_shapes(q, k, v)
    _gate_shapes(gate, raw, T, hv, dk)
    N = cu_seqlens.numel() - 1
    if N < 0:
        raise ValueError("cu_seqlens must hold N + 1 >= 1 offsets")
    pool = state_indices is not None
    if pool and initial_state is None:
        raise ValueError("pool mode needs the pool as initial_state")
    if initial_state is not None:
        if pool:
            if initial_state.shape[0] < 1:
                raise ValueError("the pool must have at least one row")
            _rows(initial_state, "state pool", 1, (hv, dv, dk))
        else:
            _rows(initial_state, "initial_state", N, (hv, dv, dk))
    if pool:
        _rows(state_indices, "state_indices", N, ())
    dev = _on_device(q, (k, v, *gate, cu_seqlens, initial_state, state_indices))
    sd = initial_state.dtype if initial_state is not None else (state_dtype or torch.float32)
    desc = prefill_desc(q, v, gate[0], N, sd, scale, initial_state.shape[0] if pool else 0)
    o = torch.empty(T, hv, dv, dtype=q.dtype, device=dev)
    if pool:
        final = initial_state
        fptr = None
    else:
        final = torch.empty(N, hv, dv, dk, dtype=sd, device=dev) if output_final_state else None
        fptr = _ptr(final)
    stream = _stream(dev)
    if noalloc:   # the library's own workspace
        with torch.cuda.device(dev):
            _check(lib().kda_chunk_prefill_noalloc(
                ctypes.byref(desc), _ptr(q), _ptr(k), _ptr(v), *(_ptr(t) for t in gate), _ptr(cu_seqlens),
                _ptr(initial_state), _ptr(state_indices), fptr, _ptr(o), stream))
        return o, final
    need = workspace_size(desc)
    ws = _workspace(dev, stream, need)
    fn = lib().kda_chunk_prefill_fused_gate if raw else lib().kda_chunk_prefill
    with torch.cuda.device(dev):
        _check(fn(ctypes.byref(desc), _ptr(q), _ptr(k), _ptr(v), *(_ptr(t) for t in gate),
                  _ptr(cu_seqlens), _ptr(initial_state), _ptr(state_indices), fptr,
                  _ptr(o), _ptr(ws), ws.numel(), stream))
    return o, final


def chunk_prefill(q, k, v, g, beta, cu_seqlens, *, initial_state=None, state_indices=None,
                  scale=1.0, output_final_state=True, state_dtype=None):
    """Chunked prefill over packed sequences.  Returns (o, final_state).

    Dense mode (state_indices is None): initial_state [N, Hv, V, K] or None
    (zeros); final_state is a new [N, Hv, V, K] tensor (or None when
    output_final_state is False).  Pool mode: initial_state is the pool
    [slots, Hv, V, K], updated in place at state_indices (negative -> last
    slot), and returned as final_state."""
    gate = _gate_args(q, g, beta, None)
    return _prefill(q, k, v, gate, cu_seqlens, initial_state, state_indices, scale,
                    output_final_state, state_dtype, False)


def chunk_prefill_noalloc(q, k, v, g, beta, cu_seqlens, *, initial_state=None, state_indices=None,
                          scale=1.0, output_final_state=True, state_dtype=None):
    """chunk_prefill through kda_chunk_prefill_noalloc: the library's own
    per-GPU workspace of SCRATCH_BYTES is used, so the library allocates
    nothing (o and a dense final state are still allocated here).  Calls that
    overlap in time on one GPU race on that workspace."""
    gate = _gate_args(q, g, beta, None)
    return _prefill(q, k, v, gate, cu_seqlens, initial_state, state_indices, scale,
                    output_final_state, state_dtype, False, noalloc=True)


def chunk_prefill_fused_gate(q, k, v, gate_x, A_log, dt_bias, beta_x, cu_seqlens, *,
                             initial_state=None, state_indices=None, scale=1.0,
                             output_final_state=True, state_dtype=None):
    """chunk_prefill with g = -exp(A_log) softplus(gate_x + dt_bias) and
    beta = sigmoid(beta_x) computed inside the kernels."""
    gate = _gate_args(q, None, None, (gate_x, A_log, dt_bias, beta_x))
    return _prefill(q, k, v, gate, cu_seqlens, initial_state, state_indices, scale,
                    output_final_state, state_dtype, True)


def _decode(q, k, v, gate, state_pool, state_indices, scale, raw):
    for t, n in ((q, "q"), (k, "k"), (v, "v")):
        _need(t, n, q.dtype, 3)
    _need(state_pool, "state_pool", None, 4)
    _need(state_indices, "state_indices", torch.int32, 1)
    B, hk, dk, hv, dv = _head_shapes(q, k, v)
    _gate_shapes(gate, raw, B, hv, dk)
    _rows(state_pool, "state_pool", 1, (hv, dv, dk))
    _rows(state_indices, "state_indices", B, ())
    dev = _on_device(q, (k, v, *gate, state_pool, state_indices))
    desc = DecodeDesc(B, hk, hv, dk, dv, _io_dtype(q), _DT[state_pool.dtype],
                      GATE_SCALAR if gate[0].dim() == 2 else GATE_CHANNEL, float(scale), state_pool.shape[0])
    o = torch.empty(B, hv, dv, dtype=q.dtype, device=dev)
    fn = lib().kda_recurrent_decode_fused_gate if raw else lib().kda_recurrent_decode
    with torch.cuda.device(dev):
        _check(fn(ctypes.byref(desc), _ptr(q), _ptr(k), _ptr(v), *(_ptr(t) for t in gate),
                  _ptr(state_pool), _ptr(state_indices), _ptr(o), _stream(dev)))
    return o


def recurrent_decode(q, k, v, g, beta, state_pool, state_indices, scale=1.0):
    """One-token decode for B requests, in place on the state pool.  Returns o."""
    return _decode(q, k, v, _gate_args(q, g, beta, None), state_pool, state_indices, scale, False)


def recurrent_decode_fused_gate(q, k, v, gate_x, A_log, dt_bias, beta_x, state_pool, state_indices,
                                scale=1.0):
    """recurrent_decode with the gate activation computed inside the kernel."""
    gate = _gate_args(q, None, None, (gate_x, A_log, dt_bias, beta_x))
    return _decode(q, k, v, gate, state_pool, state_indices, scale, True)


def _cache_pitch(cache, n, hv, dv, dk, dtype):
    """Step pitch of an intermediate-state cache [N', steps, Hv, V, K]: taken
    from stride(0), the per-request pitch fixed at allocation, so a view that
    keeps only the first few steps of a larger cache is accepted."""
    if cache is None:
        return 0
    if cache.dtype != dtype:
        raise ValueError("intermediate_states must have the pool's dtype %s" % dtype)
    if cache.dim() != 5 or tuple(cache.shape[2:]) != (hv, dv, dk) or cache.shape[0] < n:
        raise ValueError("intermediate_states must be [>= N, steps, Hv, V, K]")
    unit = hv * dv * dk
    st = cache.stride()
    if st[1:] != (unit, dv * dk, dk, 1) or st[0] % unit != 0 or st[0] // unit < cache.shape[1]:
        raise ValueError("intermediate_states must be contiguous within each request")
    return st[0] // unit


def _decode_multi(q, k, v, gate, cu_seqlens, state_pool, state_indices, cache, update_pool, scale, raw):
    for t, n in ((q, "q"), (k, "k"), (v, "v")):
        _need(t, n, q.dtype, 3)
    _need(cu_seqlens, "cu_seqlens", torch.int32, 1)
    _need(state_pool, "state_pool", None, 4)
    _need(state_indices, "state_indices", torch.int32, 1)
    T, hk, dk, hv, dv = _head_shapes(q, k, v)
    _gate_shapes(gate, raw, T, hv, dk)
    N = cu_seqlens.numel() - 1
    if N < 0:
        raise ValueError("cu_seqlens must hold N + 1 >= 1 offsets")
    _rows(state_pool, "state_pool", 1, (hv, dv, dk))
    _rows(state_indices, "state_indices", N, ())
    dev = _on_device(q, (k, v, *gate, cu_seqlens, state_pool, state_indices, cache))
    pitch = _cache_pitch(cache, N, hv, dv, dk, state_pool.dtype)
    desc = MultiDecodeDesc(N, T, hk, hv, dk, dv, _io_dtype(q), _DT[state_pool.dtype],
                           GATE_SCALAR if gate[0].dim() == 2 else GATE_CHANNEL, float(scale),
                           state_pool.shape[0], pitch, 1 if update_pool else 0)
    o = torch.empty(T, hv, dv, dtype=q.dtype, device=dev)
    fn = lib().kda_recurrent_decode_multi_fused_gate if raw else lib().kda_recurrent_decode_multi
    with torch.cuda.device(dev):
        _check(fn(ctypes.byref(desc), _ptr(q), _ptr(k), _ptr(v), *(_ptr(t) for t in gate), _ptr(cu_seqlens),
                  _ptr(state_pool), _ptr(state_indices), _ptr(cache) if pitch else None, _ptr(o),
                  _stream(dev)))
    return o


def recurrent_decode_multi(q, k, v, g, beta, cu_seqlens, state_pool, state_indices, *,
                           intermediate_states=None, update_pool=True, scale=1.0):
    """Multi-token decode (speculative verify): request n runs tokens
    [cu[n], cu[n+1]) from pool row state_indices[n]; the state after its j-th
    token goes to intermediate_states[n, j] ([N', steps, Hv, V, K], pitch from
    stride(0); steps beyond the pitch are not cached).  With update_pool the
    last state is written back to the pool row.  Returns o [T, Hv, V]."""
    return _decode_multi(q, k, v, _gate_args(q, g, beta, None), cu_seqlens, state_pool, state_indices,
                         intermediate_states, update_pool, scale, False)


def recurrent_decode_multi_fused_gate(q, k, v, gate_x, A_log, dt_bias, beta_x, cu_seqlens, state_pool,
                                      state_indices, *, intermediate_states=None, update_pool=True,
                                      scale=1.0):
    """recurrent_decode_multi with the gate activation computed inside the kernel."""
    gate = _gate_args(q, None, None, (gate_x, A_log, dt_bias, beta_x))
    return _decode_multi(q, k, v, gate, cu_seqlens, state_pool, state_indices, intermediate_states,
                         update_pool, scale, True)


def _decode_packed(qkv, gate, state_pool, state_indices, hk, hv, dk, dv, scale, raw):
    if qkv.dim() != 2 or qkv.shape[1] != 2 * hk * dk + hv * dv:
        raise ValueError("qkv must be [B, 2 hk dk + hv dv]")
    _need(qkv, "qkv", None, 2)
    _need(state_pool, "state_pool", None, 4)
    _need(state_indices, "state_indices", torch.int32, 1)
    B = qkv.shape[0]
    if hk <= 0 or hv % hk != 0:
        raise ValueError("value heads (%d) must be a multiple of key heads (%d)" % (hv, hk))
    _gate_shapes(gate, raw, B, hv, dk)
    _rows(state_pool, "state_pool", 1, (hv, dv, dk))
    _rows(state_indices, "state_indices", B, ())
    dev = _on_device(qkv, (*gate, state_pool, state_indices))
    desc = DecodeDesc(B, hk, hv, dk, dv, _io_dtype(qkv), _DT[state_pool.dtype],
                      GATE_SCALAR if gate[0].dim() == 2 else GATE_CHANNEL, float(scale), state_pool.shape[0])
    o = torch.empty(B, hv, dv, dtype=qkv.dtype, device=dev)
    fn = lib().kda_recurrent_decode_packed_fused_gate if raw else lib().kda_recurrent_decode_packed
    with torch.cuda.device(dev):
        _check(fn(ctypes.byref(desc), _ptr(qkv), *(_ptr(t) for t in gate), _ptr(state_pool), _ptr(state_indices),
                  _ptr(o), _stream(dev)))
    return o


def recurrent_decode_packed(qkv, g, beta, state_pool, state_indices, *, hk, hv, dk, dv, scale=1.0):
    """recurrent_decode with q, k, v read from one packed row per request:
    qkv [B, 2 hk dk + hv dv] = [q | k | v].  Returns o [B, Hv, V]."""
    _need(g, "g", torch.float32)
    _need(beta, "beta", torch.float32, 2)
    return _decode_packed(qkv, (g, beta), state_pool, state_indices, hk, hv, dk, dv, scale, False)


def recurrent_decode_packed_fused_gate(qkv, gate_x, A_log, dt_bias, beta_x, state_pool, state_indices, *,
                                       hk, hv, dk, dv, scale=1.0):
    """recurrent_decode_packed with the gate activation computed inside the kernel."""
    _need(gate_x, "gate_x", qkv.dtype)
    _need(beta_x, "beta_x", qkv.dtype, 2)
    _need(A_log, "A_log", torch.float32, gate_x.dim() - 1)
    _need(dt_bias, "dt_bias", torch.float32, gate_x.dim() - 1)
    return _decode_packed(qkv, (gate_x, A_log, dt_bias, beta_x), state_pool, state_indices, hk, hv, dk, dv,
                          scale, True)
