"""CPU oracle for the KDA gated delta rule — TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this module.  The product package never imports it,
and it imports nothing from the product package.

Contents
--------
* ``prefill`` / ``decode``: the fp64 token-by-token recurrence in C
  (``kda_oracle.c``, loaded with ctypes), plus the state-pool bookkeeping
  (gather initial rows, run dense, scatter final rows into a copy).
* ``recurrent_np``: the same recurrence written again in numpy (cross-check of
  the C code for implementation slips; not a pin by itself).
* ``transition_np``: the recurrence in transition-matrix form
  ``S_t = (I - b_t k_t k_t^T) D_t S_{t-1} + b_t k_t v_t^T`` (brute force).
* ``chunked_np``: the chunk-parallel (UT-transform) form with an explicit
  triangular solve, exposing per-chunk intermediates; its agreement with the
  recurrence pins the algebra the GPU kernels are built on.

Sources (the pages never print the recurrence; see ``kda_oracle.c``):
  * sglang PR 27488 digest (KDA SM100 CuteDSL prefill): section 功能与动机
    (per-channel decay gate; outputs compared with a token-by-token
    baseline), section 实现拆解 (chunk size 64; KKT inverse + U/W step; the
    per-chunk cumsum of the gate).
  * sglang PR 30169 digest (pool-state I/O fused into the state kernel):
    section 实现拆解 and the key-code test (state pool [slots, Hv, V, K],
    per-sequence slot indices, padding index -1 maps to the last slot, pool
    rows that are not indexed stay untouched).

Parity status: every function here is pinned by ``tests/test_oracle_pins.py``
(closed forms, invariants, the transition-matrix brute force and the
chunked-vs-recurrent equivalence).
"""
from __future__ import annotations

import contextlib
import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "kda_oracle.c")
_LIB = os.path.join(_HERE, "libkda_oracle.so")
_lib = None


def build(force: bool = True) -> str:
    """Compile the C oracle with gcc (fp64, OpenMP).  Returns the .so path."""
    if force or not os.path.exists(_LIB):
        tmp = _LIB + ".tmp%d" % os.getpid()
        cmd = ["gcc", "-O2", "-std=c99", "-fopenmp", "-fPIC", "-shared",
               "-o", tmp, _SRC, "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(tmp, _LIB)
    return _LIB


def _bind(lib):
    lib.kdaref_prefill.restype = ctypes.c_int
    lib.kdaref_prefill.argtypes = [
        ctypes.c_int32, ctypes.c_void_p,
        ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32,
        ctypes.c_int32, ctypes.c_double,
        ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
        ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
        ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int32]
    lib.kdaref_max_threads.restype = ctypes.c_int
    lib.kdaref_max_threads.argtypes = []
    return lib


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB):
            build(force=False)
        _lib = _bind(ctypes.CDLL(_LIB))
    return _lib


@contextlib.contextmanager
def use_library(path):
    """Temporarily route the ctypes calls to another build of kda_oracle.c
    (the mutation tests compile deliberately broken copies and check that the
    pins reject them)."""
    global _lib
    saved = _lib
    _lib = _bind(ctypes.CDLL(path))
    try:
        yield
    finally:
        _lib = saved


def max_threads() -> int:
    return int(_load().kdaref_max_threads())


def _f32(x):
    """Exact conversion of a bf16/fp32 host array (numpy or torch) to float32."""
    if hasattr(x, "detach"):  # torch tensor on the CPU
        x = x.detach().cpu().float().numpy()
    return np.ascontiguousarray(np.asarray(x, dtype=np.float32))


def _f64(x):
    """Exact conversion of a bf16/fp32/fp64 host array (numpy or torch) to float64."""
    if hasattr(x, "detach"):  # torch tensor on the CPU
        x = x.detach().cpu().double().numpy()
    return np.ascontiguousarray(np.asarray(x, dtype=np.float64))


def _ptr(a):
    return None if a is None else a.ctypes.data


def prefill(q, k, v, g, beta, cu_seqlens, h0=None, scale=1.0,
            want_state=True, nthreads=0):
    """Dense-mode prefill in fp64.

    q, k: [T, Hk, K]; v: [T, Hv, V]; g: [T, Hv, K] or [T, Hv] (scalar gate);
    beta: [T, Hv]; cu_seqlens: [N + 1]; h0: [N, Hv, V, K] or None (zeros).
    Returns (o [T, Hv, V] float64, ht [N, Hv, V, K] float64 or None).
    """
    q, k, v = (_f32(x) for x in (q, k, v))
    g, beta = _f64(g), _f64(beta)
    cu = np.ascontiguousarray(np.asarray(
        cu_seqlens.cpu() if hasattr(cu_seqlens, "cpu") else cu_seqlens, dtype=np.int32))
    n = cu.shape[0] - 1
    T, hk, dk = q.shape
    hv, dv = v.shape[1], v.shape[2]
    assert k.shape == q.shape and v.shape[0] == T and beta.shape == (T, hv)
    gate_scalar = 1 if g.ndim == 2 else 0
    assert g.shape == ((T, hv) if gate_scalar else (T, hv, dk))
    assert int(cu[-1]) == T
    h0f = None if h0 is None else _f32(h0)
    if h0f is not None:
        assert h0f.shape == (n, hv, dv, dk)
    o = np.zeros((T, hv, dv), dtype=np.float64)
    ht = np.zeros((n, hv, dv, dk), dtype=np.float64) if want_state else None
    rc = _load().kdaref_prefill(n, _ptr(cu), hk, hv, dk, dv, gate_scalar, float(scale),
                                _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta),
                                _ptr(h0f), _ptr(o), _ptr(ht), int(nthreads))
    if rc != 0:
        raise ValueError("kdaref_prefill rejected the shapes")
    return o, ht


# ---------------------------------------------------------------------------
# gate activation (fp64)
# ---------------------------------------------------------------------------
#
# The log-decay gate and the write strength are produced from raw per-token
# projections: g = -exp(A_log) * softplus(x + dt_bias) and beta = sigmoid(b)
# (GDN pool-mode digest, sglang PR 30169, key-code test: per value head A_log
# and dt_bias, raw a and b of shape [T, Hv]; KDA prefill digest, sglang
# PR 27488, key-code extend wrapper: A_log and dt_bias handed to the kernel
# entry).  For the per-channel (KDA) gate, x is [T, Hv, K] and A_log, dt_bias
# are [Hv, K] (one pair per value head and key channel); for the scalar (GDN)
# gate x is [T, Hv] and A_log, dt_bias are [Hv].

def softplus(z):
    """log(1 + e^z) in fp64, written as max(z, 0) + log1p(e^-|z|) so that
    neither branch overflows."""
    z = _f64(z)
    return np.maximum(z, 0.0) + np.log1p(np.exp(-np.abs(z)))


def sigmoid(b):
    """1 / (1 + e^-b) in fp64, evaluated through e^-|b| (no overflow)."""
    b = _f64(b)
    e = np.exp(-np.abs(b))
    return np.where(b >= 0, 1.0 / (1.0 + e), e / (1.0 + e))


def gate_activation(x, A_log, dt_bias):
    """g = -exp(A_log) * softplus(x + dt_bias), fp64, broadcast over tokens.

    x: [T, Hv, K] with A_log, dt_bias [Hv, K] (per channel), or x: [T, Hv]
    with A_log, dt_bias [Hv] (scalar gate).  Returns g with the shape of x."""
    x, A_log, dt_bias = _f64(x), _f64(A_log), _f64(dt_bias)
    assert A_log.shape == x.shape[1:] and dt_bias.shape == x.shape[1:]
    return -np.exp(A_log)[None] * softplus(x + dt_bias[None])


def prefill_fused_gate(q, k, v, x, A_log, dt_bias, b, cu_seqlens, h0=None, scale=1.0,
                       want_state=True, nthreads=0):
    """Dense-mode prefill from raw gate inputs: the activation above, then the
    recurrence (``prefill``) on the fp64 g and beta."""
    return prefill(q, k, v, gate_activation(x, A_log, dt_bias), sigmoid(b), cu_seqlens,
                   h0=h0, scale=scale, want_state=want_state, nthreads=nthreads)


def decode_steps(q, k, v, g, beta, cu_seqlens, h0, scale=1.0, nthreads=0):
    """Multi-token decode (speculative draft / verify) with the state after
    every token, fp64.

    Request n runs its tokens [cu[n], cu[n+1]) from h0[n].  Returns (o
    [T, Hv, V], states [T, Hv, V, K]) where states[t] is the state right after
    token t: the per-step intermediate states a verify step caches so that the
    state at any accepted draft length can be restored (FLA/MoE shape-limits
    digest, sglang PR 37317, 实现拆解 item 2 and the key-code snippet: a
    per-request cache of per-step states whose step pitch is fixed at
    allocation while the draft count varies from call to call).

    Written as the plain recurrence on every prefix: the state after token j
    of request n is the final state of the prefix [cu[n], cu[n] + j] run from
    h0[n] (all prefixes go through ``prefill`` in one batched call)."""
    cu = np.asarray(cu_seqlens.cpu() if hasattr(cu_seqlens, "cpu") else cu_seqlens, dtype=np.int64)
    q, k, v = (_f32(x) for x in (q, k, v))
    g, beta = _f64(g), _f64(beta)
    h0 = _f32(h0)
    T = q.shape[0]
    idx, pcu, ph0 = [], [0], []
    for n in range(len(cu) - 1):
        for end in range(cu[n] + 1, cu[n + 1] + 1):
            idx.extend(range(cu[n], end))
            pcu.append(len(idx))
            ph0.append(h0[n])
    hv, dv, dk = v.shape[1], v.shape[2], q.shape[2]
    if T == 0:
        return np.zeros((0, hv, dv)), np.zeros((0, hv, dv, dk))
    idx = np.asarray(idx)
    o_all, ht = prefill(q[idx], k[idx], v[idx], g[idx], beta[idx], np.asarray(pcu, np.int32),
                        h0=np.stack(ph0), scale=scale, nthreads=nthreads)
    # prefix p ends at token t = idx[pcu[p + 1] - 1]; its last output row is o_t
    ends = np.asarray(pcu[1:]) - 1
    order = idx[ends]
    o = np.zeros((T, hv, dv))
    states = np.zeros((T, hv, dv, dk))
    o[order] = o_all[ends]
    states[order] = ht
    return o, states


def map_slot(idx, num_slots):
    """Padding index -1 (any negative) selects the last (sentinel) slot
    (PR 30169 digest, 实现拆解 item 3 and the wrapper code)."""
    idx = np.asarray(idx, dtype=np.int64)
    return np.where(idx >= 0, idx, num_slots - 1)


def prefill_pool(q, k, v, g, beta, cu_seqlens, pool, indices, scale=1.0, nthreads=0):
    """Pool-mode prefill: gather the indexed rows as h0, run dense, scatter the
    final states into a float64 copy of the pool.  Returns (o, new_pool)."""
    pool64 = _f32(pool).astype(np.float64)
    slots = map_slot(indices, pool64.shape[0])
    h0 = pool64[slots].astype(np.float32)  # exact: the pool holds floats
    o, ht = prefill(q, k, v, g, beta, cu_seqlens, h0=h0, scale=scale, nthreads=nthreads)
    for i, s in enumerate(slots):
        pool64[s] = ht[i]
    return o, pool64


def decode(q, k, v, g, beta, h0, scale=1.0, nthreads=0):
    """One-token step for B independent requests (the recurrence with T = 1).

    q, k: [B, Hk, K]; v: [B, Hv, V]; g: [B, Hv, K] or [B, Hv]; beta: [B, Hv];
    h0: [B, Hv, V, K] (the requests' gathered states).  Returns (o, ht)."""
    B = q.shape[0]
    cu = np.arange(B + 1, dtype=np.int32)
    return prefill(q, k, v, g, beta, cu, h0=h0, scale=scale, nthreads=nthreads)


# ---------------------------------------------------------------------------
# numpy forms (fp64) for small inputs
# ---------------------------------------------------------------------------

def _gate_vec(g, t, h, dk):
    return np.full(dk, g[t, h]) if g.ndim == 2 else g[t, h]


def recurrent_np(q, k, v, g, beta, cu_seqlens, h0=None, scale=1.0):
    """The recurrence again, in numpy: decay, residual, rank-1 write, read-out."""
    q, k, v, g, beta = (_f64(x) for x in (q, k, v, g, beta))
    cu = np.asarray(cu_seqlens, dtype=np.int64)
    T, hk, dk = q.shape
    hv, dv = v.shape[1:]
    grp = hv // hk
    o = np.zeros((T, hv, dv))
    ht = np.zeros((len(cu) - 1, hv, dv, dk))
    for n in range(len(cu) - 1):
        for h in range(hv):
            S = np.zeros((dk, dv)) if h0 is None else np.asarray(_f32(h0[n, h]), np.float64).T.copy()
            for t in range(cu[n], cu[n + 1]):
                kt, qt = k[t, h // grp], q[t, h // grp]
                S = np.exp(_gate_vec(g, t, h, dk))[:, None] * S
                u = beta[t, h] * (v[t, h] - S.T @ kt)
                S = S + np.outer(kt, u)
                o[t, h] = scale * (S.T @ qt)
            ht[n, h] = S.T
    return o, ht


def transition_np(q, k, v, g, beta, h0=None, scale=1.0):
    """Single sequence, brute force through explicit K x K transition matrices:
    S_t = (I - b_t k_t k_t^T) diag(exp g_t) S_{t-1} + b_t k_t v_t^T.
    Algebraically equal to the recurrence; shares none of its steps."""
    q, k, v, g, beta = (_f64(x) for x in (q, k, v, g, beta))
    T, hk, dk = q.shape
    hv, dv = v.shape[1:]
    grp = hv // hk
    o = np.zeros((T, hv, dv))
    ht = np.zeros((hv, dv, dk))
    eye = np.eye(dk)
    for h in range(hv):
        S = np.zeros((dk, dv)) if h0 is None else np.asarray(_f32(h0[h]), np.float64).T.copy()
        for t in range(T):
            kt = k[t, h // grp]
            M = (eye - beta[t, h] * np.outer(kt, kt)) @ np.diag(np.exp(_gate_vec(g, t, h, dk)))
            S = M @ S + beta[t, h] * np.outer(kt, v[t, h])
            o[t, h] = scale * (S.T @ q[t, h // grp])
        ht[h] = S.T
    return o, ht


def chunked_np(q, k, v, g, beta, cu_seqlens, h0=None, scale=1.0, chunk=64,
               keep_intermediates=False):
    """Chunk-parallel form of the same recurrence, fp64, pairwise gate factors.

    Per (sequence, head, chunk of L <= ``chunk`` tokens), with G the in-chunk
    inclusive cumsum of g (PR 27488 digest, 实现拆解 and key-file list: the
    prologue's per-chunk cumsum, the KKT-inverse + U/W kernel, the state kernel
    and the output kernel):

      A[r,i] = beta_r * sum_c k[r,c] k[i,c] exp(G[r,c] - G[i,c])   (i < r)
      Tm     = (I + A)^-1                     (explicit triangular solve)
      Ut     = Tm diag(beta) V
      W      = Tm diag(beta) (K * exp(G))
      U      = Ut - W S0                      (the true residuals u_r)
      O      = scale * ((Q * exp(G)) S0 + M U),
               M[r,i] = sum_c q[r,c] k[i,c] exp(G[r,c] - G[i,c])  (i <= r)
      S_L    = diag(exp(G_last)) S0 + (K * exp(G_last - G))^T U

    Every exp argument here is a later-minus-earlier cumsum difference (<= 0
    for g <= 0).  Returns (o, ht) and, if asked, a list of per-chunk dicts
    (seq, head, t0, L, G, A, Tm, Ut, W, U, S0) in the GPU's storage orientation
    where that matters (S0 as [V, K])."""
    q, k, v, g, beta = (_f64(x) for x in (q, k, v, g, beta))
    cu = np.asarray(cu_seqlens, dtype=np.int64)
    T, hk, dk = q.shape
    hv, dv = v.shape[1:]
    grp = hv // hk
    o = np.zeros((T, hv, dv))
    ht = np.zeros((len(cu) - 1, hv, dv, dk))
    inter = [] if keep_intermediates else None
    for n in range(len(cu) - 1):
        for h in range(hv):
            S = np.zeros((dk, dv)) if h0 is None else np.asarray(_f32(h0[n, h]), np.float64).T.copy()
            for t0 in range(cu[n], cu[n + 1], chunk):
                t1 = min(t0 + chunk, cu[n + 1])
                L = t1 - t0
                Kc = k[t0:t1, h // grp]
                Qc = q[t0:t1, h // grp]
                Vc = v[t0:t1, h]
                bc = beta[t0:t1, h]
                gc = (np.repeat(g[t0:t1, h][:, None], dk, axis=1) if g.ndim == 2 else g[t0:t1, h])
                G = np.cumsum(gc, axis=0)                      # [L, K]
                D = G[:, None, :] - G[None, :, :]              # D[r,i,c] = G_r - G_i
                low = np.tril(np.ones((L, L), dtype=bool), -1)
                lowd = np.tril(np.ones((L, L), dtype=bool), 0)
                E = np.where(lowd[:, :, None], np.exp(np.where(lowd[:, :, None], D, 0.0)), 0.0)
                A = bc[:, None] * np.einsum("rc,ic,ric->ri", Kc, Kc, E) * low
                Tm = np.linalg.solve(np.eye(L) + A, np.eye(L))
                Ut = Tm @ (bc[:, None] * Vc)
                W = Tm @ (bc[:, None] * (Kc * np.exp(G)))
                S0 = S.copy()
                U = Ut - W @ S0
                M = np.einsum("rc,ic,ric->ri", Qc, Kc, E) * lowd
                o[t0:t1, h] = scale * ((Qc * np.exp(G)) @ S0 + M @ U)
                S = np.exp(G[-1])[:, None] * S0 + (Kc * np.exp(G[-1][None, :] - G)).T @ U
                if inter is not None:
                    inter.append(dict(seq=n, head=h, t0=int(t0), L=int(L), G=G, A=A, Tm=Tm,
                                      Ut=Ut, W=W, U=U, S0=S0.T.copy()))
            ht[n, h] = S.T
    if keep_intermediates:
        return o, ht, inter
    return o, ht
