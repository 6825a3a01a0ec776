"""Why the prefill's MFMA operands are fp16, not bf16: a CPU simulation.

The chunk form of the recurrence (one chunk of L <= 64 tokens, S0 the state
entering it, G the in-chunk cumsum of g):
    A[r,i] = beta_r sum_c k[r,c] k[i,c] exp(G[r,c] - G[i,c])   (i < r)
    T = (I + A)^-1,  W = T diag(beta) (K exp(G)),  Ut = T diag(beta) V
    U = Ut - W S0,   O = scale ((Q exp(G)) S0 + M U)
    S_L = diag(exp(G_L)) S0 + (K exp(G_L - G))^T U
is evaluated here in fp64, except that every matrix-core operand the GPU
path rounds is rounded to the operand type under test, at the same points:
the gate-scaled key and query rows that form A and M (each factor
exp(G_r - G_p), exp(G_p - G_i) split at the pivot p of the pair's aligned
block, rounded, then multiplied with the rounded k or q and rounded again),
T, K beta exp(G), W, T diag(beta), M, Q exp(G), K exp(G_L - G), V, S0 and
U; products accumulate exactly (the GPU accumulates in fp32).  T = (I+A)^-1,
the state and exp(G_L) stay unrounded (fp32 on the GPU).

On the 5-sequence GQA batch (Hk = 4, Hv = 8, K = V = 128, bf16 q/k/v,
random fp32 initial states) fp16 operands keep the final states within the
1e-3 relative-L2 bound with room to spare; bf16 operands, whose significand
is three bits shorter, do not.  The GPU path (fp16) measures 3.2e-4 on this
batch.  The oracle is the fp64 token recurrence.
"""
import numpy as np

import kda_workloads as W


def rnd_f16(x):
    return np.asarray(x, np.float64).astype(np.float16).astype(np.float64)


def rnd_bf16(x):
    """Round to bfloat16, nearest even (via the fp32 bit pattern)."""
    b = np.asarray(x, np.float64).astype(np.float32).view(np.uint32).astype(np.uint64)
    b = (b + 0x7FFF + ((b >> 16) & 1)) & 0xFFFF0000
    return b.astype(np.uint32).view(np.float32).astype(np.float64)


def simulate(inp, rnd, C=64):
    """Chunked prefill with operands rounded by ``rnd``.  Returns (o, ht)."""
    f = lambda t: t.double().numpy()
    q, k, v, g, beta = f(inp.q), f(inp.k), f(inp.v), f(inp.g), f(inp.beta)
    h0 = f(inp.h0)
    cu = inp.cu_seqlens.numpy()
    T, hk, K = q.shape
    hv, V = v.shape[1], v.shape[2]
    o = np.zeros((T, hv, V))
    ht = np.zeros_like(h0)
    tok = np.arange(C)
    for n in range(len(cu) - 1):
        for h in range(hv):
            kh = h // (hv // hk)
            S = h0[n, h].T.copy()                      # K x V
            for t0 in range(cu[n], cu[n + 1], C):
                L = min(C, cu[n + 1] - t0)
                pad = lambda x: np.concatenate([x, np.zeros((C - L,) + x.shape[1:])])
                kc, qc = rnd(pad(k[t0:t0 + L, kh])), rnd(pad(q[t0:t0 + L, kh]))
                vc, bc = pad(v[t0:t0 + L, h]), pad(beta[t0:t0 + L, h])
                G = np.cumsum(pad(g[t0:t0 + L, h]), axis=0)   # padded tokens: g = 0
                A = np.zeros((C, C))
                M = np.zeros((C, C))
                for lvl in range(6):
                    bs = 1 << lvl
                    piv = ((tok >> (lvl + 1)) << (lvl + 1)) + bs - 1
                    row = (tok >> lvl) & 1 == 1
                    Gp = G[piv]
                    fr = rnd(np.exp(np.where(row[:, None], G - Gp, 0.0)))
                    fc = rnd(np.exp(np.where(row[:, None], 0.0, Gp - G)))
                    Rk, Rq, Ck = rnd(kc * fr), rnd(qc * fr), rnd(kc * fc)
                    same = (tok[:, None] >> (lvl + 1)) == (tok[None, :] >> (lvl + 1))
                    mask = same & row[:, None] & ~row[None, :]
                    A += np.where(mask, bc[:, None] * (Rk @ Ck.T), 0.0)
                    M += np.where(mask, Rq @ Ck.T, 0.0)
                M += np.diag(np.sum(qc * kc, axis=1))
                Tm = np.linalg.inv(np.eye(C) + A)
                gam = np.exp(G)
                Wm = rnd(rnd(Tm) @ rnd(kc * (bc[:, None] * gam)))
                Tb = rnd(Tm * bc[None, :])
                QG = rnd(qc * gam)
                KL = rnd(kc * np.exp(G[-1] - G))
                Ut = Tb @ rnd(vc)
                Sr = rnd(S)
                U = rnd(Ut - Wm @ Sr)
                O = inp.scale * (QG @ Sr + rnd(M) @ U)
                o[t0:t0 + L, h] = O[:L]
                S = np.exp(G[-1])[:, None] * S + KL.T @ U
            ht[n, h] = S.T
    return o, ht


def rel(a, b):
    return float(np.linalg.norm(a - b) / np.linalg.norm(b))


def test_fp16_operands_meet_the_state_bound_bf16_do_not(oracle):
    inp = W.varlen_gqa5()
    o_ref, ht_ref = oracle.prefill(inp.q, inp.k, inp.v, inp.g, inp.beta, inp.cu_seqlens, h0=inp.h0)
    o16, h16 = simulate(inp, rnd_f16)
    obf, hbf = simulate(inp, rnd_bf16)
    e16, ebf = rel(h16, ht_ref), rel(hbf, ht_ref)
    m16, mbf = float(np.abs(o16 - o_ref).max()), float(np.abs(obf - o_ref).max())
    print("final-state rel-L2: fp16 operands %.2e, bf16 operands %.2e; o max-abs: fp16 %.2e, bf16 %.2e"
          % (e16, ebf, m16, mbf))
    assert e16 < 6e-4          # inside the 1e-3 bound with room (GPU: 3.2e-4)
    assert ebf > 1.5e-3        # outside it
    assert m16 < 2e-2 and ebf / e16 > 4


def test_simulation_without_rounding_is_the_recurrence(oracle):
    """With no rounding the simulated chunk form is the fp64 recurrence (a
    check that the simulation's algebra, pivots and masks are right)."""
    inp = W.make_prefill(31, [70, 3, 130], 1, 2, 32, 32, gate="realistic", h0="random")
    o_ref, ht_ref = oracle.prefill(inp.q, inp.k, inp.v, inp.g, inp.beta, inp.cu_seqlens, h0=inp.h0)
    o, ht = simulate(inp, lambda x: np.asarray(x, np.float64))
    assert rel(ht, ht_ref) < 1e-10 and float(np.abs(o - o_ref).max()) < 1e-10
