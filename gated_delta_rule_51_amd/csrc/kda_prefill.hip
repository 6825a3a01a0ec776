// Chunked prefill of the KDA gated delta rule (chunk C = 64) on gfx950.
//
// Method (chunk form of the per-head recurrence; sglang PR 27488 digest,
// sections 实现拆解 and 关键文件: per-chunk gate cumsum and pre-scaled keys, a
// KKT-inverse + U/W kernel, a state kernel and an output kernel).  For one
// chunk of L <= 64 tokens, with G_r the in-chunk inclusive cumsum of g and S0
// the state entering the chunk:
//     A[r,i] = beta_r sum_c k[r,c] k[i,c] exp(G[r,c] - G[i,c])        (i < r)
//     T = (I + A)^-1,  Ut = T diag(beta) V,  W = T diag(beta) (K * exp(G))
//     U = Ut - W S0                                  (true residual rows)
//     O = scale ((Q * exp(G)) S0 + M U),  M[r,i] = sum_c q k exp(G_r - G_i)  (i <= r)
//     S_L = diag(exp(G_last)) S0 + (K * exp(G_last - G))^T U
// Every gate factor is a product of exp(g) over a later-minus-earlier range, so
// no exponent is positive (the digest's 功能与动机 describes exp overflow to
// NaN under realistic gates; its 实现拆解 item 1 fixes it with sub-chunk
// normalisation).  Here the pairwise factor exp(G_r - G_i) is split at a pivot
// p with i <= p < r into exp(G_r - G_p) * exp(G_p - G_i), both <= 1, using a
// hierarchy of aligned blocks: the pair (r, i) belongs to the level of the
// highest bit in which r and i differ, and the pivot is the last token of the
// first half of that block.  Each level is one set of 16x16 MFMA tiles.
//
// Kernels (all on the caller's stream, no host synchronisation):
//   meta   : chunk map (sequence, local chunk) per chunk slot, from cu_seqlens
//   intra  : per (chunk, value head): gate factors, A and M on fp16 MFMA,
//            T = (I + A)^-1 by blocked inversion on fp32 MFMA, W and Ut on
//            fp16 MFMA; writes W, Ut, M, Q*exp(G), (K*exp(G_last-G))^T and
//            exp(G_last) to the workspace
//   state  : per (value tile, sequence, value head), sequential over chunks:
//            U = Ut - W S, O, state update; reads h0 and writes the final state
//            at the sequence's dense row or pool slot (sglang PR 30169 digest,
//            实现拆解 item 1), a negative slot meaning the last pool row.
//
// Operands are fp16 (bf16 q/k/v inputs convert exactly; fp16's 11-bit
// significand keeps the final-state error near 4e-4 relative, where bf16
// operands would exceed 1e-3); accumulation is fp32; the state stays fp32.
#include "kda_device.h"
#include "kda_internal.h"

namespace kda {

namespace {

constexpr int C = kChunk;   // 64
constexpr int NT = 256;     // threads per workgroup
constexpr int PADH = 8;     // fp16 row padding (16 B) against LDS bank conflicts

__device__ __forceinline__ f32x4 mfma_f16(const f16x8 &a, const f16x8 &b, const f32x4 &c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mfma_f32(float a, float b, const f32x4 &c) {
    return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 zero4() { return f32x4{0.f, 0.f, 0.f, 0.f}; }

// Insert bit value `v` at position `pos` of a 4-bit index m (result has 5 bits).
__device__ __forceinline__ int insert_bit(int m, int pos, int v) {
    return ((m >> pos) << (pos + 1)) | (v << pos) | (m & ((1 << pos) - 1));
}

// Load 8 consecutive io elements as fp16 (exact for bf16 inputs in range).
template <typename IO> __device__ __forceinline__ f16x8 load8_f16(const IO *p);
template <> __device__ __forceinline__ f16x8 load8_f16<float>(const float *p) {
    f32x4 a = *reinterpret_cast<const f32x4 *>(p), b = *reinterpret_cast<const f32x4 *>(p + 4);
    f16x8 r;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        r[i] = (_Float16)a[i];
        r[4 + i] = (_Float16)b[i];
    }
    return r;
}
template <> __device__ __forceinline__ f16x8 load8_f16<bf16>(const bf16 *p) {
    u32x4 w = *reinterpret_cast<const u32x4 *>(p);
    f16x8 r;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        r[2 * i] = (_Float16)__uint_as_float(w[i] << 16);
        r[2 * i + 1] = (_Float16)__uint_as_float(w[i] & 0xffff0000u);
    }
    return r;
}

__device__ __forceinline__ f16x8 lds8(const _Float16 *p) { return *reinterpret_cast<const f16x8 *>(p); }

// ---------------------------------------------------------------------------
// Workspace layout (per chunk slot s and value head h; all offsets 256-aligned)
// ---------------------------------------------------------------------------
struct Layout {
    size_t chunk_map, chunk_off, W, Ut, M, QG, KLt, GL, total;
    int slots;
};

__host__ __device__ inline size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

__host__ inline Layout make_layout(int num_seqs, int total_tokens, int hv, int dk, int dv) {
    Layout l{};
    const long slots = ((long)total_tokens + 63L * num_seqs) / C;
    l.slots = (int)slots;
    const size_t per = (size_t)slots * hv;
    size_t o = 0;
    l.chunk_map = o; o = align256(o + (size_t)slots * 2 * 4);
    l.chunk_off = o; o = align256(o + (size_t)(num_seqs + 1) * 4);
    l.W = o;   o = align256(o + per * C * dk * 2);
    l.Ut = o;  o = align256(o + per * C * dv * 2);
    l.M = o;   o = align256(o + per * C * C * 2);
    l.QG = o;  o = align256(o + per * C * dk * 2);
    l.KLt = o; o = align256(o + per * dk * C * 2);
    l.GL = o;  o = align256(o + per * dk * 4);
    l.total = o;
    return l;
}

struct Work {
    int2 *chunk_map;       // [slots] (seq, local chunk) or (-1, -1)
    int32_t *chunk_off;    // [N + 1] first chunk slot of each sequence
    _Float16 *W, *Ut, *M, *QG, *KLt;
    float *GL;
    int slots;
};

// ---------------------------------------------------------------------------
// meta: chunk offsets and chunk map from cu_seqlens (one workgroup)
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(1024) void meta_kernel(const int32_t *cu, int n, Work w) {
    __shared__ int32_t part[1024];
    __shared__ int32_t carry;
    const int tid = threadIdx.x;
    if (tid == 0) carry = 0;
    __syncthreads();
    for (int base = 0; base < n; base += 1024) {
        const int s = base + tid;
        int cnt = 0;
        if (s < n) {
            const int len = cu[s + 1] - cu[s];
            cnt = (len + C - 1) / C;
        }
        part[tid] = cnt;
        __syncthreads();
        for (int off = 1; off < 1024; off <<= 1) {   // inclusive scan
            const int x = tid >= off ? part[tid - off] : 0;
            __syncthreads();
            part[tid] += x;
            __syncthreads();
        }
        const int excl = carry + part[tid] - cnt;
        if (s < n) {
            w.chunk_off[s] = excl;
            for (int j = 0; j < cnt && excl + j < w.slots; ++j) w.chunk_map[excl + j] = make_int2(s, j);
        }
        __syncthreads();
        if (tid == 1023) carry += part[1023];
        __syncthreads();
    }
    const int total = carry;
    if (tid == 0) w.chunk_off[n] = total;
    for (int s = total + tid; s < w.slots; s += 1024) w.chunk_map[s] = make_int2(-1, -1);
}

// ---------------------------------------------------------------------------
// intra: per (chunk slot, value head)
// ---------------------------------------------------------------------------
template <int DK, int DV> struct IntraSmem {
    _Float16 k16[C][DK + PADH];
    _Float16 q16[C][DK + PADH];
    union {
        _Float16 F[C][DK + PADH];  // gate factors of the current level
        float scr[4][3][256];      // per-wave 16x16 fp32 scratch (inversion)
    };
    float A[C][C + 1];             // beta-scaled strictly-lower A; later T
    float M[C][C + 1];             // M, then reused as T
    _Float16 KGt[DK][C + PADH];    // (beta * K * exp(G))^T
    _Float16 Vt[DV][C + PADH];     // (beta * V)^T
    float beta[C];
    float tot[2][DK];              // per-half gate totals
};

template <int DK, int DV, typename IO, bool SCALAR>
__global__ __launch_bounds__(NT) void intra_kernel(PrefillArgs a, Work w) {
    extern __shared__ __align__(16) unsigned char smem_raw[];
    IntraSmem<DK, DV> &sm = *reinterpret_cast<IntraSmem<DK, DV> *>(smem_raw);

    const int slot = blockIdx.x, h = blockIdx.y;
    const int2 cm = w.chunk_map[slot];
    if (cm.x < 0) return;
    const int n = cm.x, jc = cm.y;
    const int t0 = a.cu_seqlens[n] + C * jc;
    const int L = min(C, a.cu_seqlens[n + 1] - t0);
    const int hk = h / (a.hv / a.hk);
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const size_t sh = (size_t)slot * a.hv + h;   // (slot, head) index

    const IO *qg = reinterpret_cast<const IO *>(a.q);
    const IO *kg = reinterpret_cast<const IO *>(a.k);
    const IO *vg = reinterpret_cast<const IO *>(a.v);

    // ---- phase 0: k, q -> fp16 LDS; beta; beta*V transposed; clear A, M ----
    constexpr int KCH = DK / 8;   // 8-element chunks per row
    for (int e = tid; e < C * KCH; e += NT) {
        const int r = e / KCH, c8 = (e % KCH) * 8;
        f16x8 kv = {}, qv = {};
        if (r < L) {
            const size_t off = ((size_t)(t0 + r) * a.hk + hk) * DK + c8;
            kv = load8_f16<IO>(kg + off);
            qv = load8_f16<IO>(qg + off);
        }
        *reinterpret_cast<f16x8 *>(&sm.k16[r][c8]) = kv;
        *reinterpret_cast<f16x8 *>(&sm.q16[r][c8]) = qv;
    }
    if (tid < C) sm.beta[tid] = tid < L ? a.beta[(size_t)(t0 + tid) * a.hv + h] : 0.f;
    for (int e = tid; e < C * (C + 1); e += NT) {
        (&sm.A[0][0])[e] = 0.f;
        (&sm.M[0][0])[e] = 0.f;
    }
    __syncthreads();
    {
        constexpr int TPJ = NT / DV;       // threads per value column
        constexpr int TOK = C / TPJ;       // tokens per thread
        const int j = tid % DV, part = tid / DV;
        for (int i = 0; i < TOK; ++i) {
            const int r = part * TOK + i;
            float x = 0.f;
            if (r < L) x = sm.beta[r] * io_traits<IO>::load(vg, ((size_t)(t0 + r) * a.hv + h) * DV + j);
            sm.Vt[j][r] = (_Float16)x;
        }
    }

    // ---- phase 1: gate factor chains, thread = (channel, half) ----
    // P[tau]: inclusive prefix product of exp(g) within the aligned 2^l block,
    // S[tau]: exclusive suffix product within the aligned 2^l block.
    const bool fthread = tid < 2 * DK;
    const int fc = tid % DK, fh = tid / DK;   // channel, half (valid if fthread)
    float P[32], S[32];
    if (fthread) {
#pragma unroll
        for (int tau = 0; tau < 32; ++tau) {
            const int r = 32 * fh + tau;
            float gv = 0.f;
            if (r < L) {
                if constexpr (SCALAR) gv = a.g[(size_t)(t0 + r) * a.hv + h];
                else gv = a.g[((size_t)(t0 + r) * a.hv + h) * DK + fc];
            }
            P[tau] = exp_f(gv);
            S[tau] = 1.f;
        }
    }

#pragma unroll
    for (int lvl = 0; lvl < 6; ++lvl) {
        if (fthread) {
            if (lvl > 0) {
                const int hb = 1 << (lvl - 1);     // sub-block size
#pragma unroll
                for (int tau = 0; tau < 32; ++tau) {
                    // S update first (reads P of the previous level)
                    if (((tau >> (lvl - 1)) & 1) == 0) {
                        const int last2 = tau | ((hb << 1) - 1);   // last of 2nd sub-block
                        S[tau] *= P[last2];
                    }
                }
#pragma unroll
                for (int tau = 31; tau >= 0; --tau) {
                    if ((tau >> (lvl - 1)) & 1) {
                        const int last1 = (tau & ~((hb << 1) - 1)) + hb - 1;   // last of 1st sub-block
                        P[tau] *= P[last1];
                    }
                }
            }
            const int bitsrc = lvl;   // bit of the token index that selects row/col
#pragma unroll
            for (int tau = 0; tau < 32; ++tau) {
                const int r = 32 * fh + tau;
                const bool row = (r >> bitsrc) & 1;
                sm.F[r][fc] = (_Float16)(row ? P[tau] : S[tau]);
            }
        }
        __syncthreads();

        // ---- MFMA tiles of this level: A (kind 0) and M (kind 1) ----
        const int njobs = lvl < 5 ? 4 : 8;
        for (int job = wave; job < njobs; job += 4) {
            int kind, rows_base, cols_base, t_half;
            if (lvl < 5) {
                t_half = job & 1;
                kind = job >> 1;
                rows_base = cols_base = 0;
            } else {
                t_half = 0;
                kind = job & 1;
                const int tile = job >> 1;   // 0..3 -> (row tile, col tile)
                rows_base = 32 + 16 * (tile >> 1);
                cols_base = 16 * (tile & 1);
            }
            const int m = lane & 15, kq = lane >> 4;
            int rtok, ctok;
            if (lvl < 5) {
                rtok = 32 * t_half + insert_bit(m, lvl, 1);
                ctok = 32 * t_half + insert_bit(m, lvl, 0);
            } else {
                rtok = rows_base + m;
                ctok = cols_base + m;
            }
            const _Float16 *src = kind == 0 ? &sm.k16[0][0] : &sm.q16[0][0];
            f32x4 acc = zero4();
#pragma unroll
            for (int kk = 0; kk < DK / 32; ++kk) {
                const int c8 = kk * 32 + kq * 8;
                f16x8 xr = lds8(src + rtok * (DK + PADH) + c8) * lds8(&sm.F[rtok][c8]);
                f16x8 yc = lds8(&sm.k16[ctok][c8]) * lds8(&sm.F[ctok][c8]);
                acc = mfma_f16(xr, yc, acc);
            }
            // scatter the valid pairs (same aligned 2^(lvl+1) block)
#pragma unroll
            for (int jj = 0; jj < 4; ++jj) {
                const int orow = 4 * kq + jj, ocol = m;
                int r, i;
                if (lvl < 5) {
                    r = 32 * t_half + insert_bit(orow, lvl, 1);
                    i = 32 * t_half + insert_bit(ocol, lvl, 0);
                } else {
                    r = rows_base + orow;
                    i = cols_base + ocol;
                }
                if ((r >> (lvl + 1)) == (i >> (lvl + 1))) {
                    if (kind == 0) sm.A[r][i] = sm.beta[r] * acc[jj];
                    else sm.M[r][i] = acc[jj];
                }
            }
        }
        __syncthreads();
    }

    // ---- diagonal of M: q_r . k_r (factor 1), from 16x16 diagonal tiles ----
    {
        const int m = lane & 15, kq = lane >> 4;
        const int base = 16 * wave;
        f32x4 acc = zero4();
#pragma unroll
        for (int kk = 0; kk < DK / 32; ++kk) {
            const int c8 = kk * 32 + kq * 8;
            acc = mfma_f16(lds8(&sm.q16[base + m][c8]), lds8(&sm.k16[base + m][c8]), acc);
        }
#pragma unroll
        for (int jj = 0; jj < 4; ++jj)
            if (4 * kq + jj == m) sm.M[base + m][base + m] = acc[jj];
    }

    // ---- chunk-level factors: exp(G_r) and exp(G_last - G_r) ----
    if (fthread) {
        // P[tau] now = prefix product within the half, S[tau] = suffix within the half
        sm.tot[fh][fc] = P[31];
    }
    __syncthreads();
    const size_t qg_off = sh * C * DK, kl_off = sh * DK * C;
    if (fthread) {
        const float t0v = sm.tot[0][fc], t1v = sm.tot[1][fc];
        if (fh == 0) w.GL[sh * DK + fc] = t0v * t1v;
#pragma unroll
        for (int tau = 0; tau < 32; ++tau) {
            const int r = 32 * fh + tau;
            const float gam = fh ? P[tau] * t0v : P[tau];          // exp(G_r)
            const float rest = fh ? S[tau] : S[tau] * t1v;         // exp(G_last - G_r)
            const float kv = (float)sm.k16[r][fc];
            const float qv = (float)sm.q16[r][fc];
            sm.KGt[fc][r] = (_Float16)(sm.beta[r] * kv * gam);
            w.QG[qg_off + (size_t)r * DK + fc] = (_Float16)(qv * gam);
            w.KLt[kl_off + (size_t)fc * C + r] = (_Float16)(kv * rest);
        }
    }
    __syncthreads();

    // ---- store M (fp16) ----
    for (int e = tid; e < C * C; e += NT) {
        const int r = e / C, i = e % C;
        w.M[sh * C * C + e] = (_Float16)sm.M[r][i];
    }
    __syncthreads();
    // the T blocks above the block diagonal are zero
    for (int e = tid; e < C * C; e += NT) {
        const int r = e / C, i = e % C;
        if ((i >> 4) > (r >> 4)) sm.M[r][i] = 0.f;
    }

    // ---- T = (I + A)^-1 into sm.M (blocked, fp32 MFMA) ----
    // scratch for 16x16 fp32 blocks: reuse F (>= 4 waves x 3 x 1 KB)
    float *scr = &sm.scr[wave][0][0];
    auto mm16 = [&](const float *X, int ldx, const float *Y, int ldy) {
        // 16x16 = X[16x16] * Y[16x16], fp32
        const int m = lane & 15, kq = lane >> 4;
        f32x4 acc = zero4();
#pragma unroll
        for (int kk = 0; kk < 4; ++kk)
            acc = mfma_f32(X[m * ldx + 4 * kk + kq], Y[(4 * kk + kq) * ldy + m], acc);
        return acc;
    };
    auto st16 = [&](float *Z, int ldz, const f32x4 &v) {
        const int m = lane & 15, kq = lane >> 4;
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) Z[(4 * kq + jj) * ldz + m] = v[jj];
    };
    auto ld16 = [&](const float *Z, int ldz) {
        const int m = lane & 15, kq = lane >> 4;
        f32x4 v;
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) v[jj] = Z[(4 * kq + jj) * ldz + m];
        return v;
    };
    constexpr int LD = C + 1;
    {
        // diagonal block b = wave: (I + A)^-1 = (I - A)(I + A^2)(I + A^4)(I + A^8)
        const int b = wave;
        const float *Ab = &sm.A[16 * b][16 * b];
        float *A2 = scr, *A4 = scr + 256, *X = scr + 512;
        f32x4 v = mm16(Ab, LD, Ab, LD);
        st16(A2, 16, v);
        __builtin_amdgcn_s_waitcnt(0);
        __builtin_amdgcn_wave_barrier();
        v = mm16(A2, 16, A2, 16);
        st16(A4, 16, v);
        // X = I - A + A^2 - A^3
        f32x4 a3 = mm16(Ab, LD, A2, 16);
        {
            const int m = lane & 15, kq = lane >> 4;
            f32x4 xv;
#pragma unroll
            for (int jj = 0; jj < 4; ++jj) {
                const int r = 4 * kq + jj;
                xv[jj] = (r == m ? 1.f : 0.f) - Ab[r * LD + m] + A2[r * 16 + m] - a3[jj];
            }
            __builtin_amdgcn_s_waitcnt(0);
            __builtin_amdgcn_wave_barrier();
            st16(X, 16, xv);
            __builtin_amdgcn_s_waitcnt(0);
            __builtin_amdgcn_wave_barrier();
            // X = X + X A^4
            f32x4 t = mm16(X, 16, A4, 16);
#pragma unroll
            for (int jj = 0; jj < 4; ++jj) xv[jj] += t[jj];
            // A^8 into A2
            f32x4 a8 = mm16(A4, 16, A4, 16);
            __builtin_amdgcn_s_waitcnt(0);
            __builtin_amdgcn_wave_barrier();
            st16(A2, 16, a8);
            st16(X, 16, xv);
            __builtin_amdgcn_s_waitcnt(0);
            __builtin_amdgcn_wave_barrier();
            t = mm16(X, 16, A2, 16);
#pragma unroll
            for (int jj = 0; jj < 4; ++jj) xv[jj] += t[jj];
            st16(&sm.M[16 * b][16 * b], LD, xv);
        }
    }
    __syncthreads();
    // off-diagonal blocks, by distance d = 1..3:  T_ab = -T_aa sum_{c=b}^{a-1} A_ac T_cb
    for (int d = 1; d <= 3; ++d) {
        const int nb = 4 - d;
        if (wave < nb) {
            const int b = wave, aa = b + d;
            float *X = scr;
            f32x4 acc = zero4();
            for (int c = b; c < aa; ++c) {
                f32x4 t = mm16(&sm.A[16 * aa][16 * c], LD, &sm.M[16 * c][16 * b], LD);
#pragma unroll
                for (int jj = 0; jj < 4; ++jj) acc[jj] += t[jj];
            }
            st16(X, 16, acc);
            __builtin_amdgcn_s_waitcnt(0);
            __builtin_amdgcn_wave_barrier();
            f32x4 tv = mm16(&sm.M[16 * aa][16 * aa], LD, X, 16);
#pragma unroll
            for (int jj = 0; jj < 4; ++jj) tv[jj] = -tv[jj];
            st16(&sm.M[16 * aa][16 * b], LD, tv);
        }
        __syncthreads();
    }
    // Inside each diagonal block the product form yields exact zeros above
    // the diagonal (every term there is a sum of zero products).

    // ---- W = T (beta K exp(G)),  Ut = T (beta V): wave = row tile ----
    {
        const int m = lane & 15, kq = lane >> 4;
        const int rt = wave;                    // rows 16 rt .. 16 rt + 15
        f16x8 ta[2];
#pragma unroll
        for (int kk = 0; kk < 2; ++kk) {
            const float *tp = &sm.M[16 * rt + m][kk * 32 + kq * 8];
#pragma unroll
            for (int e = 0; e < 8; ++e) ta[kk][e] = (_Float16)tp[e];
        }
        const int nk = (rt >> 1) + 1;           // k-steps that can be non-zero
        _Float16 *Wg = w.W + sh * C * DK;
        _Float16 *Ug = w.Ut + sh * C * DV;
#pragma unroll
        for (int ct = 0; ct < DK / 16; ++ct) {
            f32x4 acc = zero4();
            for (int kk = 0; kk < nk; ++kk)
                acc = mfma_f16(ta[kk], lds8(&sm.KGt[16 * ct + m][kk * 32 + kq * 8]), acc);
#pragma unroll
            for (int jj = 0; jj < 4; ++jj)
                Wg[(size_t)(16 * rt + 4 * kq + jj) * DK + 16 * ct + m] = (_Float16)acc[jj];
        }
#pragma unroll
        for (int ct = 0; ct < DV / 16; ++ct) {
            f32x4 acc = zero4();
            for (int kk = 0; kk < nk; ++kk)
                acc = mfma_f16(ta[kk], lds8(&sm.Vt[16 * ct + m][kk * 32 + kq * 8]), acc);
#pragma unroll
            for (int jj = 0; jj < 4; ++jj)
                Ug[(size_t)(16 * rt + 4 * kq + jj) * DV + 16 * ct + m] = (_Float16)acc[jj];
        }
    }
}

// ---------------------------------------------------------------------------
// state: per (value tile, sequence, value head), sequential over chunks
// ---------------------------------------------------------------------------
template <int DK, int BV> struct StateSmem {
    _Float16 Sh[BV][DK + PADH];   // S^T as fp16 (B operand of W S and Q S)
    _Float16 Vn[BV][C + PADH];    // U^T as fp16 (B operand of M U and K^T U)
};

template <typename ST> __device__ __forceinline__ f32x4 load_state4(const ST *p);
template <> __device__ __forceinline__ f32x4 load_state4<float>(const float *p) {
    return *reinterpret_cast<const f32x4 *>(p);
}
template <> __device__ __forceinline__ f32x4 load_state4<bf16>(const bf16 *p) { return load4(p); }
__device__ __forceinline__ void store_state4(float *p, const f32x4 &v) { *reinterpret_cast<f32x4 *>(p) = v; }
__device__ __forceinline__ void store_state4(bf16 *p, const f32x4 &v) {
    u32x2 w;
    w[0] = pack_bf16x2(v[0], v[1]);
    w[1] = pack_bf16x2(v[2], v[3]);
    *reinterpret_cast<u32x2 *>(p) = w;
}

template <int DK, int DV, int BV, typename IO, typename ST>
__global__ __launch_bounds__(NT) void state_kernel(PrefillArgs a, Work w) {
    __shared__ __align__(16) StateSmem<DK, BV> sm;
    const int vt = blockIdx.x, n = blockIdx.y, h = blockIdx.z;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int m = lane & 15, kq = lane >> 4;
    const int j0 = vt * BV;
    const int tbeg = a.cu_seqlens[n], tend = a.cu_seqlens[n + 1];
    const int nchunks = (tend - tbeg + C - 1) / C;
    const int s0 = w.chunk_off[n];

    // state tiles (rows = key channel c, cols = value j): wave owns tiles
    // st = wave + 4 k, (rt, ct) = (st / (BV/16), st % (BV/16))
    constexpr int CT = BV / 16;
    constexpr int NST = (DK / 16) * CT;
    constexpr int SPW = (NST + 3) / 4;   // state tiles per wave
    f32x4 S[SPW];

    long row_in = -1, row_out = -1;
    if (a.indices) {
        int s = a.indices[n];
        if (s < 0) s = a.num_slots - 1;
        row_in = row_out = s;
    } else {
        if (a.state_in) row_in = n;
        if (a.state_out) row_out = n;
    }
    const ST *sin = row_in >= 0 ? reinterpret_cast<const ST *>(a.state_in) + ((size_t)row_in * a.hv + h) * DV * DK
                                : nullptr;
#pragma unroll
    for (int q = 0; q < SPW; ++q) {
        const int st = wave + 4 * q;
        S[q] = zero4();
        if (st < NST && sin) {
            const int rt = st / CT, ct = st % CT;
            // lane holds S[c = 16 rt + 4 kq + jj][j = 16 ct + m]; stored [V][K]
            S[q] = load_state4<ST>(sin + (size_t)(j0 + 16 * ct + m) * DK + 16 * rt + 4 * kq);
        }
    }

    IO *og = reinterpret_cast<IO *>(a.o);

    for (int ch = 0; ch < nchunks; ++ch) {
        const size_t sh = (size_t)(s0 + ch) * a.hv + h;
        const int t0 = tbeg + ch * C;
        const int L = min(C, tend - t0);
        // (a) S^T -> fp16 LDS
#pragma unroll
        for (int q = 0; q < SPW; ++q) {
            const int st = wave + 4 * q;
            if (st < NST) {
                const int rt = st / CT, ct = st % CT;
                f16x4 hv4;
#pragma unroll
                for (int jj = 0; jj < 4; ++jj) hv4[jj] = (_Float16)S[q][jj];
                *reinterpret_cast<f16x4 *>(&sm.Sh[16 * ct + m][16 * rt + 4 * kq]) = hv4;
            }
        }
        __syncthreads();
        // (b) U = Ut - W S  -> U^T fp16 in LDS; tiles (row tile rv = token, ct)
        const _Float16 *Wg = w.W + sh * C * DK;
        const _Float16 *Ug = w.Ut + sh * C * DV;
        for (int ut = wave; ut < 4 * CT; ut += 4) {
            const int rv = ut / CT, ct = ut % CT;
            f32x4 acc = zero4();
#pragma unroll
            for (int kk = 0; kk < DK / 32; ++kk) {
                const int c8 = kk * 32 + kq * 8;
                acc = mfma_f16(lds8(Wg + (size_t)(16 * rv + m) * DK + c8), lds8(&sm.Sh[16 * ct + m][c8]), acc);
            }
            f16x4 uv;
#pragma unroll
            for (int jj = 0; jj < 4; ++jj) {
                const int r = 16 * rv + 4 * kq + jj;
                const float u = (float)Ug[(size_t)r * DV + j0 + 16 * ct + m] - acc[jj];
                uv[jj] = (_Float16)u;
            }
            *reinterpret_cast<f16x4 *>(&sm.Vn[16 * ct + m][16 * rv + 4 * kq]) = uv;
        }
        __syncthreads();
        // (c) O = scale (QG S + M U)
        const _Float16 *Qg = w.QG + sh * C * DK;
        const _Float16 *Mg = w.M + sh * C * C;
        for (int ot = wave; ot < 4 * CT; ot += 4) {
            const int rv = ot / CT, ct = ot % CT;
            f32x4 acc = zero4();
#pragma unroll
            for (int kk = 0; kk < DK / 32; ++kk) {
                const int c8 = kk * 32 + kq * 8;
                acc = mfma_f16(lds8(Qg + (size_t)(16 * rv + m) * DK + c8), lds8(&sm.Sh[16 * ct + m][c8]), acc);
            }
#pragma unroll
            for (int kk = 0; kk < 2; ++kk) {
                const int i8 = kk * 32 + kq * 8;
                acc = mfma_f16(lds8(Mg + (size_t)(16 * rv + m) * C + i8), lds8(&sm.Vn[16 * ct + m][i8]), acc);
            }
#pragma unroll
            for (int jj = 0; jj < 4; ++jj) {
                const int r = 16 * rv + 4 * kq + jj;
                if (r < L)
                    io_traits<IO>::store(og, ((size_t)(t0 + r) * a.hv + h) * DV + j0 + 16 * ct + m,
                                         a.scale * acc[jj]);
            }
        }
        // (d) S = diag(exp G_last) S + (K exp(G_last - G))^T U
        const _Float16 *Kl = w.KLt + sh * DK * C;
        const float *GLg = w.GL + sh * DK;
#pragma unroll
        for (int q = 0; q < SPW; ++q) {
            const int st = wave + 4 * q;
            if (st < NST) {
                const int rt = st / CT, ct = st % CT;
#pragma unroll
                for (int jj = 0; jj < 4; ++jj) S[q][jj] *= GLg[16 * rt + 4 * kq + jj];
#pragma unroll
                for (int kk = 0; kk < 2; ++kk) {
                    const int t8 = kk * 32 + kq * 8;
                    S[q] = mfma_f16(lds8(Kl + (size_t)(16 * rt + m) * C + t8), lds8(&sm.Vn[16 * ct + m][t8]), S[q]);
                }
            }
        }
        __syncthreads();
    }

    if (row_out >= 0) {
        ST *sout = reinterpret_cast<ST *>(a.state_out) + ((size_t)row_out * a.hv + h) * DV * DK;
#pragma unroll
        for (int q = 0; q < SPW; ++q) {
            const int st = wave + 4 * q;
            if (st < NST) {
                const int rt = st / CT, ct = st % CT;
                store_state4(sout + (size_t)(j0 + 16 * ct + m) * DK + 16 * rt + 4 * kq, S[q]);
            }
        }
    }
}

// ---------------------------------------------------------------------------
// launch
// ---------------------------------------------------------------------------
template <int DK, int DV, typename IO>
hipError_t launch_intra(PrefillArgs &a, Work &w, hipStream_t s) {
    const size_t smem = sizeof(IntraSmem<DK, DV>);
    dim3 grid(w.slots, a.hv);
    if (a.scalar_gate) {
        auto kern = intra_kernel<DK, DV, IO, true>;
        hipFuncSetAttribute((const void *)kern, hipFuncAttributeMaxDynamicSharedMemorySize, (int)smem);
        kern<<<grid, NT, smem, s>>>(a, w);
    } else {
        auto kern = intra_kernel<DK, DV, IO, false>;
        hipFuncSetAttribute((const void *)kern, hipFuncAttributeMaxDynamicSharedMemorySize, (int)smem);
        kern<<<grid, NT, smem, s>>>(a, w);
    }
    return hipGetLastError();
}

template <int DK, int DV, typename IO>
hipError_t launch_state(PrefillArgs &a, Work &w, hipStream_t s) {
    constexpr int BV = DV < 32 ? DV : 32;
    dim3 grid(DV / BV, a.num_seqs, a.hv);
    if (a.state_bf16) state_kernel<DK, DV, BV, IO, bf16><<<grid, NT, 0, s>>>(a, w);
    else state_kernel<DK, DV, BV, IO, float><<<grid, NT, 0, s>>>(a, w);
    return hipGetLastError();
}

template <int DK, int DV, typename IO>
hipError_t launch_all(PrefillArgs &a, Work &w, hipStream_t s) {
    hipError_t e = hipSuccess;
    if (w.slots > 0) {
        e = launch_intra<DK, DV, IO>(a, w, s);
        if (e != hipSuccess) return e;
    }
    return launch_state<DK, DV, IO>(a, w, s);
}

template <int DK, int DV>
hipError_t launch_io(PrefillArgs &a, Work &w, hipStream_t s) {
    return a.io_bf16 ? launch_all<DK, DV, bf16>(a, w, s) : launch_all<DK, DV, float>(a, w, s);
}

template <int DK>
hipError_t launch_dv(PrefillArgs &a, Work &w, hipStream_t s) {
    switch (a.dv) {
    case 32: return launch_io<DK, 32>(a, w, s);
    case 64: return launch_io<DK, 64>(a, w, s);
    default: return launch_io<DK, 128>(a, w, s);
    }
}

}  // namespace

size_t prefill_workspace_bytes(int num_seqs, int total_tokens, int hv, int dk, int dv) {
    return make_layout(num_seqs, total_tokens, hv, dk, dv).total;
}

hipError_t launch_prefill(PrefillArgs &a, void *workspace, hipStream_t stream) {
    const Layout l = make_layout(a.num_seqs, a.total_tokens, a.hv, a.dk, a.dv);
    char *base = static_cast<char *>(workspace);
    Work w;
    w.chunk_map = reinterpret_cast<int2 *>(base + l.chunk_map);
    w.chunk_off = reinterpret_cast<int32_t *>(base + l.chunk_off);
    w.W = reinterpret_cast<_Float16 *>(base + l.W);
    w.Ut = reinterpret_cast<_Float16 *>(base + l.Ut);
    w.M = reinterpret_cast<_Float16 *>(base + l.M);
    w.QG = reinterpret_cast<_Float16 *>(base + l.QG);
    w.KLt = reinterpret_cast<_Float16 *>(base + l.KLt);
    w.GL = reinterpret_cast<float *>(base + l.GL);
    w.slots = l.slots;

    meta_kernel<<<1, 1024, 0, stream>>>(a.cu_seqlens, a.num_seqs, w);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    switch (a.dk) {
    case 32: return launch_dv<32>(a, w, stream);
    case 64: return launch_dv<64>(a, w, stream);
    default: return launch_dv<128>(a, w, stream);
    }
}

}  // namespace kda
