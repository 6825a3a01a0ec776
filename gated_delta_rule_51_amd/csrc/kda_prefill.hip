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
// first half of that block.  Each level is one set of 16x16 MFMA tiles (with
// K = 128 the three levels inside a block of eight tokens are formed per wave).
//
// Kernels (all on the caller's stream, no host synchronisation):
//   meta   : chunk map (sequence, local chunk) per chunk slot, from cu_seqlens
//   intra  : per (chunk, value head): gate factors, A and M on fp16 MFMA,
//            T = (I + A)^-1 by blocked inversion on fp32 MFMA, W on fp16
//            MFMA; writes W, T diag(beta), M, Q*exp(G), (K*exp(G_last-G))^T
//            and exp(G_last) to the workspace (it never reads v)
//   state  : per (sequence, value head), its value columns split over wave
//            groups of one workgroup, sequential over chunks:
//            Ut = (T diag(beta)) V from the v rows it streams once, U = Ut - W S,
//            O, state update; reads h0 and writes the final state
//            at the sequence's dense row or pool slot (sglang PR 30169 digest,
//            实现拆解 item 1), a negative slot meaning the last pool row.
//
// Operands are fp16 (bf16 q/k/v inputs convert exactly; fp16's 11-bit
// significand keeps the final-state error near 4e-4 relative, where bf16
// operands would exceed 1e-3); accumulation is fp32; the state stays fp32.
#include <type_traits>

#include "kda_device.h"
#include "kda_internal.h"

namespace kda {

namespace {

constexpr int C = kChunk;   // 64
constexpr int PADH = 8;     // fp16 row padding (16 B) against LDS bank conflicts
constexpr int kOrderMax = 4096;   // sequences ranked by length in the meta kernel

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

__device__ __forceinline__ f16x8 lds8(const _Float16 *p) { return *reinterpret_cast<const f16x8 *>(p); }

// ---------------------------------------------------------------------------
// Workspace layout (per chunk slot s and value head h; all offsets 256-aligned)
// ---------------------------------------------------------------------------
struct Layout {
    size_t chunk_map, chunk_off, seq_order, W, Tb, M, QG, KLt, GL, total;
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
    l.seq_order = o; o = align256(o + (size_t)num_seqs * 4);
    l.W = o;   o = align256(o + per * C * dk * 2);
    l.Tb = o;  o = align256(o + per * C * C * 2);
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
    int32_t *seq_order;    // [N] sequences by decreasing length (state-kernel order)
    _Float16 *W, *Tb, *M, *QG, *KLt;   // Tb: T diag(beta)
    float *GL;
    int slots;
};

// ---------------------------------------------------------------------------
// meta: chunk offsets and chunk map from cu_seqlens (one workgroup)
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(1024) void meta_kernel(const int32_t *cu, int n, Work w) {
    __shared__ int32_t part[1024];
    __shared__ int32_t carry;
    __shared__ int32_t off[kOrderMax + 1];   // chunk offsets, when n <= kOrderMax
    const int tid = threadIdx.x;
    const bool staged = n <= kOrderMax;
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
        for (int o = 1; o < 1024; o <<= 1) {   // inclusive scan
            const int x = tid >= o ? part[tid - o] : 0;
            __syncthreads();
            part[tid] += x;
            __syncthreads();
        }
        const int excl = carry + part[tid] - cnt;
        if (s < n) {
            w.chunk_off[s] = excl;
            if (staged) off[s] = excl;
            else   // (each thread fills its own sequences' entries)
                for (int j = 0; j < cnt && excl + j < w.slots; ++j) w.chunk_map[excl + j] = make_int2(s, j);
        }
        __syncthreads();
        if (tid == 1023) carry += part[1023];
        __syncthreads();
    }
    const int total = carry;
    if (tid == 0) w.chunk_off[n] = total;
    if (staged) {
        // One chunk slot per thread: its sequence is the last one whose first
        // chunk slot is at or before it (binary search over the staged
        // offsets; empty sequences share the next one's offset and are
        // passed over), so one long sequence does not leave one thread to
        // write all of its entries.
        __syncthreads();
        for (int c = tid; c < w.slots; c += 1024) {
            int2 e = make_int2(-1, -1);
            if (c < total) {
                int lo = 0, hi = n - 1;   // off[lo] <= c holds throughout
                while (lo < hi) {
                    const int mid = (lo + hi + 1) >> 1;
                    if (off[mid] <= c) lo = mid;
                    else hi = mid - 1;
                }
                e = make_int2(lo, c - off[lo]);
            }
            w.chunk_map[c] = e;
        }
    } else {
        for (int c = total + tid; c < w.slots; c += 1024) w.chunk_map[c] = make_int2(-1, -1);
    }

    // Longest sequences first, so the state kernel's long sequential chains
    // start in the first wave of workgroups; equal lengths (and lengths past
    // kLenCap tokens) keep index order.  The order sorts the unique keys
    // ((kLenCap - length) << 12) | index.  Up to kRankMax sequences a thread
    // per sequence counts the keys below its own.  Beyond that, a bitonic
    // sort of the keys padded to a power of two P: thread t holds elements
    // 4t .. 4t+3, so partners up to 2 apart are in its own registers, up to
    // 128 apart in another lane of its wave (lane shuffles), and only those
    // 256 or more apart go through LDS, with a barrier per pass.  Beyond
    // kOrderMax sequences the natural order is kept.
    static_assert(kOrderMax == 4 * 1024, "four keys per thread; 12-bit index");
    constexpr uint32_t kLenCap = (1u << 20) - 2;   // the largest key stays below the padding key
    constexpr int kRankMax = 512;
    if (staged) {
        __shared__ __align__(16) uint32_t key[kOrderMax];
        auto make_key = [&](int i) -> uint32_t {
            const uint32_t len = (uint32_t)min(max(cu[i + 1] - cu[i], 0), (int)kLenCap);
            return ((kLenCap - len) << 12) | (uint32_t)i;
        };
        if (n <= kRankMax) {
            for (int i = tid; i < ((n + 3) & ~3); i += 1024) key[i] = i < n ? make_key(i) : ~0u;
            __syncthreads();
            if (tid < n) {
                const uint32_t ks = key[tid];
                int rank = 0;
                for (int m = 0; m < n; m += 4) {
                    const u32x4 km = *reinterpret_cast<const u32x4 *>(key + m);
                    rank += (km[0] < ks) + (km[1] < ks) + (km[2] < ks) + (km[3] < ks);
                }
                w.seq_order[rank] = tid;
            }
        } else {
            int P = 1;
            while (P < n) P <<= 1;
            const int lane = tid & 63;
            uint32_t x[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) x[e] = 4 * tid + e < n ? make_key(4 * tid + e) : ~0u;
            for (int k = 2; k <= P; k <<= 1) {
                int j = k >> 1;
                if (j >= 256) {   // partners in other waves
#pragma unroll
                    for (int e = 0; e < 4; ++e) key[4 * tid + e] = x[e];
                    __syncthreads();
                    for (; j >= 256; j >>= 1) {
                        for (int i = tid; i < P; i += 1024) {
                            const int ixj = i ^ j;
                            if (ixj > i) {
                                const uint32_t a = key[i], b = key[ixj];
                                if ((a > b) == ((i & k) == 0)) {
                                    key[i] = b;
                                    key[ixj] = a;
                                }
                            }
                        }
                        __syncthreads();
                    }
#pragma unroll
                    for (int e = 0; e < 4; ++e) x[e] = key[4 * tid + e];
                    __syncthreads();
                }
                for (; j >= 4; j >>= 1) {   // partners in lane tid ^ (j / 4) of this wave
                    const int m = j >> 2;
                    const bool lower = (lane & m) == 0;
                    uint32_t y[4];
#pragma unroll
                    for (int e = 0; e < 4; ++e) y[e] = __shfl_xor(x[e], m, 64);
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        const bool keep_min = lower == (((4 * tid + e) & k) == 0);
                        x[e] = keep_min ? min(x[e], y[e]) : max(x[e], y[e]);
                    }
                }
                // partners in this thread (j = 2, then 1)
#pragma unroll
                for (int jj = 2; jj >= 1; jj >>= 1) {
                    if (jj <= j) {
#pragma unroll
                        for (int e = 0; e < 4; ++e) {
                            if ((e & jj) == 0) {
                                const uint32_t a = x[e], b = x[e | jj];
                                const bool asc = ((4 * tid + e) & k) == 0;
                                x[e] = asc ? min(a, b) : max(a, b);
                                x[e | jj] = asc ? max(a, b) : min(a, b);
                            }
                        }
                    }
                }
            }
#pragma unroll
            for (int e = 0; e < 4; ++e)
                if (4 * tid + e < n) w.seq_order[4 * tid + e] = (int32_t)(x[e] & 0xfffu);
        }
    } else {
        for (int s = tid; s < n; s += 1024) w.seq_order[s] = s;
    }
}



// 16x16 fp32 block helpers for one wave (lane layout of the 16x16x4 f32 MFMA).
__device__ __forceinline__ f32x4 mm16(const float *X, int ldx, const float *Y, int ldy, int lane) {
    const int m = lane & 15, kq = lane >> 4;
    f32x4 acc = zero4();
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) acc = mfma_f32(X[m * ldx + 4 * kk + kq], Y[(4 * kk + kq) * ldy + m], acc);
    return acc;
}
__device__ __forceinline__ void st16(float *Z, int ldz, const f32x4 &v, int lane) {
    const int m = lane & 15, kq = lane >> 4;
#pragma unroll
    for (int jj = 0; jj < 4; ++jj) Z[(4 * kq + jj) * ldz + m] = v[jj];
}
// LDS writes of this wave are complete and visible to its other lanes.  Only
// the LDS counter is waited on (gfx9 s_waitcnt fields: vmcnt [3:0] and
// [15:14], expcnt [6:4], lgkmcnt [11:8]; the others are left at their
// maxima), so outstanding global stores and loads stay in flight.
__device__ __forceinline__ void wave_sync() {
    __builtin_amdgcn_s_waitcnt(0xC07F);
    __builtin_amdgcn_wave_barrier();
}

// ---------------------------------------------------------------------------
// intra: per (chunk slot, value head), 512 threads
//
// Gate factors.  Thread f = (channel c, quarter q) owns tokens t = 16 q + tau,
// tau = 0..15, of one key channel and keeps, per level l, the inclusive prefix
// product P (within the aligned 2^l block) and the exclusive suffix product S
// of a_t = exp(g_t).  At level l the pairs (r, i) whose highest differing bit
// is l are split at the pivot p = last token of the first half of their
// aligned 2^(l+1) block: exp(G_r - G_i) = P_l(r) * S_l(i), both <= 1.  Row
// tokens (bit l set) give k P and q P, column tokens give k S; these operand
// rows go to LDS in fp16 and two 16x16 MFMA tiles per t-half build A and M.
// ---------------------------------------------------------------------------
constexpr int NTI = 512;   // threads of the intra kernel
constexpr int kXcd = 8;    // XCDs of the device; workgroup ids go round robin over them

template <int DK, int DV> struct IntraMain {
    union {
        struct {
            _Float16 Fk[C][DK + PADH];        // k * factor, every token
            _Float16 Fq[C / 2][DK + PADH];    // q * factor, row tokens (bit l removed)
        } f;
        _Float16 stage[C][DK + PADH];         // Q exp(G) staging, later W staging
        float scr[9][16][20];                 // inversion scratch (16x16 fp32 blocks)
    } r1;
    _Float16 KGt[DK][C + PADH];               // (beta K exp(G))^T
    struct {
        float A[C][C + 1];                    // beta-scaled strictly-lower A
    } r3;
    float T[C][C + 1];                        // M during the levels, then T = (I + A)^-1
};
// Wave-local gate levels 0..2 (K = 128): each wave's 36 operand rows (k P,
// q P and k S for the four row / column tokens of each level in its own
// eight tokens), padded like the level rows.
constexpr int kWlRows = 36;

template <int DK, int DV> struct IntraSmem {
    float beta[C];
    float mdiag[C];   // q_t . k_t, the diagonal of M
    union {
        IntraMain<DK, DV> m;
        _Float16 wl[8][kWlRows][DK + PADH];
    } u;
};


// Gate threads: thread = (channel pair cp: channels 2cp, 2cp+1; eighth e8:
// tokens t = 8 e8 + tau, tau = 0..7).  Token bit LVL says whether t is a row
// (later half) or a column at level LVL.
template <int LVL> __device__ __forceinline__ bool row_bit(int e8, int tau) {
    if constexpr (LVL < 3) return (tau >> LVL) & 1;
    else return (e8 >> (LVL - 3)) & 1;
}

// Per-eighth gate totals exchanged during the levels (KGt is unused until the
// chunk-level phase, so its space holds them).
template <int DK, int DV> __device__ __forceinline__ float (*eighth_totals(IntraSmem<DK, DV> &sm))[DK] {
    return reinterpret_cast<float (*)[DK]>(&sm.u.m.KGt[0][0]);
}

// Empty volatile statements that differ per arm: they keep a branch on a
// wave-uniform condition from being merged into per-lane selects of both arms
// (or into one loop over a selected array, which would leave the arrays in
// scratch memory).
template <int ARM> __device__ __forceinline__ void keep_branch() {
    if constexpr (ARM == 0) asm volatile("; arm 0");
    else asm volatile("; arm 1");
}

// Advance the chains from level LVL-1 to LVL and write this level's operand
// rows: P[tau] / S[tau] hold (channel 2cp, channel 2cp+1) products as float2.
// Chains from level LVL-1 to LVL inside a thread's eight tokens (LVL = 1..3).
template <int LVL> __device__ __forceinline__ void chain_in_eighth(f32x2 (&P)[8], f32x2 (&S)[8]) {
    constexpr int hb = 1 << (LVL - 1);
#pragma unroll
    for (int tau = 0; tau < 8; ++tau)   // S first: it reads P of level LVL-1
        if (((tau >> (LVL - 1)) & 1) == 0) S[tau] *= P[tau | (2 * hb - 1)];
#pragma unroll
    for (int tau = 7; tau >= 0; --tau)
        if ((tau >> (LVL - 1)) & 1) P[tau] *= P[(tau & ~(2 * hb - 1)) + hb - 1];
}

template <int LVL, int DK, int DV>
__device__ __forceinline__ void factor_level(f32x2 (&P)[8], f32x2 (&S)[8], const f16x2 (&kr)[8],
                                             const f16x2 (&qr)[8], IntraSmem<DK, DV> &sm, int cp, int e8,
                                             f32x2 &H0, f32x2 &H1) {
    float (*etot)[DK] = eighth_totals(sm);
    if constexpr (LVL >= 1 && LVL <= 3) {
        chain_in_eighth<LVL>(P, S);
    } else if constexpr (LVL == 4) {
        // 16-token blocks = eighths (2j, 2j+1): the partner eighth's total
        const int pe = e8 ^ 1;
        const f32x2 tot = {etot[pe][2 * cp], etot[pe][2 * cp + 1]};
        if ((e8 & 1) == 0) {
#pragma unroll
            for (int tau = 0; tau < 8; ++tau) S[tau] *= tot;
            keep_branch<0>();
        } else {
#pragma unroll
            for (int tau = 0; tau < 8; ++tau) P[tau] *= tot;
            keep_branch<1>();
        }
    } else if constexpr (LVL == 5) {
        // 32-token blocks = eighths 4j..4j+3: the partner 16-token block's total
        f32x2 et[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) et[e] = f32x2{etot[e][2 * cp], etot[e][2 * cp + 1]};
        H0 = et[0] * et[1] * et[2] * et[3];
        H1 = et[4] * et[5] * et[6] * et[7];
        f32x2 tot;   // total of the other 16-token block of this half
        if ((e8 & 4) == 0) tot = (e8 & 2) ? et[0] * et[1] : et[2] * et[3];
        else tot = (e8 & 2) ? et[4] * et[5] : et[6] * et[7];
        if ((e8 & 2) == 0) {
#pragma unroll
            for (int tau = 0; tau < 8; ++tau) S[tau] *= tot;
            keep_branch<0>();
        } else {
#pragma unroll
            for (int tau = 0; tau < 8; ++tau) P[tau] *= tot;
            keep_branch<1>();
        }
    }
    // operand rows: two channels per 4-byte write.  The row/column role is
    // compile-time for LVL < 3 and uniform per thread otherwise.
    auto emit = [&](int tau, bool row, const f32x2 f) {
        const int t = 8 * e8 + tau;
        const f16x2 fac = {(_Float16)f[0], (_Float16)f[1]};
        *reinterpret_cast<f16x2 *>(&sm.u.m.r1.f.Fk[t][2 * cp]) = kr[tau] * fac;
        if (row) {
            const int ridx = ((t >> (LVL + 1)) << LVL) | (t & ((1 << LVL) - 1));
            *reinterpret_cast<f16x2 *>(&sm.u.m.r1.f.Fq[ridx][2 * cp]) = qr[tau] * fac;
        }
    };
    if constexpr (LVL < 3) {
#pragma unroll
        for (int tau = 0; tau < 8; ++tau) {
            if ((tau >> LVL) & 1) emit(tau, true, P[tau]);
            else emit(tau, false, S[tau]);
        }
    } else {
        if (row_bit<LVL>(e8, 0)) {
#pragma unroll
            for (int tau = 0; tau < 8; ++tau) emit(tau, true, P[tau]);
            keep_branch<0>();
        } else {
#pragma unroll
            for (int tau = 0; tau < 8; ++tau) emit(tau, false, S[tau]);
            keep_branch<1>();
        }
    }
    if constexpr (LVL == 3)   // eighth total (P over the whole eighth), read at levels 4 and 5
        *reinterpret_cast<f32x2 *>(&etot[e8][2 * cp]) = P[7];
}

// MFMA tiles of level LVL: A (kind 0) and M (kind 1); valid pairs scattered to LDS.
template <int LVL, int DK, int DV>
__device__ __forceinline__ void mfma_level(IntraSmem<DK, DV> &sm, int wave, int lane) {
    const int m = lane & 15, kq = lane >> 4;
    int kind, rtok, ridx, ctok, rbase, cbase;
    if constexpr (LVL < 5) {
        if (wave >= 4) return;
        const int th = wave & 1;
        kind = wave >> 1;
        rtok = 32 * th + insert_bit(m, LVL, 1);
        ridx = 16 * th + m;
        ctok = 32 * th + insert_bit(m, LVL, 0);
        rbase = cbase = 32 * th;
    } else {
        const int tile = wave >> 1;
        kind = wave & 1;
        rbase = 32 + 16 * (tile >> 1);
        cbase = 16 * (tile & 1);
        rtok = rbase + m;
        ridx = rtok - 32;
        ctok = cbase + m;
    }
    const _Float16 *arow = kind == 0 ? &sm.u.m.r1.f.Fk[rtok][0] : &sm.u.m.r1.f.Fq[ridx][0];
    f32x4 acc = zero4();
#pragma unroll
    for (int kk = 0; kk < DK / 32; ++kk) {
        const int c8 = kk * 32 + kq * 8;
        acc = mfma_f16(lds8(arow + c8), lds8(&sm.u.m.r1.f.Fk[ctok][c8]), acc);
    }
#pragma unroll
    for (int jj = 0; jj < 4; ++jj) {
        const int orow = 4 * kq + jj;
        int r, i;
        bool valid;
        if constexpr (LVL < 5) {
            r = rbase + insert_bit(orow, LVL, 1);
            i = cbase + insert_bit(m, LVL, 0);
            valid = (orow >> LVL) == (m >> LVL);
        } else {
            r = rbase + orow;
            i = cbase + m;
            valid = true;
        }
        if (valid) {
            if (kind == 0) sm.u.m.r3.A[r][i] = sm.beta[r] * acc[jj];
            else sm.u.m.T[r][i] = acc[jj];
        }
    }
}

// Levels 0..2 pair tokens inside one aligned block of eight, which with
// K = 128 is one wave's (the gate thread of lane cp holds channels 2cp, 2cp+1
// of its eight tokens).  Each wave writes the operand rows of all three
// levels to its own LDS block and forms its pairs with two 16x16 MFMA tiles
// (A: k P rows, M: q P rows, against the k S column rows), row / column
// 4 l + index of the token among the level's four row / column tokens; the
// valid pairs lie in the three 4x4 diagonal blocks.  No workgroup barrier is
// needed until the results are scattered.  Returns the two accumulators.
template <int DK, int DV>
__device__ __forceinline__ void wave_levels_012(f32x2 (&P)[8], f32x2 (&S)[8], const f16x2 (&kr)[8],
                                                const f16x2 (&qr)[8], IntraSmem<DK, DV> &sm, int cp, int wave,
                                                int lane, f32x4 &accA, f32x4 &accM) {
    static_assert(DK == 128, "one eighth per wave");
    _Float16 (*wb)[DK + PADH] = sm.u.wl[wave];
    auto emit = [&](auto lc) {
        constexpr int L = decltype(lc)::value;
#pragma unroll
        for (int tau = 0; tau < 8; ++tau) {
            const int idx = ((tau >> (L + 1)) << L) | (tau & ((1 << L) - 1));
            if ((tau >> L) & 1) {
                const f16x2 fac = {(_Float16)P[tau][0], (_Float16)P[tau][1]};
                *reinterpret_cast<f16x2 *>(&wb[4 * L + idx][2 * cp]) = kr[tau] * fac;
                *reinterpret_cast<f16x2 *>(&wb[12 + 4 * L + idx][2 * cp]) = qr[tau] * fac;
            } else {
                const f16x2 fac = {(_Float16)S[tau][0], (_Float16)S[tau][1]};
                *reinterpret_cast<f16x2 *>(&wb[24 + 4 * L + idx][2 * cp]) = kr[tau] * fac;
            }
        }
    };
    emit(std::integral_constant<int, 0>{});
    chain_in_eighth<1>(P, S);
    emit(std::integral_constant<int, 1>{});
    chain_in_eighth<2>(P, S);
    emit(std::integral_constant<int, 2>{});
    wave_sync();
    const int m = lane & 15, kq = lane >> 4;
    const int rm = m < 12 ? m : 0;   // tile rows / columns 12..15 are unused
    accA = zero4();
    accM = zero4();
#pragma unroll
    for (int kk = 0; kk < DK / 32; ++kk) {
        const int c8 = kk * 32 + kq * 8;
        const f16x8 col = lds8(&wb[24 + rm][c8]);
        accA = mfma_f16(lds8(&wb[rm][c8]), col, accA);
        accM = mfma_f16(lds8(&wb[12 + rm][c8]), col, accM);
    }
}

template <int DK, int DV, typename IO, bool SCALAR, bool RAW>
__global__ __launch_bounds__(NTI, 4) void intra_kernel(PrefillArgs a, Work w) {
    extern __shared__ __align__(16) unsigned char smem_raw[];
    IntraSmem<DK, DV> &sm = *reinterpret_cast<IntraSmem<DK, DV> *>(smem_raw);

    // 1-D grid over (chunk slot, head) items, head fastest, so that resident
    // workgroups read neighbouring tokens of every head (contiguous rows).
    // Block ids go round-robin over the XCDs, so each XCD takes every
    // kXcd-th head of the chunks in flight.
    const int n_items = w.slots * a.hv;
    const int item = (int)blockIdx.x;
    if (item >= n_items) return;
    const int slot = item / a.hv, h = item % a.hv;
    const int2 cm = w.chunk_map[slot];
    if (cm.x < 0) return;
    const int n = cm.x, jc = cm.y;
    const int t0 = a.cu_seqlens[n] + C * jc;
    const int L = min(C, a.cu_seqlens[n + 1] - t0);
    const int hk = h / (a.hv / a.hk);
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // uniform per wave
    const size_t sh = (size_t)slot * a.hv + h;

    const IO *qg = reinterpret_cast<const IO *>(a.q);
    const IO *kg = reinterpret_cast<const IO *>(a.k);

    // ---- phase 0: every input load issued at once ----
    // Gate threads (channel pair cp: channels 2cp, 2cp+1; eighth e8: tokens
    // 8 e8 .. 8 e8 + 7) load their k, q and g values straight into registers:
    // one wave-wide load covers a whole token row.  With K = 128 the eighth is
    // the wave.  (v is read by the state kernel only.)
    // Chunk bases are uniform; per-lane byte offsets stay below 64 rows of one
    // token stride (< 2^32 for any grid the launch accepts).
    const char *kb = reinterpret_cast<const char *>(kg + ((size_t)t0 * a.hk + hk) * DK);
    const char *qb = reinterpret_cast<const char *>(qg + ((size_t)t0 * a.hk + hk) * DK);
    // The gate arrives either as fp32 log-decays g and fp32 beta, or (RAW) as
    // the raw projections x, b in the io dtype, activated here per element.
    using GE = typename std::conditional<RAW, IO, float>::type;   // stored gate / beta element
    const char *gb = reinterpret_cast<const char *>(RAW ? a.gx : static_cast<const void *>(a.g)) +
                     ((size_t)t0 * a.hv + h) * (SCALAR ? 1 : DK) * sizeof(GE);
    const GE *bb = reinterpret_cast<const GE *>(RAW ? a.bx : static_cast<const void *>(a.beta)) +
                   (size_t)t0 * a.hv + h;
    const unsigned kq_row = (unsigned)a.hk * DK * sizeof(IO);
    const unsigned g_row = (unsigned)a.hv * (SCALAR ? 1 : DK) * sizeof(GE);
    const bool fthread = tid < 4 * DK;
    const int cp = tid % (DK / 2), e8 = DK == 128 ? wave : tid / (DK / 2);
    using Pair = typename std::conditional<sizeof(IO) == 2, unsigned, f32x2>::type;   // two io values
    using GPair = typename std::conditional<sizeof(GE) == 2, unsigned, f32x2>::type;  // two gate values
    using GRaw = typename std::conditional<SCALAR, GE, GPair>::type;
    Pair kraw[8], qraw[8];
    GRaw graw[8];
#pragma unroll
    for (int tau = 0; tau < 8; ++tau) {
        const int r = 8 * e8 + tau;
        kraw[tau] = qraw[tau] = Pair{};
        graw[tau] = GRaw{};
        if (fthread && r < L) {
            const unsigned off = (unsigned)r * kq_row + (unsigned)cp * 2 * sizeof(IO);
            kraw[tau] = __builtin_nontemporal_load(reinterpret_cast<const Pair *>(kb + off));
            qraw[tau] = __builtin_nontemporal_load(reinterpret_cast<const Pair *>(qb + off));
            graw[tau] = *reinterpret_cast<const GRaw *>(gb + (unsigned)r * g_row +
                                                        (SCALAR ? 0u : (unsigned)cp * 2 * sizeof(GE)));
        }
    }
    GE braw{};
    if (tid < C && tid < L) braw = bb[(unsigned)tid * a.hv];
    // per-(head, channel) activation parameters: a2 = exp(A_log), dtb = dt_bias log2(e)
    f32x2 a2 = {0.f, 0.f}, dtb = {0.f, 0.f};
    if constexpr (RAW) {
        if (fthread) {
            if constexpr (SCALAR) {
                a2 = f32x2{exp_f(a.A_log[h]), 0.f};
                dtb = f32x2{a.dt_bias[h] * kLog2e, 0.f};
            } else {
                const f32x2 al = *reinterpret_cast<const f32x2 *>(a.A_log + (size_t)h * DK + 2 * cp);
                const f32x2 db = *reinterpret_cast<const f32x2 *>(a.dt_bias + (size_t)h * DK + 2 * cp);
                a2 = f32x2{exp_f(al[0]), exp_f(al[1])};
                dtb = f32x2{db[0] * kLog2e, db[1] * kLog2e};
            }
        }
    }
    // A: the diagonal blocks' diagonal and upper triangle are zero (while the
    // loads are in flight; with K = 128 after the wave-local levels, whose
    // operand blocks overlay A)
    auto zero_a_diag = [&]() {
        for (int e = tid; e < 4 * 256; e += NTI) {
            const int b = e >> 8, rr = (e >> 4) & 15, ii = e & 15;
            if (ii >= rr) sm.u.m.r3.A[16 * b + rr][16 * b + ii] = 0.f;
        }
    };
    if constexpr (DK != 128) zero_a_diag();
    if (tid < C) {
        if constexpr (RAW) sm.beta[tid] = tid < L ? sigmoid_f(io_traits<IO>::load(&braw, 0)) : 0.f;
        else sm.beta[tid] = braw;
    }

    // ---- gate-thread registers and the diagonal of M (q_t . k_t, gate factor 1) ----
    f32x2 P[8], S[8], H0, H1;
    f16x2 kr[8], qr[8];   // k, q of channels (2cp, 2cp+1), rounded to fp16 (exact for bf16 in range)
    if (fthread) {
        float dpart[8];   // this thread's two-channel part of q_t . k_t
#pragma unroll
        for (int tau = 0; tau < 8; ++tau) {
            if constexpr (sizeof(IO) == 2) {
                kr[tau] = f16x2{(_Float16)__uint_as_float(kraw[tau] << 16), (_Float16)__uint_as_float(kraw[tau] & 0xffff0000u)};
                qr[tau] = f16x2{(_Float16)__uint_as_float(qraw[tau] << 16), (_Float16)__uint_as_float(qraw[tau] & 0xffff0000u)};
            } else {
                kr[tau] = f16x2{(_Float16)kraw[tau][0], (_Float16)kraw[tau][1]};
                qr[tau] = f16x2{(_Float16)qraw[tau][0], (_Float16)qraw[tau][1]};
            }
            f32x2 gx;   // the two gate values of this token as fp32
            if constexpr (SCALAR) {
                const float x = io_traits<GE>::load(&graw[tau], 0);
                gx = f32x2{x, x};
            } else if constexpr (sizeof(GE) == 2) {
                gx = f32x2{__uint_as_float(graw[tau] << 16), __uint_as_float(graw[tau] & 0xffff0000u)};
            } else {
                gx = graw[tau];
            }
            // (RAW: tokens past the chunk's end must keep factor 1, as a zero g does)
            if constexpr (RAW && SCALAR) {
                const float d = 8 * e8 + tau < L ? gate_decay(__builtin_fmaf(gx[0], kLog2e, dtb[0]), a2[0]) : 1.f;
                P[tau] = f32x2{d, d};
            } else if constexpr (RAW) {
                P[tau] = 8 * e8 + tau < L ? f32x2{gate_decay(__builtin_fmaf(gx[0], kLog2e, dtb[0]), a2[0]),
                                                  gate_decay(__builtin_fmaf(gx[1], kLog2e, dtb[1]), a2[1])}
                                          : f32x2{1.f, 1.f};
            } else if constexpr (SCALAR) {
                const float d = exp_f(gx[0]);
                P[tau] = f32x2{d, d};
            } else {
                P[tau] = f32x2{exp_f(gx[0]), exp_f(gx[1])};
            }
            S[tau] = f32x2{1.f, 1.f};
            dpart[tau] = (float)qr[tau][0] * (float)kr[tau][0] + (float)qr[tau][1] * (float)kr[tau][1];
        }
        // Sum over the DK / 2 lanes of this eighth by recursive halving: the
        // first three exchange steps halve the eight partial sums, the rest
        // are plain butterflies.  Afterwards the lane holds the total of token
        // index 4 [bit G/2] + 2 [bit G/4] + [bit G/8] of its lane id.
        constexpr int G = DK / 2;
        auto halve = [&](int o, auto half) {   // keep one half of the values, add the partner's copy
            constexpr int H = decltype(half)::value;
            const bool up = (lane & o) != 0;
#pragma unroll
            for (int i = 0; i < H; ++i) {
                const float send = up ? dpart[i] : dpart[i + H];
                const float keep = up ? dpart[i + H] : dpart[i];
                dpart[i] = keep + __shfl_xor(send, o, 64);
            }
        };
        halve(G / 2, std::integral_constant<int, 4>{});
        halve(G / 4, std::integral_constant<int, 2>{});
        halve(G / 8, std::integral_constant<int, 1>{});
#pragma unroll
        for (int o = G / 16; o >= 1; o >>= 1) dpart[0] += __shfl_xor(dpart[0], o, 64);
        const int idx = 4 * ((lane & (G / 2)) != 0) + 2 * ((lane & (G / 4)) != 0) + ((lane & (G / 8)) != 0);
        if ((lane & (G / 8 - 1)) == 0) sm.mdiag[8 * e8 + idx] = dpart[0];
    }
    __syncthreads();

    // ---- levels 0..5: gate factors, then A and M tiles ----
    // (K = 128: levels 0..2 wave-local, then their pairs scattered into A and M)
    constexpr int LVL0 = DK == 128 ? 3 : 0;
    if constexpr (DK == 128) {
        f32x4 accA, accM;
        wave_levels_012(P, S, kr, qr, sm, cp, wave, lane, accA, accM);
        __syncthreads();   // every wave is done with its operand block
        zero_a_diag();
        const int m = lane & 15, kq = lane >> 4;
        // accumulator element jj: tile row 4 kq + jj (level kq, row token index jj),
        // column m (level m / 4, column token index m % 4)
        if (kq < 3 && (m >> 2) == kq) {
#pragma unroll
            for (int jj = 0; jj < 4; ++jj) {
                const int tr = insert_bit(jj, kq, 1), tc = insert_bit(m & 3, kq, 0);
                if ((tr >> (kq + 1)) == (tc >> (kq + 1))) {
                    const int r = 8 * wave + tr, i = 8 * wave + tc;
                    sm.u.m.r3.A[r][i] = sm.beta[r] * accA[jj];
                    sm.u.m.T[r][i] = accM[jj];
                }
            }
        }
    }
#pragma unroll
    for (int lvl = LVL0; lvl < 6; ++lvl) {
        if (fthread) {
            switch (lvl) {
            case 0: factor_level<0>(P, S, kr, qr, sm, cp, e8, H0, H1); break;
            case 1: factor_level<1>(P, S, kr, qr, sm, cp, e8, H0, H1); break;
            case 2: factor_level<2>(P, S, kr, qr, sm, cp, e8, H0, H1); break;
            case 3: factor_level<3>(P, S, kr, qr, sm, cp, e8, H0, H1); break;
            case 4: factor_level<4>(P, S, kr, qr, sm, cp, e8, H0, H1); break;
            default: factor_level<5>(P, S, kr, qr, sm, cp, e8, H0, H1); break;
            }
        }
        __syncthreads();
        switch (lvl) {
        case 0: mfma_level<0>(sm, wave, lane); break;
        case 1: mfma_level<1>(sm, wave, lane); break;
        case 2: mfma_level<2>(sm, wave, lane); break;
        case 3: mfma_level<3>(sm, wave, lane); break;
        case 4: mfma_level<4>(sm, wave, lane); break;
        default: mfma_level<5>(sm, wave, lane); break;
        }
        __syncthreads();
    }

    // ---- chunk-level factors: exp(G_t), exp(G_last - G_t) ----
    const size_t qg_off = sh * C * DK, kl_off = sh * DK * C;
    if (fthread) {
        if (e8 == 0) {
            const f32x2 gl = H0 * H1;
            w.GL[sh * DK + 2 * cp] = gl[0];
            w.GL[sh * DK + 2 * cp + 1] = gl[1];
        }
        f16x8 kg0, kg1, kl0, kl1;   // channels 2cp and 2cp+1, tokens 8 e8 .. 8 e8 + 7
        const f32x2 one = {1.f, 1.f};
        const f32x2 hp = e8 >= 4 ? H0 : one, hs = e8 < 4 ? H1 : one;
#pragma unroll
        for (int tau = 0; tau < 8; ++tau) {
            const int t = 8 * e8 + tau;
            const f32x2 gam = P[tau] * hp;     // exp(G_t)
            const f32x2 rest = S[tau] * hs;    // exp(G_last - G_t)
            const f32x2 bg = gam * sm.beta[t];
            // fp16 x fp32 products rounded once to fp16 (mixed-precision FMA)
            const float k0 = (float)kr[tau][0], k1 = (float)kr[tau][1];
            kg0[tau] = (_Float16)__builtin_fmaf(k0, bg[0], 0.f);
            kg1[tau] = (_Float16)__builtin_fmaf(k1, bg[1], 0.f);
            kl0[tau] = (_Float16)__builtin_fmaf(k0, rest[0], 0.f);
            kl1[tau] = (_Float16)__builtin_fmaf(k1, rest[1], 0.f);
            const f16x2 qgam = {(_Float16)__builtin_fmaf((float)qr[tau][0], gam[0], 0.f),
                                (_Float16)__builtin_fmaf((float)qr[tau][1], gam[1], 0.f)};
            *reinterpret_cast<f16x2 *>(&sm.u.m.r1.stage[t][2 * cp]) = qgam;
        }
        // (the eighth totals held in the KGt space were last read at level 5)
        *reinterpret_cast<f16x8 *>(&sm.u.m.KGt[2 * cp][8 * e8]) = kg0;
        *reinterpret_cast<f16x8 *>(&sm.u.m.KGt[2 * cp + 1][8 * e8]) = kg1;
        // (K exp(G_last - G))^T in A-operand tile layout: rows c, k index t
#pragma unroll
        for (int u = 0; u < 2; ++u) {
            const int c = 2 * cp + u;
            const int ln = (c & 15) + 16 * (e8 & 3);
            __builtin_nontemporal_store(u ? kl1 : kl0,
                reinterpret_cast<f16x8 *>(w.KLt + kl_off + ((size_t)((c >> 4) * 2 + (e8 >> 2)) * 64 + ln) * 8));
        }
    }
    __syncthreads();

    // ---- wave 0: diagonal blocks of T = (I + A)^-1 by forward substitution,
    //      into registers; waves 1..7 meanwhile store the Q exp(G) and M tiles ----
    // Each lane of wave 0 owns one column c of one 16x16 diagonal block b and
    // runs the unit lower triangular forward substitution in fp32:
    //   T_bb[r][c] = [r == c] - sum_{j < r} A_bb[r][j] T_bb[j][c]
    // (rows above c come out exactly 0).  It reads only A; the stores read the
    // Q exp(G) staging rows and M (held in the T region), so the two overlap.
    // (Every workspace operand is written nontemporally: it is read back only
    // by the state kernel, after this kernel, so it need not stay in the caches.)
    constexpr int LD = C + 1;
    float tdiag[16];
    if (wave == 0) {
        const int b = lane >> 4, c = lane & 15;
        const float *Ab = &sm.u.m.r3.A[16 * b][16 * b];
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            float acc = r == c ? 1.f : 0.f;
#pragma unroll
            for (int j = 0; j < r; ++j) acc = __builtin_fmaf(-Ab[r * LD + j], tdiag[j], acc);
            tdiag[r] = acc;
        }
    } else {
        constexpr int NS = NTI - 64;   // storing threads
        const int ts = tid - 64;
        for (int e = ts; e < (C / 16) * (DK / 32) * 64; e += NS) {
            const int tile = e >> 6, l = e & 63;
            const int rt = tile / (DK / 32), kk = tile % (DK / 32);
            __builtin_nontemporal_store(lds8(&sm.u.m.r1.stage[16 * rt + (l & 15)][32 * kk + 8 * (l >> 4)]),
                reinterpret_cast<f16x8 *>(w.QG + qg_off + (size_t)e * 8));
        }
        for (int e = ts; e < (C / 16) * (C / 32) * 64; e += NS) {   // M: lower triangle incl. diagonal
            const int tile = e >> 6, l = e & 63;
            if ((tile & 1) && (tile >> 1) < 2) continue;   // rows < 32, columns >= 32: zero, never read
            const int r = 16 * (tile >> 1) + (l & 15), i0 = 32 * (tile & 1) + 8 * (l >> 4);
            f16x8 v;
#pragma unroll
            for (int u = 0; u < 8; ++u)
                v[u] = (_Float16)(i0 + u < r ? sm.u.m.T[r][i0 + u] : i0 + u == r ? sm.mdiag[r] : 0.f);
            __builtin_nontemporal_store(v, reinterpret_cast<f16x8 *>(w.M + sh * C * C + (size_t)e * 8));
        }
    }
    __syncthreads();
    // T: the blocks above the block diagonal are zero; wave 0 writes the diagonal blocks
    for (int e = tid; e < C * C; e += NTI) {
        const int r = e / C, i = e % C;
        if ((i >> 4) > (r >> 4)) sm.u.m.T[r][i] = 0.f;
    }
    if (wave == 0) {
        const int b = lane >> 4, c = lane & 15;
#pragma unroll
        for (int r = 0; r < 16; ++r) sm.u.m.T[16 * b + r][16 * b + c] = tdiag[r];
    }
    __syncthreads();
    // Off-diagonal blocks.  With D = I + (diagonal blocks of A), N = D^-1 A_off
    // (N_ab = T_aa A_ab for a > b) is block strictly lower, so
    // T = (I + N)^-1 D^-1 = (I - N + N^2 - N^3) D^-1, i.e. T_ab = Y_ab T_bb with
    //   Y_10 = -N_10, Y_20 = -N_20 + N_21 N_10, Y_31 = -N_31 + N_32 N_21,
    //   Y_30 = -N_30 + N_31 N_10 - N_32 Y_20,
    // in three steps of independent 16x16 products (six, five, three waves).
    {
        constexpr int LS = 20;   // scratch leading dimension (bank spread of the fragment reads)
        float(*scr)[16][LS] = sm.u.m.r1.scr;
        float *Tm = &sm.u.m.T[0][0];
        auto Tb = [&](int r, int c) { return Tm + (16 * r) * LD + 16 * c; };
        auto Ab = [&](int r, int c) { return &sm.u.m.r3.A[16 * r][16 * c]; };
        const int m = lane & 15, kq = lane >> 4;
        // scratch blocks: 0..5 = N_10, N_21, N_32, N_20, N_31, N_30; 6 = Y_20, 7 = Y_31, 8 = Y_30
        if (wave < 6) {
            constexpr int pa[6] = {1, 2, 3, 2, 3, 3}, pb[6] = {0, 1, 2, 0, 1, 0};
            const int ia = pa[wave], ib = pb[wave];
            st16(&scr[wave][0][0], LS, mm16(Tb(ia, ia), LD, Ab(ia, ib), LD, lane), lane);
        }
        __syncthreads();
        if (wave < 3) {   // T_{b+1,b} = -N_{b+1,b} T_bb
            f32x4 t = mm16(&scr[wave][0][0], LS, Tb(wave, wave), LD, lane);
#pragma unroll
            for (int jj = 0; jj < 4; ++jj) t[jj] = -t[jj];
            st16(Tb(wave + 1, wave), LD, t, lane);
        } else if (wave < 5) {   // Y_20 (wave 3), Y_31 (wave 4)
            const int i2 = wave == 3 ? 1 : 2, i1 = wave == 3 ? 0 : 1, in = wave == 3 ? 3 : 4;
            f32x4 y = mm16(&scr[i2][0][0], LS, &scr[i1][0][0], LS, lane);
#pragma unroll
            for (int jj = 0; jj < 4; ++jj) y[jj] -= scr[in][4 * kq + jj][m];
            st16(&scr[wave + 3][0][0], LS, y, lane);
        }
        __syncthreads();
        if (wave < 2) {   // T_20 = Y_20 T_00, T_31 = Y_31 T_11
            st16(Tb(wave + 2, wave), LD, mm16(&scr[6 + wave][0][0], LS, Tb(wave, wave), LD, lane), lane);
        } else if (wave == 2) {   // Y_30, then T_30 = Y_30 T_00
            const f32x4 t1 = mm16(&scr[4][0][0], LS, &scr[0][0][0], LS, lane);
            const f32x4 t2 = mm16(&scr[2][0][0], LS, &scr[6][0][0], LS, lane);
            f32x4 y;
#pragma unroll
            for (int jj = 0; jj < 4; ++jj) y[jj] = t1[jj] - t2[jj] - scr[5][4 * kq + jj][m];
            st16(&scr[8][0][0], LS, y, lane);
            wave_sync();
            st16(Tb(3, 0), LD, mm16(&scr[8][0][0], LS, Tb(0, 0), LD, lane), lane);
        }
        __syncthreads();
    }

    // ---- W = T (beta K exp(G)) -> LDS stage -> global A-operand tiles: waves
    //      w and w + 4 share token row tile w and split W's 32-column tiles
    //      (all of them on waves 0..3 when K = 32); waves 4..7 also store
    //      T diag(beta) as A-operand tiles ----
    {
        const int m = lane & 15, kq = lane >> 4;
        const int rt = wave & 3, which = wave >> 2;
        const bool k1 = rt >= 2;   // T rows < 32 vanish for columns >= 32
        constexpr int KT = DK / 32;                 // 32-column tiles of W
        constexpr int SPLIT = KT >= 2 ? 2 : 1;      // wave groups sharing them
        if (SPLIT == 2 || which == 0) {
            const int kt0 = SPLIT == 2 ? which * (KT / 2) : 0;
            f16x8 ta[2];
#pragma unroll
            for (int kk = 0; kk < 2; ++kk) {
                const float *tp = &sm.u.m.T[16 * rt + m][kk * 32 + kq * 8];
#pragma unroll
                for (int e = 0; e < 8; ++e) ta[kk][e] = (_Float16)tp[e];
            }
#pragma unroll
            for (int c2 = 0; c2 < 2 * KT / SPLIT; ++c2) {
                const int ct = 2 * kt0 + c2;   // 16-column tile
                f32x4 acc = mfma_f16(ta[0], lds8(&sm.u.m.KGt[16 * ct + m][kq * 8]), zero4());
                if (k1) acc = mfma_f16(ta[1], lds8(&sm.u.m.KGt[16 * ct + m][32 + kq * 8]), acc);
#pragma unroll
                for (int jj = 0; jj < 4; ++jj) sm.u.m.r1.stage[16 * rt + 4 * kq + jj][16 * ct + m] = (_Float16)acc[jj];
            }
            // this wave's staged block (16 rows, its columns) -> its A-operand
            // tiles (rt, kk) of W, with no workgroup barrier (the block is its own)
            wave_sync();
            _Float16 *Wg = w.W + sh * C * DK + (size_t)rt * KT * 512;
#pragma unroll
            for (int k2 = 0; k2 < KT / SPLIT; ++k2) {
                const int kk = kt0 + k2;
                __builtin_nontemporal_store(lds8(&sm.u.m.r1.stage[16 * rt + m][32 * kk + 8 * kq]),
                    reinterpret_cast<f16x8 *>(Wg + ((size_t)kk * 64 + lane) * 8));
            }
        }
        if (which == 1) {
            // Ut = T diag(beta) V is formed by the state kernel from the v rows
            // it streams; T diag(beta) goes out as A-operand tiles (rt, kk),
            // the zero tile (rt < 2, kk = 1) not stored.
            _Float16 *Tg = w.Tb + sh * C * C + (size_t)rt * 2 * 512;
#pragma unroll
            for (int kk = 0; kk < 2; ++kk) {
                if (kk == 0 || k1) {
                    const float *tp = &sm.u.m.T[16 * rt + m][kk * 32 + kq * 8];
                    const float *bp = &sm.beta[kk * 32 + kq * 8];
                    f16x8 tb;
#pragma unroll
                    for (int e = 0; e < 8; ++e) tb[e] = (_Float16)(tp[e] * bp[e]);
                    __builtin_nontemporal_store(tb, reinterpret_cast<f16x8 *>(Tg + ((size_t)kk * 64 + lane) * 8));
                }
            }
        }
    }
}

// ---------------------------------------------------------------------------
// state: per (sequence, value head), sequential over chunks
//
// Operand layouts written by the intra kernel (fp16):
//   A-operand tiles: tile (rt, kk) of an R x K matrix X holds, for lane l,
//     X[16 rt + l % 16][32 kk + 8 (l / 16) + e], e = 0..7   (16 B per lane)
//   accumulator tiles: tile (rt, ct) holds, for lane l,
//     X[16 rt + 4 (l / 16) + jj][16 ct + l % 16], jj = 0..3  (8 B per lane)
// so every operand load is one contiguous 16 B (or 8 B) access per lane.
//
// Eight waves own one column part (all of V <= 64, or 64 of 128 value
// columns) of one (sequence, head) chain and that part of the K x V state;
// a chain's parts share one workgroup.  Per chunk:
//   (a) every wave writes its state tiles to LDS as fp16 (S^T, B operand);
//   (b) waves 0..3 (token row tile rt = wave): U = Ut - W S -> LDS (U^T),
//       where Ut = (T diag(beta)) V was formed at the end of the previous
//       step from V^T staged in LDS (v is streamed once, by this kernel only);
//       waves 4..7 (rt = wave - 4): the inter-chunk output part Q exp(G) S;
//   (c) waves 4..7: O = scale (Q exp(G) S + M U), staged, stored as rows;
//   (d) every wave: its state tiles S <- exp(G_last) S + (K exp(G_last - G))^T U;
//       waves 0..3 then form the next chunk's Ut (off the chain's critical path).
// Each operand register is reloaded with the next chunk's tile right after
// its last use, so its load has a whole chunk step to arrive with a single
// register copy; the register budget (<= 128 VGPRs) then admits sixteen
// waves per CU: one chain of 128 value columns, or two of at most 64.  With
// at most 64 chains a chain's 128 columns are split into four parts of 32.
// ---------------------------------------------------------------------------
constexpr int NTS = 512;   // threads of the state kernel per column part
constexpr long kFewChains = 256;   // at most this many chains: one workgroup per column part
constexpr long kVeryFewChains = 64;   // at most this many: four parts of 32 value columns

template <int DK, int DV, typename IO> struct StateSmem {
    _Float16 Sh[DV][DK + PADH];   // S^T as fp16 (B operand of W S and Q exp(G) S)
    _Float16 Vn[DV][C + PADH];    // U^T as fp16 (B operand of M U and KLt U)
    _Float16 Vs[2][DV][C + PADH]; // V^T of a chunk as fp16 (B operand of (T diag(beta)) V), two buffers
    IO Ost[4][16][DV + 16 / sizeof(IO)];   // output rows of waves 4..7, for 16-byte stores
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


// Keeps the loads issued before it from being sunk past it by the compiler
// (a prefetch sunk to its use would expose the full memory latency).
__device__ __forceinline__ void pin_loads() { asm volatile("" ::: "memory"); }

// A wave-uniform element offset made opaque (both halves through
// readfirstlane).  Added to a kernel-argument pointer it keeps the global
// address space, and the compiler cannot fold per-lane offsets into a
// loop-invariant 64-bit per-lane pointer per operand stream.
__device__ __forceinline__ size_t uniform_off(size_t x) {
    const unsigned lo = __builtin_amdgcn_readfirstlane((unsigned)x);
    const unsigned hi = __builtin_amdgcn_readfirstlane((unsigned)(x >> 32));
    return ((size_t)hi << 32) | lo;
}

// Per-wave part of one (sequence, head) chain; UW selects the role (U wave or
// output wave).  Both roles pass the same barriers in the same order.
template <bool UW, int DK, int DV, int DVW, typename IO, typename ST>
__device__ __forceinline__ void state_chain(const PrefillArgs &a, const Work &w, StateSmem<DK, DVW, IO> &sm,
                                            int n, int h, int j0, int wave, int lane) {
    // This workgroup owns value columns j0 .. j0 + DVW - 1 of the chain (the
    // columns of S, U and O never mix, so a chain may be split over several
    // workgroups by columns); memory strides use the full width DV.
    constexpr int KK = DK / 32;               // k-steps over key channels
    constexpr int CT = DVW / 16;              // value column tiles of this workgroup
    constexpr int R = DK / 16;                // key row tiles of the state
    constexpr int NST = R * CT;               // state tiles
    constexpr int NTW = NST >= 8 ? NST / 8 : 1;   // state tiles per wave (one key row tile)
    static_assert(NTW <= CT, "a wave's state tiles share one key row tile");
    const int m = lane & 15, kq = lane >> 4;
    const int rt = wave & 3;                  // token row tile of (b) and (c)
    const bool swave = NST >= 8 || wave * NTW < NST;   // holds state tiles
    const int kr = (wave * NTW) / CT;         // its key row tile
    const int ct0 = (wave * NTW) % CT;        // its first value column tile
    const int tbeg = a.cu_seqlens[n], tend = a.cu_seqlens[n + 1];
    const int nchunks = (tend - tbeg + C - 1) / C;
    const int s0 = w.chunk_off[n];

    long row_in = -1, row_out = -1;
    if (a.indices) {
        int s = a.indices[n];
        if (s < 0) s = a.num_slots - 1;
        row_in = row_out = s;
    } else {
        if (a.state_in) row_in = n;
        if (a.state_out) row_out = n;
    }
    // S[c] holds state rows (key) 16 kr + 4 kq + jj, columns (value) 16 (ct0 + c) + m
    f32x4 S[NTW];
    {
        const ST *sin = row_in >= 0 ? reinterpret_cast<const ST *>(a.state_in) + ((size_t)row_in * a.hv + h) * DV * DK
                                    : nullptr;
#pragma unroll
        for (int c = 0; c < NTW; ++c)
            S[c] = (sin && swave) ? load_state4<ST>(sin + (size_t)(j0 + 16 * (ct0 + c) + m) * DK + 16 * kr + 4 * kq)
                                  : zero4();
    }

    // Operand registers of the current chunk (single copies, reloaded with
    // the next chunk's tiles right after their last use).  Chunk bases are
    // wave-uniform (see uniform_off); each lane adds a 32-bit byte offset.
    f16x8 Xa[KK];                   // W (U waves) or Q exp(G) (output waves), row tile rt
    f16x8 Ta[UW ? 2 : 1];           // T diag(beta) of row tile rt (U waves)
    f16x8 Ma[UW ? 1 : 2];           // M of row tile rt (output waves)
    f16x8 Ka[2];                    // (K exp(G_last - G))^T, key row tile kr
    f32x4 gl;                       // exp(G_last) of key rows 16 kr + 4 kq + jj
    auto chunk_base = [&](int ch) { return (size_t)(s0 + ch) * a.hv + h; };
    const bool t_hi = rt >= 2;      // token row tile rt reaches columns 32..63 of T and M
    const unsigned lane16 = (unsigned)lane * 16u;
    // The lane offset is re-derived behind an empty asm at every use, so the
    // compiler cannot pre-add it to loop-invariant 64-bit per-lane pointers.
    auto lane_off = [&](unsigned scale16) {
        unsigned o = scale16 == 16u ? lane16 : lane16 >> 1;
        asm volatile("" : "+v"(o));
        return o;
    };
    auto ld8 = [](const _Float16 *base, unsigned off) {
        return *reinterpret_cast<const f16x8 *>(reinterpret_cast<const char *>(base) + off);
    };
    auto load_x = [&](int ch) {
        const size_t sh = chunk_base(ch);
        const _Float16 *Xg = (UW ? w.W : w.QG) + uniform_off(sh * C * DK + (size_t)rt * KK * 512);
        const unsigned lo16 = lane_off(16u);
#pragma unroll
        for (int kk = 0; kk < KK; ++kk) Xa[kk] = ld8(Xg, lo16 + kk * 1024u);
    };
    // T diag(beta) of row tile rt (U waves): its tile of columns 32..63 is zero for rt < 2
    [[maybe_unused]] auto load_t = [&](int ch) {
        if constexpr (UW) {
            const _Float16 *Tg = w.Tb + uniform_off(chunk_base(ch) * C * C + (size_t)rt * 2 * 512);
            const unsigned lo16 = lane_off(16u);
            Ta[0] = ld8(Tg, lo16);
            Ta[1] = ld8(Tg, lo16 + 1024u);   // unused (and not stored) for rt < 2
        }
    };
    // M is lower triangular: the tile of token rows 16 rt.. and columns 32..63
    // is zero (and not stored) for rt < 2.
    const bool m_hi = t_hi;
    auto load_m = [&](int ch) {
        if constexpr (!UW) {
            const _Float16 *Mg = w.M + uniform_off(chunk_base(ch) * C * C + (size_t)rt * 2 * 512);
            const unsigned lo16 = lane_off(16u);
            Ma[0] = ld8(Mg, lo16);
            Ma[1] = ld8(Mg, lo16 + 1024u);   // unused (and not stored) for rt < 2
        }
    };
    auto load_k = [&](int ch) {
        const size_t sh = chunk_base(ch);
        const _Float16 *Kg = w.KLt + uniform_off(sh * DK * C + (size_t)kr * 2 * 512);
        const unsigned lo16 = lane_off(16u);
        Ka[0] = ld8(Kg, lo16);
        Ka[1] = ld8(Kg, lo16 + 1024u);
        const float *Gg = w.GL + uniform_off(sh * DK + 16 * kr);
        unsigned go = (unsigned)kq * 16u;
        asm volatile("" : "+v"(go));
        gl = *reinterpret_cast<const f32x4 *>(reinterpret_cast<const char *>(Gg) + go);
    };
    // V staging (U waves): unit u = (token pair p, column group g), with g
    // fastest, moves 16 bytes (VPT columns) of token rows 2p and 2p + 1 of
    // this part's columns, so a wave's loads cover whole row segments.  The
    // loads go through a buffer whose range is the chunk's valid rows (rows
    // past the sequence end read as zero) and are nontemporal: v is read once.
    constexpr int VPT = 16 / (int)sizeof(IO);   // io columns per 16-byte load
    constexpr int NVU = 32 * (DVW / VPT);       // units
    constexpr int NVI = (NVU + 255) / 256;      // units per U-wave thread
    static_assert(NVU % 64 == 0, "V staging units cover whole waves");
    [[maybe_unused]] u32x4 Vr[UW ? NVI : 1][2];
    const int vrow = a.hv * DV * (int)sizeof(IO);   // token stride of v, bytes
    [[maybe_unused]] auto load_v = [&](int ch) {
        if constexpr (UW) {
            const int t0c = tbeg + ch * C, Lc = min(C, tend - t0c);
            char *vb = reinterpret_cast<char *>(const_cast<void *>(a.v)) +
                       uniform_off((((size_t)t0c * a.hv + h) * DV + j0) * sizeof(IO));
            const int nrec = __builtin_amdgcn_readfirstlane(Lc > 0 ? (Lc - 1) * vrow + DVW * (int)sizeof(IO) : 0);
            const __amdgpu_buffer_rsrc_t vr = __builtin_amdgcn_make_buffer_rsrc(vb, 0, nrec, kBufferWord3);
#pragma unroll
            for (int it = 0; it < NVI; ++it) {
                const int u = wave * 64 + lane + 256 * it;
                if (NVU % 256 == 0 || u < NVU) {   // wave-uniform
                    const int off = 2 * (u / (NVU / 32)) * vrow + (u % (NVU / 32)) * 16;
                    Vr[it][0] = __builtin_amdgcn_raw_buffer_load_b128(vr, off, 0, 2);
                    Vr[it][1] = __builtin_amdgcn_raw_buffer_load_b128(vr, off + vrow, 0, 2);
                }
            }
        }
    };
    [[maybe_unused]] auto write_vs = [&](int buf) {
        if constexpr (UW) {
#pragma unroll
            for (int it = 0; it < NVI; ++it) {
                const int u = wave * 64 + lane + 256 * it;
                if (NVU % 256 == 0 || u < NVU) {
                    const int p = u / (NVU / 32), g = u % (NVU / 32);
#pragma unroll
                    for (int e = 0; e < VPT; ++e) {
                        float x0, x1;
                        if constexpr (VPT == 8) {
                            x0 = __uint_as_float(e & 1 ? (Vr[it][0][e >> 1] & 0xffff0000u) : (Vr[it][0][e >> 1] << 16));
                            x1 = __uint_as_float(e & 1 ? (Vr[it][1][e >> 1] & 0xffff0000u) : (Vr[it][1][e >> 1] << 16));
                        } else {
                            x0 = __uint_as_float(Vr[it][0][e]);
                            x1 = __uint_as_float(Vr[it][1][e]);
                        }
                        *reinterpret_cast<f16x2 *>(&sm.Vs[buf][g * VPT + e][2 * p]) = f16x2{(_Float16)x0, (_Float16)x1};
                    }
                }
            }
        }
    };

    // Ut = (T diag(beta)) V of row tile rt for the chunk whose V^T is in buffer buf (U waves)
    [[maybe_unused]] f32x4 Ut[UW ? CT : 1];
    [[maybe_unused]] auto form_ut = [&](int buf) {
        if constexpr (UW) {
#pragma unroll
            for (int ct = 0; ct < CT; ++ct) {
                Ut[ct] = mfma_f16(Ta[0], lds8(&sm.Vs[buf][16 * ct + m][kq * 8]), zero4());
                if (t_hi) Ut[ct] = mfma_f16(Ta[1], lds8(&sm.Vs[buf][16 * ct + m][32 + kq * 8]), Ut[ct]);
            }
        }
    };

    // The prologue ends with the loads the loop issues between a chunk's V
    // loads and the next loop head (x, k, t for U waves; x, m, k for output
    // waves), in the same order and number, so the compiler's vector-memory
    // waits at the loop head are exact on both incoming paths and the loads
    // of the next chunk stay in flight.
    if (nchunks > 0) {
        load_t(0);
        load_v(0);
        write_vs(0);                        // V^T of chunk 0
        __syncthreads();
        form_ut(0);
        load_v(min(1, nchunks - 1));
        load_x(0);
        load_m(0);
        if (swave) load_k(0);
        load_t(min(1, nchunks - 1));
    }

    IO *og = reinterpret_cast<IO *>(a.o);
    for (int ch = 0; ch < nchunks; ++ch) {
        const int t0 = tbeg + ch * C;
        const int L = min(C, tend - t0);
        // Operand reloads are unconditional (the last chunk reloads itself), so
        // the number of memory operations between a load and its use is the
        // same on every path and the waits stay exact.
        const int nxt = min(ch + 1, nchunks - 1);

        // V^T of the next chunk into the other buffer (its previous chunk was
        // read before this step's first barrier), the chunk after it into registers
        if constexpr (UW) {
            write_vs((ch + 1) & 1);
            load_v(min(ch + 2, nchunks - 1));
            pin_loads();
        }

        // (a) S^T -> fp16 LDS
        if (swave) {
#pragma unroll
            for (int c = 0; c < NTW; ++c) {
                f16x4 hv4;
#pragma unroll
                for (int jj = 0; jj < 4; ++jj) hv4[jj] = (_Float16)S[c][jj];
                *reinterpret_cast<f16x4 *>(&sm.Sh[16 * (ct0 + c) + m][16 * kr + 4 * kq]) = hv4;
            }
        }
        __syncthreads();

        // (b) U = (T diag(beta)) V - W S (U waves) | Q exp(G) S (output waves), row tile rt
        [[maybe_unused]] f32x4 Oacc[UW ? 1 : CT];
#pragma unroll
        for (int ct = 0; ct < CT; ++ct) {
            f32x4 acc = zero4();
#pragma unroll
            for (int kk = 0; kk < KK; ++kk)
                acc = mfma_f16(Xa[kk], lds8(&sm.Sh[16 * ct + m][kk * 32 + kq * 8]), acc);
            if constexpr (UW) {
                f16x4 uv;
#pragma unroll
                for (int jj = 0; jj < 4; ++jj) uv[jj] = (_Float16)(Ut[ct][jj] - acc[jj]);
                *reinterpret_cast<f16x4 *>(&sm.Vn[16 * ct + m][16 * rt + 4 * kq]) = uv;
            } else {
                Oacc[ct] = acc;
            }
        }
        load_x(nxt);
        pin_loads();
        __syncthreads();

        // (c) O = scale (Q exp(G) S + M U), output waves; valid rows stored
        if constexpr (!UW) {
            const int ow = wave - 4;
#pragma unroll
            for (int ct = 0; ct < CT; ++ct) {
                Oacc[ct] = mfma_f16(Ma[0], lds8(&sm.Vn[16 * ct + m][kq * 8]), Oacc[ct]);
                if (m_hi) Oacc[ct] = mfma_f16(Ma[1], lds8(&sm.Vn[16 * ct + m][32 + kq * 8]), Oacc[ct]);
#pragma unroll
                for (int jj = 0; jj < 4; ++jj)
                    io_traits<IO>::store(&sm.Ost[ow][4 * kq + jj][0], 16 * ct + m, a.scale * Oacc[ct][jj]);
            }
            load_m(nxt);
            pin_loads();
            wave_sync();
            // 16 rows x DV values of this wave -> 16-byte buffer stores.  The
            // buffer's range is the valid rows of this tile, so the stores of
            // rows past the sequence end are dropped by the hardware range
            // check and no store is under a branch.
            constexpr int EPV = 16 / sizeof(IO), VPR = DVW / EPV;  // elements per vector, vectors per row
            char *ob = reinterpret_cast<char *>(og + uniform_off(((size_t)(t0 + 16 * rt) * a.hv + h) * DV + j0));
            const int orow = a.hv * DV * (int)sizeof(IO);
            const int nrec = __builtin_amdgcn_readfirstlane(max(0, min(16, L - 16 * rt)) * orow);   // bytes
            const __amdgpu_buffer_rsrc_t orsrc = __builtin_amdgcn_make_buffer_rsrc(ob, 0, nrec, kBufferWord3);
#pragma unroll
            for (int e = lane; e < 16 * VPR; e += 64) {
                const int rr = e / VPR, c0 = (e % VPR) * EPV;
                __builtin_amdgcn_raw_buffer_store_b128(*reinterpret_cast<const u32x4 *>(&sm.Ost[ow][rr][c0]), orsrc,
                                                       rr * orow + c0 * (int)sizeof(IO), 0, 2);
            }
        }

        // (d) S = diag(exp G_last) S + KLt U, this wave's state tiles
        if (swave) {
#pragma unroll
            for (int c = 0; c < NTW; ++c) {
#pragma unroll
                for (int jj = 0; jj < 4; ++jj) S[c][jj] *= gl[jj];
#pragma unroll
                for (int kk = 0; kk < 2; ++kk)
                    S[c] = mfma_f16(Ka[kk], lds8(&sm.Vn[16 * (ct0 + c) + m][kk * 32 + kq * 8]), S[c]);
            }
            load_k(nxt);
            pin_loads();
        }
        // the next chunk's Ut (its V^T was written before this step's first
        // barrier, its T diag(beta) tiles loaded a step ago), then the tiles
        // of the chunk after it
        if constexpr (UW) {
            form_ut((ch + 1) & 1);
            load_t(min(ch + 2, nchunks - 1));
            pin_loads();
        }
    }

    if (row_out >= 0 && swave) {
        ST *sout = reinterpret_cast<ST *>(a.state_out) + ((size_t)row_out * a.hv + h) * DV * DK;
#pragma unroll
        for (int c = 0; c < NTW; ++c)
            store_state4(sout + (size_t)(j0 + 16 * (ct0 + c) + m) * DK + 16 * kr + 4 * kq, S[c]);
    }
}

// One workgroup per (sequence, head) chain.  With DV / DVW column parts it
// has eight waves per part; the parts keep their own LDS blocks and share
// only the barriers, so they step through the chunks in lockstep and the
// operand tiles both parts load (W, Q exp(G), M, the key factors, T diag(beta))
// are fetched from HBM once and served to the second part by the caches.
//
// With PPW = 1 and two column parts, each part is a workgroup of its own
// instead (used for few chains, where the parts' operand re-reads cost little
// and an eight-wave barrier is cheaper than a sixteen-wave one); the two
// parts of a chain get block ids kXcd apart inside one group of kXcd chains,
// so they run on one XCD and share its L2.
template <int DK, int DV, int DVW, int PPW, typename IO, typename ST>
__global__ __launch_bounds__(NTS * PPW, PPW < DV / DVW ? 2 : 4) void state_kernel(PrefillArgs a, Work w) {
    extern __shared__ __align__(16) unsigned char smem_raw[];
    StateSmem<DK, DVW, IO> *parts = reinterpret_cast<StateSmem<DK, DVW, IO> *>(smem_raw);
    // (sequence rank, head) chains, rank-major: the longest sequences come first
    constexpr int NPART = DV / DVW;
    static_assert(PPW == NPART || PPW == 1, "parts per workgroup");
    int chain = blockIdx.x, part0 = 0;
    if constexpr (PPW < NPART) {
        const int grp = blockIdx.x / (kXcd * NPART), r = blockIdx.x % (kXcd * NPART);
        part0 = r / kXcd;
        chain = grp * kXcd + r % kXcd;
    }
    const int h = chain % a.hv, rank = chain / a.hv;
    if (rank >= a.num_seqs) return;
    const int n = w.seq_order[rank];
    const int lane = threadIdx.x & 63;
    const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int part = part0 + wv / 8, wave = wv % 8;
    StateSmem<DK, DVW, IO> &sm = parts[wv / 8];
    if (wave < 4) state_chain<true, DK, DV, DVW, IO, ST>(a, w, sm, n, h, part * DVW, wave, lane);    // U waves
    else state_chain<false, DK, DV, DVW, IO, ST>(a, w, sm, n, h, part * DVW, wave, lane);   // output waves
}

// ---------------------------------------------------------------------------
// launch
// ---------------------------------------------------------------------------
template <int DK, int DV, typename IO>
hipError_t launch_intra(PrefillArgs &a, Work &w, hipStream_t s) {
    const size_t smem = sizeof(IntraSmem<DK, DV>);
    const long items = (long)w.slots * a.hv;
    dim3 grid((unsigned)items);
    auto kern = a.raw_gate ? (a.scalar_gate ? intra_kernel<DK, DV, IO, true, true> : intra_kernel<DK, DV, IO, false, true>)
                           : (a.scalar_gate ? intra_kernel<DK, DV, IO, true, false> : intra_kernel<DK, DV, IO, false, false>);
    const hipError_t e = hipFuncSetAttribute((const void *)kern, hipFuncAttributeMaxDynamicSharedMemorySize, (int)smem);
    if (e != hipSuccess) return e;
    kern<<<grid, NTI, smem, s>>>(a, w);
    return hipGetLastError();
}

template <int DK, int DV, int DVW, int PPW, typename IO, typename ST>
hipError_t launch_state_w(PrefillArgs &a, Work &w, hipStream_t s) {
    // 1-D grid over (sequence rank, head) chains, rank-major; eight waves per column part
    constexpr int NPART = DV / DVW;
    const size_t smem = PPW * sizeof(StateSmem<DK, DVW, IO>);
    auto kern = state_kernel<DK, DV, DVW, PPW, IO, ST>;
    const hipError_t e = hipFuncSetAttribute((const void *)kern, hipFuncAttributeMaxDynamicSharedMemorySize, (int)smem);
    if (e != hipSuccess) return e;
    const long chains = (long)a.hv * a.num_seqs;
    const long blocks = PPW == NPART ? chains : (chains + kXcd - 1) / kXcd * kXcd * NPART;
    kern<<<dim3((unsigned)blocks), NTS * PPW, smem, s>>>(a, w);
    return hipGetLastError();
}

template <int DK, int DV, typename IO, typename ST>
hipError_t launch_state_st(PrefillArgs &a, Work &w, hipStream_t s) {
    // A chain's 128 value columns are split over two column parts of one
    // workgroup: the per-chunk critical path of a chain halves (the longest
    // chains set the kernel's end), and each part's LDS blocks stay at 64
    // value columns.
    constexpr int DVW = DV == 128 ? 64 : DV;
    constexpr int NPART = DV / DVW;
    static_assert(NPART == (DV == 128 ? 2 : 1), "column parts");
    if constexpr (NPART > 1) {
        // With few chains the chain step's latency, not the operand stream,
        // sets the time: shorter dependent MFMA chains per part pay for the
        // extra (cache-served) operand reads.  Measured on MI355X, one
        // workgroup per part: 1 x 32768 tokens x 32 heads 1.415 ms with two
        // parts, 1.28 ms with four; 1 x 4096 x 1 0.135 -> 0.108 ms; at 128
        // chains and more two parts are faster.
        // With many short chains (at most 1024 tokens per sequence on
        // average) each chain's initial-state load and final-state store
        // weigh more than its few steps; two part-workgroups per CU overlap
        // one chain's state traffic with another's steps: 32 heads, 1024 x 32
        // tokens 2.43 -> 2.37 ms, 256 x 128 1.12 -> 1.10 ms, 64 x 512
        // 0.930 -> 0.924 ms (whole prefill).  Longer sequences keep one
        // sixteen-wave workgroup per chain (16 x 2048 0.891 against 0.901 ms).
        const long chains = (long)a.hv * a.num_seqs;
        if (chains <= kVeryFewChains) return launch_state_w<DK, DV, 32, 1, IO, ST>(a, w, s);
        if (chains <= kFewChains || (long)a.total_tokens <= 1024L * a.num_seqs)
            return launch_state_w<DK, DV, DVW, 1, IO, ST>(a, w, s);
    }
    return launch_state_w<DK, DV, DVW, NPART, IO, ST>(a, w, s);
}

template <int DK, int DV, typename IO>
hipError_t launch_state(PrefillArgs &a, Work &w, hipStream_t s) {
    return a.state_bf16 ? launch_state_st<DK, DV, IO, bf16>(a, w, s) : launch_state_st<DK, DV, IO, float>(a, w, s);
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
    w.seq_order = reinterpret_cast<int32_t *>(base + l.seq_order);
    w.W = reinterpret_cast<_Float16 *>(base + l.W);
    w.Tb = reinterpret_cast<_Float16 *>(base + l.Tb);
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
