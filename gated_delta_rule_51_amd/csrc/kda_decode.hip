// Recurrent decode of the gated delta rule against a state pool: one token per
// request (decode_kernel), or a short run of tokens per request with the state
// after every token cached (multi_decode_kernel, the verify step of
// speculative decoding).
//
// Per (value tile, request b, value head h) one workgroup streams the BV rows
// of the stored state pool[slot(b), h] ([V, K], K contiguous), applies
//     S' = Diag(exp g) S;  u = beta (v - S'^T k);  S = S' + k u^T;  o = scale S^T q
// row by row (each stored row j is one value channel, so rows are independent
// given k, q, g), and writes the rows back in place.  The grid keeps batch and
// head on separate axes (sglang PR 37317 digest, 实现拆解 item 1: folding them
// into one axis overflowed the 65535 limit at large decode batches): x runs
// over (head, value tile), head-major, so consecutive workgroups stream the
// contiguous [Hv, V, K] block of one pool row, and the batch is spread over
// y and z (request b = y + z * gridDim.y), so it is not held to one axis's
// 65535 either (the digest's 风险与影响 item 5 notes that per-axis limit after
// the split).  A negative slot index selects the last pool row (PR 30169
// digest, 实现拆解 item 3).
//
// Memory-bound: the state row block is read once and written once with
// 16-byte nontemporal accesses that are contiguous across the workgroup.
#include "kda_device.h"
#include "kda_internal.h"

namespace kda {

// Thread layout over one workgroup's BV stored rows: LPR lanes per row, each
// holding VEC consecutive channels (16 bytes of state); NP passes of RPP rows.
template <int DK, int BV, typename ST> struct RowTile {
    static constexpr int VEC = (sizeof(ST) == 4) ? 4 : 8;  // state elements per 16 B
    static constexpr int LPR = DK / VEC;                    // lanes per stored row
    static constexpr int RPP = 256 / LPR;                   // rows per pass
    static constexpr int NP = (BV + RPP - 1) / RPP;         // passes
    static_assert(DK % VEC == 0 && LPR <= 64, "tile");
};

// Element offsets of this thread's rows within a block of BV stored rows.
// With OPAQUE they are formed once and hidden from the compiler, which
// otherwise re-forms the row addresses between the row stores at the end of
// the one-token decode; the stores then go out back to back (measured 3.7%
// faster for the B = 4096 decode).
template <int DK, int BV, typename ST, bool OPAQUE = false>
__device__ __forceinline__ void row_offs(int r0, int cg, unsigned (&ro)[RowTile<DK, BV, ST>::NP]) {
    using R = RowTile<DK, BV, ST>;
#pragma unroll
    for (int p = 0; p < R::NP; ++p) {
        ro[p] = (unsigned)((r0 + p * R::RPP) * DK + cg * R::VEC);
        if constexpr (OPAQUE) asm volatile("" : "+v"(ro[p]));
    }
}

// Whether pass p holds a row of the block (always, when the passes tile it).
template <int DK, int BV, typename ST> __device__ __forceinline__ bool row_in(int r0, int p) {
    using R = RowTile<DK, BV, ST>;
    return R::NP * R::RPP == BV || r0 + p * R::RPP < BV;
}

// Load this thread's part of the rows at st (offsets ro) into s.
template <int DK, int BV, typename ST, bool NT>
__device__ __forceinline__ void load_rows(const ST *st, const unsigned (&ro)[RowTile<DK, BV, ST>::NP], int r0,
                                          float (&s)[RowTile<DK, BV, ST>::NP][RowTile<DK, BV, ST>::VEC]) {
    using R = RowTile<DK, BV, ST>;
#pragma unroll
    for (int p = 0; p < R::NP; ++p) {
        if (row_in<DK, BV, ST>(r0, p)) {
            const ST *src = st + ro[p];
            if constexpr (R::VEC == 4) {
                f32x4 x = NT ? __builtin_nontemporal_load(reinterpret_cast<const f32x4 *>(src)) : load4(src);
#pragma unroll
                for (int i = 0; i < 4; ++i) s[p][i] = x[i];
            } else {
                u32x4 w = NT ? __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(src))
                             : *reinterpret_cast<const u32x4 *>(src);
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    s[p][2 * i] = __uint_as_float(w[i] << 16);
                    s[p][2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
                }
            }
        }
    }
}

// Store this thread's part of the rows to st (offsets ro; bf16 storage rounds
// to nearest even).
template <int DK, int BV, typename ST, bool NT>
__device__ __forceinline__ void store_rows(ST *st, const unsigned (&ro)[RowTile<DK, BV, ST>::NP], int r0,
                                           const float (&s)[RowTile<DK, BV, ST>::NP][RowTile<DK, BV, ST>::VEC]) {
    using R = RowTile<DK, BV, ST>;
#pragma unroll
    for (int p = 0; p < R::NP; ++p) {
        if (row_in<DK, BV, ST>(r0, p)) {
            ST *dst = st + ro[p];
            if constexpr (R::VEC == 4) {
                f32x4 x;
#pragma unroll
                for (int i = 0; i < 4; ++i) x[i] = s[p][i];
                if constexpr (NT) __builtin_nontemporal_store(x, reinterpret_cast<f32x4 *>(dst));
                else *reinterpret_cast<f32x4 *>(dst) = x;
            } else {
                u32x4 w;
#pragma unroll
                for (int i = 0; i < 4; ++i) w[i] = pack_bf16x2(s[p][2 * i], s[p][2 * i + 1]);
                if constexpr (NT) __builtin_nontemporal_store(w, reinterpret_cast<u32x4 *>(dst));
                else *reinterpret_cast<u32x4 *>(dst) = w;
            }
        }
    }
}

// Cache policy of the state stores that stream out of the verify decode: the
// nontemporal and device-scope bits (nt, sc1).  Its cached steps measured on
// MI355X (1024 requests x 4 tokens): nt alone 1.885 ms, nt with sc1
// 1.842 ms, sc0 with sc1 and no nt 2.10 ms.
constexpr int kStreamStore = 2 | 16;

// Store this thread's part of the rows through a buffer resource covering the
// row block: the lane's offset is one register and each pass adds a scalar
// offset, so the stores need no address arithmetic between them and go out
// back to back; the range check bounds them to the block.
template <int DK, int BV, typename ST>
__device__ __forceinline__ void store_rows_buf(const __amdgpu_buffer_rsrc_t rsrc, unsigned voff, int r0,
                                               const float (&s)[RowTile<DK, BV, ST>::NP][RowTile<DK, BV, ST>::VEC]) {
    using R = RowTile<DK, BV, ST>;
#pragma unroll
    for (int p = 0; p < R::NP; ++p) {
        if (row_in<DK, BV, ST>(r0, p)) {
            u32x4 w;
            if constexpr (R::VEC == 4) {
#pragma unroll
                for (int i = 0; i < 4; ++i) w[i] = __float_as_uint(s[p][i]);
            } else {
#pragma unroll
                for (int i = 0; i < 4; ++i) w[i] = pack_bf16x2(s[p][2 * i], s[p][2 * i + 1]);
            }
            __builtin_amdgcn_raw_buffer_store_b128(w, rsrc, voff, p * R::RPP * DK * (int)sizeof(ST), kStreamStore);
        }
    }
}

// The per-token inputs of one (token t, value head h) for channels c0 .. c0+VEC-1:
// k, q, the decay factors exp(g) and beta (activated here from raw inputs if RAW).
template <int DK, int VEC, typename IO, bool SCALAR, bool RAW>
__device__ __forceinline__ void token_inputs(const DecodeArgs &a, long t, int h, int hk_idx, int c0,
                                             float (&kk)[VEC], float (&qq)[VEC], float (&dec)[VEC],
                                             float &beta) {
    const IO *kp = reinterpret_cast<const IO *>(a.k) + t * a.qk_stride + hk_idx * DK + c0;
    const IO *qp = reinterpret_cast<const IO *>(a.q) + t * a.qk_stride + hk_idx * DK + c0;
#pragma unroll
    for (int i = 0; i < VEC; i += 4) {
        f32x4 x = load4(kp + i), y = load4(qp + i);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            kk[i + e] = x[e];
            qq[i + e] = y[e];
        }
    }
    if constexpr (RAW) {
        // raw gate x (io dtype) activated here: exp(g), g = -exp(A_log) softplus(x + dt_bias)
        const IO *xp = reinterpret_cast<const IO *>(a.gx);
        if constexpr (SCALAR) {
            const float x = io_traits<IO>::load(xp, t * a.hv + h);
            const float d = gate_decay((x + a.dt_bias[h]) * kLog2e, exp_f(a.A_log[h]));
#pragma unroll
            for (int i = 0; i < VEC; ++i) dec[i] = d;
        } else {
#pragma unroll
            for (int i = 0; i < VEC; i += 4) {
                const f32x4 x = load4(xp + (t * a.hv + h) * DK + c0 + i);
                const f32x4 al = *reinterpret_cast<const f32x4 *>(a.A_log + (long)h * DK + c0 + i);
                const f32x4 db = *reinterpret_cast<const f32x4 *>(a.dt_bias + (long)h * DK + c0 + i);
#pragma unroll
                for (int e = 0; e < 4; ++e) dec[i + e] = gate_decay((x[e] + db[e]) * kLog2e, exp_f(al[e]));
            }
        }
        beta = sigmoid_f(io_traits<IO>::load(reinterpret_cast<const IO *>(a.bx), t * a.hv + h));
    } else {
        if constexpr (SCALAR) {
            const float d = exp_f(a.g[t * a.hv + h]);
#pragma unroll
            for (int i = 0; i < VEC; ++i) dec[i] = d;
        } else {
            const float *gp = a.g + (t * a.hv + h) * DK + c0;
#pragma unroll
            for (int i = 0; i < VEC; i += 4) {
                f32x4 x = *reinterpret_cast<const f32x4 *>(gp + i);
#pragma unroll
                for (int e = 0; e < 4; ++e) dec[i + e] = exp_f(x[e]);
            }
        }
        beta = a.beta[t * a.hv + h];
    }
}

// One token applied to this thread's rows: decay, residual against v, rank-1
// write, read-out; lane cg == 0 of each row writes o.  vrow(p, row) gives the
// token's v value of the thread's row p (stored row `row`).  With DEFER the
// o values are kept until every row is done and then stored together: memory
// operations complete in issue order, so an o store between two rows makes
// the next row's v load wait for it, a memory round trip per row.  The
// multi-token decode defers (without a step cache 1024 requests x 8 tokens
// x 32 heads 2.26 -> 1.89 ms, 4096 x 4 5.13 -> 4.14 ms; the cached verify
// decode unchanged); the one-token decode does not (its other resident
// workgroups hide those waits, and o stores last measured 0.7% slower).
template <int DK, int BV, typename IO, typename ST, bool DEFER = false, typename VF>
__device__ __forceinline__ void token_update(VF vrow, IO *op, float scale, int r0, int cg,
                                             float (&s)[RowTile<DK, BV, ST>::NP][RowTile<DK, BV, ST>::VEC],
                                             const float (&kk)[RowTile<DK, BV, ST>::VEC],
                                             const float (&qq)[RowTile<DK, BV, ST>::VEC],
                                             const float (&dec)[RowTile<DK, BV, ST>::VEC], float beta) {
    using R = RowTile<DK, BV, ST>;
    float ov[R::NP];
#pragma unroll
    for (int p = 0; p < R::NP; ++p) {
        const int row = r0 + p * R::RPP;
        ov[p] = 0.f;
        if (row_in<DK, BV, ST>(r0, p)) {
            float pk = 0.f;
#pragma unroll
            for (int i = 0; i < R::VEC; ++i) {
                s[p][i] *= dec[i];
                pk += s[p][i] * kk[i];
            }
            pk = group_sum<R::LPR>(pk);
            const float u = beta * (vrow(p, row) - pk);
            float pq = 0.f;
#pragma unroll
            for (int i = 0; i < R::VEC; ++i) {
                s[p][i] += kk[i] * u;
                pq += s[p][i] * qq[i];
            }
            pq = scale * group_sum<R::LPR>(pq);
            if constexpr (DEFER) ov[p] = pq;
            else if (cg == 0) io_traits<IO>::store(op, row, pq);
        }
    }
    if constexpr (DEFER) {
        if (cg == 0) {
#pragma unroll
            for (int p = 0; p < R::NP; ++p)
                if (row_in<DK, BV, ST>(r0, p)) io_traits<IO>::store(op, r0 + p * R::RPP, ov[p]);
        }
    }
}

template <int DK, int BV, typename IO, typename ST, bool SCALAR, bool RAW, bool NT>
__global__ __launch_bounds__(256) void decode_kernel(DecodeArgs a) {
    using R = RowTile<DK, BV, ST>;
    const int tid = threadIdx.x;
    const int cg = tid % R::LPR;
    const int r0 = tid / R::LPR;
    constexpr int NT_MAX = 128 / BV;
    const int nt = a.dv / BV;   // value tiles per head (1 when BV = dv)
    const int b = (int)blockIdx.y + (int)blockIdx.z * (int)gridDim.y;   // request
    if (b >= a.batch) return;   // the last z slab may be partly empty
    const int h = NT_MAX == 1 ? (int)blockIdx.x : (int)blockIdx.x / nt;
    const int j0 = NT_MAX == 1 ? 0 : ((int)blockIdx.x % nt) * BV;
    const int hk_idx = h / (a.hv / a.hk);

    int slot = a.indices[b];
    if (slot < 0) slot = a.num_slots - 1;
    ST *st = reinterpret_cast<ST *>(a.state) + (((long)slot * a.hv + h) * a.dv + j0) * (long)DK;

    // Issue every state load first.
    unsigned ro[R::NP];
    row_offs<DK, BV, ST, true>(r0, cg, ro);
    float s[R::NP][R::VEC];
    load_rows<DK, BV, ST, NT>(st, ro, r0, s);

    float dec[R::VEC], kk[R::VEC], qq[R::VEC], beta;
    token_inputs<DK, R::VEC, IO, SCALAR, RAW>(a, b, h, hk_idx, cg * R::VEC, kk, qq, dec, beta);
    const IO *vp = reinterpret_cast<const IO *>(a.v) + (long)b * a.v_stride + (long)h * a.dv + j0;
    IO *op = reinterpret_cast<IO *>(a.o) + ((long)b * a.hv + h) * a.dv + j0;
    token_update<DK, BV, IO, ST>([&](int, int row) { return io_traits<IO>::load(vp, row); }, op, a.scale,
                                 r0, cg, s, kk, qq, dec, beta);

    store_rows<DK, BV, ST, NT>(st, ro, r0, s);
}

// Multi-token decode: request b runs its tokens [cu[b], cu[b+1]) one after
// the other with the state held in registers, writes o for each, caches the
// state after step j at cache[b * pitch + j] (j < pitch; the pitch is the
// per-request step count the cache was allocated with, sglang PR 37317
// digest, 实现拆解 item 2), and with update_pool writes the last state back to
// the pool row.  A request with no tokens writes nothing.
template <int DK, int BV, typename IO, typename ST, bool SCALAR, bool RAW>
__global__ __launch_bounds__(256) void multi_decode_kernel(DecodeArgs a) {
    using R = RowTile<DK, BV, ST>;
    const int tid = threadIdx.x;
    const int cg = tid % R::LPR;
    const int r0 = tid / R::LPR;
    constexpr int NT_MAX = 128 / BV;
    const int nt = a.dv / BV;
    const int b = (int)blockIdx.y + (int)blockIdx.z * (int)gridDim.y;   // request
    if (b >= a.batch) return;   // the last z slab may be partly empty
    const int h = NT_MAX == 1 ? (int)blockIdx.x : (int)blockIdx.x / nt;
    const int j0 = NT_MAX == 1 ? 0 : ((int)blockIdx.x % nt) * BV;
    const int hk_idx = h / (a.hv / a.hk);
    const int t0 = a.cu_seqlens[b], t1 = a.cu_seqlens[b + 1];
    if (t1 <= t0) return;

    int slot = a.indices[b];
    if (slot < 0) slot = a.num_slots - 1;
    ST *st = reinterpret_cast<ST *>(a.state) + (((long)slot * a.hv + h) * a.dv + j0) * (long)DK;
    unsigned ro[R::NP];
    row_offs<DK, BV, ST>(r0, cg, ro);
    float s[R::NP][R::VEC];
    load_rows<DK, BV, ST, true>(st, ro, r0, s);

    const long step_elems = (long)a.hv * a.dv * DK;   // one cached step of one request
    ST *cache = reinterpret_cast<ST *>(a.cache);
    float dec[R::VEC], kk[R::VEC], qq[R::VEC], beta;
    token_inputs<DK, R::VEC, IO, SCALAR, RAW>(a, t0, h, hk_idx, cg * R::VEC, kk, qq, dec, beta);
    for (int t = t0; t < t1; ++t) {
        // next token's inputs first (the last token reloads itself)
        float dec2[R::VEC], kk2[R::VEC], qq2[R::VEC], beta2;
        token_inputs<DK, R::VEC, IO, SCALAR, RAW>(a, min(t + 1, t1 - 1), h, hk_idx, cg * R::VEC, kk2, qq2, dec2, beta2);
        const IO *vp = reinterpret_cast<const IO *>(a.v) + (long)t * a.v_stride + (long)h * a.dv + j0;
        IO *op = reinterpret_cast<IO *>(a.o) + ((long)t * a.hv + h) * a.dv + j0;
        token_update<DK, BV, IO, ST, true>([&](int, int row) { return io_traits<IO>::load(vp, row); }, op,
                                           a.scale, r0, cg, s, kk, qq, dec, beta);
        const int j = t - t0;
        if (cache != nullptr && j < a.cache_pitch) {
            ST *cb = cache + ((long)b * a.cache_pitch + j) * step_elems + ((long)h * a.dv + j0) * DK;
            const __amdgpu_buffer_rsrc_t cr =
                __builtin_amdgcn_make_buffer_rsrc(cb, 0, BV * DK * (int)sizeof(ST), kBufferWord3);
            store_rows_buf<DK, BV, ST>(cr, ro[0] * (unsigned)sizeof(ST), r0, s);
        }
#pragma unroll
        for (int i = 0; i < R::VEC; ++i) { dec[i] = dec2[i]; kk[i] = kk2[i]; qq[i] = qq2[i]; }
        beta = beta2;
    }
    if (a.update_pool) {
        // the row offsets re-formed here, so that those of the initial load
        // are not kept live through the token loop
        int r0x = r0, cgx = cg;
        asm volatile("" : "+v"(r0x), "+v"(cgx));
        unsigned rx[R::NP];
        row_offs<DK, BV, ST>(r0x, cgx, rx);
        store_rows<DK, BV, ST, true>(st, rx, r0x, s);
    }
}

template <int DK, int BV, typename IO, typename ST, bool SCALAR>
static hipError_t launch_t(const DecodeArgs &a, bool multi, hipStream_t stream) {
    // The state block is touched once per call: stream it past the caches.
    dim3 grid(a.hv * (a.dv / BV), decode_grid_y(a.batch), decode_grid_z(a.batch));
    if (multi) {
        if (a.raw_gate)
            multi_decode_kernel<DK, BV, IO, ST, SCALAR, true><<<grid, 256, 0, stream>>>(a);
        else
            multi_decode_kernel<DK, BV, IO, ST, SCALAR, false><<<grid, 256, 0, stream>>>(a);
    } else {
        if (a.raw_gate)
            decode_kernel<DK, BV, IO, ST, SCALAR, true, true><<<grid, 256, 0, stream>>>(a);
        else
            decode_kernel<DK, BV, IO, ST, SCALAR, false, true><<<grid, 256, 0, stream>>>(a);
    }
    return hipGetLastError();
}

template <int DK, int BV, typename IO, typename ST>
static hipError_t launch_g(const DecodeArgs &a, bool m, hipStream_t s) {
    return a.scalar_gate ? launch_t<DK, BV, IO, ST, true>(a, m, s) : launch_t<DK, BV, IO, ST, false>(a, m, s);
}
template <int DK, int BV, typename IO>
static hipError_t launch_s(const DecodeArgs &a, bool m, hipStream_t s) {
    return a.state_bf16 ? launch_g<DK, BV, IO, bf16>(a, m, s) : launch_g<DK, BV, IO, float>(a, m, s);
}
template <int DK, int BV>
static hipError_t launch_i(const DecodeArgs &a, bool m, hipStream_t s) {
    return a.io_bf16 ? launch_s<DK, BV, bf16>(a, m, s) : launch_s<DK, BV, float>(a, m, s);
}
template <int DK>
static hipError_t launch_v(const DecodeArgs &a, int bv, bool m, hipStream_t s) {
    switch (bv) {
    case 32: return launch_i<DK, 32>(a, m, s);
    case 64: return launch_i<DK, 64>(a, m, s);
    default: return launch_i<DK, 128>(a, m, s);
    }
}

static hipError_t launch_any(const DecodeArgs &a, bool multi, hipStream_t stream) {
    const int bv = decode_tile(a.dv, a.batch, a.hv, multi);
    switch (a.dk) {
    case 32: return launch_v<32>(a, bv, multi, stream);
    case 64: return launch_v<64>(a, bv, multi, stream);
    default: return launch_v<128>(a, bv, multi, stream);
    }
}

// Batch split over grid y and z: z slabs of at most 65535 requests each.
int decode_grid_z(int batch) { return batch <= 0 ? 1 : (batch + 65534) / 65535; }
int decode_grid_y(int batch) {
    const int z = decode_grid_z(batch);
    return batch <= 0 ? 1 : (batch + z - 1) / z;
}

// Value rows per workgroup.  A whole head (up to 128 rows) once the batch
// fills the chip; 32-row tiles for small batches, where four times as many
// shorter workgroups cut the latency.  Kernel times on MI355X (K = V = 128,
// Hv = 32), whole head against 32-row tiles: one-token decode B = 1 9.2 and
// 4.4 us, B = 16 16.9 and 12.5 us, B = 256 198 and 188 us, B = 512 374 and
// 385 us, B = 4096 2.87 and 3.21 ms; verify with 4 tokens per request B = 1
// 29 and 10 us, B = 16 41 and 32 us, B = 64 124 and 130 us.  The results
// are the same either way (a row's arithmetic does not depend on its tile).
int decode_tile(int dv, long batch, int hv, bool multi) {
    const long rows = batch * hv * (long)dv;   // state rows of the call
    const long small = (multi ? 32L : 256L) * 32 * 128;
    if (dv > 32 && rows <= small) return 32;
    return dv < 128 ? dv : 128;
}

hipError_t launch_decode(const DecodeArgs &a, hipStream_t stream) { return launch_any(a, false, stream); }

hipError_t launch_decode_multi(const DecodeArgs &a, hipStream_t stream) { return launch_any(a, true, stream); }

}  // namespace kda
