// C ABI of libkda: host-side validation, workspace sizing and launch sequencing.
// Declarations and the contract live in include/kda.h.
#include <hip/hip_runtime.h>

#include <mutex>

#include "../../include/kda.h"
#include "kda_internal.h"

// Workspace of the allocation-free prefill entry point: one copy of this
// array per GPU, placed by the code-object loader when the library is first
// used on that GPU and held until the process ends.  Host code never passes
// its name to a kernel (on the host it is only a stand-in); it uses the
// device address looked up once per device by scratch_ptr().
static __device__ __align__(256) unsigned char scratch[KDA_SCRATCH_BYTES];

namespace {

bool dim_ok(int d) { return d == 32 || d == 64 || d == 128; }
bool dtype_ok(int t) { return t == KDA_F32 || t == KDA_BF16; }
bool gate_ok(int t) { return t == KDA_GATE_CHANNEL || t == KDA_GATE_SCALAR; }
bool aligned(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
size_t io_size(int t) { return t == KDA_BF16 ? 2 : 4; }

// Byte ranges [p, p + n) overlap?
bool overlap(const void *a, size_t na, const void *b, size_t nb) {
    if (!a || !b || na == 0 || nb == 0) return false;
    const uintptr_t x = reinterpret_cast<uintptr_t>(a), y = reinterpret_cast<uintptr_t>(b);
    return x < y + nb && y < x + na;
}

kda_status check_desc(const kda_prefill_desc *d) {
    if (!d) return KDA_ERR_NULL;
    if (d->num_seqs < 0 || d->total_tokens < 0 || d->hk <= 0 || d->hv <= 0 || d->dk <= 0 ||
        d->dv <= 0 || d->hv % d->hk != 0)
        return KDA_ERR_SHAPE;
    if (!dim_ok(d->dk) || !dim_ok(d->dv) || !dtype_ok(d->io_dtype) || !dtype_ok(d->state_dtype) ||
        !gate_ok(d->gate))
        return KDA_ERR_UNSUPPORTED;
    return KDA_OK;
}

kda_status check_decode_desc(const kda_decode_desc *d) {
    if (!d) return KDA_ERR_NULL;
    if (d->batch < 0 || d->hk <= 0 || d->hv <= 0 || d->dk <= 0 || d->dv <= 0 ||
        d->hv % d->hk != 0 || d->num_slots <= 0)
        return KDA_ERR_SHAPE;
    if (!dim_ok(d->dk) || !dim_ok(d->dv) || !dtype_ok(d->io_dtype) || !dtype_ok(d->state_dtype) ||
        !gate_ok(d->gate))
        return KDA_ERR_UNSUPPORTED;
    return KDA_OK;
}

kda_status hip_status(hipError_t e) { return e == hipSuccess ? KDA_OK : KDA_ERR_HIP; }

// The gate inputs of one call: activated fp32 g and beta, or (raw) the raw
// projections x, b in the io dtype plus fp32 A_log and dt_bias.
struct GateIn {
    const void *g, *beta;
    const float *A_log, *dt_bias;
    bool raw;
};

kda_status prefill_impl(const kda_prefill_desc *d, const void *q, const void *k, const void *v,
                        const GateIn &gi, const int32_t *cu_seqlens, void *state,
                        const int32_t *state_indices, void *final_state, void *o, void *workspace,
                        size_t workspace_bytes, void *stream) {
    kda_status st = check_desc(d);
    if (st != KDA_OK) return st;
    const bool pool = state_indices != nullptr;
    const long T = d->total_tokens, N = d->num_seqs;
    if (!cu_seqlens) return KDA_ERR_NULL;
    if (T > 0 && (!q || !k || !v || !gi.g || !gi.beta || !o)) return KDA_ERR_NULL;
    if (T > 0 && gi.raw && (!gi.A_log || !gi.dt_bias)) return KDA_ERR_NULL;
    if (pool) {
        if (!state) return KDA_ERR_NULL;
        if (d->num_slots <= 0) return KDA_ERR_SHAPE;
        if (final_state && final_state != state) return KDA_ERR_ALIAS;
    }
    const void *ptrs[] = {q, k, v, gi.g, gi.beta, gi.A_log, gi.dt_bias, cu_seqlens, state, state_indices,
                          final_state, o, workspace};
    for (const void *p : ptrs)
        if (p && !aligned(p)) return KDA_ERR_ALIGN;
    const size_t need = kda::prefill_workspace_bytes(d->num_seqs, d->total_tokens, d->hv, d->dk, d->dv);
    if (need > 0 && (!workspace || workspace_bytes < need)) return KDA_ERR_WORKSPACE;

    // o must not alias any input; a dense final_state must not alias inputs
    // other than the initial state.
    const size_t isz = io_size(d->io_dtype), ssz = io_size(d->state_dtype), gsz = gi.raw ? isz : 4;
    const size_t gw = d->gate == KDA_GATE_SCALAR ? 1 : (size_t)d->dk;
    const size_t qk_b = (size_t)T * d->hk * d->dk * isz, v_b = (size_t)T * d->hv * d->dv * isz;
    const size_t g_b = (size_t)T * d->hv * gw * gsz;
    const size_t be_b = (size_t)T * d->hv * gsz, cu_b = (size_t)(N + 1) * 4;
    const size_t par_b = gi.raw ? (size_t)d->hv * gw * 4 : 0;
    const size_t rows = pool ? (size_t)d->num_slots : (size_t)N;
    const size_t s_b = rows * d->hv * d->dv * d->dk * ssz;
    const size_t o_b = (size_t)T * d->hv * d->dv * isz;
    struct R { const void *p; size_t n; } ins[] = {{q, qk_b}, {k, qk_b}, {v, v_b}, {gi.g, g_b}, {gi.beta, be_b},
                                                   {gi.A_log, par_b}, {gi.dt_bias, par_b},
                                                   {cu_seqlens, cu_b}, {state, s_b},
                                                   {state_indices, pool ? (size_t)N * 4 : 0},
                                                   {workspace, need}};
    for (const R &r : ins)
        if (overlap(o, o_b, r.p, r.n)) return KDA_ERR_ALIAS;
    if (!pool && final_state) {
        const size_t f_b = (size_t)N * d->hv * d->dv * d->dk * ssz;
        for (const R &r : ins)
            if (r.p != state && overlap(final_state, f_b, r.p, r.n)) return KDA_ERR_ALIAS;
        if (state && final_state != state && overlap(final_state, f_b, state, s_b)) return KDA_ERR_ALIAS;
    }
    if (N == 0) return KDA_OK;
    if (T == 0 && !final_state) return KDA_OK;

    // Grids, all 1-D: intra over (chunk slot, head) items; state over
    // (sequence, head) chains, one workgroup per chain, or one per column
    // part (two, or four with at most 64 chains) with at most 256 chains or
    // short sequences.
    int dev = 0, max_x = 0;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&max_x, hipDeviceAttributeMaxGridDimX, dev) != hipSuccess)
        return KDA_ERR_HIP;
    const long slots = (T + 63L * N) / 64;
    const long intra_wgs = slots * d->hv;
    // up to four column-part workgroups per (sequence, head) chain, in groups of eight chains
    const long state_wgs = ((long)d->hv * N + 8) * 4;
    if (intra_wgs > max_x || state_wgs > max_x) return KDA_ERR_UNSUPPORTED;

    kda::PrefillArgs a{};
    a.q = q; a.k = k; a.v = v; a.cu_seqlens = cu_seqlens;
    if (gi.raw) {
        a.gx = gi.g; a.bx = gi.beta; a.A_log = gi.A_log; a.dt_bias = gi.dt_bias;
    } else {
        a.g = static_cast<const float *>(gi.g); a.beta = static_cast<const float *>(gi.beta);
    }
    a.state_in = state;
    a.state_out = pool ? state : final_state;
    a.indices = state_indices;
    a.o = o;
    a.num_seqs = d->num_seqs; a.total_tokens = d->total_tokens;
    a.hk = d->hk; a.hv = d->hv; a.dk = d->dk; a.dv = d->dv;
    a.num_slots = pool ? d->num_slots : 0;
    a.scale = d->scale;
    a.io_bf16 = d->io_dtype == KDA_BF16;
    a.state_bf16 = d->state_dtype == KDA_BF16;
    a.scalar_gate = d->gate == KDA_GATE_SCALAR;
    a.raw_gate = gi.raw;
    return hip_status(kda::launch_prefill(a, workspace, static_cast<hipStream_t>(stream)));
}

// packed: q points at one [q | k | v] row per request (k and v are offsets into it).
kda_status decode_impl(const kda_decode_desc *d, const void *q, const void *k, const void *v,
                       const GateIn &gi, void *state_pool, const int32_t *state_indices, void *o,
                       void *stream, bool packed = false) {
    kda_status st = check_decode_desc(d);
    if (st != KDA_OK) return st;
    if (d->batch == 0) return KDA_OK;
    const size_t isz0 = io_size(d->io_dtype);
    const long qk_w = (long)d->hk * d->dk, v_w = (long)d->hv * d->dv;
    if (packed && q) {
        k = static_cast<const char *>(q) + qk_w * isz0;
        v = static_cast<const char *>(q) + 2 * qk_w * isz0;
    }
    if (!q || !k || !v || !gi.g || !gi.beta || !state_pool || !state_indices || !o) return KDA_ERR_NULL;
    if (gi.raw && (!gi.A_log || !gi.dt_bias)) return KDA_ERR_NULL;
    const void *ptrs[] = {q, k, v, gi.g, gi.beta, gi.A_log, gi.dt_bias, state_pool, state_indices, o};
    for (const void *p : ptrs)
        if (p && !aligned(p)) return KDA_ERR_ALIGN;
    const size_t isz = io_size(d->io_dtype), B = d->batch, gsz = gi.raw ? isz : 4;
    const size_t gw = d->gate == KDA_GATE_SCALAR ? 1 : (size_t)d->dk;
    const size_t o_b = B * d->hv * d->dv * isz;
    const size_t par_b = gi.raw ? (size_t)d->hv * gw * 4 : 0;
    const size_t qkv_b = packed ? B * (size_t)(2 * qk_w + v_w) * isz : 0;
    struct R { const void *p; size_t n; } ins[] = {
        {q, packed ? qkv_b : B * d->hk * d->dk * isz}, {k, packed ? 0 : B * d->hk * d->dk * isz},
        {v, packed ? 0 : o_b},
        {gi.g, B * d->hv * gw * gsz}, {gi.beta, B * d->hv * gsz}, {gi.A_log, par_b}, {gi.dt_bias, par_b},
        {state_pool, (size_t)d->num_slots * d->hv * d->dv * d->dk * io_size(d->state_dtype)},
        {state_indices, B * 4}};
    for (const R &r : ins)
        if (overlap(o, o_b, r.p, r.n)) return KDA_ERR_ALIAS;

    // Grid (hv x dv / tile, requests per z slab, z slabs) must fit the
    // device's per-axis limits.
    int dev = 0, max_x = 0, max_y = 0, max_z = 0;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&max_x, hipDeviceAttributeMaxGridDimX, dev) != hipSuccess ||
        hipDeviceGetAttribute(&max_y, hipDeviceAttributeMaxGridDimY, dev) != hipSuccess ||
        hipDeviceGetAttribute(&max_z, hipDeviceAttributeMaxGridDimZ, dev) != hipSuccess)
        return KDA_ERR_HIP;
    const long xdim = (long)d->hv * (d->dv / kda::decode_tile(d->dv, d->batch, d->hv, false));
    if (xdim > max_x || kda::decode_grid_y(d->batch) > max_y || kda::decode_grid_z(d->batch) > max_z)
        return KDA_ERR_UNSUPPORTED;

    kda::DecodeArgs a{};
    a.q = q; a.k = k; a.v = v; a.state = state_pool;
    if (gi.raw) {
        a.gx = gi.g; a.bx = gi.beta; a.A_log = gi.A_log; a.dt_bias = gi.dt_bias;
    } else {
        a.g = static_cast<const float *>(gi.g); a.beta = static_cast<const float *>(gi.beta);
    }
    a.indices = state_indices; a.o = o;
    a.batch = d->batch; a.hk = d->hk; a.hv = d->hv; a.dk = d->dk; a.dv = d->dv;
    a.num_slots = d->num_slots; a.scale = d->scale;
    a.io_bf16 = d->io_dtype == KDA_BF16;
    a.state_bf16 = d->state_dtype == KDA_BF16;
    a.scalar_gate = d->gate == KDA_GATE_SCALAR;
    a.raw_gate = gi.raw;
    a.qk_stride = packed ? 2 * qk_w + v_w : qk_w;
    a.v_stride = packed ? 2 * qk_w + v_w : v_w;
    return hip_status(kda::launch_decode(a, static_cast<hipStream_t>(stream)));
}

kda_status check_multi_desc(const kda_multi_decode_desc *d) {
    if (!d) return KDA_ERR_NULL;
    if (d->batch < 0 || d->total_tokens < 0 || d->hk <= 0 || d->hv <= 0 || d->dk <= 0 || d->dv <= 0 ||
        d->hv % d->hk != 0 || d->num_slots <= 0 || d->cache_pitch < 0)
        return KDA_ERR_SHAPE;
    if (!dim_ok(d->dk) || !dim_ok(d->dv) || !dtype_ok(d->io_dtype) || !dtype_ok(d->state_dtype) ||
        !gate_ok(d->gate))
        return KDA_ERR_UNSUPPORTED;
    return KDA_OK;
}

kda_status multi_decode_impl(const kda_multi_decode_desc *d, const void *q, const void *k, const void *v,
                             const GateIn &gi, const int32_t *cu_seqlens, void *state_pool,
                             const int32_t *state_indices, void *cache, void *o, void *stream) {
    kda_status st = check_multi_desc(d);
    if (st != KDA_OK) return st;
    if (d->batch == 0) return KDA_OK;
    if (!cu_seqlens || !state_pool || !state_indices) return KDA_ERR_NULL;
    if (d->cache_pitch > 0 && !cache) return KDA_ERR_NULL;
    const long T = d->total_tokens;
    if (T > 0 && (!q || !k || !v || !gi.g || !gi.beta || !o)) return KDA_ERR_NULL;
    if (T > 0 && gi.raw && (!gi.A_log || !gi.dt_bias)) return KDA_ERR_NULL;
    if (d->cache_pitch == 0) cache = nullptr;
    const void *ptrs[] = {q, k, v, gi.g, gi.beta, gi.A_log, gi.dt_bias, cu_seqlens, state_pool, state_indices,
                          cache, o};
    for (const void *p : ptrs)
        if (p && !aligned(p)) return KDA_ERR_ALIGN;
    const size_t isz = io_size(d->io_dtype), ssz = io_size(d->state_dtype), gsz = gi.raw ? isz : 4;
    const size_t gw = d->gate == KDA_GATE_SCALAR ? 1 : (size_t)d->dk, N = d->batch;
    const size_t unit = (size_t)d->hv * d->dv * d->dk * ssz;   // one state row of all heads
    const size_t o_b = (size_t)T * d->hv * d->dv * isz;
    const size_t par_b = gi.raw ? (size_t)d->hv * gw * 4 : 0;
    const size_t cache_b = cache ? N * (size_t)d->cache_pitch * unit : 0;
    struct R { const void *p; size_t n; } ins[] = {
        {q, (size_t)T * d->hk * d->dk * isz}, {k, (size_t)T * d->hk * d->dk * isz}, {v, o_b},
        {gi.g, (size_t)T * d->hv * gw * gsz}, {gi.beta, (size_t)T * d->hv * gsz}, {gi.A_log, par_b},
        {gi.dt_bias, par_b}, {cu_seqlens, (N + 1) * 4}, {state_pool, (size_t)d->num_slots * unit},
        {state_indices, N * 4}};
    for (const R &r : ins) {
        if (overlap(o, o_b, r.p, r.n)) return KDA_ERR_ALIAS;
        if (overlap(cache, cache_b, r.p, r.n)) return KDA_ERR_ALIAS;
    }
    if (overlap(cache, cache_b, o, o_b)) return KDA_ERR_ALIAS;
    if (T == 0) return KDA_OK;   // every request is empty: nothing is read or written

    int dev = 0, max_x = 0, max_y = 0, max_z = 0;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&max_x, hipDeviceAttributeMaxGridDimX, dev) != hipSuccess ||
        hipDeviceGetAttribute(&max_y, hipDeviceAttributeMaxGridDimY, dev) != hipSuccess ||
        hipDeviceGetAttribute(&max_z, hipDeviceAttributeMaxGridDimZ, dev) != hipSuccess)
        return KDA_ERR_HIP;
    const long xdim = (long)d->hv * (d->dv / kda::decode_tile(d->dv, d->batch, d->hv, true));
    if (xdim > max_x || kda::decode_grid_y(d->batch) > max_y || kda::decode_grid_z(d->batch) > max_z)
        return KDA_ERR_UNSUPPORTED;

    kda::DecodeArgs a{};
    a.q = q; a.k = k; a.v = v; a.state = state_pool;
    if (gi.raw) {
        a.gx = gi.g; a.bx = gi.beta; a.A_log = gi.A_log; a.dt_bias = gi.dt_bias;
    } else {
        a.g = static_cast<const float *>(gi.g); a.beta = static_cast<const float *>(gi.beta);
    }
    a.indices = state_indices; a.o = o;
    a.batch = d->batch; a.hk = d->hk; a.hv = d->hv; a.dk = d->dk; a.dv = d->dv;
    a.num_slots = d->num_slots; a.scale = d->scale;
    a.io_bf16 = d->io_dtype == KDA_BF16;
    a.state_bf16 = d->state_dtype == KDA_BF16;
    a.scalar_gate = d->gate == KDA_GATE_SCALAR;
    a.raw_gate = gi.raw;
    a.qk_stride = (long)d->hk * d->dk;
    a.v_stride = (long)d->hv * d->dv;
    a.cu_seqlens = cu_seqlens;
    a.cache = cache;
    a.cache_pitch = d->cache_pitch;
    a.update_pool = d->update_pool != 0;
    return hip_status(kda::launch_decode_multi(a, static_cast<hipStream_t>(stream)));
}

// Device address of `scratch` on the current device, looked up once per
// device with that device current (each GPU holds its own copy at its own
// address).  nullptr on failure.
void *scratch_ptr() {
    constexpr int kMaxDevices = 64;
    static std::mutex mu;
    static void *ptrs[kMaxDevices] = {};
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
    std::lock_guard<std::mutex> lock(mu);
    if (!ptrs[dev]) {
        void *p = nullptr;
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess) return nullptr;
        ptrs[dev] = p;
    }
    return ptrs[dev];
}

}  // namespace

extern "C" {

const char *kda_status_string(kda_status s) {
    switch (s) {
    case KDA_OK: return "ok";
    case KDA_ERR_NULL: return "a required pointer or descriptor is NULL";
    case KDA_ERR_SHAPE: return "inconsistent or non-positive sizes";
    case KDA_ERR_UNSUPPORTED: return "unsupported head dim, dtype, gate kind or grid size";
    case KDA_ERR_WORKSPACE: return "workspace missing or too small";
    case KDA_ERR_ALIAS: return "an output aliases an input";
    case KDA_ERR_HIP: return "HIP launch or runtime error";
    case KDA_ERR_ALIGN: return "a tensor pointer is not 16-byte aligned";
    }
    return "unknown status";
}

int32_t kda_version(void) { return 200; }

size_t kda_chunk_prefill_workspace_size(const kda_prefill_desc *d) {
    if (check_desc(d) != KDA_OK) return 0;
    return kda::prefill_workspace_bytes(d->num_seqs, d->total_tokens, d->hv, d->dk, d->dv);
}

kda_status kda_chunk_prefill(const kda_prefill_desc *d, const void *q, const void *k, const void *v,
                             const float *g, const float *beta, const int32_t *cu_seqlens,
                             void *state, const int32_t *state_indices, void *final_state, void *o,
                             void *workspace, size_t workspace_bytes, void *stream) {
    const GateIn gi{g, beta, nullptr, nullptr, false};
    return prefill_impl(d, q, k, v, gi, cu_seqlens, state, state_indices, final_state, o, workspace,
                        workspace_bytes, stream);
}

kda_status kda_chunk_prefill_fused_gate(const kda_prefill_desc *d, const void *q, const void *k,
                                        const void *v, const void *gate_x, const float *A_log,
                                        const float *dt_bias, const void *beta_x,
                                        const int32_t *cu_seqlens, void *state,
                                        const int32_t *state_indices, void *final_state, void *o,
                                        void *workspace, size_t workspace_bytes, void *stream) {
    const GateIn gi{gate_x, beta_x, A_log, dt_bias, true};
    return prefill_impl(d, q, k, v, gi, cu_seqlens, state, state_indices, final_state, o, workspace,
                        workspace_bytes, stream);
}

kda_status kda_chunk_prefill_noalloc(const kda_prefill_desc *d, const void *q, const void *k, const void *v,
                                     const float *g, const float *beta, const int32_t *cu_seqlens,
                                     void *state, const int32_t *state_indices, void *final_state, void *o,
                                     void *stream) {
    // Sizes beyond the array are refused before any HIP call.
    const kda_status st = check_desc(d);
    if (st != KDA_OK) return st;
    if (kda::prefill_workspace_bytes(d->num_seqs, d->total_tokens, d->hv, d->dk, d->dv) > KDA_SCRATCH_BYTES)
        return KDA_ERR_WORKSPACE;
    void *ws = scratch_ptr();
    if (!ws) return KDA_ERR_HIP;
    const GateIn gi{g, beta, nullptr, nullptr, false};
    return prefill_impl(d, q, k, v, gi, cu_seqlens, state, state_indices, final_state, o, ws, KDA_SCRATCH_BYTES,
                        stream);
}

kda_status kda_recurrent_decode(const kda_decode_desc *d, const void *q, const void *k, const void *v,
                                const float *g, const float *beta, void *state_pool,
                                const int32_t *state_indices, void *o, void *stream) {
    const GateIn gi{g, beta, nullptr, nullptr, false};
    return decode_impl(d, q, k, v, gi, state_pool, state_indices, o, stream);
}

kda_status kda_recurrent_decode_fused_gate(const kda_decode_desc *d, const void *q, const void *k,
                                           const void *v, const void *gate_x, const float *A_log,
                                           const float *dt_bias, const void *beta_x, void *state_pool,
                                           const int32_t *state_indices, void *o, void *stream) {
    const GateIn gi{gate_x, beta_x, A_log, dt_bias, true};
    return decode_impl(d, q, k, v, gi, state_pool, state_indices, o, stream);
}

kda_status kda_recurrent_decode_packed(const kda_decode_desc *d, const void *qkv, const float *g,
                                       const float *beta, void *state_pool, const int32_t *state_indices,
                                       void *o, void *stream) {
    const GateIn gi{g, beta, nullptr, nullptr, false};
    return decode_impl(d, qkv, nullptr, nullptr, gi, state_pool, state_indices, o, stream, true);
}

kda_status kda_recurrent_decode_packed_fused_gate(const kda_decode_desc *d, const void *qkv,
                                                  const void *gate_x, const float *A_log,
                                                  const float *dt_bias, const void *beta_x, void *state_pool,
                                                  const int32_t *state_indices, void *o, void *stream) {
    const GateIn gi{gate_x, beta_x, A_log, dt_bias, true};
    return decode_impl(d, qkv, nullptr, nullptr, gi, state_pool, state_indices, o, stream, true);
}

kda_status kda_recurrent_decode_multi(const kda_multi_decode_desc *d, const void *q, const void *k,
                                      const void *v, const float *g, const float *beta,
                                      const int32_t *cu_seqlens, void *state_pool,
                                      const int32_t *state_indices, void *intermediate_states, void *o,
                                      void *stream) {
    const GateIn gi{g, beta, nullptr, nullptr, false};
    return multi_decode_impl(d, q, k, v, gi, cu_seqlens, state_pool, state_indices, intermediate_states, o,
                             stream);
}

kda_status kda_recurrent_decode_multi_fused_gate(const kda_multi_decode_desc *d, const void *q, const void *k,
                                                 const void *v, const void *gate_x, const float *A_log,
                                                 const float *dt_bias, const void *beta_x,
                                                 const int32_t *cu_seqlens, void *state_pool,
                                                 const int32_t *state_indices, void *intermediate_states,
                                                 void *o, void *stream) {
    const GateIn gi{gate_x, beta_x, A_log, dt_bias, true};
    return multi_decode_impl(d, q, k, v, gi, cu_seqlens, state_pool, state_indices, intermediate_states, o,
                             stream);
}

}  // extern "C"
