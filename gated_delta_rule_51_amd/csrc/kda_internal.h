// Internal launch interface between the C ABI (kda_api.hip) and the kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace kda {

struct DecodeArgs {
    const void *q, *k, *v;
    const float *g, *beta;             // activated gate and beta (fp32), or
    const void *gx, *bx;               // raw gate and beta inputs (io dtype) with
    const float *A_log, *dt_bias;      // per-(head, channel) activation parameters
    void *state;
    const int32_t *indices;
    void *o;
    int batch, hk, hv, dk, dv, num_slots;
    float scale;
    bool io_bf16, state_bf16, scalar_gate, raw_gate;
    // token row strides (elements) of q, k (same stride) and v: hk * dk and hv * dv
    // for separate tensors, 2 hk dk + hv dv for one packed [q | k | v] row per token
    long qk_stride, v_stride;
    // multi-token decode only: request n owns tokens [cu_seqlens[n], cu_seqlens[n+1]);
    // the state after its step j goes to cache[n * cache_pitch + j] when j < cache_pitch
    const int32_t *cu_seqlens;
    void *cache;
    int cache_pitch;
    bool update_pool;
};

hipError_t launch_decode(const DecodeArgs &a, hipStream_t stream);
hipError_t launch_decode_multi(const DecodeArgs &a, hipStream_t stream);
int decode_tile(int dv, long batch, int hv, bool multi);
int decode_grid_y(int batch);   // requests per z slab of the decode grid
int decode_grid_z(int batch);   // z slabs

// Chunked prefill.  Chunk size and the chunk-slot bound are fixed here.
constexpr int kChunk = 64;

struct PrefillArgs {
    const void *q, *k, *v;
    const float *g, *beta;             // activated gate and beta (fp32), or
    const void *gx, *bx;               // raw gate and beta inputs (io dtype) with
    const float *A_log, *dt_bias;      // per-(head, channel) activation parameters
    const int32_t *cu_seqlens;
    const void *state_in;     // dense h0, pool, or NULL
    void *state_out;          // dense ht, pool, or NULL
    const int32_t *indices;   // pool slots or NULL
    void *o;
    int num_seqs, total_tokens, hk, hv, dk, dv, num_slots;
    float scale;
    bool io_bf16, state_bf16, scalar_gate, raw_gate;
};


size_t prefill_workspace_bytes(int num_seqs, int total_tokens, int hv, int dk, int dv);
hipError_t launch_prefill(PrefillArgs &a, void *workspace, hipStream_t stream);

}  // namespace kda
