/*
 * libkda — gated delta rule (Kimi Delta Attention, KDA) on AMD Instinct MI355X
 * (gfx950): chunked prefill over packed variable-length sequences and a
 * one-token recurrent decode, both reading and writing recurrent states
 * either densely or in place in a state pool.
 *
 * The operation (per sequence and value head; S is the K x V state):
 *     S'  = Diag(exp g_t) S          decay, one factor per key channel
 *     u   = beta_t (v_t - S'^T k_t)  delta-rule residual
 *     S   = S' + k_t u^T             rank-1 write
 *     o_t = scale * S^T q_t          read-out after the write
 * GDN's scalar gate is the case of one g per (token, head) (gate = SCALAR).
 *
 * Sources (web digests of sglang pull requests):
 *   - PR 27488 digest "KDA SM100 CuteDSL prefill": sections 功能与动机 and
 *     实现拆解 (per-channel decay gate; chunk size 64; prologue cumsum, KKT
 *     inverse + U/W, state and output kernels; workspace reuse keyed by
 *     stream), and the extend wrapper in 关键源码片段 (q, k L2-normalised by
 *     the caller; g and beta trimmed to the real token count).
 *   - PR 30169 digest "fused pool-state I/O": sections 实现拆解 and 关键源码片段
 *     (state pool [slots, Hv, V, K]; per-sequence slot indices read and
 *     written in place by the state kernel; padding index -1 selects the last
 *     slot; rows not indexed are untouched; pool mode bit-identical to dense).
 *   - PR 37317 digest "grid split": section 实现拆解 item 1 (decode grid keeps
 *     batch and head on separate axes, so B * Hv may exceed 65535).
 *
 * Conventions for every entry point
 *   - All tensor pointers are DEVICE pointers owned by the caller, contiguous
 *     in the layouts below, 16-byte aligned.  The library allocates nothing,
 *     frees nothing and keeps no pointer after it returns.
 *   - Work is enqueued on `stream` (a hipStream_t; NULL = the null stream) and
 *     returns without synchronising the host.  No host<->device copies.
 *   - Errors are found from host-visible values only (descriptor, null and
 *     aligned pointers, workspace size, aliasing rules, grid limits) and are
 *     reported as a status; nothing is launched when a check fails.  A launch
 *     failure is reported as KDA_ERR_HIP.  Nothing prints, aborts or throws.
 *   - Sizes come from the descriptor only: an array may hold more rows than
 *     the call describes (a batch padded to a captured size), and rows past
 *     the described count are never read (the KDA prefill digest, sglang
 *     PR 27488, 实现拆解 item 3, trims padded g and beta to q's token count).
 *   - Not checked (preconditions): device index values lie in [-1, slots-2]
 *     and are unique apart from -1; g is finite and <= 0; cu_seqlens is
 *     non-decreasing with cu[0] = 0 and cu[N] = total_tokens.
 *   - GQA: value head h reads key head h / (hv / hk); hv % hk == 0.
 *   - Supported sizes: dk, dv in {32, 64, 128}.  io dtype f32 or bf16; state
 *     dtype f32 or bf16.  Accumulation is fp32.
 *   - Prefill precision.  The prefill's matrix-core operands are fp16 (IEEE
 *     binary16: 11-bit significand, largest finite 65504, normal down to
 *     2^-14): q, k and v, the gate-scaled key and query rows, T = (I + A)^-1,
 *     W, M, the state entering each chunk and the residual U are rounded to
 *     fp16 before each product; products accumulate in fp32 and the carried
 *     state is fp32.  bf16 inputs convert to fp16 exactly within its range.
 *     fp16 rather than bf16 keeps the final-state error near 3e-4 relative
 *     (bf16 operands: about 2.4e-3).  Preconditions (not checked): v, the
 *     initial states and every state and residual the recurrence reaches stay
 *     below 65504 in magnitude (beyond it the results overflow to inf);
 *     magnitudes below 2^-14 keep fewer significant bits.  fp32 io is
 *     accepted, but its prefill results carry the same fp16-operand rounding
 *     (about 3e-4 relative on states, not fp32's 1e-7).  The decode entry
 *     points compute in fp32 throughout.
 *   - Pool slots: a real request's index must lie in [0, num_slots - 2]; the
 *     last slot is the padding sentinel that every negative index selects.
 */
#ifndef KDA_H
#define KDA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    KDA_OK = 0,
    KDA_ERR_NULL = 1,        /* a required pointer is NULL                      */
    KDA_ERR_SHAPE = 2,       /* inconsistent or non-positive sizes              */
    KDA_ERR_UNSUPPORTED = 3, /* dk/dv/dtype/gate outside the compiled set, or a
                                grid beyond the device's limits                  */
    KDA_ERR_WORKSPACE = 4,   /* workspace NULL or smaller than required          */
    KDA_ERR_ALIAS = 5,       /* an output aliases an input it must not alias     */
    KDA_ERR_HIP = 6,         /* a HIP launch or runtime call failed              */
    KDA_ERR_ALIGN = 7        /* a tensor pointer is not 16-byte aligned          */
} kda_status;

typedef enum { KDA_F32 = 0, KDA_BF16 = 1 } kda_dtype;

typedef enum {
    KDA_GATE_CHANNEL = 0, /* KDA: g [T, hv, dk], one log-decay per key channel */
    KDA_GATE_SCALAR = 1   /* GDN: g [T, hv], one log-decay per head            */
} kda_gate;

/* Host-side description of one prefill call. */
typedef struct {
    int32_t num_seqs;     /* N >= 0                                           */
    int32_t total_tokens; /* T >= 0, equals cu_seqlens[N] on the device        */
    int32_t hk, hv;       /* key heads, value heads (hv % hk == 0)             */
    int32_t dk, dv;       /* key / value head dims                             */
    int32_t io_dtype;     /* kda_dtype of q, k, v and o                        */
    int32_t state_dtype;  /* kda_dtype of initial / final states and pools     */
    int32_t gate;         /* kda_gate                                          */
    float scale;          /* read-out scale applied to o                       */
    int32_t num_slots;    /* pool rows (pool mode only; ignored in dense mode) */
} kda_prefill_desc;

/*
 * Bytes of device workspace kda_chunk_prefill needs for `desc` (0 if the
 * descriptor is invalid).  One workspace may be reused by any number of calls
 * that are ordered on one stream; two streams must not share one at a time.
 * The size grows linearly with T and N (chunk-level intermediates of the
 * method, PR 27488 digest 实现拆解: U/W and pre-scaled operands per token).
 */
size_t kda_chunk_prefill_workspace_size(const kda_prefill_desc *desc);

/*
 * Chunked prefill over packed sequences (chunk size 64): the chunk pipeline
 * of the KDA prefill digest (sglang PR 27488, 实现拆解: a per-chunk gate
 * cumsum prologue, the KKT-inverse + U/W step, the state (h) step and the
 * output (o) step, chunked over cu_seqlens; 关键源码片段: the pipeline entry
 * chunk_kda_cutedsl returns o and the final state), with the pool-state I/O
 * of the pool-mode digest (PR 30169, 实现拆解 items 1-2: initial states read
 * from and final states written to state_indices[seq] of a pool, in place).
 *   q, k        [T, hk, dk]  io dtype (callers pass L2-normalised q, k)
 *   v           [T, hv, dv]  io dtype
 *   g           [T, hv, dk] (CHANNEL) or [T, hv] (SCALAR), fp32, <= 0
 *   beta        [T, hv] fp32
 *   cu_seqlens  [N + 1] int32 (device)
 *   state       dense mode (state_indices == NULL): initial states
 *               [N, hv, dv, dk] state dtype, or NULL for zeros;
 *               pool mode: the pool [num_slots, hv, dv, dk], required.
 *   state_indices  NULL (dense mode) or [N] int32 slot per sequence; an index
 *               < 0 selects slot num_slots - 1 (sentinel).
 *   final_state dense mode: [N, hv, dv, dk] written with the final states, or
 *               NULL (not written); may equal `state` (in place).
 *               pool mode: must be NULL or equal to `state`; the final state of
 *               sequence n is written to the same pool row it was read from.
 *               Rows not indexed are neither read nor written.  With several
 *               negative indices the sentinel row's content, and the o rows of
 *               those sequences, are unspecified.
 *   o           [T, hv, dv] io dtype; must not alias any input.
 *   workspace   device buffer of at least kda_chunk_prefill_workspace_size().
 * A sequence of length 0 writes no o rows and leaves its state unchanged
 * (copied to final_state in dense mode).  Pool mode and dense mode run the
 * same kernels with the same tiling and produce bit-identical o and states.
 * Every chunk is processed as 64 tokens, so for pool-mode batches of very
 * short sequences (at most about 8 tokens each) kda_recurrent_decode_multi
 * with update_pool set and no step cache computes the same recurrence
 * faster, in fp32 (MI355X, 32 heads, K = V = 128: 4096 sequences x 4 tokens
 * 4.2 ms against 8.8 ms here, 1024 x 8 1.8 against 2.3 ms; from about 12
 * tokens this entry point is faster).
 */
kda_status kda_chunk_prefill(const kda_prefill_desc *desc,
                             const void *q, const void *k, const void *v,
                             const float *g, const float *beta,
                             const int32_t *cu_seqlens,
                             void *state, const int32_t *state_indices,
                             void *final_state, void *o,
                             void *workspace, size_t workspace_bytes,
                             void *stream);

/*
 * Chunked prefill with the gate activation fused in: instead of fp32 g and
 * beta, the raw per-token projections are passed and activated inside the
 * first kernel,
 *     g    = -exp(A_log) * softplus(gate_x + dt_bias)
 *     beta = sigmoid(beta_x)
 * (GDN pool-mode digest, sglang PR 30169, key-code test: raw a and b in bf16
 * per (token, value head), A_log and dt_bias per value head; KDA prefill
 * digest, PR 27488, key-code extend wrapper: A_log and dt_bias handed to the
 * kernel entry).
 *   gate_x   [T, hv, dk] (CHANNEL) or [T, hv] (SCALAR), io dtype
 *   A_log    [hv, dk] (CHANNEL) or [hv] (SCALAR), fp32; a per-head A_log is
 *            passed broadcast over the channels for the CHANNEL gate
 *   dt_bias  same shape as A_log, fp32
 *   beta_x   [T, hv] io dtype
 * Everything else (shapes, pool mode, aliasing, workspace, errors) is as for
 * kda_chunk_prefill, with gate_x, A_log, dt_bias and beta_x in the roles of
 * g and beta.  The activation runs in fp32: softplus through max(z, 0) plus
 * a log1p term, so no input overflows.  Not checked: inputs are finite.
 */
kda_status kda_chunk_prefill_fused_gate(const kda_prefill_desc *desc,
                                        const void *q, const void *k, const void *v,
                                        const void *gate_x, const float *A_log,
                                        const float *dt_bias, const void *beta_x,
                                        const int32_t *cu_seqlens,
                                        void *state, const int32_t *state_indices,
                                        void *final_state, void *o,
                                        void *workspace, size_t workspace_bytes,
                                        void *stream);

/*
 * Allocation-free chunked prefill, for callers that cannot allocate device
 * memory around the call: code under HIP graph capture, serving loops and
 * harnesses that forbid hipMalloc.  It is kda_chunk_prefill with the
 * workspace taken from a buffer the library holds itself: a device array of
 * KDA_SCRATCH_BYTES per GPU, placed when the library is first used on that
 * GPU and held until the process ends.  This call allocates and frees
 * nothing; its first call on a device looks the array's address up once.
 *   Limit: kda_chunk_prefill_workspace_size(desc) <= KDA_SCRATCH_BYTES,
 *   else KDA_ERR_WORKSPACE with nothing launched.  At dk = dv = 128 the
 *   workspace is about 64.5 KB per (64-token chunk, value head) plus a few
 *   bytes per sequence: e.g. 8,000 tokens of one sequence at 32 value heads.
 *   Concurrency: every call on one GPU uses that GPU's one array.  Calls
 *   ordered on one stream are safe; calls that overlap in time on one GPU
 *   (two streams, two host threads) race and give undefined results.
 *   Nothing in the array needs to start at zero: each call writes every
 *   workspace byte it later reads.
 * Arguments, layouts, pool mode and errors are those of kda_chunk_prefill.
 */
#define KDA_SCRATCH_BYTES ((size_t)256 << 20)
kda_status kda_chunk_prefill_noalloc(const kda_prefill_desc *desc,
                                     const void *q, const void *k, const void *v,
                                     const float *g, const float *beta,
                                     const int32_t *cu_seqlens,
                                     void *state, const int32_t *state_indices,
                                     void *final_state, void *o, void *stream);

/* Host-side description of one decode call. */
typedef struct {
    int32_t batch;        /* B >= 0 requests, one token each                  */
    int32_t hk, hv, dk, dv;
    int32_t io_dtype, state_dtype, gate;
    float scale;
    int32_t num_slots;    /* pool rows                                         */
} kda_decode_desc;

/*
 * One-token recurrent decode for B requests against a state pool, in place:
 * the packed KDA decode of the FLA/MoE shape-limits digest (sglang PR 37317,
 * 实现拆解 item 1: fused_recurrent_kda_packed_decode, one recurrence step per
 * request and value head, its grid split so batch and head are separate
 * axes), reading and writing pool rows by index with the padding sentinel of
 * the pool-mode digest (PR 30169, 实现拆解 item 3).
 *   q, k  [B, hk, dk] io dtype;  v [B, hv, dv] io dtype
 *   g     [B, hv, dk] (CHANNEL) or [B, hv] (SCALAR) fp32;  beta [B, hv] fp32
 *   state_pool     [num_slots, hv, dv, dk] state dtype, read and written in place
 *   state_indices  [B] int32; an index < 0 selects slot num_slots - 1 (with
 *                  several negative indices the sentinel row's content, and
 *                  the o of those requests, are unspecified)
 *   o     [B, hv, dv] io dtype
 * The launch grid is (hv x dv / tile, ceil(B / Z), Z) with Z = ceil(B / 65535):
 * head (with value tile) on x and the batch over y and z, so batch and head
 * stay on separate axes and no product of the two, nor the batch alone,
 * meets an axis limit (B up to 2^31 - 1).
 */
kda_status kda_recurrent_decode(const kda_decode_desc *desc,
                                const void *q, const void *k, const void *v,
                                const float *g, const float *beta,
                                void *state_pool, const int32_t *state_indices,
                                void *o, void *stream);

/*
 * One-token decode with the gate activation fused in, as for
 * kda_chunk_prefill_fused_gate:
 *   gate_x   [B, hv, dk] (CHANNEL) or [B, hv] (SCALAR), io dtype
 *   A_log, dt_bias  [hv, dk] (CHANNEL) or [hv] (SCALAR), fp32
 *   beta_x   [B, hv] io dtype
 * Everything else is as for kda_recurrent_decode.
 */
kda_status kda_recurrent_decode_fused_gate(const kda_decode_desc *desc,
                                           const void *q, const void *k, const void *v,
                                           const void *gate_x, const float *A_log,
                                           const float *dt_bias, const void *beta_x,
                                           void *state_pool, const int32_t *state_indices,
                                           void *o, void *stream);

/*
 * kda_recurrent_decode / kda_recurrent_decode_fused_gate with q, k and v read
 * from one packed row per request: qkv [B, 2 hk dk + hv dv] in the io dtype,
 * each row holding q [hk, dk], then k [hk, dk], then v [hv, dv] (the layout of
 * a fused q/k/v input projection; the FLA/MoE shape-limits digest, sglang
 * PR 37317, names the packed KDA decode kernel but does not print its layout,
 * so this concatenation order is a reading).  Gates, pool, indices, o and the
 * errors are as for the unpacked calls; qkv must not overlap o.
 */
kda_status kda_recurrent_decode_packed(const kda_decode_desc *desc, const void *qkv,
                                       const float *g, const float *beta,
                                       void *state_pool, const int32_t *state_indices,
                                       void *o, void *stream);
kda_status kda_recurrent_decode_packed_fused_gate(const kda_decode_desc *desc, const void *qkv,
                                                  const void *gate_x, const float *A_log,
                                                  const float *dt_bias, const void *beta_x,
                                                  void *state_pool, const int32_t *state_indices,
                                                  void *o, void *stream);

/* Host-side description of one multi-token decode call. */
typedef struct {
    int32_t batch;        /* N >= 0 requests                                   */
    int32_t total_tokens; /* T >= 0, equals cu_seqlens[N] on the device         */
    int32_t hk, hv, dk, dv;
    int32_t io_dtype, state_dtype, gate;
    float scale;
    int32_t num_slots;    /* pool rows                                          */
    int32_t cache_pitch;  /* steps per request in the intermediate-state cache,
                             or 0 for no cache                                  */
    int32_t update_pool;  /* nonzero: write each request's last state back to
                             its pool row; 0: the pool is only read             */
} kda_multi_decode_desc;

/*
 * Multi-token recurrent decode: the verify step of speculative decoding.
 * Request n runs its tokens [cu_seqlens[n], cu_seqlens[n+1]) in order from
 * the state in pool row state_indices[n] (negative: the last row), writes o
 * for every token and caches the state after its j-th token (j = 0, 1, ...)
 * at intermediate_states[n * cache_pitch + j] for j < cache_pitch, so that the
 * state at any accepted draft length can be restored.  The pitch is the step
 * count the cache was allocated with, not the current number of drafts, which
 * may change from call to call (FLA/MoE shape-limits digest, sglang PR 37317,
 * 实现拆解 item 2: the cache stride is derived from the allocation's
 * per-request pitch).
 *   q, k  [T, hk, dk] io dtype;  v [T, hv, dv] io dtype
 *   g     [T, hv, dk] (CHANNEL) or [T, hv] (SCALAR) fp32;  beta [T, hv] fp32
 *   cu_seqlens     [N + 1] int32 (device)
 *   state_pool     [num_slots, hv, dv, dk] state dtype
 *   state_indices  [N] int32 (with update_pool and several negative indices
 *                  the sentinel row's content, and the o and cached steps of
 *                  those requests, are unspecified)
 *   intermediate_states  [N, cache_pitch, hv, dv, dk] state dtype, or NULL
 *                  when cache_pitch is 0; steps at or beyond cache_pitch are
 *                  not cached; must not overlap any other argument
 *   o     [T, hv, dv] io dtype
 * The grid is (hv x dv / tile, ceil(N / Z), Z) as for kda_recurrent_decode.  A request
 * with no tokens writes nothing.  Not checked (preconditions, besides those of
 * kda_chunk_prefill): indices of requests with update_pool set are unique.
 */
kda_status kda_recurrent_decode_multi(const kda_multi_decode_desc *desc,
                                      const void *q, const void *k, const void *v,
                                      const float *g, const float *beta,
                                      const int32_t *cu_seqlens,
                                      void *state_pool, const int32_t *state_indices,
                                      void *intermediate_states, void *o, void *stream);

/* kda_recurrent_decode_multi with the gate activation fused in, as for
 * kda_chunk_prefill_fused_gate (gate_x [T, hv, dk] or [T, hv] and beta_x
 * [T, hv] in the io dtype; A_log, dt_bias [hv, dk] or [hv] fp32). */
kda_status kda_recurrent_decode_multi_fused_gate(const kda_multi_decode_desc *desc,
                                                 const void *q, const void *k, const void *v,
                                                 const void *gate_x, const float *A_log,
                                                 const float *dt_bias, const void *beta_x,
                                                 const int32_t *cu_seqlens,
                                                 void *state_pool, const int32_t *state_indices,
                                                 void *intermediate_states, void *o, void *stream);

/* Static description of a status code. */
const char *kda_status_string(kda_status status);

/* Library version, major * 10000 + minor * 100 + patch. */
int32_t kda_version(void);

#ifdef __cplusplus
}
#endif

#endif /* KDA_H */
