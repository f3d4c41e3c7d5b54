/*
 * kda.h -- C ABI of the MI355X (gfx950) Kimi Delta Attention (KDA) token mixer.
 *
 * What is computed (page "3T models are no longer magic", affta.cn/jrzx/86753.html,
 * section "Gate 1: KDA makes it computable"): for every (batch b, head h) a
 * fixed-size d_k x d_v fp32 state S is carried over the tokens.  Each token
 *   1. forgets channel-wise:      S <- Diag(alpha_t) S, alpha_t = exp(log_alpha_t),
 *                                 with per-step retention floored at 0.67 %
 *                                 (log_alpha clamped to [ln 0.0067, 0]);
 *   2. writes with the delta rule: u_t = beta_t (v_t - S^T k_t),  S <- S + k_t u_t^T,
 *                                 i.e. S_t = (I - beta_t k_t k_t^T) Diag(alpha_t) S_{t-1}
 *                                           + beta_t k_t v_t^T;
 *   3. reads the new state:        o_t = S_t^T q_t;
 *   4. gates the read-out:         y_t = o_t * sigmoid(z_t), channel by channel.
 * The rows of S are key channels (d_k), the columns value channels (d_v).
 *
 * kda_chunk_fwd evaluates this over whole sequences in the chunkwise-parallel
 * form (page "Kimi K3 report walk-through", prism.simon-ai.net/article/6740,
 * sections "Compute paradigm" and "Hierarchical chunking of linear attention":
 * parallel inside a chunk, recurrent across chunks, with the result independent
 * of the chunk size; decay factors are kept inside the BF16 range by 16-token
 * tiles, section "Numerical stability & co-design").  kda_decode_step performs
 * one recurrent token step on a stored state.
 *
 * Conventions shared by every entry point
 *  - Tensors are dense, row-major, device-resident and 16-byte aligned.
 *  - Token tensors are token-major: q, k, log_alpha [B, T, H, Dk];
 *    v, gate, out [B, T, H, Dv]; beta [B, T, H] (decode: the same without T).
 *  - dtype applies to q, k, v, log_alpha, beta and gate (all the same type);
 *    out_dtype selects the type of out independently (KDA_F32 = 0 is the
 *    zero-initialised default).  With bf16 inputs an fp32 output is what
 *    meets a max-abs error of 2e-2 of the output RMS: rounding even the exact
 *    result to bf16 already costs about 2.8e-2 on these outputs, whose peaks
 *    are ~10x their RMS.  States are always fp32 [B, H, Dk, Dv].
 *  - Supported head sizes: Dk == Dv, 64 or 128.
 *  - The caller owns every buffer.  The library allocates nothing, keeps no
 *    global mutable state and is reentrant; calls on distinct streams may run
 *    concurrently.  The one exception is kda_chunk_fwd_noalloc, whose fixed
 *    per-device scratch buffer is shared by all its calls (see there).  Work is enqueued on `stream` and the call returns without
 *    synchronising; results are valid once the stream has completed.
 *  - Arguments are validated on the host before any HIP call; on failure the
 *    call returns a negative status and touches no memory.  A launch error
 *    reported by the runtime returns KDA_ERR_HIP.  The library never aborts,
 *    prints or throws.
 *  - Non-finite inputs are not checked for; they propagate.
 *  - Value range of the bf16 chunk-64 path (kda_chunk_fwd with bf16 inputs and
 *    chunk 0 or 64, kda_chunk_fwd_varlen, kda_chunk_summary): v, the chunk's
 *    corrected values U = beta (v - S^T k) and fp16 copies of the state are
 *    MFMA operands in fp16, so every |v|, every state entry (initial state
 *    included) and every |U| must stay below 65504; results beyond that are
 *    not defined (inf or NaN).  fp32 inputs and the bf16 chunk 16 / 32 path
 *    carry fp32 ranges.
 *  - With KDA_FLAG_NO_CLAMP, log_alpha may lie below ln 0.0067 down to about
 *    -11 per token (retention e^-11): inside a 16-token tile, the decay over
 *    any eight consecutive tokens must stay above e^-88 (the fp32 range of the
 *    tile-relative factors).  With the clamp every tile stays within e^-80.1.
 */
#ifndef KDA_H
#define KDA_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

#define KDA_VERSION 5

/* element types */
#define KDA_F32 0  /* IEEE binary32 */
#define KDA_BF16 1 /* bfloat16 */

/* status codes */
#define KDA_OK 0
#define KDA_ERR_NULL (-1)        /* a required pointer is NULL */
#define KDA_ERR_SHAPE (-2)       /* negative or overflowing sizes */
#define KDA_ERR_UNSUPPORTED (-3) /* head size, dtype, chunk or flag not supported */
#define KDA_ERR_WORKSPACE (-4)   /* workspace missing or too small */
#define KDA_ERR_ALIGN (-5)       /* a pointer is not 16-byte aligned */
#define KDA_ERR_HIP (-6)         /* the HIP runtime reported a launch error */
#define KDA_ERR_TOO_LARGE (-7)   /* needs more scratch than kda_chunk_fwd_noalloc's fixed buffer */

/* flags */
#define KDA_FLAG_NO_CLAMP 1u /* use log_alpha as given (no clamp to [ln 0.0067, 0]); range above */
/* One sequential pass per (b, h) even where the segment scan would be used (see
 * kda_chunk_fwd).  The result is the same up to rounding; the flag exists for
 * comparisons. */
#define KDA_FLAG_NO_SEGMENT_SCAN 2u
/* Fused preprocessing (page "3T models are no longer magic", section "FlashKDA":
 * the preparation step includes the forget-gate computation and Q and K
 * normalisation), accepted by kda_chunk_fwd, kda_chunk_summary and
 * kda_decode_step:
 *  KDA_FLAG_QK_L2NORM: q and k are raw projections; every token's k is divided
 *    by its L2 norm and q by its L2 norm times sqrt(Dk) (norms below 1e-12
 *    count as 1e-12), computed in fp32 from the given values.
 *  KDA_FLAG_GATE_LOGITS: log_alpha holds forget-gate logits x; the log
 *    retention is logsigmoid(x) = -log(1 + e^-x), then clamped as usual (so
 *    log alpha = max(logsigmoid(x), ln 0.0067) by default). */
#define KDA_FLAG_QK_L2NORM 4u
#define KDA_FLAG_GATE_LOGITS 8u
/* kda_chunk_fwd only (bf16 inputs, chunk 64): the workspace already holds the
 * per-chunk cards of exactly these q, k, v, log_alpha, beta, sizes and
 * preparation flags, written by a kda_chunk_summary call that was given q (or by
 * an earlier kda_chunk_fwd); the card builder is skipped.  Context-parallel use:
 * summarise a segment, combine, then re-run it from its incoming state without
 * building its cards twice.  Stale or foreign workspace contents give wrong
 * results; they are not detected. */
#define KDA_FLAG_CARDS_READY 16u

/*
 * Arguments of kda_chunk_fwd.
 *   chunk: tokens per chunk; 0 selects the default (64 for bf16 inputs, 16 for
 *     fp32 inputs); otherwise 16, 32 or 64 (fp32 inputs with Dk = 128 allow 16
 *     and 32).  The result does not depend on it beyond rounding.
 *   initial_state: fp32 [B, H, Dk, Dv] or NULL (zeros).
 *   final_state:   fp32 [B, H, Dk, Dv] or NULL (not returned).  It may alias
 *     initial_state (in-place continuation).
 *   workspace: device scratch of at least kda_chunk_fwd_workspace_size()
 *     bytes (may be NULL when that size is 0).  Its contents on entry do not
 *     matter and on return are unspecified.
 *   Segment scan (bf16 inputs, chunk 64): when B*H is small against the GPU and
 *   the sequence is long, each (b, h) sequence is cut into P segments (P is a
 *   function of B*H, T and Dk only).  A first kernel summarises every segment but
 *   the last as the affine map it applies to the incoming state (page "Kimi K3
 *   report walk-through", section "KDA Context Parallelism": the state a zero
 *   start ends in, and the product of the per-token transitions); the state pass
 *   then runs all segments at once, each from the exact incoming state that the
 *   ordered combination of the summaries gives.  The workspace then also holds
 *   the summaries (2 * Dk * Dv * 4 bytes per (b, h) and summarised segment).
 *   T may be any value >= 0; a last partial chunk is handled exactly.  For
 *   T == 0 nothing is written to out and final_state receives initial_state
 *   (or zeros).
 */
typedef struct kda_fwd_args {
    int64_t B, T, H, Dk, Dv;
    int32_t dtype;     /* KDA_F32 or KDA_BF16: q, k, v, log_alpha, beta, gate */
    int32_t out_dtype; /* KDA_F32 or KDA_BF16: out */
    int32_t chunk;
    uint32_t flags;
    const void *q;
    const void *k;
    const void *v;
    const void *log_alpha;
    const void *beta;
    const void *gate; /* output-gate logits; sigmoid is applied inside */
    void *out;
    const float *initial_state;
    float *final_state;
    void *workspace;
    size_t workspace_bytes;
} kda_fwd_args;

/*
 * Host-only query: bytes of device workspace kda_chunk_fwd needs for these
 * sizes, dtype and chunk (pointers in *a are not inspected).  Returns a status.
 */
int kda_chunk_fwd_workspace_size(const kda_fwd_args *a, size_t *bytes);

/* Chunkwise-parallel forward over whole sequences (prefill).  Returns a status. */
int kda_chunk_fwd(const kda_fwd_args *a, hipStream_t stream);

/*
 * kda_chunk_fwd without a caller workspace, for callers that cannot allocate
 * device memory: code recorded under HIP graph capture, tight serving loops and
 * harnesses that forbid allocation.  Same arguments, kernels and result as
 * kda_chunk_fwd, except that a->workspace and a->workspace_bytes are ignored:
 * the per-chunk cards (and segment summaries) go to a fixed scratch array of
 * KDA_NOALLOC_SCRATCH_BYTES that the library's device code holds on every
 * device it runs on, from the loading of that code until the process ends.
 *   - A call whose kda_chunk_fwd_workspace_size() exceeds
 *     KDA_NOALLOC_SCRATCH_BYTES returns KDA_ERR_TOO_LARGE before any HIP call
 *     (at Dk = 128, bf16, chunk 64: up to 814 (b, h, chunk) cards, e.g.
 *     B1 H8 T4096 fits; one card is 82 432 bytes).
 *   - KDA_FLAG_CARDS_READY returns KDA_ERR_UNSUPPORTED.
 *   - The first call on a device looks up the array's address on that device
 *     (hipGetSymbolAddress) and keeps it; `stream` must belong to the calling
 *     thread's current device (KDA_ERR_UNSUPPORTED otherwise).  No call
 *     allocates or frees memory.
 *   - Every call on one device shares the one array: calls that can overlap
 *     on one device (other streams, other threads) race and give wrong
 *     results.  Serialise them, e.g. on one stream.  Nothing in the array
 *     needs to start at zero; it keeps the last call's cards.
 */
#define KDA_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)
int kda_chunk_fwd_noalloc(const kda_fwd_args *a, hipStream_t stream);

/*
 * Variable-length batch with block-granular state snapshots.  N independent
 * sequences are packed along the rows of [rows, H, D] tensors (for q, k, v,
 * log_alpha, gate, out; beta is [rows, H]); sequence i is rows
 * cu_seqlens[i] .. cu_seqlens[i+1] - 1.  Page "Kimi K3 report walk-through",
 * section on RL infrastructure and the prefix-cache trade-off of linear
 * attention: storing the state after every token gives up the linear cost, not
 * storing it rules out reusing a cached prefix, so the state is kept at block
 * granularity.  With snapshot_every = P > 0 the state after every P tokens of a
 * sequence (the state a continuation from that token would start with) is
 * written to snapshots.
 *   cu_seqlens: int64 [N + 1] in device memory, non-decreasing from 0 to at most
 *     rows.  Offsets that break this are not an error: they are read as
 *     s_i = max_{j <= i} clamp(cu_seqlens[j], 0, rows), and sequence i is rows
 *     s_i .. s_{i+1} - 1 (so nothing outside the tensors is ever touched).  Rows
 *     outside [s_0, s_N) are not read, and out is not written there.
 *   initial_state / final_state: fp32 [N, H, Dk, Dv] or NULL, as in kda_chunk_fwd
 *     (final_state may alias initial_state).
 *   snapshot_every: 0 (none) or a positive multiple of 64.  snapshots: fp32
 *     [rows / snapshot_every + N, H, Dk, Dv], required when snapshot_every > 0:
 *     the k-th snapshot of sequence i (after (k + 1) * snapshot_every of its
 *     tokens, k < len_i / snapshot_every) is slot
 *     s_i / snapshot_every + i + k (integer division).  Other slots are not written.
 *   Supported: fp32 or bf16 inputs, the chunk sizes kda_chunk_fwd takes for that
 *   dtype and head size (0 picks the same default), Dk == Dv in {64, 128}; flags as
 *   in kda_chunk_fwd (KDA_FLAG_NO_SEGMENT_SCAN has no effect: no segments here).
 *   Every sequence starts its own chunks.  The workspace size comes from
 *   kda_chunk_fwd_varlen_workspace_size() (it depends on N, rows, H, Dk, dtype and
 *   chunk only).
 * The packed layout with cu_seqlens[i] = i T is the memory of a [N, T, H, D]
 * batch, so this also adds snapshots to ordinary batches.
 */
typedef struct kda_varlen_args {
    int64_t N, rows, H, Dk, Dv;
    int32_t dtype;
    int32_t out_dtype;
    int32_t chunk;
    uint32_t flags;
    const int64_t *cu_seqlens;
    const void *q;
    const void *k;
    const void *v;
    const void *log_alpha;
    const void *beta;
    const void *gate;
    void *out;
    const float *initial_state;
    float *final_state;
    int64_t snapshot_every;
    float *snapshots;
    void *workspace;
    size_t workspace_bytes;
} kda_varlen_args;

int kda_chunk_fwd_varlen_workspace_size(const kda_varlen_args *a, size_t *bytes);
int kda_chunk_fwd_varlen(const kda_varlen_args *a, hipStream_t stream);

/*
 * Segment summary of whole sequences.  Page "3T models are no longer magic",
 * section "KDA context parallelism", and page "Kimi K3 report walk-through",
 * section "KDA Context Parallelism": a run of tokens is summarised by how it
 * transforms the state it receives and by the state it produces from a zero
 * start, so that runs computed apart (on other devices, or as segments of one
 * long sequence) can be chained afterwards.  For every (b, h) the T tokens map
 * an incoming state S_0 to
 *     S_T = M S_0 + b,   M = A_T ... A_1,   A_t = (I - beta_t k_t k_t^T) Diag(alpha_t),
 * with b the state reached from S_0 = 0.
 *   Reads k, v, log_alpha, beta and the clamp flag of *a; gate, out and
 *   initial_state are not read and may be NULL.  q may be NULL; when it is
 *   given, the cards left in the workspace are complete, and a following
 *   kda_chunk_fwd over the same inputs can take them with KDA_FLAG_CARDS_READY.
 *   transition: fp32 [B, H, Dk, Dk], receives M (required).
 *   a->final_state: fp32 [B, H, Dk, Dv], receives b (required).
 *   The two outputs must not overlap each other, the inputs or the workspace.
 *   Supported: the dtypes, chunk sizes and head sizes of kda_chunk_fwd (Dk == Dv);
 *   KDA_FLAG_NO_CLAMP, KDA_FLAG_QK_L2NORM and KDA_FLAG_GATE_LOGITS apply as in
 *   kda_chunk_fwd, KDA_FLAG_NO_SEGMENT_SCAN and KDA_FLAG_CARDS_READY return
 *   KDA_ERR_UNSUPPORTED.  The workspace that kda_chunk_fwd_workspace_size() reports
 *   for the same *a is sufficient.  Cards left for a KDA_FLAG_CARDS_READY re-run:
 *   bf16 inputs with chunk 64 only.
 *   T == 0 gives M = I and b = 0.  M and b are accumulated in fp32, from the MFMA
 *   operands of the path the inputs take (fp16 for bf16 inputs, fp32 for fp32
 *   inputs), like the state of kda_chunk_fwd.
 */
int kda_chunk_summary(const kda_fwd_args *a, float *transition, hipStream_t stream);

/*
 * Ordered combination of P consecutive segment summaries (same pages and
 * sections): the state entering segment p + 1 is S_{p+1} = M_p S_p + b_p, with
 * S_0 the state entering segment 0.  Computed in fp32 (fp32 MFMA).
 *   transition: fp32 [P, B, H, Dk, Dk] (M_p); offset: fp32 [P, B, H, Dk, Dv] (b_p);
 *     both required when P > 0.
 *   initial_state: fp32 [B, H, Dk, Dv] or NULL (zeros).
 *   segment_states: fp32 [P, B, H, Dk, Dv] or NULL; receives S_0 .. S_{P-1}, the
 *     state each segment starts from (to re-run it with kda_chunk_fwd).
 *   final_state: fp32 [B, H, Dk, Dv] or NULL; receives S_P.  It may alias
 *     initial_state; no other output may overlap an input.
 *   Dk == Dv in {64, 128}.  P == 0 copies initial_state (or zeros) to
 *   final_state.
 */
typedef struct kda_combine_args {
    int64_t P, B, H, Dk, Dv;
    const float *transition;
    const float *offset;
    const float *initial_state;
    float *segment_states;
    float *final_state;
} kda_combine_args;

int kda_combine_states(const kda_combine_args *a, hipStream_t stream);

/*
 * Arguments of kda_chunk_bwd: the gradients of a scalar loss
 *   L = sum(d_out * out) + sum(d_final_state * S_T)
 * through the forward that kda_chunk_fwd computes (fp32 out, the same flags),
 * with respect to every input as passed: with KDA_FLAG_QK_L2NORM the gradients
 * of the raw q and k (through the per-token normalisation), with
 * KDA_FLAG_GATE_LOGITS that of the forget-gate logits (through logsigmoid).  The reverse mode of the per-token step
 * (page "3T models are no longer magic", section "Gate 1: KDA makes it
 * computable") is taken over the chunk-recurrent form (page "Kimi K3 report
 * walk-through", section "Compute paradigm") with 64-token chunks.
 *   q, k, v, log_alpha, beta, gate: the forward's inputs, laid out as in
 *     kda_fwd_args, all of `dtype`.
 *   d_out: [B, T, H, Dv] of `dtype`, the gradient of L with respect to out.
 *   initial_state: fp32 [B, H, Dk, Dv] or NULL (zeros), as in the forward.
 *   d_final_state: fp32 [B, H, Dk, Dv] or NULL (zeros).
 *   dq, dk, dlog_alpha: fp32 [B, T, H, Dk]; dv, dgate: fp32 [B, T, H, Dv];
 *   dbeta: fp32 [B, T, H]; all required when B*T*H > 0.  dlog_alpha is zero
 *     where the clamp of log alpha is active (its value, after logsigmoid for
 *     logits, outside [ln 0.0067, 0]).
 *   d_initial_state: fp32 [B, H, Dk, Dv] or NULL (not returned).
 *   flags: KDA_FLAG_NO_CLAMP, KDA_FLAG_QK_L2NORM, KDA_FLAG_GATE_LOGITS; other
 *     bits give KDA_ERR_UNSUPPORTED.
 *   workspace: at least kda_chunk_bwd_workspace_size bytes, 256-byte aligned.
 *     Per (b, h, 64-token chunk) it holds, in fp32 and each section rounded up
 *     to 256 bytes: a record for the state sweeps (3*64*Dk + Dk*Dv + Dk
 *     floats), a record for the gradient kernel (64*Dk + 3*64*64 floats), the
 *     state at the chunk's start and its gradient at the chunk's end (Dk*Dv
 *     floats each): 368.5 KiB per chunk at Dk = Dv = 128, e.g. 184.3 MiB for
 *     B1 H8 T4096.
 * No output may overlap an input or another output.
 */
typedef struct kda_bwd_args {
    int64_t B, T, H, Dk, Dv;
    int32_t dtype;  /* q, k, v, log_alpha, beta, gate, d_out */
    uint32_t flags;
    const void *q;
    const void *k;
    const void *v;
    const void *log_alpha;
    const void *beta;
    const void *gate;
    const void *d_out;
    const float *initial_state;
    const float *d_final_state;
    float *dq;
    float *dk;
    float *dv;
    float *dlog_alpha;
    float *dbeta;
    float *dgate;
    float *d_initial_state;
    void *workspace;
    size_t workspace_bytes;
} kda_bwd_args;

/* Workspace bytes kda_chunk_bwd needs for these sizes (host only).  Returns a status. */
int kda_chunk_bwd_workspace_size(const kda_bwd_args *a, size_t *bytes);
/* Chunkwise backward pass.  Returns a status. */
int kda_chunk_bwd(const kda_bwd_args *a, hipStream_t stream);

/*
 * Backward pass of a variable-length batch: the gradients of
 *   L = sum(d_out * out) + sum_i sum(d_final_state[i] * S_T(i))
 * through what kda_chunk_fwd_varlen computes (fp32 out, the same flags), for N
 * independent sequences packed along the rows (the layout, cu_seqlens and its
 * sanitising as in kda_varlen_args; the per-sequence reverse mode as in
 * kda_chunk_bwd: page "3T models are no longer magic", section "Gate 1: KDA makes
 * it computable", over the chunk-recurrent form of page "Kimi K3 report
 * walk-through", section "Compute paradigm").  Every sequence starts its own
 * chunks, so no chunk spans two sequences.
 *   q, k, v, log_alpha, beta, gate, d_out: [rows, H, D] ([rows, H] for beta), all of
 *     `dtype` (fp32 or bf16).
 *   initial_state, d_final_state: fp32 [N, H, Dk, Dv] or NULL (zeros).
 *   dq, dk, dlog_alpha: fp32 [rows, H, Dk]; dv, dgate: fp32 [rows, H, Dv]; dbeta:
 *     fp32 [rows, H]; all required when rows * H > 0.  Rows outside the sanitised
 *     sequences are not written.
 *   d_initial_state: fp32 [N, H, Dk, Dv] or NULL (not returned).  An empty sequence
 *     passes d_final_state through unchanged.
 *   flags: as in kda_chunk_bwd.  Dk == Dv in {64, 128}.
 *   workspace: at least kda_chunk_bwd_varlen_workspace_size bytes (a function of N,
 *     rows, H and Dk), 256-byte aligned: kda_chunk_bwd's per-chunk sections for
 *     ceil(rows / 64) + N chunks per head, then the sequence map.
 * No output may overlap an input or another output.
 */
typedef struct kda_bwd_varlen_args {
    int64_t N, rows, H, Dk, Dv;
    int32_t dtype;  /* q, k, v, log_alpha, beta, gate, d_out */
    uint32_t flags;
    const int64_t *cu_seqlens;
    const void *q;
    const void *k;
    const void *v;
    const void *log_alpha;
    const void *beta;
    const void *gate;
    const void *d_out;
    const float *initial_state;
    const float *d_final_state;
    float *dq;
    float *dk;
    float *dv;
    float *dlog_alpha;
    float *dbeta;
    float *dgate;
    float *d_initial_state;
    void *workspace;
    size_t workspace_bytes;
} kda_bwd_varlen_args;

/* Workspace bytes kda_chunk_bwd_varlen needs (host only).  Returns a status. */
int kda_chunk_bwd_varlen_workspace_size(const kda_bwd_varlen_args *a, size_t *bytes);
/* Backward pass of a variable-length batch.  Returns a status. */
int kda_chunk_bwd_varlen(const kda_bwd_varlen_args *a, hipStream_t stream);

/*
 * Arguments of kda_decode_step: one token per (b, h).
 *   q, k, log_alpha: [B, H, Dk]; v, gate, out: [B, H, Dv]; beta: [B, H];
 *   state: fp32 [B, H, Dk, Dv], required, read and overwritten in place with
 *   the state after this token (same layout as kda_fwd_args' states, so a
 *   prefill's final state continues directly into decode).
 */
typedef struct kda_decode_args {
    int64_t B, H, Dk, Dv;
    int32_t dtype;     /* inputs */
    int32_t out_dtype; /* out */
    uint32_t flags;
    uint32_t reserved; /* must be 0 */
    const void *q;
    const void *k;
    const void *v;
    const void *log_alpha;
    const void *beta;
    const void *gate;
    void *out;
    float *state;
} kda_decode_args;

/* Single-token recurrent step, state updated in place.  Returns a status. */
int kda_decode_step(const kda_decode_args *a, hipStream_t stream);

/* Static description of a status code (never NULL). */
const char *kda_status_str(int status);

/* KDA_VERSION of the built library. */
int kda_version(void);

#ifdef __cplusplus
}
#endif

#endif /* KDA_H */
