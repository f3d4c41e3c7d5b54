// Internal launch interface between the C ABI layer and the prefill / decode kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace kda {

struct PrepParams {
    const void* q;
    const void* k;
    const void* v;
    const void* la;
    const void* beta;
    void* ws;
    int64_t B, T, H, NC;
    int clamp;
    int qk_norm;  // q, k are raw: k / |k|, q / (|q| sqrt(D)) per token
    int logits;   // la holds forget-gate logits: log alpha = logsigmoid(la)
    // variable-length batch (chunk-64 path; NULL: B sequences of T tokens): the map of
    // kda_varlen.h.  Card of chunk j of sequence i, head h: (co_i + j) H + h; tokens are
    // rows s_i .. s_{i+1} - 1 of the packed [rows, H, D] tensors.
    const int64_t* vs;
    const int64_t* vco;
    const int32_t* vsoc;
    int64_t vN;
    int cards_ready;  // the workspace already holds these inputs' cards: no card builder
    // pipelined long sequences (chunk-64 path): ring_len > 0 builds the cards of chunks
    // [piece ring_len, (piece + 1) ring_len) into half piece % 2 of a two-piece ring,
    // card ((piece % 2) B H + unit) ring_len + j for chunk j of the piece
    int64_t ring_len;
    int64_t piece;
};

struct RecurParams {
    const void* gate;
    void* out;
    const float* s0;  // may be NULL (zeros)
    float* sT;        // may be NULL; may alias s0
    const void* ws;
    int64_t B, T, H, NC;
    // segment scan (chunk-64 bf16 path): the sequence is cut into nseg segments of
    // seg_len chunks (the last one may be shorter); sums holds, per (b, h) and per
    // segment p < nseg - 1, the zero-start end state b_p and the transition M_p
    // (fp32 [D][D] each).  nseg = 1: one pass over the whole sequence.
    int64_t seg_len;
    int nseg;
    float* sums;
    // where the summary kernel writes b_p and M_p of summarised segment u (= (b, h) *
    // (nseg - 1) + p): sum_b + u * sum_stride and sum_m + u * sum_stride.  Left NULL,
    // they follow `sums` (b_p then M_p per segment, stride 2 D^2).
    float* sum_b;
    float* sum_m;
    int64_t sum_stride;
    // variable-length batch (as in PrepParams; B = N, T unused)
    const int64_t* vs;
    const int64_t* vco;
    // block-granular state snapshots: after every snap_chunks chunks of C tokens of a
    // sequence the state goes to slot floor(s_i / (C snap_chunks)) + i + k of snap
    // [slots, H, D, D]
    float* snap;
    int64_t snap_chunks;
    // pipelined long sequences: ring_len > 0 runs piece `piece` only (chunks
    // [piece ring_len, ...)), from its half of the card ring (PrepParams), from s0 to sT
    int64_t ring_len;
    int64_t piece;
};

// bytes of one per-chunk card in the workspace (or -1 if unsupported)
int64_t prefill_card_bytes(int bf16, int C, int D);
bool prefill_supported(int bf16, int C, int D);
hipError_t launch_prefill(int bf16, int out_bf16, int C, int D, const PrepParams& pp,
                          const RecurParams& rp, hipStream_t stream);
// summary of whole sequences (NC >= 1) on either path: M [units, D, D] and b [units, D, D]
// in fp32 (the chunk-64 bf16 path below, else the general path's cards and state pass)
hipError_t launch_summary(int bf16, int C, int D, const PrepParams& pp, float* M, float* b,
                          hipStream_t stream);

// bf16 inputs, 64-token chunks (kda_chunk64.hip)
int64_t prefill64_card_bytes(int D);
// segments the chunk-64 path cuts a sequence into (1 = none); a function of the shape only
int prefill64_segments(int D, int64_t units, int64_t nc);
// workspace bytes beyond the cards: the per-segment summaries
int64_t prefill64_extra_bytes(int D, int64_t units, int64_t nc);
hipError_t launch_prefill64(int D, int out_bf16, const PrepParams& pp, const RecurParams& rp,
                            hipStream_t stream);
// summary of whole sequences (NC >= 1): cards, then one summarised segment of NC chunks
// per (b, h); M [units, D, D] and b [units, D, D] in fp32
hipError_t launch_summary64(int D, const PrepParams& pp, float* M, float* b, hipStream_t stream);

}  // namespace kda
