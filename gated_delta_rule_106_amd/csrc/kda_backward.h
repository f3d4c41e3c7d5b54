// Internal launch interface of the chunkwise backward pass (fp32 arithmetic).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace kda {

struct BwdParams {
    const void* q;
    const void* k;
    const void* v;
    const void* la;
    const void* beta;
    const void* gate;
    const void* dy;
    const float* s0;   // initial state [B, H, D, D] or null (zeros)
    const float* dsT;  // gradient of the final state or null (zeros)
    float* dq;
    float* dk;
    float* dv;
    float* dla;
    float* dbeta;
    float* dgate;
    float* ds0;        // gradient of the initial state or null
    float* trans;      // per chunk: W, K-bar, b, R, Gamma_C (the sweep's record)
    float* pairs;      // per chunk: g, Li, P, Bm (the gradient kernel's record)
    float* states;     // per chunk: the state at the chunk's start
    float* dstates;    // per chunk: the gradient of the state at the chunk's end
    int64_t B, T, H;
    int64_t NC;        // chunks per sequence (variable-length: the most the offsets can give)
    // variable-length batch (NULL: B sequences of T tokens): the sequence map of
    // kda_varlen.h, B = N sequences over T packed rows.  Chunk n of sequence i, head h
    // is item (co_i + n) H + h of the per-chunk sections; NC H items in all.
    const int64_t* vs;
    const int64_t* vco;
    const int32_t* vsoc;
    int clamp;
    int qk_norm;       // q, k are raw: the gradients are taken through k / |k|, q / (|q| sqrt(D))
    int logits;        // la holds forget-gate logits: log alpha = logsigmoid(la)
};

// Workspace bytes of one call (sections: trans, pairs, states, dstates).
int64_t bwd_workspace_bytes(int D, int64_t bh, int64_t nc);
// Splits the workspace into its sections.
void bwd_layout(int D, int64_t bh, int64_t nc, void* ws, BwdParams& p);
hipError_t launch_bwd(int dtype_bf16, int D, const BwdParams& p, hipStream_t stream);

}  // namespace kda
