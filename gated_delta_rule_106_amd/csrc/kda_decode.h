// Internal launch interface of the decode step.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace kda {

struct DecodeParams {
    const void* q;
    const void* k;
    const void* v;
    const void* la;
    const void* beta;
    const void* gate;
    void* out;
    float* state;
    int64_t units;  // B * H
    int clamp;
    int qk_norm;  // q, k are raw: k / |k|, q / (|q| sqrt(D))
    int logits;   // la holds forget-gate logits: log alpha = logsigmoid(la)
};

hipError_t launch_decode(int dtype_bf16, int out_bf16, int D, const DecodeParams& p,
                         hipStream_t stream);

}  // namespace kda
