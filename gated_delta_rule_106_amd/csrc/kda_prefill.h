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
};

struct RecurParams {
    const void* gate;
    void* out;
    const float* s0;  // may be NULL (zeros)
    float* sT;        // may be NULL; may alias s0
    const void* ws;
    int64_t B, T, H, NC;
};

// bytes of one per-chunk card in the workspace (or -1 if unsupported)
int64_t prefill_card_bytes(int bf16, int C, int D);
bool prefill_supported(int bf16, int C, int D);
hipError_t launch_prefill(int bf16, int out_bf16, int C, int D, const PrepParams& pp,
                          const RecurParams& rp, hipStream_t stream);

// bf16 inputs, 64-token chunks (kda_chunk64.hip)
int64_t prefill64_card_bytes(int D);
hipError_t launch_prefill64(int D, int out_bf16, const PrepParams& pp, const RecurParams& rp,
                            hipStream_t stream);

}  // namespace kda
