// Internal launch interface of the segment-summary combination (kda_segment.hip).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace kda {

struct CombineParams {
    const float* M;   // [P, units, D, D]: transition of segment p
    const float* b;   // [P, units, D, D]: zero-start end state of segment p
    const float* s0;  // [units, D, D] or NULL (zeros)
    float* seg;       // [P, units, D, D] or NULL: state entering segment p
    float* sT;        // [units, D, D] or NULL; may alias s0
    int64_t P, units;
};

// S_{p+1} = M_p S_p + b_p over p = 0..P-1, in fp32 (D = 64 or 128)
hipError_t launch_combine(int D, const CombineParams& p, hipStream_t stream);
// the summary of an empty run: M = I, b = 0 for every (b, h)
hipError_t launch_identity_summary(int D, float* M, float* b, int64_t units, hipStream_t stream);

}  // namespace kda
