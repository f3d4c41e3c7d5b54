// Internal interface of the variable-length sequence map (kda_varlen.hip).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace kda {

// Built on the device from the caller's offsets, in the workspace.
struct VarlenMap {
    int64_t* s;    // [N + 1] sanitised starts: sequence i is rows [s_i, s_{i+1})
    int64_t* co;   // [N + 1] chunk offsets: sequence i owns chunks [co_i, co_{i+1})
    int32_t* soc;  // [max chunks] sequence of every chunk g < co_N
};

// chunks a batch of N sequences over total_T rows can need, whatever the offsets
inline int64_t varlen_max_chunks(int64_t N, int64_t total_T, int C) { return (total_T + C - 1) / C + N; }

hipError_t launch_varlen_map(const VarlenMap& m, const int64_t* cu, int64_t N, int64_t total_T, int C,
                             hipStream_t stream);

}  // namespace kda
