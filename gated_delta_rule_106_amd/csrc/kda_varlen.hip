// Sequence map of a variable-length batch (packed tokens, one offset per sequence).
//
// The caller's offsets cu[0..N] live in device memory and are not trusted: with
// x_j = clamp(cu_j, 0, total_T), the sanitised starts are s_i = max_{j <= i} x_j, so
// every sequence is a non-negative, non-overlapping range of the packed rows and the
// chunk count stays at most ceil(total_T / C) + N whatever the offsets hold.  Then
// co_i = sum_{i' < i} ceil((s_{i'+1} - s_{i'}) / C), and every chunk g < co_N records
// its sequence.  One workgroup of 256 threads walks the entries in blocks of 256:
// thread e forms s_e (a max-scan with carry) and the chunk count of sequence e - 1
// (from s_e and its left neighbour), whose inclusive sum-scan with carry is co_e.
#include "kda_device.h"
#include "kda_varlen.h"

namespace kda {
namespace vl {

// inclusive scans over the 64 lanes of a wave
__device__ __forceinline__ int64_t wave_scan_max(int64_t x) {
    const int lane = lane_id();
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
        const int64_t y = __shfl_up(x, off);
        if (lane >= off) x = x > y ? x : y;
    }
    return x;
}
__device__ __forceinline__ int64_t wave_scan_sum(int64_t x) {
    const int lane = lane_id();
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
        const int64_t y = __shfl_up(x, off);
        if (lane >= off) x += y;
    }
    return x;
}

__global__ __launch_bounds__(256) void kda_varlen_map_kernel(VarlenMap m, const int64_t* cu, int64_t N,
                                                             int64_t total_T, int C) {
    __shared__ int64_t wmax[4], wsum[4];
    const int tid = threadIdx.x, lane = lane_id(), wave = wave_id();
    int64_t carry_s = 0;  // s of the entries before this block (s_{-1} = 0)
    int64_t carry_c = 0;  // chunks of the sequences before the first one this block counts
    for (int64_t base = 0; base <= N; base += 256) {
        const int64_t e = base + tid;
        int64_t x = -1;  // entries past N take no part in the max
        if (e <= N) {
            x = cu[e];
            x = x < 0 ? 0 : (x > total_T ? total_T : x);
        }
        const int64_t smax = wave_scan_max(x);
        if (lane == 63) wmax[wave] = smax;
        __syncthreads();
        int64_t pre = carry_s;  // s of everything before this wave's first entry
        for (int w = 0; w < wave; ++w) pre = pre > wmax[w] ? pre : wmax[w];
        const int64_t s_e = smax > pre ? smax : pre;
        int64_t prev = __shfl_up(s_e, 1);
        if (lane == 0) prev = pre;
        const int64_t nck = (e >= 1 && e <= N) ? (s_e - prev + C - 1) / C : 0;  // sequence e - 1
        const int64_t csum = wave_scan_sum(nck);
        if (lane == 63) wsum[wave] = csum;
        __syncthreads();
        int64_t cpre = carry_c;
        for (int w = 0; w < wave; ++w) cpre += wsum[w];
        const int64_t co_e = cpre + csum;  // chunks of sequences 0 .. e - 1
        if (e <= N) {
            m.s[e] = s_e;
            m.co[e] = co_e;
        }
        for (int64_t j = 0; j < nck; ++j) m.soc[co_e - nck + j] = (int32_t)(e - 1);
        int64_t ns = carry_s, nc = carry_c;
        for (int w = 0; w < 4; ++w) {
            ns = ns > wmax[w] ? ns : wmax[w];
            nc += wsum[w];
        }
        __syncthreads();  // wmax and wsum are rewritten by the next block
        carry_s = ns;
        carry_c = nc;
    }
}

}  // namespace vl

hipError_t launch_varlen_map(const VarlenMap& m, const int64_t* cu, int64_t N, int64_t total_T, int C,
                             hipStream_t stream) {
    hipLaunchKernelGGL(vl::kda_varlen_map_kernel, dim3(1), dim3(256), 0, stream, m, cu, N, total_T, C);
    return hipGetLastError();
}

}  // namespace kda
