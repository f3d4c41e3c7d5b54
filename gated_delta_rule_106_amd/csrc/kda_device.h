// Device-side building blocks shared by the KDA kernels (gfx950 / CDNA4).
//
// MFMA lane layouts used throughout (wave64, lane l, row-of-16 m = l % 16,
// lane group g = l / 16):
//   v_mfma_f32_16x16x32_{f16,bf16}: A[m][8g + j], B[8g + j][m], j = 0..7
//   v_mfma_f32_16x16x16_f16       : A[m][4g + j], B[4g + j][m], j = 0..3
//   v_mfma_f32_16x16x4_f32        : A[m][g],      B[g][m]
//   accumulator (all of the above): acc[i] = D[4g + i][m], i = 0..3
// Because a contraction may visit its K index in any order as long as both
// operands agree, a 16x16 accumulator tile (rows 4g..4g+3 held by lane group
// g) can feed the next MFMA as its K-major operand directly: two stacked tiles
// form one K = 32 step whose logical k = 8g + j maps to physical row
// 4g + j (j < 4, first tile) or 16 + 4g + (j - 4) (second tile).  The other
// operand is then read with the same permutation.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace kda {

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef _Float16 half4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float floatx4 __attribute__((ext_vector_type(4)));

constexpr float kLog2e = 1.4426950408889634f;
// ln(0.0067): the per-step retention floor, in natural-log units.
constexpr float kLogAlphaMin = -5.005647752585217f;

__device__ __forceinline__ int lane_id() { return threadIdx.x & 63; }
__device__ __forceinline__ int wave_id() { return threadIdx.x >> 6; }

// exp2 on the hardware transcendental unit (v_exp_f32).
__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

__device__ __forceinline__ float bf16_bits_to_float(uint16_t u) {
    return __uint_as_float(static_cast<uint32_t>(u) << 16);
}

// Input element loaders: the public dtypes are fp32 and bf16 (raw 16-bit words).
struct InF32 {
    using raw_t = float;
    static __device__ __forceinline__ float load(const raw_t* p, int64_t i) { return p[i]; }
    static __device__ __forceinline__ raw_t from_float(float x) { return x; }
};
struct InBF16 {
    using raw_t = uint16_t;
    static __device__ __forceinline__ float load(const raw_t* p, int64_t i) {
        return bf16_bits_to_float(p[i]);
    }
    static __device__ __forceinline__ raw_t from_float(float x) {
        __bf16 h = static_cast<__bf16>(x);  // round to nearest even
        return __builtin_bit_cast(uint16_t, h);
    }
};

__device__ __forceinline__ floatx4 zero4() { return floatx4{0.f, 0.f, 0.f, 0.f}; }

__device__ __forceinline__ floatx4 mma_f16_k32(const half8& a, const half8& b, floatx4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ floatx4 mma_f16_k16(const half4& a, const half4& b, floatx4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x16f16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ floatx4 mma_bf16_k32(const bf16x8& a, const bf16x8& b, floatx4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ floatx4 mma_f32_k4(float a, float b, floatx4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ void wait_vm_zero() { __builtin_amdgcn_s_waitcnt(0x0F70); }   // vmcnt(0)
__device__ __forceinline__ void wait_lgkm_zero() { __builtin_amdgcn_s_waitcnt(0xC07F); } // lgkmcnt(0)
// workgroup barrier without the implicit memory fence of __syncthreads():
// each wave waits explicitly for exactly what the next phase needs
__device__ __forceinline__ void bare_barrier() {
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}
// barrier that orders LDS only: global loads and stores issued before it stay in flight
__device__ __forceinline__ void lds_barrier() {
    wait_lgkm_zero();
    bare_barrier();
}

// Split x into bf16 hi + lo with x ~= hi + lo to about 16 significant bits.
__device__ __forceinline__ void split_bf16(float x, __bf16& hi, __bf16& lo) {
    hi = static_cast<__bf16>(x);
    lo = static_cast<__bf16>(x - static_cast<float>(hi));
}

// logistic sigmoid with the hardware exp2 and reciprocal (v_rcp_f32, about 1 ulp)
__device__ __forceinline__ float sigmoidf_(float z) {
    return __builtin_amdgcn_rcpf(1.0f + fast_exp2(-z * kLog2e));
}

// Clamp of log(alpha) to [ln 0.0067, 0] (retention floor and retention <= 1).
__device__ __forceinline__ float clamp_log_alpha(float l, bool clamp) {
    return clamp ? fminf(fmaxf(l, kLogAlphaMin), 0.0f) : l;
}

// log(1 + e) for e in [0, 1] by Kahan's correction (D. Goldberg, "What every computer
// scientist should know about floating-point arithmetic", 1991, Theorem 4): with
// u = fl(1 + e), log1p(e) = e when u == 1, else log(u) * e / (u - 1), which cancels the
// rounding of 1 + e.  log(u) from the hardware log2 (v_log_f32).
__device__ __forceinline__ float log1p_unit(float e) {
    const float u = 1.0f + e;
    const float d = u - 1.0f;
    const float l = __builtin_amdgcn_logf(u) * 0.6931471805599453f;  // ln(u)
    return d == 0.0f ? e : l * (e * __builtin_amdgcn_rcpf(d));
}

// log(sigmoid(x)) = min(x, 0) - log(1 + e^-|x|): the log retention of a forget-gate
// logit x, finite for every finite x, 0 at x = +inf; the small decays of large logits
// (about -e^-x) keep their relative accuracy.
__device__ __forceinline__ float log_sigmoid(float x) {
    return fminf(x, 0.0f) - log1p_unit(fast_exp2(-fabsf(x) * kLog2e));
}

// log(alpha) from the log_alpha input: the value itself or, for forget-gate logits,
// its log-sigmoid; then the clamp.
__device__ __forceinline__ float log_alpha_in(float x, bool logits, bool clamp) {
    return clamp_log_alpha(logits ? log_sigmoid(x) : x, clamp);
}

// 1 / max(sqrt(ss), 1e-12): the L2 normalisation factor of a vector with squared norm ss
__device__ __forceinline__ float inv_norm(float ss) { return rsqrtf(fmaxf(ss, 1e-24f)); }

}  // namespace kda
