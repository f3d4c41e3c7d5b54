// Ordered combination of segment summaries on gfx950.
//
// Page "Kimi K3 report walk-through", section "KDA Context Parallelism" (and page
// "3T models are no longer magic", section "KDA context parallelism"): a segment of
// tokens acts on the state it receives as an affine map S -> M S + b, so once every
// segment has been summarised, the state entering segment p + 1 follows from the one
// entering segment p as S_{p+1} = M_p S_p + b_p.  This is the only sequential step
// between segments; it costs one D x D by D x D product per segment and (b, h),
// independent of the segment lengths.
//
// One workgroup per ((b, h), 16-column tile of the state): the tile (D x 16 fp32)
// stays in LDS across the segments, transposed (one row per column, so that an MFMA's B
// operand and a lane's four result rows are 16-byte accesses), in two buffers (read one,
// write the other: one barrier per segment); D / 16 waves each own one block of 16 rows and
// form it with the fp32 MFMA (v_mfma_f32_16x16x4_f32) from its rows of M_p (held in
// registers as float4 A operands) and b_p (the starting accumulator).  Three register
// sets rotate: the rows of M_{p+1} and M_{p+2} (and b) are in flight while segment p
// is combined.  Every step issues its loads unconditionally (past the last segment it
// loads the last one again), so that the count of loads in flight is the same on
// every path and each step waits only for its own segment.  Everything stays in
// fp32: the state keeps its full precision from segment to segment.
#include "kda_device.h"
#include "kda_segment.h"

namespace kda {
namespace seg {

// LDS pitch (floats) of the transposed tile's rows: the lanes of a 16-lane group land on
// disjoint banks
template <int D>
constexpr int kPitch = D + 4;

// 16 k-steps of the fp32 MFMA: k = 16 kk + 4 g + c, c = 0..3 (A[m][k] from a.c,
// B[k][m] from b[c]); both operands use the same assignment of k.
__device__ __forceinline__ floatx4 mma16(const float4& a, const floatx4& b, floatx4 acc) {
    acc = mma_f32_k4(a.x, b[0], acc);
    acc = mma_f32_k4(a.y, b[1], acc);
    acc = mma_f32_k4(a.z, b[2], acc);
    acc = mma_f32_k4(a.w, b[3], acc);
    return acc;
}

template <int D>
__global__ __launch_bounds__(D * 4) void kda_combine_kernel(CombineParams p) {
    constexpr int NT = D / 16;  // column tiles per state; also waves per workgroup
    constexpr int NK = D / 16;  // 16-wide k steps of one row block
    static_assert(NK % 2 == 0, "two accumulator chains");
    constexpr int NTH = D * 4;  // threads
    constexpr int SP = kPitch<D>;
    __shared__ __align__(16) float S[2 * 16 * SP];
    const int lane = lane_id(), wave = wave_id();
    const int m = lane & 15, g = lane >> 4;
    // consecutive workgroups go to different XCDs; the NT tiles of one (b, h), which all
    // stream the same M_p, are given blocks that share bid % 8 and so one XCD's L2
    const int nblk = gridDim.x, bid = blockIdx.x;
    const int64_t logical = (int64_t)(bid % 8) * (nblk / 8) + bid / 8;
    const int64_t unit = logical / NT;
    if (unit >= p.units) return;  // padding workgroup (the whole group leaves together)
    const int col0 = 16 * (int)(logical % NT);
    const int64_t DD = (int64_t)D * D;
    const int arow = 16 * wave + m;      // row of M this lane streams
    const int crow = 16 * wave + 4 * g;  // first accumulator row of this lane
    // copies of the state tile: one float4 per thread (D x 16 = 4 NTH floats)
    static_assert(D * 16 == 4 * NTH, "one float4 of the tile per thread");
    const int tr = threadIdx.x >> 2, tc = 4 * (threadIdx.x & 3);  // row, first column

    // four columns tc .. tc + 3 of row tr of a (transposed) state tile
    auto row4 = [&](const float* St) __attribute__((always_inline)) {
        return make_float4(St[tc * SP + tr], St[(tc + 1) * SP + tr], St[(tc + 2) * SP + tr], St[(tc + 3) * SP + tr]);
    };
    // this wave's 16 rows of M_s (as MFMA A operands) and its b_s accumulator start, in
    // three register sets: segments s + 1 and s + 2 load while segment s is combined
    float4 M0[NK], M1[NK], M2[NK];
    floatx4 b0, b1, b2;
    const int64_t last = p.P - 1;
    auto load_seg = [&](int64_t s, float4(&Ma)[NK], floatx4& bb) __attribute__((always_inline)) {
        s = s < last ? s : last;
        const float* Mp = p.M + (s * p.units + unit) * DD + (int64_t)arow * D + 4 * g;
        const float* bp = p.b + (s * p.units + unit) * DD + (int64_t)crow * D + col0 + m;
#pragma unroll
        for (int kk = 0; kk < NK; ++kk) Ma[kk] = *reinterpret_cast<const float4*>(Mp + 16 * kk);
#pragma unroll
        for (int i = 0; i < 4; ++i) bb[i] = bp[(int64_t)i * D];
    };
    // combines segment s from (Ma, bb) and loads segment s + 2 into (Mn, bn); S_s is in
    // buffer s % 2, S_{s+1} goes to the other
    auto step = [&](int64_t s, const float4(&Ma)[NK], const floatx4& bb, float4(&Mn)[NK], floatx4& bn)
        __attribute__((always_inline)) {
        load_seg(s + 2, Mn, bn);
        const float* Sc = S + (s & 1) * 16 * SP;
        float* Sn = S + ((s + 1) & 1) * 16 * SP;
        if (p.seg) *reinterpret_cast<float4*>(p.seg + (s * p.units + unit) * DD + (int64_t)tr * D + col0 + tc) = row4(Sc);
        floatx4 sv[NK];  // every B operand of the step read first: one wait on LDS
#pragma unroll
        for (int kk = 0; kk < NK; ++kk) {
            const float4 v = *reinterpret_cast<const float4*>(Sc + m * SP + 16 * kk + 4 * g);
            sv[kk] = floatx4{v.x, v.y, v.z, v.w};
        }
        __builtin_amdgcn_sched_barrier(0);  // keep the reads ahead of the products
        floatx4 acc0 = bb, acc1 = zero4();  // two chains over alternate k blocks
#pragma unroll
        for (int kk = 0; kk < NK; kk += 2) {
            acc0 = mma16(Ma[kk], sv[kk], acc0);
            acc1 = mma16(Ma[kk + 1], sv[kk + 1], acc1);
        }
        *reinterpret_cast<float4*>(Sn + m * SP + crow) =
            make_float4(acc0[0] + acc1[0], acc0[1] + acc1[1], acc0[2] + acc1[2], acc0[3] + acc1[3]);
        // S_{s+1} is complete (the later segments' loads stay in flight); buffer s % 2 is
        // written again only after the next step's barrier, when every wave has read it
        lds_barrier();
    };
    // the tile of the incoming state, one float4 per thread (D x 16 = 4 NTH floats), read
    // before anything of this tile is written, so the final state may alias it; loaded
    // before the first segments' rows, so that the wait for it leaves theirs in flight
    const float4 v0 = p.s0 ? *reinterpret_cast<const float4*>(p.s0 + unit * DD + (int64_t)tr * D + col0 + tc)
                           : make_float4(0.f, 0.f, 0.f, 0.f);
    float* const sT = p.sT ? p.sT + unit * DD + (int64_t)tr * D + col0 + tc : nullptr;
    if (p.P == 0) {  // no segment: the state passes through (the whole workgroup leaves)
        if (sT) *reinterpret_cast<float4*>(sT) = v0;
        return;
    }
    // unconditional on every path, so that the wait for the state tile leaves them in flight
    load_seg(0, M0, b0);
    load_seg(1, M1, b1);
    S[tc * SP + tr] = v0.x;
    S[(tc + 1) * SP + tr] = v0.y;
    S[(tc + 2) * SP + tr] = v0.z;
    S[(tc + 3) * SP + tr] = v0.w;
    __syncthreads();
    int64_t s = 0;
    for (; s + 3 <= p.P; s += 3) {  // the register sets in turn; every step of a trip runs
        step(s, M0, b0, M2, b2);
        step(s + 1, M1, b1, M0, b0);
        step(s + 2, M2, b2, M1, b1);
    }
    if (s < p.P) step(s, M0, b0, M2, b2);
    if (s + 1 < p.P) step(s + 1, M1, b1, M0, b0);
    if (sT) *reinterpret_cast<float4*>(sT) = row4(S + (p.P & 1) * 16 * SP);
}

// M = I and b = 0 for every (b, h): one workgroup per (b, h)
template <int D>
__global__ __launch_bounds__(256) void kda_identity_summary_kernel(float* M, float* b) {
    const int64_t base = (int64_t)blockIdx.x * D * D;
    for (int e = threadIdx.x; e < D * D; e += 256) {
        M[base + e] = (e / D == e % D) ? 1.f : 0.f;
        b[base + e] = 0.f;
    }
}

}  // namespace seg

hipError_t launch_combine(int D, const CombineParams& p, hipStream_t stream) {
    if (p.units <= 0) return hipSuccess;
    const int64_t blocks = (p.units * (D / 16) + 7) / 8 * 8;  // a multiple of 8 (XCD mapping)
    if (D == 128)
        hipLaunchKernelGGL(seg::kda_combine_kernel<128>, dim3((unsigned)blocks), dim3(512), 0, stream, p);
    else if (D == 64)
        hipLaunchKernelGGL(seg::kda_combine_kernel<64>, dim3((unsigned)blocks), dim3(256), 0, stream, p);
    else
        return hipErrorInvalidValue;
    return hipGetLastError();
}

hipError_t launch_identity_summary(int D, float* M, float* b, int64_t units, hipStream_t stream) {
    if (units <= 0) return hipSuccess;
    if (D == 128)
        hipLaunchKernelGGL(seg::kda_identity_summary_kernel<128>, dim3((unsigned)units), dim3(256), 0, stream,
                           M, b);
    else if (D == 64)
        hipLaunchKernelGGL(seg::kda_identity_summary_kernel<64>, dim3((unsigned)units), dim3(256), 0, stream,
                           M, b);
    else
        return hipErrorInvalidValue;
    return hipGetLastError();
}

}  // namespace kda
