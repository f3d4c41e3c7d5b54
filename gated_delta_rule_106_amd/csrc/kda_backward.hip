// Chunkwise backward pass of KDA: gradients of L = <dY, Y> + <dS_T, S_T> with
// respect to q, k, v, log alpha, beta, the gate logits and the initial state.
//
// The forward it differentiates is the chunk-recurrent form (page "Kimi K3 report
// walk-through", section "Compute paradigm"; the per-token step is page "3T models
// are no longer magic", section "Gate 1: KDA makes it computable").  For one chunk
// of C tokens that starts from the state S0, with g the inclusive cumulative
// (clamped) log-decay per token and key channel, E = e^g and Gc = e^{g_C}:
//   Kt = K*E,  Qt = Q*E,  Kb = K*e^{g_C - g}
//   Bm_rs = sum_c k_rc k_sc e^{g_rc - g_sc} (s < r),  P_rs = sum_c q_rc k_sc e^{g_rc - g_sc} (s <= r)
//   Li = (I + diag(beta) Bm)^-1
//   X = V - Kt S0,  U = Li diag(beta) X,  O = Qt S0 + P U,  Y = O * sigmoid(Z)
//   S_C = Diag(Gc) S0 + Kb^T U
//
// Three launches:
//  1. kda_bwd_chunk_kernel, one workgroup per chunk: g, Bm, P, Li, and the sweep's
//     record W = Li diag(beta) Kt, Kb, Gc, U~ = Li diag(beta) V and
//     R = (Qt - P W)^T dO with dO = dY * sigmoid(Z); g, Li, P and Bm stay in a pair
//     record for the gradient kernel.
//  2. kda_bwd_sweep_kernel, one (direction, b, h, 16 value columns) per workgroup
//     (columns of the state evolve independently): forwards the states at every
//     chunk start, S_{n+1} = Diag(Gc) S_n - Kb^T (W S_n - U~); backwards the state
//     gradients, dS_n = Diag(Gc) dS_{n+1} - W^T (Kb dS_{n+1}) + R (the transposed
//     map).  R does not depend on the states, so the two directions run at once.
//  3. kda_bwd_grad_kernel, one workgroup per chunk: the adjoint of the chunk's steps
//     above from S_n and dS_{n+1}; log alpha's gradient is the reverse cumulative sum
//     of g's gradient within the chunk.
// All arithmetic is fp32 (the fp32 MFMA).  The chunk kernels keep every intermediate
// in registers and LDS; the pair products, and the pair terms of the gradients, are
// products over 16-token blocks with a reference point between the two blocks, so
// that no factor exceeds e^{8 tokens of decay} (the same 16-token tile the forward uses
// to keep decay factors in range, page "Kimi K3 report walk-through", section
// "Numerical stability & co-design").
#include "kda_backward.h"
#include "kda_device.h"

namespace kda {
namespace {

constexpr int C = 64;             // tokens per chunk
constexpr int NT = 256;           // threads per sweep workgroup
constexpr int TILE = 16;          // value columns per sweep workgroup

__device__ __forceinline__ float ex(float x) { return fast_exp2(x * kLog2e); }

// fp32 offsets of the per-chunk record written by the chunk kernel (row-major blocks:
// W, K-bar and U~ token x channel, R key channel x value column).
template <int D>
struct Rec {
    static constexpr int64_t CD = (int64_t)C * D, DD = (int64_t)D * D;
    static constexpr int64_t W = 0, KBAR = CD, UT = 2 * CD, R = 3 * CD, GC = 3 * CD + DD;
    static constexpr int64_t SIZE = 3 * CD + DD + D;
};

struct ChunkPos {
    int64_t row0, h;  // packed row of the chunk's first token; head
    int L;  // tokens of the chunk inside the sequence (the rest is padding); 0: no chunk
};

// Where chunk item `item` is: B sequences of T tokens (item (b H + h) NC + n), or a
// variable-length batch (item g H + h for the batch's chunk g; past the last chunk the
// item has none, L = 0, and its workgroup leaves at once).
__device__ __forceinline__ ChunkPos chunk_pos(const BwdParams& p, int64_t item) {
    ChunkPos cp;
    if (p.vs) {
        const int64_t g = item / p.H;
        cp.h = item - g * p.H;
        cp.row0 = 0;
        cp.L = 0;
        if (g < p.vco[p.B]) {
            const int64_t i = p.vsoc[g];
            cp.row0 = p.vs[i] + (g - p.vco[i]) * C;
            const int64_t left = p.vs[i + 1] - cp.row0;  // >= 1: the sequence owns this chunk
            cp.L = (int)(left < C ? left : C);
        }
    } else {
        const int64_t bh = item / p.NC, n = item - bh * p.NC;
        const int64_t b = bh / p.H;
        cp.h = bh - b * p.H;
        cp.row0 = b * p.T + n * C;
        cp.L = (int)(p.T - n * C < C ? p.T - n * C : C);
    }
    return cp;
}

template <int D>
__device__ __forceinline__ int64_t elem(const BwdParams& p, const ChunkPos& cp, int r, int c) {
    return ((cp.row0 + r) * p.H + cp.h) * D + c;
}

// LDS of the sweep kernel (fp32 offsets): two buffers of one chunk's W and K-bar (row
// pitch D + 4), the state tile and Y, both transposed (one row per value column, pitch
// D + 4 and C + 4), so that an MFMA's B operand and a lane's four accumulator rows are
// 16-byte accesses.  The pitches put the lanes of a 16-lane group on disjoint banks.
template <int D>
struct SweepLds {
    static constexpr int DP = D + 4, SP = D + 4, YP = C + 4;
    static constexpr int W = 0, KBAR = C * DP, BUF = 2 * C * DP;  // within a buffer
    static constexpr int ST = 2 * BUF, Y = ST + TILE * SP, TOTAL = Y + TILE * YP;
    static constexpr int NW4 = C * D / 4 / NT;    // float4 of W (and of K-bar) per thread
    static_assert(TOTAL * 4 <= 160 * 1024, "sweep LDS");
};

// 16 k-steps of the fp32 MFMA: lane (m, g) gives A[m][k] and B[k][m] for
// k = 16 kk + 4 g + c, c = 0..3, and accumulates D[4 g + i][m] in acc[i].
__device__ __forceinline__ floatx4 mma16x4(const float (&a)[4], const float (&b)[4], floatx4 acc) {
#pragma unroll
    for (int c = 0; c < 4; ++c) acc = mma_f32_k4(a[c], b[c], acc);
    return acc;
}

// Forwards: S <- Diag(Gc) S - Kb^T (W S - U~); backwards: dS <- Diag(Gc) dS - W^T (Kb dS) + R.
// One workgroup runs one direction.  Both products run on the fp32 MFMA: wave w
// forms rows 16 w .. 16 w + 15 of Y, then row blocks w, w + 4, .. of the new state.
// Chunk i + 1's W and K-bar are staged into the other LDS buffer while chunk i's products
// run (from registers loaded one chunk earlier), and each lane keeps the offset (U~ of its
// rows of Y, or R of its state rows) and Gamma_C entries in registers, loaded two chunks
// ahead: two barriers per chunk.  Loads past the last chunk repeat the last one (same bytes), so
// that every chunk issues the same loads.
template <int D>
__global__ __launch_bounds__(NT) __attribute__((amdgpu_waves_per_eu(1, 1))) void kda_bwd_sweep_kernel(BwdParams p) {
    using RC = Rec<D>;
    using L = SweepLds<D>;
    constexpr int DP = L::DP, SP = L::SP, YP = L::YP;
    constexpr int RBW = D / 16 / (NT / 64);  // row blocks of the state per wave
    extern __shared__ __align__(16) float lds[];
    float* St = lds + L::ST;
    float* Y = lds + L::Y;
    constexpr int tiles = D / TILE;
    // consecutive workgroups go to different XCDs: the logical order puts the column
    // tiles of one (direction, b, h), which all read the same chunk records, on blocks
    // that share blockIdx % 8 and so one XCD's L2 (the grid is a multiple of 8)
    const int64_t nblk = gridDim.x;
    const int64_t logical = (int64_t)(blockIdx.x % 8) * (nblk / 8) + blockIdx.x / 8;
    // the two sweeps are independent (R does not depend on the states): the first half
    // of the logical grid runs the forward one, the second half the backward one
    const int64_t half = nblk / 2;
    const int dir = logical >= half ? 1 : 0;
    const int64_t bid = logical - dir * half;
    const int64_t bh = bid / tiles;
    const int col0 = (int)(bid - bh * tiles) * TILE;
    const int64_t DD = (int64_t)D * D;
    // the NC chunks of this (b, h): chunk n is item cbase + n cstride (its records and
    // states); B sequences of T tokens, or sequence bh / H of a variable-length batch
    int64_t NC, cbase, cstride;
    if (p.vs) {
        const int64_t i = bh / p.H;
        NC = p.vco[i + 1] - p.vco[i];
        cbase = p.vco[i] * p.H + (bh - i * p.H);
        cstride = p.H;
    } else {
        NC = p.NC;
        cbase = bh * NC;
        cstride = 1;
    }
    // forwards: U~ (rows of Y); backwards: R (rows of the state)
    const int64_t off_base = dir == 0 ? RC::UT : RC::R;
    const int lane = lane_id(), wave = wave_id();
    const int m = lane & 15, g = lane >> 4;
    // the record of step i (chunk i forwards, NC - 1 - i backwards), clamped to the last step
    auto rec = [&](int64_t i) __attribute__((always_inline)) {
        i = i < NC - 1 ? i : NC - 1;
        return p.trans + (cbase + (dir == 0 ? i : NC - 1 - i) * cstride) * RC::SIZE;
    };
    // W and K-bar of a later chunk, in registers until staged
    float4 rw[L::NW4], rk[L::NW4];
#pragma unroll
    for (int i = 0; i < L::NW4; ++i) rw[i] = rk[i] = make_float4(0.f, 0.f, 0.f, 0.f);
    auto fetch_wk = [&](const float* tr) __attribute__((always_inline)) {
        const float4* w4 = reinterpret_cast<const float4*>(tr + RC::W);
        const float4* k4 = reinterpret_cast<const float4*>(tr + RC::KBAR);
#pragma unroll
        for (int i = 0; i < L::NW4; ++i) {
            rw[i] = w4[threadIdx.x + i * NT];
            rk[i] = k4[threadIdx.x + i * NT];
        }
    };
    auto stage_one = [&](float* buf, int i) __attribute__((always_inline)) {
        const int q = threadIdx.x + i * NT;  // row q / (D / 4), columns 4 (q % (D / 4)) ..
        const int at = (q / (D / 4)) * DP + 4 * (q % (D / 4));
        *reinterpret_cast<float4*>(buf + L::W + at) = rw[i];
        *reinterpret_cast<float4*>(buf + L::KBAR + at) = rk[i];
    };
    auto stage = [&](float* buf) __attribute__((always_inline)) {
#pragma unroll
        for (int i = 0; i < L::NW4; ++i) stage_one(buf, i);
    };
    static_assert(L::NW4 == D / 16, "one staged pair of float4 per K-block of Y");
    // this lane's rows 16 (wave + j (NT / 64)) + 4 g + r, column col0 + m, in two register
    // sets: Gamma_C of its state rows, and the offset: backwards R of its state rows,
    // forwards U~ of its rows of Y (j = 0; the state update takes none)
    float oA[RBW][4], gA[RBW][4], oB[RBW][4], gB[RBW][4];
#pragma unroll
    for (int j = 0; j < RBW; ++j)
#pragma unroll
        for (int r = 0; r < 4; ++r) oA[j][r] = gA[j][r] = oB[j][r] = gB[j][r] = 0.f;
    auto fetch_rows = [&](const float* tr, float (&o)[RBW][4], float (&gm)[RBW][4]) __attribute__((always_inline)) {
#pragma unroll
        for (int j = 0; j < RBW; ++j)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int row = 16 * (wave + j * (NT / 64)) + 4 * g + r;
                o[j][r] = (dir == 1 || j == 0) ? tr[off_base + (int64_t)row * D + col0 + m] : 0.f;
                gm[j][r] = tr[RC::GC + row];
            }
    };
    // the state tile to its (row-major, D x D) place in HBM, four columns of a row per
    // 16-byte store
    static_assert(D * TILE % (4 * NT) == 0, "whole float4 of the tile per thread");
    auto put_state = [&](float* out) __attribute__((always_inline)) {
#pragma unroll
        for (int q = 0; q < D * TILE / 4 / NT; ++q) {
            const int idx = threadIdx.x + q * NT, c = idx >> 2, j = 4 * (idx & 3);
            *reinterpret_cast<float4*>(out + c * D + col0 + j) =
                make_float4(St[j * SP + c], St[(j + 1) * SP + c], St[(j + 2) * SP + c], St[(j + 3) * SP + c]);
        }
    };
    // step i: the state of its chunk out, Y = A1 S, chunk i + 1 staged, the new state from
    // the rows in (o, gm), which then take chunk i + 2's
    auto step = [&](int64_t i, float (&o)[RBW][4], float (&gm)[RBW][4]) __attribute__((always_inline)) {
        const int64_t n = dir == 0 ? i : NC - 1 - i;
        const float* buf = lds + (i & 1) * L::BUF;
        float* out = (dir == 0 ? p.states : p.dstates) + (cbase + n * cstride) * DD;
        put_state(out);
        // Y = W S - U~ (forwards) or Kb dS (backwards): wave w owns rows 16 w ..
        const float* A1 = buf + (dir == 0 ? L::W : L::KBAR);
        const float* A2 = buf + (dir == 0 ? L::KBAR : L::W);
        // chunk i + 1 goes into the other buffer (read by step i - 1, which every wave has
        // left), one piece after each K-block of Y so that the LDS stores run beside the MFMAs;
        // then chunk i + 2's W and K-bar into the registers
        float* nbuf = lds + ((i + 1) & 1) * L::BUF;
        {
            // two accumulator chains (even and odd K-blocks), summed at the end; forwards the
            // first starts from -U~
            floatx4 acc0 = zero4(), acc1 = zero4();
            if (dir == 0) acc0 = floatx4{-o[0][0], -o[0][1], -o[0][2], -o[0][3]};
#pragma unroll
            for (int kk = 0; kk < D / 16; ++kk) {
                const int k0 = 16 * kk + 4 * g;
                const float4 av = *reinterpret_cast<const float4*>(A1 + (16 * wave + m) * DP + k0);
                const float4 bv = *reinterpret_cast<const float4*>(St + m * SP + k0);
                const float a[4] = {av.x, av.y, av.z, av.w};
                const float b[4] = {bv.x, bv.y, bv.z, bv.w};
                if (kk & 1)
                    acc1 = mma16x4(a, b, acc1);
                else
                    acc0 = mma16x4(a, b, acc0);
                stage_one(nbuf, kk);
            }
            *reinterpret_cast<float4*>(Y + m * YP + 16 * wave + 4 * g) =
                make_float4(acc0[0] + acc1[0], acc0[1] + acc1[1], acc0[2] + acc1[2], acc0[3] + acc1[3]);
        }
        fetch_wk(rec(i + 2));
        __syncthreads();  // Y and the staged chunk are complete
        // state <- Diag(Gc) state - A2^T Y (+ R backwards), row blocks wave, wave + 4, ..
        // (their accumulator chains interleaved)
        floatx4 acc[RBW];
#pragma unroll
        for (int j = 0; j < RBW; ++j) acc[j] = zero4();
#pragma unroll
        for (int kk = 0; kk < C / 16; ++kk) {
            const int k0 = 16 * kk + 4 * g;
            const float4 yv = *reinterpret_cast<const float4*>(Y + m * YP + k0);
            const float b[4] = {yv.x, yv.y, yv.z, yv.w};
#pragma unroll
            for (int j = 0; j < RBW; ++j) {
                const int rb = wave + j * (NT / 64);
                const float a[4] = {A2[(k0 + 0) * DP + 16 * rb + m], A2[(k0 + 1) * DP + 16 * rb + m],
                                    A2[(k0 + 2) * DP + 16 * rb + m], A2[(k0 + 3) * DP + 16 * rb + m]};
                acc[j] = mma16x4(a, b, acc[j]);
            }
        }
#pragma unroll
        for (int j = 0; j < RBW; ++j) {
            float4* sp = reinterpret_cast<float4*>(St + m * SP + 16 * (wave + j * (NT / 64)) + 4 * g);
            float4 sv = *sp;
            const bool off = dir == 1;
            sv.x = gm[j][0] * sv.x - acc[j][0] + (off ? o[j][0] : 0.f);
            sv.y = gm[j][1] * sv.y - acc[j][1] + (off ? o[j][1] : 0.f);
            sv.z = gm[j][2] * sv.z - acc[j][2] + (off ? o[j][2] : 0.f);
            sv.w = gm[j][3] * sv.w - acc[j][3] + (off ? o[j][3] : 0.f);
            *sp = sv;
        }
        fetch_rows(rec(i + 2), o, gm);
        __syncthreads();  // the new state is complete; buffer i % 2 is no longer read
    };
    {
        const float* init = dir == 0 ? p.s0 : p.dsT;
        for (int idx = threadIdx.x; idx < D * TILE; idx += NT) {
            const int c = idx / TILE, j = idx - c * TILE;
            St[j * SP + c] = init ? init[bh * DD + c * D + col0 + j] : 0.f;
        }
        if (NC > 0) {
            fetch_wk(rec(0));
            stage(lds);
            fetch_wk(rec(1));
            fetch_rows(rec(0), oA, gA);
            fetch_rows(rec(1), oB, gB);
        }
        __syncthreads();
        int64_t i = 0;
        for (; i + 2 <= NC; i += 2) {  // the register sets in turn
            step(i, oA, gA);
            step(i + 1, oB, gB);
        }
        if (i < NC) step(i, oA, gA);
    }
    if (dir == 1 && p.ds0) put_state(p.ds0 + bh * DD);
}

// fp32 offsets of the per-chunk pair record the chunk kernel leaves for the gradient
// kernel: g (C x D), Li, P and Bm (C x C, row-major).
template <int D>
struct Pr {
    static constexpr int64_t CD = (int64_t)C * D, CC = (int64_t)C * C;
    static constexpr int64_t G = 0, LI = CD, PM = CD + CC, BM = CD + 2 * CC, SIZE = CD + 3 * CC;
};

// Four K-steps of the fp32 MFMA: lane (g, l) gives A[l][k_j] and B[k_j][l] with
// k_j = 16 t + 4 g + j for j = 0..3 (any K-block t).  An accumulator tile, whose lane
// (g, l) holds rows 16 t + 4 g + i of column l, is such a B operand as it stands.
__device__ __forceinline__ floatx4 mma4(const float4& a, const float4& b, floatx4 acc) {
    acc = mma_f32_k4(a.x, b.x, acc);
    acc = mma_f32_k4(a.y, b.y, acc);
    acc = mma_f32_k4(a.z, b.z, acc);
    return mma_f32_k4(a.w, b.w, acc);
}
__device__ __forceinline__ float4 f4(const floatx4& x) { return make_float4(x[0], x[1], x[2], x[3]); }
__device__ __forceinline__ float4 ld4(const float* p) { return *reinterpret_cast<const float4*>(p); }
__device__ __forceinline__ float4 mul4(const float4& a, const float4& b) {
    return make_float4(a.x * b.x, a.y * b.y, a.z * b.z, a.w * b.w);
}

// Eight consecutive input elements (channels c8 .. c8 + 7, c8 a multiple of 8) of token row
// r of the chunk as fp32: one 16-byte load for bf16, two for fp32; zero past the end.
template <int D, class In>
__device__ __forceinline__ void in8(const BwdParams& p, const ChunkPos& cp, const void* ptr, int r, int c8,
                                    float (&o)[8]) {
    // the load itself is unconditional (a row inside the sequence; cp.L >= 1), so that a
    // run of them issues at once; rows past the end are zeroed afterwards
    const bool in_seq = r < cp.L;
    const int64_t e = elem<D>(p, cp, in_seq ? r : cp.L - 1, c8);
    if constexpr (sizeof(typename In::raw_t) == 2) {
        const uint4 w = *reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(ptr) + e);
        const uint32_t ws[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
        for (int j = 0; j < 4; ++j) {  // little-endian: element 2 j is the low half-word
            o[2 * j] = __uint_as_float(ws[j] << 16);
            o[2 * j + 1] = __uint_as_float(ws[j] & 0xffff0000u);
        }
    } else {
        const float4 a = *reinterpret_cast<const float4*>(static_cast<const float*>(ptr) + e);
        const float4 b = *reinterpret_cast<const float4*>(static_cast<const float*>(ptr) + e + 4);
        o[0] = a.x, o[1] = a.y, o[2] = a.z, o[3] = a.w, o[4] = b.x, o[5] = b.y, o[6] = b.z, o[7] = b.w;
    }
#pragma unroll
    for (int j = 0; j < 8; ++j) o[j] = in_seq ? o[j] : 0.f;
}
__device__ __forceinline__ void st8(float* d, const float (&v)[8]) {
    *reinterpret_cast<float4*>(d) = make_float4(v[0], v[1], v[2], v[3]);
    *reinterpret_cast<float4*>(d + 4) = make_float4(v[4], v[5], v[6], v[7]);
}
__device__ __forceinline__ void ld8(const float* s, float (&v)[8]) {
    const float4 a = *reinterpret_cast<const float4*>(s), b = *reinterpret_cast<const float4*>(s + 4);
    v[0] = a.x, v[1] = a.y, v[2] = a.z, v[3] = a.w, v[4] = b.x, v[5] = b.y, v[6] = b.z, v[7] = b.w;
}

// Block (a, b), b <= a, of the 4 x 4 grid of 16 x 16 blocks, for task 0..9.
__device__ __forceinline__ void lower_block(int task, int& a, int& b) {
    a = 0;
    while ((a + 1) * (a + 2) / 2 <= task) ++a;
    b = task - a * (a + 1) / 2;
}

// Sum over the D / 8 neighbouring lanes that hold one token's channels in the staging
// loops (eight channels per lane, consecutive lanes on consecutive groups).
template <int D>
__device__ __forceinline__ float token_sum(float v) {
#pragma unroll
    for (int m = 1; m < D / 8; m <<= 1) v += __shfl_xor(v, m);
    return v;
}
// Per-token L2 normalisation of raw q or k (the fused preparation): scales a lane's
// eight channels by s = 1 / (c max(|x|, 1e-12)) and returns s; c = 1 for k, sqrt(D)
// for q.  Every lane of the wave takes part.
template <int D>
__device__ __forceinline__ float unit8(float (&x)[8], float inv_c) {
    float ss = 0.f;
#pragma unroll
    for (int j = 0; j < 8; ++j) ss = fmaf(x[j], x[j], ss);
    const float s = inv_norm(token_sum<D>(ss)) * inv_c;
#pragma unroll
    for (int j = 0; j < 8; ++j) x[j] *= s;
    return s;
}
template <int D>
constexpr float kInvSqrtD = D == 128 ? 0.08838834764831845f : 0.125f;

// LDS of the chunk kernel (floats; C x D blocks with row pitch D + 4, C x C with C + 4).
template <int D>
struct ChunkL {
    static constexpr int DP = D + 4, CP = C + 4;
    static constexpr int SK = 0, SQ = C * DP, SG = 2 * C * DP, SLI = 3 * C * DP, SP = SLI + C * CP,
                         SBM = SP + C * CP, BETA = SBM + C * CP, TOTAL = BETA + C;
    static_assert(TOTAL * 4 <= 160 * 1024, "chunk kernel LDS");
};

// Chunk kernel: one workgroup of D / 16 waves per (b, h, chunk).  From the chunk's
// inputs: g, the pair blocks Bm (strictly lower) and P (lower), Li = (I + diag(beta) Bm)^-1,
// then, wave w on the value (or key) columns 16 w .. 16 w + 15: W = Li diag(beta) Kt,
// U~ = Li diag(beta) V, Qe = Qt - P W, Kb, Gamma_C and R = Qe^T dO.  Writes the sweep's
// record (W, Kb, U~, R, Gamma_C) and the pair record (g, Li, P, Bm).
// Pairs: block (a, b) is a product over the channels with a reference point rho between
// the two tiles, k_r e^{g_r - rho} against k_s e^{rho - g_s}: the end of tile a - 1 for
// b < a (both factors <= 1), token 7 of the tile for a diagonal block (each factor spans
// at most eight tokens of decay).
// PREP: the inputs take the fused preparation first (flags qk_norm, logits).
template <int D, class In, bool PREP>
__global__ __launch_bounds__(64 * (D / 16)) void kda_bwd_chunk_kernel(BwdParams p) {
    using L = ChunkL<D>;
    using RC = Rec<D>;
    using PR = Pr<D>;
    using raw = typename In::raw_t;
    constexpr int NW = D / 16, NTT = 64 * NW, DP = L::DP, CP = L::CP;
    extern __shared__ __align__(16) float lds[];
    float* sk = lds + L::SK;
    float* sq = lds + L::SQ;
    float* sg = lds + L::SG;
    float* sli = lds + L::SLI;
    float* sp = lds + L::SP;
    float* sbm = lds + L::SBM;
    float* sbeta = lds + L::BETA;
    const int64_t item = blockIdx.x;
    const ChunkPos cp = chunk_pos(p, item);
    if (cp.L == 0) return;  // no chunk here (the whole workgroup leaves)
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, l = lane & 15, g = lane >> 4;
    float* pr = p.pairs + item * PR::SIZE;
    float* tr = p.trans + item * RC::SIZE;
    // element (r, c) of a token tensor, zero past the sequence's end: the load itself is
    // unconditional (from a row inside the sequence), so that a run of them issues at once
    auto in = [&](const void* ptr, int r, int c) -> float {
        const float x = In::load(static_cast<const raw*>(ptr), elem<D>(p, cp, r < cp.L ? r : cp.L - 1, c));
        return r < cp.L ? x : 0.f;
    };

    // inputs; tokens past the sequence's end are identity steps (all zero, log alpha 0)
    // eight neighbouring channels per lane and step, every load of a thread issued first
    constexpr int G8 = C * D / 8 / NTT;
    static_assert(G8 * 8 * NTT == C * D, "groups of eight");
    {
        float k8[G8][8], q8[G8][8], l8[G8][8];
#pragma unroll
        for (int u = 0; u < G8; ++u) {
            const int grp = tid + u * NTT, r = grp / (D / 8), c8 = 8 * (grp - r * (D / 8));
            in8<D, In>(p, cp, p.k, r, c8, k8[u]);
            in8<D, In>(p, cp, p.q, r, c8, q8[u]);
            in8<D, In>(p, cp, p.la, r, c8, l8[u]);
        }
#pragma unroll
        for (int u = 0; u < G8; ++u) {
            const int grp = tid + u * NTT, r = grp / (D / 8), c8 = 8 * (grp - r * (D / 8));
            if (PREP && p.qk_norm) {
                unit8<D>(k8[u], 1.f);
                unit8<D>(q8[u], kInvSqrtD<D>);
            }
#pragma unroll
            for (int j = 0; j < 8; ++j)
                l8[u][j] = r < cp.L ? log_alpha_in(l8[u][j], PREP && p.logits, p.clamp != 0) : 0.f;
            st8(sk + r * DP + c8, k8[u]);
            st8(sq + r * DP + c8, q8[u]);
            st8(sg + r * DP + c8, l8[u]);
        }
    }
    if (tid < C)
        sbeta[tid] = tid < cp.L
                         ? In::load(static_cast<const raw*>(p.beta), (cp.row0 + tid) * p.H + cp.h)
                         : 0.f;
    __syncthreads();
    if (tid < D) {  // g: inclusive cumulative sum over the chunk per key channel
        float gv[C];  // every load issued before the sums
#pragma unroll
        for (int r = 0; r < C; ++r) gv[r] = sg[r * DP + tid];
        float acc = 0.f;
#pragma unroll
        for (int r = 0; r < C; ++r) {
            acc += gv[r];
            sg[r * DP + tid] = acc;
            pr[PR::G + r * D + tid] = acc;
        }
    }
    // the blocks above the diagonal are zero
    for (int i = tid; i < C * C; i += NTT) {
        const int r = i / C, s = i - r * C;
        if (s / 16 > r / 16) {
            sbm[r * CP + s] = sp[r * CP + s] = sli[r * CP + s] = 0.f;
            pr[PR::BM + i] = pr[PR::PM + i] = 0.f;
        }
    }
    __syncthreads();

    // pair blocks
    for (int task = wave; task < 10; task += NW) {
        int a, bt;
        lower_block(task, a, bt);
        const int rref = bt < a ? 16 * a - 1 : 16 * a + 7;
        const float* gr = sg + (16 * a + l) * DP;
        const float* gs = sg + (16 * bt + l) * DP;
        const float* gf = sg + rref * DP;
        floatx4 accB = zero4(), accP = zero4();
#pragma unroll 4
        for (int t = 0; t < D / 16; ++t) {
            const int c0 = 16 * t + 4 * g;
            const float4 rho = ld4(gf + c0), g4r = ld4(gr + c0), g4s = ld4(gs + c0);
            const float4 k4r = ld4(sk + (16 * a + l) * DP + c0), q4r = ld4(sq + (16 * a + l) * DP + c0);
            const float4 k4s = ld4(sk + (16 * bt + l) * DP + c0);
            const float4 ea = make_float4(ex(g4r.x - rho.x), ex(g4r.y - rho.y), ex(g4r.z - rho.z), ex(g4r.w - rho.w));
            const float4 eb = make_float4(ex(rho.x - g4s.x), ex(rho.y - g4s.y), ex(rho.z - g4s.z), ex(rho.w - g4s.w));
            const float4 ks = mul4(k4s, eb);
            accB = mma4(mul4(k4r, ea), ks, accB);
            accP = mma4(mul4(q4r, ea), ks, accP);
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int r = 16 * a + 4 * g + i, s = 16 * bt + l;
            const float bm = s < r ? accB[i] : 0.f, pm = s <= r ? accP[i] : 0.f;
            sbm[r * CP + s] = bm;
            sp[r * CP + s] = pm;
            pr[PR::BM + r * C + s] = bm;
            pr[PR::PM + r * C + s] = pm;
        }
    }
    __syncthreads();
    // Li = (I + F)^-1 with F = diag(beta) Bm, blocked by 16 tokens: the diagonal blocks
    // X_a = (I + F_aa)^-1 by forward substitution in wave 0 (lane group = block, lane =
    // column, the column in registers), then block diagonal d = 1, 2, 3:
    //   Li_{a,a-d} = -X_a sum_{c = a-d}^{a-1} F_{a,c} Li_{c,a-d}
    // on the fp32 MFMA, one block per wave
    if (wave == 0) {
        const int a = g, j = l;
        const float* fb = sbm + (16 * a) * CP + 16 * a;
        float x[16];
        x[0] = j == 0 ? 1.f : 0.f;
#pragma unroll
        for (int r = 1; r < 16; ++r) {
            float acc = 0.f;
#pragma unroll
            for (int q = 0; q < r; ++q) acc = fmaf(fb[r * CP + q], x[q], acc);
            x[r] = (r == j ? 1.f : 0.f) - sbeta[16 * a + r] * acc;  // zero above the column
        }
#pragma unroll
        for (int r = 0; r < 16; ++r) sli[(16 * a + r) * CP + 16 * a + j] = x[r];
    }
    __syncthreads();
#pragma unroll
    for (int d = 1; d < 4; ++d) {
        if (wave < 4 - d) {
            const int a = wave + d, bb = a - d;
            const float br = sbeta[16 * a + l];
            floatx4 y = zero4();
            for (int c = bb; c < a; ++c) {
                const float4 f = ld4(sbm + (16 * a + l) * CP + 16 * c + 4 * g);
                const int r0 = 16 * c + 4 * g;
                const float4 lv = make_float4(sli[(r0 + 0) * CP + 16 * bb + l], sli[(r0 + 1) * CP + 16 * bb + l],
                                              sli[(r0 + 2) * CP + 16 * bb + l], sli[(r0 + 3) * CP + 16 * bb + l]);
                y = mma4(make_float4(br * f.x, br * f.y, br * f.z, br * f.w), lv, y);
            }
            const floatx4 z = mma4(ld4(sli + (16 * a + l) * CP + 16 * a + 4 * g), f4(y), zero4());
#pragma unroll
            for (int i = 0; i < 4; ++i) sli[(16 * a + 4 * g + i) * CP + 16 * bb + l] = -z[i];
        }
        __syncthreads();
    }
    for (int i = tid; i < C * C; i += NTT) pr[PR::LI + i] = sli[(i / C) * CP + (i % C)];

    // the products of the value (and key) columns c = 16 w + l; K-block t of a token
    // operand holds tokens 16 t + 4 g + j
    const int c = 16 * wave + l;
    float4 ktb[4], vb[4], dob[4];
#pragma unroll
    for (int t = 0; t < 4; ++t) {
        float kt[4], vv[4], dd[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int r = 16 * t + 4 * g + j;
            kt[j] = sk[r * DP + c] * ex(sg[r * DP + c]);
            vv[j] = in(p.v, r, c);
            dd[j] = in(p.dy, r, c) * sigmoidf_(in(p.gate, r, c));
        }
        ktb[t] = make_float4(kt[0], kt[1], kt[2], kt[3]);
        vb[t] = make_float4(vv[0], vv[1], vv[2], vv[3]);
        dob[t] = make_float4(dd[0], dd[1], dd[2], dd[3]);
    }
    floatx4 Wt[4], Ut[4], Qe[4];
#pragma unroll
    for (int ma = 0; ma < 4; ++ma) {
        floatx4 aw = zero4(), au = zero4();
#pragma unroll
        for (int t = 0; t <= ma; ++t) {
            const float4 a4 = mul4(ld4(sli + (16 * ma + l) * CP + 16 * t + 4 * g), ld4(sbeta + 16 * t + 4 * g));
            aw = mma4(a4, ktb[t], aw);
            au = mma4(a4, vb[t], au);
        }
        Wt[ma] = aw;
        Ut[ma] = au;
    }
#pragma unroll
    for (int ma = 0; ma < 4; ++ma) {
        floatx4 pw = zero4();
#pragma unroll
        for (int t = 0; t <= ma; ++t) pw = mma4(ld4(sp + (16 * ma + l) * CP + 16 * t + 4 * g), f4(Wt[t]), pw);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int r = 16 * ma + 4 * g + i;
            Qe[ma][i] = sq[r * DP + c] * ex(sg[r * DP + c]) - pw[i];
        }
    }
    float kbv[4][4];
    const float gC = sg[(C - 1) * DP + c];
#pragma unroll
    for (int ma = 0; ma < 4; ++ma)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int r = 16 * ma + 4 * g + i;
            kbv[ma][i] = sk[r * DP + c] * ex(gC - sg[r * DP + c]);
            tr[RC::W + r * D + c] = Wt[ma][i];
            tr[RC::KBAR + r * D + c] = kbv[ma][i];
            tr[RC::UT + r * D + c] = Ut[ma][i];
        }
    if (g == 0) tr[RC::GC + c] = ex(gC);
    __syncthreads();  // q no longer read: its block takes Qe
#pragma unroll
    for (int ma = 0; ma < 4; ++ma)
#pragma unroll
        for (int i = 0; i < 4; ++i) sq[(16 * ma + 4 * g + i) * DP + c] = Qe[ma][i];
    __syncthreads();
    // R = Qe^T dO: rows = key channels (D / 16 blocks), columns c
#pragma unroll 2
    for (int mb = 0; mb < D / 16; ++mb) {
        floatx4 ar = zero4();
#pragma unroll
        for (int t = 0; t < 4; ++t) {
            const int r0 = 16 * t + 4 * g;
            const float4 qe4 = make_float4(sq[(r0 + 0) * DP + 16 * mb + l], sq[(r0 + 1) * DP + 16 * mb + l],
                                           sq[(r0 + 2) * DP + 16 * mb + l], sq[(r0 + 3) * DP + 16 * mb + l]);
            ar = mma4(qe4, dob[t], ar);
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) tr[RC::R + (16 * mb + 4 * g + i) * D + c] = ar[i];
    }
}

// LDS of the gradient kernel (floats): three C x D blocks (pitch D + 4), three C x C
// blocks (pitch C + 4), beta, and the per-wave partial sums of dGamma_C and dbeta.
template <int D>
struct GradL {
    static constexpr int NW = D / 16, DP = D + 4, CP = C + 4;
    static constexpr int RA = 0, RB = C * DP, RCc = 2 * C * DP, RL = 3 * C * DP, RP = RL + C * CP,
                         RQ = RP + C * CP, BETA = RQ + C * CP, DGC = BETA + C, DB1 = DGC + NW * D,
                         SCL = DB1 + NW * C, TOTAL = SCL + 2 * C;
    static_assert(TOTAL * 4 <= 160 * 1024, "gradient kernel LDS");
};

// Sum over the 16 lanes l of a lane group (lanes 16 g .. 16 g + 15).
__device__ __forceinline__ float sum16(float v) {
    v += __shfl_xor(v, 1);
    v += __shfl_xor(v, 2);
    v += __shfl_xor(v, 4);
    v += __shfl_xor(v, 8);
    return v;
}

// Gradient kernel: one workgroup of D / 16 waves per (b, h, chunk), from the state at the
// chunk's start S0, the gradient of the state at its end dS_C and the pair record; the
// adjoint of the chunk's steps (X = V - Kt S0, U = Li diag(beta) X, O = Qt S0 + P U,
// S_C = Diag(Gamma_C) S0 + Kb^T U, Y = O sigmoid(Z)).  Every intermediate stays in
// registers or LDS: wave w carries the value columns 16 w .. of X, U, O, dO, dU and dX
// (left products read their other operand from LDS), and then forms the key columns
// 16 w .. of the products over the value dimension (dO S0^T, dX S0^T, U dS_C^T) and of the
// pair terms of dq, dk and dg.
// PREP: the inputs take the fused preparation (flags qk_norm, logits); the gradients of
// q and k go back through the normalisation, that of log alpha through logsigmoid.
template <int D, class In, bool PREP>
__global__ __launch_bounds__(64 * (D / 16)) void kda_bwd_grad_kernel(BwdParams p) {
    using L = GradL<D>;
    using PR = Pr<D>;
    using raw = typename In::raw_t;
    constexpr int NW = L::NW, NTT = 64 * NW, DP = L::DP, CP = L::CP;
    constexpr int NT4 = D / 16;  // K-blocks of 16 over a D-long index
    extern __shared__ __align__(16) float lds[];
    float* ra = lds + L::RA;
    float* rb = lds + L::RB;
    float* rc = lds + L::RCc;
    float* rl = lds + L::RL;
    float* rp = lds + L::RP;
    float* rq = lds + L::RQ;
    float* sbeta = lds + L::BETA;
    float* dgcp = lds + L::DGC;
    float* db1p = lds + L::DB1;
    float* sclq = lds + L::SCL;  // per token: the normalisation factors of q and k
    float* sclk = sclq + C;
    const int64_t item = blockIdx.x;
    const ChunkPos cp = chunk_pos(p, item);
    if (cp.L == 0) return;  // no chunk here (the whole workgroup leaves)
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, l = lane & 15, g = lane >> 4;
    const int64_t DD = (int64_t)D * D;
    const float* pr = p.pairs + item * PR::SIZE;
    const float* gg = pr + PR::G;
    const float* S0 = p.states + item * DD;
    const float* dSC = p.dstates + item * DD;
    // element (r, c) of a token tensor, zero past the sequence's end: the load itself is
    // unconditional (from a row inside the sequence), so that a run of them issues at once
    auto in = [&](const void* ptr, int r, int c) -> float {
        const float x = In::load(static_cast<const raw*>(ptr), elem<D>(p, cp, r < cp.L ? r : cp.L - 1, c));
        return r < cp.L ? x : 0.f;
    };

    const int c = 16 * wave + l;  // this wave's value column (and, later, key channel)
    // (issued first: their latency overlaps the staging below)
    // S0 and dS_C columns as B operands: K-block t holds key channels 16 t + 4 g + j
    float4 s0b[NT4], dsb[NT4];
#pragma unroll
    for (int t = 0; t < NT4; ++t) {
        const int k0 = 16 * t + 4 * g;
        s0b[t] = make_float4(S0[(k0 + 0) * D + c], S0[(k0 + 1) * D + c], S0[(k0 + 2) * D + c], S0[(k0 + 3) * D + c]);
        dsb[t] = make_float4(dSC[(k0 + 0) * D + c], dSC[(k0 + 1) * D + c], dSC[(k0 + 2) * D + c],
                             dSC[(k0 + 3) * D + c]);
    }
    // Li, P, beta; Kt and Qt (Li and P four neighbouring entries per thread and step,
    // every load issued first)
    {
        constexpr int N4 = C * C / 4 / NTT;
        static_assert(N4 * 4 * NTT == C * C, "Li and P in float4");
        float4 li4[N4], pm4[N4];
#pragma unroll
        for (int u = 0; u < N4; ++u) {
            const int i = 4 * (tid + u * NTT);
            li4[u] = ld4(pr + PR::LI + i);
            pm4[u] = ld4(pr + PR::PM + i);
        }
#pragma unroll
        for (int u = 0; u < N4; ++u) {
            const int i = 4 * (tid + u * NTT), r = i / C, s = i - r * C;
            *reinterpret_cast<float4*>(rl + r * CP + s) = li4[u];
            *reinterpret_cast<float4*>(rp + r * CP + s) = pm4[u];
        }
    }
    if (tid < C)
        sbeta[tid] = tid < cp.L
                         ? In::load(static_cast<const raw*>(p.beta), (cp.row0 + tid) * p.H + cp.h)
                         : 0.f;
    constexpr int G8 = C * D / 8 / NTT;
    static_assert(G8 * 8 * NTT == C * D, "groups of eight");
    {
        float k8[G8][8], q8[G8][8], g8[G8][8];
#pragma unroll
        for (int u = 0; u < G8; ++u) {
            const int grp = tid + u * NTT, r = grp / (D / 8), c8 = 8 * (grp - r * (D / 8));
            in8<D, In>(p, cp, p.k, r, c8, k8[u]);
            in8<D, In>(p, cp, p.q, r, c8, q8[u]);
            ld8(gg + r * D + c8, g8[u]);
        }
#pragma unroll
        for (int u = 0; u < G8; ++u) {
            const int grp = tid + u * NTT, r = grp / (D / 8), c8 = 8 * (grp - r * (D / 8));
            if (PREP && p.qk_norm) {
                unit8<D>(k8[u], 1.f);
                unit8<D>(q8[u], kInvSqrtD<D>);
            }
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                const float e = ex(g8[u][j]);
                k8[u][j] *= e;
                q8[u][j] *= e;
            }
            st8(ra + r * DP + c8, k8[u]);
            st8(rb + r * DP + c8, q8[u]);
        }
    }
    __syncthreads();

    // dGamma_C over this wave's value columns: sum of dS_C S0 along the row
#pragma unroll
    for (int t = 0; t < NT4; ++t) {
        const float4 pv = mul4(s0b[t], dsb[t]);
        const float v0 = sum16(pv.x), v1 = sum16(pv.y), v2 = sum16(pv.z), v3 = sum16(pv.w);
        if (l == 0) {
            const int k0 = 16 * t + 4 * g;
            dgcp[wave * D + k0 + 0] = v0;
            dgcp[wave * D + k0 + 1] = v1;
            dgcp[wave * D + k0 + 2] = v2;
            dgcp[wave * D + k0 + 3] = v3;
        }
    }
    // X = V - Kt S0, O = Qt S0 (V, dY and Z of this wave's value column loaded first, ahead
    // of the products and of the dZ stores)
    floatx4 X[4], O[4];
    float vv[4][4], dyv[4][4], zv[4][4];
#pragma unroll
    for (int ma = 0; ma < 4; ++ma)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int r = 16 * ma + 4 * g + i;
            vv[ma][i] = in(p.v, r, c);
            dyv[ma][i] = in(p.dy, r, c);
            zv[ma][i] = in(p.gate, r, c);
        }
#pragma unroll
    for (int ma = 0; ma < 4; ++ma) {
        floatx4 ax = zero4(), ao = zero4();
#pragma unroll
        for (int t = 0; t < NT4; ++t) {
            ax = mma4(ld4(ra + (16 * ma + l) * DP + 16 * t + 4 * g), s0b[t], ax);
            ao = mma4(ld4(rb + (16 * ma + l) * DP + 16 * t + 4 * g), s0b[t], ao);
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) X[ma][i] = vv[ma][i] - ax[i];
        O[ma] = ao;
    }
    // U = Li diag(beta) X;  O += P U
    floatx4 U[4];
#pragma unroll
    for (int ma = 0; ma < 4; ++ma) {
        floatx4 au = zero4();
#pragma unroll
        for (int t = 0; t <= ma; ++t)
            au = mma4(mul4(ld4(rl + (16 * ma + l) * CP + 16 * t + 4 * g), ld4(sbeta + 16 * t + 4 * g)), f4(X[t]), au);
        U[ma] = au;
    }
#pragma unroll
    for (int ma = 0; ma < 4; ++ma)
#pragma unroll
        for (int t = 0; t <= ma; ++t) O[ma] = mma4(ld4(rp + (16 * ma + l) * CP + 16 * t + 4 * g), f4(U[t]), O[ma]);
    // dO = dY sigmoid(Z);  dZ = dY O sigmoid'(Z)
    floatx4 dO[4];
#pragma unroll
    for (int ma = 0; ma < 4; ++ma)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int r = 16 * ma + 4 * g + i;
            const float dy = dyv[ma][i], sz = sigmoidf_(zv[ma][i]);
            dO[ma][i] = dy * sz;
            if (r < cp.L) p.dgate[elem<D>(p, cp, r, c)] = dy * O[ma][i] * sz * (1.f - sz);
        }
    __syncthreads();  // Kt, Qt no longer read: U and dO take their blocks, Kb the third
#pragma unroll
    for (int ma = 0; ma < 4; ++ma)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int r = 16 * ma + 4 * g + i;
            ra[r * DP + c] = U[ma][i];
            rb[r * DP + c] = dO[ma][i];
        }
    {
        float k8[G8][8], g8[G8][8], c8v[G8][8];
#pragma unroll
        for (int u = 0; u < G8; ++u) {
            const int grp = tid + u * NTT, r = grp / (D / 8), c8 = 8 * (grp - r * (D / 8));
            in8<D, In>(p, cp, p.k, r, c8, k8[u]);
            ld8(gg + r * D + c8, g8[u]);
            ld8(gg + (C - 1) * D + c8, c8v[u]);
        }
#pragma unroll
        for (int u = 0; u < G8; ++u) {
            const int grp = tid + u * NTT, r = grp / (D / 8), c8 = 8 * (grp - r * (D / 8));
            if (PREP && p.qk_norm) unit8<D>(k8[u], 1.f);
#pragma unroll
            for (int j = 0; j < 8; ++j) k8[u][j] *= ex(c8v[u][j] - g8[u][j]);
            st8(rc + r * DP + c8, k8[u]);
        }
    }
    __syncthreads();
    // dU = P^T dO + Kb dS_C
    floatx4 dU[4];
#pragma unroll
    for (int ma = 0; ma < 4; ++ma) {
        floatx4 acc = zero4();
#pragma unroll
        for (int t = ma; t < 4; ++t) {
            const int r0 = 16 * t + 4 * g;
            const float4 a4 = make_float4(rp[(r0 + 0) * CP + 16 * ma + l], rp[(r0 + 1) * CP + 16 * ma + l],
                                          rp[(r0 + 2) * CP + 16 * ma + l], rp[(r0 + 3) * CP + 16 * ma + l]);
            acc = mma4(a4, f4(dO[t]), acc);
        }
#pragma unroll
        for (int t = 0; t < NT4; ++t) acc = mma4(ld4(rc + (16 * ma + l) * DP + 16 * t + 4 * g), dsb[t], acc);
        dU[ma] = acc;
    }
    // dW = Li^T dU;  dX = diag(beta) dW = dV;  dbeta (first part) = rowsum(dW X)
    floatx4 dX[4];
#pragma unroll
    for (int ma = 0; ma < 4; ++ma) {
        floatx4 acc = zero4();
#pragma unroll
        for (int t = ma; t < 4; ++t) {
            const int r0 = 16 * t + 4 * g;
            const float4 a4 = make_float4(rl[(r0 + 0) * CP + 16 * ma + l], rl[(r0 + 1) * CP + 16 * ma + l],
                                          rl[(r0 + 2) * CP + 16 * ma + l], rl[(r0 + 3) * CP + 16 * ma + l]);
            acc = mma4(a4, f4(dU[t]), acc);
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int r = 16 * ma + 4 * g + i;
            dX[ma][i] = sbeta[r] * acc[i];
            const float db = sum16(acc[i] * X[ma][i]);
            if (l == 0) db1p[wave * C + r] = db;
            if (r < cp.L) p.dv[elem<D>(p, cp, r, c)] = dX[ma][i];
        }
    }
    __syncthreads();  // Kb no longer read: dX takes its block
#pragma unroll
    for (int ma = 0; ma < 4; ++ma)
#pragma unroll
        for (int i = 0; i < 4; ++i) rc[(16 * ma + 4 * g + i) * DP + c] = dX[ma][i];
    __syncthreads();
    // dQt = dO S0^T, dKt = -dX S0^T, dKb = U dS_C^T: key channel c = 16 w + l as column
    floatx4 dQt[4], dKt[4], dKb[4];
#pragma unroll
    for (int ma = 0; ma < 4; ++ma) dQt[ma] = dKt[ma] = dKb[ma] = zero4();
#pragma unroll 2
    for (int t = 0; t < NT4; ++t) {
        const int v0 = 16 * t + 4 * g;
        const float4 bs = ld4(S0 + (int64_t)c * D + v0), bd = ld4(dSC + (int64_t)c * D + v0);
#pragma unroll
        for (int ma = 0; ma < 4; ++ma) {
            const int ro = (16 * ma + l) * DP + v0;
            dQt[ma] = mma4(ld4(rb + ro), bs, dQt[ma]);
            dKt[ma] = mma4(ld4(rc + ro), bs, dKt[ma]);
            dKb[ma] = mma4(ld4(ra + ro), bd, dKb[ma]);
        }
    }
    // dP = lower(dO U^T), into the P block (P is no longer read)
    for (int task = wave; task < 10; task += NW) {
        int a, bt;
        lower_block(task, a, bt);
        floatx4 acc = zero4();
#pragma unroll 4
        for (int t = 0; t < NT4; ++t)
            acc = mma4(ld4(rb + (16 * a + l) * DP + 16 * t + 4 * g), ld4(ra + (16 * bt + l) * DP + 16 * t + 4 * g), acc);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int r = 16 * a + 4 * g + i, s = 16 * bt + l;
            rp[r * CP + s] = s <= r ? acc[i] : 0.f;
        }
    }
    __syncthreads();  // U, dO, dX no longer read
    // dLinv = dU (diag(beta) X)^T, strictly lower part (only it reaches the free entries of A)
#pragma unroll
    for (int ma = 0; ma < 4; ++ma)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int r = 16 * ma + 4 * g + i;
            ra[r * DP + c] = dU[ma][i];
            rb[r * DP + c] = sbeta[r] * X[ma][i];
        }
    __syncthreads();
    for (int task = wave; task < 10; task += NW) {
        int a, bt;
        lower_block(task, a, bt);
        floatx4 acc = zero4();
#pragma unroll 4
        for (int t = 0; t < NT4; ++t)
            acc = mma4(ld4(ra + (16 * a + l) * DP + 16 * t + 4 * g), ld4(rb + (16 * bt + l) * DP + 16 * t + 4 * g), acc);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int r = 16 * a + 4 * g + i, s = 16 * bt + l;
            rq[r * CP + s] = s < r ? acc[i] : 0.f;
        }
    }
    for (int i = tid; i < C * C; i += NTT) {
        const int r = i / C, s = i - r * C;
        if (s / 16 > r / 16) rq[r * CP + s] = 0.f;
    }
    __syncthreads();
    // Z = dLinv Li^T (strictly lower part is all that dA reads), over the dU block
    float* rz = ra;  // pitch C + 4
    for (int task = wave; task < 10; task += NW) {
        int a, bt;
        lower_block(task, a, bt);
        floatx4 acc = zero4();
        for (int t = 0; t <= bt; ++t)
            acc = mma4(ld4(rq + (16 * a + l) * CP + 16 * t + 4 * g), ld4(rl + (16 * bt + l) * CP + 16 * t + 4 * g), acc);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int r = 16 * a + 4 * g + i, s = 16 * bt + l;
            rz[r * CP + s] = s < r ? acc[i] : 0.f;
        }
    }
    for (int i = tid; i < C * C; i += NTT) {
        const int r = i / C, s = i - r * C;
        if (s / 16 > r / 16) rz[r * CP + s] = 0.f;
    }
    __syncthreads();
    // dA = strict_lower(-Li^T Z), over the (beta X) block (pitch C + 4)
    float* rda = rb;
    for (int task = wave; task < 10; task += NW) {
        int mr, sb;
        lower_block(task, mr, sb);
        floatx4 acc = zero4();
        for (int t = mr; t < 4; ++t) {
            const int a0 = 16 * t + 4 * g;
            const float4 a4 = make_float4(rl[(a0 + 0) * CP + 16 * mr + l], rl[(a0 + 1) * CP + 16 * mr + l],
                                          rl[(a0 + 2) * CP + 16 * mr + l], rl[(a0 + 3) * CP + 16 * mr + l]);
            const float4 b4 = make_float4(rz[(a0 + 0) * CP + 16 * sb + l], rz[(a0 + 1) * CP + 16 * sb + l],
                                          rz[(a0 + 2) * CP + 16 * sb + l], rz[(a0 + 3) * CP + 16 * sb + l]);
            acc = mma4(a4, b4, acc);
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int r = 16 * mr + 4 * g + i, s = 16 * sb + l;
            rda[r * CP + s] = s < r ? -acc[i] : 0.f;
        }
    }
    for (int i = tid; i < C * C; i += NTT) {
        const int r = i / C, s = i - r * C;
        if (s / 16 > r / 16) rda[r * CP + s] = 0.f;
    }
    __syncthreads();
    // k, q and g of the chunk for the pair terms, over the blocks no longer read: g over
    // Z's, k over dX's, q over Li's (rows 0 .. 31) and dLinv's (rows 32 .. 63); pitch D
    float* sgg = ra;
    float* skk = rc;
    {
        float k8[G8][8], q8[G8][8], g8[G8][8];
#pragma unroll
        for (int u = 0; u < G8; ++u) {
            const int grp = tid + u * NTT, r = grp / (D / 8), c8 = 8 * (grp - r * (D / 8));
            in8<D, In>(p, cp, p.k, r, c8, k8[u]);
            in8<D, In>(p, cp, p.q, r, c8, q8[u]);
            ld8(gg + r * D + c8, g8[u]);
        }
#pragma unroll
        for (int u = 0; u < G8; ++u) {
            const int grp = tid + u * NTT, r = grp / (D / 8), c8 = 8 * (grp - r * (D / 8));
            const int i = r * D + c8;
            if (PREP && p.qk_norm) {
                const float ks = unit8<D>(k8[u], 1.f), qs = unit8<D>(q8[u], kInvSqrtD<D>);
                if (c8 == 0) {
                    sclk[r] = ks;
                    sclq[r] = qs;
                }
            }
            st8(sgg + i, g8[u]);
            st8(skk + i, k8[u]);
            st8(r < C / 2 ? rl + i : rq + (i - (C / 2) * D), q8[u]);
        }
    }
    // dbeta = rowsum(dW X) + rowsum(dA Bm): each row split over neighbouring threads, a
    // slice of its columns each (dA and Bm are zero on and above the diagonal)
    {
        constexpr int TPR = NTT / C, SPAN = C / TPR;  // threads per row, columns per thread
        static_assert(TPR * C == NTT && (TPR & (TPR - 1)) == 0 && SPAN % 4 == 0, "row split");
        const int r = tid / TPR, s0 = (tid % TPR) * SPAN;
        const float* bm = pr + PR::BM + r * C + s0;
        float acc = 0.f;
#pragma unroll
        for (int s4 = 0; s4 < SPAN; s4 += 4) {
            const float4 b4 = ld4(bm + s4), d4 = ld4(rda + r * CP + s0 + s4);
            acc = fmaf(d4.x, b4.x, acc);
            acc = fmaf(d4.y, b4.y, acc);
            acc = fmaf(d4.z, b4.z, acc);
            acc = fmaf(d4.w, b4.w, acc);
        }
#pragma unroll
        for (int m = 1; m < TPR; m <<= 1) acc += __shfl_xor(acc, m);
        if (tid % TPR == 0) {
            for (int w = 0; w < NW; ++w) acc += db1p[w * C + r];
            if (r < cp.L) p.dbeta[(cp.row0 + r) * p.H + cp.h] = acc;
        }
    }
    __syncthreads();
    // pair terms over F = diag(beta) dA (strictly lower) and dP (lower), key channel c:
    //   query side QP_r = sum_s dP_rs k_s e^{g_r - g_s},  QB_r = sum_s F_rs k_s e^{g_r - g_s}
    //   key side   KP_s = sum_r dP_rs q_r e^{g_r - g_s},  KB_s = sum_r F_rs k_r e^{g_r - g_s}
    // with the reference points of the chunk kernel's pair blocks
    auto gat = [&](int r) { return sgg[r * D + c]; };
    auto kin = [&](int r) { return skk[r * D + c]; };
    auto qin = [&](int r) { return r < C / 2 ? rl[r * D + c] : rq[(r - C / 2) * D + c]; };
    const float gC = gat(C - 1);
    float dg[4][4];
    float dgc = 0.f;
#pragma unroll
    for (int a = 0; a < 4; ++a) {
        // query side, row tile a: the earlier tiles against the end of tile a - 1, then the tile itself
        floatx4 QP = zero4(), QB = zero4();
        if (a > 0) {
            const float rho = gat(16 * a - 1);
            const float br = sbeta[16 * a + l];
            for (int t = 0; t < a; ++t) {
                const int s0 = 16 * t + 4 * g;
                const float4 k4 = make_float4(kin(s0) * ex(rho - gat(s0)), kin(s0 + 1) * ex(rho - gat(s0 + 1)),
                                              kin(s0 + 2) * ex(rho - gat(s0 + 2)), kin(s0 + 3) * ex(rho - gat(s0 + 3)));
                QP = mma4(ld4(rp + (16 * a + l) * CP + s0), k4, QP);
                const float4 f = ld4(rda + (16 * a + l) * CP + s0);
                QB = mma4(make_float4(br * f.x, br * f.y, br * f.z, br * f.w), k4, QB);
            }
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const float e = ex(gat(16 * a + 4 * g + i) - rho);
                QP[i] *= e;
                QB[i] *= e;
            }
        }
        {
            const float rho = gat(16 * a + 7);
            const int s0 = 16 * a + 4 * g;
            const float4 k4 = make_float4(kin(s0) * ex(rho - gat(s0)), kin(s0 + 1) * ex(rho - gat(s0 + 1)),
                                          kin(s0 + 2) * ex(rho - gat(s0 + 2)), kin(s0 + 3) * ex(rho - gat(s0 + 3)));
            const float br = sbeta[16 * a + l];
            const floatx4 dp = mma4(ld4(rp + (16 * a + l) * CP + s0), k4, zero4());
            const float4 f = ld4(rda + (16 * a + l) * CP + s0);
            const floatx4 db = mma4(make_float4(br * f.x, br * f.y, br * f.z, br * f.w), k4, zero4());
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const float e = ex(gat(16 * a + 4 * g + i) - rho);
                QP[i] += dp[i] * e;
                QB[i] += db[i] * e;
            }
        }
        // key side, column tile a: the later tiles against the end of tile a, then the tile itself
        floatx4 KP = zero4(), KB = zero4();
        if (a < 3) {
            const float rho = gat(16 * a + 15);
            for (int t = a + 1; t < 4; ++t) {
                const int r0 = 16 * t + 4 * g;
                float qv[4], kv[4], ap[4], af[4];
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const float e = ex(gat(r0 + j) - rho);
                    qv[j] = qin(r0 + j) * e;
                    kv[j] = kin(r0 + j) * e;
                    ap[j] = rp[(r0 + j) * CP + 16 * a + l];
                    af[j] = sbeta[r0 + j] * rda[(r0 + j) * CP + 16 * a + l];
                }
                KP = mma4(make_float4(ap[0], ap[1], ap[2], ap[3]), make_float4(qv[0], qv[1], qv[2], qv[3]), KP);
                KB = mma4(make_float4(af[0], af[1], af[2], af[3]), make_float4(kv[0], kv[1], kv[2], kv[3]), KB);
            }
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const float e = ex(rho - gat(16 * a + 4 * g + i));
                KP[i] *= e;
                KB[i] *= e;
            }
        }
        {
            const float rho = gat(16 * a + 7);
            const int r0 = 16 * a + 4 * g;
            float qv[4], kv[4], ap[4], af[4];
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const float e = ex(gat(r0 + j) - rho);
                qv[j] = qin(r0 + j) * e;
                kv[j] = kin(r0 + j) * e;
                ap[j] = rp[(r0 + j) * CP + 16 * a + l];
                af[j] = sbeta[r0 + j] * rda[(r0 + j) * CP + 16 * a + l];
            }
            const floatx4 dp =
                mma4(make_float4(ap[0], ap[1], ap[2], ap[3]), make_float4(qv[0], qv[1], qv[2], qv[3]), zero4());
            const floatx4 db =
                mma4(make_float4(af[0], af[1], af[2], af[3]), make_float4(kv[0], kv[1], kv[2], kv[3]), zero4());
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const float e = ex(rho - gat(16 * a + 4 * g + i));
                KP[i] += dp[i] * e;
                KB[i] += db[i] * e;
            }
        }
        // back to q, k and g for the rows of tile a
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int r = 16 * a + 4 * g + i;
            const float gr = gat(r), E = ex(gr), eb = ex(gC - gr), kv = kin(r), qv = qin(r);
            const float dqt = dQt[a][i] * E, dkt = -dKt[a][i] * E, dkb = dKb[a][i] * eb;
            const float dq = QP[i] + dqt;
            const float dk = QB[i] + KP[i] + KB[i] + dkt + dkb;
            dg[a][i] = qv * dq + kv * (QB[i] + dkt - KP[i] - KB[i] - dkb);
            dgc += kv * dkb;
            if (r < cp.L) {  // with the normalisation, the gradients of y: finished below
                const int64_t e = elem<D>(p, cp, r, c);
                p.dq[e] = dq;
                p.dk[e] = dk;
            }
        }
    }
    // log alpha's gradient: the reverse cumulative sum of g's, plus that of g_C
    dgc += __shfl_xor(dgc, 16);
    dgc += __shfl_xor(dgc, 32);
    {
        float dG = 0.f;
        for (int w = 0; w < NW; ++w) dG += dgcp[w * D + c];
        dgc += dG * ex(gC);
    }
    // log alpha as given (for the clamp's mask and the logits' derivative), every load issued
    // ahead of the gradient's stores
    const bool logits = PREP && p.logits;
    float xla[4][4];
#pragma unroll
    for (int ma = 0; ma < 4; ++ma)
#pragma unroll
        for (int i = 0; i < 4; ++i) xla[ma][i] = (p.clamp || logits) ? in(p.la, 16 * ma + 4 * g + i, c) : 0.f;
    // rows 16 ma + 4 g + i: suffix sums within the lane, then over the lane groups and blocks
    float tot[4];
#pragma unroll
    for (int ma = 0; ma < 4; ++ma) {
        float acc = 0.f;
#pragma unroll
        for (int i = 3; i >= 0; --i) {
            acc += dg[ma][i];
            dg[ma][i] = acc;
        }
        tot[ma] = acc;
    }
    float later = dgc;  // the sum over every row after the current block, plus dg_C
#pragma unroll
    for (int ma = 3; ma >= 0; --ma) {
        const float t0 = __shfl(tot[ma], l), t1 = __shfl(tot[ma], 16 + l), t2 = __shfl(tot[ma], 32 + l),
                    t3 = __shfl(tot[ma], 48 + l);
        const float after_g = g == 0 ? t1 + t2 + t3 : g == 1 ? t2 + t3 : g == 2 ? t3 : 0.f;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int r = 16 * ma + 4 * g + i;
            if (r < cp.L) {
                const int64_t e = elem<D>(p, cp, r, c);
                float d = dg[ma][i] + after_g + later;
                if (p.clamp || logits) {
                    const float x = xla[ma][i];
                    const float lv = logits ? log_sigmoid(x) : x;  // log alpha before the clamp
                    if (p.clamp && !(lv >= kLogAlphaMin && lv <= 0.f)) d = 0.f;
                    if (logits) d *= sigmoidf_(-x);                 // d logsigmoid(x) / dx
                }
                p.dla[e] = d;
            }
        }
        later += t0 + t1 + t2 + t3;
    }
    if (PREP && p.qk_norm) {
        // back through the normalisation, a token's channels eight to a lane as in the
        // staging: dx = s (dy - c^2 y (y . dy)) for y = s x, s = 1 / (c |x|) (c = sqrt(D)
        // for q, 1 for k), dy read back from the outputs once every wave has written them
        __syncthreads();
#pragma unroll
        for (int u = 0; u < G8; ++u) {
            const int grp = tid + u * NTT, r = grp / (D / 8), c8 = 8 * (grp - r * (D / 8));
            if (r < cp.L) {  // uniform over the D / 8 lanes of a token
                const int64_t e = elem<D>(p, cp, r, c8);
                float dq8[8], dk8[8], yq[8], yk[8];
                ld8(p.dq + e, dq8);
                ld8(p.dk + e, dk8);
                ld8(r < C / 2 ? rl + r * D + c8 : rq + (r - C / 2) * D + c8, yq);
                ld8(skk + r * D + c8, yk);
                float pq = 0.f, pk = 0.f;
#pragma unroll
                for (int j = 0; j < 8; ++j) {
                    pq = fmaf(yq[j], dq8[j], pq);
                    pk = fmaf(yk[j], dk8[j], pk);
                }
                pq = token_sum<D>(pq) * (float)D;
                pk = token_sum<D>(pk);
                const float sq = sclq[r], sk = sclk[r];
#pragma unroll
                for (int j = 0; j < 8; ++j) {
                    dq8[j] = sq * (dq8[j] - yq[j] * pq);
                    dk8[j] = sk * (dk8[j] - yk[j] * pk);
                }
                st8(p.dq + e, dq8);
                st8(p.dk + e, dk8);
            }
        }
    }
}

int64_t align256(int64_t x) { return (x + 255) / 256 * 256; }

// Workspace sections: the sweep's record per chunk, the pair record per chunk, the state
// at every chunk start and the state gradient at every chunk end (each 256-byte aligned).
template <int D>
int64_t section_bytes(int64_t bh, int64_t nc, int64_t* trans, int64_t* pairs, int64_t* states) {
    const int64_t items = bh * nc;
    *trans = align256(items * Rec<D>::SIZE * 4);
    *pairs = align256(items * Pr<D>::SIZE * 4);
    *states = align256(items * (int64_t)D * D * 4);
    return *trans + *pairs + 2 * *states;
}

template <int D, class In, bool PREP>
hipError_t launch_d(const BwdParams& p, hipStream_t stream) {
    const int64_t items = p.vs ? p.NC * p.H : p.B * p.H * p.NC;  // one workgroup per chunk item
    constexpr int NTC = 64 * (D / 16);
    if (items > 0) {
        auto kc = kda_bwd_chunk_kernel<D, In, PREP>;
        constexpr int lds = ChunkL<D>::TOTAL * 4;
        hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kc),
                                           hipFuncAttributeMaxDynamicSharedMemorySize, lds);
        if (e != hipSuccess) return e;
        hipLaunchKernelGGL(kc, dim3((unsigned)items), dim3(NTC), lds, stream, p);
        e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    const int64_t bh = p.B * p.H;
    if (bh > 0) {
        auto ks = kda_bwd_sweep_kernel<D>;
        constexpr int lds = SweepLds<D>::TOTAL * 4;
        hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(ks),
                                           hipFuncAttributeMaxDynamicSharedMemorySize, lds);
        if (e != hipSuccess) return e;
        static_assert((2 * (D / TILE)) % 8 == 0, "the sweep grid is a multiple of 8 (XCD mapping)");
        hipLaunchKernelGGL(ks, dim3((unsigned)(2 * bh * (D / TILE))), dim3(NT), lds, stream, p);
        e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    if (items > 0) {
        auto kg = kda_bwd_grad_kernel<D, In, PREP>;
        constexpr int lds = GradL<D>::TOTAL * 4;
        hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kg),
                                           hipFuncAttributeMaxDynamicSharedMemorySize, lds);
        if (e != hipSuccess) return e;
        hipLaunchKernelGGL(kg, dim3((unsigned)items), dim3(NTC), lds, stream, p);
    }
    return hipGetLastError();
}

}  // namespace

int64_t bwd_workspace_bytes(int D, int64_t bh, int64_t nc) {
    int64_t t, r, s;
    return D == 64 ? section_bytes<64>(bh, nc, &t, &r, &s) : section_bytes<128>(bh, nc, &t, &r, &s);
}

void bwd_layout(int D, int64_t bh, int64_t nc, void* ws, BwdParams& p) {
    int64_t t, r, s;
    if (D == 64)
        section_bytes<64>(bh, nc, &t, &r, &s);
    else
        section_bytes<128>(bh, nc, &t, &r, &s);
    unsigned char* w = static_cast<unsigned char*>(ws);
    p.trans = reinterpret_cast<float*>(w);
    p.pairs = reinterpret_cast<float*>(w + t);
    p.states = reinterpret_cast<float*>(w + t + r);
    p.dstates = reinterpret_cast<float*>(w + t + r + s);
}

template <bool PREP>
hipError_t launch_prep(int dtype_bf16, int D, const BwdParams& p, hipStream_t stream) {
    if (D == 64) return dtype_bf16 ? launch_d<64, InBF16, PREP>(p, stream) : launch_d<64, InF32, PREP>(p, stream);
    return dtype_bf16 ? launch_d<128, InBF16, PREP>(p, stream) : launch_d<128, InF32, PREP>(p, stream);
}

hipError_t launch_bwd(int dtype_bf16, int D, const BwdParams& p, hipStream_t stream) {
    return p.qk_norm || p.logits ? launch_prep<true>(dtype_bf16, D, p, stream)
                                 : launch_prep<false>(dtype_bf16, D, p, stream);
}

}  // namespace kda
