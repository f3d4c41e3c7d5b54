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
// Every pair factor is e^{g_r - g_s} with r >= s, so none exceeds 1.
//
// Three launches:
//  1. kda_bwd_prep_kernel, one chunk per workgroup: W = Li diag(beta) Kt, Kb, Gc,
//     b = Kb^T Li diag(beta) V and R = (Qt - P W)^T dO with dO = dY * sigmoid(Z).
//  2. kda_bwd_sweep_kernel, one (direction, b, h, 16 value columns) per workgroup
//     (columns of the state evolve independently): forwards the states at every
//     chunk start, S_{n+1} = Diag(Gc) S_n - Kb^T (W S_n) + b; backwards the state
//     gradients, dS_n = Diag(Gc) dS_{n+1} - W^T (Kb dS_{n+1}) + R (the transposed
//     map).  R does not depend on the states, so the two directions run at once.
//  3. kda_bwd_grad_kernel, one chunk per workgroup: the adjoint of the chunk's
//     steps above from S_n and dS_{n+1}; log alpha's gradient is the reverse
//     cumulative sum of g's gradient within the chunk.
// All arithmetic is fp32; the chunk kernels keep their intermediates in a scratch
// slot of the workspace (one per workgroup, reused chunk after chunk).  When every
// chunk has a slot of its own, the gradient kernel finds the shared per-chunk steps
// where the prep kernel left them instead of recomputing them.
#include "kda_backward.h"
#include "kda_device.h"

namespace kda {
namespace {

constexpr int C = 64;             // tokens per chunk
constexpr int NT = 256;           // threads per workgroup
constexpr int TILE = 16;          // value columns per sweep workgroup
constexpr int64_t kMaxSlots = 512;

__device__ __forceinline__ float ex(float x) { return fast_exp2(x * kLog2e); }

// fp32 offsets of the per-chunk record written by the prep kernel.
template <int D>
struct Rec {
    static constexpr int64_t CD = (int64_t)C * D, DD = (int64_t)D * D;
    static constexpr int64_t W = 0, KBAR = CD, BV = 2 * CD, R = 2 * CD + DD, GC = 2 * CD + 2 * DD;
    static constexpr int64_t SIZE = 2 * CD + 2 * DD + D;
};

// fp32 offsets inside one scratch slot: C x D row-major blocks, then C x C blocks,
// then two C-vectors.
template <int D>
struct Scr {
    static constexpr int64_t CD = (int64_t)C * D, CC = (int64_t)C * C;
    static constexpr int64_t K = 0, Q = CD, V = 2 * CD, G = 3 * CD, DO = 4 * CD, EG = 5 * CD, KT = 6 * CD,
                             QT = 7 * CD, KB = 8 * CD, X = 9 * CD, U = 10 * CD, O = 11 * CD, DU = 12 * CD,
                             DW = 13 * CD, DKB = 14 * CD, DQ = 15 * CD, DKT = 16 * CD;
    static constexpr int64_t BM = 17 * CD, PM = BM + CC, LI = BM + 2 * CC, DP = BM + 3 * CC,
                             DLI = BM + 4 * CC, EM = BM + 5 * CC, DA = BM + 6 * CC;
    static constexpr int64_t BETA = BM + 7 * CC, DBX = BETA + C;
    static constexpr int64_t SIZE = DBX + C;
};

// out(m, n) for m < M, n < N of sum_{k < K} a(m, k) b(k, n) over the workgroup, on
// the fp32 MFMA.  A and B are first copied into LDS (row pitches K + 4 and N + 4, so
// the lane groups of an operand read fall on different banks), in the order of their
// sources' contiguous index (TA, TB: that source is stored transposed), one element
// per lane and step or (V4) four neighbours per lane merged into a 16-byte load.  Wave w then
// forms the 16 x 16 output tiles w, w + 4, ..: lane (l, g) gives A[l][k] and B[k][l] for
// k = 16 kk + 4 g + c in the c-th MFMA of a 16-wide k step and receives
// out[4 g + i][l] in acc[i].  Starts with a barrier (LDS free) and ends without one.
template <int D, int M, int N, int K, bool TA = false, bool TB = false, bool V4 = false, class FA, class FB,
          class FO>
__device__ __forceinline__ void mm(FA a, FB b, FO o, float* lds) {
    constexpr int KP = K + 4, NP = N + 4;
    static_assert(M % 16 == 0 && N % 16 == 0 && K % 16 == 0, "16 x 16 tiles");
    static_assert(M * KP + K * NP <= 3 * C * D + 2 * C * C, "fits the chunk kernels' LDS");
    float* la = lds;
    float* lb = lds + M * KP;
    __syncthreads();
    if (V4) {
        // each lane copies four neighbours along the source's contiguous index, which the
        // compiler merges into one 16-byte load
        constexpr int NA = TA ? M * K / 16 : M * K / 4, NB4 = TB ? K * N / 16 : K * N / 4;
#pragma unroll 2
        for (int i = threadIdx.x; i < NA; i += NT) {
            if (TA) {
                // a(m, k) is read from a k-major source: a 4 x 4 block per lane, four
                // 16-byte loads along m, transposed in registers into four rows of LDS
                const int k = 4 * (i / (M / 4)), m = 4 * (i - (i / (M / 4)) * (M / 4));
                float v[4][4];
#pragma unroll
                for (int t = 0; t < 4; ++t)
#pragma unroll
                    for (int j = 0; j < 4; ++j) v[t][j] = a(m + j, k + t);
#pragma unroll
                for (int j = 0; j < 4; ++j)
                    *reinterpret_cast<float4*>(la + (m + j) * KP + k) = make_float4(v[0][j], v[1][j], v[2][j], v[3][j]);
            } else {
                const int m = i / (K / 4), k = 4 * (i - m * (K / 4));
                *reinterpret_cast<float4*>(la + m * KP + k) = make_float4(a(m, k), a(m, k + 1), a(m, k + 2), a(m, k + 3));
            }
        }
#pragma unroll 2
        for (int i = threadIdx.x; i < NB4; i += NT) {
            if (TB) {
                // b(k, n) is read from an n-major source: a 4 x 4 block per lane, four
                // 16-byte loads along k, transposed in registers into four rows of LDS
                const int n = 4 * (i / (K / 4)), k = 4 * (i - (i / (K / 4)) * (K / 4));
                float v[4][4];
#pragma unroll
                for (int t = 0; t < 4; ++t)
#pragma unroll
                    for (int j = 0; j < 4; ++j) v[t][j] = b(k + j, n + t);
#pragma unroll
                for (int j = 0; j < 4; ++j)
                    *reinterpret_cast<float4*>(lb + (k + j) * NP + n) = make_float4(v[0][j], v[1][j], v[2][j], v[3][j]);
            } else {
                const int k = i / (N / 4), n = 4 * (i - k * (N / 4));
                *reinterpret_cast<float4*>(lb + k * NP + n) = make_float4(b(k, n), b(k, n + 1), b(k, n + 2), b(k, n + 3));
            }
        }
    } else {
        // one element per lane and step, consecutive lanes along the source's contiguous index
#pragma unroll 8
        for (int i = threadIdx.x; i < M * K; i += NT) {
            const int m = TA ? i % M : i / K, k = TA ? i / M : i % K;
            la[m * KP + k] = a(m, k);
        }
#pragma unroll 8
        for (int i = threadIdx.x; i < K * N; i += NT) {
            const int k = TB ? i % K : i / N, n = TB ? i / K : i % N;
            lb[k * NP + n] = b(k, n);
        }
    }
    __syncthreads();
    const int lane = lane_id(), wave = wave_id();
    const int l = lane & 15, g = lane >> 4;
    constexpr int TN = N / 16, TILES = (M / 16) * TN;
    for (int t = wave; t < TILES; t += NT / 64) {
        const int tm = t / TN, tn = t - tm * TN;
        floatx4 acc = zero4();
#pragma unroll 4
        for (int kk = 0; kk < K / 16; ++kk) {
            const int k0 = 16 * kk + 4 * g;
            const float4 av = *reinterpret_cast<const float4*>(la + (16 * tm + l) * KP + k0);
            const float* bp = lb + k0 * NP + 16 * tn + l;
            acc = mma_f32_k4(av.x, bp[0], acc);
            acc = mma_f32_k4(av.y, bp[NP], acc);
            acc = mma_f32_k4(av.z, bp[2 * NP], acc);
            acc = mma_f32_k4(av.w, bp[3 * NP], acc);
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) o(16 * tm + 4 * g + i, 16 * tn + l, acc[i]);
    }
}

struct ChunkPos {
    int64_t b, h, t0;
    int L;  // tokens of the chunk inside the sequence (the rest is padding)
};

__device__ __forceinline__ ChunkPos chunk_pos(const BwdParams& p, int64_t item) {
    ChunkPos cp;
    const int64_t bh = item / p.NC, n = item - bh * p.NC;
    cp.b = bh / p.H;
    cp.h = bh - cp.b * p.H;
    cp.t0 = n * C;
    cp.L = (int)(p.T - cp.t0 < C ? p.T - cp.t0 : C);
    return cp;
}

template <int D>
__device__ __forceinline__ int64_t elem(const BwdParams& p, const ChunkPos& cp, int r, int c) {
    return ((cp.b * p.T + cp.t0 + r) * p.H + cp.h) * D + c;
}

// LDS of the chunk kernels (fp32 offsets).  The pair products and the inverse read
// three channel-major C x D blocks and two C x C blocks; the gradient's pair terms
// read three row-major C x D blocks, two C x C blocks and beta.
template <int D>
struct ChunkLds {
    static constexpr int CP = C + 4;  // pitch of the channel-major copies (bank spread)
    static constexpr int CC = C * C, DCP = D * CP;
    static constexpr int A0 = 0, A1 = DCP, A2 = 2 * DCP, B0 = 3 * DCP, B1 = 3 * DCP + CC, BETA = 3 * DCP + 2 * CC;
    static constexpr int TOTAL = BETA + C;
};

// dst[c * (C + 4) + r] = src[r * D + c] for a C x D row-major block of scratch: a 4 x 4
// block per lane and step, four 16-byte loads along the channels, four 16-byte LDS
// stores along the tokens.
template <int D>
__device__ __forceinline__ void to_lds_cm(float* dst, const float* src) {
    constexpr int CP = C + 4;
    for (int i = threadIdx.x; i < (C / 4) * (D / 4); i += NT) {
        const int rb = i / (D / 4), c = 4 * (i - rb * (D / 4)), r = 4 * rb;
        float4 v[4];
#pragma unroll
        for (int t = 0; t < 4; ++t) v[t] = *reinterpret_cast<const float4*>(src + (r + t) * D + c);
        *reinterpret_cast<float4*>(dst + (c + 0) * CP + r) = make_float4(v[0].x, v[1].x, v[2].x, v[3].x);
        *reinterpret_cast<float4*>(dst + (c + 1) * CP + r) = make_float4(v[0].y, v[1].y, v[2].y, v[3].y);
        *reinterpret_cast<float4*>(dst + (c + 2) * CP + r) = make_float4(v[0].z, v[1].z, v[2].z, v[3].z);
        *reinterpret_cast<float4*>(dst + (c + 3) * CP + r) = make_float4(v[0].w, v[1].w, v[2].w, v[3].w);
    }
}

// Copies n floats (a multiple of 4 * NT) from global scratch to LDS, all loads of a
// thread issued before its stores.
template <int N>
__device__ __forceinline__ void to_lds(float* dst, const float* src) {
    constexpr int per = N / 4 / NT;
    float4 v[per];
#pragma unroll
    for (int i = 0; i < per; ++i) v[i] = reinterpret_cast<const float4*>(src)[threadIdx.x + i * NT];
#pragma unroll
    for (int i = 0; i < per; ++i) reinterpret_cast<float4*>(dst)[threadIdx.x + i * NT] = v[i];
}

// Eight consecutive input elements as fp32 (e is a multiple of 8, so the bf16 load is
// 16-byte aligned and the fp32 loads 32-byte aligned), and eight fp32 to scratch.
__device__ __forceinline__ void load8(const uint16_t* p, int64_t e, float (&o)[8]) {
    const uint4 w = *reinterpret_cast<const uint4*>(p + e);
    const uint32_t ws[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
    for (int j = 0; j < 4; ++j) {  // little-endian: element 2 j is the low half-word
        o[2 * j] = __uint_as_float(ws[j] << 16);
        o[2 * j + 1] = __uint_as_float(ws[j] & 0xffff0000u);
    }
}
__device__ __forceinline__ void load8(const float* p, int64_t e, float (&o)[8]) {
    const float4 a = *reinterpret_cast<const float4*>(p + e);
    const float4 b = *reinterpret_cast<const float4*>(p + e + 4);
    o[0] = a.x, o[1] = a.y, o[2] = a.z, o[3] = a.w, o[4] = b.x, o[5] = b.y, o[6] = b.z, o[7] = b.w;
}
__device__ __forceinline__ void store8(float* d, const float (&v)[8]) {
    *reinterpret_cast<float4*>(d) = make_float4(v[0], v[1], v[2], v[3]);
    *reinterpret_cast<float4*>(d + 4) = make_float4(v[4], v[5], v[6], v[7]);
}

// Steps shared by the prep and gradient kernels: the chunk's inputs in fp32 (zero
// past the sequence's end, which makes the padding tokens identity steps), g, the
// decayed operands, Bm, P and Li.
template <int D, class In>
__device__ void chunk_common(const BwdParams& p, const ChunkPos& cp, float* s, float* lds) {
    using S = Scr<D>;
    using LL = ChunkLds<D>;
    using raw = typename In::raw_t;
    // eight neighbouring channels of one token per lane and step (one 16-byte load per
    // bf16 input), two steps in flight
    constexpr int G8 = C * D / 8 / NT;  // groups of eight per thread
    static_assert(G8 % 2 == 0, "pairs of groups");
#pragma unroll 1
    for (int g0 = 0; g0 < G8; g0 += 2) {
        float k8[2][8], q8[2][8], v8[2][8], l8[2][8], y8[2][8], z8[2][8];
#pragma unroll
        for (int u = 0; u < 2; ++u) {
            const int grp = threadIdx.x + (g0 + u) * NT;
            const int r = grp / (D / 8), c8 = 8 * (grp - r * (D / 8));
            if (r < cp.L) {
                const int64_t e = elem<D>(p, cp, r, c8);
                load8(static_cast<const raw*>(p.k), e, k8[u]);
                load8(static_cast<const raw*>(p.q), e, q8[u]);
                load8(static_cast<const raw*>(p.v), e, v8[u]);
                load8(static_cast<const raw*>(p.la), e, l8[u]);
                load8(static_cast<const raw*>(p.dy), e, y8[u]);
                load8(static_cast<const raw*>(p.gate), e, z8[u]);
            } else {
#pragma unroll
                for (int j = 0; j < 8; ++j) k8[u][j] = q8[u][j] = v8[u][j] = l8[u][j] = y8[u][j] = z8[u][j] = 0.f;
            }
        }
#pragma unroll
        for (int u = 0; u < 2; ++u) {
            const int grp = threadIdx.x + (g0 + u) * NT;
            const int r = grp / (D / 8), c8 = 8 * (grp - r * (D / 8));
            const bool live = r < cp.L;
            float lv[8], dov[8];
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                lv[j] = live ? clamp_log_alpha(l8[u][j], p.clamp != 0) : 0.f;
                dov[j] = live ? y8[u][j] * sigmoidf_(z8[u][j]) : 0.f;
            }
            const int idx = r * D + c8;
            store8(s + S::K + idx, k8[u]);
            store8(s + S::Q + idx, q8[u]);
            store8(s + S::V + idx, v8[u]);
            store8(s + S::G + idx, lv);
            store8(s + S::DO + idx, dov);
        }
    }
    if (threadIdx.x < C) {
        const int r = threadIdx.x;
        const float b =
            r < cp.L ? In::load(static_cast<const raw*>(p.beta), (cp.b * p.T + cp.t0 + r) * p.H + cp.h) : 0.f;
        s[S::BETA + r] = b;
        lds[LL::BETA + r] = b;
    }
    __syncthreads();
    // g_r = sum_{s <= r} lambda_s, per key channel (the column read whole, then summed)
    if (threadIdx.x < D) {
        const int c = threadIdx.x;
        float acc = 0.f;
#pragma unroll 1
        for (int r0 = 0; r0 < C; r0 += 16) {
            float col[16];
#pragma unroll
            for (int u = 0; u < 16; ++u) col[u] = s[S::G + (r0 + u) * D + c];
#pragma unroll
            for (int u = 0; u < 16; ++u) {
                acc += col[u];
                s[S::G + (r0 + u) * D + c] = acc;
            }
        }
    }
    __syncthreads();
    to_lds_cm<D>(lds + LL::A0, s + S::K);
    to_lds_cm<D>(lds + LL::A1, s + S::Q);
    to_lds_cm<D>(lds + LL::A2, s + S::G);
    // decayed operands, eight neighbouring channels per lane and step
#pragma unroll 2
    for (int grp = threadIdx.x; grp < C * D / 8; grp += NT) {
        const int idx = 8 * grp, c8 = idx % D;
        float g[8], gc[8], kv[8], qv[8], eg[8], kt[8], qt[8], kb[8];
        load8(s + S::G + idx, 0, g);
        load8(s + S::G + (C - 1) * D + c8, 0, gc);
        load8(s + S::K + idx, 0, kv);
        load8(s + S::Q + idx, 0, qv);
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            eg[j] = ex(g[j]);
            kt[j] = kv[j] * eg[j];
            qt[j] = qv[j] * eg[j];
            kb[j] = kv[j] * ex(gc[j] - g[j]);
        }
        store8(s + S::EG + idx, eg);
        store8(s + S::KT + idx, kt);
        store8(s + S::QT + idx, qt);
        store8(s + S::KB + idx, kb);
    }
    __syncthreads();
    // pair products from LDS: channel-major k (A0), q (A1) and g (A2), row pitch C + 4
    for (int idx = threadIdx.x; idx < C * C; idx += NT) {
        const int r = idx / C, sc = idx - r * C;
        float bs = 0.f, ps = 0.f;
        if (sc <= r) {
#pragma unroll 8
            for (int c = 0; c < D; ++c) {
                const float e = ex(lds[LL::A2 + c * LL::CP + r] - lds[LL::A2 + c * LL::CP + sc]);
                const float ks = lds[LL::A0 + c * LL::CP + sc] * e;
                bs = fmaf(lds[LL::A0 + c * LL::CP + r], ks, bs);
                ps = fmaf(lds[LL::A1 + c * LL::CP + r], ks, ps);
            }
        }
        const float bm = sc < r ? bs : 0.f;
        s[S::BM + idx] = bm;
        s[S::PM + idx] = sc <= r ? ps : 0.f;
        lds[LL::B0 + idx] = bm;
    }
    __syncthreads();
    // Li = (I + diag(beta) Bm)^-1 by forward substitution in LDS, one column per lane
    if (threadIdx.x < C) {
        const int sc = threadIdx.x;
        float* li = lds + LL::B1;
        for (int r = 0; r < C; ++r) {
            float acc = 0.f;
            for (int m = 0; m < r; ++m) acc = fmaf(lds[LL::B0 + r * C + m], li[m * C + sc], acc);
            const float v = r == sc ? 1.f : (r < sc ? 0.f : -lds[LL::BETA + r] * acc);
            li[r * C + sc] = v;
            s[S::LI + r * C + sc] = v;
        }
    }
    __syncthreads();
}

template <int D, class In>
__global__ __launch_bounds__(NT) void kda_bwd_prep_kernel(BwdParams p) {
    using S = Scr<D>;
    extern __shared__ __align__(16) float lds[];
    using RC = Rec<D>;
    float* s = p.scratch + (int64_t)blockIdx.x * S::SIZE;
    const int64_t items = p.B * p.H * p.NC;
    for (int64_t item = blockIdx.x; item < items; item += gridDim.x) {
        const ChunkPos cp = chunk_pos(p, item);
        chunk_common<D, In>(p, cp, s, lds);
        float* tr = p.trans + item * RC::SIZE;
        const float* beta = s + S::BETA;
        // W = Li diag(beta) Kt;  U~ = Li diag(beta) V (kept in the X block)
        mm<D, C, D, C>([&](int m, int k) { return s[S::LI + m * C + k] * beta[k]; },
                    [&](int k, int n) { return s[S::KT + k * D + n]; },
                    [&](int m, int n, float a) { tr[RC::W + m * D + n] = a; }, lds);
        mm<D, C, D, C>([&](int m, int k) { return s[S::LI + m * C + k] * beta[k]; },
                    [&](int k, int n) { return s[S::V + k * D + n]; },
                    [&](int m, int n, float a) { s[S::X + m * D + n] = a; }, lds);
        for (int idx = threadIdx.x; idx < C * D; idx += NT) tr[RC::KBAR + idx] = s[S::KB + idx];
        if (threadIdx.x < D) tr[RC::GC + threadIdx.x] = s[S::EG + (C - 1) * D + threadIdx.x];
        __syncthreads();
        // Qe = Qt - P W (kept in the U block);  b = Kb^T U~
        mm<D, C, D, C>([&](int m, int k) { return s[S::PM + m * C + k]; },
                    [&](int k, int n) { return tr[RC::W + k * D + n]; },
                    [&](int m, int n, float a) { s[S::U + m * D + n] = s[S::QT + m * D + n] - a; }, lds);
        mm<D, D, D, C, true, false>([&](int m, int k) { return s[S::KB + k * D + m]; },
                    [&](int k, int n) { return s[S::X + k * D + n]; },
                    [&](int m, int n, float a) { tr[RC::BV + m * D + n] = a; }, lds);
        __syncthreads();
        // R = Qe^T dO
        mm<D, D, D, C, true, false>([&](int m, int k) { return s[S::U + k * D + m]; },
                    [&](int k, int n) { return s[S::DO + k * D + n]; },
                    [&](int m, int n, float a) { tr[RC::R + m * D + n] = a; }, lds);
        __syncthreads();  // the slot is reused by the next chunk
    }
}

// LDS of the sweep kernel (fp32 offsets): the chunk's W and K-bar (row pitch D + 4),
// the 16 columns of its offset (b forwards, R backwards), Gamma_C, the state tile and
// Y (row pitch 20).  The pitches put the four lane groups of an MFMA operand read on
// disjoint banks.
template <int D>
struct SweepLds {
    static constexpr int DP = D + 4, TP = 20;
    static constexpr int W = 0, KBAR = C * DP, OFF = 2 * C * DP, GC = OFF + D * TP, ST = GC + D,
                         Y = ST + D * TP, TOTAL = Y + C * TP;
    static constexpr int NW4 = C * D / 4 / NT;    // float4 of W (and of K-bar) per thread
    static constexpr int NO4 = D * TILE / 4 / NT; // float4 of the offset tile per thread
};

// 16 k-steps of the fp32 MFMA: lane (m, g) gives A[m][k] and B[k][m] for
// k = 16 kk + 4 g + c, c = 0..3, and accumulates D[4 g + i][m] in acc[i].
__device__ __forceinline__ floatx4 mma16x4(const float (&a)[4], const float (&b)[4], floatx4 acc) {
#pragma unroll
    for (int c = 0; c < 4; ++c) acc = mma_f32_k4(a[c], b[c], acc);
    return acc;
}

// Forwards: S <- Diag(Gc) S - Kb^T (W S) + b; backwards: dS <- Diag(Gc) dS - W^T (Kb dS) + R.
// One workgroup runs one direction.  Both products run on the fp32 MFMA: wave w
// forms rows 16 w .. 16 w + 15 of Y, then row blocks w, w + 4, .. of the new state.
// The record of the next chunk is read into registers while the current one is used.
template <int D>
__global__ __launch_bounds__(NT) void kda_bwd_sweep_kernel(BwdParams p) {
    using RC = Rec<D>;
    using L = SweepLds<D>;
    constexpr int DP = L::DP, TP = L::TP;
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
    const float* rec0 = p.trans + bh * p.NC * RC::SIZE;
    const int lane = lane_id(), wave = wave_id();
    const int m = lane & 15, g = lane >> 4;
    // the next chunk's W, K-bar, offset tile and Gamma_C, in registers
    float4 rw[L::NW4], rk[L::NW4], ro[L::NO4];
    float4 rg = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
    for (int i = 0; i < L::NW4; ++i) rw[i] = rk[i] = rg;
#pragma unroll
    for (int i = 0; i < L::NO4; ++i) ro[i] = rg;
    auto fetch = [&](const float* tr, int64_t off_base) {
        const float4* w4 = reinterpret_cast<const float4*>(tr + RC::W);
        const float4* k4 = reinterpret_cast<const float4*>(tr + RC::KBAR);
#pragma unroll
        for (int i = 0; i < L::NW4; ++i) {
            rw[i] = w4[threadIdx.x + i * NT];
            rk[i] = k4[threadIdx.x + i * NT];
        }
#pragma unroll
        for (int i = 0; i < L::NO4; ++i) {
            const int q = threadIdx.x + i * NT;  // row q / 4, columns col0 + 4 (q % 4) ..
            ro[i] = *reinterpret_cast<const float4*>(tr + off_base + (q >> 2) * D + col0 + 4 * (q & 3));
        }
        if (threadIdx.x < D / 4) rg = reinterpret_cast<const float4*>(tr + RC::GC)[threadIdx.x];
    };
    auto stage = [&]() {
#pragma unroll
        for (int i = 0; i < L::NW4; ++i) {
            const int q = threadIdx.x + i * NT;  // row q / (D / 4), columns 4 (q % (D / 4)) ..
            const int at = (q / (D / 4)) * DP + 4 * (q % (D / 4));
            *reinterpret_cast<float4*>(lds + L::W + at) = rw[i];
            *reinterpret_cast<float4*>(lds + L::KBAR + at) = rk[i];
        }
#pragma unroll
        for (int i = 0; i < L::NO4; ++i) {
            const int q = threadIdx.x + i * NT;
            *reinterpret_cast<float4*>(lds + L::OFF + (q >> 2) * TP + 4 * (q & 3)) = ro[i];
        }
        if (threadIdx.x < D / 4) reinterpret_cast<float4*>(lds + L::GC)[threadIdx.x] = rg;
    };
    {
        const float* init = dir == 0 ? p.s0 : p.dsT;
        for (int idx = threadIdx.x; idx < D * TILE; idx += NT) {
            const int c = idx / TILE, j = idx - c * TILE;
            St[c * TP + j] = init ? init[bh * DD + c * D + col0 + j] : 0.f;
        }
        const int64_t off_base = dir == 0 ? RC::BV : RC::R;
        if (p.NC > 0) fetch(rec0 + (dir == 0 ? 0 : p.NC - 1) * RC::SIZE, off_base);
        for (int64_t i = 0; i < p.NC; ++i) {
            const int64_t n = dir == 0 ? i : p.NC - 1 - i;
            __syncthreads();  // the previous chunk's operands are no longer read
            stage();
            __syncthreads();
            if (i + 1 < p.NC) fetch(rec0 + (dir == 0 ? n + 1 : n - 1) * RC::SIZE, off_base);
            float* out = (dir == 0 ? p.states : p.dstates) + (bh * p.NC + n) * DD;
            for (int idx = threadIdx.x; idx < D * TILE; idx += NT) {
                const int c = idx / TILE, j = idx - c * TILE;
                out[c * D + col0 + j] = St[c * TP + j];
            }
            // Y = W S (forwards) or Kb dS (backwards): wave w owns rows 16 w ..
            const float* A1 = lds + (dir == 0 ? L::W : L::KBAR);
            const float* A2 = lds + (dir == 0 ? L::KBAR : L::W);
            {
                floatx4 acc = zero4();
#pragma unroll
                for (int kk = 0; kk < D / 16; ++kk) {
                    const int k0 = 16 * kk + 4 * g;
                    const float4 av = *reinterpret_cast<const float4*>(A1 + (16 * wave + m) * DP + k0);
                    const float a[4] = {av.x, av.y, av.z, av.w};
                    const float b[4] = {St[(k0 + 0) * TP + m], St[(k0 + 1) * TP + m], St[(k0 + 2) * TP + m],
                                        St[(k0 + 3) * TP + m]};
                    acc = mma16x4(a, b, acc);
                }
#pragma unroll
                for (int r = 0; r < 4; ++r) Y[(16 * wave + 4 * g + r) * TP + m] = acc[r];
            }
            __syncthreads();
            // state <- Diag(Gc) state - A2^T Y + offset, row blocks wave, wave + 4, ..
            for (int rb = wave; rb < D / 16; rb += NT / 64) {
                floatx4 acc = zero4();
#pragma unroll
                for (int kk = 0; kk < C / 16; ++kk) {
                    const int k0 = 16 * kk + 4 * g;
                    const float a[4] = {A2[(k0 + 0) * DP + 16 * rb + m], A2[(k0 + 1) * DP + 16 * rb + m],
                                        A2[(k0 + 2) * DP + 16 * rb + m], A2[(k0 + 3) * DP + 16 * rb + m]};
                    const float b[4] = {Y[(k0 + 0) * TP + m], Y[(k0 + 1) * TP + m], Y[(k0 + 2) * TP + m],
                                        Y[(k0 + 3) * TP + m]};
                    acc = mma16x4(a, b, acc);
                }
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int row = 16 * rb + 4 * g + r;
                    St[row * TP + m] = lds[L::GC + row] * St[row * TP + m] - acc[r] + lds[L::OFF + row * TP + m];
                }
            }
        }
        __syncthreads();
    }
    if (dir == 1 && p.ds0) {
        for (int idx = threadIdx.x; idx < D * TILE; idx += NT) {
            const int c = idx / TILE, j = idx - c * TILE;
            p.ds0[bh * DD + c * D + col0 + j] = St[c * TP + j];
        }
    }
}

template <int D, class In>
__global__ __launch_bounds__(NT) void kda_bwd_grad_kernel(BwdParams p) {
    using S = Scr<D>;
    using LL = ChunkLds<D>;
    extern __shared__ __align__(16) float lds[];
    using raw = typename In::raw_t;
    float* s = p.scratch + (int64_t)blockIdx.x * S::SIZE;
    const int64_t items = p.B * p.H * p.NC;
    const int64_t DD = (int64_t)D * D;
    for (int64_t item = blockIdx.x; item < items; item += gridDim.x) {
        const ChunkPos cp = chunk_pos(p, item);
        if (items <= p.slots) {
            // one chunk per slot: the prep kernel ran this chunk's shared steps in this
            // same slot (workgroup b takes chunk b in both launches) and left them there
            if (threadIdx.x < C) lds[LL::BETA + threadIdx.x] = s[S::BETA + threadIdx.x];
            __syncthreads();
        } else {
            chunk_common<D, In>(p, cp, s, lds);
        }
        const float* S0 = p.states + item * DD;
        const float* dSC = p.dstates + item * DD;
        const float* beta = s + S::BETA;
        // X = V - Kt S0
        mm<D, C, D, D, false, false, true>([&](int m, int k) { return s[S::KT + m * D + k]; },
                    [&](int k, int n) { return S0[k * D + n]; },
                    [&](int m, int n, float a) { s[S::X + m * D + n] = s[S::V + m * D + n] - a; }, lds);
        __syncthreads();
        // U = Li diag(beta) X
        mm<D, C, D, C, false, false, true>([&](int m, int k) { return s[S::LI + m * C + k] * beta[k]; },
                    [&](int k, int n) { return s[S::X + k * D + n]; },
                    [&](int m, int n, float a) { s[S::U + m * D + n] = a; }, lds);
        __syncthreads();
        // O = Qt S0 + P U;  dP = lower(dO U^T);  dKb = U dS_C^T;  dU = P^T dO + Kb dS_C
        mm<D, C, D, D, false, false, true>([&](int m, int k) { return s[S::QT + m * D + k]; },
                    [&](int k, int n) { return S0[k * D + n]; },
                    [&](int m, int n, float a) { s[S::O + m * D + n] = a; }, lds);
        mm<D, C, D, C, false, false, true>([&](int m, int k) { return s[S::PM + m * C + k]; },
                    [&](int k, int n) { return s[S::U + k * D + n]; },
                    [&](int m, int n, float a) { s[S::O + m * D + n] += a; }, lds);
        mm<D, C, C, D, false, true, true>([&](int m, int k) { return s[S::DO + m * D + k]; },
                    [&](int k, int n) { return s[S::U + n * D + k]; },
                    [&](int m, int n, float a) { s[S::DP + m * C + n] = n <= m ? a : 0.f; }, lds);
        mm<D, C, D, D, false, true, true>([&](int m, int k) { return s[S::U + m * D + k]; },
                    [&](int k, int n) { return dSC[n * D + k]; },
                    [&](int m, int n, float a) { s[S::DKB + m * D + n] = a; }, lds);
        mm<D, C, D, C, true, false, true>([&](int m, int k) { return s[S::PM + k * C + m]; },
                    [&](int k, int n) { return s[S::DO + k * D + n]; },
                    [&](int m, int n, float a) { s[S::DU + m * D + n] = a; }, lds);
        mm<D, C, D, D, false, false, true>([&](int m, int k) { return s[S::KB + m * D + k]; },
                    [&](int k, int n) { return dSC[k * D + n]; },
                    [&](int m, int n, float a) { s[S::DU + m * D + n] += a; }, lds);
        __syncthreads();
        // dZ = dY * O * sigmoid'(Z);  dLi = dU (diag(beta) X)^T, strictly lower part;  dW = Li^T dU
#pragma unroll 2
        for (int grp = threadIdx.x; grp < cp.L * D / 8; grp += NT) {
            const int idx = 8 * grp, r = idx / D, c8 = idx - r * D;
            const int64_t e = elem<D>(p, cp, r, c8);
            float z[8], y[8], o[8], dz[8];
            load8(static_cast<const raw*>(p.gate), e, z);
            load8(static_cast<const raw*>(p.dy), e, y);
            load8(s + S::O + idx, 0, o);
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                const float sg = sigmoidf_(z[j]);
                dz[j] = y[j] * o[j] * sg * (1.f - sg);
            }
            store8(p.dgate + e, dz);
        }
        mm<D, C, C, D, false, true, true>([&](int m, int k) { return s[S::DU + m * D + k]; },
                    [&](int k, int n) { return beta[n] * s[S::X + n * D + k]; },
                    [&](int m, int n, float a) { s[S::DLI + m * C + n] = n < m ? a : 0.f; }, lds);
        mm<D, C, D, C, true, false, true>([&](int m, int k) { return s[S::LI + k * C + m]; },
                    [&](int k, int n) { return s[S::DU + k * D + n]; },
                    [&](int m, int n, float a) { s[S::DW + m * D + n] = a; }, lds);
        __syncthreads();
        // dV = diag(beta) dW;  dbeta's X part;  E = Li^T dLi;  the S0 parts of dQ and dKt
#pragma unroll 2
        for (int grp = threadIdx.x; grp < cp.L * D / 8; grp += NT) {
            const int idx = 8 * grp, r = idx / D, c8 = idx - r * D;
            float w[8];
            load8(s + S::DW + idx, 0, w);
            const float br = beta[r];
#pragma unroll
            for (int j = 0; j < 8; ++j) w[j] *= br;
            store8(p.dv + elem<D>(p, cp, r, c8), w);
        }
        if (threadIdx.x < C) {
            const int r = threadIdx.x;
            float acc = 0.f;
            for (int j = 0; j < D; ++j) acc = fmaf(s[S::DW + r * D + j], s[S::X + r * D + j], acc);
            s[S::DBX + r] = acc;
        }
        mm<D, C, C, C, true, false, true>([&](int m, int k) { return s[S::LI + k * C + m]; },
                    [&](int k, int n) { return s[S::DLI + k * C + n]; },
                    [&](int m, int n, float a) { s[S::EM + m * C + n] = a; }, lds);
        mm<D, C, D, D, false, true, true>([&](int m, int k) { return s[S::DO + m * D + k]; },
                    [&](int k, int n) { return S0[n * D + k]; },
                    [&](int m, int n, float a) { s[S::DQ + m * D + n] = a * s[S::EG + m * D + n]; }, lds);
        mm<D, C, D, D, false, true, true>([&](int m, int k) { return beta[m] * s[S::DW + m * D + k]; },
                    [&](int k, int n) { return S0[n * D + k]; },
                    [&](int m, int n, float a) { s[S::DKT + m * D + n] = -a * s[S::EG + m * D + n]; }, lds);
        __syncthreads();
        // dA = -(E Li^T), strictly lower part (the gradient with respect to diag(beta) Bm)
        mm<D, C, C, C, false, true, true>([&](int m, int k) { return s[S::EM + m * C + k]; },
                    [&](int k, int n) { return s[S::LI + n * C + k]; },
                    [&](int m, int n, float a) { s[S::DA + m * C + n] = n < m ? -a : 0.f; }, lds);
        __syncthreads();
        // pair terms of dq and dk (through P and Bm), the K-bar term, dg; dbeta.  The
        // loops read k, q, g (row-major), dP, dA and beta from LDS.
        to_lds<C * D>(lds + LL::A0, s + S::K);
        to_lds<C * D>(lds + LL::A1, s + S::Q);
        to_lds<C * D>(lds + LL::A2, s + S::G);
        to_lds<C * C>(lds + LL::B0, s + S::DP);
        to_lds<C * C>(lds + LL::B1, s + S::DA);
        __syncthreads();
        const float* lk = lds + LL::A0;
        const float* lq = lds + LL::A1;
        const float* lg = lds + LL::A2;
        const float* ldp = lds + LL::B0;
        const float* lda = lds + LL::B1;
        const float* lbeta = lds + LL::BETA;
        for (int idx = threadIdx.x; idx < C * D; idx += NT) {
            const int r = idx / D, c = idx - r * D;
            const float gr = lg[idx];
            // scratch values first: their latency is covered by the LDS loops below
            const float dq0 = s[S::DQ + idx], dkt0 = s[S::DKT + idx], dkb0 = s[S::DKB + idx];
            float pq = 0.f, aq = 0.f, ak = 0.f, pk = 0.f;
#pragma unroll 4
            for (int j = 0; j <= r; ++j) {
                const float ke = lk[j * D + c] * ex(gr - lg[j * D + c]);
                pq = fmaf(ldp[r * C + j], ke, pq);
                aq = fmaf(lda[r * C + j], ke, aq);
            }
#pragma unroll 4
            for (int j = r; j < C; ++j) {
                const float e = ex(lg[j * D + c] - gr);
                ak = fmaf(lbeta[j] * lda[j * C + r], lk[j * D + c] * e, ak);
                pk = fmaf(ldp[j * C + r], lq[j * D + c] * e, pk);
            }
            const float dqf = dq0 + pq;
            const float dktf = dkt0 + lbeta[r] * aq;
            const float dkif = ak + pk;
            const float dkbf = dkb0 * ex(lg[(C - 1) * D + c] - gr);
            const float kv = lk[idx], qv = lq[idx];
            if (r < cp.L) {
                const int64_t e = elem<D>(p, cp, r, c);
                p.dq[e] = dqf;
                p.dk[e] = dktf + dkif + dkbf;
            }
            s[S::DQ + idx] = qv * dqf + kv * (dktf - dkif - dkbf);  // gradient of g
            s[S::DKT + idx] = kv * dkbf;                             // its g_C share
        }
        if (threadIdx.x < C) {
            const int r = threadIdx.x;
            float acc = s[S::DBX + r];
            for (int j = 0; j < r; ++j) acc = fmaf(s[S::DA + r * C + j], s[S::BM + r * C + j], acc);
            if (r < cp.L) p.dbeta[(cp.b * p.T + cp.t0 + r) * p.H + cp.h] = acc;
        }
        __syncthreads();
        // dlambda_r = sum_{r' >= r} dg_r', with g_C's extra terms from Kb and Diag(Gc) S0
        if (threadIdx.x < D) {
            const int c = threadIdx.x;
            float dgc = 0.f;
            for (int j = 0; j < D; ++j) dgc = fmaf(dSC[c * D + j], S0[c * D + j], dgc);
            float acc = dgc * s[S::EG + (C - 1) * D + c];
            for (int r = 0; r < C; ++r) acc += s[S::DKT + r * D + c];
#pragma unroll 1
            for (int r0 = C - 16; r0 >= 0; r0 -= 16) {
                // 16 rows of g's gradient and of the raw log alpha, read before their stores
                float col[16], raw_la[16];
#pragma unroll
                for (int u = 0; u < 16; ++u) {
                    col[u] = s[S::DQ + (r0 + u) * D + c];
                    raw_la[u] = r0 + u < cp.L ? In::load(static_cast<const raw*>(p.la), elem<D>(p, cp, r0 + u, c)) : 0.f;
                }
#pragma unroll
                for (int u = 15; u >= 0; --u) {
                    const int r = r0 + u;
                    acc += col[u];
                    if (r < cp.L) {
                        const float l = raw_la[u];
                        const bool live = p.clamp == 0 || (l >= kLogAlphaMin && l <= 0.f);
                        p.dla[elem<D>(p, cp, r, c)] = live ? acc : 0.f;
                    }
                }
            }
        }
        __syncthreads();  // the slot is reused by the next chunk
    }
}

int64_t align256(int64_t x) { return (x + 255) / 256 * 256; }

template <int D>
int64_t section_bytes(int64_t bh, int64_t nc, int64_t* trans, int64_t* states, int64_t* slots) {
    const int64_t items = bh * nc;
    *trans = align256(items * Rec<D>::SIZE * 4);
    *states = align256(items * (int64_t)D * D * 4);
    *slots = items < kMaxSlots ? items : kMaxSlots;
    return *trans + 2 * *states + align256(*slots * Scr<D>::SIZE * 4);
}

template <int D, class In>
hipError_t launch_d(const BwdParams& p, hipStream_t stream) {
    const int64_t items = p.B * p.H * p.NC;
    constexpr int clds = ChunkLds<D>::TOTAL * 4;
    if (items > 0) {
        auto kp = kda_bwd_prep_kernel<D, In>;
        hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kp),
                                           hipFuncAttributeMaxDynamicSharedMemorySize, clds);
        if (e != hipSuccess) return e;
        hipLaunchKernelGGL(kp, dim3((unsigned)p.slots), dim3(NT), clds, stream, p);
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
        auto kg = kda_bwd_grad_kernel<D, In>;
        hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kg),
                                           hipFuncAttributeMaxDynamicSharedMemorySize, clds);
        if (e != hipSuccess) return e;
        hipLaunchKernelGGL(kg, dim3((unsigned)p.slots), dim3(NT), clds, stream, p);
    }
    return hipGetLastError();
}

}  // namespace

int64_t bwd_workspace_bytes(int D, int64_t bh, int64_t nc) {
    int64_t t, s, k;
    return D == 64 ? section_bytes<64>(bh, nc, &t, &s, &k) : section_bytes<128>(bh, nc, &t, &s, &k);
}

void bwd_layout(int D, int64_t bh, int64_t nc, void* ws, BwdParams& p) {
    int64_t t, s, k;
    if (D == 64)
        section_bytes<64>(bh, nc, &t, &s, &k);
    else
        section_bytes<128>(bh, nc, &t, &s, &k);
    unsigned char* w = static_cast<unsigned char*>(ws);
    p.trans = reinterpret_cast<float*>(w);
    p.states = reinterpret_cast<float*>(w + t);
    p.dstates = reinterpret_cast<float*>(w + t + s);
    p.scratch = reinterpret_cast<float*>(w + t + 2 * s);
    p.slots = k;
}

hipError_t launch_bwd(int dtype_bf16, int D, const BwdParams& p, hipStream_t stream) {
    if (D == 64) return dtype_bf16 ? launch_d<64, InBF16>(p, stream) : launch_d<64, InF32>(p, stream);
    return dtype_bf16 ? launch_d<128, InBF16>(p, stream) : launch_d<128, InF32>(p, stream);
}

}  // namespace kda
