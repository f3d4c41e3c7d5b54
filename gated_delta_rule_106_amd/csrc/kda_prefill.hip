// Chunkwise-parallel KDA forward (prefill) for gfx950.
//
// The per-token recurrence (page "3T models are no longer magic", section
// "Gate 1: KDA makes it computable")
//     S_t = (I - beta_t k_t k_t^T) Diag(alpha_t) S_{t-1} + beta_t k_t v_t^T,
//     y_t = (S_t^T q_t) * sigmoid(z_t)
// is evaluated chunk by chunk, parallel inside a chunk and recurrent across
// chunks (page "Kimi K3 report walk-through", sections "Compute paradigm" and
// "Hierarchical chunking of linear attention").  Inside a chunk of C tokens
// with start state S0, g_r = sum_{s<=r} log alpha_s (per key channel):
//     K~ = k e^{g},  Q~ = q e^{g},  Kbar = k e^{g_C - g},  Gamma = e^{g_C}
//     A_rs = beta_r sum_c k_rc k_sc e^{g_rc - g_sc}   (s < r)
//     P_rs =        sum_c q_rc k_sc e^{g_rc - g_sc}   (s <= r)
//     T = (I + A)^{-1} diag(beta),  W = T K~,  U~ = T V
//     U = U~ - W S0,  O = Q~ S0 + P U,  S_C = Diag(Gamma) S0 + Kbar^T U
// and, folding the output, O = Qe S0 + Uo with Qe = Q~ - P W, Uo = P U~.
// Decay is applied to one side and inverse decay to the other as an
// absolute-position rescaling (page "Kimi K3 report walk-through", section
// "Numerical stability & co-design"); the pair products that need the inverse
// factor are formed in 16-token tiles around a reference point at the middle
// of each tile, so every factor stays within e^{+-8 |ln 0.0067|} ~ e^{+-40}
// and inter-tile factors are <= 1: nothing overflows for any chunk size.
//
// Two kernels:
//   kda_prep_kernel   one workgroup per (b, h, chunk), fully parallel: the
//                     chunk's "update card" (W, Qe, Kbar^T, U~, Uo, Gamma) into
//                     the workspace.
//   kda_recur_kernel  one workgroup per (b, h, group of value columns): walks
//                     the chunks in order with the fp32 state in MFMA
//                     accumulator registers, fusing the output read and gate.
//
// Numerics (16-bit path, bf16 inputs): the pair products A and P use a
// three-pass bf16 hi/lo split (their operands span e^{+-40}); every other
// contraction uses fp16 operands (bounded quantities, 11-bit significand) with
// fp32 accumulation; the state stays fp32.  The fp32 path uses fp32 MFMA.
#include "kda_device.h"
#include "kda_prefill.h"

namespace kda {

template <bool F32>
struct Op;
template <>
struct Op<true> {
    using t = float;
};
template <>
struct Op<false> {
    using t = _Float16;
};

// ---------------------------------------------------------------------------
// workspace geometry of one (b, h, chunk) "update card"
template <int C, int D, bool F32>
struct Card {
    using op_t = typename Op<F32>::t;
    static constexpr int64_t kCD = (int64_t)C * D;
    static constexpr int64_t W = 0;            // [C][D]
    static constexpr int64_t QE = W + kCD;     // [C][D]
    static constexpr int64_t KBT = QE + kCD;   // [D][C]
    static constexpr int64_t UT = KBT + kCD;   // fragment-major [D/16][C/16][64][4]
    static constexpr int64_t UO = UT + kCD;    // fragment-major
    static constexpr int64_t OP_ELEMS = UO + kCD;
    static constexpr int64_t BYTES = OP_ELEMS * (int64_t)sizeof(op_t) + (int64_t)D * 4;  // + Gamma
    static_assert(BYTES % 16 == 0, "card alignment");
};

__host__ __device__ constexpr int64_t align16(int64_t x) { return (x + 15) / 16 * 16; }

// ---------------------------------------------------------------------------
// kernel 1: per-chunk preparation
template <int C, int D, bool F32, class In>
struct PrepLds {
    using op_t = typename Op<F32>::t;
    using raw_t = typename In::raw_t;
    static constexpr int NSUB = C / 16;
    static constexpr int SX = D + 4;                    // fp32 [C][D] row stride
    static constexpr int SV = D + (sizeof(raw_t) == 2 ? 8 : 4);
    static constexpr int SC = C + 4;                    // fp32 [C][C] row stride
    static constexpr int SU = D + (sizeof(op_t) == 2 ? 8 : 4);
    static constexpr int64_t B_TILE = align16((int64_t)C * SX * 4);
    static constexpr int64_t B_SQ = align16((int64_t)C * SC * 4);
    static constexpr int64_t B_V = align16((int64_t)C * SV * sizeof(raw_t));
    static constexpr int64_t B_U = align16((int64_t)C * SU * sizeof(op_t));
    static constexpr bool U_IN_A = B_U <= B_SQ;
    static constexpr int NPAIR = NSUB * (NSUB - 1) / 2 > 0 ? NSUB * (NSUB - 1) / 2 : 1;
    static constexpr int TPC = 256 / D;                 // threads per channel in the scan
    static constexpr int64_t OFF_KF = 0;                // k * F      -> later W (fp32)
    static constexpr int64_t OFF_QF = OFF_KF + B_TILE;  // q * F
    static constexpr int64_t OFF_KG = OFF_QF + B_TILE;  // k * G      -> later Linv / T
    static constexpr int64_t OFF_V = OFF_KG + B_TILE;   // v (raw input type)
    static constexpr int64_t OFF_A = OFF_V + B_V;       // A (fp32)   -> later U~ if it fits
    static constexpr int64_t OFF_P = OFF_A + B_SQ;      // P (fp32)
    static constexpr int64_t OFF_U = U_IN_A ? OFF_A : OFF_P + B_SQ;
    // one scratch region shared by phase-separated temporaries: scan partials
    // (phase 0), inter-tile decay vectors (phase 1) and solve temporaries (phase 2)
    static constexpr int64_t B_Y = align16((int64_t)(NSUB > 1 ? NSUB - 1 : 1) * 256 * 4);
    static constexpr int64_t B_EV = align16((int64_t)NPAIR * D * 4);
    static constexpr int64_t B_PT = align16((int64_t)TPC * D * 4);
    static constexpr int64_t B_SCR = B_Y > B_EV ? (B_Y > B_PT ? B_Y : B_PT) : (B_EV > B_PT ? B_EV : B_PT);
    static constexpr int64_t OFF_Y = U_IN_A ? OFF_P + B_SQ : OFF_U + B_U;
    static constexpr int64_t OFF_EV = OFF_Y;
    static constexpr int64_t OFF_PT = OFF_Y;
    static constexpr int64_t OFF_ML = OFF_Y + B_SCR;    // log2 midpoint refs [NSUB][D]
    static constexpr int64_t OFF_EA = OFF_ML + align16((int64_t)NSUB * D * 4);   // e^{m_a}
    static constexpr int64_t OFF_GE = OFF_EA + align16((int64_t)NSUB * D * 4);   // log2 g_C
    static constexpr int64_t OFF_BT = OFF_GE + align16((int64_t)D * 4);          // beta
    static constexpr int64_t OFF_NS = OFF_BT + align16((int64_t)C * 4);          // q, k scales [2][C]
    static constexpr int64_t TOTAL = OFF_NS + align16((int64_t)2 * C * 4);
    static_assert(TOTAL <= 160 * 1024, "prep LDS budget");
};

template <int C, int D, bool F32, class In>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 2)))
void kda_prep_kernel(PrepParams p) {
    using L = PrepLds<C, D, F32, In>;
    using CD = Card<C, D, F32>;
    using op_t = typename Op<F32>::t;
    using raw_t = typename In::raw_t;
    constexpr int NT = 256, NW = 4;
    constexpr int NSUB = L::NSUB, SX = L::SX, SV = L::SV, SC = L::SC, SU = L::SU;
    extern __shared__ __align__(16) unsigned char smem[];
    float* XF = reinterpret_cast<float*>(smem + L::OFF_KF);
    float* XQ = reinterpret_cast<float*>(smem + L::OFF_QF);
    float* XG = reinterpret_cast<float*>(smem + L::OFF_KG);
    raw_t* XV = reinterpret_cast<raw_t*>(smem + L::OFF_V);
    float* SA = reinterpret_cast<float*>(smem + L::OFF_A);
    float* SP = reinterpret_cast<float*>(smem + L::OFF_P);
    op_t* SUt = reinterpret_cast<op_t*>(smem + L::OFF_U);
    float* SY = reinterpret_cast<float*>(smem + L::OFF_Y);
    float* ML = reinterpret_cast<float*>(smem + L::OFF_ML);
    float* EA = reinterpret_cast<float*>(smem + L::OFF_EA);
    float* EV = reinterpret_cast<float*>(smem + L::OFF_EV);
    float* GE = reinterpret_cast<float*>(smem + L::OFF_GE);
    float* PT = reinterpret_cast<float*>(smem + L::OFF_PT);
    float* BT = reinterpret_cast<float*>(smem + L::OFF_BT);
    float* LI = XG;  // Linv / T after Kbar has been written out
    float* WF = XF;  // W (fp32) after K~ has been consumed

    const int tid = threadIdx.x, lane = lane_id(), wave = wave_id();
    const int m16 = lane & 15, g4 = lane >> 4;
    const int64_t H = p.H;
    // this card's chunk n of a sequence of T tokens from packed row tb, head h: B
    // sequences of p.T tokens (card (b H + h) NC + n), or a variable-length batch (card
    // g H + h for the batch's chunk g); either way the card index is blockIdx.x
    int64_t n, h, tb, T;
    if (p.vco) {
        const int64_t g = blockIdx.x / H;
        h = blockIdx.x - g * H;
        if (g >= p.vco[p.vN]) return;  // no chunk here (the whole group leaves)
        const int64_t i = p.vsoc[g];
        n = g - p.vco[i];
        tb = p.vs[i];
        T = p.vs[i + 1] - tb;  // >= 1: the sequence owns this chunk
    } else {
        const int64_t bh = blockIdx.x / p.NC;
        n = blockIdx.x - bh * p.NC;
        h = bh % H;
        tb = (bh / H) * p.T;
        T = p.T;
    }
    const int64_t t0 = (int64_t)n * C;
    const raw_t* gq = static_cast<const raw_t*>(p.q);
    const raw_t* gk = static_cast<const raw_t*>(p.k);
    const raw_t* gv = static_cast<const raw_t*>(p.v);
    const raw_t* gla = static_cast<const raw_t*>(p.la);
    const raw_t* gbeta = static_cast<const raw_t*>(p.beta);
    const bool clamp = p.clamp != 0, logits = p.logits != 0;
    float* NS = reinterpret_cast<float*>(smem + L::OFF_NS);  // [0][r]: q scale, [1][r]: k scale
    // row of token t of the sequence (head h) in a packed [rows, H, D] tensor
    auto row = [&](int64_t t) { return (tb + t) * H + h; };

    // per-token L2 normalisation factors of raw q and k (one wave per token, visible
    // after the first barrier below; 1 for inputs that arrive normalised)
    for (int r = wave; r < C; r += NW) {
        const int64_t t = t0 + r;
        float sq = 0.f, sk = 0.f;
        if (p.qk_norm && t < T) {
            for (int cc = lane; cc < D; cc += 64) {
                const float qv = In::load(gq, row(t) * D + cc), kv = In::load(gk, row(t) * D + cc);
                sq += qv * qv;
                sk += kv * kv;
            }
#pragma unroll
            for (int off = 32; off > 0; off >>= 1) {
                sq += __shfl_xor(sq, off);
                sk += __shfl_xor(sk, off);
            }
        }
        if (lane == 0) {
            NS[r] = p.qk_norm ? inv_norm(sq) * (1.0f / __builtin_sqrtf((float)D)) : 1.f;
            NS[C + r] = p.qk_norm ? inv_norm(sk) : 1.f;
        }
    }

    // ---- phase 0: cumulative log-decay (log2 units), references, rescaled tiles
    constexpr int TPC = L::TPC;        // threads per channel
    constexpr int TPT = C / TPC;       // tokens per thread
    static_assert(TPT >= 1 && C % TPC == 0, "scan split");
    const int c = tid % D, part = tid / D, r0 = part * TPT;
    float gl[TPT];
    {
        // every load issued first, each from a token inside the sequence (T >= 1 here);
        // tokens past the end count as zero
#pragma unroll
        for (int j = 0; j < TPT; ++j) {
            const int64_t t = t0 + r0 + j;
            gl[j] = In::load(gla, row(t < T ? t : T - 1) * D + c);
        }
        float acc = 0.f;
#pragma unroll
        for (int j = 0; j < TPT; ++j) {
            const float l = t0 + r0 + j < T ? log_alpha_in(gl[j], logits, clamp) : 0.f;
            acc += l * kLog2e;
            gl[j] = acc;
        }
        PT[part * D + c] = acc;
    }
    for (int i = tid; i < C * SC; i += NT) { SA[i] = 0.f; SP[i] = 0.f; }
    if (tid < C) {
        const int64_t t = t0 + tid;
        BT[tid] = t < T ? In::load(gbeta, row(t)) : 0.f;
    }
    __syncthreads();
    {
        float off = 0.f;
        for (int q2 = 0; q2 < part; ++q2) off += PT[q2 * D + c];
#pragma unroll
        for (int j = 0; j < TPT; ++j) {
            gl[j] += off;
            const int r = r0 + j;
            if ((r & 15) == 7) ML[(r >> 4) * D + c] = gl[j];
            if (r == C - 1) GE[c] = gl[j];
        }
    }
    __syncthreads();
#pragma unroll
    for (int j = 0; j < TPT; ++j) {
        const int r = r0 + j;
        const int64_t t = t0 + r;
        const float mref = ML[(r >> 4) * D + c];
        const float F = fast_exp2(gl[j] - mref), G = fast_exp2(mref - gl[j]);
        const int64_t tr = row(t < T ? t : T - 1) * D + c;  // a token inside the sequence
        const float kl = In::load(gk, tr), ql = In::load(gq, tr);
        const raw_t vl = gv[tr];
        const float kk = t < T ? kl * NS[C + r] : 0.f, qq = t < T ? ql * NS[r] : 0.f;
        const raw_t vv = t < T ? vl : In::from_float(0.f);
        XF[r * SX + c] = kk * F;
        XQ[r * SX + c] = qq * F;
        XG[r * SX + c] = kk * G;
        XV[r * SV + c] = vv;
    }
    for (int i = tid; i < NSUB * D; i += NT) EA[i] = fast_exp2(ML[i]);
    for (int i = tid; i < NSUB * NSUB * D; i += NT) {
        const int a = i / (NSUB * D), bb = (i / D) % NSUB, cc = i % D;
        if (bb < a) EV[(a * (a - 1) / 2 + bb) * D + cc] = fast_exp2(ML[a * D + cc] - ML[bb * D + cc]);
    }
    __syncthreads();

    // ---- phase 1: pair products A (strict lower, beta-scaled) and P (lower)
    {
        constexpr int NJOB = NSUB * (NSUB + 1) / 2;
        for (int job = wave; job < NJOB; job += NW) {
            int a = 0;
            while ((a + 1) * (a + 2) / 2 <= job) ++a;
            const int bb = job - a * (a + 1) / 2;
            const float* ev = (bb < a) ? EV + (a * (a - 1) / 2 + bb) * D : nullptr;
            floatx4 accA = zero4(), accP = zero4();
            const float* xr_k = XF + (16 * a + m16) * SX;
            const float* xr_q = XQ + (16 * a + m16) * SX;
            const float* xc = XG + (16 * bb + m16) * SX;
            if constexpr (F32) {
                for (int ks = 0; ks < D; ks += 4) {
                    const int cc = ks + g4;
                    const float col = ev ? xc[cc] * ev[cc] : xc[cc];
                    accA = mma_f32_k4(xr_k[cc], col, accA);
                    accP = mma_f32_k4(xr_q[cc], col, accP);
                }
            } else {
                for (int ks = 0; ks < D; ks += 32) {
                    bf16x8 kh, kl, qh, ql, ch, cl;
#pragma unroll
                    for (int j = 0; j < 8; ++j) {
                        const int cc = ks + 8 * g4 + j;
                        const float col = ev ? xc[cc] * ev[cc] : xc[cc];
                        __bf16 hi, lo;
                        split_bf16(xr_k[cc], hi, lo); kh[j] = hi; kl[j] = lo;
                        split_bf16(xr_q[cc], hi, lo); qh[j] = hi; ql[j] = lo;
                        split_bf16(col, hi, lo); ch[j] = hi; cl[j] = lo;
                    }
                    accA = mma_bf16_k32(kh, ch, accA);
                    accA = mma_bf16_k32(kh, cl, accA);
                    accA = mma_bf16_k32(kl, ch, accA);
                    accP = mma_bf16_k32(qh, ch, accP);
                    accP = mma_bf16_k32(qh, cl, accP);
                    accP = mma_bf16_k32(ql, ch, accP);
                }
            }
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int r = 16 * a + 4 * g4 + i, s = 16 * bb + m16;
                SA[r * SC + s] = (s < r) ? BT[r] * accA[i] : 0.f;
                SP[r * SC + s] = (s <= r) ? accP[i] : 0.f;
            }
        }
    }
    __syncthreads();

    // ---- phase 1.5: Kbar^T and Gamma to the card (frees the k*G tile)
    const int64_t chunk_index = blockIdx.x;
    op_t* card = reinterpret_cast<op_t*>(static_cast<unsigned char*>(p.ws) + chunk_index * CD::BYTES);
    float* gam = reinterpret_cast<float*>(card + CD::OP_ELEMS);
    for (int i = tid; i < D * (C / 8); i += NT) {
        const int cc = i / (C / 8), r8 = (i % (C / 8)) * 8;
        const float gend = GE[cc];
        op_t* dst = card + CD::KBT + (int64_t)cc * C + r8;
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            const int r = r8 + j;
            dst[j] = static_cast<op_t>(XG[r * SX + cc] * fast_exp2(gend - ML[(r >> 4) * D + cc]));
        }
    }
    for (int i = tid; i < D; i += NT) gam[i] = fast_exp2(GE[i]);
    __syncthreads();

    // ---- phase 2: T = (I + A)^{-1} diag(beta), fp32, blocked forward substitution
    for (int i = tid; i < C * SC; i += NT) LI[i] = 0.f;
    __syncthreads();
    if (tid < NSUB * 16) {  // inverse of each unit-lower diagonal 16x16 block, one column per thread
        const int a = tid >> 4, j = tid & 15, base = 16 * a;
        float x[16];
#pragma unroll
        for (int r = 0; r < 16; ++r) x[r] = 0.f;
        x[j] = 1.f;
#pragma unroll
        for (int r = 1; r < 16; ++r) {
            if (r > j) {
                float s = 0.f;
                for (int q2 = j; q2 < r; ++q2) s += SA[(base + r) * SC + base + q2] * x[q2];
                x[r] = -s;
            }
        }
#pragma unroll
        for (int r = 0; r < 16; ++r) LI[(base + r) * SC + base + j] = x[r];
    }
    __syncthreads();
    for (int d = 1; d < NSUB; ++d) {
        const int nb = NSUB - d;
        // Y_(a) = sum_{c=a-d}^{a-1} A_{a,c} Linv_{c,a-d}
        for (int e = tid; e < nb * 256; e += NT) {
            const int a = d + e / 256, rr = (e % 256) / 16, cc = e % 16, bb = a - d;
            float s = 0.f;
            for (int q2 = 16 * bb; q2 < 16 * a; ++q2)
                s += SA[(16 * a + rr) * SC + q2] * LI[q2 * SC + 16 * bb + cc];
            SY[e] = s;
        }
        __syncthreads();
        // Linv_{a,a-d} = -X_a Y_(a)
        for (int e = tid; e < nb * 256; e += NT) {
            const int a = d + e / 256, rr = (e % 256) / 16, cc = e % 16, bb = a - d;
            float s = 0.f;
            for (int q2 = 0; q2 <= rr; ++q2)
                s += LI[(16 * a + rr) * SC + 16 * a + q2] * SY[(e / 256) * 256 + q2 * 16 + cc];
            LI[(16 * a + rr) * SC + 16 * bb + cc] = -s;
        }
        __syncthreads();
    }
    for (int i = tid; i < C * C; i += NT) {
        const int r = i / C, s = i % C;
        LI[r * SC + s] *= BT[s];
    }
    __syncthreads();

    // ---- phase 3: W = T K~ and U~ = T V  (K = tokens 0 .. 16(mt+1))
    constexpr int NMT = C / 16, NNT = D / 16, NTILE = NMT * NNT;
    constexpr int JOBS3 = 2 * NTILE;
    constexpr int PERW = (JOBS3 + NW - 1) / NW;
    floatx4 res[PERW];
#pragma unroll
    for (int jj = 0; jj < PERW; ++jj) {
        const int job = wave + jj * NW;
        floatx4 acc = zero4();
        if (job < JOBS3) {
            const bool isU = job >= NTILE;
            const int tile = isU ? job - NTILE : job;
            const int mt = tile / NNT, nt = tile % NNT;
            const int kend = 16 * (mt + 1);
            const float* arow = LI + (16 * mt + m16) * SC;
            const int col = 16 * nt + m16;
            auto bval = [&](int s) -> float {
                return isU ? In::load(XV, (int64_t)s * SV + col)
                           : XF[s * SX + col] * EA[(s >> 4) * D + col];
            };
            if constexpr (F32) {
                for (int k0 = 0; k0 < kend; k0 += 4) acc = mma_f32_k4(arow[k0 + g4], bval(k0 + g4), acc);
            } else {
                int k0 = 0;
                for (; k0 + 32 <= kend; k0 += 32) {
                    half8 av, bv;
#pragma unroll
                    for (int j = 0; j < 8; ++j) {
                        av[j] = static_cast<_Float16>(arow[k0 + 8 * g4 + j]);
                        bv[j] = static_cast<_Float16>(bval(k0 + 8 * g4 + j));
                    }
                    acc = mma_f16_k32(av, bv, acc);
                }
                if (k0 < kend) {  // last 16 tokens: a K = 32 step with its upper half zeroed
                    half8 av, bv;
#pragma unroll
                    for (int j = 0; j < 4; ++j) {
                        av[j] = static_cast<_Float16>(arow[k0 + 4 * g4 + j]);
                        bv[j] = static_cast<_Float16>(bval(k0 + 4 * g4 + j));
                        av[4 + j] = bv[4 + j] = static_cast<_Float16>(0.f);
                    }
                    acc = mma_f16_k32(av, bv, acc);
                }
            }
        }
        res[jj] = acc;
    }
    __syncthreads();  // every wave is done reading k*F and v
#pragma unroll
    for (int jj = 0; jj < PERW; ++jj) {
        const int job = wave + jj * NW;
        if (job >= JOBS3) continue;
        const bool isU = job >= NTILE;
        const int tile = isU ? job - NTILE : job;
        const int mt = tile / NNT, nt = tile % NNT;
        const floatx4 acc = res[jj];
        if (!isU) {
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int r = 16 * mt + 4 * g4 + i, cc = 16 * nt + m16;
                WF[r * SX + cc] = acc[i];
                card[CD::W + (int64_t)r * D + cc] = static_cast<op_t>(acc[i]);
            }
        } else {
            op_t* dst = card + CD::UT + ((int64_t)(nt * NMT + mt) * 64 + lane) * 4;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int r = 16 * mt + 4 * g4 + i, cc = 16 * nt + m16;
                SUt[r * SU + cc] = static_cast<op_t>(acc[i]);
                dst[i] = static_cast<op_t>(acc[i]);
            }
        }
    }
    __syncthreads();

    // ---- phase 4: Qe = Q~ - P W and Uo = P U~
#pragma unroll
    for (int jj = 0; jj < PERW; ++jj) {
        const int job = wave + jj * NW;
        if (job >= JOBS3) continue;
        const bool isU = job >= NTILE;
        const int tile = isU ? job - NTILE : job;
        const int mt = tile / NNT, nt = tile % NNT;
        const int kend = 16 * (mt + 1);
        const float* arow = SP + (16 * mt + m16) * SC;
        const int col = 16 * nt + m16;
        auto bval = [&](int s) -> float {
            return isU ? static_cast<float>(SUt[s * SU + col]) : WF[s * SX + col];
        };
        floatx4 acc = zero4();
        if constexpr (F32) {
            for (int k0 = 0; k0 < kend; k0 += 4) acc = mma_f32_k4(arow[k0 + g4], bval(k0 + g4), acc);
        } else {
            int k0 = 0;
            for (; k0 + 32 <= kend; k0 += 32) {
                half8 av, bv;
#pragma unroll
                for (int j = 0; j < 8; ++j) {
                    av[j] = static_cast<_Float16>(arow[k0 + 8 * g4 + j]);
                    bv[j] = static_cast<_Float16>(bval(k0 + 8 * g4 + j));
                }
                acc = mma_f16_k32(av, bv, acc);
            }
            if (k0 < kend) {  // last 16 tokens: a K = 32 step with its upper half zeroed
                half8 av, bv;
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    av[j] = static_cast<_Float16>(arow[k0 + 4 * g4 + j]);
                    bv[j] = static_cast<_Float16>(bval(k0 + 4 * g4 + j));
                    av[4 + j] = bv[4 + j] = static_cast<_Float16>(0.f);
                }
                acc = mma_f16_k32(av, bv, acc);
            }
        }
        if (!isU) {
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int r = 16 * mt + 4 * g4 + i, cc = 16 * nt + m16;
                const float qt = XQ[r * SX + cc] * EA[(r >> 4) * D + cc];
                card[CD::QE + (int64_t)r * D + cc] = static_cast<op_t>(qt - acc[i]);
            }
        } else {
            op_t* dst = card + CD::UO + ((int64_t)(nt * NMT + mt) * 64 + lane) * 4;
#pragma unroll
            for (int i = 0; i < 4; ++i) dst[i] = static_cast<op_t>(acc[i]);
        }
    }
}

// ---------------------------------------------------------------------------
// kernel 2: sequential pass over the chunks, state in registers, output fused
template <int C, int D, bool F32>
struct RecurLds {
    using op_t = typename Op<F32>::t;
    static constexpr int SW = D + (sizeof(op_t) == 2 ? 8 : 4);  // [C][D] row stride
    static constexpr int SK = C + (sizeof(op_t) == 2 ? 8 : 4);  // [D][C] row stride
    static constexpr int64_t B_W = align16((int64_t)C * SW * sizeof(op_t));
    static constexpr int64_t B_K = align16((int64_t)D * SK * sizeof(op_t));
    static constexpr int64_t B_BUF = 2 * B_W + B_K + align16((int64_t)D * 4);
    static constexpr int64_t TOTAL = 2 * B_BUF;
    static_assert(TOTAL <= 160 * 1024, "recur LDS budget");
};

// One workgroup per CU (LDS-bound): let each wave use the whole register file.
// SUM: the segment summary instead of the outputs (page "Kimi K3 report walk-through",
// section "KDA Context Parallelism"): blocks of the first half of each (b, h)'s range
// carry b (the state from zero, U = U~ - W S), the second half M (from the identity,
// U = -W S: the same map on a state whose columns are the unit vectors, without the
// values); nothing is read out, and the end state goes to p.sum_b or p.sum_m.
template <int C, int D, bool F32, class In, class Out, int NWV, bool SUM>
__global__ __launch_bounds__(NWV * 64) __attribute__((amdgpu_waves_per_eu(1, 1)))
void kda_recur_kernel(RecurParams p) {
    using L = RecurLds<C, D, F32>;
    using CD = Card<C, D, F32>;
    using op_t = typename Op<F32>::t;
    using raw_t = typename In::raw_t;
    constexpr int NT = NWV * 64;
    constexpr int SW = L::SW, SK = L::SK;
    constexpr int NMT = C / 16, NCT = D / 16;
    extern __shared__ __align__(16) unsigned char smem[];

    const int lane = lane_id(), wave = wave_id(), tid = threadIdx.x;
    const int m16 = lane & 15, g4 = lane >> 4;
    // XCD-aware mapping: consecutive logical blocks (same head) land on one XCD
    const int nblk = gridDim.x;
    const int bid = blockIdx.x;
    const int logical = (nblk % 8 == 0) ? (bid % 8) * (nblk / 8) + bid / 8 : bid;
    constexpr int GROUPS = D / (16 * NWV);
    constexpr int PARTS = SUM ? 2 : 1;  // SUM: b, then M
    const int cgrp = logical % GROUPS;
    const int part = SUM ? (logical / GROUPS) % PARTS : 0;  // 1: this block carries M
    const int64_t unit = logical / (GROUPS * PARTS);  // b * H + h
    const int64_t H = p.H;
    const int64_t b = unit / H, h = unit % H;
    // the sequence of this (b, h): T tokens from packed row tb, NC chunks whose cards are
    // cbase + ci cstride (B sequences of p.T tokens, or a variable-length batch)
    int64_t T, NC, tb, cbase, cstride;
    if (p.vco) {
        tb = p.vs[b];
        T = p.vs[b + 1] - tb;
        NC = (T + C - 1) / C;
        cbase = p.vco[b] * H + h;
        cstride = H;
    } else {
        T = p.T;
        NC = p.NC;
        tb = b * T;
        cbase = unit * NC;
        cstride = 1;
    }
    const int col = 16 * (cgrp * NWV + wave) + m16;  // this lane's value column
    const int nt = col >> 4;

    // state S[ct] rows 16ct + 4g + i, column col
    floatx4 S[NCT];
    if (SUM && part == 1) {  // M starts from the identity
#pragma unroll
        for (int ct = 0; ct < NCT; ++ct)
#pragma unroll
            for (int i = 0; i < 4; ++i) S[ct][i] = (16 * ct + 4 * g4 + i == col) ? 1.f : 0.f;
    } else {
        const float* s0 = (!SUM && p.s0) ? p.s0 + unit * (int64_t)D * D : nullptr;
#pragma unroll
        for (int ct = 0; ct < NCT; ++ct)
#pragma unroll
            for (int i = 0; i < 4; ++i) S[ct][i] = s0 ? s0[(16 * ct + 4 * g4 + i) * D + col] : 0.f;
    }

    const unsigned char* cards = static_cast<const unsigned char*>(p.ws) + cbase * CD::BYTES;
    const int64_t cbytes = cstride * CD::BYTES;  // from one chunk's card to the next
    // cooperative copy of one card's W, Qe, Kbar^T (+ Gamma) into an LDS buffer
    constexpr int VPR_W = D * (int)sizeof(op_t) / 16;   // 16-byte vectors per [C][D] row
    constexpr int VPR_K = C * (int)sizeof(op_t) / 16;   // per [D][C] row
    constexpr int NV_W = C * VPR_W, NV_K = D * VPR_K, NV_G = D * 4 / 16;
    constexpr int NV = 2 * NV_W + NV_K + NV_G;
    constexpr int PER = (NV + NT - 1) / NT;
    // W, Qe and Kbar^T are contiguous at the start of a card, Gamma follows the
    // op-typed part.  Vector v of the staging set -> card vector index / LDS byte offset.
    auto src_vec = [&](int v) -> int {
        return v < 2 * NV_W + NV_K ? v : (int)(CD::OP_ELEMS * sizeof(op_t) / 16) + (v - 2 * NV_W - NV_K);
    };
    auto lds_off = [&](int v) -> int64_t {
        if (v < 2 * NV_W) {
            const int mat = v / NV_W, w = v % NV_W, r = w / VPR_W, cv = w % VPR_W;
            return mat * L::B_W + ((int64_t)r * SW) * (int64_t)sizeof(op_t) + cv * 16;
        }
        if (v < 2 * NV_W + NV_K) {
            const int w = v - 2 * NV_W, r = w / VPR_K, cv = w % VPR_K;
            return 2 * L::B_W + ((int64_t)r * SK) * (int64_t)sizeof(op_t) + cv * 16;
        }
        return 2 * L::B_W + L::B_K + (int64_t)(v - 2 * NV_W - NV_K) * 16;
    };

    const raw_t* gz = static_cast<const raw_t*>(p.gate);
    typename Out::raw_t* gy = static_cast<typename Out::raw_t*>(p.out);
    uint4 reg[PER];
#pragma unroll
    for (int j = 0; j < PER; ++j) reg[j] = make_uint4(0u, 0u, 0u, 0u);
    if (NC > 0) {
        const uint4* src = reinterpret_cast<const uint4*>(cards);
#pragma unroll
        for (int j = 0; j < PER; ++j) {
            const int v = tid + j * NT;
            if (v < NV) *reinterpret_cast<uint4*>(smem + lds_off(v)) = src[src_vec(v)];
        }
    }
    __syncthreads();

    for (int64_t ci = 0; ci < NC; ++ci) {
        const int buf = (int)(ci & 1);
        const bool more = ci + 1 < NC;
        {   // prefetch the next card into registers (unconditional loads keep them in VGPRs)
            const uint4* src = reinterpret_cast<const uint4*>(cards + (more ? ci + 1 : ci) * cbytes);
#pragma unroll
            for (int j = 0; j < PER; ++j) {
                const int v = tid + j * NT;
                reg[j] = src[src_vec(v < NV ? v : 0)];
            }
        }
        const op_t* Wl = reinterpret_cast<const op_t*>(smem + buf * L::B_BUF);
        const op_t* Ql = reinterpret_cast<const op_t*>(smem + buf * L::B_BUF + L::B_W);
        const op_t* Kl = reinterpret_cast<const op_t*>(smem + buf * L::B_BUF + 2 * L::B_W);
        const float* Gl = reinterpret_cast<const float*>(smem + buf * L::B_BUF + 2 * L::B_W + L::B_K);
        const op_t* card = reinterpret_cast<const op_t*>(cards + ci * cbytes);
        const int64_t tbase = ci * C;
        // this lane's gate logits of the chunk (rows 16 mt + 4 g4 + i, column col), loaded ahead
        // of the products and of the output stores, each from a token inside the sequence
        float zl[NMT][4];
#pragma unroll
        for (int mt = 0; mt < NMT; ++mt)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int64_t t = tbase + 16 * mt + 4 * g4 + i;
                zl[mt][i] = SUM ? 0.f : In::load(gz, ((tb + (t < T ? t : T - 1)) * H + h) * D + col);
            }

        floatx4 U[NMT];
        if constexpr (F32) {
#pragma unroll
            for (int mt = 0; mt < NMT; ++mt) {
                floatx4 aw = zero4(), aq = zero4();
                const op_t* wr = Wl + (16 * mt + m16) * SW;
                const op_t* qr = Ql + (16 * mt + m16) * SW;
#pragma unroll
                for (int ct = 0; ct < NCT; ++ct)
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        const int cc = 16 * ct + 4 * g4 + i;
                        aw = mma_f32_k4(wr[cc], S[ct][i], aw);
                        if constexpr (!SUM) aq = mma_f32_k4(qr[cc], S[ct][i], aq);
                    }
                const float4 ut = *reinterpret_cast<const float4*>(card + CD::UT + ((int64_t)(nt * NMT + mt) * 64 + lane) * 4);
                const float4 uo = *reinterpret_cast<const float4*>(card + CD::UO + ((int64_t)(nt * NMT + mt) * 64 + lane) * 4);
                const float utv[4] = {ut.x, ut.y, ut.z, ut.w}, uov[4] = {uo.x, uo.y, uo.z, uo.w};
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    U[mt][i] = ((SUM && part == 1) ? 0.f : utv[i]) - aw[i];
                    const int64_t t = tbase + 16 * mt + 4 * g4 + i;
                    if (!SUM && t < T) {
                        const int64_t gi = ((tb + t) * H + h) * D + col;
                        gy[gi] = Out::from_float((uov[i] + aq[i]) * sigmoidf_(zl[mt][i]));
                    }
                }
            }
#pragma unroll
            for (int ct = 0; ct < NCT; ++ct) {
                floatx4 acc;
#pragma unroll
                for (int i = 0; i < 4; ++i) acc[i] = Gl[16 * ct + 4 * g4 + i] * S[ct][i];
                const op_t* kr = Kl + (16 * ct + m16) * SK;
#pragma unroll
                for (int u = 0; u < NMT; ++u)
#pragma unroll
                    for (int i = 0; i < 4; ++i) acc = mma_f32_k4(kr[16 * u + 4 * g4 + i], U[u][i], acc);
                S[ct] = acc;
            }
        } else {
            half8 Sb[NCT / 2];
#pragma unroll
            for (int kb = 0; kb < NCT / 2; ++kb)
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    Sb[kb][i] = static_cast<_Float16>(S[2 * kb][i]);
                    Sb[kb][4 + i] = static_cast<_Float16>(S[2 * kb + 1][i]);
                }
#pragma unroll
            for (int mt = 0; mt < NMT; ++mt) {
                floatx4 aw = zero4(), aq = zero4();
                const op_t* wr = Wl + (16 * mt + m16) * SW;
                const op_t* qr = Ql + (16 * mt + m16) * SW;
#pragma unroll
                for (int kb = 0; kb < NCT / 2; ++kb) {
                    const int c0 = 32 * kb + 4 * g4;
                    half8 a1, a2;
                    const half4 w0 = *reinterpret_cast<const half4*>(wr + c0);
                    const half4 w1 = *reinterpret_cast<const half4*>(wr + c0 + 16);
                    const half4 q0 = *reinterpret_cast<const half4*>(qr + c0);
                    const half4 q1 = *reinterpret_cast<const half4*>(qr + c0 + 16);
#pragma unroll
                    for (int j = 0; j < 4; ++j) {
                        a1[j] = w0[j]; a1[4 + j] = w1[j];
                        a2[j] = q0[j]; a2[4 + j] = q1[j];
                    }
                    aw = mma_f16_k32(a1, Sb[kb], aw);
                    if constexpr (!SUM) aq = mma_f16_k32(a2, Sb[kb], aq);
                }
                const half4 ut = *reinterpret_cast<const half4*>(card + CD::UT + ((int64_t)(nt * NMT + mt) * 64 + lane) * 4);
                const half4 uo = *reinterpret_cast<const half4*>(card + CD::UO + ((int64_t)(nt * NMT + mt) * 64 + lane) * 4);
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    U[mt][i] = ((SUM && part == 1) ? 0.f : static_cast<float>(ut[i])) - aw[i];
                    const int64_t t = tbase + 16 * mt + 4 * g4 + i;
                    if (!SUM && t < T) {
                        const int64_t gi = ((tb + t) * H + h) * D + col;
                        gy[gi] = Out::from_float((static_cast<float>(uo[i]) + aq[i]) * sigmoidf_(zl[mt][i]));
                    }
                }
            }
#pragma unroll
            for (int ct = 0; ct < NCT; ++ct) {
                floatx4 acc;
#pragma unroll
                for (int i = 0; i < 4; ++i) acc[i] = Gl[16 * ct + 4 * g4 + i] * S[ct][i];
                const op_t* kr = Kl + (16 * ct + m16) * SK;
#pragma unroll
                for (int u = 0; u + 1 < NMT; u += 2) {
                    const int t0_ = 32 * (u / 2) + 4 * g4;
                    const half4 k0 = *reinterpret_cast<const half4*>(kr + t0_);
                    const half4 k1 = *reinterpret_cast<const half4*>(kr + t0_ + 16);
                    half8 av, bv;
#pragma unroll
                    for (int j = 0; j < 4; ++j) {
                        av[j] = k0[j]; av[4 + j] = k1[j];
                        bv[j] = static_cast<_Float16>(U[u][j]);
                        bv[4 + j] = static_cast<_Float16>(U[u + 1][j]);
                    }
                    acc = mma_f16_k32(av, bv, acc);
                }
                if constexpr (NMT % 2 == 1) {  // odd tile count: a K = 32 step with its upper half zeroed
                    const int u = NMT - 1;
                    const half4 a4 = *reinterpret_cast<const half4*>(kr + 16 * u + 4 * g4);
                    half8 av, bv;
#pragma unroll
                    for (int j = 0; j < 4; ++j) {
                        av[j] = a4[j];
                        bv[j] = static_cast<_Float16>(U[u][j]);
                        av[4 + j] = bv[4 + j] = static_cast<_Float16>(0.f);
                    }
                    acc = mma_f16_k32(av, bv, acc);
                }
                S[ct] = acc;
            }
        }
        if (!SUM && p.snap && (ci + 1) % p.snap_chunks == 0 && (ci + 1) * C <= T) {
            // block-granular snapshot: the state after (ci + 1) C tokens of the sequence
            const int64_t slot = tb / (C * p.snap_chunks) + b + (ci + 1) / p.snap_chunks - 1;
            float* dst = p.snap + (slot * H + h) * (int64_t)D * D;
#pragma unroll
            for (int ct = 0; ct < NCT; ++ct)
#pragma unroll
                for (int i = 0; i < 4; ++i) dst[(16 * ct + 4 * g4 + i) * D + col] = S[ct][i];
        }
        if (more) {
            unsigned char* base = smem + (buf ^ 1) * L::B_BUF;
#pragma unroll
            for (int j = 0; j < PER; ++j) {
                const int v = tid + j * NT;
                if (v < NV) *reinterpret_cast<uint4*>(base + lds_off(v)) = reg[j];
            }
        }
        __syncthreads();
    }

    if (SUM) {
        float* dst = (part == 1 ? p.sum_m : p.sum_b) + unit * p.sum_stride;
#pragma unroll
        for (int ct = 0; ct < NCT; ++ct)
#pragma unroll
            for (int i = 0; i < 4; ++i) dst[(16 * ct + 4 * g4 + i) * D + col] = S[ct][i];
    } else if (p.sT) {
        float* sT = p.sT + unit * (int64_t)D * D;
#pragma unroll
        for (int ct = 0; ct < NCT; ++ct)
#pragma unroll
            for (int i = 0; i < 4; ++i) sT[(16 * ct + 4 * g4 + i) * D + col] = S[ct][i];
    }
}

// ---------------------------------------------------------------------------
// host side
int64_t prefill_card_bytes(int bf16, int C, int D) {
    const bool f = !bf16;
#define KDA_CARD(CC, DD)                                                     \
    if (C == CC && D == DD) return f ? Card<CC, DD, true>::BYTES : Card<CC, DD, false>::BYTES;
    KDA_CARD(16, 64) KDA_CARD(32, 64) KDA_CARD(64, 64)
    KDA_CARD(16, 128) KDA_CARD(32, 128) KDA_CARD(64, 128)
#undef KDA_CARD
    return -1;
}

template <int C, int D, bool F32, class In, class Out, int NWV, bool SUM = false>
static hipError_t launch_t(const PrepParams& pp, const RecurParams& rp, hipStream_t stream) {
    using LP = PrepLds<C, D, F32, In>;
    using LR = RecurLds<C, D, F32>;
    if (pp.NC > 0) {
        auto kp = kda_prep_kernel<C, D, F32, In>;
        hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kp),
                                           hipFuncAttributeMaxDynamicSharedMemorySize, (int)LP::TOTAL);
        if (e != hipSuccess) return e;
        // a variable-length grid covers the most chunks its offsets can give (pp.NC)
        dim3 grid((unsigned)(pp.vco ? pp.NC * pp.H : pp.NC * pp.H * pp.B));
        hipLaunchKernelGGL(kp, grid, dim3(256), LP::TOTAL, stream, pp);
        e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    auto kr = kda_recur_kernel<C, D, F32, In, Out, NWV, SUM>;
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kr),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)LR::TOTAL);
    if (e != hipSuccess) return e;
    const int64_t blocks = rp.B * rp.H * (D / (16 * NWV)) * (SUM ? 2 : 1);
    hipLaunchKernelGGL(kr, dim3((unsigned)blocks), dim3(NWV * 64), LR::TOTAL, stream, rp);
    return hipGetLastError();
}

bool prefill_supported(int bf16, int C, int D) {
    if (D != 64 && D != 128) return false;
    if (C != 16 && C != 32 && C != 64) return false;
    if (!bf16 && D == 128 && C == 64) return false;  // fp32 tiles exceed the LDS budget
    return true;
}

template <int C, int D, bool F32, class In>
static hipError_t launch_o(int out_bf16, const PrepParams& pp, const RecurParams& rp,
                           hipStream_t stream) {
    constexpr int NWV = D == 128 ? 4 : 2;
    return out_bf16 ? launch_t<C, D, F32, In, InBF16, NWV>(pp, rp, stream)
                    : launch_t<C, D, F32, In, InF32, NWV>(pp, rp, stream);
}

// Segment summary on the general path: the cards, then one state pass per (b, h) that
// carries b (from zero) and M (from the identity) in separate column blocks.
hipError_t launch_summary(int bf16, int C, int D, const PrepParams& pp, float* M, float* b,
                          hipStream_t stream) {
    if (C == 64 && bf16) return launch_summary64(D, pp, M, b, stream);
    RecurParams rp{};
    rp.B = pp.B;
    rp.T = pp.T;
    rp.H = pp.H;
    rp.NC = pp.NC;
    rp.ws = pp.ws;
    rp.nseg = 1;
    rp.seg_len = pp.NC;
    rp.sum_b = b;
    rp.sum_m = M;
    rp.sum_stride = (int64_t)D * D;
    if (pp.NC < 1) return hipErrorInvalidValue;
#define KDA_S(CC, DD)                                                                                     \
    if (C == CC && D == DD)                                                                               \
        return bf16 ? launch_t<CC, DD, false, InBF16, InF32, DD == 128 ? 4 : 2, true>(pp, rp, stream)    \
                    : launch_t<CC, DD, true, InF32, InF32, DD == 128 ? 4 : 2, true>(pp, rp, stream);
    KDA_S(16, 64) KDA_S(32, 64) KDA_S(64, 64) KDA_S(16, 128) KDA_S(32, 128)
#undef KDA_S
    return hipErrorInvalidValue;
}

hipError_t launch_prefill(int bf16, int out_bf16, int C, int D, const PrepParams& pp,
                          const RecurParams& rp, hipStream_t stream) {
#define KDA_L(CC, DD)                                                              \
    if (C == CC && D == DD)                                                        \
        return bf16 ? launch_o<CC, DD, false, InBF16>(out_bf16, pp, rp, stream)   \
                    : launch_o<CC, DD, true, InF32>(out_bf16, pp, rp, stream);
    if (C == 64 && bf16) return launch_prefill64(D, out_bf16, pp, rp, stream);
    KDA_L(16, 64) KDA_L(32, 64) KDA_L(64, 64) KDA_L(16, 128) KDA_L(32, 128)
#undef KDA_L
    if (C == 64 && bf16) return launch_prefill64(D, out_bf16, pp, rp, stream);
    return hipErrorInvalidValue;
}

}  // namespace kda
