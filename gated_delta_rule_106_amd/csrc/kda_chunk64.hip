// Chunkwise KDA forward for bf16 inputs with 64-token chunks (gfx950).
//
// Same algebra as the general kernels (the per-token recurrence of page "3T
// models are no longer magic", section "Gate 1: KDA makes it computable",
// evaluated chunk by chunk as on page "Kimi K3 report walk-through", sections
// "Compute paradigm" and "Hierarchical chunking of linear attention"), laid out
// for throughput on CDNA4:
//
// kda_prep64_kernel  persistent workgroups of 4 waves, one (b, h, chunk) item at a
//   time with the next item's inputs prefetched into registers.  Wave a owns the
//   16-token tile a of the chunk and keeps it in registers in MFMA operand
//   layout (lane = token, 4 consecutive key channels per 16-channel tile).  The
//   cumulative log-decay is a DPP prefix scan across the 16 lanes of a row.
//   Decay is folded into q and k as an absolute-position rescaling measured
//   from the start of each 16-token tile (page "Kimi K3 report walk-through",
//   section "Numerical stability & co-design": inside one tile the inverse
//   factor stays below 2^116 given the 0.67 % retention floor):
//       KR = k 2^{P},  QR = q 2^{P},  KC = k 2^{-P},  KE = k 2^{tau - P},
//   P = prefix sum of log2(alpha) inside the tile, tau = its total.  Pair
//   products inside a tile use KR.KC^T on the fp32 MFMA (the operands span
//   2^{+-116}); across tiles both operands are <= |k| and one fp16 pass
//   suffices.  The unit-lower-triangular system (I + A) is solved
//   with register forward substitution on the four 16x16 diagonal blocks and
//   fp32 MFMA block products for the rest.  The remaining contractions are
//   arranged so that their accumulators come out in exactly the fragment
//   layout the sequential kernel consumes, so the "update card" of the chunk
//   is written with coalesced 16-byte stores.
//
// kda_rec64_kernel  one workgroup per (b, h, group of NCONS 16-column value
//   tiles): per tile a chain wave carries the fp32 state of its columns in MFMA
//   accumulators across all chunks and an output wave forms the chunk's
//   read-out; four producer waves stage the next cards through registers into
//   a double-buffered LDS ring and gate and store y.
//   Workgroups of one head are placed on one XCD so its cards are fetched
//   into one L2.
//
// Card of one (b, h, chunk), fp16 unless noted (lane l = 16 g + m):
//   W   [mt][kb] 64 lanes x 8: -W[16mt + m][c(kb, g, j)]
//   QE  [mt][kb] 64 lanes x 8:  Qe[16mt + m][c(kb, g, j)]        Qe = Q~ - P W
//   KBT [ct][u]  64 lanes x 8:  Kbar[c(u, g, j)][16ct + m]
//   UT  [nt][mt] 64 lanes x 4:  U~[16mt + 4g + i][16nt + m]
//   UO  [nt][mt] 64 lanes x 4:  Uo[16mt + 4g + i][16nt + m]       Uo = P U~
//   GAM [D] fp32: 2^{gamma_C}, the decay of the whole chunk per key channel
// with c(x, g, j) = 32x + 4g + j (j < 4), 32x + 16 + 4g + (j - 4) (j >= 4):
// the K-index order in which two stacked accumulator tiles (rows 4g .. 4g+3
// in lane group g) feed the next MFMA directly as its B operand.
#include <type_traits>

#include "kda_device.h"
#include "kda_prefill.h"

namespace kda {
namespace c64 {

constexpr int C = 64;
constexpr int NSUB = 4;

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

template <int CTRL>
__device__ __forceinline__ float dpp_mov(float x) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xf, 0xf, true));
}

// inclusive prefix sum over the 16 lanes of a DPP row (lanes 16g .. 16g+15)
__device__ __forceinline__ float row_scan16(float x) {
    x += dpp_mov<0x111>(x);  // row_shr:1
    x += dpp_mov<0x112>(x);  // row_shr:2
    x += dpp_mov<0x114>(x);  // row_shr:4
    x += dpp_mov<0x118>(x);  // row_shr:8
    return x;
}

// value held by lane 15 of this lane's 16-lane row
__device__ __forceinline__ float row_last(float x) {
    return __int_as_float(__builtin_amdgcn_ds_swizzle(__float_as_int(x), 0x1F0));
}

// physical index of logical K element j (0..7) of lane group g in K-step x
__device__ __forceinline__ constexpr int cmap(int x, int g, int j) {
    return 32 * x + 4 * g + (j & 3) + ((j >> 2) << 4);
}

__device__ __forceinline__ half4 ld_h4(const _Float16* p) { return *reinterpret_cast<const half4*>(p); }
__device__ __forceinline__ half8 ld_h8(const _Float16* p) { return *reinterpret_cast<const half8*>(p); }

__device__ __forceinline__ half8 cat_h8(const half4& lo, const half4& hi) {
    half8 r;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        r[j] = lo[j];
        r[4 + j] = hi[j];
    }
    return r;
}

__device__ __forceinline__ half8 pack_h8(const floatx4& lo, const floatx4& hi) {
    half8 r;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        r[j] = static_cast<_Float16>(lo[j]);
        r[4 + j] = static_cast<_Float16>(hi[j]);
    }
    return r;
}

__device__ __forceinline__ half4 pack_h4(const floatx4& x) {
    half4 r;
#pragma unroll
    for (int j = 0; j < 4; ++j) r[j] = static_cast<_Float16>(x[j]);
    return r;
}

__device__ __forceinline__ floatx4 unpack_h4(const half4& x) {
    floatx4 r;
#pragma unroll
    for (int j = 0; j < 4; ++j) r[j] = static_cast<float>(x[j]);
    return r;
}

__device__ __forceinline__ floatx4 mma_f32_k16(const float4& a, const floatx4& b, floatx4 acc) {
    acc = mma_f32_k4(a.x, b[0], acc);
    acc = mma_f32_k4(a.y, b[1], acc);
    acc = mma_f32_k4(a.z, b[2], acc);
    acc = mma_f32_k4(a.w, b[3], acc);
    return acc;
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
// barrier that orders LDS only: global stores issued before it keep draining
__device__ __forceinline__ void lds_barrier() {
    wait_lgkm_zero();
    bare_barrier();
}

// ---------------------------------------------------------------------------
template <int D>
struct Card {
    static constexpr int KB = D / 32, NCT = D / 16;
    static constexpr int64_t FRAG = 1024;  // 64 lanes x 16 B
    static constexpr int64_t HFRAG = 512;  // 64 lanes x 8 B
    static constexpr int64_t W = 0;
    static constexpr int64_t QE = W + 4 * KB * FRAG;
    static constexpr int64_t KBT = QE + 4 * KB * FRAG;
    static constexpr int64_t UT = KBT + NCT * 2 * FRAG;
    static constexpr int64_t UO = UT + NCT * 4 * HFRAG;
    static constexpr int64_t GAM = UO + NCT * 4 * HFRAG;
    static constexpr int64_t BYTES = GAM + D * 4;
    static_assert(BYTES % 16 == 0, "card alignment");
};

template <int D>
struct PrepL {
    static constexpr int KB = D / 32;
    static constexpr int SR = D + 8;  // fp16 [token][channel] row stride (halves)
    static constexpr int ST = C + 8;  // fp16 [channel][token] row stride (halves)
    static constexpr int SA = C + 4;  // fp32 [64][64] row stride (floats)
    static constexpr int SP = C + 8;  // fp16 [64][64] row stride (halves)
    static constexpr int64_t B_KEF = (int64_t)NSUB * KB * 64 * 16;  // KE fragments
    static constexpr int64_t B_LINV = 64 * SA * 4;
    static constexpr int64_t B_KE = B_KEF > B_LINV ? B_KEF : B_LINV;
    static constexpr int64_t OFF_BETA = 0;                     // fp32 [64]
    static constexpr int64_t OFF_ETAU = 256;                   // fp32 [4][D]: decay over each tile
    static constexpr int64_t OFF_KE = OFF_ETAU + 4 * D * 4;    // KE fragments; later Linv fp32 [64][SA]
    static constexpr int64_t OFF_KT = OFF_KE + B_KE;           // fp16 K~^T [D][ST]; later -W^T
    static constexpr int64_t OFF_KBT = OFF_KT + D * ST * 2;    // fp16 Kbar^T [D][ST]
    static constexpr int64_t OFF_VT = OFF_KBT + D * ST * 2;    // fp16 V^T [D][ST]
    static constexpr int64_t OFF_Q = OFF_VT + D * ST * 2;      // fp16 Q~ [64][SR]
    static constexpr int64_t OFF_A = OFF_Q + 64 * SR * 2;      // fp32 A [64][SA]
    static constexpr int64_t OFF_P = OFF_A + 64 * SA * 4;      // fp16 P [64][SP]
    static constexpr int64_t OFF_T = OFF_P + 64 * SP * 2;      // fp16 T [64][SP]
    static constexpr int64_t TOTAL = OFF_T + 64 * SP * 2;
    static_assert(TOTAL <= 160 * 1024, "prep LDS budget");
    static_assert(OFF_KE % 16 == 0 && OFF_KT % 16 == 0 && OFF_KBT % 16 == 0 && OFF_VT % 16 == 0 &&
                      OFF_Q % 16 == 0 && OFF_A % 16 == 0 && OFF_P % 16 == 0 && OFF_T % 16 == 0,
                  "prep LDS alignment");
};

// ---------------------------------------------------------------------------
// kernel 1: update cards.  Persistent: each workgroup walks (b, h, chunk) items
// with a stride of the grid size and prefetches the next item's raw inputs into
// registers while it builds the current card.
template <int D>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1)))
void kda_prep64_kernel(PrepParams p) {
    using L = PrepL<D>;
    using CD = Card<D>;
    constexpr int NCT = D / 16, KB = D / 32;
    constexpr int SR = L::SR, ST = L::ST, SA = L::SA, SP = L::SP;
    extern __shared__ __align__(16) unsigned char smem[];
    float* s_beta = reinterpret_cast<float*>(smem + L::OFF_BETA);
    float* s_etau = reinterpret_cast<float*>(smem + L::OFF_ETAU);
    _Float16* s_ke = reinterpret_cast<_Float16*>(smem + L::OFF_KE);
    float* s_linv = reinterpret_cast<float*>(smem + L::OFF_KE);
    _Float16* s_kt = reinterpret_cast<_Float16*>(smem + L::OFF_KT);
    _Float16* s_kbt = reinterpret_cast<_Float16*>(smem + L::OFF_KBT);
    _Float16* s_vt = reinterpret_cast<_Float16*>(smem + L::OFF_VT);
    _Float16* s_q = reinterpret_cast<_Float16*>(smem + L::OFF_Q);
    float* s_a = reinterpret_cast<float*>(smem + L::OFF_A);
    _Float16* s_p = reinterpret_cast<_Float16*>(smem + L::OFF_P);
    _Float16* s_t = reinterpret_cast<_Float16*>(smem + L::OFF_T);

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int m16 = lane & 15, g4 = lane >> 4;
    const int a = wave;             // this wave's 16-token tile
    const int rl = 16 * a + m16;    // this lane's token within the chunk
    const int64_t NC = p.NC, T = p.T, H = p.H;
    const int64_t items = p.B * H * NC;
    const uint16_t* gq = static_cast<const uint16_t*>(p.q);
    const uint16_t* gk = static_cast<const uint16_t*>(p.k);
    const uint16_t* gv = static_cast<const uint16_t*>(p.v);
    const uint16_t* gla = static_cast<const uint16_t*>(p.la);
    const uint16_t* gbeta = static_cast<const uint16_t*>(p.beta);
    const bool clamp = p.clamp != 0;

    // raw inputs of token rl: per 16-channel tile ct, the 4 bf16 channels 16ct + 4g4 .. +3
    uint2 nq[NCT], nk[NCT], nv[NCT], nla[NCT];
    uint16_t nbeta;
    auto fetch = [&](int64_t it) {
        const int64_t n = it % NC, unit = it / NC;
        const int64_t b = unit / H, h = unit % H;
        const int64_t tok = n * C + rl;
        const int64_t row = (b * T + (tok < T ? tok : T - 1)) * H + h;  // in bounds; zeroed below
#pragma unroll
        for (int ct = 0; ct < NCT; ++ct) {
            const int64_t off = row * D + 16 * ct + 4 * g4;
            nq[ct] = *reinterpret_cast<const uint2*>(gq + off);
            nk[ct] = *reinterpret_cast<const uint2*>(gk + off);
            nv[ct] = *reinterpret_cast<const uint2*>(gv + off);
            nla[ct] = *reinterpret_cast<const uint2*>(gla + off);
        }
        nbeta = gbeta[row];
    };
    auto elem = [](const uint2& w, int i) -> float {
        const uint32_t x = (i < 2) ? w.x : w.y;
        return (i & 1) ? __uint_as_float(x & 0xffff0000u) : __uint_as_float(x << 16);
    };

    int64_t item = blockIdx.x;
    if (item < items) fetch(item);
    for (; item < items; item += gridDim.x) {
        const int64_t n = item % NC;
        const int64_t t0 = n * C;
        const bool valid = t0 + rl < T;
        unsigned char* card = static_cast<unsigned char*>(p.ws) + item * CD::BYTES;
        uint2 rq[NCT], rk[NCT], rv[NCT], rla[NCT];
#pragma unroll
        for (int ct = 0; ct < NCT; ++ct) {  // identity tokens past the end: q = k = v = log alpha = 0
            const uint2 z2 = make_uint2(0u, 0u);
            rq[ct] = valid ? nq[ct] : z2;
            rk[ct] = valid ? nk[ct] : z2;
            rv[ct] = valid ? nv[ct] : z2;
            rla[ct] = valid ? nla[ct] : z2;
        }
        const float beta_mine = valid ? bf16_bits_to_float(nbeta) : 0.f;
        if (item + gridDim.x < items) fetch(item + gridDim.x);

        // ---- phase 1 (per tile): decay inside the tile, in-tile pair products
        if (g4 == 0) s_beta[rl] = beta_mine;
        half8 kr16[KB], qr16[KB];
        floatx4 accA = zero4(), accP = zero4();
#pragma unroll
        for (int kb = 0; kb < KB; ++kb) {
            half8 ke;
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                const int ct = 2 * kb + (j >> 2), i = j & 3;
                const float l = clamp_log_alpha(elem(rla[ct], i), clamp) * kLog2e;
                const float P = row_scan16(l);      // log2 decay from the tile start, inclusive
                const float E = fast_exp2(P);       // <= 1
                const float Einv = fast_exp2(-P);   // >= 1, < 2^116 under the floor
                const float Et = row_last(E);       // decay over the whole tile
                const float kf = elem(rk[ct], i), qf = elem(rq[ct], i);
                const float KR = kf * E, QR = qf * E, KC = kf * Einv;
                // K-step (kb, j): lane group g4 supplies channel cmap(kb, g4, j) to both operands
                accA = mma_f32_k4(KR, KC, accA);
                accP = mma_f32_k4(QR, KC, accP);
                kr16[kb][j] = static_cast<_Float16>(KR);
                qr16[kb][j] = static_cast<_Float16>(QR);
                ke[j] = static_cast<_Float16>(kf * (Einv * Et));  // decay from after this token to the tile end
                const int c = cmap(kb, g4, j);
                if (m16 == 0) s_etau[a * D + c] = Et;
                s_vt[c * ST + rl] = static_cast<_Float16>(elem(rv[ct], i));
            }
            // KE fragment of this tile: the B operand of the pairs (later tile, this tile)
            *reinterpret_cast<half8*>(s_ke + ((a * KB + kb) * 64 + lane) * 8) = ke;
        }
        // diagonal blocks of A (strictly lower, rows scaled by beta) and P (lower)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int r = 4 * g4 + i, s = m16;
            const float br = __shfl(beta_mine, r);
            s_a[(16 * a + r) * SA + 16 * a + s] = (s < r) ? br * accA[i] : 0.f;
            s_p[(16 * a + r) * SP + 16 * a + s] = static_cast<_Float16>((s <= r) ? accP[i] : 0.f);
#pragma unroll
            for (int bb = 0; bb < NSUB; ++bb)
                if (bb > a) s_p[(16 * a + r) * SP + 16 * bb + s] = static_cast<_Float16>(0.f);
        }
        lds_barrier();  // (1) tile decays, KE fragments, V^T and beta are in LDS

        // ---- phase 2 (per tile): chunk-relative operands and the pairs with earlier tiles.
        // Decay factors across tiles are products of the per-tile decays 2^{tau}.
        floatx4 pa[NSUB - 1], pp[NSUB - 1];
#pragma unroll
        for (int bb = 0; bb < NSUB - 1; ++bb) pa[bb] = pp[bb] = zero4();
#pragma unroll
        for (int kb = 0; kb < KB; ++kb) {
            float et[NSUB][8];
#pragma unroll
            for (int a2 = 0; a2 < NSUB; ++a2) {
                const float4 lo = *reinterpret_cast<const float4*>(s_etau + a2 * D + 32 * kb + 4 * g4);
                const float4 hi = *reinterpret_cast<const float4*>(s_etau + a2 * D + 32 * kb + 16 + 4 * g4);
                et[a2][0] = lo.x; et[a2][1] = lo.y; et[a2][2] = lo.z; et[a2][3] = lo.w;
                et[a2][4] = hi.x; et[a2][5] = hi.y; et[a2][6] = hi.z; et[a2][7] = hi.w;
            }
            half8 q8;
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                const int c = cmap(kb, g4, j);
                float erho = 1.f, eaft = 1.f;  // decay before this tile / after this tile
#pragma unroll
                for (int a2 = 0; a2 < NSUB; ++a2) {
                    if (a2 < a) erho *= et[a2][j];
                    if (a2 > a) eaft *= et[a2][j];
                }
                const float ke = static_cast<float>(s_ke[((a * KB + kb) * 64 + lane) * 8 + j]);
                s_kt[c * ST + rl] = static_cast<_Float16>(static_cast<float>(kr16[kb][j]) * erho);  // K~ = k 2^{g}
                s_kbt[c * ST + rl] = static_cast<_Float16>(ke * eaft);                             // Kbar = k 2^{g_C - g}
                q8[j] = static_cast<_Float16>(static_cast<float>(qr16[kb][j]) * erho);             // Q~ = q 2^{g}
            }
            half4 qlo, qhi;
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                qlo[j] = q8[j];
                qhi[j] = q8[4 + j];
            }
            *reinterpret_cast<half4*>(s_q + rl * SR + 32 * kb + 4 * g4) = qlo;
            *reinterpret_cast<half4*>(s_q + rl * SR + 32 * kb + 16 + 4 * g4) = qhi;
            // pairs (a, bb), bb < a: reference point at the end of tile a-1; both operands <= |k|
#pragma unroll
            for (int bb = 0; bb < NSUB - 1; ++bb) {
                if (bb < a) {
                    const half8 keb = ld_h8(s_ke + ((bb * KB + kb) * 64 + lane) * 8);
                    half8 col;
#pragma unroll
                    for (int j = 0; j < 8; ++j) {
                        float f = 1.f;  // decay over the tiles strictly between bb and a
#pragma unroll
                        for (int a2 = 1; a2 < NSUB - 1; ++a2)
                            if (a2 > bb && a2 < a) f *= et[a2][j];
                        col[j] = static_cast<_Float16>(static_cast<float>(keb[j]) * f);
                    }
                    pa[bb] = mma_f16_k32(kr16[kb], col, pa[bb]);
                    pp[bb] = mma_f16_k32(qr16[kb], col, pp[bb]);
                }
            }
        }
#pragma unroll
        for (int bb = 0; bb < NSUB - 1; ++bb) {
            if (bb < a) {
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int r = 4 * g4 + i;
                    s_a[(16 * a + r) * SA + 16 * bb + m16] = s_beta[16 * a + r] * pa[bb][i];
                    s_p[(16 * a + r) * SP + 16 * bb + m16] = static_cast<_Float16>(pp[bb][i]);
                }
            }
        }
        // Gamma = 2^{g_C} per key channel
        if (tid < D) {
            float gm = 1.f;
#pragma unroll
            for (int a2 = 0; a2 < NSUB; ++a2) gm *= s_etau[a2 * D + tid];
            reinterpret_cast<float*>(card + CD::GAM)[tid] = gm;
        }
        lds_barrier();  // (2) A, P, K~^T, Kbar^T, Q~ complete

        // ---- phase 3: Linv = (I + A)^{-1} (unit lower triangular, blocked by 16) and
        //      T = Linv diag(beta) in fp16
        if (wave == 0) {  // diagonal blocks: lane group g4 = block, lane m16 = column
            const int ab = g4, j = m16;
            const float* Ab = s_a + (16 * ab) * SA + 16 * ab;
            float x[16];
#pragma unroll
            for (int r = 0; r < 16; ++r) x[r] = (r == j) ? 1.f : 0.f;
#pragma unroll
            for (int r = 1; r < 16; ++r) {
                float acc = x[r];
#pragma unroll
                for (int q = 0; q < r; ++q) acc -= Ab[r * SA + q] * x[q];
                x[r] = acc;
            }
            const float bj = s_beta[16 * ab + j];
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                s_linv[(16 * ab + r) * SA + 16 * ab + j] = x[r];
                s_t[(16 * ab + r) * SP + 16 * ab + j] = static_cast<_Float16>(x[r] * bj);
            }
        }
        lds_barrier();
        // off-diagonal blocks by block diagonal d: Linv_{a,a-d} = -X_a sum_c A_{a,c} Linv_{c,a-d}
        auto blk_a = [&](int r, int c) { return s_a + (16 * r) * SA + 16 * c; };
        auto blk_x = [&](int r, int c) { return s_linv + (16 * r) * SA + 16 * c; };
        auto mm = [&](const float* mp, const float* np, floatx4 acc) {  // acc += M N (row-major blocks)
            const float4 av = *reinterpret_cast<const float4*>(mp + m16 * SA + 4 * g4);
            floatx4 bv;
#pragma unroll
            for (int s = 0; s < 4; ++s) bv[s] = np[(4 * g4 + s) * SA + m16];
            return mma_f32_k16(av, bv, acc);
        };
#pragma unroll
        for (int d = 1; d < NSUB; ++d) {
            if (wave >= d) {
                floatx4 y = zero4();
                for (int c = wave - d; c < wave; ++c) y = mm(blk_a(wave, c), blk_x(c, wave - d), y);
                const float4 xv = *reinterpret_cast<const float4*>(blk_x(wave, wave) + m16 * SA + 4 * g4);
                const floatx4 z = mma_f32_k16(xv, y, zero4());
                float* dst = blk_x(wave, wave - d);
                const float bcol = s_beta[16 * (wave - d) + m16];
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    dst[(4 * g4 + i) * SA + m16] = -z[i];
                    s_t[(16 * wave + 4 * g4 + i) * SP + 16 * (wave - d) + m16] = static_cast<_Float16>(-z[i] * bcol);
                }
            }
            lds_barrier();
        }

        // ---- phase 4: card.  Jobs 0..KB-1: key-channel pair kb (W, Qe, Kbar^T);
        //      jobs KB..2KB-1: value-column pair (U~, Uo)
        // sum over tokens s < 16 (mt + 1) of A_row[s] * B_row[s] (rows in LDS, tokens contiguous).
        // A trailing 16-token step is a K = 32 step with its upper half zeroed: one MFMA shape
        // per accumulator chain.
        auto kloop = [&](const _Float16* arow, const _Float16* brow, int mt, floatx4 acc) {
            const int kend = 16 * (mt + 1);
            int s0 = 0;
            for (; s0 + 32 <= kend; s0 += 32)
                acc = mma_f16_k32(ld_h8(arow + s0 + 8 * g4), ld_h8(brow + s0 + 8 * g4), acc);
            if (s0 < kend) {
                const half4 z4 = {0, 0, 0, 0};
                acc = mma_f16_k32(cat_h8(ld_h4(arow + s0 + 4 * g4), z4), cat_h8(ld_h4(brow + s0 + 4 * g4), z4), acc);
            }
            return acc;
        };
        for (int job = wave; job < 2 * KB; job += 4) {
            if (job < KB) {
                const int kb = job;
                floatx4 wt[2][4];
#pragma unroll
                for (int cl = 0; cl < 2; ++cl)
#pragma unroll
                    for (int mt = 0; mt < 4; ++mt)  // W^T tile = K~^T T^T
                        wt[cl][mt] = kloop(s_kt + (16 * (2 * kb + cl) + m16) * ST, s_t + (16 * mt + m16) * SP, mt,
                                           zero4());
#pragma unroll
                for (int mt = 0; mt < 4; ++mt) {
                    floatx4 n0, n1;
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        n0[i] = -wt[0][mt][i];
                        n1[i] = -wt[1][mt][i];
                    }
                    *reinterpret_cast<half8*>(card + CD::W + ((mt * KB + kb) * 64 + lane) * 16) = pack_h8(n0, n1);
                }
                // -W^T over this pair's rows of K~^T (only this wave reads them)
#pragma unroll
                for (int cl = 0; cl < 2; ++cl)
#pragma unroll
                    for (int mt = 0; mt < 4; ++mt)
#pragma unroll
                        for (int i = 0; i < 4; ++i)
                            s_kt[(16 * (2 * kb + cl) + 4 * g4 + i) * ST + 16 * mt + m16] =
                                static_cast<_Float16>(-wt[cl][mt][i]);
                // Qe^T tile = Q~^T + (-W^T) P^T
#pragma unroll
                for (int mt = 0; mt < 4; ++mt) {
                    floatx4 qe[2];
#pragma unroll
                    for (int cl = 0; cl < 2; ++cl) {
                        const floatx4 init =
                            unpack_h4(ld_h4(s_q + (16 * mt + m16) * SR + 16 * (2 * kb + cl) + 4 * g4));
                        qe[cl] = kloop(s_kt + (16 * (2 * kb + cl) + m16) * ST, s_p + (16 * mt + m16) * SP, mt, init);
                    }
                    *reinterpret_cast<half8*>(card + CD::QE + ((mt * KB + kb) * 64 + lane) * 16) =
                        pack_h8(qe[0], qe[1]);
                }
                // Kbar^T fragments of the two 16-channel tiles
#pragma unroll
                for (int cl = 0; cl < 2; ++cl) {
                    const int ct = 2 * kb + cl;
                    const _Float16* kr = s_kbt + (16 * ct + m16) * ST;
#pragma unroll
                    for (int u = 0; u < 2; ++u)
                        *reinterpret_cast<half8*>(card + CD::KBT + ((ct * 2 + u) * 64 + lane) * 16) =
                            cat_h8(ld_h4(kr + 32 * u + 4 * g4), ld_h4(kr + 32 * u + 16 + 4 * g4));
                }
            } else {
                const int np = job - KB;
                floatx4 ut[2][4];
#pragma unroll
                for (int cl = 0; cl < 2; ++cl) {
                    const int nt = 2 * np + cl;
#pragma unroll
                    for (int mt = 0; mt < 4; ++mt) {  // U~ tile = T V
                        ut[cl][mt] = kloop(s_t + (16 * mt + m16) * SP, s_vt + (16 * nt + m16) * ST, mt, zero4());
                        *reinterpret_cast<half4*>(card + CD::UT + ((nt * 4 + mt) * 64 + lane) * 8) =
                            pack_h4(ut[cl][mt]);
                    }
#pragma unroll
                    for (int mt = 0; mt < 4; ++mt) {  // Uo tile = P U~ (U~ accumulators as the B operand)
                        floatx4 acc = zero4();
                        const _Float16* prow = s_p + (16 * mt + m16) * SP;
#pragma unroll
                        for (int u = 0; u < 2; ++u)
                            if (2 * u <= mt)
                                acc = mma_f16_k32(
                                    cat_h8(ld_h4(prow + 32 * u + 4 * g4), ld_h4(prow + 32 * u + 16 + 4 * g4)),
                                    pack_h8(ut[cl][2 * u], ut[cl][2 * u + 1]), acc);
                        *reinterpret_cast<half4*>(card + CD::UO + ((nt * 4 + mt) * 64 + lane) * 8) = pack_h4(acc);
                    }
                }
            }
        }
        lds_barrier();  // LDS is reused by the next item
    }
}

// ---------------------------------------------------------------------------
// kernel 2: sequential pass over the cards
//
// Per workgroup, for each of its NCONS 16-column value tiles, a chain wave and an
// output wave, plus NP producer waves.  Iteration n, around the barriers A and B:
//   chain     S_n (fp16 copy) -> LDS before A; after A: U = U~ - W S_n,
//             S_{n+1} = Diag(Gamma) S_n + Kbar^T U (fp32 state in accumulators)
//   output    after A: O = Uo + Qe S_n -> LDS tile
//   producers before A: issue the loads of chunk n+2 into one of two register
//             sets, compute sigmoid(z) of chunk n and store y = O * sigmoid(z) of
//             chunk n-1 (a quarter of the tokens each, 16-byte stores);
//             after A: wait for chunk n+1 (loaded one iteration earlier) and
//             write it into LDS ring slot (n+1) % 2.
// A card is therefore in flight for two iterations, while LDS holds only two.
template <int D, int NCONS>
struct RecL {
    using CD = Card<D>;
    static constexpr int KB = D / 32;
    static constexpr int NP = 4;                          // producer waves
    static constexpr int64_t SH = CD::UT;                 // W, QE, KBT: shared by all tiles
    // per 16-column tile: U~ slice (2 KiB), Uo slice (2 KiB), gate logits [64][16] bf16 (2 KiB)
    static constexpr int64_t PER = 6 * 1024;
    static constexpr int64_t OFF_U = SH;                  // tile t2 at OFF_U + t2 * PER
    static constexpr int64_t UO_IN = 2048, Z_IN = 4096;   // offsets inside a tile block
    static constexpr int64_t OFF_G = SH + NCONS * PER;
    static constexpr int64_t STAGE = OFF_G + 1024;        // Gamma (D * 4 bytes) in a 1 KiB piece
    static constexpr int NSTAGE = 2;
    static constexpr int NPC = (int)(STAGE / 1024);       // 1 KiB pieces per card
    static constexpr int KP = (NPC + NP - 1) / NP;        // pieces per producer
    static constexpr int OST = 20;                        // [token][16 columns] row stride (elements)
    static constexpr int64_t OTILE = 64 * OST * 4;        // one tile's 64 x 16 fp32 read-out
    // sigmoid(z) tiles: fp32 with one tile; fp16 (relative error 2^-11) when two tiles
    // must share the LDS budget
    using sig_t = typename std::conditional<NCONS == 1, float, _Float16>::type;
    static constexpr int64_t STILE = 64 * OST * (int64_t)sizeof(sig_t);
    static constexpr int64_t SBX = (int64_t)KB * 64 * 16;  // fp16 copy of one tile's state (B operand)
    static constexpr int64_t OFF_O = NSTAGE * STAGE;                 // read-out O [2][NCONS]
    static constexpr int64_t OFF_S = OFF_O + 2 * NCONS * OTILE;      // sigmoid(z) [2][NCONS]
    static constexpr int64_t OFF_X = OFF_S + 2 * NCONS * STILE;      // state copies [NCONS]
    static constexpr int64_t TOTAL = OFF_X + NCONS * SBX;
    static constexpr int WAVES = 2 * NCONS + NP;
    static_assert(STAGE % 1024 == 0 && D * 4 <= 1024, "card pieces");
    static_assert(TOTAL <= 160 * 1024, "recurrence LDS budget");
    static_assert(OFF_O % 16 == 0 && OFF_X % 16 == 0, "alignment");
    static_assert(KP <= 63, "outstanding-load counter");
};

// vmcnt(n) for small compile-time n (expcnt and lgkmcnt left unconstrained)
template <int N>
__device__ __forceinline__ void wait_vm() {
    static_assert(N >= 0 && N <= 63, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | 0x0F70);
}

template <int I>
struct Int {
    static constexpr int value = I;
};

template <int D, class Out, int NCONS>
__global__ __launch_bounds__((2 * NCONS + 4) * 64) __attribute__((amdgpu_waves_per_eu(1, 2)))
void kda_rec64_kernel(RecurParams p) {
    using CD = Card<D>;
    using L = RecL<D, NCONS>;
    constexpr int NCT = D / 16, KB = D / 32, NP = L::NP, KP = L::KP;
    constexpr int G = D / (16 * NCONS);  // workgroups per head
    constexpr int OST = L::OST;
    static_assert(L::WAVES == 2 * NCONS + 4, "launch bounds");
    extern __shared__ __align__(16) unsigned char smem[];

    const int lane = lane_id(), wave = wave_id();
    const int m16 = lane & 15, g4 = lane >> 4;
    // XCD-aware placement: the G workgroups of one head share bid % 8
    const int nblk = gridDim.x, bid = blockIdx.x;
    const int logical = (bid % 8) * (nblk / 8) + bid / 8;
    const int64_t unit = logical / G;
    const int grp = logical % G;
    const int64_t units = p.B * p.H;
    if (unit >= units) return;  // padding workgroup (the whole group leaves together)
    const int64_t H = p.H, T = p.T, NC = p.NC;
    const int64_t b = unit / H, h = unit % H;
    const unsigned char* cards = static_cast<const unsigned char*>(p.ws) + unit * NC * CD::BYTES;
    const bool chain = wave < NCONS;
    const bool outw = wave >= NCONS && wave < 2 * NCONS;
    const bool prod = wave >= 2 * NCONS;
    const int pw = prod ? wave - 2 * NCONS : 0;               // producer index
    const int cs = chain ? wave : (outw ? wave - NCONS : 0);  // value tile of a chain / output wave
    const uint16_t* gz = static_cast<const uint16_t*>(p.gate);
    float* obuf = reinterpret_cast<float*>(smem + L::OFF_O);
    using sig_t = typename L::sig_t;
    sig_t* sbuf = reinterpret_cast<sig_t*>(smem + L::OFF_S);
    _Float16* sbx = reinterpret_cast<_Float16*>(smem + L::OFF_X + cs * L::SBX);
    auto zrow = [&](int64_t t) { return ((b * T + t) * H + h) * D; };  // element offset of (b, t, h, 0)

    // ---- producers: 1 KiB pieces of a card, piece j handled by producer j % NP.
    // Every piece is one 16-byte load per lane from a valid address (gate rows past T
    // are clamped to the last token; their values are never stored).
    // every producer moves exactly KP pieces; a producer short of work repeats the last
    // piece (same data to the same LDS address), which keeps its load count uniform
    auto piece_of = [&](int k) { const int j = pw + k * NP; return j < L::NPC ? j : L::NPC - 1; };
    auto piece_src = [&](int64_t c, int j) __attribute__((always_inline)) -> const u32x4* {
        const unsigned char* card = cards + c * CD::BYTES;
        if (j < (int)(L::SH / 1024)) return reinterpret_cast<const u32x4*>(card + j * 1024) + lane;
        int r = j - (int)(L::SH / 1024);
        if (r < NCONS * 6) {
            const int t2 = r / 6, q = r % 6, nt = grp * NCONS + t2;
            if (q < 4)  // U~ (q = 0, 1) and Uo (q = 2, 3) slices of tile nt
                return reinterpret_cast<const u32x4*>(card + (q < 2 ? CD::UT : CD::UO) + nt * 2048 + (q & 1) * 1024) + lane;
            int64_t t = c * C + 32 * (q - 4) + (lane >> 1);
            t = t < T ? t : T - 1;
            return reinterpret_cast<const u32x4*>(gz + zrow(t) + 16 * nt + 8 * (lane & 1));
        }
        return reinterpret_cast<const u32x4*>(card + CD::GAM) + (lane % (D / 4));  // Gamma, replicated
    };
    auto piece_dst = [&](int64_t c, int j) __attribute__((always_inline)) -> u32x4* {
        return reinterpret_cast<u32x4*>(smem + (c % L::NSTAGE) * L::STAGE + (int64_t)j * 1024) + lane;
    };
    // sigmoid and output work of one producer: 16 tokens x 4 columns per lane group
    const int tq = 16 * pw + (lane >> 2), cq = 4 * (lane & 3);
    auto sigmoid_part = [&](int64_t c) __attribute__((always_inline)) {
        const unsigned char* st = smem + (c % L::NSTAGE) * L::STAGE;
#pragma unroll
        for (int t2 = 0; t2 < NCONS; ++t2) {
            const uint2 zw = *reinterpret_cast<const uint2*>(st + L::OFF_U + t2 * L::PER + L::Z_IN + tq * 32 + cq * 2);
            sig_t* srow = sbuf + ((c & 1) * NCONS + t2) * (64 * OST) + tq * OST + cq;
            srow[0] = static_cast<sig_t>(sigmoidf_(__uint_as_float(zw.x << 16)));
            srow[1] = static_cast<sig_t>(sigmoidf_(__uint_as_float(zw.x & 0xffff0000u)));
            srow[2] = static_cast<sig_t>(sigmoidf_(__uint_as_float(zw.y << 16)));
            srow[3] = static_cast<sig_t>(sigmoidf_(__uint_as_float(zw.y & 0xffff0000u)));
        }
    };
    typename Out::raw_t* gy = static_cast<typename Out::raw_t*>(p.out);
    auto output_part = [&](int64_t c) __attribute__((always_inline)) {
        const int64_t t = c * C + tq;
#pragma unroll
        for (int t2 = 0; t2 < NCONS; ++t2) {
            const float4 o = *reinterpret_cast<const float4*>(obuf + ((c & 1) * NCONS + t2) * (64 * OST) + tq * OST + cq);
            const sig_t* srow = sbuf + ((c & 1) * NCONS + t2) * (64 * OST) + tq * OST + cq;
            const float y0 = o.x * static_cast<float>(srow[0]), y1 = o.y * static_cast<float>(srow[1]);
            const float y2 = o.z * static_cast<float>(srow[2]), y3 = o.w * static_cast<float>(srow[3]);
            if (t < T) {
                typename Out::raw_t* dst = gy + zrow(t) + 16 * (grp * NCONS + t2) + cq;
                if constexpr (sizeof(typename Out::raw_t) == 4) {
                    *reinterpret_cast<float4*>(dst) = make_float4(y0, y1, y2, y3);
                } else {
                    *reinterpret_cast<uint2*>(dst) =
                        make_uint2((uint32_t)Out::from_float(y0) | ((uint32_t)Out::from_float(y1) << 16),
                                   (uint32_t)Out::from_float(y2) | ((uint32_t)Out::from_float(y3) << 16));
                }
            }
        }
    };

    // chain state: S[ct][i] = S[16ct + 4g4 + i][col]
    const int nt = grp * NCONS + cs;
    const int col = 16 * nt + m16;
    floatx4 S[NCT];
    if (chain) {
        const float* s0 = p.s0 ? p.s0 + unit * (int64_t)D * D : nullptr;
#pragma unroll
        for (int ct = 0; ct < NCT; ++ct)
#pragma unroll
            for (int i = 0; i < 4; ++i) S[ct][i] = s0 ? s0[(16 * ct + 4 * g4 + i) * D + col] : 0.f;
    }


    // each role runs its own loop (so that no role carries another's registers); all of them
    // pass the same barriers: A and B once per chunk
    if (chain) {
        lds_barrier();  // the first card is resident
        for (int64_t ci = 0; ci < NC; ++ci) {
            const unsigned char* st = smem + (ci % L::NSTAGE) * L::STAGE;
            const _Float16* sw = reinterpret_cast<const _Float16*>(st + CD::W);
            const _Float16* sk = reinterpret_cast<const _Float16*>(st + CD::KBT);
            const _Float16* su = reinterpret_cast<const _Float16*>(st + L::OFF_U + cs * L::PER);
            const float* sg = reinterpret_cast<const float*>(st + L::OFF_G);
            // the state at the chunk start, as the B operand (logical k = 8g4 + j of step kb is
            // channel cmap(kb, g4, j)), for this wave and for the output wave
            half8 Sb[KB];
#pragma unroll
            for (int kb = 0; kb < KB; ++kb) {
                Sb[kb] = pack_h8(S[2 * kb], S[2 * kb + 1]);
                *reinterpret_cast<half8*>(sbx + (kb * 64 + lane) * 8) = Sb[kb];
            }
            half8 wf[4][KB];
            half4 ut[4];
            float4 gm[NCT];
#pragma unroll
            for (int mt = 0; mt < 4; ++mt) {
#pragma unroll
                for (int kb = 0; kb < KB; ++kb) wf[mt][kb] = ld_h8(sw + ((mt * KB + kb) * 64 + lane) * 8);
                ut[mt] = ld_h4(su + (mt * 64 + lane) * 4);
            }
#pragma unroll
            for (int ct = 0; ct < NCT; ++ct) gm[ct] = *reinterpret_cast<const float4*>(sg + 16 * ct + 4 * g4);
            lds_barrier();  // A: the state copy is visible to the output wave
            half8 kf[NCT][2];  // read while the U chain runs
#pragma unroll
            for (int ct = 0; ct < NCT; ++ct) {
                kf[ct][0] = ld_h8(sk + ((ct * 2 + 0) * 64 + lane) * 8);
                kf[ct][1] = ld_h8(sk + ((ct * 2 + 1) * 64 + lane) * 8);
            }
            floatx4 U[4];
#pragma unroll
            for (int mt = 0; mt < 4; ++mt) U[mt] = unpack_h4(ut[mt]);  // U~
#pragma unroll
            for (int ct = 0; ct < NCT; ++ct) {  // Diag(Gamma) S, off the U chain
                S[ct][0] *= gm[ct].x;
                S[ct][1] *= gm[ct].y;
                S[ct][2] *= gm[ct].z;
                S[ct][3] *= gm[ct].w;
            }
#pragma unroll
            for (int kb = 0; kb < KB; ++kb)
#pragma unroll
                for (int mt = 0; mt < 4; ++mt) U[mt] = mma_f16_k32(wf[mt][kb], Sb[kb], U[mt]);  // U~ - W S
            half8 Ub[2];
#pragma unroll
            for (int u = 0; u < 2; ++u) Ub[u] = pack_h8(U[2 * u], U[2 * u + 1]);
#pragma unroll
            for (int u = 0; u < 2; ++u)
#pragma unroll
                for (int ct = 0; ct < NCT; ++ct) S[ct] = mma_f16_k32(kf[ct][u], Ub[u], S[ct]);  // + Kbar^T U
            lds_barrier();  // B
        }
    } else if (outw) {
        lds_barrier();  // the first card is resident
        for (int64_t ci = 0; ci < NC; ++ci) {
            const unsigned char* st = smem + (ci % L::NSTAGE) * L::STAGE;
            const _Float16* sq = reinterpret_cast<const _Float16*>(st + CD::QE);
            const _Float16* su = reinterpret_cast<const _Float16*>(st + L::OFF_U + cs * L::PER);
            half8 qf[4][KB];
            half4 uo[4];
#pragma unroll
            for (int mt = 0; mt < 4; ++mt) {
#pragma unroll
                for (int kb = 0; kb < KB; ++kb) qf[mt][kb] = ld_h8(sq + ((mt * KB + kb) * 64 + lane) * 8);
                uo[mt] = ld_h4(su + L::UO_IN / 2 + (mt * 64 + lane) * 4);
            }
            lds_barrier();  // A
            half8 Sb[KB];
#pragma unroll
            for (int kb = 0; kb < KB; ++kb) Sb[kb] = ld_h8(sbx + (kb * 64 + lane) * 8);
            floatx4 O[4];
#pragma unroll
            for (int mt = 0; mt < 4; ++mt) O[mt] = unpack_h4(uo[mt]);  // Uo
#pragma unroll
            for (int kb = 0; kb < KB; ++kb)
#pragma unroll
                for (int mt = 0; mt < 4; ++mt) O[mt] = mma_f16_k32(qf[mt][kb], Sb[kb], O[mt]);  // + Qe S
            float* orow = obuf + ((ci & 1) * NCONS + cs) * (64 * OST);
#pragma unroll
            for (int mt = 0; mt < 4; ++mt)
#pragma unroll
                for (int i = 0; i < 4; ++i) orow[(16 * mt + 4 * g4 + i) * OST + m16] = O[mt][i];
            lds_barrier();  // B
        }
    } else {
        // two register sets: while one is in flight (chunk n+2), the other (chunk n+1,
        // loaded one iteration earlier) is written to LDS
        u32x4 ra[KP], rb[KP];
        auto load_set = [&](u32x4 (&r)[KP], int64_t c) __attribute__((always_inline)) {
#pragma unroll
            for (int k = 0; k < KP; ++k) r[k] = *piece_src(c, piece_of(k));
        };
        auto store_set = [&](const u32x4 (&r)[KP], int64_t c) __attribute__((always_inline)) {
#pragma unroll
            for (int k = 0; k < KP; ++k) *piece_dst(c, piece_of(k)) = r[k];
        };
        // Branch-free: past the end the producers reload the last chunk and rewrite the slot
        // that nobody reads any more, so both register sets follow the same code path.
        auto step = [&](u32x4 (&ld)[KP], const u32x4 (&wr)[KP], int64_t ci) __attribute__((always_inline)) {
            load_set(ld, ci + 2 < NC ? ci + 2 : NC - 1);  // the set that held chunk ci
            sigmoid_part(ci);
            if (ci >= 1) output_part(ci - 1);
            lds_barrier();  // A
            wait_vm<KP>();          // chunk ci + 1, loaded one iteration ago into the other set
            store_set(wr, ci + 1);  // the slot of chunk ci - 1, released by barrier B
            lds_barrier();  // B
        };
        if (NC > 0) {
            load_set(ra, 0);
            load_set(rb, NC > 1 ? 1 : 0);
            wait_vm<KP>();
            store_set(ra, 0);
        }
        lds_barrier();  // the first card is resident
        for (int64_t ci = 0; ci < NC; ci += 2) {
            step(ra, rb, ci);
            if (ci + 1 < NC) step(rb, ra, ci + 1);
        }
    }
    if (prod && NC > 0) output_part(NC - 1);

    if (chain && p.sT) {
        float* sT = p.sT + unit * (int64_t)D * D;
#pragma unroll
        for (int ct = 0; ct < NCT; ++ct)
#pragma unroll
            for (int i = 0; i < 4; ++i) sT[(16 * ct + 4 * g4 + i) * D + col] = S[ct][i];
    }
}

// ---------------------------------------------------------------------------
template <int D, class Out, int NCONS>
static hipError_t launch_d(const PrepParams& pp, const RecurParams& rp, hipStream_t stream) {
    using LP = PrepL<D>;
    using LR = RecL<D, NCONS>;
    const int64_t units = rp.B * rp.H;
    if (pp.NC > 0) {
        auto kp = kda_prep64_kernel<D>;
        hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kp),
                                           hipFuncAttributeMaxDynamicSharedMemorySize, (int)LP::TOTAL);
        if (e != hipSuccess) return e;
        int dev = 0, cus = 256;
        if (hipGetDevice(&dev) != hipSuccess ||
            hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0)
            cus = 256;
        const int64_t items = units * pp.NC;
        const int64_t grid = items < cus ? items : cus;  // one persistent workgroup per CU (LDS-bound)
        hipLaunchKernelGGL(kp, dim3((unsigned)grid), dim3(256), LP::TOTAL, stream, pp);
        e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    auto kr = kda_rec64_kernel<D, Out, NCONS>;
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kr),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)LR::TOTAL);
    if (e != hipSuccess) return e;
    constexpr int G = D / (16 * NCONS);
    const int64_t blocks = (units * G + 7) / 8 * 8;
    hipLaunchKernelGGL(kr, dim3((unsigned)blocks), dim3(LR::WAVES * 64), LR::TOTAL, stream, rp);
    return hipGetLastError();
}

}  // namespace c64

int64_t prefill64_card_bytes(int D) {
    return D == 128 ? c64::Card<128>::BYTES : D == 64 ? c64::Card<64>::BYTES : -1;
}

int64_t prefill64_blocks(int D, int64_t units, int64_t nc) {
    (void)D;
    return units * nc;
}

hipError_t launch_prefill64(int D, int out_bf16, const PrepParams& pp, const RecurParams& rp,
                            hipStream_t stream) {
    // one consumer per workgroup has the shortest chain per chunk; with enough (b, h)
    // sequences to fill the GPU, two consumers share each streamed card instead
    const bool wide = rp.B * rp.H >= 64;
    if (D == 128) {
        if (wide)
            return out_bf16 ? c64::launch_d<128, InBF16, 2>(pp, rp, stream)
                            : c64::launch_d<128, InF32, 2>(pp, rp, stream);
        return out_bf16 ? c64::launch_d<128, InBF16, 1>(pp, rp, stream)
                        : c64::launch_d<128, InF32, 1>(pp, rp, stream);
    }
    if (D == 64)
        return out_bf16 ? c64::launch_d<64, InBF16, 1>(pp, rp, stream)
                        : c64::launch_d<64, InF32, 1>(pp, rp, stream);
    return hipErrorInvalidValue;
}

}  // namespace kda
