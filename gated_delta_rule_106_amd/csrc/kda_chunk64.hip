// Chunkwise KDA forward for bf16 inputs with 64-token chunks (gfx950).
//
// Same algebra as the general kernels (the per-token recurrence of page "3T
// models are no longer magic", section "Gate 1: KDA makes it computable",
// evaluated chunk by chunk as on page "Kimi K3 report walk-through", sections
// "Compute paradigm" and "Hierarchical chunking of linear attention"), laid out
// for throughput on CDNA4:
//
// kda_prep64_kernel  one workgroup of 4 waves per (b, h, chunk) card, two
//   workgroups per CU.  Wave a owns the 16-token tile a of the chunk, keeps it
//   in registers in MFMA operand layout (lane = token, 4 consecutive key
//   channels per 16-channel tile) and is compiled for its tile index.  The
//   cumulative log-decay is a DPP prefix scan across the 16 lanes of a row.
//   Decay is folded into q and k as an absolute-position rescaling measured
//   from the start of each 16-token tile (page "Kimi K3 report walk-through",
//   section "Numerical stability & co-design": inside one tile the inverse
//   factor stays below 2^116 given the 0.67 % retention floor):
//       KR = k 2^{P},  QR = q 2^{P},  KC = k 2^{-P},  KE = k 2^{tau - P},
//   P = prefix sum of log2(alpha) inside the tile, tau = its total.  Pair
//   products inside a tile use KR.KC^T on the fp32 MFMA (the operands span
//   2^{+-116}); across tiles both operands are <= |k| and one fp16 pass
//   suffices.  The unit-lower-triangular system (I + A) is solved with
//   register forward substitution on the four 16x16 diagonal blocks and fp32
//   MFMA block products for the rest.  Tiles are turned to lane = channel by
//   an MFMA against a 0/1 selection operand.  With M = P T, every card block of
//   the tile is one product of its T or M rows with the K~ or V fragments:
//       U~ = T V,  Uo = M V,  W^T = K~^T T^T,  Qe^T = Q~^T - K~^T M^T,
//   whose accumulators are the card's fragments (coalesced stores).
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
//   KBT [ct][u][h] 64 lanes x 4: Kbar[32u + 16h + 4g + i][16ct + m]; the two
//                halves h = 0, 1 concatenated are the 8 K-elements c(u, g, j)
//   UT  [nt][mt] 64 lanes x 4:  U~[16mt + 4g + i][16nt + m]
//   UO  [nt][mt] 64 lanes x 4:  Uo[16mt + 4g + i][16nt + m]       Uo = P U~
//   GAM [D] fp32: 2^{gamma_C}, the decay of the whole chunk per key channel
// with c(x, g, j) = 32x + 4g + j (j < 4), 32x + 16 + 4g + (j - 4) (j >= 4):
// the K-index order in which two stacked accumulator tiles (rows 4g .. 4g+3
// in lane group g) feed the next MFMA directly as its B operand.
#include <type_traits>

#include "kda_device.h"
#include "kda_prefill.h"
#include "kda_varlen.h"

namespace kda {
namespace c64 {

constexpr int C = 64;
constexpr int NSUB = 4;

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

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

// value held by lane 7 of this lane's 16-lane row (swizzle bitmask mode: lane & 16 | 7)
__device__ __forceinline__ float row_mid(float x) {
    return __int_as_float(__builtin_amdgcn_ds_swizzle(__float_as_int(x), 0x0F0));
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
    static constexpr int KB = D / 32, NCT = D / 16;
    static constexpr int SAB = 17;                         // fp32 16x16 block row stride (floats)
    static constexpr int BLK = 16 * SAB;                   // floats per block
    static constexpr int NBLK = NSUB * (NSUB + 1) / 2;     // blocks on and below the diagonal
    static constexpr int SP = C + 8;                       // fp16 [64][64] row stride (halves)
    static constexpr int64_t FR = 1024;                    // 64 lanes x 16 B
    static constexpr int64_t B_BLK = (int64_t)NBLK * BLK * 4;
    static constexpr int64_t B_KEF = (int64_t)NSUB * KB * FR;
    static constexpr int64_t B_R1 = B_KEF > B_BLK ? B_KEF : B_BLK;
    static constexpr int64_t B_MAT = 64 * SP * 2;
    static constexpr int64_t B_R2 = B_BLK > B_MAT ? B_BLK : B_MAT;
    static constexpr int64_t OFF_BETA = 0;                      // fp32 [64]
    static constexpr int64_t OFF_ETAU = 256;                    // fp32 [NSUB][D]: decay over each tile
    static constexpr int64_t OFF_KE = OFF_ETAU + NSUB * D * 4;  // KE fragments [tile][kb]; later Linv blocks
    static constexpr int64_t OFF_KF = OFF_KE + B_R1;            // K~ fragments [ct][u][half][lane] 8 B
    static constexpr int64_t OFF_VF = OFF_KF + NCT * 2 * FR;    // V fragments, same layout
    static constexpr int64_t OFF_A = OFF_VF + NCT * 2 * FR;     // fp32 A blocks; later fp16 M [64][SP]
    static constexpr int64_t OFF_P = OFF_A + B_R2;              // fp16 P [64][SP]
    static constexpr int64_t OFF_T = OFF_P + B_MAT;             // fp16 T [64][SP]
    static constexpr int64_t TOTAL = OFF_T + B_MAT;
    // two workgroups per CU
    static_assert(2 * TOTAL <= 160 * 1024, "prep LDS budget");
    static_assert(OFF_KE % 16 == 0 && OFF_KF % 16 == 0 && OFF_VF % 16 == 0 && OFF_A % 16 == 0 &&
                      OFF_P % 16 == 0 && OFF_T % 16 == 0,
                  "prep LDS alignment");
};

// index of the 16x16 block (r, c), c <= r, among the blocks on and below the diagonal
__device__ __forceinline__ constexpr int bidx(int r, int c) { return r * (r + 1) / 2 + c; }

// Operand of a K = 32 step over the channels 32 kb .. 32 kb + 31 (lane group g
// supplies 8 g .. 8 g + 7) that picks the 16 channels 32 kb + 16 cl + n: as the B
// operand, D = A Sel holds a tile in A-operand layout (lane = token) transposed, with
// lane = channel and the four registers = tokens 4g .. 4g + 3; as the A operand,
// D = Sel B turns a B-operand tile (lane = token) into the accumulator layout (lane =
// token, registers = channels 16 (2 kb + cl) + 4g .. +3).  Products with 1.0 and sums
// with zeros keep fp16 values exact.
__device__ __forceinline__ half8 sel_operand(int cl, int lane) {
    const int g = lane >> 4, n = lane & 15;
    half8 r;
#pragma unroll
    for (int j = 0; j < 8; ++j) r[j] = static_cast<_Float16>((g == 2 * cl + (n >> 3) && j == (n & 7)) ? 1.f : 0.f);
    return r;
}

// 64 lanes x 8 B fragment piece [ct][u][half]: lane (g, n) holds rows
// 32u + 16 half + 4g .. +3 of column 16 ct + n
__device__ __forceinline__ constexpr int64_t frag_piece(int ct, int u, int hf) { return ((ct * 2 + u) * 2 + hf) * 512; }

// 16 bytes of an input row; non-temporal with STREAM (below).
template <bool STREAM>
__device__ __forceinline__ u32x4 in_ld(const uint16_t* p) {
    if constexpr (STREAM)
        return __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
    else
        return *reinterpret_cast<const u32x4*>(p);
}

// A card store.  STREAM (the pipelined pass, whose cards are read a whole piece later,
// from other XCDs): the store is non-temporal, so the cards stream past the L2 rather than
// evicting the lines the state pass running beside the card builder reuses.  Otherwise the
// state pass reads the cards right after this launch and the ordinary policy keeps them
// close.
template <bool STREAM, class T>
__device__ __forceinline__ void card_st(unsigned char* p, const T& v) {
    if constexpr (STREAM)
        __builtin_nontemporal_store(v, reinterpret_cast<T*>(p));
    else
        *reinterpret_cast<T*>(p) = v;
}

// ---------------------------------------------------------------------------
// kernel 1: one update card per workgroup.  Wave A owns the 16-token tile A of the
// chunk; everything that depends on A is resolved at compile time.
// MODE bit 0: raw q, k (per-token L2 normalisation); bit 1: log_alpha holds forget
// logits.  Compile-time, so the decay loop of the plain mode carries no extra work.
// MODE bit 2 (taken with the clamp off, where a token's log alpha may lie below the
// floor): the in-tile pairs take their reference point at token 7 of the tile instead of
// the tile start, so each of their factors spans at most eight tokens of decay and stays
// finite down to about -11 nats per token (the clamp's floor keeps a whole tile within
// 80.1 nats, so the default mode needs no such care).
constexpr int kModeQkNorm = 1, kModeLogits = 2, kModeWide = 4, kModeStream = 8;

// Where a card's tokens are: chunk n of a sequence of slen tokens starting at packed
// row tb, head h; item is the card's index in the workspace.  Formed once per
// workgroup, outside the four per-tile bodies (the kernel's code is about the size of
// the instruction cache, so nothing is repeated in them that need not be).
struct CardPos {
    int64_t item, n, h, tb, slen;
};

template <int D, int A, int MODE>
__device__ __forceinline__ void prep_tile(const PrepParams& p, unsigned char* smem, const CardPos& cp) {
    using L = PrepL<D>;
    using CD = Card<D>;
    constexpr int NCT = D / 16, KB = D / 32, SAB = L::SAB, BLK = L::BLK, SP = L::SP;
    float* s_beta = reinterpret_cast<float*>(smem + L::OFF_BETA);
    float* s_etau = reinterpret_cast<float*>(smem + L::OFF_ETAU);
    _Float16* s_ke = reinterpret_cast<_Float16*>(smem + L::OFF_KE);
    float* s_linv = reinterpret_cast<float*>(smem + L::OFF_KE);
    unsigned char* s_kf = smem + L::OFF_KF;
    unsigned char* s_vf = smem + L::OFF_VF;
    float* s_ab = reinterpret_cast<float*>(smem + L::OFF_A);
    _Float16* s_m = reinterpret_cast<_Float16*>(smem + L::OFF_A);
    _Float16* s_p = reinterpret_cast<_Float16*>(smem + L::OFF_P);
    _Float16* s_t = reinterpret_cast<_Float16*>(smem + L::OFF_T);

    const int lane = threadIdx.x & 63;
    const int m16 = lane & 15, g4 = lane >> 4;
    const int rl = 16 * A + m16;  // this lane's token within the chunk
    const int64_t H = p.H;
    constexpr bool logits = (MODE & kModeLogits) != 0, qk_norm = (MODE & kModeQkNorm) != 0;
    constexpr bool wide = (MODE & kModeWide) != 0;
    constexpr bool clamp = !wide;  // the wide mode is taken exactly when the clamp is off
    constexpr bool stream = (MODE & kModeStream) != 0;

    // raw inputs of token rl: per 32-channel block kb, the 8 bf16 channels 32 kb + 8 g4 .. +7
    // (16 bytes; the four lane groups of a token cover 64 contiguous bytes of its row).
    // STREAM: non-temporal loads, which leave the L2's lines to the state pass beside.
    u32x4 rq[KB], rk[KB], rv[KB], rla[KB];
    uint32_t rbeta;
    const int64_t item = cp.item, n = cp.n, h = cp.h, tb = cp.tb, slen = cp.slen;
    auto fetch = [&]() __attribute__((always_inline)) {
        const int64_t tok = n * C + rl;
        const int64_t row = (tb + (tok < slen ? tok : slen - 1)) * H + h;  // in bounds; zeroed at use
        const uint16_t* gq = static_cast<const uint16_t*>(p.q);
        const uint16_t* gk = static_cast<const uint16_t*>(p.k);
        const uint16_t* gv = static_cast<const uint16_t*>(p.v);
        const uint16_t* gla = static_cast<const uint16_t*>(p.la);
        rbeta = static_cast<const uint16_t*>(p.beta)[row];
        // in the order the decay phase consumes them, so that it starts on the first channel
        // block while the later ones are still arriving
#pragma unroll
        for (int kb = 0; kb < KB; ++kb) {
            const int64_t off = row * D + 32 * kb + 8 * g4;
            rla[kb] = in_ld<stream>(gla + off);
            rk[kb] = in_ld<stream>(gk + off);
            rq[kb] = in_ld<stream>(gq + off);
            rv[kb] = in_ld<stream>(gv + off);
        }
    };
    auto elem = [](const u32x4 w, int j) -> float {  // bf16 element j of 8
        const uint32_t x = w[j >> 1];
        return (j & 1) ? __uint_as_float(x & 0xffff0000u) : __uint_as_float(x << 16);
    };
    const half8 sel0 = sel_operand(0, lane), sel1 = sel_operand(1, lane);
    // a 16 x 32 tile in operand layout -> two transposed 16 x 16 pieces of a fragment
    auto put_transposed = [&](unsigned char* base, int kb, const half8& x) __attribute__((always_inline)) {
        const floatx4 t0 = mma_f16_k32(x, sel0, zero4());
        const floatx4 t1 = mma_f16_k32(x, sel1, zero4());
        *reinterpret_cast<half4*>(base + frag_piece(2 * kb, A >> 1, A & 1) + lane * 8) = pack_h4(t0);
        *reinterpret_cast<half4*>(base + frag_piece(2 * kb + 1, A >> 1, A & 1) + lane * 8) = pack_h4(t1);
    };

    fetch();
    const bool valid = n * C + rl < slen;  // tokens past the end are identity tokens
    if (!valid) {  // all of their inputs count as zero (log alpha 0: no decay)
        // a forget-gate logit of +inf (bf16 0x7f80) has log-sigmoid 0
        constexpr uint32_t la0 = logits ? 0x7f807f80u : 0u;
#pragma unroll
        for (int kb = 0; kb < KB; ++kb) {
            rk[kb] = rq[kb] = rv[kb] = u32x4{0u, 0u, 0u, 0u};
            rla[kb] = u32x4{la0, la0, la0, la0};
        }
    }
    // per-token L2 normalisation of raw q and k: the four lane groups of a token hold
    // its channels; factors stay 1 for inputs that arrive normalised
    float ks = 1.f, qs = 1.f;
    if constexpr (qk_norm) {
        float sk = 0.f, sq = 0.f;
#pragma unroll
        for (int kb = 0; kb < KB; ++kb)
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                const float kf = elem(rk[kb], j), qf = elem(rq[kb], j);
                sk += kf * kf;
                sq += qf * qf;
            }
        sk += __shfl_xor(sk, 16);
        sq += __shfl_xor(sq, 16);
        sk += __shfl_xor(sk, 32);
        sq += __shfl_xor(sq, 32);
        ks = inv_norm(sk);
        qs = inv_norm(sq) * (1.0f / __builtin_sqrtf((float)D));
    }
    unsigned char* card = static_cast<unsigned char*>(p.ws) + item * CD::BYTES;
    const float beta_mine = valid ? bf16_bits_to_float(static_cast<uint16_t>(rbeta)) : 0.f;

    // ---- phase 1: decay inside the tile, in-tile pair products, V fragments
    s_beta[rl] = beta_mine;  // the four lane groups store the same value
    half8 kr16[KB], qr16[KB], ke16[KB];
    floatx4 accA = zero4(), accP = zero4();
#pragma unroll
    for (int kb = 0; kb < KB; ++kb) {
        half8 v16;
        float et8[8];  // decay over the whole tile of this lane's eight channels
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            const float x = elem(rla[kb], j);
            float la = x;
            if constexpr (logits) la = log_sigmoid(x);
            // log2 units; clamping after the scaling gives the same bits (the scaling is
            // monotone) and leaves no product for the scan's first add to fuse with
            const float l = clamp ? __builtin_amdgcn_fmed3f(la * kLog2e, kLogAlphaMin * kLog2e, 0.f) : la * kLog2e;
            const float P = row_scan16(l);      // log2 decay from the tile start, inclusive
            const float E = fast_exp2(P);       // <= 1
            const float Et = row_last(E);       // decay over the whole tile
            float kf = elem(rk[kb], j), qf = elem(rq[kb], j);
            if constexpr (qk_norm) {
                kf *= ks;
                qf *= qs;
            }
            const float KR = kf * E, QR = qf * E;
            // K-step (kb, j): lane group g4 supplies channel 32 kb + 8 g4 + j to both operands
            if constexpr (wide) {
                const float Pm = P - row_mid(P);  // from token 7 of the tile
                const float Em = fast_exp2(Pm), Emi = fast_exp2(-Pm);
                accA = mma_f32_k4(kf * Em, kf * Emi, accA);
                accP = mma_f32_k4(qf * Em, kf * Emi, accP);
                ke16[kb][j] = static_cast<_Float16>(kf * fast_exp2(row_last(P) - P));
            } else {
                const float Einv = fast_exp2(-P);  // >= 1, < 2^116 under the floor
                const float KC = kf * Einv;
                accA = mma_f32_k4(KR, KC, accA);
                accP = mma_f32_k4(QR, KC, accP);
                ke16[kb][j] = static_cast<_Float16>(KC * Et);  // decay from after this token to the tile end
            }
            kr16[kb][j] = static_cast<_Float16>(KR);
            qr16[kb][j] = static_cast<_Float16>(QR);
            v16[j] = static_cast<_Float16>(elem(rv[kb], j));
            et8[j] = Et;
        }
        if (m16 == 0) {  // the 16 lanes of a row hold the same values
            float* et = s_etau + A * D + 32 * kb + 8 * g4;
            *reinterpret_cast<float4*>(et) = make_float4(et8[0], et8[1], et8[2], et8[3]);
            *reinterpret_cast<float4*>(et + 4) = make_float4(et8[4], et8[5], et8[6], et8[7]);
        }
        // KE fragment of this tile: the B operand of the pairs (later tile, this tile)
        *reinterpret_cast<half8*>(s_ke + ((A * KB + kb) * 64 + lane) * 8) = ke16[kb];
        put_transposed(s_vf, kb, v16);
        __builtin_amdgcn_sched_barrier(0);  // one K-block at a time: bounded register lifetimes
    }
    // diagonal blocks of A (strictly lower, rows scaled by beta) and P (lower)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int r = 4 * g4 + i, s = m16;
        const float br = __shfl(beta_mine, r);
        s_ab[bidx(A, A) * BLK + r * SAB + s] = (s < r) ? br * accA[i] : 0.f;
        s_p[(16 * A + r) * SP + 16 * A + s] = static_cast<_Float16>((s <= r) ? accP[i] : 0.f);
    }
    lds_barrier();  // (1) tile decays, KE and V fragments, beta

    // ---- phase 2: chunk-relative operands and the pairs with earlier tiles.  Decay
    //      factors across tiles are products of the per-tile decays 2^{tau}.
    half8 q16[KB];  // Q~ of this tile (B-operand layout): the initial value of its Qe rows
    floatx4 pa[NSUB - 1], pp[NSUB - 1];
#pragma unroll
    for (int bb = 0; bb < NSUB - 1; ++bb) pa[bb] = pp[bb] = zero4();
#pragma unroll
    for (int kb = 0; kb < KB; ++kb) {
        float et[NSUB][8];
#pragma unroll
        for (int a2 = 0; a2 < NSUB; ++a2) {
            if (a2 == A) continue;
            const float4 lo = *reinterpret_cast<const float4*>(s_etau + a2 * D + 32 * kb + 8 * g4);
            const float4 hi = *reinterpret_cast<const float4*>(s_etau + a2 * D + 32 * kb + 8 * g4 + 4);
            et[a2][0] = lo.x; et[a2][1] = lo.y; et[a2][2] = lo.z; et[a2][3] = lo.w;
            et[a2][4] = hi.x; et[a2][5] = hi.y; et[a2][6] = hi.z; et[a2][7] = hi.w;
        }
        // decay before this tile and after it, formed in fp32 and applied to the fp16 operands
        // as packed fp16 products
        half8 erho, eaft;
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            float e0 = 1.f, e1 = 1.f;
#pragma unroll
            for (int a2 = 0; a2 < A; ++a2) e0 *= et[a2][j];
#pragma unroll
            for (int a2 = A + 1; a2 < NSUB; ++a2) e1 *= et[a2][j];
            erho[j] = static_cast<_Float16>(e0);
            eaft[j] = static_cast<_Float16>(e1);
        }
        const half8 kt = A == 0 ? kr16[kb] : kr16[kb] * erho;                // K~ = k 2^{g}
        q16[kb] = A == 0 ? qr16[kb] : qr16[kb] * erho;                      // Q~ = q 2^{g}
        const half8 kbar = A == NSUB - 1 ? ke16[kb] : ke16[kb] * eaft;      // Kbar = k 2^{g_C - g}
        put_transposed(s_kf, kb, kt);
        {
            const floatx4 t0 = mma_f16_k32(kbar, sel0, zero4());
            const floatx4 t1 = mma_f16_k32(kbar, sel1, zero4());
            card_st<stream>(card + CD::KBT + frag_piece(2 * kb, A >> 1, A & 1) + lane * 8, pack_h4(t0));
            card_st<stream>(card + CD::KBT + frag_piece(2 * kb + 1, A >> 1, A & 1) + lane * 8, pack_h4(t1));
        }
        // pairs (A, bb), bb < A: reference point at the end of tile A-1; both operands <= |k|
        float f[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) f[j] = 1.f;
#pragma unroll
        for (int bb = A - 1; bb >= 0; --bb) {  // f = decay over the tiles strictly between bb and A
            const half8 keb = ld_h8(s_ke + ((bb * KB + kb) * 64 + lane) * 8);
            half8 col = keb;
            if (bb != A - 1) {
                half8 fh;
#pragma unroll
                for (int j = 0; j < 8; ++j) fh[j] = static_cast<_Float16>(f[j]);
                col = keb * fh;
            }
            pa[bb] = mma_f16_k32(kr16[kb], col, pa[bb]);
            pp[bb] = mma_f16_k32(qr16[kb], col, pp[bb]);
            if (bb > 0) {
#pragma unroll
                for (int j = 0; j < 8; ++j) f[j] *= et[bb][j];
            }
        }
    }
#pragma unroll
    for (int bb = 0; bb < A; ++bb) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int r = 4 * g4 + i;
            const float br = __shfl(beta_mine, r);
            s_ab[bidx(A, bb) * BLK + r * SAB + m16] = br * pa[bb][i];
            s_p[(16 * A + r) * SP + 16 * bb + m16] = static_cast<_Float16>(pp[bb][i]);
        }
    }
    // Gamma = 2^{g_C} per key channel
    if (64 * A < D) {
        const int c = 64 * A + lane;
        float gm = 1.f;
#pragma unroll
        for (int a2 = 0; a2 < NSUB; ++a2) gm *= s_etau[a2 * D + c];
        card_st<stream>(card + CD::GAM + 4 * c, gm);
    }
    lds_barrier();  // (2) A, P, K~ fragments complete; KE fragments no longer needed

    // ---- phase 3: Linv = (I + A)^{-1} (unit lower triangular, blocked by 16) and
    //      T = Linv diag(beta) in fp16
    if constexpr (A == 0) {  // diagonal blocks: lane group g4 = block, lane m16 = column
        const int ab = g4, j = m16;
        const float* Ab = s_ab + bidx(ab, ab) * BLK;
        float x[16];
#pragma unroll
        for (int r = 0; r < 16; ++r) x[r] = (r == j) ? 1.f : 0.f;
#pragma unroll
        for (int r = 1; r < 16; ++r) {
            float acc = x[r];
#pragma unroll
            for (int q = 0; q < r; ++q) acc -= Ab[r * SAB + q] * x[q];
            x[r] = acc;
        }
        const float bj = s_beta[16 * ab + j];
        float* Xb = s_linv + bidx(ab, ab) * BLK;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            Xb[r * SAB + j] = x[r];
            s_t[(16 * ab + r) * SP + 16 * ab + j] = static_cast<_Float16>(x[r] * bj);
        }
    }
    lds_barrier();  // (3)
    // off-diagonal blocks by block diagonal d: Linv_{A,A-d} = -X_A sum_c A_{A,c} Linv_{c,A-d}
    auto mm = [&](const float* mp, const float* np, floatx4 acc) {  // acc += M N (16x16 blocks)
        float4 av;
        av.x = mp[m16 * SAB + 4 * g4 + 0];
        av.y = mp[m16 * SAB + 4 * g4 + 1];
        av.z = mp[m16 * SAB + 4 * g4 + 2];
        av.w = mp[m16 * SAB + 4 * g4 + 3];
        floatx4 bv;
#pragma unroll
        for (int s = 0; s < 4; ++s) bv[s] = np[(4 * g4 + s) * SAB + m16];
        return mma_f32_k16(av, bv, acc);
    };
#pragma unroll
    for (int d = 1; d < NSUB; ++d) {
        if (A >= d) {
            floatx4 y = zero4();
#pragma unroll
            for (int c = A - d; c < A; ++c) y = mm(s_ab + bidx(A, c) * BLK, s_linv + bidx(c, A - d) * BLK, y);
            const float* Xa = s_linv + bidx(A, A) * BLK;
            float4 xv;
            xv.x = Xa[m16 * SAB + 4 * g4 + 0];
            xv.y = Xa[m16 * SAB + 4 * g4 + 1];
            xv.z = Xa[m16 * SAB + 4 * g4 + 2];
            xv.w = Xa[m16 * SAB + 4 * g4 + 3];
            const floatx4 zz = mma_f32_k16(xv, y, zero4());
            float* dst = s_linv + bidx(A, A - d) * BLK;
            const float bcol = s_beta[16 * (A - d) + m16];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                dst[(4 * g4 + i) * SAB + m16] = -zz[i];
                s_t[(16 * A + 4 * g4 + i) * SP + 16 * (A - d) + m16] = static_cast<_Float16>(-zz[i] * bcol);
            }
        }
        lds_barrier();  // (4), (5), (6)
    }

    // ---- M = P T (rows of this tile; lower triangular), fp16, over the dead A blocks.
    //      K-steps of 32 tokens; a 16-token half outside [16c, 16A + 16) is zero.
    const half4 z4 = {0, 0, 0, 0};
#pragma unroll
    for (int c = 0; c <= A; ++c) {
        floatx4 acc = zero4();
#pragma unroll
        for (int u = c >> 1; u <= (A >> 1); ++u) {
            const bool lo_ok = c <= 2 * u, hi_ok = 2 * u + 1 <= A;
            const _Float16* prow = s_p + (16 * A + m16) * SP + 32 * u + 4 * g4;
            const half8 pa8 = cat_h8(lo_ok ? ld_h4(prow) : z4, hi_ok ? ld_h4(prow + 16) : z4);
            half8 tb;
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                const int s = 32 * u + 16 * (j >> 2) + 4 * g4 + (j & 3);
                const bool ok = (j < 4) ? lo_ok : hi_ok;
                tb[j] = ok ? s_t[s * SP + 16 * c + m16] : static_cast<_Float16>(0.f);
            }
            acc = mma_f16_k32(pa8, tb, acc);
        }
        // lane (g4, m16) holds M[16A + 4g4 + i][16c + m16]
#pragma unroll
        for (int i = 0; i < 4; ++i) s_m[(16 * A + 4 * g4 + i) * SP + 16 * c + m16] = static_cast<_Float16>(acc[i]);
    }
    lds_barrier();  // (7)

    // ---- phase 4: the card rows of this tile.  With the T and M rows of the tile as
    //      operands (A side for T V and M V, B side for the transposed products):
    //      U~ = T V, Uo = M V, W^T = K~^T T^T, Qe^T = Q~^T - K~^T M^T.
    half8 ta[2], ma[2];
#pragma unroll
    for (int u = 0; u <= (A >> 1); ++u) {
        const bool hi_ok = 2 * u + 1 <= A;
        const _Float16* trow = s_t + (16 * A + m16) * SP + 32 * u + 4 * g4;
        const _Float16* mrow = s_m + (16 * A + m16) * SP + 32 * u + 4 * g4;
        ta[u] = cat_h8(ld_h4(trow), hi_ok ? ld_h4(trow + 16) : z4);
        ma[u] = cat_h8(ld_h4(mrow), hi_ok ? ld_h4(mrow + 16) : z4);
    }
    floatx4 wt[2], qe[2];
#pragma unroll
    for (int x = 0; x < NCT; ++x) {
        floatx4 ut = zero4(), uo = zero4(), w = zero4(), qm = zero4();
#pragma unroll
        for (int u = 0; u <= (A >> 1); ++u) {
            const half8 vf = cat_h8(*reinterpret_cast<const half4*>(s_vf + frag_piece(x, u, 0) + lane * 8),
                                    *reinterpret_cast<const half4*>(s_vf + frag_piece(x, u, 1) + lane * 8));
            const half8 kf = cat_h8(*reinterpret_cast<const half4*>(s_kf + frag_piece(x, u, 0) + lane * 8),
                                    *reinterpret_cast<const half4*>(s_kf + frag_piece(x, u, 1) + lane * 8));
            ut = mma_f16_k32(ta[u], vf, ut);
            uo = mma_f16_k32(ma[u], vf, uo);
            w = mma_f16_k32(kf, ta[u], w);
            qm = mma_f16_k32(kf, ma[u], qm);
        }
        card_st<stream>(card + CD::UT + ((x * 4 + A) * 64 + lane) * 8, pack_h4(ut));
        card_st<stream>(card + CD::UO + ((x * 4 + A) * 64 + lane) * 8, pack_h4(uo));
        const int kb = x >> 1, cl = x & 1;
        const floatx4 q0 = mma_f16_k32(cl ? sel1 : sel0, q16[kb], zero4());  // Q~^T rows of this tile
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            wt[cl][i] = -w[i];
            qe[cl][i] = q0[i] - qm[i];
        }
        if (cl == 1) {
            card_st<stream>(card + CD::W + ((A * KB + kb) * 64 + lane) * 16, pack_h8(wt[0], wt[1]));
            card_st<stream>(card + CD::QE + ((A * KB + kb) * 64 + lane) * 16, pack_h8(qe[0], qe[1]));
        }
    }
}

// One card: workgroup item `item` of the card builder's grid, 16-token tile `tile` of it
// (one wave per tile).  Returns without a barrier when the item has no card.
template <int D, int MODE>
__device__ __forceinline__ void prep64_card(const PrepParams& p, unsigned char* smem, int64_t item, int tile) {
    // a variable-length grid is sized for the most chunks the offsets can give
    CardPos cp;
    cp.item = item;
    if (p.ring_len > 0) {  // one piece of the sequences, chunk-major, into its half of the ring
        const int64_t units = p.B * p.H;
        const int64_t j = cp.item / units;  // chunk within the piece
        const int64_t unit = cp.item - j * units;
        cp.n = p.piece * p.ring_len + j;
        cp.item = ((p.piece & 1) * units + unit) * p.ring_len + j;
        const int64_t b = unit / p.H;
        cp.h = unit - b * p.H;
        cp.tb = b * p.T;
        cp.slen = p.T;
    } else if (p.vco) {  // variable-length batch: card (co_i + n) H + h
        const int64_t g = cp.item / p.H;
        if (g >= p.vco[p.vN]) return;  // the whole group leaves
        const int64_t i = p.vsoc[g];
        cp.h = cp.item - g * p.H;
        cp.n = g - p.vco[i];
        cp.tb = p.vs[i];
        cp.slen = p.vs[i + 1] - cp.tb;  // >= 1: the sequence owns this chunk
    } else {  // B sequences of T tokens: card unit NC + n
        // workgroups build the last chunks of every sequence first, so that the cards the
        // state pass reads first are the most recently written (still in the Infinity Cache)
        const int64_t units = p.B * p.H;
        const int64_t back = cp.item / units;  // chunks from the end
        const int64_t unit = cp.item - back * units;
        cp.n = p.NC - 1 - back;
        cp.item = unit * p.NC + cp.n;
        const int64_t b = unit / p.H;
        cp.h = unit - b * p.H;
        cp.tb = b * p.T;
        cp.slen = p.T;
    }
    switch (__builtin_amdgcn_readfirstlane(tile)) {
        case 0: prep_tile<D, 0, MODE>(p, smem, cp); break;
        case 1: prep_tile<D, 1, MODE>(p, smem, cp); break;
        case 2: prep_tile<D, 2, MODE>(p, smem, cp); break;
        default: prep_tile<D, 3, MODE>(p, smem, cp); break;
    }
}

template <int D, int MODE>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2, 2)))
void kda_prep64_kernel(PrepParams p) {
    extern __shared__ __align__(16) unsigned char smem[];
    prep64_card<D, MODE>(p, smem, blockIdx.x, threadIdx.x >> 6);
}

// ---------------------------------------------------------------------------
// kernel 2: sequential pass over the cards
//
// Per workgroup, for each of its NCONS 16-column value tiles, a chain wave and an
// output wave, plus NP producer waves, pipelined around one barrier X(n) per chunk:
//   chain     iteration n: S_n (fp16 copy) -> LDS buffer n % 2, U = U~ - W S_n,
//             S_{n+1} = Diag(Gamma) S_n + Kbar^T U (fp32 state in accumulators)
//   output    iteration n + 1: O_n = Uo + Qe S_n from that copy -> LDS buffer n % 2
//             (Qe and Uo loaded into registers one chunk ahead)
//   producers iteration n: y_{n-2} = O_{n-2} sigmoid(z_{n-2}) (a quarter of the
//             tokens each, 16-byte stores), direct-to-LDS copies of chunk n+2 (W,
//             Kbar^T, the U~ slices, the gate logits, Gamma) into ring slot
//             (n+2) % 3, the gate logits of chunk n into registers; before X(n) they
//             wait for the copies of chunk n+1 (issued one iteration earlier).
// A chunk's copy is in flight for about two iterations; the LDS ring holds three.
template <int D, int NCONS>
struct RecL {
    using CD = Card<D>;
    static constexpr int KB = D / 32;
    static constexpr int NP = 4;                              // producer waves
    static constexpr int NW = 4 * KB;                         // 1 KiB pieces of W; as many of Kbar^T
    static constexpr int64_t OFF_WS = 0;                      // W fragments (card order)
    static constexpr int64_t OFF_KS = (int64_t)NW * 1024;     // Kbar^T fragments (card order)
    static constexpr int64_t OFF_US = 2 * OFF_KS;             // U~ slices, 2 KiB per tile
    static constexpr int64_t OFF_ZS = OFF_US + NCONS * 2048;  // gate logits [64][16] bf16, 2 KiB per tile
    static constexpr int64_t OFF_GS = OFF_ZS + NCONS * 2048;  // Gamma (D * 4 bytes) in a 1 KiB piece
    static constexpr int64_t STAGE = OFF_GS + 1024;
    static constexpr int NSTAGE = 3;
    static constexpr int NPC = (int)(STAGE / 1024);           // pieces per stage
    static constexpr int KP = (NPC + NP - 1) / NP;            // pieces per producer
    static constexpr int OST = 20;                            // [token][16 columns] fp32 row stride
    static constexpr int64_t OTILE = 64 * OST * 4;            // one tile's 64 x 16 fp32 tile
    static constexpr int64_t SBX = (int64_t)KB * 64 * 16;     // fp16 copy of one tile's state (B operand)
    static constexpr int64_t OFF_O = NSTAGE * STAGE;          // read-out O [2][NCONS]
    static constexpr int64_t OFF_X = OFF_O + 2 * NCONS * OTILE;  // state copies [2][NCONS]
    static constexpr int64_t TOTAL = OFF_X + 2 * NCONS * SBX;
    static constexpr int WAVES = 2 * NCONS + NP;
    static_assert(STAGE % 1024 == 0 && D * 4 <= 1024, "card pieces");
    static_assert(TOTAL <= 160 * 1024, "recurrence LDS budget");
    static_assert(OFF_O % 16 == 0 && OFF_X % 16 == 0, "alignment");
    static_assert(KP + NCONS <= 63, "outstanding-load counter");
    static_assert(NP == 4 && C == 64, "gate pieces: 32 tokens x 32 bytes per piece");
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

// 16 bytes per lane from global memory straight into LDS: lane l's bytes land at LDS
// byte offset lds + 16 l (lds is the same for the whole wave).  Written as inline
// assembly so that the compiler does not treat the copy as a pending LDS store: it
// would otherwise wait for every copy in flight before this wave's next LDS access.
// The copy is counted by vmcnt like any load; its completion is awaited explicitly
// (wait_vm) before the barrier that hands the slot to the consumers.  M0 holds the
// LDS base (the kernels keep nothing else in M0).
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
__device__ __forceinline__ void lds_copy16(const void* g, uint32_t lds) {
    asm volatile("s_mov_b32 m0, %1\n\tglobal_load_lds_dwordx4 %0, off" ::"v"(g), "s"(lds) : "memory", "m0");
}
#pragma clang diagnostic pop
__device__ __forceinline__ uint32_t lds_offset(const void* p) { return (uint32_t)(uintptr_t)p; }

// PF: one more wave that touches the cards (and gate rows) of chunk n + 2 + kPfAhead in
// iteration n, a G-th of each card per workgroup, so that the producers' and the output
// wave's loads of cards the card builder wrote long before (no longer in the Infinity
// Cache) find them in the L2 their XCD shares.  Two chunks beyond the producers' copies:
// 1, 2, 3, 4, 6 and 8 gave 1 395, 1 387, 1 399, 1 397, 1 424 and 1 449 us for B1 H16
// T65536 in pieces of 128 chunks (the touched lines must still be in the L2 when read).
constexpr int kPfAhead = 2;

// Workgroup `bid` of the `nblk` (a multiple of 8) state-pass workgroups of a launch;
// waves past the roles (and the prefetch wave) only keep the barrier count.
template <int D, class Out, int NCONS, bool PF>
__device__ __forceinline__ void rec64_body(const RecurParams& p, unsigned char* smem, int bid, int nblk) {
    using CD = Card<D>;
    using L = RecL<D, NCONS>;
    constexpr int NCT = D / 16, KB = D / 32, NP = L::NP, KP = L::KP;
    constexpr int G = D / (16 * NCONS);  // workgroups per head
    constexpr int OST = L::OST;
    static_assert(L::WAVES == 2 * NCONS + 4, "launch bounds");

    const int lane = lane_id(), wave = wave_id();
    const int m16 = lane & 15, g4 = lane >> 4;
    // XCD-aware placement: the G workgroups of one head share bid % 8
    const int logical = (bid % 8) * (nblk / 8) + bid / 8;
    const int64_t useg = logical / G;  // (b, h) * nseg + segment
    const int grp = logical % G;
    const int64_t units = p.B * p.H, nseg = p.nseg;
    if (useg >= units * nseg) return;  // padding workgroup (the whole group leaves together)
    const int64_t unit = useg / nseg, seg = useg % nseg;
    const int64_t H = p.H;
    const int64_t b = unit / H, h = unit % H;
    // the sequence of this (b, h): T tokens from row tb, NC chunks; its chunk c is card
    // cbase + c * cstride (B sequences of p.T tokens, or a variable-length batch)
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
    // this workgroup's chunks: [c0, c0 + NL) of its (b, h); card0 is chunk c0's card
    int64_t c0, NL;
    const unsigned char* card0;
    if (p.ring_len > 0) {  // one piece, whose cards are that piece's half of the ring
        c0 = p.piece * p.ring_len;
        NL = (c0 + p.ring_len < NC ? c0 + p.ring_len : NC) - c0;
        card0 = static_cast<const unsigned char*>(p.ws) + ((p.piece & 1) * units + unit) * p.ring_len * CD::BYTES;
    } else {
        c0 = seg * p.seg_len;
        NL = p.vco ? NC : (c0 + p.seg_len < NC ? c0 + p.seg_len : NC) - c0;
        card0 = static_cast<const unsigned char*>(p.ws) + (cbase + c0 * cstride) * CD::BYTES;
    }
    const int64_t cbytes = cstride * CD::BYTES;  // from one chunk's card to the next
    const bool chain = wave < NCONS;
    const bool outw = wave >= NCONS && wave < 2 * NCONS;
    const bool pfw = PF && wave == L::WAVES;  // the prefetch wave
    const bool idle = wave > L::WAVES || (!PF && wave == L::WAVES);
    const int pw = wave - 2 * NCONS;                          // producer index (producers only)
    const int cs = chain ? wave : (outw ? wave - NCONS : 0);  // value tile of a chain / output wave
    const uint16_t* gz = static_cast<const uint16_t*>(p.gate);
    // O read-out and fp16 state copy of tile t2 for chunk n: buffer n % 2
    auto obuf = [&](int64_t n, int t2) { return reinterpret_cast<float*>(smem + L::OFF_O + ((n & 1) * NCONS + t2) * L::OTILE); };
    auto sbx = [&](int64_t n) { return reinterpret_cast<_Float16*>(smem + L::OFF_X + ((n & 1) * NCONS + cs) * L::SBX); };
    const int64_t zrow0 = (tb * H + h) * D, zstride = H * D;  // element offset of (b, t, h, 0)
    typename Out::raw_t* gy = static_cast<typename Out::raw_t*>(p.out);
    auto slot = [&](int64_t ci) { return smem + (ci % L::NSTAGE) * L::STAGE; };  // local chunk index

    // each role runs its own loop (so that no role carries another's registers); all of them
    // pass the same barriers: one before the first chunk, then A and B once per chunk
    if (chain) {
        // chain state: S[ct][i] = S[16ct + 4g4 + i][col]
        const int nt = grp * NCONS + cs;
        const int col = 16 * nt + m16;
        floatx4 S[NCT];
        const float* s0 = p.s0 ? p.s0 + unit * (int64_t)D * D : nullptr;
#pragma unroll
        for (int ct = 0; ct < NCT; ++ct)
#pragma unroll
            for (int i = 0; i < 4; ++i) S[ct][i] = s0 ? s0[(16 * ct + 4 * g4 + i) * D + col] : 0.f;
        // segment scan: the state entering segment seg, S_{q+1} = M_q S_q + b_q for q < seg
        // (page "Kimi K3 report walk-through", section "KDA Context Parallelism"),
        // M_q S_q on the fp16 MFMA like every state product of the chain
        for (int64_t q = 0; q < seg; ++q) {
            const float* bq = p.sums + ((unit * (nseg - 1) + q) * 2) * (int64_t)D * D;
            const float* Mq = bq + (int64_t)D * D;
            half8 Sb[KB];
#pragma unroll
            for (int kb = 0; kb < KB; ++kb) Sb[kb] = pack_h8(S[2 * kb], S[2 * kb + 1]);
#pragma unroll
            for (int mt = 0; mt < NCT; ++mt) {
                floatx4 acc;
#pragma unroll
                for (int i = 0; i < 4; ++i) acc[i] = bq[(16 * mt + 4 * g4 + i) * D + col];
#pragma unroll
                for (int kb = 0; kb < KB; ++kb) {
                    const float* mrow = Mq + (16 * mt + m16) * D + 32 * kb + 4 * g4;  // channels cmap(kb, g4, j)
                    const float4 lo = *reinterpret_cast<const float4*>(mrow);
                    const float4 hi = *reinterpret_cast<const float4*>(mrow + 16);
                    half8 a;
                    a[0] = static_cast<_Float16>(lo.x); a[1] = static_cast<_Float16>(lo.y);
                    a[2] = static_cast<_Float16>(lo.z); a[3] = static_cast<_Float16>(lo.w);
                    a[4] = static_cast<_Float16>(hi.x); a[5] = static_cast<_Float16>(hi.y);
                    a[6] = static_cast<_Float16>(hi.z); a[7] = static_cast<_Float16>(hi.w);
                    acc = mma_f16_k32(a, Sb[kb], acc);
                }
                S[mt] = acc;  // S[mt] is not read again in this step: Sb holds the old state
            }
        }
        lds_barrier();  // the first card is resident
        for (int64_t ci = 0; ci < NL; ++ci) {
            const unsigned char* st = slot(ci);
            const _Float16* sw = reinterpret_cast<const _Float16*>(st + L::OFF_WS);
            const _Float16* sk = reinterpret_cast<const _Float16*>(st + L::OFF_KS);
            const _Float16* su = reinterpret_cast<const _Float16*>(st + L::OFF_US + cs * 2048);
            const float* sg = reinterpret_cast<const float*>(st + L::OFF_GS);
            // the state at the chunk start, as the B operand (logical k = 8g4 + j of step kb is
            // channel cmap(kb, g4, j)), for this wave and for the output wave
            half8 Sb[KB];
            _Float16* sx = sbx(ci);
#pragma unroll
            for (int kb = 0; kb < KB; ++kb) {
                Sb[kb] = pack_h8(S[2 * kb], S[2 * kb + 1]);
                *reinterpret_cast<half8*>(sx + (kb * 64 + lane) * 8) = Sb[kb];
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
            half8 kf[NCT][2];  // read while the U chain runs
#pragma unroll
            for (int ct = 0; ct < NCT; ++ct) {
#pragma unroll
                for (int u = 0; u < 2; ++u)
                    kf[ct][u] = cat_h8(ld_h4(sk + frag_piece(ct, u, 0) / 2 + lane * 4),
                                       ld_h4(sk + frag_piece(ct, u, 1) / 2 + lane * 4));
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
            if (p.snap && (ci + 1) % p.snap_chunks == 0 && (ci + 1) * C <= T) {
                // block-granular snapshot: the state after (ci + 1) C tokens of the sequence
                const int64_t slot = tb / (C * p.snap_chunks) + b + (ci + 1) / p.snap_chunks - 1;
                float* dst = p.snap + (slot * H + h) * (int64_t)D * D;
#pragma unroll
                for (int ct = 0; ct < NCT; ++ct)
#pragma unroll
                    for (int i = 0; i < 4; ++i) dst[(16 * ct + 4 * g4 + i) * D + col] = S[ct][i];
            }
            lds_barrier();  // X(ci): the state copy is visible to the output wave
        }
        lds_barrier();  // X(NL): the output wave forms its last read-out
        if (p.sT && seg == nseg - 1) {
            float* sT = p.sT + unit * (int64_t)D * D;
#pragma unroll
            for (int ct = 0; ct < NCT; ++ct)
#pragma unroll
                for (int i = 0; i < 4; ++i) sT[(16 * ct + 4 * g4 + i) * D + col] = S[ct][i];
        }
    } else if (pfw) {
        // a G-th of each card, one 4-byte load per 128-byte line, and 64 / G tokens' gate
        // rows (the head's 256 bytes of z per token, two lines); every value is folded into
        // `sink` kPfAhead iterations later, so each load has that long to land
        constexpr int64_t PART = (CD::BYTES + G - 1) / G;
        constexpr int NPF = (int)((PART + 128 * 64 - 1) / (128 * 64));
        constexpr int ZT = 64 / G;  // tokens whose gate rows this workgroup touches
        static_assert(2 * ZT <= 64, "gate lines");
        uint32_t ring[kPfAhead][NPF + 1];
#pragma unroll
        for (int s2 = 0; s2 < kPfAhead; ++s2)
#pragma unroll
            for (int j = 0; j <= NPF; ++j) ring[s2][j] = 0u;
        uint32_t sink = 0u;
        auto touch = [&](uint32_t (&r)[NPF + 1], int64_t ci) __attribute__((always_inline)) {
#pragma unroll
            for (int j = 0; j <= NPF; ++j) sink ^= r[j];
            if (ci >= NL) return;
            const unsigned char* card = card0 + ci * cbytes;
#pragma unroll
            for (int j = 0; j < NPF; ++j) {
                int64_t off = grp * PART + 128 * (int64_t)(j * 64 + lane);
                off = off < CD::BYTES - 4 ? off : CD::BYTES - 4;
                r[j] = *reinterpret_cast<const uint32_t*>(card + off);
            }
            int64_t t = (c0 + ci) * C + grp * ZT + ((lane >> 1) % ZT);
            t = t < T ? t : T - 1;
            const int zline = D == 128 ? (lane & 1) : 0;  // a head's gate row is D * 2 bytes
            r[NPF] = *reinterpret_cast<const uint32_t*>(gz + zrow0 + t * zstride + 64 * zline);
        };
        // the producers copy chunks 0 and 1 before the first barrier and chunk n + 2 in
        // iteration n: chunks 2 .. 1 + kPfAhead now, chunk n + 2 + kPfAhead in iteration n
#pragma unroll
        for (int s2 = 0; s2 < kPfAhead; ++s2) touch(ring[s2], 2 + s2);
        lds_barrier();  // the first card is resident
        for (int64_t n = 0; n <= NL; n += kPfAhead) {
#pragma unroll
            for (int s2 = 0; s2 < kPfAhead; ++s2) {
                if (n + s2 <= NL) {
                    touch(ring[s2], n + s2 + 2 + kPfAhead);
                    lds_barrier();  // X(n + s2)
                }
            }
        }
#pragma unroll
        for (int s2 = 0; s2 < kPfAhead; ++s2)
#pragma unroll
            for (int j = 0; j <= NPF; ++j) sink ^= ring[s2][j];
        asm volatile("" ::"v"(sink));  // every load has landed before the wave ends
    } else if (idle) {
        for (int64_t n = 0; n < NL + 2; ++n) lds_barrier();  // as many barriers as every role
    } else if (outw) {
        // Qe and Uo of one chunk, straight from the card into registers; two sets, the next
        // chunk's in flight while this one is used
        const int nt = grp * NCONS + cs;
        auto load_q = [&](half8 (&qf)[4][KB], half4 (&uo)[4], int64_t c) __attribute__((always_inline)) {
            if (NL == 0) return;  // an empty sequence has no card to read (nothing is read out)
            const unsigned char* card = card0 + (c < NL ? c : NL - 1) * cbytes;
#pragma unroll
            for (int mt = 0; mt < 4; ++mt) {
#pragma unroll
                for (int kb = 0; kb < KB; ++kb)
                    qf[mt][kb] = *reinterpret_cast<const half8*>(card + CD::QE + ((mt * KB + kb) * 64 + lane) * 16);
                uo[mt] = *reinterpret_cast<const half4*>(card + CD::UO + ((nt * 4 + mt) * 64 + lane) * 8);
            }
        };
        // iteration n (1 .. NL): the read-out of chunk n - 1 from the state copy the chain
        // wave left before X(n - 1); the next chunk's Qe and Uo load meanwhile
        auto step = [&](half8 (&qf)[4][KB], half4 (&uo)[4], half8 (&qn)[4][KB], half4 (&un)[4], int64_t n)
                        __attribute__((always_inline)) {
            load_q(qn, un, n);
            const _Float16* sx = sbx(n - 1);
            half8 Sb[KB];
#pragma unroll
            for (int kb = 0; kb < KB; ++kb) Sb[kb] = ld_h8(sx + (kb * 64 + lane) * 8);
            floatx4 O[4];
#pragma unroll
            for (int mt = 0; mt < 4; ++mt) O[mt] = unpack_h4(uo[mt]);  // Uo
#pragma unroll
            for (int kb = 0; kb < KB; ++kb)
#pragma unroll
                for (int mt = 0; mt < 4; ++mt) O[mt] = mma_f16_k32(qf[mt][kb], Sb[kb], O[mt]);  // + Qe S
            float* orow = obuf(n - 1, cs);
#pragma unroll
            for (int mt = 0; mt < 4; ++mt)
#pragma unroll
                for (int i = 0; i < 4; ++i) orow[(16 * mt + 4 * g4 + i) * OST + m16] = O[mt][i];
            lds_barrier();  // X(n)
        };
        half8 qa[4][KB], qb[4][KB];
        half4 ua[4], ub[4];
        load_q(qa, ua, 0);
        lds_barrier();  // the first card is resident
        lds_barrier();  // X(0): the first state copy
        // both steps in every trip (see the producers)
        int64_t n = 1;
        for (; n + 1 <= NL; n += 2) {
            step(qa, ua, qb, ub, n);
            step(qb, ub, qa, ua, n + 1);
        }
        if (n <= NL) step(qa, ua, qb, ub, n);
    } else {
        // Each producer is compiled for its index, so that the source of every piece it
        // copies is fixed at compile time (straight-line address arithmetic, no branches).
        auto producer = [&](auto pwc) __attribute__((always_inline)) {
            constexpr int PW = decltype(pwc)::value;
            // piece j of a stage is copied by producer j % NP; every producer issues exactly
            // KP copies per chunk (one short of work repeats its last piece: same bytes to
            // the same place), so that its count of outstanding loads is fixed
            auto piece = [&](int64_t ci, int k) __attribute__((always_inline)) {
                const int j0 = PW + k * NP, j = j0 < L::NPC ? j0 : L::NPC - 1;
                const int64_t c = c0 + ci;  // chunk of the sequence
                const unsigned char* card = card0 + ci * cbytes;
                const void* src;
                if (j < L::NW) {
                    src = card + CD::W + j * 1024 + lane * 16;
                } else if (j < 2 * L::NW) {
                    src = card + CD::KBT + (j - L::NW) * 1024 + lane * 16;
                } else if (j < 2 * L::NW + 2 * NCONS) {
                    const int r = j - 2 * L::NW;
                    src = card + CD::UT + (grp * NCONS + r / 2) * 2048 + (r % 2) * 1024 + lane * 16;
                } else if (j < 2 * L::NW + 4 * NCONS) {
                    // gate logits: 32 tokens per piece, lane pair (2m, 2m+1) = token m's 16 columns
                    const int r = j - 2 * L::NW - 2 * NCONS;
                    int64_t t = c * C + 32 * (r % 2) + (lane >> 1);
                    t = t < T ? t : T - 1;  // in bounds; rows past the end are never stored
                    src = gz + zrow0 + t * zstride + 16 * (grp * NCONS + r / 2) + 8 * (lane & 1);
                } else {
                    src = card + CD::GAM + (lane % (D / 4)) * 16;  // Gamma, replicated
                }
                lds_copy16(src, lds_offset(slot(ci) + (int64_t)j * 1024));
            };
            auto copy_chunk = [&](int64_t ci) __attribute__((always_inline)) {
                if (NL == 0) return;                       // no tokens: nothing to stream
                const int64_t cc = ci < NL ? ci : NL - 1;  // past the end: the last chunk again
#pragma unroll
                for (int k = 0; k < KP; ++k) piece(cc, k);
            };
            // gate and output: 16 tokens x 4 columns per lane group, per tile
            const int tq = 16 * PW + (lane >> 2), cq = 4 * (lane & 3);
            auto load_z = [&](uint2 (&z)[NCONS], int64_t n) __attribute__((always_inline)) {
                const unsigned char* st = slot(n);
#pragma unroll
                for (int t2 = 0; t2 < NCONS; ++t2)
                    z[t2] = *reinterpret_cast<const uint2*>(st + L::OFF_ZS + t2 * 2048 + tq * 32 + cq * 2);
            };
            auto output_part = [&](const uint2 (&z)[NCONS], int64_t n) __attribute__((always_inline)) {
                const int64_t t = (c0 + n) * C + tq;
#pragma unroll
                for (int t2 = 0; t2 < NCONS; ++t2) {
                    const float4 o = *reinterpret_cast<const float4*>(obuf(n, t2) + tq * OST + cq);
                    const float y0 = o.x * sigmoidf_(__uint_as_float(z[t2].x << 16));
                    const float y1 = o.y * sigmoidf_(__uint_as_float(z[t2].x & 0xffff0000u));
                    const float y2 = o.z * sigmoidf_(__uint_as_float(z[t2].y << 16));
                    const float y3 = o.w * sigmoidf_(__uint_as_float(z[t2].y & 0xffff0000u));
                    if (t < T) {
                        typename Out::raw_t* dst = gy + zrow0 + t * zstride + 16 * (grp * NCONS + t2) + cq;
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
            // Iteration n (vmcnt is in order): y of chunk n-2 (at most NCONS stores; O from the
            // output wave before X(n-1), z held in registers since iteration n-2), then the KP
            // copies of chunk n+2 into the slot of chunk n-1 (released by X(n-1)), then the gate
            // logits of chunk n.  vmcnt(KP) before X(n) leaves only this iteration's copies in
            // flight: chunk n+1's, issued one iteration earlier, have landed.
            uint2 z1[NCONS], z2[NCONS];  // gate logits of chunks n-1 and n-2
            auto step = [&](int64_t n) __attribute__((always_inline)) {
                if (n >= 2) output_part(z2, n - 2);
                copy_chunk(n + 2);
#pragma unroll
                for (int t2 = 0; t2 < NCONS; ++t2) z2[t2] = z1[t2];
                if (n < NL) load_z(z1, n);
                wait_vm<KP>();
                lds_barrier();  // X(n)
            };
            copy_chunk(0);
            copy_chunk(1);
            wait_vm<KP>();  // chunk 0
            lds_barrier();  // the first card is resident
            for (int64_t n = 0; n <= NL; ++n) step(n);
            if (NL > 0) output_part(z1, NL - 1);
            wait_vm_zero();  // the last (redundant) copies land before the workgroup's LDS is released
        };
        static_assert(NP == 4, "producer dispatch");
        switch (__builtin_amdgcn_readfirstlane(pw)) {
            case 0: producer(Int<0>{}); break;
            case 1: producer(Int<1>{}); break;
            case 2: producer(Int<2>{}); break;
            default: producer(Int<3>{}); break;
        }
    }
}

template <int D, class Out, int NCONS, bool PF>
__global__ __launch_bounds__((2 * NCONS + 4 + (PF ? 1 : 0)) * 64) __attribute__((amdgpu_waves_per_eu(1, 2)))
void kda_rec64_kernel(RecurParams p) {
    extern __shared__ __align__(16) unsigned char smem[];
    rec64_body<D, Out, NCONS, PF>(p, smem, blockIdx.x, gridDim.x);
}

// One launch of the pipelined long-sequence pass: workgroups 0 .. nstate - 1 run the state
// pass over piece rp.piece from its half of the card ring (one value tile each, with the
// prefetch wave and one more wave that only keeps the barriers), while the others build
// the cards of piece pp.piece = rp.piece + 1 into the other half, two cards per workgroup
// (waves 0-3 and 4-7, each pair of 16-token-tile waves with its own half of the LDS).
// Nothing in a launch waits on another workgroup: the pieces are ordered by the stream.
template <int D, class Out>
__global__ __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(2, 2)))
void kda_piece64_kernel(PrepParams pp, RecurParams rp, int nstate) {
    extern __shared__ __align__(16) unsigned char smem[];
    if ((int)blockIdx.x < nstate) {
        rec64_body<D, Out, 1, true>(rp, smem, blockIdx.x, nstate);
    } else {
        const int half = wave_id() >> 2;
        const int64_t c0 = pp.piece * pp.ring_len;
        const int64_t nl = (c0 + pp.ring_len < pp.NC ? c0 + pp.ring_len : pp.NC) - c0;
        const int64_t items = pp.B * pp.H * nl;
        int64_t item = 2 * ((int64_t)blockIdx.x - nstate) + half;
        item = item < items ? item : items - 1;  // an odd count: the last card twice, same bytes
        prep64_card<D, kModeStream>(pp, smem + half * PrepL<D>::TOTAL, item, wave_id() & 3);
    }
}

// ---------------------------------------------------------------------------
// kernel 3 (segment scan): the summary of one segment of chunks.  Page "Kimi K3
// report walk-through", section "KDA Context Parallelism": a segment acts on the
// state it receives as an affine map S -> M S + b, where b is the state the segment
// ends in from a zero start and M = prod (I - beta k k^T) Diag(alpha) over its tokens.
// Chunkwise, both follow the state recurrence of the cards: b with U = U~ - W S from
// S = 0, and M (d_k columns) with U = -W M from M = I.  One workgroup per (b, h,
// segment, NS of the 2 D/16 column tiles of [b | M]); per tile a chain wave, plus
// two copier waves streaming W, Kbar^T, the U~ slices and Gamma into a three-slot LDS
// ring (one barrier per chunk: the copies of chunk n+2 go into the slot of chunk n-1).
template <int D, int NS>
struct SumL {
    using CD = Card<D>;
    static constexpr int KB = D / 32, NCT = D / 16;
    static constexpr int NPW = 2;                             // copier waves
    static constexpr int NW = 4 * KB;                         // 1 KiB pieces of W; as many of Kbar^T
    static constexpr int64_t OFF_WS = 0;
    static constexpr int64_t OFF_KS = (int64_t)NW * 1024;
    static constexpr int64_t OFF_US = 2 * OFF_KS;             // U~ slices of the b tiles, 2 KiB each
    static constexpr int64_t OFF_GS = OFF_US + NS * 2048;
    static constexpr int64_t STAGE = OFF_GS + 1024;
    static constexpr int NSTAGE = 3;
    static constexpr int NPC = (int)(STAGE / 1024);
    static constexpr int KP = (NPC + NPW - 1) / NPW;
    static constexpr int64_t TOTAL = NSTAGE * STAGE;
    static constexpr int WAVES = NS + NPW;
    static constexpr int GW = 2 * NCT / NS;                   // workgroups per (b, h, segment)
    static_assert(NCT % NS == 0, "a workgroup's tiles are all b or all M");
    static_assert(TOTAL <= 160 * 1024 && KP <= 63, "summary budget");
};

template <int D, int NS>
__global__ __launch_bounds__((NS + 2) * 64) __attribute__((amdgpu_waves_per_eu(1, 2)))
void kda_sum64_kernel(RecurParams p) {
    using CD = Card<D>;
    using L = SumL<D, NS>;
    constexpr int NCT = D / 16, KB = D / 32, KP = L::KP;
    constexpr int GW = L::GW;
    extern __shared__ __align__(16) unsigned char smem[];

    const int lane = lane_id(), wave = wave_id();
    const int g4 = lane >> 4, m16 = lane & 15;
    // the GW workgroups of one (b, h, segment) share bid % 8, so their card reads meet in one L2
    const int nblk = gridDim.x, bid = blockIdx.x;
    const int logical = (bid % 8) * (nblk / 8) + bid / 8;
    const int64_t useg = logical / GW;  // (b, h) * (nseg - 1) + segment
    const int grp = logical % GW;
    const int64_t units = p.B * p.H, nsum = p.nseg - 1;
    if (useg >= units * nsum) return;  // padding workgroup (the whole group leaves together)
    const int64_t unit = useg / nsum, seg = useg % nsum;
    const int64_t NC = p.NC, c0 = seg * p.seg_len;
    const int64_t nloc = p.seg_len;  // every summarised segment is a full one
    const unsigned char* cards = static_cast<const unsigned char*>(p.ws) + unit * NC * CD::BYTES;
    const bool mtile = grp * NS >= NCT;  // this workgroup's tiles are columns of M (else of b)
    auto slot = [&](int64_t ci) { return smem + (ci % L::NSTAGE) * L::STAGE; };

    if (wave < NS) {
        const int tt = grp * NS + wave;           // tile of [b | M]
        const int col = 16 * (tt % NCT) + m16;    // column within b or M
        floatx4 S[NCT];
#pragma unroll
        for (int ct = 0; ct < NCT; ++ct)
#pragma unroll
            for (int i = 0; i < 4; ++i) S[ct][i] = (mtile && 16 * ct + 4 * g4 + i == col) ? 1.f : 0.f;
        lds_barrier();  // the first card is resident
        for (int64_t ci = 0; ci < nloc; ++ci) {
            const unsigned char* st = slot(ci);
            const _Float16* sw = reinterpret_cast<const _Float16*>(st + L::OFF_WS);
            const _Float16* sk = reinterpret_cast<const _Float16*>(st + L::OFF_KS);
            const _Float16* su = reinterpret_cast<const _Float16*>(st + L::OFF_US + wave * 2048);
            const float* sg = reinterpret_cast<const float*>(st + L::OFF_GS);
            half8 Sb[KB];
#pragma unroll
            for (int kb = 0; kb < KB; ++kb) Sb[kb] = pack_h8(S[2 * kb], S[2 * kb + 1]);
            floatx4 U[4];
#pragma unroll
            for (int mt = 0; mt < 4; ++mt) U[mt] = mtile ? zero4() : unpack_h4(ld_h4(su + (mt * 64 + lane) * 4));
#pragma unroll
            for (int ct = 0; ct < NCT; ++ct) {
                const float4 gm = *reinterpret_cast<const float4*>(sg + 16 * ct + 4 * g4);
                S[ct][0] *= gm.x;
                S[ct][1] *= gm.y;
                S[ct][2] *= gm.z;
                S[ct][3] *= gm.w;
            }
#pragma unroll
            for (int kb = 0; kb < KB; ++kb)
#pragma unroll
                for (int mt = 0; mt < 4; ++mt)
                    U[mt] = mma_f16_k32(ld_h8(sw + ((mt * KB + kb) * 64 + lane) * 8), Sb[kb], U[mt]);
            half8 Ub[2];
#pragma unroll
            for (int u = 0; u < 2; ++u) Ub[u] = pack_h8(U[2 * u], U[2 * u + 1]);
#pragma unroll
            for (int u = 0; u < 2; ++u)
#pragma unroll
                for (int ct = 0; ct < NCT; ++ct)
                    S[ct] = mma_f16_k32(cat_h8(ld_h4(sk + frag_piece(ct, u, 0) / 2 + lane * 4),
                                               ld_h4(sk + frag_piece(ct, u, 1) / 2 + lane * 4)),
                                        Ub[u], S[ct]);
            lds_barrier();  // the slot of chunk ci is free; chunk ci + 1 is resident
        }
        float* dst = (mtile ? p.sum_m : p.sum_b) + useg * p.sum_stride;
#pragma unroll
        for (int ct = 0; ct < NCT; ++ct)
#pragma unroll
            for (int i = 0; i < 4; ++i) dst[(16 * ct + 4 * g4 + i) * D + col] = S[ct][i];
    } else {
        auto copier = [&](auto pwc) __attribute__((always_inline)) {
            constexpr int PW = decltype(pwc)::value;
            auto piece = [&](int64_t ci, int k) __attribute__((always_inline)) {
                const int j0 = PW + k * L::NPW, j = j0 < L::NPC ? j0 : L::NPC - 1;
                const unsigned char* card = cards + (c0 + ci) * CD::BYTES;
                const void* src;
                if (j < L::NW) {
                    src = card + CD::W + j * 1024 + lane * 16;
                } else if (j < 2 * L::NW) {
                    src = card + CD::KBT + (j - L::NW) * 1024 + lane * 16;
                } else if (j < 2 * L::NW + 2 * NS) {
                    // U~ slices (unused by M tiles, copied all the same: fixed counts)
                    const int r = j - 2 * L::NW;
                    src = card + CD::UT + ((grp * NS) % NCT + r / 2) * 2048 + (r % 2) * 1024 + lane * 16;
                } else {
                    src = card + CD::GAM + (lane % (D / 4)) * 16;  // Gamma, replicated
                }
                lds_copy16(src, lds_offset(slot(ci) + (int64_t)j * 1024));
            };
            auto copy_chunk = [&](int64_t ci) __attribute__((always_inline)) {
                const int64_t cc = ci < nloc ? ci : nloc - 1;  // past the end: the last chunk again
#pragma unroll
                for (int k = 0; k < KP; ++k) piece(cc, k);
            };
            copy_chunk(0);
            copy_chunk(1);
            wait_vm<KP>();  // chunk 0
            lds_barrier();  // the first card is resident
            for (int64_t ci = 0; ci < nloc; ++ci) {
                copy_chunk(ci + 2);  // the slot of chunk ci - 1, released by the previous barrier
                wait_vm<KP>();       // chunk ci + 1, issued one iteration earlier
                lds_barrier();
            }
        };
        if (__builtin_amdgcn_readfirstlane(wave - NS) == 0)
            copier(Int<0>{});
        else
            copier(Int<1>{});
    }
}

// ---------------------------------------------------------------------------
// Segment scan: worth it only when the state pass alone leaves most of the GPU idle.
// With P segments the sequential depth becomes about 2 NC / P chunks (summaries, then
// the re-run), on P times the workgroups, plus a fixed cost (a third launch, the
// ordered combination of the summaries, two pipeline fills) of roughly 30 us on
// MI355X; measured, it pays off from segments of about 32 chunks.  The rule depends
// on the shape only, so that the workspace size is known on the host without a
// device query.
constexpr int kSumTiles = 2;  // column tiles of [b | M] per summary workgroup
constexpr int64_t kSlots = 256;  // workgroups one round may hold (one per CU)

int segments(int D, int64_t units, int64_t nc) {
    const int64_t g = D / 16;  // state-pass workgroups per (b, h) with one tile each
    for (int P = 8; P >= 2; P /= 2) {
        const int64_t len = (nc + P - 1) / P;
        if (P * units * g <= kSlots && (P - 1) * units * (2 * g / kSumTiles) <= kSlots && len >= 32 &&
            (P - 1) * len < nc && 2 * len + 4 < nc)
            return P;
    }
    return 1;
}

#ifndef KDA_PREFETCH_MIN_BYTES
#define KDA_PREFETCH_MIN_BYTES (256ll << 20)
#endif
bool prefetch_cards(int64_t card_bytes) { return card_bytes >= KDA_PREFETCH_MIN_BYTES; }

// Pipelined pass over few, long sequences: when the one-tile state pass leaves at least
// half of the CUs idle, the sequence is cut into pieces of piece_len() chunks and launch
// i runs the state pass over piece i beside the card builder of piece i + 1 (pieces are
// ordered by the stream alone).  The cards live in a ring of two pieces at the start of
// the workspace, followed by the fp32 state carried from one piece to the next.  Pieces
// of 128 chunks where at least four fit (each launch boundary costs the state pass a
// refill of its card pipeline), else of 64.  (Pieces that grow from a short first one
// to a long last one, which runs without the card builder beside it, measured slower:
// a launch whose card builder has more chunks than its state pass waits for the
// builder, which runs at about 3/4 of the state pass's pace per chunk when the two
// share the GPU.)
constexpr int64_t kPieceLen = 64;

int64_t piece_len(int64_t nc) { return nc >= 8 * kPieceLen ? 2 * kPieceLen : kPieceLen; }

bool use_pieces(int D, int64_t units, int64_t nc) {
    return D == 128 && units * (D / 16) <= kSlots / 2 && nc >= 4 * kPieceLen;
}

template <int D, class Out>
static hipError_t launch_pieces(const PrepParams& pp, const RecurParams& rp0, hipStream_t stream) {
    using LP = PrepL<D>;
    using LR = RecL<D, 1>;
    using CD = Card<D>;
    const int64_t units = rp0.B * rp0.H, NC = pp.NC, L = piece_len(NC);
    const int64_t npieces = (NC + L - 1) / L;
    float* carry = reinterpret_cast<float*>(static_cast<unsigned char*>(pp.ws) + 2 * units * L * CD::BYTES);
    PrepParams q = pp;
    q.ring_len = L;
    RecurParams r = rp0;
    r.ring_len = L;
    r.nseg = 1;
    r.seg_len = NC;
    const int nstate = (int)((units * (D / 16) + 7) / 8 * 8);
    // piece 0's cards: the card builder alone, on every CU
    auto k0 = kda_prep64_kernel<D, kModeStream>;
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(k0), hipFuncAttributeMaxDynamicSharedMemorySize,
                                       (int)LP::TOTAL);
    if (e != hipSuccess) return e;
    q.piece = 0;
    hipLaunchKernelGGL(k0, dim3((unsigned)(units * (L < NC ? L : NC))), dim3(256), LP::TOTAL, stream, q);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    auto kp = kda_piece64_kernel<D, Out>;
    constexpr int64_t LDS2 = 2 * LP::TOTAL;
    static_assert(LDS2 >= LR::TOTAL && LDS2 <= 160 * 1024, "two cards or one state tile per workgroup");
    if ((e = hipFuncSetAttribute(reinterpret_cast<const void*>(kp), hipFuncAttributeMaxDynamicSharedMemorySize,
                                 (int)LDS2)) != hipSuccess)
        return e;
    auto kr = kda_rec64_kernel<D, Out, 1, true>;
    if ((e = hipFuncSetAttribute(reinterpret_cast<const void*>(kr), hipFuncAttributeMaxDynamicSharedMemorySize,
                                 (int)LR::TOTAL)) != hipSuccess)
        return e;
    for (int64_t i = 0; i < npieces; ++i) {
        r.piece = i;
        r.s0 = i == 0 ? rp0.s0 : carry;
        r.sT = i == npieces - 1 ? rp0.sT : carry;
        if (i + 1 < npieces) {
            q.piece = i + 1;
            const int64_t c1 = (i + 1) * L, items = units * ((c1 + L < NC ? c1 + L : NC) - c1);
            hipLaunchKernelGGL(kp, dim3((unsigned)(nstate + (items + 1) / 2)), dim3(512), LDS2, stream, q, r, nstate);
        } else {
            hipLaunchKernelGGL(kr, dim3((unsigned)nstate), dim3((LR::WAVES + 1) * 64), LR::TOTAL, stream, r);
        }
        if ((e = hipGetLastError()) != hipSuccess) return e;
    }
    return hipSuccess;
}

// Launches the card builder, the segment summaries (rp.nseg > 1) and, unless
// summary_only, the state pass.
template <int D, class Out, int NCONS>
static hipError_t launch_d(const PrepParams& pp, const RecurParams& rp0, hipStream_t stream,
                           bool summary_only = false) {
    using LP = PrepL<D>;
    using LR = RecL<D, NCONS>;
    using LS = SumL<D, kSumTiles>;
    const int64_t units = rp0.B * rp0.H;
    if constexpr (NCONS == 1 && D == 128) {
        if (!summary_only && !pp.vco && !pp.cards_ready && !pp.qk_norm && !pp.logits && pp.clamp &&
            rp0.nseg <= 1 && use_pieces(D, units, pp.NC))
            return launch_pieces<D, Out>(pp, rp0, stream);
    }
    RecurParams rp = rp0;
    // one workgroup per card, two per CU; a variable-length grid covers the most chunks
    // its offsets can give (pp.T = packed rows) and the surplus groups leave at once
    const int64_t items = pp.vco ? varlen_max_chunks(pp.vN, pp.T, C) * pp.H : units * pp.NC;
    if (items > 0 && !pp.cards_ready) {
        const int mode = (pp.qk_norm ? kModeQkNorm : 0) | (pp.logits ? kModeLogits : 0) |
                         (pp.clamp ? 0 : kModeWide);
        auto kp = mode == 0   ? kda_prep64_kernel<D, 0>
                  : mode == 1 ? kda_prep64_kernel<D, 1>
                  : mode == 2 ? kda_prep64_kernel<D, 2>
                  : mode == 3 ? kda_prep64_kernel<D, 3>
                  : mode == 4 ? kda_prep64_kernel<D, 4>
                  : mode == 5 ? kda_prep64_kernel<D, 5>
                  : mode == 6 ? kda_prep64_kernel<D, 6>
                              : kda_prep64_kernel<D, 7>;
        hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kp),
                                           hipFuncAttributeMaxDynamicSharedMemorySize, (int)LP::TOTAL);
        if (e != hipSuccess) return e;
        hipLaunchKernelGGL(kp, dim3((unsigned)items), dim3(256), LP::TOTAL, stream, pp);
        e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    if (rp.nseg > 1) {
        if (!rp.sum_b) {  // the state pass's layout: b_p then M_p per segment
            rp.sum_b = rp.sums;
            rp.sum_m = rp.sums + (int64_t)D * D;
            rp.sum_stride = 2 * (int64_t)D * D;
        }
        auto ks = kda_sum64_kernel<D, kSumTiles>;
        hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(ks),
                                           hipFuncAttributeMaxDynamicSharedMemorySize, (int)LS::TOTAL);
        if (e != hipSuccess) return e;
        const int64_t blocks = (units * (rp.nseg - 1) * LS::GW + 7) / 8 * 8;
        hipLaunchKernelGGL(ks, dim3((unsigned)blocks), dim3(LS::WAVES * 64), LS::TOTAL, stream, rp);
        e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    if (summary_only) return hipSuccess;
    // the prefetch wave pays where the cards outgrow the 256 MB Infinity Cache; with two
    // value tiles per workgroup a ninth wave would leave too few registers per wave
    const bool pf = NCONS == 1 && prefetch_cards(items * Card<D>::BYTES);
    auto kr = pf ? kda_rec64_kernel<D, Out, NCONS, NCONS == 1> : kda_rec64_kernel<D, Out, NCONS, false>;
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kr),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)LR::TOTAL);
    if (e != hipSuccess) return e;
    constexpr int G = D / (16 * NCONS);
    const int64_t blocks = (units * rp.nseg * G + 7) / 8 * 8;
    hipLaunchKernelGGL(kr, dim3((unsigned)blocks), dim3((LR::WAVES + (pf ? 1 : 0)) * 64), LR::TOTAL, stream, rp);
    return hipGetLastError();
}

}  // namespace c64

int64_t prefill64_card_bytes(int D) {
    return D == 128 ? c64::Card<128>::BYTES : D == 64 ? c64::Card<64>::BYTES : -1;
}

int prefill64_segments(int D, int64_t units, int64_t nc) { return c64::segments(D, units, nc); }

int64_t prefill64_extra_bytes(int D, int64_t units, int64_t nc) {
    const int P = c64::segments(D, units, nc);
    return P > 1 ? units * (P - 1) * 2 * (int64_t)D * D * 4 : 0;  // b_p and M_p, fp32
}

hipError_t launch_prefill64(int D, int out_bf16, const PrepParams& pp, const RecurParams& rp0,
                            hipStream_t stream) {
    // the caller fills seg_len / nseg / sums only when it wants the segment scan
    RecurParams rp = rp0;
    if (rp.nseg < 1 || !rp.sums) {
        rp.nseg = 1;
        rp.seg_len = rp.NC;
    }
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

hipError_t launch_summary64(int D, const PrepParams& pp, float* M, float* b, hipStream_t stream) {
    // one summarised segment spanning all NC chunks: the summary kernel's segment 0 of
    // nseg = 2 (the second, never summarised, segment is empty); the padding tokens of
    // a last partial chunk are identity steps, so the summary is exact for any T
    RecurParams rp{};
    rp.B = pp.B;
    rp.T = pp.T;
    rp.H = pp.H;
    rp.NC = pp.NC;
    rp.ws = pp.ws;
    rp.nseg = 2;
    rp.seg_len = pp.NC;
    rp.sum_b = b;
    rp.sum_m = M;
    rp.sum_stride = (int64_t)D * D;
    if (pp.NC < 1) return hipErrorInvalidValue;
    if (D == 128) return c64::launch_d<128, InF32, 1>(pp, rp, stream, true);
    if (D == 64) return c64::launch_d<64, InF32, 1>(pp, rp, stream, true);
    return hipErrorInvalidValue;
}

}  // namespace kda
