// Single-token recurrent KDA step on a stored fp32 state (decode).
//
// Per (b, h), following the per-token order of page "3T models are no longer
// magic", section "Gate 1: KDA makes it computable" (forget, delta-rule
// corrective write, read the new state, output gate):
//   S' = Diag(alpha) S                     alpha = exp(clamp(log_alpha))
//   r  = S'^T k,  o' = S'^T q              (one pass over the decayed state)
//   u  = beta (v - r)
//   S  = S' + k u^T                         (written back in place)
//   o  = S^T q = o' + (q . k) u             (no second pass needed)
//   y  = o * sigmoid(z)
// The state is read once and written once: the step is HBM-bound (about
// 0.86 flop per byte), so it runs on the vector ALUs with coalesced 16-byte
// accesses, one workgroup per (b, h) and the 64 KiB state held in registers
// between the read and the write.  The state moves with non-temporal loads and
// stores: it is touched once per step, and keeping it out of the caches lets the
// read-modify-write stream closer to the HBM rate.
#include "kda_device.h"
#include "kda_decode.h"

namespace kda {

template <class In, class Out, int DK, int DV>
__global__ __launch_bounds__(256) void kda_decode_kernel(DecodeParams p) {
    constexpr int NT = 256;
    constexpr int COLS = DV / 4;      // threads across a row (one float4 each)
    constexpr int RG = NT / COLS;     // row groups
    constexpr int RPT = DK / RG;      // rows per thread
    static_assert(DK % RG == 0 && RPT >= 1, "decode tiling");
    using raw_t = typename In::raw_t;

    __shared__ float s_q[DK], s_k[DK], s_a[DK];
    __shared__ float s_red_r[RG][DV], s_red_o[RG][DV];
    __shared__ float s_u[DV];
    __shared__ float s_qk;
    __shared__ float s_ss[2][DK / 64 > 0 ? DK / 64 : 1];  // per-wave partial |q|^2, |k|^2

    const int64_t unit = blockIdx.x;
    if (unit >= p.units) return;
    const int tid = threadIdx.x;
    const raw_t* q = static_cast<const raw_t*>(p.q);
    const raw_t* k = static_cast<const raw_t*>(p.k);
    const raw_t* la = static_cast<const raw_t*>(p.la);
    // this thread's value-column inputs (tid < DV), loaded first so that their latency
    // overlaps the state's
    float vin = 0.f, zin = 0.f, bin = 0.f;
    if (tid < DV) {
        vin = In::load(static_cast<const raw_t*>(p.v), unit * DV + tid);
        zin = In::load(static_cast<const raw_t*>(p.gate), unit * DV + tid);
        bin = In::load(static_cast<const raw_t*>(p.beta), unit);
    }

    if (tid < DK) {
        const float qv = In::load(q, unit * DK + tid), kv = In::load(k, unit * DK + tid);
        s_q[tid] = qv;
        s_k[tid] = kv;
        const float l = log_alpha_in(In::load(la, unit * DK + tid), p.logits != 0, p.clamp != 0);
        s_a[tid] = fast_exp2(l * kLog2e);
        if (p.qk_norm) {  // squared norms of raw q and k, one partial per wave
            float sq = qv * qv, sk = kv * kv;
#pragma unroll
            for (int off = 32; off > 0; off >>= 1) {
                sq += __shfl_xor(sq, off);
                sk += __shfl_xor(sk, off);
            }
            if ((tid & 63) == 0) {
                s_ss[0][tid >> 6] = sq;
                s_ss[1][tid >> 6] = sk;
            }
        }
    }

    const int cg = tid % COLS, rg = tid / COLS;
    float4* st = reinterpret_cast<float4*>(p.state + unit * (int64_t)DK * DV);
    float4 s[RPT];
#pragma unroll
    for (int i = 0; i < RPT; ++i) {
        const floatx4 v = __builtin_nontemporal_load(reinterpret_cast<const floatx4*>(st) + (rg * RPT + i) * COLS + cg);
        s[i] = make_float4(v[0], v[1], v[2], v[3]);
    }
    __syncthreads();

    // normalisation factors of raw q and k (1 for inputs that arrive normalised)
    float qs = 1.f, ks = 1.f;
    if (p.qk_norm) {
        float sq = 0.f, sk = 0.f;
#pragma unroll
        for (int w = 0; w < (DK / 64 > 0 ? DK / 64 : 1); ++w) {
            sq += s_ss[0][w];
            sk += s_ss[1][w];
        }
        qs = inv_norm(sq) * (1.0f / __builtin_sqrtf((float)DK));
        ks = inv_norm(sk);
    }

    // q . k on wave 0
    if (tid < 64) {
        float part = 0.f;
        for (int c = tid; c < DK; c += 64) part += s_q[c] * s_k[c];
#pragma unroll
        for (int off = 32; off > 0; off >>= 1) part += __shfl_xor(part, off);
        if (tid == 0) s_qk = part * (qs * ks);
    }

    float4 pr = {0.f, 0.f, 0.f, 0.f}, po = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int i = 0; i < RPT; ++i) {
        const int r = rg * RPT + i;
        const float a = s_a[r], kr = s_k[r] * ks, qr = s_q[r] * qs;
        s[i].x *= a; s[i].y *= a; s[i].z *= a; s[i].w *= a;
        pr.x += s[i].x * kr; pr.y += s[i].y * kr; pr.z += s[i].z * kr; pr.w += s[i].w * kr;
        po.x += s[i].x * qr; po.y += s[i].y * qr; po.z += s[i].z * qr; po.w += s[i].w * qr;
    }
    *reinterpret_cast<float4*>(&s_red_r[rg][4 * cg]) = pr;
    *reinterpret_cast<float4*>(&s_red_o[rg][4 * cg]) = po;
    __syncthreads();

    if (tid < DV) {
        float r = 0.f, o = 0.f;
#pragma unroll
        for (int g = 0; g < RG; ++g) { r += s_red_r[g][tid]; o += s_red_o[g][tid]; }
        const float u = bin * (vin - r);
        s_u[tid] = u;
        const float y = (o + s_qk * u) * sigmoidf_(zin);
        static_cast<typename Out::raw_t*>(p.out)[unit * DV + tid] = Out::from_float(y);
    }
    __syncthreads();

    const float4 u4 = *reinterpret_cast<const float4*>(&s_u[4 * cg]);
#pragma unroll
    for (int i = 0; i < RPT; ++i) {
        const float kr = s_k[rg * RPT + i] * ks;
        s[i].x += kr * u4.x; s[i].y += kr * u4.y; s[i].z += kr * u4.z; s[i].w += kr * u4.w;
        const floatx4 v = {s[i].x, s[i].y, s[i].z, s[i].w};
        __builtin_nontemporal_store(v, reinterpret_cast<floatx4*>(st) + (rg * RPT + i) * COLS + cg);
    }
}

template <class In, class Out, int D>
static hipError_t launch_decode_t(const DecodeParams& p, hipStream_t stream) {
    hipLaunchKernelGGL((kda_decode_kernel<In, Out, D, D>), dim3((unsigned)p.units), dim3(256), 0,
                       stream, p);
    return hipGetLastError();
}

template <class In, class Out>
static hipError_t launch_decode_d(int D, const DecodeParams& p, hipStream_t stream) {
    return D == 128 ? launch_decode_t<In, Out, 128>(p, stream) : launch_decode_t<In, Out, 64>(p, stream);
}

// Host launcher used by the C ABI (arguments already validated).
hipError_t launch_decode(int dtype_bf16, int out_bf16, int D, const DecodeParams& p,
                         hipStream_t stream) {
    if (p.units == 0) return hipSuccess;
    if (dtype_bf16)
        return out_bf16 ? launch_decode_d<InBF16, InBF16>(D, p, stream)
                        : launch_decode_d<InBF16, InF32>(D, p, stream);
    return out_bf16 ? launch_decode_d<InF32, InBF16>(D, p, stream)
                    : launch_decode_d<InF32, InF32>(D, p, stream);
}

}  // namespace kda
