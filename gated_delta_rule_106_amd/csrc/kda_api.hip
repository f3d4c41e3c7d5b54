// C ABI of the KDA library: host-side validation, workspace sizing, dispatch.
// Every check runs before the first HIP call; see include/kda.h for the contract.
#include <limits.h>

#include <mutex>

#include "../../include/kda.h"
#include "kda_backward.h"
#include "kda_decode.h"
#include "kda_prefill.h"
#include "kda_segment.h"
#include "kda_varlen.h"

// Scratch of kda_chunk_fwd_noalloc: the per-chunk cards (and segment summaries) that
// kda_chunk_fwd keeps in the caller's workspace.  Each device holds its own copy from the
// loading of the library's code until the process ends; every call on a device shares it.
static __device__ __align__(256) unsigned char scratch[KDA_NOALLOC_SCRATCH_BYTES];

namespace {

constexpr int kDefaultChunkBf16 = 64;
constexpr uint32_t kPrepFlags = KDA_FLAG_QK_L2NORM | KDA_FLAG_GATE_LOGITS;
constexpr int kDefaultChunkF32 = 16;

bool mul_ok(int64_t a, int64_t b, int64_t* out) {
    if (a < 0 || b < 0) return false;
    if (a != 0 && b > INT64_MAX / a) return false;
    *out = a * b;
    return true;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// elements of one state tensor [B, H, Dk, Dv] (sizes already checked not to overflow)
int64_t bh_elems(const kda_fwd_args* a) { return a->B * a->H * a->Dk * a->Dv; }

int resolve_chunk(const kda_fwd_args* a) {
    if (a->chunk != 0) return a->chunk;
    return a->dtype == KDA_BF16 ? kDefaultChunkBf16 : kDefaultChunkF32;
}

// Sizes, dtype, head size, chunk and flags; fills the chunk count and card size.
int check_shape(const kda_fwd_args* a, int* chunk, int64_t* nchunks, int64_t* card, int64_t* ws_total) {
    if (!a) return KDA_ERR_NULL;
    if (a->B < 0 || a->T < 0 || a->H < 0 || a->Dk <= 0 || a->Dv <= 0) return KDA_ERR_SHAPE;
    if (a->dtype != KDA_F32 && a->dtype != KDA_BF16) return KDA_ERR_UNSUPPORTED;
    if (a->Dk != a->Dv || (a->Dk != 64 && a->Dk != 128)) return KDA_ERR_UNSUPPORTED;
    if (a->out_dtype != KDA_F32 && a->out_dtype != KDA_BF16) return KDA_ERR_UNSUPPORTED;
    if ((a->flags & ~(KDA_FLAG_NO_CLAMP | KDA_FLAG_NO_SEGMENT_SCAN | kPrepFlags | KDA_FLAG_CARDS_READY)) != 0)
        return KDA_ERR_UNSUPPORTED;
    const int c = resolve_chunk(a);
    if (!kda::prefill_supported(a->dtype == KDA_BF16, c, (int)a->Dk)) return KDA_ERR_UNSUPPORTED;
    // cards can only have come from the chunk-64 bf16 path (summary or prefill)
    if ((a->flags & KDA_FLAG_CARDS_READY) && (a->dtype != KDA_BF16 || c != 64)) return KDA_ERR_UNSUPPORTED;
    // every element index of every tensor must fit in int64
    int64_t bt, bth, elems, bh, st;
    if (!mul_ok(a->B, a->T, &bt) || !mul_ok(bt, a->H, &bth) || !mul_ok(bth, a->Dk, &elems) ||
        !mul_ok(a->B, a->H, &bh) || !mul_ok(bh, a->Dk * a->Dv, &st))
        return KDA_ERR_SHAPE;
    if (a->H > INT_MAX || bh > INT_MAX) return KDA_ERR_SHAPE;  // grid dimensions
    const int64_t nc = (a->T + c - 1) / c;
    if (nc > INT_MAX) return KDA_ERR_SHAPE;
    const int64_t cb = kda::prefill_card_bytes(a->dtype == KDA_BF16, c, (int)a->Dk);
    int64_t tmp, total;
    if (cb <= 0 || !mul_ok(bh, nc, &tmp) || !mul_ok(tmp, cb, &total)) return KDA_ERR_SHAPE;
    if (tmp > INT_MAX) return KDA_ERR_SHAPE;  // one workgroup per (b, h, chunk)
    // segment-scan summaries (chunk-64 bf16 path; small only when B*H is small)
    const int64_t extra = (a->dtype == KDA_BF16 && c == 64) ? kda::prefill64_extra_bytes((int)a->Dk, bh, nc) : 0;
    if (extra > INT64_MAX - total) return KDA_ERR_SHAPE;
    *chunk = c;
    *nchunks = nc;
    *card = cb;
    *ws_total = total + extra;
    return KDA_OK;
}

// Varlen: sizes, dtype, chunk, flags and snapshot interval; fills the workspace
// layout (cards, then the sequence map).
struct VarlenLayout {
    int chunk;
    int64_t max_chunks, card, cards_bytes, off_s, off_co, off_soc, total;
};

int64_t align256(int64_t x) { return (x + 255) / 256 * 256; }

int check_varlen(const kda_varlen_args* a, VarlenLayout* L) {
    if (!a) return KDA_ERR_NULL;
    if (a->N < 0 || a->rows < 0 || a->H < 0 || a->Dk <= 0 || a->Dv <= 0 || a->snapshot_every < 0)
        return KDA_ERR_SHAPE;
    if (a->dtype != KDA_F32 && a->dtype != KDA_BF16) return KDA_ERR_UNSUPPORTED;
    if (a->Dk != a->Dv || (a->Dk != 64 && a->Dk != 128)) return KDA_ERR_UNSUPPORTED;
    const int c = a->chunk != 0 ? a->chunk : (a->dtype == KDA_BF16 ? kDefaultChunkBf16 : kDefaultChunkF32);
    if (!kda::prefill_supported(a->dtype == KDA_BF16, c, (int)a->Dk)) return KDA_ERR_UNSUPPORTED;
    if (a->out_dtype != KDA_F32 && a->out_dtype != KDA_BF16) return KDA_ERR_UNSUPPORTED;
    if ((a->flags & ~(KDA_FLAG_NO_CLAMP | KDA_FLAG_NO_SEGMENT_SCAN | kPrepFlags)) != 0) return KDA_ERR_UNSUPPORTED;
    if (a->snapshot_every % 64 != 0) return KDA_ERR_UNSUPPORTED;
    int64_t elems, nh, st;
    if (!mul_ok(a->rows, a->H, &elems) || !mul_ok(elems, a->Dk, &elems) || !mul_ok(a->N, a->H, &nh) ||
        !mul_ok(nh, a->Dk * a->Dv, &st))
        return KDA_ERR_SHAPE;
    if (a->N >= INT32_MAX || a->H > INT_MAX || nh > INT_MAX) return KDA_ERR_SHAPE;
    const int64_t mc = kda::varlen_max_chunks(a->N, a->rows, c);
    const int64_t cb = kda::prefill_card_bytes(a->dtype == KDA_BF16, c, (int)a->Dk);
    int64_t items, cards;
    if (!mul_ok(mc, a->H, &items) || items > INT_MAX || !mul_ok(items, cb, &cards)) return KDA_ERR_SHAPE;
    if (a->snapshot_every > 0) {
        int64_t slots = a->rows / a->snapshot_every + a->N, sb;
        if (!mul_ok(slots, st / (a->N > 0 ? a->N : 1), &sb)) return KDA_ERR_SHAPE;
    }
    L->chunk = c;
    L->max_chunks = mc;
    L->card = cb;
    L->cards_bytes = align256(cards);
    L->off_s = L->cards_bytes;
    L->off_co = L->off_s + align256((a->N + 1) * 8);
    L->off_soc = L->off_co + align256((a->N + 1) * 8);
    L->total = L->off_soc + align256(mc * 4);
    return KDA_OK;
}

// Backward: sizes, dtype, head size and flags; fills the chunk count and workspace bytes.
int check_bwd(const kda_bwd_args* a, int64_t* nchunks, int64_t* ws_total) {
    if (!a) return KDA_ERR_NULL;
    if (a->B < 0 || a->T < 0 || a->H < 0 || a->Dk <= 0 || a->Dv <= 0) return KDA_ERR_SHAPE;
    if (a->dtype != KDA_F32 && a->dtype != KDA_BF16) return KDA_ERR_UNSUPPORTED;
    if (a->Dk != a->Dv || (a->Dk != 64 && a->Dk != 128)) return KDA_ERR_UNSUPPORTED;
    if ((a->flags & ~(KDA_FLAG_NO_CLAMP | KDA_FLAG_QK_L2NORM | KDA_FLAG_GATE_LOGITS)) != 0)
        return KDA_ERR_UNSUPPORTED;
    int64_t bt, bth, elems, bh, st, items, tmp;
    if (!mul_ok(a->B, a->T, &bt) || !mul_ok(bt, a->H, &bth) || !mul_ok(bth, a->Dk, &elems) ||
        !mul_ok(a->B, a->H, &bh) || !mul_ok(bh, a->Dk * a->Dv, &st))
        return KDA_ERR_SHAPE;
    if (bh > INT_MAX / 16) return KDA_ERR_SHAPE;  // two sweep workgroups per (b, h, 16 value columns)
    const int64_t nc = (a->T + 63) / 64;
    // per chunk: the two records and two states stay below 1 MiB
    if (!mul_ok(bh, nc, &items) || !mul_ok(items, (int64_t)1 << 20, &tmp)) return KDA_ERR_SHAPE;
    if (items > INT_MAX) return KDA_ERR_SHAPE;  // one workgroup per (b, h, chunk)
    *nchunks = nc;
    *ws_total = kda::bwd_workspace_bytes((int)a->Dk, bh, nc);
    return KDA_OK;
}

// Variable-length backward: sizes, dtype, head size and flags; the workspace layout (the
// per-chunk sections for the most chunks the offsets can give, then the sequence map).
struct BwdVarlenLayout {
    int64_t max_chunks, off_s, off_co, off_soc, total;
};

int check_bwd_varlen(const kda_bwd_varlen_args* a, BwdVarlenLayout* L) {
    if (!a) return KDA_ERR_NULL;
    if (a->N < 0 || a->rows < 0 || a->H < 0 || a->Dk <= 0 || a->Dv <= 0) return KDA_ERR_SHAPE;
    if (a->dtype != KDA_F32 && a->dtype != KDA_BF16) return KDA_ERR_UNSUPPORTED;
    if (a->Dk != a->Dv || (a->Dk != 64 && a->Dk != 128)) return KDA_ERR_UNSUPPORTED;
    if ((a->flags & ~(KDA_FLAG_NO_CLAMP | KDA_FLAG_QK_L2NORM | KDA_FLAG_GATE_LOGITS)) != 0)
        return KDA_ERR_UNSUPPORTED;
    int64_t elems, nh, st, items, tmp;
    if (!mul_ok(a->rows, a->H, &elems) || !mul_ok(elems, a->Dk, &elems) || !mul_ok(a->N, a->H, &nh) ||
        !mul_ok(nh, a->Dk * a->Dv, &st))
        return KDA_ERR_SHAPE;
    if (a->N >= INT32_MAX || nh > INT_MAX / 16) return KDA_ERR_SHAPE;  // sequence ids; sweep grid
    const int64_t mc = kda::varlen_max_chunks(a->N, a->rows, 64);
    // per chunk: the two records and two states stay below 1 MiB; one workgroup per chunk
    if (!mul_ok(mc, a->H, &items) || !mul_ok(items, (int64_t)1 << 20, &tmp) || items > INT_MAX)
        return KDA_ERR_SHAPE;
    L->max_chunks = mc;
    L->off_s = kda::bwd_workspace_bytes((int)a->Dk, a->H, mc);
    L->off_co = L->off_s + align256((a->N + 1) * 8);
    L->off_soc = L->off_co + align256((a->N + 1) * 8);
    L->total = L->off_soc + align256(mc * 4);
    return KDA_OK;
}

// Token tensors present and aligned, states aligned (after check_shape).
int check_fwd_tensors(const kda_fwd_args* a) {
    if (a->B * a->T * a->H > 0) {
        const void* req[] = {a->q, a->k, a->v, a->log_alpha, a->beta, a->gate, a->out};
        for (const void* p : req)
            if (!p) return KDA_ERR_NULL;
        for (const void* p : req)
            if (!aligned16(p)) return KDA_ERR_ALIGN;
    }
    if (!aligned16(a->initial_state) || !aligned16(a->final_state)) return KDA_ERR_ALIGN;
    return KDA_OK;
}

int run_chunk_fwd(const kda_fwd_args* a, int c, int64_t nc, int64_t cb, void* workspace, hipStream_t stream);

// Device address of `scratch` on the stream's device, looked up once per device (with
// that device current) and kept.  The array's host-side name is only a handle for the
// runtime: kernels and copies take the address returned here.
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices];

int scratch_address(hipStream_t stream, void** out) {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return KDA_ERR_HIP;
    if (stream) {  // the work goes to the stream's device: it must be the current one
        hipDevice_t sdev = -1;
        if (hipStreamGetDevice(stream, &sdev) != hipSuccess) return KDA_ERR_HIP;
        if ((int)sdev != dev) return KDA_ERR_UNSUPPORTED;
    }
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void* p = nullptr;
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return KDA_ERR_HIP;
        g_scratch_ptr[dev] = p;
    }
    *out = g_scratch_ptr[dev];
    return KDA_OK;
}

}  // namespace

extern "C" {

int kda_chunk_fwd_varlen_workspace_size(const kda_varlen_args* a, size_t* bytes) {
    if (!a || !bytes) return KDA_ERR_NULL;
    VarlenLayout L;
    const int st = check_varlen(a, &L);
    if (st != KDA_OK) return st;
    *bytes = (size_t)L.total;
    return KDA_OK;
}

int kda_chunk_fwd_varlen(const kda_varlen_args* a, hipStream_t stream) {
    VarlenLayout L;
    const int st = check_varlen(a, &L);
    if (st != KDA_OK) return st;
    if (a->N == 0 || a->H == 0) return KDA_OK;
    if (!a->cu_seqlens) return KDA_ERR_NULL;
    if (a->rows > 0) {
        const void* req[] = {a->q, a->k, a->v, a->log_alpha, a->beta, a->gate, a->out};
        for (const void* p : req)
            if (!p) return KDA_ERR_NULL;
        for (const void* p : req)
            if (!aligned16(p)) return KDA_ERR_ALIGN;
    }
    if (a->snapshot_every > 0 && !a->snapshots) return KDA_ERR_NULL;
    const void* opt[] = {a->initial_state, a->final_state, a->snapshots, a->workspace};
    for (const void* p : opt)
        if (!aligned16(p)) return KDA_ERR_ALIGN;
    if ((reinterpret_cast<uintptr_t>(a->cu_seqlens) & 7u) != 0) return KDA_ERR_ALIGN;
    if (!a->workspace || (int64_t)a->workspace_bytes < L.total) return KDA_ERR_WORKSPACE;

    unsigned char* ws = static_cast<unsigned char*>(a->workspace);
    kda::VarlenMap m{reinterpret_cast<int64_t*>(ws + L.off_s), reinterpret_cast<int64_t*>(ws + L.off_co),
                     reinterpret_cast<int32_t*>(ws + L.off_soc)};
    hipError_t e = kda::launch_varlen_map(m, a->cu_seqlens, a->N, a->rows, L.chunk, stream);
    if (e != hipSuccess) return KDA_ERR_HIP;
    // NC: the most chunks the offsets can give (the card builder's grid)
    kda::PrepParams pp{a->q, a->k, a->v, a->log_alpha, a->beta, a->workspace,
                       1, a->rows, a->H, L.max_chunks, (a->flags & KDA_FLAG_NO_CLAMP) ? 0 : 1,
                       (a->flags & KDA_FLAG_QK_L2NORM) ? 1 : 0, (a->flags & KDA_FLAG_GATE_LOGITS) ? 1 : 0,
                       m.s, m.co, m.soc, a->N};
    kda::RecurParams rp{a->gate, a->out, a->initial_state, a->final_state, a->workspace,
                        a->N, 0, a->H, 0, 0, 1, nullptr};
    rp.vs = m.s;
    rp.vco = m.co;
    rp.snap = a->snapshot_every > 0 ? a->snapshots : nullptr;
    rp.snap_chunks = a->snapshot_every > 0 ? a->snapshot_every / L.chunk : 1;
    e = kda::launch_prefill(a->dtype == KDA_BF16, a->out_dtype == KDA_BF16, L.chunk, (int)a->Dk, pp, rp, stream);
    return e == hipSuccess ? KDA_OK : KDA_ERR_HIP;
}

int kda_version(void) { return KDA_VERSION; }

const char* kda_status_str(int status) {
    switch (status) {
        case KDA_OK: return "ok";
        case KDA_ERR_NULL: return "a required pointer is NULL";
        case KDA_ERR_SHAPE: return "negative or overflowing sizes";
        case KDA_ERR_UNSUPPORTED: return "unsupported head size, dtype, chunk size or flag";
        case KDA_ERR_WORKSPACE: return "workspace missing or too small";
        case KDA_ERR_ALIGN: return "a pointer is not 16-byte aligned";
        case KDA_ERR_HIP: return "the HIP runtime reported a launch error";
        case KDA_ERR_TOO_LARGE: return "the call needs more scratch than the fixed no-allocation buffer holds";
        default: return "unknown status";
    }
}

int kda_chunk_fwd_workspace_size(const kda_fwd_args* a, size_t* bytes) {
    if (!a || !bytes) return KDA_ERR_NULL;
    int c;
    int64_t nc, cb, ws;
    const int st = check_shape(a, &c, &nc, &cb, &ws);
    if (st != KDA_OK) return st;
    *bytes = (size_t)ws;
    return KDA_OK;
}

int kda_chunk_fwd(const kda_fwd_args* a, hipStream_t stream) {
    if (!a) return KDA_ERR_NULL;
    int c;
    int64_t nc, cb, need;
    int st = check_shape(a, &c, &nc, &cb, &need);
    if (st != KDA_OK) return st;
    st = check_fwd_tensors(a);
    if (st != KDA_OK) return st;
    if (need > 0) {
        if (!a->workspace) return KDA_ERR_WORKSPACE;
        if ((int64_t)a->workspace_bytes < need) return KDA_ERR_WORKSPACE;
        if (!aligned16(a->workspace)) return KDA_ERR_ALIGN;
    }
    return run_chunk_fwd(a, c, nc, cb, a->workspace, stream);
}

int kda_chunk_fwd_noalloc(const kda_fwd_args* a, hipStream_t stream) {
    if (!a) return KDA_ERR_NULL;
    int c;
    int64_t nc, cb, need;
    int st = check_shape(a, &c, &nc, &cb, &need);
    if (st != KDA_OK) return st;
    // the cards of an earlier call are not known to be in the shared buffer
    if (a->flags & KDA_FLAG_CARDS_READY) return KDA_ERR_UNSUPPORTED;
    if ((uint64_t)need > (uint64_t)KDA_NOALLOC_SCRATCH_BYTES) return KDA_ERR_TOO_LARGE;
    st = check_fwd_tensors(a);
    if (st != KDA_OK) return st;
    if (a->B * a->H == 0) return KDA_OK;
    if (a->B * a->T * a->H == 0 && !a->final_state) return KDA_OK;
    void* ws = nullptr;
    st = scratch_address(stream, &ws);
    if (st != KDA_OK) return st;
    return run_chunk_fwd(a, c, nc, cb, ws, stream);
}

}  // extern "C"

namespace {

int run_chunk_fwd(const kda_fwd_args* a, int c, int64_t nc, int64_t cb, void* workspace, hipStream_t stream) {
    const bool has_tokens = a->B * a->T * a->H > 0;
    if (a->B * a->H == 0) return KDA_OK;
    if (!has_tokens && !a->final_state) return KDA_OK;

    kda::PrepParams pp{a->q, a->k, a->v, a->log_alpha, a->beta, workspace,
                       a->B, a->T, a->H, nc, (a->flags & KDA_FLAG_NO_CLAMP) ? 0 : 1,
                       (a->flags & KDA_FLAG_QK_L2NORM) ? 1 : 0, (a->flags & KDA_FLAG_GATE_LOGITS) ? 1 : 0};
    pp.cards_ready = (a->flags & KDA_FLAG_CARDS_READY) ? 1 : 0;
    kda::RecurParams rp{a->gate, a->out, a->initial_state, a->final_state, workspace,
                        a->B, a->T, a->H, nc, nc, 1, nullptr};
    // the state pass of every segment reads initial_state at its start while the last
    // segment writes final_state at its end: no segments when the two overlap
    const bool states_overlap =
        a->initial_state && a->final_state &&
        a->final_state < a->initial_state + bh_elems(a) && a->initial_state < a->final_state + bh_elems(a);
    if (a->dtype == KDA_BF16 && c == 64 && !(a->flags & KDA_FLAG_NO_SEGMENT_SCAN) && !states_overlap) {
        const int P = kda::prefill64_segments((int)a->Dk, a->B * a->H, nc);
        if (P > 1) {
            rp.nseg = P;
            rp.seg_len = (nc + P - 1) / P;
            rp.sums = reinterpret_cast<float*>(static_cast<unsigned char*>(workspace) + a->B * a->H * nc * cb);
        }
    }
    const hipError_t e = kda::launch_prefill(a->dtype == KDA_BF16, a->out_dtype == KDA_BF16, c,
                                             (int)a->Dk, pp, rp, stream);
    return e == hipSuccess ? KDA_OK : KDA_ERR_HIP;
}

}  // namespace

extern "C" {

int kda_chunk_summary(const kda_fwd_args* a, float* transition, hipStream_t stream) {
    if (!a) return KDA_ERR_NULL;
    int c;
    int64_t nc, cb, need;
    int st = check_shape(a, &c, &nc, &cb, &need);
    if (st != KDA_OK) return st;
    if (a->flags & ~(KDA_FLAG_NO_CLAMP | kPrepFlags)) return KDA_ERR_UNSUPPORTED;
    const int64_t units = a->B * a->H;
    if (!aligned16(a->q)) return KDA_ERR_ALIGN;
    if (units == 0) return KDA_OK;
    if (units * (a->Dk / 16) > INT_MAX) return KDA_ERR_SHAPE;  // combine-style grids
    if (!transition || !a->final_state) return KDA_ERR_NULL;
    if (!aligned16(transition) || !aligned16(a->final_state)) return KDA_ERR_ALIGN;
    const int D = (int)a->Dk;
    if (a->T == 0) {
        const hipError_t e = kda::launch_identity_summary(D, transition, a->final_state, units, stream);
        return e == hipSuccess ? KDA_OK : KDA_ERR_HIP;
    }
    const void* req[] = {a->k, a->v, a->log_alpha, a->beta};
    for (const void* p : req)
        if (!p) return KDA_ERR_NULL;
    for (const void* p : req)
        if (!aligned16(p)) return KDA_ERR_ALIGN;
    const int64_t cards = units * nc * cb;  // only the cards: no segment-scan summaries here
    if (!a->workspace || (int64_t)a->workspace_bytes < cards) return KDA_ERR_WORKSPACE;
    if (!aligned16(a->workspace)) return KDA_ERR_ALIGN;
    // the card builder also forms the query-side blocks of each card, which the summary
    // never reads: without q, k stands in for it (and the cards serve the summary only)
    kda::PrepParams pp{a->q ? a->q : a->k, a->k, a->v, a->log_alpha, a->beta, a->workspace,
                       a->B, a->T, a->H, nc, (a->flags & KDA_FLAG_NO_CLAMP) ? 0 : 1,
                       (a->flags & KDA_FLAG_QK_L2NORM) ? 1 : 0, (a->flags & KDA_FLAG_GATE_LOGITS) ? 1 : 0};
    const hipError_t e = kda::launch_summary(a->dtype == KDA_BF16, c, D, pp, transition, a->final_state, stream);
    return e == hipSuccess ? KDA_OK : KDA_ERR_HIP;
}

int kda_combine_states(const kda_combine_args* a, hipStream_t stream) {
    if (!a) return KDA_ERR_NULL;
    if (a->P < 0 || a->B < 0 || a->H < 0 || a->Dk <= 0 || a->Dv <= 0) return KDA_ERR_SHAPE;
    if (a->Dk != a->Dv || (a->Dk != 64 && a->Dk != 128)) return KDA_ERR_UNSUPPORTED;
    int64_t bh, st, pst;
    if (!mul_ok(a->B, a->H, &bh) || !mul_ok(bh, a->Dk * a->Dv, &st) || !mul_ok(st, a->P, &pst))
        return KDA_ERR_SHAPE;
    if (bh * (a->Dk / 16) > INT_MAX) return KDA_ERR_SHAPE;  // one workgroup per (b, h, 16 columns)
    if (bh == 0) return KDA_OK;
    if (a->P > 0 && (!a->transition || !a->offset)) return KDA_ERR_NULL;
    const void* ptrs[] = {a->transition, a->offset, a->initial_state, a->segment_states, a->final_state};
    for (const void* p : ptrs)
        if (!aligned16(p)) return KDA_ERR_ALIGN;
    if (!a->segment_states && !a->final_state) return KDA_OK;
    kda::CombineParams p{a->transition, a->offset, a->initial_state, a->segment_states, a->final_state,
                         a->P, bh};
    const hipError_t e = kda::launch_combine((int)a->Dk, p, stream);
    return e == hipSuccess ? KDA_OK : KDA_ERR_HIP;
}

int kda_chunk_bwd_workspace_size(const kda_bwd_args* a, size_t* bytes) {
    if (!a || !bytes) return KDA_ERR_NULL;
    int64_t nc, ws;
    const int st = check_bwd(a, &nc, &ws);
    if (st != KDA_OK) return st;
    *bytes = (size_t)ws;
    return KDA_OK;
}

int kda_chunk_bwd(const kda_bwd_args* a, hipStream_t stream) {
    if (!a) return KDA_ERR_NULL;
    int64_t nc, need;
    const int st = check_bwd(a, &nc, &need);
    if (st != KDA_OK) return st;
    const bool has_tokens = a->B * a->T * a->H > 0;
    if (has_tokens) {
        const void* req[] = {a->q, a->k, a->v, a->log_alpha, a->beta, a->gate, a->d_out,
                             a->dq, a->dk, a->dv, a->dlog_alpha, a->dbeta, a->dgate};
        for (const void* p : req)
            if (!p) return KDA_ERR_NULL;
        for (const void* p : req)
            if (!aligned16(p)) return KDA_ERR_ALIGN;
    }
    if (!aligned16(a->initial_state) || !aligned16(a->d_final_state) || !aligned16(a->d_initial_state))
        return KDA_ERR_ALIGN;
    if (need > 0) {
        if (!a->workspace) return KDA_ERR_WORKSPACE;
        if ((int64_t)a->workspace_bytes < need) return KDA_ERR_WORKSPACE;
        if (!aligned16(a->workspace)) return KDA_ERR_ALIGN;
    }
    if (a->B * a->H == 0) return KDA_OK;
    if (!has_tokens && !a->d_initial_state) return KDA_OK;
    kda::BwdParams p{a->q, a->k, a->v, a->log_alpha, a->beta, a->gate, a->d_out,
                     a->initial_state, a->d_final_state, a->dq, a->dk, a->dv, a->dlog_alpha,
                     a->dbeta, a->dgate, a->d_initial_state};
    p.B = a->B;
    p.T = a->T;
    p.H = a->H;
    p.NC = nc;
    p.clamp = (a->flags & KDA_FLAG_NO_CLAMP) ? 0 : 1;
    p.qk_norm = (a->flags & KDA_FLAG_QK_L2NORM) ? 1 : 0;
    p.logits = (a->flags & KDA_FLAG_GATE_LOGITS) ? 1 : 0;
    kda::bwd_layout((int)a->Dk, a->B * a->H, nc, a->workspace, p);
    const hipError_t e = kda::launch_bwd(a->dtype == KDA_BF16, (int)a->Dk, p, stream);
    return e == hipSuccess ? KDA_OK : KDA_ERR_HIP;
}

int kda_chunk_bwd_varlen_workspace_size(const kda_bwd_varlen_args* a, size_t* bytes) {
    if (!a || !bytes) return KDA_ERR_NULL;
    BwdVarlenLayout L;
    const int st = check_bwd_varlen(a, &L);
    if (st != KDA_OK) return st;
    *bytes = (size_t)L.total;
    return KDA_OK;
}

int kda_chunk_bwd_varlen(const kda_bwd_varlen_args* a, hipStream_t stream) {
    BwdVarlenLayout L;
    const int st = check_bwd_varlen(a, &L);
    if (st != KDA_OK) return st;
    if (a->N == 0 || a->H == 0) return KDA_OK;
    if (!a->cu_seqlens) return KDA_ERR_NULL;
    if ((reinterpret_cast<uintptr_t>(a->cu_seqlens) & 7u) != 0) return KDA_ERR_ALIGN;
    const bool has_rows = a->rows > 0;
    if (has_rows) {
        const void* req[] = {a->q, a->k, a->v, a->log_alpha, a->beta, a->gate, a->d_out,
                             a->dq, a->dk, a->dv, a->dlog_alpha, a->dbeta, a->dgate};
        for (const void* p : req)
            if (!p) return KDA_ERR_NULL;
        for (const void* p : req)
            if (!aligned16(p)) return KDA_ERR_ALIGN;
    }
    if (!aligned16(a->initial_state) || !aligned16(a->d_final_state) || !aligned16(a->d_initial_state))
        return KDA_ERR_ALIGN;
    if (!has_rows && !a->d_initial_state) return KDA_OK;
    if (!a->workspace || (int64_t)a->workspace_bytes < L.total) return KDA_ERR_WORKSPACE;
    if (!aligned16(a->workspace)) return KDA_ERR_ALIGN;
    unsigned char* ws = static_cast<unsigned char*>(a->workspace);
    kda::VarlenMap m{reinterpret_cast<int64_t*>(ws + L.off_s), reinterpret_cast<int64_t*>(ws + L.off_co),
                     reinterpret_cast<int32_t*>(ws + L.off_soc)};
    hipError_t e = kda::launch_varlen_map(m, a->cu_seqlens, a->N, a->rows, 64, stream);
    if (e != hipSuccess) return KDA_ERR_HIP;
    kda::BwdParams p{a->q, a->k, a->v, a->log_alpha, a->beta, a->gate, a->d_out,
                     a->initial_state, a->d_final_state, a->dq, a->dk, a->dv, a->dlog_alpha,
                     a->dbeta, a->dgate, a->d_initial_state};
    p.B = a->N;
    p.T = a->rows;
    p.H = a->H;
    p.NC = L.max_chunks;
    p.vs = m.s;
    p.vco = m.co;
    p.vsoc = m.soc;
    p.clamp = (a->flags & KDA_FLAG_NO_CLAMP) ? 0 : 1;
    p.qk_norm = (a->flags & KDA_FLAG_QK_L2NORM) ? 1 : 0;
    p.logits = (a->flags & KDA_FLAG_GATE_LOGITS) ? 1 : 0;
    kda::bwd_layout((int)a->Dk, a->H, L.max_chunks, a->workspace, p);
    e = kda::launch_bwd(a->dtype == KDA_BF16, (int)a->Dk, p, stream);
    return e == hipSuccess ? KDA_OK : KDA_ERR_HIP;
}

int kda_decode_step(const kda_decode_args* a, hipStream_t stream) {
    if (!a) return KDA_ERR_NULL;
    if (a->B < 0 || a->H < 0 || a->Dk <= 0 || a->Dv <= 0) return KDA_ERR_SHAPE;
    if (a->dtype != KDA_F32 && a->dtype != KDA_BF16) return KDA_ERR_UNSUPPORTED;
    if (a->Dk != a->Dv || (a->Dk != 64 && a->Dk != 128)) return KDA_ERR_UNSUPPORTED;
    if (a->out_dtype != KDA_F32 && a->out_dtype != KDA_BF16) return KDA_ERR_UNSUPPORTED;
    if ((a->flags & ~(KDA_FLAG_NO_CLAMP | kPrepFlags)) != 0 || a->reserved != 0) return KDA_ERR_UNSUPPORTED;
    int64_t bh, st;
    if (!mul_ok(a->B, a->H, &bh) || !mul_ok(bh, a->Dk * a->Dv, &st)) return KDA_ERR_SHAPE;
    if (bh > INT_MAX) return KDA_ERR_SHAPE;
    if (bh == 0) return KDA_OK;
    const void* req[] = {a->q, a->k, a->v, a->log_alpha, a->beta, a->gate, a->out, a->state};
    for (const void* p : req)
        if (!p) return KDA_ERR_NULL;
    for (const void* p : req)
        if (!aligned16(p)) return KDA_ERR_ALIGN;
    kda::DecodeParams p{a->q, a->k, a->v, a->log_alpha, a->beta, a->gate, a->out, a->state,
                        bh, (a->flags & KDA_FLAG_NO_CLAMP) ? 0 : 1, (a->flags & KDA_FLAG_QK_L2NORM) ? 1 : 0,
                        (a->flags & KDA_FLAG_GATE_LOGITS) ? 1 : 0};
    const hipError_t e =
        kda::launch_decode(a->dtype == KDA_BF16, a->out_dtype == KDA_BF16, (int)a->Dk, p, stream);
    return e == hipSuccess ? KDA_OK : KDA_ERR_HIP;
}

}  // extern "C"
