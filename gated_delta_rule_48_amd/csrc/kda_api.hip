// kda_api.hip -- the C ABI of libkda (see include/kda.h): argument validation,
// workspace layout and kernel dispatch. Host code only; it never synchronises.

#include <math.h>

#include <algorithm>
#include <mutex>
#include <stdint.h>

#include "../../include/kda.h"
#include "kda_internal.hpp"
#include "kda_attn.hpp"
#include "kda_bwd.hpp"

#define KDA_EXPORT extern "C" __attribute__((visibility("default")))

static_assert(KDA_GATE_CHANNEL == kda::kGateChannel && KDA_GATE_HEAD == kda::kGateHead &&
                  KDA_GATE_NONE == kda::kGateNone,
              "gate kinds of the ABI and the kernels");

namespace {

using kda::ChunkBuffers;

bool supported_dim(int d) { return d == 64 || d == 128; }
bool aligned(const void *p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }
size_t round_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

// [lo, lo + bytes) ranges overlap?
bool overlaps(const void *a, size_t na, const void *b, size_t nb) {
    if (!a || !b || na == 0 || nb == 0) return false;
    const uintptr_t x = reinterpret_cast<uintptr_t>(a), y = reinterpret_cast<uintptr_t>(b);
    return x < y + nb && y < x + na;
}

// The fused pass (the state of a (sequence, head) in one workgroup's registers,
// nothing staged in memory, 64-row chunks) serves bf16 input with d_k = d_v = 128,
// for equal-length and for packed sequences, whatever chunk size is asked (chunking
// is an exact refactoring of the recurrence: 64 and 128 give the same results up to
// rounding). When the (sequence, head) pairs alone fill the chip it runs one
// workgroup per pair. Otherwise it cuts the sequences into segments and runs one
// workgroup per (segment, head) in two launches of at most one workgroup per compute
// unit: segment 0 of every sequence with its outputs and the maps S_out = M S_in + N
// of the middle segments, then (after the maps' composition) the other segments from
// their entering states. Other inputs (fp32, d = 64) take the split pass (parallel
// chunk preparation, then state propagation over d_v slices) at the asked chunk size.
constexpr int kFusedMinPairs = 256;
constexpr int kComputeUnits = 256;  // MI355X
bool use_fused(int B, int T, int H, int dk, int dv, int C, bool varlen, int io, int n_seqs) {
    (void)B;
    (void)H;
    (void)C;
    (void)varlen;
    (void)n_seqs;
    return io == KDA_BF16 && dk == 128 && dv == 128 && T > 0;
}

struct FusedPlan {
    int u;      // units per head in each of the two launches (0: no segments)
    int T;      // equal-length sequences: the budget (chunks per unit)
    int P;      // equal-length sequences: segments of each
    int slots;  // segment slots per head (entering states and maps): at least launch C's units
};

// Below 256 (sequence, head) pairs the pass runs on the plan (kda_internal.hpp): per head u =
// 256 / H units in each of two launches. For packed sequences the device works out the plan
// from the offsets (kda_seg_plan_kernel); for B equal sequences of c chunks the host does: from
// the smallest budget T for which B plan_units_a(c, T) <= u, the budget of plan_budget. Both
// launches then take about T chunk-steps (the 4 packed sequences of 32,768 + 16,384 + 12,288 +
// 4,096 tokens x 32 heads: T = 103 of their 1,024 chunks per head, 8 units in launch A and 7 in
// launch C; 1 x 4,096 tokens x 16 heads: T = 4, 15 units each). Sequences of fewer than
// kMinSegChunks chunks are not cut (T = the longest: one unit per sequence): below that the
// composition and the second launch cost about what the segments save. Either way the usual
// body runs in the same kernel, so equal-length and packed layouts of the same sequences agree
// bit for bit.
FusedPlan fused_plan(int B, int T, int H, bool varlen, int n_seqs) {
    const int64_t pairs = (int64_t)(varlen ? n_seqs : B) * H;
    if (pairs >= kFusedMinPairs || T <= 0) return FusedPlan{0, 0, 0, 0};
    const int u = kComputeUnits / H;  // (>= the number of sequences: fewer than 256 pairs)
    const int64_t c = ((int64_t)T + 63) / 64;  // chunks of one sequence, or at most of a packed one
    // (launch C's units have a chunk each at least: no more than the chunks of all sequences)
    if (varlen) return FusedPlan{u, 0, 0, (int)std::min<int64_t>(u, c + n_seqs)};
    int lo = 1, hi = (int)c;
    if (c < kda::kMinSegChunks) lo = hi;
    while (lo < hi) {
        const int mid = (lo + hi) / 2;
        if ((int64_t)B * kda::plan_units_a((int)c, mid) <= u) hi = mid; else lo = mid + 1;
    }
    const int T_b = kda::plan_budget((int)c, lo);
    const int P = kda::plan_segments((int)c, T_b);
    return FusedPlan{u, T_b, P, B * (P - 1)};
}

struct WsLayout {
    size_t W, U, QO, KtT, Aqk, eg, strong, discard, choff, total;
    size_t seg_tab, seg_state, seg_map;  // fused pass with segments
    int64_t n_chunks;  // upper bound on the number of chunks over all sequences
};

// Workspace layout: per-chunk buffers (chunk-major, see ChunkBuffers) and, for
// packed variable-length input, the chunk offsets of the sequences.
bool ws_layout(int B, int T, int H, int dk, int dv, int C, int n_seqs, bool varlen, int io,
               WsLayout *L) {
    *L = WsLayout{};
    if (T <= 0) return true;
    size_t off = 0;
    auto take = [&](size_t bytes) {
        const size_t at = off;
        off = round_up(off + bytes, 256);
        return at;
    };
    if (use_fused(B, T, H, dk, dv, C, varlen, io, n_seqs)) {
        // the discard slot; one byte per (sequence or segment, head): left to the strong-decay
        // instance; with segments, their table, entering states and maps (fp32, 64 KB each)
        const FusedPlan fp = fused_plan(B, T, H, varlen, n_seqs);
        const size_t slots = (size_t)fp.slots * H;
        L->discard = take(256);
        L->strong = take(fp.u > 0 ? (size_t)2 * fp.u * H : (size_t)(varlen ? n_seqs : B) * H);
        if (fp.u > 0) {
            L->seg_tab = varlen ? take((size_t)kda::PlanTab::ints(n_seqs) * sizeof(int32_t)) : 0;
            L->seg_state = take(slots * dk * dv * sizeof(float));
            L->seg_map = take(slots * 2 * dk * dv * sizeof(float));
        }
        L->total = off;
        return true;
    }
    const size_t esz = io == KDA_BF16 ? 2 : 4;
    const int64_t per_seq = ((int64_t)T + C - 1) / C;
    L->n_chunks = varlen ? per_seq + n_seqs : (int64_t)B * per_seq;
    const size_t nch = (size_t)L->n_chunks * (size_t)H;
    L->W = take(nch * C * dk * esz);
    L->U = take(nch * C * dv * esz);
    L->QO = take(nch * C * dk * esz);
    L->KtT = take(nch * dk * C * esz);
    L->Aqk = take(nch * C * C * esz);
    L->eg = take(nch * dk * sizeof(float));
    L->strong = take(nch);  // one byte per (chunk, head)
    L->discard = take(256);  // absorbs stores of rows past a sequence's end
    // chunk offsets [n_seqs + 1], then sequence begins and ends [n_seqs] each
    L->choff = varlen ? take(((size_t)3 * n_seqs + 1) * sizeof(int32_t)) : 0;
    L->total = off;
    return true;
}

kda_status check_sizes(int B, int T, int H, int dk, int dv, int chunk, int io, bool varlen,
                       int n_seqs) {
    if (io != KDA_F32 && io != KDA_BF16) return KDA_ERR_UNSUPPORTED;
    if (B < 1 || T < 0 || H < 1) return KDA_ERR_INVALID_ARG;
    if (varlen && (B != 1 || n_seqs < 1)) return KDA_ERR_INVALID_ARG;
    if (!supported_dim(dk) || !supported_dim(dv)) return KDA_ERR_UNSUPPORTED;
    if (chunk != 64 && chunk != 128) return KDA_ERR_UNSUPPORTED;
    if (H > 65535) return KDA_ERR_UNSUPPORTED;  // grid y limit of the prep kernel
    const int64_t tokens = (int64_t)B * T;
    if (tokens > INT32_MAX) return KDA_ERR_UNSUPPORTED;
    const int64_t nseq = varlen ? n_seqs : B;
    if (nseq * H * 4 > INT32_MAX) return KDA_ERR_UNSUPPORTED;
    return KDA_OK;
}

}  // namespace

KDA_EXPORT int kda_abi_version(void) { return KDA_ABI_VERSION; }

KDA_EXPORT const char *kda_status_string(int status) {
    switch (status) {
        case KDA_OK: return "ok";
        case KDA_ERR_INVALID_ARG: return "invalid argument";
        case KDA_ERR_UNSUPPORTED: return "unsupported size or dtype";
        case KDA_ERR_WORKSPACE: return "workspace missing, misaligned or too small";
        case KDA_ERR_HIP: return "HIP launch failed";
        default: return "unknown status";
    }
}

KDA_EXPORT size_t kda_chunk_fwd_workspace_bytes(int B, int T, int H, int d_k, int d_v, int chunk,
                                                int n_seqs, int io) {
    const bool varlen = n_seqs > 0 && B == 1;
    if (check_sizes(B, T, H, d_k, d_v, chunk, io, varlen, varlen ? n_seqs : 0) != KDA_OK) return 0;
    WsLayout L;
    ws_layout(B, T, H, d_k, d_v, chunk, varlen ? n_seqs : 0, varlen, io, &L);
    return L.total;
}

// ---------------------------------------------------------------- the workspace of kda_chunk_fwd_noalloc
//
// A fixed device array that takes the place of the caller's workspace. Each GPU the
// library runs on holds its own copy until the process ends. In host code `scratch`
// names a host-side stand-in, not the array's device address, so host code never
// uses it directly: the address is looked up once per device (with that device
// current) and kept in scratch_dev; kernels receive that pointer. Calls on one GPU
// share the array, so calls that overlap in time on one GPU race (the workspace of
// kda_chunk_fwd is caller-owned instead). Nothing in the chunked passes' workspace
// has to start at zero: every byte a kernel reads was written earlier in the same call.
static __device__ __align__(256) unsigned char scratch[KDA_NOALLOC_MAX_WORKSPACE];

namespace {

constexpr int kMaxDevices = 64;
std::mutex scratch_mu;
void *scratch_dev[kMaxDevices] = {};

// The current device's address of `scratch` (looked up on the first call per device).
hipError_t scratch_address(void **out) {
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(scratch_mu);
    if (!scratch_dev[dev]) {
        void *p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return e;
        if (!p) return hipErrorInvalidSymbol;
        scratch_dev[dev] = p;
    }
    *out = scratch_dev[dev];
    return hipSuccess;
}

}  // namespace

namespace {

// kda_chunk_fwd_gated (gate = a kda_gate value) and kda_chunk_fwd_preact (gate =
// kda::kGatePreact, pre = its pre-activations; log_alpha unused, beta = b). With
// use_scratch (kda_chunk_fwd_noalloc) the workspace is the device array `scratch`,
// looked up once every argument has been validated.
int chunk_fwd_impl(int gate, const kda::PreactArgs &pre, int B, int T, int H, int d_k, int d_v, int chunk, int io,
                   const void *q, const void *k, const void *v, const float *log_alpha, const float *beta,
                   float scale, const float *h0, const int32_t *cu_seqlens, int n_seqs, void *o, float *hT,
                   void *workspace, size_t workspace_bytes, void *stream, bool use_scratch = false) {
    const bool varlen = cu_seqlens != nullptr;
    kda_status st = check_sizes(B, T, H, d_k, d_v, chunk, io, varlen, n_seqs);
    if (st != KDA_OK) return st;
    if (!isfinite(scale)) return KDA_ERR_INVALID_ARG;
    const int nseq = varlen ? n_seqs : B;
    const size_t tokens = (size_t)B * T;
    const size_t esz = io == KDA_BF16 ? 2 : 4;
    if (tokens > 0) {
        if (!q || !k || !v || !beta || !o) return KDA_ERR_INVALID_ARG;
        if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(o, 16) || !aligned(beta, 4))
            return KDA_ERR_INVALID_ARG;
        const size_t ob = tokens * H * d_v * esz;
        if (overlaps(o, ob, q, tokens * H * d_k * esz) || overlaps(o, ob, k, tokens * H * d_k * esz) ||
            overlaps(o, ob, v, ob) || overlaps(o, ob, beta, tokens * H * 4))
            return KDA_ERR_INVALID_ARG;
        if (gate == kda::kGatePreact) {
            if (!pre.a || !pre.A_log || !pre.dt_bias || !aligned(pre.a, 16) || !aligned(pre.A_log, 4) ||
                !aligned(pre.dt_bias, 16) || overlaps(o, ob, pre.a, tokens * H * d_k * esz) ||
                overlaps(o, ob, pre.A_log, (size_t)H * 4) || overlaps(o, ob, pre.dt_bias, (size_t)H * d_k * 4))
                return KDA_ERR_INVALID_ARG;
        } else if (gate != KDA_GATE_NONE) {
            const size_t gb = tokens * H * (gate == KDA_GATE_CHANNEL ? (size_t)d_k : 1) * 4;
            if (!log_alpha || !aligned(log_alpha, gate == KDA_GATE_CHANNEL ? 16 : 4) || overlaps(o, ob, log_alpha, gb))
                return KDA_ERR_INVALID_ARG;
        }
    }
    if (gate == KDA_GATE_NONE || gate == kda::kGatePreact) log_alpha = nullptr;  // never read
    if ((h0 && !aligned(h0, 16)) || (hT && !aligned(hT, 16))) return KDA_ERR_INVALID_ARG;
    if (varlen && !aligned(cu_seqlens, 4)) return KDA_ERR_INVALID_ARG;

    WsLayout L;
    ws_layout(B, T, H, d_k, d_v, chunk, varlen ? n_seqs : 0, varlen, io, &L);
    if (use_scratch) {
        if (L.total > KDA_NOALLOC_MAX_WORKSPACE) return KDA_ERR_WORKSPACE;
        workspace = nullptr;
        workspace_bytes = 0;
        if (L.total > 0) {
            if (scratch_address(&workspace) != hipSuccess) return KDA_ERR_HIP;
            workspace_bytes = KDA_NOALLOC_MAX_WORKSPACE;
        }
    }
    if (L.total > 0 && (!workspace || !aligned(workspace, 256) || workspace_bytes < L.total))
        return KDA_ERR_WORKSPACE;

    hipStream_t hs = reinterpret_cast<hipStream_t>(stream);
    char *ws = static_cast<char *>(workspace);
    const bool bf = io == KDA_BF16;
    if (use_fused(B, T, H, d_k, d_v, chunk, varlen, io, n_seqs)) {
        const FusedPlan fp = fused_plan(B, T, H, varlen, n_seqs);
        kda::FusedArgs fa{q,  k,     v,  log_alpha, beta, scale, h0, hT,   o, ws + L.discard, H,
                          T,  varlen ? cu_seqlens : nullptr, (int)tokens, gate, pre,
                          reinterpret_cast<uint8_t *>(ws + L.strong)};
        fa.n_seqs = nseq;
        fa.plan_u = fp.u;
        fa.plan_T = fp.T;
        fa.plan_P = fp.P;
        if (fp.u > 0) {
            fa.seg_state = reinterpret_cast<float *>(ws + L.seg_state);
            fa.seg_map = reinterpret_cast<float *>(ws + L.seg_map);
            if (varlen) {
                int32_t *tab = reinterpret_cast<int32_t *>(ws + L.seg_tab);
                fa.plan_tab = tab;
                if (kda::launch_seg_plan(cu_seqlens, n_seqs, (int)tokens, fp.u, tab, hs) != hipSuccess)
                    return KDA_ERR_HIP;
            }
        }
        return kda::launch_fused(fa, d_k, d_v, bf, nseq, hs) == hipSuccess ? KDA_OK : KDA_ERR_HIP;
    }
    ChunkBuffers buf{};
    if (L.total > 0) {
        buf = ChunkBuffers{ws + L.W, ws + L.U, ws + L.QO, ws + L.KtT, ws + L.Aqk,
                           reinterpret_cast<float *>(ws + L.eg), reinterpret_cast<uint8_t *>(ws + L.strong)};
    }

    kda::SeqMap map{};
    map.C = chunk;
    map.n_seqs = nseq;
    if (varlen && tokens > 0) {
        int32_t *off = reinterpret_cast<int32_t *>(ws + L.choff);
        map.varlen = 1;
        map.chunk_off = off;
        map.seq_begin = off + n_seqs + 1;
        map.seq_end = off + 2 * n_seqs + 1;
        map.seq_len = 0;
        if (kda::launch_chunk_offsets(cu_seqlens, n_seqs, (int)tokens, chunk, off, off + n_seqs + 1,
                                      off + 2 * n_seqs + 1, hs) != hipSuccess)
            return KDA_ERR_HIP;
    } else {  // B equal sequences (or no tokens at all: every sequence is empty)
        map.varlen = 0;
        map.seq_len = tokens > 0 ? T : 0;
    }

    if (tokens > 0) {
        kda::PrepArgs pa{q, k, v, log_alpha, beta, scale, H, gate, pre, map, buf};
        if (kda::launch_prep(pa, chunk, d_k, d_v, bf, (int)L.n_chunks, hs) != hipSuccess)
            return KDA_ERR_HIP;
    }
    kda::StateArgs sa{h0, hT, o, L.total > 0 ? ws + L.discard : nullptr, H, 0, map, buf};
    if (kda::launch_state(sa, chunk, d_k, d_v, bf, nseq, hs) != hipSuccess) return KDA_ERR_HIP;
    return KDA_OK;
}

int recurrent_step_impl(int gate, const kda::PreactArgs &pre, int N, int H, int d_k, int d_v, int io,
                        const void *q, const void *k, const void *v, const float *log_alpha,
                        const float *beta, float scale, float *state, void *o, void *stream);

}  // namespace


KDA_EXPORT int kda_chunk_fwd_gated(int gate, int B, int T, int H, int d_k, int d_v, int chunk, int io,
                                   const void *q, const void *k, const void *v,
                                   const float *log_alpha, const float *beta, float scale,
                                   const float *h0, const int32_t *cu_seqlens, int n_seqs,
                                   void *o, float *hT, void *workspace, size_t workspace_bytes,
                                   void *stream) {
    if (gate != KDA_GATE_CHANNEL && gate != KDA_GATE_HEAD && gate != KDA_GATE_NONE) return KDA_ERR_INVALID_ARG;
    return chunk_fwd_impl(gate, kda::PreactArgs{}, B, T, H, d_k, d_v, chunk, io, q, k, v, log_alpha, beta, scale,
                          h0, cu_seqlens, n_seqs, o, hT, workspace, workspace_bytes, stream);
}

KDA_EXPORT int kda_chunk_fwd_preact(int flags, int B, int T, int H, int d_k, int d_v, int chunk, int io,
                                    const void *q, const void *k, const void *v,
                                    const void *a, const float *A_log, const float *dt_bias, const float *b,
                                    float scale, const float *h0, const int32_t *cu_seqlens, int n_seqs,
                                    void *o, float *hT, void *workspace, size_t workspace_bytes, void *stream) {
    if (flags & ~KDA_PREACT_QK_NORM) return KDA_ERR_INVALID_ARG;
    const kda::PreactArgs pre{a, A_log, dt_bias, (flags & KDA_PREACT_QK_NORM) ? 1 : 0};
    return chunk_fwd_impl(kda::kGatePreact, pre, B, T, H, d_k, d_v, chunk, io, q,
                          k, v, nullptr, b, scale, h0, cu_seqlens, n_seqs, o, hT, workspace, workspace_bytes,
                          stream);
}

KDA_EXPORT int kda_chunk_fwd_noalloc(int gate, int B, int T, int H, int d_k, int d_v, int chunk, int io,
                                     const void *q, const void *k, const void *v,
                                     const float *log_alpha, const float *beta, float scale,
                                     const float *h0, const int32_t *cu_seqlens, int n_seqs,
                                     void *o, float *hT, void *stream) {
    if (gate != KDA_GATE_CHANNEL && gate != KDA_GATE_HEAD && gate != KDA_GATE_NONE) return KDA_ERR_INVALID_ARG;
    return chunk_fwd_impl(gate, kda::PreactArgs{}, B, T, H, d_k, d_v, chunk, io, q, k, v, log_alpha, beta, scale,
                          h0, cu_seqlens, n_seqs, o, hT, nullptr, 0, stream, true);
}

KDA_EXPORT int kda_chunk_fwd(int B, int T, int H, int d_k, int d_v, int chunk, int io,
                             const void *q, const void *k, const void *v,
                             const float *log_alpha, const float *beta, float scale,
                             const float *h0, const int32_t *cu_seqlens, int n_seqs,
                             void *o, float *hT, void *workspace, size_t workspace_bytes,
                             void *stream) {
    return kda_chunk_fwd_gated(KDA_GATE_CHANNEL, B, T, H, d_k, d_v, chunk, io, q, k, v, log_alpha, beta, scale,
                               h0, cu_seqlens, n_seqs, o, hT, workspace, workspace_bytes, stream);
}

namespace {

int recurrent_step_impl(int gate, const kda::PreactArgs &pre, int N, int H, int d_k, int d_v, int io,
                        const void *q, const void *k, const void *v, const float *log_alpha,
                        const float *beta, float scale, float *state, void *o, void *stream) {
    if (io != KDA_F32 && io != KDA_BF16) return KDA_ERR_UNSUPPORTED;
    if (N < 0 || H < 1) return KDA_ERR_INVALID_ARG;
    if (!supported_dim(d_k) || !supported_dim(d_v)) return KDA_ERR_UNSUPPORTED;
    if ((int64_t)N * H > INT32_MAX) return KDA_ERR_UNSUPPORTED;
    if (!isfinite(scale)) return KDA_ERR_INVALID_ARG;
    if (N == 0) return KDA_OK;
    if (!q || !k || !v || !beta || !state || !o) return KDA_ERR_INVALID_ARG;
    if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(o, 16) || !aligned(beta, 4) ||
        !aligned(state, 16))
        return KDA_ERR_INVALID_ARG;
    if (gate == kda::kGatePreact) {
        if (!pre.a || !pre.A_log || !pre.dt_bias || !aligned(pre.a, 16) || !aligned(pre.A_log, 4) ||
            !aligned(pre.dt_bias, 16))
            return KDA_ERR_INVALID_ARG;
    } else if (gate != KDA_GATE_NONE && (!log_alpha || !aligned(log_alpha, gate == KDA_GATE_CHANNEL ? 16 : 4))) {
        return KDA_ERR_INVALID_ARG;
    }
    if (gate == KDA_GATE_NONE || gate == kda::kGatePreact) log_alpha = nullptr;  // never read
    const size_t nh = (size_t)N * H, esz = io == KDA_BF16 ? 2 : 4;
    if (overlaps(o, nh * d_v * esz, state, nh * d_k * d_v * 4)) return KDA_ERR_INVALID_ARG;
    kda::DecodeArgs da{q, k, v, log_alpha, beta, scale, state, o, (int)nh, gate, H, pre};
    if (kda::launch_decode(da, d_k, d_v, io == KDA_BF16, reinterpret_cast<hipStream_t>(stream)) !=
        hipSuccess)
        return KDA_ERR_HIP;
    return KDA_OK;
}

}  // namespace

KDA_EXPORT int kda_recurrent_step_gated(int gate, int N, int H, int d_k, int d_v, int io,
                                        const void *q, const void *k, const void *v,
                                        const float *log_alpha, const float *beta, float scale,
                                        float *state, void *o, void *stream) {
    if (gate != KDA_GATE_CHANNEL && gate != KDA_GATE_HEAD && gate != KDA_GATE_NONE) return KDA_ERR_INVALID_ARG;
    return recurrent_step_impl(gate, kda::PreactArgs{}, N, H, d_k, d_v, io, q, k, v, log_alpha, beta, scale, state,
                               o, stream);
}

KDA_EXPORT int kda_recurrent_step_preact(int flags, int N, int H, int d_k, int d_v, int io,
                                         const void *q, const void *k, const void *v,
                                         const void *a, const float *A_log, const float *dt_bias, const float *b,
                                         float scale, float *state, void *o, void *stream) {
    if (flags & ~KDA_PREACT_QK_NORM) return KDA_ERR_INVALID_ARG;
    const kda::PreactArgs pre{a, A_log, dt_bias, (flags & KDA_PREACT_QK_NORM) ? 1 : 0};
    return recurrent_step_impl(kda::kGatePreact, pre, N, H, d_k, d_v, io, q, k, v,
                               nullptr, b, scale, state, o, stream);
}

KDA_EXPORT int kda_recurrent_step(int N, int H, int d_k, int d_v, int io,
                                  const void *q, const void *k, const void *v,
                                  const float *log_alpha, const float *beta, float scale,
                                  float *state, void *o, void *stream) {
    return kda_recurrent_step_gated(KDA_GATE_CHANNEL, N, H, d_k, d_v, io, q, k, v, log_alpha, beta, scale,
                                    state, o, stream);
}

namespace {

// Splits of the attention decode's cache: enough workgroups to fill the chip
// several times over, each over at least kAttnMinSplit rows (its fixed costs are
// the query, one merge and one partial write), in whole iterations.
constexpr int64_t kAttnTargetGroups = kda::kAttnMaxSplits;  // so no cached head takes more splits
constexpr int64_t kAttnMinSplit = 1024;

struct AttnSplit {
    int n, len;
};

AttnSplit attn_split(int B, int H_kv, int D, int T_max) {
    const int64_t rows = kda::attn_rows_per_iter(D);
    if (T_max <= 0) return {1, (int)rows};
    const int64_t units = (int64_t)B * H_kv;
    int64_t n = (kAttnTargetGroups + units - 1) / units;
    n = std::min<int64_t>(n, std::max<int64_t>(1, T_max / kAttnMinSplit));
    n = std::max<int64_t>(n, 1);
    const int64_t L = ((T_max + n - 1) / n + rows - 1) / rows * rows;
    return {(int)((T_max + L - 1) / L), (int)L};
}

int check_attn(int B, int H, int H_kv, int d, int T_max, int io) {
    if (io != KDA_F32 && io != KDA_BF16) return KDA_ERR_UNSUPPORTED;
    if (B < 0 || H < 1 || H_kv < 1 || T_max < 0 || H % H_kv != 0) return KDA_ERR_INVALID_ARG;
    const int G = H / H_kv;
    if (!supported_dim(d) || (G != 1 && G != 2 && G != 4 && G != 8)) return KDA_ERR_UNSUPPORTED;
    // grid limits, and 32-bit row offsets within one cached head
    if (B > 65535 || H_kv > 65535 || (int64_t)T_max * d > INT32_MAX) return KDA_ERR_UNSUPPORTED;
    return KDA_OK;
}

size_t attn_ws_bytes(int B, int H, int d, const AttnSplit &sp, size_t *ml_off) {
    if (sp.n <= 1) {
        *ml_off = 0;
        return 0;
    }
    const size_t n = (size_t)B * H * sp.n;
    *ml_off = round_up(n * d * sizeof(float), 256);
    return *ml_off + round_up(n * 2 * sizeof(float), 256);
}

}  // namespace

KDA_EXPORT size_t kda_attn_decode_workspace_bytes(int B, int H, int H_kv, int d, int T_max, int io) {
    if (check_attn(B, H, H_kv, d, T_max, io) != KDA_OK || B == 0) return 0;
    size_t ml_off;
    return attn_ws_bytes(B, H, d, attn_split(B, H_kv, d, T_max), &ml_off);
}

KDA_EXPORT int kda_attn_decode(int B, int H, int H_kv, int d, int T_max, int io, const void *q,
                               const void *k_cache, const void *v_cache, const int32_t *seq_lens, float scale,
                               void *o, void *workspace, size_t workspace_bytes, void *stream) {
    const int st = check_attn(B, H, H_kv, d, T_max, io);
    if (st != KDA_OK) return st;
    if (!isfinite(scale)) return KDA_ERR_INVALID_ARG;
    if (B == 0) return KDA_OK;
    if (!q || !o || (T_max > 0 && (!k_cache || !v_cache))) return KDA_ERR_INVALID_ARG;
    if (!aligned(q, 16) || !aligned(o, 16) || !aligned(k_cache, 16) || !aligned(v_cache, 16) ||
        !aligned(seq_lens, 4))
        return KDA_ERR_INVALID_ARG;
    const size_t esz = io == KDA_BF16 ? 2 : 4;
    const size_t o_bytes = (size_t)B * H * d * esz, cache_bytes = (size_t)B * H_kv * T_max * d * esz;
    if (overlaps(o, o_bytes, q, o_bytes) || overlaps(o, o_bytes, k_cache, cache_bytes) ||
        overlaps(o, o_bytes, v_cache, cache_bytes) || overlaps(o, o_bytes, seq_lens, (size_t)B * 4))
        return KDA_ERR_INVALID_ARG;
    const AttnSplit sp = attn_split(B, H_kv, d, T_max);
    size_t ml_off;
    const size_t need = attn_ws_bytes(B, H, d, sp, &ml_off);
    float *part_acc = nullptr, *part_ml = nullptr;
    if (need > 0) {
        if (!workspace || workspace_bytes < need || !aligned(workspace, 256)) return KDA_ERR_WORKSPACE;
        if (overlaps(workspace, need, o, o_bytes) || overlaps(workspace, need, q, o_bytes) ||
            overlaps(workspace, need, k_cache, cache_bytes) || overlaps(workspace, need, v_cache, cache_bytes))
            return KDA_ERR_INVALID_ARG;
        part_acc = static_cast<float *>(workspace);
        part_ml = reinterpret_cast<float *>(static_cast<unsigned char *>(workspace) + ml_off);
    }
    const kda::AttnArgs a{q, k_cache, v_cache, seq_lens, scale, o, part_acc, part_ml,
                          H_kv, H / H_kv, T_max, sp.len, sp.n};
    if (kda::launch_attn_decode(a, B, d, io == KDA_BF16, reinterpret_cast<hipStream_t>(stream)) != hipSuccess)
        return KDA_ERR_HIP;
    return KDA_OK;
}

namespace {

struct BwdPlan {
    size_t per_bytes, scratch_off, total;
    int n_chunks, n_groups;
    // the matrix-core pass (bf16, d_k = d_v = 128): offsets of its workspace buffers
    bool fast;
    size_t W, U, QO, KtT, Aqk, eg, strong, st, ut, ds, du, discard, choff;
    int64_t fast_chunks;  // chunks over all sequences (an upper bound with cu_seqlens)
    // the token pass (kda_bwd_tok.hip): its chunk flags (direct pass; the matrix-core pass
    // reads the chunk preparation's), its workgroups' checkpoints
    size_t tok_flags, tok_scratch, tok_slot_floats;
    int tok_slots, tok_nblk;
};

// The token pass's checkpoints from offset off (one slot per workgroup, as many as the
// budget holds, at most one per pair); the end of them.
size_t tok_layout(size_t off, int64_t n_pairs, int64_t n_blk_max, int d_k, int d_v, BwdPlan *p) {
    p->tok_nblk = (int)n_blk_max;
    p->tok_slot_floats = (size_t)(n_blk_max + 16) * d_k * d_v;
    const size_t slot_bytes = p->tok_slot_floats * sizeof(float);
    int64_t slots = (int64_t)(kda::kTokScratchBudget / slot_bytes);
    slots = std::max<int64_t>(1, std::min<int64_t>(slots, std::min<int64_t>(n_pairs, 1024)));
    p->tok_slots = n_pairs > 0 && n_blk_max > 0 ? (int)slots : 0;
    p->tok_scratch = off;
    return round_up(off + (size_t)p->tok_slots * slot_bytes, 256);
}

// The matrix-core pass's workspace: per (chunk, head) the forward's chunk quantities, then
// S^T, U^T, dS'^T and dU^T (bf16); with packed sequences, the chunk-offset table.
void bwd_fast_layout(int64_t chunks, int H, int d_k, int d_v, int C, int n_seqs_varlen, int64_t n_pairs,
                     int64_t n_blk_max, BwdPlan *p) {
    const size_t u = (size_t)chunks * H, e = 2;
    size_t off = 0;
    auto take = [&](size_t bytes) {
        const size_t at = off;
        off = round_up(off + bytes, 256);
        return at;
    };
    p->W = take(u * C * d_k * e);
    p->U = take(u * C * d_v * e);
    p->QO = take(u * C * d_k * e);
    p->KtT = take(u * d_k * C * e);
    p->Aqk = take(u * C * C * e);
    p->eg = take(u * d_k * 4);
    p->strong = take(u);
    p->st = take(u * d_v * d_k * e);
    p->ut = take(u * d_v * C * e);
    p->ds = take(u * d_v * d_k * e);
    p->du = take(u * d_v * C * e);
    p->discard = take(256);
    p->choff = n_seqs_varlen > 0 ? take(((size_t)3 * n_seqs_varlen + 1) * sizeof(int32_t)) : 0;
    p->fast_chunks = chunks;
    off = tok_layout(off, n_pairs, n_blk_max, d_k, d_v, p);
    p->total = u > 0 || n_seqs_varlen > 0 ? off : 0;
}

// bf16 I/O with d_k = d_v = 128 takes the matrix-core backward pass (kda_bwd_bf16.hip);
// everything else the direct one (kda_bwd.hip).
bool bwd_fast(int d_k, int d_v, int io) { return io == KDA_BF16 && d_k == 128 && d_v == 128; }

int check_bwd(int B, int T, int H, int d_k, int d_v, int chunk, int io, BwdPlan *p) {
    if (io != KDA_F32 && io != KDA_BF16) return KDA_ERR_UNSUPPORTED;
    if (B < 0 || T < 0 || H < 1) return KDA_ERR_INVALID_ARG;
    if (chunk != kda::kBwdChunk || !supported_dim(d_k) || !supported_dim(d_v)) return KDA_ERR_UNSUPPORTED;
    if (B > 65535 || H > 65535 || (int64_t)B * T * H > INT32_MAX) return KDA_ERR_UNSUPPORTED;
    *p = BwdPlan{};
    p->n_chunks = (T + chunk - 1) / chunk;
    const int64_t units = (int64_t)B * p->n_chunks * H;
    p->fast = bwd_fast(d_k, d_v, io);
    if (p->fast) {
        bwd_fast_layout((int64_t)B * p->n_chunks, H, d_k, d_v, chunk, 0, (int64_t)B * H, p->n_chunks, p);
        return KDA_OK;
    }
    const kda::BwdLayout L{d_k, d_v};
    p->n_groups = (int)std::min<int64_t>(units, kda::kBwdMaxGroups);
    p->per_bytes = (size_t)L.per_chunk() * sizeof(float);
    p->scratch_off = round_up((size_t)units * p->per_bytes, 256);
    p->tok_flags = p->scratch_off + round_up((size_t)p->n_groups * L.scratch() * sizeof(float), 256);
    const size_t end = tok_layout(round_up(p->tok_flags + (size_t)units, 256), (int64_t)B * H, p->n_chunks, d_k, d_v, p);
    p->total = units > 0 ? end : 0;
    return KDA_OK;
}

// After either backward pass: the token pass over the pairs whose chunks `flags` marks.
int launch_tok_after(const BwdPlan &p, unsigned char *w8, const uint8_t *flags, const kda::SeqMap &map, int H,
                     int d_k, int d_v, int io, const void *q, const void *k, const void *v, const float *log_alpha,
                     const float *beta, float scale, const float *h0, const void *dout, const float *dhT, void *dq,
                     void *dk, void *dv, float *dlog_alpha, float *dbeta, float *dh0, size_t ntok, hipStream_t hs) {
    if (p.total == 0 || ntok == 0 || p.tok_slots == 0) return KDA_OK;
    kda::TokArgs t{};
    t.q = q, t.k = k, t.v = v, t.dout = dout, t.log_alpha = log_alpha, t.beta = beta, t.h0 = h0, t.dhT = dhT;
    t.scale = scale;
    t.dq = dq, t.dk = dk, t.dv = dv, t.dlog_alpha = dlog_alpha, t.dbeta = dbeta, t.dh0 = dh0;
    t.map = map;
    t.H = H;
    t.flags = flags;
    t.scratch = reinterpret_cast<float *>(w8 + p.tok_scratch);
    t.slot_floats = p.tok_slot_floats;
    t.n_blk_max = p.tok_nblk;
    return kda::launch_bwd_tok(t, d_k, d_v, io == KDA_BF16, p.tok_slots, hs) == hipSuccess ? KDA_OK : KDA_ERR_HIP;
}

}  // namespace

KDA_EXPORT size_t kda_chunk_bwd_workspace_bytes(int B, int T, int H, int d_k, int d_v, int chunk, int io) {
    BwdPlan p;
    if (check_bwd(B, T, H, d_k, d_v, chunk, io, &p) != KDA_OK) return 0;
    return p.total;
}

KDA_EXPORT int kda_chunk_bwd(int B, int T, int H, int d_k, int d_v, int chunk, int io, const void *q,
                             const void *k, const void *v, const float *log_alpha, const float *beta, float scale,
                             const float *h0, const void *dout, const float *dhT, void *dq, void *dk, void *dv,
                             float *dlog_alpha, float *dbeta, float *dh0, void *workspace, size_t workspace_bytes,
                             void *stream) {
    BwdPlan p;
    const int st = check_bwd(B, T, H, d_k, d_v, chunk, io, &p);
    if (st != KDA_OK) return st;
    if (!isfinite(scale)) return KDA_ERR_INVALID_ARG;
    const size_t ntok = (size_t)B * T * H, esz = io == KDA_BF16 ? 2 : 4;
    const size_t nk = ntok * d_k * esz, nv = ntok * d_v * esz, nb = ntok * 4, ns = (size_t)B * H * d_k * d_v * 4;
    const size_t nla = ntok * d_k * 4;  // log_alpha and dlog_alpha are fp32
    if (ntok > 0 && (!q || !k || !v || !log_alpha || !beta || !dout || !dq || !dk || !dv || !dlog_alpha || !dbeta))
        return KDA_ERR_INVALID_ARG;
    const void *in16[] = {q, k, v, log_alpha, dout, h0, dhT, dq, dk, dv, dlog_alpha, dh0};
    for (const void *x : in16)
        if (!aligned(x, 16)) return KDA_ERR_INVALID_ARG;
    if (!aligned(beta, 4) || !aligned(dbeta, 4)) return KDA_ERR_INVALID_ARG;
    // no output may overlap any argument or another output
    const void *ins[] = {q, k, v, log_alpha, beta, h0, dout, dhT};
    const size_t in_n[] = {nk, nk, nv, nla, nb, ns, nv, ns};
    const void *outs[] = {dq, dk, dv, dlog_alpha, dbeta, dh0};
    const size_t out_n[] = {nk, nk, nv, nla, nb, ns};
    for (int i = 0; i < 6; ++i) {
        for (int j = 0; j < 8; ++j)
            if (overlaps(outs[i], out_n[i], ins[j], in_n[j])) return KDA_ERR_INVALID_ARG;
        for (int j = i + 1; j < 6; ++j)
            if (overlaps(outs[i], out_n[i], outs[j], out_n[j])) return KDA_ERR_INVALID_ARG;
    }
    if (p.total > 0) {
        if (!workspace || workspace_bytes < p.total || !aligned(workspace, 256)) return KDA_ERR_WORKSPACE;
        for (int j = 0; j < 8; ++j)
            if (overlaps(workspace, p.total, ins[j], in_n[j])) return KDA_ERR_INVALID_ARG;
        for (int i = 0; i < 6; ++i)
            if (overlaps(workspace, p.total, outs[i], out_n[i])) return KDA_ERR_INVALID_ARG;
    }
    if (ntok == 0 && !(dh0 && B > 0)) return KDA_OK;
    if (p.fast) {
        unsigned char *w8 = static_cast<unsigned char *>(workspace);
        kda::BwdFastArgs a{};
        a.q = q, a.k = k, a.v = v, a.log_alpha = log_alpha, a.beta = beta, a.h0 = h0, a.dout = dout, a.dhT = dhT;
        a.scale = scale;
        a.dq = dq, a.dk = dk, a.dv = dv, a.dlog_alpha = dlog_alpha, a.dbeta = dbeta, a.dh0 = dh0;
        a.H = H;
        a.map = kda::SeqMap{nullptr, nullptr, nullptr, 0, B, T, kda::kBwdChunk};
        if (p.total > 0) {
            a.buf = kda::ChunkBuffers{w8 + p.W, w8 + p.U, w8 + p.QO, w8 + p.KtT, w8 + p.Aqk,
                                      reinterpret_cast<float *>(w8 + p.eg), w8 + p.strong};
            a.st = w8 + p.st, a.ut = w8 + p.ut, a.ds = w8 + p.ds, a.du = w8 + p.du, a.discard = w8 + p.discard;
        }
        const hipStream_t hs = reinterpret_cast<hipStream_t>(stream);
        if (kda::launch_chunk_bwd_bf16(a, B, B * p.n_chunks, hs) != hipSuccess) return KDA_ERR_HIP;
        return launch_tok_after(p, w8, w8 + p.strong, a.map, H, d_k, d_v, io, q, k, v, log_alpha, beta, scale, h0,
                                dout, dhT, dq, dk, dv, dlog_alpha, dbeta, dh0, ntok, hs);
    }
    float *ws = static_cast<float *>(workspace);
    const kda::BwdArgs a{q,  k,  v,  log_alpha, beta,       h0,    dout, dhT, scale,
                         dq, dk, dv, dlog_alpha, dbeta, dh0, ws,
                         p.total > 0 ? reinterpret_cast<float *>(static_cast<unsigned char *>(workspace) + p.scratch_off)
                                     : nullptr,
                         B, T, H, p.n_chunks, p.n_groups};
    const hipStream_t hs = reinterpret_cast<hipStream_t>(stream);
    if (kda::launch_chunk_bwd(a, d_k, d_v, io == KDA_BF16, hs) != hipSuccess) return KDA_ERR_HIP;
    if (p.total == 0 || ntok == 0) return KDA_OK;
    unsigned char *w8 = static_cast<unsigned char *>(workspace);
    const kda::SeqMap map{nullptr, nullptr, nullptr, 0, B, T, kda::kBwdChunk};
    if (kda::launch_bwd_tok_detect(log_alpha, map, H, d_k, B * p.n_chunks, w8 + p.tok_flags, hs) != hipSuccess)
        return KDA_ERR_HIP;
    return launch_tok_after(p, w8, w8 + p.tok_flags, map, H, d_k, d_v, io, q, k, v, log_alpha, beta, scale, h0, dout,
                            dhT, dq, dk, dv, dlog_alpha, dbeta, dh0, ntok, hs);
}

namespace {

int check_bwd_varlen(int T, int H, int d_k, int d_v, int chunk, int n_seqs, int io, BwdPlan *p) {
    if (io != KDA_F32 && io != KDA_BF16) return KDA_ERR_UNSUPPORTED;
    if (T < 0 || H < 1 || n_seqs < 1) return KDA_ERR_INVALID_ARG;
    if (chunk != kda::kBwdChunk || !bwd_fast(d_k, d_v, io)) return KDA_ERR_UNSUPPORTED;
    if (H > 65535 || n_seqs > 65535 || (int64_t)T * H > INT32_MAX) return KDA_ERR_UNSUPPORTED;
    *p = BwdPlan{};
    p->fast = true;
    bwd_fast_layout(((int64_t)T + chunk - 1) / chunk + n_seqs, H, d_k, d_v, chunk, n_seqs, (int64_t)n_seqs * H,
                    ((int64_t)T + chunk - 1) / chunk, p);
    return KDA_OK;
}

}  // namespace

KDA_EXPORT size_t kda_chunk_bwd_varlen_workspace_bytes(int T, int H, int d_k, int d_v, int chunk, int n_seqs,
                                                       int io) {
    BwdPlan p;
    if (check_bwd_varlen(T, H, d_k, d_v, chunk, n_seqs, io, &p) != KDA_OK) return 0;
    return p.total;
}

KDA_EXPORT int kda_chunk_bwd_varlen(int T, int H, int d_k, int d_v, int chunk, int io, const void *q, const void *k,
                                    const void *v, const float *log_alpha, const float *beta, float scale,
                                    const float *h0, const int32_t *cu_seqlens, int n_seqs, const void *dout,
                                    const float *dhT, void *dq, void *dk, void *dv, float *dlog_alpha, float *dbeta,
                                    float *dh0, void *workspace, size_t workspace_bytes, void *stream) {
    BwdPlan p;
    const int st = check_bwd_varlen(T, H, d_k, d_v, chunk, n_seqs, io, &p);
    if (st != KDA_OK) return st;
    if (!isfinite(scale)) return KDA_ERR_INVALID_ARG;
    const size_t ntok = (size_t)T * H, esz = 2;
    const size_t nk = ntok * d_k * esz, nv = ntok * d_v * esz, nb = ntok * 4, ns = (size_t)n_seqs * H * d_k * d_v * 4;
    const size_t nla = ntok * d_k * 4;
    if (!cu_seqlens || !aligned(cu_seqlens, 4)) return KDA_ERR_INVALID_ARG;
    if (ntok > 0 && (!q || !k || !v || !log_alpha || !beta || !dout || !dq || !dk || !dv || !dlog_alpha || !dbeta))
        return KDA_ERR_INVALID_ARG;
    const void *in16[] = {q, k, v, log_alpha, dout, h0, dhT, dq, dk, dv, dlog_alpha, dh0};
    for (const void *x : in16)
        if (!aligned(x, 16)) return KDA_ERR_INVALID_ARG;
    if (!aligned(beta, 4) || !aligned(dbeta, 4)) return KDA_ERR_INVALID_ARG;
    const size_t ncu = ((size_t)n_seqs + 1) * sizeof(int32_t);
    const void *ins[] = {q, k, v, log_alpha, beta, h0, dout, dhT, cu_seqlens};
    const size_t in_n[] = {nk, nk, nv, nla, nb, ns, nv, ns, ncu};
    const void *outs[] = {dq, dk, dv, dlog_alpha, dbeta, dh0};
    const size_t out_n[] = {nk, nk, nv, nla, nb, ns};
    for (int i = 0; i < 6; ++i) {
        for (int j = 0; j < 9; ++j)
            if (overlaps(outs[i], out_n[i], ins[j], in_n[j])) return KDA_ERR_INVALID_ARG;
        for (int j = i + 1; j < 6; ++j)
            if (overlaps(outs[i], out_n[i], outs[j], out_n[j])) return KDA_ERR_INVALID_ARG;
    }
    if (!workspace || workspace_bytes < p.total || !aligned(workspace, 256)) return KDA_ERR_WORKSPACE;
    for (int j = 0; j < 9; ++j)
        if (overlaps(workspace, p.total, ins[j], in_n[j])) return KDA_ERR_INVALID_ARG;
    for (int i = 0; i < 6; ++i)
        if (overlaps(workspace, p.total, outs[i], out_n[i])) return KDA_ERR_INVALID_ARG;
    const hipStream_t hs = reinterpret_cast<hipStream_t>(stream);
    unsigned char *w8 = static_cast<unsigned char *>(workspace);
    int32_t *tab = reinterpret_cast<int32_t *>(w8 + p.choff);
    if (kda::launch_chunk_offsets(cu_seqlens, n_seqs, T, kda::kBwdChunk, tab, tab + n_seqs + 1, tab + 2 * n_seqs + 1,
                                  hs) != hipSuccess)
        return KDA_ERR_HIP;
    kda::BwdFastArgs a{};
    a.q = q, a.k = k, a.v = v, a.log_alpha = log_alpha, a.beta = beta, a.h0 = h0, a.dout = dout, a.dhT = dhT;
    a.scale = scale;
    a.dq = dq, a.dk = dk, a.dv = dv, a.dlog_alpha = dlog_alpha, a.dbeta = dbeta, a.dh0 = dh0;
    a.H = H;
    a.map = kda::SeqMap{tab, tab + n_seqs + 1, tab + 2 * n_seqs + 1, 1, n_seqs, 0, kda::kBwdChunk};
    a.buf = kda::ChunkBuffers{w8 + p.W, w8 + p.U, w8 + p.QO, w8 + p.KtT, w8 + p.Aqk,
                              reinterpret_cast<float *>(w8 + p.eg), w8 + p.strong};
    a.st = w8 + p.st, a.ut = w8 + p.ut, a.ds = w8 + p.ds, a.du = w8 + p.du, a.discard = w8 + p.discard;
    if (kda::launch_chunk_bwd_bf16(a, n_seqs, (int)p.fast_chunks, hs) != hipSuccess) return KDA_ERR_HIP;
    return launch_tok_after(p, w8, w8 + p.strong, a.map, H, d_k, d_v, io, q, k, v, log_alpha, beta, scale, h0, dout,
                            dhT, dq, dk, dv, dlog_alpha, dbeta, dh0, ntok, hs);
}
