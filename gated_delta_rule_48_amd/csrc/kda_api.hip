// kda_api.hip -- the C ABI of libkda (see include/kda.h): argument validation,
// workspace layout and kernel dispatch. Host code only; it never synchronises.

#include <math.h>

#include <algorithm>
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

// The fused pass (one workgroup per (sequence, head), nothing staged in
// memory) is used for bf16 input with d_k = d_v = 128 and chunk 64 when the
// (sequence, head) pairs alone fill the chip, for equal-length and for packed
// sequences; otherwise the split pass (parallel chunk preparation, then state
// propagation over d_v slices). With packed sequences the longest one sets the
// fused pass's time, as it does the split pass's state propagation.
constexpr int kFusedMinPairs = 256;
bool use_fused(int B, int T, int H, int dk, int dv, int C, bool varlen, int io, int n_seqs) {
    return C == 64 && io == KDA_BF16 && dk == 128 && dv == 128 && T > 0 &&
           (int64_t)(varlen ? n_seqs : B) * H >= kFusedMinPairs;
}

struct WsLayout {
    size_t W, U, QO, KtT, Aqk, eg, discard, choff, total;
    int64_t n_chunks;  // upper bound on the number of chunks over all sequences
};

// Workspace layout: per-chunk buffers (chunk-major, see ChunkBuffers) and, for
// packed variable-length input, the chunk offsets of the sequences.
bool ws_layout(int B, int T, int H, int dk, int dv, int C, int n_seqs, bool varlen, int io,
               WsLayout *L) {
    if (T <= 0) {
        *L = WsLayout{0, 0, 0, 0, 0, 0, 0, 0, 0, 0};
        return true;
    }
    if (use_fused(B, T, H, dk, dv, C, varlen, io, n_seqs)) {  // only the discard slot
        *L = WsLayout{0, 0, 0, 0, 0, 0, 0, 0, 256, 0};
        L->n_chunks = 0;
        return true;
    }
    const size_t esz = io == KDA_BF16 ? 2 : 4;
    const int64_t per_seq = ((int64_t)T + C - 1) / C;
    L->n_chunks = varlen ? per_seq + n_seqs : (int64_t)B * per_seq;
    const size_t nch = (size_t)L->n_chunks * (size_t)H;
    size_t off = 0;
    auto take = [&](size_t bytes) {
        const size_t at = off;
        off = round_up(off + bytes, 256);
        return at;
    };
    L->W = take(nch * C * dk * esz);
    L->U = take(nch * C * dv * esz);
    L->QO = take(nch * C * dk * esz);
    L->KtT = take(nch * dk * C * esz);
    L->Aqk = take(nch * C * C * esz);
    L->eg = take(nch * dk * sizeof(float));
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

namespace {

// kda_chunk_fwd_gated (gate = a kda_gate value) and kda_chunk_fwd_preact (gate =
// kda::kGatePreact, pre = its pre-activations; log_alpha unused, beta = b).
int chunk_fwd_impl(int gate, const kda::PreactArgs &pre, int B, int T, int H, int d_k, int d_v, int chunk, int io,
                   const void *q, const void *k, const void *v, const float *log_alpha, const float *beta,
                   float scale, const float *h0, const int32_t *cu_seqlens, int n_seqs, void *o, float *hT,
                   void *workspace, size_t workspace_bytes, void *stream) {
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
    if (L.total > 0 && (!workspace || !aligned(workspace, 256) || workspace_bytes < L.total))
        return KDA_ERR_WORKSPACE;

    hipStream_t hs = reinterpret_cast<hipStream_t>(stream);
    char *ws = static_cast<char *>(workspace);
    const bool bf = io == KDA_BF16;
    if (use_fused(B, T, H, d_k, d_v, chunk, varlen, io, n_seqs)) {
        kda::FusedArgs fa{q,  k,     v,  log_alpha, beta, scale, h0, hT,   o, ws + L.discard, H,
                          T,  varlen ? cu_seqlens : nullptr, (int)tokens, gate, pre};
        return kda::launch_fused(fa, d_k, d_v, bf, nseq, hs) == hipSuccess ? KDA_OK : KDA_ERR_HIP;
    }
    ChunkBuffers buf{};
    if (L.total > 0) {
        buf = ChunkBuffers{ws + L.W, ws + L.U, ws + L.QO, ws + L.KtT, ws + L.Aqk,
                           reinterpret_cast<float *>(ws + L.eg)};
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
};

int check_bwd(int B, int T, int H, int d_k, int d_v, int chunk, int io, BwdPlan *p) {
    if (io != KDA_F32 && io != KDA_BF16) return KDA_ERR_UNSUPPORTED;
    if (B < 0 || T < 0 || H < 1) return KDA_ERR_INVALID_ARG;
    if (chunk != kda::kBwdChunk || !supported_dim(d_k) || !supported_dim(d_v)) return KDA_ERR_UNSUPPORTED;
    if (B > 65535 || H > 65535 || (int64_t)B * T * H > INT32_MAX) return KDA_ERR_UNSUPPORTED;
    const kda::BwdLayout L{d_k, d_v};
    p->n_chunks = (T + chunk - 1) / chunk;
    const int64_t units = (int64_t)B * p->n_chunks * H;
    p->n_groups = (int)std::min<int64_t>(units, kda::kBwdMaxGroups);
    p->per_bytes = (size_t)L.per_chunk() * sizeof(float);
    p->scratch_off = round_up((size_t)units * p->per_bytes, 256);
    p->total = units > 0 ? p->scratch_off + round_up((size_t)p->n_groups * L.scratch() * sizeof(float), 256) : 0;
    return KDA_OK;
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
    float *ws = static_cast<float *>(workspace);
    const kda::BwdArgs a{q,  k,  v,  log_alpha, beta,       h0,    dout, dhT, scale,
                         dq, dk, dv, dlog_alpha, dbeta, dh0, ws,
                         p.total > 0 ? reinterpret_cast<float *>(static_cast<unsigned char *>(workspace) + p.scratch_off)
                                     : nullptr,
                         B, T, H, p.n_chunks, p.n_groups};
    if (kda::launch_chunk_bwd(a, d_k, d_v, io == KDA_BF16, reinterpret_cast<hipStream_t>(stream)) != hipSuccess)
        return KDA_ERR_HIP;
    return KDA_OK;
}
