// kda_internal.hpp -- launch interfaces between libkda's C ABI and its kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "kda_device.hpp"

namespace kda {

// Decay granularity of log_alpha (the kda_gate values of kda.h): one decay per key
// channel, one per token and head, or none.
constexpr int kGateChannel = 0, kGateHead = 1, kGateNone = 2;
// Gates formed from pre-activations: log_alpha = -exp(A_log[h]) softplus(a + dt_bias[h, c])
// per key channel (a in the io dtype, [T, H, d_k]) and beta = sigmoid(b).
constexpr int kGatePreact = 3;
// kGatePreact with q and k given before silu and per-row L2 normalisation (kernel
// template argument only; the arguments carry kGatePreact and PreactArgs::qk_norm).
constexpr int kGatePreactQK = 4;

// softplus(x) = log(1 + e^x) without overflow, and sigmoid(x) = 1 / (1 + e^-x).
__device__ __forceinline__ float softplus_f(float x) { return fmaxf(x, 0.f) + log1pf(expf(-fabsf(x))); }
__device__ __forceinline__ float sigmoid_f(float x) { return 1.f / (1.f + expf(-x)); }
// silu(x) = x sigmoid(x); rows normalised to unit L2 length with this floor on the norm.
__device__ __forceinline__ float silu_f(float x) { return x / (1.f + expf(-x)); }
constexpr float kNormEps = 1e-12f;

// The gate pre-activations' per-head parameters (kGatePreact only).
struct PreactArgs {
    const void *a;          // [T, H, d_k] io dtype
    const float *A_log;     // [H]
    const float *dt_bias;   // [H, d_k]
    int qk_norm;            // q and k are given before silu and L2 normalisation per row
};

// Per-chunk quantities produced by the chunk-preparation kernel and consumed by
// the state/output kernel. All are indexed chunk-major: [chunk j][head h][...],
// where j runs over the chunks of all sequences in order.
struct ChunkBuffers {
    void *W;     // [C][d_k]  io dtype: T (beta k exp(g))            (WY "w")
    void *U;     // [C][d_v]  io dtype: T (beta v)                   (WY "u", before the state term)
    void *QO;    // [C][d_k]  io dtype: scale q exp(g)               (readout of the entering state)
    void *KtT;   // [d_k][C]  io dtype: (k exp(gamma - g))^T         (write-back into the state)
    void *Aqk;   // [C][C]    io dtype: scale <q_r exp(g_r - g_i), k_i>, i <= r, else 0
    float *eg;   // [d_k]     fp32:     exp(gamma), gamma = g at the chunk's last row
    uint8_t *strong;  // [1]  chunk left to the strong-decay instance of the prep kernel (0 / 1)
};

struct PrepArgs {
    const void *q, *k, *v;
    const float *log_alpha, *beta;
    float scale;
    int H;
    int gate;  // kGateChannel: log_alpha [T, H, d_k]; kGateHead: [T, H]; kGateNone: not read;
               // kGatePreact: pre (log_alpha not read) and beta holds its pre-activation
    PreactArgs pre;
    SeqMap map;
    ChunkBuffers buf;
};

struct StateArgs {
    const float *h0;
    float *hT;
    void *o;        // null: no outputs (the backward pass runs this kernel for its states only)
    void *discard;  // 64 io-dtype elements of workspace that absorb writes of rows past a sequence end
    int H;
    int xcd_group;  // set by the launcher: map a pair's d_v slices onto one XCD
    SeqMap map;
    ChunkBuffers buf;
    // Optional (backward pass), per (chunk, head) in the io dtype: the state entering the
    // chunk as fragment-ordered S^T ([d_v][d_k]: row j = value column j, contraction over key
    // channels), and the chunk's corrected writes U as fragment-ordered U^T ([d_v][C]).
    void *st_out;
    void *ut_out;
};

struct FusedArgs {
    const void *q, *k, *v;
    const float *log_alpha, *beta;
    float scale;
    const float *h0;
    float *hT;
    void *o;
    void *discard;  // absorbs stores of rows past a sequence end (256 bytes)
    int H;
    int seq_len;    // every sequence has seq_len tokens (cu_seqlens null), or
    const int32_t *cu_seqlens;  // [n_seqs + 1] offsets of packed sequences (clamped to [0, T_total], monotone)
    int T_total;
    int gate;       // as in PrepArgs
    PreactArgs pre;
    uint8_t *redo;  // [n_seqs * H] (or [n_seg * H] with segments): 1 where the usual instance met
                    // a chunk of strong decay and left the (sequence, head) to the strong instance
    // Segments: each sequence cut into runs of seg_len tokens (a multiple of 64), one
    // workgroup per (segment, head); seg_len = 0: one workgroup per (sequence, head).
    int seg_len;
    int n_seqs;
    int segs_per_seq;          // equal-length sequences: segments of each
    const int32_t *seg_off;    // packed sequences: [n_seqs + 1] segments before each sequence,
    const int32_t *seg_tb;     // then each sequence's clamped begin and end ([n_seqs] each)
    const int32_t *seg_te;
    float *seg_state;          // [n_seg, H, d_k, d_v] fp32: the state entering each segment (p > 0)
    float *seg_map;            // [n_seg, H, 2, d_k * d_k] fp32: M and N of each segment (S_out = M S_in + N),
                               // in the order the composition reads them (seg_m_index, seg_n_index)
};

// Positions of M[r][c] and N[r][c] (d_k = d_v = 128, channel order) within a segment's map.
// The composition's wave w, lane n + 16 g reads M[16 w + n][32 kb + 8 g + 4 j .. + 3] with one
// 16-byte load per (kb, j), and N[16 w + 4 g + i][16 cb + n] with one 4-byte load per i: in
// these orders every such load instruction reads one contiguous run of 1 KB (M) or 256 B (N).
__host__ __device__ constexpr int seg_m_index(int r, int c) {
    return ((((r >> 4) * 4 + (c >> 5)) * 2 + ((c >> 2) & 1)) * 64 + (r & 15) + 16 * ((c >> 3) & 3)) * 4 + (c & 3);
}
__host__ __device__ constexpr int seg_n_index(int r, int c) {
    return (((c >> 4) * 8 + (r >> 4)) * 4 + (r & 3)) * 64 + (c & 15) + 16 * ((r >> 2) & 3);
}

// The composition of segment maps: per (sequence, head, 16 value columns), in order,
// S_in(1) = N(0) (segment 0's map starts from h0) and S_in(p + 1) = M(p) S_in(p) + N(p).
hipError_t launch_segment_chain(const FusedArgs &a, hipStream_t stream);

struct DecodeArgs {
    const void *q, *k, *v;
    const float *log_alpha, *beta;
    float scale;
    float *state;
    void *o;
    int NH;    // N * H
    int gate;  // as in PrepArgs (log_alpha [N, H, d_k] or [N, H])
    int H;
    PreactArgs pre;
};

// Each returns hipSuccess or the launch error.
// min_one: count at least one chunk (segment) for an empty sequence
hipError_t launch_chunk_offsets(const int32_t *cu, int n_seqs, int T_total, int C, int32_t *off,
                                int32_t *tb, int32_t *te, hipStream_t stream, int min_one = 0);
hipError_t launch_prep(const PrepArgs &a, int C, int dk, int dv, bool bf16, int n_chunks_grid,
                       hipStream_t stream);
hipError_t launch_state(const StateArgs &a, int C, int dk, int dv, bool bf16, int n_seqs,
                        hipStream_t stream);
// n_seg_grid: with segments (a.seg_len > 0), an upper bound on the number of segments
hipError_t launch_fused(const FusedArgs &a, int dk, int dv, bool bf16, int n_seqs, int n_seg_grid,
                        hipStream_t stream);
hipError_t launch_decode(const DecodeArgs &a, int dk, int dv, bool bf16, hipStream_t stream);

}  // namespace kda
