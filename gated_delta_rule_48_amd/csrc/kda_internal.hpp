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
    uint8_t *redo;  // one byte per unit (see below): 1 where the unit met a chunk of strong decay
                    // and left its (sequence, head) to the strong instance
    // Segments (plan_u > 0: fewer (sequence, head) pairs than compute units). Each sequence of
    // c chunks is cut, for a budget of plan_T chunks, into P = max(1, ceil(c / plan_T))
    // segments: segment 0 of min(c, plan_T) chunks, then P - 1 near-equal ones. Launch A runs,
    // per head, every sequence's segment 0 (outputs, and the state at its end) and the maps of
    // segments 1 .. P - 2 (S_out = M S_in + N, from S_in = 0); the composition then forms the
    // states entering segments 2 .. P - 1; launch C runs segments 1 .. P - 1 from their
    // entering states. Each launch has at most plan_u units per head (one per compute unit).
    // The budget is the longest sequence (one segment each: launch A alone does the work) if
    // that has fewer than kMinSegChunks chunks. plan_u = 0 (256 pairs or more): one workgroup
    // per (sequence, head), redo [n_seqs * H].
    int plan_u;
    int plan_T;               // equal-length sequences: the budget (chunks)
    int plan_P;               // equal-length sequences: segments of each
    const int32_t *plan_tab;  // packed sequences: the plan (PlanTab layout), written by kda_seg_plan_kernel
    int n_seqs;
    float *seg_state;  // [slots, H, d_k, d_v] fp32: the state entering segment p >= 1 (slot of the segment)
    float *seg_map;    // [slots, H, 128 KB]: M (split into two bf16 parts) and N of segment p = 1 .. P - 2
                       // (its slot), in the order the composition reads them (seg_mh_index, seg_n_index)
    // With segments, redo holds [2 plan_u, H]: launch A's unit u at u H + h, launch C's at
    // (plan_u + u) H + h. The slot of segment p >= 1 of sequence s is the index of its unit in
    // launch C: c_off(s) + p - 1.
};

// A segment's map (d_k = d_v = 128, channel order), 128 KB: M split as M = Mh + Ml (Mh = M
// rounded to bf16, Ml = the rest rounded to bf16), Mh then Ml as bf16 [16384] each at
// seg_mh_index, then N as fp32 [16384] at seg_n_index. The composition's wave w, lane n + 16 g
// reads Mh and Ml [16 w + n][32 kb + 8 g .. + 7] with one 16-byte load each per kb, and
// N[16 w + 4 g + i][16 cb + n] with one 4-byte load per i: in these orders every such load
// instruction reads one contiguous run of 1 KB (Mh, Ml) or 256 B (N).
__host__ __device__ constexpr int seg_mh_index(int r, int c) {
    return ((((r >> 4) * 4 + (c >> 5)) * 64 + (r & 15) + 16 * ((c >> 3) & 3)) * 8 + (c & 7));
}
__host__ __device__ constexpr int seg_n_index(int r, int c) {
    return (((c >> 4) * 8 + (r >> 4)) * 4 + (r & 3)) * 64 + (c & 15) + 16 * ((r >> 2) & 3);
}

// The plan table of packed sequences (n = n_seqs): [0] the budget T (chunks); then a_off
// [n + 1] (launch A's units before each sequence), c_off [n + 1] (launch C's), tb [n] and te
// [n] (each sequence's token range, clamped to [0, T_total] and made monotone).
struct PlanTab {
    static constexpr int ints(int n) { return 4 * n + 3; }
    const int32_t *t;
    int n;
    __host__ __device__ int T() const { return t[0]; }
    __host__ __device__ const int32_t *a_off() const { return t + 1; }
    __host__ __device__ const int32_t *c_off() const { return t + n + 2; }
    __host__ __device__ const int32_t *tb() const { return t + 2 * n + 3; }
    __host__ __device__ const int32_t *te() const { return t + 3 * n + 3; }
};

// Sequences are cut into segments only if the longest has this many chunks or more.
constexpr int kMinSegChunks = 8;

// Segments of a sequence of c chunks under budget T, and its units in launch A (segment 0
// and the maps of segments 1 .. P - 2; at least one unit, for segment 0).
__host__ __device__ inline int plan_segments(int c, int T) { return c <= T ? 1 : (c + T - 1) / T; }
__host__ __device__ inline int plan_units_a(int c, int T) {
    const int P = plan_segments(c, T);
    return P > 1 ? P - 1 : 1;
}

// The budget from the smallest that fits the compute units (t_min) and the longest sequence
// (c_max chunks): both launches take about T chunk-steps (about 5.5 us each) and the composition
// max(P - 2, 0) dependent steps (about 1.4 us each), so the budget minimises 8 T + max(P - 2, 0).
// With many units per head (few heads) that is longer than t_min: one sequence of 64 chunks and
// 64 units per head takes T = 3 (44 against 70 for T = 1, whose composition has 62 steps). The
// cost only grows with T once 8 T passes the best cost found.
__host__ __device__ inline int plan_budget(int c_max, int t_min) {
    auto cost = [&](int T) {
        const int P = plan_segments(c_max, T);
        return 8 * T + (P > 2 ? P - 2 : 0);
    };
    int best = t_min, best_cost = cost(t_min);
    for (int T = t_min + 1; T <= c_max && 8 * T <= best_cost; ++T) {
        const int c = cost(T);
        if (c < best_cost) {
            best = T;
            best_cost = c;
        }
    }
    return best;
}

// Chunk range [*sc, *sc + *lc) of segment p of a sequence of c chunks under budget T.
__host__ __device__ inline void plan_segment_chunks(int c, int T, int p, int *sc, int *lc) {
    const int f = c < T ? c : T;
    if (p == 0) {
        *sc = 0;
        *lc = f;
        return;
    }
    const int parts = plan_segments(c, T) - 1, R = c - f, q = R / parts, e = R % parts;
    *sc = f + (p - 1) * q + (p - 1 < e ? p - 1 : e);
    *lc = q + (p - 1 < e ? 1 : 0);
}

// The composition of segment maps: per (sequence, head, 16 value columns) with P >= 3
// segments, in order, S_in(p + 1) = M(p) S_in(p) + N(p) for p = 1 .. P - 2, from S_in(1)
// (the state at the end of segment 0, written by launch A).
hipError_t launch_segment_chain(const FusedArgs &a, hipStream_t stream);
// The plan of packed sequences: clamped token ranges, the smallest budget T for which
// every head's units in launch A number at most u_max, and the units' offsets.
hipError_t launch_seg_plan(const int32_t *cu, int n_seqs, int T_total, int u_max, int32_t *tab,
                           hipStream_t stream);

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
hipError_t launch_fused(const FusedArgs &a, int dk, int dv, bool bf16, int n_seqs, hipStream_t stream);
hipError_t launch_decode(const DecodeArgs &a, int dk, int dv, bool bf16, hipStream_t stream);

}  // namespace kda
