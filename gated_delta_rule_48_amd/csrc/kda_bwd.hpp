// kda_bwd.hpp -- launch arguments of the chunked backward pass (kda_bwd.hip),
// shared by the kernels and the C ABI.
#pragma once

#include "kda_internal.hpp"

namespace kda {

constexpr int kBwdChunk = 64;     // rows per chunk
constexpr int kBwdThreads = 256;  // four waves
constexpr int kBwdCols = 16;      // state columns per workgroup of the sequential passes
constexpr int kBwdMaxGroups = 1024;  // persistent workgroups of the chunk-local kernels, at most

// Per (chunk, head) buffers in the workspace, fp32, in this order: T (C x C), Aqk^T
// (C x C), W (C x dk), U~ (C x dv), R (C x dk), QO (C x dk), exp(gamma) (dk), the
// state at the chunk's start (dk x dv) and the loss gradient with respect to the
// state at its end (dk x dv).
struct BwdLayout {
    int dk, dv;
    __host__ __device__ constexpr int oT() const { return 0; }
    __host__ __device__ constexpr int oAqk() const { return kBwdChunk * kBwdChunk; }
    __host__ __device__ constexpr int oW() const { return 2 * kBwdChunk * kBwdChunk; }
    __host__ __device__ constexpr int oUt() const { return oW() + kBwdChunk * dk; }
    __host__ __device__ constexpr int oR() const { return oUt() + kBwdChunk * dv; }
    __host__ __device__ constexpr int oQO() const { return oR() + kBwdChunk * dk; }
    __host__ __device__ constexpr int oEg() const { return oQO() + kBwdChunk * dk; }
    __host__ __device__ constexpr int oS() const { return oEg() + dk; }
    __host__ __device__ constexpr int oDS() const { return oS() + dk * dv; }
    __host__ __device__ constexpr int per_chunk() const { return oDS() + dk * dv; }
    // scratch of one workgroup of the chunk-local kernels: 15 C x dk, 6 C x dv and
    // 5 C x C matrices, C betas and 2 dk vectors
    __host__ __device__ constexpr int scratch() const {
        return 15 * kBwdChunk * dk + 6 * kBwdChunk * dv + 5 * kBwdChunk * kBwdChunk + kBwdChunk + 2 * dk;
    }
};

struct BwdArgs {
    const void *q, *k, *v;  // io dtype (fp32 or bf16), as dout and dq, dk, dv
    const float *log_alpha, *beta, *h0;
    const void *dout;
    const float *dhT;
    float scale;
    void *dq, *dk, *dv;
    float *dlog_alpha, *dbeta, *dh0;
    float *ws;       // B * n_chunks * H per-chunk buffers (BwdLayout)
    float *scratch;  // n_groups * BwdLayout::scratch() floats
    int B, T, H, n_chunks, n_groups;
};

// hipSuccess or the first launch error.
hipError_t launch_chunk_bwd(const BwdArgs &a, int dk, int dv, bool bf16, hipStream_t stream);

// The backward pass on the matrix cores (kda_bwd_bf16.hip): bf16 I/O, d_k = d_v = 128,
// chunk 64. Its workspace holds the forward's chunk quantities (buf, as the split forward
// pass lays them out) and four bf16 matrices per (chunk, head), fragment-ordered: the
// state entering the chunk as S^T [d_v][d_k], the corrected writes as U^T [d_v][C], the
// gradient with respect to the state at the chunk's end as dS'^T [d_v][d_k], and dU^T
// [d_v][C].
struct BwdFastArgs {
    const void *q, *k, *v;  // bf16, as dout and dq, dk, dv
    const float *log_alpha, *beta, *h0;
    const void *dout;
    const float *dhT;
    float scale;
    void *dq, *dk, *dv;
    float *dlog_alpha, *dbeta, *dh0;
    int H;
    SeqMap map;
    ChunkBuffers buf;
    void *st, *ut, *ds, *du;
    void *discard;  // 256 bytes
};

hipError_t launch_chunk_bwd_bf16(const BwdFastArgs &a, int n_seqs, int total_chunks, hipStream_t stream);

// The backward token by token (kda_bwd_tok.hip), run after either pass for the (sequence,
// head) pairs holding a chunk whose summed log_alpha falls below -kStrongDecay on some key
// channel (flags, one byte per (chunk, head) in the chunk order of map: such chunks leave
// the range of the chunked passes' midpoint factors). It overwrites every gradient of those
// pairs. Each of its workgroups keeps the checkpoints of one pair at a time in scratch.
constexpr size_t kTokScratchBudget = size_t(512) << 20;  // bytes of checkpoints, at most
struct TokArgs {
    const void *q, *k, *v, *dout;  // io dtype
    const float *log_alpha, *beta, *h0, *dhT;
    float scale;
    void *dq, *dk, *dv;  // io dtype
    float *dlog_alpha, *dbeta, *dh0;
    SeqMap map;          // chunks of 64 rows from each sequence's start
    int H;
    const uint8_t *flags;   // [chunk][head]
    float *scratch;         // n_slots x slot_floats
    size_t slot_floats;     // (n_blk_max + 16) d_k d_v: a state per 64-token block, then per 4-token group
    int n_blk_max;          // 64-token blocks of the longest sequence, at most
};

// flags[j][h] for every chunk j of map (n_chunks_grid: an upper bound of map's chunk count).
hipError_t launch_bwd_tok_detect(const float *log_alpha, const SeqMap &map, int H, int dk, int n_chunks_grid,
                                 uint8_t *flags, hipStream_t stream);
hipError_t launch_bwd_tok(const TokArgs &a, int dk, int dv, bool io_bf16, int n_slots, hipStream_t stream);

}  // namespace kda
