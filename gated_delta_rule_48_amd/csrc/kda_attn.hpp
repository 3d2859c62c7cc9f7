// kda_attn.hpp -- launch arguments of the softmax-attention decode step over a
// KV cache (kda_attn.hip), shared by the kernels and the C ABI.
#pragma once

#include "kda_internal.hpp"

namespace kda {

// The cache of each (sequence, cached head) is split along time into n_splits
// ranges of split_len rows, one workgroup each; with more than one, the splits'
// partial results go to part_acc [B, H, n_splits, D] and part_ml
// [B, H, n_splits, 2] (running maximum and sum), and a second kernel combines
// them.
constexpr int kAttnThreads = 256;         // four waves
constexpr int kAttnRowsPerLane = 4;       // cache rows per lane group per iteration
constexpr int kAttnMaxSplits = 4096;      // splits per cached head, at most (the combine keeps a weight each in LDS)
constexpr int kAttnCombineChannels = 32;  // channels per combine workgroup
__host__ __device__ constexpr int attn_rows_per_iter(int D) { return 4 * (64 / (D / 8)) * kAttnRowsPerLane; }

struct AttnArgs {
    const void *q, *k, *v;      // q [B, H, D]; k, v caches [B, H_kv, T_max, D]
    const int32_t *seq_lens;    // [B] rows in use per sequence, or null (all T_max)
    float scale;
    void *o;                    // [B, H, D]
    float *part_acc, *part_ml;  // split partials (n_splits > 1)
    int H_kv, G, T_max, split_len, n_splits;
};

// hipSuccess or the launch error.
hipError_t launch_attn_decode(const AttnArgs &a, int B, int D, bool bf16, hipStream_t stream);

}  // namespace kda
