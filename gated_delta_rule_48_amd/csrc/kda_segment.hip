// kda_segment.hip -- the composition of segment maps for the segmented fused pass.
//
// A long sequence is cut into segments of seg_len tokens. A chunk acts on the state as
// an affine map, and so does a run of chunks: S_out = M S_in + N, M = prod over the
// chunks of (Diag(exp(gamma)) - (k exp(gamma - g))^T W), N the state reached from zero
// (unrolling the recurrence over the segment; the same identity as the chunk form of
// the essay "22,580: from GPT-2 to Kimi K3", section 6.3, applied to a run of chunks).
// The map instance of kda_fused_kernel forms (M, N) of every segment but a sequence's
// last, in parallel (segment 0's N from h0, so that N(0) = S_in(1)); this kernel then
// walks each sequence's segments in order, S_in(p + 1) = M(p) S_in(p) + N(p), and the
// usual instance runs every segment from its S_in in parallel.
//
// One workgroup of 4 waves per (sequence, head, 16 value columns): the columns of the
// state evolve independently. Each step is a 128 x 128 by 128 x 16 product in fp32 on
// the matrix cores (v_mfma_f32_16x16x4_f32), wave w forming rows 32 w .. 32 w + 31. Each
// lane reads its share of M(p) straight from memory (the contraction index of operand
// slot g of product kk is 32 g + kk, so a lane's share of a row is 32 adjacent values),
// M(p + 1) while step p computes; the 16 columns of S_in stay in LDS between steps. All
// buffers hold states in channel order, row-major (row = key channel), like h0 and hT.

#include "kda_internal.hpp"

namespace kda {
namespace {

constexpr int kD = 128;

__global__ __launch_bounds__(256) void kda_segment_chain_kernel(FusedArgs a) {
    __shared__ __align__(16) float Sb[kD * 16];
    const int H = a.H;
    const int pair = blockIdx.x >> 3, cb = blockIdx.x & 7;
    const int s = pair / H, h = pair % H;
    if (s >= a.n_seqs) return;
    const int g0 = a.cu_seqlens ? a.seg_off[s] : s * a.segs_per_seq;
    const int P = a.cu_seqlens ? a.seg_off[s + 1] - g0 : a.segs_per_seq;
    if (P <= 1) return;
    const int tid = threadIdx.x, w = tid >> 6, l = tid & 63, g = l >> 4, n = l & 15;
    const size_t DD = (size_t)kD * kD;
    auto map_of = [&](int p) { return a.seg_map + ((size_t)(g0 + p) * H + h) * 2 * DD; };
    auto state_of = [&](int p) { return a.seg_state + ((size_t)(g0 + p) * H + h) * DD; };

    // S_in(1) = N(0): this workgroup's 16 columns, to LDS and to segment 1's entering state
    {
        const float *N0 = map_of(0) + DD;
        float *S1 = state_of(1);
        for (int e = tid; e < kD * 16; e += 256) {
            const int r = e >> 4, c = e & 15;
            const float x = N0[r * kD + 16 * cb + c];
            Sb[e] = x;
            S1[r * kD + 16 * cb + c] = x;
        }
    }
    // this lane's A operands of M(p): rows 32 w + 16 t + n, columns 32 g .. 32 g + 31, in two
    // sets used in turn (step p computes from one while M(p + 1) arrives in the other)
    f32x4 amA[2][8], amB[2][8];
    auto fetch = [&](int p, f32x4 (&dst)[2][8]) {
        const float *M = map_of(p);
#pragma unroll
        for (int t = 0; t < 2; ++t)
#pragma unroll
            for (int j = 0; j < 8; ++j)
                dst[t][j] = *reinterpret_cast<const f32x4 *>(M + (32 * w + 16 * t + n) * kD + 32 * g + 4 * j);
    };
    auto step = [&](int p, const f32x4 (&am)[2][8]) {
        __syncthreads();  // Sb holds S_in(p)
        const float *N = map_of(p) + DD;
        f32x4 acc[2];
#pragma unroll
        for (int t = 0; t < 2; ++t) {
            acc[t] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int j = 0; j < 8; ++j)
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int kk = 4 * j + e;
                    acc[t] = __builtin_amdgcn_mfma_f32_16x16x4f32(am[t][j][e], Sb[(32 * g + kk) * 16 + n], acc[t], 0, 0, 0);
                }
        }
        __syncthreads();  // every wave has read Sb
        float *Sn = state_of(p + 1);
#pragma unroll
        for (int t = 0; t < 2; ++t)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int r = 32 * w + 16 * t + 4 * g + i;
                const float x = acc[t][i] + N[r * kD + 16 * cb + n];
                Sb[r * 16 + n] = x;
                Sn[r * kD + 16 * cb + n] = x;
            }
    };
    if (P > 2) fetch(1, amA);
    for (int p = 1; p + 1 < P; p += 2) {
        if (p + 2 < P) fetch(p + 1, amB);
        step(p, amA);
        if (p + 2 >= P) break;
        if (p + 3 < P) fetch(p + 2, amA);
        step(p + 1, amB);
    }
}

}  // namespace

hipError_t launch_segment_chain(const FusedArgs &a, hipStream_t stream) {
    hipLaunchKernelGGL(kda_segment_chain_kernel, dim3(a.n_seqs * a.H * 8), dim3(256), 0, stream, a);
    return hipGetLastError();
}

}  // namespace kda
