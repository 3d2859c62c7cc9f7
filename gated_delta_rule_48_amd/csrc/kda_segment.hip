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
// One workgroup of 8 waves per (sequence, head, 16 value columns): the columns of the
// state evolve independently. Each step is a 128 x 128 by 128 x 16 product on the matrix
// cores, wave w forming rows 16 w .. 16 w + 15. M(p) and S_in(p) are fp32; each operand is
// split as x = hi + lo (hi = x rounded to bf16, lo = the rest rounded to bf16) and the
// product taken as hi hi' + hi lo' + lo hi' with v_mfma_f32_16x16x32_bf16 (lane l supplies
// A[l%16][8 (l/16) .. + 7] and B[8 (l/16) .. + 7][l%16]), fp32 accumulation: about 16
// significant bits per product, at a fifth of the matrix-core time of fp32 instructions.
// Each lane reads its share of M(p) and N(p) straight from memory, those of steps p + 1
// and p + 2 in flight while step p computes. The 16 columns of S_in stay in LDS, split into
// hi and lo once, by the lanes that form them (transposed; two sets of buffers used in turn,
// so one barrier per step). The 8 workgroups of one (sequence, head) run on one
// XCD (block ids 8 apart), so M(p) is fetched into one L2 and read there 8 times. The maps
// are stored in the order of these reads (seg_m_index, seg_n_index: one contiguous 1 KB run
// per load instruction of M, where row-major order would touch 16 cache lines per
// instruction, half of each); the entering states are row-major (row = key channel), like h0
// and hT.

#include "kda_internal.hpp"

namespace kda {
namespace {

constexpr int kD = 128;
constexpr int kChainThreads = 512;
constexpr int kStPitch = kD + 8;  // bf16 per row of the transposed S_in buffers
constexpr int kBlockSteps = 15;   // steps per straight-line block (a multiple of the three operand sets)

// hi = bf16(x), lo = bf16(x - hi) for 8 values
__device__ __forceinline__ void split_hi_lo(const f32x4 &x0, const f32x4 &x1, bf16x8 &hi, bf16x8 &lo) {
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        hi[e] = static_cast<bf16>(x0[e]);
        lo[e] = static_cast<bf16>(x0[e] - static_cast<float>(hi[e]));
        hi[e + 4] = static_cast<bf16>(x1[e]);
        lo[e + 4] = static_cast<bf16>(x1[e] - static_cast<float>(hi[e + 4]));
    }
}

__global__ __launch_bounds__(kChainThreads) void kda_segment_chain_kernel(FusedArgs a) {
    // S_in's 16 columns as the B operand, already split: Sh[b][n * kStPitch + k] = hi of S_in[k][n],
    // Sl the rest (each value is split once, by the lane that forms it, for all eight waves)
    __shared__ __align__(16) bf16 Sh[2][16 * kStPitch], Sl[2][16 * kStPitch];
    const int H = a.H;
    // blocks are dealt round-robin to the 8 XCDs: block id = xcd + 8 (cb + 8 q), pair = xcd + 8 q
    const int xcd = blockIdx.x & 7, rest = blockIdx.x >> 3;
    const int cb = rest & 7, pair = xcd + 8 * (rest >> 3);
    if (pair >= a.n_seqs * H) return;
    const int s = pair / H, h = pair % H;
    const int g0 = a.cu_seqlens ? a.seg_off[s] : s * a.segs_per_seq;
    const int P = a.cu_seqlens ? a.seg_off[s + 1] - g0 : a.segs_per_seq;
    if (P <= 1) return;
    const int tid = threadIdx.x, w = tid >> 6, l = tid & 63, g = l >> 4, n = l & 15;
    const size_t DD = (size_t)kD * kD;
    auto map_of = [&](int p) { return a.seg_map + ((size_t)(g0 + p) * H + h) * 2 * DD; };
    auto state_of = [&](int p) { return a.seg_state + ((size_t)(g0 + p) * H + h) * DD; };

    // S_in(1) = N(0): this workgroup's 16 columns, to LDS and to segment 1's entering state
    // (its loads are issued first, the first two steps' operands right behind them, so that
    // the three wait out one memory latency together)
    float n0[kD * 16 / kChainThreads];
#pragma unroll
    for (int k = 0; k < kD * 16 / kChainThreads; ++k) {
        const int e = tid + k * kChainThreads, r = e >> 4, c = e & 15;
        n0[k] = map_of(0)[DD + seg_n_index(r, 16 * cb + c)];
    }
    // this lane's A operands of M(p) (row 16 w + n, contraction indices 32 kb + 8 g .. + 7) and
    // the four entries of N(p) its outputs add, in three sets used in turn: step p computes
    // from one while the maps of steps p + 1 and p + 2 are in flight (a step is much shorter
    // than a load of M from memory)
    f32x4 amA[4][2], amB[4][2], amC[4][2];
    float nA[4], nB[4], nC[4];
    auto fetch = [&](int p, f32x4 (&a4)[4][2], float (&n4)[4]) {
        const float *M = map_of(p);
#pragma unroll
        for (int kb = 0; kb < 4; ++kb)
#pragma unroll
            for (int j = 0; j < 2; ++j)
                a4[kb][j] = *reinterpret_cast<const f32x4 *>(M + seg_m_index(16 * w + n, 32 * kb + 8 * g + 4 * j));
#pragma unroll
        for (int i = 0; i < 4; ++i) n4[i] = M[DD + seg_n_index(16 * w + 4 * g + i, 16 * cb + n)];
    };
    // S_in(p + 1) = M(p) S_in(p) + N(p); S_in(p) is in buffer p & 1
    auto step = [&](int p, const f32x4 (&a4)[4][2], const float (&nv)[4]) {
        bf16x8 ah[4], al[4];  // M's split does not wait for S_in
#pragma unroll
        for (int kb = 0; kb < 4; ++kb) split_hi_lo(a4[kb][0], a4[kb][1], ah[kb], al[kb]);
        __syncthreads();  // S_in(p) complete; every wave is done with the other buffer
        const bf16 *sh = Sh[p & 1], *sl = Sl[p & 1];
        f32x4 hh = {0.f, 0.f, 0.f, 0.f}, hl = hh, lh = hh;
#pragma unroll
        for (int kb = 0; kb < 4; ++kb) {
            const bf16x8 bh = *reinterpret_cast<const bf16x8 *>(sh + n * kStPitch + 32 * kb + 8 * g);
            const bf16x8 bl = *reinterpret_cast<const bf16x8 *>(sl + n * kStPitch + 32 * kb + 8 * g);
            hh = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ah[kb], bh, hh, 0, 0, 0);
            hl = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ah[kb], bl, hl, 0, 0, 0);
            lh = __builtin_amdgcn_mfma_f32_16x16x32_bf16(al[kb], bh, lh, 0, 0, 0);
        }
        bf16 *dh = Sh[(p + 1) & 1], *dl = Sl[(p + 1) & 1];
        float x[4];
        bf16 xh[4], xl[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            x[i] = hh[i] + (hl[i] + lh[i]) + nv[i];
            xh[i] = static_cast<bf16>(x[i]);
            xl[i] = static_cast<bf16>(x[i] - static_cast<float>(xh[i]));
        }
        // rows 16 w + 4 g .. + 3 of column n: four adjacent entries of each buffer's row n (the
        // next step's operand first: the stores to memory below may wait behind loads in flight)
        *reinterpret_cast<uint2 *>(dh + n * kStPitch + 16 * w + 4 * g) = *reinterpret_cast<const uint2 *>(xh);
        *reinterpret_cast<uint2 *>(dl + n * kStPitch + 16 * w + 4 * g) = *reinterpret_cast<const uint2 *>(xl);
        float *Sn = state_of(p + 1);
#pragma unroll
        for (int i = 0; i < 4; ++i) Sn[(16 * w + 4 * g + i) * kD + 16 * cb + n] = x[i];
    };
    // Every fetch is unconditional (past the last step a set re-reads map P - 1, which lies
    // inside the workspace and is not used), so that the number of loads in flight is the
    // same on every path and each step waits for exactly its own operands. The steps run in
    // straight-line blocks of kBlockSteps: at the header of a loop the compiler's wait for
    // the loads in flight has to hold for the entry and for the back edge alike, and there
    // it waits for nearly all of them, so the pipeline drains once per block.
    if (P > 2) {
        fetch(1, amA, nA);
        fetch(min(2, P - 1), amB, nB);
    }
    {
        float *S1 = state_of(1);
#pragma unroll
        for (int k = 0; k < kD * 16 / kChainThreads; ++k) {
            const int e = tid + k * kChainThreads, r = e >> 4, c = e & 15;
            const bf16 xh = static_cast<bf16>(n0[k]);
            Sh[1][c * kStPitch + r] = xh;
            Sl[1][c * kStPitch + r] = static_cast<bf16>(n0[k] - static_cast<float>(xh));
            S1[r * kD + 16 * cb + c] = n0[k];
        }
    }
    if (P <= 2) return;
    for (int p0 = 1; p0 + 1 < P; p0 += kBlockSteps) {
#pragma unroll
        for (int j = 0; j < kBlockSteps; j += 3) {
            const int p = p0 + j;
            if (p + 1 >= P) break;
            fetch(min(p + 2, P - 1), amC, nC);
            step(p, amA, nA);
            if (p + 2 >= P) break;
            fetch(min(p + 3, P - 1), amA, nA);
            step(p + 1, amB, nB);
            if (p + 3 >= P) break;
            fetch(min(p + 4, P - 1), amB, nB);
            step(p + 2, amC, nC);
        }
    }
}

}  // namespace

hipError_t launch_segment_chain(const FusedArgs &a, hipStream_t stream) {
    const int groups = (a.n_seqs * a.H + 7) / 8;  // of 8 (sequence, head) pairs, one per XCD
    hipLaunchKernelGGL(kda_segment_chain_kernel, dim3(groups * 64), dim3(kChainThreads), 0, stream, a);
    return hipGetLastError();
}

}  // namespace kda
