// kda_segment.hip -- the plan and the composition of segment maps for the segmented fused pass.
//
// With fewer (sequence, head) pairs than compute units, long sequences are cut into segments.
// A chunk acts on the state as an affine map, and so does a run of chunks: S_out = M S_in + N,
// M = prod over the chunks of (Diag(exp(gamma)) - (k exp(gamma - g))^T W), N the state reached
// from zero (unrolling the recurrence over the segment; the same identity as the chunk form of
// the essay "22,580: from GPT-2 to Kimi K3", section 6.3, applied to a run of chunks).
// Launch A of kda_fused_kernel runs segment 0 of every sequence (outputs, and the state at its
// end, S_in(1)) and, in parallel, the maps (M, N) of the middle segments 1 .. P - 2; this
// kernel then walks each sequence's maps in order, S_in(p + 1) = M(p) S_in(p) + N(p); launch C
// runs segments 1 .. P - 1 from their S_in in parallel.
//
// The plan (kda_seg_plan_kernel for packed sequences; the host computes the same for equal
// lengths): for a budget of T chunks, a sequence of c chunks has P = ceil(c / T) segments, the
// first of min(c, T) chunks and the others near-equal (at most T each). Per head, launch A
// holds one unit per sequence with P = 1 and P - 1 units per sequence with P > 1, launch C
// P - 1 per sequence. T starts from the smallest budget for which launch A's units fit the
// compute units (u_max per head) and grows while that shortens the composition by more than
// it lengthens the two launches (plan_budget). If the longest sequence has fewer than
// kMinSegChunks chunks, T is its length: no sequence is cut.
//
// Composition: one workgroup of 8 waves per (sequence, head, 16 value columns): the columns of
// the state evolve independently. Each step is a 128 x 128 by 128 x 16 product on the matrix
// cores, wave w forming rows 16 w .. 16 w + 15. M(p) and S_in(p) are fp32; each operand is
// split as x = hi + lo (hi = x rounded to bf16, lo = the rest rounded to bf16) and the
// product taken as hi hi' + hi lo' + lo hi' with v_mfma_f32_16x16x32_bf16 (lane l supplies
// A[l%16][8 (l/16) .. + 7] and B[8 (l/16) .. + 7][l%16]), fp32 accumulation: about 16
// significant bits per product, at a fifth of the matrix-core time of fp32 instructions.
// M(p) arrives split: the map instance stores its two bf16 parts (split there once, not in
// every step of the eight workgroups that read it). Each lane reads its share of M(p) and N(p)
// straight from memory, those of steps p + 1 and p + 2 in flight while step p computes. The
// 16 columns of S_in stay in LDS, split into hi and lo once, by the lanes that form them
// (transposed; two sets of buffers used in turn, so one barrier per step). The 8 workgroups of
// one (sequence, head) run on one XCD (block ids 8 apart), so M(p) is fetched into one L2 and
// read there 8 times. The maps are stored in the order of these reads (seg_mh_index,
// seg_n_index: one contiguous 1 KB run per load instruction of M's parts, where row-major
// order would touch 16 cache lines per instruction, half of each); the entering states are
// row-major (row = key channel), like h0 and hT.

#include "kda_internal.hpp"

namespace kda {
namespace {

constexpr int kD = 128;
constexpr int kChainThreads = 512;
constexpr int kStPitch = kD + 8;  // bf16 per row of the transposed S_in buffers
constexpr int kBlockSteps = 15;   // steps per straight-line block (a multiple of the three operand sets)

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
    // segments of the sequence, and the slot of its segment 1 (segment p >= 1 at c0 + p - 1)
    int P, c0;
    if (a.plan_tab) {
        const PlanTab t{a.plan_tab, a.n_seqs};
        P = plan_segments((t.te()[s] - t.tb()[s] + 63) / 64, t.T());
        c0 = t.c_off()[s];
    } else {
        P = a.plan_P;
        c0 = s * (P - 1);
    }
    if (P <= 2) return;  // segment 1's entering state is segment 0's end state
    const int tid = threadIdx.x, w = tid >> 6, l = tid & 63, g = l >> 4, n = l & 15;
    const size_t DD = (size_t)kD * kD;
    auto map_of = [&](int p) { return a.seg_map + ((size_t)(c0 + p - 1) * H + h) * 2 * DD; };
    auto state_of = [&](int p) { return a.seg_state + ((size_t)(c0 + p - 1) * H + h) * DD; };

    // S_in(1), written by segment 0's workgroup in launch A: this workgroup's 16 columns, to
    // LDS (its loads are issued first, the first two steps' operands right behind them, so
    // that the three wait out one memory latency together)
    float n0[kD * 16 / kChainThreads];
#pragma unroll
    for (int k = 0; k < kD * 16 / kChainThreads; ++k) {
        const int e = tid + k * kChainThreads, r = e >> 4, c = e & 15;
        n0[k] = state_of(1)[r * kD + 16 * cb + c];
    }
    // this lane's A operands of M(p) (row 16 w + n, contraction indices 32 kb + 8 g .. + 7) and
    // the four entries of N(p) its outputs add, in three sets used in turn: step p computes
    // from one while the maps of steps p + 1 and p + 2 are in flight (a step is much shorter
    // than a load of M from memory)
    // (M arrives split: the map instance stores its two bf16 parts)
    bf16x8 amA[2][4], amB[2][4], amC[2][4];
    float nA[4], nB[4], nC[4];
    auto fetch = [&](int p, bf16x8 (&a8)[2][4], float (&n4)[4]) {
        const float *M = map_of(p);
        const bf16 *Mh = reinterpret_cast<const bf16 *>(M);
#pragma unroll
        for (int part = 0; part < 2; ++part)
#pragma unroll
            for (int kb = 0; kb < 4; ++kb)
                a8[part][kb] = *reinterpret_cast<const bf16x8 *>(Mh + part * kD * kD + seg_mh_index(16 * w + n, 32 * kb + 8 * g));
#pragma unroll
        for (int i = 0; i < 4; ++i) n4[i] = M[DD + seg_n_index(16 * w + 4 * g + i, 16 * cb + n)];
    };
    // S_in(p + 1) = M(p) S_in(p) + N(p); S_in(p) is in buffer p & 1
    auto step = [&](int p, const bf16x8 (&a8)[2][4], const float (&nv)[4]) {
        const bf16x8(&ah)[4] = a8[0];
        const bf16x8(&al)[4] = a8[1];
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
    // Every fetch is unconditional (past the last step a set re-reads the slot of segment P - 1,
    // which lies inside the workspace and is not used), so that the number of loads in flight is the
    // same on every path and each step waits for exactly its own operands. The steps run in
    // straight-line blocks of kBlockSteps: at the header of a loop the compiler's wait for
    // the loads in flight has to hold for the entry and for the back edge alike, and there
    // it waits for nearly all of them, so the pipeline drains once per block.
    fetch(1, amA, nA);
    fetch(2, amB, nB);  // (map P - 1 = 2 is read past the last step: inside the workspace, not used)
#pragma unroll
    for (int k = 0; k < kD * 16 / kChainThreads; ++k) {
        const int e = tid + k * kChainThreads, r = e >> 4, c = e & 15;
        const bf16 xh = static_cast<bf16>(n0[k]);
        Sh[1][c * kStPitch + r] = xh;
        Sl[1][c * kStPitch + r] = static_cast<bf16>(n0[k] - static_cast<float>(xh));
    }
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

// The plan of packed sequences, one thread per sequence (n_seqs < 256). The token ranges
// are the offsets clamped to [0, T_total] and made monotone: begin = min(T_total, max(0,
// cu[0 .. s])), end = min(T_total, max(0, cu[0 .. s + 1])), a running maximum.
constexpr int kPlanThreads = 256;

__device__ int block_sum(int v, int *red) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
    __syncthreads();  // every thread is done with red's previous use
    if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = v;
    __syncthreads();
    int t = 0;
#pragma unroll
    for (int i = 0; i < kPlanThreads / 64; ++i) t += red[i];
    return t;
}

__global__ __launch_bounds__(kPlanThreads) void kda_seg_plan_kernel(const int32_t *cu, int n, int T_total,
                                                                    int u_max, int32_t *tab) {
    __shared__ int pm[2][kPlanThreads + 1];
    __shared__ int red[kPlanThreads / 64];
    const int t = threadIdx.x;
    // running maximum of the clamped offsets 0 .. n (n + 1 <= 256 values)
    int x = t <= n ? min(max(cu[t], 0), T_total) : 0;
    pm[0][t] = x;
    int b = 0;
    for (int o = 1; o < kPlanThreads; o <<= 1) {
        __syncthreads();
        const int y = t >= o ? max(pm[b][t], pm[b][t - o]) : pm[b][t];
        pm[b ^ 1][t] = y;
        b ^= 1;
    }
    __syncthreads();
    const int tb = t < n ? pm[b][t] : 0, te = t < n ? pm[b][t + 1] : 0;
    const int c = (te - tb + 63) / 64;  // chunks (0 past the last sequence)
    // the smallest budget whose units in launch A fit u_max per head (T = max c always fits:
    // one unit per sequence, n <= u_max)
    int cmax = c;
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) cmax = max(cmax, __shfl_xor(cmax, o));
    if ((t & 63) == 0) red[t >> 6] = cmax;
    __syncthreads();
    cmax = 1;
#pragma unroll
    for (int i = 0; i < kPlanThreads / 64; ++i) cmax = max(cmax, red[i]);
    int lo = 1, hi = cmax;
    if (cmax < kMinSegChunks) lo = hi;  // (no segments)
    while (lo < hi) {  // (uniform across the block)
        const int mid = (lo + hi) >> 1;
        const int units = block_sum(t < n ? plan_units_a(c, mid) : 0, red);
        if (units <= u_max) hi = mid; else lo = mid + 1;
    }
    const int T = plan_budget(cmax, lo);  // (uniform: every thread works it out)
    // exclusive prefix sums of the units of launches A and C
    const int ua = t < n ? plan_units_a(c, T) : 0, uc = t < n ? plan_segments(c, T) - 1 : 0;
    __syncthreads();
    pm[0][t] = ua;
    pm[1][t] = uc;
    for (int o = 1; o < kPlanThreads; o <<= 1) {
        __syncthreads();
        const int ya = t >= o ? pm[0][t - o] : 0, yc = t >= o ? pm[1][t - o] : 0;
        __syncthreads();
        pm[0][t] += ya;
        pm[1][t] += yc;
    }
    __syncthreads();
    int32_t *a_off = tab + 1, *c_off = tab + n + 2, *tbo = tab + 2 * n + 3, *teo = tab + 3 * n + 3;  // (PlanTab)
    if (t == 0) {
        tab[0] = T;
        a_off[0] = 0;
        c_off[0] = 0;
    }
    if (t < n) {
        a_off[t + 1] = pm[0][t];
        c_off[t + 1] = pm[1][t];
        tbo[t] = tb;
        teo[t] = te;
    }
}

}  // namespace

hipError_t launch_seg_plan(const int32_t *cu, int n_seqs, int T_total, int u_max, int32_t *tab,
                           hipStream_t stream) {
    if (n_seqs < 1 || n_seqs >= kPlanThreads) return hipErrorInvalidValue;
    hipLaunchKernelGGL(kda_seg_plan_kernel, dim3(1), dim3(kPlanThreads), 0, stream, cu, n_seqs, T_total, u_max,
                       tab);
    return hipGetLastError();
}

hipError_t launch_segment_chain(const FusedArgs &a, hipStream_t stream) {
    const int groups = (a.n_seqs * a.H + 7) / 8;  // of 8 (sequence, head) pairs, one per XCD
    hipLaunchKernelGGL(kda_segment_chain_kernel, dim3(groups * 64), dim3(kChainThreads), 0, stream, a);
    return hipGetLastError();
}

}  // namespace kda
