// kda_solve.hpp -- (I + A)^{-1} for the strictly lower triangular C x C matrix
// of one chunk, in LDS, by one workgroup. Internal to libkda.
//
// This is the inverse that the WY reparametrisation needs (the essay "22,580:
// from GPT-2 to Kimi K3", yichencityu.github.io, section 6.3, obtains it by
// forward substitution row by row). Here, in place: the 16 x 16 diagonal blocks
// by forward substitution, one thread per column, then blocks are doubled,
// [[T1, 0], [X, T2]] with X = -T2 A21 T1, for block sizes 16, 32 and 64.
#pragma once

#include "kda_device.hpp"

namespace kda {

// M = (I + A)^{-1} in place, for A strictly lower triangular (C x C, fp32, pitch
// PT, zero on and above the diagonal). 16x16 diagonal blocks by forward
// substitution (one thread per column), then doubling: [[T1, 0], [X, T2]] with
// X = -T2 (A21 T1), for block sizes 16, 32, 64. Each X is formed in the slot of
// its A21, which no other block reads: the blocks A21 of a level lie below the
// diagonal blocks of all lower levels. Ends with a barrier.
template <int C, int PT, typename T, int NT>
__device__ __forceinline__ void unit_lower_inverse(float *M) {
    const int tid = threadIdx.x;
    {
        const int base = tid & ~15, c = tid & 15;
        float x[16];
        if (tid < C) {
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                // row r of the diagonal block, read as four 16-byte vectors
                float arow[16];
#pragma unroll
                for (int v4 = 0; v4 < 4; ++v4) {
                    const f32x4 t = *reinterpret_cast<const f32x4 *>(M + (base + r) * PT + base + 4 * v4);
#pragma unroll
                    for (int e = 0; e < 4; ++e) arow[4 * v4 + e] = t[e];
                }
                float acc = 0.f;
#pragma unroll
                for (int i = 0; i < 16; ++i)
                    if (i < r) acc += arow[i] * x[i];
                x[r] = (r < c) ? 0.f : (r == c ? 1.f : -acc);
            }
        }
        __syncthreads();  // every diagonal block read
        if (tid < C) {
#pragma unroll
            for (int r = 0; r < 16; ++r) M[(base + r) * PT + base + c] = x[r];
        }
    }

    // Level n = 16 on the vector ALUs: C/32 pairs of 16x16 blocks, 256 entries each.
    {
        constexpr int NP = C / 32;
        constexpr int PER = (NP * 256 + NT - 1) / NT;
        float y[PER];
        __syncthreads();
#pragma unroll
        for (int u = 0; u < PER; ++u) {  // Y = A21 T1
            const int e = tid + u * NT;
            y[u] = 0.f;
            if (e < NP * 256) {
                const int p = e >> 8, r = (e >> 4) & 15, c = e & 15;
                const int r0 = (2 * p + 1) * 16, c0 = 2 * p * 16;
                float acc = 0.f;
#pragma unroll
                for (int m = 0; m < 16; ++m) acc += M[(r0 + r) * PT + c0 + m] * M[(c0 + m) * PT + c0 + c];
                y[u] = acc;
            }
        }
        __syncthreads();
#pragma unroll
        for (int u = 0; u < PER; ++u) {  // Y replaces A21
            const int e = tid + u * NT;
            if (e < NP * 256) {
                const int p = e >> 8, r = (e >> 4) & 15, c = e & 15;
                M[((2 * p + 1) * 16 + r) * PT + 2 * p * 16 + c] = y[u];
            }
        }
        __syncthreads();
#pragma unroll
        for (int u = 0; u < PER; ++u) {  // X = -T2 Y
            const int e = tid + u * NT;
            if (e < NP * 256) {
                const int p = e >> 8, r = (e >> 4) & 15, c = e & 15;
                const int r0 = (2 * p + 1) * 16, c0 = 2 * p * 16;
                float acc = 0.f;
#pragma unroll
                for (int m = 0; m < 16; ++m) acc += M[(r0 + r) * PT + r0 + m] * M[(r0 + m) * PT + c0 + c];
                y[u] = -acc;
            }
        }
        __syncthreads();
#pragma unroll
        for (int u = 0; u < PER; ++u) {
            const int e = tid + u * NT;
            if (e < NP * 256) {
                const int p = e >> 8, r = (e >> 4) & 15, c = e & 15;
                M[((2 * p + 1) * 16 + r) * PT + 2 * p * 16 + c] = y[u];
            }
        }
    }

    // Levels n = 32, 64 on the matrix cores: (n/16)^2 output tiles per pair.
    constexpr int NW = NT / 64;
    const int w = tid >> 6;
#pragma unroll
    for (int n = 32; 2 * n <= C; n *= 2) {
        const int NP = C / (2 * n), TPP = (n / 16) * (n / 16), NTL = NP * TPP;
        constexpr int MAXT = (C * 64 / 512 + NW - 1) / NW;  // tiles per wave at the largest level
        f32x4 res[MAXT];
        __syncthreads();
#pragma unroll
        for (int u = 0; u < MAXT; ++u) {  // Y = A21 T1
            const int t = w + NW * u;
            res[u] = f32x4{0.f, 0.f, 0.f, 0.f};
            if (t < NTL) {
                const int p = t / TPP, ti = (t % TPP) / (n / 16), tj = t % (n / 16);
                const int r0 = (2 * p + 1) * n + ti * 16, c0 = 2 * p * n + tj * 16;
                res[u] = mma_nn_f32<T>(res[u], M + r0 * PT + 2 * p * n, PT, M + (2 * p * n) * PT + c0, PT, 0, n);
            }
        }
        __syncthreads();
#pragma unroll
        for (int u = 0; u < MAXT; ++u) {  // Y replaces A21
            const int t = w + NW * u;
            if (t < NTL) {
                const int p = t / TPP, ti = (t % TPP) / (n / 16), tj = t % (n / 16);
                const int r0 = (2 * p + 1) * n + ti * 16, c0 = 2 * p * n + tj * 16;
#pragma unroll
                for (int i = 0; i < 4; ++i) M[(r0 + acc_row(i)) * PT + c0 + acc_col()] = res[u][i];
            }
        }
        __syncthreads();
#pragma unroll
        for (int u = 0; u < MAXT; ++u) {  // X = -T2 Y
            const int t = w + NW * u;
            if (t < NTL) {
                const int p = t / TPP, ti = (t % TPP) / (n / 16), tj = t % (n / 16);
                const int r0 = (2 * p + 1) * n + ti * 16, c0 = 2 * p * n + tj * 16;
                res[u] = -mma_nn_f32<T>(f32x4{0.f, 0.f, 0.f, 0.f}, M + r0 * PT + (2 * p + 1) * n, PT,
                                        M + ((2 * p + 1) * n) * PT + c0, PT, 0, n);
            }
        }
        __syncthreads();
#pragma unroll
        for (int u = 0; u < MAXT; ++u) {
            const int t = w + NW * u;
            if (t < NTL) {
                const int p = t / TPP, ti = (t % TPP) / (n / 16), tj = t % (n / 16);
                const int r0 = (2 * p + 1) * n + ti * 16, c0 = 2 * p * n + tj * 16;
#pragma unroll
                for (int i = 0; i < 4; ++i) M[(r0 + acc_row(i)) * PT + c0 + acc_col()] = res[u][i];
            }
        }
    }
    __syncthreads();
}

}  // namespace kda
