// kda_solve.hpp -- (I + A)^{-1} for the strictly lower triangular C x C matrix
// of one chunk, in LDS, by one workgroup. Internal to libkda.
//
// This is the inverse that the WY reparametrisation needs (the essay "22,580:
// from GPT-2 to Kimi K3", yichencityu.github.io, section 6.3, obtains it by
// forward substitution row by row). Here: the 16 x 16 diagonal blocks by
// forward substitution, one thread per column, then blocks are doubled,
// [[T1, 0], [X, T2]] with X = -T2 A21 T1, for block sizes 16, 32 and 64.
#pragma once

#include "kda_device.hpp"

namespace kda {

// Tm = (I + A)^{-1} for A strictly lower triangular (C x C, fp32, pitch PT).
// 16x16 diagonal blocks by forward substitution (one thread per column), then
// doubling: [[T1, 0], [X, T2]] with X = -T2 A21 T1, for block sizes 16, 32, 64.
template <int C, int PT, typename T, int NT>
__device__ __forceinline__ void unit_lower_inverse(const float *A, float *Tm) {
    const int tid = threadIdx.x;
    for (int e = tid; e < C * PT / 4; e += NT) reinterpret_cast<f32x4 *>(Tm)[e] = f32x4{0.f, 0.f, 0.f, 0.f};
    __syncthreads();
    if (tid < C) {
        const int base = tid & ~15, c = tid & 15;
        float x[16];
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            // row r of the diagonal block, read as four 16-byte vectors
            float arow[16];
#pragma unroll
            for (int v4 = 0; v4 < 4; ++v4) {
                const f32x4 t = *reinterpret_cast<const f32x4 *>(A + (base + r) * PT + base + 4 * v4);
#pragma unroll
                for (int e = 0; e < 4; ++e) arow[4 * v4 + e] = t[e];
            }
            float acc = 0.f;
#pragma unroll
            for (int i = 0; i < 16; ++i)
                if (i < r) acc += arow[i] * x[i];
            x[r] = (r < c) ? 0.f : (r == c ? 1.f : -acc);
        }
#pragma unroll
        for (int r = 0; r < 16; ++r) Tm[(base + r) * PT + base + c] = x[r];
    }

    // Level n = 16 on the vector ALUs: C/32 pairs of 16x16 blocks, 256 entries each.
    {
        constexpr int NP = C / 32;
        constexpr int PER = (NP * 256 + NT - 1) / NT;
        __syncthreads();
#pragma unroll
        for (int u = 0; u < PER; ++u) {  // Y = A21 T1, written into the X slot
            const int e = tid + u * NT;
            if (e < NP * 256) {
                const int p = e >> 8, r = (e >> 4) & 15, c = e & 15;
                const int r0 = (2 * p + 1) * 16, c0 = 2 * p * 16;
                float acc = 0.f;
#pragma unroll
                for (int m = 0; m < 16; ++m) acc += A[(r0 + r) * PT + c0 + m] * Tm[(c0 + m) * PT + c0 + c];
                Tm[(r0 + r) * PT + c0 + c] = acc;
            }
        }
        __syncthreads();
        float res[PER];
#pragma unroll
        for (int u = 0; u < PER; ++u) {  // X = -T2 Y
            const int e = tid + u * NT;
            res[u] = 0.f;
            if (e < NP * 256) {
                const int p = e >> 8, r = (e >> 4) & 15, c = e & 15;
                const int r0 = (2 * p + 1) * 16, c0 = 2 * p * 16;
                float acc = 0.f;
#pragma unroll
                for (int m = 0; m < 16; ++m) acc += Tm[(r0 + r) * PT + r0 + m] * Tm[(r0 + m) * PT + c0 + c];
                res[u] = -acc;
            }
        }
        __syncthreads();
#pragma unroll
        for (int u = 0; u < PER; ++u) {
            const int e = tid + u * NT;
            if (e < NP * 256) {
                const int p = e >> 8, r = (e >> 4) & 15, c = e & 15;
                Tm[((2 * p + 1) * 16 + r) * PT + 2 * p * 16 + c] = res[u];
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
        __syncthreads();
        for (int t = w; t < NTL; t += NW) {  // Y = A21 T1 into the X slot (X is not read here)
            const int p = t / TPP, ti = (t % TPP) / (n / 16), tj = t % (n / 16);
            const int r0 = (2 * p + 1) * n + ti * 16, c0 = 2 * p * n + tj * 16;
            f32x4 acc = {0.f, 0.f, 0.f, 0.f};
            acc = mma_nn_f32<T>(acc, A + r0 * PT + 2 * p * n, PT, Tm + (2 * p * n) * PT + c0, PT, 0, n);
#pragma unroll
            for (int i = 0; i < 4; ++i) Tm[(r0 + acc_row(i)) * PT + c0 + acc_col()] = acc[i];
        }
        __syncthreads();
        f32x4 res[MAXT];
#pragma unroll
        for (int u = 0; u < MAXT; ++u) {  // X = -T2 Y
            const int t = w + NW * u;
            res[u] = f32x4{0.f, 0.f, 0.f, 0.f};
            if (t < NTL) {
                const int p = t / TPP, ti = (t % TPP) / (n / 16), tj = t % (n / 16);
                const int r0 = (2 * p + 1) * n + ti * 16, c0 = 2 * p * n + tj * 16;
                res[u] = -mma_nn_f32<T>(res[u], Tm + r0 * PT + (2 * p + 1) * n, PT,
                                        Tm + ((2 * p + 1) * n) * PT + c0, PT, 0, n);
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
                for (int i = 0; i < 4; ++i) Tm[(r0 + acc_row(i)) * PT + c0 + acc_col()] = res[u][i];
            }
        }
    }
    __syncthreads();
}

}  // namespace kda
