// kda_prep.hip -- chunk preparation for the chunked KDA forward pass.
//
// One workgroup (4 waves) per (chunk, head). Everything it computes depends
// only on the chunk's own inputs, never on the state, so all chunks of all
// sequences run in parallel. Within a chunk of rows r = 0..L-1 (L <= C):
//
//   g[r]    = sum_{j<=r} log_alpha[j]           per key channel, inclusive
//   gamma   = g[L-1]                            the chunk's total decay
//   A[r,i]  = beta_r sum_c k[r,c] k[i,c] exp(g[r,c] - g[i,c])          (i < r)
//   T       = (I + A)^{-1}                      unit lower triangular
//   W       = T (beta k exp(g))                 U~ = T (beta v)
//   QO      = scale q exp(g)                    KtT = (k exp(gamma - g))^T
//   Aqk     = scale sum_c q[r,c] k[i,c] exp(g[r,c] - g[i,c])           (i <= r)
//
// These follow from unrolling the recurrence over one chunk: with S0 the state
// entering the chunk, the corrected writes are U = U~ - W S0, the outputs are
// O = QO S0 + Aqk U and the state leaving the chunk is
// exp(gamma) S0 + KtT U. For alpha = 1 it is the WY form of DeltaNet in the
// essay "22,580: from GPT-2 to Kimi K3" (yichencityu.github.io, section 6.3:
// T from the strictly lower triangle of diag(beta) K K^T by forward
// substitution, W = T K_beta, U = T V_beta); the exp(g[r] - g[i]) factors are
// the cumulative decay between a write and a later read that the aidehub.top
// summary describes in its Gated DeltaNet section (a multiplicative prefix sum).
//
// exp(g[r] - g[i]) is not a product of two matrices, so the decayed Gram is
// formed as (k exp(g - m)) (k exp(m - g))^T with m = gamma / 2, which keeps both
// factors within exp(+-|gamma|/2) and needs no per-element exponential; the
// factors' exponents are clamped to +-85 (fp32 and bf16 share that range).
// Entries above the diagonal would carry huge factors and are dropped by
// selection, never by multiplying with a zero mask.

#include "kda_internal.hpp"

namespace kda {
namespace {

constexpr int kThreads = 256;

// Row pitches (in elements) of the LDS tiles. The +8 / +4 padding spreads rows
// over LDS banks while keeping 16-byte alignment for vector reads.
template <int C> struct PrepPitch {
    static constexpr int P64 = 64 + 8;  // [C][64] operand tiles
    static constexpr int PC = C + 8;    // [64][C] transposed operand tiles
    static constexpr int PT = C + 4;    // [C][C] fp32 matrices
};

template <int C, int DK, typename T> constexpr size_t prep_smem_bytes() {
    typedef PrepPitch<C> P;
    constexpr size_t small = (size_t)(5 * DK + C) * sizeof(float);
    constexpr size_t gram = (size_t)(3 * C * P::P64 + 64 * P::PC) * sizeof(T);
    constexpr size_t tmat = (size_t)C * P::PT * sizeof(float);
    constexpr size_t opt = (size_t)64 * P::PC * sizeof(T);
    constexpr size_t solve = tmat + (tmat > opt ? tmat : opt);
    return small + (gram > solve ? gram : solve);
}

__device__ __forceinline__ float clamp85(float x) { return fminf(fmaxf(x, -85.f), 85.f); }

// Lower-triangular 16x16 tile list: tile t <-> (ti, tj), tj <= ti, row by row.
__device__ __forceinline__ void tri_tile(int t, int &ti, int &tj) {
    ti = 0;
    while ((ti + 1) * (ti + 2) / 2 <= t) ++ti;
    tj = t - ti * (ti + 1) / 2;
}

// Tm = (I + A)^{-1} for A strictly lower triangular (C x C, fp32, pitch PT).
// 16x16 diagonal blocks by forward substitution (one thread per column), then
// doubling: [[T1, 0], [X, T2]] with X = -T2 A21 T1, for block sizes 16, 32, 64.
template <int C, int PT, typename T>
__device__ void unit_lower_inverse(const float *A, float *Tm) {
    const int tid = threadIdx.x;
    for (int e = tid; e < C * PT; e += kThreads) Tm[e] = 0.f;
    __syncthreads();
    if (tid < C) {
        const int base = tid & ~15, c = tid & 15;
        float x[16];
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            float acc = 0.f;
#pragma unroll
            for (int i = 0; i < 16; ++i)
                if (i < r) acc += A[(base + r) * PT + base + i] * x[i];
            x[r] = (r < c) ? 0.f : (r == c ? 1.f : -acc);
        }
#pragma unroll
        for (int r = 0; r < 16; ++r) Tm[(base + r) * PT + base + c] = x[r];
    }

    // Level n = 16 on the vector ALUs: C/32 pairs of 16x16 blocks.
    {
        constexpr int NP = C / 32;
        constexpr int PER = (NP * 256 + kThreads - 1) / kThreads;
        __syncthreads();
        // Y = A21 T1, written into the X slot
#pragma unroll
        for (int u = 0; u < PER; ++u) {
            const int e = tid + u * kThreads;
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
        for (int u = 0; u < PER; ++u) {
            const int e = tid + u * kThreads;
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
            const int e = tid + u * kThreads;
            if (e < NP * 256) {
                const int p = e >> 8, r = (e >> 4) & 15, c = e & 15;
                Tm[((2 * p + 1) * 16 + r) * PT + 2 * p * 16 + c] = res[u];
            }
        }
    }

    // Levels n = 32, 64 on the matrix cores: (n/16)^2 output tiles per pair.
    const int w = tid >> 6;
#pragma unroll
    for (int n = 32; 2 * n <= C; n *= 2) {
        const int NP = C / (2 * n), TPP = (n / 16) * (n / 16), NT = NP * TPP;
        constexpr int MAXT = (C * 64 / 512 + 3) / 4;  // tiles per wave at the largest level
        __syncthreads();
        for (int t = w; t < NT; t += 4) {  // Y = A21 T1 into the X slot (X region is not read)
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
            const int t = w + 4 * u;
            res[u] = f32x4{0.f, 0.f, 0.f, 0.f};
            if (t < NT) {
                const int p = t / TPP, ti = (t % TPP) / (n / 16), tj = t % (n / 16);
                const int r0 = (2 * p + 1) * n + ti * 16, c0 = 2 * p * n + tj * 16;
                res[u] = -mma_nn_f32<T>(res[u], Tm + r0 * PT + (2 * p + 1) * n, PT,
                                        Tm + ((2 * p + 1) * n) * PT + c0, PT, 0, n);
            }
        }
        __syncthreads();
#pragma unroll
        for (int u = 0; u < MAXT; ++u) {
            const int t = w + 4 * u;
            if (t < NT) {
                const int p = t / TPP, ti = (t % TPP) / (n / 16), tj = t % (n / 16);
                const int r0 = (2 * p + 1) * n + ti * 16, c0 = 2 * p * n + tj * 16;
#pragma unroll
                for (int i = 0; i < 4; ++i) Tm[(r0 + acc_row(i)) * PT + c0 + acc_col()] = res[u][i];
            }
        }
    }
    __syncthreads();
}

template <int C, int DK, int DV, typename T>
__global__ __launch_bounds__(kThreads) void kda_prep_kernel(PrepArgs a) {
    typedef PrepPitch<C> P;
    constexpr int RS = C / 4;  // rows per wave in the channel scan
    constexpr int NKB = DK / 64, NVB = DV / 64;
    constexpr int TR = C / 16, NTILE = TR * (TR + 1) / 2, TPW = (NTILE + 3) / 4;
    constexpr int KK = Mma<T>::kK;

    extern __shared__ __align__(16) unsigned char smem[];
    float *segtot = reinterpret_cast<float *>(smem);  // [4][DK]
    float *gam = segtot + 4 * DK;                       // [DK]
    float *bet = gam + DK;                              // [C]
    unsigned char *un = reinterpret_cast<unsigned char *>(bet + C);
    T *Kp = reinterpret_cast<T *>(un);                  // [C][P64]  k exp(g - m)
    T *Km = Kp + C * P::P64;                            // [C][P64]  k exp(m - g)
    T *Qp = Km + C * P::P64;                            // [C][P64]  scale q exp(g - m)
    T *KtS = Qp + C * P::P64;                           // [64][PC]  staging of KtT
    float *Tm = reinterpret_cast<float *>(un);          // [C][PT]   (after the Gram phase)
    float *Am = Tm + C * P::PT;                         // [C][PT]
    T *OpT = reinterpret_cast<T *>(Am);                 // [64][PC]  (after the solve, over Am)

    const int j = blockIdx.x, h = blockIdx.y;
    int s, t0, L;
    if (!a.map.locate(j, s, t0, L)) return;  // past the last chunk (same for the whole block)
    (void)s;
    const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63;
    const int H = a.H;
    const T *q = static_cast<const T *>(a.q);
    const T *k = static_cast<const T *>(a.k);
    const T *v = static_cast<const T *>(a.v);
    const size_t jh = (size_t)j * H + h;
    T *Wg = static_cast<T *>(a.buf.W) + jh * C * DK;
    T *Ug = static_cast<T *>(a.buf.U) + jh * C * DV;
    T *QOg = static_cast<T *>(a.buf.QO) + jh * C * DK;
    T *KtTg = static_cast<T *>(a.buf.KtT) + jh * DK * C;
    T *Aqkg = static_cast<T *>(a.buf.Aqk) + jh * C * C;

    if (tid < C) bet[tid] = (tid < L) ? a.beta[(size_t)(t0 + tid) * H + h] : 0.f;

    // ---- 1. inclusive running sum of log alpha per key channel
    // thread (w, lane): channels lane + 64 b, rows w*RS .. w*RS + RS - 1
    float g[NKB][RS];
#pragma unroll
    for (int b = 0; b < NKB; ++b) {
        float run = 0.f;
#pragma unroll
        for (int r = 0; r < RS; ++r) {
            const int row = w * RS + r;
            const float la = (row < L) ? a.log_alpha[((size_t)(t0 + row) * H + h) * DK + b * 64 + lane] : 0.f;
            run += la;
            g[b][r] = run;
        }
        segtot[w * DK + b * 64 + lane] = run;
    }
    __syncthreads();
    float gtot[NKB];
#pragma unroll
    for (int b = 0; b < NKB; ++b) {
        const int c = b * 64 + lane;
        float off = 0.f, tot = 0.f;
#pragma unroll
        for (int ww = 0; ww < 4; ++ww) {
            const float x = segtot[ww * DK + c];
            if (ww < w) off += x;
            tot += x;
        }
#pragma unroll
        for (int r = 0; r < RS; ++r) g[b][r] += off;
        gtot[b] = tot;
        if (w == 0) gam[c] = tot;
    }

    // ---- 2. decayed Gram matrices, accumulated over 64-channel blocks
    f32x4 akk[TPW], aqk[TPW];
#pragma unroll
    for (int t = 0; t < TPW; ++t) {
        akk[t] = f32x4{0.f, 0.f, 0.f, 0.f};
        aqk[t] = f32x4{0.f, 0.f, 0.f, 0.f};
    }
#pragma unroll
    for (int b = 0; b < NKB; ++b) {
        const int c = b * 64 + lane;
        const float m = 0.5f * gtot[b];
#pragma unroll
        for (int r = 0; r < RS; ++r) {
            const int row = w * RS + r;
            const size_t src = ((size_t)(t0 + row) * H + h) * DK + c;
            const float kv = (row < L) ? to_f32(k[src]) : 0.f;
            const float qv = (row < L) ? to_f32(q[src]) : 0.f;
            const float x = g[b][r];
            const float ep = expf(clamp85(x - m));
            const float em = expf(clamp85(m - x));
            Kp[row * P::P64 + lane] = from_f32<T>(kv * ep);
            Km[row * P::P64 + lane] = from_f32<T>(kv * em);
            Qp[row * P::P64 + lane] = from_f32<T>(a.scale * qv * ep);
            QOg[row * DK + c] = from_f32<T>(a.scale * qv * expf(x));
            KtS[lane * P::PC + row] = from_f32<T>(kv * expf(gtot[b] - x));
        }
        __syncthreads();
        for (int e = tid; e < 64 * C; e += kThreads) {
            const int cc = e / C, rr = e - cc * C;
            KtTg[(b * 64 + cc) * C + rr] = KtS[cc * P::PC + rr];
        }
#pragma unroll
        for (int t = 0; t < TPW; ++t) {
            const int tile = w + 4 * t;
            if (tile < NTILE) {
                int ti, tj;
                tri_tile(tile, ti, tj);
                akk[t] = mma_nt<T>(akk[t], Kp + ti * 16 * P::P64, P::P64, Km + tj * 16 * P::P64, P::P64, 0, 64);
                aqk[t] = mma_nt<T>(aqk[t], Qp + ti * 16 * P::P64, P::P64, Km + tj * 16 * P::P64, P::P64, 0, 64);
            }
        }
        __syncthreads();
    }

    // ---- 3. A (strictly lower, rows scaled by beta) into LDS; Aqk (lower) to memory
    for (int e = tid; e < C * P::PT; e += kThreads) Am[e] = 0.f;
    __syncthreads();
#pragma unroll
    for (int t = 0; t < TPW; ++t) {
        const int tile = w + 4 * t;
        if (tile < NTILE) {
            int ti, tj;
            tri_tile(tile, ti, tj);
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int r = ti * 16 + acc_row(i), c = tj * 16 + acc_col();
                Am[r * P::PT + c] = (c < r) ? bet[r] * akk[t][i] : 0.f;
                Aqkg[r * C + c] = from_f32<T>((c <= r) ? aqk[t][i] : 0.f);
            }
        }
    }
    for (int e = tid; e < C * C; e += kThreads) {
        const int r = e / C, c = e - r * C;
        if ((c >> 4) > (r >> 4)) Aqkg[e] = from_f32<T>(0.f);
    }
    __syncthreads();

    // ---- 4. T = (I + A)^{-1}
    unit_lower_inverse<C, P::PT, T>(Am, Tm);

    // ---- 5. W = T (beta k exp(g)) and U~ = T (beta v), 64 output columns at a time
    constexpr int WPW = C / 16;  // output tiles per wave per 64-column block
#pragma unroll
    for (int b = 0; b < NKB + NVB; ++b) {
        const bool isW = b < NKB;
        const int cb = isW ? b : b - NKB;
        const int c = cb * 64 + lane;
#pragma unroll
        for (int r = 0; r < RS; ++r) {
            const int row = w * RS + r;
            float val = 0.f;
            if (row < L) {
                if (isW) {
                    val = bet[row] * to_f32(k[((size_t)(t0 + row) * H + h) * DK + c]) * expf(g[isW ? b : 0][r]);
                } else {
                    val = bet[row] * to_f32(v[((size_t)(t0 + row) * H + h) * DV + c]);
                }
            }
            OpT[lane * P::PC + row] = from_f32<T>(val);
        }
        __syncthreads();
#pragma unroll
        for (int t = 0; t < WPW; ++t) {
            const int tile = w * WPW + t;
            const int ti = tile >> 2, tn = tile & 3;
            const int kmax = min(C, ((ti + 1) * 16 + KK - 1) / KK * KK);
            f32x4 acc = {0.f, 0.f, 0.f, 0.f};
            acc = mma_nt_f32a<T>(acc, Tm + ti * 16 * P::PT, P::PT, OpT + tn * 16 * P::PC, P::PC, 0, kmax);
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int r = ti * 16 + acc_row(i), cc = cb * 64 + tn * 16 + acc_col();
                if (isW) Wg[r * DK + cc] = from_f32<T>(acc[i]);
                else Ug[r * DV + cc] = from_f32<T>(acc[i]);
            }
        }
        __syncthreads();
    }
    if (tid < DK) a.buf.eg[jh * DK + tid] = expf(gam[tid]);
}

template <int C, int DK, int DV, typename T>
hipError_t launch_prep_t(const PrepArgs &a, int n_chunks_grid, hipStream_t stream) {
    constexpr size_t smem = prep_smem_bytes<C, DK, T>();
    static_assert(smem <= 160 * 1024, "prep LDS budget");
    auto kern = kda_prep_kernel<C, DK, DV, T>;
    hipError_t err = hipFuncSetAttribute(reinterpret_cast<const void *>(kern),
                                         hipFuncAttributeMaxDynamicSharedMemorySize, (int)smem);
    if (err != hipSuccess) return err;
    hipLaunchKernelGGL(kern, dim3(n_chunks_grid, a.H), dim3(kThreads), smem, stream, a);
    return hipGetLastError();
}

template <int C, typename T>
hipError_t dispatch_d(const PrepArgs &a, int dk, int dv, int n, hipStream_t st) {
    if (dk == 64 && dv == 64) return launch_prep_t<C, 64, 64, T>(a, n, st);
    if (dk == 64 && dv == 128) return launch_prep_t<C, 64, 128, T>(a, n, st);
    if (dk == 128 && dv == 64) return launch_prep_t<C, 128, 64, T>(a, n, st);
    return launch_prep_t<C, 128, 128, T>(a, n, st);
}

// Sequence ranges and chunk offsets of packed sequences. Sequence s spans
// [tb, te) with tb = clamp(cu[s], end of sequence s-1, T) and te = clamp(cu[s+1],
// tb, T): ordered, non-overlapping and inside the token range whatever the table
// holds. off[s] = sum_{s' < s} ceil((te - tb) / C) <= ceil(T / C) + n_seqs.
// One thread; the loop is over sequences only.
__global__ void kda_chunk_offsets_kernel(const int32_t *cu, int n_seqs, int T_total, int C,
                                         int32_t *off, int32_t *tb_out, int32_t *te_out) {
    if (threadIdx.x != 0 || blockIdx.x != 0) return;
    int acc = 0, prev_end = 0;
    for (int s = 0; s < n_seqs; ++s) {
        const int tb = min(max(cu[s], prev_end), T_total);
        const int te = min(max(cu[s + 1], tb), T_total);
        off[s] = acc;
        tb_out[s] = tb;
        te_out[s] = te;
        acc += (te - tb + C - 1) / C;
        prev_end = te;
    }
    off[n_seqs] = acc;
}

}  // namespace

hipError_t launch_chunk_offsets(const int32_t *cu, int n_seqs, int T_total, int C, int32_t *off,
                                int32_t *tb, int32_t *te, hipStream_t stream) {
    hipLaunchKernelGGL(kda_chunk_offsets_kernel, dim3(1), dim3(64), 0, stream, cu, n_seqs, T_total,
                       C, off, tb, te);
    return hipGetLastError();
}

hipError_t launch_prep(const PrepArgs &a, int C, int dk, int dv, bool bf16, int n_chunks_grid,
                       hipStream_t stream) {
    if (C == 64) return bf16 ? dispatch_d<64, kda::bf16>(a, dk, dv, n_chunks_grid, stream)
                             : dispatch_d<64, float>(a, dk, dv, n_chunks_grid, stream);
    return bf16 ? dispatch_d<128, kda::bf16>(a, dk, dv, n_chunks_grid, stream)
                : dispatch_d<128, float>(a, dk, dv, n_chunks_grid, stream);
}

}  // namespace kda
