// kda_prep.hip -- chunk preparation for the chunked KDA forward pass.
//
// One workgroup (4*C threads, C/16 waves) per (chunk, head). Everything it
// computes depends only on the chunk's own inputs, never on the state, so all
// chunks of all sequences run in parallel. Within a chunk of rows r = 0..L-1:
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
// O = QO S0 + Aqk U and the state leaving the chunk is exp(gamma) S0 + KtT U.
// For alpha = 1 it is the WY form of DeltaNet in the essay "22,580: from GPT-2
// to Kimi K3" (yichencityu.github.io, section 6.3: T from the strictly lower
// triangle of diag(beta) K K^T by forward substitution, W = T K_beta,
// U = T V_beta); the exp(g[r] - g[i]) factors are the cumulative decay between
// a write and a later read that the aidehub.top summary describes in its Gated
// DeltaNet section (a multiplicative prefix sum).
//
// exp(g[r] - g[i]) is not a product of two matrices, so the decayed Gram is
// formed as (k exp(g - m)) (k exp(m - g))^T with m = gamma / 2, which keeps both
// factors within exp(+-|gamma|/2); their exponents are clamped to +-85 (fp32
// and bf16 share that range). Entries above the diagonal would carry huge
// factors and are dropped by selection, never by multiplying with a zero mask.
//
// Memory access: each thread owns 8 adjacent channels of C/(4*C/(d/8)) rows and
// issues all of its 16-byte loads before any computation; every output goes
// through LDS and leaves as fully coalesced 16-byte stores, in the
// fragment-ordered layouts the state kernel reads.

#include "kda_internal.hpp"

namespace kda {
namespace {

template <int C, int DK, int DV, typename T> struct PrepCfg {
    static constexpr int NT = 4 * C, NW = NT / 64;
    static constexpr int CGK = DK / 8, RPK = CGK / 4, RGK = NT / CGK;  // key-side thread tiles
    static constexpr int CGV = DV / 8, RPV = CGV / 4;                  // value-side thread tiles
    static constexpr int P64 = 64 + 8;  // pitch of the [C][64] Gram operand blocks
    static constexpr int PT = C + 4;    // pitch of the fp32 [C][C] matrices
    static constexpr size_t SMALL = (size_t)(RGK * DK + C) * 4;
    static constexpr size_t STAGE = (size_t)C * (DK > DV ? DK : DV) * sizeof(T);
    static constexpr size_t GRAM = (size_t)3 * C * P64 * sizeof(T);
    static constexpr size_t MATF = (size_t)C * PT * 4;
    static constexpr size_t OPB = (size_t)64 * C * sizeof(T);
    static constexpr size_t mx(size_t a, size_t b) { return a > b ? a : b; }
    static constexpr size_t REGION = mx(mx(STAGE, GRAM), mx(2 * MATF, MATF + 2 * OPB));
    static constexpr size_t SMEM = SMALL + REGION;
};

__device__ __forceinline__ float clamp85(float x) { return fminf(fmaxf(x, -85.f), 85.f); }

// Lower-triangular 16x16 tile list: tile t <-> (ti, tj), tj <= ti, row by row.
__device__ __forceinline__ void tri_tile(int t, int &ti, int &tj) {
    ti = 0;
    while ((ti + 1) * (ti + 2) / 2 <= t) ++ti;
    tj = t - ti * (ti + 1) / 2;
}

template <typename T> __device__ __forceinline__ void load8(const T *p, float v[8]);
template <> __device__ __forceinline__ void load8<bf16>(const bf16 *p, float v[8]) {
    const bf16x8 x = *reinterpret_cast<const bf16x8 *>(p);
#pragma unroll
    for (int e = 0; e < 8; ++e) v[e] = static_cast<float>(x[e]);
}
template <> __device__ __forceinline__ void load8<float>(const float *p, float v[8]) {
    const f32x4 a = *reinterpret_cast<const f32x4 *>(p);
    const f32x4 b = *reinterpret_cast<const f32x4 *>(p + 4);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        v[e] = a[e];
        v[4 + e] = b[e];
    }
}

// Store 8 values of row r, columns c0..c0+7 (c0 % 8 == 0), of a
// fragment-ordered matrix with R rows.
template <typename T>
__device__ __forceinline__ void frag_store_row8(T *base, int r, int c0, const float v[8], int R) {
    if constexpr (sizeof(T) == 2) {
        bf16x8 x;
#pragma unroll
        for (int e = 0; e < 8; ++e) x[e] = static_cast<bf16>(v[e]);
        *reinterpret_cast<bf16x8 *>(base + frag_off<T>(r, c0, R)) = x;
    } else {
#pragma unroll
        for (int e = 0; e < 8; ++e) base[frag_off<T>(r, c0 + e, R)] = v[e];
    }
}

// Store n consecutive contraction indices k0..k0+n-1 (n = 2 or 4, k0 % n == 0)
// of row r of a fragment-ordered matrix with R rows.
template <typename T, int N>
__device__ __forceinline__ void frag_store_col(T *base, int r, int k0, const float *v, int R) {
    if constexpr (sizeof(T) == 2) {
        bf16 x[N];
#pragma unroll
        for (int i = 0; i < N; ++i) x[i] = static_cast<bf16>(v[i]);
        T *dst = base + frag_off<T>(r, k0, R);
        if constexpr (N == 4) {
            *reinterpret_cast<uint2 *>(dst) = *reinterpret_cast<const uint2 *>(x);
        } else {
            *reinterpret_cast<uint32_t *>(dst) = *reinterpret_cast<const uint32_t *>(x);
        }
    } else {
#pragma unroll
        for (int i = 0; i < N; ++i) base[frag_off<T>(r, k0 + i, R)] = v[i];
    }
}

template <typename T, int NT>
__device__ __forceinline__ void copy_out(T *dst, const T *src, int n) {
    typedef typename Frag<T>::Vec V;
    for (int i = threadIdx.x; i < n / Frag<T>::EPL; i += NT)
        reinterpret_cast<V *>(dst)[i] = reinterpret_cast<const V *>(src)[i];
}

// A-operand fragment group kg of row block `row0` taken from an fp32 row-major
// matrix (pitch ld), rounded to T.
template <typename T>
__device__ __forceinline__ typename Frag<T>::Vec a_frag_f32(const float *M, int ld, int row0, int kg) {
    const int l = threadIdx.x & 63;
    typename Frag<T>::Vec v;
    const float *p = M + (row0 + (l & 15)) * ld + kg * Frag<T>::KG;
    if constexpr (sizeof(T) == 2) {
        const f32x4 a = *reinterpret_cast<const f32x4 *>(p + 8 * (l >> 4));
        const f32x4 b = *reinterpret_cast<const f32x4 *>(p + 8 * (l >> 4) + 4);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            v[e] = static_cast<bf16>(a[e]);
            v[4 + e] = static_cast<bf16>(b[e]);
        }
    } else {
#pragma unroll
        for (int s = 0; s < 4; ++s) v[s] = p[4 * s + (l >> 4)];
    }
    return v;
}

// Tm = (I + A)^{-1} for A strictly lower triangular (C x C, fp32, pitch PT).
// 16x16 diagonal blocks by forward substitution (one thread per column), then
// doubling: [[T1, 0], [X, T2]] with X = -T2 A21 T1, for block sizes 16, 32, 64.
template <int C, int PT, typename T, int NT>
__device__ void unit_lower_inverse(const float *A, float *Tm) {
    const int tid = threadIdx.x;
    for (int e = tid; e < C * PT; e += NT) Tm[e] = 0.f;
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

template <int C, int DK, int DV, typename T>
__global__ __launch_bounds__(4 * C) void kda_prep_kernel(PrepArgs a) {
    typedef PrepCfg<C, DK, DV, T> P;
    typedef Frag<T> F;
    constexpr int NT = P::NT, NW = P::NW, RPK = P::RPK, RPV = P::RPV;
    constexpr int P64 = P::P64, PT = P::PT;
    constexpr int TR = C / 16, NTILE = TR * (TR + 1) / 2, TPW = (NTILE + NW - 1) / NW;

    extern __shared__ __align__(16) unsigned char smem[];
    float *tot = reinterpret_cast<float *>(smem);  // [RGK][DK] row-group sums of log alpha
    float *bet = tot + P::RGK * DK;                 // [C]
    unsigned char *R = smem + P::SMALL;
    T *stage = reinterpret_cast<T *>(R);            // output staging (fragment order)
    T *Kp = reinterpret_cast<T *>(R);               // [C][P64] k exp(g - m), one 64-channel block
    T *Km = Kp + C * P64;                           // [C][P64] k exp(m - g)
    T *Qp = Km + C * P64;                           // [C][P64] scale q exp(g - m)
    float *Tm = reinterpret_cast<float *>(R);       // [C][PT]
    float *Am = Tm + C * PT;                        // [C][PT]
    T *OpB = reinterpret_cast<T *>(R + P::MATF);    // [64][C] B operand block, fragment order
    T *Wst = reinterpret_cast<T *>(R + P::MATF + P::OPB);  // [C][64] W block, fragment order

    const int j = blockIdx.x, h = blockIdx.y;
    int s, t0, L;
    if (!a.map.locate(j, s, t0, L)) return;  // past the last chunk (same for the whole block)
    (void)s;
    const int tid = threadIdx.x, w = tid >> 6;
    const int H = a.H;
    const size_t jh = (size_t)j * H + h;
    const int rk0 = (tid / P::CGK) * RPK, ck0 = 8 * (tid % P::CGK);  // key tile: rows, channels
    const int rv0 = (tid / P::CGV) * RPV, cv0 = 8 * (tid % P::CGV);  // value tile

    // ---- 0. the key-side global loads of this thread, before anything else
    float kr[RPK][8], qr[RPK][8], g[RPK][8], bk[RPK];
#pragma unroll
    for (int i = 0; i < RPK; ++i) {
        const int row = rk0 + i;
        if (row < L) {
            const size_t o = ((size_t)(t0 + row) * H + h) * DK + ck0;
            load8<T>(static_cast<const T *>(a.k) + o, kr[i]);
            load8<T>(static_cast<const T *>(a.q) + o, qr[i]);
            load8<float>(a.log_alpha + o, g[i]);
            bk[i] = a.beta[(size_t)(t0 + row) * H + h];
        } else {
#pragma unroll
            for (int e = 0; e < 8; ++e) kr[i][e] = qr[i][e] = g[i][e] = 0.f;
            bk[i] = 0.f;
        }
    }
    if (tid < C) bet[tid] = (tid < L) ? a.beta[(size_t)(t0 + tid) * H + h] : 0.f;

    // ---- 1. inclusive running sum of log alpha: within the thread's rows, then
    //         across row groups (sums added in row-group order, so the last row's
    //         g equals gamma exactly)
#pragma unroll
    for (int i = 1; i < RPK; ++i)
#pragma unroll
        for (int e = 0; e < 8; ++e) g[i][e] += g[i - 1][e];
#pragma unroll
    for (int e = 0; e < 8; ++e) tot[(tid / P::CGK) * DK + ck0 + e] = g[RPK - 1][e];
    __syncthreads();
    float off[8], gam[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) off[e] = gam[e] = 0.f;
    for (int gg = 0; gg < P::RGK; ++gg) {
        const bool before = gg < tid / P::CGK;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const float x = tot[gg * DK + ck0 + e];
            if (before) off[e] += x;
            gam[e] += x;
        }
    }

#pragma unroll
    for (int i = 0; i < RPK; ++i)
#pragma unroll
        for (int e = 0; e < 8; ++e) g[i][e] += off[e];
    float mid[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) mid[e] = 0.5f * gam[e];

    T *chunk_QO = static_cast<T *>(a.buf.QO) + jh * C * DK;
    T *chunk_KtT = static_cast<T *>(a.buf.KtT) + jh * DK * C;
    T *chunk_Aqk = static_cast<T *>(a.buf.Aqk) + jh * C * C;
    T *chunk_W = static_cast<T *>(a.buf.W) + jh * C * DK;
    T *chunk_U = static_cast<T *>(a.buf.U) + jh * C * DV;

    // ---- 2. QO = scale q exp(g)  (A operand [C][DK])
#pragma unroll
    for (int i = 0; i < RPK; ++i) {
        float x[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) x[e] = a.scale * qr[i][e] * __expf(g[i][e]);
        frag_store_row8<T>(stage, rk0 + i, ck0, x, C);
    }
    __syncthreads();
    copy_out<T, NT>(chunk_QO, stage, C * DK);
    __syncthreads();

    // ---- 3. KtT = (k exp(gamma - g))^T  (A operand [DK][C])
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        float x[RPK];
#pragma unroll
        for (int i = 0; i < RPK; ++i) x[i] = kr[i][e] * __expf(gam[e] - g[i][e]);
        frag_store_col<T, RPK>(stage, ck0 + e, rk0, x, DK);
    }
    __syncthreads();
    copy_out<T, NT>(chunk_KtT, stage, DK * C);
    __syncthreads();

    // ---- 4. decayed Gram matrices, 64 key channels at a time
    f32x4 akk[TPW], aqk[TPW];
#pragma unroll
    for (int t = 0; t < TPW; ++t) akk[t] = aqk[t] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int b = 0; b < DK / 64; ++b) {
        if (ck0 / 64 == b) {
            const int cl = ck0 - 64 * b;
#pragma unroll
            for (int i = 0; i < RPK; ++i) {
                float xp[8], xm[8], xq[8];
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    const float ep = __expf(clamp85(g[i][e] - mid[e]));
                    const float em = __expf(clamp85(mid[e] - g[i][e]));
                    xp[e] = kr[i][e] * ep;
                    xm[e] = kr[i][e] * em;
                    xq[e] = a.scale * qr[i][e] * ep;
                }
                T *dp = Kp + (rk0 + i) * P64 + cl, *dm = Km + (rk0 + i) * P64 + cl, *dq = Qp + (rk0 + i) * P64 + cl;
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    dp[e] = from_f32<T>(xp[e]);
                    dm[e] = from_f32<T>(xm[e]);
                    dq[e] = from_f32<T>(xq[e]);
                }
            }
        }
        __syncthreads();
#pragma unroll
        for (int t = 0; t < TPW; ++t) {
            const int tile = w + NW * t;
            if (tile < NTILE) {
                int ti, tj;
                tri_tile(tile, ti, tj);
                akk[t] = mma_nt<T>(akk[t], Kp + ti * 16 * P64, P64, Km + tj * 16 * P64, P64, 0, 64);
                aqk[t] = mma_nt<T>(aqk[t], Qp + ti * 16 * P64, P64, Km + tj * 16 * P64, P64, 0, 64);
            }
        }
        __syncthreads();
    }

    // ---- 5. A (strictly lower, rows scaled by beta) -> fp32 LDS;
    //         Aqk (lower, diagonal included) -> memory (A operand [C][C])
    for (int e = tid; e < C * PT; e += NT) Am[e] = 0.f;
    for (int e = tid; e < C * C; e += NT) stage[e] = from_f32<T>(0.f);
    __syncthreads();
#pragma unroll
    for (int t = 0; t < TPW; ++t) {
        const int tile = w + NW * t;
        if (tile < NTILE) {
            int ti, tj;
            tri_tile(tile, ti, tj);
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int r = ti * 16 + acc_row(i), c = tj * 16 + acc_col();
                Am[r * PT + c] = (c < r) ? bet[r] * akk[t][i] : 0.f;
                stage[frag_off<T>(r, c, C)] = from_f32<T>((c <= r) ? aqk[t][i] : 0.f);
            }
        }
    }
    __syncthreads();
    copy_out<T, NT>(chunk_Aqk, stage, C * C);
    __syncthreads();

    // ---- 6. T = (I + A)^{-1}, with the value rows in flight meanwhile
    float vx[RPV][8], bv[RPV];
#pragma unroll
    for (int i = 0; i < RPV; ++i) {
        const int row = rv0 + i;
        if (row < L) {
            load8<T>(static_cast<const T *>(a.v) + ((size_t)(t0 + row) * H + h) * DV + cv0, vx[i]);
            bv[i] = a.beta[(size_t)(t0 + row) * H + h];
        } else {
#pragma unroll
            for (int e = 0; e < 8; ++e) vx[i][e] = 0.f;
            bv[i] = 0.f;
        }
    }
    unit_lower_inverse<C, PT, T, NT>(Am, Tm);

    // ---- 7. W = T (beta k exp(g)) and U~ = T (beta v), 64 output columns at a time
#pragma unroll
    for (int b = 0; b < DK / 64 + DV / 64; ++b) {
        const bool isW = b < DK / 64;
        const int cb = isW ? b : b - DK / 64;
        if (isW && ck0 / 64 == cb) {
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                float x[RPK];
#pragma unroll
                for (int i = 0; i < RPK; ++i) x[i] = bk[i] * kr[i][e] * __expf(g[i][e]);
                frag_store_col<T, RPK>(OpB, ck0 - 64 * cb + e, rk0, x, 64);
            }
        }
        if (!isW && cv0 / 64 == cb) {
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                float x[RPV];
#pragma unroll
                for (int i = 0; i < RPV; ++i) x[i] = bv[i] * vx[i][e];
                frag_store_col<T, RPV>(OpB, cv0 - 64 * cb + e, rv0, x, 64);
            }
        }
        __syncthreads();
        const int kgmax = ((w + 1) * 16 + F::KG - 1) / F::KG;  // T is lower triangular
#pragma unroll
        for (int tn = 0; tn < 4; ++tn) {
            f32x4 acc = {0.f, 0.f, 0.f, 0.f};
            for (int kg = 0; kg < kgmax; ++kg)
                acc = F::mma(acc, a_frag_f32<T>(Tm, PT, w * 16, kg), frag_load<T>(OpB, kg, tn, 64));
            if (isW) {
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    Wst[frag_off<T>(w * 16 + acc_row(i), tn * 16 + acc_col(), C)] = from_f32<T>(acc[i]);
            } else {
                T *dst = chunk_U + acc_tile_off(w, (64 * cb + 16 * tn) >> 4, DV);
                if constexpr (sizeof(T) == 2) {
                    bf16 x[4];
#pragma unroll
                    for (int i = 0; i < 4; ++i) x[i] = static_cast<bf16>(acc[i]);
                    *reinterpret_cast<uint2 *>(dst) = *reinterpret_cast<const uint2 *>(x);
                } else {
                    *reinterpret_cast<f32x4 *>(dst) = acc;
                }
            }
        }
        __syncthreads();
        if (isW) {
            copy_out<T, NT>(chunk_W + 64 * cb * C, Wst, C * 64);
            __syncthreads();
        }
    }
    if (tid < DK / 8 && rk0 == 0) {
#pragma unroll
        for (int e = 0; e < 8; ++e) a.buf.eg[jh * DK + ck0 + e] = __expf(gam[e]);
    }
}

template <int C, int DK, int DV, typename T>
hipError_t launch_prep_t(const PrepArgs &a, int n_chunks_grid, hipStream_t stream) {
    constexpr size_t smem = PrepCfg<C, DK, DV, T>::SMEM;
    static_assert(smem <= 160 * 1024, "prep LDS budget");
    auto kern = kda_prep_kernel<C, DK, DV, T>;
    hipError_t err = hipFuncSetAttribute(reinterpret_cast<const void *>(kern),
                                         hipFuncAttributeMaxDynamicSharedMemorySize, (int)smem);
    if (err != hipSuccess) return err;
    hipLaunchKernelGGL(kern, dim3(n_chunks_grid, a.H), dim3(4 * C), smem, stream, a);
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
