// kda_bwd.hip -- the chunked backward pass of the KDA recurrence: the gradients
// of a loss with respect to q, k, v, log alpha, beta and the initial state, from
// its gradients with respect to every output and to the final state.
//
// The pages derive no gradient. This pass is the reverse-mode derivative of the
// chunked forward (the chunk form of the essay "22,580: from GPT-2 to Kimi K3"
// sections 6.2-6.3 with the per-channel decay of its Gated DeltaNet section),
// taken identity by identity. Per chunk of C rows, with the prefix
// g = cumsum(log alpha) inside the chunk, gamma = g[C-1], m = gamma / 2, the
// scale s and the state S at the chunk's start:
//
//   P = k e^(g-m),  N = k e^(m-g),  Qe = q e^(g-m),  R = k e^(gamma-g)
//   A = strict_lower(diag(beta) P N^T),  T = (I + A)^-1
//   Bk = diag(beta) k e^g,  Bv = diag(beta) v,  W = T Bk,  U~ = T Bv
//   QO = s q e^g,  Aqk = s lower(Qe N^T)
//   U = U~ - W S,  O = QO S + Aqk U,  S' = Diag(e^gamma) S + R^T U
//
// Given dO and dS' (the loss gradient with respect to the state at the chunk's
// end):
//
//   dU = Aqk^T dO + R dS'
//   dS = QO^T dO + Diag(e^gamma) dS' - W^T dU          (the reverse recursion)
//   dQO = dO S^T, dAqk = lower(dO U^T), dR = U dS'^T, dW = -dU S^T
//   dT = dU Bv^T + dW Bk^T, dBv = T^T dU, dBk = T^T dW
//   dA = strict_lower(-T^T dT T^T)
//   dbeta = rowsum(dBv * v) + rowsum(dBk * k e^g) + rowsum(dA * P N^T)
//   dv = diag(beta) dBv
//   dP = diag(beta) dA N,  dN = (diag(beta) dA)^T P + s dAqk^T Qe,  dQe = s dAqk N
//   dq = s dQO e^g + dQe e^(g-m)
//   dk = diag(beta) dBk e^g + dP e^(g-m) + dN e^(m-g) + dR e^(gamma-g)
//   dg = s dQO q e^g + dQe Qe + diag(beta) dBk k e^g + dP P - dN N - dR R
//   dgamma = colsum(dR * R) + e^gamma rowsum(dS' * S), added to dg's last row
//   dlog_alpha = the reverse prefix sum of dg down the chunk
//
// (m cancels in P N^T and Qe N^T and carries no gradient.) Rows past a
// sequence's end are zero in q, k, v, dO, beta and log alpha, which leaves every
// quantity of the valid rows unchanged.
//
// Four kernels: (1) the chunk-local forward quantities T, Aqk^T, W, U~, R, QO and
// e^gamma, in parallel over (chunk, head); (2) the chunk-start states, in order
// over the chunks of each (sequence, head, 16 state columns); (3) the state
// gradients dS', in reverse order likewise, and dh0; (4) the chunk-local
// gradients, in parallel over (chunk, head). q, k, v, dout and dq, dk, dv are fp32
// or bf16; everything else, and all arithmetic, is fp32, the chunk
// matrices in a per-workgroup scratch in global memory, the products on the
// matrix cores in fp32 with their operands read straight from that memory: the
// direct form of this pass, not tuned further.

#include "kda_bwd.hpp"

namespace kda {
namespace {

constexpr int C = kBwdChunk;

// Staging buffers of gemm in LDS: all of op(A) (C x K) and op(B) (K x N), K and N
// up to 128 (rows padded against bank conflicts).
constexpr int kMaxK = 128;
struct Stage {
    float a[C][kMaxK + 1];
    float b[kMaxK][128 + 4];
};

// D = alpha op(A) op(B) + beta D over the workgroup (beta = 0 overwrites D);
// every thread of the workgroup calls it. op(A) is C x K: A row-major with leading
// dimension lda, or stored K x C (TA). op(B) is K x N: B stored K x N with leading
// dimension ldb, or N x K (TB). N is 64 or 128, K 64 or 128. Both operands are
// first copied whole into LDS (all loads in flight at once), then each wave
// computes 16 x 16 tiles of D on the matrix cores (v_mfma_f32_16x16x4_f32: lane l
// supplies op(A)[l%16][k + l/16] and op(B)[k + l/16][l%16] and holds
// D[4 (l/16) + i][l%16]). A later call with the same N gives every lane the same
// elements of D, so it may accumulate into D without a barrier of its own.
template <bool TA, bool TB, int N, int K>
__device__ void gemm(Stage &st, float alpha, const float *A, int lda, const float *B, int ldb, float beta, float *D,
                     int ldd) {
    static_assert((N == 64 || N == 128) && (K == 64 || K == 128), "gemm shape");
    constexpr int M = C, tn = N / 16, tiles = (M / 16) * tn, kMaxTiles = tiles / (kBwdThreads / 64);
    const int tid = threadIdx.x, l = tid & 63, w = tid >> 6, r = l & 15, kq = l >> 4;
    // op(A) into st.a[m][k], four consecutive elements of A per load
    for (int idx = tid; idx < M * K / 4; idx += kBwdThreads) {
        if (TA) {  // A row kk holds op(A)[.][kk]
            const int kk = idx / (M / 4), m = 4 * (idx % (M / 4));
            const f32x4 v = *reinterpret_cast<const f32x4 *>(A + kk * lda + m);
#pragma unroll
            for (int e = 0; e < 4; ++e) st.a[m + e][kk] = v[e];
        } else {
            const int m = idx / (K / 4), kk = 4 * (idx % (K / 4));
            const f32x4 v = *reinterpret_cast<const f32x4 *>(A + m * lda + kk);
#pragma unroll
            for (int e = 0; e < 4; ++e) st.a[m][kk + e] = v[e];
        }
    }
    __builtin_amdgcn_sched_barrier(0);  // op(A)'s loads before op(B)'s: fewer registers in flight
    // op(B) into st.b[k][n]
    for (int idx = tid; idx < K * N / 4; idx += kBwdThreads) {
        if (TB) {  // B row n holds op(B)[.][n]
            const int n = idx / (K / 4), kk = 4 * (idx % (K / 4));
            const f32x4 v = *reinterpret_cast<const f32x4 *>(B + n * ldb + kk);
#pragma unroll
            for (int e = 0; e < 4; ++e) st.b[kk + e][n] = v[e];
        } else {
            const int kk = idx / (N / 4), n = 4 * (idx % (N / 4));
            const f32x4 v = *reinterpret_cast<const f32x4 *>(B + kk * ldb + n);
#pragma unroll
            for (int e = 0; e < 4; ++e) st.b[kk][n + e] = v[e];
        }
    }
    __syncthreads();
#pragma unroll
    for (int q = 0; q < kMaxTiles; ++q) {
        const int t = w + 4 * q, i0 = (t / tn) * 16, j0 = (t % tn) * 16;
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll 4
        for (int k = 0; k < K; k += 4)
            acc = __builtin_amdgcn_mfma_f32_16x16x4f32(st.a[i0 + r][k + kq], st.b[k + kq][j0 + r], acc, 0, 0, 0);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            float *d = D + (i0 + 4 * kq + i) * ldd + j0 + r;
            *d = beta == 0.f ? alpha * acc[i] : fmaf(alpha, acc[i], beta * *d);
        }
    }
    __syncthreads();  // the staging buffers are free again
}

// The scratch of one workgroup of the chunk-local kernels (BwdLayout::scratch()):
// 15 C x dk, 6 C x dv and 5 C x C matrices at fixed offsets from one base (so that
// only the base stays in registers). The prefix g (later its gradient), gamma, m and
// beta are kept in LDS instead (the members G, gam, m, bet).
template <int DK, int DV> struct Scr {
    static constexpr int ck = C * DK, cv = C * DV, cc = C * C;
    float *base;
    float *G, *m, *gam, *bet;
    __device__ explicit Scr(float *p) : base(p), G(nullptr), m(nullptr), gam(nullptr), bet(nullptr) {}
    __device__ __forceinline__ float *Q() const { return base + 0 * ck; }
    __device__ __forceinline__ float *K() const { return base + 1 * ck; }
    __device__ __forceinline__ float *Gs() const { return base + 2 * ck; }
    __device__ __forceinline__ float *P() const { return base + 3 * ck; }
    __device__ __forceinline__ float *N() const { return base + 4 * ck; }
    __device__ __forceinline__ float *Qe() const { return base + 5 * ck; }
    __device__ __forceinline__ float *Bk() const { return base + 6 * ck; }
    __device__ __forceinline__ float *dQO() const { return base + 7 * ck; }
    __device__ __forceinline__ float *dR() const { return base + 8 * ck; }
    __device__ __forceinline__ float *dW() const { return base + 9 * ck; }
    __device__ __forceinline__ float *dBk() const { return base + 10 * ck; }
    __device__ __forceinline__ float *dQe() const { return base + 11 * ck; }
    __device__ __forceinline__ float *dP() const { return base + 12 * ck; }
    __device__ __forceinline__ float *dN() const { return base + 13 * ck; }
    __device__ __forceinline__ float *dG() const { return base + 14 * ck; }
    __device__ __forceinline__ float *V() const { return base + 15 * ck + 0 * cv; }
    __device__ __forceinline__ float *dO() const { return base + 15 * ck + 1 * cv; }
    __device__ __forceinline__ float *Bv() const { return base + 15 * ck + 2 * cv; }
    __device__ __forceinline__ float *U() const { return base + 15 * ck + 3 * cv; }
    __device__ __forceinline__ float *dU() const { return base + 15 * ck + 4 * cv; }
    __device__ __forceinline__ float *dBv() const { return base + 15 * ck + 5 * cv; }
    __device__ __forceinline__ float *PN() const { return base + 15 * ck + 6 * cv + 0 * cc; }
    __device__ __forceinline__ float *dAqk() const { return base + 15 * ck + 6 * cv + 1 * cc; }
    __device__ __forceinline__ float *dT() const { return base + 15 * ck + 6 * cv + 2 * cc; }
    __device__ __forceinline__ float *Tmp() const { return base + 15 * ck + 6 * cv + 3 * cc; }
    __device__ __forceinline__ float *dA() const { return base + 15 * ck + 6 * cv + 4 * cc; }
};

__device__ __forceinline__ size_t row_of(const BwdArgs &a, int b, int t, int h) {
    return ((size_t)b * a.T + t) * a.H + h;
}

// One chunk's inputs into the scratch (rows past the end zero), beta, the prefix
// g of log alpha, gamma and m (these four in LDS). Every thread calls it.
template <typename T, int DK, int DV>
__device__ void load_chunk(const BwdArgs &a, int b, int h, int t0, int n, const Scr<DK, DV> &S, bool with_dout) {
    const int tid = threadIdx.x;
    for (int idx = tid; idx < C * DK; idx += kBwdThreads) {
        const int r = idx / DK, i = idx % DK;
        const size_t off = row_of(a, b, t0 + r, h) * DK + i;
        S.Q()[idx] = r < n ? to_f32(static_cast<const T *>(a.q)[off]) : 0.f;
        S.K()[idx] = r < n ? to_f32(static_cast<const T *>(a.k)[off]) : 0.f;
    }
    for (int idx = tid; idx < C * DV; idx += kBwdThreads) {
        const int r = idx / DV, j = idx % DV;
        const size_t off = row_of(a, b, t0 + r, h) * DV + j;
        S.V()[idx] = r < n ? to_f32(static_cast<const T *>(a.v)[off]) : 0.f;
        if (with_dout) S.dO()[idx] = r < n ? to_f32(static_cast<const T *>(a.dout)[off]) : 0.f;
    }
    for (int r = tid; r < C; r += kBwdThreads) S.bet[r] = r < n ? a.beta[row_of(a, b, t0 + r, h)] : 0.f;
    for (int idx = tid; idx < C * DK; idx += kBwdThreads) {
        const int r = idx / DK;
        S.G[idx] = r < n ? a.log_alpha[row_of(a, b, t0 + r, h) * DK + idx % DK] : 0.f;
    }
    __syncthreads();
    for (int i = tid; i < DK; i += kBwdThreads) {  // the prefix down each channel (G is in LDS)
        float g = 0.f;
        for (int r = 0; r < C; ++r) {
            g += S.G[r * DK + i];
            S.G[r * DK + i] = g;
        }
        S.gam[i] = g;
        S.m[i] = 0.5f * g;
    }
}

// x from the lane that a quad permutation (DPP) selects.
template <int CTRL> __device__ __forceinline__ float quad_swap(float x) {
    return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, x), CTRL, 0xf, 0xf, false));
}

// Sum over the 64 lanes of a wave, left in every lane.
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
    return v;
}

// P, N, Qe and Bk over C x dk, Bv over C x dv (after load_chunk and a barrier).
template <int DK, int DV>
__device__ void chunk_factors(const Scr<DK, DV> &S) {
    for (int idx = threadIdx.x; idx < C * DK; idx += kBwdThreads) {
        const int r = idx / DK, i = idx % DK;
        const float g = S.G[idx], m = S.m[i], kv = S.K()[idx];
        S.P()[idx] = kv * expf(g - m);
        S.N()[idx] = kv * expf(m - g);
        S.Qe()[idx] = S.Q()[idx] * expf(g - m);
        S.Bk()[idx] = S.bet[r] * kv * expf(g);
    }
    for (int idx = threadIdx.x; idx < C * DV; idx += kBwdThreads) S.Bv()[idx] = S.bet[idx / DV] * S.V()[idx];
}

// (1) T, Aqk^T, W, U~, R, QO and e^gamma of every (chunk, head).
template <typename T, int DK, int DV>
__global__ __launch_bounds__(kBwdThreads) void kda_bwd_chunk_fwd_kernel(BwdArgs a) {
    constexpr BwdLayout L{DK, DV};
    __shared__ float sA[C][C + 1];
    __shared__ Stage st;
    __shared__ float lg[C * DK], lm[DK], lgam[DK], lbet[C];
    Scr<DK, DV> S(a.scratch + (size_t)blockIdx.x * L.scratch());
    S.G = lg;  // the prefix, gamma, m and beta live in LDS
    S.m = lm;
    S.gam = lgam;
    S.bet = lbet;
    const int tid = threadIdx.x, total = a.B * a.n_chunks * a.H;
    for (int ch = blockIdx.x; ch < total; ch += gridDim.x) {
        const int h = ch % a.H, c = (ch / a.H) % a.n_chunks, b = ch / (a.H * a.n_chunks);
        const int t0 = c * C, n = min(C, a.T - t0);
        float *cb = a.ws + (size_t)ch * L.per_chunk();
        load_chunk<T, DK, DV>(a, b, h, t0, n, S, false);
        __syncthreads();
        chunk_factors<DK, DV>(S);
        for (int idx = tid; idx < C * DK; idx += kBwdThreads) {
            const int i = idx % DK;
            const float g = S.G[idx];
            cb[L.oR() + idx] = S.K()[idx] * expf(S.gam[i] - g);
            cb[L.oQO() + idx] = a.scale * S.Q()[idx] * expf(g);
        }
        for (int i = tid; i < DK; i += kBwdThreads) cb[L.oEg() + i] = expf(S.gam[i]);
        __syncthreads();
        gemm<false, true, C, DK>(st, 1.f, S.P(), DK, S.N(), DK, 0.f, S.PN(), C);
        gemm<false, true, C, DK>(st, a.scale, S.N(), DK, S.Qe(), DK, 0.f, cb + L.oAqk(), C);  // Aqk^T
        __syncthreads();
        for (int idx = tid; idx < C * C; idx += kBwdThreads) {
            const int r = idx / C, i = idx % C;
            sA[r][i] = i < r ? S.bet[r] * S.PN()[idx] : 0.f;
            if (r > i) cb[L.oAqk() + idx] = 0.f;  // Aqk^T: zero below the diagonal
        }
        __syncthreads();
        // T = (I + A)^-1 by forward substitution: column j on the four lanes of quad j, lane q
        // holding x_i for i = q mod 4 and summing those terms; the quad's partial sums meet by
        // two DPP swaps, so each step waits on one product and two exchanges
        {
            const int j = tid >> 2, q = tid & 3;
            float x[C / 4];  // zero until solved: a zero coefficient may meet it before then
#pragma unroll
            for (int m = 0; m < C / 4; ++m) x[m] = 0.f;
#pragma unroll
            for (int r = 0; r < C; ++r) {
                float part = 0.f;
#pragma unroll
                for (int m = 0; m < C / 4; ++m)
                    if (4 * m < r) part = fmaf(4 * m + q < r ? sA[r][4 * m + q] : 0.f, x[m], part);
                part += quad_swap<0xB1>(part);  // quad_perm [1, 0, 3, 2]
                part += quad_swap<0x4E>(part);  // quad_perm [2, 3, 0, 1]
                const float xr = (r == j ? 1.f : 0.f) - part;
                if ((r & 3) == q) x[r >> 2] = xr;
            }
#pragma unroll
            for (int m = 0; m < C / 4; ++m) cb[L.oT() + (4 * m + q) * C + j] = x[m];
        }
        __syncthreads();
        gemm<false, false, DK, C>(st, 1.f, cb + L.oT(), C, S.Bk(), DK, 0.f, cb + L.oW(), DK);
        gemm<false, false, DV, C>(st, 1.f, cb + L.oT(), C, S.Bv(), DV, 0.f, cb + L.oUt(), DV);
        __syncthreads();
    }
}

// (2) The state at every chunk's start, for 16 columns of one (sequence, head).
// Each thread computes four adjacent outputs, the chunk matrices read as float4
// rows of the workspace, the state and U from LDS.
template <int DK, int DV>
__global__ __launch_bounds__(kBwdThreads) void kda_bwd_states_kernel(BwdArgs a) {
    constexpr BwdLayout L{DK, DV};
    constexpr int NB = kBwdCols;
    __shared__ __align__(16) float sS[DK][NB];
    __shared__ __align__(16) float sU[C][NB];
    const int j0 = blockIdx.x * NB, h = blockIdx.y, b = blockIdx.z, tid = threadIdx.x;
    for (int idx = tid; idx < DK * NB; idx += kBwdThreads) {
        const int i = idx / NB, j = idx % NB;
        sS[i][j] = a.h0 ? a.h0[(((size_t)b * a.H + h) * DK + i) * DV + j0 + j] : 0.f;
    }
    __syncthreads();
    for (int c = 0; c < a.n_chunks; ++c) {
        float *cb = a.ws + (((size_t)b * a.n_chunks + c) * a.H + h) * L.per_chunk();
        for (int idx = tid; idx < DK * NB; idx += kBwdThreads) {
            const int i = idx / NB, j = idx % NB;
            cb[L.oS() + i * DV + j0 + j] = sS[i][j];
        }
        for (int it = tid; it < C * NB / 4; it += kBwdThreads) {  // U[r][4 jg ..] = U~ - W S
            const int r = it / (NB / 4), jc = 4 * (it % (NB / 4));
            f32x4 u = *reinterpret_cast<const f32x4 *>(cb + L.oUt() + r * DV + j0 + jc);
            const f32x4 *w4 = reinterpret_cast<const f32x4 *>(cb + L.oW() + r * DK);
            for (int i4 = 0; i4 < DK / 4; ++i4) {
                const f32x4 w = w4[i4];
#pragma unroll
                for (int e = 0; e < 4; ++e) u -= w[e] * *reinterpret_cast<const f32x4 *>(&sS[4 * i4 + e][jc]);
            }
            *reinterpret_cast<f32x4 *>(&sU[r][jc]) = u;
        }
        __syncthreads();
        for (int it = tid; it < DK / 4 * NB; it += kBwdThreads) {  // S'[4 ig ..][j] = e^gamma S + R^T U
            const int i0 = 4 * (it / NB), j = it % NB;
            const f32x4 eg = *reinterpret_cast<const f32x4 *>(cb + L.oEg() + i0);
            f32x4 sv = {eg[0] * sS[i0][j], eg[1] * sS[i0 + 1][j], eg[2] * sS[i0 + 2][j], eg[3] * sS[i0 + 3][j]};
            for (int r = 0; r < C; ++r) sv += *reinterpret_cast<const f32x4 *>(cb + L.oR() + r * DK + i0) * sU[r][j];
#pragma unroll
            for (int e = 0; e < 4; ++e) sS[i0 + e][j] = sv[e];
        }
        __syncthreads();
    }
}

// (3) dS' of every chunk (the gradient at its end), last chunk first, and dh0;
// arranged as kernel (2), with Aqk stored transposed.
template <typename T, int DK, int DV>
__global__ __launch_bounds__(kBwdThreads) void kda_bwd_state_grads_kernel(BwdArgs a) {
    constexpr BwdLayout L{DK, DV};
    constexpr int NB = kBwdCols;
    __shared__ __align__(16) float sD[DK][NB];
    __shared__ __align__(16) float sdU[C][NB];
    __shared__ __align__(16) float sdO[C][NB];
    const int j0 = blockIdx.x * NB, h = blockIdx.y, b = blockIdx.z, tid = threadIdx.x;
    for (int idx = tid; idx < DK * NB; idx += kBwdThreads) {
        const int i = idx / NB, j = idx % NB;
        sD[i][j] = a.dhT ? a.dhT[(((size_t)b * a.H + h) * DK + i) * DV + j0 + j] : 0.f;
    }
    for (int c = a.n_chunks - 1; c >= 0; --c) {
        const int t0 = c * C, n = min(C, a.T - t0);
        float *cb = a.ws + (((size_t)b * a.n_chunks + c) * a.H + h) * L.per_chunk();
        for (int idx = tid; idx < C * NB; idx += kBwdThreads) {
            const int r = idx / NB, j = idx % NB;
            sdO[r][j] = r < n ? to_f32(static_cast<const T *>(a.dout)[row_of(a, b, t0 + r, h) * DV + j0 + j]) : 0.f;
        }
        __syncthreads();
        for (int idx = tid; idx < DK * NB; idx += kBwdThreads) {
            const int i = idx / NB, j = idx % NB;
            cb[L.oDS() + i * DV + j0 + j] = sD[i][j];
        }
        for (int it = tid; it < C * NB / 4; it += kBwdThreads) {  // dU[r][4 jg ..] = Aqk^T dO + R dS'
            const int r = it / (NB / 4), jc = 4 * (it % (NB / 4));
            f32x4 u = {0.f, 0.f, 0.f, 0.f};
            const f32x4 *a4 = reinterpret_cast<const f32x4 *>(cb + L.oAqk() + r * C);
            for (int q4 = 0; q4 < C / 4; ++q4) {
                const f32x4 x = a4[q4];
#pragma unroll
                for (int e = 0; e < 4; ++e) u += x[e] * *reinterpret_cast<const f32x4 *>(&sdO[4 * q4 + e][jc]);
            }
            const f32x4 *r4 = reinterpret_cast<const f32x4 *>(cb + L.oR() + r * DK);
            for (int i4 = 0; i4 < DK / 4; ++i4) {
                const f32x4 x = r4[i4];
#pragma unroll
                for (int e = 0; e < 4; ++e) u += x[e] * *reinterpret_cast<const f32x4 *>(&sD[4 * i4 + e][jc]);
            }
            *reinterpret_cast<f32x4 *>(&sdU[r][jc]) = u;
        }
        __syncthreads();
        for (int it = tid; it < DK / 4 * NB; it += kBwdThreads) {  // dS = QO^T dO + e^gamma dS' - W^T dU
            const int i0 = 4 * (it / NB), j = it % NB;
            const f32x4 eg = *reinterpret_cast<const f32x4 *>(cb + L.oEg() + i0);
            f32x4 sv = {eg[0] * sD[i0][j], eg[1] * sD[i0 + 1][j], eg[2] * sD[i0 + 2][j], eg[3] * sD[i0 + 3][j]};
            for (int r = 0; r < C; ++r) {
                sv += *reinterpret_cast<const f32x4 *>(cb + L.oQO() + r * DK + i0) * sdO[r][j];
                sv -= *reinterpret_cast<const f32x4 *>(cb + L.oW() + r * DK + i0) * sdU[r][j];
            }
#pragma unroll
            for (int e = 0; e < 4; ++e) sD[i0 + e][j] = sv[e];
        }
        __syncthreads();
    }
    if (a.dh0) {
        __syncthreads();
        for (int idx = tid; idx < DK * NB; idx += kBwdThreads) {
            const int i = idx / NB, j = idx % NB;
            a.dh0[(((size_t)b * a.H + h) * DK + i) * DV + j0 + j] = sD[i][j];
        }
    }
}

// (4) dq, dk, dv, dlog_alpha and dbeta of every (chunk, head).
template <typename T, int DK, int DV>
__global__ __launch_bounds__(kBwdThreads) void kda_bwd_chunk_grads_kernel(BwdArgs a) {
    constexpr BwdLayout L{DK, DV};
    __shared__ Stage st;
    __shared__ float lg[C * DK], lm[DK], lgam[DK], lbet[C];
    // Partial sums, one slot per wave step (64 consecutive elements of a loop) or per thread,
    // added up in a fixed order at the end: dbeta's three row sums, and dgamma's column sums
    // of dR R and dS' S. No atomics, so every run gives the same bits.
    static_assert(C % 64 == 0 && DK % 64 == 0 && DV % 64 == 0 && kBwdThreads % DK == 0, "wave-aligned rows");
    __shared__ float lb1[C * C / 64], lb2[C * DV / 64], lb3[C * DK / 64], lgp[kBwdThreads], lsp[DK * DV / 64];
    Scr<DK, DV> S(a.scratch + (size_t)blockIdx.x * L.scratch());
    S.G = lg;  // the prefix (later its gradient), gamma, m and beta live in LDS
    S.m = lm;
    S.gam = lgam;
    S.bet = lbet;
    const int tid = threadIdx.x, total = a.B * a.n_chunks * a.H;
    const float s = a.scale;
    for (int ch = blockIdx.x; ch < total; ch += gridDim.x) {
        const int h = ch % a.H, c = (ch / a.H) % a.n_chunks, b = ch / (a.H * a.n_chunks);
        const int t0 = c * C, n = min(C, a.T - t0);
        const float *cb = a.ws + (size_t)ch * L.per_chunk();
        const float *Tm = cb + L.oT(), *AqkT = cb + L.oAqk(), *W = cb + L.oW(), *Ut = cb + L.oUt();
        const float *Rm = cb + L.oR(), *S0 = cb + L.oS(), *dS1 = cb + L.oDS();
        load_chunk<T, DK, DV>(a, b, h, t0, n, S, true);
        __syncthreads();
        chunk_factors<DK, DV>(S);
        for (int idx = tid; idx < C * DV; idx += kBwdThreads) S.U()[idx] = Ut[idx];
        __syncthreads();
        gemm<false, true, C, DK>(st, 1.f, S.P(), DK, S.N(), DK, 0.f, S.PN(), C);           // P N^T
        gemm<false, false, DV, DK>(st, -1.f, W, DK, S0, DV, 1.f, S.U(), DV);          // U = U~ - W S
        gemm<false, false, DV, C>(st, 1.f, AqkT, C, S.dO(), DV, 0.f, S.dU(), DV);       // dU = Aqk^T dO
        gemm<false, false, DV, DK>(st, 1.f, Rm, DK, dS1, DV, 1.f, S.dU(), DV);        //    + R dS'
        gemm<false, true, DK, DV>(st, 1.f, S.dO(), DV, S0, DV, 0.f, S.dQO(), DK);       // dQO = dO S^T
        __syncthreads();
        gemm<false, true, C, DV>(st, 1.f, S.dO(), DV, S.U(), DV, 0.f, S.dAqk(), C);       // dO U^T
        gemm<false, true, DK, DV>(st, 1.f, S.U(), DV, dS1, DV, 0.f, S.dR(), DK);        // dR = U dS'^T
        gemm<false, true, DK, DV>(st, -1.f, S.dU(), DV, S0, DV, 0.f, S.dW(), DK);       // dW = -dU S^T
        gemm<true, false, DV, C>(st, 1.f, Tm, C, S.dU(), DV, 0.f, S.dBv(), DV);         // dBv = T^T dU
        gemm<false, true, C, DV>(st, 1.f, S.dU(), DV, S.Bv(), DV, 0.f, S.dT(), C);        // dT = dU Bv^T
        __syncthreads();
        for (int idx = tid; idx < C * C; idx += kBwdThreads)
            if (idx % C > idx / C) S.dAqk()[idx] = 0.f;                               // lower, diagonal included
        gemm<false, true, C, DK>(st, 1.f, S.dW(), DK, S.Bk(), DK, 1.f, S.dT(), C);        //    + dW Bk^T
        gemm<true, false, DK, C>(st, 1.f, Tm, C, S.dW(), DK, 0.f, S.dBk(), DK);         // dBk = T^T dW
        __syncthreads();
        gemm<true, false, C, C>(st, 1.f, Tm, C, S.dT(), C, 0.f, S.Tmp(), C);            // T^T dT
        __syncthreads();
        gemm<false, true, C, C>(st, -1.f, S.Tmp(), C, Tm, C, 0.f, S.dA(), C);           // dA = -T^T dT T^T
        __syncthreads();
        // dA strictly lower; dbeta's third term, rowsum(dA * P N^T), over the strictly lower
        // part only (above the diagonal P N^T can overflow, e^(g_r - g_i) with i after r).
        // A wave covers one row per step here and in the two loops below.
        #pragma unroll 2
        for (int idx = tid; idx < C * C; idx += kBwdThreads) {
            const int r = idx / C, i = idx % C;
            float d = S.dA()[idx], t = 0.f;
            if (i >= r)
                S.dA()[idx] = 0.f;
            else
                t = d * S.PN()[idx];
            t = wave_sum(t);
            if ((tid & 63) == 0) lb1[idx >> 6] = t;
        }
        __syncthreads();
        #pragma unroll 2
        for (int idx = tid; idx < C * DV; idx += kBwdThreads) {  // dv, and dbeta's rowsum(dBv * v)
            const int r = idx / DV;
            const float dbv = S.dBv()[idx];
            if (r < n) static_cast<T *>(a.dv)[row_of(a, b, t0 + r, h) * DV + idx % DV] = from_f32<T>(S.bet[r] * dbv);
            const float t = wave_sum(dbv * S.V()[idx]);
            if ((tid & 63) == 0) lb2[idx >> 6] = t;
        }
        for (int idx = tid; idx < C * C; idx += kBwdThreads) S.dA()[idx] *= S.bet[idx / C];  // diag(beta) dA
        __syncthreads();
        gemm<false, false, DK, C>(st, 1.f, S.dA(), C, S.N(), DK, 0.f, S.dP(), DK);        // dP = diag(beta) dA N
        gemm<true, false, DK, C>(st, 1.f, S.dA(), C, S.P(), DK, 0.f, S.dN(), DK);         // dN = (diag(beta) dA)^T P
        gemm<true, false, DK, C>(st, s, S.dAqk(), C, S.Qe(), DK, 1.f, S.dN(), DK);        //    + s dAqk^T Qe
        gemm<false, false, DK, C>(st, s, S.dAqk(), C, S.N(), DK, 0.f, S.dQe(), DK);       // dQe = s dAqk N
        __syncthreads();
        // dq, dk; dg into LDS in place of g; dbeta's rowsum(dBk * k e^g); this thread's
        // share of colsum(dR * R) (its channel is fixed: 256 is a multiple of dk)
        float dgr = 0.f;
        #pragma unroll 2
        for (int idx = tid; idx < C * DK; idx += kBwdThreads) {
            const int r = idx / DK, i = idx % DK;
            const float g = S.G[idx], m = S.m[i], kv = S.K()[idx], qv = S.Q()[idx], bb = S.bet[r];
            const float eG = expf(g), eGm = expf(g - m), emG = expf(m - g), eR = expf(S.gam[i] - g);
            const float dQO = S.dQO()[idx], dQe = S.dQe()[idx], dBk = S.dBk()[idx], dP = S.dP()[idx], dN = S.dN()[idx],
                        dR = S.dR()[idx];
            S.G[idx] = s * dQO * qv * eG + dQe * qv * eGm + bb * dBk * kv * eG + dP * kv * eGm - dN * kv * emG -
                       dR * kv * eR;
            dgr = fmaf(dR, kv * eR, dgr);
            if (r < n) {
                const size_t off = row_of(a, b, t0 + r, h) * DK + i;
                static_cast<T *>(a.dq)[off] = from_f32<T>(s * dQO * eG + dQe * eGm);
                static_cast<T *>(a.dk)[off] = from_f32<T>(bb * dBk * eG + dP * eGm + dN * emG + dR * eR);
            }
            const float t = wave_sum(dBk * kv * eG);
            if ((tid & 63) == 0) lb3[idx >> 6] = t;
        }
        lgp[tid] = dgr;
        #pragma unroll 2
        for (int idx = tid; idx < DK * DV; idx += kBwdThreads) {  // rowsum(dS' * S), a wave per row
            const float t = wave_sum(dS1[idx] * S0[idx]);
            if ((tid & 63) == 0) lsp[idx >> 6] = t;
        }
        __syncthreads();
        for (int r = tid; r < n; r += kBwdThreads) {
            float acc = 0.f;
            for (int j = 0; j < C / 64; ++j) acc += lb1[r * (C / 64) + j];
            for (int j = 0; j < DV / 64; ++j) acc += lb2[r * (DV / 64) + j];
            for (int j = 0; j < DK / 64; ++j) acc += lb3[r * (DK / 64) + j];
            a.dbeta[row_of(a, b, t0 + r, h)] = acc;
        }
        for (int i = tid; i < DK; i += kBwdThreads) {  // dgamma, then the reverse prefix of dg
            float gs = 0.f, ss = 0.f;
            for (int j = 0; j < kBwdThreads / DK; ++j) gs += lgp[j * DK + i];
            for (int j = 0; j < DV / 64; ++j) ss += lsp[i * (DV / 64) + j];
            float acc = fmaf(expf(S.gam[i]), ss, gs);
            for (int r = C - 1; r >= 0; --r) {
                acc += S.G[r * DK + i];
                if (r < n) a.dlog_alpha[row_of(a, b, t0 + r, h) * DK + i] = acc;
            }
        }
        __syncthreads();
    }
}

template <typename T, int DK, int DV>
hipError_t launch_bwd_t(const BwdArgs &a, hipStream_t st) {
    const int total = a.B * a.n_chunks * a.H;
    if (total > 0) {
        hipLaunchKernelGGL((kda_bwd_chunk_fwd_kernel<T, DK, DV>), dim3(a.n_groups), dim3(kBwdThreads), 0, st, a);
        if (hipGetLastError() != hipSuccess) return hipErrorLaunchFailure;
        hipLaunchKernelGGL((kda_bwd_states_kernel<DK, DV>), dim3(DV / kBwdCols, a.H, a.B), dim3(kBwdThreads), 0, st,
                           a);
        if (hipGetLastError() != hipSuccess) return hipErrorLaunchFailure;
    }
    if (total > 0 || a.dh0) {
        hipLaunchKernelGGL((kda_bwd_state_grads_kernel<T, DK, DV>), dim3(DV / kBwdCols, a.H, a.B), dim3(kBwdThreads), 0,
                           st, a);
        if (hipGetLastError() != hipSuccess) return hipErrorLaunchFailure;
    }
    if (total > 0) {
        hipLaunchKernelGGL((kda_bwd_chunk_grads_kernel<T, DK, DV>), dim3(a.n_groups), dim3(kBwdThreads), 0, st, a);
        return hipGetLastError();
    }
    return hipSuccess;
}

template <typename T>
hipError_t dispatch_bwd(const BwdArgs &a, int dk, int dv, hipStream_t stream) {
    if (dk == 64 && dv == 64) return launch_bwd_t<T, 64, 64>(a, stream);
    if (dk == 64 && dv == 128) return launch_bwd_t<T, 64, 128>(a, stream);
    if (dk == 128 && dv == 64) return launch_bwd_t<T, 128, 64>(a, stream);
    return launch_bwd_t<T, 128, 128>(a, stream);
}

}  // namespace

hipError_t launch_chunk_bwd(const BwdArgs &a, int dk, int dv, bool is_bf16, hipStream_t stream) {
    return is_bf16 ? dispatch_bwd<bf16>(a, dk, dv, stream) : dispatch_bwd<float>(a, dk, dv, stream);
}

}  // namespace kda
