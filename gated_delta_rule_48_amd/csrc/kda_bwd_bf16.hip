// kda_bwd_bf16.hip -- the chunked backward pass on the matrix cores, for bf16 I/O with
// d_k = d_v = 128 and chunks of 64 rows.
//
// The same derivative as kda_bwd.hip (the reverse-mode derivative of the chunk form of
// the essay "22,580: from GPT-2 to Kimi K3", sections 6.2-6.3, with the per-channel decay
// of its Gated DeltaNet section; the identities are listed in that file's header), taken
// in four launches whose products all run on the matrix cores with bf16 operands and fp32
// accumulation:
//
//  1. the forward's chunk preparation (kda_prep.hip): W, U~, QO, KtT, Aqk and e^gamma of
//     every (chunk, head), in parallel;
//  2. the forward's state recursion (kda_state.hip) without outputs, which records the
//     state entering every chunk (as S^T) and the chunk's corrected writes U = U~ - W S
//     (as U^T);
//  3. the reverse recursion (kda_bwd_rev_kernel, this file), last chunk first: with dS' the
//     loss gradient with respect to the state at a chunk's end,
//         dU = Aqk^T dO + R dS',   dS = QO^T dO + Diag(e^gamma) dS' - W^T dU,
//     recording dS' (as dS'^T) and dU (as dU^T) of every chunk, and dh0;
//  4. the chunk-local gradients (kda_bwd_chunk_kernel, this file), in parallel over
//     (chunk, head): everything else, from q, k, v, log alpha, beta, dO and the four
//     recorded matrices, with the chunk's matrices in LDS and registers.
//
// Fragment-ordered operands (kda_device.hpp): F(X) is X stored as the A operand of a
// product that contracts over X's columns (rows of X = rows of the product); a product
// D = X Y^T takes F(X) and F(Y). A 16x16 accumulator tile of D is, lane for lane, four
// consecutive operand slots of F(D^T), so D^T is stored with one 8-byte write per lane;
// F(D) needs four 2-byte writes.

#include "kda_bwd.hpp"

namespace kda {
namespace {

constexpr int kC = 64;     // rows per chunk
constexpr int kD = 128;    // d_k = d_v
typedef Frag<bf16> FB;
typedef FB::Vec V8;

__device__ __forceinline__ f32x4 zero4() { return f32x4{0.f, 0.f, 0.f, 0.f}; }

// The lane index, opaque to the compiler: element addresses derived from it are formed
// afresh where they are used instead of being kept in registers from one phase to the next.
__device__ __forceinline__ int fresh_lane() {
    int l = threadIdx.x & 63;
    asm volatile("" : "+v"(l));
    return l;
}

// Sum over the 16 lanes of each DPP row (lanes 16m .. 16m + 15), left in every lane.
__device__ __forceinline__ float row16_sum(float x) {
#pragma unroll
    for (int o = 8; o > 0; o >>= 1) x += __shfl_xor(x, o);
    return x;
}

__device__ __forceinline__ int fresh_tid() {
    int t = threadIdx.x;
    asm volatile("" : "+v"(t));
    return t;
}

// x, opaque to the compiler: an exponential of it is computed again instead of being kept
// in a register from an earlier phase.
__device__ __forceinline__ float fresh(float x) {
    asm volatile("" : "+v"(x));
    return x;
}

// acc tile (rows 16 rb .., columns 16 cb ..) of D into F(D^T) (R = D's column count).
__device__ __forceinline__ void store_t(bf16 *base, int rb, int cb, f32x4 v, int R) {
    const int l = threadIdx.x & 63;
    bf16 x[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) x[i] = static_cast<bf16>(v[i]);
    const int kg = rb >> 1;
    *reinterpret_cast<uint2 *>(base + (((size_t)kg * (R >> 4) + cb) * 64 + l) * 8 + 4 * (rb & 1)) =
        *reinterpret_cast<const uint2 *>(x);
}

// acc tile (rows 16 rb .., columns 16 cb ..) of D into F(D) (R = D's row count).
__device__ __forceinline__ void store_n(bf16 *base, int rb, int cb, f32x4 v, int R) {
    const int l = fresh_lane();
#pragma unroll
    for (int i = 0; i < 4; ++i)
        base[frag_off<bf16>(16 * rb + 4 * (l >> 4) + i, 16 * cb + (l & 15), R)] = static_cast<bf16>(v[i]);
}

// acc[u] += sum over NK contraction groups of F(A)[kg][rbA] x F(B)[kg][cb0 + u]
template <int NU, int NK>
__device__ __forceinline__ void prod(f32x4 (&acc)[NU], const bf16 *A, int RA, int rbA, const bf16 *B, int RB, int cb0) {
#pragma unroll
    for (int kg = 0; kg < NK; ++kg) {
        const V8 a = frag_load<bf16>(A, kg, rbA, RA);
#pragma unroll
        for (int u = 0; u < NU; ++u) acc[u] = FB::mma(acc[u], a, frag_load<bf16>(B, kg, cb0 + u, RB));
    }
}

// One thread's share of a fragment-ordered [R][K] bf16 matrix: slots tid, tid + NT, ...
// (whole 16-byte operand shares), and those shares written transposed into F(X^T) ([K][R])
// in LDS.
template <int R, int K, int NT> struct Shares {
    static constexpr int N = R * K / 8 / NT;
    V8 x[N];
    __device__ __forceinline__ void load(const bf16 *src) {
#pragma unroll
        for (int m = 0; m < N; ++m) x[m] = *reinterpret_cast<const V8 *>(src + ((size_t)threadIdx.x + NT * m) * 8);
    }
    __device__ __forceinline__ void store_transposed(bf16 *dst, bool negate) const {
        const int l = threadIdx.x & 63, hi = l >> 4;
#pragma unroll
        for (int m = 0; m < N; ++m) {
            const int gi = (threadIdx.x + NT * m) >> 6, kg = gi / (R / 16), rb = gi % (R / 16);
            const int r = 16 * rb + (l & 15);
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                const float f = static_cast<float>(x[m][j]);
                dst[frag_off<bf16>(frag_chan<bf16>(kg, hi, j), r, K)] = static_cast<bf16>(negate ? -f : f);
            }
        }
    }
};

template <int R, int K, int NT>
__device__ __forceinline__ void transpose_into(bf16 *dst, const bf16 *src, bool negate) {
    Shares<R, K, NT> sh;
    sh.load(src);
    sh.store_transposed(dst, negate);
}

// ------------------------------------------------------------------ (3) reverse recursion
//
// One workgroup of 8 waves per (sequence, head), two per SIMD so that one wave's loads and
// LDS waits overlap the other's products; the state gradient dS' (128 x 128 fp32) in
// matrix-core accumulators, wave w owning key channels 16 w .. 16 w + 15. Per chunk,
// last first: the chunk's Aqk, KtT, QO and W (fragment-ordered for the forward's uses)
// are transposed into LDS for the reverse uses, and dO's rows into F(dO^T).
struct RevLds {
    bf16 AqT[kC * kC];   // F(Aqk^T): rows i, contraction r
    bf16 Rf[kC * kD];    // F(R), R = KtT^T: rows r, contraction key channel
    bf16 QOt[kD * kC];   // F(QO^T): rows key channel, contraction r
    bf16 Wn[kD * kC];    // F(-W^T)
    bf16 dOt[kD * kC];   // F(dO^T): rows value column, contraction r
    bf16 dSt[kD * kD];   // F(dS'^T): rows value column, contraction key channel
    bf16 dUt[kD * kC];   // F(dU^T)
};

__global__ __launch_bounds__(512) void kda_bwd_rev_kernel(BwdFastArgs a) {
    __shared__ __align__(16) RevLds L;
    const int H = a.H, sh = blockIdx.x, h = sh % H, s = sh / H;
    const int w = threadIdx.x >> 6, l = threadIdx.x & 63;
    // dS' tiles of this wave: key-channel block w, value blocks nt
    f32x4 acc[8];
    {
        const float *dhT = a.dhT ? a.dhT + ((size_t)s * H + h) * kD * kD : nullptr;
#pragma unroll
        for (int nt = 0; nt < 8; ++nt)
#pragma unroll
            for (int i = 0; i < 4; ++i)
                acc[nt][i] = dhT ? dhT[(16 * w + acc_row(i)) * kD + 16 * nt + acc_col()] : 0.f;
    }
    int tb, te;
    a.map.seq_range(s, tb, te);
    const int c_begin = a.map.chunks_before(s);
    const int n_c = (te - tb + kC - 1) / kC;
    const bf16 *dout = static_cast<const bf16 *>(a.dout);

    // One chunk's operands as loaded (this thread's shares), the next chunk's in flight while
    // one computes. Every load is unconditional (rows past the sequence's end re-read its last
    // row and are then zeroed), so that the compiler waits for exactly the set it needs.
    struct Ops {
        Shares<kC, kC, 512> aq;
        Shares<kD, kC, 512> kt;
        Shares<kC, kD, 512> qo, wm;
        V8 o[2];
        f32x4 eg;
    };
    auto load_ops = [&](int ci, Ops &op) {
        const int t0 = tb + ci * kC, L_rows = min(kC, te - t0);
        const size_t jh = (size_t)(c_begin + ci) * H + h;
        op.aq.load(static_cast<const bf16 *>(a.buf.Aqk) + jh * kC * kC);
        op.kt.load(static_cast<const bf16 *>(a.buf.KtT) + jh * kD * kC);
        op.qo.load(static_cast<const bf16 *>(a.buf.QO) + jh * kC * kD);
        op.wm.load(static_cast<const bf16 *>(a.buf.W) + jh * kC * kD);
#pragma unroll
        for (int m = 0; m < 2; ++m) {  // dO: 8 adjacent value columns of one row per share
            const int u = threadIdx.x + 512 * m, r = u / (kD / 8), j0 = 8 * (u % (kD / 8));
            op.o[m] = *reinterpret_cast<const V8 *>(dout + ((size_t)(t0 + min(r, L_rows - 1)) * H + h) * kD + j0);
            if (r >= L_rows) {
#pragma unroll
                for (int e = 0; e < 8; ++e) op.o[m][e] = static_cast<bf16>(0.f);
            }
        }
        op.eg = *reinterpret_cast<const f32x4 *>(a.buf.eg + jh * kD + 16 * w + 4 * (l >> 4));
    };
    Ops op;
    if (n_c > 0) load_ops(n_c - 1, op);

    for (int ci = n_c - 1; ci >= 0; --ci) {
        const size_t jh = (size_t)(c_begin + ci) * H + h;
        // dS' (the gradient at this chunk's end) into LDS
#pragma unroll
        for (int nt = 0; nt < 8; ++nt) store_t(L.dSt, w, nt, acc[nt], kD);
        // this chunk's operands, transposed
        op.aq.store_transposed(L.AqT, false);
        op.kt.store_transposed(L.Rf, false);
        op.qo.store_transposed(L.QOt, false);
        op.wm.store_transposed(L.Wn, true);
#pragma unroll
        for (int m = 0; m < 2; ++m) {
            const int u = threadIdx.x + 512 * m, r = u / (kD / 8), j0 = 8 * (u % (kD / 8));
#pragma unroll
            for (int e = 0; e < 8; ++e) L.dOt[frag_off<bf16>(j0 + e, r, kD)] = op.o[m][e];
        }
        const f32x4 eg = op.eg;
        load_ops(ci > 0 ? ci - 1 : 0, op);  // the next chunk's (the first re-reads itself)
        __syncthreads();
        // record dS'^T of this chunk
        {
            bf16 *dst = static_cast<bf16 *>(a.ds) + jh * kD * kD;
            for (int u = threadIdx.x; u < kD * kD / 8; u += 512)
                *reinterpret_cast<uint4 *>(dst + (size_t)u * 8) = *reinterpret_cast<const uint4 *>(L.dSt + (size_t)u * 8);
        }
        // dU = Aqk^T dO + R dS': rows 16 (w % 4) .. of the chunk, value blocks 4 (w / 4) .. + 3
        {
            const int rb = w & 3, cb0 = 4 * (w >> 2);
            f32x4 du[4];
#pragma unroll
            for (int nt = 0; nt < 4; ++nt) du[nt] = zero4();
            prod<4, kC / 32>(du, L.AqT, kC, rb, L.dOt, kD, cb0);
            prod<4, kD / 32>(du, L.Rf, kC, rb, L.dSt, kD, cb0);
#pragma unroll
            for (int nt = 0; nt < 4; ++nt) store_t(L.dUt, rb, cb0 + nt, du[nt], kD);
        }
        __syncthreads();
        {
            bf16 *dst = static_cast<bf16 *>(a.du) + jh * kD * kC;
            for (int u = threadIdx.x; u < kD * kC / 8; u += 512)
                *reinterpret_cast<uint4 *>(dst + (size_t)u * 8) = *reinterpret_cast<const uint4 *>(L.dUt + (size_t)u * 8);
        }
        // dS = Diag(e^gamma) dS' + QO^T dO - W^T dU
        {
            f32x4 t[8];
#pragma unroll
            for (int nt = 0; nt < 8; ++nt) t[nt] = acc[nt] * eg;
            prod<8, kC / 32>(t, L.QOt, kD, w, L.dOt, kD, 0);
            prod<8, kC / 32>(t, L.Wn, kD, w, L.dUt, kD, 0);
#pragma unroll
            for (int nt = 0; nt < 8; ++nt) acc[nt] = t[nt];
        }
        __syncthreads();  // LDS free for the next chunk
    }
    if (a.dh0) {
        float *dh0 = a.dh0 + ((size_t)s * H + h) * kD * kD;
#pragma unroll
        for (int nt = 0; nt < 8; ++nt)
#pragma unroll
            for (int i = 0; i < 4; ++i) dh0[(16 * w + acc_row(i)) * kD + 16 * nt + acc_col()] = acc[nt][i];
    }
}

// ------------------------------------------------------------------ (4) chunk-local gradients
//
// One workgroup of 8 waves per (chunk, head). Outputs of shape C x 128 are 16x16 tiles
// dealt as: wave w takes row block w & 3 and column blocks 4 (w >> 2) .. + 3 (so every
// such product leaves element (r, c) in the same lane and register, and dq, dk and the
// decay gradient accumulate in registers); outputs of shape C x C: row block w & 3,
// column blocks 2 (w >> 2) .. + 1.
//
// With g the prefix of log alpha in the chunk, gamma = g[C - 1], m = gamma / 2, the
// elementwise gradients are collected as
//     dq = e^g (s dQO) + e^(g-m) dQe
//     dk = e^g (beta dBk) + e^(g-m) dP + e^(m-g) dN + e^(gamma-g) dR
//     dg = q dq + k dk - 2 k Z,   Z = e^(m-g) dN + e^(gamma-g) dR
// (dg of the header's list regrouped), then dlog alpha = the reverse prefix of dg plus
// dgamma = colsum(dR * R) + e^gamma rowsum(dS' * S) on every row.

// LDS map (bytes). The large region is reused from phase to phase; the persistent part
// holds T, T^T and the two layouts of dAqk.
namespace cl {
constexpr int Lg = 0;             // fp32 [C][132]: g, later dg
constexpr int LgP = kD + 4;
constexpr int As = 34816;         // fp32 [C][68]: A, then T
constexpr int AsP = kC + 4;
constexpr int FP = 52224, FN = 68608;      // phase 1: F(P), F(N)
constexpr int FdO = 0, FS = 16384, FU = 49152, FdU = 65536, FdW = 81920, FdWt = 98304;  // phase 2
constexpr int FBv = 0, FBk = 16384, FdTt = 32768;                                         // phase 3
constexpr int FX = 40960, FdAp = 49152, FdApt = 57344;                                    // phase 4
constexpr int FNt = 65536, FPt = 81920, FQet = 98304;                                     // phase 5
constexpr int REGION = 114688;
constexpr int FT = REGION, FTt = REGION + 8192, FdAqk = REGION + 16384, FdAqkt = REGION + 24576;
constexpr int SMALL = REGION + 32768;
constexpr int bet = SMALL;                 // fp32 [C]
constexpr int gam = bet + 4 * kC;          // fp32 [128]
constexpr int bpart = gam + 4 * kD;        // fp32 [3 terms][2 halves][C]: dbeta partial sums
constexpr int gpart = bpart + 4 * 6 * kC;  // fp32 [4 row blocks][128]: colsum(dR R)
constexpr int spart = gpart + 4 * 4 * kD;  // fp32 [8 value blocks][128]: rowsum(dS' S)
constexpr int qpart = spart + 4 * 8 * kD;  // fp32 [4 quarters][128]: row-quarter sums of the scans
constexpr int TOTAL = qpart + 4 * 4 * kD;
static_assert(As >= Lg + 4 * kC * LgP && FP >= As + 4 * kC * AsP && FN + 16384 <= REGION, "phase 1 layout");
static_assert(TOTAL <= 160 * 1024, "LDS budget");
}  // namespace cl

// x from the lane that a quad permutation (DPP) selects.
template <int CTRL> __device__ __forceinline__ float quad_swap(float x) {
    return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, x), CTRL, 0xf, 0xf, false));
}

__global__ __launch_bounds__(512) void kda_bwd_chunk_kernel(BwdFastArgs a) {
    extern __shared__ __align__(16) unsigned char smem[];
    auto fbuf = [&](int off) { return reinterpret_cast<bf16 *>(smem + off); };
    auto ffl = [&](int off) { return reinterpret_cast<float *>(smem + off); };
    const int tid = threadIdx.x, w = tid >> 6, l = tid & 63, hi = l >> 4, n = l & 15;
    const int H = a.H, h = blockIdx.x % H, j = blockIdx.x / H;
    int s_, t0, L;
    if (!a.map.locate(j, s_, t0, L)) return;
    const size_t jh = (size_t)j * H + h;
    const float sc = a.scale;
    const int rb = w & 3, half = w >> 2;
    const int cbD = 4 * half;  // first 16-column block of this wave's C x 128 tiles
    const int cbC = 2 * half;  // first 16-column block of this wave's C x C tiles
    auto row_of = [&](int i) { return 16 * rb + acc_row(i); };
    auto colD = [&](int u) { return 16 * (cbD + u) + n; };
    const bf16 *q_g = static_cast<const bf16 *>(a.q), *k_g = static_cast<const bf16 *>(a.k);
    const bf16 *v_g = static_cast<const bf16 *>(a.v), *o_g = static_cast<const bf16 *>(a.dout);
    auto tok = [&](int r) { return ((size_t)(t0 + r) * H + h); };

    // ---- phase 0: g (prefix of log alpha down each channel), beta
    {
        float *Lg = ffl(cl::Lg);
        for (int u = tid; u < kC * kD / 4; u += 512) {
            const int r = u / (kD / 4), c4 = 4 * (u % (kD / 4));
            f32x4 x = zero4();
            if (r < L) x = *reinterpret_cast<const f32x4 *>(a.log_alpha + tok(r) * kD + c4);
            *reinterpret_cast<f32x4 *>(Lg + r * cl::LgP + c4) = x;
        }
        if (tid < kC) ffl(cl::bet)[tid] = tid < L ? a.beta[tok(tid)] : 0.f;
        __syncthreads();
        // thread (channel c, quarter qq): the prefix over rows 16 qq .. 16 qq + 15 in registers,
        // then the quarters' totals through LDS
        const int ft = fresh_tid(), c = ft & (kD - 1), qq = ft >> 7;
        float x[16];
#pragma unroll
        for (int r = 0; r < 16; ++r) x[r] = Lg[(16 * qq + r) * cl::LgP + c];
#pragma unroll
        for (int r = 1; r < 16; ++r) x[r] += x[r - 1];
        ffl(cl::qpart)[qq * kD + c] = x[15];
        __syncthreads();
        float off = 0.f;
#pragma unroll
        for (int b = 0; b < 3; ++b) off += b < qq ? ffl(cl::qpart)[b * kD + c] : 0.f;
#pragma unroll
        for (int r = 0; r < 16; ++r) Lg[(16 * qq + r) * cl::LgP + c] = x[r] + off;
        if (qq == 3) ffl(cl::gam)[c] = x[15] + off;
        __syncthreads();
    }
    // this thread's elements of the C x 128 layout: k, g (q is read again where needed); m and
    // gamma of its columns; beta of its rows
    float kv[4][4], gv[4][4], mcol[4], gcol[4], brow[4];
    // element (u, i) of this thread: row 16 rb + 4 hi + i, column 16 (cbD + u) + n (addresses
    // from fresh_lane(), see there)
#define KDA_ROW(i) (16 * rb + 4 * (fl >> 4) + (i))
#define KDA_COL(u) (16 * (cbD + (u)) + (fl & 15))
    {
        const int fl = fresh_lane();
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            gcol[u] = ffl(cl::gam)[KDA_COL(u)];
            mcol[u] = 0.5f * gcol[u];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int r = KDA_ROW(i), c = KDA_COL(u);
                gv[u][i] = ffl(cl::Lg)[r * cl::LgP + c];
                kv[u][i] = r < L ? static_cast<float>(k_g[tok(r) * kD + c]) : 0.f;
            }
        }
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) brow[i] = ffl(cl::bet)[row_of(i)];

    // ---- phase 1: G = P N^T, A = strict_lower(beta G), T = (I + A)^-1
#pragma unroll
    for (int u = 0; u < 4; ++u) {
        f32x4 pp, nn;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const float d = gv[u][i] - mcol[u];
            pp[i] = kv[u][i] * __expf(d);
            nn[i] = kv[u][i] * __expf(-d);
        }
        store_n(fbuf(cl::FP), rb, cbD + u, pp, kC);
        store_n(fbuf(cl::FN), rb, cbD + u, nn, kC);
    }
    __syncthreads();
    f32x4 G[2];
    G[0] = G[1] = zero4();
    prod<2, kD / 32>(G, fbuf(cl::FP), kC, rb, fbuf(cl::FN), kC, cbC);
    {
        float *As = ffl(cl::As);
#pragma unroll
        for (int u = 0; u < 2; ++u)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int r = row_of(i), c = 16 * (cbC + u) + n;
                As[r * cl::AsP + c] = c < r ? brow[i] * G[u][i] : 0.f;
            }
    }
    __syncthreads();
    // forward substitution on all eight waves: column jc on the eight lanes jc * 8 .., lane qd
    // holding x_i for i = qd mod 8 and summing those terms; the partial sums meet by three DPP
    // swaps (pairs, quads, then the two quads of the half row)
    float xs[kC / 8];
    {
        const float *As = ffl(cl::As);
        const int jc = tid >> 3, qd = tid & 7;
#pragma unroll
        for (int mm = 0; mm < kC / 8; ++mm) xs[mm] = 0.f;
#pragma unroll
        for (int r = 0; r < kC; ++r) {
            float part = 0.f;
#pragma unroll
            for (int mm = 0; mm < kC / 8; ++mm)
                if (8 * mm < r) part = fmaf(8 * mm + qd < r ? As[r * cl::AsP + 8 * mm + qd] : 0.f, xs[mm], part);
            part += quad_swap<0xB1>(part);
            part += quad_swap<0x4E>(part);
            part += quad_swap<0x141>(part);
            const float xr = (r == jc ? 1.f : 0.f) - part;
            if ((r & 7) == qd) xs[r >> 3] = xr;
        }
    }
    __syncthreads();  // every read of A done
    {
        float *As = ffl(cl::As);
        const int jc = tid >> 3, qd = tid & 7;
#pragma unroll
        for (int mm = 0; mm < kC / 8; ++mm) As[(8 * mm + qd) * cl::AsP + jc] = xs[mm];
    }
    __syncthreads();
    // F(T) (rows r, contraction i) and F(T^T) (rows i, contraction r): one slot of 8 each per thread
    {
        const float *Ts = ffl(cl::As);
        const int gi = tid >> 6, kg = gi / (kC / 16), rbs = gi % (kC / 16), rr = 16 * rbs + n;
        V8 x, y;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const int kk = frag_chan<bf16>(kg, hi, e);
            x[e] = static_cast<bf16>(Ts[rr * cl::AsP + kk]);
            y[e] = static_cast<bf16>(Ts[kk * cl::AsP + rr]);
        }
        *reinterpret_cast<V8 *>(fbuf(cl::FT) + (size_t)tid * 8) = x;
        *reinterpret_cast<V8 *>(fbuf(cl::FTt) + (size_t)tid * 8) = y;
    }
    __syncthreads();  // phase-1 buffers free

    // ---- phase 2: products with S, dS', U and dU
    // F(dO): rows r, contraction value column (two runs of 4 adjacent columns per slot)
    for (int u = tid; u < kC * kD / 8; u += 512) {
        const int gi = u >> 6, kg = gi / (kC / 16), rbs = gi % (kC / 16), r = 16 * rbs + n;
        uint4 x = {0u, 0u, 0u, 0u};
        if (r < L) {
            const bf16 *p = o_g + tok(r) * kD + 32 * kg + 4 * hi;
            const uint2 lo = *reinterpret_cast<const uint2 *>(p), hi2 = *reinterpret_cast<const uint2 *>(p + 16);
            x = uint4{lo.x, lo.y, hi2.x, hi2.y};
        }
        *reinterpret_cast<uint4 *>(fbuf(cl::FdO) + (size_t)u * 8) = x;
    }
    // F(S) and F(U) and F(dU) from the recorded transposes; rowsum(dS' * S) on the way
    const bf16 *stg = static_cast<const bf16 *>(a.st) + jh * kD * kD;
    const bf16 *dsg = static_cast<const bf16 *>(a.ds) + jh * kD * kD;
    {
        float sp[4][8];
#pragma unroll
        for (int qq = 0; qq < 4; ++qq) {
            const int u = tid + 512 * qq;  // group w + 8 qq: contraction group qq, value block w
            const V8 sv = *reinterpret_cast<const V8 *>(stg + (size_t)u * 8);
            const V8 dsv = *reinterpret_cast<const V8 *>(dsg + (size_t)u * 8);
            const int jv = 16 * w + n;
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const int c = frag_chan<bf16>(qq, hi, e);
                fbuf(cl::FS)[frag_off<bf16>(c, jv, kD)] = sv[e];
                sp[qq][e] = row16_sum(static_cast<float>(sv[e]) * static_cast<float>(dsv[e]));
            }
        }
        if (n == 0) {
#pragma unroll
            for (int qq = 0; qq < 4; ++qq)
#pragma unroll
                for (int e = 0; e < 8; ++e) ffl(cl::spart)[w * kD + frag_chan<bf16>(qq, hi, e)] = sp[qq][e];
        }
    }
    transpose_into<kD, kC, 512>(fbuf(cl::FU), static_cast<const bf16 *>(a.ut) + jh * kD * kC, false);
    transpose_into<kD, kC, 512>(fbuf(cl::FdU), static_cast<const bf16 *>(a.du) + jh * kD * kC, false);
    __syncthreads();

    float dq[4][4], dk[4][4], Z[4][4];
    // dQO = dO S^T: dq += s e^g dQO
    {
        f32x4 t[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) t[u] = zero4();
        prod<4, kD / 32>(t, fbuf(cl::FdO), kC, rb, fbuf(cl::FS), kD, cbD);
#pragma unroll
        for (int u = 0; u < 4; ++u)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                dq[u][i] = sc * __expf(gv[u][i]) * t[u][i];
                dk[u][i] = 0.f;
                Z[u][i] = 0.f;
            }
    }
    // dW = -dU S^T, into F(dW) and F(dW^T)
    {
        f32x4 t[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) t[u] = zero4();
        prod<4, kD / 32>(t, fbuf(cl::FdU), kC, rb, fbuf(cl::FS), kD, cbD);
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            t[u] = -t[u];
            store_n(fbuf(cl::FdW), rb, cbD + u, t[u], kC);
            store_t(fbuf(cl::FdWt), rb, cbD + u, t[u], kD);
        }
    }
    // dAqk = s lower(dO U^T), into F(dAqk) and F(dAqk^T)
    {
        f32x4 t[2];
        t[0] = t[1] = zero4();
        prod<2, kD / 32>(t, fbuf(cl::FdO), kC, rb, fbuf(cl::FU), kC, cbC);
#pragma unroll
        for (int u = 0; u < 2; ++u) {
#pragma unroll
            for (int i = 0; i < 4; ++i) t[u][i] = (16 * (cbC + u) + n) <= row_of(i) ? sc * t[u][i] : 0.f;
            store_n(fbuf(cl::FdAqk), rb, cbC + u, t[u], kC);
            store_t(fbuf(cl::FdAqkt), rb, cbC + u, t[u], kC);
        }
    }
    __syncthreads();  // F(S) read by every wave
    // F(dS') (rows key channel, contraction value column) where F(S) was
#pragma unroll
    for (int qq = 0; qq < 4; ++qq) {
        const V8 dsv = *reinterpret_cast<const V8 *>(dsg + (size_t)(tid + 512 * qq) * 8);
#pragma unroll
        for (int e = 0; e < 8; ++e) fbuf(cl::FS)[frag_off<bf16>(frag_chan<bf16>(qq, hi, e), 16 * w + n, kD)] = dsv[e];
    }
    __syncthreads();
    // dR = U dS'^T: dk += e^(gamma-g) dR, Z += e^(gamma-g) dR; colsum(dR * R) partials
    {
        f32x4 t[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) t[u] = zero4();
        prod<4, kD / 32>(t, fbuf(cl::FU), kC, rb, fbuf(cl::FS), kD, cbD);
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            float cs = 0.f;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const float e = __expf(gcol[u] - gv[u][i]) * t[u][i];
                dk[u][i] += e;
                Z[u][i] += e;
                cs = fmaf(e, kv[u][i], cs);
            }
            cs += __shfl_xor(cs, 16);
            cs += __shfl_xor(cs, 32);
            if (hi == 0) ffl(cl::gpart)[rb * kD + colD(u)] = cs;
        }
    }
    __syncthreads();  // phase-2 buffers but dU, dW, dW^T free

    // ---- phase 3: dT, dBv, dBk
    // F(Bv): rows i, contraction value column; F(Bk): rows i, contraction key channel
    for (int u = tid; u < kC * kD / 8; u += 512) {
        const int gi = u >> 6, kg = gi / (kC / 16), rbs = gi % (kC / 16), r = 16 * rbs + n;
        V8 x;
        const float b = ffl(cl::bet)[r];
#pragma unroll
        for (int e = 0; e < 8; ++e) x[e] = static_cast<bf16>(0.f);
        if (r < L) {
            const bf16 *p = v_g + tok(r) * kD + 32 * kg + 4 * hi;
            const uint2 lo = *reinterpret_cast<const uint2 *>(p), hi2 = *reinterpret_cast<const uint2 *>(p + 16);
            const bf16 *vl = reinterpret_cast<const bf16 *>(&lo), *vh = reinterpret_cast<const bf16 *>(&hi2);
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                x[e] = static_cast<bf16>(b * static_cast<float>(vl[e]));
                x[e + 4] = static_cast<bf16>(b * static_cast<float>(vh[e]));
            }
        }
        *reinterpret_cast<V8 *>(fbuf(cl::FBv) + (size_t)u * 8) = x;
    }
#pragma unroll
    for (int u = 0; u < 4; ++u) {
        f32x4 bk;
#pragma unroll
        for (int i = 0; i < 4; ++i) bk[i] = brow[i] * kv[u][i] * __expf(gv[u][i]);
        store_n(fbuf(cl::FBk), rb, cbD + u, bk, kC);
    }
    __syncthreads();
    // dT = dU Bv^T + dW Bk^T, into F(dT^T)
    {
        f32x4 t[2];
        t[0] = t[1] = zero4();
        prod<2, kD / 32>(t, fbuf(cl::FdU), kC, rb, fbuf(cl::FBv), kC, cbC);
        prod<2, kD / 32>(t, fbuf(cl::FdW), kC, rb, fbuf(cl::FBk), kC, cbC);
#pragma unroll
        for (int u = 0; u < 2; ++u) store_t(fbuf(cl::FdTt), rb, cbC + u, t[u], kC);
    }
    // dBv = T^T dU: dv = beta dBv; rowsum(dBv * v) partials
    {
        f32x4 t[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) t[u] = zero4();
        const bf16 *dut = static_cast<const bf16 *>(a.du) + jh * kD * kC;
        prod<4, kC / 32>(t, fbuf(cl::FTt), kC, rb, dut, kD, cbD);
        float rs[4] = {0.f, 0.f, 0.f, 0.f};
        bf16 *dv = static_cast<bf16 *>(a.dv);
        const int fl = fresh_lane();
#pragma unroll
        for (int u = 0; u < 4; ++u)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int r = KDA_ROW(i), c = KDA_COL(u);
                if (r < L) {
                    dv[tok(r) * kD + c] = static_cast<bf16>(brow[i] * t[u][i]);
                    rs[i] = fmaf(t[u][i], static_cast<float>(v_g[tok(r) * kD + c]), rs[i]);
                }
            }
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            rs[i] = row16_sum(rs[i]);
            if (n == 0) ffl(cl::bpart)[(0 * 2 + half) * kC + row_of(i)] = rs[i];
        }
    }
    // dBk = T^T dW: dk += beta e^g dBk; rowsum(dBk * k e^g) partials
    {
        f32x4 t[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) t[u] = zero4();
        prod<4, kC / 32>(t, fbuf(cl::FTt), kC, rb, fbuf(cl::FdWt), kD, cbD);
        float rs[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int u = 0; u < 4; ++u)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const float eg = __expf(gv[u][i]);
                dk[u][i] = fmaf(brow[i] * eg, t[u][i], dk[u][i]);
                rs[i] = fmaf(t[u][i], kv[u][i] * eg, rs[i]);
            }
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            rs[i] = row16_sum(rs[i]);
            if (n == 0) ffl(cl::bpart)[(1 * 2 + half) * kC + row_of(i)] = rs[i];
        }
    }
    __syncthreads();

    // ---- phase 4: X = T^T dT, dA = strict_lower(-X T^T), dA' = beta dA
    {
        f32x4 t[2];
        t[0] = t[1] = zero4();
        prod<2, kC / 32>(t, fbuf(cl::FTt), kC, rb, fbuf(cl::FdTt), kC, cbC);
#pragma unroll
        for (int u = 0; u < 2; ++u) store_n(fbuf(cl::FX), rb, cbC + u, t[u], kC);
    }
    __syncthreads();
    {
        f32x4 t[2];
        t[0] = t[1] = zero4();
        prod<2, kC / 32>(t, fbuf(cl::FX), kC, rb, fbuf(cl::FT), kC, cbC);
        float rs[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int u = 0; u < 2; ++u) {
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                // above the diagonal G = P N^T can overflow (e^(g_r - g_i) with i after r): selected
                // away, never multiplied by a zero
                const bool low = (16 * (cbC + u) + n) < row_of(i);
                const float dA = low ? -t[u][i] : 0.f;
                rs[i] = low ? fmaf(dA, G[u][i], rs[i]) : rs[i];
                t[u][i] = brow[i] * dA;
            }
            store_n(fbuf(cl::FdAp), rb, cbC + u, t[u], kC);
            store_t(fbuf(cl::FdApt), rb, cbC + u, t[u], kC);
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            rs[i] = row16_sum(rs[i]);
            if (n == 0) ffl(cl::bpart)[(2 * 2 + half) * kC + row_of(i)] = rs[i];
        }
    }
    // ---- phase 5: F(N^T), F(P^T), F(Qe^T) (rows key channel, contraction r)
    float qv[4][4];
    {
        const int fl = fresh_lane();
#pragma unroll
        for (int u = 0; u < 4; ++u)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int r = KDA_ROW(i);
                qv[u][i] = r < L ? static_cast<float>(q_g[tok(r) * kD + KDA_COL(u)]) : 0.f;
            }
    }
#pragma unroll
    for (int u = 0; u < 4; ++u) {
        f32x4 nn, pp, qe;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const float d = fresh(gv[u][i] - mcol[u]), ep = __expf(d), em = __expf(-d);
            nn[i] = kv[u][i] * em;
            pp[i] = kv[u][i] * ep;
            qe[i] = qv[u][i] * ep;
        }
        store_t(fbuf(cl::FNt), rb, cbD + u, nn, kD);
        store_t(fbuf(cl::FPt), rb, cbD + u, pp, kD);
        store_t(fbuf(cl::FQet), rb, cbD + u, qe, kD);
    }
    __syncthreads();
    // dP = dA' N (dk), dQe = dAqk N (dq): both e^(g-m)
    {
        f32x4 tp[4], tq[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) tp[u] = tq[u] = zero4();
        prod<4, kC / 32>(tp, fbuf(cl::FdAp), kC, rb, fbuf(cl::FNt), kD, cbD);
        prod<4, kC / 32>(tq, fbuf(cl::FdAqk), kC, rb, fbuf(cl::FNt), kD, cbD);
#pragma unroll
        for (int u = 0; u < 4; ++u)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const float ep = __expf(gv[u][i] - mcol[u]);
                dk[u][i] = fmaf(ep, tp[u][i], dk[u][i]);
                dq[u][i] = fmaf(ep, tq[u][i], dq[u][i]);
            }
    }
    // dN = dA'^T P + dAqk^T Qe: dk, Z += e^(m-g) dN
    {
        f32x4 t[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) t[u] = zero4();
        prod<4, kC / 32>(t, fbuf(cl::FdApt), kC, rb, fbuf(cl::FPt), kD, cbD);
        prod<4, kC / 32>(t, fbuf(cl::FdAqkt), kC, rb, fbuf(cl::FQet), kD, cbD);
#pragma unroll
        for (int u = 0; u < 4; ++u)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const float e = __expf(mcol[u] - gv[u][i]) * t[u][i];
                dk[u][i] += e;
                Z[u][i] += e;
            }
    }
    __syncthreads();  // region free: dg goes where g was

    // ---- outputs: dq, dk; dg into LDS; then dlog alpha and dbeta
    {
        bf16 *dqg = static_cast<bf16 *>(a.dq), *dkg = static_cast<bf16 *>(a.dk);
        float *Lg = ffl(cl::Lg);
        const int fl = fresh_lane();
#pragma unroll
        for (int u = 0; u < 4; ++u)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int r = KDA_ROW(i), c = KDA_COL(u);
                if (r < L) {
                    dqg[tok(r) * kD + c] = static_cast<bf16>(dq[u][i]);
                    dkg[tok(r) * kD + c] = static_cast<bf16>(dk[u][i]);
                }
                Lg[r * cl::LgP + c] = qv[u][i] * dq[u][i] + kv[u][i] * (dk[u][i] - 2.f * Z[u][i]);
            }
    }
    __syncthreads();
    // dlog alpha: thread (channel c, quarter qq) forms the suffix sums of its 16 rows, then adds
    // the later quarters' totals and dgamma
    {
        const int ft = fresh_tid(), c = ft & (kD - 1), qq = ft >> 7;
        const float *Lg = ffl(cl::Lg);
        float x[16];
#pragma unroll
        for (int r = 0; r < 16; ++r) x[r] = Lg[(16 * qq + r) * cl::LgP + c];
#pragma unroll
        for (int r = 14; r >= 0; --r) x[r] += x[r + 1];
        ffl(cl::qpart)[qq * kD + c] = x[0];
        if (tid < kC) {  // dbeta, rows 0 .. C - 1: its six partial sums in a fixed order
            const float *bp = ffl(cl::bpart);
            float acc = 0.f;
#pragma unroll
            for (int t = 0; t < 6; ++t) acc += bp[t * kC + tid];
            if (tid < L) a.dbeta[tok(tid)] = acc;
        }
        __syncthreads();
        const float *gp = ffl(cl::gpart), *sp = ffl(cl::spart);
        float cs = 0.f, ss = 0.f;
#pragma unroll
        for (int b = 0; b < 4; ++b) cs += gp[b * kD + c];
#pragma unroll
        for (int b = 0; b < 8; ++b) ss += sp[b * kD + c];
        float off = fmaf(__expf(ffl(cl::gam)[c]), ss, cs);
#pragma unroll
        for (int b = 1; b < 4; ++b) off += b > qq ? ffl(cl::qpart)[b * kD + c] : 0.f;
#pragma unroll
        for (int r = 0; r < 16; ++r)
            if (16 * qq + r < L) a.dlog_alpha[tok(16 * qq + r) * kD + c] = x[r] + off;
    }
}
#undef KDA_ROW
#undef KDA_COL

}  // namespace

hipError_t launch_chunk_bwd_bf16(const BwdFastArgs &a, int n_seqs, int total_chunks, hipStream_t stream) {
    // (1) the forward's chunk preparation and (2) state recursion, states recorded
    hipError_t err;
    if (total_chunks > 0) {
        PrepArgs pa{a.q, a.k, a.v, a.log_alpha, a.beta, a.scale, a.H, kGateChannel, PreactArgs{}, a.map, a.buf};
        if ((err = launch_prep(pa, kC, kD, kD, true, total_chunks, stream)) != hipSuccess) return err;
        StateArgs sa{a.h0, nullptr, nullptr, a.discard, a.H, 0, a.map, a.buf, a.st, a.ut};
        if ((err = launch_state(sa, kC, kD, kD, true, n_seqs, stream)) != hipSuccess) return err;
    }
    // (3) the reverse recursion
    hipLaunchKernelGGL(kda_bwd_rev_kernel, dim3(n_seqs * a.H), dim3(512), 0, stream, a);
    if ((err = hipGetLastError()) != hipSuccess) return err;
    // (4) the chunk-local gradients
    if (total_chunks > 0) {
        err = hipFuncSetAttribute(reinterpret_cast<const void *>(kda_bwd_chunk_kernel),
                                  hipFuncAttributeMaxDynamicSharedMemorySize, cl::TOTAL);
        if (err != hipSuccess) return err;
        hipLaunchKernelGGL(kda_bwd_chunk_kernel, dim3(total_chunks * a.H), dim3(512), cl::TOTAL, stream, a);
        if ((err = hipGetLastError()) != hipSuccess) return err;
    }
    return hipSuccess;
}

}  // namespace kda
