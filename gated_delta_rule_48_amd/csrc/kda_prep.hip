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
// Memory access: each thread owns one chunk row's 8 (bf16) or 4 (fp32) adjacent
// channels per operand group and issues all of its loads before any computation.
// The outputs leave in the fragment-ordered layouts the state kernel reads: QO as
// row groups, KtT, Aqk and W as accumulator tiles of their transposes, which the
// matrix cores form (a product with an identity operand, or the operands of a
// product with their roles swapped) and which are each lane's four consecutive
// operand slots; U~ as accumulator tiles.

#include "kda_internal.hpp"
#include "kda_solve.hpp"

namespace kda {
namespace {

template <int C, int DK, int DV, typename T> struct PrepCfg {
    typedef Frag<T> F;
    static constexpr int NW = C / 16, NT = 64 * NW;   // wave w owns chunk rows 16w .. 16w+15
    static constexpr int NKG = DK / F::KG, NVG = DV / F::KG;
    static constexpr int PT = C + 4;                  // pitch of the fp32 [C][C] matrix A (then T)
    // columns of W / U~ per pass of the final product (LDS budget)
    static constexpr int PW = (sizeof(T) == 4 && C == 128) ? 64 : 128;
    static constexpr size_t mx(size_t a, size_t b) { return a > b ? a : b; }
    // sums, offsets, exp(gamma/2), beta; the strong-decay path's block prefixes and gamma
    // (log2 units), its flags and the diagonal blocks of A
    static constexpr size_t SMALL =
        (size_t)(2 * NW * DK + DK + C + (NW + 1) * DK + 4 + NW * (NW + 1) / 2 * 256 + NW * DK) * 4;
    static constexpr size_t MATF = (size_t)C * PT * 4;                   // A, then T in place
    static constexpr size_t KMB = (size_t)C * DK * sizeof(T);            // Km (Gram operand)
    static constexpr size_t OPB = (size_t)PW * C * sizeof(T);            // B operand of one W / U~ pass
    static constexpr size_t REGION = mx(mx(KMB, MATF), OPB);
    static constexpr size_t SMEM = SMALL + REGION;
};

// This lane's operand share of group kg of one row (the values at channels
// frag_chan<T>(kg, hi, 0..EPL-1)), from a row in global memory: runs of 4
// consecutive channels.
template <typename T>
__device__ __forceinline__ typename Frag<T>::Vec load_row_frag(const T *row, int kg, int hi) {
    typedef Frag<T> F;
    typename F::Vec v;
    if constexpr (sizeof(T) == 2) {
        const uint2 a = *reinterpret_cast<const uint2 *>(row + frag_chan<T>(kg, hi, 0));
        const uint2 b = *reinterpret_cast<const uint2 *>(row + frag_chan<T>(kg, hi, 4));
        const bf16 *pa = reinterpret_cast<const bf16 *>(&a), *pb = reinterpret_cast<const bf16 *>(&b);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            v[e] = pa[e];
            v[4 + e] = pb[e];
        }
    } else {
        v = *reinterpret_cast<const f32x4 *>(row + frag_chan<T>(kg, hi, 0));
    }
    return v;
}

// The fp32 values at the same channels (log alpha is fp32 for both dtypes).
template <typename T>
__device__ __forceinline__ void load_row_f32(const float *row, int kg, int hi, float *out) {
#pragma unroll
    for (int r4 = 0; r4 < Frag<T>::EPL / 4; ++r4) {
        const f32x4 a = *reinterpret_cast<const f32x4 *>(row + frag_chan<T>(kg, hi, 4 * r4));
#pragma unroll
        for (int e = 0; e < 4; ++e) out[4 * r4 + e] = a[e];
    }
}

template <typename T> __device__ __forceinline__ typename Frag<T>::Vec pack_frag(const float *x) {
    typename Frag<T>::Vec v;
#pragma unroll
    for (int j = 0; j < Frag<T>::EPL; ++j) v[j] = from_f32<T>(x[j]);
    return v;
}

// A-operand fragment group kg of row block `row0` taken from an fp32 row-major
// matrix (pitch ld), rounded to T.
template <typename T>
__device__ __forceinline__ typename Frag<T>::Vec a_frag_f32(const float *M, int ld, int row0, int kg) {
    const int l = threadIdx.x & 63;
    typename Frag<T>::Vec v;
    const float *p = M + (row0 + (l & 15)) * ld;
#pragma unroll
    for (int r4 = 0; r4 < Frag<T>::EPL / 4; ++r4) {
        const f32x4 a = *reinterpret_cast<const f32x4 *>(p + frag_chan<T>(kg, l >> 4, 4 * r4));
#pragma unroll
        for (int e = 0; e < 4; ++e) v[4 * r4 + e] = from_f32<T>(a[e]);
    }
    return v;
}

// The identity of tile t of a contraction group as a B operand: lane (n, hi) has a
// one in the slot whose contraction index is 16 t + n. The product of a row group X
// (16 rows x KG contraction indices) with it is the 16 x 16 accumulator tile
// X[:, 16 t .. 16 t + 15], exactly (each entry is one product with 1).
template <typename T> __device__ __forceinline__ typename Frag<T>::Vec ident_op(int t) {
    const int l = threadIdx.x & 63, n = l & 15, hi = l >> 4;
    typename Frag<T>::Vec v;
#pragma unroll
    for (int j = 0; j < Frag<T>::EPL; ++j) v[j] = from_f32<T>(frag_chan<T>(0, hi, j) == 16 * t + n ? 1.f : 0.f);
    return v;
}

// Accumulator tile acc (lane n + 16 hi holds its entries (4 hi + i, n)) stored
// transposed into the fragment-ordered [R][K] matrix at base: entry (4 hi + i, n)
// becomes row 16 rb + n, contraction index 16 kb + 4 hi + i. Those are four
// consecutive slots of the same lane: one 8-byte (bf16) or 16-byte (fp32) store.
template <typename T>
__device__ __forceinline__ void store_tile_t(T *base, int R, int kb, int rb, f32x4 acc) {
    constexpr int WPG = Frag<T>::KG / 16;
    const int l = threadIdx.x & 63;
    T *p = base + (((kb / WPG) * (R >> 4) + rb) * 64 + l) * Frag<T>::EPL + 4 * (kb % WPG);
    if constexpr (sizeof(T) == 2) {
        typedef __bf16 b4 __attribute__((ext_vector_type(4)));
        *reinterpret_cast<b4 *>(p) = __builtin_convertvector(acc, b4);
    } else {
        *reinterpret_cast<f32x4 *>(p) = acc;
    }
}

// kStrong = false: the usual kernel. A chunk whose decay some channel sums below
// -kStrongDecay is left to the second instance: this one records it in a.buf.strong and
// writes nothing else for it. kStrong = true: runs after the first, on the recorded
// chunks only (the others return at once), with every exponent <= 0 (steps 3 and 4 below).
template <int C, int DK, int DV, typename T, bool kStrong>
__global__ __launch_bounds__(4 * C) void kda_prep_kernel(PrepArgs a) {
    typedef PrepCfg<C, DK, DV, T> P;
    typedef Frag<T> F;
    typedef typename F::Vec V;
    constexpr int NW = P::NW, NT = P::NT, NKG = P::NKG, NVG = P::NVG, PT = P::PT, PW = P::PW;
    constexpr int EPL = F::EPL, KG = F::KG, TPG = KG / 16;  // 16-column tiles per contraction group
    constexpr float kL2E = 1.4426950408889634f;             // exponents in base 2
    constexpr float kClamp = 85.f * kL2E;                    // |exponent| limit of the Gram factors

    extern __shared__ __align__(16) unsigned char smem[];
    float *tot = reinterpret_cast<float *>(smem);  // [NW][DK] per-wave sums of log alpha
    float *off = tot + NW * DK;                     // [NW][DK] (sum before row block w - gamma/2) log2(e)
    float *eh = off + NW * DK;                      // [DK] exp(gamma / 2)
    float *bet = eh + DK;                           // [C] beta per chunk row
    float *gpre = bet + C;                          // [NW + 1][DK] log2 decay before row block w (strong path)
    float *gam2 = gpre + NW * DK;                   // [DK]: row NW of gpre, gamma log2(e)
    int *sflag = reinterpret_cast<int *>(gam2 + DK);  // [4] some channel of the chunk decays strongly
    // [NW (NW + 1) / 2][256] A's tiles (w, tj <= w), rows scaled by beta (strong path): tile
    // w (w + 1) / 2 + tj; the diagonal ones row-major, the others in accumulator order
    float *ast = gam2 + DK + 4;
    float *gpost = ast + NW * (NW + 1) / 2 * 256;   // [NW][DK] log2 decay after row block w (strong path)
    unsigned char *R = smem + P::SMALL;
    T *Km = reinterpret_cast<T *>(R);               // [C][DK] frag order: k exp(m - g)  (Gram)
    float *Am = reinterpret_cast<float *>(R);       // [C][PT] A, then T = (I + A)^{-1} in place
    T *OpB = reinterpret_cast<T *>(R);              // [PW][C] frag order: B operand of a W / U~ pass

    const int j = blockIdx.x, h = blockIdx.y;
    int s, t0, L;
    if (!a.map.locate(j, s, t0, L)) return;  // past the last chunk (same for the whole block)
    (void)s;
    if constexpr (kStrong) {
        if (a.buf.strong[(size_t)j * a.H + h] == 0) return;  // done by the usual instance
    }
    const int tid = threadIdx.x, w = tid >> 6, l = tid & 63, lr = l & 15, hi = l >> 4;
    const int r = 16 * w + lr;  // the chunk row this lane holds
    const bool valid = r < L;
    const int H = a.H;
    const size_t tok = (size_t)(t0 + (valid ? r : 0)) * H + h;
    const size_t jh = (size_t)j * H + h;
    const float scale = a.scale;
    const f32x4 zero4 = {0.f, 0.f, 0.f, 0.f};

    // ---- 0. this lane's row of k, q and log alpha, in matrix-core operand order (q, k
    //         activated and normalised when asked), and the inclusive running sum of log
    //         alpha within the wave's 16 rows (DPP scan)
    float gsuf[NKG][EPL];  // strong instance: log alpha summed over the later rows of the block
    auto load_kqg = [&](V (&kr_)[NKG], V (&qr_)[NKG], float (&g_)[NKG][EPL]) {
#pragma unroll
        for (int kg = 0; kg < NKG; ++kg) {
            if (valid) {
                kr_[kg] = load_row_frag<T>(static_cast<const T *>(a.k) + tok * DK, kg, hi);
                qr_[kg] = load_row_frag<T>(static_cast<const T *>(a.q) + tok * DK, kg, hi);
                if (a.gate == kGateChannel) {
                    load_row_f32<T>(a.log_alpha + tok * DK, kg, hi, g_[kg]);
                } else if (a.gate == kGatePreact) {  // -exp(A_log) softplus(a + dt_bias)
                    const V ar = load_row_frag<T>(static_cast<const T *>(a.pre.a) + tok * DK, kg, hi);
                    const float eA = expf(a.pre.A_log[h]);
                    float db[EPL];
                    load_row_f32<T>(a.pre.dt_bias + (size_t)h * DK, kg, hi, db);
#pragma unroll
                    for (int e = 0; e < EPL; ++e) g_[kg][e] = -eA * softplus_f(to_f32(ar[e]) + db[e]);
                } else {  // one decay for every channel of the row, or none
                    const float x = a.gate == kGateHead ? a.log_alpha[tok] : 0.f;
#pragma unroll
                    for (int e = 0; e < EPL; ++e) g_[kg][e] = x;
                }
            } else {
#pragma unroll
                for (int e = 0; e < EPL; ++e) {
                    kr_[kg][e] = from_f32<T>(0.f);
                    qr_[kg][e] = from_f32<T>(0.f);
                    g_[kg][e] = 0.f;
                }
            }
        }
        if (a.pre.qk_norm) {
            // q, k = silu(.) / ||silu(.)|| over the row, whose channels lie in lanes lr + 16 hi:
            // the sums of squares by two lane exchanges, then silu again, scaled (rows past the
            // end are zero and stay zero)
            float sk = 0.f, sq = 0.f;
#pragma unroll
            for (int kg = 0; kg < NKG; ++kg)
#pragma unroll
                for (int e = 0; e < EPL; ++e) {
                    const float x = silu_f(to_f32(kr_[kg][e])), y = silu_f(to_f32(qr_[kg][e]));
                    sk += x * x;
                    sq += y * y;
                }
            sk += __shfl_xor(sk, 16);
            sk += __shfl_xor(sk, 32);
            sq += __shfl_xor(sq, 16);
            sq += __shfl_xor(sq, 32);
            const float rk = 1.f / fmaxf(sqrtf(sk), kNormEps), rq = 1.f / fmaxf(sqrtf(sq), kNormEps);
#pragma unroll
            for (int kg = 0; kg < NKG; ++kg)
#pragma unroll
                for (int e = 0; e < EPL; ++e) {
                    kr_[kg][e] = from_f32<T>(silu_f(to_f32(kr_[kg][e])) * rk);
                    qr_[kg][e] = from_f32<T>(silu_f(to_f32(qr_[kg][e])) * rq);
                }
        }
#pragma unroll
        for (int kg = 0; kg < NKG; ++kg)
#pragma unroll
            for (int e = 0; e < EPL; ++e) {
                if constexpr (kStrong) gsuf[kg][e] = row16_exclusive_suffix_sum(g_[kg][e]);
                g_[kg][e] = row16_inclusive_sum(g_[kg][e]);
            }
    };
    V kr[NKG], qr[NKG], vr[NVG];
    float g[NKG][EPL];
    float b = 0.f;
    load_kqg(kr, qr, g);
#pragma unroll
    for (int kg = 0; kg < NVG; ++kg) {
        if (valid) {
            vr[kg] = load_row_frag<T>(static_cast<const T *>(a.v) + tok * DV, kg, hi);
        } else {
#pragma unroll
            for (int e = 0; e < EPL; ++e) vr[kg][e] = from_f32<T>(0.f);
        }
    }
    if (valid) b = a.gate == kGatePreact ? sigmoid_f(a.beta[tok]) : a.beta[tok];
    if (hi == 0) bet[r] = b;

    // ---- 1. the row blocks' sums of log alpha to LDS
#pragma unroll
    for (int kg = 0; kg < NKG; ++kg)
#pragma unroll
        for (int e = 0; e < EPL; ++e)
            if (lr == 15) tot[w * DK + frag_chan<T>(kg, hi, e)] = g[kg][e];
    __syncthreads();

    // ---- 2. per key channel (one thread each): each row block's offset, summed in
    //         row-block order, less gamma / 2 (in base 2); exp(gamma / 2) to LDS and
    //         exp(gamma) to memory
    if (tid < DK) {
        float pre[NW], acc = 0.f;
#pragma unroll
        for (int ww = 0; ww < NW; ++ww) {
            pre[ww] = acc;
            acc += tot[ww * DK + tid];
        }
        const float m = 0.5f * acc;
#pragma unroll
        for (int ww = 0; ww < NW; ++ww) {
            off[ww * DK + tid] = (pre[ww] - m) * kL2E;
            gpre[ww * DK + tid] = pre[ww] * kL2E;
        }
        gam2[tid] = acc * kL2E;
        float post = 0.f;  // the later row blocks' decay, summed from the end
#pragma unroll
        for (int ww = NW - 1; ww >= 0; --ww) {
            gpost[ww * DK + tid] = post * kL2E;
            post += tot[ww * DK + tid];
        }
        eh[tid] = __builtin_amdgcn_exp2f(m * kL2E);
        a.buf.eg[jh * DK + tid] = __builtin_amdgcn_exp2f(acc * kL2E);
        const unsigned long long st = __ballot(acc < -kStrongDecay);
        if ((tid & 63) == 0) sflag[tid >> 6] = st != 0ull;
    }
    __syncthreads();
    if constexpr (!kStrong) {
        // a chunk past the midpoint factors' range goes to the strong instance
        const bool strong = __builtin_amdgcn_readfirstlane(DK > 64 ? (sflag[0] | sflag[1]) : sflag[0]) != 0;
        if (tid == 0) a.buf.strong[jh] = strong ? 1 : 0;
        if (strong) return;
    }

    // ---- 3. elementwise, with d = (g - gamma/2) log2(e) clamped, ep = 2^d, em = 2^-d
    //         and E = exp(gamma/2): the Gram factors Kp = k ep and Qp = scale q ep
    //         (registers) and Km = k em (LDS); QO = Qp E (memory); KtT = (Km E)^T,
    //         transposed by the matrix cores (memory); and the rows beta Kp E of W's
    //         operand (registers). In this instance's range (|gamma| <= 160) no factor
    //         is clamped, so Qp E = scale q exp(g) and Km E = k exp(gamma - g).
    T *gQO = static_cast<T *>(a.buf.QO) + jh * C * DK;
    T *gKtT = static_cast<T *>(a.buf.KtT) + jh * DK * C;
    V idt[TPG];
#pragma unroll
    for (int t = 0; t < TPG; ++t) idt[t] = ident_op<T>(t);
    V kb[NKG];
    T *gAqk = static_cast<T *>(a.buf.Aqk) + jh * C * C;
    f32x4 akk[NW];
    // ---- 4. decayed Gram tiles of this wave's row block: A's tiles (w, tj <= w), and,
    //         with the operands' roles swapped, the tiles of Aqk^T = Km Qp^T, whose
    //         entries are Aqk's operand slots (stored to memory, zero above the diagonal)
    // (each path runs steps 3 and 4 as one block: the values one path keeps from step 3
    // to step 4 are never live in the other)
    if constexpr (kStrong) {
        // QO = scale q 2^ga, KtT = (k 2^(gamma - ga))^T and W's rows beta k 2^ga, with ga the
        // chunk's log2 decay up to the row (each exponent <= 0: underflow gives the value's
        // own negligible size); and this block's Gram column operand k 2^(b - ga) in Km,
        // b = the decay up to the block's last row (<= 1 as well). gamma - ga and b - ga are
        // formed from suffix sums.
#pragma unroll
        for (int kg = 0; kg < NKG; ++kg) {
            float xo[EPL], xk[EPL], xb[EPL], xc[EPL];
#pragma unroll
            for (int e = 0; e < EPL; ++e) {
                const int ch = frag_chan<T>(kg, hi, e);
                // the decay from the chunk's start to the row (a prefix) and from the row to the
                // block's and the chunk's end (suffix sums, exact where they are small)
                const float ga = g[kg][e] * kL2E + gpre[w * DK + ch], sb = gsuf[kg][e] * kL2E;
                const float eg = __builtin_amdgcn_exp2f(ga), egr = __builtin_amdgcn_exp2f(sb + gpost[w * DK + ch]);
                const float kv = to_f32(kr[kg][e]), qv = scale * to_f32(qr[kg][e]);
                xo[e] = qv * eg;
                xk[e] = kv * egr;
                xb[e] = b * kv * eg;
                xc[e] = kv * __builtin_amdgcn_exp2f(fminf(sb, 0.f));
            }
            *reinterpret_cast<V *>(gQO + ((kg * NW + w) * 64 + l) * EPL) = pack_frag<T>(xo);
            kb[kg] = pack_frag<T>(xb);
            *reinterpret_cast<V *>(Km + ((kg * NW + w) * 64 + l) * EPL) = pack_frag<T>(xc);
            const V kk = pack_frag<T>(xk);
#pragma unroll
            for (int t = 0; t < TPG; ++t) store_tile_t<T>(gKtT, DK, w, TPG * kg + t, F::mma(zero4, kk, idt[t]));
            __builtin_amdgcn_sched_barrier(0);
        }
        __syncthreads();  // Km complete
        // the diagonal tile pair by pair, 8 channels at a time: A's entries to LDS (ast),
        // Aqk's (as its transposed tile) to memory
        {
            float ad16[16], aqd[16];
#pragma unroll
            for (int i = 0; i < 16; ++i) ad16[i] = aqd[i] = 0.f;
            constexpr int GPB = 8 / EPL;  // operand groups per 8-channel batch
#pragma unroll
            for (int kb0 = 0; kb0 < NKG; kb0 += GPB) {
                float kf[8], qf[8];
#pragma unroll
                for (int x = 0; x < GPB; ++x)
#pragma unroll
                    for (int e = 0; e < EPL; ++e) {
                        kf[x * EPL + e] = to_f32(kr[kb0 + x][e]);
                        qf[x * EPL + e] = scale * to_f32(qr[kb0 + x][e]);
                    }
                diag_pairs_accum<8>(kf, qf, &g[kb0][0], ad16, aqd);
            }
            diag_pairs_reduce(ad16, aqd);
            const f32x4 a4 = group4(ad16, hi), q4 = group4(aqd, hi);
            f32x4 aq;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                // A[r][16 w + 4 hi + i], strictly lower, rows scaled by beta; entry (4 hi + i, lr)
                // of this tile of Aqk^T is Aqk[16 w + lr][16 w + 4 hi + i], kept for i <= r
                ast[(w * (w + 1) / 2 + w) * 256 + lr * 16 + 4 * hi + i] = 4 * hi + i < lr ? b * a4[i] : 0.f;
                aq[i] = (4 * hi + i <= lr) ? q4[i] : 0.f;
            }
            store_tile_t<T>(gAqk, C, w, w, aq);
        }
        // the tiles left of the diagonal, (w, tj < w), with the end of block tj as the
        // reference: rows k 2^(ga - b_tj) and scale q 2^(ga - b_tj), columns Km of block tj
        // (both <= 1); A's tiles to LDS (ast, rows scaled by beta)
        const f32x4 bv = *reinterpret_cast<const f32x4 *>(bet + 16 * w + 4 * hi);
#pragma unroll
        for (int tj = 0; tj < NW; ++tj) {
            f32x4 aq = zero4;
            if (tj == w) continue;  // stored above
            if (tj < w) {
                f32x4 at = zero4;
#pragma unroll
                for (int kg = 0; kg < NKG; ++kg) {
                    float xr[EPL], xs[EPL];
#pragma unroll
                    for (int e = 0; e < EPL; ++e) {
                        const int ch = frag_chan<T>(kg, hi, e);
                        const float f = __builtin_amdgcn_exp2f(
                            fminf(g[kg][e] * kL2E + gpre[w * DK + ch] - gpre[(tj + 1) * DK + ch], 0.f));
                        xr[e] = to_f32(kr[kg][e]) * f;
                        xs[e] = scale * to_f32(qr[kg][e]) * f;
                    }
                    const V bm = frag_load<T>(Km, kg, tj, C);
                    at = F::mma(at, pack_frag<T>(xr), bm);
                    aq = F::mma(aq, bm, pack_frag<T>(xs));
                    __builtin_amdgcn_sched_barrier(0);  // (keeps each group's LDS reads next to their use)
                }
                *reinterpret_cast<f32x4 *>(ast + (w * (w + 1) / 2 + tj) * 256 + 4 * l) = at * bv;
            }
            store_tile_t<T>(gAqk, C, tj, w, aq);
        }
    } else {
        V kp[NKG], qp[NKG];
    #pragma unroll
        for (int kg = 0; kg < NKG; ++kg) {
            float xo[EPL], xp[EPL], xq[EPL], xm[EPL], xk[EPL], xb[EPL];
    #pragma unroll
            for (int e = 0; e < EPL; ++e) {
                const int ch = frag_chan<T>(kg, hi, e);
                const float d = __builtin_amdgcn_fmed3f(fmaf(g[kg][e], kL2E, off[w * DK + ch]), -kClamp, kClamp);
                const float ep = __builtin_amdgcn_exp2f(d), em = __builtin_amdgcn_exp2f(-d), E = eh[ch];
                const float kv = to_f32(kr[kg][e]), qv = scale * to_f32(qr[kg][e]);
                xp[e] = kv * ep;
                xq[e] = qv * ep;
                xm[e] = kv * em;
                xo[e] = xq[e] * E;
                xk[e] = xm[e] * E;
                xb[e] = b * xp[e] * E;
            }
            *reinterpret_cast<V *>(gQO + ((kg * NW + w) * 64 + l) * EPL) = pack_frag<T>(xo);
            kp[kg] = pack_frag<T>(xp);
            qp[kg] = pack_frag<T>(xq);
            kb[kg] = pack_frag<T>(xb);
            *reinterpret_cast<V *>(Km + ((kg * NW + w) * 64 + l) * EPL) = pack_frag<T>(xm);
            const V kk = pack_frag<T>(xk);
    #pragma unroll
            for (int t = 0; t < TPG; ++t) store_tile_t<T>(gKtT, DK, w, TPG * kg + t, F::mma(zero4, kk, idt[t]));
        }
        __syncthreads();  // Km complete
    #pragma unroll
        for (int tj = 0; tj < NW; ++tj) {
            akk[tj] = zero4;
            f32x4 aq = zero4;
            if (tj <= w) {
    #pragma unroll
                for (int kg = 0; kg < NKG; ++kg) {
                    const V bm = frag_load<T>(Km, kg, tj, C);
                    akk[tj] = F::mma(akk[tj], kp[kg], bm);
                    aq = F::mma(aq, bm, qp[kg]);
                }
                if (tj == w) {  // entry (4 hi + i, lr) is Aqk[16 w + lr][16 w + 4 hi + i]: kept for i <= r
    #pragma unroll
                    for (int i = 0; i < 4; ++i) aq[i] = (4 * hi + i <= lr) ? aq[i] : 0.f;
                }
            }
            store_tile_t<T>(gAqk, C, tj, w, aq);
        }
    }
    __syncthreads();  // Km is no longer read: the region takes A
    // A (strictly lower, rows scaled by beta, zero elsewhere) -> fp32 LDS
    if constexpr (kStrong) {
#pragma unroll
        for (int tj = 0; tj < NW; ++tj) {
            const float *st = ast + (w * (w + 1) / 2 + tj) * 256;
            if (tj == w) {  // the diagonal block (row r, columns 4 hi ..), zero above it
                const f32x4 x = *reinterpret_cast<const f32x4 *>(st + lr * 16 + 4 * hi);
                *reinterpret_cast<f32x4 *>(Am + r * PT + 16 * w + 4 * hi) = x;
            } else {
                const f32x4 x = tj < w ? *reinterpret_cast<const f32x4 *>(st + 4 * l) : zero4;
#pragma unroll
                for (int i = 0; i < 4; ++i) Am[(16 * w + acc_row(i)) * PT + 16 * tj + acc_col()] = x[i];
            }
        }
    } else {
#pragma unroll
        for (int tj = 0; tj < NW; ++tj)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int rr = 16 * w + acc_row(i), cc = 16 * tj + acc_col();
                Am[rr * PT + cc] = (tj <= w && cc < rr) ? bet[rr] * akk[tj][i] : 0.f;
            }
    }
    __syncthreads();

    // ---- 5. T = (I + A)^{-1}, in place
    unit_lower_inverse<C, PT, T, NT>(Am);

    // ---- 6. W = T (beta k exp(g)) and U~ = T (beta v), PW output columns per pass
    constexpr int NCG = C / KG;
    const int kgmax = ((w + 1) * 16 + KG - 1) / KG;  // T is lower triangular
    V tf[NCG];
#pragma unroll
    for (int kg = 0; kg < NCG; ++kg)
        if (kg < kgmax) tf[kg] = a_frag_f32<T>(Am, PT, 16 * w, kg);
    __syncthreads();  // T is in registers: the region takes the B operands
    T *gW = static_cast<T *>(a.buf.W) + jh * C * DK;
    T *gU = static_cast<T *>(a.buf.U) + jh * C * DV;
    // one pass: output columns [c0, c0 + width) of W (isW) or of U~
    auto pass = [&](bool isW, int c0, int width) {
        // B operand [width][C]: this wave's rows of beta k exp(g) (W) or beta v (U~),
        // transposed by the matrix cores
#pragma unroll
        for (int kg = 0; kg < (isW ? NKG : NVG); ++kg) {
            V x;
            if (isW) {
                x = kb[kg];
            } else {
                float xv[EPL];
#pragma unroll
                for (int e = 0; e < EPL; ++e) xv[e] = b * to_f32(vr[kg][e]);
                x = pack_frag<T>(xv);
            }
#pragma unroll
            for (int t = 0; t < TPG; ++t) {
                const int cb = TPG * kg + t;
                if (16 * cb >= c0 && 16 * cb < c0 + width)
                    store_tile_t<T>(OpB, width, w, cb - c0 / 16, F::mma(zero4, x, idt[t]));
            }
        }
        __syncthreads();
        for (int tc = 0; tc < width / 16; ++tc) {
            f32x4 acc = zero4;
            if (isW) {
                // W^T's tile (columns c0 + 16 tc .., rows 16 w ..), from the operands with
                // their roles swapped: its entries are W's operand slots
#pragma unroll
                for (int kg = 0; kg < NCG; ++kg)
                    if (kg < kgmax) acc = F::mma(acc, frag_load<T>(OpB, kg, tc, width), tf[kg]);
                store_tile_t<T>(gW, C, c0 / 16 + tc, w, acc);
            } else {
#pragma unroll
                for (int kg = 0; kg < NCG; ++kg)
                    if (kg < kgmax) acc = F::mma(acc, tf[kg], frag_load<T>(OpB, kg, tc, width));
                T *dst = gU + acc_tile_off(w, (c0 >> 4) + tc, DV);
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
    };
    constexpr int PWK = DK < PW ? DK : PW, PWV = DV < PW ? DV : PW;
#pragma unroll
    for (int p = 0; p < DK / PWK; ++p) pass(true, p * PWK, PWK);
#pragma unroll
    for (int p = 0; p < DV / PWV; ++p) pass(false, p * PWV, PWV);
}

template <int C, int DK, int DV, typename T>
hipError_t launch_prep_t(const PrepArgs &a, int n_chunks_grid, hipStream_t stream) {
    constexpr size_t smem = PrepCfg<C, DK, DV, T>::SMEM;
    static_assert(smem <= 160 * 1024, "prep LDS budget");
    // the usual instance, then the strong-decay one over the chunks the first left to it
    auto fast = kda_prep_kernel<C, DK, DV, T, false>;
    auto strong = kda_prep_kernel<C, DK, DV, T, true>;
    for (auto kern : {fast, strong}) {
        hipError_t err = hipFuncSetAttribute(reinterpret_cast<const void *>(kern),
                                             hipFuncAttributeMaxDynamicSharedMemorySize, (int)smem);
        if (err != hipSuccess) return err;
        hipLaunchKernelGGL(kern, dim3(n_chunks_grid, a.H), dim3(4 * C), smem, stream, a);
        err = hipGetLastError();
        if (err != hipSuccess) return err;
    }
    return hipSuccess;
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
// holds. off[s] = sum_{s' < s} ceil((te - tb) / C) (at least min_one each) <= ceil(T / C) + n_seqs.
// One thread; the loop is over sequences only.
__global__ void kda_chunk_offsets_kernel(const int32_t *cu, int n_seqs, int T_total, int C,
                                         int32_t *off, int32_t *tb_out, int32_t *te_out, int min_one) {
    if (threadIdx.x != 0 || blockIdx.x != 0) return;
    int acc = 0, prev_end = 0;
    for (int s = 0; s < n_seqs; ++s) {
        const int tb = min(max(cu[s], prev_end), T_total);
        const int te = min(max(cu[s + 1], tb), T_total);
        off[s] = acc;
        tb_out[s] = tb;
        te_out[s] = te;
        acc += max((te - tb + C - 1) / C, min_one);
        prev_end = te;
    }
    off[n_seqs] = acc;
}

}  // namespace

hipError_t launch_chunk_offsets(const int32_t *cu, int n_seqs, int T_total, int C, int32_t *off,
                                int32_t *tb, int32_t *te, hipStream_t stream, int min_one) {
    hipLaunchKernelGGL(kda_chunk_offsets_kernel, dim3(1), dim3(64), 0, stream, cu, n_seqs, T_total,
                       C, off, tb, te, min_one);
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
