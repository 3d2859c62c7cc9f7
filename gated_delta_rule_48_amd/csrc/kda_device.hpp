// kda_device.hpp -- device-side building blocks shared by libkda's kernels
// (gfx950, wave64). Internal to the library.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace kda {

typedef __bf16 bf16;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kWave = 64;

// ---------------------------------------------------------------- conversions

__device__ __forceinline__ float to_f32(float x) { return x; }
__device__ __forceinline__ float to_f32(bf16 x) { return static_cast<float>(x); }

template <typename T> __device__ __forceinline__ T from_f32(float x);
template <> __device__ __forceinline__ float from_f32<float>(float x) { return x; }
template <> __device__ __forceinline__ bf16 from_f32<bf16>(float x) { return static_cast<bf16>(x); }

// ---------------------------------------------------------------- MFMA
//
// One 16x16 fp32 output tile, accumulated over K with the matrix cores.
// Both operands are "K-contiguous": A is row-major [16][K] (row m at A + m*lda)
// and B is given as its transpose, row-major [16][K] (column n of B at
// B + n*ldb). Accumulator layout (both instructions): lane l holds
// C[4*(l/16) + i][l%16] in element i.
//
//  bf16: v_mfma_f32_16x16x32_bf16, lane l supplies A[l%16][8*(l/16) .. +7] and
//        B^T[l%16][8*(l/16) .. +7]  (one 16-byte load each).
//  fp32: v_mfma_f32_16x16x4_f32,   lane l supplies A[l%16][l/16] and B^T[l%16][l/16].

template <typename T> struct Mma;

template <> struct Mma<bf16> {
    typedef bf16x8 Frag;
    static constexpr int kK = 32;   // K per instruction
    static constexpr int kPer = 8;  // consecutive K elements per lane
    __device__ __forceinline__ static Frag load(const bf16 *p) {
        return *reinterpret_cast<const bf16x8 *>(p);
    }
    // kPer fp32 values `stride` apart, rounded to bf16 (to nearest even).
    __device__ __forceinline__ static Frag load_f32(const float *p, int stride) {
        Frag f;
#pragma unroll
        for (int i = 0; i < 8; ++i) f[i] = static_cast<bf16>(p[i * stride]);
        return f;
    }
    __device__ __forceinline__ static f32x4 mma(Frag a, Frag b, f32x4 c) {
        return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
    }
};

template <> struct Mma<float> {
    typedef float Frag;
    static constexpr int kK = 4;
    static constexpr int kPer = 1;
    __device__ __forceinline__ static Frag load(const float *p) { return *p; }
    __device__ __forceinline__ static Frag load_f32(const float *p, int) { return *p; }
    __device__ __forceinline__ static f32x4 mma(Frag a, Frag b, f32x4 c) {
        return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
    }
};

// acc += A[0:16, k0:k1] * (Bt[0:16, k0:k1])^T. A is row-major [16][K] (row m at
// A + m*lda) and Bt is B transposed, row-major [16][K]; both already offset to
// their first row. k0 and k1 are multiples of Mma<T>::kK.
template <typename T>
__device__ __forceinline__ f32x4 mma_nt(f32x4 acc, const T *A, int lda, const T *Bt, int ldb,
                                        int k0, int k1) {
    typedef Mma<T> M;
    const int l = threadIdx.x & (kWave - 1);
    const T *a = A + (l & 15) * lda + (l >> 4) * M::kPer;
    const T *b = Bt + (l & 15) * ldb + (l >> 4) * M::kPer;
    for (int k = k0; k < k1; k += M::kK) acc = M::mma(M::load(a + k), M::load(b + k), acc);
    return acc;
}

// Same with A taken from fp32 storage (rounded to T).
template <typename T>
__device__ __forceinline__ f32x4 mma_nt_f32a(f32x4 acc, const float *A, int lda, const T *Bt,
                                             int ldb, int k0, int k1) {
    typedef Mma<T> M;
    const int l = threadIdx.x & (kWave - 1);
    const float *a = A + (l & 15) * lda + (l >> 4) * M::kPer;
    const T *b = Bt + (l & 15) * ldb + (l >> 4) * M::kPer;
    for (int k = k0; k < k1; k += M::kK) acc = M::mma(M::load_f32(a + k, 1), M::load(b + k), acc);
    return acc;
}

// acc += A[0:16, k0:k1] * B[k0:k1, 0:16] with both in fp32 storage: A row-major
// [16][K], B row-major [K][16] (row k at B + k*ldb), rounded to T.
template <typename T>
__device__ __forceinline__ f32x4 mma_nn_f32(f32x4 acc, const float *A, int lda, const float *B,
                                            int ldb, int k0, int k1) {
    typedef Mma<T> M;
    const int l = threadIdx.x & (kWave - 1);
    const float *a = A + (l & 15) * lda + (l >> 4) * M::kPer;
    const float *b = B + (l >> 4) * M::kPer * ldb + (l & 15);
    for (int k = k0; k < k1; k += M::kK)
        acc = M::mma(M::load_f32(a + k, 1), M::load_f32(b + k * ldb, ldb), acc);
    return acc;
}

// ---------------------------------------------------------------- fragment-ordered tiles
//
// Matrix-core operands stored so that each lane's share of one instruction
// group is 16 contiguous bytes, and the 64 lanes' shares are contiguous: one
// wave reads a whole operand group with a single fully coalesced 1 KB access
// (global memory) or a conflict-free ds_read_b128 (LDS).
//
// A group covers 16 rows x KG contraction indices (KG = 32 for bf16, 16 for
// fp32), EPL = KG / 4 values per lane. Lane l = r + 16*hi holds, in slot j,
// the contraction index
//
//     k = 16 * (j / 4) + 4 * hi + (j % 4)
//
// For bf16 that is one v_mfma_f32_16x16x32_bf16 operand; for fp32 slot j is
// the operand of the j-th of four v_mfma_f32_16x16x4_f32 steps. The order is a
// permutation of the natural one, applied identically to both operands of
// every product, so it does not change any result. It is chosen because a
// 16x16 accumulator tile holds rows 4*hi + 0..3 of column r in lane r + 16*hi:
// the accumulator tiles of contraction indices 0..15 and 16..31 are, slot for
// slot, the operand of the next product, with no data movement.
//
// Groups are stored contraction-major: group (kg, row block rb) of an [R][K]
// matrix starts at element (kg * (R/16) + rb) * 64 * EPL. The same layout serves
// A operands ([M][K]) and transposed B operands ([N][K]).
template <typename T> struct Frag;
template <> struct Frag<bf16> {
    static constexpr int KG = 32, EPL = 8;
    typedef bf16x8 Vec;
    __device__ __forceinline__ static f32x4 mma(f32x4 acc, Vec a, Vec b) {
        return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, acc, 0, 0, 0);
    }
};
template <> struct Frag<float> {
    static constexpr int KG = 16, EPL = 4;
    typedef f32x4 Vec;
    __device__ __forceinline__ static f32x4 mma(f32x4 acc, Vec a, Vec b) {
#pragma unroll
        for (int s = 0; s < 4; ++s) acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a[s], b[s], acc, 0, 0, 0);
        return acc;
    }
};
// contraction index of slot j held by lane group hi, in group kg
template <typename T> __device__ __forceinline__ int frag_chan(int kg, int hi, int j) {
    return Frag<T>::KG * kg + 16 * (j >> 2) + 4 * hi + (j & 3);
}

// Element offset of (r, k) in a fragment-ordered matrix with R rows.
template <typename T>
__device__ __forceinline__ int frag_off(int r, int k, int R) {
    typedef Frag<T> F;
    const int kg = k / F::KG, kk = k % F::KG;
    const int lane = (r & 15) + 16 * ((kk & 15) >> 2), slot = (kk & 3) + 4 * (kk >> 4);
    return ((kg * (R >> 4) + (r >> 4)) * 64 + lane) * F::EPL + slot;
}

// This lane's 16-byte share of group (kg, rb) of a fragment-ordered matrix.
template <typename T>
__device__ __forceinline__ typename Frag<T>::Vec frag_load(const T *base, int kg, int rb, int R) {
    const int l = threadIdx.x & 63;
    return *reinterpret_cast<const typename Frag<T>::Vec *>(
        base + ((kg * (R >> 4) + rb) * 64 + l) * Frag<T>::EPL);
}

// Accumulator-ordered [R][NC] matrix: 16x16 tiles row-block-major, lane l of a
// tile holding rows 4*(l/16) + 0..3 of column l%16 contiguously (the layout of
// a 16x16 matrix-core accumulator).
__device__ __forceinline__ int acc_tile_off(int rb, int cb, int NC) {
    return ((rb * (NC >> 4) + cb) * 64 + (threadIdx.x & 63)) * 4;
}

// Inclusive prefix sum over the 16 lanes of each DPP row (lanes 16m .. 16m+15),
// by shifted adds; lanes shifted in from outside the row contribute zero.
template <int D> __device__ __forceinline__ float dpp_row_shr(float x) {
    return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x),
                                                                 0x110 | D, 0xf, 0xf, true));
}
template <int D> __device__ __forceinline__ float dpp_row_shl(float x) {
    return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x),
                                                                 0x100 | D, 0xf, 0xf, true));
}
// Sum over the later lanes of each 16-lane DPP row (lanes i + 1 .. 15 for lane i): the
// exclusive suffix sum, formed from the values themselves (not as a difference of
// prefix sums, which would cancel where the prefixes are large).
__device__ __forceinline__ float row16_exclusive_suffix_sum(float x) {
    x = dpp_row_shl<1>(x);
    x += dpp_row_shl<1>(x);
    x += dpp_row_shl<2>(x);
    x += dpp_row_shl<4>(x);
    x += dpp_row_shl<8>(x);
    return x;
}
__device__ __forceinline__ float row16_inclusive_sum(float x) {
    x += dpp_row_shr<1>(x);
    x += dpp_row_shr<2>(x);
    x += dpp_row_shr<4>(x);
    x += dpp_row_shr<8>(x);
    return x;
}

// Value of lane I of this lane's 16-lane DPP row (row_newbcast).
template <int I> __device__ __forceinline__ float dpp_row_bcast(float x) {
    return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, x), 0x150 + I, 0xf, 0xf, true));
}

// ---------------------------------------------------------------- strong decay: diagonal Gram tiles pair by pair
//
// Inside one 16-row block of a chunk, the decayed Gram entries
//     A[r][i]   = sum_c k[r][c] k[i][c] e^(g[r][c] - g[i][c])        (i < r)
//     Aqk[r][i] = sum_c q[r][c] k[i][c] e^(g[r][c] - g[i][c])        (i <= r)
// (g: the running sum of log alpha, which does not increase with r) carry a factor
// in (0, 1] for every pair that counts. When the block's decay spans more than the
// fp32 range, no factorisation e^(g[r] - m) e^(m - g[i]) with one reference m keeps
// both factors finite, so these entries are formed one pair at a time, each factor
// from its own exponent. Lane (r, hi) of the calling wave holds N channels of row r
// (the same channels in every lane of its group hi): kf, qf (q times the query scale)
// and g, the prefix local to the block (its offset cancels in g[r] - g[i]).
// diag_pairs_accum adds this lane's share to a[i] (A[r][i]) and aq[i] (Aqk[r][i]) for
// the 16 rows i of the block; diag_pairs_reduce then sums the four lane groups, so that
// every lane of row r holds the totals. Entries with i > r (and a's entry i = r) are
// finite values to be discarded.
template <int I, int N>
__device__ __forceinline__ void diag_pair_sums(const float *kf, const float *qf, const float *g, float *a, float *aq) {
    constexpr float kL2E = 1.4426950408889634f;
    float sa = a[I], sq = aq[I];
#pragma unroll
    for (int c = 0; c < N; ++c) {
        const float ki = dpp_row_bcast<I>(kf[c]);
        const float gi = dpp_row_bcast<I>(g[c]);
        const float kd = ki * __builtin_amdgcn_exp2f(fminf((g[c] - gi) * kL2E, 0.f));
        sa = fmaf(kf[c], kd, sa);
        sq = fmaf(qf[c], kd, sq);
    }
    a[I] = sa;
    aq[I] = sq;
    // one column i at a time: interleaving the sixteen keeps all their broadcasts live
    __builtin_amdgcn_sched_barrier(0);
}

template <int N>
__device__ __forceinline__ void diag_pairs_accum(const float *kf, const float *qf, const float *g, float *a, float *aq) {
    diag_pair_sums<0, N>(kf, qf, g, a, aq);
    diag_pair_sums<1, N>(kf, qf, g, a, aq);
    diag_pair_sums<2, N>(kf, qf, g, a, aq);
    diag_pair_sums<3, N>(kf, qf, g, a, aq);
    diag_pair_sums<4, N>(kf, qf, g, a, aq);
    diag_pair_sums<5, N>(kf, qf, g, a, aq);
    diag_pair_sums<6, N>(kf, qf, g, a, aq);
    diag_pair_sums<7, N>(kf, qf, g, a, aq);
    diag_pair_sums<8, N>(kf, qf, g, a, aq);
    diag_pair_sums<9, N>(kf, qf, g, a, aq);
    diag_pair_sums<10, N>(kf, qf, g, a, aq);
    diag_pair_sums<11, N>(kf, qf, g, a, aq);
    diag_pair_sums<12, N>(kf, qf, g, a, aq);
    diag_pair_sums<13, N>(kf, qf, g, a, aq);
    diag_pair_sums<14, N>(kf, qf, g, a, aq);
    diag_pair_sums<15, N>(kf, qf, g, a, aq);
}

__device__ __forceinline__ void diag_pairs_reduce(float *a, float *aq) {
#pragma unroll
    for (int i = 0; i < 16; ++i) {
        a[i] += __shfl_xor(a[i], 16);
        a[i] += __shfl_xor(a[i], 32);
        aq[i] += __shfl_xor(aq[i], 16);
        aq[i] += __shfl_xor(aq[i], 32);
    }
}

// x[4 hi .. 4 hi + 3] for the lane group hi (0..3), by selects among values held in
// registers (every index is a constant, so the array never needs a memory copy).
__device__ __forceinline__ f32x4 group4(const float *x, int hi) {
    const f32x4 v0 = {x[0], x[1], x[2], x[3]}, v1 = {x[4], x[5], x[6], x[7]};
    const f32x4 v2 = {x[8], x[9], x[10], x[11]}, v3 = {x[12], x[13], x[14], x[15]};
    f32x4 v = v0;
    v = hi == 1 ? v1 : v;
    v = hi == 2 ? v2 : v;
    v = hi == 3 ? v3 : v;
    return v;
}

// Chunks whose summed log alpha falls below -kStrongDecay on some key channel take the
// pair-by-pair path above (the midpoint factors 2^(+-|gamma|/2) of the usual path stay
// within the fp32 range, e^(+-85), only above -170).
constexpr float kStrongDecay = 160.f;

__device__ __forceinline__ int acc_row(int i) { return 4 * ((threadIdx.x & 63) >> 4) + i; }
__device__ __forceinline__ int acc_col() { return threadIdx.x & 15; }

// ---------------------------------------------------------------- sequences and chunks
//
// Sequences are packed along the token axis. Without cu_seqlens there are
// n_seqs sequences of seq_len tokens each. With cu_seqlens, the ranges are the
// ones kda_chunk_offsets_kernel derived from it: clamped into [0, T_total] and
// made non-overlapping and ordered (a malformed table therefore can neither
// move an access out of the buffers nor produce more chunks than the
// workspace holds); chunk_off[s] is the number of chunks of all earlier
// sequences.
struct SeqMap {
    const int32_t *chunk_off; // device [n_seqs + 1] when varlen
    const int32_t *seq_begin; // device [n_seqs] when varlen
    const int32_t *seq_end;   // device [n_seqs] when varlen
    int varlen;
    int n_seqs;
    int seq_len;              // uniform length when !varlen
    int C;

    __device__ __forceinline__ void seq_range(int s, int &t_begin, int &t_end) const {
        if (!varlen) {
            t_begin = s * seq_len;
            t_end = t_begin + seq_len;
        } else {
            t_begin = seq_begin[s];
            t_end = seq_end[s];
        }
    }
    __device__ __forceinline__ int chunks_before(int s) const {
        return !varlen ? s * ((seq_len + C - 1) / C) : chunk_off[s];
    }
    __device__ __forceinline__ int total_chunks() const { return chunks_before(n_seqs); }
    // Global chunk j -> its sequence, first token and length. False if j is past the end.
    __device__ __forceinline__ bool locate(int j, int &s, int &t0, int &len) const {
        if (j >= total_chunks()) return false;
        if (!varlen) {
            s = j / ((seq_len + C - 1) / C);
        } else {  // last s with chunk_off[s] <= j (empty sequences share offsets)
            int lo = 0, hi = n_seqs - 1;
            while (lo < hi) {
                const int mid = (lo + hi + 1) >> 1;
                if (chunk_off[mid] <= j) lo = mid; else hi = mid - 1;
            }
            s = lo;
        }
        int tb, te;
        seq_range(s, tb, te);
        t0 = tb + (j - chunks_before(s)) * C;
        len = min(C, te - t0);
        return true;
    }
};

}  // namespace kda
