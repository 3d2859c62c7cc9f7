// kda_state.hip -- state propagation and outputs of the chunked KDA forward.
//
// One workgroup (C/16 waves) per (sequence, head, slice of DVS value columns).
// The columns of the state evolve independently (every term of the update acts
// on S from the left or row-wise), so a head's d_v columns split over
// workgroups without any exchange. The workgroup walks its sequence's chunks
// in order, keeping its d_k x DVS slice of the fp32 state in registers
// (matrix-core accumulators), and for each chunk computes, with the per-chunk
// quantities of kda_prep.hip:
//
//   U   = U~ - W S                 the chunk's corrected writes
//   O   = QO S + Aqk U             outputs: entering state plus in-chunk part
//   S  <- exp(gamma) S + KtT U     state leaving the chunk
//
// This is the chunk loop of the WY algorithm in the essay "22,580: from GPT-2
// to Kimi K3" (yichencityu.github.io, section 6.3: u = U - w S,
// o = q S + tril(q k^T) u, S += k^T u), with KDA's per-channel decay folded
// into W, QO, Aqk, KtT and exp(gamma).
//
// The per-chunk operands are stored fragment-ordered, so each wave fetches its
// share with fully coalesced 16-byte-per-lane loads; on the bf16 path the next
// chunk's share is fetched while the current chunk computes. Only S (rounded
// to the operand type) and U pass through LDS, as transposed B operands.

#include "kda_internal.hpp"

namespace kda {
namespace {

template <typename T> struct Acc4;  // four io-dtype values of one accumulator lane
template <> struct Acc4<bf16> {
    typedef uint2 Raw;
    __device__ __forceinline__ static float get(Raw r, int i) {
        return static_cast<float>(reinterpret_cast<const bf16 *>(&r)[i]);
    }
};
template <> struct Acc4<float> {
    typedef f32x4 Raw;
    __device__ __forceinline__ static float get(Raw r, int i) { return r[i]; }
};

// Store 4 consecutive contraction indices k0..k0+3 (k0 % 4 == 0) of row n of a
// fragment-ordered matrix with R rows.
template <typename T>
__device__ __forceinline__ void frag_store4(T *base, int n, int k0, f32x4 v, int R) {
    if constexpr (sizeof(T) == 2) {
        bf16 x[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) x[i] = static_cast<bf16>(v[i]);
        *reinterpret_cast<uint2 *>(base + frag_off<T>(n, k0, R)) = *reinterpret_cast<const uint2 *>(x);
    } else {
#pragma unroll
        for (int i = 0; i < 4; ++i) base[frag_off<T>(n, k0 + i, R)] = v[i];
    }
}

// kRecord: the backward pass's instance, which also records S^T and U^T of every chunk
// (StateArgs::st_out, ut_out) and writes no outputs.
template <int C, int DK, int DV, int DVS, typename T, bool kRecord>
__global__ __launch_bounds__(4 * C) void kda_state_kernel(StateArgs a) {
    typedef Frag<T> F;
    typedef typename F::Vec V;
    typedef typename Acc4<T>::Raw R4;
    constexpr int NW = C / 16;
    constexpr int NSL = DV / DVS, NTL = DVS / 16;
    constexpr int NKG = DK / F::KG, NCG = C / F::KG;
    constexpr int STOT = (DK / 16) * NTL;  // 16x16 state tiles of the slice
    static_assert(STOT % NW == 0, "state tiles must split evenly over the waves");
    constexpr int SPW = STOT / NW;                       // state tiles per wave
    constexpr int TPB = SPW < NTL ? SPW : NTL;           // tiles per row block
    constexpr int NSB = SPW / TPB;                       // row blocks per wave
    constexpr bool kPrefetch = sizeof(T) == 2;

    __shared__ __align__(16) T St[DVS * DK];  // S^T, fragment order [DVS][DK]
    __shared__ __align__(16) T Ut[DVS * C];   // U^T, fragment order [DVS][C]

    const int H = a.H;
    // Workgroups are dispatched round-robin over the 8 XCDs. When the number
    // of (sequence, head) pairs is a multiple of 8, the NSL slices of one pair
    // get block ids 8 apart, i.e. the same XCD, so the pair's shared operands
    // (W, QO, Aqk, KtT) are fetched into one L2 once and read there NSL times.
    int sl, sh;
    if (NSL > 1 && a.xcd_group) {
        const int xcd = blockIdx.x & 7, idx = blockIdx.x >> 3;
        sl = idx % NSL;
        sh = (idx / NSL) * 8 + xcd;
    } else {
        sl = blockIdx.x % NSL;
        sh = blockIdx.x / NSL;
    }
    const int h = sh % H, s = sh / H;
    const int w = threadIdx.x >> 6, l = threadIdx.x & 63;
    const int col0 = sl * DVS;

    // state tile u of this wave: rows 16*sb(u) .., columns 16*nt(u) .. of the slice
    auto tile_sb = [&](int sbi, int u) { return (w * SPW + sbi * TPB + u) / NTL; };
    auto tile_nt = [&](int sbi, int u) { return (w * SPW + sbi * TPB + u) % NTL; };

    f32x4 accS[NSB][TPB];
    {
        const float *h0 = a.h0 ? a.h0 + ((size_t)s * H + h) * DK * DV : nullptr;
#pragma unroll
        for (int sbi = 0; sbi < NSB; ++sbi)
#pragma unroll
            for (int u = 0; u < TPB; ++u)
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int r = 16 * tile_sb(sbi, u) + acc_row(i);
                    const int c = col0 + 16 * tile_nt(sbi, u) + acc_col();
                    accS[sbi][u][i] = h0 ? h0[r * DV + c] : 0.f;
                }
    }
    auto write_state_t = [&]() {
#pragma unroll
        for (int sbi = 0; sbi < NSB; ++sbi)
#pragma unroll
            for (int u = 0; u < TPB; ++u)
                frag_store4<T>(St, 16 * tile_nt(sbi, u) + acc_col(), 16 * tile_sb(sbi, u) + acc_row(0),
                               accS[sbi][u], DVS);
    };
    write_state_t();
    __syncthreads();

    int tb, te;
    a.map.seq_range(s, tb, te);
    const int c_begin = a.map.chunks_before(s);
    const int n_c = (te - tb + C - 1) / C;
    T *o = static_cast<T *>(a.o);
    const int kgq = (16 * w + 15) / F::KG;  // last Aqk group this wave needs

    struct Ops {
        V wf[NKG], qf[NKG], af[NCG], kf[NSB][NCG];
        R4 ut[NTL];
        f32x4 eg[NSB];
    };
    // Every load is unconditional (Aqk groups past the diagonal are stored as
    // zeros) so that the number of memory operations in flight is the same on
    // every path and the compiler can wait for exactly the group it needs.
    auto load_ops = [&](int ci, Ops &op) {
        const size_t jh = (size_t)(c_begin + ci) * H + h;
        const T *W = static_cast<const T *>(a.buf.W) + jh * C * DK;
        const T *QO = static_cast<const T *>(a.buf.QO) + jh * C * DK;
        const T *Aqk = static_cast<const T *>(a.buf.Aqk) + jh * C * C;
        const T *KtT = static_cast<const T *>(a.buf.KtT) + jh * DK * C;
        const T *Ug = static_cast<const T *>(a.buf.U) + jh * C * DV;
        const float *eg = a.buf.eg + jh * DK;
#pragma unroll
        for (int kg = 0; kg < NKG; ++kg) {
            op.wf[kg] = frag_load<T>(W, kg, w, C);
            op.qf[kg] = frag_load<T>(QO, kg, w, C);
        }
#pragma unroll
        for (int kg = 0; kg < NCG; ++kg) op.af[kg] = frag_load<T>(Aqk, kg, w, C);
#pragma unroll
        for (int sbi = 0; sbi < NSB; ++sbi) {
            const int sb = tile_sb(sbi, 0);
#pragma unroll
            for (int kg = 0; kg < NCG; ++kg) op.kf[sbi][kg] = frag_load<T>(KtT, kg, sb, DK);
            op.eg[sbi] = *reinterpret_cast<const f32x4 *>(eg + 16 * sb + 4 * (l >> 4));
        }
#pragma unroll
        for (int nt = 0; nt < NTL; ++nt)
            op.ut[nt] = *reinterpret_cast<const R4 *>(Ug + acc_tile_off(w, (col0 >> 4) + nt, DV));
    };

    // A fragment-ordered [DVS][K] slice in LDS (rows = this workgroup's value columns) to
    // rows col0 .. of the [DV][K] matrix of chunk ci in global memory: whole groups of 64
    // lanes x 16 bytes (EPL values of T).
    auto copy_slice = [&](const T *src, void *dst_base, int K, int ci) {
        static_assert(F::EPL * sizeof(T) == 16, "one 16-byte share per lane");
        const size_t jh = (size_t)(c_begin + ci) * H + h;
        T *dst = static_cast<T *>(dst_base) + jh * DV * K;
        const int ngroups = (K / F::KG) * (DVS / 16);
        for (int gi = w; gi < ngroups; gi += NW) {
            const int kg = gi / (DVS / 16), rb = gi % (DVS / 16);
            *reinterpret_cast<uint4 *>(dst + (((size_t)kg * (DV / 16) + (col0 >> 4) + rb) * 64 + l) * F::EPL) =
                *reinterpret_cast<const uint4 *>(src + ((size_t)gi * 64 + l) * F::EPL);
        }
    };

    // One chunk: U = U~ - W S, O = QO S + Aqk U, S <- exp(gamma) S + KtT U.
    auto chunk_step = [&](int ci, const Ops &op) {
        const int t0 = tb + ci * C;
        const int L = min(C, te - t0);
        if constexpr (kRecord) copy_slice(St, a.st_out, DK, ci);  // S^T entering the chunk
        f32x4 accU[NTL], accO[NTL];
#pragma unroll
        for (int nt = 0; nt < NTL; ++nt) {
            accU[nt] = accO[nt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int kg = 0; kg < NKG; ++kg) {
                const V sf = frag_load<T>(St, kg, nt, DVS);
                accU[nt] = F::mma(accU[nt], op.wf[kg], sf);
                accO[nt] = F::mma(accO[nt], op.qf[kg], sf);
            }
#pragma unroll
            for (int i = 0; i < 4; ++i) accU[nt][i] = Acc4<T>::get(op.ut[nt], i) - accU[nt][i];
            frag_store4<T>(Ut, 16 * nt + acc_col(), 16 * w + acc_row(0), accU[nt], DVS);
        }
        __syncthreads();  // U^T complete; every wave is done reading S^T
        if constexpr (kRecord) copy_slice(Ut, a.ut_out, C, ci);

        // O += Aqk U (zero above the diagonal; the groups past it are skipped)
#pragma unroll
        for (int nt = 0; nt < NTL; ++nt) {
            if constexpr (kRecord) break;
#pragma unroll
            for (int kg = 0; kg < NCG; ++kg)
                if (kg <= kgq) accO[nt] = F::mma(accO[nt], op.af[kg], frag_load<T>(Ut, kg, nt, DVS));
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                // rows past the end of the sequence go to a discard slot, not through a branch
                const int r = 16 * w + acc_row(i);
                T *dst = r < L ? o + ((size_t)(t0 + r) * H + h) * DV + col0 + 16 * nt + acc_col()
                               : static_cast<T *>(a.discard) + (threadIdx.x & 63);
                *dst = from_f32<T>(accO[nt][i]);
            }
        }

        // S <- exp(gamma) S + KtT U
#pragma unroll
        for (int sbi = 0; sbi < NSB; ++sbi)
#pragma unroll
            for (int u = 0; u < TPB; ++u) {
                accS[sbi][u] *= op.eg[sbi];
                const int nt = tile_nt(sbi, u);
#pragma unroll
                for (int kg = 0; kg < NCG; ++kg)
                    accS[sbi][u] = F::mma(accS[sbi][u], op.kf[sbi][kg], frag_load<T>(Ut, kg, nt, DVS));
            }
        write_state_t();
        __syncthreads();  // S^T ready for the next chunk; U^T free again
    };

    if constexpr (kPrefetch) {
        // Two operand sets used in turn: while one chunk computes, the next
        // chunk's operands are in flight (the last chunk re-fetches itself).
        Ops A, B;
        if (n_c > 0) load_ops(0, A);
        for (int ci = 0; ci < n_c; ci += 2) {
            load_ops(min(ci + 1, n_c - 1), B);
            chunk_step(ci, A);
            if (ci + 1 >= n_c) break;
            load_ops(min(ci + 2, n_c - 1), A);
            chunk_step(ci + 1, B);
        }
    } else {
        Ops A;
        for (int ci = 0; ci < n_c; ++ci) {
            load_ops(ci, A);
            chunk_step(ci, A);
        }
    }

    if (a.hT) {
        float *hT = a.hT + ((size_t)s * H + h) * DK * DV;
#pragma unroll
        for (int sbi = 0; sbi < NSB; ++sbi)
#pragma unroll
            for (int u = 0; u < TPB; ++u)
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int r = 16 * tile_sb(sbi, u) + acc_row(i);
                    const int c = col0 + 16 * tile_nt(sbi, u) + acc_col();
                    hT[r * DV + c] = accS[sbi][u][i];
                }
    }
}

template <int C, int DK, int DV, int DVS, typename T>
hipError_t launch_state_t(const StateArgs &a, int n_seqs, hipStream_t stream) {
    auto kern = kda_state_kernel<C, DK, DV, DVS, T, false>;
    if (a.st_out) {  // recording instance: built for the backward pass's shape only
        if constexpr (C == 64 && DK == 128 && DV == 128 && sizeof(T) == 2)
            kern = kda_state_kernel<C, DK, DV, DVS, T, true>;
        else
            return hipErrorInvalidValue;
    }
    hipLaunchKernelGGL(kern, dim3(n_seqs * a.H * (DV / DVS)), dim3(4 * C), 0, stream, a);
    return hipGetLastError();
}

// Slice width: the whole of d_v per workgroup when the (sequence, head) pairs
// alone fill the chip (no operand is then read twice), else 32 columns so that
// short batches still spread over the compute units.
template <int C, int DK, int DV, typename T>
hipError_t launch_state_w(StateArgs a, int n_seqs, hipStream_t stream) {
    const int pairs = n_seqs * a.H;
    a.xcd_group = (pairs % 8) == 0;
    if constexpr (sizeof(T) == 2) {
        // (the backward's recording instance: two slices of 64 columns per pair, which
        // keep two workgroups on each compute unit)
        if (a.st_out) return launch_state_t<C, DK, DV, (DV > 64 ? 64 : DV), T>(a, n_seqs, stream);
        if (pairs >= 256) return launch_state_t<C, DK, DV, DV, T>(a, n_seqs, stream);
    }
    return launch_state_t<C, DK, DV, 32, T>(a, n_seqs, stream);
}

template <int C, typename T>
hipError_t dispatch_d(const StateArgs &a, int dk, int dv, int n, hipStream_t st) {
    if (dk == 64 && dv == 64) return launch_state_w<C, 64, 64, T>(a, n, st);
    if (dk == 64 && dv == 128) return launch_state_w<C, 64, 128, T>(a, n, st);
    if (dk == 128 && dv == 64) return launch_state_w<C, 128, 64, T>(a, n, st);
    return launch_state_w<C, 128, 128, T>(a, n, st);
}

}  // namespace

hipError_t launch_state(const StateArgs &a, int C, int dk, int dv, bool bf16, int n_seqs,
                        hipStream_t stream) {
    if (C == 64) return bf16 ? dispatch_d<64, kda::bf16>(a, dk, dv, n_seqs, stream)
                             : dispatch_d<64, float>(a, dk, dv, n_seqs, stream);
    return bf16 ? dispatch_d<128, kda::bf16>(a, dk, dv, n_seqs, stream)
                : dispatch_d<128, float>(a, dk, dv, n_seqs, stream);
}

}  // namespace kda
