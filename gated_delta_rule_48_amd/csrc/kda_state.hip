// kda_state.hip -- state propagation and outputs of the chunked KDA forward.
//
// One workgroup (4 waves) per (sequence, head, slice of DVS value columns).
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
// into W, QO, Aqk, KtT and exp(gamma). Only S (rounded to the operand type)
// and U pass through LDS, transposed so that every matrix-core operand is
// contiguous along the contraction.

#include "kda_internal.hpp"

namespace kda {
namespace {

constexpr int kThreads = 256;

template <int C, int DK, int DV, int DVS, typename T>
__global__ __launch_bounds__(kThreads) void kda_state_kernel(StateArgs a) {
    constexpr int NSL = DV / DVS;
    constexpr int RW = C / 4, MB = RW / 16;     // U / O rows per wave
    constexpr int RSW = DK / 4, SB = RSW / 16;  // state rows per wave
    constexpr int NTL = DVS / 16;               // 16-column tiles in the slice
    constexpr int PS = DK + 8;                  // pitch of the S^T copy [DVS][DK]
    constexpr int PU = C + 8;                   // pitch of the U^T copy [DVS][C]
    constexpr int KK = Mma<T>::kK;

    __shared__ __align__(16) T St[DVS * PS];
    __shared__ __align__(16) T Ut[DVS * PU];

    const int H = a.H;
    const int sl = blockIdx.x % NSL;
    const int sh = blockIdx.x / NSL;
    const int h = sh % H, s = sh / H;
    const int w = threadIdx.x >> 6;
    const int col0 = sl * DVS;

    f32x4 accS[SB][NTL];
    const float *h0 = a.h0 ? a.h0 + ((size_t)s * H + h) * DK * DV : nullptr;
#pragma unroll
    for (int sb = 0; sb < SB; ++sb)
#pragma unroll
        for (int nt = 0; nt < NTL; ++nt)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int r = w * RSW + sb * 16 + acc_row(i), c = col0 + nt * 16 + acc_col();
                accS[sb][nt][i] = h0 ? h0[r * DV + c] : 0.f;
            }

    auto write_state_t = [&]() {
#pragma unroll
        for (int sb = 0; sb < SB; ++sb)
#pragma unroll
            for (int nt = 0; nt < NTL; ++nt)
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int r = w * RSW + sb * 16 + acc_row(i), c = nt * 16 + acc_col();
                    St[c * PS + r] = from_f32<T>(accS[sb][nt][i]);
                }
    };
    write_state_t();
    __syncthreads();

    int tb, te;
    a.map.seq_range(s, tb, te);
    const int c_begin = a.map.chunks_before(s);
    const int n_c = (te - tb + C - 1) / C;
    T *o = static_cast<T *>(a.o);

    for (int ci = 0; ci < n_c; ++ci) {
        const int t0 = tb + ci * C;
        const int L = min(C, te - t0);
        const size_t jh = (size_t)(c_begin + ci) * H + h;
        const T *W = static_cast<const T *>(a.buf.W) + jh * C * DK;
        const T *QO = static_cast<const T *>(a.buf.QO) + jh * C * DK;
        const T *KtT = static_cast<const T *>(a.buf.KtT) + jh * DK * C;
        const T *Aqk = static_cast<const T *>(a.buf.Aqk) + jh * C * C;
        const T *Ug = static_cast<const T *>(a.buf.U) + jh * C * DV + col0;
        const float *eg = a.buf.eg + jh * DK;

        // U = U~ - W S and the entering-state part of O
        f32x4 accU[MB][NTL], accO[MB][NTL];
#pragma unroll
        for (int mb = 0; mb < MB; ++mb) {
            const int r0 = w * RW + mb * 16;
#pragma unroll
            for (int nt = 0; nt < NTL; ++nt) {
                const f32x4 z = {0.f, 0.f, 0.f, 0.f};
                accU[mb][nt] = mma_nt<T>(z, W + r0 * DK, DK, St + nt * 16 * PS, PS, 0, DK);
                accO[mb][nt] = mma_nt<T>(z, QO + r0 * DK, DK, St + nt * 16 * PS, PS, 0, DK);
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int r = r0 + acc_row(i), c = nt * 16 + acc_col();
                    const float u = to_f32(Ug[r * DV + c]) - accU[mb][nt][i];
                    accU[mb][nt][i] = u;
                    Ut[c * PU + r] = from_f32<T>(u);
                }
            }
        }
        __syncthreads();  // U^T complete; every wave is done reading S^T

        // O += Aqk U (Aqk is zero above the diagonal; stop at the diagonal tile)
#pragma unroll
        for (int mb = 0; mb < MB; ++mb) {
            const int r0 = w * RW + mb * 16;
            const int kmax = min(C, (r0 + 16 + KK - 1) / KK * KK);
#pragma unroll
            for (int nt = 0; nt < NTL; ++nt) {
                accO[mb][nt] = mma_nt<T>(accO[mb][nt], Aqk + r0 * C, C, Ut + nt * 16 * PU, PU, 0, kmax);
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int r = r0 + acc_row(i), c = col0 + nt * 16 + acc_col();
                    if (r < L) o[((size_t)(t0 + r) * H + h) * DV + c] = from_f32<T>(accO[mb][nt][i]);
                }
            }
        }

        // S <- exp(gamma) S + KtT U
#pragma unroll
        for (int sb = 0; sb < SB; ++sb) {
            const int r0 = w * RSW + sb * 16;
#pragma unroll
            for (int nt = 0; nt < NTL; ++nt) {
#pragma unroll
                for (int i = 0; i < 4; ++i) accS[sb][nt][i] *= eg[r0 + acc_row(i)];
                accS[sb][nt] = mma_nt<T>(accS[sb][nt], KtT + r0 * C, C, Ut + nt * 16 * PU, PU, 0, C);
            }
        }
        write_state_t();
        __syncthreads();  // S^T ready for the next chunk; U^T free again
    }

    if (a.hT) {
        float *hT = a.hT + ((size_t)s * H + h) * DK * DV;
#pragma unroll
        for (int sb = 0; sb < SB; ++sb)
#pragma unroll
            for (int nt = 0; nt < NTL; ++nt)
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int r = w * RSW + sb * 16 + acc_row(i), c = col0 + nt * 16 + acc_col();
                    hT[r * DV + c] = accS[sb][nt][i];
                }
    }
}

template <int C, int DK, int DV, typename T>
hipError_t launch_state_t(const StateArgs &a, int n_seqs, hipStream_t stream) {
    constexpr int DVS = 32;
    auto kern = kda_state_kernel<C, DK, DV, DVS, T>;
    hipLaunchKernelGGL(kern, dim3(n_seqs * a.H * (DV / DVS)), dim3(kThreads), 0, stream, a);
    return hipGetLastError();
}

template <int C, typename T>
hipError_t dispatch_d(const StateArgs &a, int dk, int dv, int n, hipStream_t st) {
    if (dk == 64 && dv == 64) return launch_state_t<C, 64, 64, T>(a, n, st);
    if (dk == 64 && dv == 128) return launch_state_t<C, 64, 128, T>(a, n, st);
    if (dk == 128 && dv == 64) return launch_state_t<C, 128, 64, T>(a, n, st);
    return launch_state_t<C, 128, 128, T>(a, n, st);
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
