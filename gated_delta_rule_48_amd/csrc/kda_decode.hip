// kda_decode.hip -- one KDA decode step: a single token for each of N sequences.
//
// The step in the order of the bra-ket derivation page (mynewscn.com, the KDA
// state-update equations at its start), in the d_k x d_v orientation:
//
//   S~ = Diag(alpha) S;  e = beta (v - S~^T k);  S <- S~ + k e^T;
//   o  = scale S^T q = scale (S~^T q + (k . q) e)
//
// The second form of o lets one pass over the state produce both reductions
// (S~^T k and S~^T q) before anything is written, so each state is read once
// and written once. The step is a pure HBM read-modify-write (about one flop
// per byte), so the kernel is built around the memory access: one workgroup of
// 1024 threads per (sequence, head), each thread owning 4 adjacent columns of
// RPT rows (4 at d = 128), 16-byte loads and stores covering whole rows per
// wave instruction, and the column sums reduced across row groups through LDS
// in two levels: the row groups of a wave by lane exchanges, then one thread per
// column (and sum) adds the waves' partials in wave order. (Every thread adding all
// 32 row groups' partials itself read 0.5 to 1 MB of LDS per workgroup between its
// state reads and writes; the two-level sums took the step from 194 to 181 us.)

#include "kda_internal.hpp"

namespace kda {
namespace {

constexpr int kThreads = 1024;

template <int DK, int DV, typename T>
__global__ __launch_bounds__(kThreads) void kda_decode_kernel(DecodeArgs a) {
    constexpr int CG = DV / 4;          // float4 column groups
    constexpr int RG = kThreads / CG;   // row groups
    constexpr int RPT = DK / RG;        // rows per thread
    static_assert(RPT * RG == DK, "rows must split evenly");

    constexpr int NW = kThreads / 64;   // waves
    constexpr int GPW = 64 / CG;        // row groups per wave (lanes l, l + CG, ... share a column group)
    __shared__ float ks[DK], qs[DK], al[DK];
    __shared__ f32x4 red_k[NW][CG], red_q[NW][CG];  // per-wave partial column sums
    __shared__ float col_k[DV], col_q[DV];          // the full column sums
    __shared__ float kq_part[kThreads / 64];
    __shared__ float ss_part[2][kThreads / 64];  // sums of squares of silu(k), silu(q) (qk_norm)

    const int nh = blockIdx.x;
    const int tid = threadIdx.x;
    const int cg = tid % CG, rg = tid / CG;

    // 1. this thread's state rows first: they are the step's traffic, and
    //    nothing below waits for them until the token is staged. Streamed once
    //    per step (the states exceed the last-level cache), hence nontemporal.
    f32x4 *S = reinterpret_cast<f32x4 *>(a.state + (size_t)nh * DK * DV);
    f32x4 sv[RPT];
#pragma unroll
    for (int it = 0; it < RPT; ++it) sv[it] = __builtin_nontemporal_load(&S[(it * RG + rg) * CG + cg]);

    // 2. the token: k, q and alpha per key channel into LDS, k . q by reduction
    const T *q = static_cast<const T *>(a.q) + (size_t)nh * DK;
    const T *k = static_cast<const T *>(a.k) + (size_t)nh * DK;
    const T *v = static_cast<const T *>(a.v) + (size_t)nh * DV;
    float kq = 0.f, ssk = 0.f, ssq = 0.f;
    if (tid < DK) {
        float kv = to_f32(k[tid]), qv = to_f32(q[tid]);
        if (a.pre.qk_norm) {  // silu here; the row norms are applied to the sums below
            kv = silu_f(kv);
            qv = silu_f(qv);
            ssk = kv * kv;
            ssq = qv * qv;
        }
        ks[tid] = kv;
        qs[tid] = qv;
        if (a.gate == kGatePreact) {  // alpha = exp(-exp(A_log) softplus(a + dt_bias))
            const int hh = nh % a.H;
            const float x = to_f32(static_cast<const T *>(a.pre.a)[(size_t)nh * DK + tid]) +
                            a.pre.dt_bias[(size_t)hh * DK + tid];
            al[tid] = expf(-expf(a.pre.A_log[hh]) * softplus_f(x));
        } else {
            al[tid] = a.gate == kGateChannel ? __expf(a.log_alpha[(size_t)nh * DK + tid])
                      : a.gate == kGateHead  ? __expf(a.log_alpha[nh])
                                             : 1.f;
        }
        kq = kv * qv;
    }
    f32x4 vv;
#pragma unroll
    for (int i = 0; i < 4; ++i) vv[i] = to_f32(v[4 * cg + i]);
    const float beta = a.gate == kGatePreact ? sigmoid_f(a.beta[nh]) : a.beta[nh];
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) kq += __shfl_xor(kq, off);
    if ((tid & 63) == 0) kq_part[tid >> 6] = kq;
    if (a.pre.qk_norm) {
#pragma unroll
        for (int off = 32; off > 0; off >>= 1) {
            ssk += __shfl_xor(ssk, off);
            ssq += __shfl_xor(ssq, off);
        }
        if ((tid & 63) == 0) {
            ss_part[0][tid >> 6] = ssk;
            ss_part[1][tid >> 6] = ssq;
        }
    }
    __syncthreads();

    // 3. decay, and the partial column sums of S~^T k and S~^T q over this thread's rows
    f32x4 rk = {0.f, 0.f, 0.f, 0.f}, rq = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int it = 0; it < RPT; ++it) {
        const int row = it * RG + rg;
        sv[it] *= al[row];
        rk += ks[row] * sv[it];
        rq += qs[row] * sv[it];
    }
    // the wave's row groups first (lane exchanges), then its partial to LDS
#pragma unroll
    for (int off = CG; off < 64; off <<= 1) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            rk[i] += __shfl_xor(rk[i], off);
            rq[i] += __shfl_xor(rq[i], off);
        }
    }
    if ((tid & 63) < CG) {
        red_k[tid >> 6][cg] = rk;
        red_q[tid >> 6][cg] = rq;
    }
    __syncthreads();
    // each of the first 2 DV threads adds the waves' partials of one column, in wave order
    if (tid < 2 * DV) {
        const int c = tid % DV;
        const float *red = reinterpret_cast<const float *>(tid < DV ? red_k : red_q);
        float t = 0.f;
#pragma unroll
        for (int w = 0; w < NW; ++w) t += red[w * DV + c];
        (tid < DV ? col_k : col_q)[c] = t;
    }
    __syncthreads();

    // 4. full column sums, the error e = beta (v - S~^T k) and the output
    const f32x4 tk0 = *reinterpret_cast<const f32x4 *>(col_k + 4 * cg);
    const f32x4 tq0 = *reinterpret_cast<const f32x4 *>(col_q + 4 * cg);
    f32x4 tk = tk0, tq = tq0;
    float kqs = 0.f;
#pragma unroll
    for (int i = 0; i < kThreads / 64; ++i) kqs += kq_part[i];
    // with qk_norm, k and q are silu(.) / ||silu(.)||: the sums above were taken with
    // silu(.), and each is linear in k or q
    float rk_inv = 1.f;
    if (a.pre.qk_norm) {
        float sk = 0.f, sq = 0.f;
#pragma unroll
        for (int i = 0; i < kThreads / 64; ++i) {
            sk += ss_part[0][i];
            sq += ss_part[1][i];
        }
        rk_inv = 1.f / fmaxf(sqrtf(sk), kNormEps);
        const float rq_inv = 1.f / fmaxf(sqrtf(sq), kNormEps);
        tk *= rk_inv;
        tq *= rq_inv;
        kqs *= rk_inv * rq_inv;
    }
    const f32x4 e = beta * (vv - tk);
    if (rg == 0) {
        T *o = static_cast<T *>(a.o) + (size_t)nh * DV;
#pragma unroll
        for (int i = 0; i < 4; ++i) o[4 * cg + i] = from_f32<T>(a.scale * (tq[i] + kqs * e[i]));
    }

    // 5. write back S~ + k e^T
#pragma unroll
    for (int it = 0; it < RPT; ++it) {
        const int row = it * RG + rg;
        __builtin_nontemporal_store(sv[it] + (ks[row] * rk_inv) * e, &S[row * CG + cg]);
    }
}

template <int DK, int DV, typename T>
hipError_t launch_decode_t(const DecodeArgs &a, hipStream_t stream) {
    hipLaunchKernelGGL((kda_decode_kernel<DK, DV, T>), dim3(a.NH), dim3(kThreads), 0, stream, a);
    return hipGetLastError();
}

template <typename T>
hipError_t dispatch_d(const DecodeArgs &a, int dk, int dv, hipStream_t st) {
    if (dk == 64 && dv == 64) return launch_decode_t<64, 64, T>(a, st);
    if (dk == 64 && dv == 128) return launch_decode_t<64, 128, T>(a, st);
    if (dk == 128 && dv == 64) return launch_decode_t<128, 64, T>(a, st);
    return launch_decode_t<128, 128, T>(a, st);
}

}  // namespace

hipError_t launch_decode(const DecodeArgs &a, int dk, int dv, bool bf16, hipStream_t stream) {
    return bf16 ? dispatch_d<kda::bf16>(a, dk, dv, stream) : dispatch_d<float>(a, dk, dv, stream);
}

}  // namespace kda
