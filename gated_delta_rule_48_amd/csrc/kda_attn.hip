// kda_attn.hip -- softmax attention for one new token per sequence over a KV
// cache: the full-attention decode step that the KDA decode step is weighed
// against.
//
// The operation is the essay "22,580: from GPT-2 to Kimi K3" section 2.2's
// causal softmax attention, evaluated for the newest position only against the
// keys and values kept from all positions so far (its section 2.3, the KV
// cache):
//
//   o[b, h] = sum_{t < len_b} w_t v[b, j, t],   w = softmax_t(scale q[b, h] . k[b, j, t]),
//
// with j = h / G: G = H / H_kv consecutive query heads share one cached head
// (G = 1 is plain multi-head attention). The "ten questions" page (Q10) counts
// what such a step costs: every cached key and value is read once, so it is
// bound by HBM at about G flops per byte, against one fixed-size state for KDA.
//
// Design (gfx950): the cache of each (sequence, cached head) is split along time
// over enough workgroups to fill the chip ("flash decoding"). In a workgroup of
// four waves, 8 channels of one cache row sit in each lane, so D / 8 adjacent
// lanes (a DPP row or half row) hold a row and each wave load instruction
// covers 4 (D = 128) or 8 (D = 64) whole, consecutive rows of 256 or 128 bytes.
// Each group of lanes runs the streaming softmax over its own rows (running
// maximum, sum and weighted value sum, in base 2 with log2(e) folded into the
// query); the groups are merged by lane exchanges, the waves through LDS, and
// the splits by a second kernel. The dot products stay on the vector ALUs: at
// G <= 8 there are at most 8 flops per cached byte (bf16), below the point where
// the matrix cores would pay.

#include "kda_attn.hpp"

namespace kda {
namespace {

constexpr float kL2E = 1.4426950408889634f;  // log2(e)

__device__ __forceinline__ float exp2_fast(float x) { return __builtin_amdgcn_exp2f(x); }

template <int CTRL> __device__ __forceinline__ float dpp_mov(float x) {
    return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, x), CTRL, 0xf, 0xf, false));
}

// Sum over the LPT adjacent lanes that hold one cache row, left in every one of
// them: swaps within quads, then between the quads of a half row (half-row
// mirror), then between the halves of a row (row mirror).
template <int LPT> __device__ __forceinline__ float row_sum(float x) {
    x += dpp_mov<0xB1>(x);   // quad_perm [1, 0, 3, 2]
    x += dpp_mov<0x4E>(x);   // quad_perm [2, 3, 0, 1]
    x += dpp_mov<0x141>(x);  // row_half_mirror
    if constexpr (LPT == 16) x += dpp_mov<0x140>(x);  // row_mirror
    return x;
}

// 8 consecutive elements of a row, as fp32
template <typename T> struct Row8;
template <> struct Row8<bf16> {
    bf16x8 v;
    __device__ __forceinline__ void load(const bf16 *p) {
        v = __builtin_nontemporal_load(reinterpret_cast<const bf16x8 *>(p));
    }
    __device__ __forceinline__ float operator[](int e) const { return static_cast<float>(v[e]); }
};
template <> struct Row8<float> {
    f32x4 a, b;
    __device__ __forceinline__ void load(const float *p) {
        a = __builtin_nontemporal_load(reinterpret_cast<const f32x4 *>(p));
        b = __builtin_nontemporal_load(reinterpret_cast<const f32x4 *>(p) + 1);
    }
    __device__ __forceinline__ float operator[](int e) const { return e < 4 ? a[e] : b[e - 4]; }
};

// Streaming softmax state of one group of lanes (or, merged, of a wave or a
// split): m the running maximum of the base-2 scores (-inf before any row),
// l the sum of 2^(s - m), acc the sum of 2^(s - m) v over this lane's channels.
// Merging (m, l, acc) with (mo, lo, acco) rescales both to max(m, mo); the
// reference point is 0 while both are empty, so no -inf - -inf is formed.
__device__ __forceinline__ float ref_of(float m) { return m == -INFINITY ? 0.f : m; }

template <int D, int G, typename T>
__global__ __launch_bounds__(kAttnThreads) void kda_attn_decode_kernel(AttnArgs a) {
    constexpr int LPT = D / 8;               // lanes per cache row
    constexpr int RPW = 64 / LPT;            // rows per wave load instruction
    constexpr int U = kAttnRowsPerLane;      // rows per lane group per iteration
    constexpr int ROWS = 4 * RPW * U;        // rows per workgroup iteration
    static_assert(ROWS == attn_rows_per_iter(D), "iteration size shared with the host");
    __shared__ float red_acc[4][G][D];
    __shared__ float red_ml[4][G][2];

    const int split = blockIdx.x, j = blockIdx.y, b = blockIdx.z;
    const int tid = threadIdx.x, w = tid >> 6, l = tid & 63, lrow = l / LPT, c0 = 8 * (l % LPT);
    const int H = a.H_kv * G;

    int len = a.seq_lens ? a.seq_lens[b] : a.T_max;
    len = min(max(len, 0), a.T_max);
    const int t_begin = split * a.split_len;
    const int t_end = min(t_begin + a.split_len, len);

    // this lane's 8 query channels of each head of the group, times scale log2(e)
    float qs[G][8];
#pragma unroll
    for (int g = 0; g < G; ++g) {
        Row8<T> qr;
        qr.load(static_cast<const T *>(a.q) + ((size_t)b * H + (size_t)j * G + g) * D + c0);
#pragma unroll
        for (int e = 0; e < 8; ++e) qs[g][e] = qr[e] * (a.scale * kL2E);
    }
    float m[G], ls[G], acc[G][8];
#pragma unroll
    for (int g = 0; g < G; ++g) {
        m[g] = -INFINITY;
        ls[g] = 0.f;
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[g][e] = 0.f;
    }

    const size_t head = ((size_t)b * a.H_kv + j) * (size_t)a.T_max * D + c0;
    const T *Kc = static_cast<const T *>(a.k) + head;
    const T *Vc = static_cast<const T *>(a.v) + head;
    for (int t0 = t_begin; t0 < t_end; t0 += ROWS) {
        // rows t0 + (U w + u) RPW + lrow: each wave instruction reads RPW consecutive rows.
        // Rows past the end read the split's last row and are masked below.
        Row8<T> kr[U], vr[U];
        int tt[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            tt[u] = t0 + (U * w + u) * RPW + lrow;
            const unsigned tc = (unsigned)min(tt[u], t_end - 1);
            kr[u].load(Kc + tc * D);
            vr[u].load(Vc + tc * D);
        }
#pragma unroll
        for (int g = 0; g < G; ++g) {
            float sc[U];
#pragma unroll
            for (int u = 0; u < U; ++u) {
                float p = 0.f;
#pragma unroll
                for (int e = 0; e < 8; ++e) p = fmaf(qs[g][e], kr[u][e], p);
                p = row_sum<LPT>(p);
                sc[u] = tt[u] < t_end ? p : -INFINITY;
            }
            float mx = m[g];
#pragma unroll
            for (int u = 0; u < U; ++u) mx = fmaxf(mx, sc[u]);
            const float ref = ref_of(mx);
            const float corr = exp2_fast(m[g] - ref);
            float p[U], psum = 0.f;
#pragma unroll
            for (int u = 0; u < U; ++u) {
                p[u] = exp2_fast(sc[u] - ref);
                psum += p[u];
            }
            m[g] = mx;
            ls[g] = fmaf(ls[g], corr, psum);
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                float x = acc[g][e] * corr;
#pragma unroll
                for (int u = 0; u < U; ++u) x = fmaf(p[u], vr[u][e], x);
                acc[g][e] = x;
            }
        }
    }

    // merge the wave's lane groups (rows of lanes LPT apart)
#pragma unroll
    for (int s = LPT; s < 64; s *= 2) {
#pragma unroll
        for (int g = 0; g < G; ++g) {
            const float mo = __shfl_xor(m[g], s), lo = __shfl_xor(ls[g], s);
            const float mx = fmaxf(m[g], mo), ref = ref_of(mx);
            const float f = exp2_fast(m[g] - ref), fo = exp2_fast(mo - ref);
            ls[g] = ls[g] * f + lo * fo;
#pragma unroll
            for (int e = 0; e < 8; ++e) acc[g][e] = acc[g][e] * f + __shfl_xor(acc[g][e], s) * fo;
            m[g] = mx;
        }
    }
    if (l < LPT) {
#pragma unroll
        for (int g = 0; g < G; ++g) {
#pragma unroll
            for (int e = 0; e < 8; ++e) red_acc[w][g][c0 + e] = acc[g][e];
            if (l == 0) {
                red_ml[w][g][0] = m[g];
                red_ml[w][g][1] = ls[g];
            }
        }
    }
    __syncthreads();

    // merge the four waves: one (head, channel) per thread
    for (int idx = tid; idx < G * D; idx += kAttnThreads) {
        const int g = idx / D, c = idx % D;
        float mx = -INFINITY;
#pragma unroll
        for (int v = 0; v < 4; ++v) mx = fmaxf(mx, red_ml[v][g][0]);
        const float ref = ref_of(mx);
        float lsum = 0.f, val = 0.f;
#pragma unroll
        for (int v = 0; v < 4; ++v) {
            const float f = exp2_fast(red_ml[v][g][0] - ref);
            lsum = fmaf(red_ml[v][g][1], f, lsum);
            val = fmaf(red_acc[v][g][c], f, val);
        }
        const size_t bh = (size_t)b * H + (size_t)j * G + g;
        if (a.n_splits == 1) {  // the whole cache: normalise (an empty one gives 0)
            static_cast<T *>(a.o)[bh * D + c] = from_f32<T>(lsum > 0.f ? val / lsum : 0.f);
        } else {
            const size_t ps = bh * a.n_splits + split;
            a.part_acc[ps * D + c] = val;
            if (c == 0) {
                a.part_ml[2 * ps] = mx;
                a.part_ml[2 * ps + 1] = lsum;
            }
        }
    }
}

// o[b, h] from the splits' (m, l, acc). A workgroup takes kAttnCombineChannels
// channels of one (sequence, query head): its threads first form the common
// maximum and each split's weight 2^(m_s - max) (one split per thread in turn,
// the weights kept in LDS), then sum the weighted partial vectors, every channel
// over P interleaved groups of splits, merged through LDS. The loads of a
// thread's splits are independent, so they overlap.
template <int D, typename T>
__global__ __launch_bounds__(kAttnThreads) void kda_attn_combine_kernel(AttnArgs a) {
    constexpr int CB = kAttnCombineChannels;
    constexpr int P = kAttnThreads / CB;
    __shared__ float wgt[kAttnMaxSplits];
    __shared__ float red[2][kAttnThreads / 64];
    __shared__ float part[P][CB];
    const int h = blockIdx.x, b = blockIdx.y, tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
    const int n = a.n_splits;
    const size_t bh = (size_t)b * a.H_kv * a.G + h;
    const float *ml = a.part_ml + bh * n * 2;

    float mx = -INFINITY;
    for (int s = tid; s < n; s += kAttnThreads) mx = fmaxf(mx, ml[2 * s]);
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) mx = fmaxf(mx, __shfl_xor(mx, o));
    if (lane == 0) red[0][wv] = mx;
    __syncthreads();
    mx = fmaxf(fmaxf(red[0][0], red[0][1]), fmaxf(red[0][2], red[0][3]));
    const float ref = ref_of(mx);
    float lsum = 0.f;
    for (int s = tid; s < n; s += kAttnThreads) {
        const float f = exp2_fast(ml[2 * s] - ref);
        wgt[s] = f;
        lsum = fmaf(ml[2 * s + 1], f, lsum);
    }
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) lsum += __shfl_xor(lsum, o);
    if (lane == 0) red[1][wv] = lsum;
    __syncthreads();  // the weights and the partial sums are complete
    lsum = (red[1][0] + red[1][1]) + (red[1][2] + red[1][3]);

    const int c = blockIdx.z * CB + tid % CB, pg = tid / CB;
    const float *pa = a.part_acc + bh * n * D + c;
    float val = 0.f;
#pragma unroll 4
    for (int s = pg; s < n; s += P) val = fmaf(pa[(size_t)s * D], wgt[s], val);
    part[pg][tid % CB] = val;
    __syncthreads();
    if (tid < CB) {
        float v = 0.f;
#pragma unroll
        for (int p = 0; p < P; ++p) v += part[p][tid];
        static_cast<T *>(a.o)[bh * D + blockIdx.z * CB + tid] = from_f32<T>(lsum > 0.f ? v / lsum : 0.f);
    }
}

template <int D, int G, typename T>
hipError_t launch_attn_t(const AttnArgs &a, int B, hipStream_t stream) {
    hipLaunchKernelGGL((kda_attn_decode_kernel<D, G, T>), dim3(a.n_splits, a.H_kv, B), dim3(kAttnThreads), 0,
                       stream, a);
    hipError_t err = hipGetLastError();
    if (err != hipSuccess || a.n_splits == 1) return err;
    hipLaunchKernelGGL((kda_attn_combine_kernel<D, T>), dim3(a.H_kv * G, B, D / kAttnCombineChannels),
                       dim3(kAttnThreads), 0, stream, a);
    return hipGetLastError();
}

template <int D, typename T>
hipError_t dispatch_g(const AttnArgs &a, int B, hipStream_t st) {
    if (a.G == 1) return launch_attn_t<D, 1, T>(a, B, st);
    if (a.G == 2) return launch_attn_t<D, 2, T>(a, B, st);
    if (a.G == 4) return launch_attn_t<D, 4, T>(a, B, st);
    return launch_attn_t<D, 8, T>(a, B, st);
}

}  // namespace

hipError_t launch_attn_decode(const AttnArgs &a, int B, int D, bool is_bf16, hipStream_t stream) {
    if (D == 64) return is_bf16 ? dispatch_g<64, bf16>(a, B, stream) : dispatch_g<64, float>(a, B, stream);
    return is_bf16 ? dispatch_g<128, bf16>(a, B, stream) : dispatch_g<128, float>(a, B, stream);
}

}  // namespace kda
