// kda_bwd_tok.hip -- the backward pass token by token, for the (sequence, head) pairs in
// which some chunk's summed log-decay on a key channel falls below -kStrongDecay.
//
// The chunked backward passes factor the decay inside a chunk around the chunk's midpoint;
// those factors leave the fp32 range once a chunk's summed log_alpha on some channel falls
// below about -170. For the pairs holding such a chunk this pass recomputes every
// gradient from the token recurrence itself: the update formula of "Kimi K3 KDA math for
// beginners: ten questions" (jokeuncle.github.io), in the step order of the bra-ket
// derivation page (mynewscn.com, opening equations: the decay first, then the delta
// correction of the decayed state, the readout after the write). Every decay enters as
// alpha = exp(log_alpha) <= 1, so nothing can overflow, and decays that underflow are the
// negligible values they stand for.
//
// Per token t, with S~ = Diag(alpha_t) S_{t-1}, u = v_t - S~^T k_t, S_t = S~ + beta_t k_t u^T
// and o_t = S_t^T (scale q_t), reverse mode gives, for dS = dL/dS_t (the gradient arriving
// from the later tokens and from hT) and do = dL/do_t:
//     dS'  = dS + scale q do^T,      dq = scale S_t do
//     du   = beta dS'^T k,           dv = du,         dbeta = k^T dS' u
//     dk   = beta dS' u - S~ du,     dS~ = dS' - k du^T
//     dlog_alpha = rowsum(S~ (.) dS~),  dL/dS_{t-1} = Diag(alpha) dS~
// The states S_{t-1} are recomputed forward from checkpoints: the state entering every
// 64-token block (stored by a first pass over the sequence), the state entering every
// 4-token group of the block being reversed (from the block's), and inside a group from
// the group's, kept in registers.
//
// Work split: one workgroup of four waves per pair, a fixed number of workgroups (the
// workspace holds one set of checkpoints per workgroup) each taking the pairs i, i + grid,
// ... Thread (bi, bj) = (t / 16, t % 16) holds rows RB bi .. RB bi + RB - 1 and columns
// CB bj .. CB bj + CB - 1 of every d_k x d_v matrix (RB = d_k / 16, CB = d_v / 16): sums
// along a row meet within the 16 lanes of a DPP row, sums down a column across lanes and
// waves through LDS. Every sum is taken in a fixed order.
#include "kda_bwd.hpp"

namespace kda {
namespace {

constexpr int kTokThreads = 256;
constexpr int kTokBlock = 64;  // tokens between stored checkpoints
constexpr int kTokGroup = 4;   // tokens between the checkpoints of the block being reversed

template <int CTRL> __device__ __forceinline__ float dppf(float x) {
    return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, x), CTRL, 0xf, 0xf, false));
}

// The sum over the 16 lanes of this lane's DPP row, in every lane of the row (pairs, then
// quads, then halves: every lane adds the same two partial sums).
__device__ __forceinline__ float row16_allsum(float x) {
    x += dppf<0xB1>(x);   // quad_perm [1, 0, 3, 2]
    x += dppf<0x4E>(x);   // quad_perm [2, 3, 0, 1]
    x += dppf<0x141>(x);  // row_half_mirror
    x += dppf<0x140>(x);  // row_mirror
    return x;
}

template <typename T, int DK, int DV>
struct TokPass {
    static constexpr int RB = DK / 16, CB = DV / 16;
    static constexpr int RED = 32 * CB;  // one wave's column partials (two matrices)

    const TokArgs &a;
    float *stg_k, *stg_q, *stg_a, *stg_v, *stg_do, *stg_b, *red;
    int tid, w, l, bi, bj, r0, c0, h;
    int rbuf = 0;  // the reduction buffer of the next column sum

    // Column sums over all d_k rows of per-thread partials (NV values per thread: this
    // thread's CB columns of one or two matrices): in-wave across the four row groups, then
    // across the waves in LDS. Every thread receives the sums. One barrier; the two buffers
    // alternate, so a buffer is written again only after every thread has passed the next
    // barrier, that is, after every thread has read it.
    template <int NV> __device__ __forceinline__ void col_allsum(float (&p)[NV]) {
        static_assert(16 * NV <= RED, "reduction buffer");
#pragma unroll
        for (int c = 0; c < NV; ++c) {
            p[c] += __shfl_xor(p[c], 16);
            p[c] += __shfl_xor(p[c], 32);
        }
        float *rb = red + rbuf * 4 * RED;
        rbuf ^= 1;
        if (l < 16) {
#pragma unroll
            for (int c = 0; c < NV; ++c) rb[w * RED + NV * bj + c] = p[c];
        }
        __syncthreads();
#pragma unroll
        for (int c = 0; c < NV; ++c)
            p[c] = (rb[NV * bj + c] + rb[RED + NV * bj + c]) + (rb[2 * RED + NV * bj + c] + rb[3 * RED + NV * bj + c]);
    }

    // One 4-token group's inputs (this thread's elements, as loaded): requested by fetch()
    // one group ahead and stored, converted, into the staging slots by put() when the group
    // is reached, so that the loads overlap the work in between.
    static constexpr int NEK = (kTokGroup * DK + kTokThreads - 1) / kTokThreads;
    static constexpr int NEV = (kTokGroup * DV + kTokThreads - 1) / kTokThreads;
    struct Fetch {
        T k[NEK], q[NEK], v[NEV], d[NEV];
        float la[NEK], b;
    };
    // Tokens [row0, row0 + n) of the pair (packed row indices): k, log_alpha, v, beta, and with
    // with_q also q and dout.
    __device__ __forceinline__ void fetch(Fetch &f, int row0, int n, bool with_q) {
        const int H = a.H;
#pragma unroll
        for (int e = 0; e < NEK; ++e) {
            const int idx = tid + kTokThreads * e;
            if (idx < n * DK) {
                const size_t g = ((size_t)(row0 + idx / DK) * H + h) * DK + idx % DK;
                f.k[e] = static_cast<const T *>(a.k)[g];
                f.la[e] = a.log_alpha[g];
                if (with_q) f.q[e] = static_cast<const T *>(a.q)[g];
            }
        }
#pragma unroll
        for (int e = 0; e < NEV; ++e) {
            const int idx = tid + kTokThreads * e;
            if (idx < n * DV) {
                const size_t g = ((size_t)(row0 + idx / DV) * H + h) * DV + idx % DV;
                f.v[e] = static_cast<const T *>(a.v)[g];
                if (with_q) f.d[e] = static_cast<const T *>(a.dout)[g];
            }
        }
        if (tid < n) f.b = a.beta[(size_t)(row0 + tid) * H + h];
    }
    // The fetched group into the staging slots: k, alpha = exp(log_alpha), v, beta (and q,
    // dout), fp32, slot i at offset i * d.
    __device__ __forceinline__ void put(const Fetch &f, int n, bool with_q) {
#pragma unroll
        for (int e = 0; e < NEK; ++e) {
            const int idx = tid + kTokThreads * e;
            if (idx < n * DK) {
                stg_k[idx] = to_f32(f.k[e]);
                stg_a[idx] = expf(f.la[e]);
                if (with_q) stg_q[idx] = to_f32(f.q[e]);
            }
        }
#pragma unroll
        for (int e = 0; e < NEV; ++e) {
            const int idx = tid + kTokThreads * e;
            if (idx < n * DV) {
                stg_v[idx] = to_f32(f.v[e]);
                if (with_q) stg_do[idx] = to_f32(f.d[e]);
            }
        }
        if (tid < n) stg_b[tid] = f.b;
    }

    __device__ __forceinline__ void load_state(const float *src, float (&S)[RB][CB]) {
#pragma unroll
        for (int r = 0; r < RB; ++r)
#pragma unroll
            for (int c4 = 0; c4 < CB / 4; ++c4) {
                const f32x4 x = *reinterpret_cast<const f32x4 *>(src + (size_t)(r0 + r) * DV + c0 + 4 * c4);
#pragma unroll
                for (int i = 0; i < 4; ++i) S[r][4 * c4 + i] = x[i];
            }
    }
    __device__ __forceinline__ void store_state(float *dst, const float (&S)[RB][CB]) {
#pragma unroll
        for (int r = 0; r < RB; ++r)
#pragma unroll
            for (int c4 = 0; c4 < CB / 4; ++c4)
                *reinterpret_cast<f32x4 *>(dst + (size_t)(r0 + r) * DV + c0 + 4 * c4) =
                    f32x4{S[r][4 * c4], S[r][4 * c4 + 1], S[r][4 * c4 + 2], S[r][4 * c4 + 3]};
    }

    // S <- S_i from S_{i-1} = S, the token in staging slot i.
    __device__ __forceinline__ void forward_step(float (&S)[RB][CB], int i) {
        float kr[RB], ar[RB], p[CB];
#pragma unroll
        for (int r = 0; r < RB; ++r) {
            kr[r] = stg_k[i * DK + r0 + r];
            ar[r] = stg_a[i * DK + r0 + r];
        }
        const float b = stg_b[i];
#pragma unroll
        for (int c = 0; c < CB; ++c) p[c] = 0.f;
#pragma unroll
        for (int r = 0; r < RB; ++r)
#pragma unroll
            for (int c = 0; c < CB; ++c) {
                S[r][c] *= ar[r];
                p[c] = fmaf(S[r][c], kr[r], p[c]);
            }
        col_allsum(p);  // p = S~^T k
#pragma unroll
        for (int c = 0; c < CB; ++c) p[c] = stg_v[i * DV + c0 + c] - p[c];  // u
#pragma unroll
        for (int r = 0; r < RB; ++r)
#pragma unroll
            for (int c = 0; c < CB; ++c) S[r][c] = fmaf(b * kr[r], p[c], S[r][c]);
    }

    // The gradients of the token in staging slot i (packed row `row`), from Sp = S_{i-1}
    // (overwritten) and dS = dL/dS_i, which becomes dL/dS_{i-1}.
    __device__ __forceinline__ void reverse_step(float (&Sp)[RB][CB], float (&dS)[RB][CB], int i, int row) {
        const float scale = a.scale;
        float kr[RB], qr[RB], ar[RB], u[CB], dc[CB], p[CB];
#pragma unroll
        for (int r = 0; r < RB; ++r) {
            kr[r] = stg_k[i * DK + r0 + r];
            qr[r] = stg_q[i * DK + r0 + r];
            ar[r] = stg_a[i * DK + r0 + r];
        }
        const float b = stg_b[i];
#pragma unroll
        for (int c = 0; c < CB; ++c) dc[c] = stg_do[i * DV + c0 + c];
        // S~; dS' = dS + scale q do^T; one column sum for u = v - S~^T k and du = beta dS'^T k
        float pp[2 * CB];
#pragma unroll
        for (int c = 0; c < 2 * CB; ++c) pp[c] = 0.f;
#pragma unroll
        for (int r = 0; r < RB; ++r) {
            const float sq = scale * qr[r];
#pragma unroll
            for (int c = 0; c < CB; ++c) {
                Sp[r][c] *= ar[r];
                dS[r][c] = fmaf(sq, dc[c], dS[r][c]);
                pp[c] = fmaf(Sp[r][c], kr[r], pp[c]);
                pp[CB + c] = fmaf(dS[r][c], kr[r], pp[CB + c]);
            }
        }
        col_allsum(pp);
        // dbeta = k^T dS' u = (dS'^T k) . u, summed over this thread's columns, then the row
        float eb = 0.f;
#pragma unroll
        for (int c = 0; c < CB; ++c) {
            u[c] = stg_v[i * DV + c0 + c] - pp[c];
            eb = fmaf(pp[CB + c], u[c], eb);
            p[c] = b * pp[CB + c];  // du
        }
        eb = row16_allsum(eb);
        // x1 = S_t do (S_t = S~ + beta k u^T); x2 = dS' u
        float x1[RB], x2[RB];
#pragma unroll
        for (int r = 0; r < RB; ++r) {
            const float bk = b * kr[r];
            float s1 = 0.f, s2 = 0.f;
#pragma unroll
            for (int c = 0; c < CB; ++c) {
                s1 = fmaf(fmaf(bk, u[c], Sp[r][c]), dc[c], s1);
                s2 = fmaf(dS[r][c], u[c], s2);
            }
            x1[r] = row16_allsum(s1);
            x2[r] = row16_allsum(s2);
        }
        // y1 = S~ du; dS~ = dS' - k du^T; y2 = rowsum(S~ (.) dS~); dS <- Diag(alpha) dS~
        float y1[RB], y2[RB];
#pragma unroll
        for (int r = 0; r < RB; ++r) {
            float s1 = 0.f, s2 = 0.f;
#pragma unroll
            for (int c = 0; c < CB; ++c) {
                s1 = fmaf(Sp[r][c], p[c], s1);
                const float dt = fmaf(-kr[r], p[c], dS[r][c]);
                s2 = fmaf(Sp[r][c], dt, s2);
                dS[r][c] = ar[r] * dt;
            }
            y1[r] = row16_allsum(s1);
            y2[r] = row16_allsum(s2);
        }
        const size_t gk = ((size_t)row * a.H + h) * DK + r0, gv = ((size_t)row * a.H + h) * DV + c0;
        if (bj == 0) {
#pragma unroll
            for (int r = 0; r < RB; ++r) {
                static_cast<T *>(a.dq)[gk + r] = from_f32<T>(scale * x1[r]);
                static_cast<T *>(a.dk)[gk + r] = from_f32<T>(fmaf(b, x2[r], -y1[r]));
                a.dlog_alpha[gk + r] = y2[r];
            }
        }
        if (bi == 0) {
#pragma unroll
            for (int c = 0; c < CB; ++c) static_cast<T *>(a.dv)[gv + c] = from_f32<T>(p[c]);
        }
        if (tid == 0) a.dbeta[(size_t)row * a.H + h] = eb;
    }

    // The whole backward of sequence s, head h, from the checkpoint area ck.
    __device__ void run(int s, float *ck) {
        int tb, te;
        a.map.seq_range(s, tb, te);
        const int T_len = te - tb;
        const int n_blk = (T_len + kTokBlock - 1) / kTokBlock;
        float *grp = ck + (size_t)a.n_blk_max * DK * DV;  // the block's group checkpoints
        const size_t pair = (size_t)s * a.H + h;

        // forward over the sequence: the state entering every block
        float S[RB][CB];
        if (a.h0) {
            load_state(a.h0 + pair * DK * DV, S);
        } else {
#pragma unroll
            for (int r = 0; r < RB; ++r)
#pragma unroll
                for (int c = 0; c < CB; ++c) S[r][c] = 0.f;
        }
        Fetch f;
        const int n_all = (T_len + kTokGroup - 1) / kTokGroup;  // groups (blocks hold whole groups)
        if (n_all > 0) fetch(f, tb, min(kTokGroup, T_len), false);
        for (int gi = 0; gi < n_all; ++gi) {
            const int g0 = tb + gi * kTokGroup, n = min(kTokGroup, te - g0);
            if ((gi * kTokGroup) % kTokBlock == 0) store_state(ck + (size_t)(gi * kTokGroup / kTokBlock) * DK * DV, S);
            __syncthreads();  // the previous group's staging is read
            put(f, n, false);
            if (gi + 1 < n_all) fetch(f, g0 + kTokGroup, min(kTokGroup, te - g0 - kTokGroup), false);
            __syncthreads();
            for (int i = 0; i < n; ++i) forward_step(S, i);
        }

        // reverse, block by block
        float dS[RB][CB];
        if (a.dhT) {
            load_state(a.dhT + pair * DK * DV, dS);
        } else {
#pragma unroll
            for (int r = 0; r < RB; ++r)
#pragma unroll
                for (int c = 0; c < CB; ++c) dS[r][c] = 0.f;
        }
        // the first group of the last block
        if (n_blk > 0) {
            const int b0 = tb + (n_blk - 1) * kTokBlock;
            fetch(f, b0, min(kTokGroup, te - b0), false);
        }
        for (int bk = n_blk - 1; bk >= 0; --bk) {
            const int b0 = tb + bk * kTokBlock, b1 = min(b0 + kTokBlock, te);
            const int n_grp = (b1 - b0 + kTokGroup - 1) / kTokGroup;
            const int g_last = b0 + (n_grp - 1) * kTokGroup;
            // the state entering every group of the block (its first group is in flight)
            load_state(ck + (size_t)bk * DK * DV, S);
            for (int gi = 0; gi < n_grp; ++gi) {
                const int g0 = b0 + gi * kTokGroup, n = min(kTokGroup, b1 - g0);
                store_state(grp + (size_t)gi * DK * DV, S);
                __syncthreads();
                put(f, n, false);
                if (gi + 1 < n_grp)
                    fetch(f, g0 + kTokGroup, min(kTokGroup, b1 - g0 - kTokGroup), false);
                else
                    fetch(f, g_last, b1 - g_last, true);  // the reverse's first group
                __syncthreads();
                for (int i = 0; i < n; ++i) forward_step(S, i);
            }
            // the groups in reverse; inside a group, S_{i-1} from the group's checkpoint
            for (int gi = n_grp - 1; gi >= 0; --gi) {
                const int g0 = b0 + gi * kTokGroup, n = min(kTokGroup, b1 - g0);
                __syncthreads();
                put(f, n, true);
                if (gi > 0)
                    fetch(f, g0 - kTokGroup, kTokGroup, true);
                else if (bk > 0)
                    fetch(f, b0 - kTokBlock, kTokGroup, false);  // the previous block's first group
                __syncthreads();
                float Sg[RB][CB];
                load_state(grp + (size_t)gi * DK * DV, Sg);
                for (int i = n - 1; i >= 0; --i) {
                    float Sp[RB][CB];
#pragma unroll
                    for (int r = 0; r < RB; ++r)
#pragma unroll
                        for (int c = 0; c < CB; ++c) Sp[r][c] = Sg[r][c];
                    for (int j = 0; j < i; ++j) forward_step(Sp, j);
                    reverse_step(Sp, dS, i, g0 + i);
                }
            }
        }
        if (a.dh0) store_state(a.dh0 + pair * DK * DV, dS);
    }
};

template <typename T, int DK, int DV>
__global__ __launch_bounds__(kTokThreads, 1) void kda_bwd_tok_kernel(TokArgs a) {
    constexpr int RED = TokPass<T, DK, DV>::RED;
    __shared__ float stg[kTokGroup * (3 * DK + 2 * DV + 1)];
    __shared__ float red[2 * 4 * RED];
    TokPass<T, DK, DV> p{a};
    p.stg_k = stg;
    p.stg_q = stg + kTokGroup * DK;
    p.stg_a = stg + 2 * kTokGroup * DK;
    p.stg_v = stg + 3 * kTokGroup * DK;
    p.stg_do = stg + 3 * kTokGroup * DK + kTokGroup * DV;
    p.stg_b = stg + 3 * kTokGroup * DK + 2 * kTokGroup * DV;
    p.red = red;
    p.tid = threadIdx.x;
    p.w = threadIdx.x >> 6;
    p.l = threadIdx.x & 63;
    p.bi = 4 * p.w + (p.l >> 4);
    p.bj = p.l & 15;
    p.r0 = p.bi * (DK / 16);
    p.c0 = p.bj * (DV / 16);
    float *ck = a.scratch + (size_t)blockIdx.x * a.slot_floats;
    const int n_pairs = a.map.n_seqs * a.H;
    for (int pi = blockIdx.x; pi < n_pairs; pi += gridDim.x) {
        const int s = pi / a.H, h = pi % a.H;
        // whether a chunk of this pair lies past the chunked passes' range
        const int j0 = a.map.chunks_before(s), j1 = a.map.chunks_before(s + 1);
        int any = 0;
        for (int j = j0 + (int)threadIdx.x; j < j1; j += kTokThreads) any |= a.flags[(size_t)j * a.H + h];
        if (__syncthreads_or(any) == 0) continue;
        p.h = h;
        p.run(s, ck);
    }
}

// flags[j][h] = 1 where chunk j of head h (chunks of kTokBlock rows from each sequence's
// start) sums log_alpha below -kStrongDecay on some key channel, else 0.
template <int DK>
__global__ __launch_bounds__(128) void kda_bwd_tok_detect_kernel(const float *log_alpha, SeqMap map, int H,
                                                                 uint8_t *flags) {
    const int j = blockIdx.x, h = blockIdx.y, c = threadIdx.x;
    int s, t0, len;
    if (!map.locate(j, s, t0, len)) return;
    float sum = 0.f;
    if (c < DK)
        for (int t = 0; t < len; ++t) sum += log_alpha[((size_t)(t0 + t) * H + h) * DK + c];
    const int strong = __syncthreads_or(c < DK && sum < -kStrongDecay);
    if (c == 0) flags[(size_t)j * H + h] = strong ? 1 : 0;
}

template <typename T, int DK, int DV>
hipError_t launch_tok(const TokArgs &a, int n_slots, hipStream_t stream) {
    hipLaunchKernelGGL((kda_bwd_tok_kernel<T, DK, DV>), dim3(n_slots), dim3(kTokThreads), 0, stream, a);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_bwd_tok_detect(const float *log_alpha, const SeqMap &map, int H, int dk, int n_chunks_grid,
                                 uint8_t *flags, hipStream_t stream) {
    if (n_chunks_grid <= 0) return hipSuccess;
    if (dk == 128)
        hipLaunchKernelGGL(kda_bwd_tok_detect_kernel<128>, dim3(n_chunks_grid, H), dim3(128), 0, stream, log_alpha,
                           map, H, flags);
    else
        hipLaunchKernelGGL(kda_bwd_tok_detect_kernel<64>, dim3(n_chunks_grid, H), dim3(128), 0, stream, log_alpha,
                           map, H, flags);
    return hipGetLastError();
}

hipError_t launch_bwd_tok(const TokArgs &a, int dk, int dv, bool io_bf16, int n_slots, hipStream_t stream) {
    if (n_slots <= 0) return hipSuccess;
    if (io_bf16) {
        if (dk == 128 && dv == 128) return launch_tok<bf16, 128, 128>(a, n_slots, stream);
        if (dk == 128 && dv == 64) return launch_tok<bf16, 128, 64>(a, n_slots, stream);
        if (dk == 64 && dv == 128) return launch_tok<bf16, 64, 128>(a, n_slots, stream);
        return launch_tok<bf16, 64, 64>(a, n_slots, stream);
    }
    if (dk == 128 && dv == 128) return launch_tok<float, 128, 128>(a, n_slots, stream);
    if (dk == 128 && dv == 64) return launch_tok<float, 128, 64>(a, n_slots, stream);
    if (dk == 64 && dv == 128) return launch_tok<float, 64, 128>(a, n_slots, stream);
    return launch_tok<float, 64, 64>(a, n_slots, stream);
}

}  // namespace kda
