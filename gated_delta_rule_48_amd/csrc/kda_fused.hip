// kda_fused.hip -- the whole chunked KDA forward pass of one (sequence, head)
// in one workgroup of 8 waves: chunk preparation and state propagation fused,
// the fp32 128 x 128 state resident in matrix-core accumulators for the whole
// sequence. Built for bf16 q/k/v/o, d_k = d_v = 128 and chunks of 64 rows.
//
// Per chunk the workgroup computes the quantities of the split pass (kda_prep.hip
// then kda_state.hip) without writing any of them to memory: decay prefix g and
// gamma, the decayed Gram matrices, T = (I + A)^{-1}, U~ = T (beta v), and the
// state-side products. With m = gamma/2, E = Diag(exp(m)), Kp = k exp(g - m),
// Qp = q exp(g - m) and Km = k exp(m - g) (the midpoint factors of the Gram
// matrices), the chunk identities read
//     W S      = (T Diag(beta) Kp) (E S)              (k exp(g) = Kp E)
//     QO S     = scale Qp (E S)                      (q exp(g) = Qp E)
//     S_next   = E (E S + Km^T U)                    (exp(gamma) = E^2)
// so E scales the state's rows inside the state phase and every per-element
// product is one of Kp, Qp, Km. Between chunks the accumulators hold
// Q = E S + Km^T U (S_next = E Q), and the next chunk's E S is E_next (E Q),
// applied at the start of the next state phase: as one factor E_next E while
// that stays in the normal fp32 range, else one factor after the other (the
// product underflows long before either factor does).
// The only traffic is the inputs q, k, v,
// log_alpha, beta (read once, ahead of use), the outputs o, and h0 / hT.
//
// The method is the chunk algorithm of the essay "22,580: from GPT-2 to Kimi K3"
// (yichencityu.github.io, section 6.3: T by forward substitution, W = T K_beta,
// U = T V_beta, then u = U - w S, o = q S + tril(q k^T) u, S += k^T u) with the
// per-channel cumulative decay of KDA (aidehub.top summary, Gated DeltaNet
// section); kda_prep.hip states the chunk identities.
//
// Work split. Two waves share each SIMD, so one wave's latencies (exp, LDS,
// matrix-core results) overlap the other's work. Wave w = rb + 4 hf:
//   scan, elementwise  chunk rows 16 rb .. 16 rb + 15, key/value channels of
//                      half hf (64 of 128), lane l = r + 16 hi holding row r;
//   Gram               hf = 0: the diagonal block rb of A = beta K+ K-^T, then the
//                      inverse of (I + that block) by forward substitution in
//                      registers (DPP row broadcasts); hf = 1: the off-diagonal
//                      blocks of A's rows rb and Aqk's rows 3 - rb (four tiles);
//   solve              hf = 1, rb < 3: the off-diagonal blocks of column block rb
//                      of T' = T Diag(beta), one small matrix-core chain each;
//   state              state columns 16 w .. 16 w + 15, all 128 rows: U = T' (v -
//                      Kp P) for those columns (so neither W nor U~ is formed for
//                      the whole chunk), then O and the state update.
// Intermediates pass between phases in LDS in the permuted fragment order of
// kda_device.hpp, in which two adjacent accumulator tiles are one operand.

#include "kda_internal.hpp"

namespace kda {
namespace {

typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));

constexpr int kC = 64, kDK = 128, kDV = 128, kNT = 512;
constexpr int kPT = kC + 4;                  // pitch of the fp32 [C][C] matrix A
constexpr float kL2E = 1.4426950408889634f;  // log2(e): exponents are kept in base 2
constexpr float kClamp = 85.f * kL2E;        // |exponent| limit of the midpoint factors (e^85)

// LDS layout (bytes): operands written by the elementwise and Gram phases and read
// by the later phases, in the permuted fragment order.
struct Lds {
    static constexpr int QP = 0;                        // [C][DK]  bf16 fragments: Qp (Gram and state)
    static constexpr int KTT = QP + kC * kDK * 2;       // [DK][C]  bf16 fragments: Km^T
    static constexpr int AQK = KTT + kDK * kC * 2;      // [C][C]   bf16 fragments: masked scale Qp Km^T
    static constexpr int EHALF = AQK + kC * kC * 2;     // [2][DK]  exp(gamma_prev / 2), exp(gamma / 2), in e_slot order
    static constexpr int TOT = EHALF + 2 * kDK * 4;     // [4][DK]  log-decay sum of each row block
    static constexpr int OFFM = TOT + 4 * kDK * 4;      // [4][DK]  (row-block offset - gamma/2) log2(e)
    static constexpr int BET = OFFM + 4 * kDK * 4;      // [C]      beta (0 past the end)
    static constexpr int VT = BET + kC * 4;             // [DV][C]  bf16 fragments: v^T
    static constexpr int AM = VT + kDV * kC * 2;        // [C][PT]  fp32 A (strictly lower)
    static constexpr int TF = AM + kC * kPT * 4;        // [C][C]   bf16 fragments: T Diag(beta)
    static constexpr int DG = TF + kC * kC * 2;         // [4][64]  bf16x4 per lane: diagonal blocks of T
    static constexpr int KM = DG + 4 * 64 * 4 * 2;      // [C][DK]  bf16 fragments: Km (Gram)
    static constexpr int KP = KM + kC * kDK * 2;        // [C][DK]  bf16 fragments: Kp (Gram and state)
    static constexpr int IDN = KP + kC * kDK * 2;       // [2][64]  bf16x8: each lane's identity operands (ident_frag)
    static constexpr int FLG = IDN + 2 * 64 * 16;       // [4]      int: E E_prev leaves the normal fp32 range (0, 1);
                                                        //          some channel decays strongly (2, 3)
    static constexpr int DTB = FLG + 16;                // [DK]     fp32: dt_bias of the head (pre-activation gates)
    static constexpr int QKS = DTB + kDK * 4;           // [2][C][2] fp32: per half, each row's sums of squares of
                                                        //           silu(k) (scan phase), silu(q) (elementwise phase)
    static constexpr int QNR = QKS + 2 * kC * 2 * 4;   // [C] fp32: inverse norms of the rows of silu(q)
    // strong-decay instance only:
    static constexpr int GPRE = QNR + kC * 4;          // [5][DK] fp32: log2 decay before row block 0..3, gamma
    static constexpr int EGAM = GPRE + 5 * kDK * 4;    // [DK] fp32 (e_slot order): exp(gamma)
    static constexpr int SAQ = EGAM + kDK * 4;         // [10][256] fp32: half 1's partial Aqk tiles (rb, tj <= rb)
    static constexpr int SIZE = SAQ + 10 * 256 * 4;
};
static_assert(Lds::SIZE <= 160 * 1024, "fused LDS budget");

template <int I> struct IntTag { static constexpr int value = I; };

__device__ __forceinline__ f32x4 mma16(bf16x4 a, bf16x4 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ float exp2_fast(float x) { return __builtin_amdgcn_exp2f(x); }

// Value of lane I of this lane's 16-lane DPP row.
template <int I> __device__ __forceinline__ float row_bcast(float x) {
    return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, x), 0x150 + I, 0xf, 0xf, true));
}

typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef unsigned u32x2 __attribute__((ext_vector_type(2)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));

// Two floats rounded to bf16 (nearest even) in one 32-bit word.
__device__ __forceinline__ unsigned pack2(float a, float b) {
    return __builtin_bit_cast(unsigned, __builtin_convertvector(f32x2{a, b}, bf16x2));
}

__device__ __forceinline__ bf16x4 to_bf16x4(f32x4 x) {
    return __builtin_bit_cast(bf16x4, u32x2{pack2(x[0], x[1]), pack2(x[2], x[3])});
}

__device__ __forceinline__ bf16x8 pack8(const float *x) {
    return __builtin_bit_cast(bf16x8, u32x4{pack2(x[0], x[1]), pack2(x[2], x[3]), pack2(x[4], x[5]), pack2(x[6], x[7])});
}

// Two accumulator tiles (contraction indices 0..15 and 16..31 of a group) as one operand.
__device__ __forceinline__ bf16x8 tiles_to_frag(f32x4 lo, f32x4 hi) {
    return __builtin_bit_cast(bf16x8, u32x4{pack2(lo[0], lo[1]), pack2(lo[2], lo[3]), pack2(hi[0], hi[1]), pack2(hi[2], hi[3])});
}

// The lane index as a value the compiler cannot hoist: addresses derived from it
// are rebuilt where they are used instead of being kept as loop-carried values.
__device__ __forceinline__ int opaque_lane() {
    int l = threadIdx.x & 63;
    asm volatile("" : "+v"(l));
    return l;
}

// Key and value channels are held in a fixed permuted order: in registers, in LDS
// and in the state, position p = 32 kg + 16 t + 4 hi + i of a channel group (the
// operand slot 4 t + i of lane group hi) holds channel 32 kg + 8 hi + 4 t + i. Each
// lane's eight slots of a group are then eight adjacent channels of the tensor,
// one 16-byte load of a bf16 row. The contractions over channels do not depend on
// their order; only the global loads and stores map positions to channels.
__device__ __forceinline__ int chan_of_pos(int p) {
    return (p & ~31) | (((p >> 2) & 3) << 3) | (((p >> 4) & 1) << 2) | (p & 3);
}

// Slot of key position p = 16 tm + 4 hi + i in the per-channel factor array: lane
// group hi's 32 factors (tm = 0..7, i = 0..3) are contiguous, two per lane of its
// 16-lane row, so that one 8-byte read per lane and row broadcasts give every
// lane all of them.
__device__ __forceinline__ int e_slot(int p) { return ((p >> 2) & 3) * 32 + ((p >> 4) << 2) + (p & 3); }

// Channels 32 kg + 8 hi .. + 7 of a bf16 row: the operand slots of lane group hi
// for channel group kg.
__device__ __forceinline__ bf16x8 load_row8(const bf16 *row, int kg, int hi) {
    return *reinterpret_cast<const bf16x8 *>(row + 32 * kg + 8 * hi);
}

// The 16 x 16 identity as the B operand of mma16: lane (c, hi) has a one (bf16
// 0x3f80) in slot c - 4 hi when that is 0..3.
__device__ __forceinline__ unsigned long long ident4_bits() {
    const int l = opaque_lane();
    const unsigned d = (unsigned)((l & 15) - 4 * (l >> 4));
    return d < 4 ? 0x3f80ull << (16 * d) : 0ull;
}

// Identity operand for transposing with the matrix cores: as B^T of a 16-column
// tile t within a contraction group, lane l (column l%16) has a one in the slot
// whose contraction index is 16 t + l%16 (slots 4 t .. 4 t + 3 hold indices
// 16 t + 4 hi .. 16 t + 4 hi + 3).
__device__ __forceinline__ bf16x8 ident_frag(int t) {
    const unsigned long long b = ident4_bits();
    const unsigned lo = (unsigned)b, hi = (unsigned)(b >> 32);
    return __builtin_bit_cast(bf16x8, t ? u32x4{0u, 0u, lo, hi} : u32x4{lo, hi, 0u, 0u});
}

// The LDS helpers below take the lane index l explicitly (each phase declares it).

// Store accumulator tile `acc` as slots 4 t .. 4 t + 3 of lane l's share of
// group (kg, rb) of a fragment-ordered matrix with R rows.
__device__ __forceinline__ void store_slots(bf16 *base, int kg, int rb, int R, int t, f32x4 acc, int l) {
    *reinterpret_cast<bf16x4 *>(base + ((kg * (R >> 4) + rb) * 64 + l) * 8 + 4 * t) = to_bf16x4(acc);
}

// Lane l's slots 4 t .. 4 t + 3 (one 16 x 16 block's operand) of group (kg, rb).
__device__ __forceinline__ bf16x4 load_slots(const bf16 *base, int kg, int rb, int R, int t, int l) {
    return *reinterpret_cast<const bf16x4 *>(base + ((kg * (R >> 4) + rb) * 64 + l) * 8 + 4 * t);
}

// Lane l's 16-byte share of group (kg, rb) of a fragment-ordered matrix with R rows.
__device__ __forceinline__ bf16x8 fld(const bf16 *base, int kg, int rb, int R, int l) {
    return *reinterpret_cast<const bf16x8 *>(base + ((kg * (R >> 4) + rb) * 64 + l) * 8);
}

// Lane l's element offset in tile (rb, cb) of an accumulator-ordered [R][NC] matrix.
__device__ __forceinline__ int ato(int rb, int cb, int NC, int l) { return ((rb * (NC >> 4) + cb) * 64 + l) * 4; }

// States pass to and from memory through LDS (before the first chunk and after the last,
// when no operand lives there): memory sees whole 16-byte pieces of consecutive rows, while
// each lane's accumulator share (rows 16 tm + 4 hi + i of one column) is scattered in a row-
// major state. Staging buffer: [d_k][kSP] fp32 from the start of LDS.
constexpr int kSP = kDV + 4;
static_assert(kDK * kSP * 4 <= 123 * 1024, "state staging below the identity operands");

// accS <- the [d_k][d_v] fp32 state at src (row = key channel), in the permuted positions of
// the accumulators (tile tm, lane (lr, hi) of wave w: rows 16 tm + 4 hi + i of column 16 w + lr).
__device__ __forceinline__ void load_state(const float *src, f32x4 (&acc)[8], float *stg, int tid, int w, int lr,
                                           int hi) {
#pragma unroll
    for (int k = 0; k < kDK * kDV / 4 / kNT; ++k) {
        const int piece = tid + kNT * k, row = piece / (kDV / 4), c4 = piece % (kDV / 4);
        *reinterpret_cast<f32x4 *>(stg + row * kSP + 4 * c4) =
            *reinterpret_cast<const f32x4 *>(src + (size_t)row * kDV + 4 * c4);
    }
    __syncthreads();
    const int col = chan_of_pos(16 * w + lr);
#pragma unroll
    for (int tm = 0; tm < 8; ++tm)
#pragma unroll
        for (int i = 0; i < 4; ++i) acc[tm][i] = stg[chan_of_pos(16 * tm + 4 * hi + i) * kSP + col];
    __syncthreads();  // the buffer is free again
}

// The [d_k][d_v] fp32 state at dst <- acc (the layout of load_state). The caller has passed a
// barrier after the last read of LDS operands.
__device__ __forceinline__ void store_state(float *dst, const f32x4 (&acc)[8], float *stg, int tid, int w, int lr,
                                            int hi) {
    const int col = chan_of_pos(16 * w + lr);
#pragma unroll
    for (int tm = 0; tm < 8; ++tm)
#pragma unroll
        for (int i = 0; i < 4; ++i) stg[chan_of_pos(16 * tm + 4 * hi + i) * kSP + col] = acc[tm][i];
    __syncthreads();
#pragma unroll
    for (int k = 0; k < kDK * kDV / 4 / kNT; ++k) {
        const int piece = tid + kNT * k, row = piece / (kDV / 4), c4 = piece % (kDV / 4);
        *reinterpret_cast<f32x4 *>(dst + (size_t)row * kDV + 4 * c4) =
            *reinterpret_cast<const f32x4 *>(stg + row * kSP + 4 * c4);
    }
}

// Declares this lane's index l, its row lr and lane group hi, and its chunk row r
// (within the wave's row block rb), for the enclosing phase.
#define KDA_PHASE_LANE                                                         \
    const int l = threadIdx.x & 63, lr = l & 15, hi = l >> 4, r = 16 * rb + lr; \
    (void)lr;                                                                  \
    (void)hi;                                                                  \
    (void)r;

// Bodies (kMode):
//   kUsual  the usual pass over one run of chunks (a whole sequence, or a segment of one).
//           Where a chunk's decay sums below -kStrongDecay on some channel (the midpoint
//           factors would leave the fp32 range), it flags its unit and stops.
//   kStrongPass  runs after it, on the flagged (sequence, head) pairs only, from the start
//           of the sequence, with every exponent <= 0: the state-side factors taken from the
//           chunk's start, the Gram tiles left of the diagonal from the end of their column
//           block, the diagonal tiles pair by pair.
//   kMap    for a middle segment of a long sequence: its map S_out = M S_in + N, with M
//           (d_k x d_k) carried from I and N from zero through the segment's chunks as a
//           second state, no outputs. A chunk of strong decay flags the unit and stops.
// Kernels (the same template argument): kUsual over the (sequence, head) pairs, kStrongPass
// over the pairs, and with segments kPlanA (segment 0 of every sequence with the kUsual body,
// the maps of segments 1 .. P - 2 with the kMap body) and kPlanC (segments 1 .. P - 1 with
// the kUsual body, each from its entering state).
constexpr int kUsual = 0, kStrongPass = 1, kMap = 2, kPlanA = 3, kPlanC = 4;

// One workgroup's run of chunks.
struct Unit {
    int h;
    size_t seq0;          // its first token
    int T_len;            // its tokens
    const float *h0src;   // the state it starts from ([d_k][d_v] fp32), or null (zero)
    float *out_state;     // where the state at its end goes ([d_k][d_v] fp32), or null
    float *map_out;       // kMap: M (bf16 parts) and N (seg_mh_index, seg_n_index)
    uint8_t *redo;        // its flag: 1 if it left its pair to the strong instance, else 0
};

template <int G, int kMode>
__device__ __forceinline__ void fused_body(const FusedArgs &a, const Unit &u) {
    constexpr bool kStrong = kMode == kStrongPass;
    constexpr bool kMapMode = kMode == kMap;
    // G: the kda_gate kinds, kGatePreact, and kGatePreactQK (kGatePreact with q and k
    // normalised here as well)
    constexpr bool kPreact = G == kGatePreact || G == kGatePreactQK;
    constexpr bool kQK = G == kGatePreactQK;
    // a decay per key channel, given or formed from pre-activations
    constexpr bool kPerChannel = G == kGateChannel || kPreact;
    extern __shared__ __align__(16) unsigned char smem[];
    bf16 *Qp = reinterpret_cast<bf16 *>(smem + Lds::QP);
    bf16 *KtT = reinterpret_cast<bf16 *>(smem + Lds::KTT);
    bf16 *Aqk = reinterpret_cast<bf16 *>(smem + Lds::AQK);
    float *tot = reinterpret_cast<float *>(smem + Lds::TOT);
    float *offm = reinterpret_cast<float *>(smem + Lds::OFFM);
    float *ehalf = reinterpret_cast<float *>(smem + Lds::EHALF);
    float *bet = reinterpret_cast<float *>(smem + Lds::BET);
    bf16 *Vt = reinterpret_cast<bf16 *>(smem + Lds::VT);
    float *Am = reinterpret_cast<float *>(smem + Lds::AM);
    bf16 *Tf = reinterpret_cast<bf16 *>(smem + Lds::TF);
    bf16 *Dg = reinterpret_cast<bf16 *>(smem + Lds::DG);
    bf16 *Km = reinterpret_cast<bf16 *>(smem + Lds::KM);
    bf16 *Kp = reinterpret_cast<bf16 *>(smem + Lds::KP);
    bf16 *idn = reinterpret_cast<bf16 *>(smem + Lds::IDN);
    int *flg = reinterpret_cast<int *>(smem + Lds::FLG);
    float *dtb = reinterpret_cast<float *>(smem + Lds::DTB);
    float *qks = reinterpret_cast<float *>(smem + Lds::QKS);
    float *qnr = reinterpret_cast<float *>(smem + Lds::QNR);
    float *gpre = reinterpret_cast<float *>(smem + Lds::GPRE);
    float *egam = reinterpret_cast<float *>(smem + Lds::EGAM);
    float *saq = reinterpret_cast<float *>(smem + Lds::SAQ);

    const int H = a.H;
    const int h = u.h;
    const int tid = threadIdx.x, l = tid & 63, lr = l & 15, hi = l >> 4;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int rb = w & 3, hf = w >> 2;
    const float scale = a.scale;
    const int T_len = u.T_len;
    const size_t seq0 = u.seq0;
    const float *h0src = u.h0src;
    const int n_c = (T_len + kC - 1) / kC;
    const int T_ld = max(T_len, 1);  // the rows the loads may touch (row 0 for an empty sequence)

    // ---- state columns (value positions) 16 w .. 16 w + 15: tile tm holds rows (key
    //      positions) 16 tm + 4 hi + i of column 16 w + lr
    f32x4 accS[8];
    if (h0src) {
        load_state(h0src, accS, reinterpret_cast<float *>(smem), tid, w, lr, hi);
    } else {
#pragma unroll
        for (int tm = 0; tm < 8; ++tm) accS[tm] = f32x4{0.f, 0.f, 0.f, 0.f};
    }
    // map instance: M, from the identity (rows and columns are key positions)
    f32x4 accM[8];
    if constexpr (kMapMode) {
#pragma unroll
        for (int tm = 0; tm < 8; ++tm)
#pragma unroll
            for (int i = 0; i < 4; ++i) accM[tm][i] = (16 * tm + 4 * hi + i == 16 * w + lr) ? 1.f : 0.f;
    }

    // ---- this lane's inputs of one chunk: row r, channel groups 2 hf and 2 hf + 1.
    //      The next chunk's are requested in three parts, each just before a
    //      barrier: decay and beta after the scan, key rows after the elementwise
    //      phase, query and value rows after the off-diagonal blocks of T.
    //      Issuing a load stalls a wave while the CU's address units
    //      are busy; at the end of a phase the waves arrive one or two thousand
    //      cycles apart (the first ones would only wait at the barrier), so few
    //      requests compete, and no phase starts with a burst of them.
    bf16x8 kr[2], qr[2], vr[2];
    float gl[2][8];
    bf16x8 gar[2];  // decay pre-activations (kGatePreact)
    float bta;
    // uniform base of chunk ci's first row (head h) + 32-bit lane offsets
    auto tok0_of = [&](int ci) { return (seq0 + (size_t)ci * kC) * H + h; };
    // Each request derives the lane's row and column group afresh (opaque_lane), so
    // the per-lane addresses are not kept as loop-carried pointers in registers.
    auto row_off = [&](int ci, int lane) {  // rows past the end read the last row; beta and decay are zeroed at use
        return (unsigned)(min(16 * rb + (lane & 15), T_ld - 1 - ci * kC) * H);
    };
    auto load_k = [&](int ci) {
        const int ln = opaque_lane();
        const bf16 *base = static_cast<const bf16 *>(a.k) + tok0_of(ci) * kDK;
        const unsigned ro = row_off(ci, ln) * kDK;
#pragma unroll
        for (int x = 0; x < 2; ++x) kr[x] = load_row8(base + ro, 2 * hf + x, ln >> 4);
    };
    auto load_q = [&](int ci) {
        if constexpr (kMapMode) return;  // (no outputs: q is not read)
        const int ln = opaque_lane();
        const bf16 *base = static_cast<const bf16 *>(a.q) + tok0_of(ci) * kDK;
        const unsigned ro = row_off(ci, ln) * kDK;
#pragma unroll
        for (int x = 0; x < 2; ++x) qr[x] = load_row8(base + ro, 2 * hf + x, ln >> 4);
    };
    auto load_v = [&](int ci) {
        const int ln = opaque_lane();
        const bf16 *base = static_cast<const bf16 *>(a.v) + tok0_of(ci) * kDV;
        const unsigned ro = row_off(ci, ln) * kDV;
#pragma unroll
        for (int x = 0; x < 2; ++x) vr[x] = load_row8(base + ro, 2 * hf + x, ln >> 4);
    };
    auto load_g = [&](int ci) {
        const int ln = opaque_lane();
        const size_t t0b = tok0_of(ci);
        const unsigned ro = row_off(ci, ln);
        if constexpr (kPreact) {
            const bf16 *ap = static_cast<const bf16 *>(a.pre.a) + t0b * kDK + ro * kDK;
#pragma unroll
            for (int x = 0; x < 2; ++x) gar[x] = load_row8(ap, 2 * hf + x, ln >> 4);
        } else if constexpr (G == kGateChannel) {
            const float *gp = a.log_alpha + t0b * kDK + ro * kDK;
#pragma unroll
            for (int x = 0; x < 2; ++x) {
                const f32x4 g0 = *reinterpret_cast<const f32x4 *>(gp + 32 * (2 * hf + x) + 8 * (ln >> 4));
                const f32x4 g1 = *reinterpret_cast<const f32x4 *>(gp + 32 * (2 * hf + x) + 8 * (ln >> 4) + 4);
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    gl[x][e] = g0[e];
                    gl[x][4 + e] = g1[e];
                }
            }
        } else {  // one decay for every channel of the row (log_alpha [T, H]), or none
            const float gv = G == kGateHead ? a.log_alpha[t0b + ro] : 0.f;
#pragma unroll
            for (int x = 0; x < 2; ++x)
#pragma unroll
                for (int e = 0; e < 8; ++e) gl[x][e] = gv;
        }
        bta = a.beta[t0b + ro];
    };
    // pre-activation gates: the head's dt_bias in LDS, complete before the first scan reads
    // it, and its decay-rate scale exp(A_log)
    float eA = 0.f;
    if constexpr (kPreact) {
        if (tid < kDK) dtb[tid] = a.pre.dt_bias[(size_t)h * kDK + tid];
        eA = exp2_fast(a.pre.A_log[h] * kL2E);
        __syncthreads();
    }
    // the identity operands, formed once and read back where a transpose needs them
    // (the first barrier of the loop precedes every read)
    if (w == 0) {
#pragma unroll
        for (int t = 0; t < 2; ++t) *reinterpret_cast<bf16x8 *>(idn + (t * 64 + l) * 8) = ident_frag(t);
    }
    load_g(0);
    load_k(0);
    load_q(0);
    load_v(0);

    bf16 *o = static_cast<bf16 *>(a.o);
    const f32x4 zero4 = {0.f, 0.f, 0.f, 0.f};

    // The accumulators carry Q = P + Km^T U of the last chunk (P = E S at its start);
    // the next chunk's P is E_next (E Q), E = Diag(exp(gamma / 2)). m_prev is the
    // previous chunk's gamma / 2 (zero before the first chunk), kept by the threads
    // that form the per-channel factors.
    float m_prev = 0.f;
    for (int ci = 0; ci < n_c; ++ci) {
        const int t0 = ci * kC;
        const bool more = ci + 1 < n_c;  // the next chunk's inputs are requested below
        const bool full = t0 + kC <= T_len;  // no row of the chunk is past the end

        // ---- 1. inclusive prefix of log(alpha) down the chunk: DPP scan over the
        //      wave's 16 rows, step-major so consecutive DPP operations are
        //      independent; row-block sums to LDS, their prefix by one thread per channel
        float g[2][8], bt;
        {
        KDA_PHASE_LANE
        bt = bta;
        if constexpr (kPreact) {
            // log alpha = -exp(A_log) softplus(a + dt_bias) (channels 32 kg + 8 hi + e of the
            // row), beta = sigmoid(b); softplus(x) = max(x, 0) + log(1 + e^-|x|)
#pragma unroll
            for (int x = 0; x < 2; ++x) {
                const int c0 = 32 * (2 * hf + x) + 8 * hi;
                const f32x4 d0 = *reinterpret_cast<const f32x4 *>(dtb + c0);
                const f32x4 d1 = *reinterpret_cast<const f32x4 *>(dtb + c0 + 4);
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    const float xv = static_cast<float>(gar[x][e]) + (e < 4 ? d0[e] : d1[e - 4]);
                    const float sp = fmaxf(xv, 0.f) +
                                     __builtin_amdgcn_logf(1.f + exp2_fast(-fabsf(xv) * kL2E)) * (1.f / kL2E);
                    g[x][e] = -eA * sp;
                }
            }
            bt = __builtin_amdgcn_rcpf(1.f + exp2_fast(-bta * kL2E));
            if constexpr (kQK) {
                // silu of this chunk's key rows (kept, rounded to bf16, for the
                // elementwise phase) and the sum of their squares over the row's 64
                // channels of this half: lanes lr + 16 hi hold the row. The query rows
                // follow in the elementwise phase: their norm is only needed from the
                // Gram phase on, and it scales rows of Aqk and of O.
                float sk = 0.f;
#pragma unroll
                for (int x = 0; x < 2; ++x) {
                    float fk[8];
#pragma unroll
                    for (int e = 0; e < 8; ++e) {
                        const float kx = static_cast<float>(kr[x][e]);
                        fk[e] = kx * __builtin_amdgcn_rcpf(1.f + exp2_fast(-kx * kL2E));
                        sk += fk[e] * fk[e];
                    }
                    kr[x] = pack8(fk);
                }
                sk += __shfl_xor(sk, 16);
                sk += __shfl_xor(sk, 32);
                if (hi == 0) qks[(hf * kC + r) * 2] = sk;
            }
        } else {
#pragma unroll
            for (int x = 0; x < 2; ++x)
#pragma unroll
                for (int e = 0; e < 8; ++e) g[x][e] = gl[x][e];
        }
        if (!full) {  // rows past the end: no decay, no update
            const bool valid = t0 + r < T_len;
#pragma unroll
            for (int x = 0; x < 2; ++x)
#pragma unroll
                for (int e = 0; e < 8; ++e) g[x][e] = valid ? g[x][e] : 0.f;
            bt = valid ? bt : 0.f;
        }
        if constexpr (kPerChannel) {
#pragma unroll
            for (int x = 0; x < 2; ++x)
#pragma unroll
                for (int e = 0; e < 8; ++e) g[x][e] += dpp_row_shr<1>(g[x][e]);
#pragma unroll
            for (int x = 0; x < 2; ++x)
#pragma unroll
                for (int e = 0; e < 8; ++e) g[x][e] += dpp_row_shr<2>(g[x][e]);
#pragma unroll
            for (int x = 0; x < 2; ++x)
#pragma unroll
                for (int e = 0; e < 8; ++e) g[x][e] += dpp_row_shr<4>(g[x][e]);
#pragma unroll
            for (int x = 0; x < 2; ++x)
#pragma unroll
                for (int e = 0; e < 8; ++e) g[x][e] += dpp_row_shr<8>(g[x][e]);
        } else if constexpr (G == kGateHead) {  // the row's one decay, for every slot
            const float s0 = row16_inclusive_sum(g[0][0]);
#pragma unroll
            for (int x = 0; x < 2; ++x)
#pragma unroll
                for (int e = 0; e < 8; ++e) g[x][e] = s0;
        }
        if (lr == 15) {
#pragma unroll
            for (int x = 0; x < 2; ++x)
#pragma unroll
                for (int e4 = 0; e4 < 2; ++e4)
                    *reinterpret_cast<f32x4 *>(tot + rb * kDK + frag_chan<bf16>(2 * hf + x, hi, 4 * e4)) =
                        f32x4{g[x][4 * e4], g[x][4 * e4 + 1], g[x][4 * e4 + 2], g[x][4 * e4 + 3]};
        }
        if (hf == 0 && hi == 0) bet[r] = bt;
        }
        if (more) load_g(ci + 1);  // decay and beta of this chunk are consumed
        __syncthreads();
        float rk = 1.f;  // inverse row norm of silu(k) (kQK)
        if constexpr (kQK) {
            KDA_PHASE_LANE
            rk = __builtin_amdgcn_rcpf(fmaxf(__builtin_sqrtf(qks[r * 2] + qks[(kC + r) * 2]), kNormEps));
        }
        if (tid < kDK) {
            const float t0v = tot[tid], t1 = tot[kDK + tid], t2 = tot[2 * kDK + tid], t3 = tot[3 * kDK + tid];
            const float gam = (t0v + t1) + (t2 + t3), m = 0.5f * gam;
            offm[tid] = -m * kL2E;
            offm[kDK + tid] = (t0v - m) * kL2E;
            offm[2 * kDK + tid] = ((t0v + t1) - m) * kL2E;
            offm[3 * kDK + tid] = ((t0v + t1 + t2) - m) * kL2E;
            ehalf[e_slot(tid)] = exp2_fast(m_prev * kL2E);
            ehalf[kDK + e_slot(tid)] = exp2_fast(m * kL2E);
            // whether E E_prev of some channel falls below the normal fp32 range
            const unsigned long long tiny = __ballot((m + m_prev) * kL2E < -120.f);
            // whether some channel decays past the midpoint factors' range
            const unsigned long long strong = __ballot(gam < -kStrongDecay);
            if ((tid & 63) == 0) {
                flg[tid >> 6] = tiny != 0ull;
                flg[2 + (tid >> 6)] = strong != 0ull;
            }
            m_prev = m;
            if constexpr (kStrong) {  // block prefixes and gamma in log2 units; exp(gamma)
                gpre[tid] = 0.f;
                gpre[kDK + tid] = t0v * kL2E;
                gpre[2 * kDK + tid] = (t0v + t1) * kL2E;
                gpre[3 * kDK + tid] = (t0v + t1 + t2) * kL2E;
                gpre[4 * kDK + tid] = gam * kL2E;
                egam[e_slot(tid)] = exp2_fast(gam * kL2E);
            }
        }
        __syncthreads();
        if constexpr (!kStrong) {
            // a chunk of strong decay: the pair is left to the strong instance
            if (__builtin_amdgcn_readfirstlane(flg[2] | flg[3]) != 0) {
                if (tid == 0 && u.redo) *u.redo = 1;
                return;
            }
        }

        // ---- 2. elementwise, with d = g - gamma/2 (clamped), u = exp(d), 1/u = exp(-d):
        //      Kp = k u, Qp = q u and Km = k / u (registers and LDS; the query scale is
        //      applied to Aqk and O); Km^T, Kp^T and v^T transposed by the matrix cores
        //      into LDS (beta is carried by T's columns)
        bf16x8 kpf[2], qpf[2];
        // strong instance: the diagonal Gram tiles' sums over this half's channels (row r,
        // columns 16 rb + 4 hi + i)
        f32x4 sad4, saq4;
        if constexpr (kStrong) {
        KDA_PHASE_LANE
        float sq = 0.f;
        float skf[2][8], sqf[2][8], sad[16], saqd[16];
        const bf16x8 id0 = *reinterpret_cast<const bf16x8 *>(idn + l * 8);
        const bf16x8 id1 = *reinterpret_cast<const bf16x8 *>(idn + (64 + l) * 8);
#pragma unroll
        for (int i = 0; i < 16; ++i) sad[i] = saqd[i] = 0.f;
#pragma unroll
        for (int x = 0; x < 2; ++x) {
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                float qv = static_cast<float>(qr[x][e]);
                if constexpr (kQK) {  // silu(q); its row norm is applied to Aqk and O
                    qv *= __builtin_amdgcn_rcpf(1.f + exp2_fast(-qv * kL2E));
                    sq = fmaf(qv, qv, sq);
                }
                skf[x][e] = kQK ? static_cast<float>(kr[x][e]) * rk : static_cast<float>(kr[x][e]);
                sqf[x][e] = qv;
            }
            diag_pairs_accum<8>(skf[x], sqf[x], g[x], sad, saqd);
        }
        diag_pairs_reduce(sad, saqd);
        sad4 = group4(sad, hi);
        saq4 = group4(saqd, hi);
        // state-side operands from the chunk's start: Kp = k 2^ga, Qp = q 2^ga, Km^T =
        // (k 2^(gamma - ga))^T; the Gram's column operand of this block from its end, in Km:
        // k 2^(b - ga), b the decay up to the block's last row (every factor <= 1)
        // (LDS positions from an opaque lane index, so that they are not hoisted out of the
        // chunk loop and kept live across it)
        const int ho = opaque_lane() >> 4;
#pragma unroll
        for (int x = 0; x < 2; ++x) {
            const int kg = 2 * hf + x;
            float xp[8], xq[8], xm[8], xc[8];
            const int c0 = frag_chan<bf16>(kg, ho, 0), c4 = frag_chan<bf16>(kg, ho, 4);
            const f32x4 gp[2] = {*reinterpret_cast<const f32x4 *>(gpre + rb * kDK + c0),
                                 *reinterpret_cast<const f32x4 *>(gpre + rb * kDK + c4)};
            const f32x4 gg[2] = {*reinterpret_cast<const f32x4 *>(gpre + 4 * kDK + c0),
                                 *reinterpret_cast<const f32x4 *>(gpre + 4 * kDK + c4)};
            const f32x4 tb[2] = {*reinterpret_cast<const f32x4 *>(tot + rb * kDK + c0),
                                 *reinterpret_cast<const f32x4 *>(tot + rb * kDK + c4)};
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const float gl = g[x][e] * kL2E, ga = gl + gp[e >> 2][e & 3];
                const float u = exp2_fast(ga), um = exp2_fast(gg[e >> 2][e & 3] - ga);
                xp[e] = skf[x][e] * u;
                xq[e] = sqf[x][e] * u;
                xm[e] = skf[x][e] * um;
                xc[e] = skf[x][e] * exp2_fast(fminf(tb[e >> 2][e & 3] * kL2E - gl, 0.f));
            }
            kpf[x] = pack8(xp);
            qpf[x] = pack8(xq);
            const bf16x8 km = pack8(xm);
            const int off = ((kg * 4 + rb) * 64 + l) * 8;
            *reinterpret_cast<bf16x8 *>(Kp + off) = kpf[x];
            *reinterpret_cast<bf16x8 *>(Qp + off) = qpf[x];
            *reinterpret_cast<bf16x8 *>(Km + off) = pack8(xc);
#pragma unroll
            for (int t = 0; t < 2; ++t)
                store_slots(KtT, rb >> 1, 2 * kg + t, kDK, rb & 1, Frag<bf16>::mma(zero4, km, t ? id1 : id0), l);
        }
#pragma unroll
        for (int x = 0; x < 2; ++x)
#pragma unroll
            for (int t = 0; t < 2; ++t)
                store_slots(Vt, rb >> 1, 2 * (2 * hf + x) + t, kDV, rb & 1, Frag<bf16>::mma(zero4, vr[x], t ? id1 : id0), l);
        if constexpr (kQK) {
            sq += __shfl_xor(sq, 16);
            sq += __shfl_xor(sq, 32);
            if (hi == 0) qks[(hf * kC + r) * 2 + 1] = sq;
        }
        } else {
        KDA_PHASE_LANE
        float sq = 0.f;  // sum of squares of silu(q) over the lane's channels (kQK)
        const bf16x8 id0 = *reinterpret_cast<const bf16x8 *>(idn + l * 8);
        const bf16x8 id1 = *reinterpret_cast<const bf16x8 *>(idn + (64 + l) * 8);
#pragma unroll
        for (int x = 0; x < 2; ++x) {
            const int kg = 2 * hf + x;
            const int c0 = frag_chan<bf16>(kg, hi, 0), c4 = frag_chan<bf16>(kg, hi, 4);
            const f32x4 om0 = *reinterpret_cast<const f32x4 *>(offm + rb * kDK + c0);
            const f32x4 om1 = *reinterpret_cast<const f32x4 *>(offm + rb * kDK + c4);
            float xp[8], xq[8], xm[8];
            if constexpr (kPerChannel) {
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    const float om = e < 4 ? om0[e] : om1[e - 4];
                    const float d = __builtin_amdgcn_fmed3f(fmaf(g[x][e], kL2E, om), -kClamp, kClamp);
                    const float u = exp2_fast(d), ui = exp2_fast(-d);
                    const float kv = kQK ? static_cast<float>(kr[x][e]) * rk : static_cast<float>(kr[x][e]);
                    float qv = static_cast<float>(qr[x][e]);
                    if constexpr (kQK) {  // silu(q); its row norm is applied to Aqk and O
                        qv *= __builtin_amdgcn_rcpf(1.f + exp2_fast(-qv * kL2E));
                        sq = fmaf(qv, qv, sq);
                    }
                    xp[e] = kv * u;
                    xq[e] = qv * u;
                    xm[e] = kv * ui;
                }
            } else {  // one factor pair for the whole row (none without decay)
                float u = 1.f, ui = 1.f;
                if constexpr (G == kGateHead) {
                    const float d = __builtin_amdgcn_fmed3f(fmaf(g[0][0], kL2E, om0[0]), -kClamp, kClamp);
                    u = exp2_fast(d);
                    ui = exp2_fast(-d);
                }
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    const float kv = static_cast<float>(kr[x][e]);
                    xp[e] = kv * u;
                    xq[e] = static_cast<float>(qr[x][e]) * u;
                    xm[e] = kv * ui;
                }
            }
            kpf[x] = pack8(xp);
            const bf16x8 km = pack8(xm);
            const int off = ((kg * 4 + rb) * 64 + l) * 8;
            *reinterpret_cast<bf16x8 *>(Kp + off) = kpf[x];
            if constexpr (!kMapMode) {  // (the map instance has no outputs)
                qpf[x] = pack8(xq);
                *reinterpret_cast<bf16x8 *>(Qp + off) = qpf[x];
            }
            *reinterpret_cast<bf16x8 *>(Km + off) = km;
            // chunk rows 16 rb .. are contraction slots 4 (rb % 2) .. of group rb / 2
#pragma unroll
            for (int t = 0; t < 2; ++t)
                store_slots(KtT, rb >> 1, 2 * kg + t, kDK, rb & 1, Frag<bf16>::mma(zero4, km, t ? id1 : id0), l);
        }
#pragma unroll
        for (int x = 0; x < 2; ++x)
#pragma unroll
            for (int t = 0; t < 2; ++t)
                store_slots(Vt, rb >> 1, 2 * (2 * hf + x) + t, kDV, rb & 1, Frag<bf16>::mma(zero4, vr[x], t ? id1 : id0), l);
        if constexpr (kQK && !kMapMode) {
            sq += __shfl_xor(sq, 16);
            sq += __shfl_xor(sq, 32);
            if (hi == 0) qks[(hf * kC + r) * 2 + 1] = sq;
        }
        }
        if (more && !kStrong) load_k(ci + 1);  // key rows consumed (the strong instance reads them again below)
        __syncthreads();  // Kp, Qp, Km, Km^T, Kp^T, v^T complete

        // (used by the waves of half 0, which hold the diagonal block rb of A in LDS)
        auto diag_inverse = [&](const f32x4 bv) {
            KDA_PHASE_LANE
            // (I + L)^{-1} of the diagonal block L = A[16rb.., 16rb..] by forward
            // substitution: lane (r, hi) holds X[r][4 hi + j]; step i subtracts
            // L[r][i] times row i (broadcast within the 16-lane row). The block's
            // rows were written by this wave, and the LDS operations of one wave
            // are performed in order.
            float Lr[16];
#pragma unroll
            for (int v4 = 0; v4 < 4; ++v4) {
                const f32x4 t = *reinterpret_cast<const f32x4 *>(Am + r * kPT + 16 * rb + 4 * v4);
#pragma unroll
                for (int e = 0; e < 4; ++e) Lr[4 * v4 + e] = t[e];
            }
            float xs[4];
#pragma unroll
            for (int j = 0; j < 4; ++j) xs[j] = (lr == 4 * hi + j) ? 1.f : 0.f;
#define KDA_SUBST_STEP(I) \
    _Pragma("unroll") for (int j = 0; j < 4; ++j) xs[j] = fmaf(-Lr[I], row_bcast<I>(xs[j]), xs[j]);
            KDA_SUBST_STEP(0) KDA_SUBST_STEP(1) KDA_SUBST_STEP(2) KDA_SUBST_STEP(3)
            KDA_SUBST_STEP(4) KDA_SUBST_STEP(5) KDA_SUBST_STEP(6) KDA_SUBST_STEP(7)
            KDA_SUBST_STEP(8) KDA_SUBST_STEP(9) KDA_SUBST_STEP(10) KDA_SUBST_STEP(11)
            KDA_SUBST_STEP(12) KDA_SUBST_STEP(13) KDA_SUBST_STEP(14)
#undef KDA_SUBST_STEP
            // T fragments of row block rb: the diagonal block in slots 4 (rb % 2) ..,
            // and the zero block above the diagonal for even rb
            // (the unscaled block for the off-diagonal chain; T Diag(beta) for the state phase,
            // beta of the block's columns 16 rb + 4 hi + j)
            *reinterpret_cast<bf16x4 *>(Dg + (rb * 64 + l) * 4) = to_bf16x4(f32x4{xs[0], xs[1], xs[2], xs[3]});
            store_slots(Tf, rb >> 1, rb, kC, rb & 1, f32x4{xs[0] * bv[0], xs[1] * bv[1], xs[2] * bv[2], xs[3] * bv[3]}, l);
            if ((rb & 1) == 0) store_slots(Tf, rb >> 1, rb, kC, 1, zero4, l);
        };

        // ---- 3. Gram rows of block rb, contraction over all 128 channels (own half
        //      from registers, the other half from LDS)
        if constexpr (kStrong) {
            KDA_PHASE_LANE
            // Each wave: its half's share of A's tiles (rb, tj < rb) and of Aqk^T's tiles (tj, rb),
            // with the end of block tj as the reference (rows k 2^(ga - b_tj), q 2^(ga - b_tj);
            // columns Km of block tj), and of the diagonal tiles (pair sums of phase 2). Half 1
            // leaves its shares in A's place and in saq; half 0 adds its own, scales and masks,
            // and inverts the diagonal block as the usual instance does.
            const f32x4 bv = *reinterpret_cast<const f32x4 *>(bet + 16 * rb + 4 * hi);
            f32x4 at[3], qt[3];
#pragma unroll
            for (int tj = 0; tj < 3; ++tj) {
                at[tj] = qt[tj] = zero4;
                if (tj < rb) {
                    bf16x8 rk2[2], rq2[2];
                    const int ho = opaque_lane() >> 4;
#pragma unroll
                    for (int x = 0; x < 2; ++x) {
                        float xr[8], xs2[8];
                        const int c0 = frag_chan<bf16>(2 * hf + x, ho, 0), c4 = frag_chan<bf16>(2 * hf + x, ho, 4);
                        const f32x4 d[2] = {*reinterpret_cast<const f32x4 *>(gpre + rb * kDK + c0) -
                                                *reinterpret_cast<const f32x4 *>(gpre + (tj + 1) * kDK + c0),
                                            *reinterpret_cast<const f32x4 *>(gpre + rb * kDK + c4) -
                                                *reinterpret_cast<const f32x4 *>(gpre + (tj + 1) * kDK + c4)};
#pragma unroll
                        for (int e = 0; e < 8; ++e) {
                            float qv = static_cast<float>(qr[x][e]);
                            if constexpr (kQK) qv *= __builtin_amdgcn_rcpf(1.f + exp2_fast(-qv * kL2E));
                            const float kv = kQK ? static_cast<float>(kr[x][e]) * rk : static_cast<float>(kr[x][e]);
                            const float f = exp2_fast(fminf(fmaf(g[x][e], kL2E, d[e >> 2][e & 3]), 0.f));
                            xr[e] = kv * f;
                            xs2[e] = qv * f;
                        }
                        rk2[x] = pack8(xr);
                        rq2[x] = pack8(xs2);
                    }
                    const bf16x8 c0 = fld(Km, 2 * hf, tj, kC, l), c1 = fld(Km, 2 * hf + 1, tj, kC, l);
                    at[tj] = Frag<bf16>::mma(Frag<bf16>::mma(zero4, rk2[0], c0), rk2[1], c1);
                    qt[tj] = Frag<bf16>::mma(Frag<bf16>::mma(zero4, c0, rq2[0]), c1, rq2[1]);
                }
            }
            const f32x4 ad4 = sad4, aq4 = saq4;  // row r, columns 16 rb + 4 hi + i
            float *sq_rb = saq + (rb * (rb + 1) / 2) * 256;
            if (more) load_k(ci + 1);  // key rows consumed
            if (hf == 1) {
#pragma unroll
                for (int tj = 0; tj < 3; ++tj) {
                    if (tj < rb) {
#pragma unroll
                        for (int i = 0; i < 4; ++i) Am[(16 * rb + 4 * hi + i) * kPT + 16 * tj + lr] = at[tj][i];
                        *reinterpret_cast<f32x4 *>(sq_rb + tj * 256 + 4 * l) = qt[tj];
                    }
                }
                *reinterpret_cast<f32x4 *>(Am + r * kPT + 16 * rb + 4 * hi) = ad4;
                *reinterpret_cast<f32x4 *>(sq_rb + rb * 256 + 4 * l) = aq4;
            }
            __syncthreads();  // half 1's shares in place
            if (hf == 0) {
#pragma unroll
                for (int tj = 0; tj < 3; ++tj) {
                    if (tj < rb) {
#pragma unroll
                        for (int i = 0; i < 4; ++i) {
                            float *p = Am + (16 * rb + 4 * hi + i) * kPT + 16 * tj + lr;
                            *p = bv[i] * (*p + at[tj][i]);
                        }
                    }
                }
                {
                    const float br = bet[r];
                    float *p = Am + r * kPT + 16 * rb + 4 * hi;
                    const f32x4 o4 = *reinterpret_cast<const f32x4 *>(p);
                    f32x4 d4;
#pragma unroll
                    for (int i = 0; i < 4; ++i) d4[i] = (4 * hi + i < lr) ? br * (o4[i] + ad4[i]) : 0.f;
                    *reinterpret_cast<f32x4 *>(p) = d4;
                }
                // Aqk's scale, times the inverse norm of silu(q)'s row r (kQK; kept for O)
                float aqs = scale;
                if constexpr (kQK) {
                    const float n = __builtin_amdgcn_rcpf(
                        fmaxf(__builtin_sqrtf(qks[r * 2 + 1] + qks[(kC + r) * 2 + 1]), kNormEps));
                    if (hi == 0) qnr[r] = n;
                    aqs *= n;
                }
#pragma unroll
                for (int tj = 0; tj < 4; ++tj) {
                    if (tj < 2 * ((rb >> 1) + 1)) {
                        f32x4 acc = zero4;
                        if (tj < rb) {
                            acc = (qt[tj < 3 ? tj : 0] + *reinterpret_cast<const f32x4 *>(sq_rb + tj * 256 + 4 * l)) * aqs;
                        } else if (tj == rb) {
                            acc = (aq4 + *reinterpret_cast<const f32x4 *>(sq_rb + rb * 256 + 4 * l)) * aqs;
#pragma unroll
                            for (int i = 0; i < 4; ++i) acc[i] = (4 * hi + i <= lr) ? acc[i] : 0.f;
                        }
                        store_slots(Aqk, tj >> 1, rb, kC, tj & 1, acc, l);
                    }
                }
                diag_inverse(bv);
            }
        } else if (hf == 0) {
            KDA_PHASE_LANE
            // the diagonal block of A[r][i] = beta_r <Kp_r, Km_i> (i < r), then the
            // inverse of (I + that block)
            const bf16x8 ka[4] = {kpf[0], kpf[1], fld(Kp, 2, rb, kC, l), fld(Kp, 3, rb, kC, l)};
            const f32x4 bv = *reinterpret_cast<const f32x4 *>(bet + 16 * rb + 4 * hi);
            bf16x8 kmb[4];
#pragma unroll
            for (int kg = 0; kg < 4; ++kg) kmb[kg] = fld(Km, kg, rb, kC, l);
            f32x4 acc = zero4;
#pragma unroll
            for (int kg = 0; kg < 4; ++kg) acc = Frag<bf16>::mma(acc, ka[kg], kmb[kg]);
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int rr = 16 * rb + 4 * hi + i, cc = 16 * rb + lr;
                Am[rr * kPT + cc] = (cc < rr) ? bv[i] * acc[i] : 0.f;
            }
            diag_inverse(bv);
        } else {
            KDA_PHASE_LANE
            // The off-diagonal blocks of A's rows rb, A[r][i] = beta_r <Kp_r, Km_i> (i < 16 rb),
            // and Aqk[r][i] = scale <Qp_r, Km_i> (i <= r) for the rows of block rq = 3 - rb:
            // four tiles on every wave of this half, with the diagonal blocks of A on the
            // other half. Tiles of Aqk^T = Km Qp^T are the operand slots of Aqk's rows rq.
            // Each Km column block is read once (the next one while the current one is
            // multiplied) and serves both products.
            const int rq = 3 - rb;
            bf16x8 qb[4];
            if constexpr (!kMapMode) {  // (the map instance forms no Aqk)
#pragma unroll
                for (int kg = 0; kg < 4; ++kg) qb[kg] = fld(Qp, kg, rq, kC, l);
            }
            // (read unconditionally: a conditional read would be merged with an undefined
            // value at the branch's end, which costs register copies on every path)
            bf16x8 ka[4];
#pragma unroll
            for (int kg = 0; kg < 4; ++kg) ka[kg] = fld(Kp, kg, rb, kC, l);
            const f32x4 bv = *reinterpret_cast<const f32x4 *>(bet + 16 * rb + 4 * hi);
            // Aqk's scale, times the inverse norm of silu(q)'s row 16 rq + lr (kQK; kept
            // for the state phase's O)
            float aqs = scale;
            if constexpr (kQK && !kMapMode) {
                const int qrow = 16 * rq + lr;
                const float n = __builtin_amdgcn_rcpf(
                    fmaxf(__builtin_sqrtf(qks[qrow * 2 + 1] + qks[(kC + qrow) * 2 + 1]), kNormEps));
                if (hi == 0) qnr[qrow] = n;
                aqs *= n;
            }
            bf16x8 kmb[2][4];
#pragma unroll
            for (int kg = 0; kg < 4; ++kg) kmb[0][kg] = fld(Km, kg, 0, kC, l);
#pragma unroll
            for (int tj = 0; tj < 4; ++tj) {
                if (tj < 3) {  // block tj + 1 (read even when unused, see ka)
#pragma unroll
                    for (int kg = 0; kg < 4; ++kg) kmb[(tj + 1) & 1][kg] = fld(Km, kg, tj + 1, kC, l);
                }
                __builtin_amdgcn_sched_barrier(0);
                if (tj < rb) {
                    f32x4 acc = zero4;
#pragma unroll
                    for (int kg = 0; kg < 4; ++kg) acc = Frag<bf16>::mma(acc, ka[kg], kmb[tj & 1][kg]);
#pragma unroll
                    for (int i = 0; i < 4; ++i) Am[(16 * rb + 4 * hi + i) * kPT + 16 * tj + lr] = bv[i] * acc[i];
                }
                if (!kMapMode && tj < 2 * ((rq >> 1) + 1)) {
                    f32x4 acc = zero4;
                    if (tj <= rq) {
#pragma unroll
                        for (int kg = 0; kg < 4; ++kg) acc = Frag<bf16>::mma(acc, kmb[tj & 1][kg], qb[kg]);
#pragma unroll
                        for (int i = 0; i < 4; ++i) acc[i] *= aqs;
                        if (tj == rq) {  // the diagonal tile: i <= r only (the others lie below it)
#pragma unroll
                            for (int i = 0; i < 4; ++i) acc[i] = (4 * hi + i <= lr) ? acc[i] : 0.f;
                        }
                    }
                    store_slots(Aqk, tj >> 1, rq, kC, tj & 1, acc, l);
                }
            }
        }
        __syncthreads();  // A, the diagonal blocks of T and Aqk complete

        // ---- 4. off-diagonal blocks of T' = T Diag(beta), column block j = rb by wave
        //      (rb, 1): T'_ij = -D_i Y, Y = sum_{k=j}^{i-1} A_ik T'_kj (D_i = T_ii, the
        //      unscaled diagonal block; the column scaling passes through the sum).
        //      Both orientations of each block are formed from Y: T'_ij (as the B
        //      operand of the next Y) and T'_ij^T (whose tile is T'_ij's A operand, stored).
        if (hf == 1 && rb < 3) {
            KDA_PHASE_LANE
            const int j = rb;
            // every operand of the chain is read first: T'_jj, the blocks A_ik (j <= k < i)
            // and the diagonal blocks D_i (i > j); one wait, then the dependent products
            f32x4 ar[4][3];
            bf16x4 dg[4];
            const bf16x4 tjj = load_slots(Tf, j >> 1, j, kC, j & 1, l);
            // (all below-diagonal blocks, whichever j needs: conditional reads would be
            // merged with undefined values at the branches' ends, at the cost of copies)
#pragma unroll
            for (int i = 1; i < 4; ++i) {
                dg[i] = *reinterpret_cast<const bf16x4 *>(Dg + (i * 64 + l) * 4);
#pragma unroll
                for (int k = 0; k < 3; ++k)
                    if (k < i) ar[i][k] = *reinterpret_cast<const f32x4 *>(Am + (16 * i + lr) * kPT + 16 * k + 4 * hi);
            }
            __builtin_amdgcn_sched_barrier(0);
            // Right-looking order, with the column block j as a compile-time constant (so
            // that the accumulators stay in registers): as soon as T'_kj is known, its
            // contribution A_ik T'_kj is added to every later row block i, so that each
            // level waits on one product and the multiplication by D_i, not on the sum.
            auto chain = [&](auto jt) {
                constexpr int J = decltype(jt)::value;
                f32x4 y[4] = {zero4, zero4, zero4, zero4};
                {
                    const bf16x4 tb = to_bf16x4(mma16(tjj, *reinterpret_cast<const bf16x4 *>(idn + l * 8), zero4));
#pragma unroll
                    for (int i = J + 1; i < 4; ++i) y[i] = mma16(to_bf16x4(ar[i][J]), tb, y[i]);
                }
#pragma unroll
                for (int i = J + 1; i < 4; ++i) {
                    const bf16x4 yb = to_bf16x4(y[i]);
                    store_slots(Tf, J >> 1, i, kC, J & 1, -mma16(yb, dg[i], zero4), l);
                    if (i < 3) {
                        const bf16x4 tb = to_bf16x4(-mma16(dg[i], yb, zero4));
#pragma unroll
                        for (int i2 = i + 1; i2 < 4; ++i2) y[i2] = mma16(to_bf16x4(ar[i2][i]), tb, y[i2]);
                    }
                }
            };
            if (j == 0)
                chain(IntTag<0>{});
            else if (j == 1)
                chain(IntTag<1>{});
            else
                chain(IntTag<2>{});
        }
        // the next chunk's query and value rows: the waves without a chain above (half 0
        // and the last row block) request them at once, the others after their chain
        if (more) {
            load_q(ci + 1);
            load_v(ci + 1);
        }
        __syncthreads();  // T complete

        // ---- 5. state phase (columns 16 w ..): P = E (E_prev Q); Y = v - Kp P;
        //      U = T' Y (that is U~ - W' P with U~ = T' v, W' = T' Kp); O = scale Qp P
        //      + Aqk U (stored); Q = P + Km^T U, so that S_next = E Q. The shared
        //      operands come from LDS one row block ahead of the products that use
        //      them (the scheduling barriers keep those reads ahead of the
        //      matrix-core work).
        if constexpr (kMapMode) {
            // The map instance: the same update for N (accS, with v) and for M (accM, whose
            // "values" are zero: Y = -Kp P), no outputs.
            KDA_PHASE_LANE
            auto scale_rows = [&](f32x4 (&acc)[8]) {  // P = E (E_prev Q), as below
                if constexpr (G == kGateHead) {
                    const float ep0 = ehalf[0], ec0 = ehalf[kDK];
                    if (__builtin_amdgcn_readfirstlane(flg[0] | flg[1]) != 0) {
#pragma unroll
                        for (int tm = 0; tm < 8; ++tm) acc[tm] = acc[tm] * ep0 * ec0;
                    } else {
#pragma unroll
                        for (int tm = 0; tm < 8; ++tm) acc[tm] *= ep0 * ec0;
                    }
                }
                if constexpr (kPerChannel) {
                    const f32x2 ep = *reinterpret_cast<const f32x2 *>(ehalf + 32 * hi + 2 * lr);
                    const f32x2 ec = *reinterpret_cast<const f32x2 *>(ehalf + kDK + 32 * hi + 2 * lr);
                    if (__builtin_amdgcn_readfirstlane(flg[0] | flg[1]) != 0) {
#define KDA_EROW(TM)                                                                     \
    acc[TM][0] = acc[TM][0] * row_bcast<2 * TM>(ep[0]) * row_bcast<2 * TM>(ec[0]);         \
    acc[TM][1] = acc[TM][1] * row_bcast<2 * TM>(ep[1]) * row_bcast<2 * TM>(ec[1]);         \
    acc[TM][2] = acc[TM][2] * row_bcast<2 * TM + 1>(ep[0]) * row_bcast<2 * TM + 1>(ec[0]); \
    acc[TM][3] = acc[TM][3] * row_bcast<2 * TM + 1>(ep[1]) * row_bcast<2 * TM + 1>(ec[1]);
                        KDA_EROW(0) KDA_EROW(1) KDA_EROW(2) KDA_EROW(3) KDA_EROW(4) KDA_EROW(5) KDA_EROW(6) KDA_EROW(7)
#undef KDA_EROW
                    } else {
                        const f32x2 e2 = ep * ec;
#define KDA_EROW(TM)                                   \
    acc[TM][0] *= row_bcast<2 * TM>(e2[0]);            \
    acc[TM][1] *= row_bcast<2 * TM>(e2[1]);            \
    acc[TM][2] *= row_bcast<2 * TM + 1>(e2[0]);        \
    acc[TM][3] *= row_bcast<2 * TM + 1>(e2[1]);
                        KDA_EROW(0) KDA_EROW(1) KDA_EROW(2) KDA_EROW(3) KDA_EROW(4) KDA_EROW(5) KDA_EROW(6) KDA_EROW(7)
#undef KDA_EROW
                    }
                }
            };
            auto advance = [&](f32x4 (&acc)[8], bool with_v) {  // Y = v - Kp P; U = T' Y; Q = P + Km^T U
                bf16x8 sb[4];
#pragma unroll
                for (int kg = 0; kg < 4; ++kg) sb[kg] = tiles_to_frag(acc[2 * kg], acc[2 * kg + 1]);
                const bf16x8 vf[2] = {fld(Vt, 0, w, kDV, l), fld(Vt, 1, w, kDV, l)};
                bf16x8 fa[2][4];
#pragma unroll
                for (int kg = 0; kg < 4; ++kg) fa[0][kg] = fld(Kp, kg, 0, kC, l);
                bf16x8 tq[6];
                f32x4 ya[4];
#pragma unroll
                for (int rr = 0; rr < 4; ++rr) {
                    if (rr < 3) {
#pragma unroll
                        for (int kg = 0; kg < 4; ++kg) fa[(rr + 1) & 1][kg] = fld(Kp, kg, rr + 1, kC, l);
                    } else {
#pragma unroll
                        for (int q = 0; q < 4; ++q) tq[q] = fld(Tf, 0, q, kC, l);
                        tq[4] = fld(Tf, 1, 2, kC, l);
                        tq[5] = fld(Tf, 1, 3, kC, l);
                    }
                    __builtin_amdgcn_sched_barrier(0);
                    f32x4 pk = zero4;
#pragma unroll
                    for (int kg = 0; kg < 4; ++kg) pk = Frag<bf16>::mma(pk, fa[rr & 1][kg], sb[kg]);
#pragma unroll
                    for (int i = 0; i < 4; ++i)
                        ya[rr][i] = (with_v ? static_cast<float>(vf[rr >> 1][4 * (rr & 1) + i]) : 0.f) - pk[i];
                }
                const bf16x8 yb[2] = {tiles_to_frag(ya[0], ya[1]), tiles_to_frag(ya[2], ya[3])};
                f32x4 ua[4];
#pragma unroll
                for (int rr = 0; rr < 4; ++rr) {
                    ua[rr] = Frag<bf16>::mma(zero4, tq[rr], yb[0]);
                    if (rr >= 2) ua[rr] = Frag<bf16>::mma(ua[rr], tq[rr + 2], yb[1]);
                }
                bf16x8 ub[2];
#pragma unroll
                for (int kc = 0; kc < 2; ++kc) ub[kc] = tiles_to_frag(ua[2 * kc], ua[2 * kc + 1]);
                bf16x8 kf[2][2];
#pragma unroll
                for (int kc = 0; kc < 2; ++kc) kf[0][kc] = fld(KtT, kc, 0, kDK, l);
#pragma unroll
                for (int tm = 0; tm < 8; ++tm) {
                    if (tm < 7) {
#pragma unroll
                        for (int kc = 0; kc < 2; ++kc) kf[(tm + 1) & 1][kc] = fld(KtT, kc, tm + 1, kDK, l);
                    }
                    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
                    for (int kc = 0; kc < 2; ++kc) acc[tm] = Frag<bf16>::mma(acc[tm], kf[tm & 1][kc], ub[kc]);
                }
            };
            scale_rows(accS);
            scale_rows(accM);
            advance(accS, true);
            advance(accM, false);
        } else {
            KDA_PHASE_LANE
            {
                // P = E (E_prev Q). Q can be as large as E_prev is small, so where the
                // product E E_prev leaves the normal fp32 range (fast-forgetting channels)
                // the two factors are applied one after the other; otherwise their product
                // is. Lane (c, hi) needs the factors of key positions 16 tm + 4 hi + i;
                // lane lr of the row holds those of 4 tm + i = 2 lr, 2 lr + 1.
                // (The strong instance holds S itself: no factor.)
                if constexpr (G == kGateHead && !kStrong) {  // one factor pair for every row
                    const float ep0 = ehalf[0], ec0 = ehalf[kDK];
                    if (__builtin_amdgcn_readfirstlane(flg[0] | flg[1]) != 0) {
#pragma unroll
                        for (int tm = 0; tm < 8; ++tm) accS[tm] = accS[tm] * ep0 * ec0;
                    } else {
                        const float e2 = ep0 * ec0;
#pragma unroll
                        for (int tm = 0; tm < 8; ++tm) accS[tm] *= e2;
                    }
                }
                if constexpr (kPerChannel && !kStrong) {
                const f32x2 ep = *reinterpret_cast<const f32x2 *>(ehalf + 32 * hi + 2 * lr);
                const f32x2 ec = *reinterpret_cast<const f32x2 *>(ehalf + kDK + 32 * hi + 2 * lr);
                if (__builtin_amdgcn_readfirstlane(flg[0] | flg[1]) != 0) {
#define KDA_EROW(TM)                                                                       \
    accS[TM][0] = accS[TM][0] * row_bcast<2 * TM>(ep[0]) * row_bcast<2 * TM>(ec[0]);         \
    accS[TM][1] = accS[TM][1] * row_bcast<2 * TM>(ep[1]) * row_bcast<2 * TM>(ec[1]);         \
    accS[TM][2] = accS[TM][2] * row_bcast<2 * TM + 1>(ep[0]) * row_bcast<2 * TM + 1>(ec[0]); \
    accS[TM][3] = accS[TM][3] * row_bcast<2 * TM + 1>(ep[1]) * row_bcast<2 * TM + 1>(ec[1]);
                    KDA_EROW(0) KDA_EROW(1) KDA_EROW(2) KDA_EROW(3) KDA_EROW(4) KDA_EROW(5) KDA_EROW(6) KDA_EROW(7)
#undef KDA_EROW
                } else {
                    const f32x2 e2 = ep * ec;
#define KDA_EROW(TM)                                     \
    accS[TM][0] *= row_bcast<2 * TM>(e2[0]);             \
    accS[TM][1] *= row_bcast<2 * TM>(e2[1]);             \
    accS[TM][2] *= row_bcast<2 * TM + 1>(e2[0]);         \
    accS[TM][3] *= row_bcast<2 * TM + 1>(e2[1]);
                    KDA_EROW(0) KDA_EROW(1) KDA_EROW(2) KDA_EROW(3) KDA_EROW(4) KDA_EROW(5) KDA_EROW(6) KDA_EROW(7)
#undef KDA_EROW
                }
                }  // (no decay: no factor)
            }
            bf16x8 sb[4];
#pragma unroll
            for (int kg = 0; kg < 4; ++kg) sb[kg] = tiles_to_frag(accS[2 * kg], accS[2 * kg + 1]);
            // v of the wave's columns: fragment group kc of v^T's column block w holds the
            // accumulator tiles 2 kc and 2 kc + 1 of v (chunk rows 16 rr + 4 hi + i in
            // slots 4 (rr % 2) + i)
            const bf16x8 vf[2] = {fld(Vt, 0, w, kDV, l), fld(Vt, 1, w, kDV, l)};
            bf16x8 fa[2][4];
#pragma unroll
            for (int kg = 0; kg < 4; ++kg) fa[0][kg] = fld(Kp, kg, 0, kC, l);
            bf16x8 tq[6];  // T' operand groups (rows rr, contraction group kc <= rr / 2)
            f32x4 ya[4];
#pragma unroll
            for (int rr = 0; rr < 4; ++rr) {
                if (rr < 3) {
#pragma unroll
                    for (int kg = 0; kg < 4; ++kg) fa[(rr + 1) & 1][kg] = fld(Kp, kg, rr + 1, kC, l);
                } else {  // next: T', then Qp rows 0
#pragma unroll
                    for (int q = 0; q < 4; ++q) tq[q] = fld(Tf, 0, q, kC, l);
                    tq[4] = fld(Tf, 1, 2, kC, l);
                    tq[5] = fld(Tf, 1, 3, kC, l);
#pragma unroll
                    for (int kg = 0; kg < 4; ++kg) fa[0][kg] = fld(Qp, kg, 0, kC, l);
                }
                __builtin_amdgcn_sched_barrier(0);
                f32x4 acc = zero4;
#pragma unroll
                for (int kg = 0; kg < 4; ++kg) acc = Frag<bf16>::mma(acc, fa[rr & 1][kg], sb[kg]);
#pragma unroll
                for (int i = 0; i < 4; ++i) ya[rr][i] = static_cast<float>(vf[rr >> 1][4 * (rr & 1) + i]) - acc[i];
            }
            const bf16x8 yb[2] = {tiles_to_frag(ya[0], ya[1]), tiles_to_frag(ya[2], ya[3])};
            f32x4 ua[4];
#pragma unroll
            for (int rr = 0; rr < 4; ++rr) {
                ua[rr] = Frag<bf16>::mma(zero4, tq[rr], yb[0]);
                if (rr >= 2) ua[rr] = Frag<bf16>::mma(ua[rr], tq[rr + 2], yb[1]);
            }
            bf16x8 ub[2];
#pragma unroll
            for (int kc = 0; kc < 2; ++kc) ub[kc] = tiles_to_frag(ua[2 * kc], ua[2 * kc + 1]);
            bf16x8 kf[2][2];
            // value positions 16 w + 4 hi + i are channels 32 (w / 2) + 8 hi + 4 (w % 2) + i
            bf16 *o_chunk = o + ((seq0 + t0) * H + h) * kDV + 32 * (w >> 1) + 4 * (w & 1);
#pragma unroll
            for (int rr = 0; rr < 4; ++rr) {
                bf16x8 aq[2];
#pragma unroll
                for (int kc = 0; kc < 2; ++kc)
                    if (kc <= (rr >> 1)) aq[kc] = fld(Aqk, kc, rr, kC, l);
                if (rr < 3) {
#pragma unroll
                    for (int kg = 0; kg < 4; ++kg) fa[(rr + 1) & 1][kg] = fld(Qp, kg, rr + 1, kC, l);
                } else {
#pragma unroll
                    for (int kc = 0; kc < 2; ++kc) kf[0][kc] = fld(KtT, kc, 0, kDK, l);
                }
                __builtin_amdgcn_sched_barrier(0);
                // O^T = S^T (scale Qp)^T + U^T Aqk^T: the operands of O's products with
                // their roles swapped (A-layout(X^T) is B-layout(X)), so that the
                // accumulator tile is O^T and lane (r, hi) holds 4 adjacent columns
                // of chunk row 16 rr + r, stored as 8 bytes
                f32x4 ot = zero4;
#pragma unroll
                for (int kg = 0; kg < 4; ++kg) ot = Frag<bf16>::mma(ot, sb[kg], fa[rr & 1][kg]);
                ot *= kQK ? scale * qnr[16 * rr + lr] : scale;
#pragma unroll
                for (int kc = 0; kc < 2; ++kc)
                    if (kc <= (rr >> 1)) ot = Frag<bf16>::mma(ot, ub[kc], aq[kc]);
                bf16 *dst = o_chunk + (unsigned)(((16 * rr + lr) * H) * kDV + 8 * hi);
                if (!full && t0 + 16 * rr + lr >= T_len) dst = static_cast<bf16 *>(a.discard) + 4 * (l & 31);
                *reinterpret_cast<bf16x4 *>(dst) = to_bf16x4(ot);
            }
            if constexpr (kStrong) {
                // S_next = Diag(exp(gamma)) S + Km^T U
                const f32x2 eg2 = *reinterpret_cast<const f32x2 *>(egam + 32 * hi + 2 * lr);
#define KDA_EROW(TM)                                 \
    accS[TM][0] *= row_bcast<2 * TM>(eg2[0]);        \
    accS[TM][1] *= row_bcast<2 * TM>(eg2[1]);        \
    accS[TM][2] *= row_bcast<2 * TM + 1>(eg2[0]);    \
    accS[TM][3] *= row_bcast<2 * TM + 1>(eg2[1]);
                KDA_EROW(0) KDA_EROW(1) KDA_EROW(2) KDA_EROW(3) KDA_EROW(4) KDA_EROW(5) KDA_EROW(6) KDA_EROW(7)
#undef KDA_EROW
            }
#pragma unroll
            for (int tm = 0; tm < 8; ++tm) {
                if (tm < 7) {
#pragma unroll
                    for (int kc = 0; kc < 2; ++kc) kf[(tm + 1) & 1][kc] = fld(KtT, kc, tm + 1, kDK, l);
                }
                __builtin_amdgcn_sched_barrier(0);
#pragma unroll
                for (int kc = 0; kc < 2; ++kc) accS[tm] = Frag<bf16>::mma(accS[tm], kf[tm & 1][kc], ub[kc]);
            }
        }
        // No barrier here: before the next chunk writes anything the state phase
        // reads (from the per-channel factors on), every wave passes its first barrier.
    }

    // The last chunk's factor exp(gamma / 2) on the rows of what leaves (S = E_last Q), once
    // every wave has read that chunk's factors; then the buffer that held them may be reused.
    auto last_factor = [&](f32x4 (&acc)[8]) {
#pragma unroll
        for (int tm = 0; tm < 8; ++tm) {
            const f32x4 e4 = {ehalf[e_slot(16 * tm + 4 * hi)], ehalf[e_slot(16 * tm + 4 * hi + 1)],
                              ehalf[e_slot(16 * tm + 4 * hi + 2)], ehalf[e_slot(16 * tm + 4 * hi + 3)]};
            acc[tm] = acc[tm] * e4;
        }
    };
    float *stg = reinterpret_cast<float *>(smem);
    if constexpr (kMapMode) {
        // M = E_last Q_M and N = E_last Q_N, each staged in LDS in the order the composition
        // reads it, then copied out in whole 16-byte pieces: first M as its two bf16 parts
        // (hi = M rounded, lo = the rest rounded, seg_mh_index), then N in fp32 (seg_n_index)
        __syncthreads();
        if (tid < kDK) ehalf[e_slot(tid)] = exp2_fast(m_prev * kL2E);
        __syncthreads();
        last_factor(accM);
        last_factor(accS);
        __syncthreads();
        const int cc = chan_of_pos(16 * w + lr);
        bf16 *stg_h = reinterpret_cast<bf16 *>(smem);
#pragma unroll
        for (int half = 0; half < 2; ++half) {
#pragma unroll
            for (int tm = 0; tm < 8; ++tm)
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int r = chan_of_pos(16 * tm + 4 * hi + i);
                    if (half == 0) {
                        const bf16 mh = static_cast<bf16>(accM[tm][i]);
                        stg_h[seg_mh_index(r, cc)] = mh;
                        stg_h[kDK * kDK + seg_mh_index(r, cc)] = static_cast<bf16>(accM[tm][i] - static_cast<float>(mh));
                    } else {
                        stg[seg_n_index(r, cc)] = accS[tm][i];
                    }
                }
            __syncthreads();
            float *dst = u.map_out + half * kDK * kDK;
#pragma unroll
            for (int k = 0; k < kDK * kDK / 4 / kNT; ++k) {
                const int piece = tid + kNT * k;
                *reinterpret_cast<f32x4 *>(dst + 4 * piece) = *reinterpret_cast<const f32x4 *>(stg + 4 * piece);
            }
            if (half == 0) __syncthreads();
        }
        if (tid == 0) *u.redo = 0;  // no chunk of strong decay in this segment
        return;
    } else if constexpr (!kStrong) {
        if (tid == 0 && u.redo) *u.redo = 0;  // no chunk of strong decay in this run
    } else {
        if (u.out_state) {
            __syncthreads();  // every wave is done with the last chunk's operands
            store_state(u.out_state, accS, stg, tid, w, lr, hi);
        }
        return;
    }
    if (u.out_state) {
        __syncthreads();
        if (tid < kDK) ehalf[e_slot(tid)] = exp2_fast(m_prev * kL2E);
        __syncthreads();
        last_factor(accS);
        __syncthreads();
        store_state(u.out_state, accS, stg, tid, w, lr, hi);
    }
}

// Segment p of sequence s under the plan: its token range [*beg, *beg + *len).
__device__ __forceinline__ void plan_range(int tb, int te, int T, int p, size_t *beg, int *len) {
    int sc, lc;
    plan_segment_chunks((te - tb + kC - 1) / kC, T, p, &sc, &lc);
    const int b = min(tb + sc * kC, te);
    *beg = (size_t)b;
    *len = min(tb + (sc + lc) * kC, te) - b;
}

// The plan's view of sequence s: token range, segments, and its units in launches A
// and C ([a0, a1), [c0, c1)).
struct PlanSeq {
    int tb, te, T, P, a0, a1, c0, c1;
};
__device__ __forceinline__ PlanSeq plan_seq(const FusedArgs &a, int s) {
    PlanSeq q;
    if (a.plan_tab) {
        const PlanTab t{a.plan_tab, a.n_seqs};
        q.tb = t.tb()[s];
        q.te = t.te()[s];
        q.T = t.T();
        q.P = plan_segments((q.te - q.tb + kC - 1) / kC, q.T);
        q.a0 = t.a_off()[s];
        q.a1 = t.a_off()[s + 1];
        q.c0 = t.c_off()[s];
        q.c1 = t.c_off()[s + 1];
    } else {
        q.tb = s * a.seq_len;
        q.te = q.tb + a.seq_len;
        q.T = a.plan_T;
        q.P = a.plan_P;
        const int ua = max(q.P - 1, 1);
        q.a0 = s * ua;
        q.a1 = q.a0 + ua;
        q.c0 = s * (q.P - 1);
        q.c1 = q.c0 + q.P - 1;
    }
    return q;
}

// The sequence that unit u of a launch belongs to: the last s with off[s] <= u (sequences
// without units in that launch have off[s] = off[s + 1] and are passed over).
__device__ __forceinline__ int plan_find(const int32_t *off, int n, int u) {
    int lo = 0, hi2 = n - 1;
    while (lo < hi2) {
        const int mid = (lo + hi2 + 1) >> 1;
        if (off[mid] <= u) lo = mid; else hi2 = mid - 1;
    }
    return lo;
}

template <int G, int kMode>
__global__ __launch_bounds__(kNT) void kda_fused_kernel(FusedArgs a) {
    const int H = a.H;
    const size_t DD = (size_t)kDK * kDV;
    if constexpr (kMode == kUsual) {
        // one workgroup per (sequence, head): equal lengths, or packed at the (clamped)
        // offsets cu_seqlens
        const int s = blockIdx.x / H, h = blockIdx.x % H;
        Unit u;
        u.h = h;
        u.T_len = a.seq_len;
        u.seq0 = (size_t)s * a.seq_len;
        if (a.cu_seqlens) {
            const int b0 = min(max(a.cu_seqlens[s], 0), a.T_total);
            const int b1 = min(max(a.cu_seqlens[s + 1], b0), a.T_total);
            u.T_len = b1 - b0;
            // an empty sequence runs no chunk; its first chunk's loads (issued before the
            // loop) then read row 0 of the batch, which exists, and are never used
            u.seq0 = u.T_len > 0 ? (size_t)b0 : 0;
        }
        u.h0src = a.h0 ? a.h0 + ((size_t)s * H + h) * DD : nullptr;
        u.out_state = a.hT ? a.hT + ((size_t)s * H + h) * DD : nullptr;
        u.map_out = nullptr;
        u.redo = a.redo + blockIdx.x;
        fused_body<G, kUsual>(a, u);
    } else if constexpr (kMode == kStrongPass) {
        // the whole pair again, from h0, if any of its units flagged it
        const int s = blockIdx.x / H, h = blockIdx.x % H;
        Unit u;
        u.h = h;
        bool any = false;
        if (a.plan_u > 0) {
            const PlanSeq q = plan_seq(a, s);
            for (int i = q.a0; i < q.a1; ++i) any |= a.redo[(size_t)i * H + h] != 0;
            for (int i = q.c0; i < q.c1; ++i) any |= a.redo[(size_t)(a.plan_u + i) * H + h] != 0;
            u.T_len = q.te - q.tb;
            u.seq0 = u.T_len > 0 ? (size_t)q.tb : 0;
        } else {
            any = a.redo[blockIdx.x] != 0;
            u.T_len = a.seq_len;
            u.seq0 = (size_t)s * a.seq_len;
            if (a.cu_seqlens) {
                const int b0 = min(max(a.cu_seqlens[s], 0), a.T_total);
                const int b1 = min(max(a.cu_seqlens[s + 1], b0), a.T_total);
                u.T_len = b1 - b0;
                u.seq0 = u.T_len > 0 ? (size_t)b0 : 0;
            }
        }
        if (!any) return;
        u.h0src = a.h0 ? a.h0 + ((size_t)s * H + h) * DD : nullptr;
        u.out_state = a.hT ? a.hT + ((size_t)s * H + h) * DD : nullptr;
        u.map_out = nullptr;
        u.redo = nullptr;
        fused_body<G, kStrongPass>(a, u);
    } else {
        // launch A (segment 0 of every sequence, the maps of its middle segments) or C
        // (segments 1 .. P - 1): unit ui of head h
        const int ui = blockIdx.x / H, h = blockIdx.x % H;
        int s, j;
        if (a.plan_tab) {
            const PlanTab t{a.plan_tab, a.n_seqs};
            const int32_t *off = kMode == kPlanA ? t.a_off() : t.c_off();
            if (ui >= off[a.n_seqs]) return;
            s = plan_find(off, a.n_seqs, ui);
            j = ui - off[s];
        } else {
            const int per = kMode == kPlanA ? max(a.plan_P - 1, 1) : a.plan_P - 1;
            if (per <= 0) return;
            s = ui / per;
            j = ui - s * per;
            if (s >= a.n_seqs) return;
        }
        const PlanSeq q = plan_seq(a, s);
        const int p = kMode == kPlanA ? j : j + 1;  // the segment
        Unit u;
        u.h = h;
        plan_range(q.tb, q.te, q.T, p, &u.seq0, &u.T_len);
        if (u.T_len <= 0) u.seq0 = 0;  // (an empty sequence: row 0 is read, never used)
        u.map_out = nullptr;
        u.redo = a.redo + (size_t)((kMode == kPlanA ? 0 : a.plan_u) + ui) * H + h;
        // slot of segment p >= 1: the state entering it, and its map
        auto slot = [&](int pp) { return (size_t)(q.c0 + pp - 1) * H + h; };
        float *hT_pair = a.hT ? a.hT + ((size_t)s * H + h) * DD : nullptr;
        if constexpr (kMode == kPlanC) {
            u.h0src = a.seg_state + slot(p) * DD;
            u.out_state = p == q.P - 1 ? hT_pair : nullptr;
            fused_body<G, kUsual>(a, u);
        } else {
            // (the condition is uniform and opaque to the compiler: otherwise it kept values
            // of one body live across the other, in scratch)
            int first = __builtin_amdgcn_readfirstlane(p == 0 ? 1 : 0);
            asm volatile("" : "+s"(first));
            if (first) {
                u.h0src = a.h0 ? a.h0 + ((size_t)s * H + h) * DD : nullptr;
                u.out_state = q.P == 1 ? hT_pair : a.seg_state + slot(1) * DD;
                fused_body<G, kUsual>(a, u);
            } else {
                u.h0src = nullptr;
                u.out_state = nullptr;
                u.map_out = a.seg_map + slot(p) * 2 * DD;
                fused_body<G, kMap>(a, u);
            }
        }
    }
}

}  // namespace

hipError_t launch_fused(const FusedArgs &a, int dk, int dv, bool bf16, int n_seqs, hipStream_t stream) {
    // the fused pass is built for bf16 input and d_k = d_v = 128 only
    if (!bf16 || dk != kDK || dv != kDV) return hipErrorInvalidValue;
    constexpr size_t smem = Lds::SIZE;
    // Without segments: the usual instance over the (sequence, head) pairs, then the strong
    // one over the pairs the first left to it. With segments: launch A (segment 0 of every
    // sequence and the maps of the middle segments), the composition of the maps, launch C
    // (segments 1 .. P - 1), then the strong instance over the (sequence, head) pairs any of
    // whose units was left to it. (Without a decay, no chunk can leave anything to it.)
    typedef void (*Kern)(FusedArgs);
    struct Set { Kern usual, strong, plan_a, plan_c; };
    auto set_of = [](auto gt) {
        constexpr int Gk = decltype(gt)::value;
        Set r{kda_fused_kernel<Gk, kUsual>, nullptr, kda_fused_kernel<Gk, kPlanA>, kda_fused_kernel<Gk, kPlanC>};
        if constexpr (Gk != kGateNone) r.strong = kda_fused_kernel<Gk, kStrongPass>;
        return r;
    };
    Set k;
    if (a.gate == kGateHead) k = set_of(IntTag<kGateHead>{});
    else if (a.gate == kGateNone) k = set_of(IntTag<kGateNone>{});
    else if (a.gate == kGatePreact && a.pre.qk_norm) k = set_of(IntTag<kGatePreactQK>{});
    else if (a.gate == kGatePreact) k = set_of(IntTag<kGatePreact>{});
    else k = set_of(IntTag<kGateChannel>{});
    auto go = [&](Kern kern, int grid) {
        hipError_t err = hipFuncSetAttribute(reinterpret_cast<const void *>(kern),
                                             hipFuncAttributeMaxDynamicSharedMemorySize, (int)smem);
        if (err != hipSuccess) return err;
        hipLaunchKernelGGL(kern, dim3(grid), dim3(kNT), smem, stream, a);
        return hipGetLastError();
    };
    hipError_t err;
    if (a.plan_u > 0) {
        if ((err = go(k.plan_a, a.plan_u * a.H)) != hipSuccess) return err;
        if (a.plan_tab || a.plan_P > 1) {  // (equal lengths in one segment each: nothing more)
            if ((err = launch_segment_chain(a, stream)) != hipSuccess) return err;
            if ((err = go(k.plan_c, a.plan_u * a.H)) != hipSuccess) return err;
        }
    } else {
        if ((err = go(k.usual, n_seqs * a.H)) != hipSuccess) return err;
    }
    if (k.strong && (err = go(k.strong, n_seqs * a.H)) != hipSuccess) return err;
    return hipSuccess;
}

}  // namespace kda
