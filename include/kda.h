/*
 * kda.h -- C ABI of libkda: the KDA (Kimi Delta Attention) gated delta rule on
 * AMD Instinct MI355X (gfx950).
 *
 * The operation, per (sequence, head), for t = 1..T:
 *
 *     S_t = (I - beta_t k_t k_t^T) Diag(alpha_t) S_{t-1} + beta_t k_t v_t^T
 *     o_t = S_t^T (scale * q_t),           alpha_t = exp(log_alpha_t) per key channel
 *
 * as written on the "ten questions" page (jokeuncle.github.io, Kimi K3 KDA math
 * for beginners: the closing symbol-by-symbol reading of the update; Q4 for the
 * readout o = S^T q, Q8 for Diag(alpha) acting on the rows of S), with the
 * d_k^{-1/2} query scale of the bra-ket derivation page (mynewscn.com, the KDA
 * state-update equations at its start). S is d_k x d_v, row i = key channel i.
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 *  - Every tensor argument is a caller-owned DEVICE pointer on the current HIP
 *    device, contiguous, 16-byte aligned. The library allocates nothing, never
 *    synchronises and never prints. Its only global state belongs to
 *    kda_chunk_fwd_noalloc: a fixed device array per GPU and its address.
 *  - Layouts are token-major: q, k [T_total, H, d_k]; v, o [T_total, H, d_v];
 *    log_alpha [T_total, H, d_k] fp32; beta [T_total, H] fp32; states
 *    [n_seqs, H, d_k, d_v] fp32 row-major (row = key channel).
 *  - `io` selects the dtype of q, k, v and o: KDA_F32 (float) or KDA_BF16
 *    (bfloat16). Gates, states and the workspace's fp32 parts are always fp32.
 *  - `stream` is a hipStream_t passed as void* (NULL = the null stream). All
 *    work is enqueued on it in order; the call returns before it runs.
 *  - Supported sizes: d_k, d_v in {64, 128}; chunk in {64, 128}; H >= 1;
 *    any T >= 0 (a ragged last chunk is handled).
 *  - Errors: arguments are validated on the host before anything is launched;
 *    on KDA_ERR_INVALID_ARG, KDA_ERR_UNSUPPORTED or KDA_ERR_WORKSPACE nothing is
 *    written and nothing is enqueued. KDA_ERR_HIP reports a failed launch.
 *    Device-side faults surface at the caller's next synchronisation. Input
 *    VALUES are not checked: gates must be finite (log_alpha <= 0 and beta in
 *    [0, 1] in the method's own use). The chunked prefill has no limit on how
 *    fast a channel forgets: it factors the in-chunk decay around the chunk's
 *    midpoint, whose factors e^(+-|sum|/2) stay in the fp32 range while a
 *    chunk's summed log_alpha is >= -160 on every key channel; a chunk below
 *    that is computed by a second instance of the kernels in which every
 *    exponent is <= 0 (the decay from the chunk's start, or from the end of a
 *    16-row block, and the pairs inside a block one by one), so factors that
 *    underflow are the negligible values they stand for. Tested at chunk sums
 *    near -500 and -2000 for every gate kind. On the fused pass (bf16,
 *    d_k = d_v = 128) such a chunk sends its whole (sequence, head) pair to the
 *    second instance, which runs it again from the start, one workgroup per
 *    pair. kda_chunk_bwd has no limit either: the (sequence, head) pairs holding
 *    such a chunk are recomputed token by token after its chunked pass.
 */
#ifndef KDA_H_
#define KDA_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define KDA_ABI_VERSION 6

typedef enum {
    KDA_OK = 0,
    KDA_ERR_INVALID_ARG = 1, /* NULL / misaligned pointer, negative or inconsistent size */
    KDA_ERR_UNSUPPORTED = 2, /* well-formed but unsupported: d_k, d_v, chunk or dtype */
    KDA_ERR_WORKSPACE = 3,   /* workspace missing, misaligned (256 B) or too small */
    KDA_ERR_HIP = 4          /* a HIP launch or runtime call failed */
} kda_status;

typedef enum { KDA_F32 = 0, KDA_BF16 = 1 } kda_dtype;

/*
 * Granularity of the decay, for the *_gated entry points. The essay "22,580:
 * from GPT-2 to Kimi K3" (yichencityu.github.io) builds the method in steps:
 * section 06, DeltaNet (the delta rule, no decay); section 08, Gated DeltaNet
 * (one data-dependent decay alpha_t in (0, 1] that scales the whole previous
 * state; alpha = 1 gives back the delta rule); section 9.1, KDA (a decay per
 * key channel). The recurrence above covers all three: a per-head decay is
 * the same alpha_t on every key channel, and none is alpha_t = 1.
 */
typedef enum {
    KDA_GATE_CHANNEL = 0, /* log_alpha [T_total, H, d_k] fp32, 16-byte aligned (KDA) */
    KDA_GATE_HEAD = 1,    /* log_alpha [T_total, H] fp32, 4-byte aligned: one decay per
                             token and head (Gated DeltaNet) */
    KDA_GATE_NONE = 2     /* no decay: log_alpha is not read and may be NULL (DeltaNet) */
} kda_gate;

/* KDA_ABI_VERSION of the built library. */
int kda_abi_version(void);

/* Static English text for a kda_status value ("unknown status" otherwise). */
const char *kda_status_string(int status);

/*
 * Workspace bytes kda_chunk_fwd needs for these sizes (0 when T == 0). For
 * packed variable-length input pass B = 1, T = total tokens and n_seqs = the
 * number of sequences; otherwise n_seqs is ignored. Returns 0 for unsupported
 * or invalid sizes as well, so check kda_chunk_fwd's status.
 */
size_t kda_chunk_fwd_workspace_bytes(int B, int T, int H, int d_k, int d_v, int chunk,
                                     int n_seqs, int io);

/*
 * kda_chunk_fwd -- chunked prefill ("chunked program"): o for every token and
 * the final state of every sequence.
 *
 * Method: the sequence is cut into chunks of `chunk` tokens (the essay
 * "22,580: from GPT-2 to Kimi K3", yichencityu.github.io, section 6.2: masked
 * attention inside a chunk, a recurrent state between chunks; section 6.3: the
 * WY reparametrisation that solves a chunk's delta corrections with one
 * unit-lower-triangular solve), extended with the per-channel decay of KDA
 * (the aidehub.top summary of the same essay, Gated DeltaNet section: a write
 * at one position read at a later one is decayed by the product of the alphas
 * in between). Chunking is an exact refactoring of the recurrence; results
 * differ from the token loop only by rounding.
 *
 * Arguments
 *   B, T        without cu_seqlens: B sequences of T tokens each, tensors
 *               [B, T, H, d] (the same memory as packed [B*T, H, d]).
 *   H, d_k, d_v heads and head dims.  io: kda_dtype.
 *   chunk       64 or 128: rows per chunk of the split pass (fp32, or d = 64).
 *               The fused pass (bf16, d_k = d_v = 128) works in chunks of 64
 *               rows for either value; since chunking is exact, only rounding
 *               differs. With fewer than 256 (sequence, head) pairs the fused
 *               pass cuts long sequences into segments sized so that two
 *               launches of at most one workgroup per compute unit cover them:
 *               segment 0 of every sequence together with the affine maps the
 *               middle segments apply to their entering states, the maps
 *               composed in order, then the other segments from their own
 *               entering states.
 *   q, k, v     [B*T, H, d_k|d_k|d_v], dtype io.
 *   log_alpha   [B*T, H, d_k] fp32, log of the per-channel decay (<= 0 normally).
 *   beta        [B*T, H] fp32, write strength.
 *   scale       query scale (callers normally pass d_k^{-1/2}).
 *   h0          [n_seq, H, d_k, d_v] fp32 initial states, or NULL for zeros.
 *               May alias hT (in-place carry).
 *   cu_seqlens  NULL, or device int32 [n_seqs + 1] offsets of packed sequences
 *               (then B must be 1): cu_seqlens[0] = 0, non-decreasing,
 *               cu_seqlens[n_seqs] = T. Values outside [0, T] are clamped on
 *               the device so that no access leaves the buffers.
 *   n_seqs      number of packed sequences (ignored when cu_seqlens is NULL;
 *               then n_seq = B).
 *   o           [B*T, H, d_v] dtype io, written for every token. Must not alias
 *               any input.
 *   hT          [n_seq, H, d_k, d_v] fp32 final states, or NULL to skip.
 *   workspace   device scratch of at least kda_chunk_fwd_workspace_bytes(...)
 *               bytes, 256-byte aligned; owned by the caller, contents
 *               undefined before and after. Two calls in flight at once need
 *               two workspaces.
 */
int kda_chunk_fwd(int B, int T, int H, int d_k, int d_v, int chunk, int io,
                  const void *q, const void *k, const void *v,
                  const float *log_alpha, const float *beta, float scale,
                  const float *h0, const int32_t *cu_seqlens, int n_seqs,
                  void *o, float *hT, void *workspace, size_t workspace_bytes, void *stream);

/*
 * kda_chunk_fwd_gated -- kda_chunk_fwd with the decay granularity `gate` (a
 * kda_gate value; any other value is KDA_ERR_INVALID_ARG). log_alpha's shape and
 * alignment follow kda_gate; with KDA_GATE_NONE it is not read. Every other
 * argument, the workspace size and the error behaviour are those of
 * kda_chunk_fwd, which is this call with KDA_GATE_CHANNEL.
 */
int kda_chunk_fwd_gated(int gate, int B, int T, int H, int d_k, int d_v, int chunk, int io,
                        const void *q, const void *k, const void *v,
                        const float *log_alpha, const float *beta, float scale,
                        const float *h0, const int32_t *cu_seqlens, int n_seqs,
                        void *o, float *hT, void *workspace, size_t workspace_bytes,
                        void *stream);

/*
 * kda_chunk_fwd_noalloc -- kda_chunk_fwd_gated without a workspace argument, for callers
 * that cannot allocate device memory: code under HIP graph capture, tight serving loops,
 * harnesses that forbid allocation. The library allocates nothing here either: the
 * workspace is a fixed device array of KDA_NOALLOC_MAX_WORKSPACE bytes inside the
 * library, one per GPU, held until the process ends.
 *
 * Arguments, results and errors are those of kda_chunk_fwd_gated. In addition, sizes whose
 * workspace (kda_chunk_fwd_workspace_bytes) exceeds KDA_NOALLOC_MAX_WORKSPACE are
 * rejected with KDA_ERR_WORKSPACE before anything is enqueued. The fused pass (bf16,
 * d_k = d_v = 128) with at least 256 (sequence, head) pairs needs 256 bytes plus one per
 * pair, so all such calls fit; with fewer pairs it cuts long sequences into segments and
 * needs 192 KB per (segment, head) after each sequence's first, which fits up to about 170
 * of them (a sequence of fewer than 512 tokens is never cut, and at most 256 // H
 * segments per head are used); split-pass calls
 * (fp32 or d = 64) fit up to about 25,000 to 30,000 token-heads at d = 128. The first call
 * on a device looks up the array's device address (KDA_ERR_HIP if that fails).
 *
 * All calls on one GPU share the array: calls whose work overlaps in time on one GPU
 * (other streams, other host threads) race and give undefined results. Calls in order on
 * one stream are safe. The array keeps the last call's contents; no call reads what an
 * earlier one left.
 */
#define KDA_NOALLOC_MAX_WORKSPACE ((size_t)32 << 20)

int kda_chunk_fwd_noalloc(int gate, int B, int T, int H, int d_k, int d_v, int chunk, int io,
                          const void *q, const void *k, const void *v,
                          const float *log_alpha, const float *beta, float scale,
                          const float *h0, const int32_t *cu_seqlens, int n_seqs,
                          void *o, float *hT, void *stream);

/*
 * kda_chunk_fwd_preact -- kda_chunk_fwd with the gates formed inside the kernels
 * from their pre-activations, as the gate line of KDA's open-source layer that
 * the "ten questions" page quotes (jokeuncle.github.io, Kimi K3 KDA math for
 * beginners, Q9: g = -exp(A_log) softplus(f(x) + dt_bias), alpha = e^g, and beta
 * through a sigmoid):
 *
 *     log_alpha[t, h, c] = -exp(A_log[h]) * softplus(a[t, h, c] + dt_bias[h, c])
 *     beta[t, h]         = sigmoid(b[t, h])
 *
 * so the decay is read in the io dtype (half the bytes of fp32 log_alpha in bf16)
 * and no separate pass forms it. softplus(x) = log(1 + e^x), sigmoid(x) =
 * 1 / (1 + e^-x).
 *
 * With KDA_PREACT_QK_NORM in `flags`, q and k are given before their activation
 * and normalisation too, and each row is formed as the delta-rule layer of the
 * essay "22,580: from GPT-2 to Kimi K3" (section 5.2's forward) writes it:
 * x -> silu(x) / max(||silu(x)||_2, 1e-12) over the head dimension, silu(x) =
 * x sigmoid(x). Other flag bits are KDA_ERR_INVALID_ARG.
 *
 * Arguments (others as kda_chunk_fwd; the workspace size is the same):
 *   a        [B*T, H, d_k] dtype io, 16-byte aligned: the decay's pre-activation.
 *   A_log    [H] fp32: per-head log of the decay rate's scale.
 *   dt_bias  [H, d_k] fp32, 16-byte aligned: per-channel bias.
 *   b        [B*T, H] fp32: beta's pre-activation.
 * Chunks whose formed decay sums below -160 are handled as for kda_chunk_fwd.
 */
enum { KDA_PREACT_QK_NORM = 1 };

int kda_chunk_fwd_preact(int flags, int B, int T, int H, int d_k, int d_v, int chunk, int io,
                         const void *q, const void *k, const void *v,
                         const void *a, const float *A_log, const float *dt_bias, const float *b,
                         float scale, const float *h0, const int32_t *cu_seqlens, int n_seqs,
                         void *o, float *hT, void *workspace, size_t workspace_bytes, void *stream);

/*
 * kda_recurrent_step -- one decode step ("recurrent program") for N sequences:
 * every (sequence, head) state is read once and written once, in place.
 *
 * Method: the step in the order of the bra-ket derivation page (mynewscn.com,
 * the KDA state-update equations at its start), in the d_k x d_v orientation:
 * S~ = Diag(alpha) S; e = beta (v - S~^T k); S <- S~ + k e^T;
 * o = scale (S~^T q + (k . q) e), which equals S_t^T (scale q).
 *
 * Arguments
 *   N, H, d_k, d_v, io   as above (d_k, d_v in {64, 128}).
 *   q, k        [N, H, d_k] dtype io;  v, o [N, H, d_v] dtype io.
 *   log_alpha   [N, H, d_k] fp32;  beta [N, H] fp32;  scale as above.
 *   state       [N, H, d_k, d_v] fp32, updated in place. Must not alias o.
 */
int kda_recurrent_step(int N, int H, int d_k, int d_v, int io,
                       const void *q, const void *k, const void *v,
                       const float *log_alpha, const float *beta, float scale,
                       float *state, void *o, void *stream);

/*
 * kda_recurrent_step_gated -- kda_recurrent_step with the decay granularity
 * `gate`: log_alpha [N, H, d_k] (KDA_GATE_CHANNEL), [N, H] (KDA_GATE_HEAD), or not
 * read (KDA_GATE_NONE). kda_recurrent_step is this call with KDA_GATE_CHANNEL.
 */
int kda_recurrent_step_gated(int gate, int N, int H, int d_k, int d_v, int io,
                             const void *q, const void *k, const void *v,
                             const float *log_alpha, const float *beta, float scale,
                             float *state, void *o, void *stream);

/*
 * kda_recurrent_step_preact -- kda_recurrent_step with the gates formed from
 * pre-activations as in kda_chunk_fwd_preact: a [N, H, d_k] dtype io, A_log [H],
 * dt_bias [H, d_k], b [N, H] fp32; `flags` as there.
 */
int kda_recurrent_step_preact(int flags, int N, int H, int d_k, int d_v, int io,
                              const void *q, const void *k, const void *v,
                              const void *a, const float *A_log, const float *dt_bias, const float *b,
                              float scale, float *state, void *o, void *stream);

/*
 * kda_chunk_bwd -- the backward pass of kda_chunk_fwd: the gradients of a loss
 * with respect to q, k, v, log_alpha, beta and h0, given its gradients with
 * respect to o (dout) and to the final state (dhT).
 *
 * The pages derive no gradient (the essay "22,580: from GPT-2 to Kimi K3" notes
 * that training runs the chunked form of sections 6.2-6.3); this is the exact
 * reverse-mode derivative of the recurrence at the top of this header, computed
 * chunk by chunk: the chunk-local forward quantities, the chunk-start states in
 * order, the state gradients in reverse order, then the chunk-local gradients.
 *
 * Two implementations: bf16 I/O with d_k = d_v = 128 runs the matrix-core pass (the
 * forward's chunk preparation and state recursion, recording the state entering every
 * chunk; the state gradients in reverse; one fused kernel per (chunk, head) for the
 * chunk-local gradients), whose products take bf16 operands with fp32 accumulation as
 * the forward's bf16 passes do; every other case runs the direct pass, all arithmetic
 * fp32. Both add every sum in a fixed order: repeated calls give the same bits.
 *
 * Both factor the decay inside a chunk around the chunk's midpoint, which holds while a
 * chunk's summed log_alpha is >= -160 on every key channel. After either pass, the
 * (sequence, head) pairs holding a chunk below that are recomputed token by token (fp32
 * arithmetic, every decay applied as alpha = exp(log_alpha) <= 1): the exact reverse mode
 * of the recurrence, with the states recomputed from checkpoints (one per 64 tokens, then
 * one per 4 tokens of the block being reversed). This pass is sequential over the tokens of
 * a pair (about 7 us per token on one MI355X compute unit) and runs on as many pairs at once
 * as its share of the workspace holds checkpoints for (at most 512 MiB, at least one pair at
 * a time); calls without such chunks spend only the check on it.
 *
 * Arguments
 *   B, T, H, d_k, d_v   equal-length sequences [B, T, H, d] (packed sequences:
 *               kda_chunk_bwd_varlen); d_k, d_v in {64, 128}; B, H <= 65535.
 *   chunk       64.   io   dtype of q, k, v, dout and dq, dk, dv (KDA_F32 or KDA_BF16);
 *               gates, states and their gradients are fp32.
 *   q, k, v, log_alpha, beta, scale, h0   the forward call's inputs (h0 NULL =
 *               zero initial state).
 *   dout        [B, T, H, d_v] dtype io, the gradient with respect to o.
 *   dhT         [B, H, d_k, d_v] fp32 or NULL (zero): with respect to hT.
 *   dq, dk      [B, T, H, d_k], dv [B, T, H, d_v]: dtype io;  dlog_alpha [B, T, H, d_k]
 *               and dbeta [B, T, H]: fp32. Written, none overlapping any argument.
 *   dh0         [B, H, d_k, d_v] fp32 or NULL (not computed).
 *   workspace   kda_chunk_bwd_workspace_bytes(...) bytes, 256-byte aligned: on the
 *               matrix-core pass about 170 KB per (chunk, head) (the forward's chunk
 *               quantities and four bf16 matrices); on the direct pass about 300 KB per
 *               (chunk, head) at d = 128 plus a fixed scratch of at most 1024 x 770 KB;
 *               on both, the token pass's checkpoints: (ceil(T / 64) + 16) d_k d_v fp32
 *               per pair it runs at once, within 512 MiB.
 * Gate values: any finite log_alpha (<= 0 in the method's use) and beta. Errors as for
 * the other entry points.
 */
size_t kda_chunk_bwd_workspace_bytes(int B, int T, int H, int d_k, int d_v, int chunk, int io);

int kda_chunk_bwd(int B, int T, int H, int d_k, int d_v, int chunk, int io,
                  const void *q, const void *k, const void *v,
                  const float *log_alpha, const float *beta, float scale,
                  const float *h0, const void *dout, const float *dhT,
                  void *dq, void *dk, void *dv, float *dlog_alpha, float *dbeta, float *dh0,
                  void *workspace, size_t workspace_bytes, void *stream);

/*
 * kda_chunk_bwd_varlen -- kda_chunk_bwd for packed variable-length sequences, the
 * layout of kda_chunk_fwd with cu_seqlens: q, k, dq, dk, log_alpha, dlog_alpha
 * [T, H, d_k]; v, dout, dv [T, H, d_v]; beta, dbeta [T, H]; h0, dhT, dh0
 * [n_seqs, H, d_k, d_v] (h0, dhT NULL = zero; dh0 NULL = not computed). cu_seqlens is
 * a device int32 [n_seqs + 1] table with the meaning, and the clamping of malformed
 * values, of kda_chunk_fwd's; n_seqs >= 1.
 *
 * Served by the matrix-core pass: io = KDA_BF16, d_k = d_v = 128, chunk 64; any other
 * size returns KDA_ERR_UNSUPPORTED. Workspace: kda_chunk_bwd_varlen_workspace_bytes
 * (sized for up to ceil(T / 64) + n_seqs chunks). Empty sequences give dh0 = dhT.
 * Everything else as kda_chunk_bwd.
 */
size_t kda_chunk_bwd_varlen_workspace_bytes(int T, int H, int d_k, int d_v, int chunk, int n_seqs, int io);

int kda_chunk_bwd_varlen(int T, int H, int d_k, int d_v, int chunk, int io,
                         const void *q, const void *k, const void *v,
                         const float *log_alpha, const float *beta, float scale,
                         const float *h0, const int32_t *cu_seqlens, int n_seqs,
                         const void *dout, const float *dhT,
                         void *dq, void *dk, void *dv, float *dlog_alpha, float *dbeta, float *dh0,
                         void *workspace, size_t workspace_bytes, void *stream);

/*
 * Full-attention decode over a KV cache: the comparator of the decode step
 * -----------------------------------------------------------------------
 * The step that a softmax-attention layer takes for each new token, against
 * which kda_recurrent_step is measured. The essay "22,580: from GPT-2 to Kimi
 * K3" defines causal softmax attention in section 2.2 and the KV cache in
 * section 2.3: at decode time the keys and values of all earlier positions are
 * kept, and the new token's query is compared with every one of them. The "ten
 * questions" page (Q10) counts the cost: the cache grows by one key and one
 * value per token and per head, and every decode step reads all of it, while
 * KDA keeps one d_k x d_v state per head.
 *
 *   o[b, h] = sum_{t < len_b} w_t v_cache[b, j, t],
 *   w_t = exp(s_t) / sum_{t' < len_b} exp(s_t'),  s_t = scale q[b, h] . k_cache[b, j, t],
 *   j = h / (H / H_kv)   (consecutive query heads share a cached head; H_kv = H
 *                         is multi-head attention)
 *
 * Arguments
 *   B, H, H_kv  sequences, query heads, cached heads; H % H_kv == 0 and
 *               H / H_kv in {1, 2, 4, 8}; B <= 65535, H_kv <= 65535.
 *   d           head dimension, 64 or 128 (queries, keys and values).
 *   T_max       rows allocated per cached head; T_max * d < 2^31.
 *   io          dtype of q, the caches and o (KDA_F32 or KDA_BF16).
 *   q           [B, H, d];  o [B, H, d] (must not overlap any input).
 *   k_cache, v_cache  [B, H_kv, T_max, d], row t of a head = position t. The
 *               new token's key and value are expected in the cache already
 *               (row len_b - 1): the query attends to itself.
 *   seq_lens    [B] int32, rows in use per sequence (len_b), or NULL for
 *               T_max everywhere. Values are clamped to [0, T_max]; rows at
 *               and past len_b are never read. len_b = 0 gives o = 0.
 *   scale       the score scale (d^{-1/2} for the usual attention).
 *   workspace   kda_attn_decode_workspace_bytes(B, H, H_kv, d, T_max, io)
 *               bytes, 256-byte aligned (NULL allowed when that is 0): the
 *               partial results when a cache is split over several workgroups.
 * Scores are formed in fp32 with the usual running-maximum rescaling, so any
 * finite scores are safe. Errors as for the other entry points.
 */
size_t kda_attn_decode_workspace_bytes(int B, int H, int H_kv, int d, int T_max, int io);

int kda_attn_decode(int B, int H, int H_kv, int d, int T_max, int io,
                    const void *q, const void *k_cache, const void *v_cache,
                    const int32_t *seq_lens, float scale, void *o,
                    void *workspace, size_t workspace_bytes, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* KDA_H_ */
