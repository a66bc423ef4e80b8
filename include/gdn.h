/*
 * gdn.h -- C ABI of the MI355X (gfx950) gated-delta-rule token mixer library
 * (libgdn.so).
 *
 * The operation is the gated delta rule of the "Delta-rule layers" row of the
 * Architecture table on the "Agnes-3.0-Flash" model card (ModelScope): 16 key
 * heads shared by 48 value heads, head dim 128, a kernel-4 causal conv in
 * front, a gated RMS-norm after, and an fp32 recurrent state.  The rule itself
 * (the "erase, then write" update with a forget gate described in the
 * explanatory paragraph on the Gated Delta Rule that follows the
 * "Feed-Forward and Positional Encoding" section of "Agnes-3.0-Flash Deep
 * Dive: A 33B Hybrid-Attention Multimodal Model") is, per value head h with key head
 * kh = h / (Hv / Hk):
 *
 *     S_t = S_{t-1} * alpha_t (I - beta_t k_t k_t^T) + beta_t v_t k_t^T
 *     o_t = scale * S_t q_t,        alpha_t = exp(g_t)
 *
 * S is dv x dk with the VALUE channel as row index (S k is a value vector).
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 *  - All tensor pointers are DEVICE pointers, owned by the caller.  The library
 *    allocates no device memory (scratch space comes from the caller's
 *    workspace, or for gdn_chunk_fwd_noalloc from a fixed static device array)
 *    and keeps no pointer after returning.  Its other state: a thread-local
 *    error string, and per device, made on first need and kept until the
 *    process ends, one extra HIP stream and two events (the overlapped
 *    prefill of gdn_chunk_fwd).
 *  - bf16 tensors travel as uint16_t bit patterns.
 *  - Strides are in elements; the innermost (head-dim) dimension is contiguous.
 *  - `stream` is a hipStream_t (NULL = the default stream).  Work is enqueued
 *    asynchronously; no call synchronises the host unless stated.
 *  - Argument errors are detected before anything is enqueued: a negative
 *    status is returned and no output is touched.  Launch failures return
 *    GDN_ERR_HIP with detail text in gdn_last_error().  Device faults surface
 *    at the caller's next synchronisation, as usual for HIP.
 *  - Data pointers of tensors with no elements (T_total == 0, n_seqs == 0,
 *    rows == 0) may be NULL.
 *  - Supported domain: head dim 128 (dk = dv = 128), Hv % Hk == 0.
 *  - Matrix products inside the prefill kernels take fp16 operands with fp32
 *    accumulation.  q and k convert from bf16 exactly for components of
 *    magnitude 2^-17 or more (bf16's 8 significant bits fit fp16's, down to
 *    its subnormal step 2^-24); smaller components round to a multiple of
 *    2^-24.  The state S0 at chunk starts and the per-chunk products built from
 *    v (b v - b gamma K S0^T, the solve's U, the decayed U) are rounded to
 *    fp16 too: they must stay below 65504 in magnitude, and lose relative
 *    precision where most of them fall under 2^-14 (fp16 subnormals).  The
 *    accuracy bar is tested with v ~ N(0, s^2) and S0 ~ N(0, (0.02 s)^2) for
 *    s = 2^-12 .. 2^8, and with |v| ~ 200 outliers among N(0, 1) values; the
 *    rule is linear in (S0, v), so inputs outside that range can be scaled by
 *    a power of two (exact) and the results scaled back.  The conv front's L2
 *    normalisation keeps q and k at unit norm.
 */
#ifndef GDN_H
#define GDN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef int32_t gdn_status;

#define GDN_OK 0
#define GDN_ERR_NULL (-1)        /* a required pointer is NULL                        */
#define GDN_ERR_SHAPE (-2)       /* a size, stride or head count is invalid           */
#define GDN_ERR_UNSUPPORTED (-3) /* valid but outside the supported domain (e.g. d)   */
#define GDN_ERR_WORKSPACE (-4)   /* workspace NULL or smaller than required          */
#define GDN_ERR_ALIAS (-5)       /* an input overlaps an output it must not overlap   */
#define GDN_ERR_HIP (-6)         /* the HIP runtime reported an error                 */
#define GDN_ERR_SEQLENS (-7)     /* cu_seqlens failed the opt-in host validation      */

#define GDN_ABI_VERSION 8

/* Human-readable name of a status code (static storage). */
const char* gdn_status_string(gdn_status s);

/* Detail text of the last failure on the calling thread (empty if none). */
const char* gdn_last_error(void);

/* GDN_ABI_VERSION of the built library. */
int32_t gdn_abi_version(void);

/*
 * gdn_conv1d_fwd -- causal depthwise conv (kernel 4) + SiLU + per-head L2 norm.
 *
 * The "causal conv (kernel 4) in front" of the "Delta-rule layers" row of the
 * model card's Architecture table, applied to the projected q|k|v channels:
 *
 *     y[t][c] = silu( sum_{i=0..3} w[c][i] * x[t-3+i][c]  + bias[c] )
 *
 * where x before the start of a sequence is read from that sequence's
 * conv_state (oldest first) or is zero when conv_state is NULL.  Then every
 * head of head_dim channels among the first n_l2_heads heads is normalised:
 *     y <- y / sqrt(sum y^2 + l2_eps)
 * Arithmetic is fp32; y is rounded to bf16 (nearest, ties to even).
 *
 *   x          [T_total, C] bf16, row stride x_row_stride (>= C)
 *   w          [C, 4] bf16; w[c][3] multiplies the current token
 *   bias       [C] fp32 or NULL
 *   y          [T_total, C] bf16, row stride y_row_stride (>= C); must not
 *              overlap x
 *   conv_state [n_seqs, C, 3] bf16 or NULL.  In: the three inputs preceding
 *              each sequence, oldest first.  Out (in place): the last three
 *              inputs of (old state ++ sequence); an empty sequence keeps it.
 *   cu_seqlens [n_seqs + 1] int32 device array or NULL.  NULL means n_seqs
 *              sequences of T_total / n_seqs tokens each (T_total % n_seqs == 0;
 *              decode is T_total == n_seqs).  Precondition: cu[0] = 0,
 *              non-decreasing, cu[n_seqs] = T_total (checked only by
 *              gdn_validate_cu_seqlens or when GDN_VALIDATE_CU_SEQLENS=1).
 *   n_l2_heads heads [0, n_l2_heads) of head_dim channels are L2-normalised
 *              (32 for the layer: 16 q heads then 16 k heads).
 *   head_dim   must be 128.  C must be a multiple of 8.
 */
gdn_status gdn_conv1d_fwd(const uint16_t* x, int64_t x_row_stride, const uint16_t* w,
                          const float* bias, uint16_t* y, int64_t y_row_stride,
                          uint16_t* conv_state, const int32_t* cu_seqlens, int32_t n_seqs,
                          int32_t T_total, int32_t C, int32_t n_l2_heads, int32_t head_dim,
                          float l2_eps, void* stream);

/*
 * gdn_chunk_fwd -- chunked prefill of the rule over packed sequences.
 *
 * Computes exactly the sequential rule above for every token of every
 * sequence (the state restarts at each sequence start from its initial state),
 * organised in chunks of 64 tokens with the WY / UT form inside each chunk.
 *
 *   q, k           [T_total, Hk, dk] bf16, token strides q_tok_stride,
 *                  k_tok_stride (>= Hk * dk)
 *   v              [T_total, Hv, dv] bf16, token stride v_tok_stride (>= Hv * dv)
 *   g, beta        [T_total, Hv] fp32, contiguous (alpha = exp(g))
 *   o              [T_total, Hv, dv] fp32, contiguous; must not overlap q, k, v
 *   initial_state  [n_seqs, Hv, dv, dk] fp32 or NULL (zeros)
 *   final_state    [n_seqs, Hv, dv, dk] fp32 or NULL; may be the same buffer as
 *                  initial_state (each block reads its slice before writing it)
 *   cu_seqlens     [n_seqs + 1] int32 device array or NULL (n_seqs equal
 *                  sequences, T_total % n_seqs == 0); same precondition as above
 *   scale          multiplies o (1.0 for the plain rule)
 *   workspace      device scratch of at least gdn_chunk_fwd_workspace_bytes()
 *                  bytes, 256-byte aligned (may be NULL only when n_seqs == 0),
 *                  not overlapping any tensor.  Per call it receives the chunk
 *                  map (as gdn_chunk_map), then the state-independent part of
 *                  every chunk (fp16 K rows and Q, -A, the inverted diagonal
 *                  blocks of I + A, the masked decayed Q K^T and the decay
 *                  tables, mostly in MFMA fragment order), which the
 *                  sequential scan then reads.  About 17.9 KB per token for
 *                  16 key / 48 value heads; sequences of 32768 tokens or more
 *                  (T_total / n_seqs) add n_seqs * Hv * dv * dk * 4 bytes for
 *                  the state carried between segments (below).  Contents are
 *                  scratch: nothing is kept across calls.
 *
 * Overlapped launch: with equal lengths of at least 32768 tokens, no
 * cu_seqlens and a scan that leaves 32 or more compute units idle (n_seqs = 1
 * at 16/48 heads), the call runs in 16384-token segments.  The state-
 * independent part of segment i + 1 is computed on the library's second
 * stream of the device, on the idle units, while the scan of segment i runs
 * on `stream`; `stream` waits for that work before each later segment's scan,
 * so the caller sees ordinary stream order (work enqueued on `stream` after
 * the call starts after all of it).  Results are bit-identical to the one-
 * pass launch.  Concurrent calls on one device serialise their enqueueing.
 */
size_t gdn_chunk_fwd_workspace_bytes(int32_t n_seqs, int32_t T_total, int32_t Hk, int32_t Hv,
                                     int32_t d);

gdn_status gdn_chunk_fwd(const uint16_t* q, int64_t q_tok_stride, const uint16_t* k,
                         int64_t k_tok_stride, const uint16_t* v, int64_t v_tok_stride,
                         const float* g, const float* beta, float* o,
                         const float* initial_state, float* final_state,
                         const int32_t* cu_seqlens, int32_t n_seqs, int32_t T_total, int32_t Hk,
                         int32_t Hv, int32_t dk, int32_t dv, float scale, void* workspace,
                         size_t workspace_bytes, void* stream);

/*
 * gdn_chunk_fwd_noalloc -- gdn_chunk_fwd for callers that cannot allocate
 * device memory or hand over a workspace: code under HIP graph capture,
 * tight serving loops, harnesses that forbid hipMalloc.  Same arguments,
 * result and errors as gdn_chunk_fwd, without the workspace arguments; the
 * call allocates nothing (no hipMalloc, hipFree or allocating library call).
 * The workspace is instead a static 64 MiB device array of the library, one
 * copy per GPU, held from the library's load until the process ends:
 *   - the call is rejected with GDN_ERR_WORKSPACE when
 *     gdn_chunk_fwd_workspace_bytes(n_seqs, T_total, Hk, Hv, dk) exceeds
 *     64 MiB (about 3,700 tokens at 16 key / 48 value heads);
 *   - every call on one GPU uses that GPU's array, which keeps the last
 *     call's contents (each call overwrites what it reads; nothing has to
 *     start at zero), so calls that may run concurrently on one GPU (several
 *     streams or host threads) race and must be ordered by the caller;
 *   - the first call on a device looks the array's device address up
 *     (hipGetSymbolAddress) with that device current; argument errors are
 *     found before that, as for gdn_chunk_fwd.
 */
gdn_status gdn_chunk_fwd_noalloc(const uint16_t* q, int64_t q_tok_stride, const uint16_t* k,
                                 int64_t k_tok_stride, const uint16_t* v, int64_t v_tok_stride,
                                 const float* g, const float* beta, float* o,
                                 const float* initial_state, float* final_state,
                                 const int32_t* cu_seqlens, int32_t n_seqs, int32_t T_total,
                                 int32_t Hk, int32_t Hv, int32_t dk, int32_t dv, float scale,
                                 void* stream);

/*
 * gdn_chunk_fwd_bf16o -- gdn_chunk_fwd with o written as bf16 (each element
 * the fp32 result rounded to nearest, ties to even): half the output bytes.
 * o is [T_total, Hv, dv] bf16, contiguous, 16-byte aligned; every other
 * argument, the states and the errors are as for gdn_chunk_fwd.
 */
gdn_status gdn_chunk_fwd_bf16o(const uint16_t* q, int64_t q_tok_stride, const uint16_t* k,
                               int64_t k_tok_stride, const uint16_t* v, int64_t v_tok_stride,
                               const float* g, const float* beta, uint16_t* o,
                               const float* initial_state, float* final_state,
                               const int32_t* cu_seqlens, int32_t n_seqs, int32_t T_total,
                               int32_t Hk, int32_t Hv, int32_t dk, int32_t dv, float scale,
                               void* workspace, size_t workspace_bytes, void* stream);

/*
 * gdn_chunk_fwd_pooled -- gdn_chunk_fwd for sequences that continue from, and
 * return to, a pool of per-sequence states (continuous batching: one call may
 * mix long prefills with sequences of one or a few new tokens), as serving
 * many concurrent requests needs (the model card's Hardware Requirements
 * table); the rule is that of gdn_chunk_fwd.
 *   state       [n_slots, Hv, dv, dk] fp32, 16-byte aligned, read and written
 *               in place: sequence n starts from state[state_slot[n]] and
 *               leaves its final state there; an empty sequence leaves its
 *               slot unchanged; slots not named are not touched
 *   state_slot  [n_seqs] int32 device array, required when n_seqs > 0; the
 *               slots in [0, n_slots) must be distinct; a slot outside
 *               [0, n_slots) (say -1) marks a padding sequence: no state is
 *               read or written for it and its rows of o are not written
 *   o           [T_total, Hv, dv] fp32 (o_is_bf16 == 0) or bf16 (as
 *               gdn_chunk_fwd_bf16o), must not overlap the state pool
 * Every other argument, the workspace and the errors as for gdn_chunk_fwd.
 */
gdn_status gdn_chunk_fwd_pooled(const uint16_t* q, int64_t q_tok_stride, const uint16_t* k,
                                int64_t k_tok_stride, const uint16_t* v, int64_t v_tok_stride,
                                const float* g, const float* beta, void* o, int32_t o_is_bf16,
                                float* state, const int32_t* state_slot, int32_t n_slots,
                                const int32_t* cu_seqlens, int32_t n_seqs, int32_t T_total,
                                int32_t Hk, int32_t Hv, int32_t dk, int32_t dv, float scale,
                                void* workspace, size_t workspace_bytes, void* stream);

/*
 * gdn_chunk_fwd_gated -- gdn_chunk_fwd with the gates formed inside the prep
 * kernel from the per-head projections instead of read as g and beta.  The
 * Deep Dive article's paragraph on the Gated Delta Rule names a forget gate
 * without its form; the form taken is a per-head decay rate times a
 * data-dependent softplus step, and a sigmoid write strength:
 *     g[t][h]    = -exp(A_log[h]) * softplus(a[t][h] + dt_bias[h])
 *     beta[t][h] = sigmoid(b[t][h])
 * (fp32 arithmetic on the bf16 inputs).
 *   a, b         [T_total, Hv] bf16 with token strides a_tok_stride,
 *                b_tok_stride (elements, >= Hv), 2-byte aligned; may be
 *                columns of a wider projection output
 *   A_log, dt_bias  [Hv] fp32
 * Every other argument, the workspace and the errors as for gdn_chunk_fwd.
 */
gdn_status gdn_chunk_fwd_gated(const uint16_t* q, int64_t q_tok_stride, const uint16_t* k,
                               int64_t k_tok_stride, const uint16_t* v, int64_t v_tok_stride,
                               const uint16_t* a, int64_t a_tok_stride, const uint16_t* b,
                               int64_t b_tok_stride, const float* A_log, const float* dt_bias,
                               float* o, const float* initial_state, float* final_state,
                               const int32_t* cu_seqlens, int32_t n_seqs, int32_t T_total,
                               int32_t Hk, int32_t Hv, int32_t dk, int32_t dv, float scale,
                               void* workspace, size_t workspace_bytes, void* stream);

/*
 * gdn_mixer_fwd -- the whole token mixer over a prefill in one call (the
 * "Delta-rule layers" row of the model card's Architecture table: causal
 * conv in front, the rule, gated RMS-norm after).  The causal conv (kernel 4)
 * + SiLU + per-head L2 of q and k runs inside the chunk-prep kernel and the
 * conv + SiLU of v inside the scan kernel, so no conv output goes to HBM;
 * then the conv-window update and the gated RMSNorm.  The result equals gdn_conv1d_fwd -> gdn_chunk_fwd ->
 * gdn_gated_rmsnorm on the same inputs bit for bit (same operations in the
 * same order).
 *   x           [T_total, C] bf16 pre-conv rows [q | k | v], C = (2 Hk + Hv) d,
 *               row stride x_stride (>= C, a multiple of 8)
 *   conv_w      [C, 4] bf16, tap 3 = the current token; conv_bias [C] fp32 or NULL
 *   conv_state  [n_seqs, C, 3] bf16 or NULL: the inputs before each sequence
 *               (oldest first), replaced by each sequence's last three
 *   g, beta     [T_total, Hv] fp32, or both NULL and the gates formed from
 *               the projections as in gdn_chunk_fwd_gated: a, b [T_total, Hv]
 *               bf16 (token strides a_stride, b_stride >= Hv), A_log, dt_bias
 *               [Hv] fp32 (pass NULL for these when g, beta are given)
 *   z           [T_total, Hv, d] bf16 gate input, row stride z_stride (>= Hv d,
 *               a multiple of 8); norm_w [d] fp32
 *   out         [T_total, Hv, d] fp32 (out_is_bf16 == 0) or bf16, contiguous;
 *               overlaps no other buffer
 *   initial_state, final_state, cu_seqlens, n_seqs, scale: as gdn_chunk_fwd
 *   state_slot  [n_seqs] int32 device array or NULL.  With it, states and conv
 *               windows are pools of n_slots rows updated in place (serving):
 *               initial_state == final_state = [n_slots, Hv, d, d] and
 *               conv_state [n_slots, C, 3]; sequence n uses row
 *               state_slot[n] of both (slots in [0, n_slots) distinct), other
 *               rows are not touched.  A slot outside [0, n_slots) (say -1)
 *               marks a padding sequence: no state or conv-window row is read
 *               or written for it (its conv history is taken as zeros) and its
 *               rows of out are unspecified
 *   l2_eps, norm_eps  the L2 and RMS epsilons (finite, >= 0)
 *   workspace   gdn_mixer_fwd_workspace_bytes() bytes, 256-byte aligned: the
 *               prefill workspace and, for bf16 out, the fp32 o
 * Every pointer 16-byte aligned except g, beta, A_log, dt_bias and
 * cu_seqlens (4 bytes) and a, b (2 bytes).
 * d = 128.  Errors as for gdn_chunk_fwd.
 */
size_t gdn_mixer_fwd_workspace_bytes(int32_t n_seqs, int32_t T_total, int32_t Hk, int32_t Hv,
                                     int32_t d, int32_t out_is_bf16);

gdn_status gdn_mixer_fwd(const uint16_t* x, int64_t x_stride, const uint16_t* conv_w,
                         const float* conv_bias, uint16_t* conv_state, const float* g,
                         const float* beta, const uint16_t* a, int64_t a_stride, const uint16_t* b,
                         int64_t b_stride, const float* A_log, const float* dt_bias,
                         const uint16_t* z, int64_t z_stride,
                         const float* norm_w, void* out, int32_t out_is_bf16,
                         const float* initial_state, float* final_state,
                         const int32_t* state_slot, int32_t n_slots,
                         const int32_t* cu_seqlens, int32_t n_seqs, int32_t T_total, int32_t Hk,
                         int32_t Hv, int32_t d, float scale, float l2_eps, float norm_eps,
                         void* workspace, size_t workspace_bytes, void* stream);

/*
 * gdn_chunk_map -- the varlen chunk map used by gdn_chunk_fwd, exposed so its
 * integer results can be checked bit for bit.  From cu_seqlens it writes
 *   order      [n_seqs]      sequence ids sorted by length, longest first
 *                            (ties by id)
 *   chunk_off  [n_seqs + 1]  exclusive prefix sum of ceil(len / 64)
 *   chunk_tab  [n_chunks, 3] (sequence id, first token, token count) per chunk,
 *                            sequences in id order, chunks restart at each
 *                            sequence start; n_chunks = chunk_off[n_seqs]
 *                            <= T_total / 64 + n_seqs
 * All arrays are device int32.  cu_seqlens must be non-NULL here.
 */
gdn_status gdn_chunk_map(const int32_t* cu_seqlens, int32_t n_seqs, int32_t T_total,
                         int32_t* order, int32_t* chunk_off, int32_t* chunk_tab, void* stream);

/*
 * gdn_decode_step -- one token per sequence, state updated in place.
 *
 * The rule above with T = 1: per (sequence n, value head h)
 *     S <- alpha S + beta (v - alpha S k) k^T,   o = scale * S q
 * computed in fp32 from one pass over the state.
 *
 *   q, k        [n_seqs, Hk, dk] bf16, sequence strides q_stride, k_stride
 *   v           [n_seqs, Hv, dv] bf16, sequence stride v_stride
 *   g, beta     [n_seqs, Hv] fp32, contiguous
 *   state       [n_slots, Hv, dv, dk] fp32, read and written in place
 *   state_slot  [n_seqs] int32 device array or NULL: sequence n uses slot
 *               state_slot[n] (NULL: slot n).  Slots in [0, n_slots) must be
 *               distinct; a slot outside [0, n_slots) (say -1 for a padding
 *               row of a fixed-size batch) makes the kernel skip sequence n:
 *               no state is read or written and its row of o is not written.
 *   o           [n_seqs, Hv, dv] fp32; must not overlap state or the inputs
 */
gdn_status gdn_decode_step(const uint16_t* q, int64_t q_stride, const uint16_t* k,
                           int64_t k_stride, const uint16_t* v, int64_t v_stride, const float* g,
                           const float* beta, float* state, const int32_t* state_slot,
                           int32_t n_slots, float* o, int32_t n_seqs, int32_t Hk, int32_t Hv,
                           int32_t dk, int32_t dv, float scale, void* stream);

/*
 * gdn_decode_tokens -- n_tokens (1..8) consecutive tokens per sequence, state
 * updated in place: the rule above applied to the tokens in order, as
 * n_tokens successive gdn_decode_step calls would, but reading and writing
 * each state once.  For serving steps that append several tokens to each
 * cached sequence (e.g. verifying drafted tokens).  Token t of sequence n is
 * row n * n_tokens + t of every per-token array:
 *
 *   q, k        [n_seqs * n_tokens, Hk, dk] bf16, row strides q_stride, k_stride
 *   v           [n_seqs * n_tokens, Hv, dv] bf16, row stride v_stride
 *   g, beta     [n_seqs * n_tokens, Hv] fp32, contiguous
 *   state       [n_slots, Hv, dv, dk] fp32, read and written in place
 *   state_slot  [n_seqs] int32 device array or NULL, as for gdn_decode_step
 *   o           [n_seqs * n_tokens, Hv, dv] fp32; must not overlap state or
 *               the inputs
 *
 * n_tokens outside 1..8 returns GDN_ERR_UNSUPPORTED; other errors as for
 * gdn_decode_step.
 */
gdn_status gdn_decode_tokens(const uint16_t* q, int64_t q_stride, const uint16_t* k,
                             int64_t k_stride, const uint16_t* v, int64_t v_stride,
                             const float* g, const float* beta, float* state,
                             const int32_t* state_slot, int32_t n_slots, float* o,
                             int32_t n_seqs, int32_t n_tokens, int32_t Hk, int32_t Hv,
                             int32_t dk, int32_t dv, float scale, void* stream);

/*
 * gdn_decode_mixer_step -- one decode step of the whole mixer in one kernel
 * (model card, Architecture table, row "Delta-rule layers": conv in front,
 * the rule with its fp32 state, gated RMS-norm after).  Per sequence n and
 * value head h, with the new token's projected channels x:
 *     y = silu(conv4(conv_state, x) + bias)   (conv state shifted in place)
 *     q, k = y / sqrt(sum y^2 + l2_eps) per head; q, k, v rounded to bf16
 *     S <- alpha S + beta (v - alpha S k) k^T,  o = scale * S q
 *     out = o / sqrt(mean(o^2) + norm_eps) * norm_w * z * sigmoid(z)
 * i.e. gdn_conv1d_fwd in decode batch mode (n_l2_heads = Hk), gdn_decode_step
 * and gdn_gated_rmsnorm in sequence, without the intermediate tensors.
 *
 *   x           [n_seqs, C] bf16, row stride x_stride >= C, C = (2 Hk + Hv) * d,
 *               channels [q heads | k heads | v heads]
 *   conv_w      [C, 4] bf16; conv_bias [C] fp32 or NULL
 *   conv_state  [n_slots, C, 3] bf16, oldest first, updated in place
 *   g, beta     [n_seqs, Hv] fp32, contiguous; or both NULL and the gates
 *               formed from the projections a, b [n_seqs, Hv] bf16 (token
 *               strides a_stride, b_stride >= Hv) and A_log, dt_bias [Hv] fp32
 *               as in gdn_chunk_fwd_gated (NULL when g, beta are given)
 *   z           [n_seqs, Hv * d] bf16, row stride z_stride >= Hv * d
 *   norm_w      [d] fp32
 *   state       [n_slots, Hv, d, d] fp32, updated in place
 *   state_slot  [n_seqs] int32 device array or NULL: sequence n uses slot
 *               state_slot[n] of both conv_state and state (NULL: slot n);
 *               slots in [0, n_slots) distinct; a slot outside [0, n_slots)
 *               (say -1) skips sequence n: neither pool is read or written and
 *               its row of out is not written
 *   out         [n_seqs, Hv, d], fp32 (out_is_bf16 == 0) or bf16 (rounded to
 *               nearest even); must not overlap any other tensor
 *   d           must be 128; Hv / Hk must be 1, 2, 3 or 4
 */
gdn_status gdn_decode_mixer_step(const uint16_t* x, int64_t x_stride, const uint16_t* conv_w,
                                 const float* conv_bias, uint16_t* conv_state, const float* g,
                                 const float* beta, const uint16_t* a, int64_t a_stride,
                                 const uint16_t* b, int64_t b_stride, const float* A_log,
                                 const float* dt_bias, const uint16_t* z, int64_t z_stride,
                                 const float* norm_w, float* state, const int32_t* state_slot,
                                 int32_t n_slots, void* out, int32_t out_is_bf16, int32_t n_seqs,
                                 int32_t Hk, int32_t Hv, int32_t d, float scale, float l2_eps,
                                 float norm_eps, void* stream);

/*
 * gdn_gated_rmsnorm -- the "gated RMS-norm" after the rule (model card,
 * Architecture table, row "Delta-rule layers"), per (row, value head):
 *     out_i = o_i / sqrt(mean_j o_j^2 + eps) * w_i * z_i * sigmoid(z_i)
 *
 *   o      [rows, Hv, dv] fp32, contiguous
 *   z      [rows, Hv * dv] bf16, row stride z_row_stride (>= Hv * dv)
 *   w      [dv] fp32, shared by all heads
 *   out    [rows, Hv, dv], fp32 (out_is_bf16 == 0) or bf16 (out_is_bf16 != 0,
 *          rounded to nearest, ties to even); may be the same buffer as o when
 *          fp32
 *   dv     must be 128
 */
gdn_status gdn_gated_rmsnorm(const float* o, const uint16_t* z, int64_t z_row_stride,
                             const float* w, void* out, int32_t out_is_bf16, int64_t rows,
                             int32_t Hv, int32_t dv, float eps, void* stream);

/*
 * gdn_backward -- gradients of the rule for training: the derivatives of
 *     L = sum(grad_o * o) + sum(grad_final_state * S_T)
 * (o and S_T as gdn_chunk_fwd computes them from the same inputs) with
 * respect to q, k, v, g, beta and the initial states.  The chain rule is
 * taken through the chunk-parallel form of the erase-then-write update (the
 * deep-dive page's paragraph on the Gated Delta Rule), chunks of 64 tokens,
 * in fp32 (fp32 matrix-core products, and for the products with the states
 * and their gradients fp32 operands split into bf16 hi + lo parts, about 17
 * significant bits per product; the gradients keep their relative accuracy
 * whatever the scale of grad_o): a per-chunk pass forms
 * (I + A)^-1 and the masked Q K^T of every (chunk, value head), a forward
 * chain records each chunk's initial state and its U, E, a reverse chain
 * carries dL/dS through the chunks and records it, and a per-(chunk, key
 * head) pass forms dq, dk (summed over the key head's value heads), dg and
 * dbeta.  The workspace holds per chunk slot (T_total / 64 + n_seqs) and value
 * head about 240 KB: roughly 190 KB per token at 48 value heads.
 *
 *   q, k, v, g, beta, initial_state, cu_seqlens, n_seqs, T_total, sizes
 *                     as gdn_chunk_fwd (initial_state NULL = zeros)
 *   grad_o            [T_total, Hv, dv] fp32, contiguous
 *   grad_final_state  [n_seqs, Hv, dv, dk] fp32 or NULL (= zeros)
 *   grad_q, grad_k    [T_total, Hk, dk] fp32, contiguous
 *   grad_v            [T_total, Hv, dv] fp32, contiguous
 *   grad_g, grad_beta [T_total, Hv] fp32, contiguous (grad_g is dL/dg, g
 *                     being the log of the decay alpha)
 *   grad_initial_state [n_seqs, Hv, dv, dk] fp32 or NULL (not written)
 *   workspace         >= gdn_backward_workspace_bytes(n_seqs, T_total, Hv) bytes,
 *                     256-byte aligned, contents ignored on entry
 *
 * No output may overlap an input, another output or the workspace
 * (GDN_ERR_ALIAS).  Errors as gdn_chunk_fwd.
 */
size_t gdn_backward_workspace_bytes(int32_t n_seqs, int32_t T_total, int32_t Hv);
gdn_status gdn_backward(const uint16_t* q, int64_t q_tok_stride, const uint16_t* k,
                        int64_t k_tok_stride, const uint16_t* v, int64_t v_tok_stride,
                        const float* g, const float* beta, const float* initial_state,
                        const float* grad_o, const float* grad_final_state,
                        const int32_t* cu_seqlens, int32_t n_seqs, int32_t T_total, int32_t Hk,
                        int32_t Hv, int32_t dk, int32_t dv, float scale, float* grad_q,
                        float* grad_k, float* grad_v, float* grad_g, float* grad_beta,
                        float* grad_initial_state, void* workspace, size_t workspace_bytes,
                        void* stream);

/*
 * gdn_validate_cu_seqlens -- opt-in host check of a device cu_seqlens array:
 * cu[0] == 0, non-decreasing, cu[n_seqs] == T_total.  Copies the array to the
 * host and therefore SYNCHRONISES the stream.  Returns GDN_OK or
 * GDN_ERR_SEQLENS.  When the environment variable GDN_VALIDATE_CU_SEQLENS=1
 * is set, gdn_conv1d_fwd and gdn_chunk_fwd call it before enqueuing.
 */
gdn_status gdn_validate_cu_seqlens(const int32_t* cu_seqlens, int32_t n_seqs, int32_t T_total,
                                   void* stream);

/*
 * gdn_calib_mfma_loop -- a measurement aid, not part of the rule: the dense
 * fp16 matrix-unit ceiling of the running device, against which the prefill's
 * matrix products are judged (beside the HBM ceiling a plain device copy
 * gives).  n_blocks work-groups of 4 waves; every wave runs n_iter rounds of 8
 * independent v_mfma_f32_16x16x32_f16 products and writes one float (the sum
 * of its accumulators) to out[wave], so out holds 4 * n_blocks floats.
 * gdn_calib_mfma_loop_flops gives the flops of such a launch (2*16*16*32 per
 * product); divide by the launch time.  n_iter, n_blocks >= 1, n_blocks <=
 * 2^20, out 4-byte aligned; GDN_ERR_SHAPE / GDN_ERR_NULL otherwise.
 */
double gdn_calib_mfma_loop_flops(int32_t n_iter, int32_t n_blocks);
gdn_status gdn_calib_mfma_loop(int32_t n_iter, int32_t n_blocks, float* out, void* stream);

/*
 * gdn_calib_stream_inplace -- a measurement aid, not part of the rule: the
 * HBM ceiling of the decode step's traffic pattern on the running device.
 * Every 16-byte piece of buf [bytes] is read and written back unchanged with
 * nontemporal accesses by n_blocks work-groups of 256 threads (grid-stride),
 * so 2 * bytes cross HBM per launch; divide by the launch time.  bytes a
 * positive multiple of 16, buf 16-byte aligned, 1 <= n_blocks <= 2^20;
 * GDN_ERR_SHAPE / GDN_ERR_NULL otherwise.  The contents are left as they were.
 */
gdn_status gdn_calib_stream_inplace(void* buf, int64_t bytes, int32_t n_blocks, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* GDN_H */
