/*
 * based.h -- C ABI of the Based sequence-mixing layer for AMD Instinct MI355X
 * (gfx950).
 *
 * The layer pairs two attentions over the same q, k, v (HazyResearch/based
 * README, introduction):
 *   - a global causal linear attention whose kernel is the 2nd-order Taylor
 *     expansion of exp(q.k), realised by the feature map
 *       phi(x) = [1, x_1..x_16, x_a x_b / sqrt(2) for a = 1..16, b = 1..16]
 *     (273 features for d_k = 16; blog post "Базированная модель, часть 2",
 *     feature-map pseudocode), normalised:
 *       y_i = sum_{j<=i} phi(q_i).phi(k_j) v_j / sum_{j<=i} phi(q_i).phi(k_j);
 *   - an exact softmax attention over a short causal sliding window (64).
 * The recurrent form keeps a numerator KV-state S = sum_j phi(k_j) v_j^T and a
 * denominator K-state z = sum_j phi(k_j) (same blog post, paragraph on the
 * state); the decode entry point advances that state one token at a time.
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * Tensors are dense, row-major, [B, H, L, d] with d fastest (d = d_k, d_qk or
 * d_v), base pointers 16-byte aligned, living in device memory of the current
 * HIP device.  Inputs q, k, v have the element type `dtype`; outputs and
 * states are fp32.  Causal means inclusive: row i sees positions j <= i.
 * One (batch, head) block of any [L, d] tensor must span fewer than 2^31
 * bytes in fp32, L * d * 4 < 2^31 for every d of the call (the kernels
 * address a head through 32-bit offsets): L < 4,194,304 at d = 128 and
 * L < 8,388,608 at d = 64; longer sequences return BASED_ERR_SHAPE (split
 * them with S_in / S_out).
 *
 * State layout (S_in, S_out, decode S: [B, H, 273, d_v]; z: [B, H, 273]):
 * row 0 is the constant feature, row 1 + a the linear feature x_a, row
 * 17 + 16 a + b the quadratic feature x_a x_b / sqrt(2) (a, b in 0..15).
 * States written by this library are symmetric in (a, b).  A state read by
 * this library enters every output only through S[ab] + S[ba].
 *
 * Ownership: the caller allocates and frees every buffer; the library never
 * allocates, keeps no mutable global state and is re-entrant on distinct
 * buffers.  All work is enqueued asynchronously on `stream` (a hipStream_t;
 * NULL is the default stream); nothing synchronises and nothing copies
 * between host and device.
 *
 * Errors: arguments are validated on the host before anything is enqueued; a
 * failed check returns a negative BASED_ERR_* code and touches no memory.
 * A failed kernel launch returns BASED_ERR_HIP.  Faults inside a kernel
 * surface at the caller's next synchronisation.  NaN and Inf inputs are not
 * checked; they propagate to the outputs they reach.
 */
#ifndef BASED_H
#define BASED_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define BASED_ABI_VERSION 9

/* element type of q, k, v (and of the decode ring buffers) */
enum {
  BASED_F32 = 0,  /* fp32: arithmetic in fp32 throughout                       */
  BASED_BF16 = 1  /* bf16: products on the matrix cores, accumulation in fp32 */
};

enum {
  BASED_OK = 0,
  BASED_ERR_NULL = -1,        /* a required pointer is NULL                     */
  BASED_ERR_SHAPE = -2,       /* a size is out of range                         */
  BASED_ERR_UNSUPPORTED = -3, /* a head dimension this library does not handle  */
  BASED_ERR_DTYPE = -4,       /* dtype is not BASED_F32 or BASED_BF16           */
  BASED_ERR_ALIGN = -5,       /* a base pointer is not 16-byte aligned          */
  BASED_ERR_WORKSPACE = -6,   /* workspace NULL or smaller than required        */
  BASED_ERR_WINDOW = -7,      /* window outside 1..64                           */
  BASED_ERR_HIP = -8,         /* a HIP runtime call or kernel launch failed     */
  BASED_ERR_ALIAS = -9        /* an output overlaps an input it must not overlap */
};

#define BASED_DK 16        /* q/k head dimension of the Taylor linear attention */
#define BASED_DPHI 273     /* 1 + 16 + 16*16 Taylor features                    */
#define BASED_DCMP 153     /* compact decode state: 1 + 16 + 16*17/2 rows       */
#define BASED_MAX_WINDOW 64
#define BASED_MAX_CONV 4     /* longest BaseConv filter (taps)                   */

/* ABI version compiled into the library (BASED_ABI_VERSION). */
int based_abi_version(void);

/* Static, NUL-terminated description of a status code. */
const char* based_status_string(int status);

/*
 * Bytes of device workspace based_linattn_fwd needs for this shape (0 when
 * none).  Depends only on the arguments.  Returns 0 for invalid arguments
 * as well; based_linattn_fwd reports those.
 */
size_t based_linattn_workspace_bytes(int B, int H, int L, int d_k, int d_v, int dtype);

/*
 * Causal Taylor linear attention, forward (blog post, linear-attention
 * paragraph and feature-map pseudocode; README intro "dense, global linear
 * attention").
 *
 *   q, k   [B,H,L,d_k] dtype, d_k must be 16
 *   v      [B,H,L,d_v] dtype, d_v in {16, 32, 48, ..., 128}
 *   y      [B,H,L,d_v] fp32 out: y_i = (phi(q_i)^T S_i) / (phi(q_i)^T z_i) with
 *          S_i = S_in + sum_{j<=i} phi(k_j) v_j^T, z_i likewise
 *   S_in   [B,H,273,d_v] fp32 or NULL (zero state)  -- initial state, e.g. the
 *   z_in   [B,H,273]     fp32 or NULL (zero state)     S_out of an earlier call
 *          S_in and z_in must be both NULL or both set.
 *   S_out  [B,H,273,d_v] fp32 or NULL  -- state after position L-1
 *   z_out  [B,H,273]     fp32 or NULL     (both NULL or both set)
 *   B, H >= 1; L >= 0 (L = 0 only copies the state through).
 *   workspace: device memory of at least based_linattn_workspace_bytes(...)
 *          bytes (may be NULL when that is 0); contents on entry are ignored.
 *
 * With zero initial state the denominator of row i is at least (i + 1) / 2,
 * so no epsilon is added.  y must not overlap q, k, v, S_in or z_in.
 * S_out may be S_in itself and z_out z_in itself (in-place state update);
 * any other overlap of S_out or z_out with an input, with each other, with
 * y or with the workspace, and any overlap of the workspace with an input,
 * returns BASED_ERR_ALIAS.
 *
 * BASED_BF16 with d_v in {32, 64, 96, 128} runs on the matrix cores with fp16
 * operands (bf16 inputs convert exactly): Taylor features and the state copy
 * read out by each chunk are rounded to fp16 once (relative 2^-11; the state
 * is scaled by a power of two, so its size is not limited), the in-chunk
 * weights are split into fp16 hi + lo, and all sums are fp32.  With a
 * non-NULL S_in the readout instead takes both the query features and the
 * state copy as fp16 hi + lo (three matrix passes), so that a caller's state
 * of any make-up -- whose readout may cancel over its 272 feature rows -- is
 * read to the same relative precision as a state the recurrence builds.
 * Inputs must stay in fp16 range there: |q|, |k| < 128 per coordinate,
 * |q.k| < 256 and |v| < 32768.  Other d_v, and BASED_F32, use fp32 vector
 * arithmetic.
 */
int based_linattn_fwd(const void* q, const void* k, const void* v, float* y,
                      const float* S_in, const float* z_in, float* S_out, float* z_out,
                      int B, int H, int L, int d_k, int d_v, int dtype,
                      void* workspace, size_t workspace_bytes, void* stream);

/*
 * Causal Taylor linear attention with a per-head state decay, forward: the
 * based/train README's optional decay strategy, read (no formula on the
 * pages) as S_i = gamma_h S_{i-1} + phi(k_i) v_i^T and z_i = gamma_h z_{i-1} +
 * phi(k_i), y_i = phi(q_i)^T S_i / phi(q_i)^T z_i -- the kernel weight of key j
 * in row i becomes K_ij gamma_h^(i-j); gamma_h = 1 is based_linattn_fwd.
 *
 *   gamma  [H] fp32, device memory; each gamma_h is taken clamped to [0, 1]
 *          (NaN reads as 0).  gamma_h = 0 keeps each position's own term
 *          only (gamma^0 = 1; powers d >= 1 of 0 are flushed below 2^-126)
 *   every other argument as for based_linattn_fwd (same workspace size; S_in
 *   decays like the rest: position i sees gamma^(i+1) S_in).
 * BASED_BF16 with d_v in {32, 64, 96, 128} runs on the matrix cores,
 * numerics as for based_linattn_fwd with the per-key decay weights of the
 * state update rounded to fp16; BASED_F32 and other d_v use fp32 vector
 * arithmetic throughout (the decay weights gamma^d from exp2 of d log2 gamma).
 */
int based_linattn_decay_fwd(const void* q, const void* k, const void* v, const float* gamma, float* y,
                            const float* S_in, const float* z_in, float* S_out, float* z_out,
                            int B, int H, int L, int d_k, int d_v, int dtype,
                            void* workspace, size_t workspace_bytes, void* stream);

/*
 * Causal sliding-window softmax attention, forward (README intro: exact
 * softmax attention over a short window).
 *
 *   q, k   [B,H,L,d_qk] dtype, d_qk in {16, 32, ..., 128}
 *   v      [B,H,L,d_v]  dtype, d_v in {16, 32, ..., 128}
 *   y      [B,H,L,d_v]  fp32 out
 *   Row i attends to the `window` positions max(0, i-window+1) .. i (itself
 *   included) with weights softmax_j(scale * q_i.k_j).  1 <= window <= 64.
 *   B, H >= 1, L >= 0.  y must not overlap q, k or v.
 */
int based_swa_fwd(const void* q, const void* k, const void* v, float* y,
                  int B, int H, int L, int d_qk, int d_v, int window, float scale,
                  int dtype, void* stream);

/*
 * Bytes of device workspace based_linattn_bwd needs for this shape (0 for
 * invalid arguments; based_linattn_bwd reports those).
 */
size_t based_linattn_bwd_workspace_bytes(int B, int H, int L, int d_k, int d_v, int dtype);

/*
 * Causal Taylor linear attention, backward: gradients of based_linattn_fwd's
 * y (zero initial state) with respect to q, k and v -- the derivative of the
 * forward above, which the based/train README's training views train
 * through.
 *
 *   q, k, v    as for based_linattn_fwd (d_k = 16)
 *   y          [B,H,L,d_v] fp32 -- based_linattn_fwd's output for these q, k, v
 *   dy         [B,H,L,d_v] fp32 -- gradient of the loss with respect to y
 *   dq, dk     [B,H,L,16]  fp32 out;  dv [B,H,L,d_v] fp32 out
 *   workspace: at least based_linattn_bwd_workspace_bytes(...) bytes of
 *          device memory; contents on entry are ignored.
 *
 * With x_ij = q_i.k_j, K_ij = 1 + x_ij + x_ij^2/2, den_i = sum_{j<=i} K_ij,
 * g_i = dy_i / den_i and h_i = -(dy_i . y_i) / den_i:
 *   dq_i = sum_{j<=i} c_ij k_j,  dk_j = sum_{i>=j} c_ij q_i,
 *   dv_j = sum_{i>=j} K_ij g_i,  c_ij = (g_i . v_j + h_i)(1 + x_ij).
 * No output may overlap an input, another output or the workspace.
 * Numerics: BASED_F32 is fp32 throughout; BASED_BF16 as for the forward.
 */
int based_linattn_bwd(const void* q, const void* k, const void* v, const float* y, const float* dy,
                      float* dq, float* dk, float* dv, int B, int H, int L, int d_k, int d_v, int dtype,
                      void* workspace, size_t workspace_bytes, void* stream);

/*
 * The decayed linear attention, backward: gradients of based_linattn_decay_fwd's
 * y (zero initial state) with respect to q, k and v -- based_linattn_bwd with
 * every kernel entry weighed by gamma_h^(i-j) (K_ij -> K_ij gamma_h^(i-j) in
 * den_i, dq_i, dk_j and dv_j; the train README's decay strategy, read as for
 * the forward).
 *
 *   gamma      [H] fp32, device memory, clamped to [0, 1] as in
 *              based_linattn_decay_fwd
 *   q, k, v, y, dy, dq, dk, dv: as for based_linattn_bwd (y from
 *              based_linattn_decay_fwd with the same gamma)
 *   workspace: at least 2 * B * H * L * 4 bytes of device memory; contents
 *              on entry are ignored.
 * With BASED_BF16, d_v in {32, 64, 96, 128} and a workspace of at least
 * based_linattn_bwd_workspace_bytes for the shape, the matrix-core passes of
 * based_linattn_bwd with the decay (the carried states decay per position and
 * per chunk, the in-chunk terms carry gamma^(i-j); the same numerics).
 * Otherwise (fp32, other widths, or the smaller workspace) the chunked fp32
 * vector form of based_linattn_bwd with the same decay weights.
 * Errors as for based_linattn_bwd, and BASED_ERR_NULL for a null gamma; gamma
 * must not overlap an output or the workspace.
 */
int based_linattn_decay_bwd(const void* q, const void* k, const void* v, const float* gamma, const float* y,
                            const float* dy, float* dq, float* dk, float* dv, int B, int H, int L, int d_k,
                            int d_v, int dtype, void* workspace, size_t workspace_bytes, void* stream);

/*
 * Sliding-window softmax attention, backward: gradients of based_swa_fwd's y
 * with respect to q, k and v (the exact softmax Jacobian).
 *
 *   q, k       [B,H,L,d_qk] dtype, d_qk must be 16 (the layer's)
 *   v          [B,H,L,d_v]  dtype, d_v in {16, 32, ..., 128}
 *   y          [B,H,L,d_v]  fp32 -- based_swa_fwd's output for these inputs
 *   dy         [B,H,L,d_v]  fp32 -- gradient of the loss with respect to y
 *   dq, dk, dv fp32 out, shaped like q, k, v
 *   window, scale: as for based_swa_fwd.
 * With p_ij the window softmax weights, dP_ij = dy_i . v_j and D_i = dy_i . y_i:
 *   dS_ij = p_ij (dP_ij - D_i); dq_i = scale sum_j dS_ij k_j;
 *   dk_j = scale sum_i dS_ij q_i; dv_j = sum_i p_ij dy_i.
 * Arithmetic is fp32 for both dtypes.  No output may overlap an input or
 * another output.
 */
int based_swa_bwd(const void* q, const void* k, const void* v, const float* y, const float* dy,
                  float* dq, float* dk, float* dv, int B, int H, int L, int d_qk, int d_v,
                  int window, float scale, int dtype, void* stream);

/*
 * BaseConv gate, forward: the gated short convolution of the BaseConv block
 * (blog post "Базированная модель, часть 1", BaseConv: y = linear(x) * conv(h, x);
 * README acknowledgements: a short causal conv1d).  linear(x) is the caller's
 * projection of x (a plain matrix product) and enters as u.
 *
 *   x, u   [B,L,D] dtype, token-major (channels fastest); D a multiple of 4
 *   h      [D,K] fp32 filter, tap s applied to x_{t-s}; 1 <= K <= BASED_MAX_CONV
 *   bias   [D] fp32 or NULL
 *   y      [B,L,D] fp32 out:
 *            y[b,t,c] = u[b,t,c] * (bias[c] + sum_{s<K} h[c,s] x[b,t-s,c]),
 *          x before position 0 taken as zero (causal; each sequence apart).
 *   B >= 1, L >= 0.  y must not overlap x, u, h or bias.
 * Arithmetic is fp32 for both dtypes.
 */
int based_baseconv_fwd(const void* x, const void* u, const float* h, const float* bias, float* y,
                       int B, int L, int D, int K, int dtype, void* stream);

/*
 * The Based layer's two attentions over the same q, k, v in one pass: the
 * outputs of based_linattn_fwd (y_lin, with its state arguments) and of
 * based_swa_fwd with d_qk = d_k (y_swa) from a single read of the inputs
 * (README intro: the layer pairs a global linear attention with a short
 * sliding-window softmax attention).
 *
 *   q, k, v, S_in, z_in, S_out, z_out, workspace: as for based_linattn_fwd
 *          (workspace size from based_linattn_workspace_bytes)
 *   y_lin  [B,H,L,d_v] fp32 out -- based_linattn_fwd's y
 *   y_swa  [B,H,L,d_v] fp32 out -- based_swa_fwd's y (d_qk = d_k = 16)
 *   window, scale: as for based_swa_fwd.
 * Neither output may overlap an input, a state or the other output.
 * BASED_BF16 with d_v in {32, 64, 96, 128} is one fused matrix-core pass (with
 * the input ranges of based_linattn_fwd); otherwise L <= 512 with no S_in and
 * no S_out is one fused vector pass (fp32 arithmetic), and the rest runs the
 * two attentions as separate kernels.
 */
int based_layer_fwd(const void* q, const void* k, const void* v, float* y_lin, float* y_swa,
                    const float* S_in, const float* z_in, float* S_out, float* z_out,
                    int B, int H, int L, int d_k, int d_v, int window, float scale, int dtype,
                    void* workspace, size_t workspace_bytes, void* stream);

/*
 * based_layer_fwd with the linear attention's state decayed per head, as in
 * based_linattn_decay_fwd (gamma [H] fp32 device memory, clamped to [0, 1];
 * y_lin is based_linattn_decay_fwd's y); the window attention
 * (y_swa) has no decay.  Every other argument, and the workspace size, as for
 * based_layer_fwd; BASED_ERR_NULL for a null gamma, BASED_ERR_ALIAS when
 * gamma overlaps an output.  BASED_BF16 with d_v in {32, 64, 96, 128} is one
 * fused matrix-core pass; otherwise L <= 512 with no S_in and no S_out is one
 * fused vector pass, and the rest runs the two attentions as separate
 * kernels.
 */
int based_layer_decay_fwd(const void* q, const void* k, const void* v, const float* gamma, float* y_lin,
                          float* y_swa, const float* S_in, const float* z_in, float* S_out, float* z_out,
                          int B, int H, int L, int d_k, int d_v, int window, float scale, int dtype,
                          void* workspace, size_t workspace_bytes, void* stream);

/*
 * based_layer_fwd without a workspace argument, for callers that cannot
 * allocate device memory (code under HIP graph capture, serving loops,
 * harnesses that forbid hipMalloc).  The segment records live in a static
 * device array of BASED_NOALLOC_SCRATCH_MB MiB that each GPU the library
 * runs on holds until the process ends; this entry point allocates nothing
 * (no hipMalloc, no allocating library call).  That array is larger than
 * the workspace of every shape the layer splits into segments (at most
 * about 41 MiB); a shape whose workspace would not fit returns
 * BASED_ERR_WORKSPACE.  Its contents on entry are ignored, so nothing needs
 * clearing between calls.  All calls on one GPU share the array: calls that
 * overlap in time on one GPU (on different streams, or from several host
 * threads) race, and must be serialised by the caller.  Every other
 * argument, result and error as for based_layer_fwd; BASED_ERR_HIP if the
 * array's device address cannot be obtained.
 */
#define BASED_NOALLOC_SCRATCH_MB 48
int based_layer_fwd_noalloc(const void* q, const void* k, const void* v, float* y_lin, float* y_swa,
                            const float* S_in, const float* z_in, float* S_out, float* z_out,
                            int B, int H, int L, int d_k, int d_v, int window, float scale, int dtype,
                            void* stream);

/*
 * Fill the decode ring buffers from a context and set the positions
 * (the set-up of generation after a prefill).
 *
 *   k      [B,H,L,d_k] dtype, v [B,H,L,d_v] dtype -- the context (L >= 0)
 *   ring_k [B,H,window,d_k] dtype out, ring_v [B,H,window,d_v] dtype out:
 *          slot (t mod window) receives position t for the last min(L, window)
 *          positions; other slots are left untouched (they are never read).
 *   pos    [B] int32 out: set to L.
 * The linear-attention state comes from based_linattn_fwd's S_out / z_out
 * over the same context.
 */
int based_decode_prefill(const void* k, const void* v, void* ring_k, void* ring_v, int32_t* pos,
                         int B, int H, int L, int d_k, int d_v, int window, int dtype,
                         void* stream);

/*
 * One generation step of the layer for B sequences x H heads (blog post,
 * paragraph on the state: constant-size KV-state and K-state instead of a
 * KV cache; README intro: window attention over the last 64 tokens).
 *
 *   q, k   [B,H,d_k] dtype (d_k = 16), v [B,H,d_v] dtype (d_v in {16..128})
 *   S      [B,H,273,d_v] fp32 in/out, z [B,H,273] fp32 in/out
 *   ring_k [B,H,window,d_k] dtype in/out, ring_v [B,H,window,d_v] in/out
 *   pos    [B] int32 in/out: position t of this token; incremented by one.
 *   y_lin  [B,H,d_v] fp32 out, y_swa [B,H,d_v] fp32 out
 * Per (b, h), with t = pos[b]:
 *   S += phi(k) v^T;  z += phi(k);  y_lin = phi(q)^T S / phi(q)^T z
 *   ring slot (t mod window) <- (k, v)
 *   y_swa = sum_j p_j v_j / sum_j p_j over positions max(0, t-window+1)..t,
 *           p_j = exp(scale * q.k_j - max)
 * The token attends to itself in both attentions.  1 <= window <= 64; the
 * ring's slot count equals `window`.  Sequences are independent: each may be
 * at a different position.
 */
int based_decode_step(const void* q, const void* k, const void* v,
                      float* S, float* z, void* ring_k, void* ring_v, int32_t* pos,
                      float* y_lin, float* y_swa,
                      int B, int H, int d_k, int d_v, int window, float scale, int dtype,
                      void* stream);

/*
 * based_decode_step for the decayed linear attention (the train README's
 * optional decay strategy, read as a per-head factor on the state, as in
 * based_linattn_decay_fwd):
 *   S <- gamma[h] S + phi(k) v^T;  z <- gamma[h] z + phi(k);
 *   y_lin = phi(q)^T S / phi(q)^T z
 * gamma: [H] fp32 device pointer, each entry taken clamped to [0, 1] (NaN as
 * 0), read only, shared by the batch; it must not overlap any output.  The window attention
 * and the ring are as in based_decode_step.  A state prefilled by
 * based_linattn_decay_fwd's S_out / z_out over the context continues the
 * decayed forward exactly.  Both dtypes, d_v in {16..128}.  Errors as
 * based_decode_step, and BASED_ERR_NULL for a null gamma.
 */
int based_decode_step_decay(const void* q, const void* k, const void* v, const float* gamma,
                            float* S, float* z, void* ring_k, void* ring_v, int32_t* pos,
                            float* y_lin, float* y_swa,
                            int B, int H, int d_k, int d_v, int window, float scale, int dtype,
                            void* stream);

/*
 * based_decode_step (and, with a non-NULL gamma, based_decode_step_decay) on
 * a state in the compact layout: one row per unordered pair of the quadratic
 * features.  Every state the recurrence builds has S[(a,b)] = S[(b,a)] for the
 * rows of the ordered pairs (k_a k_b / sqrt2 both), and the readout and the
 * update use only their sum, so one row per pair carries the same state
 * (blog post, paragraph on the state; feature map of the linear attention):
 *   S  [B,H,153,d_v] fp32: row 0 the constant feature, rows 1..16 the linear
 *      features, then for a = 0..15, b = a..15 in that order the pair (a, b),
 *      holding S[(a,b)] + S[(b,a)] for a < b and S[(a,a)] on the diagonal;
 *   z  [B,H,153] fp32 likewise.
 * The step moves 56 % of the state bytes of based_decode_step and gives its
 * results for a symmetric 273-row state up to rounding order (pair rows are
 * updated once with sqrt2 k_a k_b v instead of twice with k_a k_b v / sqrt2).
 * Convert with based_state_compact / based_state_expand.  gamma: [H] fp32 or
 * NULL (no decay), as in based_decode_step_decay.  Every other argument and
 * every error as in based_decode_step.
 */
int based_decode_step_compact(const void* q, const void* k, const void* v, const float* gamma,
                              float* S, float* z, void* ring_k, void* ring_v, int32_t* pos,
                              float* y_lin, float* y_swa,
                              int B, int H, int d_k, int d_v, int window, float scale, int dtype,
                              void* stream);

/*
 * State layout conversions for based_decode_step_compact (layouts as there).
 *   based_state_compact: S [B,H,273,d_v], z [B,H,273] -> Sc [B,H,153,d_v],
 *     zc [B,H,153]; a pair row is the sum of the two ordered rows.
 *   based_state_expand: Sc, zc -> S, z; both ordered rows of a pair get half
 *     the pair row (so expand(compact(S)) = S for a symmetric S, and
 *     compact(expand(Sc)) = Sc).
 * All fp32 device pointers; outputs must not overlap inputs or each other.
 * d_v in {16, 32, ..., 128}.  Errors: BASED_ERR_SHAPE (B, H < 1 or too
 * large), BASED_ERR_UNSUPPORTED (d_v), BASED_ERR_NULL, BASED_ERR_ALIGN
 * (pointers not 16-byte aligned), BASED_ERR_ALIAS, BASED_ERR_HIP (launch).
 */
int based_state_compact(const float* S, const float* z, float* Sc, float* zc, int B, int H, int d_v,
                        void* stream);
int based_state_expand(const float* Sc, const float* zc, float* S, float* z, int B, int H, int d_v,
                       void* stream);

#ifdef __cplusplus
}
#endif

#endif /* BASED_H */
