/*
 * kdtopk.h - C ABI of the MI355X (gfx950) fused top-K knowledge-distillation
 * library: the chunked LM head + sparse top-K KD loss (forward and backward)
 * and the companion teacher-cache build.
 *
 * Sources, cited by title and section:
 *  [TG]  "The Gradient That Top-k Distillation Never Computes" (Khanbayov,
 *        Kurban): abstract; Figure 2 (renormalized objective, tail masses);
 *        Figure 3 (top-k cache of the teacher's logits; z = U g + b from a
 *        hidden-state cache, 2dV FLOP per token).
 *  [TA]  "Tail-Aware Top-k On-Policy Distillation" (Huang, Wei), abstract:
 *        top-k bins plus one tail bin carrying the tail probability.
 *  [TT]  "Unbiased Top-k Estimation for On-Policy Distillation" (Meng et
 *        al.), abstract and Table 2: reverse KL over normalized top-k
 *        distributions, the student's own top-16 as the support.
 *  [FK]  "Efficient Knowledge Distillation for LLMs: Offline Top-K Logits
 *        and a Fused Chunked KL Loss": section 3.2, identity (2) (partial
 *        retained mass, only log Z spans the vocabulary) and Eq. (3) (logit
 *        gradient = M * softmax minus a sparse teacher term); the fused
 *        chunked loss never materialises the [T, V] logits.
 *  [SS]  "Sparse Teacher Support Cuts LLM Distillation Cost Without Losing
 *        Accuracy": the adaptive support k_rho = min{k : top-k mass >= rho}.
 *
 * Conventions for every call:
 *  - All array pointers are DEVICE pointers (HIP device memory of the
 *    current device) unless marked "host".  Row-major, no strides.
 *  - bf16 arrays are passed as their 16-bit patterns (kd_bf16).
 *  - The caller owns every buffer, including the workspace `ws`, whose size
 *    comes from the matching *_workspace() query.  The library allocates no
 *    device memory.
 *  - Work is enqueued asynchronously on `stream` (a hipStream_t, NULL = the
 *    default stream).  Argument errors are detected on the host before any
 *    launch and return a non-zero status with nothing enqueued; a launch
 *    failure returns KD_EHIP.  kd_last_error() then describes the problem.
 *  - No atomics touch floating-point results: outputs are bitwise
 *    reproducible from run to run on the same device.
 *  - Shape limits: 1 <= K <= min(V, 1024); d % 64 == 0; d <= 16384;
 *    T >= 0; V >= 1.
 *  - The matrices h, W, g, U, dh, dW and the workspace are accessed with
 *    16-byte vector loads and stores and must be 16-byte aligned (hipMalloc
 *    and PyTorch's allocator return 256-byte aligned blocks); a misaligned
 *    one is refused with KD_EINVAL.
 */
#ifndef KDTOPK_H
#define KDTOPK_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef uint16_t kd_bf16;

typedef enum {
  KD_OK = 0,
  KD_EINVAL = 1,        /* invalid argument (shape, null pointer, mode) */
  KD_EUNSUPPORTED = 2,  /* valid but outside this build's limits */
  KD_ENOWS = 3,         /* workspace too small */
  KD_EHIP = 4           /* a HIP runtime call or launch failed */
} kd_status;

/* Loss modes.  Per token t, with z = W h_t, p = softmax(z), S = the cached
 * indices, q_v = exp(teacher_logp_v) on S, Q = sum_S q, m_p = sum of p
 * outside S (= 1 - sum_S p; computed as the sum over the tokens outside S),
 * p_hat / q_hat = p / q renormalized over S:
 *   KD_RENORM  L = KL(q_hat || p_hat)                    [TG abstract, Fig. 2]
 *   KD_TAIL    L = sum_S q log(q/p) + m_q log(m_q/m_p)   [TA abstract; the
 *              (K+1)-bin KL, read in the forward direction]
 *   KD_FULL    L = sum_S q (log q - z) + Q * logsumexp(z) [FK sec. 3.2, (2);
 *              equals the dense KL(q || p) when S covers the vocabulary]
 *   KD_REVERSE L = KL(p_hat || q_hat)                    [TT abstract]
 *   KD_TAIL_REVERSE  L = sum_S p log(p/q) + m_p log(m_p/m_q) [TA abstract: the
 *              reverse KL over the top-k tokens plus a tail token]
 *   KD_REVERSE_TT    L = sum_S p log(p/q) (+ the sampled-token tail correction of
 *              kd_topk_loss_fwd_bwd_tt) [TT abstract, Figure 1]
 * For KD_RENORM, KD_TAIL, KD_FULL, KD_REVERSE and KD_TAIL_REVERSE the
 * gradient dL/dz is the exact derivative of L (for KD_FULL it is Eq. (3)).
 * KD_REVERSE_TT is an estimator: its dz is sum_S a_v grad p_v with
 * a = log p - log q held fixed, i.e. the S-part of the full reverse-KL
 * gradient, which leaves out the p (1_S - P_S) term that differentiating the
 * reported L through a would add (see kd_topk_loss_fwd_bwd_tt).
 * Tail masses inside logarithms are floored at the smallest normal float. */
typedef enum {
  KD_RENORM = 0, KD_TAIL = 1, KD_FULL = 2, KD_REVERSE = 3, KD_TAIL_REVERSE = 4, KD_REVERSE_TT = 5
} kd_mode;

/* Bytes of device workspace kd_topk_loss_fwd_bwd needs for these sizes.
 * Linear in T for fixed (d, V, K, chunk).  Returns 0 for invalid sizes. */
size_t kd_topk_loss_workspace(int64_t T, int64_t d, int64_t V, int32_t K, kd_mode mode, int32_t chunk);

/* Fused chunked LM head + top-K KD loss, forward and backward [FK sec. 3.2].
 *
 * In:  h            [T, d] bf16   student final hidden states
 *      W            [V, d] bf16   LM-head (unembedding) rows
 *      idx          [T, K] int32  retained indices per token, distinct within a
 *                                 row, in [0, V) or -1 for an ignored padding slot;
 *                                 any order.  Values >= V are rejected on the
 *                                 device by writing NaN to *loss.
 *      teacher_logp [T, K] fp32   teacher log-probabilities at idx.  KD_TAIL,
 *                                 KD_TAIL_REVERSE and KD_FULL expect
 *                                 full-vocabulary-normalised values;
 *                                 KD_RENORM and KD_REVERSE accept any per-row shift.
 *      m_q          [T]    fp32   teacher tail mass (KD_TAIL, KD_TAIL_REVERSE; may be NULL
 *                                 for the other modes)
 *      mode         kd_mode
 *      chunk        vocabulary rows per chunk of the backward (> 0; e.g. 8192;
 *                   rounded up to 256).  chunk x d, T x d and T x chunk bf16
 *                   arrays must each stay below 4 GiB.
 *                   Vocabulary-sized scratch is bounded by chunk rows.
 *      scale        loss = scale * sum_t L_t (e.g. 1/T for the token mean)
 * Out: loss         [1]    fp32   the scalar loss
 *      loss_tok     [T]    fp32   per-token L_t (unscaled), or NULL
 *      lse          [T]    fp32   logsumexp of each token's logits, or NULL
 *      m_p          [T]    fp32   student tail mass outside S, or NULL
 *      dh           [T, d] fp32   dloss/dh, fully written
 *      dW           [V, d] fp32   dloss/dW, fully written
 * The [T, V] logits are never stored: the forward keeps only per-token
 * partial logsumexps and the K gathered logits; the backward recomputes
 * one vocabulary chunk of logits at a time and folds the closed-form dz
 * into dh and dW. */
kd_status kd_topk_loss_fwd_bwd(const kd_bf16* h, const kd_bf16* W, const int32_t* idx,
                               const float* teacher_logp, const float* m_q,
                               int64_t T, int64_t d, int64_t V, int32_t K, kd_mode mode,
                               int32_t chunk, float scale,
                               float* loss, float* loss_tok, float* lse, float* m_p,
                               float* dh, float* dW,
                               void* ws, size_t ws_bytes, void* stream);

/* Bytes of device workspace kd_topk_loss_fwd_bwd_tokblock needs (0 for
 * invalid sizes, or when token_block (rounded up to 256) times V (rounded
 * up to 256) bf16 elements reach 4 GiB).  Linear in T plus the logit block
 * token_block x V x 2 bytes for the dense modes. */
size_t kd_topk_loss_tokblock_workspace(int64_t T, int64_t d, int64_t V, int32_t K, kd_mode mode,
                                       int32_t token_block);

/* kd_topk_loss_fwd_bwd without the backward's recompute: the token-block
 * option of the dense modes (KD_TAIL, KD_FULL, KD_TAIL_REVERSE, KD_REVERSE_TT
 * without sampled tokens).  [FK sec. 4.3] weighs chunking against
 * recomputation: the vocabulary-chunked call evaluates the LM head twice
 * (8 T d V FLOP for a 6 T d V step); here tokens are taken token_block at a
 * time (rounded up to 256) and the block's logits are kept in the
 * workspace as bf16 exp(z - m) (m a per-256-row maximum), so the head is
 * evaluated once and dz = A exp(z - B) is formed from them in place.  The
 * [T, V] logits are never stored: scratch is token_block x V x 2 bytes plus
 * terms linear in T.  dW accumulates over the blocks in the GEMM epilogue
 * (no atomics; outputs are bitwise reproducible).
 *
 * In / out as kd_topk_loss_fwd_bwd (no chunk argument).  The forward
 * outputs (loss, loss_tok, lse, m_p) equal those of kd_topk_loss_fwd_bwd
 * bitwise; dh and dW differ by the rounding of dz (two bf16 roundings
 * instead of one).  The sparse modes (KD_RENORM, KD_REVERSE), which have no
 * dense backward to recompute, take the kd_topk_loss_fwd_bwd path.
 * token_block <= 0 is KD_EINVAL. */
kd_status kd_topk_loss_fwd_bwd_tokblock(const kd_bf16* h, const kd_bf16* W, const int32_t* idx,
                                        const float* teacher_logp, const float* m_q,
                                        int64_t T, int64_t d, int64_t V, int32_t K, kd_mode mode,
                                        int32_t token_block, float scale,
                                        float* loss, float* loss_tok, float* lse, float* m_p,
                                        float* dh, float* dW,
                                        void* ws, size_t ws_bytes, void* stream);

/* Bytes of device workspace kd_topk_loss_fwd_bwd_ce needs (0 for invalid
 * sizes).  A nonzero ce_weight sends every mode through the dense backward. */
size_t kd_topk_loss_ce_workspace(int64_t T, int64_t d, int64_t V, int32_t K, kd_mode mode, int32_t chunk,
                                 float ce_weight);

/* kd_topk_loss_fwd_bwd plus a hard-label cross-entropy term [TG abstract:
 * the top-k student trained with and without the cross-entropy term]:
 *   L_t += ce_weight * (logsumexp(z) - z_y),  dL_t/dz += ce_weight * (p - e_y)
 * for each token with labels[t] = y >= 0.
 *
 * In:  labels    [T] int32  data-token label per token, -1 for none; labels
 *                           >= V are rejected on the device (NaN loss).  May be
 *                           NULL when ce_weight == 0.
 *      ce_weight finite, >= 0; 0 gives exactly kd_topk_loss_fwd_bwd.
 * All other arguments, outputs and errors as kd_topk_loss_fwd_bwd; loss_tok
 * includes the term.  The workspace size comes from kd_topk_loss_ce_workspace. */
kd_status kd_topk_loss_fwd_bwd_ce(const kd_bf16* h, const kd_bf16* W, const int32_t* idx,
                                  const float* teacher_logp, const float* m_q,
                                  const int32_t* labels, float ce_weight,
                                  int64_t T, int64_t d, int64_t V, int32_t K, kd_mode mode,
                                  int32_t chunk, float scale,
                                  float* loss, float* loss_tok, float* lse, float* m_p,
                                  float* dh, float* dW,
                                  void* ws, size_t ws_bytes, void* stream);

/* Tail-corrected top-k reverse KL [TT abstract and Figure 1: the selected
 * top-k tokens plus the token the student sampled, under a stop-gradient,
 * give an unbiased estimate of the full reverse-KL gradient].  Per token,
 * with S the selected tokens (e.g. the student's top-k), a = log p - log q
 * on S, y the sampled token and l = log p_y - log q_y:
 *   L_t   = sum_S p a + [y not in S] l          (unbiased for KL(p || q))
 *   dz    = p (a [v in S] - sum_S p a) + [y not in S] l (e_y - p)
 * dz is the estimator's gradient, sum_S a_v grad p_v + l grad log p_y with
 * a and l held fixed (stop-gradient), not the derivative of L_t: that would
 * add p_u ([u in S] - sum_S p) from differentiating a = log p - log q.
 *
 * In:  idx, teacher_logp  [T, K]  S and log q on S, full-vocabulary normalised
 *      sampled            [T] int32  y per token, -1 for none (no correction);
 *                                    values >= V give a NaN loss
 *      teacher_logp_sampled [T] fp32 log q_y
 * Everything else as kd_topk_loss_fwd_bwd with mode KD_REVERSE_TT (whose
 * workspace size kd_topk_loss_workspace gives). */
kd_status kd_topk_loss_fwd_bwd_tt(const kd_bf16* h, const kd_bf16* W, const int32_t* idx,
                                  const float* teacher_logp, const int32_t* sampled,
                                  const float* teacher_logp_sampled,
                                  int64_t T, int64_t d, int64_t V, int32_t K, int32_t chunk, float scale,
                                  float* loss, float* loss_tok, float* lse, float* m_p,
                                  float* dh, float* dW,
                                  void* ws, size_t ws_bytes, void* stream);

/* kd_topk_loss_fwd_bwd (any mode) when the student's logsumexp and its
 * logits at idx are already known, so the forward pass over the vocabulary
 * is skipped.  The reverse modes choose S as the student's own top-k [TT
 * abstract, Table 2]: kd_topk_cache_build(h, W, NULL, K) returns exactly
 * idx, student_logits (its val) and student_lse (its lse), computed from the
 * same fp32 logits this call would form, so a step that selects and then
 * distils evaluates the student head once for the forward instead of twice.
 *
 * In:  student_lse    [T]    fp32  logsumexp of each token's student logits
 *      student_logits [T, K] fp32  the student's logits at idx, same order
 *                                  (padding slots ignored)
 *      sampled, teacher_logp_sampled  as kd_topk_loss_fwd_bwd_tt (mode
 *                                  KD_REVERSE_TT only), else NULL
 * Everything else, the outputs (lse receives student_lse) and the
 * workspace (kd_topk_loss_workspace) as kd_topk_loss_fwd_bwd.  Values that
 * are not those of h and W give the loss of the values given, not of the
 * model; the backward still uses h and W. */
kd_status kd_topk_loss_fwd_bwd_selected(const kd_bf16* h, const kd_bf16* W, const int32_t* idx,
                                        const float* teacher_logp, const float* m_q,
                                        const float* student_lse, const float* student_logits,
                                        const int32_t* sampled, const float* teacher_logp_sampled,
                                        int64_t T, int64_t d, int64_t V, int32_t K, kd_mode mode,
                                        int32_t chunk, float scale,
                                        float* loss, float* loss_tok, float* lse, float* m_p,
                                        float* dh, float* dW,
                                        void* ws, size_t ws_bytes, void* stream);

/* Bytes of device workspace kd_kl_hidden_fwd_bwd needs (0 for invalid sizes).
 * Linear in T for fixed (d, dt, V, chunk). */
size_t kd_kl_hidden_workspace(int64_t T, int64_t d, int64_t dt, int64_t V, int32_t chunk);

/* Exact full-vocabulary KL(q || p) with the teacher rebuilt from a cached
 * hidden state [TG Fig. 3 bottom: caching the teacher's final hidden state
 * reconstructs its full distribution at 2 dt V FLOP per token]:
 *   q = softmax(U g_t + b), p = softmax(W h_t),
 *   L_t = sum_v q_v (log q_v - log p_v),  dL_t/dz = p - q.
 *
 * In:  h  [T, d]  bf16  student final hidden states
 *      W  [V, d]  bf16  student LM-head rows
 *      g  [T, dt] bf16  cached teacher final hidden states
 *      U  [V, dt] bf16  teacher LM-head rows
 *      b  [V]     fp32  teacher bias, or NULL
 *      d, dt multiples of 64 (<= 16384); chunk as kd_topk_loss_fwd_bwd
 *      (chunk x max(d, dt) bf16, T x max(d, dt) bf16 and T x chunk fp32 each
 *      below 4 GiB); scale: loss = scale * sum_t L_t
 * Out: loss [1], loss_tok [T] or NULL, lse [T] or NULL (student), lse_t [T]
 *      or NULL (teacher), dh [T, d] fp32, dW [V, d] fp32 (fully written).
 * Neither [T, V] logit tensor is stored: both heads are evaluated one
 * vocabulary chunk at a time (twice, forward and backward). */
kd_status kd_kl_hidden_fwd_bwd(const kd_bf16* h, const kd_bf16* W, const kd_bf16* g, const kd_bf16* U,
                               const float* b, int64_t T, int64_t d, int64_t dt, int64_t V,
                               int32_t chunk, float scale,
                               float* loss, float* loss_tok, float* lse, float* lse_t,
                               float* dh, float* dW,
                               void* ws, size_t ws_bytes, void* stream);

/* int8 hidden-state cache [TG Table A2: d + 4 bytes per position]: per
 * position t, scale[t] = max_j |g[t][j]| / 127 and codes[t][j] =
 * rint(g[t][j] / scale[t]) clamped to [-127, 127], computed in fp32 with
 * IEEE division and round-half-even (a zero row: scale 0, zero codes).
 * In: g [T, d] bf16.  Out: codes [T, d] int8, scale [T] fp32.  No workspace. */
kd_status kd_hidden_quantize_int8(const kd_bf16* g, int64_t T, int64_t d, int8_t* codes, float* scale,
                                  void* stream);

/* Bytes of device workspace kd_kl_hidden_int8_fwd_bwd needs (0 for invalid
 * sizes): kd_kl_hidden_workspace plus 2 * T * dt. */
size_t kd_kl_hidden_int8_workspace(int64_t T, int64_t d, int64_t dt, int64_t V, int32_t chunk);

/* kd_kl_hidden_fwd_bwd with the teacher hidden states cached as int8 codes
 * and a per-position scale (kd_hidden_quantize_int8): the teacher logits are
 * scale[t] * (U codes[t]) + b, exact for the quantized states.  Arguments,
 * outputs and errors otherwise as kd_kl_hidden_fwd_bwd. */
kd_status kd_kl_hidden_int8_fwd_bwd(const kd_bf16* h, const kd_bf16* W, const int8_t* codes,
                                    const float* scale_g, const kd_bf16* U, const float* b,
                                    int64_t T, int64_t d, int64_t dt, int64_t V, int32_t chunk, float scale,
                                    float* loss, float* loss_tok, float* lse, float* lse_t,
                                    float* dh, float* dW,
                                    void* ws, size_t ws_bytes, void* stream);

/* The hidden-state KL with the teacher's logsumexp read from the cache
 * instead of recomputed.  [TG Fig. 3] prices the rebuild of the teacher's
 * full distribution from a cached hidden state at one head evaluation
 * (2 dt V FLOP) per token; without a cached normalizer the chunked loss has
 * to evaluate the teacher head twice (once for its logsumexp, once for q).
 * Here it is evaluated once:
 *   teacher_lse [T] fp32  logsumexp_v (U g_t + b)_v, as written to lse_t by an
 *                         earlier kd_kl_hidden_fwd_bwd / _int8_fwd_bwd call on
 *                         the same cached states, U and b (q is formed as
 *                         exp(U g_t + b - teacher_lse_t); a different value
 *                         leaves q unnormalized and the result is not the KL)
 * The teacher states are given either as g [T, dt] bf16 (codes, scale_g
 * NULL; workspace kd_kl_hidden_workspace) or as int8 codes [T, dt] with
 * scale_g [T] (g NULL; workspace kd_kl_hidden_int8_workspace).  lse_t, if not
 * NULL, receives teacher_lse.  Other arguments, outputs and errors as
 * kd_kl_hidden_fwd_bwd. */
kd_status kd_kl_hidden_cached_lse_fwd_bwd(const kd_bf16* h, const kd_bf16* W, const kd_bf16* g,
                                          const int8_t* codes, const float* scale_g, const kd_bf16* U,
                                          const float* b, const float* teacher_lse, int64_t T, int64_t d,
                                          int64_t dt, int64_t V, int32_t chunk, float scale,
                                          float* loss, float* loss_tok, float* lse, float* lse_t,
                                          float* dh, float* dW, void* ws, size_t ws_bytes, void* stream);

/* Bytes of device workspace kd_topk_cache_build needs.  Returns 0 for
 * invalid sizes. */
size_t kd_topk_cache_build_workspace(int64_t T, int64_t d, int64_t V, int32_t K, int32_t n_rho);

/* Teacher-cache build [TG Fig. 3; FK sec. 3.2; SS]: z = U g + b per token,
 * then per row the top-K logits, logsumexp, tail mass and adaptive k_rho.
 *
 * In:  g        [T, d] bf16   teacher final hidden states
 *      U        [V, d] bf16   teacher LM-head rows
 *      b        [V]    fp32   bias, or NULL for none
 *      K        entries kept per token (1 <= K <= min(V, 1024))
 *      rho_host [n_rho] fp32  HOST array of target masses in (0, 1], or NULL
 *               when n_rho == 0 (0 <= n_rho <= 8)
 * Out: idx      [T, K] int32  retained indices, ordered by logit descending,
 *                             ties to the lower index (-0.0 ties with +0.0)
 *      val      [T, K] fp32   the fp32 logits z at idx (bitwise)
 *      lse      [T]    fp32   logsumexp of z
 *      m_q      [T]    fp32   1 - sum_{top-K} exp(val - lse), the tail mass
 *      k_rho    [T, n_rho] int32  smallest k whose top-k mass reaches rho[j]
 *               over the full row (may exceed K), or NULL when n_rho == 0
 *      teacher_logp [T, K] fp32  the cached teacher log-probabilities
 *               val - lse at idx, the loss's teacher_logp input, rounded to
 *               fp32 from the fp64 difference with the row's fp64
 *               logsumexp [TG Fig. 3: the top-k cache; FK sec. 3.2: the
 *               cached top-K teacher values feed the loss]; or NULL (not
 *               written) */
kd_status kd_topk_cache_build(const kd_bf16* g, const kd_bf16* U, const float* b,
                              int64_t T, int64_t d, int64_t V, int32_t K,
                              const float* rho_host, int32_t n_rho,
                              int32_t* idx, float* val, float* lse, float* m_q, int32_t* k_rho,
                              float* teacher_logp, void* ws, size_t ws_bytes, void* stream);

/* Bytes of device workspace kd_topk_rows needs (0 for invalid sizes): 4
 * bytes per row (fallback flags) rounded up to 256, and with k_rho targets
 * (n_rho > 0, V < 2^18) a record of 240 bytes per row plus 4 KiB per row and
 * target for the crossing bins whose count and mass do not pin k_rho (those
 * rows are finished by a second launch that reads them with several
 * workgroups). */
size_t kd_topk_rows_workspace(int64_t T, int64_t V, int32_t K, int32_t n_rho);

/* The row pass of the cache build on caller-provided fp32 logits z [T, V]
 * (no NaN) [TG Fig. 3: keep the k largest teacher logits of each row, with
 * the discarded tail mass; SS: the adaptive support k_rho]: same outputs
 * (teacher_logp may be NULL) and ordering rules as kd_topk_cache_build.  On
 * identical fp32 inputs the selected indices and values are exact.  ws must
 * be 16-byte aligned and hold kd_topk_rows_workspace(T, V, K, n_rho) bytes
 * (KD_ENOWS otherwise); its contents need no initialization. */
kd_status kd_topk_rows(const float* z, int64_t T, int64_t V, int32_t K,
                       const float* rho_host, int32_t n_rho,
                       int32_t* idx, float* val, float* lse, float* m_q, int32_t* k_rho,
                       float* teacher_logp, void* ws, size_t ws_bytes, void* stream);

/* kd_topk_rows for callers that cannot allocate device memory (code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc):
 * no workspace argument; the per-row fallback flags live in a static
 * device array of the library (1,048,576 rows, 4 MiB per device, held
 * until the process ends).  Calls nothing that allocates.
 * Same inputs, outputs and results as kd_topk_rows; T above 1,048,576 is
 * refused with KD_EUNSUPPORTED.  The array is the current device's: all
 * calls on one device share it, and every call rewrites the flags of its
 * rows before reading them, so calls in stream order are independent;
 * calls that overlap on one device (two streams, or two host threads at
 * once) race on it and must not be issued. */
kd_status kd_topk_rows_noalloc(const float* z, int64_t T, int64_t V, int32_t K,
                               const float* rho_host, int32_t n_rho,
                               int32_t* idx, float* val, float* lse, float* m_q, int32_t* k_rho,
                               float* teacher_logp, void* stream);

/* Teacher hidden-state recovery from k cached log-probabilities [TG abstract
 * and Table 1: the retained set determines the teacher's distribution from
 * k = d + 1 on].  Per position t, the least-squares solution of
 *   [U_S, -1] (g; c) = teacher_logp_S - b_S,   S = idx[t, :]
 * in fp64 (Householder QR), g the teacher's final hidden state and c its
 * logsumexp; softmax(U g + b) is then the full teacher distribution.
 *
 * In:  idx          [T, k] int32  cached indices (distinct, in [0, V))
 *      teacher_logp [T, k] fp32   cached teacher log-probabilities at idx
 *      U            [V, d] bf16   teacher LM-head rows;  b [V] fp32 or NULL
 *      d + 1 <= k <= V and (d + 2) * (k rounded up to odd) <= 19968
 *      (KD_EUNSUPPORTED otherwise: one workgroup holds the system in LDS)
 * Out: g_hat [T, d] fp32, c_hat [T] fp32; NaN for a position whose indices
 *      are out of range (and non-finite values when [U_S, -1] is singular). */
kd_status kd_teacher_recover(const int32_t* idx, const float* teacher_logp, const kd_bf16* U, const float* b,
                             int64_t T, int64_t d, int64_t V, int32_t k, float* g_hat, float* c_hat,
                             void* stream);

/* Bytes of device workspace kd_teacher_recover_ws needs (0 for invalid
 * sizes): per position one fp64 copy of the system (max(k, d+1) rows, even
 * pitch) plus four fp64 vectors, and one int32 flag. */
size_t kd_teacher_recover_workspace(int64_t T, int64_t d, int32_t k);

/* kd_teacher_recover at the widths of real teachers (d in the thousands;
 * k and d + 2 up to 65,536), with the system in a caller-owned workspace
 * and solved by many workgroups [TG abstract and Table 1: from k = d + 1
 * cached log-probabilities on, the teacher's distribution is determined].
 * Per position, fp64:
 *   k >= d + 1: the least-squares solution of [U_S, -1] (g; c) = log q_S - b_S
 *               by Householder QR (column by column, every trailing column
 *               updated in parallel) and back substitution;
 *   k <= d:     the system is underdetermined (the teacher is not
 *               identifiable from S): the minimum-norm solution, by
 *               Householder QR of the transposed system, R^T w = y and
 *               x = Q [w; 0].
 * In / out as kd_teacher_recover (1 <= k <= V; at most 65,535 positions per
 * call); ws of kd_teacher_recover_workspace(T, d, k) bytes, 8-byte aligned.
 * Non-finite outputs when the system is singular; NaN for a position with an
 * index out of range. */
kd_status kd_teacher_recover_ws(const int32_t* idx, const float* teacher_logp, const kd_bf16* U, const float* b,
                                int64_t T, int64_t d, int64_t V, int32_t k, float* g_hat, float* c_hat,
                                void* ws, size_t ws_bytes, void* stream);

/* Message describing the last non-KD_OK status returned on this thread. */
const char* kd_last_error(void);

/* Launch profiler (diagnostics).  After kd_profile_begin(), every kernel the
 * library enqueues from this thread is bracketed by a pair of HIP events on
 * its stream.  kd_profile_end() waits for those events, stops recording and
 * reports, per distinct kernel name (at most max_kernels entries), the summed
 * event time in milliseconds and the launch count; it returns the number of
 * distinct kernels.  names[i] point to static strings.  Any pointer may be
 * NULL.  Not for use inside HIP graph capture. */
kd_status kd_profile_begin(void);
int32_t kd_profile_end(int32_t max_kernels, const char** names, float* total_ms, int32_t* launches);

/* Library version string. */
const char* kd_version(void);

#ifdef __cplusplus
}
#endif
#endif /* KDTOPK_H */
