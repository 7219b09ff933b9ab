/*
 * atlasmem -- the neural-memory test-time update and retrieval (Titans / ATLAS)
 * on one MI355X (gfx950), behind a plain C ABI.
 *
 * What is computed (per memory m = (b, h), all memories independent):
 *
 *   memory     M_W(x) = W x                      (LINEAR, W: d_value x d_in)
 *              M_W(x) = W2 silu(W1 x)            (MLP2_SILU, W1: d_hidden x d_in,
 *                                                 W2: d_value x d_hidden)
 *              M_W(x) = x + W2 silu(W1 x)        (MLP2_SILU_RESIDUAL, d_in == d_value: the
 *                                                 default memory of ATLAS, "ATLAS ... |
 *                                                 Summary", section 5.1)
 *              M_W(x) = W2 (silu(W1 x) * (W3 x)) (MLP2_GATED, W3 like W1: the gated memory
 *                                                 of ATLAS++, same section; parameters
 *                                                 [W1 | W3 | W2])
 *   loss       l(W; x, v) = ||M_W(x) - v||^2      -- "Titans: Learning to Memorize at
 *              Test Time" (titans-pytorch-mlx README), Core Equations, Eq. 12
 *   momentum   S_t = eta_t S_{t-1} - theta_t G_t  -- same page, Eq. 14
 *   forgetting W_t = (1 - alpha_t) W_{t-1} + S_t  -- same page, Eq. 13; titans-torch
 *              0.1.2 (PyPI), API Reference, inner-loop update rule
 *   chunks     the sequence is cut into chunks of `chunk` tokens; every gradient of a
 *              chunk is taken at the chunk-start weights and every query of the chunk
 *              is answered with them, y_t = M_{W_start}(phi(q_t)) ("ATLAS: Learning to
 *              Optimally Memorize the Context at Test Time | Summary", section 3.3;
 *              titans-pytorch-mlx README, MAC Eq. 21)
 *   Omega      G_t = sum_{i=t-c+1..t} gamma_i grad l(W_start; phi(k_i), v_i) for a
 *              window c > 1 (gamma_i per token; the window crosses chunk boundaries and
 *              is clipped only at the start of the sequence); G_t = grad l(...; k_t, v_t)
 *              for c = 1 (ATLAS summary, section 3.2; Atlas-Torch README, Atlas
 *              Extensions table, Omega Rule)
 *   features   phi(x) = [1, x_i, x_i x_j / 2 (i <= j)] in combinations_with_replacement
 *              order, C(d_key + 2, 2) features, for poly_degree = 2 (Atlas-Torch README,
 *              Atlas Extensions table, Polynomial Features); identity for poly_degree = 1
 *   per chunk  (gate_mode = PER_CHUNK) one summed gradient G_c per chunk, optionally
 *              orthogonalised per weight matrix by ns_steps quintic Newton-Schulz
 *              iterations X <- aX + (b A + c A^2) X, A = X X^T, on X0 = G/(||G||_F + eps)
 *              in the orientation with rows <= cols, then S_c = eta_c S - theta_c NS(G_c),
 *              W_c = (1 - alpha_c) W + S_c (Atlas-Torch README, Atlas Extensions table,
 *              Muon / Newton-Schulz; Bug Fixes table, no-omega ablation row)
 *
 * Conventions for every call:
 *   - Every array pointer is a DEVICE pointer (HIP device memory on the handle's
 *     device) unless stated otherwise; the caller owns it.  Arrays are dense and
 *     row-major with the shapes given below; M = batch * heads, memory m = b*heads + h.
 *   - `stream` is a hipStream_t passed as void* (NULL = the default stream).  Work is
 *     enqueued on it asynchronously; a call returns once its work is enqueued.
 *   - Status codes are returned synchronously.  Argument and shape errors are
 *     detected before anything is enqueued and leave the handle unchanged.
 *   - A handle is not re-entrant: calls on one handle must not overlap; distinct
 *     handles are independent.
 */
#ifndef ATLASMEM_H
#define ATLASMEM_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define ATLASMEM_ABI_VERSION 2

typedef enum {
  ATLASMEM_OK = 0,
  ATLASMEM_E_INVALID = 1,      /* null pointer, negative size, bad enum value, wrong abi_version */
  ATLASMEM_E_SHAPE = 2,        /* sizes beyond the stated limits; stand-alone stages: T % chunk */
  ATLASMEM_E_UNSUPPORTED = 3,  /* a valid but unsupported combination of options                  */
  ATLASMEM_E_DEVICE = 4,       /* no usable gfx950 device, or a HIP runtime / launch error        */
  ATLASMEM_E_NOMEM = 5,        /* device allocation failed (create only)                          */
  ATLASMEM_E_NONFINITE = 6     /* a state element became NaN/Inf (reported by get_state)          */
} atlasmem_status;

typedef enum {
  ATLASMEM_LINEAR = 0,
  ATLASMEM_MLP2_SILU = 1,
  ATLASMEM_MLP2_SILU_RESIDUAL = 2,
  ATLASMEM_MLP2_GATED = 3
} atlasmem_memory_kind;
typedef enum { ATLASMEM_PER_TOKEN = 0, ATLASMEM_PER_CHUNK = 1 } atlasmem_gate_mode;
typedef enum { ATLASMEM_F32 = 0, ATLASMEM_BF16 = 1 } atlasmem_dtype;

/* Operand precision of the matrix-core products (state and accumulation are fp32 always).
 * BF16X3 splits every fp32 operand x into hi = bf16(x), lo = bf16(x - hi) and sums
 * hi*hi + hi*lo + lo*hi (two products where one side is an exact bf16 input).
 * F32 keeps every operand in fp32 (the matrix cores' fp32 path, v_mfma_f32_16x16x4_f32, and
 * fp32 fused multiply-adds for Newton-Schulz): for inputs whose rounding the Newton-Schulz
 * feedback amplifies beyond what the split holds (e.g. keys that are not normalised); it runs the
 * general per-product path only (no fused whole-call kernel, no chunk loop, no decode kernel) and
 * the outer-loop backward of the 2-layer memories rejects it (E_UNSUPPORTED).
 * AUTO = BF16X3.  The linear memory always runs in fp32 FMA. */
typedef enum {
  ATLASMEM_PREC_AUTO = 0,
  ATLASMEM_PREC_BF16 = 1,
  ATLASMEM_PREC_BF16X3 = 2,
  ATLASMEM_PREC_F32 = 3
} atlasmem_precision;

typedef struct {
  int32_t abi_version;   /* ATLASMEM_ABI_VERSION                                           */
  int32_t memory_kind;   /* atlasmem_memory_kind                                            */
  int32_t batch;         /* B >= 1                                                          */
  int32_t heads;         /* H >= 1                                                          */
  int32_t d_key;         /* raw key/query width, 1..1024                                    */
  int32_t d_value;       /* value width, 1..1024                                            */
  int32_t d_hidden;      /* MLP hidden width, 1..4096 (ignored for LINEAR)                  */
  int32_t poly_degree;   /* 1 (identity) or 2 (degree <= 2 monomials, 1/deg!)               */
  int32_t chunk;         /* tokens per chunk, 1..1024                                       */
  int32_t omega_window;  /* c >= 1, c <= 64                                                 */
  int32_t gate_mode;     /* atlasmem_gate_mode                                              */
  int32_t ns_steps;      /* 0 (none) or 1..16 Newton-Schulz iterations (PER_CHUNK only)     */
  float ns_a, ns_b, ns_c;/* quintic coefficients (Muon: 3.4445, -4.7750, 2.0315)            */
  float ns_eps;          /* added to ||G||_F before normalising (e.g. 1e-7)                 */
  int32_t input_dtype;   /* atlasmem_dtype of K, Q, V                                       */
  int32_t output_dtype;  /* atlasmem_dtype of Y                                             */
  int32_t precision;     /* atlasmem_precision                                              */
  int32_t flags;         /* bit set of ATLASMEM_FLAG_* (0 = defaults)                       */
} atlasmem_config;

/* Force the general per-chunk kernel sequence even where a fused whole-call kernel exists
 * (the fused kernels cover the 64 -> 128 -> 64 MLP memory, plain, residual or gated, with
 * per-chunk gates and Newton-Schulz, bf16 inputs, split precision, and the plain or residual one
 * with per-token gates in chunks of 64).  Results agree within rounding. */
#define ATLASMEM_FLAG_NO_FUSED 1
/* Per-token retrieval: Y[t] = M_{W_t}(phi(Q[t])) with W_t the state right after token t's
 * update, instead of the chunk-start weights (Atlas-Torch README, "Known deviations from the
 * paper's MAC": the Atlas configuration reads the post-update per-token state).  Per-token gates
 * only (E_UNSUPPORTED otherwise).  No per-token weights are formed: inside a chunk W_t is the
 * chunk-start state plus a masked sum of the chunk's rank-one gradients, so the queries are
 * answered through query-key score products.  Streaming calls (tokens of an unfinished chunk)
 * are answered from the buffered rows of that chunk, which W_t depends on alone, so decoding
 * equals one call (Atlas-Torch README, "Status and scope", limitation 4: the decode path must read
 * the state the parallel path reads); for the LINEAR memory such calls return E_UNSUPPORTED. */
#define ATLASMEM_FLAG_PER_TOKEN_RETRIEVE 2
/* Run the chunks of a call as one separate launch per matrix product (five per chunk) instead of
 * the chunk-loop kernel, which walks every chunk of a block inside one launch with one workgroup
 * per memory and is used where a memory's per-chunk products are small (the general MLP path
 * with per-token gates, or per-chunk gates without Newton-Schulz).  Both compute the same
 * products and epilogues; results agree to rounding. */
#define ATLASMEM_FLAG_NO_CHUNK_LOOP 4
/* Run every matrix product of the per-product launches over its whole k range in one launch.
 * By default a product with few 64 x 64 output tiles and a long k range (the first-layer
 * product of degree-2 features, the wide memory's output products) is split into k-slices whose
 * partial tiles a second launch sums in slice order, so the slices' global-load round trips run
 * in parallel.  Results agree to rounding. */
#define ATLASMEM_FLAG_NO_SPLIT_K 8

typedef struct atlasmem_handle_s* atlasmem_handle;

/* Parameter count P per memory: d_value*d_in (LINEAR) or d_hidden*d_in + d_value*d_hidden,
 * with d_in = d_key (poly_degree 1) or C(d_key + 2, 2) (poly_degree 2).  The state layout
 * of one memory is W1 (row-major) followed by W2 (row-major); LINEAR: W.  Returns -1 for an
 * invalid config. */
int64_t atlasmem_param_count(const atlasmem_config* cfg);

int atlasmem_abi_version(void);
const char* atlasmem_status_string(int status);

/* Validates `cfg`, selects the device's kernels, allocates every buffer the handle will
 * need (state, momentum, window history, per-chunk workspace) and copies the initial
 * state in, ordered on `stream`.
 *   W0: [M, P] fp32 initial weights, or NULL for zeros.
 *   S0: [M, P] fp32 initial momentum, or NULL for zeros.
 * The window history starts empty (start of a sequence).  The handle is bound to the
 * device current at the call.  On error *out is set to NULL and nothing is leaked. */
atlasmem_status atlasmem_create(const atlasmem_config* cfg, const float* W0, const float* S0,
                                void* stream, atlasmem_handle* out);

/* Consumes T >= 0 tokens of every memory.  Tokens are grouped into chunks of cfg.chunk in
 * stream order across calls (titans-pytorch-mlx README, Core Equations, Eq. 12-14 with the
 * gradients of a chunk at its start weights; ATLAS summary, section 3.3): every token's
 * retrieved row Y = M_{W_start}(phi(Q)) uses the weights at the start of its chunk, and (W, S)
 * advance each time a chunk is complete.  The tokens of an unfinished chunk are buffered by the
 * handle (their Y is written by this call), so the result does not depend on how a sequence is
 * cut into calls: token-by-token decoding equals one call over the whole sequence.  A final
 * partial chunk is applied by atlasmem_flush.  The window history (last c - 1 keys, values and
 * gammas) carries over likewise.
 *   K, Q:  [M, T, d_key]   input_dtype
 *   V:     [M, T, d_value] input_dtype
 *   theta, eta, alpha: fp32 [M, T] (PER_TOKEN), or [M, n] (PER_CHUNK) with n the number of
 *          chunks this call completes, (pending + T) / chunk; may be NULL when n = 0
 *   gamma: fp32 [M, T] for omega_window > 1, must be NULL for omega_window == 1
 *   Y:     [M, T, d_value] output_dtype, or NULL to skip retrieval
 * Never allocates. */
atlasmem_status atlasmem_update_chunked(atlasmem_handle h, const void* K, const void* Q, const void* V,
                                        const float* theta, const float* eta, const float* alpha,
                                        const float* gamma, int64_t T, void* Y, void* stream);

/* The causal short convolution of the keys, queries and values (kernel 4, depthwise, one filter per
 * (head, channel); keys and queries optionally L2-normalised after it) folded into the update:
 * Atlas-Torch README, Atlas Extensions table, "Short Convolution"; titans-pytorch-mlx README,
 * Configuration table (use_conv, conv_kernel_size 4).  Tap j multiplies token t - 3 + j, exactly as
 * atlasmem_short_conv below. */
typedef struct atlasmem_short_conv_params_s {
  const float* taps_k;  /* [heads, d_key, 4] fp32 (device, 16-byte aligned; likewise taps_q, v) */
  const float* taps_q;  /* [heads, d_key, 4]                                                      */
  const float* taps_v;  /* [heads, d_value, 4]                                                    */
  const float* bias_k;  /* [heads, d_key] fp32 or NULL (zero); bias_q, bias_v likewise            */
  const float* bias_q;
  const float* bias_v;
  int32_t l2norm_k;     /* 1: each convolved key row divided by max(its L2 norm, 1e-12)           */
  int32_t l2norm_q;     /* the same for the query rows (values are never normalised)              */
} atlasmem_short_conv_params;

/* atlasmem_update_chunked on the convolved rows without writing them: given the RAW rows K, Q, V,
 * the update reads conv(K), conv(Q), conv(V) (fp32 arithmetic, the normalisation, one rounding to
 * input_dtype: the rows atlasmem_short_conv would produce) while staging each chunk's operands,
 * so only a 4-byte inverse norm per key and query row passes through memory.  The handle carries
 * the three raw rows before the next call of each tensor (zeros at the start of a sequence and
 * after atlasmem_reset_history), so a sequence cut into calls gives the same result as one call.
 * Scope: the 2-layer memories (plain, residual, gated) without per-token retrieval, d_key and
 * d_value <= 512, calls of whole chunks with nothing pending (E_UNSUPPORTED otherwise); runs the
 * general per-product path.  Arguments as atlasmem_update_chunked; Q is required; `conv` is a
 * HOST pointer to the parameters.  Never allocates. */
atlasmem_status atlasmem_update_chunked_conv(atlasmem_handle h, const void* K, const void* Q, const void* V,
                                             const atlasmem_short_conv_params* conv, const float* theta,
                                             const float* eta, const float* alpha, const float* gamma, int64_t T,
                                             void* Y, void* stream);

/* Applies the buffered tokens of an unfinished chunk (r = atlasmem_pending(h) > 0 of them) as
 * one final chunk of r tokens, e.g. at the end of a sequence; no-op when none are buffered.
 *   theta, eta, alpha: PER_CHUNK: fp32 [M, 1], the gates of that chunk; PER_TOKEN: ignored (the
 *   buffered per-token gates are used), may be NULL.
 * Never allocates. */
atlasmem_status atlasmem_flush(atlasmem_handle h, const float* theta, const float* eta, const float* alpha,
                               void* stream);

/* Tokens of the unfinished chunk buffered by the handle (0 .. chunk - 1); -1 for NULL. */
int64_t atlasmem_pending(atlasmem_handle h);

/* Retrieval with no update (titans-torch 0.1.2, forward(): inference without updating the
 * memory): Y[m, t] = M_W(phi(Q[m, t])) with the current weights, for T >= 0 tokens.
 *   Q: [M, T, d_key] input_dtype;  Y: [M, T, d_value] output_dtype.  Never allocates. */
atlasmem_status atlasmem_retrieve(atlasmem_handle h, const void* Q, int64_t T, void* Y, void* stream);

/* Copies the current weights / momentum out to W, S ([M, P] fp32 device arrays; either may be
 * NULL).  Synchronises `stream` to read the device's non-finite flag and returns
 * E_NONFINITE if any update since create / set_state produced a NaN or Inf (the copies are
 * still made). */
atlasmem_status atlasmem_get_state(atlasmem_handle h, float* W, float* S, void* stream);

/* Replaces the weights / momentum ([M, P] fp32 device arrays; NULL = zeros) and clears the
 * non-finite flag.  The window history and any buffered tokens are left as they are. */
atlasmem_status atlasmem_set_state(atlasmem_handle h, const float* W, const float* S, void* stream);

/* Forgets the window history and any buffered tokens of an unfinished chunk (start of a new
 * sequence).  State is unchanged. */
atlasmem_status atlasmem_reset_history(atlasmem_handle h, void* stream);

/* Waits for the handle's work and frees everything it owns.  NULL is a no-op. */
void atlasmem_destroy(atlasmem_handle h);

/* For callers that cannot allocate device memory (code under HIP graph capture, tight serving
 * loops, harnesses that forbid hipMalloc): atlasmem_update_chunked without a handle, for the
 * configurations the fused whole-call kernel covers (the 64 -> 128 -> 64 SiLU memory, plain or
 * residual, PER_CHUNK gates, ns_steps >= 1, window 1, poly_degree 1, bf16 inputs, AUTO / BF16X3
 * precision, chunk a multiple of 64, flags 0; E_UNSUPPORTED otherwise, the gated memory
 * included).  Same results as update_chunked from the same state over the same tokens, bit for
 * bit (the handle may run each memory over two workgroups, this entry point one).
 *   cfg:   validated as by atlasmem_create (batch * heads <= ATLASMEM_STATIC_MAX_MEMORIES, else
 *          E_SHAPE)
 *   K, Q, V, theta, eta, alpha, Y: as in atlasmem_update_chunked, with T a multiple of the chunk
 *          (E_SHAPE otherwise; no tokens are buffered between calls)
 *   W, S:  [M, P] fp32 device arrays, the weights and momentum before the call, overwritten in
 *          place with the state after it
 *   nonfinite: optional device int32, set to 1 if a state element became NaN/Inf, else 0
 * The kernel's per-memory scratch (the second-layer state between chunks, 64 KB per memory) lives
 * in a static device array of the library: at most ATLASMEM_STATIC_MAX_MEMORIES memories (8 MB per
 * device, held from the first call on a device until the process ends).  Nothing is allocated;
 * the first call on a device looks the array's address up once.  Every call on one GPU shares that
 * array, so calls that overlap on one GPU (concurrent streams or threads) race and must be
 * serialised by the caller. */
#define ATLASMEM_STATIC_MAX_MEMORIES 128
atlasmem_status atlasmem_update_chunked_static(const atlasmem_config* cfg, const void* K, const void* Q,
                                               const void* V, const float* theta, const float* eta,
                                               const float* alpha, int64_t T, float* W, float* S, void* Y,
                                               int32_t* nonfinite, void* stream);

/* ---------------------------------------------------------------------------------------
 * Stand-alone stages of the path (the same kernels the update runs), for callers that
 * want one stage and for measuring each against its own roofline.  Device pointers,
 * asynchronous on `stream`.
 * ------------------------------------------------------------------------------------- */

/* Gate scan over the chunk-internal recurrence (derived from Eq. 13-14 with all gradients
 * of a chunk at the chunk-start weights).  For every memory and chunk [s, s+C) of the
 * per-token gates theta, eta, alpha ([M, T] fp32, T a multiple of C):
 *   e_j = prod_{l=j+1..C} eta_l,  b_j = prod_{l=j+1..C} (1 - alpha_l),
 *   w_C = 1, w_j = b_j + eta_{j+1} w_{j+1},
 *   cS[m, s+j] = theta_j e_j,  cW[m, s+j] = theta_j w_j            ([M, T] fp32)
 *   chunk_scalars[m, k, 0..2] = (prod eta, prod (1 - alpha), eta_1 w_1)   ([M, T/C, 3])
 * so that S_end = P S_0 - sum_j cS_j g_j and W_end = beta W_0 + a_S S_0 - sum_j cW_j g_j. */
atlasmem_status atlasmem_gate_scan(const float* theta, const float* eta, const float* alpha, int64_t M,
                                   int64_t T, int32_t chunk, float* cW, float* cS, float* chunk_scalars,
                                   void* stream);

/* Omega window coefficients: for chunk k = [s, s+C) and row r in [0, C + c - 1), token
 * i = s - (c - 1) + r (ATLAS summary, section 3.2):
 *   oW[m, k, r] = gamma_i * sum_{t = max(i, s)}^{min(i + c - 1, s + C - 1)} cW[m, t]   (same for oS)
 * gamma: [M, T]; tokens before 0 take gamma from `gamma_hist` ([M, c-1], the c - 1 tokens
 * before this T, oldest first; NULL = none, i.e. the start of the sequence, weight 0).
 * cW, cS: [M, T];  oW, oS: [M, T/C, C + c - 1] fp32. */
atlasmem_status atlasmem_omega_coeffs(const float* cW, const float* cS, const float* gamma,
                                      const float* gamma_hist, int64_t M, int64_t T, int32_t chunk,
                                      int32_t window, float* oW, float* oS, void* stream);

/* Polynomial feature map phi (poly_degree 2) of n vectors of width d (1..1024):
 *   X: [n, d] (in_dtype),  F: [n, C(d+2, 2)] fp32 (exact: every monomial of bf16 inputs
 *   is representable in fp32). */
atlasmem_status atlasmem_poly_features(const void* X, int32_t in_dtype, int64_t n, int32_t d, float* F,
                                       void* stream);

/* Newton-Schulz orthogonalisation of n_mat independent rows x cols fp32 matrices
 * (G, out: [n_mat, rows, cols]; out may not alias G), with the handle-free semantics of
 * the per-chunk path above.  precision as in atlasmem_config.  Never allocates when
 * rows, cols <= 128 and min(rows, cols) <= 64; larger matrices return E_UNSUPPORTED. */
atlasmem_status atlasmem_newton_schulz(const float* G, int64_t n_mat, int32_t rows, int32_t cols,
                                       int32_t steps, float a, float b, float c, float eps,
                                       int32_t precision, float* out, void* stream);

/* Outer-loop backward (the training path): runs the update over T tokens exactly as
 * atlasmem_update_chunked does (advancing the handle's state and writing Y when Y != NULL), and
 * returns the gradients of an outer loss L, given dY = dL/dY and the adjoints dW_T, dS_T of the
 * final state, with respect to every input of the update and the state it started from
 * (Atlas-Torch README, "How the memory works": the outer loop trains through the inner updates;
 * the derivative of the recurrence includes that of the inner gradient).
 * Scope: every memory kind without per-token retrieval, with either PER_TOKEN gates (ns_steps 0),
 * any Omega window and poly_degree 1 or 2 (gradients reach the raw keys and queries through the
 * feature map), or, for the 2-layer memories, PER_CHUNK gates (window 1, poly_degree 1) with or
 * without the Newton-Schulz orthogonalisation of the chunk gradient (its iteration
 * differentiated step by step) (E_UNSUPPORTED otherwise).  With a window > 1 the c - 1 rows of
 * window history the call starts with are constants of the call: gradients flow to this call's
 * tokens only (ATLAS summary, sections 3.2-3.3: the Omega rule over a sliding window);
 * T a multiple of the chunk and nothing pending (E_SHAPE otherwise).
 *   theta, eta, alpha: as in atlasmem_update_chunked ([M, T] per token, [M, T/C] per chunk)
 *   gamma: fp32 [M, T], the Omega-rule gates (window > 1; ignored, may be NULL, otherwise)
 *   dY: fp32 [M, T, d_value];  dW_T, dS_T: fp32 [M, P] or NULL (zero)
 *   workspace: device memory of atlasmem_backward_workspace_bytes(h, T) bytes (the chunk-start
 *          states of the forward and the backward's buffers); the call allocates nothing
 *   dK, dQ: fp32 [M, T, d_key]; dV: fp32 [M, T, d_value];
 *   dtheta, deta, dalpha: fp32, the gates' shape ([M, T] or [M, T/C]); dgamma: fp32 [M, T]
 *          (window > 1; may be NULL otherwise);
 *   dW0, dS0: fp32 [M, P] (gradients with respect to the state at the start of the call) */
int64_t atlasmem_backward_workspace_bytes(atlasmem_handle h, int64_t T);
atlasmem_status atlasmem_update_backward(atlasmem_handle h, const void* K, const void* Q, const void* V,
                                         const float* theta, const float* eta, const float* alpha,
                                         const float* gamma, int64_t T, void* Y, const float* dY,
                                         const float* dW_T, const float* dS_T, void* workspace,
                                         int64_t workspace_bytes, float* dK, float* dQ, float* dV, float* dtheta,
                                         float* deta, float* dalpha, float* dgamma, float* dW0, float* dS0,
                                         void* stream);

/* Feature map of n rows of width d: every monomial of degree 0..degree (degree 1..3), degree-major
 * and in combinations_with_replacement order inside a degree, the degree-k monomials multiplied
 * by coeffs[k] -- and, with P, projected back (Atlas-Torch README, Atlas Extensions table,
 * "Polynomial Features": exact monomial expansion, learnable coefficients initialised to 1/d!,
 * optional project_back; ATLAS summary, section 4.3: Dot pairs these exponential-kernel features
 * with the Omega rule, which the update then applies to the mapped rows).
 *   X:      [n, d] in_dtype (d <= 1024, C(d + degree, degree) <= 2^20 features)
 *   coeffs: HOST pointer to degree + 1 floats, or NULL for 1/k!
 *   P:      fp32 [d_out, C(d + degree, degree)] (device) or NULL; d_out <= 65536
 *   out:    fp32 [n, d_out] = phi_c(X) P^T, or [n, C(d + degree, degree)] = phi_c(X) without P
 * With P the product runs on the matrix cores in split bf16 (hi/lo) with fp32 accumulation.
 * Errors: E_INVALID for bad sizes, dtype or null pointers; E_SHAPE beyond the limits. */
atlasmem_status atlasmem_feature_map(const void* X, int32_t in_dtype, int64_t n, int32_t d, int32_t degree,
                                     const float* coeffs, const float* P, int32_t d_out, float* out,
                                     void* stream);

/* ---------------------------------------------------------------------------------------
 * Input prologue: the steps just before the update, producing its K, Q, V and gates.
 * ------------------------------------------------------------------------------------- */

/* Causal depthwise short convolution, kernel 4, along the token axis, one filter per (head,
 * channel), for keys, queries or values (Atlas-Torch README, Atlas Extensions table, "Short
 * Convolution"; titans-pytorch-mlx README, Configuration table, use_conv / conv_kernel_size 4):
 *   out[m, t, i] = bias[h, i] + sum_{j=0..3} taps[h, i, j] * X[m, t - 3 + j, i],  h = m % heads
 * then, with l2norm = 1, each output row divided by max(its L2 norm, 1e-12) (keys, queries).
 *   X:     [M, T, d] in_dtype (d 1..512); memory m = b * heads + h
 *   taps:  fp32 [heads, d, 4];  bias: fp32 [heads, d] or NULL (zero)
 *   hist:  [M, 3, d] in_dtype, the three rows before token 0 (oldest first), or NULL (the
 *          start of a sequence: zeros)
 *   out:   [M, T, d] out_dtype (fp32 arithmetic, one rounding to bf16); must not overlap X
 *   hist_out: [M, 3, d] in_dtype or NULL: the three rows before the next call's first token (the
 *          last three of hist ++ X), for streaming; must not overlap X or hist
 * T = 0 is valid (only hist_out is written).  Errors: E_INVALID for bad sizes, enums, null or
 * overlapping pointers; E_SHAPE for d > 512. */
atlasmem_status atlasmem_short_conv(const void* X, int32_t in_dtype, int64_t M, int64_t T, int32_t d,
                                    int32_t heads, const float* taps, const float* bias, const void* hist,
                                    int32_t l2norm, void* out, int32_t out_dtype, void* hist_out, void* stream);

/* Data-dependent gates (titans-pytorch-mlx README, Key Innovations item 4, and the
 * Configuration table: memory_lr 0.1, memory_momentum 0.9, memory_decay 0.01, each scaled by a
 * gate; titans-torch 0.1.2, "Inner-loop update rule"): for gate g (e.g. theta, eta, alpha and
 * the Omega gamma), head h and token t of sequence b,
 *   out[g, b, h, t] = scale[g] * sigmoid(Wg[g, h, :] . U[b, t, :] + bg[g, h])        (chunk = 1)
 * and with chunk > 1 (the per-chunk path) one value per chunk, the gate of the chunk's
 * mean-pooled input: sigmoid of the mean of its tokens' logits (Atlas-Torch README, Bug Fixes
 * table, "no-omega ablation" row); a final short chunk pools its own tokens.
 *   U:  [B, T, d_model] bf16 (d_model a multiple of 16, at most 512)
 *   Wg: fp32 [n_gates, heads, d_model];  bg: fp32 [n_gates, heads];  scale: fp32 [n_gates]
 *   chunk: 1, or a multiple of 32
 *   out: fp32 [n_gates, B, heads, n], n = T or ceil(T / chunk): row (g, b, h) is memory
 *        b * heads + h's gate array as atlasmem_update_chunked takes it
 * Errors: E_INVALID for bad sizes or null pointers; E_UNSUPPORTED for other d_model / chunk;
 * E_SHAPE for (T + 32) * d_model * 2 > 2^31 - 1. */
atlasmem_status atlasmem_gates(const void* U, int64_t B, int64_t T, int32_t d_model, int32_t heads,
                               int32_t n_gates, const float* Wg, const float* bg, const float* scale,
                               int32_t chunk, float* out, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* ATLASMEM_H */
