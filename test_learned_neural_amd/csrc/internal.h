// Internal declarations shared by the atlasmem translation units.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/atlasmem.h"

namespace am {

// Derived sizes of a validated configuration.
struct Dims {
  int M;        // memories = batch * heads
  int dk, dv, dh, din;
  int poly;
  int C, c;     // chunk, Omega window
  int Rk;       // key rows per chunk incl. window history = C + c - 1
  int Rt;       // key rows + query rows = Rk + C
  int64_t P;    // parameters per memory
  int64_t P1;   // size of W1 (MLP) / W (linear)
  int kind, gate_mode, ns_steps;  // kind: LINEAR or MLP2_SILU (also for the residual memory)
  bool residual;                  // M(x) = x + W2 silu(W1 x)
  bool gated;                     // M(x) = W2 (silu(W1 x) * (W3 x)), W3 stored after W1
  int dz;                         // first-layer rows: d_hidden, or 2 d_hidden when gated
  bool ptr;                       // per-token retrieval: y_t from the state right after token t
  float ns_a, ns_b, ns_c, ns_eps;
  int in_bf16, out_bf16;
  bool split;   // bf16 hi/lo split products
  int prec;     // operand precision of the products: 0 plain bf16, 1 split bf16 (hi/lo), 2 fp32
  bool no_fused;
  bool no_loop;  // one launch per product and chunk instead of the chunk-loop kernel
  bool no_splitk;  // every product over its whole k range in one launch
  bool conv;       // this call's rows are convolved while they are read (update_chunked_conv)
};

// The token arrays of one launch sequence: T tokens; per memory, token stride `ld` of K, Q, V, Y,
// gamma and per-token gates, and stride `ldg` of per-chunk gates.
struct Span {
  int64_t T, ld, ldg;
};

// Per-token retrieval coefficients of one chunk (k_scan.hip): for query t of the chunk starting at
// token s0, beta_t and a_t of W_t = beta_t W0 + a_t S0 - sum_i Om[t][r] g_i (key row r <-> token
// i = s0 - (c - 1) + r).
atlasmem_status launch_ptr_coeffs(const float* theta, const float* eta, const float* alpha, const float* gamma,
                                  int64_t ld, const float* ghist, int M, int64_t s0, int C, int c, float* bA,
                                  float* Om, hipStream_t st);

// Feature map stage (k_features.hip): phi_c of degree <= 3, optionally projected by P.
int64_t feature_count_host(int d, int degree);
atlasmem_status launch_feature_map(const void* X, bool in_bf16, int64_t n, int d, int degree, const float* c4,
                                   const float* P, int d_out, float* out, hipStream_t st);

// Short convolution folded into the update (k_prologue.hip): inverse L2 norms of the convolved
// rows [t0, t0 + n) of every memory (X token stride ld; taps / bias as atlasmem_short_conv), written
// to inv[m * ld_inv + (t - t0)]; and the carried rows: hist_out = the last three of hist ++ X[0, T).
atlasmem_status launch_conv_inv_norm(const void* X, const void* hist, bool in_bf16, int M, int64_t ld, int64_t t0,
                                     int64_t n, int d, int heads, const float* taps, const float* bias, float* inv,
                                     int64_t ld_inv, hipStream_t st);
atlasmem_status launch_conv_carry(const void* X, const void* hist, bool in_bf16, int M, int64_t ld, int64_t T, int d,
                                  void* hist_out, hipStream_t st);

// Input prologue (k_prologue.hip)
atlasmem_status launch_short_conv(const void* X, bool in_bf16, int64_t M, int64_t T, int d, int heads,
                                  const float* taps, const float* bias, const void* hist, bool l2norm, void* out,
                                  bool out_bf16, void* hist_out, hipStream_t st);
bool gates_supported(int dm, int chunk);
atlasmem_status launch_gates(const void* U, int64_t B, int64_t T, int dm, int H, int n_gates, const float* Wg,
                             const float* bg, const float* scale, int chunk, float* out, hipStream_t st);

}  // namespace am

// The opaque handle of the C ABI.
struct atlasmem_handle_s {
  atlasmem_config cfg;
  am::Dims d;
  int device;
  void* arena;
  size_t arena_bytes;
  // state, ping-pong
  float* W[2];
  float* S[2];
  int cur;
  // window history (raw keys fp32, values fp32, gamma), ping-pong
  float* hk[2];
  float* hv[2];
  float* hg[2];
  int hcur;
  // per-chunk workspace (MLP path)
  float* Z;      // [M][Rt][dh]
  float* D2;     // [M][Rk][dv]
  float* D1;     // [M][Rk][dh]
  float* sk;     // split-K partial products of the per-product launches
  int64_t sk_floats;
  // gate coefficients for a batch of up to ncb chunks
  int ncb;
  float* cW;     // [M][ncb*C]
  float* cS;     // [M][ncb*C]
  float* oW;     // [M][ncb][Rk]  (window > 1)
  float* oS;
  float* scal;   // [M][ncb][3]
  // per-chunk gradient (PER_CHUNK path)
  float* G;      // [M][P]
  // hidden-split chunk kernel (k_hsplit.hip): partial outputs and key-row pre-activations of two
  // chunks, or null when the configuration does not qualify
  float* hsw;
  // the fused Newton-Schulz kernel's two-workgroup form (k_fused.hip): exchange slots and the
  // workgroup pairs' counts, or null when the configuration does not qualify
  float* fxs;
  // retrieval workspace
  int rb;        // rows per retrieval block
  float* Zr;     // [M][rb][dh]
  int* flag;     // non-finite flag (device)
  // per-token retrieval workspace (one chunk): [Zq | ...] [M][C][dz], scores [M][C][Rk], Y
  // accumulator [M][C][dv], per-token (beta, a) [M][C][2] and window coefficients [M][C][Rk]
  float* pZS;
  float* pA1;
  float* pYB;
  float* pbA;
  float* pOm;
  // tokens of the current, unfinished chunk (streaming calls): input rows of K and V (input
  // dtype), gamma and per-token gates, [M][C] each; `pending` of them are filled
  void* pK;
  void* pV;
  void* pQ;   // per-token retrieval: the unfinished chunk's query rows [M][C][d_key] (input dtype)
  void* pYs;  // ... and its answers [M][C][d_value] (output dtype), rows 0..pending-1
  float* pg;
  float* pth;
  float* pet;
  float* pal;
  int64_t pending;
  // short convolution folded into the update (update_chunked_conv): the three raw rows before the
  // next call of keys, queries and values ([M][3][d], input dtype, ping-pong), the inverse row
  // norms of a block of chunks' keys (window rows included) and queries, and the call's taps
  void* chk[2];
  void* chq[2];
  void* chv[2];
  int chcur;
  float* cinvk;  // [M][ncb * C + c - 1]
  float* cinvq;  // [M][ncb * C]
  const struct atlasmem_short_conv_params_s* conv;  // set during update_chunked_conv only
  const void* conv_v;                                // the call's raw value rows (with conv)
  int64_t cinv_t0k, cinv_t0q;                        // first token of cinvk / cinvq
};

namespace am {

using Handle = ::atlasmem_handle_s;

// Outer-loop backward (k_backward.hip)
bool backward_supported(const Dims& d);
int64_t backward_workspace_bytes(const Dims& d, int64_t T);
// Streaming calls of at most a few tokens (k_decode.hip): the queries' retrieval from the current
// state and, with `append`, the key / value rows and per-token gates appended to the unfinished
// chunk, in one launch.  E_UNSUPPORTED when the configuration or the call does not qualify.
// One update of T tokens (api.hip): the MLP path or the linear memory's, with the window history.
atlasmem_status run_update(Handle* h, const Dims& d, const void* K, const void* Q, const void* V, const float* theta,
                           const float* eta, const float* alpha, const float* gamma, const Span& sp, void* Y,
                           hipStream_t st);
bool decode_supported(const Dims& d, int64_t n);
// Per-token retrieval of the unfinished chunk's r buffered tokens (2-layer memories): the chunk's
// forward at its start weights over the buffered rows and their per-token-state answers into
// h->pYs, without the update (k_mlp.hip).
atlasmem_status ptr_partial_retrieve(Handle* h, int64_t r, hipStream_t st);
atlasmem_status launch_decode(Handle* h, const void* Q, const void* K, const void* V, const float* theta,
                              const float* eta, const float* alpha, const float* gamma, int64_t ld, int64_t n,
                              void* Y, bool append, hipStream_t st);
atlasmem_status backward(Handle* h, const void* K, const void* Q, const void* V, const float* theta, const float* eta,
                         const float* alpha, const float* gamma, int64_t T, void* Y, const float* dY,
                         const float* dWT, const float* dST, void* workspace, float* dK, float* dQ, float* dV,
                         float* dth, float* det, float* dal, float* dgamma, float* dW0, float* dS0, hipStream_t st);



// Launchers (enqueue only; return ATLASMEM_OK or ATLASMEM_E_DEVICE on a launch error).
atlasmem_status launch_gate_scan(const float* theta, const float* eta, const float* alpha, int M, int64_t ld_gate,
                                 int64_t t0, int nchunks, int C, float* cW, float* cS, int64_t ld_c, float* scal,
                                 int64_t ld_s, hipStream_t st);
atlasmem_status launch_omega(const float* cW, const float* cS, int64_t ld_c, const float* gamma, int64_t ld_g,
                             const float* ghist, int M, int64_t s0, int nchunks, int C, int c, float* oW, float* oS,
                             int64_t ld_o, hipStream_t st);
atlasmem_status launch_history_update(const Handle* h, const void* K, const void* V, const float* gamma, int64_t T,
                                      int64_t ld, hipStream_t st);
atlasmem_status launch_poly(const void* X, int in_bf16, int64_t n, int d, float* F, hipStream_t st);
// The update launchers take the sizes from `d` (the handle's, or a copy with a shorter chunk for
// a final partial chunk) and advance the handle's state over sp.T tokens (a multiple of d.C).
atlasmem_status launch_linear_update(Handle* h, const Dims& d, const void* K, const void* Q, const void* V,
                                     const float* theta, const float* eta, const float* alpha, const float* gamma,
                                     const Span& sp, void* Y, hipStream_t st);
atlasmem_status launch_linear_retrieve(Handle* h, const void* Q, int64_t T, int64_t ld, void* Y, hipStream_t st);
atlasmem_status mlp_update(Handle* h, const Dims& d, const void* K, const void* Q, const void* V, const float* theta,
                           const float* eta, const float* alpha, const float* gamma, const Span& sp, void* Y,
                           hipStream_t st);
atlasmem_status mlp_retrieve(Handle* h, const void* Q, int64_t T, int64_t ld, void* Y, hipStream_t st);
// Newton-Schulz on [n_mat] matrices of rows x cols, followed by an optional momentum/forgetting
// epilogue.  When `upd` is null the result is written to `out` ([n_mat, rows, cols]).
struct NsUpdate {
  const float* Win;
  const float* Sin;
  float* Wout;
  float* Sout;
  int64_t P;          // parameters per memory
  int64_t off;        // offset of this matrix inside a memory's parameters
  int mats_per_mem;   // matrices in the batch belonging to one memory (1)
  const float* theta; // per-chunk gates [M][ld_gate] at column k
  const float* eta;
  const float* alpha;
  int64_t ld_gate;
  int64_t k;
  int* flag;
};
atlasmem_status launch_ns(const float* G, int64_t ldG_mat, int n_mat, int rows, int cols, int steps, float a, float b,
                          float c, float eps, int prec, float* out, const NsUpdate* upd, hipStream_t st);
bool ns_supported(int rows, int cols);
// Several matrices of each memory in one launch (up to three groups of n_mat matrices, memory m's
// matrix of group i at G + goff_i + m ldG_mat, rows_i x cols_i), each followed by the momentum /
// forgetting epilogue at state offset uoff_i (upd.off is not used).
struct NsGroup {
  int rows, cols;
  int64_t goff, uoff;
};
atlasmem_status launch_ns_groups(const float* G, int64_t ldG_mat, int n_mat, int ngroups, const NsGroup* grp, int steps,
                                 float a, float b, float c, float eps, int prec, const NsUpdate& upd,
                                 hipStream_t st);
bool fused_supported(const Dims& d);
// Newton-Schulz forward recomputation and reverse of the outer-loop backward, one workgroup per
// 64 x 128 working slab (k_nsbwd.hip).  Slab z is matrix z / M (of nm <= 3) of memory z % M, at
// goff in the memory's P parameters, transposed to its working orientation when tr.  Workspace per
// slab: X [steps][128][64] (the iterates' transposes), A and B [steps][64][64], sq (|G|^2).
struct NsSlabGeo {
  int M, nm;
  int64_t P;
  int64_t goff[3];
  int tr[3];
};
bool ns_slab_supported(int rows, int cols, int steps);
atlasmem_status launch_ns_slab_forward(const NsSlabGeo& g, const float* G, float* X, float* A, float* B, float* sq,
                                       float* N, int steps, float a, float b, float c, float eps, hipStream_t st);
atlasmem_status launch_ns_slab_reverse(const NsSlabGeo& g, const float* G, const float* Na, const float* X,
                                       const float* A, const float* B, const float* sq, float* Ga, int steps, float a,
                                       float b, float c, float eps, hipStream_t st);
int64_t fused_split_workspace_floats(const Dims& d);
// The hidden-split chunk kernel for per-token gates (2-layer SiLU memory, Omega window, features of
// degree <= 2): chunks [kb0, kb0 + nb) of a call, after the gate scan (and window coefficients) of
// that block, in nb + 1 launches.
bool hsplit_supported(const Dims& d);
int64_t hsplit_workspace_floats(const Dims& d);
atlasmem_status launch_hsplit(Handle* h, const Dims& d, const void* K, const void* Q, const void* V, int64_t kb0,
                              int nb, int64_t ld, void* Y, hipStream_t st);
// The fused kernel for per-token gates (the same memory, chunks of 64): chunks [kb0, kb0 + nb) of a
// call, after the gate scan of that block of chunks.
bool fused_pt_supported(const Dims& d);
atlasmem_status launch_fused_pt(Handle* h, const Dims& d, const void* K, const void* Q, const void* V, int64_t kb0,
                                int nb, int64_t ld, void* Y, hipStream_t st);
// The fused update without a handle and without allocating: the caller's W, S ([M, P]) updated in
// place, the kernel's scratch in a static device array (k_fused.hip).
int fused_static_max_memories();
atlasmem_status launch_fused_static(const Dims& d, const void* K, const void* Q, const void* V, const float* theta,
                                    const float* eta, const float* alpha, const Span& sp, void* Y, float* W, float* S,
                                    int* nonfinite, hipStream_t st);
atlasmem_status launch_fused(Handle* h, const Dims& d, const void* K, const void* Q, const void* V,
                             const float* theta, const float* eta, const float* alpha, const Span& sp, void* Y,
                             hipStream_t st);

// Per-token retrieval coefficients of one chunk (k_scan.hip): for query t of the chunk starting at
// token s0, beta_t and a_t of W_t = beta_t W0 + a_t S0 - sum_i Om[t][r] g_i (key row r <-> token
// i = s0 - (c - 1) + r).
atlasmem_status launch_ptr_coeffs(const float* theta, const float* eta, const float* alpha, const float* gamma,
                                  int64_t ld, const float* ghist, int M, int64_t s0, int C, int c, float* bA,
                                  float* Om, hipStream_t st);

// Feature map stage (k_features.hip): phi_c of degree <= 3, optionally projected by P.
int64_t feature_count_host(int d, int degree);
atlasmem_status launch_feature_map(const void* X, bool in_bf16, int64_t n, int d, int degree, const float* c4,
                                   const float* P, int d_out, float* out, hipStream_t st);

// Input prologue (k_prologue.hip)
atlasmem_status launch_short_conv(const void* X, bool in_bf16, int64_t M, int64_t T, int d, int heads,
                                  const float* taps, const float* bias, const void* hist, bool l2norm, void* out,
                                  bool out_bf16, void* hist_out, hipStream_t st);
bool gates_supported(int dm, int chunk);
atlasmem_status launch_gates(const void* U, int64_t B, int64_t T, int dm, int H, int n_gates, const float* Wg,
                             const float* bg, const float* scale, int chunk, float* out, hipStream_t st);

}  // namespace am
