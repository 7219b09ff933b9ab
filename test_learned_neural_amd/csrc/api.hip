// C ABI of the atlasmem library: validation, the handle and its device arena, dispatch.
#include <stdlib.h>
#include <string.h>

#include <new>

#include "common.h"
#include "internal.h"

using namespace am;

namespace {

struct DeviceGuard {
  int prev = -1;
  bool ok = false;
  explicit DeviceGuard(int dev) {
    if (hipGetDevice(&prev) != hipSuccess) return;
    ok = (prev == dev) || (hipSetDevice(dev) == hipSuccess);
  }
  ~DeviceGuard() {
    if (ok && prev >= 0) (void)hipSetDevice(prev);
  }
};

int64_t feature_count(int dk, int poly) { return poly == 1 ? dk : 1 + dk + (int64_t)dk * (dk + 1) / 2; }

atlasmem_status validate(const atlasmem_config* c) {
  if (!c) return ATLASMEM_E_INVALID;
  if (c->abi_version != ATLASMEM_ABI_VERSION) return ATLASMEM_E_INVALID;
  if (c->memory_kind < ATLASMEM_LINEAR || c->memory_kind > ATLASMEM_MLP2_GATED) return ATLASMEM_E_INVALID;
  const bool mlp = c->memory_kind != ATLASMEM_LINEAR;
  if (c->batch < 1 || c->heads < 1 || c->d_key < 1 || c->d_value < 1 || c->chunk < 1 || c->omega_window < 1)
    return ATLASMEM_E_INVALID;
  if (mlp && c->d_hidden < 1) return ATLASMEM_E_INVALID;
  if (c->poly_degree != 1 && c->poly_degree != 2) return ATLASMEM_E_INVALID;
  if (c->gate_mode != ATLASMEM_PER_TOKEN && c->gate_mode != ATLASMEM_PER_CHUNK) return ATLASMEM_E_INVALID;
  if (c->ns_steps < 0 || c->ns_steps > 16) return ATLASMEM_E_INVALID;
  if ((c->input_dtype != ATLASMEM_F32 && c->input_dtype != ATLASMEM_BF16) ||
      (c->output_dtype != ATLASMEM_F32 && c->output_dtype != ATLASMEM_BF16))
    return ATLASMEM_E_INVALID;
  if (c->precision < ATLASMEM_PREC_AUTO || c->precision > ATLASMEM_PREC_F32) return ATLASMEM_E_INVALID;
  if (c->ns_steps > 0 && !(c->ns_eps >= 0.0f)) return ATLASMEM_E_INVALID;
  if (c->flags & ~(ATLASMEM_FLAG_NO_FUSED | ATLASMEM_FLAG_PER_TOKEN_RETRIEVE | ATLASMEM_FLAG_NO_CHUNK_LOOP |
                   ATLASMEM_FLAG_NO_SPLIT_K))
    return ATLASMEM_E_INVALID;
  if ((int64_t)c->batch * c->heads > (1 << 20)) return ATLASMEM_E_SHAPE;
  if (c->d_key > 1024 || c->d_value > 1024 || c->d_hidden > 4096 || c->chunk > 1024 || c->omega_window > 64)
    return ATLASMEM_E_SHAPE;
  const int64_t din = feature_count(c->d_key, c->poly_degree);
  if (din > 16384) return ATLASMEM_E_SHAPE;
  // the residual memory adds its input to its output
  if (c->memory_kind == ATLASMEM_MLP2_SILU_RESIDUAL && din != c->d_value) return ATLASMEM_E_INVALID;
  // valid but not provided
  if (c->gate_mode == ATLASMEM_PER_CHUNK && c->omega_window > 1) return ATLASMEM_E_UNSUPPORTED;
  if (c->gate_mode == ATLASMEM_PER_TOKEN && c->ns_steps > 0) return ATLASMEM_E_UNSUPPORTED;
  if ((c->flags & ATLASMEM_FLAG_PER_TOKEN_RETRIEVE) && c->gate_mode != ATLASMEM_PER_TOKEN)
    return ATLASMEM_E_UNSUPPORTED;
  if (c->memory_kind == ATLASMEM_LINEAR) {
    if (din > 64 || c->d_value > 64 || c->omega_window > 8 || c->ns_steps > 0) return ATLASMEM_E_UNSUPPORTED;
  } else if (c->ns_steps > 0) {
    if (!ns_supported(c->d_hidden, (int)din) || !ns_supported(c->d_value, c->d_hidden)) return ATLASMEM_E_UNSUPPORTED;
  }
  return ATLASMEM_OK;
}

Dims make_dims(const atlasmem_config* c) {
  Dims d;
  d.M = c->batch * c->heads;
  d.dk = c->d_key;
  d.dv = c->d_value;
  d.dh = c->memory_kind != ATLASMEM_LINEAR ? c->d_hidden : 0;
  d.poly = c->poly_degree;
  d.din = (int)feature_count(c->d_key, c->poly_degree);
  d.C = c->chunk;
  d.c = c->omega_window;
  d.Rk = d.C + d.c - 1;
  d.Rt = d.Rk + d.C;
  // both 2-layer memories run the MLP path; the residual one adds its input in the epilogues
  d.kind = c->memory_kind == ATLASMEM_LINEAR ? ATLASMEM_LINEAR : ATLASMEM_MLP2_SILU;
  d.residual = c->memory_kind == ATLASMEM_MLP2_SILU_RESIDUAL;
  d.gated = c->memory_kind == ATLASMEM_MLP2_GATED;
  // first-layer rows: W1 (and W3 below it, gated); the hidden buffers hold [Z1 | Z3] per row
  d.dz = d.gated ? 2 * d.dh : d.dh;
  if (d.kind == ATLASMEM_LINEAR) {
    d.P1 = (int64_t)d.dv * d.din;
    d.P = d.P1;
  } else {
    d.P1 = (int64_t)d.dz * d.din;
    d.P = d.P1 + (int64_t)d.dv * d.dh;
  }
  d.gate_mode = c->gate_mode;
  d.ns_steps = c->ns_steps;
  d.ns_a = c->ns_a;
  d.ns_b = c->ns_b;
  d.ns_c = c->ns_c;
  d.ns_eps = c->ns_eps;
  d.in_bf16 = c->input_dtype == ATLASMEM_BF16;
  d.out_bf16 = c->output_dtype == ATLASMEM_BF16;
  d.prec = c->precision == ATLASMEM_PREC_BF16 ? 0 : (c->precision == ATLASMEM_PREC_F32 ? 2 : 1);
  d.split = d.prec == 1;
  d.no_fused = (c->flags & ATLASMEM_FLAG_NO_FUSED) != 0;
  d.no_loop = (c->flags & ATLASMEM_FLAG_NO_CHUNK_LOOP) != 0;
  d.no_splitk = (c->flags & ATLASMEM_FLAG_NO_SPLIT_K) != 0;
  d.ptr = (c->flags & ATLASMEM_FLAG_PER_TOKEN_RETRIEVE) != 0;
  d.conv = false;
  return d;
}

struct Carver {
  size_t off = 0;
  size_t take(size_t bytes) {
    size_t o = off;
    off += (bytes + 255) & ~(size_t)255;
    return o;
  }
};

bool device_is_gfx950(int dev) {
  hipDeviceProp_t prop;
  if (hipGetDeviceProperties(&prop, dev) != hipSuccess) return false;
  return strncmp(prop.gcnArchName, "gfx950", 6) == 0;
}

hipStream_t S(void* p) { return (hipStream_t)p; }

}  // namespace

extern "C" {

int atlasmem_abi_version(void) { return ATLASMEM_ABI_VERSION; }

const char* atlasmem_status_string(int status) {
  switch (status) {
    case ATLASMEM_OK: return "ok";
    case ATLASMEM_E_INVALID: return "invalid argument";
    case ATLASMEM_E_SHAPE: return "bad shape";
    case ATLASMEM_E_UNSUPPORTED: return "unsupported combination";
    case ATLASMEM_E_DEVICE: return "device or launch error";
    case ATLASMEM_E_NOMEM: return "out of device memory";
    case ATLASMEM_E_NONFINITE: return "non-finite state";
    default: return "unknown status";
  }
}

int64_t atlasmem_param_count(const atlasmem_config* cfg) {
  if (!cfg) return -1;
  atlasmem_status s = validate(cfg);
  if (s == ATLASMEM_E_INVALID) return -1;
  return make_dims(cfg).P;
}

atlasmem_status atlasmem_create(const atlasmem_config* cfg, const float* W0, const float* S0, void* stream,
                                atlasmem_handle* out) {
  if (!out) return ATLASMEM_E_INVALID;
  *out = nullptr;
  atlasmem_status s = validate(cfg);
  if (s != ATLASMEM_OK) return s;
  int ndev = 0;
  if (hipGetDeviceCount(&ndev) != hipSuccess || ndev < 1) return ATLASMEM_E_DEVICE;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return ATLASMEM_E_DEVICE;
  if (!device_is_gfx950(dev)) return ATLASMEM_E_DEVICE;

  Handle* h = new (std::nothrow) Handle();
  if (!h) return ATLASMEM_E_NOMEM;
  h->cfg = *cfg;
  h->d = make_dims(cfg);
  h->device = dev;
  const Dims& d = h->d;
  const int64_t M = d.M;
  const int H = d.c - 1 > 0 ? d.c - 1 : 1;

  Carver cv;
  size_t oW[2], oS[2], ohk[2], ohv[2], ohg[2];
  for (int i = 0; i < 2; ++i) {
    oW[i] = cv.take(sizeof(float) * M * d.P);
    oS[i] = cv.take(sizeof(float) * M * d.P);
    ohk[i] = cv.take(sizeof(float) * M * H * d.dk);
    ohv[i] = cv.take(sizeof(float) * M * H * d.dv);
    ohg[i] = cv.take(sizeof(float) * M * H);
  }
  const size_t oflag = cv.take(256);
  // the tokens of an unfinished chunk (streaming calls)
  const size_t esz = d.in_bf16 ? 2 : 4;
  const size_t opK = cv.take(esz * M * d.C * d.dk), opV = cv.take(esz * M * d.C * d.dv);
  const size_t opg = cv.take(sizeof(float) * M * d.C), opth = cv.take(sizeof(float) * M * d.C);
  const size_t opet = cv.take(sizeof(float) * M * d.C), opal = cv.take(sizeof(float) * M * d.C);
  // per-token retrieval: the unfinished chunk's queries and their answers
  const size_t oesz = d.out_bf16 ? 2 : 4;
  const size_t opQ = d.ptr ? cv.take(esz * M * d.C * d.dk) : 0, opYs = d.ptr ? cv.take(oesz * M * d.C * d.dv) : 0;
  // the raw rows before the next call for the folded short convolution (zero: sequence start)
  size_t ochk[2], ochq[2], ochv[2];
  for (int i = 0; i < 2; ++i) {
    ochk[i] = cv.take(esz * M * 3 * d.dk);
    ochq[i] = cv.take(esz * M * 3 * d.dk);
    ochv[i] = cv.take(esz * M * 3 * d.dv);
  }
  const size_t state_end = cv.off;
  size_t oZ = 0, oD2 = 0, oD1 = 0, osk = 0, ocW = 0, ocS = 0, ooW = 0, ooS = 0, oscal = 0, oG = 0, oZr = 0;
  size_t opZS = 0, opA1 = 0, opYB = 0, opbA = 0, opOm = 0, ocik = 0, ociq = 0, ohs = 0, ofxs = 0;
  if (d.kind == ATLASMEM_MLP2_SILU) {
    oZ = cv.take(sizeof(float) * M * d.Rt * d.dz);
    oD2 = cv.take(sizeof(float) * M * d.Rk * d.dv);
    oD1 = cv.take(sizeof(float) * M * d.Rk * d.dz);
    {  // room for 16 k-slices of the chunk's row products, at most 16 MB
      const int64_t w = d.dz > d.dv ? d.dz : d.dv;
      int64_t f = 16 * M * (int64_t)d.Rt * w;
      h->sk_floats = f < ((int64_t)4 << 20) ? f : ((int64_t)4 << 20);
      osk = cv.take(sizeof(float) * h->sk_floats);
    }
    const int64_t per_chunk_floats = M * (2 * (int64_t)d.C + 2 * (int64_t)d.Rk + 3);
    int64_t ncb = ((int64_t)32 << 20) / 4 / per_chunk_floats;
    ncb = ncb < 1 ? 1 : (ncb > 4096 ? 4096 : ncb);
    h->ncb = (int)ncb;
    if (d.gate_mode == ATLASMEM_PER_TOKEN) {
      ocW = cv.take(sizeof(float) * M * ncb * d.C);
      ocS = cv.take(sizeof(float) * M * ncb * d.C);
      oscal = cv.take(sizeof(float) * M * ncb * 3);
      if (d.c > 1) {
        ooW = cv.take(sizeof(float) * M * ncb * d.Rk);
        ooS = cv.take(sizeof(float) * M * ncb * d.Rk);
      }
    }
    // the per-chunk gradient (Newton-Schulz), or the fused kernels' transposed second-layer state
    oG = cv.take(sizeof(float) * M * d.P);
    if (hsplit_supported(d)) ohs = cv.take(sizeof(float) * hsplit_workspace_floats(d));
    if (fused_split_workspace_floats(d) > 0) ofxs = cv.take(sizeof(float) * fused_split_workspace_floats(d));
    ocik = cv.take(sizeof(float) * M * (ncb * d.C + d.c - 1));
    ociq = cv.take(sizeof(float) * M * ncb * d.C);
    int64_t rb = 1024;
    while (rb > 64 && (int64_t)M * rb * d.dz * 4 > ((int64_t)256 << 20)) rb /= 2;
    h->rb = (int)rb;
    oZr = cv.take(sizeof(float) * M * rb * d.dz);
    if (d.ptr) {
      opZS = cv.take(sizeof(float) * M * d.C * d.dz);
      opA1 = cv.take(sizeof(float) * M * d.C * d.Rk);
      opYB = cv.take(sizeof(float) * M * d.C * d.dv);
      opbA = cv.take(sizeof(float) * M * d.C * 2);
      opOm = cv.take(sizeof(float) * M * d.C * d.Rk);
    }
  }
  h->arena_bytes = cv.off;
  if (hipMalloc(&h->arena, h->arena_bytes) != hipSuccess) {
    (void)hipGetLastError();
    delete h;
    return ATLASMEM_E_NOMEM;
  }
  char* base = (char*)h->arena;
  for (int i = 0; i < 2; ++i) {
    h->W[i] = (float*)(base + oW[i]);
    h->S[i] = (float*)(base + oS[i]);
    h->hk[i] = (float*)(base + ohk[i]);
    h->hv[i] = (float*)(base + ohv[i]);
    h->hg[i] = (float*)(base + ohg[i]);
  }
  h->flag = (int*)(base + oflag);
  h->pK = base + opK;
  h->pV = base + opV;
  h->pQ = d.ptr ? base + opQ : nullptr;
  h->pYs = d.ptr ? base + opYs : nullptr;
  h->pg = (float*)(base + opg);
  h->pth = (float*)(base + opth);
  h->pet = (float*)(base + opet);
  h->pal = (float*)(base + opal);
  h->pending = 0;
  for (int i = 0; i < 2; ++i) {
    h->chk[i] = base + ochk[i];
    h->chq[i] = base + ochq[i];
    h->chv[i] = base + ochv[i];
  }
  h->chcur = 0;
  h->conv = nullptr;
  h->conv_v = nullptr;
  h->cinvk = h->cinvq = nullptr;
  h->cinv_t0k = h->cinv_t0q = 0;
  if (d.kind == ATLASMEM_MLP2_SILU) {
    h->cinvk = (float*)(base + ocik);
    h->cinvq = (float*)(base + ociq);
    h->Z = (float*)(base + oZ);
    h->D2 = (float*)(base + oD2);
    h->D1 = (float*)(base + oD1);
    h->sk = (float*)(base + osk);
    h->cW = ocW ? (float*)(base + ocW) : nullptr;
    h->cS = ocS ? (float*)(base + ocS) : nullptr;
    h->oW = ooW ? (float*)(base + ooW) : nullptr;
    h->oS = ooS ? (float*)(base + ooS) : nullptr;
    h->scal = oscal ? (float*)(base + oscal) : nullptr;
    h->G = oG ? (float*)(base + oG) : nullptr;
    h->hsw = ohs ? (float*)(base + ohs) : nullptr;
    h->fxs = ofxs ? (float*)(base + ofxs) : nullptr;
    h->Zr = (float*)(base + oZr);
    h->pZS = d.ptr ? (float*)(base + opZS) : nullptr;
    h->pA1 = d.ptr ? (float*)(base + opA1) : nullptr;
    h->pYB = d.ptr ? (float*)(base + opYB) : nullptr;
    h->pbA = d.ptr ? (float*)(base + opbA) : nullptr;
    h->pOm = d.ptr ? (float*)(base + opOm) : nullptr;
  }
  h->cur = 0;
  h->hcur = 0;
  hipStream_t st = S(stream);
  bool ok = hipMemsetAsync(h->arena, 0, state_end, st) == hipSuccess;
  if (ok && W0) ok = hipMemcpyAsync(h->W[0], W0, sizeof(float) * M * d.P, hipMemcpyDeviceToDevice, st) == hipSuccess;
  if (ok && S0) ok = hipMemcpyAsync(h->S[0], S0, sizeof(float) * M * d.P, hipMemcpyDeviceToDevice, st) == hipSuccess;
  if (!ok) {
    (void)hipGetLastError();
    (void)hipStreamSynchronize(st);
    (void)hipFree(h->arena);
    delete h;
    return ATLASMEM_E_DEVICE;
  }
  *out = h;
  return ATLASMEM_OK;
}

}  // extern "C"

namespace am {

// One launch sequence of the update over sp.T tokens (a multiple of d.C), then the window
// history of those tokens.
atlasmem_status run_update(Handle* h, const Dims& d, const void* K, const void* Q, const void* V, const float* theta,
                           const float* eta, const float* alpha, const float* gamma, const Span& sp, void* Y,
                           hipStream_t st) {
  if (sp.T == 0) return ATLASMEM_OK;
  if (d.kind == ATLASMEM_MLP2_SILU) return mlp_update(h, d, K, Q, V, theta, eta, alpha, gamma, sp, Y, st);
  atlasmem_status s = launch_linear_update(h, d, K, Q, V, theta, eta, alpha, gamma, sp, Y, st);
  if (s != ATLASMEM_OK) return s;
  if (d.c > 1) {
    s = launch_history_update(h, K, V, gamma, sp.T, sp.ld, st);
    if (s != ATLASMEM_OK) return s;
    h->hcur = 1 - h->hcur;
  }
  return ATLASMEM_OK;
}

}  // namespace am

namespace {

atlasmem_status retrieve_rows(Handle* h, const void* Q, int64_t T, int64_t ld, void* Y, hipStream_t st) {
  if (T == 0) return ATLASMEM_OK;
  if (h->d.kind == ATLASMEM_LINEAR) return launch_linear_retrieve(h, Q, T, ld, Y, st);
  return mlp_retrieve(h, Q, T, ld, Y, st);
}

// Copies tokens [0, n) of every memory of a row array (token stride ld, `row` bytes per token)
// to rows [r0, r0 + n) of the matching pending buffer.
bool to_pending(void* dst, const void* src, int64_t ld, int64_t r0, int64_t n, size_t row, const Dims& d,
                hipStream_t st) {
  if (n == 0 || !src) return true;
  return hipMemcpy2DAsync((char*)dst + r0 * row, (size_t)d.C * row, src, (size_t)ld * row, (size_t)n * row, d.M,
                          hipMemcpyDeviceToDevice, st) == hipSuccess;
}

bool append_pending(Handle* h, const void* K, const void* V, const float* theta, const float* eta, const float* alpha,
                    const float* gamma, int64_t ld, int64_t n, hipStream_t st) {
  const Dims& d = h->d;
  const size_t esz = d.in_bf16 ? 2 : 4;
  const int64_t r0 = h->pending;
  bool ok = to_pending(h->pK, K, ld, r0, n, esz * d.dk, d, st) && to_pending(h->pV, V, ld, r0, n, esz * d.dv, d, st);
  if (ok && d.c > 1) ok = to_pending(h->pg, gamma, ld, r0, n, sizeof(float), d, st);
  if (ok && d.gate_mode == ATLASMEM_PER_TOKEN)
    ok = to_pending(h->pth, theta, ld, r0, n, sizeof(float), d, st) &&
         to_pending(h->pet, eta, ld, r0, n, sizeof(float), d, st) &&
         to_pending(h->pal, alpha, ld, r0, n, sizeof(float), d, st);
  if (!ok) {
    (void)hipGetLastError();
    return false;
  }
  h->pending += n;
  return true;
}

const char* at_token(const void* base, int64_t t, size_t row) { return base ? (const char*)base + t * row : nullptr; }

// Tokens [0, n) of a streaming call that join the unfinished chunk: their queries are answered
// from the current state (the chunk's start weights) and their rows appended.  A call of a few
// tokens takes one decode launch; otherwise the GEMM-engine retrieval and strided copies.
static atlasmem_status stream_rows(Handle* h, const void* Q, const void* K, const void* V, const float* theta,
                                   const float* eta, const float* alpha, const float* gamma, int64_t ld, int64_t n,
                                   void* Y, hipStream_t st) {
  if (n == 0) return ATLASMEM_OK;
  if (h->d.ptr) {
    // per-token retrieval: each query reads the state right after its own token, which depends on
    // the unfinished chunk's rows up to that token only, so the rows are buffered first and the
    // buffered chunk's queries answered from them (the state is not updated until the chunk is
    // complete); the new tokens' answers are copied out
    const Dims& d = h->d;
    const int64_t r0 = h->pending;
    if (Q && !to_pending(h->pQ, Q, ld, r0, n, (d.in_bf16 ? 2 : 4) * (size_t)d.dk, d, st)) return ATLASMEM_E_DEVICE;
    if (!append_pending(h, K, V, theta, eta, alpha, gamma, ld, n, st)) return ATLASMEM_E_DEVICE;
    if (!Y) return ATLASMEM_OK;
    const atlasmem_status s = ptr_partial_retrieve(h, h->pending, st);
    if (s != ATLASMEM_OK) return s;
    const size_t row = (d.out_bf16 ? 2 : 4) * (size_t)d.dv;
    if (hipMemcpy2DAsync(Y, (size_t)ld * row, (const char*)h->pYs + r0 * row, (size_t)d.C * row, (size_t)n * row, d.M,
                         hipMemcpyDeviceToDevice, st) != hipSuccess) {
      (void)hipGetLastError();
      return ATLASMEM_E_DEVICE;
    }
    return ATLASMEM_OK;
  }
  const atlasmem_status s = launch_decode(h, Q, K, V, theta, eta, alpha, gamma, ld, n, Y, true, st);
  if (s != ATLASMEM_E_UNSUPPORTED) return s;
  atlasmem_status r;
  if (Y && (r = retrieve_rows(h, Q, n, ld, Y, st)) != ATLASMEM_OK) return r;
  if (!append_pending(h, K, V, theta, eta, alpha, gamma, ld, n, st)) return ATLASMEM_E_DEVICE;
  return ATLASMEM_OK;
}

}  // namespace

extern "C" {

atlasmem_status atlasmem_update_chunked_static(const atlasmem_config* cfg, const void* K, const void* Q,
                                               const void* V, const float* theta, const float* eta,
                                               const float* alpha, int64_t T, float* W, float* Sm, void* Y,
                                               int32_t* nonfinite, void* stream) {
  const atlasmem_status v = validate(cfg);
  if (v != ATLASMEM_OK) return v;
  const Dims d = make_dims(cfg);
  if (cfg->flags != 0 || d.prec != 1 || d.gated || !fused_supported(d)) return ATLASMEM_E_UNSUPPORTED;
  if (d.M > fused_static_max_memories()) return ATLASMEM_E_SHAPE;
  if (T < 0 || !W || !Sm) return ATLASMEM_E_INVALID;
  if (T % d.C != 0) return ATLASMEM_E_SHAPE;
  if (T == 0) return ATLASMEM_OK;
  if (!K || !V || !theta || !eta || !alpha || (Y && !Q)) return ATLASMEM_E_INVALID;
  if (T > INT64_MAX / d.C) return ATLASMEM_E_SHAPE;
  return launch_fused_static(d, K, Q, V, theta, eta, alpha, Span{T, T, T / d.C}, Y, W, Sm, (int*)nonfinite,
                             S(stream));
}

atlasmem_status atlasmem_update_chunked_conv(atlasmem_handle hh, const void* K, const void* Q, const void* V,
                                             const atlasmem_short_conv_params* conv, const float* theta,
                                             const float* eta, const float* alpha, const float* gamma, int64_t T,
                                             void* Y, void* stream) {
  Handle* h = (Handle*)hh;
  if (!h || !conv || T < 0) return ATLASMEM_E_INVALID;
  const Dims& d = h->d;
  if (d.kind != ATLASMEM_MLP2_SILU || d.ptr) return ATLASMEM_E_UNSUPPORTED;
  if (d.dk > 512 || d.dv > 512) return ATLASMEM_E_SHAPE;
  if (h->pending != 0 || T % d.C != 0) return ATLASMEM_E_UNSUPPORTED;
  if (T == 0) return ATLASMEM_OK;
  if (!K || !Q || !V || !theta || !eta || !alpha) return ATLASMEM_E_INVALID;
  if (!conv->taps_k || !conv->taps_q || !conv->taps_v) return ATLASMEM_E_INVALID;
  // each channel's four taps are read as one 16-byte vector
  if ((((uintptr_t)conv->taps_k) | ((uintptr_t)conv->taps_q) | ((uintptr_t)conv->taps_v)) & 15)
    return ATLASMEM_E_INVALID;
  if ((d.c > 1) != (gamma != nullptr)) return ATLASMEM_E_INVALID;
  DeviceGuard g(h->device);
  if (!g.ok) return ATLASMEM_E_DEVICE;
  hipStream_t st = S(stream);
  Dims dc = d;
  dc.conv = true;
  const atlasmem_short_conv_params params = *conv;
  h->conv = &params;
  h->conv_v = V;
  atlasmem_status s = mlp_update(h, dc, K, Q, V, theta, eta, alpha, gamma,
                                 Span{T, T, d.gate_mode == ATLASMEM_PER_TOKEN ? T : T / d.C}, Y, st);
  h->conv = nullptr;
  h->conv_v = nullptr;
  if (s != ATLASMEM_OK) return s;
  // the three raw rows of each tensor before the next call
  const int nx = 1 - h->chcur;
  if ((s = launch_conv_carry(K, h->chk[h->chcur], d.in_bf16, d.M, T, T, d.dk, h->chk[nx], st)) != ATLASMEM_OK ||
      (s = launch_conv_carry(Q, h->chq[h->chcur], d.in_bf16, d.M, T, T, d.dk, h->chq[nx], st)) != ATLASMEM_OK ||
      (s = launch_conv_carry(V, h->chv[h->chcur], d.in_bf16, d.M, T, T, d.dv, h->chv[nx], st)) != ATLASMEM_OK)
    return s;
  h->chcur = nx;
  return ATLASMEM_OK;
}

atlasmem_status atlasmem_update_chunked(atlasmem_handle hh, const void* K, const void* Q, const void* V,
                                        const float* theta, const float* eta, const float* alpha, const float* gamma,
                                        int64_t T, void* Y, void* stream) {
  Handle* h = (Handle*)hh;
  if (!h || T < 0) return ATLASMEM_E_INVALID;
  const Dims& d = h->d;
  if (T == 0) return ATLASMEM_OK;
  const int64_t C = d.C;
  const bool per_token = d.gate_mode == ATLASMEM_PER_TOKEN;
  const int64_t p0 = h->pending;
  const int64_t ncomp = (p0 + T) / C;  // chunks this call completes
  if (!K || !V || (Y && !Q)) return ATLASMEM_E_INVALID;
  if ((per_token || ncomp > 0) && (!theta || !eta || !alpha)) return ATLASMEM_E_INVALID;
  if ((d.c > 1) != (gamma != nullptr)) return ATLASMEM_E_INVALID;
  DeviceGuard g(h->device);
  if (!g.ok) return ATLASMEM_E_DEVICE;
  hipStream_t st = S(stream);
  const int64_t ldg = per_token ? T : ncomp;
  // per-token retrieval of an unfinished chunk's queries runs on the 2-layer memories' path
  if (d.ptr && d.kind == ATLASMEM_LINEAR && (p0 != 0 || T % C != 0)) return ATLASMEM_E_UNSUPPORTED;
  if (p0 == 0 && T % C == 0)
    return run_update(h, d, K, Q, V, theta, eta, alpha, gamma, Span{T, T, ldg}, Y, st);

  const size_t ek = (d.in_bf16 ? 2 : 4) * (size_t)d.dk, ev = (d.in_bf16 ? 2 : 4) * (size_t)d.dv;
  const size_t ey = (d.out_bf16 ? 2 : 4) * (size_t)d.dv;
  atlasmem_status s;
  int64_t pos = 0, gpos = 0;  // tokens and (per-chunk) gates consumed
  if (p0 > 0) {
    // tokens of the unfinished chunk: retrieved now, at its start weights (the current state),
    // and buffered until the chunk is complete
    const int64_t a = T < C - p0 ? T : C - p0;
    if ((s = stream_rows(h, Q, K, V, theta, eta, alpha, gamma, T, a, Y, st)) != ATLASMEM_OK) return s;
    pos = a;
    if (h->pending == C) {
      const float* th = per_token ? h->pth : theta;
      const float* et = per_token ? h->pet : eta;
      const float* al = per_token ? h->pal : alpha;
      s = run_update(h, d, h->pK, nullptr, h->pV, th, et, al, d.c > 1 ? h->pg : nullptr,
                     Span{C, C, per_token ? C : ldg}, nullptr, st);
      if (s != ATLASMEM_OK) return s;
      h->pending = 0;
      gpos = 1;
    }
  }
  // whole chunks straight from the caller's arrays
  const int64_t nfull = (T - pos) / C * C;
  if (nfull > 0) {
    const int64_t go = per_token ? pos : gpos;
    s = run_update(h, d, at_token(K, pos, ek), at_token(Q, pos, ek), at_token(V, pos, ev), theta + go, eta + go,
                   alpha + go, gamma ? gamma + pos : nullptr, Span{nfull, T, ldg}, Y ? (void*)at_token(Y, pos, ey) : nullptr,
                   st);
    if (s != ATLASMEM_OK) return s;
    pos += nfull;
  }
  // the rest starts a new chunk
  const int64_t r = T - pos;
  if (r > 0) {
    if ((s = stream_rows(h, Q ? at_token(Q, pos, ek) : nullptr, at_token(K, pos, ek), at_token(V, pos, ev),
                         per_token ? theta + pos : nullptr, per_token ? eta + pos : nullptr,
                         per_token ? alpha + pos : nullptr, gamma ? gamma + pos : nullptr, T, r,
                         Y ? (void*)at_token(Y, pos, ey) : nullptr, st)) != ATLASMEM_OK)
      return s;
  }
  return ATLASMEM_OK;
}

atlasmem_status atlasmem_flush(atlasmem_handle hh, const float* theta, const float* eta, const float* alpha,
                               void* stream) {
  Handle* h = (Handle*)hh;
  if (!h) return ATLASMEM_E_INVALID;
  const int64_t r = h->pending;
  if (r == 0) return ATLASMEM_OK;
  const bool per_token = h->d.gate_mode == ATLASMEM_PER_TOKEN;
  if (!per_token && (!theta || !eta || !alpha)) return ATLASMEM_E_INVALID;
  DeviceGuard g(h->device);
  if (!g.ok) return ATLASMEM_E_DEVICE;
  // the buffered tokens form one final chunk of r tokens
  Dims dr = h->d;
  dr.C = (int)r;
  dr.Rk = dr.C + dr.c - 1;
  dr.Rt = dr.Rk + dr.C;
  const atlasmem_status s =
      run_update(h, dr, h->pK, nullptr, h->pV, per_token ? h->pth : theta, per_token ? h->pet : eta,
                 per_token ? h->pal : alpha, dr.c > 1 ? h->pg : nullptr, Span{r, h->d.C, per_token ? h->d.C : 1},
                 nullptr, S(stream));
  if (s != ATLASMEM_OK) return s;
  h->pending = 0;
  return ATLASMEM_OK;
}

int64_t atlasmem_pending(atlasmem_handle hh) {
  const Handle* h = (const Handle*)hh;
  return h ? h->pending : -1;
}

atlasmem_status atlasmem_retrieve(atlasmem_handle hh, const void* Q, int64_t T, void* Y, void* stream) {
  Handle* h = (Handle*)hh;
  if (!h || T < 0) return ATLASMEM_E_INVALID;
  if (T == 0) return ATLASMEM_OK;
  if (!Q || !Y) return ATLASMEM_E_INVALID;
  DeviceGuard g(h->device);
  if (!g.ok) return ATLASMEM_E_DEVICE;
  if (decode_supported(h->d, T))
    return launch_decode(h, Q, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, T, T, Y, false, S(stream));
  return retrieve_rows(h, Q, T, T, Y, S(stream));
}

atlasmem_status atlasmem_get_state(atlasmem_handle hh, float* W, float* Sm, void* stream) {
  Handle* h = (Handle*)hh;
  if (!h) return ATLASMEM_E_INVALID;
  DeviceGuard g(h->device);
  if (!g.ok) return ATLASMEM_E_DEVICE;
  const size_t bytes = sizeof(float) * h->d.M * h->d.P;
  hipStream_t st = S(stream);
  if (W && hipMemcpyAsync(W, h->W[h->cur], bytes, hipMemcpyDeviceToDevice, st) != hipSuccess) return ATLASMEM_E_DEVICE;
  if (Sm && hipMemcpyAsync(Sm, h->S[h->cur], bytes, hipMemcpyDeviceToDevice, st) != hipSuccess)
    return ATLASMEM_E_DEVICE;
  int flag = 0;
  if (hipMemcpyAsync(&flag, h->flag, sizeof(int), hipMemcpyDeviceToHost, st) != hipSuccess) return ATLASMEM_E_DEVICE;
  if (hipStreamSynchronize(st) != hipSuccess) return ATLASMEM_E_DEVICE;
  return flag ? ATLASMEM_E_NONFINITE : ATLASMEM_OK;
}

atlasmem_status atlasmem_set_state(atlasmem_handle hh, const float* W, const float* Sm, void* stream) {
  Handle* h = (Handle*)hh;
  if (!h) return ATLASMEM_E_INVALID;
  DeviceGuard g(h->device);
  if (!g.ok) return ATLASMEM_E_DEVICE;
  const size_t bytes = sizeof(float) * h->d.M * h->d.P;
  hipStream_t st = S(stream);
  bool ok = true;
  ok = ok && (W ? hipMemcpyAsync(h->W[h->cur], W, bytes, hipMemcpyDeviceToDevice, st)
                : hipMemsetAsync(h->W[h->cur], 0, bytes, st)) == hipSuccess;
  ok = ok && (Sm ? hipMemcpyAsync(h->S[h->cur], Sm, bytes, hipMemcpyDeviceToDevice, st)
                 : hipMemsetAsync(h->S[h->cur], 0, bytes, st)) == hipSuccess;
  ok = ok && hipMemsetAsync(h->flag, 0, sizeof(int), st) == hipSuccess;
  return ok ? ATLASMEM_OK : ATLASMEM_E_DEVICE;
}

atlasmem_status atlasmem_reset_history(atlasmem_handle hh, void* stream) {
  Handle* h = (Handle*)hh;
  if (!h) return ATLASMEM_E_INVALID;
  DeviceGuard g(h->device);
  if (!g.ok) return ATLASMEM_E_DEVICE;
  const Dims& d = h->d;
  const int H = d.c - 1 > 0 ? d.c - 1 : 1;
  hipStream_t st = S(stream);
  for (int i = 0; i < 2; ++i) {
    if (hipMemsetAsync(h->hk[i], 0, sizeof(float) * d.M * H * d.dk, st) != hipSuccess ||
        hipMemsetAsync(h->hv[i], 0, sizeof(float) * d.M * H * d.dv, st) != hipSuccess ||
        hipMemsetAsync(h->hg[i], 0, sizeof(float) * d.M * H, st) != hipSuccess)
      return ATLASMEM_E_DEVICE;
  }
  const size_t esz = d.in_bf16 ? 2 : 4;
  if (hipMemsetAsync(h->chk[h->chcur], 0, esz * d.M * 3 * d.dk, st) != hipSuccess ||
      hipMemsetAsync(h->chq[h->chcur], 0, esz * d.M * 3 * d.dk, st) != hipSuccess ||
      hipMemsetAsync(h->chv[h->chcur], 0, esz * d.M * 3 * d.dv, st) != hipSuccess)
    return ATLASMEM_E_DEVICE;
  h->pending = 0;  // a new sequence starts with a new chunk
  return ATLASMEM_OK;
}

void atlasmem_destroy(atlasmem_handle hh) {
  Handle* h = (Handle*)hh;
  if (!h) return;
  {
    DeviceGuard g(h->device);
    (void)hipDeviceSynchronize();
    (void)hipFree(h->arena);
  }
  delete h;
}

atlasmem_status atlasmem_gate_scan(const float* theta, const float* eta, const float* alpha, int64_t M, int64_t T,
                                   int32_t chunk, float* cW, float* cS, float* chunk_scalars, void* stream) {
  if (M < 0 || T < 0 || chunk < 1) return ATLASMEM_E_INVALID;
  if (T % chunk != 0) return ATLASMEM_E_SHAPE;
  if (M == 0 || T == 0) return ATLASMEM_OK;
  if (!theta || !eta || !alpha || !cW || !cS || !chunk_scalars) return ATLASMEM_E_INVALID;
  if (M > INT32_MAX || T / chunk > INT32_MAX) return ATLASMEM_E_SHAPE;
  return launch_gate_scan(theta, eta, alpha, (int)M, T, 0, (int)(T / chunk), chunk, cW, cS, T, chunk_scalars,
                          (T / chunk) * 3, S(stream));
}

atlasmem_status atlasmem_omega_coeffs(const float* cW, const float* cS, const float* gamma, const float* gamma_hist,
                                      int64_t M, int64_t T, int32_t chunk, int32_t window, float* oW, float* oS,
                                      void* stream) {
  if (M < 0 || T < 0 || chunk < 1 || window < 1 || window > 64) return ATLASMEM_E_INVALID;
  if (T % chunk != 0) return ATLASMEM_E_SHAPE;
  if (M == 0 || T == 0) return ATLASMEM_OK;
  if (!cW || !cS || !gamma || !oW || !oS) return ATLASMEM_E_INVALID;
  if (M > INT32_MAX || T / chunk > INT32_MAX) return ATLASMEM_E_SHAPE;
  const int Rk = chunk + window - 1;
  return launch_omega(cW, cS, T, gamma, T, gamma_hist, (int)M, 0, (int)(T / chunk), chunk, window, oW, oS,
                      (T / chunk) * Rk, S(stream));
}

atlasmem_status atlasmem_poly_features(const void* X, int32_t in_dtype, int64_t n, int32_t d, float* F,
                                       void* stream) {
  if (n < 0 || d < 1 || d > 1024 || (in_dtype != ATLASMEM_F32 && in_dtype != ATLASMEM_BF16))
    return ATLASMEM_E_INVALID;
  if (n == 0) return ATLASMEM_OK;
  if (!X || !F) return ATLASMEM_E_INVALID;
  return launch_poly(X, in_dtype == ATLASMEM_BF16, n, d, F, S(stream));
}

atlasmem_status atlasmem_newton_schulz(const float* G, int64_t n_mat, int32_t rows, int32_t cols, int32_t steps,
                                       float a, float b, float c, float eps, int32_t precision, float* out,
                                       void* stream) {
  if (n_mat < 0 || rows < 1 || cols < 1 || steps < 0 || steps > 16 || !(eps >= 0.0f)) return ATLASMEM_E_INVALID;
  if (precision < ATLASMEM_PREC_AUTO || precision > ATLASMEM_PREC_F32) return ATLASMEM_E_INVALID;
  if (!ns_supported(rows, cols)) return ATLASMEM_E_UNSUPPORTED;
  if (n_mat == 0) return ATLASMEM_OK;
  if (!G || !out || G == out) return ATLASMEM_E_INVALID;
  if (n_mat > INT32_MAX) return ATLASMEM_E_SHAPE;
  return launch_ns(G, (int64_t)rows * cols, (int)n_mat, rows, cols, steps, a, b, c, eps,
                   precision == ATLASMEM_PREC_BF16 ? 0 : (precision == ATLASMEM_PREC_F32 ? 2 : 1), out, nullptr,
                   S(stream));
}

atlasmem_status atlasmem_short_conv(const void* X, int32_t in_dtype, int64_t M, int64_t T, int32_t d, int32_t heads,
                                    const float* taps, const float* bias, const void* hist, int32_t l2norm, void* out,
                                    int32_t out_dtype, void* hist_out, void* stream) {
  const bool dt_ok = (in_dtype == ATLASMEM_F32 || in_dtype == ATLASMEM_BF16) &&
                     (out_dtype == ATLASMEM_F32 || out_dtype == ATLASMEM_BF16);
  if (M < 0 || T < 0 || d < 1 || heads < 1 || !dt_ok || (l2norm != 0 && l2norm != 1)) return ATLASMEM_E_INVALID;
  if (d > 512) return ATLASMEM_E_SHAPE;
  if (M == 0 || (T == 0 && !hist_out)) return ATLASMEM_OK;
  if (!taps || (T > 0 && (!X || !out)) || (hist_out && (!X && T > 0))) return ATLASMEM_E_INVALID;
  // the output and the carried rows must not overlap what is still being read
  if ((out && out == X) || (hist_out && (hist_out == hist || hist_out == X))) return ATLASMEM_E_INVALID;
  return launch_short_conv(X, in_dtype == ATLASMEM_BF16, M, T, d, heads, taps, bias, hist, l2norm != 0, out,
                           out_dtype == ATLASMEM_BF16, hist_out, S(stream));
}

atlasmem_status atlasmem_gates(const void* U, int64_t B, int64_t T, int32_t d_model, int32_t heads, int32_t n_gates,
                               const float* Wg, const float* bg, const float* scale, int32_t chunk, float* out,
                               void* stream) {
  if (B < 0 || T < 0 || d_model < 1 || heads < 1 || n_gates < 1 || chunk < 1) return ATLASMEM_E_INVALID;
  if (!gates_supported(d_model, chunk)) return ATLASMEM_E_UNSUPPORTED;
  if ((int64_t)n_gates * heads > (1 << 20)) return ATLASMEM_E_SHAPE;
  // per-sequence byte offsets of U (plus one 32-row block past the end) stay within 32 bits
  if ((T + 32) * (int64_t)d_model * 2 > INT32_MAX) return ATLASMEM_E_SHAPE;
  if (B == 0 || T == 0) return ATLASMEM_OK;
  if (!U || !Wg || !bg || !scale || !out) return ATLASMEM_E_INVALID;
  return launch_gates(U, B, T, d_model, heads, n_gates, Wg, bg, scale, chunk, out, S(stream));
}

atlasmem_status atlasmem_feature_map(const void* X, int32_t in_dtype, int64_t n, int32_t d, int32_t degree,
                                     const float* coeffs, const float* P, int32_t d_out, float* out, void* stream) {
  if (n < 0 || d < 1 || degree < 1 || degree > 3 || (in_dtype != ATLASMEM_F32 && in_dtype != ATLASMEM_BF16))
    return ATLASMEM_E_INVALID;
  if (P && d_out < 1) return ATLASMEM_E_INVALID;
  if (d > 1024 || feature_count_host(d, degree) > (1 << 20) || (P && d_out > (1 << 16))) return ATLASMEM_E_SHAPE;
  if (n == 0) return ATLASMEM_OK;
  if (!X || !out) return ATLASMEM_E_INVALID;
  float c4[4] = {1.0f, 1.0f, 0.5f, 1.0f / 6.0f};  // 1/k!
  if (coeffs)
    for (int k = 0; k <= degree; ++k) c4[k] = coeffs[k];
  return launch_feature_map(X, in_dtype == ATLASMEM_BF16, n, d, degree, c4, P, P ? d_out : 0, out, S(stream));
}

int64_t atlasmem_backward_workspace_bytes(atlasmem_handle hh, int64_t T) {
  const Handle* h = (const Handle*)hh;
  if (!h || T < 0 || !backward_supported(h->d)) return -1;
  return backward_workspace_bytes(h->d, T);
}

atlasmem_status atlasmem_update_backward(atlasmem_handle hh, const void* K, const void* Q, const void* V,
                                         const float* theta, const float* eta, const float* alpha,
                                         const float* gamma, int64_t T, void* Y, const float* dY,
                                         const float* dW_T, const float* dS_T, void* workspace,
                                         int64_t workspace_bytes, float* dK, float* dQ, float* dV, float* dtheta,
                                         float* deta, float* dalpha, float* dgamma, float* dW0, float* dS0,
                                         void* stream) {
  Handle* h = (Handle*)hh;
  if (!h || T < 0) return ATLASMEM_E_INVALID;
  const Dims& d = h->d;
  if (!backward_supported(d)) return ATLASMEM_E_UNSUPPORTED;
  if (T % d.C != 0 || h->pending != 0) return ATLASMEM_E_SHAPE;
  if (T == 0) return ATLASMEM_OK;
  if (!K || !Q || !V || !theta || !eta || !alpha || !dY || !workspace || !dK || !dQ || !dV || !dtheta || !deta ||
      !dalpha || !dW0 || !dS0 || (d.c > 1 && (!gamma || !dgamma)))
    return ATLASMEM_E_INVALID;
  if (workspace_bytes < backward_workspace_bytes(d, T)) return ATLASMEM_E_INVALID;
  DeviceGuard g(h->device);
  if (!g.ok) return ATLASMEM_E_DEVICE;
  return backward(h, K, Q, V, theta, eta, alpha, gamma, T, Y, dY, dW_T, dS_T, workspace, dK, dQ, dV, dtheta, deta,
                  dalpha, dgamma, dW0, dS0, S(stream));
}

}  // extern "C"
