// Fused chunk loop for the 64 -> 128 -> 64 SiLU MLP memory with per-chunk gates and
// Newton-Schulz orthogonalisation: one 256-thread workgroup per memory runs every chunk of
// the call, with no launch between chunks and no per-chunk round trip of intermediates
// through global memory.
//
// What each chunk computes (titans-pytorch-mlx README, Core Equations, Eq. 12-14; ATLAS
// summary, section 3.3 (chunk-start weights) and section 5 (Newton-Schulz); Atlas-Torch
// README, Atlas Extensions and Bug Fixes tables (one summed gradient per chunk, eta and
// theta outside the orthogonalisation)):
//   retrieval   Y = W2 silu(W1 q)                         (chunk-start weights)
//   forward     Z = X W1^T, H = silu(Z), Yh = H W2^T      (keys X of the chunk)
//   backward    D2 = 2 (Yh - V), D1 = (D2 W2) * silu'(Z)
//   gradient    G1^T = X^T D1 (64 x 128), G2 = D2^T H (64 x 128)
//   NS          X0 = G / (||G||_F + eps); steps x {A = X X^T; B = bA + cA^2; X = aX + BX}
//   update      S = eta_c S - theta_c NS(G), W = (1 - alpha_c) W + S      (per matrix)
//
// Layout on the matrix cores (v_mfma_f32_32x32x16_bf16 unless noted; every fp32 operand is
// split into bf16 hi + lo and multiplied as hi*hi + hi*lo + lo*hi, exact bf16 inputs as
// x*hi + x*lo):
//  - A 32 x 32 output tile leaves lane l with rows 8q + 4(l/32) + u (q, u = 0..3) of column
//    l % 32.  Read as a k-operand, registers 8kl..8kl+7 of a tile hold the 16 consecutive k of
//    k-step kl in the fixed order {4h..4h+3, 8+4h..8+4h+3} (h = l/32); the partner operand is
//    read from memory in the same order.  Chained products therefore take tiles straight
//    from registers: H and D1 feed the gradient products, the updated weights feed the next
//    chunk's forward products, the Newton-Schulz iterate feeds B X.
//  - 512 threads = two sets of four waves, two waves per SIMD, so that one wave's vector and
//    LDS work overlaps the other's matrix-core work.  Wave w of either set owns hidden units
//    [32w, 32w + 32): its slice of W1 (the B operand of X W1^T) lives in its registers; W2 is
//    kept in LDS in both orientations (B operand of H W2^T, contraction over hidden units, and
//    of D2 W2, contraction over values).
//  - A chunk is processed in groups of 64 rows, set s taking rows [32s, 32s + 32); H, D2 (both
//    orientations) and X^T of a group go through LDS, and each wave accumulates its partial
//    gradients over its set's rows in registers.  At the end of the chunk the sets swap
//    partials through LDS, so that set 0 holds all of G1 and set 1 all of G2; each set then
//    orthogonalises and applies its own matrix, and the new W1 slices pass from set 0 to set 1
//    through LDS.
#include <string.h>

#include <mutex>

#include "common.h"
#include "internal.h"
#include "mfma_tiles.h"

namespace am {
namespace fz {

constexpr int D = 64;        // key / value width
constexpr int HD = 128;      // hidden width
constexpr int NT = 512;      // threads per workgroup: two sets of four waves
constexpr int GR = 32;       // rows per set in a group
constexpr int GROWS = 64;    // rows per group
// LDS row strides (bf16 units).  Rows read 16 bytes per lane by 16 consecutive lanes want a
// byte stride of 16 (mod 256) times an odd number, rows read 8 bytes per lane by 32
// consecutive lanes want 8 (mod 256) times an odd number: either way every lane of a pass
// lands on its own banks.
constexpr int LH = HD + 8;      // [*][128], 16-byte row reads (272 B)
constexpr int LD = D + 8;       // [*][64],  16-byte row reads (144 B)
constexpr int LE = D + 4;       // [*][64],  8-byte row reads (136 B)
constexpr int LR = GROWS + 4;   // [*][64 rows], 8-byte row reads (136 B)

// LDS map in uint16 units.
// Weights: W2 [v][h] (B operand of H W2^T) and W2^T [h][v] (B operand of D2 W2), hi and lo.
constexpr int W2H = 0, W2L = W2H + 64 * LH;
constexpr int WTH = W2L + 64 * LH, WTL = WTH + HD * LE;
// Group buffers: region A holds D2 [row][v], D2^T [v][row] and X^T [d][row] of the key rows,
// region B their H [row][h] (hi, then lo), HQ the H of the query rows (where W2 [v][h] would be:
// H W2^T reads W2 from W2^T).
constexpr int RA = WTL + HD * LE;
constexpr int D2H = RA, D2L = D2H + GROWS * LE;
constexpr int DTH = D2L + GROWS * LE, DTL = DTH + D * LR;
constexpr int XTH = DTL + D * LR;
constexpr int RA_END = XTH + D * LR;
constexpr int HSZ = GROWS * LH;                  // one of H hi / H lo
constexpr int RB = RA_END;
constexpr int GEND = RB + 2 * HSZ;
constexpr int HQ = 0;
static_assert(HQ + 2 * HSZ <= WTH, "query H below W2^T");
// Newton-Schulz phase, matrix j (set j): X^T [col][row] hi/lo (128 x 64, rows of 128 bytes, 8-byte
// chunks swizzled), A and B [64][64] hi/lo.  The X buffers lie under the weight copies, which
// the update rewrites after the last read of X.
constexpr int NX = 0, NXS = 2 * HD * 64;
constexpr int NA = 2 * NXS, NAS = 2 * 64 * LD;
constexpr int NB = NA + 2 * NAS, NBS = 2 * 64 * LE;
constexpr int NEND = NB + 2 * NBS;
// Partial-gradient exchange at the end of a chunk (fp32, [wave][tile][quad][lane] float4):
// G2 partials of set 0 under W2 (read last by the group's H W2^T), G1 partials of set 1 in
// region B (read last by the same product).
constexpr int XG2 = 0, XG1 = RB;
constexpr int XG_U16 = 4 * 2 * 4 * 64 * 4 * 2;
static_assert(XG_U16 <= 2 * 64 * LH && XG_U16 <= 2 * HSZ, "exchange slots");
// New W1 operand words from set 0 to set 1 ([wave][k-step word][lane] u32x4), over the
// Newton-Schulz A buffers, which are dead after the last A^2 product.
constexpr int HOFF = RA;
constexpr int HOFF_U16 = 4 * 8 * 64 * 8;
static_assert(HOFF >= NA && HOFF + HOFF_U16 <= NB, "handoff must lie in the A buffers");
constexpr int LDS_U16 = (GEND > NEND ? GEND : NEND);
constexpr int LDS_BYTES = LDS_U16 * 2 + 16 * 4;
static_assert(LDS_BYTES <= 160 * 1024, "LDS");

struct Args {
  const uint16_t* K;     // token 0 of this launch, memory 0; memory m at + m * ldT * D
  const uint16_t* Q;
  const uint16_t* V;
  const float* theta;    // chunk 0 of this launch, memory 0; memory m at + m * ld_gate
  const float* eta;
  const float* alpha;
  int64_t ldT;           // tokens per memory in the caller's arrays
  int64_t ld_gate;       // chunks per memory in the caller's gate arrays
  int C;
  int nchunks;           // chunks of this launch
  const float* Win;
  const float* Sin;
  float* Wout;
  float* Sout;
  float* T2;   // per memory [W2^T (h, v) | S2^T (h, v)]: the W2 state between chunks of a launch
  void* Y;
  int out_bf16;
  int ns_steps;
  float ns_a, ns_b, ns_c, ns_eps;
  int* flag;
  // Two workgroups per memory (one per set; null otherwise): per memory two exchange slots of
  // 64 x 128 floats (the partial gradient each set passes to the other) and a count of arrivals at
  // the pair's waits (one int, 128 bytes apart), zero at the launch.
  float* xs;
  int* sync;
  int M;
};

typedef unsigned short v2u16 __attribute__((ext_vector_type(2)));

// LDS buffer bases as opaque scalars: the bases lie beyond the 64 KB reach of a ds
// instruction's immediate offset, so folding them into constants would cost one address
// register per (buffer, constant) pair; kept opaque, only the small in-buffer constants fold.
__device__ __forceinline__ int opq(int x) {
  asm volatile("" : "+s"(x));
  return x;
}
// A per-lane value made opaque where it is used, so that the compiler recomputes it there
// instead of keeping many such addresses alive across the whole kernel.
__device__ __forceinline__ int opv(int x) {
  asm volatile("" : "+v"(x));
  return x;
}

constexpr int64_t P1 = (int64_t)HD * D;        // W1 size
constexpr int64_t P = P1 + (int64_t)D * HD;    // parameters per memory
constexpr int P2 = D * HD;                     // W2 size

// Write a 32x32 fp32 tile into an LDS matrix [row][col] as hi/lo (2-byte stores).
__device__ __forceinline__ void store_tile(uint16_t* sm, int offh, int offl, int ld, const f32x16& t, int r0, int c0,
                                           int lane) {
  const int hf = lane >> 5, col = c0 + (lane & 31);
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    uint32_t h, l;
    split_bf16(t[r], h, l);
    const int row = r0 + 8 * (r >> 2) + 4 * hf + (r & 3);
    sm[offh + row * ld + col] = (uint16_t)h;
    sm[offl + row * ld + col] = (uint16_t)l;
  }
}

// Store the packed operand words of one k-step (16 rows starting at r0, one column) into a
// row-major LDS matrix [row][col]: word p holds rows r0 + 8(p/2) + 4h + 2(p%2) and the next.
template <bool PL = false>
__device__ __forceinline__ void store_rows(uint16_t* sm, int offh, int offl, int ld, const u32x4& hi, const u32x4& lo,
                                           int r0, int col, int hf) {
#pragma unroll
  for (int p = 0; p < 4; ++p) {
    const int r = r0 + 8 * (p >> 1) + 4 * hf + 2 * (p & 1);
    sm[offh + r * ld + col] = (uint16_t)hi[p];
    sm[offh + (r + 1) * ld + col] = (uint16_t)(hi[p] >> 16);
    if constexpr (!PL) {
      sm[offl + r * ld + col] = (uint16_t)lo[p];
      sm[offl + (r + 1) * ld + col] = (uint16_t)(lo[p] >> 16);
    }
  }
}
// The same k-step words into a transposed LDS matrix [col][row] (two 8-byte stores each).
template <bool PL = false>
__device__ __forceinline__ void store_rows_T(uint16_t* sm, int offh, int offl, int ld, const u32x4& hi,
                                             const u32x4& lo, int r0, int col, int hf) {
  const int o = col * ld + r0 + 4 * hf;
  *(uint2*)(sm + offh + o) = uint2{hi[0], hi[1]};
  *(uint2*)(sm + offh + o + 8) = uint2{hi[2], hi[3]};
  if constexpr (!PL) {
    *(uint2*)(sm + offl + o) = uint2{lo[0], lo[1]};
    *(uint2*)(sm + offl + o + 8) = uint2{lo[2], lo[3]};
  }
}

// Barrier of the four waves of one set, for the Newton-Schulz iterations, where the two sets work
// on disjoint LDS buffers: a set does not wait for the other, so the sets drift apart and one
// set's matrix work overlaps the other's splits and stores.  A per-set count in LDS only grows
// (each wave adds one per barrier; `target` counts the set's barriers times four).  The release
// fence completes this wave's LDS accesses before its arrival, the acquire fence orders the next
// phase's accesses after the wait.  The wait is bounded, so every wave ends whatever happens; a
// wave that gives up sets `stuck` (raised to the kernel's error flag).
__device__ __forceinline__ void set_barrier(int* ctr, int& target, bool& stuck, int lane) {
  target += 4;
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
  if (lane == 0) __hip_atomic_fetch_add(ctr, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
  int spins = 0;
  while (__hip_atomic_load(ctr, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP) < target) {
    __builtin_amdgcn_s_sleep(1);
    if (++spins > (1 << 22)) {
      stuck = true;
      break;
    }
  }
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
}

// Wait of the two workgroups of a memory (one per set, on different CUs): one lane counts the
// workgroup's arrival and waits until the pair has made `target` arrivals in all.  Ordering:
//  - the pair on one XCD (`local`, the case under round-robin placement), which shares that XCD's
//    L2: before the barrier each wave waits until its stores have reached L2 (vector L1 writes
//    through); after it, the CU's L1 is invalidated (`buffer_inv sc0`, the invalidate that the
//    compiler uses when one workgroup's waves span CUs), so the other workgroup's data is read
//    from L2.  Neither touches L2 itself;
//  - otherwise device-scope release and acquire fences, which write back and invalidate L2.
// The wait is bounded, so every wave ends whatever happens; one that gives up sets `stuck` (raised
// to the kernel's error flag), and after that the workgroup no longer waits at all, so a broken
// pair costs one bounded wait, not one per chunk.
__device__ __forceinline__ void pair_sync(int* ctr, int& target, bool& stuck, bool local) {
  target += 2;
  if (local) asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  else __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");
  __syncthreads();
  if (threadIdx.x == 0 && !stuck) {
    __hip_atomic_fetch_add(ctr, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    int spins = 0;
    while (__hip_atomic_load(ctr, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) < target) {
      __builtin_amdgcn_s_sleep(1);
      if (++spins > (1 << 20)) {
        stuck = true;
        break;
      }
    }
  }
  __syncthreads();
  if (local) asm volatile("buffer_inv sc0" ::: "memory");
  else __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
}

// Newton-Schulz on one 64 x 128 matrix held by the four waves of a set as two 32 x 32 tiles
// per wave (wave w: columns 32w..32w+31), in place.  xh/xl/ah/al/bh/bl: the set's LDS buffers;
// red: the set's four partial sums of squares.
template <int P>
struct Part {
  static constexpr int value = P;
};
// pre(Part<p>) (p = 0..3) is called before iteration p: it issues the p-th quarter of the state
// loads, so that they stream in under the matrix work instead of stalling the vector memory path
// all at once.
// KEEP: B X takes its X operand from the split words this lane stored for X^T (kept in registers,
// one wave per SIMD has the room) instead of reading them back.
template <bool PL, bool KEEP = false, class Pre, class Bar>
__device__ __forceinline__ void newton_schulz1(f32x16 (&x)[2], uint16_t* sm, int bxh, int bxl, int bah, int bal,
                                               int bbh, int bbl, float* red, const Args& a, int lane, int w,
                                               Pre&& pre, Bar&& set_bar) {
  const int hf = lane >> 5, l32 = lane & 31;
  float ss = 0.0f;
#pragma unroll
  for (int t = 0; t < 2; ++t)
#pragma unroll
    for (int r = 0; r < 16; ++r) ss = fmaf(x[t][r], x[t][r], ss);
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) ss += __shfl_xor(ss, off, 64);
  if (lane == 0) red[w] = ss;
  __syncthreads();
  const float inv = 1.0f / (sqrtf(red[0] + red[1] + red[2] + red[3]) + a.ns_eps);
#pragma unroll
  for (int t = 0; t < 2; ++t)
#pragma unroll
    for (int r = 0; r < 16; ++r) x[t][r] *= inv;

  const int rt = w >> 1, ct = w & 1;
  // this lane's column c = 32w + l32 of X: X^T row base and swizzle
  const int cx = opv(32 * w + l32);
  const int xrow = cx * 64, xsw = swz(cx) ^ (4 * hf);
  // operands of A = X X^T by transposing reads: lane (g, e, q) of 16-lane group g reads the
  // chunk of X^T row c = 16ks + 8(g/2) + e (+4 for the second half of the k-step) at rows
  // rb + 16(g%2) + 4q; the swizzle of c + 16 differs from that of c by 16 (XOR).
  const int ln = opv(lane);
  const int g = ln >> 4, e = (ln >> 2) & 3, q4 = 4 * (ln & 3);
  const int c1 = 8 * (g >> 1) + e, c2 = c1 + 4;
  const int ra = 32 * rt + 16 * (g & 1) + q4, rb = 32 * ct + 16 * (g & 1) + q4;
  const int ta1 = c1 * 64 + (ra ^ swz(c1)), ta2 = c2 * 64 + (ra ^ swz(c2));
  const int tb1 = c1 * 64 + (rb ^ swz(c1)), tb2 = c2 * 64 + (rb ^ swz(c2));
  auto iteration = [&]() __attribute__((always_inline)) {
    // X^T to LDS: tile t, quad q of this lane = rows 32t + 8q + 4hf .. +3 of column cx (with KEEP
    // also the k-step words of B X: k-step 2t + q/2, words 2(q%2) and 2(q%2) + 1)
    u32x4 kh[4], kl[4];
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        uint32_t h0, l0, h1, l1;
        split2(x[t][4 * q], x[t][4 * q + 1], h0, l0);
        split2(x[t][4 * q + 2], x[t][4 * q + 3], h1, l1);
        const int o = opv(xrow + ((32 * t + 8 * q) ^ xsw));
        *(uint2*)(sm + bxh + o) = uint2{h0, h1};
        if constexpr (!PL) *(uint2*)(sm + bxl + o) = uint2{l0, l1};
        if constexpr (KEEP) {
          kh[2 * t + (q >> 1)][2 * (q & 1)] = h0;
          kh[2 * t + (q >> 1)][2 * (q & 1) + 1] = h1;
          kl[2 * t + (q >> 1)][2 * (q & 1)] = l0;
          kl[2 * t + (q >> 1)][2 * (q & 1) + 1] = l1;
        }
      }
    set_bar();
    // A = X X^T, tile (rt, ct), k = the 128 columns in steps of 16 (natural order)
    f32x16 A = zero16();
    {
      const int pa1 = opv(ta1), pa2 = opv(ta2), pb1 = opv(tb1), pb2 = opv(tb2);
#pragma unroll
      for (int ks = 0; ks < HD / 16; ++ks) {
        const int f = (ks & 1) ? 16 : 0, kb = ks * 16 * 64;
        const u32x4 ah = cat2(lds_tr16(sm + bxh + kb + (pa1 ^ f)), lds_tr16(sm + bxh + kb + (pa2 ^ f)));
        const u32x4 al = cat2(lds_tr16(sm + bxl + kb + (pa1 ^ f)), lds_tr16(sm + bxl + kb + (pa2 ^ f)));
        const u32x4 bh = cat2(lds_tr16(sm + bxh + kb + (pb1 ^ f)), lds_tr16(sm + bxh + kb + (pb2 ^ f)));
        const u32x4 bl = cat2(lds_tr16(sm + bxl + kb + (pb1 ^ f)), lds_tr16(sm + bxl + kb + (pb2 ^ f)));
        A = mmp<PL>(ah, al, bh, bl, A);
      }
    }
    store_tile_T<PL>(sm, bah, bal, LD, A, 32 * rt, 32 * ct, lane);
    set_bar();
    // B = b A + c A^2, tile (rt, ct), accumulated in place of A as c (A^2 + (b/c) A)
    if (a.ns_c != 0.0f) {
      const float r_bc = a.ns_b / a.ns_c;
#pragma unroll
      for (int r = 0; r < 16; ++r) A[r] *= r_bc;
      const int ara = opv((32 * rt + l32) * LD + 8 * hf), arb = opv((32 * ct + l32) * LD + 8 * hf);
#pragma unroll
      for (int ks = 0; ks < D / 16; ++ks) {
        const int oa = ara + 16 * ks;
        const int ob = arb + 16 * ks;
        A = mmp<PL>(lds16(sm, bah + oa), lds16(sm, bal + oa), lds16(sm, bah + ob), lds16(sm, bal + ob), A);
      }
#pragma unroll
      for (int r = 0; r < 16; ++r) A[r] *= a.ns_c;
    } else {
#pragma unroll
      for (int r = 0; r < 16; ++r) A[r] *= a.ns_b;
    }
    store_tile_T<PL>(sm, bbh, bbl, LE, A, 32 * rt, 32 * ct, lane);
    set_bar();
    // X = a X + B X: rows 0..63, columns 32w..32w+31; B X's k-operand X (rows of column cx in
    // the order 4hf..4hf+3, 8+4hf..8+4hf+3 of each k-step) comes back from X^T
    // (accumulated onto a X in place)
    const int brow = opv(l32 * LE + 4 * hf);
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
      for (int r = 0; r < 16; ++r) x[t][r] *= a.ns_a;
#pragma unroll
    for (int ks = 0; ks < D / 16; ++ks) {
      u32x4 xh, xl;
      if constexpr (KEEP) {
        xh = kh[ks];
        xl = kl[ks];
      } else {
        const int o1 = opv(xrow + ((16 * ks) ^ xsw)), o2 = opv(xrow + ((16 * ks + 8) ^ xsw));
        xh = cat2(lds8(sm, bxh + o1), lds8(sm, bxh + o2));
        xl = cat2(lds8(sm, bxl + o1), lds8(sm, bxl + o2));
      }
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        const int o0 = brow + 32 * t * LE + 16 * ks;
        const u32x4 ah = cat2(lds8(sm, bbh + o0), lds8(sm, bbh + o0 + 8));
        const u32x4 al = cat2(lds8(sm, bbl + o0), lds8(sm, bbl + o0 + 8));
        x[t] = mmp<PL>(ah, al, xh, xl, x[t]);
      }
    }
    // No barrier here: B X reads only the X^T rows of this lane's own column, which this lane
    // wrote, and the other waves read X^T only in A X^T, which every wave finished before
    // barrier 2; the A / B stores of the next iteration come after its own first barrier.
  };
  pre(Part<0>());
  if (a.ns_steps > 0) iteration();
  pre(Part<1>());
  if (a.ns_steps > 1) iteration();
  pre(Part<2>());
  if (a.ns_steps > 2) iteration();
  pre(Part<3>());
  for (int it = 3; it < a.ns_steps; ++it) iteration();
}

// RES: the residual memory M(x) = x + W2 silu(W1 x) (input and output widths are both D): the
// key's own values enter the error, D2 = 2 (Yh - (V - x)); each V element register carries the
// key element of the same position in its upper half.  The query's values are added to the
// output after the launch (residual_output_kernel).
//
// SPLIT: each set is a workgroup of its own (256 threads, one wave per SIMD) on its own CU, so that
// 128 memories occupy 256 CUs.  Workgroups b and b + 8 of each run of 16 form a memory's pair (the
// same XCD under round-robin placement, so their exchanges stay in one L2; each workgroup reads its
// XCD id at the start, and a pair found on two XCDs orders its exchanges with device-scope fences
// instead).  Within a set the work
// is the same as in the one-workgroup form (the thread index is offset by 256 for set 1); what the
// sets pass each other through LDS there goes through global memory here, around two waits of the
// pair per chunk: the partial gradients (exchange slots), and the new weights, which each set reads
// back from the state it has just stored (W1 from the state, W2^T from T2).  The results are those
// of the one-workgroup form bit for bit.  The launch is cooperative, so both workgroups of a pair
// are resident together.
template <bool RES, bool PL, bool SPLIT, bool GATED = false>
__global__ void __launch_bounds__(SPLIT ? NT / 2 : NT) fused_ns_kernel(Args a) {
  static_assert(!GATED || (SPLIT && !RES && !PL), "the gated memory runs the two-workgroup form in split bf16");
  // parameters per memory and the offsets of W3 (gated) and W2 in them
  constexpr int64_t PM = GATED ? P + P1 : P, O3 = P1, O2 = GATED ? 2 * P1 : P1;
  constexpr int NSLOT = GATED ? 3 : 2;  // exchange slots per memory (two-workgroup form)
  extern __shared__ __attribute__((aligned(16))) uint16_t sm[];
  float* red = (float*)(sm + LDS_U16);
  const int blk = blockIdx.x;
  const int m = SPLIT ? (blk >> 4) * 8 + (blk & 7) : blk;
  const int s_blk = SPLIT ? (blk >> 3) & 1 : 0;
  if (SPLIT && m >= a.M) return;  // both workgroups of a pair past the last memory
  const int t0 = threadIdx.x + 256 * s_blk;
  const int w8 = __builtin_amdgcn_readfirstlane(t0 >> 6);
  const int s = w8 >> 2, w = w8 & 3;  // row set, hidden-unit slice
  int* set_count = (int*)(red + 8) + s;  // this set's barrier count (red[8], red[9])
  int set_target = 0;
  bool stuck = false;
  // the pair's words: [0] arrivals, [2 + set] the set's XCD id + 1
  int* pair_ctr = SPLIT ? a.sync + (int64_t)m * 32 : nullptr;
  int pair_target = 0;
  if (threadIdx.x == 0) {
    ((int*)(red + 8))[0] = 0;
    ((int*)(red + 8))[1] = 0;
  }
  int xcc = 0;
  if constexpr (SPLIT) {
    asm volatile("s_getreg_b32 %0, hwreg(HW_REG_XCC_ID)" : "=s"(xcc));
    xcc &= 0xF;
    if (threadIdx.x == 0) __hip_atomic_store(pair_ctr + 2 + s_blk, xcc + 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
  // Lane-dependent values are re-derived in each phase from an opaque copy of the thread index,
  // so that the compiler does not keep them (and every address made from them) live across the
  // whole chunk loop.  h_own: the hidden unit this lane owns in register slices.
#define AM_LANE_VARS                                                                \
  const int t = opv(t0), lane = t & 63, hf = lane >> 5, l32 = lane & 31;          \
  const int h_own = 32 * w + l32;                                                 \
  (void)hf; (void)l32; (void)h_own
  // this memory's token rows as buffer resources (byte offsets fit in 32 bits: a launch covers
  // at most 2^22 tokens)
  const int nT = a.nchunks * a.C;
  const rsrc_t rK = make_rsrc(a.K + (int64_t)m * a.ldT * D, (uint32_t)nT * D * 2);
  const rsrc_t rQ = (a.Y && a.Q) ? make_rsrc(a.Q + (int64_t)m * a.ldT * D, (uint32_t)nT * D * 2) : rK;
  const rsrc_t rV = make_rsrc(a.V + (int64_t)m * a.ldT * D, (uint32_t)nT * D * 2);
  const int ysz = a.out_bf16 ? 2 : 4;  // bytes per output element
  const rsrc_t rY = make_rsrc(a.Y ? (const char*)a.Y + (int64_t)m * a.ldT * D * ysz : nullptr,
                              a.Y ? (uint32_t)nT * D * ysz : 0u);
  const float* Win = a.Win + (int64_t)m * PM;
  const float* Sin = a.Sin + (int64_t)m * PM;
  float* Wout = a.Wout + (int64_t)m * PM;
  float* Sout = a.Sout + (int64_t)m * PM;
  const int wth = opq(WTH), wtl = opq(WTL);
  const int d2h = opq(D2H), d2l = opq(D2L), dth = opq(DTH), dtl = opq(DTL), xth = opq(XTH);
  const int rb = opq(RB);

  // register slice of W1[h_own][d] (B operand of X W1^T, k = d), four k-steps of 16, hi and lo;
  // the gated memory's W3 slice likewise
  u32x4 w1h[4], w1l[4], w3h[4], w3l[4];
  {
  AM_LANE_VARS;
#pragma unroll
  for (int ks = 0; ks < 4; ++ks) {
    float v[8];
    const float4 p0 = *(const float4*)(Win + (int64_t)h_own * D + 16 * ks + 4 * hf);
    const float4 p1 = *(const float4*)(Win + (int64_t)h_own * D + 16 * ks + 8 + 4 * hf);
    v[0] = p0.x; v[1] = p0.y; v[2] = p0.z; v[3] = p0.w;
    v[4] = p1.x; v[5] = p1.y; v[6] = p1.z; v[7] = p1.w;
    pack8(v, w1h[ks], w1l[ks]);
    if constexpr (GATED) {
      const float4 r0 = *(const float4*)(Win + O3 + (int64_t)h_own * D + 16 * ks + 4 * hf);
      const float4 r1 = *(const float4*)(Win + O3 + (int64_t)h_own * D + 16 * ks + 8 + 4 * hf);
      const float u[8] = {r0.x, r0.y, r0.z, r0.w, r1.x, r1.y, r1.z, r1.w};
      pack8(u, w3h[ks], w3l[ks]);
    }
  }
  // W2 in LDS as [h][v]: B operand of D2 W2 (direct reads) and of H W2^T (transposing reads)
  for (int e = SPLIT ? t - 256 * s : t; e < D * HD; e += (SPLIT ? NT / 2 : NT)) {
    const int vv = e / HD, hh = e % HD;
    uint32_t hi, lo;
    split_bf16(Win[O2 + e], hi, lo);
    sm[wth + hh * LE + vv] = (uint16_t)hi;
    sm[wtl + hh * LE + vv] = (uint16_t)lo;
  }
  // set 1 keeps the W2 part of the state transposed in T2 between chunks (16-byte accesses for
  // its register layout, see the update); each lane writes exactly the elements it reads later
  if (s == 1) {
    const rsrc_t rt2 = make_rsrc(a.T2 + (int64_t)m * 2 * P2, (uint32_t)(2 * P2 * 4));
    const int vt = (h_own * D + 4 * hf) * 4;
#pragma unroll
    for (int tt = 0; tt < 2; ++tt)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        float wv4[4], sv4[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          const int64_t o = O2 + (int64_t)(32 * tt + 8 * q + 4 * hf + u) * HD + h_own;
          wv4[u] = Win[o];
          sv4[u] = Sin[o];
        }
        buf_st4(rt2, vt, (32 * tt + 8 * q) * 4, float4{wv4[0], wv4[1], wv4[2], wv4[3]});
        buf_st4(rt2, vt + P2 * 4, (32 * tt + 8 * q) * 4, float4{sv4[0], sv4[1], sv4[2], sv4[3]});
      }
  }
  }
  __syncthreads();
  bool pair_local = false;  // both workgroups of the pair on this XCD
  if constexpr (SPLIT) {
    int* loc = (int*)(red + 10);
    if (threadIdx.x == 0) {
      int other = 0, spins = 0;
      while ((other = __hip_atomic_load(pair_ctr + 3 - s_blk, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT)) == 0) {
        __builtin_amdgcn_s_sleep(1);
        if (++spins > (1 << 20)) {
          stuck = true;
          break;
        }
      }
      *loc = other == xcc + 1 ? 1 : 0;
    }
    __syncthreads();
    pair_local = __builtin_amdgcn_readfirstlane(*loc) != 0;
  }

  // A chunk is processed in double groups: the query rows and the key rows [64g, 64g + 64)
  // together (only the key rows when nothing is retrieved), so that the two X W1^T and H W2^T
  // products run as independent chains between the same barriers.
  const int ngroups = a.C / GROWS;
  const bool withq = a.Y != nullptr;
  // The X operand rows of a double group (this set's rows) are loaded by the previous one
  // (software pipelining), right after its own X W1^T has consumed the registers they land in;
  // the query operand is loaded (from the key rows when nothing is retrieved) in every case, so
  // that every wait for these loads has a fixed count of younger loads.
  auto load_x = [&](int k, int g, u32x4 (&pq)[4], u32x4 (&pk)[4]) __attribute__((always_inline)) {
    AM_LANE_VARS;
    if (k >= a.nchunks) {  // past the end of the launch: repeat the last group's loads
      k = a.nchunks - 1;
      g = ngroups - 1;
    }
    const int rset = (k * a.C + g * GROWS + GR * s) * D * 2;
    const int vx = (l32 * D + 4 * hf) * 2;
#pragma unroll
    for (int ks = 0; ks < 4; ++ks)
      pk[ks] = cat2(buf_ld8(rK, vx + 32 * ks, rset), buf_ld8(rK, vx + 32 * ks + 16, rset));
#pragma unroll
    for (int ks = 0; ks < 4; ++ks)
      pq[ks] = cat2(buf_ld8(rQ, vx + 32 * ks, rset), buf_ld8(rQ, vx + 32 * ks + 16, rset));
  };

  bool bad = false;
  f32x16 gr[2][2], gr3[2];
  const int hq = opq(HQ);
  // One double group: Z, H and Yh of queries and keys, Y of the queries, then D2, D1 and the
  // gradient accumulation of the keys.
  auto run_group = [&](int k, int g, u32x4 (&pq)[4], u32x4 (&pk)[4]) __attribute__((always_inline)) {
    AM_LANE_VARS;
    const int vcol = 16 * w + (lane & 15);
    const int row0 = k * a.C + g * GROWS;  // the group's first row in this launch
    const int rset = row0 + GR * s;        // ... and this set's first row
    // the key rows' X^T staging words and values, used after the first barrier (issued before
    // the X operands are consumed: the wait for those then has exactly nine younger loads)
    const u32x4 xt = buf_ld16(rK, ((t >> 3) * D + (t & 7) * 8) * 2, row0 * D * 2);
    uint32_t vv[8];
#pragma unroll
    for (int rt = 0; rt < 2; ++rt)
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int vo = (4 * (lane >> 4) * D + vcol) * 2 + u * D * 2, so = (rset + 16 * rt) * D * 2;
        if (RES) {
          v2u16 pr;
          pr.x = __builtin_amdgcn_raw_buffer_load_b16(rV, vo, so, 0);
          pr.y = __builtin_amdgcn_raw_buffer_load_b16(rK, vo, so, 0);
          vv[4 * rt + u] = __builtin_bit_cast(uint32_t, pr);
        } else {
          vv[4 * rt + u] = buf_ld_u16(rV, vo, so);
        }
      }
    // Z = X W1^T of keys and queries: this set's 32 rows, hidden units of this wave
    f32x16 zk = zero16(), zq = zero16();
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      zk = mfma32(pk[ks], w1h[ks], zk);
      if constexpr (!PL) zk = mfma32(pk[ks], w1l[ks], zk);
    }
    if (withq) {
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) {
        zq = mfma32(pq[ks], w1h[ks], zq);
        if constexpr (!PL) zq = mfma32(pq[ks], w1l[ks], zq);
      }
    }
    // gated: Z3 = X W3^T of keys and queries
    f32x16 z3k, z3q;
    if constexpr (GATED) {
      z3k = zero16();
      z3q = zero16();
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) {
        z3k = mfma32(pk[ks], w3h[ks], z3k);
        z3k = mfma32(pk[ks], w3l[ks], z3k);
      }
      if (withq) {
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) {
          z3q = mfma32(pq[ks], w3h[ks], z3q);
          z3q = mfma32(pq[ks], w3l[ks], z3q);
        }
      }
    }
    if (g + 1 < ngroups) load_x(k, g + 1, pq, pk);
    else load_x(k + 1, 0, pq, pk);
    // H = silu(Z) to LDS (keys: region B, queries: HQ), silu'(Z) of the keys kept for D1.  Gated:
    // H = silu(Z1) Z3, and the keys keep Z3 silu'(Z1) (for D1) and silu(Z1) (for D3)
    f32x16 hz, zp, a3;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const float sg = sigmoidf_(zk[r]);
      if constexpr (GATED) {
        a3[r] = zk[r] * sg;
        hz[r] = a3[r] * z3k[r];
        zp[r] = z3k[r] * (sg * (1.0f + zk[r] * (1.0f - sg)));
      } else {
        hz[r] = zk[r] * sg;
        zp[r] = sg * (1.0f + zk[r] * (1.0f - sg));
      }
    }
    u32x4 hph[2], hpl[2];  // hi/lo words of the keys' H, k-steps over the set's rows
#pragma unroll
    for (int kl = 0; kl < 2; ++kl) {
      tile_op(hz, kl, hph[kl], hpl[kl]);
      store_rows<PL>(sm, rb, rb + HSZ, LH, hph[kl], hpl[kl], GR * s + 16 * kl, h_own, hf);
    }
    if (withq) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        hz[r] = zq[r] * sigmoidf_(zq[r]);
        if constexpr (GATED) hz[r] *= z3q[r];
      }
#pragma unroll
      for (int kl = 0; kl < 2; ++kl) {
        u32x4 qh, ql;
        tile_op(hz, kl, qh, ql);
        store_rows<PL>(sm, hq, hq + HSZ, LH, qh, ql, GR * s + 16 * kl, h_own, hf);
      }
    }
    __syncthreads();
    // Yh = H W2^T: 16x16 tiles, wave w owns values [16w, 16w+16), both row halves of the set;
    // the B operand (k = h, n = v) comes from W2^T [h][v] by transposing reads: lane 4e + q of
    // 16-lane group g names row 32ks + 8g + e (+4), columns 16w + 4q .. +3
    f32x4 yk[2] = {f32x4{0.f, 0.f, 0.f, 0.f}, f32x4{0.f, 0.f, 0.f, 0.f}};
    f32x4 yq[2] = {f32x4{0.f, 0.f, 0.f, 0.f}, f32x4{0.f, 0.f, 0.f, 0.f}};
    {
      const int ob = ((lane >> 4) * 8 + ((lane >> 2) & 3)) * LE + 16 * w + 4 * (lane & 3);
#pragma unroll
      for (int ks = 0; ks < HD / 32; ++ks) {
        const int o1 = ob + 32 * ks * LE, o2 = o1 + 4 * LE;
        const u32x4 bh = cat2(lds_tr16(sm + wth + o1), lds_tr16(sm + wth + o2));
        const u32x4 bl = cat2(lds_tr16(sm + wtl + o1), lds_tr16(sm + wtl + o2));
#pragma unroll
        for (int rt = 0; rt < 2; ++rt) {
          const int oa = (GR * s + 16 * rt + (lane & 15)) * LH + 32 * ks + 8 * (lane >> 4);
          yk[rt] = mmp16<PL>(lds16(sm, rb + oa), lds16(sm, rb + HSZ + oa), bh, bl, yk[rt]);
          if (withq) yq[rt] = mmp16<PL>(lds16(sm, hq + oa), lds16(sm, hq + HSZ + oa), bh, bl, yq[rt]);
        }
      }
    }
    // D2 = 2 (Yh - V): to LDS as [row][v] (operand of D2 W2) and [v][row] (operand of D2^T H)
#pragma unroll
    for (int rt = 0; rt < 2; ++rt) {
      const int rr = GR * s + 16 * rt + 4 * (lane >> 4);
      float d2[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const uint32_t pv = vv[4 * rt + u];
        d2[u] = RES ? 2.0f * (yk[rt][u] - (bf16_value(pv & 0xFFFFu) - __uint_as_float(pv & 0xFFFF0000u)))
                    : 2.0f * (yk[rt][u] - bf16_value(pv));
      }
      uint32_t h0, l0, h1, l1;
      split2(d2[0], d2[1], h0, l0);
      split2(d2[2], d2[3], h1, l1);
      const uint32_t hh[4] = {h0 & 0xFFFFu, h0 >> 16, h1 & 0xFFFFu, h1 >> 16};
      const uint32_t ll[4] = {l0 & 0xFFFFu, l0 >> 16, l1 & 0xFFFFu, l1 >> 16};
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        sm[d2h + (rr + u) * LE + vcol] = (uint16_t)hh[u];
        if constexpr (!PL) sm[d2l + (rr + u) * LE + vcol] = (uint16_t)ll[u];
      }
      *(uint2*)(sm + dth + vcol * LR + rr) = uint2{h0, h1};
      if constexpr (!PL) *(uint2*)(sm + dtl + vcol * LR + rr) = uint2{l0, l1};
    }
    {  // X^T of the group for the G1 product
      const int r = t >> 3, d0 = (t & 7) * 8;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        sm[xth + (d0 + 2 * i) * LR + r] = (uint16_t)(xt[i] & 0xFFFFu);
        sm[xth + (d0 + 2 * i + 1) * LR + r] = (uint16_t)(xt[i] >> 16);
      }
    }
    // Y of the queries (after the loads above have been waited for)
    if (withq) {
      const int vy = 4 * (lane >> 4) * D + vcol;  // element offset of this lane's first output
      if (a.out_bf16) {
#pragma unroll
        for (int rt = 0; rt < 2; ++rt)
#pragma unroll
          for (int u = 0; u < 4; ++u)
            buf_st_u16(rY, vy * 2 + u * D * 2, (rset + 16 * rt) * D * 2, bf16_bits(yq[rt][u]));
      } else {
#pragma unroll
        for (int rt = 0; rt < 2; ++rt)
#pragma unroll
          for (int u = 0; u < 4; ++u) buf_st(rY, vy * 4 + u * D * 4, (rset + 16 * rt) * D * 4, yq[rt][u]);
      }
    }
    __syncthreads();
    // Pm = D2 W2 (k = v), D1 = Pm * silu'(Z)
    f32x16 p = zero16();
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      const int o0 = (GR * s + l32) * LE + 16 * ks + 4 * hf;
      const u32x4 ah = cat2(lds8(sm, d2h + o0), lds8(sm, d2h + o0 + 8));
      const u32x4 al = cat2(lds8(sm, d2l + o0), lds8(sm, d2l + o0 + 8));
      const int ob = h_own * LE + 16 * ks + 4 * hf;
      const u32x4 bh = cat2(lds8(sm, wth + ob), lds8(sm, wth + ob + 8));
      const u32x4 bl = cat2(lds8(sm, wtl + ob), lds8(sm, wtl + ob + 8));
      p = mmp<PL>(ah, al, bh, bl, p);
    }
    f32x16 p3;  // gated: D3 = Pm * silu(Z1)
    if constexpr (GATED) {
#pragma unroll
      for (int r = 0; r < 16; ++r) p3[r] = p[r] * a3[r];
    }
#pragma unroll
    for (int r = 0; r < 16; ++r) p[r] *= zp[r];
    // G1^T += X^T D1 and G2 += D2^T H (k = the set's rows, B operands from registers); gated:
    // G3^T += X^T D3
#pragma unroll
    for (int kl = 0; kl < 2; ++kl) {
      u32x4 dh, dl, d3h, d3l;
      tile_op(p, kl, dh, dl);
      if constexpr (GATED) tile_op(p3, kl, d3h, d3l);
      const u32x4 hh = hph[kl], hl = hpl[kl];
#pragma unroll
      for (int tt = 0; tt < 2; ++tt) {
        const int o0 = (32 * tt + l32) * LR + GR * s + 16 * kl + 4 * hf;
        const u32x4 xa = cat2(lds8(sm, xth + o0), lds8(sm, xth + o0 + 8));
        gr[0][tt] = mfma32(xa, dh, gr[0][tt]);
        if constexpr (!PL) gr[0][tt] = mfma32(xa, dl, gr[0][tt]);
        if constexpr (GATED) {
          gr3[tt] = mfma32(xa, d3h, gr3[tt]);
          gr3[tt] = mfma32(xa, d3l, gr3[tt]);
        }
        const u32x4 ah = cat2(lds8(sm, dth + o0), lds8(sm, dth + o0 + 8));
        const u32x4 al = cat2(lds8(sm, dtl + o0), lds8(sm, dtl + o0 + 8));
        gr[1][tt] = mmp<PL>(ah, al, hh, hl, gr[1][tt]);
      }
    }
    // No barrier here: the next group writes H after its X W1^T (every wave is past this
    // group's second barrier, so done with H W2^T) and D2, D2^T, X^T after its first barrier,
    // which every wave reaches after finishing these reads.
  };

  u32x4 pq[4], pk[4];
  load_x(0, 0, pq, pk);
  for (int k = 0; k < a.nchunks; ++k) {
    // partial gradients over this set's rows: gr[0] = G1^T tiles (d rows 0..31 / 32..63,
    // h_own), gr[1] = G2 tiles (v rows 0..31 / 32..63, h_own)
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int j = 0; j < 2; ++j) gr[i][j] = zero16();
    if constexpr (GATED) gr3[0] = gr3[1] = zero16();
    for (int g = 0; g < ngroups; ++g) run_group(k, g, pq, pk);

    // Swap partial gradients: set 0 keeps G1 and passes its G2 partial, set 1 the reverse.
    // The slots were last read by the final group's H W2^T, before its second barrier.
    f32x16 x[2], x3[2];
    if constexpr (SPLIT) {
      // through this memory's exchange slots: slot s holds the partial this set passes on (gated:
      // slot 2 set 1's G3 partial)
      AM_LANE_VARS;
      const rsrc_t rx = make_rsrc(a.xs + (int64_t)m * NSLOT * P2, (uint32_t)(NSLOT * P2 * 4));
      const int vx = (((w * 2) * 4) * 64 + lane) * 16;  // byte offset of (tile 0, quad 0) of this lane
      if (s == 0) {
#pragma unroll
        for (int tt = 0; tt < 2; ++tt)
#pragma unroll
          for (int q = 0; q < 4; ++q)
            buf_st4(rx, vx, ((tt * 4 + q) * 64) * 16,
                    float4{gr[1][tt][4 * q], gr[1][tt][4 * q + 1], gr[1][tt][4 * q + 2], gr[1][tt][4 * q + 3]});
      } else {
#pragma unroll
        for (int tt = 0; tt < 2; ++tt)
#pragma unroll
          for (int q = 0; q < 4; ++q)
            buf_st4(rx, vx + P2 * 4, ((tt * 4 + q) * 64) * 16,
                    float4{gr[0][tt][4 * q], gr[0][tt][4 * q + 1], gr[0][tt][4 * q + 2], gr[0][tt][4 * q + 3]});
        if constexpr (GATED) {
#pragma unroll
          for (int tt = 0; tt < 2; ++tt)
#pragma unroll
            for (int q = 0; q < 4; ++q)
              buf_st4(rx, vx + 2 * P2 * 4, ((tt * 4 + q) * 64) * 16,
                      float4{gr3[tt][4 * q], gr3[tt][4 * q + 1], gr3[tt][4 * q + 2], gr3[tt][4 * q + 3]});
        }
      }
      pair_sync(pair_ctr, pair_target, stuck, pair_local);
      const int vsrc = vx + (s ? 0 : P2 * 4);
#pragma unroll
      for (int tt = 0; tt < 2; ++tt)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const float4 f = buf_ld4(rx, vsrc, ((tt * 4 + q) * 64) * 16);
          const float fv[4] = {f.x, f.y, f.z, f.w};
#pragma unroll
          for (int u = 0; u < 4; ++u) x[tt][4 * q + u] = (s ? gr[1][tt][4 * q + u] : gr[0][tt][4 * q + u]) + fv[u];
        }
      if constexpr (GATED) {
        if (s == 0) {
#pragma unroll
          for (int tt = 0; tt < 2; ++tt)
#pragma unroll
            for (int q = 0; q < 4; ++q) {
              const float4 f = buf_ld4(rx, vx + 2 * P2 * 4, ((tt * 4 + q) * 64) * 16);
              const float fv[4] = {f.x, f.y, f.z, f.w};
#pragma unroll
              for (int u = 0; u < 4; ++u) x3[tt][4 * q + u] = gr3[tt][4 * q + u] + fv[u];
            }
        }
      }
    } else {
      AM_LANE_VARS;
      float* xg1 = (float*)(sm + opq(XG1));
      float* xg2 = (float*)(sm + opq(XG2));
      if (s == 0) {
#pragma unroll
        for (int tt = 0; tt < 2; ++tt)
#pragma unroll
          for (int q = 0; q < 4; ++q)
            *(float4*)(xg2 + (((w * 2 + tt) * 4 + q) * 64 + lane) * 4) =
                float4{gr[1][tt][4 * q], gr[1][tt][4 * q + 1], gr[1][tt][4 * q + 2], gr[1][tt][4 * q + 3]};
      } else {
#pragma unroll
        for (int tt = 0; tt < 2; ++tt)
#pragma unroll
          for (int q = 0; q < 4; ++q)
            *(float4*)(xg1 + (((w * 2 + tt) * 4 + q) * 64 + lane) * 4) =
                float4{gr[0][tt][4 * q], gr[0][tt][4 * q + 1], gr[0][tt][4 * q + 2], gr[0][tt][4 * q + 3]};
      }
      __syncthreads();
      const float* src = s ? xg2 : xg1;
#pragma unroll
      for (int tt = 0; tt < 2; ++tt)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const float4 f = *(const float4*)(src + (((w * 2 + tt) * 4 + q) * 64 + lane) * 4);
          const float fv[4] = {f.x, f.y, f.z, f.w};
#pragma unroll
          for (int u = 0; u < 4; ++u) x[tt][4 * q + u] = (s ? gr[1][tt][4 * q + u] : gr[0][tt][4 * q + u]) + fv[u];
        }
    }

    const int64_t gk = (int64_t)m * a.ld_gate + k;
    const float th = a.theta[gk], et = a.eta[gk], om = 1.0f - a.alpha[gk];
    const float* Wsrc = (k == 0) ? Win : Wout;
    const float* Ssrc = (k == 0) ? Sin : Sout;
    // This set's state, loaded in quarters during the Newton-Schulz phase so that the loads
    // complete under it: register r of tile tt holds the element of row 32tt + 8(r/4) + 4hf + r%4
    // of G1^T (set 0: W1[h_own][d]) or of G2 (set 1: W2[v][h_own], kept transposed in T2 within
    // a launch).  Buffer accesses: one per-lane byte offset, per-register offsets are constants.
    const rsrc_t rt2 = make_rsrc(a.T2 + (int64_t)m * 2 * P2, (uint32_t)(2 * P2 * 4));
    const rsrc_t rs = s ? rt2 : make_rsrc(Ssrc, (uint32_t)(PM * 4));
    const rsrc_t rw = s ? rt2 : make_rsrc(Wsrc, (uint32_t)(PM * 4));
    float sv[2][16], wv[2][16];
    auto pre = [&](auto part) __attribute__((always_inline)) {
      constexpr int tt = decltype(part)::value >> 1, q0 = 2 * (decltype(part)::value & 1);
      AM_LANE_VARS;
      const int vo1 = (h_own * D + 4 * hf) * 4;  // W1[h_own][4hf], W2^T[h_own][4hf]
      const int vs = vo1 + (s ? P2 * 4 : 0);
#pragma unroll
      for (int q = q0; q < q0 + 2; ++q) {
        const float4 so = buf_ld4(rs, vs, (32 * tt + 8 * q) * 4);
        const float4 wo = buf_ld4(rw, vo1, (32 * tt + 8 * q) * 4);
        sv[tt][4 * q] = so.x; sv[tt][4 * q + 1] = so.y; sv[tt][4 * q + 2] = so.z; sv[tt][4 * q + 3] = so.w;
        wv[tt][4 * q] = wo.x; wv[tt][4 * q + 1] = wo.y; wv[tt][4 * q + 2] = wo.z; wv[tt][4 * q + 3] = wo.w;
      }
    };

    {
      AM_LANE_VARS;
      const int bxh = opq(NX + s * NXS), bah = opq(NA + s * NAS), bbh = opq(NB + s * NBS);
      auto set_bar = [&]() __attribute__((always_inline)) {
        if constexpr (SPLIT) __syncthreads();
        else set_barrier(set_count, set_target, stuck, lane);
      };
      newton_schulz1<PL, SPLIT>(x, sm, bxh, bxh + HD * 64, bah, bah + 64 * LD, bbh, bbh + 64 * LE, red + 4 * s, a,
                                lane, w, pre, set_bar);
    }
    // S = eta S - theta NS(G), W = (1 - alpha) W + S for this set's matrix
#pragma unroll
    for (int tt = 0; tt < 2; ++tt)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const float sn = et * sv[tt][r] - th * x[tt][r];
        const float wn = om * wv[tt][r] + sn;
        sv[tt][r] = sn;
        x[tt][r] = wn;
      }
    // A non-finite value never becomes finite again under the momentum, forgetting and
    // Newton-Schulz steps (its row and column turn NaN or stay infinite), so checking the state
    // after the last chunk of the launch flags every launch that produced one.
    if (k + 1 == a.nchunks) {
#pragma unroll
      for (int tt = 0; tt < 2; ++tt)
#pragma unroll
        for (int r = 0; r < 16; ++r) bad |= !(isfinite(sv[tt][r]) && isfinite(x[tt][r]));
    }
    // The W1 handoff overwrites the A buffers, dead after the last iteration's third barrier.
    // Set 1's W2^T operand copies overwrite its Newton-Schulz X^T buffer, which the last
    // iteration's B X still reads (each wave its own columns, but the copy rows of one wave span
    // columns of its neighbours): they are written after the barrier below, which every wave
    // reaches only after that product.  Until the next group's first barrier nothing reads
    // W2^T, and the group writes only its H buffers, which lie outside the copies.
    u32x4* ho = (u32x4*)(sm + opq(HOFF));
    {
    AM_LANE_VARS;
    const rsrc_t rs_out = make_rsrc(Sout, (uint32_t)(PM * 4)), rw_out = make_rsrc(Wout, (uint32_t)(PM * 4));
    const bool last = k + 1 == a.nchunks;
    const int wo1 = (h_own * D + 4 * hf) * 4, wo2 = ((int)O2 + 4 * hf * HD + h_own) * 4;
    if (s == 0 || !last) {
      const rsrc_t rs = s ? rt2 : rs_out, rw = s ? rt2 : rw_out;
      const int vs = wo1 + (s ? P2 * 4 : 0);
#pragma unroll
      for (int tt = 0; tt < 2; ++tt)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          buf_st4(rs, vs, (32 * tt + 8 * q) * 4,
                  float4{sv[tt][4 * q], sv[tt][4 * q + 1], sv[tt][4 * q + 2], sv[tt][4 * q + 3]});
          buf_st4(rw, wo1, (32 * tt + 8 * q) * 4,
                  float4{x[tt][4 * q], x[tt][4 * q + 1], x[tt][4 * q + 2], x[tt][4 * q + 3]});
        }
    } else {
#pragma unroll
      for (int tt = 0; tt < 2; ++tt)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int so = (32 * tt + 8 * (r >> 2) + (r & 3)) * HD * 4;
          buf_st(rs_out, wo2, so, sv[tt][r]);
          buf_st(rw_out, wo2, so, x[tt][r]);
        }
    }
    if constexpr (GATED) {
      // The gated memory's W3: set 0 orthogonalises and applies it after W1, in the same LDS
      // buffers (the W1 pass's last B X reads only this lane's own X^T rows, which the first
      // store of this pass overwrites; its A and B buffers are rewritten after barriers).
      if (s == 0) {
        const float* W3src = ((k == 0) ? Win : Wout) + O3;
        const float* S3src = ((k == 0) ? Sin : Sout) + O3;
        const rsrc_t rs3 = make_rsrc(S3src, (uint32_t)(P1 * 4)), rw3 = make_rsrc(W3src, (uint32_t)(P1 * 4));
        float sv3[2][16], wv3[2][16];
        auto pre3 = [&](auto part) __attribute__((always_inline)) {
          constexpr int tt = decltype(part)::value >> 1, q0 = 2 * (decltype(part)::value & 1);
          const int vo1 = (h_own * D + 4 * hf) * 4;  // W3[h_own][4hf]
#pragma unroll
          for (int q = q0; q < q0 + 2; ++q) {
            const float4 so = buf_ld4(rs3, vo1, (32 * tt + 8 * q) * 4);
            const float4 wo = buf_ld4(rw3, vo1, (32 * tt + 8 * q) * 4);
            sv3[tt][4 * q] = so.x; sv3[tt][4 * q + 1] = so.y; sv3[tt][4 * q + 2] = so.z; sv3[tt][4 * q + 3] = so.w;
            wv3[tt][4 * q] = wo.x; wv3[tt][4 * q + 1] = wo.y; wv3[tt][4 * q + 2] = wo.z; wv3[tt][4 * q + 3] = wo.w;
          }
        };
        auto bar = [&]() __attribute__((always_inline)) { __syncthreads(); };
        const int bxh = opq(NX), bah = opq(NA), bbh = opq(NB);
        newton_schulz1<PL, true>(x3, sm, bxh, bxh + HD * 64, bah, bah + 64 * LD, bbh, bbh + 64 * LE, red, a, lane, w,
                                 pre3, bar);
        const rsrc_t rs3o = make_rsrc(Sout + O3, (uint32_t)(P1 * 4)), rw3o = make_rsrc(Wout + O3, (uint32_t)(P1 * 4));
#pragma unroll
        for (int tt = 0; tt < 2; ++tt)
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            float sn[4], wn[4];
#pragma unroll
            for (int u = 0; u < 4; ++u) {
              const int r = 4 * q + u;
              sn[u] = et * sv3[tt][r] - th * x3[tt][r];
              wn[u] = om * wv3[tt][r] + sn[u];
              x3[tt][r] = wn[u];
              if (last) bad |= !(isfinite(sn[u]) && isfinite(wn[u]));
            }
            buf_st4(rs3o, wo1, (32 * tt + 8 * q) * 4, float4{sn[0], sn[1], sn[2], sn[3]});
            buf_st4(rw3o, wo1, (32 * tt + 8 * q) * 4, float4{wn[0], wn[1], wn[2], wn[3]});
          }
      }
    }
    if constexpr (!SPLIT) {
    // the handoff lies over both sets' A buffers: wait for the other set's last iteration
    __syncthreads();
    if (s == 0) {
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) {
        u32x4 wh, wl;
        tile_op(x[ks >> 1], ks & 1, wh, wl);
        ho[(w * 8 + ks) * 64 + lane] = wh;
        if constexpr (!PL) ho[(w * 8 + 4 + ks) * 64 + lane] = wl;
      }
    }
    }
    }
    if constexpr (SPLIT) {
      // Both sets' new weights are stored (set 0: W1 in the state, set 1: W2^T in T2); after the
      // pair's wait each set builds the operands of the next chunk from its own registers and the
      // other's stored matrix.  The barrier inside the wait also orders these LDS writes after the
      // last Newton-Schulz reads of the buffers below them.
      if (k + 1 < a.nchunks) {
        pair_sync(pair_ctr, pair_target, stuck, pair_local);
        AM_LANE_VARS;
        if (s == 0) {
          f32x16 y2[2];
          const int vo1 = (h_own * D + 4 * hf) * 4;  // W2^T[h_own][4hf] in T2
#pragma unroll
          for (int tt = 0; tt < 2; ++tt)
#pragma unroll
            for (int q = 0; q < 4; ++q) {
              const float4 f = buf_ld4(rt2, vo1, (32 * tt + 8 * q) * 4);
              y2[tt][4 * q] = f.x; y2[tt][4 * q + 1] = f.y; y2[tt][4 * q + 2] = f.z; y2[tt][4 * q + 3] = f.w;
            }
#pragma unroll
          for (int ks = 0; ks < 4; ++ks) {
            u32x4 wh, wl;
            tile_op(y2[ks >> 1], ks & 1, wh, wl);
            store_rows_T<PL>(sm, wth, wtl, LE, wh, wl, 16 * ks, h_own, hf);
            tile_op(x[ks >> 1], ks & 1, w1h[ks], w1l[ks]);
            if constexpr (GATED) tile_op(x3[ks >> 1], ks & 1, w3h[ks], w3l[ks]);
          }
        } else {
#pragma unroll
          for (int ks = 0; ks < 4; ++ks) {
            u32x4 wh, wl;
            tile_op(x[ks >> 1], ks & 1, wh, wl);
            store_rows_T<PL>(sm, wth, wtl, LE, wh, wl, 16 * ks, h_own, hf);
          }
          const rsrc_t rw1 = make_rsrc(Wout, (uint32_t)(P1 * 4));
          const int vw = (h_own * D + 4 * hf) * 4;  // W1[h_own][4hf] in the state
#pragma unroll
          for (int ks = 0; ks < 4; ++ks) {
            const float4 p0 = buf_ld4(rw1, vw, 16 * ks * 4);
            const float4 p1 = buf_ld4(rw1, vw, (16 * ks + 8) * 4);
            const float v[8] = {p0.x, p0.y, p0.z, p0.w, p1.x, p1.y, p1.z, p1.w};
            pack8(v, w1h[ks], w1l[ks]);
          }
          if constexpr (GATED) {
            const rsrc_t rw3 = make_rsrc(Wout + O3, (uint32_t)(P1 * 4));
#pragma unroll
            for (int ks = 0; ks < 4; ++ks) {
              const float4 p0 = buf_ld4(rw3, vw, 16 * ks * 4);
              const float4 p1 = buf_ld4(rw3, vw, (16 * ks + 8) * 4);
              const float v[8] = {p0.x, p0.y, p0.z, p0.w, p1.x, p1.y, p1.z, p1.w};
              pack8(v, w3h[ks], w3l[ks]);
            }
          }
        }
        // the next group's first LDS reads of W2^T come after its first barrier
      }
      continue;
    }
    __syncthreads();
    // both sets take the new W1 slices from LDS (the registers then hold nothing across the
    // Newton-Schulz phase)
    {
      AM_LANE_VARS;
      if (s == 1) {
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) {
          u32x4 wh, wl;
          tile_op(x[ks >> 1], ks & 1, wh, wl);
          store_rows_T<PL>(sm, wth, wtl, LE, wh, wl, 16 * ks, h_own, hf);
        }
      }
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) {
        w1h[ks] = ho[(w * 8 + ks) * 64 + lane];
        if constexpr (!PL) w1l[ks] = ho[(w * 8 + 4 + ks) * 64 + lane];
      }
    }
  }
  if (bad || stuck) a.flag[0] = 1;
#undef AM_LANE_VARS
}

// ---------------------------------------------------------------------------- per-token gates
//
// The same memory with per-token gates and no orthogonalisation, chunks of exactly 64 tokens (one
// double group per chunk).  The chunk's update is the coefficient form of the per-token recurrence
// (titans-pytorch-mlx README, Core Equations, Eq. 13-14, with every gradient of the chunk at its
// start weights: ATLAS summary, section 3.3):
//   S_end = P S0 - sum_j cS_j g_j,   W_end = beta W0 + a_S S0 - sum_j cW_j g_j,
// with cW, cS and (P, beta, a_S) from the gate scan.  The two weighted gradient sums are formed one
// after the other from the same chunk activations, kept in registers: D1 and H of the set's rows
// are weighted per row before their hi/lo split (G1^T = X^T (c D1), G2 = D2^T (c H)); each sum's
// partials are swapped between the sets like the per-chunk kernel's, so that set 0 applies W1's
// update and set 1 W2's.  The S sum comes first: S_end is stored at once and only S0 stays live
// for the W update.
struct PtArgs {
  Args a;
  const float* cW;    // chunk 0 of this launch, memory 0; memory m at + m * ld_c
  const float* cS;
  const float* scal;  // (P, beta, a_S) per chunk; memory m at + m * ld_s
  int64_t ld_c, ld_s;
};
constexpr int PT_CF = LDS_U16 * 2 + 16 * 4;            // byte offset of the chunk's coefficients
constexpr int PT_LDS_BYTES = PT_CF + (2 * GROWS + 4) * 4;
static_assert(PT_LDS_BYTES <= 160 * 1024, "LDS");

template <bool RES>
__global__ void __launch_bounds__(NT) fused_pt_kernel(PtArgs pa) {
  extern __shared__ __attribute__((aligned(16))) uint16_t sm[];
  const Args& a = pa.a;
  float* cf = (float*)((char*)sm + PT_CF);  // [cW of 64 rows | cS of 64 rows | P, beta, a_S]
  const int m = blockIdx.x;
  const int t0 = threadIdx.x;
  const int w8 = __builtin_amdgcn_readfirstlane(t0 >> 6);
  const int s = w8 >> 2, w = w8 & 3;
#define AM_LANE_VARS                                                                \
  const int t = opv(t0), lane = t & 63, hf = lane >> 5, l32 = lane & 31;          \
  const int h_own = 32 * w + l32;                                                 \
  (void)hf; (void)l32; (void)h_own
  const int nT = a.nchunks * a.C;
  const rsrc_t rK = make_rsrc(a.K + (int64_t)m * a.ldT * D, (uint32_t)nT * D * 2);
  const rsrc_t rQ = (a.Y && a.Q) ? make_rsrc(a.Q + (int64_t)m * a.ldT * D, (uint32_t)nT * D * 2) : rK;
  const rsrc_t rV = make_rsrc(a.V + (int64_t)m * a.ldT * D, (uint32_t)nT * D * 2);
  const int ysz = a.out_bf16 ? 2 : 4;
  const rsrc_t rY = make_rsrc(a.Y ? (const char*)a.Y + (int64_t)m * a.ldT * D * ysz : nullptr,
                              a.Y ? (uint32_t)nT * D * ysz : 0u);
  const float* Win = a.Win + (int64_t)m * P;
  const float* Sin = a.Sin + (int64_t)m * P;
  float* Wout = a.Wout + (int64_t)m * P;
  float* Sout = a.Sout + (int64_t)m * P;
  const int wth = opq(WTH), wtl = opq(WTL);
  const int d2h = opq(D2H), d2l = opq(D2L), dth = opq(DTH), dtl = opq(DTL), xth = opq(XTH);
  const int rb = opq(RB);

  // prologue: W1 slice in registers, W2^T in LDS, set 1's transposed W2 state (as the per-chunk kernel)
  u32x4 w1h[4], w1l[4];
  {
  AM_LANE_VARS;
#pragma unroll
  for (int ks = 0; ks < 4; ++ks) {
    float v[8];
    const float4 p0 = *(const float4*)(Win + (int64_t)h_own * D + 16 * ks + 4 * hf);
    const float4 p1 = *(const float4*)(Win + (int64_t)h_own * D + 16 * ks + 8 + 4 * hf);
    v[0] = p0.x; v[1] = p0.y; v[2] = p0.z; v[3] = p0.w;
    v[4] = p1.x; v[5] = p1.y; v[6] = p1.z; v[7] = p1.w;
    pack8(v, w1h[ks], w1l[ks]);
  }
  for (int e = t; e < D * HD; e += NT) {
    const int vv = e / HD, hh = e % HD;
    uint32_t hi, lo;
    split_bf16(Win[P1 + e], hi, lo);
    sm[wth + hh * LE + vv] = (uint16_t)hi;
    sm[wtl + hh * LE + vv] = (uint16_t)lo;
  }
  if (s == 1) {
    const rsrc_t rt2 = make_rsrc(a.T2 + (int64_t)m * 2 * P2, (uint32_t)(2 * P2 * 4));
    const int vt = (h_own * D + 4 * hf) * 4;
#pragma unroll
    for (int tt = 0; tt < 2; ++tt)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        float wv4[4], sv4[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          const int64_t o = P1 + (int64_t)(32 * tt + 8 * q + 4 * hf + u) * HD + h_own;
          wv4[u] = Win[o];
          sv4[u] = Sin[o];
        }
        buf_st4(rt2, vt, (32 * tt + 8 * q) * 4, float4{wv4[0], wv4[1], wv4[2], wv4[3]});
        buf_st4(rt2, vt + P2 * 4, (32 * tt + 8 * q) * 4, float4{sv4[0], sv4[1], sv4[2], sv4[3]});
      }
  }
  }
  __syncthreads();

  const bool withq = a.Y != nullptr;
  auto load_x = [&](int k, u32x4 (&pq)[4], u32x4 (&pk)[4]) __attribute__((always_inline)) {
    AM_LANE_VARS;
    if (k >= a.nchunks) k = a.nchunks - 1;  // past the end of the launch: repeat the last loads
    const int rset = (k * a.C + GR * s) * D * 2;
    const int vx = (l32 * D + 4 * hf) * 2;
#pragma unroll
    for (int ks = 0; ks < 4; ++ks)
      pk[ks] = cat2(buf_ld8(rK, vx + 32 * ks, rset), buf_ld8(rK, vx + 32 * ks + 16, rset));
#pragma unroll
    for (int ks = 0; ks < 4; ++ks)
      pq[ks] = cat2(buf_ld8(rQ, vx + 32 * ks, rset), buf_ld8(rQ, vx + 32 * ks + 16, rset));
  };

  bool bad = false;
  const int hq = opq(HQ);
  // The chunk's rows: Z, H and Yh of queries and keys, Y of the queries, D2 (LDS), X^T (LDS);
  // returns the keys' D1 (p) and H (hz) tiles of this set's rows, fp32.
  auto run_group = [&](int k, u32x4 (&pq)[4], u32x4 (&pk)[4], f32x16& p, f32x16& hz) __attribute__((always_inline)) {
    AM_LANE_VARS;
    const int vcol = 16 * w + (lane & 15);
    const int row0 = k * a.C;
    const int rset = row0 + GR * s;
    const u32x4 xt = buf_ld16(rK, ((t >> 3) * D + (t & 7) * 8) * 2, row0 * D * 2);
    uint32_t vv[8];
#pragma unroll
    for (int rt = 0; rt < 2; ++rt)
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int vo = (4 * (lane >> 4) * D + vcol) * 2 + u * D * 2, so = (rset + 16 * rt) * D * 2;
        if (RES) {
          v2u16 pr;
          pr.x = __builtin_amdgcn_raw_buffer_load_b16(rV, vo, so, 0);
          pr.y = __builtin_amdgcn_raw_buffer_load_b16(rK, vo, so, 0);
          vv[4 * rt + u] = __builtin_bit_cast(uint32_t, pr);
        } else {
          vv[4 * rt + u] = buf_ld_u16(rV, vo, so);
        }
      }
    f32x16 zk = zero16(), zq = zero16();
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      zk = mfma32(pk[ks], w1h[ks], zk);
      zk = mfma32(pk[ks], w1l[ks], zk);
    }
    if (withq) {
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) {
        zq = mfma32(pq[ks], w1h[ks], zq);
        zq = mfma32(pq[ks], w1l[ks], zq);
      }
    }
    load_x(k + 1, pq, pk);
    f32x16 zp;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const float sg = sigmoidf_(zk[r]);
      hz[r] = zk[r] * sg;
      zp[r] = sg * (1.0f + zk[r] * (1.0f - sg));
    }
#pragma unroll
    for (int kl = 0; kl < 2; ++kl) {
      u32x4 hh, hl;
      tile_op(hz, kl, hh, hl);
      store_rows(sm, rb, rb + HSZ, LH, hh, hl, GR * s + 16 * kl, h_own, hf);
    }
    if (withq) {
      f32x16 hqz;
#pragma unroll
      for (int r = 0; r < 16; ++r) hqz[r] = zq[r] * sigmoidf_(zq[r]);
#pragma unroll
      for (int kl = 0; kl < 2; ++kl) {
        u32x4 qh, ql;
        tile_op(hqz, kl, qh, ql);
        store_rows(sm, hq, hq + HSZ, LH, qh, ql, GR * s + 16 * kl, h_own, hf);
      }
    }
    __syncthreads();
    f32x4 yk[2] = {f32x4{0.f, 0.f, 0.f, 0.f}, f32x4{0.f, 0.f, 0.f, 0.f}};
    f32x4 yq[2] = {f32x4{0.f, 0.f, 0.f, 0.f}, f32x4{0.f, 0.f, 0.f, 0.f}};
    {
      const int ob = ((lane >> 4) * 8 + ((lane >> 2) & 3)) * LE + 16 * w + 4 * (lane & 3);
#pragma unroll
      for (int ks = 0; ks < HD / 32; ++ks) {
        const int o1 = ob + 32 * ks * LE, o2 = o1 + 4 * LE;
        const u32x4 bh = cat2(lds_tr16(sm + wth + o1), lds_tr16(sm + wth + o2));
        const u32x4 bl = cat2(lds_tr16(sm + wtl + o1), lds_tr16(sm + wtl + o2));
#pragma unroll
        for (int rt = 0; rt < 2; ++rt) {
          const int oa = (GR * s + 16 * rt + (lane & 15)) * LH + 32 * ks + 8 * (lane >> 4);
          yk[rt] = mma3_16(lds16(sm, rb + oa), lds16(sm, rb + HSZ + oa), bh, bl, yk[rt]);
          if (withq) yq[rt] = mma3_16(lds16(sm, hq + oa), lds16(sm, hq + HSZ + oa), bh, bl, yq[rt]);
        }
      }
    }
#pragma unroll
    for (int rt = 0; rt < 2; ++rt) {
      const int rr = GR * s + 16 * rt + 4 * (lane >> 4);
      float d2[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const uint32_t pv = vv[4 * rt + u];
        d2[u] = RES ? 2.0f * (yk[rt][u] - (bf16_value(pv & 0xFFFFu) - __uint_as_float(pv & 0xFFFF0000u)))
                    : 2.0f * (yk[rt][u] - bf16_value(pv));
      }
      uint32_t h0, l0, h1, l1;
      split2(d2[0], d2[1], h0, l0);
      split2(d2[2], d2[3], h1, l1);
      const uint32_t hh[4] = {h0 & 0xFFFFu, h0 >> 16, h1 & 0xFFFFu, h1 >> 16};
      const uint32_t ll[4] = {l0 & 0xFFFFu, l0 >> 16, l1 & 0xFFFFu, l1 >> 16};
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        sm[d2h + (rr + u) * LE + vcol] = (uint16_t)hh[u];
        sm[d2l + (rr + u) * LE + vcol] = (uint16_t)ll[u];
      }
      *(uint2*)(sm + dth + vcol * LR + rr) = uint2{h0, h1};
      *(uint2*)(sm + dtl + vcol * LR + rr) = uint2{l0, l1};
    }
    {
      const int r = t >> 3, d0 = (t & 7) * 8;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        sm[xth + (d0 + 2 * i) * LR + r] = (uint16_t)(xt[i] & 0xFFFFu);
        sm[xth + (d0 + 2 * i + 1) * LR + r] = (uint16_t)(xt[i] >> 16);
      }
    }
    if (withq) {
      const int vy = 4 * (lane >> 4) * D + vcol;
      if (a.out_bf16) {
#pragma unroll
        for (int rt = 0; rt < 2; ++rt)
#pragma unroll
          for (int u = 0; u < 4; ++u)
            buf_st_u16(rY, vy * 2 + u * D * 2, (rset + 16 * rt) * D * 2, bf16_bits(yq[rt][u]));
      } else {
#pragma unroll
        for (int rt = 0; rt < 2; ++rt)
#pragma unroll
          for (int u = 0; u < 4; ++u) buf_st(rY, vy * 4 + u * D * 4, (rset + 16 * rt) * D * 4, yq[rt][u]);
      }
    }
    __syncthreads();
    p = zero16();
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      const int o0 = (GR * s + l32) * LE + 16 * ks + 4 * hf;
      const u32x4 ah = cat2(lds8(sm, d2h + o0), lds8(sm, d2h + o0 + 8));
      const u32x4 al = cat2(lds8(sm, d2l + o0), lds8(sm, d2l + o0 + 8));
      const int ob = h_own * LE + 16 * ks + 4 * hf;
      const u32x4 bh = cat2(lds8(sm, wth + ob), lds8(sm, wth + ob + 8));
      const u32x4 bl = cat2(lds8(sm, wtl + ob), lds8(sm, wtl + ob + 8));
      p = mma3(ah, al, bh, bl, p);
    }
#pragma unroll
    for (int r = 0; r < 16; ++r) p[r] *= zp[r];
  };

  // One weighted gradient sum over this set's rows: G1^T += X^T (c D1), G2 += D2^T (c H), the row
  // weights c from LDS (coefficient array `co`: 0 = cW, 64 = cS).
  auto weighted_sum = [&](const f32x16& p, const f32x16& hz, int co, f32x16 (&gr)[2][2]) __attribute__((always_inline)) {
    AM_LANE_VARS;
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int j = 0; j < 2; ++j) gr[i][j] = zero16();
#pragma unroll
    for (int kl = 0; kl < 2; ++kl) {
      // registers 8kl..8kl+7 hold rows GR s + 16kl + 4hf + 0..3 and GR s + 16kl + 8 + 4hf + 0..3
      const float4 c0 = *(const float4*)(cf + co + GR * s + 16 * kl + 4 * hf);
      const float4 c1 = *(const float4*)(cf + co + GR * s + 16 * kl + 8 + 4 * hf);
      const float cr[8] = {c0.x, c0.y, c0.z, c0.w, c1.x, c1.y, c1.z, c1.w};
      float vd[8], vh[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        vd[e] = cr[e] * p[8 * kl + e];
        vh[e] = cr[e] * hz[8 * kl + e];
      }
      u32x4 dh, dl, hh, hl;
      pack8(vd, dh, dl);
      pack8(vh, hh, hl);
#pragma unroll
      for (int tt = 0; tt < 2; ++tt) {
        const int o0 = (32 * tt + l32) * LR + GR * s + 16 * kl + 4 * hf;
        const u32x4 xa = cat2(lds8(sm, xth + o0), lds8(sm, xth + o0 + 8));
        gr[0][tt] = mfma32(xa, dh, gr[0][tt]);
        gr[0][tt] = mfma32(xa, dl, gr[0][tt]);
        const u32x4 ah = cat2(lds8(sm, dth + o0), lds8(sm, dth + o0 + 8));
        const u32x4 al = cat2(lds8(sm, dtl + o0), lds8(sm, dtl + o0 + 8));
        gr[1][tt] = mma3(ah, al, hh, hl, gr[1][tt]);
      }
    }
  };
  // Swap the partial sums: set 0 ends with all of G1 (W1's sum), set 1 with all of G2.  The slots
  // are free from the group's H W2^T on; `first` tells whether a previous swap's reads must be
  // waited for.
  auto swap_partials = [&](f32x16 (&gr)[2][2], f32x16 (&g)[2], bool first) __attribute__((always_inline)) {
    AM_LANE_VARS;
    float* xg1 = (float*)(sm + opq(XG1));
    float* xg2 = (float*)(sm + opq(XG2));
    if (!first) __syncthreads();
    if (s == 0) {
#pragma unroll
      for (int tt = 0; tt < 2; ++tt)
#pragma unroll
        for (int q = 0; q < 4; ++q)
          *(float4*)(xg2 + (((w * 2 + tt) * 4 + q) * 64 + lane) * 4) =
              float4{gr[1][tt][4 * q], gr[1][tt][4 * q + 1], gr[1][tt][4 * q + 2], gr[1][tt][4 * q + 3]};
    } else {
#pragma unroll
      for (int tt = 0; tt < 2; ++tt)
#pragma unroll
        for (int q = 0; q < 4; ++q)
          *(float4*)(xg1 + (((w * 2 + tt) * 4 + q) * 64 + lane) * 4) =
              float4{gr[0][tt][4 * q], gr[0][tt][4 * q + 1], gr[0][tt][4 * q + 2], gr[0][tt][4 * q + 3]};
    }
    __syncthreads();
    const float* src = s ? xg2 : xg1;
#pragma unroll
    for (int tt = 0; tt < 2; ++tt)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const float4 f = *(const float4*)(src + (((w * 2 + tt) * 4 + q) * 64 + lane) * 4);
        const float fv[4] = {f.x, f.y, f.z, f.w};
#pragma unroll
        for (int u = 0; u < 4; ++u) g[tt][4 * q + u] = (s ? gr[1][tt][4 * q + u] : gr[0][tt][4 * q + u]) + fv[u];
      }
  };

  u32x4 pq[4], pk[4];
  load_x(0, pq, pk);
  for (int k = 0; k < a.nchunks; ++k) {
    {  // the chunk's coefficients (the previous chunk's readers are past its last barrier)
      AM_LANE_VARS;
      if (t < GROWS) cf[t] = pa.cW[(int64_t)m * pa.ld_c + (int64_t)k * GROWS + t];
      else if (t < 2 * GROWS) cf[t] = pa.cS[(int64_t)m * pa.ld_c + (int64_t)k * GROWS + (t - GROWS)];
      else if (t < 2 * GROWS + 3) cf[t] = pa.scal[(int64_t)m * pa.ld_s + (int64_t)k * 3 + (t - 2 * GROWS)];
    }
    f32x16 p, hz;
    run_group(k, pq, pk, p, hz);

    // this set's state (W1[h_own][d] or the transposed W2[v][h_own] in T2), as the per-chunk kernel
    const rsrc_t rt2 = make_rsrc(a.T2 + (int64_t)m * 2 * P2, (uint32_t)(2 * P2 * 4));
    const float* Wsrc = (k == 0) ? Win : Wout;
    const float* Ssrc = (k == 0) ? Sin : Sout;
    const rsrc_t rs = s ? rt2 : make_rsrc(Ssrc, (uint32_t)(P * 4));
    const rsrc_t rw = s ? rt2 : make_rsrc(Wsrc, (uint32_t)(P * 4));
    float sv[2][16], wv[2][16];
    {
      AM_LANE_VARS;
      const int vo1 = (h_own * D + 4 * hf) * 4;
      const int vs = vo1 + (s ? P2 * 4 : 0);
#pragma unroll
      for (int tt = 0; tt < 2; ++tt)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const float4 so = buf_ld4(rs, vs, (32 * tt + 8 * q) * 4);
          sv[tt][4 * q] = so.x; sv[tt][4 * q + 1] = so.y; sv[tt][4 * q + 2] = so.z; sv[tt][4 * q + 3] = so.w;
        }
    }
    const float cP = cf[2 * GROWS], cB = cf[2 * GROWS + 1], cA = cf[2 * GROWS + 2];
    f32x16 gr[2][2], g[2];
    // momentum: S_end = P S0 - sum_j cS_j g_j
    weighted_sum(p, hz, GROWS, gr);
    {
      AM_LANE_VARS;
      const int vo1 = (h_own * D + 4 * hf) * 4;
#pragma unroll
      for (int tt = 0; tt < 2; ++tt)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const float4 wo = buf_ld4(rw, vo1, (32 * tt + 8 * q) * 4);
          wv[tt][4 * q] = wo.x; wv[tt][4 * q + 1] = wo.y; wv[tt][4 * q + 2] = wo.z; wv[tt][4 * q + 3] = wo.w;
        }
    }
    swap_partials(gr, g, true);
    // S_end of this set's matrix, stored at once (W1 rows of set 0; set 1's W2 transposed in T2,
    // or in [v][h] after the last chunk)
    {
      AM_LANE_VARS;
      const bool last = k + 1 == a.nchunks;
      float sn[2][16];
#pragma unroll
      for (int tt = 0; tt < 2; ++tt)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          sn[tt][r] = fmaf(cP, sv[tt][r], -g[tt][r]);
          if (last) bad |= !isfinite(sn[tt][r]);
        }
      const rsrc_t rs_out = make_rsrc(Sout, (uint32_t)(P * 4));
      if (s == 0 || !last) {
        const rsrc_t rs2 = s ? rt2 : rs_out;
        const int vs = (h_own * D + 4 * hf) * 4 + (s ? P2 * 4 : 0);
#pragma unroll
        for (int tt = 0; tt < 2; ++tt)
#pragma unroll
          for (int q = 0; q < 4; ++q)
            buf_st4(rs2, vs, (32 * tt + 8 * q) * 4,
                    float4{sn[tt][4 * q], sn[tt][4 * q + 1], sn[tt][4 * q + 2], sn[tt][4 * q + 3]});
      } else {
        const int wo2 = ((int)P1 + 4 * hf * HD + h_own) * 4;
#pragma unroll
        for (int tt = 0; tt < 2; ++tt)
#pragma unroll
          for (int r = 0; r < 16; ++r) buf_st(rs_out, wo2, (32 * tt + 8 * (r >> 2) + (r & 3)) * HD * 4, sn[tt][r]);
      }
    }
    // weights: W_end = beta W0 + a_S S0 - sum_j cW_j g_j
    weighted_sum(p, hz, 0, gr);
    swap_partials(gr, g, false);
    f32x16 x[2];
#pragma unroll
    for (int tt = 0; tt < 2; ++tt)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        x[tt][r] = fmaf(cB, wv[tt][r], fmaf(cA, sv[tt][r], -g[tt][r]));
        if (k + 1 == a.nchunks) bad |= !isfinite(x[tt][r]);
      }
    // store W_end, hand the new W1 slices to set 1 (region A: D2, D2^T, X^T are dead, every wave
    // read them last before the second swap's first barrier) and write the new W2^T operand copies
    // (read last in the group's products), as the per-chunk kernel
    u32x4* ho = (u32x4*)(sm + opq(HOFF));
    {
      AM_LANE_VARS;
      const rsrc_t rw_out = make_rsrc(Wout, (uint32_t)(P * 4));
      const bool last = k + 1 == a.nchunks;
      const int wo1 = (h_own * D + 4 * hf) * 4, wo2 = ((int)P1 + 4 * hf * HD + h_own) * 4;
      if (s == 0 || !last) {
        const rsrc_t rw2 = s ? rt2 : rw_out;
#pragma unroll
        for (int tt = 0; tt < 2; ++tt)
#pragma unroll
          for (int q = 0; q < 4; ++q)
            buf_st4(rw2, wo1, (32 * tt + 8 * q) * 4,
                    float4{x[tt][4 * q], x[tt][4 * q + 1], x[tt][4 * q + 2], x[tt][4 * q + 3]});
      } else {
#pragma unroll
        for (int tt = 0; tt < 2; ++tt)
#pragma unroll
          for (int r = 0; r < 16; ++r) buf_st(rw_out, wo2, (32 * tt + 8 * (r >> 2) + (r & 3)) * HD * 4, x[tt][r]);
      }
      if (s == 0) {
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) {
          u32x4 wh, wl;
          tile_op(x[ks >> 1], ks & 1, wh, wl);
          ho[(w * 8 + ks) * 64 + lane] = wh;
          ho[(w * 8 + 4 + ks) * 64 + lane] = wl;
        }
      } else {
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) {
          u32x4 wh, wl;
          tile_op(x[ks >> 1], ks & 1, wh, wl);
          store_rows_T(sm, wth, wtl, LE, wh, wl, 16 * ks, h_own, hf);
        }
      }
    }
    __syncthreads();
    {
      AM_LANE_VARS;
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) {
        w1h[ks] = ho[(w * 8 + ks) * 64 + lane];
        w1l[ks] = ho[(w * 8 + 4 + ks) * 64 + lane];
      }
    }
    // the next chunk overwrites region A after its first barrier, which every wave reaches after
    // these handoff reads
  }
  if (bad) a.flag[0] = 1;
#undef AM_LANE_VARS
}

// The residual memory's retrieval adds the query to the fused kernel's output:
// Y[m][t][v] += q[m][t][v] over the call's tokens (fp32 output; 8 elements per thread).
__global__ void residual_output_kernel(const uint16_t* __restrict__ Q, float* __restrict__ Y, int64_t ld, int64_t n) {
  const int64_t e = ((int64_t)blockIdx.x * blockDim.x + threadIdx.x) * 8;
  if (e >= n) return;
  const int64_t o = (int64_t)blockIdx.y * ld + e;
  const u32x4 q = *(const u32x4*)(Q + o);
  float4* y = (float4*)(Y + o);
  float4 a = y[0], b = y[1];
  a.x += bf16_value(q[0] & 0xFFFFu);
  a.y += bf16_value(q[0] >> 16);
  a.z += bf16_value(q[1] & 0xFFFFu);
  a.w += bf16_value(q[1] >> 16);
  b.x += bf16_value(q[2] & 0xFFFFu);
  b.y += bf16_value(q[2] >> 16);
  b.z += bf16_value(q[3] & 0xFFFFu);
  b.w += bf16_value(q[3] >> 16);
  y[0] = a;
  y[1] = b;
}

}  // namespace fz

namespace fz {
// Memories of one launch of the two-workgroup form: 2 x 8 x ceil(M / 8) workgroups, one per CU.
constexpr int kSplitMaxMem = 128;
}  // namespace fz

bool fused_supported(const Dims& d) {
  const bool shape = d.kind == ATLASMEM_MLP2_SILU && d.gate_mode == ATLASMEM_PER_CHUNK && d.ns_steps > 0 &&
                     d.dk == fz::D && d.din == fz::D && d.dv == fz::D && d.dh == fz::HD && d.c == 1 &&
                     d.C % fz::GROWS == 0 && d.in_bf16;
  // the gated memory: only the two-workgroup form (its registers), split bf16
  if (d.gated) return shape && !d.residual && d.prec == 1 && d.M <= fz::kSplitMaxMem;
  return shape && d.prec != 2 && !(d.residual && d.out_bf16);
}

namespace fz {
__global__ void zero_ints_kernel(int* p, int n) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) p[i] = 0;
}
}  // namespace fz

int64_t fused_split_workspace_floats(const Dims& d) {
  if (!fused_supported(d) || d.M > fz::kSplitMaxMem) return 0;
  return (int64_t)d.M * ((d.gated ? 3 : 2) * fz::P2 + 32);  // exchange slots, then the pairs' counts
}

// The fused kernel sequence over sp.T tokens (a whole number of chunks).  The state moves from
// (Wb[cur], Sb[cur]) to (Wb[1 - cur], Sb[1 - cur]) in each launch segment and `cur` flips with it;
// Wb[0] == Wb[1] (and Sb likewise) updates the state in place, which the kernel allows: every
// state element it writes was read earlier by the same lane, or before a workgroup barrier (or a
// wait of the workgroup pair) that precedes the write.  T2: per memory 2 x 64 x 128 floats of
// scratch; xs: the two-workgroup form's workspace (fused_split_workspace_floats), or null for one
// workgroup per memory; flag: the non-finite flag.
static atlasmem_status launch_fused_bufs(const Dims& d, const void* K, const void* Q, const void* V,
                                         const float* theta, const float* eta, const float* alpha, const Span& sp,
                                         void* Y, float* const Wb[2], float* const Sb[2], int& cur, float* T2,
                                         float* xs, int* flag, hipStream_t st) {
  const bool pl = d.prec == 0;  // plain bf16 products
  const void* kern = d.residual ? (pl ? (const void*)fz::fused_ns_kernel<true, true, false> : (const void*)fz::fused_ns_kernel<true, false, false>)
                                : (pl ? (const void*)fz::fused_ns_kernel<false, true, false> : (const void*)fz::fused_ns_kernel<false, false, false>);
  if (hipFuncSetAttribute(kern, hipFuncAttributeMaxDynamicSharedMemorySize, fz::LDS_BYTES) != hipSuccess)
    return ATLASMEM_E_DEVICE;
  // the two-workgroup form for calls of at least four chunks (measured: a call of one or two chunks
  // takes longer in wall time with the cooperative launch than on one workgroup per memory); the
  // gated memory has only that form
  bool split = xs != nullptr && d.M <= fz::kSplitMaxMem && (sp.T / d.C >= 4 || d.gated);
  const void* kern2 = d.gated ? (const void*)fz::fused_ns_kernel<false, false, true, true>
                    : d.residual ? (pl ? (const void*)fz::fused_ns_kernel<true, true, true> : (const void*)fz::fused_ns_kernel<true, false, true>)
                                 : (pl ? (const void*)fz::fused_ns_kernel<false, true, true> : (const void*)fz::fused_ns_kernel<false, false, true>);
  if (split && hipFuncSetAttribute(kern2, hipFuncAttributeMaxDynamicSharedMemorySize, fz::LDS_BYTES) != hipSuccess)
    return ATLASMEM_E_DEVICE;
  if (d.gated) {
    // the gated memory has no one-workgroup form: without room for every pair at once the caller
    // takes the general path (decided before anything runs)
    int dev = 0, per_cu = 0, ncu = 0;
    if (!split || hipGetDevice(&dev) != hipSuccess ||
        hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kern2, fz::NT / 2, fz::LDS_BYTES) != hipSuccess ||
        hipDeviceGetAttribute(&ncu, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
        (int64_t)per_cu * ncu < 16 * ((d.M + 7) / 8)) {
      (void)hipGetLastError();
      return ATLASMEM_E_UNSUPPORTED;
    }
  }
  int* sync = split ? (int*)(xs + (int64_t)d.M * (d.gated ? 3 : 2) * fz::P2) : nullptr;
  // one launch per segment of at most 2^22 tokens, so that per-memory byte offsets fit 32 bits
  const int64_t nchunks = sp.T / d.C;
  const int64_t seg = ((int64_t)1 << 22) / d.C;
  const int ysz = d.out_bf16 ? 2 : 4;
  for (int64_t c0 = 0; c0 < nchunks; c0 += seg) {
    const int64_t nc = nchunks - c0 < seg ? nchunks - c0 : seg;
    const int64_t t0 = c0 * d.C;
    fz::Args a;
    a.K = (const uint16_t*)K + t0 * fz::D;
    a.Q = (const uint16_t*)Q + t0 * fz::D;
    a.V = (const uint16_t*)V + t0 * fz::D;
    a.theta = theta + c0;
    a.eta = eta + c0;
    a.alpha = alpha + c0;
    a.ldT = sp.ld;
    a.ld_gate = sp.ldg;
    a.C = d.C;
    a.nchunks = (int)nc;
    a.Win = Wb[cur];
    a.Sin = Sb[cur];
    a.Wout = Wb[1 - cur];
    a.Sout = Sb[1 - cur];
    a.T2 = T2;
    a.Y = Y ? (void*)((char*)Y + t0 * fz::D * ysz) : nullptr;
    a.out_bf16 = d.out_bf16;
    a.ns_steps = d.ns_steps;
    a.ns_a = d.ns_a;
    a.ns_b = d.ns_b;
    a.ns_c = d.ns_c;
    a.ns_eps = d.ns_eps;
    a.flag = flag;
    a.xs = split ? xs : nullptr;
    a.sync = sync;
    a.M = d.M;
    if (split) {
      // the pairs' counts start at zero in every launch (a kernel, not a memset)
      hipLaunchKernelGGL(fz::zero_ints_kernel, dim3((d.M * 32 + 255) / 256), dim3(256), 0, st, sync, d.M * 32);
      AM_LAUNCH_CHECK();
      void* args[] = {&a};
      const unsigned nblk = 16u * (unsigned)((d.M + 7) / 8);
      if (hipLaunchCooperativeKernel(kern2, dim3(nblk), dim3(fz::NT / 2), args, fz::LDS_BYTES, st) != hipSuccess) {
        // not every pair can be resident at once on this device: one workgroup per memory instead
        (void)hipGetLastError();
        // the gated memory has no one-workgroup form: the caller takes the general path (only the
        // pairs' counts were cleared, and a refusal repeats for every segment, so it is the first)
        if (d.gated) return ATLASMEM_E_UNSUPPORTED;
        split = false;
        a.xs = nullptr;
        a.sync = nullptr;
      } else {
        cur = 1 - cur;
        continue;
      }
    }
    if (d.residual) {
      if (pl) hipLaunchKernelGGL((fz::fused_ns_kernel<true, true, false>), dim3(d.M), dim3(fz::NT), fz::LDS_BYTES, st, a);
      else hipLaunchKernelGGL((fz::fused_ns_kernel<true, false, false>), dim3(d.M), dim3(fz::NT), fz::LDS_BYTES, st, a);
    } else {
      if (pl) hipLaunchKernelGGL((fz::fused_ns_kernel<false, true, false>), dim3(d.M), dim3(fz::NT), fz::LDS_BYTES, st, a);
      else hipLaunchKernelGGL((fz::fused_ns_kernel<false, false, false>), dim3(d.M), dim3(fz::NT), fz::LDS_BYTES, st, a);
    }
    AM_LAUNCH_CHECK();
    cur = 1 - cur;
  }
  if (d.residual && Y && sp.T > 0) {
    const int64_t n = sp.T * fz::D;  // a whole number of 8-element groups (D = 64)
    hipLaunchKernelGGL(fz::residual_output_kernel, dim3((unsigned)((n / 8 + 255) / 256), d.M), dim3(256), 0, st,
                       (const uint16_t*)Q, (float*)Y, sp.ld * fz::D, n);
    AM_LAUNCH_CHECK();
  }
  return ATLASMEM_OK;
}

bool fused_pt_supported(const Dims& d) {
  return d.kind == ATLASMEM_MLP2_SILU && !d.gated && !d.ptr && !d.conv && !d.no_fused &&
         d.gate_mode == ATLASMEM_PER_TOKEN && d.ns_steps == 0 && d.dk == fz::D && d.din == fz::D && d.dv == fz::D &&
         d.dh == fz::HD && d.c == 1 && d.C == fz::GROWS && d.in_bf16 && d.split && !(d.residual && d.out_bf16);
}

// Chunks [kb0, kb0 + nb) of a call (tokens from kb0 * C, token stride ld), with the gate scan's
// coefficients of these chunks at h->cW, h->cS, h->scal (chunk kb of the block at column kb).
atlasmem_status launch_fused_pt(Handle* h, const Dims& d, const void* K, const void* Q, const void* V, int64_t kb0,
                                int nb, int64_t ld, void* Y, hipStream_t st) {
  const void* kern = d.residual ? (const void*)fz::fused_pt_kernel<true> : (const void*)fz::fused_pt_kernel<false>;
  if (hipFuncSetAttribute(kern, hipFuncAttributeMaxDynamicSharedMemorySize, fz::PT_LDS_BYTES) != hipSuccess)
    return ATLASMEM_E_DEVICE;
  const int64_t t0 = kb0 * d.C;
  const int ysz = d.out_bf16 ? 2 : 4;
  fz::PtArgs pa;
  fz::Args& a = pa.a;
  a.K = (const uint16_t*)K + t0 * fz::D;
  a.Q = (const uint16_t*)Q + t0 * fz::D;
  a.V = (const uint16_t*)V + t0 * fz::D;
  a.theta = a.eta = a.alpha = nullptr;
  a.ldT = ld;
  a.ld_gate = 0;
  a.C = d.C;
  a.nchunks = nb;
  a.Win = h->W[h->cur];
  a.Sin = h->S[h->cur];
  a.Wout = h->W[1 - h->cur];
  a.Sout = h->S[1 - h->cur];
  a.T2 = h->G;
  a.Y = Y ? (void*)((char*)Y + t0 * fz::D * ysz) : nullptr;
  a.out_bf16 = d.out_bf16;
  a.ns_steps = 0;
  a.ns_a = a.ns_b = a.ns_c = a.ns_eps = 0.0f;
  a.flag = h->flag;
  pa.cW = h->cW;
  pa.cS = h->cS;
  pa.scal = h->scal;
  pa.ld_c = (int64_t)h->ncb * d.C;
  pa.ld_s = (int64_t)h->ncb * 3;
  if (d.residual)
    hipLaunchKernelGGL(fz::fused_pt_kernel<true>, dim3(d.M), dim3(fz::NT), fz::PT_LDS_BYTES, st, pa);
  else
    hipLaunchKernelGGL(fz::fused_pt_kernel<false>, dim3(d.M), dim3(fz::NT), fz::PT_LDS_BYTES, st, pa);
  AM_LAUNCH_CHECK();
  h->cur = 1 - h->cur;
  if (d.residual && Y) {
    const int64_t n = (int64_t)nb * d.C * fz::D;
    hipLaunchKernelGGL(fz::residual_output_kernel, dim3((unsigned)((n / 8 + 255) / 256), d.M), dim3(256), 0, st,
                       (const uint16_t*)Q + t0 * fz::D, (float*)Y + t0 * fz::D, ld * fz::D, n);
    AM_LAUNCH_CHECK();
  }
  return ATLASMEM_OK;
}

atlasmem_status launch_fused(Handle* h, const Dims& d, const void* K, const void* Q, const void* V,
                             const float* theta, const float* eta, const float* alpha, const Span& sp, void* Y,
                             hipStream_t st) {
  return launch_fused_bufs(d, K, Q, V, theta, eta, alpha, sp, Y, h->W, h->S, h->cur, h->G, h->fxs, h->flag, st);
}

// ---------------------------------------------------------------------------- no allocation
//
// For callers that cannot allocate: the same kernel with the caller's state updated in place and
// its per-memory scratch (the W2 half of the state between the chunks of a launch) in this static
// device array, 64 KB per memory for at most kStaticMaxMem memories (8 MB) plus a flag word.  Each
// device holds its own copy until the process ends; its address is looked up once per device.

namespace fz {
constexpr int kStaticMaxMem = ATLASMEM_STATIC_MAX_MEMORIES;
constexpr int64_t kStaticFloats = (int64_t)kStaticMaxMem * 2 * P2 + 64;
constexpr int kMaxDevices = 64;

__global__ void zero_flag_kernel(int* f) { f[0] = 0; }
}  // namespace fz

static __device__ __align__(256) float scratch[fz::kStaticFloats];

namespace {
std::mutex g_scratch_mu;
float* g_scratch[fz::kMaxDevices];       // device address of `scratch`, per device
bool g_scratch_gfx950[fz::kMaxDevices];  // the device is a gfx950
}  // namespace

// The device address of this device's copy of `scratch` (set up on the first call on a device).
static atlasmem_status static_scratch(int dev, float** out) {
  if (dev < 0 || dev >= fz::kMaxDevices) return ATLASMEM_E_DEVICE;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch[dev]) {
    hipDeviceProp_t prop;
    if (hipGetDeviceProperties(&prop, dev) != hipSuccess) return ATLASMEM_E_DEVICE;
    g_scratch_gfx950[dev] = strncmp(prop.gcnArchName, "gfx950", 6) == 0;
    if (!g_scratch_gfx950[dev]) return ATLASMEM_E_DEVICE;
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return ATLASMEM_E_DEVICE;
    g_scratch[dev] = (float*)p;
  }
  *out = g_scratch[dev];
  return ATLASMEM_OK;
}

int fused_static_max_memories() { return fz::kStaticMaxMem; }

atlasmem_status launch_fused_static(const Dims& d, const void* K, const void* Q, const void* V, const float* theta,
                                    const float* eta, const float* alpha, const Span& sp, void* Y, float* W, float* S,
                                    int* nonfinite, hipStream_t st) {
  if (d.M > fz::kStaticMaxMem) return ATLASMEM_E_SHAPE;
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess) return ATLASMEM_E_DEVICE;
  float* base = nullptr;
  const atlasmem_status s = static_scratch(dev, &base);
  if (s != ATLASMEM_OK) return s;
  // the flag: the caller's word (cleared by a small kernel, so the call also records into a
  // captured graph), or the scratch's last word, which nothing reads
  int* flag = nonfinite ? (int*)nonfinite : (int*)(base + fz::kStaticFloats - 1);
  if (nonfinite) {
    hipLaunchKernelGGL(fz::zero_flag_kernel, dim3(1), dim3(1), 0, st, flag);
    AM_LAUNCH_CHECK();
  }
  float* Wb[2] = {W, W};
  float* Sb[2] = {S, S};
  int cur = 0;
  return launch_fused_bufs(d, K, Q, V, theta, eta, alpha, sp, Y, Wb, Sb, cur, base, nullptr, flag, st);
}

}  // namespace am
