"""Seeded synthetic inputs for the neural-memory update workloads.

This module only draws and prepares inputs (random draws, L2 normalisation of
the drawn vectors, rounding to bf16).  It holds none of the method's
arithmetic, so both the fp64 oracle and the HIP path can be fed from it
without sharing any computation.

Five workloads are defined (sizes and distributions of the neural-memory
configurations used for parity and measurement):

  0  linear memory 16x16, fp32, B=1 H=1 T=256, chunk 1 (exact per-token
     recurrence); keys/queries N(0,1) then L2-normalised, values N(0,1);
     theta~U(.01,.1), eta~U(.8,.99), alpha~U(0,.05) per token; W0 = S0 = 0.
  1  2-layer SiLU MLP 64->128->64, B=2 H=4 T=4096 chunk 64, bf16 inputs,
     keys L2-normalised, gates as workload 0.
  2  wide single-head MLP 384->768->384, B=2 H=1 T=1024 chunk 64, bf16 N(0,1),
     theta~U(.001,.05), eta~U(.85,.99), alpha~U(0,.02).
  3  Omega window 4 + degree-2 polynomial features (32 -> 561), MLP
     561->128->64, B=4 H=8 T=8192 chunk 64, gamma~U(0,1), gates as workload 0,
     keys/queries L2-normalised before the feature map.
  4  Muon-style: MLP 64->128->64, B=8 H=16 T=32768 chunk 128, per-chunk gates
     with workload 2's distributions, 5 Newton-Schulz steps, keys L2-normalised.

Variant "stabilised" changes only the generator (the literal workloads 1-3
overflow in fp64, so a bounded variant is also provided):
workload 1 also L2-normalises V; workload 2 L2-normalises K, Q and V;
workload 3 L2-normalises K, Q, V and scales theta by 0.1.

Random stream: numpy default_rng(SeedSequence([workload, b, h])), drawn in the
order K, Q, V (N(0,1) fp64), theta, eta, alpha (uniform), gamma (U(0,1), only
for an Omega window > 1), then W1 (or W), then W2, then (gated memory) W3
(N(0, 1/fan_in)).
Preparation: cast to fp32, L2-normalise in fp32 where the workload says so,
round to bf16 once (round-to-nearest-even) for bf16 workloads.
"""

from __future__ import annotations

import dataclasses
import math

import numpy as np

LINEAR = 0
MLP2_SILU = 1
MLP2_SILU_RESIDUAL = 2
MLP2_GATED = 3
PER_TOKEN = 0
PER_CHUNK = 1
F32 = 0
BF16 = 1

NS_COEFFS = (3.4445, -4.7750, 2.0315)
NS_EPS = 1e-7


@dataclasses.dataclass(frozen=True)
class Spec:
    """Shape and distribution of one workload (per memory = per (b, h))."""

    name: str
    kind: int
    batch: int
    heads: int
    T: int
    d_key: int
    d_value: int
    d_hidden: int
    poly_degree: int
    chunk: int
    omega_window: int
    gate_mode: int
    ns_steps: int
    input_dtype: int
    theta_range: tuple
    eta_range: tuple
    alpha_range: tuple
    norm_k: bool
    norm_q: bool
    norm_v: bool
    theta_scale: float = 1.0
    zero_init: bool = False
    per_token_retrieve: bool = False   # retrieval after each token's update (per-token gates)

    @property
    def n_mem(self) -> int:
        return self.batch * self.heads

    @property
    def d_in(self) -> int:
        """Width of the memory's input after the feature map: C(d+p, p) for p = 2."""
        if self.poly_degree == 1:
            return self.d_key
        return math.comb(self.d_key + self.poly_degree, self.poly_degree)

    @property
    def param_count(self) -> int:
        if self.kind == LINEAR:
            return self.d_value * self.d_in
        if self.kind == MLP2_GATED:
            return 2 * self.d_hidden * self.d_in + self.d_value * self.d_hidden
        return self.d_hidden * self.d_in + self.d_value * self.d_hidden


_GATES_0 = dict(theta_range=(0.01, 0.1), eta_range=(0.8, 0.99), alpha_range=(0.0, 0.05))
_GATES_2 = dict(theta_range=(0.001, 0.05), eta_range=(0.85, 0.99), alpha_range=(0.0, 0.02))

SPECS = [
    Spec("linear16_T256_C1", LINEAR, 1, 1, 256, 16, 16, 0, 1, 1, 1, PER_TOKEN, 0, F32,
         norm_k=True, norm_q=True, norm_v=False, zero_init=True, **_GATES_0),
    Spec("mlp64x128_B2H4_T4096_C64", MLP2_SILU, 2, 4, 4096, 64, 64, 128, 1, 64, 1, PER_TOKEN, 0, BF16,
         norm_k=True, norm_q=False, norm_v=False, **_GATES_0),
    Spec("mlp384x768_B2H1_T1024_C64", MLP2_SILU, 2, 1, 1024, 384, 384, 768, 1, 64, 1, PER_TOKEN, 0, BF16,
         norm_k=False, norm_q=False, norm_v=False, **_GATES_2),
    Spec("omega4_poly2_mlp561x128x64_B4H8_T8192_C64", MLP2_SILU, 4, 8, 8192, 32, 64, 128, 2, 64, 4, PER_TOKEN, 0,
         BF16, norm_k=True, norm_q=True, norm_v=False, **_GATES_0),
    Spec("ns5_mlp64x128_B8H16_T32768_C128", MLP2_SILU, 8, 16, 32768, 64, 64, 128, 1, 128, 1, PER_CHUNK, 5, BF16,
         norm_k=True, norm_q=False, norm_v=False, **_GATES_2),
]

VARIANTS = ("literal", "stabilised")


def spec(index: int, variant: str = "literal", **overrides) -> Spec:
    """Workload `index` in `variant`, with optional field overrides (e.g. T=256)."""
    if variant not in VARIANTS:
        raise ValueError(f"unknown variant {variant!r}")
    s = SPECS[index]
    if variant == "stabilised":
        if index == 1:
            s = dataclasses.replace(s, norm_v=True)
        elif index == 2:
            s = dataclasses.replace(s, norm_k=True, norm_q=True, norm_v=True)
        elif index == 3:
            s = dataclasses.replace(s, norm_v=True, theta_scale=0.1)
    return dataclasses.replace(s, **overrides) if overrides else s


# ----------------------------------------------------------------------------- bf16 rounding

def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round fp32 to bf16 (round to nearest, ties to even); returns uint16 bit patterns."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    rounding = ((u >> 16) & 1) + np.uint32(0x7FFF)
    return ((u + rounding) >> 16).astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def _l2n_f32(x32: np.ndarray) -> np.ndarray:
    n = np.sqrt(np.sum(x32 * x32, axis=-1, keepdims=True, dtype=np.float32), dtype=np.float32)
    return (x32 / np.maximum(n, np.float32(1e-30))).astype(np.float32)


# ----------------------------------------------------------------------------- inputs

@dataclasses.dataclass
class Inputs:
    """Host arrays for all memories, in the device layouts.

    K, Q: [M, T, d_key]; V: [M, T, d_value] -- uint16 bf16 bits for bf16 workloads, float32 otherwise.
    theta, eta, alpha: [M, T] (per token) or [M, ceil(T / chunk)] (per chunk), float32.
    gamma: [M, T] float32 or None (window 1).
    W0: [M, P] float32 (W1 row-major then W2 row-major; linear: W), S0: zeros [M, P].
    """

    spec: Spec
    index: int
    variant: str
    K: np.ndarray
    Q: np.ndarray
    V: np.ndarray
    theta: np.ndarray
    eta: np.ndarray
    alpha: np.ndarray
    gamma: np.ndarray | None
    W0: np.ndarray
    S0: np.ndarray

    def values(self, name: str, mems=None) -> np.ndarray:
        """Exact float64 values of an input array (bf16 bits decoded), optionally for a subset of memories."""
        a = getattr(self, name)
        if mems is not None:
            a = a[np.asarray(mems)]
        if a.dtype == np.uint16:
            return bf16_bits_to_f32(a).astype(np.float64)
        return a.astype(np.float64)

    def split_params(self, flat: np.ndarray):
        """Split one memory's flat parameter vector into its matrices (W), (W1, W2) or (W1, W3, W2)."""
        s = self.spec
        flat = np.asarray(flat, dtype=np.float64)
        if s.kind == LINEAR:
            return [flat.reshape(s.d_value, s.d_in)]
        n1 = s.d_hidden * s.d_in
        if s.kind == MLP2_GATED:
            return [flat[:n1].reshape(s.d_hidden, s.d_in), flat[n1:2 * n1].reshape(s.d_hidden, s.d_in),
                    flat[2 * n1:].reshape(s.d_value, s.d_hidden)]
        return [flat[:n1].reshape(s.d_hidden, s.d_in), flat[n1:].reshape(s.d_value, s.d_hidden)]


def _draw_memory(s: Spec, index: int, b: int, h: int):
    rng = np.random.default_rng(np.random.SeedSequence([index, b, h]))
    T = s.T
    k = rng.standard_normal((T, s.d_key))
    q = rng.standard_normal((T, s.d_key))
    v = rng.standard_normal((T, s.d_value))
    n_g = T if s.gate_mode == PER_TOKEN else -(-T // s.chunk)
    theta = rng.uniform(*s.theta_range, size=n_g)
    eta = rng.uniform(*s.eta_range, size=n_g)
    alpha = rng.uniform(*s.alpha_range, size=n_g)
    gamma = rng.uniform(0.0, 1.0, size=T) if s.omega_window > 1 else None
    if s.kind == LINEAR:
        w = rng.normal(0.0, 1.0 / math.sqrt(s.d_in), size=(s.d_value, s.d_in))
        params = [w]
    else:
        w1 = rng.normal(0.0, 1.0 / math.sqrt(s.d_in), size=(s.d_hidden, s.d_in))
        w2 = rng.normal(0.0, 1.0 / math.sqrt(s.d_hidden), size=(s.d_value, s.d_hidden))
        params = [w1, w2]
        if s.kind == MLP2_GATED:  # drawn last, so the other draws match the plain memory's
            w3 = rng.normal(0.0, 1.0 / math.sqrt(s.d_in), size=(s.d_hidden, s.d_in))
            params = [w1, w3, w2]
    return k, q, v, theta, eta, alpha, gamma, params


def _prepare(x: np.ndarray, normalise: bool, dtype: int) -> np.ndarray:
    x32 = x.astype(np.float32)
    if normalise:
        x32 = _l2n_f32(x32)
    if dtype == BF16:
        return f32_to_bf16_bits(x32)
    return x32


def make_inputs(index: int, variant: str = "literal", **overrides) -> Inputs:
    """All memories' inputs for workload `index` (optionally with overridden sizes)."""
    s = spec(index, variant, **overrides)
    M, T = s.n_mem, s.T
    in_dt = np.uint16 if s.input_dtype == BF16 else np.float32
    K = np.empty((M, T, s.d_key), in_dt)
    Q = np.empty((M, T, s.d_key), in_dt)
    V = np.empty((M, T, s.d_value), in_dt)
    n_g = T if s.gate_mode == PER_TOKEN else -(-T // s.chunk)
    theta = np.empty((M, n_g), np.float32)
    eta = np.empty((M, n_g), np.float32)
    alpha = np.empty((M, n_g), np.float32)
    gamma = np.empty((M, T), np.float32) if s.omega_window > 1 else None
    W0 = np.zeros((M, s.param_count), np.float32)
    for b in range(s.batch):
        for h in range(s.heads):
            m = b * s.heads + h
            k, q, v, th, et, al, ga, params = _draw_memory(s, index, b, h)
            K[m] = _prepare(k, s.norm_k, s.input_dtype)
            Q[m] = _prepare(q, s.norm_q, s.input_dtype)
            V[m] = _prepare(v, s.norm_v, s.input_dtype)
            theta[m] = (th * s.theta_scale).astype(np.float32)
            eta[m] = et.astype(np.float32)
            alpha[m] = al.astype(np.float32)
            if gamma is not None:
                gamma[m] = ga.astype(np.float32)
            if not s.zero_init:
                W0[m] = np.concatenate([p.astype(np.float32).ravel() for p in params])
    return Inputs(s, index, variant, K, Q, V, theta, eta, alpha, gamma, W0, np.zeros_like(W0))


# ----------------------------------------------------------------------------- prologue inputs

GATE_SCALES = (0.1, 0.9, 0.01, 1.0)  # theta, eta, alpha maxima and gamma's


@dataclasses.dataclass
class PrologueInputs:
    """Host arrays for the input prologue (short convolution and gates).

    X: [B*H, T, d] raw key / query / value rows (bf16 bits or fp32), hist: [B*H, 3, d] rows
    before token 0 (same dtype); taps: [H, d, 4], bias: [H, d] fp32;
    U: [B, T, d_model] bf16 bits; Wg: [n_gates, H, d_model], bg: [n_gates, H], scale: [n_gates]."""

    X: np.ndarray
    hist: np.ndarray
    taps: np.ndarray
    bias: np.ndarray
    U: np.ndarray
    Wg: np.ndarray
    bg: np.ndarray
    scale: np.ndarray


def make_prologue_inputs(seed: int, B: int, H: int, T: int, d: int, d_model: int, n_gates: int = 3,
                         in_dtype: int = BF16) -> PrologueInputs:
    """Seeded draws: X, hist, U ~ N(0, 1); taps ~ N(0, 0.5^2); bias ~ N(0, 0.1^2);
    Wg ~ N(0, 1/d_model); bg ~ N(0, 1); scale = the first n_gates of GATE_SCALES.
    Rows are rounded to bf16 once where bf16 is asked for (U always)."""
    rng = np.random.default_rng(np.random.SeedSequence([1000 + seed, B, H, T, d, d_model]))
    M = B * H
    X = rng.standard_normal((M, T, d)).astype(np.float32)
    hist = rng.standard_normal((M, 3, d)).astype(np.float32)
    taps = (0.5 * rng.standard_normal((H, d, 4))).astype(np.float32)
    bias = (0.1 * rng.standard_normal((H, d))).astype(np.float32)
    U = rng.standard_normal((B, T, d_model)).astype(np.float32)
    Wg = (rng.standard_normal((n_gates, H, d_model)) / math.sqrt(d_model)).astype(np.float32)
    bg = rng.standard_normal((n_gates, H)).astype(np.float32)
    scale = np.array(GATE_SCALES[:n_gates], dtype=np.float32)
    if in_dtype == BF16:
        X = f32_to_bf16_bits(X)
        hist = f32_to_bf16_bits(hist)
    return PrologueInputs(X=X, hist=hist, taps=taps, bias=bias, U=f32_to_bf16_bits(U), Wg=Wg, bg=bg, scale=scale)



def make_conv_params(seed: int, heads: int, d_key: int, d_value: int):
    """Seeded short-convolution parameters for keys, queries and values: taps ~ N(0, 0.5^2)
    [heads, d, 4] and biases ~ N(0, 0.1^2) [heads, d], fp32, drawn in the order taps_k, taps_q,
    taps_v, bias_k, bias_q, bias_v."""
    rng = np.random.default_rng(np.random.SeedSequence([2000 + seed, heads, d_key, d_value]))
    tk = (0.5 * rng.standard_normal((heads, d_key, 4))).astype(np.float32)
    tq = (0.5 * rng.standard_normal((heads, d_key, 4))).astype(np.float32)
    tv = (0.5 * rng.standard_normal((heads, d_value, 4))).astype(np.float32)
    bk = (0.1 * rng.standard_normal((heads, d_key))).astype(np.float32)
    bq = (0.1 * rng.standard_normal((heads, d_key))).astype(np.float32)
    bv = (0.1 * rng.standard_normal((heads, d_value))).astype(np.float32)
    return (tk, tq, tv), (bk, bq, bv)
