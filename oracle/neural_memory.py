"""Plain, slow, fp64 CPU oracle of the neural-memory test-time update and retrieval.

TEST INFRASTRUCTURE.  Only the test suite, the smoke check and the benchmark's
CPU-baseline leg import this module.  The library never calls it, shares no
code with it, and must fail loudly rather than fall back to it.

What it computes, and where the pages define it
-----------------------------------------------
* Memory M_W: a linear map (M(x) = W x) or a 2-layer SiLU MLP
  (M(x) = W2 silu(W1 x)).  Deep memory: "Titans: Learning to Memorize at Test
  Time" (titans-pytorch-mlx README), Key Innovations item 3; titans-torch 0.1.2
  (PyPI), API Reference, NeuralLongTermMemory (num_layers = 2).  The residual
  2-layer memory M(x) = x + W2 silu(W1 x) (d_in == d_value) is ATLAS's default
  memory ("ATLAS ... | Summary", section 5.1; the pages give no formula, the
  residual adds the memory's input to its output).  ATLAS++ uses a gated MLP
  (same section); reading taken: M(x) = W2 (silu(W1 x) * (W3 x)), a SiLU branch
  gating a linear one elementwise, weights [W1, W3, W2].
* Per-token retrieval (optional, per-token gates): y_t = M_{W_t}(phi(q_t)) with
  W_t the state right after token t's update, the Atlas configuration's
  retrieve (Atlas-Torch README, "Known deviations from the paper's MAC": the
  post-update per-token state; Bug Fixes table, "no-omega ablation" row:
  per-token retrieve on the per-token path).
* Associative loss l(M; x_t) = ||M(k_t) - v_t||^2 (sum of squares, no 1/d):
  titans-pytorch-mlx README, Core Equations, Eq. 12.  For a linear memory its
  gradient is (prediction error) x (key), the delta rule: Atlas-Torch README,
  "How the memory works".
* Momentum S_t = eta_t S_{t-1} - theta_t grad, forgetting
  W_t = (1 - alpha_t) W_{t-1} + S_t: titans-pytorch-mlx README, Eq. 13 and
  Eq. 14; titans-torch 0.1.2, "Inner-loop update rule".
* Chunk-wise form: every gradient inside a chunk is taken at the memory state
  of the preceding chunk boundary, the recurrence runs across chunks:
  "ATLAS ... | Summary", section 3.3 "Parallelizing Omega Rule"; Atlas-Torch
  README, Bug Fixes table ("share the segment-start base weights").
  Retrieval uses the same chunk-start weights (y_t = M*_{t-1}(q_t) with no
  update: titans-pytorch-mlx README, MAC Eq. 21; titans-torch 0.1.2 forward()).
* Omega rule: the loss at step t sums gamma_i-weighted losses over the last c
  associations; a window of 1 is the single-token rule: "ATLAS ... | Summary",
  section 3.2; Atlas-Torch README, Atlas Extensions table (Omega Rule).
* Polynomial features: exact monomials in combinations_with_replacement order
  with coefficients 1/deg!: Atlas-Torch README, Atlas Extensions table
  (Polynomial Features); capacity O(d_k^p): "ATLAS ... | Summary", section 3.1.
* Newton-Schulz, 5 quintic iterations, on the per-chunk surprise:
  Atlas-Torch README, Atlas Extensions table (Muon / Newton-Schulz);
  "ATLAS ... | Summary", section 5.  Per-chunk path: one summed gradient per
  chunk, eta and theta outside the orthogonalisation (Atlas-Torch README, Bug
  Fixes table, "no-omega ablation" row).

Readings where the pages leave a step open (each is stated in the design notes):
the Omega window crosses chunk boundaries and is clipped only at the start of
the sequence; the halo tokens' gradients are re-taken at the current
chunk-start weights; gamma_i belongs to token i; with a window of 1 the weight
is 1 (gamma unused); the constant monomial is included in the feature map;
NS normalises by ||G||_F + eps, works on the wide orientation and handles each
weight matrix separately.

Everything here is float64; bf16 and fp32 inputs are exact in float64.
"""

from __future__ import annotations

import dataclasses
import math
from itertools import combinations_with_replacement

import numpy as np
from scipy.special import expit

LINEAR = 0
MLP2_SILU = 1
MLP2_SILU_RESIDUAL = 2      # x + W2 silu(W1 x): the default memory of ATLAS (d_in == d_value)
MLP2_GATED = 3              # W2 (silu(W1 x) * (W3 x)): the gated memory of ATLAS++
PER_TOKEN = 0
PER_CHUNK = 1


@dataclasses.dataclass(frozen=True)
class MemoryConfig:
    kind: int                 # LINEAR, MLP2_SILU, MLP2_SILU_RESIDUAL or MLP2_GATED
    d_key: int
    d_value: int
    d_hidden: int = 0
    poly_degree: int = 1      # 1: identity feature map
    chunk: int = 1
    omega_window: int = 1
    gate_mode: int = PER_TOKEN
    ns_steps: int = 0
    ns_coeffs: tuple = (3.4445, -4.7750, 2.0315)
    ns_eps: float = 1e-7
    per_token_retrieve: bool = False   # y_t read after token t's update (per-token gates only)


# ----------------------------------------------------------------------------- feature map

def poly_features(x: np.ndarray, degree: int) -> np.ndarray:
    """phi(x): every monomial of degree 0..p, coefficient 1/deg!, degree-major,
    combinations_with_replacement order inside a degree.  Identity for p = 1.
    (Atlas-Torch README, Atlas Extensions table: Polynomial Features.)"""
    x = np.asarray(x, dtype=np.float64)
    if degree == 1:
        return x.copy()
    if degree < 1:
        raise ValueError("poly_degree must be >= 1")
    n, d = x.shape
    cols = []
    for deg in range(degree + 1):
        coeff = 1.0 / math.factorial(deg)
        for combo in combinations_with_replacement(range(d), deg):
            col = np.full(n, coeff)
            for i in combo:
                col = col * x[:, i]
            cols.append(col)
    return np.stack(cols, axis=1)


# ----------------------------------------------------------------------------- memory and its gradient

def silu(z):
    return z * expit(z)


def silu_prime(z):
    s = expit(z)
    return s * (1.0 + z * (1.0 - s))


def memory_apply(params, x, residual: bool = False):
    """M_W(x) for one input vector; with `residual` the 2-layer memory adds its input,
    M(x) = x + W2 silu(W1 x) ("ATLAS ... | Summary", section 5.1: the default memory is a
    two-layer residual MLP).  Three matrices [W1, W3, W2] are the gated memory
    W2 (silu(W1 x) * (W3 x)) (same section: ATLAS++)."""
    if len(params) == 1:
        return params[0] @ x
    if len(params) == 3:
        w1, w3, w2 = params
        return w2 @ (silu(w1 @ x) * (w3 @ x))
    w1, w2 = params
    y = w2 @ silu(w1 @ x)
    return x + y if residual else y


def loss(params, x, v, residual: bool = False) -> float:
    """l = ||M_W(x) - v||^2 (titans-pytorch-mlx README, Eq. 12)."""
    r = memory_apply(params, x, residual) - v
    return float(r @ r)


def loss_grad(params, x, v, residual: bool = False):
    """Gradient of ||M_W(x) - v||^2 with respect to each weight matrix, by the chain rule.  The
    residual input x does not depend on the weights: it only shifts the prediction error."""
    if len(params) == 1:
        w = params[0]
        return [np.outer(2.0 * (w @ x - v), x)]
    if len(params) == 3:
        w1, w3, w2 = params
        z1, z3 = w1 @ x, w3 @ x
        a = silu(z1)
        hg = a * z3                                  # gated hidden activation
        e = 2.0 * (w2 @ hg - v)                      # dl/dy
        back = w2.T @ e                              # dl/dhg
        return [np.outer(back * z3 * silu_prime(z1), x), np.outer(back * a, x), np.outer(e, hg)]
    w1, w2 = params
    z = w1 @ x
    h = silu(z)
    y = w2 @ h
    if residual:
        y = x + y
    e = 2.0 * (y - v)                            # dl/dy
    g2 = np.outer(e, h)                          # dl/dW2
    g1 = np.outer((w2.T @ e) * silu_prime(z), x)  # dl/dW1
    return [g1, g2]


# ----------------------------------------------------------------------------- Newton-Schulz

def newton_schulz(g: np.ndarray, steps: int = 5, coeffs=(3.4445, -4.7750, 2.0315), eps: float = 1e-7):
    """Quintic Newton-Schulz orthogonalisation of one matrix: X0 = G / (||G||_F + eps),
    worked in the orientation with rows <= cols, `steps` times X <- aX + (bA + cA^2)X with
    A = X X^T, then returned in G's orientation.  In exact arithmetic each step maps every
    singular value s to a s + b s^3 + c s^5 and keeps the singular vectors, whatever the
    orientation; the wide orientation only makes A the smaller Gram matrix."""
    a, b, c = coeffs
    x = np.asarray(g, dtype=np.float64) / (np.linalg.norm(g) + eps)
    transposed = x.shape[0] > x.shape[1]
    if transposed:
        x = x.T
    for _ in range(steps):
        A = x @ x.T
        B = b * A + c * (A @ A)
        x = a * x + B @ x
    return x.T if transposed else x


# ----------------------------------------------------------------------------- the recurrence (one memory)

@dataclasses.dataclass
class MemoryResult:
    Y: np.ndarray             # [T, d_value] retrieved outputs
    params: list              # final weight matrices
    momenta: list             # final momentum matrices
    history: list             # last (window - 1) tokens as (phi(k), v, gamma), for the next call
    boundary_states: list     # (params, momenta) at every chunk boundary, if requested
    max_abs_w: list           # max |W| after every chunk (health report)


def run_memory(cfg: MemoryConfig, params, momenta, K, Q, V, theta, eta, alpha, gamma=None,
               history=None, keep_boundaries: bool = False) -> MemoryResult:
    """The literal recurrence for one memory over T tokens, in chunks of cfg.chunk tokens; when T
    is not a multiple of the chunk, the last chunk holds the remaining T mod chunk tokens (a
    sequence's final partial chunk: its gradients are taken at its own start weights, like any
    chunk's).

    params / momenta: weight and momentum matrices at the start of the call.
    K, Q: [T, d_key]; V: [T, d_value]; theta/eta/alpha: [T] (per token) or [ceil(T / chunk)]
    (per chunk); gamma: [T] (used only when the window is > 1).
    history: the previous call's last (window - 1) tokens as (phi(k), v, gamma); empty at the
    start of a sequence, where the window is clipped.
    """
    W = [np.array(p, dtype=np.float64) for p in params]
    S = [np.array(s, dtype=np.float64) for s in momenta]
    T = int(K.shape[0])
    C = cfg.chunk
    c = cfg.omega_window
    X = poly_features(K, cfg.poly_degree)
    Xq = poly_features(Q, cfg.poly_degree)
    V = np.asarray(V, dtype=np.float64)
    res = cfg.kind == MLP2_SILU_RESIDUAL
    ptr = cfg.per_token_retrieve
    if ptr and cfg.gate_mode != PER_TOKEN:
        raise ValueError("per-token retrieval needs per-token gates")
    if res and X.shape[1] != cfg.d_value:
        raise ValueError("a residual memory needs d_in == d_value")
    hist = list(history or [])[-(c - 1):] if c > 1 else []

    def token(i):
        """(phi(k_i), v_i, gamma_i) of call-relative token i, or None before the sequence start."""
        if i >= 0:
            return X[i], V[i], (float(gamma[i]) if c > 1 else 1.0)
        j = len(hist) + i
        return hist[j] if j >= 0 else None

    Y = np.zeros((T, cfg.d_value))
    bounds = []
    health = []
    for s in range(0, T, C):
        e = min(s + C, T)                                  # the chunk is tokens [s, e)
        if keep_boundaries:
            bounds.append(([w.copy() for w in W], [m.copy() for m in S]))
        w_bar = [w.copy() for w in W]                     # chunk-start weights
        if not ptr:
            for t in range(s, e):                          # retrieval at the chunk-start weights
                Y[t] = memory_apply(w_bar, Xq[t], res)
        if cfg.gate_mode == PER_TOKEN:
            cache = {}

            def grad_at(i):
                if i not in cache:
                    tok = token(i)
                    cache[i] = None if tok is None else (loss_grad(w_bar, tok[0], tok[1], res), tok[2])
                return cache[i]

            for t in range(s, e):
                G = [np.zeros_like(w) for w in W]
                for i in range(t - c + 1, t + 1):
                    gi = grad_at(i)
                    if gi is None:
                        continue
                    grads, weight = gi
                    for G_m, g_m in zip(G, grads):
                        G_m += weight * g_m
                for m in range(len(W)):
                    S[m] = eta[t] * S[m] - theta[t] * G[m]
                    W[m] = (1.0 - alpha[t]) * W[m] + S[m]
                if ptr:                                    # the state right after token t's update
                    Y[t] = memory_apply(W, Xq[t], res)
        else:
            G = [np.zeros_like(w) for w in W]
            for t in range(s, e):
                for G_m, g_m in zip(G, loss_grad(w_bar, X[t], V[t], res)):
                    G_m += g_m
            if cfg.ns_steps > 0:
                G = [newton_schulz(g, cfg.ns_steps, cfg.ns_coeffs, cfg.ns_eps) for g in G]
            k = s // C
            for m in range(len(W)):
                S[m] = eta[k] * S[m] - theta[k] * G[m]
                W[m] = (1.0 - alpha[k]) * W[m] + S[m]
        health.append(max(float(np.max(np.abs(w))) for w in W))
    if keep_boundaries:
        bounds.append(([w.copy() for w in W], [m.copy() for m in S]))
    if c > 1:
        tail = [token(i) for i in range(T - (c - 1), T)]
        new_hist = [t for t in tail if t is not None]
    else:
        new_hist = []
    return MemoryResult(Y, W, S, new_hist, bounds, health)


# ----------------------------------------------------------------------------- many memories

def flatten(mats) -> np.ndarray:
    return np.concatenate([np.asarray(m, dtype=np.float64).ravel() for m in mats])


def unflatten(cfg: MemoryConfig, flat) -> list:
    flat = np.asarray(flat, dtype=np.float64)
    d_in = poly_feature_count(cfg.d_key, cfg.poly_degree)
    if cfg.kind == LINEAR:
        return [flat.reshape(cfg.d_value, d_in)]
    n1 = cfg.d_hidden * d_in
    if cfg.kind == MLP2_GATED:
        return [flat[:n1].reshape(cfg.d_hidden, d_in), flat[n1:2 * n1].reshape(cfg.d_hidden, d_in),
                flat[2 * n1:].reshape(cfg.d_value, cfg.d_hidden)]
    return [flat[:n1].reshape(cfg.d_hidden, d_in), flat[n1:].reshape(cfg.d_value, cfg.d_hidden)]


def poly_feature_count(d: int, degree: int) -> int:
    """Number of features phi produces, counted by enumerating the monomials."""
    if degree == 1:
        return d
    return sum(1 for deg in range(degree + 1) for _ in combinations_with_replacement(range(d), deg))


def _one(args):
    cfg, w_flat, s_flat, K, Q, V, th, et, al, ga = args
    r = run_memory(cfg, unflatten(cfg, w_flat), unflatten(cfg, s_flat), K, Q, V, th, et, al, ga)
    return r.Y, flatten(r.params), flatten(r.momenta)


def run_many(cfg: MemoryConfig, W0, S0, K, Q, V, theta, eta, alpha, gamma=None, processes: int = 1):
    """Run every memory m (leading axis) independently; returns Y [M,T,d_v], W [M,P], S [M,P].
    With processes > 1 the memories are spread over a process pool (one memory per task)."""
    M = K.shape[0]
    tasks = [(cfg, W0[m], S0[m], K[m], Q[m], V[m], theta[m], eta[m], alpha[m],
              None if gamma is None else gamma[m]) for m in range(M)]
    if processes > 1:
        import multiprocessing as mp
        ctx = mp.get_context("fork")
        with ctx.Pool(processes) as pool:
            out = pool.map(_one, tasks, chunksize=1)
    else:
        out = [_one(t) for t in tasks]
    Y = np.stack([o[0] for o in out])
    W = np.stack([o[1] for o in out])
    S = np.stack([o[2] for o in out])
    return Y, W, S
