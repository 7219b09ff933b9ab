"""Plain fp64 CPU oracle of the input prologue that precedes the memory update: the causal
short convolution of keys, queries and values, and the data-dependent gates.

TEST INFRASTRUCTURE.  Only the test suite, the smoke check and the benchmark's CPU-baseline
leg import this module.  The library never calls it and shares no code with it.

What it computes, and where the pages define it
-----------------------------------------------
* Short convolution: a causal depthwise 1-D convolution with kernel size 4 along the token
  axis, applied to keys, queries and values separately, with one filter per channel (and per
  head): Atlas-Torch README, Atlas Extensions table ("Short Convolution", kernel 4 on
  keys/values/queries); titans-pytorch-mlx README, Configuration table (use_conv,
  conv_kernel_size 4); titans-torch 0.1.2, API Reference (NeuralLongTermMemory, use_conv).
  Tap j of channel i multiplies token t - 3 + j:
      out[t, i] = bias[i] + sum_{j=0..3} w[i, j] * x[t - 3 + j, i]
  Tokens before the sequence start are zero, or the rows carried from a previous call.  An
  empty sequence is valid (Atlas-Torch README, Bug Fixes table, "Conv empty sequence").
* L2 normalisation of the convolved key / query rows (optional): row / max(||row||, 1e-12).
* Gates: theta, eta and alpha are functions of the input, not constants (titans-pytorch-mlx
  README, Core Equations, the ranges of alpha_t, eta_t, theta_t, and Key Innovations item 4);
  each is a configured maximum times a sigmoid gate (titans-pytorch-mlx README,
  Configuration table: memory_lr 0.1, memory_momentum 0.9, memory_decay 0.01, each "scaled
  by gate"), produced from the data by a small learned map (titans-torch 0.1.2, "Inner-loop
  update rule").  The Omega rule's context gates gamma are learned the same way (Atlas-Torch
  README, Atlas Extensions table, Omega Rule), with maximum 1.  Reading taken: the map is one
  linear layer per head on the token's input vector u_t,
      gate_g[t, h] = scale_g * sigmoid(Wg[g, h] . u_t + bg[g, h]).
* Per-chunk gates (one triple per chunk, the per-chunk path of the Newton-Schulz memory):
  the chunk's gates are pooled (Atlas-Torch README, Bug Fixes table, "no-omega ablation"
  row).  Reading taken: the gate of the chunk's mean-pooled input, i.e. the sigmoid of the
  mean of its tokens' logits; a final short chunk pools its own tokens.
* Feature map stage: monomials of degree 0..p (p <= 3) with learnable per-degree coefficients
  (default 1/k!, the exponential kernel's Taylor coefficients, which Dot uses with the Omega
  rule) and the optional projection back (Atlas-Torch README, Atlas Extensions table,
  "Polynomial Features"; ATLAS summary, sections 3.1 and 4.3).
"""

from __future__ import annotations

import math

import numpy as np

CONV_TAPS = 4


def short_conv(x: np.ndarray, taps: np.ndarray, bias=None, hist=None) -> np.ndarray:
    """Causal depthwise convolution of one memory's rows.

    x: [T, d]; taps: [d, 4] (tap j on token t - 3 + j); bias: [d] or None;
    hist: [3, d], the three rows before x, oldest first (None: the sequence start, zeros).
    Returns [T, d] float64."""
    x = np.asarray(x, dtype=np.float64)
    T, d = x.shape
    w = np.asarray(taps, dtype=np.float64)
    assert w.shape == (d, CONV_TAPS)
    prev = np.zeros((CONV_TAPS - 1, d)) if hist is None else np.asarray(hist, dtype=np.float64)
    assert prev.shape == (CONV_TAPS - 1, d)
    rows = np.concatenate([prev, x], axis=0)  # row t + 3 is token t
    out = np.zeros((T, d)) if bias is None else np.tile(np.asarray(bias, dtype=np.float64), (T, 1))
    for t in range(T):
        for j in range(CONV_TAPS):
            out[t] += w[:, j] * rows[t + j]
    return out


def l2_normalise(y: np.ndarray) -> np.ndarray:
    """Each row divided by max(its Euclidean norm, 1e-12); zero rows stay zero."""
    y = np.asarray(y, dtype=np.float64)
    n = np.sqrt(np.sum(y * y, axis=-1, keepdims=True))
    return y / np.maximum(n, 1e-12)


def conv_history(x: np.ndarray, hist=None) -> np.ndarray:
    """The three rows that precede the token after x: the last three of (hist ++ x)."""
    x = np.asarray(x, dtype=np.float64)
    prev = np.zeros((CONV_TAPS - 1, x.shape[1])) if hist is None else np.asarray(hist, dtype=np.float64)
    return np.concatenate([prev, x], axis=0)[-(CONV_TAPS - 1):]


def short_conv_all(X: np.ndarray, taps: np.ndarray, heads: int, bias=None, hist=None, l2norm=False) -> np.ndarray:
    """All memories m = b * heads + h: X [M, T, d], taps [heads, d, 4], bias [heads, d],
    hist [M, 3, d]; memory m uses the filters of head m % heads."""
    M = X.shape[0]
    out = np.empty(X.shape, dtype=np.float64)
    for m in range(M):
        h = m % heads
        y = short_conv(X[m], taps[h], None if bias is None else bias[h], None if hist is None else hist[m])
        out[m] = l2_normalise(y) if l2norm else y
    return out


def sigmoid(z):
    z = np.asarray(z, dtype=np.float64)
    return 1.0 / (1.0 + np.exp(-z))


def gates(U: np.ndarray, Wg: np.ndarray, bg: np.ndarray, scale, chunk: int = 1) -> np.ndarray:
    """Gates of one sequence for every (gate, head).

    U: [T, dm] token inputs; Wg: [n_g, H, dm]; bg: [n_g, H]; scale: [n_g];
    chunk 1: per token, else one value per chunk of `chunk` tokens (the last may be short).
    Returns [n_g, H, n] with n = T (chunk 1) or ceil(T / chunk)."""
    U = np.asarray(U, dtype=np.float64)
    Wg = np.asarray(Wg, dtype=np.float64)
    bg = np.asarray(bg, dtype=np.float64)
    n_g, H, dm = Wg.shape
    T = U.shape[0]
    logits = np.einsum("ghk,tk->ght", Wg, U) + bg[:, :, None]  # [n_g, H, T]
    if chunk > 1:
        n = -(-T // chunk)
        pooled = np.empty((n_g, H, n))
        for c in range(n):
            pooled[:, :, c] = logits[:, :, c * chunk:min((c + 1) * chunk, T)].mean(axis=2)
        logits = pooled
    return np.asarray(scale, dtype=np.float64)[:, None, None] * sigmoid(logits)


def gates_all(U: np.ndarray, Wg: np.ndarray, bg: np.ndarray, scale, chunk: int = 1) -> np.ndarray:
    """U: [B, T, dm] -> [n_g, B, H, n] (memory m = b * H + h reads row [g, b, h])."""
    return np.stack([gates(U[b], Wg, bg, scale, chunk) for b in range(U.shape[0])], axis=1)


def gates_bruteforce(U, Wg, bg, scale, chunk: int = 1):
    """Pure-Python loops over tiny inputs, for pinning `gates`."""
    n_g, H, dm = len(Wg), len(Wg[0]), len(Wg[0][0])
    T = len(U)
    n = T if chunk == 1 else -(-T // chunk)
    out = [[[0.0] * n for _ in range(H)] for _ in range(n_g)]
    for g in range(n_g):
        for h in range(H):
            zs = []
            for t in range(T):
                z = float(bg[g][h])
                for k in range(dm):
                    z += float(Wg[g][h][k]) * float(U[t][k])
                zs.append(z)
            for c in range(n):
                part = zs[c:c + 1] if chunk == 1 else zs[c * chunk:min((c + 1) * chunk, T)]
                z = sum(part) / len(part)
                out[g][h][c] = float(scale[g]) / (1.0 + math.exp(-z))
    return out


# ----------------------------------------------------------------------------- feature map stage

def feature_map(x, degree: int, coeffs=None, P=None) -> np.ndarray:
    """phi_c(x) of every row: all monomials of degree 0..p in combinations_with_replacement order
    (degree-major), the monomials of degree k multiplied by coeffs[k] (default 1/k!, the Taylor
    coefficients of the exponential kernel), optionally projected back, phi_c(x) P^T.

    Atlas-Torch README, Atlas Extensions table, "Polynomial Features" (exact monomial expansion,
    learnable coefficients initialised to 1/d!, optional project_back); ATLAS summary, sections 3.1
    (polynomial features) and 4.1-4.3 (Dot: the exponential feature construction with the Omega
    rule)."""
    from itertools import combinations_with_replacement
    x = np.asarray(x, dtype=np.float64)
    n, d = x.shape
    c = [1.0 / math.factorial(k) for k in range(degree + 1)] if coeffs is None else list(coeffs)
    assert len(c) == degree + 1
    cols = []
    for k in range(degree + 1):
        for combo in combinations_with_replacement(range(d), k):
            col = np.full(n, float(c[k]))
            for i in combo:
                col = col * x[:, i]
            cols.append(col)
    F = np.stack(cols, axis=1)
    return F if P is None else F @ np.asarray(P, dtype=np.float64).T


def feature_count(d: int, degree: int) -> int:
    return math.comb(d + degree, degree)
