"""fp64 oracle of the outer-loop backward of the memory update: the gradients of an outer loss
with respect to every input of the chunked test-time update (keys, queries, values, gates,
initial state), i.e. the derivative of the inner recurrence, which itself contains the inner
gradient (the "gradient of the gradient").

TEST INFRASTRUCTURE.  Only the test suite may import this module.  The library never calls it.

What it computes, and where the pages define it
-----------------------------------------------
The outer loop trains the model through the test-time updates: the full forward pass runs the
inner updates, and the outer loss is back-propagated through them (Atlas-Torch README, "How the
memory works": the two loops; Bug Fixes table, "Store-path gradient starvation": outer-loop
gradient to the store-side parameters through the memory).  For a scalar outer loss L with
adjoints dY = dL/dY and dW_T, dS_T = dL/d(final state), the gradients are those of
    L = <dY, Y> + <dW_T, W_T> + <dS_T, S_T>
with Y, W_T, S_T from the literal chunked recurrence (the fp64 oracle's algorithm, restated
with torch operations) -- the plain definition of a vector-Jacobian product, taken here by
torch autograd as a library step.
"""

from __future__ import annotations

import math
from itertools import combinations_with_replacement

import numpy as np
import torch

from .neural_memory import LINEAR, MLP2_SILU, MLP2_SILU_RESIDUAL, PER_TOKEN, MemoryConfig


def _silu(z):
    return z * torch.sigmoid(z)


def _poly(x, degree):
    """phi of every row of x ([T, d]) with torch operations: the monomials of degree 0..p, each
    degree's coefficient 1/deg!, degree-major and in combinations_with_replacement order inside a
    degree (Atlas-Torch README, Atlas Extensions table, Polynomial Features); identity for p = 1."""
    if degree == 1:
        return x
    cols = []
    for deg in range(degree + 1):
        for combo in combinations_with_replacement(range(x.shape[1]), deg):
            col = torch.full((x.shape[0],), 1.0 / math.factorial(deg), dtype=x.dtype)
            for i in combo:
                col = col * x[:, i]
            cols.append(col)
    return torch.stack(cols, dim=1)


def _apply(params, x, residual=False):
    if len(params) == 1:
        return params[0] @ x
    if len(params) == 3:  # the gated memory [W1, W3, W2]: W2 (silu(W1 x) * (W3 x))
        return params[2] @ (_silu(params[0] @ x) * (params[1] @ x))
    y = params[1] @ _silu(params[0] @ x)
    return x + y if residual else y


def _grad(params, x, v, residual=False):
    """The inner gradient of ||M_W(x) - v||^2, written out (so that it can itself be
    differentiated): linear 2 (W x - v) x^T; MLP e = 2 (W2 h - v), (W2^T e) * silu'(z) x^T, e h^T;
    the residual memory x + W2 silu(W1 x) has e = 2 (W2 h + x - v) (ATLAS summary, section 5.1)."""
    if len(params) == 1:
        return [torch.outer(2.0 * (params[0] @ x - v), x)]
    if len(params) == 3:
        # the gated memory (ATLAS summary, section 5.1): a = silu(z1), h = a * z3, e = 2 (W2 h - v),
        # b = W2^T e: (b * z3 * silu'(z1)) x^T, (b * a) x^T, e h^T
        w1, w3, w2 = params
        z1, z3 = w1 @ x, w3 @ x
        s1 = torch.sigmoid(z1)
        a = z1 * s1
        e = 2.0 * (w2 @ (a * z3) - v)
        b = w2.T @ e
        sp = s1 * (1.0 + z1 * (1.0 - s1))
        return [torch.outer(b * z3 * sp, x), torch.outer(b * a, x), torch.outer(e, a * z3)]
    w1, w2 = params
    z = w1 @ x
    s = torch.sigmoid(z)
    h = z * s
    e = 2.0 * (w2 @ h + x - v) if residual else 2.0 * (w2 @ h - v)
    sp = s * (1.0 + z * (1.0 - s))
    return [torch.outer((w2.T @ e) * sp, x), torch.outer(e, h)]


def _newton_schulz(g, steps, coeffs, eps):
    """The quintic iteration of the oracle's newton_schulz, with torch operations."""
    a, b, c = coeffs
    x = g / (torch.linalg.norm(g) + eps)
    tr = x.shape[0] > x.shape[1]
    if tr:
        x = x.T
    for _ in range(steps):
        A = x @ x.T
        x = a * x + (b * A + c * (A @ A)) @ x
    return x.T if tr else x


def run_memory_torch(cfg: MemoryConfig, params, momenta, K, Q, V, theta, eta, alpha, gamma=None):
    """The literal chunked recurrence for one memory (keys and queries through the polynomial
    feature map; per-token gates with an Omega window of c tokens, or per-chunk gates with an
    optional Newton-Schulz orthogonalisation of the summed chunk gradient) with torch tensors:
    Y, final params, final momenta.  Plain, residual or linear memory.  The window starts with the sequence (no history
    from a previous call): token t's step uses sum_{i=t-c+1..t, i>=0} gamma_i g_i, every g_i taken
    at the weights of the chunk that holds t (ATLAS summary, sections 3.2-3.3)."""
    c = cfg.omega_window
    assert c == 1 or cfg.gate_mode == PER_TOKEN
    res = cfg.kind == MLP2_SILU_RESIDUAL
    K, Q = _poly(K, cfg.poly_degree), _poly(Q, cfg.poly_degree)  # the memory reads features
    W = list(params)
    S = list(momenta)
    T = K.shape[0]
    C = cfg.chunk
    Y = []
    for s in range(0, T, C):
        e = min(s + C, T)
        wb = list(W)
        for t in range(s, e):
            Y.append(_apply(wb, Q[t], res))
        if cfg.gate_mode == PER_TOKEN:
            grads = {}
            for t in range(s, e):
                G = None
                for i in range(max(t - c + 1, 0), t + 1):
                    if i not in grads:
                        grads[i] = _grad(wb, K[i], V[i], res)
                    w_i = 1.0 if c == 1 else gamma[i]
                    G = [w_i * g for g in grads[i]] if G is None else [G[m] + w_i * g for m, g in enumerate(grads[i])]
                S = [eta[t] * S[m] - theta[t] * G[m] for m in range(len(W))]
                W = [(1.0 - alpha[t]) * W[m] + S[m] for m in range(len(W))]
        else:
            G = [torch.zeros_like(w) for w in W]
            for t in range(s, e):
                G = [G[m] + g for m, g in enumerate(_grad(wb, K[t], V[t], res))]
            if cfg.ns_steps > 0:
                G = [_newton_schulz(g, cfg.ns_steps, cfg.ns_coeffs, cfg.ns_eps) for g in G]
            k = s // C
            S = [eta[k] * S[m] - theta[k] * G[m] for m in range(len(W))]
            W = [(1.0 - alpha[k]) * W[m] + S[m] for m in range(len(W))]
    return torch.stack(Y), W, S


def outer_grads(cfg: MemoryConfig, params, momenta, K, Q, V, theta, eta, alpha, dY, dW_T=None, dS_T=None,
                gamma=None):
    """Gradients of <dY, Y> + <dW_T, W_T> + <dS_T, S_T> (numpy in, numpy out, fp64):
    dict with K, Q, V, theta, eta, alpha, W0 (list), S0 (list), and gamma for a window > 1."""
    t = lambda a: torch.tensor(np.asarray(a, dtype=np.float64), requires_grad=True)
    P = [t(p) for p in params]
    M = [t(m) for m in momenta]
    k, q, v, th, et, al = t(K), t(Q), t(V), t(theta), t(eta), t(alpha)
    gm = t(gamma) if cfg.omega_window > 1 else None
    Y, W, S = run_memory_torch(cfg, P, M, k, q, v, th, et, al, gm)
    L = (Y * torch.tensor(np.asarray(dY, dtype=np.float64))).sum()
    if dW_T is not None:
        L = L + sum((w * torch.tensor(np.asarray(d, dtype=np.float64))).sum() for w, d in zip(W, dW_T))
    if dS_T is not None:
        L = L + sum((m * torch.tensor(np.asarray(d, dtype=np.float64))).sum() for m, d in zip(S, dS_T))
    extra = [gm] if gm is not None else []
    grads = torch.autograd.grad(L, [k, q, v, th, et, al] + P + M + extra, allow_unused=True)
    z = lambda g, ref: np.zeros(ref.shape) if g is None else g.detach().numpy()
    names = ["K", "Q", "V", "theta", "eta", "alpha"]
    srcs = [k, q, v, th, et, al]
    out = {n: z(g, s) for n, g, s in zip(names, grads[:6], srcs)}
    out["W0"] = [z(g, p) for g, p in zip(grads[6:6 + len(P)], P)]
    out["S0"] = [z(g, m) for g, m in zip(grads[6 + len(P):6 + len(P) + len(M)], M)]
    if gm is not None:
        out["gamma"] = z(grads[-1], gm)
    return out
