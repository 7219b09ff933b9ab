"""Pins of the fp64 oracle against things other than itself.

Each test ties one part of the oracle to an independent authority: a library
gradient (torch autograd), a library factorisation (numpy SVD), a closed form,
brute force on tiny inputs, or a value written out by hand from the pages.
A plausible slip in the oracle (a dropped term, a wrong sign, a wrong index, a
transposed operand, the wrong update order) fails at least one of them.
"""

import math
import os

import numpy as np
import pytest
import torch

import oracle
from oracle import MemoryConfig, LINEAR, MLP2_SILU, MLP2_SILU_RESIDUAL, MLP2_GATED, PER_TOKEN, PER_CHUNK

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
NS = (3.4445, -4.7750, 2.0315)

# ----------------------------------------------------------------------------- helpers (test-only)


def rng(seed):
    return np.random.default_rng(seed)


def rand_params(r, kind, d_in, d_v, d_h, scale=0.5):
    if kind == LINEAR:
        return [r.normal(0, scale, (d_v, d_in))]
    if kind == MLP2_GATED:
        return [r.normal(0, scale, (d_h, d_in)), r.normal(0, scale, (d_h, d_in)), r.normal(0, scale, (d_v, d_h))]
    return [r.normal(0, scale, (d_h, d_in)), r.normal(0, scale, (d_v, d_h))]


def torch_memory(params, x, residual=False):
    """M_W(x) written with torch primitives (silu from torch.nn.functional); the residual memory
    adds its input."""
    if len(params) == 1:
        return params[0] @ x
    if len(params) == 3:  # gated: W2 (silu(W1 x) * (W3 x))
        return params[2] @ (torch.nn.functional.silu(params[0] @ x) * (params[1] @ x))
    y = params[1] @ torch.nn.functional.silu(params[0] @ x)
    return x + y if residual else y


def phi_triu(x, degree):
    """Independent degree<=2 feature map: constant, x, then x_i x_j / 2 over the upper triangle
    (np.triu_indices walks i <= j row by row, the same order as combinations_with_replacement)."""
    x = np.asarray(x, dtype=np.float64)
    if degree == 1:
        return x
    iu, ju = np.triu_indices(x.shape[-1])
    return np.concatenate([np.ones(x.shape[:-1] + (1,)), x, 0.5 * x[..., iu] * x[..., ju]], axis=-1)


def autograd_window_grad(params_np, xs, vs, ws, residual=False):
    """Gradient of sum_i w_i ||M_W(x_i) - v_i||^2 with respect to every weight matrix, by autograd."""
    params = [torch.tensor(p, dtype=torch.float64, requires_grad=True) for p in params_np]
    L = torch.zeros((), dtype=torch.float64)
    for x, v, w in zip(xs, vs, ws):
        r = torch_memory(params, torch.tensor(x), residual) - torch.tensor(v)
        L = L + w * (r * r).sum()
    if not L.requires_grad:
        return [np.zeros_like(p) for p in params_np]
    grads = torch.autograd.grad(L, params, allow_unused=True)
    return [np.zeros_like(p) if g is None else g.numpy() for g, p in zip(grads, params_np)]


def ns5_svd(G, steps=5, coeffs=NS, eps=1e-7):
    """Newton-Schulz through the SVD: each singular value sigma/(||G||_F+eps) goes through the scalar
    quintic f(s) = a s + b s^3 + c s^5 `steps` times; singular vectors are unchanged."""
    a, b, c = coeffs
    U, sig, Vt = np.linalg.svd(G, full_matrices=False)
    s = sig / (np.linalg.norm(G) + eps)
    for _ in range(steps):
        s = a * s + b * s ** 3 + c * s ** 5
    return (U * s) @ Vt


def bruteforce_run(cfg, params, momenta, K, Q, V, th, et, al, ga):
    """Per-step gradient of the windowed loss at the chunk-start weights by autograd, features by
    phi_triu, retrieval by torch (at the chunk start, or right after each step for per-token
    retrieval); the momentum / forgetting updates applied step by step."""
    W = [p.copy() for p in params]
    S = [m.copy() for m in momenta]
    X = phi_triu(K, cfg.poly_degree)
    Xq = phi_triu(Q, cfg.poly_degree)
    T, C, c = K.shape[0], cfg.chunk, cfg.omega_window
    res = cfg.kind == MLP2_SILU_RESIDUAL
    Y = np.zeros((T, cfg.d_value))
    for s in range(0, T, C):
        e = min(s + C, T)  # a final partial chunk holds the rest
        wb = [w.copy() for w in W]
        tw = [torch.tensor(w) for w in wb]
        for t in range(s, e):
            Y[t] = torch_memory(tw, torch.tensor(Xq[t]), res).numpy()
        if cfg.gate_mode == PER_TOKEN:
            for t in range(s, e):
                idx = [i for i in range(t - c + 1, t + 1) if i >= 0]
                ws = [(ga[i] if c > 1 else 1.0) for i in idx]
                G = autograd_window_grad(wb, [X[i] for i in idx], [V[i] for i in idx], ws, res)
                for m in range(len(W)):
                    S[m] = et[t] * S[m] - th[t] * G[m]
                    W[m] = (1 - al[t]) * W[m] + S[m]
                if cfg.per_token_retrieve:
                    Y[t] = torch_memory([torch.tensor(w) for w in W], torch.tensor(Xq[t]), res).numpy()
        else:
            idx = list(range(s, e))
            G = autograd_window_grad(wb, [X[i] for i in idx], [V[i] for i in idx], [1.0] * len(idx), res)
            if cfg.ns_steps:
                G = [ns5_svd(g, cfg.ns_steps) for g in G]
            k = s // C
            for m in range(len(W)):
                S[m] = et[k] * S[m] - th[k] * G[m]
                W[m] = (1 - al[k]) * W[m] + S[m]
    return Y, W, S


def tiny_problem(seed, kind, T, d_k, d_v, d_h, poly, C, c, mode, ns=0, gate_scale=1.0):
    r = rng(seed)
    cfg = MemoryConfig(kind, d_k, d_v, d_h, poly, C, c, mode, ns)
    d_in = oracle.poly_feature_count(d_k, poly)
    params = rand_params(r, kind, d_in, d_v, d_h)
    momenta = [r.normal(0, 0.1, p.shape) for p in params]
    K = r.normal(0, 1, (T, d_k)) / math.sqrt(d_k)
    Q = r.normal(0, 1, (T, d_k)) / math.sqrt(d_k)
    V = r.normal(0, 1, (T, d_v))
    ng = T if mode == PER_TOKEN else -(-T // C)
    th = r.uniform(0.01, 0.1, ng) * gate_scale
    et = r.uniform(0.8, 0.99, ng)
    al = r.uniform(0.0, 0.05, ng)
    ga = r.uniform(0, 1, T)
    return cfg, params, momenta, K, Q, V, th, et, al, ga


def maxrel(a, b):
    a, b = np.asarray(a), np.asarray(b)
    return float(np.max(np.abs(a - b)) / max(np.max(np.abs(b)), 1e-300))


# ----------------------------------------------------------------------------- gradients


@pytest.mark.parametrize("kind", [LINEAR, MLP2_SILU, MLP2_SILU_RESIDUAL, MLP2_GATED])
def test_loss_gradient_matches_autograd(kind):
    r = rng(1)
    res = kind == MLP2_SILU_RESIDUAL
    d_in, d_v = (6, 6) if res else (7, 5)
    params = rand_params(r, kind, d_in, d_v, 9)
    x, v = r.normal(size=d_in), r.normal(size=d_v)
    got = oracle.loss_grad(params, x, v, res)
    ref = autograd_window_grad(params, [x], [v], [1.0], res)
    for g, h in zip(got, ref):
        assert g.shape == h.shape
        np.testing.assert_allclose(g, h, rtol=1e-13, atol=1e-13)


def test_residual_memory_identity_and_shifted_target():
    """With W2 = 0 the residual memory is the identity; its gradient equals the plain memory's
    for the target v - x (the residual only shifts the prediction error)."""
    r = rng(2)
    w1, w2 = rand_params(r, MLP2_SILU, 6, 6, 8)
    x, v = r.normal(size=6), r.normal(size=6)
    assert np.array_equal(oracle.memory_apply([w1, np.zeros_like(w2)], x, True), x)
    g_res = oracle.loss_grad([w1, w2], x, v, True)
    g_plain = oracle.loss_grad([w1, w2], x, v - x)
    for a, b in zip(g_res, g_plain):
        np.testing.assert_allclose(a, b, rtol=1e-13, atol=1e-14)
    with pytest.raises(ValueError):
        cfg = MemoryConfig(MLP2_SILU_RESIDUAL, 4, 3, 5)
        oracle.run_memory(cfg, rand_params(r, MLP2_SILU, 4, 3, 5), rand_params(r, MLP2_SILU, 4, 3, 5),
                          r.normal(size=(4, 4)), r.normal(size=(4, 4)), r.normal(size=(4, 3)), np.ones(4),
                          np.ones(4), np.zeros(4))


def test_gated_memory_reduces_to_plain_when_gate_is_one():
    """If W3 x = 1 for every hidden unit, the gated memory is the plain one and its W1 and W2
    gradients are the plain memory's; its W3 gradient is (W2^T e) * silu(W1 x) times x^T."""
    r = rng(3)
    w1, w2 = rand_params(r, MLP2_SILU, 5, 3, 7)
    x = np.zeros(5)
    x[0] = 1.0
    w3 = r.normal(size=(7, 5))
    w3[:, 0] = 1.0
    v = r.normal(size=3)
    np.testing.assert_allclose(oracle.memory_apply([w1, w3, w2], x), oracle.memory_apply([w1, w2], x), rtol=1e-15)
    g1, g3, g2 = oracle.loss_grad([w1, w3, w2], x, v)
    p1, p2 = oracle.loss_grad([w1, w2], x, v)
    np.testing.assert_allclose(g1, p1, rtol=1e-14, atol=1e-15)
    np.testing.assert_allclose(g2, p2, rtol=1e-14, atol=1e-15)
    e = 2.0 * (oracle.memory_apply([w1, w2], x) - v)
    np.testing.assert_allclose(g3, np.outer((w2.T @ e) * oracle.silu(w1 @ x), x), rtol=1e-14, atol=1e-15)


def test_linear_gradient_is_delta_rule_outer_product():
    """Linear memory: the gradient is 2 (W k - v) k^T -- checked against the loss by central differences."""
    r = rng(2)
    W = r.normal(size=(4, 6))
    k, v = r.normal(size=6), r.normal(size=4)
    g = oracle.loss_grad([W], k, v)[0]
    h = 1e-6
    fd = np.zeros_like(W)
    for i in range(W.shape[0]):
        for j in range(W.shape[1]):
            Wp, Wm = W.copy(), W.copy()
            Wp[i, j] += h
            Wm[i, j] -= h
            fd[i, j] = (oracle.loss([Wp], k, v) - oracle.loss([Wm], k, v)) / (2 * h)
    assert maxrel(g, fd) < 1e-7
    # rank one, with the key as the row factor
    assert np.linalg.matrix_rank(g) == 1
    np.testing.assert_allclose(g @ np.linalg.pinv(k[None, :]).ravel(), g @ k / (k @ k), rtol=1e-12)


def test_mlp_gradient_central_differences():
    """Tiny MLP memory (d=3, h=5, v=2): analytic gradient vs central differences of the loss."""
    r = rng(3)
    params = rand_params(r, MLP2_SILU, 3, 2, 5, scale=0.8)
    x, v = r.normal(size=3), r.normal(size=2)
    got = oracle.loss_grad(params, x, v)
    h = 1e-6
    for m, P in enumerate(params):
        fd = np.zeros_like(P)
        for idx in np.ndindex(P.shape):
            pp = [p.copy() for p in params]
            pm = [p.copy() for p in params]
            pp[m][idx] += h
            pm[m][idx] -= h
            fd[idx] = (oracle.loss(pp, x, v) - oracle.loss(pm, x, v)) / (2 * h)
        assert maxrel(got[m], fd) < 1e-7


def test_silu_and_derivative_against_torch():
    z = np.linspace(-30, 30, 241)
    tz = torch.tensor(z, requires_grad=True)
    y = torch.nn.functional.silu(tz)
    (dy,) = torch.autograd.grad(y.sum(), tz)
    np.testing.assert_allclose(oracle.silu(z), y.detach().numpy(), rtol=1e-14, atol=1e-300)
    np.testing.assert_allclose(oracle.silu_prime(z), dy.numpy(), rtol=1e-13, atol=1e-15)


# ----------------------------------------------------------------------------- recurrence


def test_delta_rule_exact_storage():
    """Linear memory, chunk 1, eta = alpha = 0, theta = 1/2, orthonormal keys: each step is the delta
    rule with step 1/(2||k||^2), which writes the association exactly, so W_T = sum v_t k_t^T and
    retrieving with the previous key returns the previous value."""
    d, T = 8, 6
    r = rng(4)
    Qm, _ = np.linalg.qr(r.normal(size=(d, d)))
    K = Qm[:T]
    V = r.normal(size=(T, 5))
    Qs = np.vstack([np.zeros(d), K[:-1]])          # q_t = k_{t-1}
    cfg = MemoryConfig(LINEAR, d, 5, 0, 1, 1, 1, PER_TOKEN, 0)
    res = oracle.run_memory(cfg, [np.zeros((5, d))], [np.zeros((5, d))], K, Qs, V,
                            np.full(T, 0.5), np.zeros(T), np.zeros(T))
    np.testing.assert_allclose(res.params[0], V.T @ K, atol=1e-14)
    np.testing.assert_allclose(res.Y[1:], V[:-1], atol=1e-14)     # y_t = W_{t-1} q_t
    np.testing.assert_allclose(res.Y[0], 0.0)


@pytest.mark.parametrize("mode", [PER_TOKEN, PER_CHUNK])
def test_zero_lr_is_pure_decay(mode):
    """theta = 0: with S0 = 0 the weights only decay, W_T = prod(1 - alpha) W_0; a non-zero S0 decays
    as S_T = prod(eta) S_0."""
    cfg, params, _, K, Q, V, th, et, al, ga = tiny_problem(5, MLP2_SILU, 16, 3, 2, 4, 1, 4, 1, mode)
    zeros = [np.zeros_like(p) for p in params]
    res = oracle.run_memory(cfg, params, zeros, K, Q, V, np.zeros_like(th), et, al)
    for w, w0 in zip(res.params, params):
        np.testing.assert_allclose(w, np.prod(1 - al) * w0, rtol=1e-13)
    S0 = [np.ones_like(p) for p in params]
    res = oracle.run_memory(cfg, params, S0, K, Q, V, np.zeros_like(th), et, al)
    for s in res.momenta:
        np.testing.assert_allclose(s, np.prod(et) * np.ones_like(s), rtol=1e-13)


def test_chunk_gradients_taken_at_chunk_start():
    """With eta = alpha = 0 and a constant theta, a single chunk's update is the sum of gradients all
    taken at W_0, so it does not depend on the order of the tokens inside the chunk; with chunk 1
    (gradient at the running weights) it does."""
    cfg, params, momenta, K, Q, V, th, et, al, ga = tiny_problem(6, MLP2_SILU, 8, 3, 2, 4, 1, 8, 1, PER_TOKEN)
    zeros = [np.zeros_like(p) for p in params]
    th = np.full(8, 0.05)
    z = np.zeros(8)
    perm = rng(0).permutation(8)
    a = oracle.run_memory(cfg, params, zeros, K, Q, V, th, z, z)
    b = oracle.run_memory(cfg, params, zeros, K[perm], Q, V[perm], th, z, z)
    for x, y in zip(a.params, b.params):
        np.testing.assert_allclose(x, y, rtol=1e-12, atol=1e-15)
    cfg1 = MemoryConfig(MLP2_SILU, 3, 2, 4, 1, 1, 1, PER_TOKEN, 0)
    a1 = oracle.run_memory(cfg1, params, zeros, K, Q, V, th, z, z)
    b1 = oracle.run_memory(cfg1, params, zeros, K[perm], Q, V[perm], th, z, z)
    assert max(maxrel(x, y) for x, y in zip(a1.params, b1.params)) > 1e-6


def test_retrieval_uses_chunk_start_weights():
    """Every query of a chunk is answered by the weights at the chunk boundary (torch forward)."""
    cfg, params, momenta, K, Q, V, th, et, al, ga = tiny_problem(7, MLP2_SILU, 12, 3, 2, 4, 1, 4, 1, PER_TOKEN)
    res = oracle.run_memory(cfg, params, momenta, K, Q, V, th, et, al, keep_boundaries=True)
    for ci in range(3):
        wb = [torch.tensor(w) for w in res.boundary_states[ci][0]]
        for t in range(ci * 4, ci * 4 + 4):
            np.testing.assert_allclose(res.Y[t], torch_memory(wb, torch.tensor(Q[t])).numpy(), rtol=1e-13)


CASES = [
    # kind, T, d_k, d_v, d_h, poly, C, c, mode, ns
    (LINEAR, 12, 4, 3, 0, 1, 1, 1, PER_TOKEN, 0),
    (LINEAR, 12, 4, 3, 0, 1, 4, 3, PER_TOKEN, 0),
    (MLP2_SILU, 12, 3, 2, 5, 1, 4, 1, PER_TOKEN, 0),
    (MLP2_SILU, 12, 3, 2, 5, 1, 4, 3, PER_TOKEN, 0),
    (MLP2_SILU, 12, 3, 2, 5, 2, 4, 4, PER_TOKEN, 0),
    (MLP2_SILU, 12, 3, 2, 5, 2, 3, 5, PER_TOKEN, 0),
    (MLP2_SILU, 12, 3, 2, 5, 1, 4, 1, PER_CHUNK, 0),
    (MLP2_SILU, 12, 3, 2, 5, 1, 4, 1, PER_CHUNK, 5),
    (MLP2_SILU, 12, 3, 4, 6, 2, 6, 1, PER_CHUNK, 5),
    (LINEAR, 12, 4, 3, 0, 1, 4, 1, PER_CHUNK, 5),
    # a final partial chunk (T not a multiple of the chunk)
    (MLP2_SILU, 14, 3, 2, 5, 1, 4, 3, PER_TOKEN, 0),
    (MLP2_SILU, 13, 3, 2, 5, 2, 5, 2, PER_TOKEN, 0),
    (MLP2_SILU, 10, 3, 2, 5, 1, 4, 1, PER_CHUNK, 5),
    (LINEAR, 7, 4, 3, 0, 1, 3, 1, PER_CHUNK, 0),
    # the residual memory x + W2 silu(W1 x) (d_in == d_v; poly 2 on d_k = 2 gives d_in = 6)
    (MLP2_SILU_RESIDUAL, 12, 3, 3, 5, 1, 4, 3, PER_TOKEN, 0),
    (MLP2_SILU_RESIDUAL, 12, 2, 6, 5, 2, 4, 2, PER_TOKEN, 0),
    (MLP2_SILU_RESIDUAL, 13, 4, 4, 6, 1, 4, 1, PER_CHUNK, 5),
    # the gated memory W2 (silu(W1 x) * (W3 x))
    (MLP2_GATED, 12, 3, 2, 5, 1, 4, 3, PER_TOKEN, 0),
    (MLP2_GATED, 12, 3, 2, 5, 2, 4, 1, PER_TOKEN, 0),
    (MLP2_GATED, 13, 3, 4, 6, 1, 4, 1, PER_CHUNK, 5),
]


@pytest.mark.parametrize("case", CASES)
def test_recurrence_against_autograd_bruteforce(case):
    """The whole recurrence vs a brute force that takes each step's gradient of the windowed loss by
    autograd (window crossing chunk boundaries, clipped at t = 0), features by an independent map and
    Newton-Schulz through the SVD."""
    kind, T, d_k, d_v, d_h, poly, C, c, mode, ns = case
    cfg, params, momenta, K, Q, V, th, et, al, ga = tiny_problem(11, kind, T, d_k, d_v, d_h, poly, C, c, mode, ns)
    res = oracle.run_memory(cfg, params, momenta, K, Q, V, th, et, al, ga)
    Y, W, S = bruteforce_run(cfg, params, momenta, K, Q, V, th, et, al, ga)
    assert maxrel(res.Y, Y) < 1e-11
    for a, b in zip(res.params, W):
        assert maxrel(a, b) < 1e-11
    for a, b in zip(res.momenta, S):
        assert maxrel(a, b) < 1e-11


PTR_CASES = [
    # kind, T, d_k, d_v, d_h, poly, C, c
    (LINEAR, 12, 4, 3, 0, 1, 4, 3),
    (MLP2_SILU, 12, 3, 2, 5, 1, 4, 1),
    (MLP2_SILU, 14, 3, 2, 5, 2, 4, 3),
    (MLP2_SILU_RESIDUAL, 12, 3, 3, 5, 1, 5, 2),
    (MLP2_GATED, 12, 3, 2, 5, 1, 4, 3),
]


@pytest.mark.parametrize("case", PTR_CASES)
def test_per_token_retrieve_against_bruteforce(case):
    """Per-token retrieval (each query answered right after its token's update) against the
    autograd brute force; the chunk-start retrieval of the same run differs from it."""
    import dataclasses
    kind, T, d_k, d_v, d_h, poly, C, c = case
    cfg, params, momenta, K, Q, V, th, et, al, ga = tiny_problem(13, kind, T, d_k, d_v, d_h, poly, C, c, PER_TOKEN)
    cfg = dataclasses.replace(cfg, per_token_retrieve=True)
    res = oracle.run_memory(cfg, params, momenta, K, Q, V, th, et, al, ga)
    Y, W, S = bruteforce_run(cfg, params, momenta, K, Q, V, th, et, al, ga)
    assert maxrel(res.Y, Y) < 1e-11
    for a, b in zip(res.params, W):
        assert maxrel(a, b) < 1e-11
    plain = oracle.run_memory(dataclasses.replace(cfg, per_token_retrieve=False), params, momenta, K, Q, V, th,
                              et, al, ga)
    for a, b in zip(plain.params, res.params):
        assert np.array_equal(a, b)  # retrieval does not touch the state
    assert maxrel(plain.Y, res.Y) > 1e-6
    with pytest.raises(ValueError):
        oracle.run_memory(dataclasses.replace(cfg, gate_mode=PER_CHUNK), params, momenta, K, Q, V, th, et, al, ga)


def coefficient_form(cfg, params, momenta, K, V, th, et, al, ga, hist=None):
    """Chunk-wise closed form built on oracle.coefficients (coefficients written out as products):
    S_end = P S0 - sum_i oS_i g_i, W_end = beta W0 + a_S S0 - sum_i oW_i g_i, every g_i at the
    chunk-start weights, i over the chunk and the window - 1 tokens before it.  `hist` = (K, V,
    gamma) of the tokens before this call (oldest first), whose gammas reach the coefficients
    through omega_coefficients' gamma_hist; None = the start of a sequence."""
    from oracle.coefficients import chunk_coefficients, omega_coefficients
    W = [p.copy() for p in params]
    S = [m.copy() for m in momenta]
    X = phi_triu(K, cfg.poly_degree)
    T, C, c = K.shape[0], cfg.chunk, cfg.omega_window
    Xh = None if hist is None else phi_triu(hist[0], cfg.poly_degree)
    cW_all = np.zeros(T)
    cS_all = np.zeros(T)
    scal = []
    for s in range(0, T, C):
        cW_all[s:s + C], cS_all[s:s + C], sc = chunk_coefficients(th[s:s + C], et[s:s + C], al[s:s + C])
        scal.append(sc)
    oW, oS = omega_coefficients(cW_all, cS_all, ga if c > 1 else np.ones(T), C, c,
                                gamma_hist=None if hist is None else hist[2])
    for k, s in enumerate(range(0, T, C)):
        P, beta, aS = scal[k]
        GW = [np.zeros_like(x) for x in W]
        GS = [np.zeros_like(x) for x in W]
        for r in range(C + c - 1):
            i = s - (c - 1) + r
            if i < 0:
                if Xh is None or len(Xh) + i < 0:
                    continue
                g = oracle.loss_grad(W, Xh[len(Xh) + i], hist[1][len(Xh) + i])
            else:
                g = oracle.loss_grad(W, X[i], V[i])
            for m in range(len(W)):
                GW[m] += oW[k, r] * g[m]
                GS[m] += oS[k, r] * g[m]
        newS = [P * S[m] - GS[m] for m in range(len(W))]
        W = [beta * W[m] + aS * S[m] - GW[m] for m in range(len(W))]
        S = newS
    return W, S


def test_chunk_coefficients_backward_recursion():
    """The product form of the coefficients equals the backward recursion e_j = eta_{j+1} e_{j+1},
    b_j = (1 - alpha_{j+1}) b_{j+1}, w_j = b_j + eta_{j+1} w_{j+1} (w_C = b_C = e_C = 1)."""
    from oracle.coefficients import chunk_coefficients
    r = rng(21)
    C = 9
    th, et, al = r.uniform(.01, .1, C), r.uniform(.8, .99, C), r.uniform(0, .05, C)
    cW, cS, (P, beta, aS) = chunk_coefficients(th, et, al)
    e, b, w = np.ones(C), np.ones(C), np.ones(C)
    for j in range(C - 2, -1, -1):
        e[j] = e[j + 1] * et[j + 1]
        b[j] = b[j + 1] * (1 - al[j + 1])
        w[j] = b[j] + et[j + 1] * w[j + 1]
    np.testing.assert_allclose(cS, th * e, rtol=1e-14)
    np.testing.assert_allclose(cW, th * w, rtol=1e-14)
    np.testing.assert_allclose([P, beta, aS], [np.prod(et), np.prod(1 - al), et[0] * w[0]], rtol=1e-14)


@pytest.mark.parametrize("c", [1, 3, 6])
@pytest.mark.parametrize("kind", [LINEAR, MLP2_SILU])
def test_recurrence_matches_derived_coefficient_form(kind, c):
    cfg, params, momenta, K, Q, V, th, et, al, ga = tiny_problem(12, kind, 12, 3, 2, 4, 1, 4, c, PER_TOKEN)
    res = oracle.run_memory(cfg, params, momenta, K, Q, V, th, et, al, ga)
    W, S = coefficient_form(cfg, params, momenta, K, V, th, et, al, ga)
    for a, b in zip(res.params, W):
        assert maxrel(a, b) < 1e-12
    for a, b in zip(res.momenta, S):
        assert maxrel(a, b) < 1e-12


@pytest.mark.parametrize("c", [2, 4, 6])
def test_omega_coefficients_with_carried_gamma_history(c):
    """The coefficient form of a second call, whose window reaches back into the first call's last
    c - 1 tokens (their gammas through gamma_hist, oldest first), equals the literal recurrence run
    as two calls with the carried history.  An index slip in the gamma_hist branch (off by one, the
    newest gamma first, gamma taken as 1) moves W and S far beyond 1e-12."""
    T, T1 = 16, 8
    cfg, params, momenta, K, Q, V, th, et, al, ga = tiny_problem(40 + c, MLP2_SILU, T, 3, 2, 4, 1, 4, c, PER_TOKEN)
    a = oracle.run_memory(cfg, params, momenta, K[:T1], Q[:T1], V[:T1], th[:T1], et[:T1], al[:T1], ga[:T1])
    b = oracle.run_memory(cfg, a.params, a.momenta, K[T1:], Q[T1:], V[T1:], th[T1:], et[T1:], al[T1:], ga[T1:],
                          history=a.history)
    h0 = T1 - (c - 1)
    hist = (K[h0:T1], V[h0:T1], ga[h0:T1])
    W, S = coefficient_form(cfg, a.params, a.momenta, K[T1:], V[T1:], th[T1:], et[T1:], al[T1:], ga[T1:], hist=hist)
    for x, y in zip(b.params + b.momenta, W + S):
        assert maxrel(y, x) < 1e-12
    # the carried gammas matter: the same history rows with their gammas taken as 1, or the
    # window clipped at the call boundary, give a different state
    flipped = (hist[0], hist[1], np.ones(c - 1))
    Wf, _ = coefficient_form(cfg, a.params, a.momenta, K[T1:], V[T1:], th[T1:], et[T1:], al[T1:], ga[T1:],
                             hist=flipped)
    Wc, _ = coefficient_form(cfg, a.params, a.momenta, K[T1:], V[T1:], th[T1:], et[T1:], al[T1:], ga[T1:])
    assert maxrel(Wf[0], b.params[0]) > 1e-9
    assert maxrel(Wc[0], b.params[0]) > 1e-9


def test_omega_window_one_is_single_token_rule():
    """A window of 1 is the single-token rule: gamma is not used at all (bitwise)."""
    cfg, params, momenta, K, Q, V, th, et, al, ga = tiny_problem(13, MLP2_SILU, 12, 3, 2, 4, 2, 4, 1, PER_TOKEN)
    a = oracle.run_memory(cfg, params, momenta, K, Q, V, th, et, al, ga)
    b = oracle.run_memory(cfg, params, momenta, K, Q, V, th, et, al, None)
    assert np.array_equal(a.Y, b.Y)
    for x, y in zip(a.params + a.momenta, b.params + b.momenta):
        assert np.array_equal(x, y)


def test_streaming_equals_whole_sequence():
    """One call over T equals two calls over T1 and T - T1 (T1 a chunk multiple) with the window's
    history carried across the call boundary."""
    cfg, params, momenta, K, Q, V, th, et, al, ga = tiny_problem(14, MLP2_SILU, 16, 3, 2, 4, 2, 4, 4, PER_TOKEN)
    whole = oracle.run_memory(cfg, params, momenta, K, Q, V, th, et, al, ga)
    a = oracle.run_memory(cfg, params, momenta, K[:8], Q[:8], V[:8], th[:8], et[:8], al[:8], ga[:8])
    b = oracle.run_memory(cfg, a.params, a.momenta, K[8:], Q[8:], V[8:], th[8:], et[8:], al[8:], ga[8:],
                          history=a.history)
    assert np.array_equal(whole.Y, np.concatenate([a.Y, b.Y]))
    for x, y in zip(whole.params + whole.momenta, b.params + b.momenta):
        assert np.array_equal(x, y)
    # without the history the window would be clipped at the call boundary instead
    c = oracle.run_memory(cfg, a.params, a.momenta, K[8:], Q[8:], V[8:], th[8:], et[8:], al[8:], ga[8:])
    assert maxrel(c.params[0], b.params[0]) > 1e-9


def test_memories_are_independent():
    cfg, *_ = tiny_problem(15, MLP2_SILU, 8, 3, 2, 4, 1, 4, 1, PER_TOKEN)
    r = rng(15)
    M, T, P = 3, 8, 4 * 3 + 2 * 4
    W0 = r.normal(0, 0.5, (M, P))
    S0 = np.zeros((M, P))
    K, Q, V = r.normal(size=(M, T, 3)), r.normal(size=(M, T, 3)), r.normal(size=(M, T, 2))
    th, et, al = r.uniform(.01, .1, (M, T)), r.uniform(.8, .99, (M, T)), r.uniform(0, .05, (M, T))
    Y, W, S = oracle.run_many(cfg, W0, S0, K, Q, V, th, et, al)
    p = [2, 0, 1]
    Y2, W2, S2 = oracle.run_many(cfg, W0[p], S0[p], K[p], Q[p], V[p], th[p], et[p], al[p])
    assert np.array_equal(Y[p], Y2) and np.array_equal(W[p], W2) and np.array_equal(S[p], S2)


# ----------------------------------------------------------------------------- feature map


def test_poly_features_golden_d3():
    rows = [ln for ln in open(os.path.join(GOLDEN, "poly_features_d3.txt")) if not ln.startswith("#")]
    expected = np.array([float(t) for t in rows[0].split()])
    got = oracle.poly_features(np.array([[1.0, 2.0, 3.0]]), 2)[0]
    np.testing.assert_array_equal(got, expected)


@pytest.mark.parametrize("d,p", [(1, 2), (3, 2), (5, 3), (32, 2), (4, 1)])
def test_poly_feature_count_is_binomial(d, p):
    expect = d if p == 1 else math.comb(d + p, p)
    assert oracle.poly_feature_count(d, p) == expect
    assert oracle.poly_features(np.zeros((1, d)), p).shape == (1, expect)
    if (d, p) == (32, 2):
        assert expect == 561


def test_poly_features_inner_product_identity():
    """<phi(x), phi(y)> = 1 + x.y + ((x.y)^2 + sum_i x_i^2 y_i^2) / 8 for the degree-2 map with 1/2 on
    every pair i <= j (sum over i <= j of x_i x_j y_i y_j is half of (x.y)^2 + sum x_i^2 y_i^2)."""
    r = rng(16)
    x, y = r.normal(size=(5, 32)), r.normal(size=(5, 32))
    px, py = oracle.poly_features(x, 2), oracle.poly_features(y, 2)
    xy = np.sum(x * y, axis=1)
    ref = 1 + xy + (xy ** 2 + np.sum(x * x * y * y, axis=1)) / 8
    np.testing.assert_allclose(np.sum(px * py, axis=1), ref, rtol=1e-12)
    np.testing.assert_allclose(px, phi_triu(x, 2), rtol=0, atol=0)


def test_poly_features_of_basis_vector():
    """phi(e_i) has exactly three non-zero entries: 1 (constant), 1 (x_i) and 1/2 (x_i^2)."""
    d = 6
    for i in range(d):
        e = np.zeros((1, d))
        e[0, i] = 1
        f = oracle.poly_features(e, 2)[0]
        nz = np.flatnonzero(f)
        assert len(nz) == 3
        assert sorted(f[nz].tolist()) == [0.5, 1.0, 1.0]
        assert f[0] == 1.0 and f[1 + i] == 1.0


# ----------------------------------------------------------------------------- Newton-Schulz


@pytest.mark.parametrize("shape", [(64, 128), (128, 64), (5, 5), (3, 7)])
def test_newton_schulz_matches_svd_form(shape):
    G = rng(17).normal(size=shape)
    np.testing.assert_allclose(oracle.newton_schulz(G), ns5_svd(G), rtol=1e-10, atol=1e-12)


def test_newton_schulz_rank_one_scalar_map():
    """G = s u v^T (unit u, v): NS5(G) = f^5(s / (s + eps)) u v^T with f(x) = a x + b x^3 + c x^5."""
    r = rng(18)
    u = r.normal(size=6)
    u /= np.linalg.norm(u)
    v = r.normal(size=9)
    v /= np.linalg.norm(v)
    s = 3.0
    x = s / (s + 1e-7)
    for _ in range(5):
        x = 3.4445 * x - 4.7750 * x ** 3 + 2.0315 * x ** 5
    np.testing.assert_allclose(oracle.newton_schulz(s * np.outer(u, v)), x * np.outer(u, v), rtol=1e-12)
    assert 0.6 < x < 0.8


def test_newton_schulz_equivariance_zero_and_transpose():
    r = rng(19)
    G = r.normal(size=(8, 12))
    U, _ = np.linalg.qr(r.normal(size=(8, 8)))
    Vm, _ = np.linalg.qr(r.normal(size=(12, 12)))
    np.testing.assert_allclose(oracle.newton_schulz(U @ G @ Vm), U @ oracle.newton_schulz(G) @ Vm,
                               rtol=1e-10, atol=1e-12)
    np.testing.assert_allclose(oracle.newton_schulz(G.T), oracle.newton_schulz(G).T, rtol=1e-12, atol=1e-14)
    assert np.array_equal(oracle.newton_schulz(np.zeros((4, 6))), np.zeros((4, 6)))


# ----------------------------------------------------------------------------- workloads' health


def test_workload_health_literal_and_stabilised():
    """The generated workloads behave as recorded in the design notes: the linear workload stays
    bounded, the literal MLP workload 1 overflows within its first 8 chunks, its stabilised variant
    stays finite, and the Newton-Schulz workload stays O(1)."""
    from test_learned_neural_amd import synth
    inp = synth.make_inputs(0)
    _, W, _ = oracle.run_inputs(inp)
    assert np.isfinite(W).all() and 1.0 < np.abs(W).max() < 3.0
    with np.errstate(all="ignore"):
        inp = synth.make_inputs(1, batch=1, heads=1, T=640)
        cfg = oracle.config_from(inp.spec)
        r = oracle.run_memory(cfg, inp.split_params(inp.W0[0]), inp.split_params(inp.S0[0]),
                              inp.values("K")[0], inp.values("Q")[0], inp.values("V")[0],
                              inp.values("theta")[0], inp.values("eta")[0], inp.values("alpha")[0])
    assert not np.isfinite(r.max_abs_w[7])
    inp = synth.make_inputs(1, "stabilised", batch=1, heads=1, T=640)
    _, W, _ = oracle.run_inputs(inp)
    assert np.isfinite(W).all()
    inp = synth.make_inputs(4, batch=1, heads=1, T=2048)
    _, W, _ = oracle.run_inputs(inp)
    assert 0.1 < np.abs(W).max() < 2.0
