"""Pins of the prologue oracle (short convolution, L2 normalisation, gates) against things other
than itself: a hand-computed example from the definition, library routines (numpy convolve,
torch normalize, scipy expit), closed forms (identity and shift filters, zero weights) and
pure-Python brute force on tiny inputs."""

import os

import numpy as np
import pytest
import scipy.special
import torch

from oracle import prologue as pro

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _golden_conv():
    vals = {}
    for ln in open(os.path.join(GOLDEN, "short_conv_d1.txt")):
        if ln.startswith("#") or not ln.strip():
            continue
        k, *v = ln.split()
        vals[k] = np.array([float(x) for x in v])
    return vals


def test_conv_golden_by_hand():
    g = _golden_conv()
    x = g["x"][:, None]
    taps = g["taps"][None, :]
    assert np.array_equal(pro.short_conv(x, taps)[:, 0], g["out"])
    assert np.array_equal(pro.short_conv(x, taps, hist=g["hist"][:, None])[:, 0], g["out_hist"])


def test_conv_identity_and_shift_filters():
    r = np.random.default_rng(0)
    x = r.standard_normal((11, 5))
    ident = np.tile([0.0, 0.0, 0.0, 1.0], (5, 1))
    assert np.array_equal(pro.short_conv(x, ident), x)
    shift = np.tile([1.0, 0.0, 0.0, 0.0], (5, 1))
    y = pro.short_conv(x, shift)
    assert np.array_equal(y[:3], np.zeros((3, 5)))
    assert np.array_equal(y[3:], x[:-3])
    hist = r.standard_normal((3, 5))
    y = pro.short_conv(x, shift, hist=hist)
    assert np.array_equal(y[:3], hist)
    b = r.standard_normal(5)
    assert np.array_equal(pro.short_conv(x, ident, bias=b), x + b)


def test_conv_matches_numpy_convolve():
    r = np.random.default_rng(1)
    T, d = 37, 6
    x = r.standard_normal((T, d))
    taps = r.standard_normal((d, 4))
    hist = r.standard_normal((3, d))
    y = pro.short_conv(x, taps, hist=hist)
    for i in range(d):
        # np.convolve flips its second argument: the kernel k[s] multiplies x[t - s], so
        # k = taps reversed (k[0] on the current token, k[3] on token t - 3)
        full = np.convolve(np.concatenate([hist[:, i], x[:, i]]), taps[i][::-1])
        np.testing.assert_allclose(y[:, i], full[3:3 + T], rtol=1e-13, atol=1e-13)


@pytest.mark.parametrize("t1", [0, 1, 2, 3, 10])
def test_conv_streaming_equals_whole(t1):
    r = np.random.default_rng(2)
    x = r.standard_normal((17, 4))
    taps = r.standard_normal((4, 4))
    b = r.standard_normal(4)
    whole = pro.short_conv(x, taps, b)
    h = pro.conv_history(x[:t1])
    parts = np.concatenate([pro.short_conv(x[:t1], taps, b), pro.short_conv(x[t1:], taps, b, hist=h)])
    assert np.array_equal(whole, parts)
    # a second cut inside the first part, hist composed through a short call
    h1 = pro.conv_history(x[:1])
    h2 = pro.conv_history(x[1:t1 + 1], h1)
    np.testing.assert_array_equal(h2, pro.conv_history(x[:t1 + 1]))


def test_conv_empty_sequence():
    y = pro.short_conv(np.zeros((0, 3)), np.ones((3, 4)))
    assert y.shape == (0, 3)


def test_l2_normalise_matches_torch():
    r = np.random.default_rng(3)
    y = r.standard_normal((9, 7)) * r.uniform(0.1, 10, (9, 1))
    y[4] = 0.0
    ref = torch.nn.functional.normalize(torch.tensor(y), dim=-1, eps=1e-12).numpy()
    out = pro.l2_normalise(y)
    np.testing.assert_allclose(out, ref, rtol=1e-14, atol=1e-15)
    assert np.all(out[4] == 0.0)
    nrm = np.linalg.norm(np.delete(out, 4, axis=0), axis=1)
    np.testing.assert_allclose(nrm, 1.0, rtol=1e-14)


def test_conv_all_uses_head_filters():
    r = np.random.default_rng(4)
    B, H, T, d = 2, 3, 9, 4
    X = r.standard_normal((B * H, T, d))
    taps = r.standard_normal((H, d, 4))
    bias = r.standard_normal((H, d))
    hist = r.standard_normal((B * H, 3, d))
    out = pro.short_conv_all(X, taps, H, bias, hist, l2norm=True)
    for m in range(B * H):
        h = m % H
        full = np.concatenate([hist[m], X[m]])
        y = np.stack([bias[h] + sum(taps[h][:, j] * full[t + j] for j in range(4)) for t in range(T)])
        np.testing.assert_allclose(out[m], y / np.linalg.norm(y, axis=1, keepdims=True), rtol=1e-13)


@pytest.mark.parametrize("chunk,T", [(1, 7), (3, 7), (4, 8), (5, 3)])
def test_gates_bruteforce(chunk, T):
    r = np.random.default_rng(5)
    n_g, H, dm = 3, 2, 5
    U = r.standard_normal((T, dm))
    Wg = r.standard_normal((n_g, H, dm))
    bg = r.standard_normal((n_g, H))
    scale = np.array([0.1, 0.9, 0.01])
    got = pro.gates(U, Wg, bg, scale, chunk)
    ref = np.array(pro.gates_bruteforce(U.tolist(), Wg.tolist(), bg.tolist(), scale.tolist(), chunk))
    np.testing.assert_allclose(got, ref, rtol=1e-13, atol=1e-15)


def test_gates_zero_weights_and_library_sigmoid():
    r = np.random.default_rng(6)
    U = r.standard_normal((6, 4))
    bg = r.standard_normal((4, 3))
    scale = np.array([0.1, 0.9, 0.01, 1.0])
    got = pro.gates(U, np.zeros((4, 3, 4)), bg, scale)
    ref = scale[:, None, None] * scipy.special.expit(bg)[:, :, None] * np.ones((1, 1, 6))
    np.testing.assert_allclose(got, ref, rtol=1e-15)
    # at logit 0 every gate is half its maximum
    half = pro.gates(np.zeros((2, 4)), np.zeros((4, 3, 4)), np.zeros((4, 3)), scale)
    assert np.array_equal(half, np.broadcast_to(scale[:, None, None] / 2, half.shape))
    z = r.standard_normal(50) * 8
    np.testing.assert_allclose(pro.sigmoid(z), scipy.special.expit(z), rtol=1e-14)


def test_pooled_gate_is_gate_of_mean_input():
    r = np.random.default_rng(7)
    T, C, dm = 13, 4, 6
    U = r.standard_normal((T, dm))
    Wg = r.standard_normal((3, 2, dm))
    bg = r.standard_normal((3, 2))
    scale = np.array([0.1, 0.9, 0.01])
    got = pro.gates(U, Wg, bg, scale, C)
    means = np.stack([U[c * C:min((c + 1) * C, T)].mean(axis=0) for c in range(-(-T // C))])
    ref = pro.gates(means, Wg, bg, scale, 1)
    np.testing.assert_allclose(got, ref, rtol=1e-13)


def test_gates_all_layout():
    r = np.random.default_rng(8)
    B, T, dm, H = 2, 5, 3, 2
    U = r.standard_normal((B, T, dm))
    Wg = r.standard_normal((3, H, dm))
    bg = r.standard_normal((3, H))
    scale = np.array([0.1, 0.9, 0.01])
    out = pro.gates_all(U, Wg, bg, scale)
    assert out.shape == (3, B, H, T)
    for b in range(B):
        np.testing.assert_array_equal(out[:, b], pro.gates(U[b], Wg, bg, scale))


# ----------------------------------------------------------------------------- feature map stage

def test_feature_map_golden_degree3():
    rows = [ln for ln in open(os.path.join(GOLDEN, "feature_map_d2_deg3.txt")) if not ln.startswith("#")]
    ref = np.array([float(v) for v in rows[0].split()])
    got = pro.feature_map(np.array([[1.0, 2.0]]), 3)[0]
    np.testing.assert_allclose(got, ref, rtol=1e-15)


@pytest.mark.parametrize("d,p", [(3, 1), (5, 2), (4, 3), (32, 3)])
def test_feature_count_is_binomial(d, p):
    import math
    assert pro.feature_map(np.ones((1, d)), p).shape[1] == math.comb(d + p, p) == pro.feature_count(d, p)


def test_feature_map_degree2_equals_update_path_map():
    import oracle
    r = np.random.default_rng(9)
    x = r.standard_normal((5, 6))
    np.testing.assert_array_equal(pro.feature_map(x, 2), oracle.poly_features(x, 2))


@pytest.mark.parametrize("p", [1, 2, 3])
def test_feature_map_inner_product_closed_form(p):
    """<phi(x), phi(y)> = sum_k c_k^2 h_k(z), z_i = x_i y_i, with the complete homogeneous symmetric
    polynomials from the power sums P_k = sum z_i^k (Newton's identities): h_0 = 1, h_1 = P_1,
    h_2 = (P_1^2 + P_2) / 2, h_3 = (P_1^3 + 3 P_1 P_2 + 2 P_3) / 6."""
    r = np.random.default_rng(10 + p)
    x, y = r.standard_normal(7), r.standard_normal(7)
    c = r.uniform(0.2, 1.5, p + 1)
    z = x * y
    P1, P2, P3 = z.sum(), (z ** 2).sum(), (z ** 3).sum()
    h = [1.0, P1, (P1 ** 2 + P2) / 2, (P1 ** 3 + 3 * P1 * P2 + 2 * P3) / 6]
    ref = sum(c[k] ** 2 * h[k] for k in range(p + 1))
    fx, fy = pro.feature_map(x[None], p, c)[0], pro.feature_map(y[None], p, c)[0]
    np.testing.assert_allclose(fx @ fy, ref, rtol=1e-12)


def test_feature_map_basis_vector_and_projection():
    d, p = 4, 3
    c = [0.7, 1.1, 0.3, 0.2]
    f = pro.feature_map(np.eye(d)[2:3], p, c)[0]
    # e_2: the constant, x_2, x_2^2 and x_2^3 are the only non-zero monomials
    assert sorted(np.round(f[f != 0], 12).tolist()) == sorted([0.7, 1.1, 0.3, 0.2])
    r = np.random.default_rng(11)
    X = r.standard_normal((6, d))
    Pm = r.standard_normal((5, pro.feature_count(d, p)))
    F = pro.feature_map(X, p, c)
    np.testing.assert_allclose(pro.feature_map(X, p, c, Pm), np.einsum("nf,of->no", F, Pm), rtol=1e-13)
    assert np.array_equal(pro.feature_map(X, p, c, np.eye(F.shape[1])), F)
