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
