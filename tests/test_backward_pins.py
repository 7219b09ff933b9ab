"""Pins of the outer-loop backward oracle: its torch restatement of the recurrence against the numpy
oracle, and its autograd gradients against central finite differences of the numpy oracle's
forward (independent of autograd), for every input group."""

import numpy as np
import pytest

import oracle
from oracle import LINEAR, MLP2_GATED, MLP2_SILU, MLP2_SILU_RESIDUAL, PER_CHUNK, PER_TOKEN, MemoryConfig
from oracle import backward as bw


def problem(seed, kind, T=8, C=4, d=3, v=2, h=5, mode=PER_TOKEN, ns=0, c=1, poly=1):
    r = np.random.default_rng(seed)
    din = oracle.poly_feature_count(d, poly)
    if kind == MLP2_SILU_RESIDUAL:
        v = din  # the residual memory adds its input (features) to its output
    cfg = MemoryConfig(kind, d, v, h if kind != LINEAR else 0, poly, C, c, mode, ns)
    if kind == LINEAR:
        params = [r.normal(0, 0.5, (v, din))]
    elif kind == MLP2_GATED:
        params = [r.normal(0, 0.5, (h, din)), r.normal(0, 0.5, (h, din)), r.normal(0, 0.5, (v, h))]
    else:
        params = [r.normal(0, 0.5, (h, din)), r.normal(0, 0.5, (v, h))]
    momenta = [r.normal(0, 0.1, p.shape) for p in params]
    K = r.normal(0, 1, (T, d)) / np.sqrt(d)
    Q = r.normal(0, 1, (T, d)) / np.sqrt(d)
    V = r.normal(0, 1, (T, v))
    ng = T if mode == PER_TOKEN else -(-T // C)
    th, et, al = r.uniform(0.01, 0.1, ng), r.uniform(0.8, 0.99, ng), r.uniform(0.0, 0.05, ng)
    dY = r.normal(size=(T, v))
    dW = [r.normal(size=p.shape) for p in params]
    dS = [r.normal(size=p.shape) for p in params]
    gm = r.uniform(0.2, 1.0, T) if c > 1 else None  # Omega-rule context gates
    return cfg, params, momenta, K, Q, V, th, et, al, dY, dW, dS, gm


def objective(cfg, params, momenta, K, Q, V, th, et, al, dY, dW, dS, gm=None):
    res = oracle.run_memory(cfg, params, momenta, K, Q, V, th, et, al, gm)
    return (np.sum(res.Y * dY) + sum(np.sum(a * b) for a, b in zip(res.params, dW))
            + sum(np.sum(a * b) for a, b in zip(res.momenta, dS)))


# (kind, gate mode, Newton-Schulz steps, Omega window, feature degree)
MODES = [(LINEAR, PER_TOKEN, 0, 1, 1), (MLP2_SILU, PER_TOKEN, 0, 1, 1), (MLP2_SILU, PER_CHUNK, 0, 1, 1),
         (MLP2_SILU, PER_CHUNK, 5, 1, 1), (LINEAR, PER_CHUNK, 5, 1, 1), (MLP2_SILU_RESIDUAL, PER_TOKEN, 0, 1, 1),
         (MLP2_SILU_RESIDUAL, PER_CHUNK, 5, 1, 1), (MLP2_SILU, PER_TOKEN, 0, 3, 1),
         (MLP2_SILU_RESIDUAL, PER_TOKEN, 0, 2, 1), (LINEAR, PER_TOKEN, 0, 3, 1), (MLP2_SILU, PER_TOKEN, 0, 6, 1),
         (MLP2_SILU, PER_TOKEN, 0, 3, 2), (MLP2_SILU, PER_TOKEN, 0, 1, 2), (MLP2_SILU_RESIDUAL, PER_TOKEN, 0, 2, 2),
         (MLP2_GATED, PER_TOKEN, 0, 1, 1), (MLP2_GATED, PER_TOKEN, 0, 3, 2), (MLP2_GATED, PER_CHUNK, 5, 1, 1)]


@pytest.mark.parametrize("kind,mode,ns,c,poly", MODES)
def test_torch_restatement_matches_oracle(kind, mode, ns, c, poly):
    import torch
    cfg, params, momenta, K, Q, V, th, et, al, _, _, _, gm = problem(1, kind, T=10, C=4, h=6, mode=mode, ns=ns, c=c,
                                                                     poly=poly)
    ref = oracle.run_memory(cfg, params, momenta, K, Q, V, th, et, al, gm)
    t = lambda a: torch.tensor(np.asarray(a, dtype=np.float64))
    Y, W, S = bw.run_memory_torch(cfg, [t(p) for p in params], [t(m) for m in momenta], t(K), t(Q), t(V), t(th),
                                  t(et), t(al), None if gm is None else t(gm))
    np.testing.assert_allclose(Y.numpy(), ref.Y, rtol=1e-13, atol=1e-14)
    for a, b in zip(W, ref.params):
        np.testing.assert_allclose(a.numpy(), b, rtol=1e-13, atol=1e-14)
    for a, b in zip(S, ref.momenta):
        np.testing.assert_allclose(a.numpy(), b, rtol=1e-13, atol=1e-14)


@pytest.mark.parametrize("kind,mode,ns,c,poly", MODES)
def test_outer_gradients_against_finite_differences(kind, mode, ns, c, poly):
    """<grad, delta> against (L(x + h delta) - L(x - h delta)) / 2h with L from the numpy oracle,
    for a random direction in every input group (a wrong sign, index or dropped term in any
    group changes its directional derivative)."""
    cfg, params, momenta, K, Q, V, th, et, al, dY, dW, dS, gm = problem(2, kind, T=9, C=4, h=6, mode=mode, ns=ns,
                                                                        c=c, poly=poly)
    g = bw.outer_grads(cfg, params, momenta, K, Q, V, th, et, al, dY, dW, dS, gamma=gm)
    r = np.random.default_rng(3)
    args = dict(params=params, momenta=momenta, K=K, Q=Q, V=V, th=th, et=et, al=al, gm=gm)
    groups = [("K", "K"), ("Q", "Q"), ("V", "V"), ("theta", "th"), ("eta", "et"), ("alpha", "al")]
    if c > 1:
        groups.append(("gamma", "gm"))
    hstep = 1e-6
    for gname, aname in groups:
        d = r.normal(size=np.shape(args[aname]))
        plus = dict(args)
        minus = dict(args)
        plus[aname] = args[aname] + hstep * d
        minus[aname] = args[aname] - hstep * d
        fd = (objective(cfg, **plus, dY=dY, dW=dW, dS=dS) - objective(cfg, **minus, dY=dY, dW=dW, dS=dS)) / (2 * hstep)
        an = float(np.sum(g[gname] * d))
        assert abs(fd - an) <= 1e-6 * max(1.0, abs(an)), (gname, fd, an)
    for gname, aname in (("W0", "params"), ("S0", "momenta")):
        ds = [r.normal(size=p.shape) for p in args[aname]]
        plus = dict(args)
        minus = dict(args)
        plus[aname] = [p + hstep * dd for p, dd in zip(args[aname], ds)]
        minus[aname] = [p - hstep * dd for p, dd in zip(args[aname], ds)]
        fd = (objective(cfg, **plus, dY=dY, dW=dW, dS=dS) - objective(cfg, **minus, dY=dY, dW=dW, dS=dS)) / (2 * hstep)
        an = float(sum(np.sum(a * b) for a, b in zip(g[gname], ds)))
        assert abs(fd - an) <= 1e-6 * max(1.0, abs(an)), (gname, fd, an)


def test_zero_adjoints_give_zero_gradients():
    cfg, params, momenta, K, Q, V, th, et, al, dY, dW, dS, _ = problem(4, MLP2_SILU)
    g = bw.outer_grads(cfg, params, momenta, K, Q, V, th, et, al, np.zeros_like(dY))
    for k in ("K", "Q", "V", "theta", "eta", "alpha"):
        assert not np.any(g[k])
