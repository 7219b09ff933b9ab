"""GPU tests of the stand-alone stages (gate scan, Omega coefficients, feature map,
Newton-Schulz) against their fp64 definitions in the oracle, through the C ABI."""

import math

import numpy as np
import pytest

import oracle
from helpers import log, maxrel, to_dev
from oracle.coefficients import omega_coefficients, sequence_coefficients
from test_learned_neural_amd import atlasmem as am
from test_learned_neural_amd import synth

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


@pytest.mark.parametrize("M,T,C", [(3, 192, 64), (2, 300, 100), (1, 256, 1), (2, 384, 128), (1, 130, 130)])
def test_gate_scan(M, T, C):
    import torch
    r = np.random.default_rng(M * 1000 + T + C)
    th = r.uniform(.01, .1, (M, T)).astype(np.float32)
    et = r.uniform(.8, .99, (M, T)).astype(np.float32)
    al = r.uniform(0, .05, (M, T)).astype(np.float32)
    cW = torch.empty((M, T), device=DEV)
    cS = torch.empty((M, T), device=DEV)
    sc = torch.empty((M, T // C, 3), device=DEV)
    am.gate_scan(to_dev(th), to_dev(et), to_dev(al), M, T, C, cW, cS, sc)
    for m in range(M):
        rW, rS, rsc = sequence_coefficients(th[m].astype(np.float64), et[m].astype(np.float64),
                                            al[m].astype(np.float64), C)
        e = (maxrel(cW[m].cpu().numpy(), rW), maxrel(cS[m].cpu().numpy(), rS), maxrel(sc[m].cpu().numpy(), rsc))
        log(f"PARITY gate_scan M={M} T={T} C={C} m={m}: cW={e[0]:.2e} cS={e[1]:.2e} scalars={e[2]:.2e}")
        assert max(e) < 1e-5


@pytest.mark.parametrize("T,C,c,hist", [(192, 64, 4, True), (192, 64, 4, False), (40, 4, 7, True), (64, 64, 1, False)])
def test_omega_coeffs(T, C, c, hist):
    import torch
    M = 2
    r = np.random.default_rng(T + C + c)
    cWv = r.uniform(0, 1, (M, T)).astype(np.float32)
    cSv = r.uniform(0, 1, (M, T)).astype(np.float32)
    ga = r.uniform(0, 1, (M, T)).astype(np.float32)
    gh = r.uniform(0, 1, (M, max(c - 1, 1))).astype(np.float32) if hist else None
    R = C + c - 1
    oW = torch.empty((M, T // C, R), device=DEV)
    oS = torch.empty((M, T // C, R), device=DEV)
    am.omega_coeffs(to_dev(cWv), to_dev(cSv), to_dev(ga), None if gh is None else to_dev(gh), M, T, C, c, oW, oS)
    for m in range(M):
        rW, rS = omega_coefficients(cWv[m].astype(np.float64), cSv[m].astype(np.float64), ga[m].astype(np.float64),
                                    C, c, None if gh is None else gh[m].astype(np.float64))
        e = max(maxrel(oW[m].cpu().numpy(), rW), maxrel(oS[m].cpu().numpy(), rS))
        log(f"PARITY omega T={T} C={C} c={c} hist={hist} m={m}: {e:.2e}")
        assert e < 1e-6


@pytest.mark.parametrize("n,d,dtype,shift", [(1000, 32, synth.BF16, 0), (37, 5, synth.F32, 0), (3, 1, synth.BF16, 0),
                                             (130, 64, synth.F32, 0), (45, 7, synth.F32, 1), (70, 200, synth.BF16, 0),
                                             (33, 200, synth.F32, 3)],
                         ids=["d32", "d5", "d1", "d64", "ragged_misaligned", "wide_no_table", "wide_misaligned"])
def test_poly_features_exact(n, d, dtype, shift):
    """The feature map against the oracle's, exact for bf16 inputs; also with an output that is not
    16-byte aligned (shift floats into the buffer) and for widths whose pair table exceeds LDS."""
    import torch
    r = np.random.default_rng(n + d)
    x32 = r.normal(size=(n, d)).astype(np.float32)
    xin = synth.f32_to_bf16_bits(x32) if dtype == synth.BF16 else x32
    xv = synth.bf16_bits_to_f32(xin).astype(np.float64) if dtype == synth.BF16 else x32.astype(np.float64)
    nf = math.comb(d + 2, 2)
    buf = torch.full((n * nf + shift,), float("nan"), device=DEV)
    F = buf[shift:].view(n, nf)
    am.poly_features(to_dev(xin), dtype, n, d, F)
    ref = oracle.poly_features(xv, 2)
    got = F.cpu().numpy().astype(np.float64)
    if dtype == synth.BF16:
        assert np.array_equal(got, ref)          # every monomial of bf16 inputs is exact in fp32
    else:
        assert maxrel(got, ref) < 1e-6


@pytest.mark.parametrize("rows,cols,prec,tol", [(64, 128, am.PREC_BF16X3, 1e-3), (128, 64, am.PREC_BF16X3, 1e-3),
                                                 (24, 56, am.PREC_BF16X3, 1e-3), (5, 3, am.PREC_BF16X3, 1e-3),
                                                 (64, 128, am.PREC_BF16, 1e-1)])
def test_newton_schulz(rows, cols, prec, tol):
    import torch
    n = 6
    r = np.random.default_rng(rows * cols)
    G = r.normal(size=(n, rows, cols)).astype(np.float32)
    G[1] *= 1e-3
    G[2] = np.outer(r.normal(size=rows), r.normal(size=cols))   # rank one
    G[3] = 0.0
    out = torch.empty((n, rows, cols), device=DEV)
    am.newton_schulz(to_dev(G), n, rows, cols, 5, synth.NS_COEFFS, synth.NS_EPS, prec, out)
    got = out.cpu().numpy().astype(np.float64)
    for i in range(n):
        ref = oracle.newton_schulz(G[i].astype(np.float64), 5, synth.NS_COEFFS, synth.NS_EPS)
        e = maxrel(got[i], ref)
        log(f"PARITY ns {rows}x{cols} prec={prec} mat={i}: {e:.2e} (tol {tol:g})")
        assert e <= tol
    assert np.array_equal(got[3], np.zeros((rows, cols)))
