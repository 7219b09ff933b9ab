"""Operand precision against the fp64 oracle.

The Newton-Schulz workload (64 -> 128 -> 64, chunk 128, per-chunk gates, 5 steps) names bf16
inputs but no key normalisation.  Two readings: keys L2-normalised (the default generator, which
the benchmark runs) and raw N(0, 1) keys.  The orthogonalisation feeds operand rounding back into
the state, about 30x with normalised keys and about 1000x with raw ones, so on raw keys the split
bf16 products (hi*hi + hi*lo + lo*hi) exceed the 2e-2 bar on W and S, while fp32 operands
(ATLASMEM_PREC_F32) hold it.  Both memories sampled here run the whole 32768-token sequence."""

import numpy as np
import pytest

from helpers import BF16_TOL, compare, log, oracle_run, run_gpu, run_gpu_states
from test_learned_neural_amd import atlasmem as am
from test_learned_neural_amd import synth

pytestmark = pytest.mark.gpu

MEMS = [5, 101]


@pytest.fixture(scope="module")
def raw_keys():
    inp = synth.make_inputs(4, "literal", norm_k=False)
    log(f"CASE raw keys {inp.spec.name} memories {MEMS}: oracle")
    return inp, oracle_run(inp, mems=MEMS)


def _one_call(inp, precision):
    Y, states = run_gpu_states(inp, MEMS, 1, inp.spec.T // inp.spec.chunk, precision=precision)
    W, S = states[-1]
    return Y, W, S


def test_raw_keys_full_length_f32(raw_keys):
    inp, ref = raw_keys
    got = _one_call(inp, am.PREC_F32)
    errs = compare("ns5_raw_keys_f32", inp.spec, got, ref, BF16_TOL)
    assert np.all(np.isfinite(got[0]))
    assert all(v <= BF16_TOL for v in errs.values()), errs


@pytest.mark.xfail(reason="split bf16 products on raw keys: Newton-Schulz amplifies their rounding about 1000x, "
                          "beyond the 2e-2 bar on W and S (PREC_F32 holds it)", strict=False)
def test_raw_keys_full_length_split_bf16_known_failure(raw_keys):
    inp, ref = raw_keys
    got = _one_call(inp, am.PREC_BF16X3)
    errs = compare("ns5_raw_keys_split_bf16", inp.spec, got, ref, BF16_TOL)
    assert all(v <= BF16_TOL for v in errs.values()), errs


@pytest.mark.parametrize("ov", [dict(batch=1, heads=2, T=512), dict(batch=1, heads=2, T=384, chunk=64)],
                         ids=["ns5_C128", "ns5_C64"])
def test_f32_matches_oracle_closely(ov):
    """fp32 operands track the fp64 oracle far inside the fp32 bar on short runs (normalised keys)."""
    inp = synth.make_inputs(4, "literal", **ov)
    ref = oracle_run(inp)
    got = run_gpu(inp, precision=am.PREC_F32)
    errs = compare(f"f32_{inp.spec.chunk}", inp.spec, got, ref, 1e-4)
    assert got[3] == am.OK
    assert all(v <= 1e-4 for v in errs.values()), errs


@pytest.mark.parametrize("index", [1, 3])
def test_f32_per_token_workloads(index):
    """fp32 operands on the per-token path: the 64 -> 128 -> 64 workload and the Omega window with
    degree-2 features, short prefixes, against the oracle at the fp32 bar."""
    inp = synth.make_inputs(index, "stabilised", batch=1, heads=2, T=256)
    ref = oracle_run(inp)
    got = run_gpu(inp, precision=am.PREC_F32)
    errs = compare(f"f32_workload_{index}", inp.spec, got, ref, 1e-4)
    assert got[3] == am.OK
    assert all(v <= 1e-4 for v in errs.values()), errs


def test_f32_newton_schulz_stage():
    """The stand-alone Newton-Schulz stage in fp32 against the oracle's iteration, both orientations."""
    import torch
    import oracle
    r = np.random.default_rng(3)
    for rows, cols in ((64, 128), (128, 64), (40, 72)):
        G = r.standard_normal((6, rows, cols)).astype(np.float32)
        g = torch.from_numpy(G).to("cuda:0")
        out = torch.empty_like(g)
        am.newton_schulz(g, 6, rows, cols, 5, synth.NS_COEFFS, synth.NS_EPS, am.PREC_F32, out)
        got = out.cpu().numpy().astype(np.float64)
        ref = np.stack([oracle.newton_schulz(G[i].astype(np.float64), 5, synth.NS_COEFFS, synth.NS_EPS)
                        for i in range(6)])
        e = float(np.max(np.abs(got - ref)) / np.max(np.abs(ref)))
        log(f"PARITY ns_f32_{rows}x{cols}: {e:.3e}")
        assert e <= 1e-4


@pytest.mark.xfail(reason="plain bf16 products (no lo terms) on the Newton-Schulz workload: the orthogonalisation "
                          "feeds their rounding back into the state, far beyond the 2e-2 bar; the split products hold it",
                   strict=False)
def test_plain_bf16_fused_full_length_known_failure():
    """The fused kernel with plain bf16 products (the benchmark's fast-mode line) over the whole
    sequence of two memories, normalised keys: recorded, not hidden."""
    inp = synth.make_inputs(4, "literal")
    ref = oracle_run(inp, mems=MEMS)
    got = _one_call(inp, am.PREC_BF16)
    assert np.all(np.isfinite(got[0]))
    errs = compare("ns5_plain_bf16_fused", inp.spec, got, ref, BF16_TOL)
    assert all(v <= BF16_TOL for v in errs.values()), errs
