"""The hidden-split chunk kernel (2-layer memory with per-token gates, an Omega window and features of
degree <= 2, each memory over d_hidden / 16 workgroups, one launch per chunk) against the general
path (per-product launches) and the fp64 oracle, through the C ABI.

Both paths form the same coefficient-weighted gradient sums at the chunk-start weights, in different
summation orders (the output product here is summed over the workgroups' 16-unit slices), so they
agree to rounding (1e-4 max relative difference per tensor; one bf16 ulp for a bf16 output); each
meets the 2e-2 bar against the oracle.  The full-size workload (4 x 8 memories, T = 8192) runs through
this kernel in test_fullsize_gpu, every chunk on its own scale."""

import pytest

from helpers import BF16_TOL, compare, log, maxrel, oracle_run, run_gpu
from test_learned_neural_amd import atlasmem as am
from test_learned_neural_amd import synth

pytestmark = pytest.mark.gpu

AGREE = 1e-4

CASES = [
    # (name, variant, overrides, call boundaries or None, output dtype, with Y)
    ("omega4_poly2_T192", "stabilised", dict(batch=1, heads=4, T=192), None, am.F32, True),
    ("streamed_calls", "stabilised", dict(batch=1, heads=3, T=320), [0, 1, 65, 130, 200, 320], am.F32, True),
    ("bf16_output", "stabilised", dict(batch=1, heads=2, T=256), None, am.BF16, True),
    ("no_retrieval", "stabilised", dict(batch=1, heads=2, T=256), None, am.F32, False),
    ("literal_gates", "literal", dict(batch=1, heads=2, T=128), None, am.F32, True),
    # degree 1 of bf16 inputs (exact features: no lo word on their side), 4 workgroups per memory
    ("poly1_exact_C48_w2", "stabilised", dict(batch=1, heads=3, T=240, d_key=64, poly_degree=1, d_hidden=64,
                                              d_value=32, chunk=48, omega_window=2), None, am.F32, True),
    # no window: the chunk coefficients themselves; 2 workgroups per memory, 153 features
    ("poly2_window1_C32", "stabilised", dict(batch=2, heads=1, T=160, d_key=16, d_hidden=32, chunk=32,
                                             omega_window=1), None, am.F32, True),
    # one workgroup per memory, 45 features, window 3 over chunks of 16
    ("one_workgroup_C16_w3", "stabilised", dict(batch=1, heads=2, T=96, d_key=8, d_hidden=16, d_value=32,
                                                chunk=16, omega_window=3), None, am.F32, True),
]


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_hsplit_matches_general_path_and_oracle(case):
    name, variant, ov, splits, od, with_y = case
    inp = synth.make_inputs(3, variant, **ov)
    log(f"CASE hsplit {name}")
    fast = run_gpu(inp, splits=splits, output_dtype=od, with_y=with_y)
    general = run_gpu(inp, splits=splits, output_dtype=od, with_y=with_y, flags=am.FLAG_NO_FUSED)
    assert fast[3] == am.OK and general[3] == am.OK
    agree = {k: maxrel(a, b) for k, a, b in zip(("Y", "W", "S"), fast[:3], general[:3]) if with_y or k != "Y"}
    log(f"AGREE hsplit_{name}: " + " ".join(f"{k}={v:.2e}" for k, v in agree.items()))
    bars = {k: (2.0 ** -8 if (k == "Y" and od == am.BF16) else AGREE) for k in agree}
    assert all(agree[k] <= bars[k] for k in agree), agree
    assert max(agree.values()) > 0.0  # different summation orders: the hidden-split kernel ran
    ref = oracle_run(inp)
    errs = compare(f"hsplit_{name}", inp.spec, fast, ref, BF16_TOL)
    if not with_y:
        errs.pop("Y")
    assert all(v <= BF16_TOL for v in errs.values()), errs


def test_hsplit_spans_coefficient_blocks():
    """2048 memories with chunks of 96: the gate coefficients of a call come in blocks of 10 chunks,
    so a 1056-token call runs the kernel over blocks of 10 and 1 chunks (nb + 1 launches each; an
    odd block flips the state buffers).  Every memory against the general path, two against the
    oracle.  561 features, 32 hidden units (two workgroups per memory), 32 outputs; the state stays
    well inside fp32's range (max |Y| falls from 0.1 to ~5e-12 over the 11 chunks)."""
    inp = synth.make_inputs(3, "stabilised", batch=256, heads=8, T=1056, d_hidden=32, d_value=32, chunk=96)
    log("CASE hsplit over two coefficient blocks")
    fast = run_gpu(inp)
    general = run_gpu(inp, flags=am.FLAG_NO_FUSED)
    agree = {k: maxrel(a, b) for k, a, b in zip(("Y", "W", "S"), fast[:3], general[:3])}
    log("AGREE hsplit_blocks: " + " ".join(f"{k}={v:.2e}" for k, v in agree.items()))
    assert all(v <= AGREE for v in agree.values()), agree
    assert max(agree.values()) > 0.0  # different summation orders: the hidden-split kernel ran
    mems = [0, 2047]
    ref = oracle_run(inp, mems=mems)
    sub = (fast[0][mems], fast[1][mems], fast[2][mems])
    errs = compare("hsplit_blocks", inp.spec, sub, ref, BF16_TOL)
    assert all(v <= BF16_TOL for v in errs.values()), errs
