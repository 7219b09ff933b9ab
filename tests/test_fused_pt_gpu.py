"""The fused kernel for per-token gates (64 -> 128 -> 64 MLP memory, chunks of 64, no Newton-Schulz:
the per-token workload's geometry) against the general path (the chunk-loop kernel) and the fp64
oracle, through the C ABI.

Both paths form the same coefficient-weighted gradient sums at the chunk-start weights, in different
summation orders, so they agree to rounding (1e-4 max relative difference per tensor; one bf16 ulp
for a bf16 output); each meets the 2e-2 bar against the oracle.  The full-size workload runs
through this kernel in test_fullsize_gpu (every chunk on its own scale)."""

import numpy as np
import pytest

from helpers import BF16_TOL, compare, log, maxrel, oracle_run, run_gpu
from test_learned_neural_amd import atlasmem as am
from test_learned_neural_amd import synth

pytestmark = pytest.mark.gpu

AGREE = 1e-4

CASES = [
    # (name, overrides, call boundaries or None, output dtype, with Y)
    ("plain_2x4_T512", dict(T=512), None, am.F32, True),
    ("streamed_calls", dict(batch=1, heads=3, T=320), [0, 1, 65, 130, 200, 320], am.F32, True),
    ("bf16_output", dict(batch=1, heads=2, T=256), None, am.BF16, True),
    ("no_retrieval", dict(batch=1, heads=2, T=256), None, am.F32, False),
    ("residual", dict(kind=synth.MLP2_SILU_RESIDUAL, batch=1, heads=2, T=256), None, am.F32, True),
    ("literal_gates_two_chunks", dict(batch=1, heads=2, T=128), None, am.F32, True),
]


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_fused_per_token_matches_general_path_and_oracle(case):
    name, ov, splits, od, with_y = case
    variant = "literal" if name.startswith("literal") else "stabilised"
    inp = synth.make_inputs(1, variant, **ov)
    log(f"CASE fused per-token {name}")
    fused = run_gpu(inp, splits=splits, output_dtype=od, with_y=with_y)
    general = run_gpu(inp, splits=splits, output_dtype=od, with_y=with_y, flags=am.FLAG_NO_FUSED)
    assert fused[3] == am.OK and general[3] == am.OK
    agree = {k: maxrel(a, b) for k, a, b in zip(("Y", "W", "S"), fused[:3], general[:3]) if with_y or k != "Y"}
    log(f"AGREE fused_pt_{name}: " + " ".join(f"{k}={v:.2e}" for k, v in agree.items()))
    bars = {k: (2.0 ** -8 if (k == "Y" and od == am.BF16) else AGREE) for k in agree}
    assert all(agree[k] <= bars[k] for k in agree), agree
    ref = oracle_run(inp)
    errs = compare(f"fused_pt_{name}", inp.spec, fused, ref, BF16_TOL)
    if not with_y:
        errs.pop("Y")
    assert all(v <= BF16_TOL for v in errs.values()), errs


def test_fused_per_token_spans_coefficient_blocks():
    """2048 memories: the gate coefficients of a call come in blocks of 15 chunks, so a 1024-token
    call runs the fused kernel over blocks of 15 and 1 chunks (an odd block flips the state
    buffers).  Every memory against the general path, three against the oracle."""
    inp = synth.make_inputs(1, "stabilised", batch=64, heads=32, T=1024)
    log("CASE fused per-token over two coefficient blocks")
    fused = run_gpu(inp)
    general = run_gpu(inp, flags=am.FLAG_NO_FUSED)
    agree = {k: maxrel(a, b) for k, a, b in zip(("Y", "W", "S"), fused[:3], general[:3])}
    log("AGREE fused_pt_blocks: " + " ".join(f"{k}={v:.2e}" for k, v in agree.items()))
    assert all(v <= AGREE for v in agree.values()), agree
    mems = [0, 1029, 2047]
    ref = oracle_run(inp, mems=mems)
    errs = compare("fused_pt_blocks", inp.spec, tuple(x[mems] for x in fused[:3]), ref, BF16_TOL)
    assert all(v <= BF16_TOL for v in errs.values()), errs
