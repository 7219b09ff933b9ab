"""The chunk-loop kernel (every chunk of a block in one launch, one workgroup per memory) against
the same update run as one launch per product and chunk, through the C ABI, and both against the
fp64 oracle.

Both paths compute the same products and epilogues, but the per-product launches split long-k
products into k-slices summed in another order, so the two agree to rounding: the check is a
1e-4 max relative difference per tensor (one bf16 ulp, 2^-8, for a bf16 output, where a rounding
difference can flip the last bit), far inside the 2e-2 bar both must meet against the oracle.  Cases cover
per-token gates (plain, residual and gated memories, Omega windows, degree-2 features, calls
that cut chunks), per-chunk gates without Newton-Schulz, bf16 output and update-only calls.
"""

import numpy as np
import pytest

from helpers import BF16_TOL, compare, log, maxrel, oracle_run, run_gpu
from test_learned_neural_amd import atlasmem as am
from test_learned_neural_amd import synth

pytestmark = pytest.mark.gpu

AGREE = 1e-4
AGREE_BF16_OUT = 2.0 ** -8

CASES = [
    # (name, workload, variant, overrides, call boundaries or None, output dtype, with Y)
    ("mlp64_per_token", 1, "stabilised", dict(T=512), None, am.F32, True),
    ("mlp64_streamed", 1, "stabilised", dict(batch=1, heads=3, T=320), [0, 1, 65, 130, 200, 320], am.F32, True),
    ("mlp64_bf16_out", 1, "stabilised", dict(batch=1, heads=2, T=256), None, am.BF16, True),
    ("mlp64_no_retrieval", 1, "stabilised", dict(batch=1, heads=2, T=256), None, am.F32, False),
    ("omega4_poly2", 3, "stabilised", dict(batch=1, heads=4, T=256), [0, 128, 256], am.F32, True),
    ("residual_window3", 3, "stabilised",
     dict(kind=synth.MLP2_SILU_RESIDUAL, batch=1, heads=3, T=144, d_key=40, poly_degree=1, d_value=40,
          d_hidden=72, chunk=48, omega_window=3), [0, 48, 96, 144], am.F32, True),
    ("gated_per_token", 1, "stabilised", dict(kind=synth.MLP2_GATED, batch=1, heads=2, T=256), None, am.F32, True),
    ("per_chunk_no_ns", 4, "literal", dict(batch=1, heads=3, T=512, ns_steps=0), None, am.F32, True),
]


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_chunk_loop_matches_per_product_launches(case):
    name, idx, variant, ov, splits, od, with_y = case
    log(f"CASE chunk loop {name}")
    inp = synth.make_inputs(idx, variant, **ov)
    # (the 64 -> 128 -> 64 per-token memory would take the fused kernel by default)
    loop = run_gpu(inp, splits=splits, output_dtype=od, with_y=with_y, flags=am.FLAG_NO_FUSED)
    launches = run_gpu(inp, splits=splits, output_dtype=od, with_y=with_y,
                       flags=am.FLAG_NO_CHUNK_LOOP | am.FLAG_NO_FUSED)
    assert loop[3] == am.OK and launches[3] == am.OK
    agree = {k: maxrel(a, b) for k, a, b in zip(("Y", "W", "S"), loop[:3], launches[:3]) if with_y or k != "Y"}
    bitwise = all(np.array_equal(a, b, equal_nan=True) for a, b in zip(loop[:3], launches[:3]))
    log(f"AGREE {name}: " + " ".join(f"{k}={v:.2e}" for k, v in agree.items()) + f" bitwise={bitwise}")
    bars = {k: (AGREE_BF16_OUT if (k == "Y" and od == am.BF16) else AGREE) for k in agree}
    assert all(agree[k] <= bars[k] for k in agree), agree
    ref = oracle_run(inp)
    errs = compare(f"chunk_loop_{name}", inp.spec, loop, ref, BF16_TOL, check_state=True)
    if not with_y:
        errs.pop("Y")
    assert all(v <= BF16_TOL for v in errs.values()), errs


SPLIT_CASES = [
    # (name, workload, variant, overrides, call boundaries or None)
    ("omega4_poly2_first_layer", 3, "stabilised", dict(batch=1, heads=4, T=256), [0, 128, 256]),
    ("wide_384x768", 2, "stabilised", dict(T=256), None),
    ("wide_residual_streamed", 2, "stabilised", dict(kind=synth.MLP2_SILU_RESIDUAL, batch=1, T=192), [0, 5, 64, 192]),
    ("wide_per_chunk_gates", 2, "stabilised", dict(batch=1, T=256, gate_mode=synth.PER_CHUNK, ns_steps=0), None),
]


@pytest.mark.parametrize("case", SPLIT_CASES, ids=[c[0] for c in SPLIT_CASES])
def test_split_k_matches_whole_k(case):
    """Products split into k-slices (partial tiles summed in slice order, then the epilogue)
    against the same products over the whole k range, and against the oracle."""
    name, idx, variant, ov, splits = case
    log(f"CASE split-K {name}")
    inp = synth.make_inputs(idx, variant, **ov)
    sk = run_gpu(inp, splits=splits)
    whole = run_gpu(inp, splits=splits, flags=am.FLAG_NO_SPLIT_K)
    assert sk[3] == am.OK and whole[3] == am.OK
    agree = {k: maxrel(a, b) for k, a, b in zip(("Y", "W", "S"), sk[:3], whole[:3])}
    log(f"AGREE {name}: " + " ".join(f"{k}={v:.2e}" for k, v in agree.items()))
    assert all(v <= AGREE for v in agree.values()), agree
    ref = oracle_run(inp)
    errs = compare(f"split_k_{name}", inp.spec, sk, ref, BF16_TOL)
    assert all(v <= BF16_TOL for v in errs.values()), errs


def test_in_workgroup_split_matches_whole_k():
    """Products of two to four k-steps with at least 128 output tiles split their k-steps over the
    groups of one workgroup (reduced in LDS) where split products are allowed.  256 memories with
    ragged widths on the per-product launches: the first-layer product over 40 key features (a
    32-step and an 8-wide step) and the gradient pairs over 72 key rows (two full steps and an
    8-wide one) take that form.  Against whole-k products (1e-4) and, on two memories, the oracle."""
    log("CASE in-workgroup k-split, 256 memories, ragged widths")
    inp = synth.make_inputs(1, "stabilised", batch=64, heads=4, T=144, chunk=72, d_key=40, d_value=20,
                            d_hidden=36)
    flags = am.FLAG_NO_FUSED | am.FLAG_NO_CHUNK_LOOP
    split = run_gpu(inp, flags=flags)
    whole = run_gpu(inp, flags=flags | am.FLAG_NO_SPLIT_K)
    assert split[3] == am.OK and whole[3] == am.OK
    agree = {k: maxrel(a, b) for k, a, b in zip(("Y", "W", "S"), split[:3], whole[:3])}
    log("AGREE kgroup: " + " ".join(f"{k}={v:.2e}" for k, v in agree.items()))
    assert all(v <= AGREE for v in agree.values()), agree
    assert max(agree.values()) > 0.0  # different summation orders: the split form ran
    mems = [0, 255]
    ref = oracle_run(inp, mems=mems)
    sub = (split[0][mems], split[1][mems], split[2][mems])
    errs = compare("kgroup_ragged", inp.spec, sub, ref, BF16_TOL)
    assert all(v <= BF16_TOL for v in errs.values()), errs


def test_chunk_loop_spans_coefficient_blocks():
    """A call longer than one block of gate coefficients: 2048 memories with chunk 16 give
    blocks of 61 chunks, so a 1024-token call runs blocks of 61 and 3 chunks (an odd first
    block flips the state buffers). The chunk loop against the per-product launches on every
    memory, and against the oracle on three memories."""
    log("CASE chunk loop over two coefficient blocks")
    inp = synth.make_inputs(1, "stabilised", batch=64, heads=32, T=1024, chunk=16, d_key=16, d_value=16,
                            d_hidden=32)
    loop = run_gpu(inp)
    launches = run_gpu(inp, flags=am.FLAG_NO_CHUNK_LOOP)
    assert loop[3] == am.OK and launches[3] == am.OK
    agree = {k: maxrel(a, b) for k, a, b in zip(("Y", "W", "S"), loop[:3], launches[:3])}
    log("AGREE blocks: " + " ".join(f"{k}={v:.2e}" for k, v in agree.items()))
    assert all(v <= AGREE for v in agree.values()), agree
    mems = [0, 1029, 2047]
    ref = oracle_run(inp, mems=mems)
    got = tuple(x[mems] for x in loop[:3])
    errs = compare("chunk_loop_blocks", inp.spec, got, ref, BF16_TOL)
    assert all(v <= BF16_TOL for v in errs.values()), errs
