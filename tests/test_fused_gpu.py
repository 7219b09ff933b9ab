"""The fused whole-call kernel (64 -> 128 -> 64 MLP memory, per-chunk gates, Newton-Schulz) against
the fp64 oracle and against the general per-chunk kernel sequence, through the C ABI."""

import numpy as np
import pytest

from helpers import BF16_TOL, compare, handle_update_run, log, maxrel, oracle_run, run_gpu, static_update_run
from test_learned_neural_amd import atlasmem as am
from test_learned_neural_amd import synth

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("ov", [dict(batch=2, heads=4, T=512), dict(batch=1, heads=3, T=384, chunk=64),
                                dict(batch=1, heads=2, T=384, chunk=192), dict(batch=1, heads=2, T=384, chunk=96)],
                         ids=["C128", "C64", "C192", "C96_general"])
def test_fused_matches_oracle_and_general_path(ov):
    inp = synth.make_inputs(4, "literal", **ov)
    ref = oracle_run(inp)
    fused = run_gpu(inp)
    general = run_gpu(inp, flags=am.FLAG_NO_FUSED)
    e1 = compare(f"fused_{inp.spec.chunk}", inp.spec, fused, ref, BF16_TOL)
    e2 = compare(f"general_{inp.spec.chunk}", inp.spec, general, ref, BF16_TOL)
    assert fused[3] == am.OK and general[3] == am.OK
    assert all(v <= BF16_TOL for v in e1.values()), e1
    assert all(v <= BF16_TOL for v in e2.values()), e2
    d = max(maxrel(a, b) for a, b in zip(fused[:3], general[:3]))
    log(f"PARITY fused_vs_general_{inp.spec.chunk}: {d:.3e}")


def test_fused_streaming_and_no_retrieval():
    inp = synth.make_inputs(4, "literal", batch=1, heads=2, T=512)
    one = run_gpu(inp)
    parts = run_gpu(inp, splits=[0, 128, 384, 512])
    for a, b in zip(one[:3], parts[:3]):
        assert np.array_equal(a, b)
    no_y = run_gpu(inp, with_y=False)
    assert np.array_equal(no_y[1], one[1]) and np.array_equal(no_y[2], one[2])
    bf = run_gpu(inp, output_dtype=am.BF16)
    assert maxrel(bf[0], one[0]) < 8e-3


def test_fused_full_size_sampled():
    """The full workload (B=8, H=16, T=32768, chunk 128) in one call, as the benchmark runs it (the
    two-workgroup form: 256 workgroups, 2 x 256 waits per pair); the oracle recomputes two sampled
    memories over the whole sequence, and every memory equals the one-workgroup form (the
    allocation-free entry point) bit for bit."""
    inp = synth.make_inputs(4, "literal")
    got = run_gpu(inp)
    assert got[3] == am.OK
    one = static_update_run(inp)
    for name, a, b in zip(("Y", "W", "S"), got[:3], one):
        assert np.array_equal(a, b), (name, maxrel(a, b))
    del one
    mems = [5, 101]
    ref = oracle_run(inp, mems=mems)
    sub = (got[0][mems], got[1][mems], got[2][mems])
    errs = compare("fused_full_size_memories_5_101", inp.spec, sub, ref, BF16_TOL)
    assert all(v <= BF16_TOL for v in errs.values()), errs


@pytest.mark.parametrize("kind,ov", [
    (synth.MLP2_SILU, dict(batch=8, heads=16, T=640)),                 # 128 memories: every CU a set
    (synth.MLP2_SILU, dict(batch=1, heads=13, T=256, chunk=64)),       # pairs past the last memory exit
    (synth.MLP2_SILU, dict(batch=1, heads=2, T=512)),                  # four chunks, the shortest call
    (synth.MLP2_SILU_RESIDUAL, dict(batch=2, heads=5, T=768, chunk=192)),
], ids=["M128_C128", "M13_C64", "M2_four_chunks", "residual_M10_C192"])
def test_two_workgroup_form_equals_one_workgroup_form(kind, ov):
    """For up to 128 memories and calls of at least four chunks a handle runs each memory's two
    sets as two workgroups on different CUs, which exchange partial gradients and new weights
    through global memory; the allocation-free entry point runs one workgroup per memory with the
    same arithmetic.  The results agree bit for bit, and the handle reports no failed wait (the
    flag that get_state checks)."""
    inp = synth.make_inputs(4, "literal", kind=kind, **ov)
    log(f"CASE fused two-workgroup form: kind {kind} memories {inp.spec.n_mem} T {inp.spec.T} "
        f"chunk {inp.spec.chunk}")
    two = handle_update_run(inp)
    one = static_update_run(inp)
    for name, a, b in zip(("Y", "W", "S"), two, one):
        assert np.array_equal(a, b), (name, maxrel(a, b))


GATED_CASES = [
    # (name, overrides, call boundaries or None)
    ("M3_C128", dict(batch=1, heads=3, T=512), None),
    ("M13_C64_streamed", dict(batch=1, heads=13, T=320, chunk=64), [0, 64, 65, 192, 320]),
    ("M2_C192_one_chunk", dict(batch=1, heads=2, T=192, chunk=192), None),
]


@pytest.mark.parametrize("case", GATED_CASES, ids=[c[0] for c in GATED_CASES])
def test_gated_fused_matches_general_path_and_oracle(case):
    """The gated memory W2 (silu(W1 x) * (W3 x)) on the two-workgroup fused form (set 0 applies W1
    and W3, set 1 W2) against the general per-chunk sequence and the fp64 oracle."""
    name, ov, splits = case
    inp = synth.make_inputs(4, "literal", kind=synth.MLP2_GATED, **ov)
    log(f"CASE fused gated {name}")
    fused = run_gpu(inp, splits=splits)
    general = run_gpu(inp, splits=splits, flags=am.FLAG_NO_FUSED)
    assert fused[3] == am.OK and general[3] == am.OK
    ref = oracle_run(inp)
    e1 = compare(f"fused_gated_{name}", inp.spec, fused, ref, BF16_TOL)
    e2 = compare(f"general_gated_{name}", inp.spec, general, ref, BF16_TOL)
    assert all(v <= BF16_TOL for v in e1.values()), e1
    assert all(v <= BF16_TOL for v in e2.values()), e2
    d = max(maxrel(a, b) for a, b in zip(fused[:3], general[:3]))
    log(f"PARITY fused_gated_vs_general_{name}: {d:.3e}")
    assert d > 0.0  # different summation orders: the fused kernel ran


def test_gated_fused_benchmark_size_sampled():
    """128 memories x 4096 tokens of the gated memory (the benchmark's stage shape) in one call; the
    oracle recomputes two sampled memories over the whole sequence."""
    inp = synth.make_inputs(4, "literal", kind=synth.MLP2_GATED, T=4096)
    log("CASE fused gated 128 x 4096")
    got = run_gpu(inp)
    assert got[3] == am.OK
    mems = [3, 126]
    ref = oracle_run(inp, mems=mems)
    sub = (got[0][mems], got[1][mems], got[2][mems])
    errs = compare("fused_gated_128x4096_memories_3_126", inp.spec, sub, ref, BF16_TOL)
    assert all(v <= BF16_TOL for v in errs.values()), errs
