"""GPU parity of the memory variants against the fp64 oracle, through the C ABI.

The residual 2-layer memory M(x) = x + W2 silu(W1 x) (ATLAS's default memory) runs the general
MLP path with its input added in the prediction and retrieval epilogues.  Tolerances as for the
plain memory: max |x - r| / max |r| per tensor within 2e-2 for bf16 inputs.
"""

import numpy as np
import pytest

from helpers import BF16_TOL, DEV, F32_TOL, compare, config_for, log, maxrel, oracle_run, run_gpu, segment, to_dev
from test_learned_neural_amd import atlasmem as am
from test_learned_neural_amd import synth

pytestmark = pytest.mark.gpu

R = synth.MLP2_SILU_RESIDUAL

RESIDUAL = [
    # (name, workload, variant, overrides, call boundaries or None)
    ("mlp64_T256", 1, "stabilised", dict(kind=R, batch=1, heads=4, T=256), None),
    ("window3_d40_history_rows", 3, "stabilised",
     dict(kind=R, batch=1, heads=3, T=144, d_key=40, poly_degree=1, d_value=40, d_hidden=72, chunk=48,
          omega_window=3), [0, 48, 96, 144]),
    ("poly2_d4_to_15_window2", 3, "stabilised",
     dict(kind=R, batch=2, heads=1, T=96, d_key=4, d_value=15, d_hidden=24, chunk=24, omega_window=2), None),
    ("ns5_per_chunk_fused", 4, "literal", dict(kind=R, batch=1, heads=3, T=512), None),
    ("ns5_fused_streamed", 4, "literal", dict(kind=R, batch=1, heads=2, T=512), [0, 1, 2, 130, 256, 300, 512]),
    ("streamed_uneven_calls", 1, "stabilised", dict(kind=R, batch=1, heads=2, T=192),
     [0, 1, 2, 3, 70, 71, 150, 192]),
]


@pytest.mark.parametrize("case", RESIDUAL, ids=[c[0] for c in RESIDUAL])
def test_residual_memory_parity(case):
    name, idx, variant, ov, splits = case
    log(f"CASE residual {name}")
    inp = synth.make_inputs(idx, variant, **ov)
    got = run_gpu(inp, splits=splits)
    ref = oracle_run(inp)
    errs = compare(f"residual_{name}", inp.spec, got, ref, BF16_TOL)
    assert got[3] == am.OK
    assert all(v <= BF16_TOL for v in errs.values()), errs


@pytest.mark.parametrize("out", ["f32", "bf16"])
def test_residual_fused_matches_general(out):
    """The fused kernel's residual variant (key values in the error, query values added to the
    output afterwards) against the general per-chunk path on the same inputs, and both against
    the oracle.  bf16 output runs the general path either way (one rounding of q + Yh)."""
    log(f"CASE residual fused vs general ({out})")
    inp = synth.make_inputs(4, "literal", kind=R, batch=1, heads=4, T=384)
    od = am.BF16 if out == "bf16" else am.F32
    fused = run_gpu(inp, output_dtype=od)
    general = run_gpu(inp, output_dtype=od, flags=am.FLAG_NO_FUSED)
    ref = oracle_run(inp)
    errs = compare(f"residual_fused_{out}", inp.spec, fused, ref, BF16_TOL)
    assert fused[3] == am.OK and general[3] == am.OK
    assert all(v <= BF16_TOL for v in errs.values()), errs
    agree = {k: maxrel(a, b) for k, a, b in zip(("Y", "W", "S"), fused[:3], general[:3])}
    log(f"PARITY residual fused vs general ({out}): " + " ".join(f"{k}={v:.3e}" for k, v in agree.items()))
    assert all(v <= 5e-4 for v in agree.values()), agree


def test_residual_retrieve_and_shape_error():
    """Retrieval alone adds the query's features too; a residual memory whose input width
    differs from its output width is refused."""
    import torch
    import oracle
    inp = synth.make_inputs(1, "stabilised", kind=R, batch=1, heads=2, T=64)
    s = inp.spec
    log("CASE residual_retrieve")
    mem = am.Memory(config_for(s), to_dev(inp.W0))
    seg = segment(inp, 0, 64)
    Y = torch.empty((s.n_mem, 64, s.d_value), dtype=torch.float32, device=DEV)
    mem.retrieve(seg["Q"], 64, Y)
    torch.cuda.synchronize()
    mem.close()
    cfg = oracle.config_from(s)
    Qf = synth.bf16_bits_to_f32(inp.Q).astype(np.float64) if s.input_dtype == synth.BF16 else inp.Q
    ref = np.stack([np.stack([oracle.memory_apply(oracle.unflatten(cfg, inp.W0[m]), Qf[m, t], True)
                              for t in range(64)]) for m in range(s.n_mem)])
    err = maxrel(Y.cpu().numpy(), ref)
    log(f"PARITY residual_retrieve: Y={err:.3e}")
    assert err <= BF16_TOL
    bad = synth.spec(1, "stabilised", kind=R, d_value=32)
    with pytest.raises(am.AtlasMemError) as e:
        am.Memory(config_for(bad))
    assert e.value.status == am.E_INVALID


G = synth.MLP2_GATED

GATED = [
    # (name, workload, variant, overrides, call boundaries or None)
    ("mlp64_T256", 1, "stabilised", dict(kind=G, batch=1, heads=4, T=256), None),
    ("window3_ragged_widths", 3, "stabilised",
     dict(kind=G, batch=1, heads=3, T=144, d_key=40, poly_degree=1, d_value=24, d_hidden=72, chunk=48,
          omega_window=3), [0, 48, 96, 144]),
    ("poly2_window2", 3, "stabilised",
     dict(kind=G, batch=2, heads=1, T=96, d_key=11, d_value=20, d_hidden=37, chunk=24, omega_window=2), None),
    ("ns5_per_chunk_three_matrices", 4, "literal", dict(kind=G, batch=1, heads=3, T=512), None),
    ("per_chunk_no_ns", 4, "literal", dict(kind=G, batch=1, heads=2, T=256, ns_steps=0), None),
    ("streamed_uneven_calls", 1, "stabilised", dict(kind=G, batch=1, heads=2, T=192),
     [0, 1, 2, 3, 70, 71, 150, 192]),
]


@pytest.mark.parametrize("case", GATED, ids=[c[0] for c in GATED])
def test_gated_memory_parity(case):
    name, idx, variant, ov, splits = case
    log(f"CASE gated {name}")
    inp = synth.make_inputs(idx, variant, **ov)
    got = run_gpu(inp, splits=splits)
    ref = oracle_run(inp)
    errs = compare(f"gated_{name}", inp.spec, got, ref, BF16_TOL)
    assert got[3] == am.OK
    assert all(v <= BF16_TOL for v in errs.values()), errs


def test_gated_retrieve():
    import torch
    import oracle
    inp = synth.make_inputs(1, "stabilised", kind=G, batch=1, heads=2, T=64)
    s = inp.spec
    log("CASE gated_retrieve")
    mem = am.Memory(config_for(s), to_dev(inp.W0))
    assert mem.P == s.param_count
    seg = segment(inp, 0, 64)
    Y = torch.empty((s.n_mem, 64, s.d_value), dtype=torch.float32, device=DEV)
    mem.retrieve(seg["Q"], 64, Y)
    torch.cuda.synchronize()
    mem.close()
    cfg = oracle.config_from(s)
    Qf = synth.bf16_bits_to_f32(inp.Q).astype(np.float64)
    ref = np.stack([np.stack([oracle.memory_apply(oracle.unflatten(cfg, inp.W0[m]), Qf[m, t])
                              for t in range(64)]) for m in range(s.n_mem)])
    err = maxrel(Y.cpu().numpy(), ref)
    log(f"PARITY gated_retrieve: Y={err:.3e}")
    assert err <= BF16_TOL


PTR = [
    # (name, workload, variant, overrides, call boundaries or None)
    ("linear_C4_w3", 0, "literal", dict(batch=2, heads=2, T=96, chunk=4, omega_window=3, d_key=20, d_value=12,
                                        per_token_retrieve=True), None),
    ("mlp64_T256", 1, "stabilised", dict(batch=1, heads=4, T=256, per_token_retrieve=True), [0, 64, 192, 256]),
    ("window3_ragged_widths", 3, "stabilised",
     dict(batch=1, heads=3, T=144, d_key=40, poly_degree=1, d_value=24, d_hidden=72, chunk=48, omega_window=3,
          per_token_retrieve=True), [0, 48, 144]),
    ("poly2_window4", 3, "stabilised", dict(batch=1, heads=2, T=192, per_token_retrieve=True), None),
    ("residual_window2", 3, "stabilised",
     dict(kind=R, batch=1, heads=2, T=96, d_key=24, poly_degree=1, d_value=24, d_hidden=40, chunk=32,
          omega_window=2, per_token_retrieve=True), None),
    ("gated_window3", 3, "stabilised",
     dict(kind=G, batch=1, heads=2, T=96, d_key=16, poly_degree=1, d_value=20, d_hidden=36, chunk=48,
          omega_window=3, per_token_retrieve=True), None),
    # a window wider than the coefficient kernel's register window (8): the token-by-token kernel
    ("window10_wide", 3, "stabilised",
     dict(batch=1, heads=2, T=96, d_key=16, poly_degree=1, d_value=16, d_hidden=32, chunk=32, omega_window=10,
          per_token_retrieve=True), [0, 32, 96]),
]


@pytest.mark.parametrize("case", PTR, ids=[c[0] for c in PTR])
def test_per_token_retrieve_parity(case):
    """Queries answered from the state right after their token's update, against the oracle."""
    name, idx, variant, ov, splits = case
    log(f"CASE per_token_retrieve {name}")
    inp = synth.make_inputs(idx, variant, **ov)
    tol = F32_TOL if inp.spec.kind == synth.LINEAR else BF16_TOL
    got = run_gpu(inp, splits=splits)
    ref = oracle_run(inp)
    errs = compare(f"ptr_{name}", inp.spec, got, ref, tol)
    assert got[3] == am.OK
    assert all(v <= tol for v in errs.values()), errs
    # the chunk-start answers of the same run are different (the test would not see a mix-up)
    import dataclasses
    base = dataclasses.replace(inp, spec=dataclasses.replace(inp.spec, per_token_retrieve=False))
    assert maxrel(oracle_run(base)[0], ref[0]) > 10 * tol


def test_per_token_retrieve_full_size_sampled():
    """The benchmark's per-token-retrieval shape (8 memories x 4096 tokens, 64 -> 128 -> 64, chunk
    64) in one call; the oracle recomputes two memories over the whole sequence, and every chunk's
    answers are compared on their own scale (the stabilised memory shrinks geometrically)."""
    from helpers import per_chunk_y_errors
    inp = synth.make_inputs(1, "stabilised", per_token_retrieve=True)
    s = inp.spec
    log(f"CASE per_token_retrieve full size {s.name}")
    got = run_gpu(inp)
    assert got[3] == am.OK
    mems = [2, 7]
    ref = oracle_run(inp, mems=mems)
    sub = tuple(x[mems] for x in got[:3])
    errs = compare("ptr_full_size_memories_2_7", s, sub, ref, BF16_TOL)
    assert all(v <= BF16_TOL for v in errs.values()), errs
    ey, counts, last = per_chunk_y_errors(sub[0], ref[0], s.chunk)
    log(f"PARITY ptr_full_size_per_chunk_Y: worst={ey:.3e} chunks checked={counts} last={last} of {s.T // s.chunk}")
    assert ey <= BF16_TOL and min(counts) >= 36  # the chunks above the floor: 39-40 of 64 for these memories


def test_per_token_retrieve_unsupported():
    s = synth.spec(4, "literal", batch=1, heads=1, T=256, per_token_retrieve=True)
    with pytest.raises(am.AtlasMemError) as e:
        am.Memory(config_for(s))
    assert e.value.status == am.E_UNSUPPORTED
    import torch
    # the linear memory answers per-token queries only for whole chunks
    inp = synth.make_inputs(0, "literal", batch=1, heads=1, T=10, chunk=4, per_token_retrieve=True)
    mem = am.Memory(config_for(inp.spec), to_dev(inp.W0))
    seg = segment(inp, 0, 10)
    Y = torch.empty((1, 10, inp.spec.d_value), dtype=torch.float32, device=DEV)
    with pytest.raises(am.AtlasMemError) as e:
        mem.update_chunked(seg["K"], seg["Q"], seg["V"], seg["theta"], seg["eta"], seg["alpha"], None, 10, Y)
    assert e.value.status == am.E_UNSUPPORTED
    assert mem.pending == 0
    mem.close()


PTR_STREAM = [
    # (name, workload, variant, overrides, call boundaries): one-token decoding and mixed calls
    ("mlp64_decode_then_calls", 1, "stabilised", dict(batch=1, heads=2, T=256, per_token_retrieve=True),
     [0, 1, 2, 3, 5, 64, 100, 128, 129, 200, 256]),
    ("window3_ragged_streamed", 3, "stabilised",
     dict(batch=1, heads=2, T=144, d_key=40, poly_degree=1, d_value=24, d_hidden=72, chunk=48, omega_window=3,
          per_token_retrieve=True), [0, 7, 40, 48, 49, 100, 144]),
    ("poly2_window4_streamed", 3, "stabilised", dict(batch=1, heads=2, T=192, per_token_retrieve=True),
     [0, 1, 33, 64, 65, 130, 192]),
    ("gated_streamed", 3, "stabilised",
     dict(kind=G, batch=1, heads=2, T=96, d_key=16, poly_degree=1, d_value=20, d_hidden=36, chunk=48,
          omega_window=3, per_token_retrieve=True), [0, 10, 11, 60, 96]),
    ("residual_streamed", 3, "stabilised",
     dict(kind=R, batch=1, heads=2, T=96, d_key=24, poly_degree=1, d_value=24, d_hidden=40, chunk=32,
          omega_window=2, per_token_retrieve=True), [0, 31, 33, 96]),
]


@pytest.mark.parametrize("case", PTR_STREAM, ids=[c[0] for c in PTR_STREAM])
def test_per_token_retrieve_streaming(case):
    """Queries of an unfinished chunk read the per-token states of its buffered rows: calls of any
    size (single tokens included) give one call's result, and the oracle's."""
    name, idx, variant, ov, splits = case
    inp = synth.make_inputs(idx, variant, **ov)
    log(f"CASE per-token retrieval streamed {name}")
    one = run_gpu(inp)
    streamed = run_gpu(inp, splits=splits)
    assert one[3] == am.OK and streamed[3] == am.OK
    agree = {k: maxrel(a, b) for k, a, b in zip(("Y", "W", "S"), streamed[:3], one[:3])}
    log(f"AGREE ptr_streamed_{name}: " + " ".join(f"{k}={v:.2e}" for k, v in agree.items()))
    assert all(v <= 1e-5 for v in agree.values()), agree
    ref = oracle_run(inp)
    errs = compare(f"ptr_streamed_{name}", inp.spec, streamed, ref, BF16_TOL)
    assert all(v <= BF16_TOL for v in errs.values()), errs
