"""GPU parity of the HIP path against the fp64 oracle, through the C ABI.

Small sizes the oracle finishes in seconds, spanning several chunks and tiles, with
ragged widths (not multiples of the 64 x 64 GEMM tile or the 16-row MFMA block).
Tolerances: max |x - r| / max |r| per tensor within 2e-2 for bf16-input workloads and
1e-4 for the fp32 linear workload (Y, each weight matrix, each momentum matrix).
"""

import numpy as np
import pytest

import oracle
from helpers import BF16_TOL, F32_TOL, compare, config_for, log, oracle_run, run_gpu, segment, to_dev
from test_learned_neural_amd import atlasmem as am
from test_learned_neural_amd import synth

pytestmark = pytest.mark.gpu

SMALL = [
    # (name, workload, variant, overrides, tol)
    ("linear16_T256_C1", 0, "literal", dict(), F32_TOL),
    ("mlp64_stab_T256", 1, "stabilised", dict(T=256), BF16_TOL),
    ("mlp384_stab_T192", 2, "stabilised", dict(T=192), BF16_TOL),
    ("omega4_poly_stab_T192", 3, "stabilised", dict(batch=1, heads=4, T=192), BF16_TOL),
    ("ns5_mlp64_T512", 4, "literal", dict(batch=2, heads=4, T=512), BF16_TOL),
    # ragged widths / other chunk and window sizes
    ("mlp_ragged_C48_w3", 3, "stabilised", dict(batch=1, heads=3, T=144, d_key=40, poly_degree=1, d_value=24,
                                                d_hidden=72, chunk=48, omega_window=3), BF16_TOL),
    ("poly_ragged_C24_w2", 3, "stabilised", dict(batch=2, heads=1, T=96, d_key=11, d_value=20, d_hidden=37,
                                                 chunk=24, omega_window=2), BF16_TOL),
    ("perchunk_nons_ragged", 4, "literal", dict(batch=1, heads=3, T=200, d_key=40, d_value=24, d_hidden=56,
                                                 chunk=40, ns_steps=0), BF16_TOL),
    ("perchunk_ns_ragged", 4, "literal", dict(batch=1, heads=3, T=200, d_key=40, d_value=24, d_hidden=56,
                                               chunk=40), BF16_TOL),
    ("linear_C4_w3", 0, "literal", dict(batch=2, heads=2, T=96, chunk=4, omega_window=3, d_key=20, d_value=12),
     F32_TOL),
    ("linear_poly_C8", 0, "literal", dict(batch=1, heads=2, T=64, chunk=8, d_key=6, poly_degree=2, d_value=9,
                                          zero_init=False), F32_TOL),
    ("linear_perchunk_C16", 0, "literal", dict(batch=1, heads=2, T=128, chunk=16, gate_mode=synth.PER_CHUNK,
                                               d_key=32, d_value=32), F32_TOL),
]


@pytest.mark.parametrize("case", SMALL, ids=[c[0] for c in SMALL])
def test_parity_small(case):
    name, idx, variant, ov, tol = case
    log(f"CASE {name}")
    inp = synth.make_inputs(idx, variant, **ov)
    got = run_gpu(inp)
    ref = oracle_run(inp)
    errs = compare(name, inp.spec, got, ref, tol)
    assert got[3] == am.OK
    assert all(v <= tol for v in errs.values()), errs


def test_parity_bf16_output_and_no_retrieval():
    inp = synth.make_inputs(1, "stabilised", batch=1, heads=4, T=192)
    ref = oracle_run(inp)
    got = run_gpu(inp, output_dtype=am.BF16)
    errs = compare("mlp64_bf16_out", inp.spec, got, ref, BF16_TOL)
    assert all(v <= BF16_TOL for v in errs.values()), errs
    no_y = run_gpu(inp, with_y=False)
    assert np.array_equal(no_y[1], got[1]) and np.array_equal(no_y[2], got[2])


def test_streaming_equals_one_call():
    """One call over T equals calls over chunk-multiple pieces (window history carried): bitwise."""
    inp = synth.make_inputs(3, "stabilised", batch=1, heads=2, T=256)
    one = run_gpu(inp)
    parts = run_gpu(inp, splits=[0, 64, 192, 256])
    for a, b in zip(one[:3], parts[:3]):
        assert np.array_equal(a, b)
    inp = synth.make_inputs(0, "literal", batch=1, heads=1, T=96, chunk=4, omega_window=3, d_key=20, d_value=12)
    one = run_gpu(inp)
    parts = run_gpu(inp, splits=[0, 8, 96])
    for a, b in zip(one[:3], parts[:3]):
        assert np.array_equal(a, b)


def test_teacher_forced_literal_chunks_up_to_horizon():
    """The literal workload 1 overflows in fp64 within 8 chunks; up to that horizon each chunk is
    checked from the oracle's own chunk-start state (set_state), one chunk at a time."""
    import torch
    inp = synth.make_inputs(1, "literal", batch=1, heads=2, T=448)
    s = inp.spec
    cfg = oracle.config_from(s)
    refs = []
    with np.errstate(all="ignore"):
        for m in range(s.n_mem):
            refs.append(oracle.run_memory(cfg, inp.split_params(inp.W0[m]), inp.split_params(inp.S0[m]),
                                          inp.values("K")[m], inp.values("Q")[m], inp.values("V")[m],
                                          inp.values("theta")[m], inp.values("eta")[m], inp.values("alpha")[m],
                                          keep_boundaries=True))
    mem = am.Memory(config_for(s))
    checked = 0
    for k in range(s.T // s.chunk):
        Wk = np.stack([oracle.flatten(r.boundary_states[k][0]) for r in refs])
        Sk = np.stack([oracle.flatten(r.boundary_states[k][1]) for r in refs])
        W1 = np.stack([oracle.flatten(r.boundary_states[k + 1][0]) for r in refs])
        S1 = np.stack([oracle.flatten(r.boundary_states[k + 1][1]) for r in refs])
        Yr = np.stack([r.Y[k * s.chunk:(k + 1) * s.chunk] for r in refs])
        # the chunk is representable in fp32 only while its start state, outputs and end state are
        if not all(np.isfinite(a).all() and np.abs(a).max() < 1e30 for a in (Wk, Sk, W1, S1, Yr)):
            log(f"literal fp32 horizon reached at chunk {k}")
            break
        mem.set_state(to_dev(Wk.astype(np.float32)), to_dev(Sk.astype(np.float32)))
        seg = segment(inp, k * s.chunk, (k + 1) * s.chunk)
        y = torch.empty((s.n_mem, s.chunk, s.d_value), dtype=torch.float32, device="cuda:0")
        mem.update_chunked(seg["K"], seg["Q"], seg["V"], seg["theta"], seg["eta"], seg["alpha"], None, s.chunk, y)
        W = torch.empty((s.n_mem, mem.P), dtype=torch.float32, device="cuda:0")
        S = torch.empty_like(W)
        mem.get_state(W, S)
        errs = compare(f"literal_mlp64_chunk{k}", s, (y.cpu().numpy(), W.cpu().numpy(), S.cpu().numpy()),
                       (Yr, W1, S1), BF16_TOL)
        assert all(v <= BF16_TOL for v in errs.values()), errs
        checked += 1
    mem.close()
    assert checked >= 4


def test_nonfinite_state_is_reported():
    """Running the literal workload 1 past its overflow sets the non-finite flag; set_state clears it."""
    inp = synth.make_inputs(1, "literal", batch=1, heads=1, T=1024)
    got = run_gpu(inp)
    assert got[3] == am.E_NONFINITE


def test_retrieve_with_generator_weights():
    """retrieve() answers with the weights it holds and does not update them."""
    import torch
    for idx, var, ov in [(1, "stabilised", dict(batch=1, heads=3, T=300)),
                         (3, "stabilised", dict(batch=1, heads=2, T=130)),
                         (0, "literal", dict(batch=1, heads=2, T=70, zero_init=False))]:
        inp = synth.make_inputs(idx, var, **ov)
        s = inp.spec
        mem = am.Memory(config_for(s), to_dev(inp.W0), to_dev(inp.S0))
        Y = torch.empty((s.n_mem, s.T, s.d_value), dtype=torch.float32, device="cuda:0")
        mem.retrieve(to_dev(inp.Q), s.T, Y)
        W = torch.empty((s.n_mem, mem.P), dtype=torch.float32, device="cuda:0")
        mem.get_state(W)
        Qv = inp.values("Q")
        ref = np.stack([[oracle.memory_apply(inp.split_params(inp.W0[m]), x)
                         for x in oracle.poly_features(Qv[m], s.poly_degree)] for m in range(s.n_mem)])
        err = float(np.abs(Y.cpu().numpy() - ref).max() / np.abs(ref).max())
        tol = F32_TOL if s.input_dtype == synth.F32 else 1e-3
        log(f"PARITY retrieve_{s.name}: Y={err:.3e} (tol {tol:g})")
        assert err <= tol
        assert np.array_equal(W.cpu().numpy(), inp.W0)
        mem.close()


def test_argument_errors_on_device():
    """Bad arguments are reported as errors and change nothing; a call of fewer tokens than a
    chunk (or a non-multiple) is valid and leaves the tail pending."""
    import torch
    inp = synth.make_inputs(3, "stabilised", batch=1, heads=1, T=128)
    s = inp.spec
    mem = am.Memory(config_for(s))
    seg = segment(inp, 0, 128)
    with pytest.raises(am.AtlasMemError) as e:
        mem.update_chunked(seg["K"], seg["Q"], seg["V"], seg["theta"], seg["eta"], seg["alpha"], None, 100)
    assert e.value.status == am.E_INVALID
    with pytest.raises(am.AtlasMemError) as e:
        mem.update_chunked(seg["K"], seg["Q"], seg["V"], None, seg["eta"], seg["alpha"], seg["gamma"], 100)
    assert e.value.status == am.E_INVALID
    with pytest.raises(am.AtlasMemError) as e:
        mem.update_chunked(seg["K"], seg["Q"], seg["V"], seg["theta"], seg["eta"], seg["alpha"], seg["gamma"], -1)
    assert e.value.status == am.E_INVALID
    assert mem.pending == 0
    mem.update_chunked(seg["K"], seg["Q"], seg["V"], seg["theta"], seg["eta"], seg["alpha"], seg["gamma"], 0)
    assert mem.pending == 0
    mem.update_chunked(seg["K"], None, seg["V"], seg["theta"], seg["eta"], seg["alpha"], seg["gamma"], 100)
    assert mem.pending == 100 - s.chunk
    mem.flush()
    assert mem.pending == 0
    torch.cuda.synchronize()
    mem.close()

    # per-chunk gates: needed only by calls that complete a chunk, and by a flush
    inp = synth.make_inputs(4, "literal", batch=1, heads=2, T=256)
    s = inp.spec
    mem = am.Memory(config_for(s))
    seg = segment(inp, 0, 256)
    mem.update_chunked(seg["K"], None, seg["V"], None, None, None, None, 100)
    assert mem.pending == 100
    with pytest.raises(am.AtlasMemError) as e:
        mem.update_chunked(seg["K"], None, seg["V"], None, None, None, None, 100)
    assert e.value.status == am.E_INVALID
    assert mem.pending == 100
    with pytest.raises(am.AtlasMemError) as e:
        mem.flush()
    assert e.value.status == am.E_INVALID
    assert mem.pending == 100
    mem.reset_history()
    assert mem.pending == 0
    torch.cuda.synchronize()
    mem.close()
