"""The general path at the workloads' full sizes against the fp64 oracle, with every chunk checked on
its own scale (stabilised variants: the literal ones leave fp32's range, which the teacher-forced
tests in test_parity_gpu cover up to that point).

The stabilised workloads' state shrinks geometrically (without biases W = 0 attracts under the
forgetting gate), so a tensor-wide relative error is set by the first chunks alone.  Each test here
therefore also scales every chunk's retrieved rows, and the weights and momenta at many chunk
boundaries (read with get_state between update calls), by their own reference magnitude, down to
helpers.FLOOR."""

import numpy as np
import pytest

from helpers import (BF16_TOL, FLOOR, boundary_state_errors, compare, log, oracle_boundaries, oracle_run,
                     per_chunk_y_errors, run_gpu, run_gpu_states)
from test_learned_neural_amd import atlasmem as am
from test_learned_neural_amd import synth

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("index", [1, 2])
def test_full_size_all_memories(index):
    """Every memory of the 64 -> 128 -> 64 (2 x 4 x 4096) and 384 -> 768 -> 384 (2 x 1 x 1024)
    workloads over the whole sequence in one call: tensor-wide errors and every chunk's Y on its own
    scale."""
    inp = synth.make_inputs(index, "stabilised")
    s = inp.spec
    log(f"CASE full_size workload {index} {s.name}")
    ref = oracle_run(inp)
    got = run_gpu(inp)
    assert got[3] == am.OK
    errs = compare(f"full_size_{index}", s, got, ref, BF16_TOL)
    assert all(v <= BF16_TOL for v in errs.values()), errs
    ey, counts, last = per_chunk_y_errors(got[0], ref[0], s.chunk)
    log(f"PARITY full_size_{index}_per_chunk_Y: worst={ey:.3e} chunks checked per memory={counts} "
        f"last chunk checked={last} of {s.T // s.chunk} (floor {FLOOR:g})")
    assert ey <= BF16_TOL
    assert min(counts) >= (40 if index == 1 else s.T // s.chunk)


@pytest.mark.parametrize("index,mems,calls,per_call", [(1, [0, 5], 16, 4), (2, [0, 1], 8, 2)])
def test_full_size_state_at_chunk_boundaries(index, mems, calls, per_call):
    """The 64 -> 128 -> 64 and 384 -> 768 -> 384 workloads fed in calls of a few chunks, with W1, W2,
    S1, S2 read after every call and each compared on its own scale with the oracle's state at that
    chunk boundary (16 and 8 boundaries), and every chunk's Y likewise."""
    inp = synth.make_inputs(index, "stabilised")
    s = inp.spec
    log(f"CASE boundaries workload {index} {s.name} memories {mems}")
    refs = oracle_boundaries(inp, mems)
    Yg, states = run_gpu_states(inp, mems, calls, per_call)
    ids = [(j + 1) * per_call for j in range(calls)]
    worst, last = 0.0, []
    for i in range(len(mems)):
        e, lk = boundary_state_errors(s, [(W[i], S[i]) for W, S in states], refs[i][1], ids)
        worst = max(worst, e)
        last.append(lk)
    ey, counts, ylast = per_chunk_y_errors(Yg, np.stack([r[0] for r in refs]), s.chunk)
    log(f"PARITY boundaries_{index}: state worst={worst:.3e} last boundary checked={last}; "
        f"per-chunk Y worst={ey:.3e} chunks checked={counts}")
    assert worst <= BF16_TOL and ey <= BF16_TOL
    assert min(last) == ids[-1]           # every boundary, to the end of the sequence


def test_full_size_omega_poly_per_chunk():
    """Polynomial keys (32 -> 561) with the Omega window 4, two sampled memories of the 4 x 8 x 8192
    workload fed in 16 calls of 8 chunks: every chunk's Y and the state at each call boundary, each on
    its own scale, down to the floor (with these gates the memory shrinks below it after about 50 of
    the 128 chunks; the window history crosses every call boundary)."""
    inp = synth.make_inputs(3, "stabilised")
    s = inp.spec
    mems = [3, 26]
    log(f"CASE full_size workload 3 {s.name} memories {mems}")
    refs = oracle_boundaries(inp, mems)
    calls, per_call = 16, 8
    Yg, states = run_gpu_states(inp, mems, calls, per_call)
    assert np.all(np.isfinite(Yg))
    ids = [(j + 1) * per_call for j in range(calls)]
    worst, last = 0.0, []
    for i in range(len(mems)):
        e, lk = boundary_state_errors(s, [(W[i], S[i]) for W, S in states], refs[i][1], ids)
        worst = max(worst, e)
        last.append(lk)
    Yr = np.stack([r[0] for r in refs])
    ey, counts, ylast = per_chunk_y_errors(Yg, Yr, s.chunk)
    log(f"PARITY full_size_3: state worst={worst:.3e} last boundary checked={last}; per-chunk Y worst={ey:.3e} "
        f"chunks checked={counts} last={ylast} of {s.T // s.chunk} (floor {FLOOR:g})")
    assert worst <= BF16_TOL and ey <= BF16_TOL
    assert min(last) >= 48 and min(counts) >= 28
    tail = float(np.max(np.abs(Yg[:, -s.chunk:])))
    log(f"last chunk: max |Y| = {tail:.3e} (oracle {float(np.max(np.abs(Yr[:, -s.chunk:]))):.3e})")
