"""The per-chunk parity checks of the GPU tests, run on the CPU against mutated oracle outputs: a
result that goes wrong after the first chunks must fail them, although the tensor-wide error (set by
the first chunks, whose magnitude dominates a shrinking memory) does not see it."""

import numpy as np

from helpers import BF16_TOL, boundary_state_errors, maxrel, oracle_boundaries, per_chunk_y_errors
from test_learned_neural_amd import synth


def _ref():
    inp = synth.make_inputs(1, "stabilised", batch=1, heads=1, T=1024)
    return inp, oracle_boundaries(inp, [0])[0]


def test_zero_y_after_chunk_3_fails_per_chunk_check():
    inp, (Y, _) = _ref()
    C = inp.spec.chunk
    bad = Y.copy()
    bad[4 * C:] = 0.0
    assert maxrel(bad, Y) <= BF16_TOL                      # invisible to the tensor-wide error
    e, counts, last = per_chunk_y_errors(bad[None], Y[None], C)
    assert e >= 1.0 - 1e-12 and counts[0] == 16 and last[0] == 15
    ok, _, _ = per_chunk_y_errors(Y[None], Y[None], C)
    assert ok == 0.0


def test_late_chunk_offset_fails_per_chunk_check():
    """Chunk k answered with chunk k - 1's rows from chunk 8 on (a chunk-offset slip)."""
    inp, (Y, _) = _ref()
    C = inp.spec.chunk
    bad = Y.copy()
    bad[8 * C:] = Y[7 * C:-C]
    assert maxrel(bad, Y) <= BF16_TOL
    e, _, _ = per_chunk_y_errors(bad[None], Y[None], C)
    assert e > BF16_TOL


def test_late_state_error_fails_boundary_check():
    """A state that stops decaying at boundary 8 (e.g. a dropped forgetting factor late in the
    sequence) fails at the later boundaries, scaled by their own magnitude."""
    inp, (_, bounds) = _ref()
    ids = list(range(1, len(bounds)))
    good = [bounds[k] for k in ids]
    e, last = boundary_state_errors(inp.spec, good, bounds, ids)
    assert e == 0.0 and last == ids[-1]
    bad = [bounds[min(k, 8)] for k in ids]
    e, _ = boundary_state_errors(inp.spec, bad, bounds, ids)
    assert e > BF16_TOL
