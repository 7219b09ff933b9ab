"""The allocation-free update (atlasmem_update_chunked_static) against atlasmem_update_chunked on a
handle, through the C ABI: two calls in a row on the shared static scratch, the second with fewer
memories and tokens, each compared with the handle's result from the same state over the same
tokens (the same kernel's arithmetic: the handle runs the two-workgroup form for up to 128
memories, the static entry point one workgroup per memory, and the two agree bit for bit); the
non-finite flag is cleared per call; sizes beyond the scratch are refused before anything runs."""

import numpy as np
import pytest

from helpers import DEV, config_for, handle_update_run, log, static_update_run
from test_learned_neural_amd import atlasmem as am
from test_learned_neural_amd import synth

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("kind", [synth.MLP2_SILU, synth.MLP2_SILU_RESIDUAL])
def test_static_update_equals_handle_update_twice(kind):
    calls = [dict(batch=8, heads=16, T=512), dict(batch=1, heads=3, T=256)]
    for i, ov in enumerate(calls):
        inp = synth.make_inputs(4, "literal", kind=kind, **ov)
        log(f"CASE no_alloc call {i}: kind {kind} memories {inp.spec.n_mem} T {inp.spec.T}")
        ref = handle_update_run(inp)
        got = static_update_run(inp)
        for name, a, b in zip(("Y", "W", "S"), got, ref):
            d = float(np.max(np.abs(a.astype(np.float64) - b)) / np.max(np.abs(b)))
            log(f"PARITY no_alloc_{i}_{name}: {d:.3e}")
            assert np.array_equal(a, b), (name, d)


def test_static_update_rejects_beyond_scratch_and_other_configs():
    import torch
    s = synth.spec(4, "literal", batch=2, heads=am.STATIC_MAX_MEMORIES, T=128)  # 256 memories
    z = torch.zeros(1, device=DEV)
    with pytest.raises(am.AtlasMemError) as e:
        am.update_chunked_static(config_for(s), z, z, z, z, z, z, 128, z, z, z)
    assert e.value.status == am.E_SHAPE
    s2 = synth.spec(1, "literal", batch=1, heads=2, T=128)  # per-token gates: not the fused kernel
    with pytest.raises(am.AtlasMemError) as e:
        am.update_chunked_static(config_for(s2), z, z, z, z, z, z, 128, z, z, z)
    assert e.value.status == am.E_UNSUPPORTED
    s3 = synth.spec(4, "literal", batch=1, heads=2, T=128)
    with pytest.raises(am.AtlasMemError) as e:  # T not a multiple of the chunk
        am.update_chunked_static(config_for(s3), z, z, z, z, z, z, 100, z, z, z)
    assert e.value.status == am.E_SHAPE
