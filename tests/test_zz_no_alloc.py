"""The allocation-free update (atlasmem_update_chunked_static) against atlasmem_update_chunked on a
handle, through the C ABI: two calls in a row on the shared static scratch, the second with fewer
memories and tokens, each compared with the handle's result from the same state over the same
tokens (the same kernel runs, so the results agree exactly); the non-finite flag is cleared per
call; sizes beyond the scratch are refused before anything runs."""

import numpy as np
import pytest

from helpers import DEV, config_for, log, segment, to_dev
from test_learned_neural_amd import atlasmem as am
from test_learned_neural_amd import synth

pytestmark = pytest.mark.gpu


def _handle_run(inp):
    import torch
    s = inp.spec
    mem = am.Memory(config_for(s), to_dev(inp.W0), to_dev(inp.S0))
    seg = segment(inp, 0, s.T)
    Y = torch.empty((s.n_mem, s.T, s.d_value), dtype=torch.float32, device=DEV)
    mem.update_chunked(seg["K"], seg["Q"], seg["V"], seg["theta"], seg["eta"], seg["alpha"], None, s.T, Y)
    W = torch.empty((s.n_mem, mem.P), dtype=torch.float32, device=DEV)
    S = torch.empty_like(W)
    assert mem.get_state(W, S) == am.OK
    torch.cuda.synchronize()
    mem.close()
    return Y.cpu().numpy(), W.cpu().numpy(), S.cpu().numpy()


def _static_run(inp):
    import torch
    s = inp.spec
    seg = segment(inp, 0, s.T)
    W = to_dev(inp.W0).clone()
    S = to_dev(inp.S0).clone()
    Y = torch.full((s.n_mem, s.T, s.d_value), float("nan"), dtype=torch.float32, device=DEV)
    flag = torch.full((1,), 7, dtype=torch.int32, device=DEV)
    st = am.update_chunked_static(config_for(s), seg["K"], seg["Q"], seg["V"], seg["theta"], seg["eta"],
                                  seg["alpha"], s.T, W, S, Y, flag)
    assert st == am.OK
    torch.cuda.synchronize()
    assert int(flag.item()) == 0
    return Y.cpu().numpy(), W.cpu().numpy(), S.cpu().numpy()


@pytest.mark.parametrize("kind", [synth.MLP2_SILU, synth.MLP2_SILU_RESIDUAL])
def test_static_update_equals_handle_update_twice(kind):
    calls = [dict(batch=8, heads=16, T=512), dict(batch=1, heads=3, T=256)]
    for i, ov in enumerate(calls):
        inp = synth.make_inputs(4, "literal", kind=kind, **ov)
        log(f"CASE no_alloc call {i}: kind {kind} memories {inp.spec.n_mem} T {inp.spec.T}")
        ref = _handle_run(inp)
        got = _static_run(inp)
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
