"""The general path at the workloads' full sizes, in one update call as the benchmark would run it,
against the fp64 oracle (stabilised variants: the literal ones leave fp32's range, which the
teacher-forced tests in test_parity_gpu cover up to that point)."""

import numpy as np
import pytest

from helpers import BF16_TOL, DEV, compare, log, oracle_run, run_gpu, segment, split_params, config_for, maxrel
from test_learned_neural_amd import atlasmem as am
from test_learned_neural_amd import synth

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("index", [1, 2])
def test_full_size_all_memories(index):
    """Every memory of the 64 -> 128 -> 64 (2 x 4 x 4096) and 384 -> 768 -> 384 (2 x 1 x 1024)
    workloads over the whole sequence."""
    inp = synth.make_inputs(index, "stabilised")
    log(f"CASE full_size workload {index} {inp.spec.name}")
    ref = oracle_run(inp)
    got = run_gpu(inp)
    assert got[3] == am.OK
    errs = compare(f"full_size_{index}", inp.spec, got, ref, BF16_TOL)
    assert all(v <= BF16_TOL for v in errs.values()), errs


def test_full_size_omega_poly_sampled():
    """Polynomial keys (32 -> 561) with the Omega window 4, 4 x 8 x 8192 in two update calls.  The
    state is compared after the first 2048 tokens, while it is still far inside fp32's range (with
    these gates the product-form memory shrinks geometrically and leaves fp32's range after about
    50 of the 128 chunks, where relative state errors stop meaning anything); Y is compared over the
    whole sequence.  The oracle recomputes two sampled memories."""
    import torch
    inp = synth.make_inputs(3, "stabilised")
    s = inp.spec
    mems = [3, 26]
    t_mid = 2048
    log(f"CASE full_size workload 3 {s.name} memories {mems}")
    ref_mid = oracle_run(inp, mems=mems, T=t_mid)
    ref = oracle_run(inp, mems=mems)

    mem = am.Memory(config_for(s), torch.from_numpy(inp.W0).to(DEV), torch.from_numpy(inp.S0).to(DEV))
    Y = torch.empty((s.n_mem, s.T, s.d_value), dtype=torch.float32, device=DEV)
    W = torch.empty((s.n_mem, mem.P), dtype=torch.float32, device=DEV)
    S = torch.empty_like(W)
    states = []
    for a, b in ((0, t_mid), (t_mid, s.T)):
        seg = segment(inp, a, b)
        y = torch.empty((s.n_mem, b - a, s.d_value), dtype=torch.float32, device=DEV)
        mem.update_chunked(seg["K"], seg["Q"], seg["V"], seg["theta"], seg["eta"], seg["alpha"], seg["gamma"],
                           b - a, y)
        Y[:, a:b] = y
        status = mem.get_state(W, S)
        states.append((status, W.cpu().numpy().astype(np.float64), S.cpu().numpy().astype(np.float64)))
    torch.cuda.synchronize()
    mem.close()
    Yg = Y.cpu().numpy().astype(np.float64)

    status, Wm, Sm = states[0]
    assert status == am.OK
    scale = max(float(np.max(np.abs(p))) for p in split_params(s, ref_mid[1]))
    log(f"state scale at token {t_mid}: max |W| = {scale:.3e}")
    assert scale > 1e-20
    errs = compare(f"full_size_3_state_at_{t_mid}", s, (Yg[mems, :t_mid], Wm[mems], Sm[mems]), ref_mid, BF16_TOL)
    assert all(v <= BF16_TOL for v in errs.values()), errs
    ey = maxrel(Yg[mems], ref[0])
    log(f"PARITY full_size_3_Y_whole_sequence: Y={ey:.3e} (tol {BF16_TOL:g})")
    assert ey <= BF16_TOL
    assert np.all(np.isfinite(Yg))
