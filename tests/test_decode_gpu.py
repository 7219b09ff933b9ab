"""GPU parity of the decode kernel (streaming calls and retrievals of at most 8 tokens answered in
one launch) against the fp64 oracle, through the C ABI.

Retrieval reads the memory at the current state (the start weights of the unfinished chunk):
y = M_W(q) for the plain, residual and gated 2-layer memories.  The kernel keeps the split-bf16
product policy, so the bar is the bf16-input workloads' 2e-2 (it lands near 1e-6), and a
retrieval of n rows must equal the same rows retrieved one by one up to fp32 accumulation order
(1e-5, the streamed-versus-one-call bar).
"""

import numpy as np
import pytest

import oracle
from helpers import BF16_TOL, DEV, config_for, log, maxrel, to_dev, y_to_np
from test_learned_neural_amd import atlasmem as am
from test_learned_neural_amd import synth

pytestmark = pytest.mark.gpu

R, G = synth.MLP2_SILU_RESIDUAL, synth.MLP2_GATED
CASES = [
    # (name, workload, variant, overrides, rows, output dtype)
    ("plain_1row", 1, "stabilised", dict(batch=1, heads=4, T=64), 1, am.F32),
    ("plain_8rows_bf16_out", 4, "literal", dict(batch=2, heads=2, T=128), 8, am.BF16),
    ("residual_3rows", 4, "literal", dict(kind=R, batch=1, heads=3, T=128), 3, am.F32),
    ("gated_5rows_ragged", 1, "stabilised", dict(kind=G, batch=1, heads=2, T=64, d_key=20, d_value=12, d_hidden=36),
     5, am.F32),
    ("fp32_inputs_2rows", 1, "stabilised", dict(batch=1, heads=2, T=64, d_key=24, d_value=16, d_hidden=44,
                                                input_dtype=synth.F32), 2, am.F32),
]


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_decode_retrieve_matches_oracle(case):
    import torch
    name, idx, variant, ov, n, od = case
    log(f"CASE decode retrieve {name}")
    inp = synth.make_inputs(idx, variant, **ov)
    s = inp.spec
    mem = am.Memory(config_for(s, output_dtype=od), to_dev(inp.W0), to_dev(inp.S0))
    q = inp.Q[:, :n]
    ydt = torch.int16 if od == am.BF16 else torch.float32
    Y = torch.zeros((s.n_mem, n, s.d_value), dtype=ydt, device=DEV)
    mem.retrieve(to_dev(np.ascontiguousarray(q)), n, Y)
    ones = []
    for t in range(n):  # the same rows one by one
        y1 = torch.zeros((s.n_mem, 1, s.d_value), dtype=ydt, device=DEV)
        mem.retrieve(to_dev(np.ascontiguousarray(q[:, t:t + 1])), 1, y1)
        ones.append(y1)
    torch.cuda.synchronize()
    mem.close()
    got = y_to_np(Y)
    one = np.concatenate([y_to_np(y) for y in ones], axis=1)
    cfg = oracle.config_from(s)
    res = s.kind == R
    Qf = synth.bf16_bits_to_f32(q).astype(np.float64) if s.input_dtype == synth.BF16 else q.astype(np.float64)
    ref = np.stack([np.stack([oracle.memory_apply(oracle.unflatten(cfg, inp.W0[m]), Qf[m, t], res)
                              for t in range(n)]) for m in range(s.n_mem)])
    err = maxrel(got, ref)
    cons = maxrel(got, one)
    log(f"PARITY decode_{name}: Y={err:.3e} rows-vs-one-by-one={cons:.3e}")
    assert err <= BF16_TOL
    # the rows of a call are split over lanes by their count, so the fp32 summation order differs
    assert cons <= (1e-2 if od == am.BF16 else 1e-5)
