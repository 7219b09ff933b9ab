"""GPU parity of the outer-loop backward against the fp64 autograd oracle, through the C ABI.

Every gradient group (keys, queries, values, the three gates, initial weights and momentum) is
compared per tensor as max |x - r| / max |r| over all memories, against the 2e-2 bar of the
bf16-input workloads (the products run in split bf16 with fp32 accumulation, the forward's
checkpoints in fp32)."""

import numpy as np
import pytest

import oracle
from oracle import backward as bw
from helpers import BF16_TOL, DEV, F32_TOL, config_for, log, maxrel, to_dev
from test_learned_neural_amd import atlasmem as am
from test_learned_neural_amd import synth

pytestmark = pytest.mark.gpu

CASES = [
    # (name, workload, variant, overrides)
    ("mlp64x128_C64_two_chunks", 1, "stabilised", dict(batch=1, heads=2, T=128)),
    ("ragged_widths_C16", 1, "stabilised", dict(batch=2, heads=1, T=48, d_key=24, d_value=20, d_hidden=36, chunk=16)),
    ("fp32_inputs_C8", 1, "stabilised", dict(batch=1, heads=2, T=32, d_key=12, d_value=10, d_hidden=20, chunk=8,
                                             input_dtype=synth.F32)),
    # per-chunk gates: the chunk gradient through 5 Newton-Schulz steps (W1 128 x 64 runs transposed)
    ("ns5_per_chunk_C128", 4, "literal", dict(batch=1, heads=2, T=384)),
    # both matrices transposed (rows > cols), ragged widths that span several 64-wide tiles
    ("ns5_both_transposed", 4, "literal", dict(batch=1, heads=2, T=160, d_key=24, d_value=72, d_hidden=40, chunk=40)),
    # neither transposed
    ("ns5_none_transposed", 4, "literal", dict(batch=2, heads=1, T=96, d_key=56, d_value=20, d_hidden=36, chunk=32)),
    ("per_chunk_no_ns", 4, "literal", dict(batch=2, heads=1, T=256, ns_steps=0)),
    # the residual memory x + W2 silu(W1 x): keys in the error, queries in the output
    ("residual_per_token_C16", 1, "stabilised", dict(kind=synth.MLP2_SILU_RESIDUAL, batch=1, heads=2, T=48, d_key=24,
                                                      d_value=24, d_hidden=40, chunk=16)),
    ("residual_ns5_per_chunk", 4, "literal", dict(kind=synth.MLP2_SILU_RESIDUAL, batch=1, heads=2, T=256)),
    # the wide memory (384 -> 768 -> 384): tiles of every product span several 64-wide blocks
    ("wide_384x768_C64", 2, "stabilised", dict(batch=1, heads=1, T=128)),
    # the Omega window (per-token gates): key rows reach c - 1 tokens into the previous chunk
    ("omega3_C64", 1, "stabilised", dict(batch=1, heads=2, T=128, omega_window=3)),
    ("omega6_ragged_C16", 1, "stabilised", dict(batch=2, heads=1, T=48, d_key=24, d_value=20, d_hidden=36, chunk=16,
                                                omega_window=6)),
    ("omega2_residual_C16", 1, "stabilised", dict(kind=synth.MLP2_SILU_RESIDUAL, batch=1, heads=2, T=32, d_key=16,
                                                  d_value=16, d_hidden=24, chunk=16, omega_window=2)),
    # degree-2 polynomial features (the memory reads phi(k), phi(q); 32 -> 561 features) with the
    # window of 4, as in the Omega workload
    ("poly2_omega4_C64", 3, "stabilised", dict(batch=1, heads=2, T=128)),
    ("poly2_no_window_C16", 3, "stabilised", dict(batch=2, heads=1, T=48, d_key=6, d_value=20, d_hidden=36,
                                                  chunk=16, omega_window=1)),
    ("poly2_residual_window2", 3, "stabilised", dict(kind=synth.MLP2_SILU_RESIDUAL, batch=1, heads=2, T=48, d_key=4,
                                                     d_value=15, d_hidden=24, chunk=16, omega_window=2)),
    # the linear memory W x (fp32 bar): one token per chunk, and chunks of 4 with a window of 3
    ("linear_C1", 0, "literal", dict(batch=1, heads=2, T=48)),
    ("linear_C4_window3", 0, "literal", dict(batch=2, heads=1, T=40, chunk=4, omega_window=3, d_key=20, d_value=12)),
    ("linear_poly2_C8", 0, "literal", dict(batch=1, heads=2, T=32, chunk=8, poly_degree=2, d_key=5, d_value=7)),
    # the gated memory W2 (silu(W1 x) * W3 x): [W1; W3] one first-layer block
    ("gated_mlp64_C64", 1, "stabilised", dict(kind=synth.MLP2_GATED, batch=1, heads=2, T=128)),
    ("gated_ragged_C16", 1, "stabilised", dict(kind=synth.MLP2_GATED, batch=2, heads=1, T=48, d_key=20, d_value=12,
                                                d_hidden=36, chunk=16)),
    ("gated_omega3_poly2", 3, "stabilised", dict(kind=synth.MLP2_GATED, batch=1, heads=2, T=48, d_key=6, d_value=20,
                                                  d_hidden=24, chunk=16, omega_window=3)),
    # gated, per-chunk gates: three Newton-Schulz matrices (one batch at 64 -> 128 -> 64; W1 and
    # W3 paired, W2 apart at ragged widths)
    ("gated_ns5_per_chunk", 4, "literal", dict(kind=synth.MLP2_GATED, batch=1, heads=2, T=256)),
    ("gated_ns5_ragged", 4, "literal", dict(kind=synth.MLP2_GATED, batch=1, heads=2, T=96, d_key=24, d_value=40,
                                            d_hidden=32, chunk=32)),
    ("gated_per_chunk_no_ns", 4, "literal", dict(kind=synth.MLP2_GATED, batch=2, heads=1, T=256, ns_steps=0)),
]


def to_f64(a, dtype):
    return synth.bf16_bits_to_f32(a).astype(np.float64) if dtype == synth.BF16 else a.astype(np.float64)


# The benchmark's backward shapes: every memory runs on the GPU, the oracle recomputes sampled ones
# over the whole sequence (thousands of tokens, dozens of chunks).
LARGE = [
    ("bench_per_token_8x4096", 1, "stabilised", dict(), [0, 5]),
    ("bench_ns5_128x4096", 4, "literal", dict(T=4096), [0, 77]),
]


@pytest.mark.parametrize("case", LARGE, ids=[c[0] for c in LARGE])
def test_backward_at_benchmark_size_sampled(case):
    name, idx, variant, ov, mems = case
    _backward_case(name, idx, variant, ov, mems)


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_backward_matches_autograd_oracle(case):
    name, idx, variant, ov = case
    _backward_case(name, idx, variant, ov, None)


def _backward_case(name, idx, variant, ov, mems):
    """The library's backward over every memory; the oracle over `mems` (None: all of them)."""
    import torch
    log(f"CASE backward {name}")
    inp = synth.make_inputs(idx, variant, **ov)
    s = inp.spec
    M, T = s.n_mem, s.T
    r = np.random.default_rng(21)
    dY = r.standard_normal((M, T, s.d_value)).astype(np.float32)
    dWT = (0.1 * r.standard_normal((M, s.param_count))).astype(np.float32)
    dST = (0.1 * r.standard_normal((M, s.param_count))).astype(np.float32)
    mem = am.Memory(config_for(s), to_dev(inp.W0), to_dev(inp.S0))
    ws = torch.empty(mem.backward_workspace_bytes(T), dtype=torch.uint8, device=DEV)
    z = lambda *shape: torch.full(shape, float("nan"), dtype=torch.float32, device=DEV)
    dK, dQ, dV = z(M, T, s.d_key), z(M, T, s.d_key), z(M, T, s.d_value)
    ng = inp.theta.shape[1]  # T per token, T / C per chunk
    dth, det, dal = z(M, ng), z(M, ng), z(M, ng)
    win = s.omega_window > 1
    dgm = z(M, T) if win else None
    dW0, dS0 = z(M, mem.P), z(M, mem.P)
    Y = z(M, T, s.d_value)
    mem.update_backward(to_dev(inp.K), to_dev(inp.Q), to_dev(inp.V), to_dev(inp.theta), to_dev(inp.eta),
                        to_dev(inp.alpha), T, to_dev(dY), dK, dQ, dV, dth, det, dal, dW0, dS0, ws, Y=Y,
                        dW_T=to_dev(dWT), dS_T=to_dev(dST), gamma=to_dev(inp.gamma) if win else None, dgamma=dgm)
    W = torch.empty((M, mem.P), dtype=torch.float32, device=DEV)
    S = torch.empty_like(W)
    status = mem.get_state(W, S)
    torch.cuda.synchronize()
    mem.close()
    assert status == am.OK
    cfg = oracle.config_from(s)
    K, Q, V = to_f64(inp.K, s.input_dtype), to_f64(inp.Q, s.input_dtype), to_f64(inp.V, s.input_dtype)
    errs = {}
    got = dict(K=dK, Q=dQ, V=dV, theta=dth, eta=det, alpha=dal)
    if win:
        got["gamma"] = dgm
    ref = {k: [] for k in got}
    ref["W0"], ref["S0"] = [], []
    ys, wts = [], []
    mems = list(range(M)) if mems is None else mems
    for m in mems:
        P0 = oracle.unflatten(cfg, inp.W0[m].astype(np.float64))
        S0m = oracle.unflatten(cfg, inp.S0[m].astype(np.float64))
        g = bw.outer_grads(cfg, P0, S0m, K[m], Q[m], V[m], inp.theta[m], inp.eta[m], inp.alpha[m], dY[m],
                           oracle.unflatten(cfg, dWT[m].astype(np.float64)),
                           oracle.unflatten(cfg, dST[m].astype(np.float64)),
                           gamma=inp.gamma[m] if win else None)
        for k in got:
            ref[k].append(g[k])
        ref["W0"].append(oracle.flatten(g["W0"]))
        ref["S0"].append(oracle.flatten(g["S0"]))
        res = oracle.run_memory(cfg, P0, S0m, K[m], Q[m], V[m], inp.theta[m], inp.eta[m], inp.alpha[m],
                                inp.gamma[m] if win else None)
        ys.append(res.Y)
        wts.append(oracle.flatten(res.params))
    for k, t in got.items():
        errs[k] = maxrel(t.cpu().numpy()[mems], np.stack(ref[k]))
    errs["W0"] = maxrel(dW0.cpu().numpy()[mems], np.stack(ref["W0"]))
    errs["S0"] = maxrel(dS0.cpu().numpy()[mems], np.stack(ref["S0"]))
    errs["Y"] = maxrel(Y.cpu().numpy()[mems], np.stack(ys))
    errs["W_T"] = maxrel(W.cpu().numpy()[mems], np.stack(wts))
    label = lambda k: k if k in ("Y", "W_T") else "d" + k  # forward outputs, then gradients
    tol = F32_TOL if s.kind == synth.LINEAR else BF16_TOL  # the linear workload's fp32 bar
    log(f"PARITY backward_{name} (memories {mems}, T {T}): " + " ".join(f"{label(k)}={v:.3e}" for k, v in errs.items())
        + f" (tol {tol:g})")
    assert all(v <= tol for v in errs.values()), errs


def test_backward_errors():
    import torch
    for s3 in (synth.spec(3, "stabilised", batch=1, heads=1, T=256, gate_mode=synth.PER_CHUNK, omega_window=1),
               synth.spec(1, "stabilised", batch=1, heads=1, T=256, per_token_retrieve=True)):
        mem = am.Memory(config_for(s3))
        assert mem.backward_workspace_bytes(256) == -1
        mem.close()
    s = synth.spec(1, "stabilised", batch=1, heads=1, T=64)
    mem = am.Memory(config_for(s))
    need = mem.backward_workspace_bytes(64)
    assert need > 0
    small = torch.empty(need - 4, dtype=torch.uint8, device=DEV)
    x = torch.zeros((1, 64, 64), dtype=torch.float32, device=DEV)
    g = torch.zeros((1, 64), dtype=torch.float32, device=DEV)
    p = torch.zeros((1, mem.P), dtype=torch.float32, device=DEV)
    xb = torch.zeros((1, 64, 64), dtype=torch.int16, device=DEV)
    with pytest.raises(am.AtlasMemError) as e:
        mem.update_backward(xb, xb, xb, g, g, g, 64, x, x, x, x, g, g, g, p, p, small)
    assert e.value.status == am.E_INVALID
    ws = torch.empty(need, dtype=torch.uint8, device=DEV)
    with pytest.raises(am.AtlasMemError) as e:
        mem.update_backward(xb, xb, xb, g, g, g, 40, x, x, x, x, g, g, g, p, p, ws)
    assert e.value.status == am.E_SHAPE
    mem.close()
    # an Omega window needs its gates and their gradient
    sw = synth.spec(1, "stabilised", batch=1, heads=1, T=64, omega_window=3)
    mem = am.Memory(config_for(sw))
    ws = torch.empty(mem.backward_workspace_bytes(64), dtype=torch.uint8, device=DEV)
    with pytest.raises(am.AtlasMemError) as e:
        mem.update_backward(xb, xb, xb, g, g, g, 64, x, x, x, x, g, g, g, p, p, ws)
    assert e.value.status == am.E_INVALID
    mem.close()
