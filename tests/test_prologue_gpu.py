"""GPU parity of the input prologue (short convolution, gates) against the fp64 oracle, through
the C ABI.

Tolerances (max |x - r| / max |r| per tensor): fp32 outputs of the convolution within 1e-5 (four
fp32 multiply-adds per element); bf16 outputs within 4e-3 (one rounding to bf16, 2^-9 relative,
on top of that); gates within 1e-4 (exact bf16 inputs times hi/lo-split weights, fp32
accumulation, hardware exp and reciprocal).  Streamed convolutions equal one call bit for bit:
every output element is computed by the same four multiply-adds in the same order.
"""

import numpy as np
import pytest

from helpers import DEV, log, maxrel, to_dev
from oracle import prologue as pro
from test_learned_neural_amd import atlasmem as am
from test_learned_neural_amd import synth

pytestmark = pytest.mark.gpu

CONV_F32_TOL = 1e-5
CONV_BF16_TOL = 4e-3
GATE_TOL = 1e-4


def as_f64(a, dtype):
    return synth.bf16_bits_to_f32(a).astype(np.float64) if dtype == am.BF16 else a.astype(np.float64)


def dev_out(shape, dtype):
    import torch
    return torch.full(shape, -7, dtype=torch.int16 if dtype == am.BF16 else torch.float32, device=DEV)


def out_np(t, dtype):
    a = t.cpu().numpy()
    return as_f64(a.view(np.uint16), dtype) if dtype == am.BF16 else a.astype(np.float64)


def run_conv(p, H, in_dt, out_dt, l2norm, with_bias=True, with_hist=True, t0=0, t1=None, hist_dev=None,
             want_hist=False):
    """One atlasmem_short_conv call over tokens [t0, t1) of p.X; returns (out, hist_out) tensors."""
    import torch
    M, T, d = p.X.shape
    t1 = T if t1 is None else t1
    X = to_dev(p.X[:, t0:t1])
    out = dev_out((M, t1 - t0, d), out_dt)
    hist = hist_dev if hist_dev is not None else (to_dev(p.hist) if with_hist else None)
    hout = torch.zeros((M, 3, d), dtype=X.dtype, device=DEV) if want_hist else None
    am.short_conv(X, in_dt, M, t1 - t0, d, H, to_dev(p.taps), to_dev(p.bias) if with_bias else None, hist, l2norm,
                  out, out_dt, hout)
    return out, hout


CONV_CASES = [
    # (name, B, H, T, d, in_dtype, out_dtype, l2norm, bias, hist)
    ("d64_bf16_norm", 2, 3, 100, 64, am.BF16, am.BF16, True, True, True),
    ("d64_bf16_raw_f32out", 2, 3, 100, 64, am.BF16, am.F32, False, True, False),
    ("d40_f32_norm", 1, 2, 77, 40, am.F32, am.F32, True, False, True),
    ("d20_bf16_ragged_width", 1, 3, 33, 20, am.BF16, am.BF16, False, True, True),
    ("d300_f32_wide_ragged", 1, 2, 45, 300, am.F32, am.BF16, True, True, False),
    ("d512_bf16_widest", 1, 1, 40, 512, am.BF16, am.F32, True, True, True),
    ("d3_f32_tiny", 2, 1, 5, 3, am.F32, am.F32, False, True, True),
]


@pytest.mark.parametrize("case", CONV_CASES, ids=[c[0] for c in CONV_CASES])
def test_short_conv_parity(case):
    import torch
    name, B, H, T, d, in_dt, out_dt, l2n, with_bias, with_hist = case
    log(f"CASE conv {name}")
    p = synth.make_prologue_inputs(1, B, H, T, d, 16, in_dtype=in_dt)
    out, _ = run_conv(p, H, in_dt, out_dt, l2n, with_bias, with_hist)
    torch.cuda.synchronize()
    ref = pro.short_conv_all(as_f64(p.X, in_dt), p.taps, H, p.bias if with_bias else None,
                             as_f64(p.hist, in_dt) if with_hist else None, l2norm=l2n)
    err = maxrel(out_np(out, out_dt), ref)
    tol = CONV_BF16_TOL if out_dt == am.BF16 else CONV_F32_TOL
    log(f"PARITY conv_{name}: {err:.3e} (tol {tol:g})")
    assert err <= tol
    if l2n:
        nrm = np.linalg.norm(out_np(out, out_dt), axis=-1)
        assert np.all(np.abs(nrm - 1.0) <= (1e-2 if out_dt == am.BF16 else 1e-5))


@pytest.mark.parametrize("cut", [[0, 1, 2, 3, 40], [0, 17, 18, 40], [0, 0, 40], [0, 32, 40]])
def test_short_conv_streaming_bitwise(cut):
    """Calls over [t0, t1) chained through hist_out equal one call, bit for bit, and the carried
    rows equal the oracle's."""
    import torch
    B, H, T, d = 1, 2, 40, 64
    p = synth.make_prologue_inputs(2, B, H, T, d, 16)
    whole, _ = run_conv(p, H, am.BF16, am.F32, True)
    parts, hist = [], to_dev(p.hist)
    for a, b in zip(cut[:-1], cut[1:]):
        out, hist = run_conv(p, H, am.BF16, am.F32, True, t0=a, t1=b, hist_dev=hist, want_hist=True)
        parts.append(out)
        ref_h = pro.conv_history(as_f64(p.X[0, :b], am.BF16), as_f64(p.hist[0], am.BF16))
        assert np.array_equal(synth.bf16_bits_to_f32(hist[0].cpu().numpy().view(np.uint16)).astype(np.float64),
                              ref_h)
    torch.cuda.synchronize()
    got = torch.cat(parts, dim=1)
    log(f"CASE conv_stream cut {cut}")
    assert torch.equal(got, whole)


def test_short_conv_edges_and_errors():
    import torch
    p = synth.make_prologue_inputs(3, 1, 2, 8, 16, 16)
    X = to_dev(p.X)
    taps = to_dev(p.taps)
    out = dev_out((2, 8, 16), am.BF16)
    # T = 0 writes only the carried rows (the old ones, since nothing new came)
    hout = torch.zeros((2, 3, 16), dtype=torch.int16, device=DEV)
    am.short_conv(X, am.BF16, 2, 0, 16, 2, taps, None, to_dev(p.hist), True, out, am.BF16, hout)
    torch.cuda.synchronize()
    assert torch.equal(hout.cpu(), torch.from_numpy(p.hist.view(np.int16)))
    for bad in (dict(d=0), dict(heads=0), dict(M=-1), dict(l2norm=2)):
        kw = dict(M=2, T=8, d=16, heads=2, l2norm=1)
        kw.update(bad)
        with pytest.raises(am.AtlasMemError) as e:
            am.short_conv(X, am.BF16, kw["M"], kw["T"], kw["d"], kw["heads"], taps, None, None, kw["l2norm"], out,
                          am.BF16)
        assert e.value.status == am.E_INVALID
    with pytest.raises(am.AtlasMemError) as e:  # in place is refused
        am.short_conv(X, am.BF16, 2, 8, 16, 2, taps, None, None, True, X, am.BF16)
    assert e.value.status == am.E_INVALID
    with pytest.raises(am.AtlasMemError) as e:
        am.short_conv(X, am.BF16, 2, 8, 600, 2, taps, None, None, True, out, am.BF16)
    assert e.value.status == am.E_SHAPE


def run_gates(p, B, T, dm, H, n_g, chunk):
    import torch
    n = T if chunk == 1 else -(-T // chunk)
    out = torch.full((n_g, B, H, n), float("nan"), dtype=torch.float32, device=DEV)
    am.gates(to_dev(p.U), B, T, dm, H, n_g, to_dev(p.Wg), to_dev(p.bg), to_dev(p.scale), chunk, out)
    torch.cuda.synchronize()
    return out.cpu().numpy().astype(np.float64)


GATE_CASES = [
    # (name, B, H, T, d_model, n_gates, chunk)
    ("per_token_dm64_ragged", 2, 3, 100, 64, 3, 1),
    ("per_token_dm512_omega", 2, 4, 70, 512, 4, 1),
    ("per_token_dm48", 1, 5, 31, 48, 3, 1),
    ("two_column_passes", 1, 20, 50, 128, 4, 1),
    ("pooled_C32", 2, 3, 128, 64, 3, 32),
    ("pooled_C64_short_tail", 2, 16, 150, 512, 3, 64),
    ("pooled_C128_one_short_chunk", 1, 2, 40, 32, 3, 128),
]


@pytest.mark.parametrize("case", GATE_CASES, ids=[c[0] for c in GATE_CASES])
def test_gates_parity(case):
    name, B, H, T, dm, n_g, chunk = case
    log(f"CASE gates {name}")
    p = synth.make_prologue_inputs(4, B, H, T, 8, dm, n_gates=n_g)
    got = run_gates(p, B, T, dm, H, n_g, chunk)
    ref = pro.gates_all(synth.bf16_bits_to_f32(p.U).astype(np.float64), p.Wg, p.bg, p.scale, chunk)
    assert np.all(np.isfinite(got))
    errs = [maxrel(got[g], ref[g]) for g in range(n_g)]
    log(f"PARITY gates_{name}: " + " ".join(f"{e:.3e}" for e in errs) + f" (tol {GATE_TOL:g})")
    assert max(errs) <= GATE_TOL
    # every gate stays inside (0, scale)
    for g in range(n_g):
        assert np.all(got[g] > 0) and np.all(got[g] <= p.scale[g])


def test_gates_errors():
    import torch
    p = synth.make_prologue_inputs(5, 1, 2, 16, 8, 64)
    out = torch.empty((3, 1, 2, 16), dtype=torch.float32, device=DEV)
    args = (to_dev(p.U), 1, 16, 64, 2, 3, to_dev(p.Wg), to_dev(p.bg), to_dev(p.scale))
    for dm, chunk, status in ((40, 1, am.E_UNSUPPORTED), (64, 48, am.E_UNSUPPORTED), (1024, 1, am.E_UNSUPPORTED),
                              (64, 0, am.E_INVALID)):
        a = list(args)
        a[3] = dm
        with pytest.raises(am.AtlasMemError) as e:
            am.gates(*a, chunk, out)
        assert e.value.status == status


def test_prologue_full_size_sampled():
    """The Newton-Schulz workload's shape (8 x 16 memories x 32768 tokens, width 64, token inputs
    of width 512): the keys' convolution and the per-chunk and per-token gates in one call
    each, checked against the oracle on sampled memories / sequences."""
    import torch
    B, H, T, d, dm, C = 8, 16, 32768, 64, 512, 128
    p = synth.make_prologue_inputs(6, B, H, T, d, dm, n_gates=3)
    log("CASE prologue_full_size")
    out, _ = run_conv(p, H, am.BF16, am.BF16, True)
    torch.cuda.synchronize()
    for m in (0, 77, 127):
        y = out_np(out[m], am.BF16)
        ref = pro.l2_normalise(pro.short_conv(as_f64(p.X[m], am.BF16), p.taps[m % H], p.bias[m % H],
                                              as_f64(p.hist[m], am.BF16)))
        err = maxrel(y, ref)
        log(f"PARITY conv_full memory {m}: {err:.3e}")
        assert err <= CONV_BF16_TOL
    del out
    for chunk in (C, 1):
        got = run_gates(p, B, T, dm, H, 3, chunk)
        for b in (0, 5):
            ref = pro.gates(synth.bf16_bits_to_f32(p.U[b]).astype(np.float64), p.Wg, p.bg, p.scale, chunk)
            errs = [maxrel(got[g, b], ref[g]) for g in range(3)]
            log(f"PARITY gates_full chunk {chunk} sequence {b}: " + " ".join(f"{e:.3e}" for e in errs))
            assert max(errs) <= GATE_TOL


# ----------------------------------------------------------------------------- feature map stage

FMAP_F32_TOL = 1e-6   # products of up to three inputs in fp32 against fp64
FMAP_PROJ_TOL = 1e-4  # the projection runs in split bf16 (hi/lo) with fp32 accumulation

FMAP_CASES = [
    # (name, n, d, degree, in_dtype, coeffs, d_out or 0)
    ("deg1_bf16", 37, 7, 1, am.BF16, None, 0),
    ("deg2_default", 37, 7, 2, am.BF16, None, 0),
    ("deg3_default_ragged", 1001, 5, 3, am.F32, None, 0),
    ("deg3_learned_coeffs_d32", 64, 32, 3, am.BF16, [0.9, 1.2, 0.4, 0.3], 0),
    ("deg2_single_row", 1, 33, 2, am.F32, [1.0, 0.5, 0.25], 0),
    ("deg2_project_d64", 300, 16, 2, am.BF16, None, 64),
    ("deg3_project_ragged_d70", 130, 6, 3, am.F32, [1.0, 1.0, 0.5, 0.2], 70),
    ("deg1_project_d5", 77, 9, 1, am.BF16, None, 5),
    ("deg3_project_d128_four_tiles", 257, 12, 3, am.BF16, [1.0, 0.8, 0.5, 0.25], 128),
    # beyond the matrix-core kernel's limits (d_out > 128, rows wider than 64): the GEMM engine
    ("deg2_project_d200_engine", 70, 8, 2, am.F32, None, 200),
    ("deg2_project_rows70_engine", 40, 70, 2, am.BF16, None, 32),
]


@pytest.mark.parametrize("case", FMAP_CASES, ids=[c[0] for c in FMAP_CASES])
def test_feature_map_parity(case):
    import torch
    name, n, d, deg, dt, coeffs, d_out = case
    log(f"CASE feature_map {name}")
    r = np.random.default_rng(7)
    x = r.standard_normal((n, d)).astype(np.float32) * 0.7
    xin = synth.f32_to_bf16_bits(x) if dt == am.BF16 else x
    xf = as_f64(xin, dt)
    F = pro.feature_count(d, deg)
    P = (r.standard_normal((d_out, F)) / np.sqrt(F)).astype(np.float32) if d_out else None
    out = torch.full((n, d_out or F), float("nan"), dtype=torch.float32, device=DEV)
    am.feature_map(to_dev(xin), dt, n, d, deg, out, coeffs=coeffs, P=None if P is None else to_dev(P), d_out=d_out)
    torch.cuda.synchronize()
    got = out.cpu().numpy().astype(np.float64)
    ref = pro.feature_map(xf, deg, coeffs, None if P is None else P.astype(np.float64))
    err = maxrel(got, ref)
    tol = FMAP_PROJ_TOL if d_out else FMAP_F32_TOL
    log(f"PARITY feature_map_{name}: {err:.3e} (tol {tol:g})")
    assert np.all(np.isfinite(got)) and err <= tol


def test_feature_map_errors():
    import torch
    out = torch.empty((4, 10), dtype=torch.float32, device=DEV)
    x = torch.zeros((4, 3), dtype=torch.float32, device=DEV)
    for kw, status in ((dict(degree=0), am.E_INVALID), (dict(degree=4), am.E_INVALID), (dict(d=0), am.E_INVALID),
                       (dict(d=200, degree=3), am.E_SHAPE)):
        a = dict(n=4, d=3, degree=2)
        a.update(kw)
        with pytest.raises(am.AtlasMemError) as e:
            am.feature_map(x, am.F32, a["n"], a["d"], a["degree"], out)
        assert e.value.status == status


def test_dot_exponential_features_with_omega_update():
    """Dot: degree-3 exponential-kernel features of the keys and queries (from the feature map
    stage) as the inputs of the Omega-window memory update, against the oracle on the same
    composition."""
    import torch
    import oracle
    from helpers import compare, config_for, BF16_TOL
    B, H, T, dk = 1, 2, 96, 4
    F = pro.feature_count(dk, 3)  # 35
    spec = synth.spec(3, "stabilised", batch=B, heads=H, T=T, d_key=F, poly_degree=1, d_value=24, d_hidden=40,
                      chunk=32, omega_window=3, input_dtype=synth.F32)
    inp = synth.make_inputs(3, "stabilised", batch=B, heads=H, T=T, d_key=F, poly_degree=1, d_value=24,
                            d_hidden=40, chunk=32, omega_window=3, input_dtype=synth.F32)
    r = np.random.default_rng(3)
    k_raw = r.standard_normal((B * H, T, dk)).astype(np.float32) * 0.5
    q_raw = r.standard_normal((B * H, T, dk)).astype(np.float32) * 0.5
    log("CASE dot_degree3_omega3")
    Kf = torch.empty((B * H * T, F), dtype=torch.float32, device=DEV)
    Qf = torch.empty_like(Kf)
    am.feature_map(to_dev(k_raw.reshape(-1, dk)), am.F32, B * H * T, dk, 3, Kf)
    am.feature_map(to_dev(q_raw.reshape(-1, dk)), am.F32, B * H * T, dk, 3, Qf)
    mem = am.Memory(config_for(spec), to_dev(inp.W0), to_dev(inp.S0))
    Y = torch.empty((B * H, T, spec.d_value), dtype=torch.float32, device=DEV)
    mem.update_chunked(Kf.view(B * H, T, F), Qf.view(B * H, T, F), to_dev(inp.V), to_dev(inp.theta),
                       to_dev(inp.eta), to_dev(inp.alpha), to_dev(inp.gamma), T, Y)
    W = torch.empty((B * H, mem.P), dtype=torch.float32, device=DEV)
    S = torch.empty_like(W)
    status = mem.get_state(W, S)
    torch.cuda.synchronize()
    mem.close()
    # the oracle on the same composition: fp64 features, then the literal recurrence
    inp.K = np.stack([pro.feature_map(k_raw[m], 3) for m in range(B * H)])
    inp.Q = np.stack([pro.feature_map(q_raw[m], 3) for m in range(B * H)])
    ref = oracle.run_inputs(inp)
    got = (Y.cpu().numpy().astype(np.float64), W.cpu().numpy().astype(np.float64),
           S.cpu().numpy().astype(np.float64))
    errs = compare("dot_degree3_omega3", spec, got, ref, BF16_TOL)
    assert status == am.OK
    assert all(v <= BF16_TOL for v in errs.values()), errs
