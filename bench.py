"""Throughput of the neural-memory update + retrieval on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload 4] [--no-cpu]

A step is one atlasmem_update_chunked call over the whole sequence of every memory
(retrieval of every query at its chunk-start weights, the chunk-wise update with the
per-chunk Newton-Schulz orthogonalisation), starting from the workload's initial state
(restored with atlasmem_set_state before each step, inside the timed region).
Inputs are seeded synthetic tensors already resident in device memory.

Prints one JSON line: tokens/s (B*H*T per second), the roofline of the dominant kernel
(algorithmic FLOPs or bytes per launch over its average duration, timed with HIP events
on the stream it runs on) and the fp64 oracle's throughput on a bounded sample on the
host's cores.
"""

from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 / fp16 matrix peak (TFLOP/s)
PEAK_HBM_GBS = 8000.0       # MI355X HBM3E (GB/s)
METRIC = "memory-update+retrieval tokens/s (B·H·T/s) per config; % of bf16 MFMA peak"


def mlp_flops_per_chunk(spec) -> dict:
    """Algorithmic FLOPs of one chunk of one memory (2 per multiply-add), by stage."""
    C, din, dh, dv = spec.chunk, spec.d_in, spec.d_hidden, spec.d_value
    R = C + spec.omega_window - 1
    f = dict(
        retrieval=2 * C * din * dh + 2 * C * dh * dv,
        forward=2 * R * din * dh + 2 * R * dh * dv,
        backward=2 * R * dv * dh,
        wgrad=(2 if spec.gate_mode == 0 else 1) * (2 * R * dv * dh + 2 * R * dh * din),
    )
    if spec.ns_steps:
        def ns(r, c):
            m, n = min(r, c), max(r, c)
            return spec.ns_steps * (2 * m * m * n + 2 * m * m * m + 2 * m * m * n)
        f["newton_schulz"] = ns(dh, din) + ns(dv, dh)
    return f


def gated_flops_per_chunk(spec) -> dict:
    """Algorithmic FLOPs of one chunk of the gated memory M(x) = W2 (silu(W1 x) * (W3 x)): the
    plain memory's products with the W1 products doubled (W3 beside W1) and three
    Newton-Schulz matrices."""
    C, din, dh, dv = spec.chunk, spec.d_in, spec.d_hidden, spec.d_value
    R = C + spec.omega_window - 1
    f = dict(
        retrieval=2 * C * 2 * din * dh + 2 * C * dh * dv,
        forward=2 * R * 2 * din * dh + 2 * R * dh * dv,
        backward=2 * R * dv * dh,
        wgrad=(2 if spec.gate_mode == 0 else 1) * (2 * R * dv * dh + 2 * 2 * R * dh * din),
    )
    if spec.ns_steps:
        f["newton_schulz"] = 2 * ns_flops_per_matrix(dh, din, spec.ns_steps) + ns_flops_per_matrix(dv, dh,
                                                                                                  spec.ns_steps)
    return f


def ptr_flops_per_chunk(spec) -> dict:
    """The plain memory's chunk with per-token retrieval: the queries read W_t = beta_t W0 +
    a_t S0 - sum_r Om[t][r] g_r through Z0 = Q W0_1^T, ZS = Q S0_1^T, the scores Q K^T, the mix
    (Om * scores) D1, the hidden scores Hq Hk^T, Hq W0_2^T, Hq S0_2^T and (Om * scores) D2."""
    C, din, dh, dv = spec.chunk, spec.d_in, spec.d_hidden, spec.d_value
    R = C + spec.omega_window - 1
    f = mlp_flops_per_chunk(spec)
    f["retrieval"] = 2 * C * (2 * din * dh + R * din + 2 * R * dh + 2 * dh * dv + R * dv)
    return f


def backward_flops_per_chunk(spec) -> int:
    """Algorithmic FLOPs of one chunk of one memory in the outer-loop backward call (window 1,
    identity features): the forward it records (as in mlp_flops_per_chunk) plus the reverse step's
    products, which recompute the chunk's activations from its checkpoint: Z of keys and queries,
    E, P, the adjoint projections (two per layer per token for per-token gates, one per layer for
    per-chunk gates, whose gradient sum G and its Newton-Schulz iterates are recomputed too), E',
    W2' (3C deep), H' and X' (3 or 2 terms), Zq', Q', W1' (2C deep), and the Newton-Schulz backward,
    twice its forward."""
    C, din, dh, dv = spec.chunk, spec.d_in, spec.d_hidden, spec.d_value
    pc = spec.gate_mode == 1
    p1, p2 = 2 * C * din * dh, 2 * C * dh * dv  # one product over the chunk's rows, per layer
    terms = 2 if pc else 3
    back = (2 * p1 + p2 + p2                      # Z (keys, queries), E, P
            + (1 if pc else 2) * (p1 + p2)        # U projections
            + p2 + 3 * p2 + terms * p2            # E', W2', H'
            + terms * p1 + p2 + p1 + 2 * p1)      # X', Zq', Q', W1'
    if pc:
        back += p1 + p2                           # G recomputed
        if spec.ns_steps:
            nsf = ns_flops_per_matrix(dh, din, spec.ns_steps) + ns_flops_per_matrix(dv, dh, spec.ns_steps)
            back += 3 * nsf                       # forward recomputed + backward (2x)
    return int(sum(mlp_flops_per_chunk(spec).values()) + back)


def ns_flops_per_matrix(rows, cols, steps):
    m, n = min(rows, cols), max(rows, cols)
    return steps * (2 * m * m * n + 2 * m * m * m + 2 * m * m * n)


TRAFFIC_FILE = os.path.join(ROOT, "profiles", "ns5_B8H16_T32768_fused_kernel_traffic.txt")
FUSED_SOURCES = [os.path.join(ROOT, "test_learned_neural_amd", "csrc", f) for f in ("k_fused.hip", "common.h",
                                                                                  "mfma_tiles.h")]


def measured_traffic():
    """HBM bytes per launch of the fused kernel from the committed counter summary, or None when
    the kernel's sources have changed since the counters were taken."""
    import hashlib
    try:
        kv = {}
        for ln in open(TRAFFIC_FILE):
            if "=" in ln and not ln.startswith("#"):
                k, v = ln.split("=", 1)
                kv[k.strip()] = v.strip()
        m = hashlib.sha256()
        for f in FUSED_SOURCES:
            m.update(open(f, "rb").read())
        if m.hexdigest()[:16] != kv["kernel_sources_sha256_16"]:
            return None
        return int(float(kv["hbm_bytes_per_launch"]))
    except (OSError, KeyError, ValueError):
        return None


STATS_FILE = os.path.join(ROOT, "profiles", "ns5_B8H16_T32768_fused_kernel_stats.md")


def sources_sha16():
    import hashlib
    m = hashlib.sha256()
    for f in FUSED_SOURCES:
        m.update(open(f, "rb").read())
    return m.hexdigest()[:16]


def rocprof_kernel_ms():
    """Average duration (ms) of the fused kernel from the committed rocprofv3 --kernel-trace --stats
    summary, or None when the kernel's sources have changed since it was taken."""
    try:
        kv = {}
        for ln in open(STATS_FILE):
            if "=" in ln and not ln.startswith("#") and not ln.startswith("|"):
                k, v = ln.split("=", 1)
                kv[k.strip()] = v.strip()
        if sources_sha16() != kv["kernel_sources_sha256_16"]:
            return None
        return float(kv["avg_ns"]) * 1e-6
    except (OSError, KeyError, ValueError):
        return None


def cpu_model() -> str:
    try:
        for ln in open("/proc/cpuinfo"):
            if ln.startswith("model name"):
                return ln.split(":", 1)[1].strip()
    except OSError:
        pass
    import platform
    return platform.processor() or "unknown"


def calibration(torch, am, dev, stream):
    """The measured ceilings: the bf16 matrix-core rate of a kernel that does nothing else (256
    workgroups of eight waves, eight independent 32x32x16 chains per wave) and the rate of a plain
    16-byte streaming copy of 1 GiB."""
    sink = torch.empty(256, dtype=torch.float32, device=dev)
    iters = 20000
    flops = 256 * 8 * iters * 8 * 32768
    am.calibrate_mfma(iters, 256, sink, stream)
    t = event_ms(lambda: am.calibrate_mfma(iters, 256, sink, stream), 5, stream)
    n = 1 << 30
    src = torch.ones(n // 4, dtype=torch.float32, device=dev)
    dst = torch.empty_like(src)
    am.calibrate_copy(src, dst, n, stream)
    tc = event_ms(lambda: am.calibrate_copy(src, dst, n, stream), 10, stream)
    del src, dst
    return dict(mfma_bf16_tflops=round(flops / (t * 1e-3) / 1e12, 1), mfma_kernel_ms=round(t, 4),
                copy_gbs=round(2 * n / (tc * 1e-3) / 1e9, 1), copy_bytes=n,
                note="am::mfma_peak_kernel (v_mfma_f32_32x32x16_bf16 chains, no memory traffic) and "
                     "am::copy16_kernel (read + write counted)")


def event_ms(fn, iters, stream):
    import torch
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    start.record(stream)
    for _ in range(iters):
        fn()
    end.record(stream)
    end.synchronize()
    return start.elapsed_time(end) / iters


def _cfg(am, s, precision=0):
    return am.make_config(kind=s.kind, batch=s.batch, heads=s.heads, d_key=s.d_key, d_value=s.d_value,
                          d_hidden=s.d_hidden, poly_degree=s.poly_degree, chunk=s.chunk, omega_window=s.omega_window,
                          gate_mode=s.gate_mode, ns_steps=s.ns_steps, input_dtype=s.input_dtype, precision=precision)


def _dev(torch, a, dev):
    if a.dtype == np.uint16:
        a = a.view(np.int16)
    return torch.from_numpy(np.ascontiguousarray(a)).to(dev)


def _oracle_backward_sample(synth, inp, Tn):
    """The fp64 autograd oracle of the outer-loop backward on memory 0's first Tn tokens."""
    import oracle
    from oracle import backward as bw
    s = inp.spec
    cfg = oracle.config_from(s)
    f64 = lambda a: synth.bf16_bits_to_f32(a).astype(np.float64) if a.dtype == np.uint16 else a.astype(np.float64)
    ng = Tn if s.gate_mode == synth.PER_TOKEN else Tn // s.chunk
    dY = np.random.default_rng(5).standard_normal((Tn, s.d_value))
    bw.outer_grads(cfg, oracle.unflatten(cfg, inp.W0[0].astype(np.float64)),
                   oracle.unflatten(cfg, inp.S0[0].astype(np.float64)), f64(inp.K[0, :Tn]), f64(inp.Q[0, :Tn]),
                   f64(inp.V[0, :Tn]), inp.theta[0, :ng], inp.eta[0, :ng], inp.alpha[0, :ng], dY)
    return Tn


def stage_rooflines(torch, am, synth, dev, stream, only=None, cpu=False):
    """Stand-alone stages, each against its own roofline: the gate scan, Omega coefficients and
    feature map against HBM bandwidth (algorithmic bytes), Newton-Schulz against the bf16 matrix
    peak (algorithmic FLOPs).  Sizes are large enough for the launch to be bandwidth- or
    compute-bound (the per-chunk sizes inside a workload are far smaller): the scans over 256
    memories x 32768 tokens in chunks of 64, the feature map over the Omega workload's 262144 keys
    (width 32 -> 561), Newton-Schulz over 4096 gradient matrices of 128 x 64; the input prologue at
    the Newton-Schulz workload's shape: the keys' short convolution (128 memories x 32768 tokens x
    64, bf16 in and out, L2-normalised) and the gates of 8 x 32768 token inputs of width 512 for 16
    heads (per token: theta, eta, alpha, gamma; per chunk of 128: theta, eta, alpha); the feature map
    stage (degree 3 of 16384 width-32 vectors, and degree 2 of the 262144 keys projected to 64); the
    outer-loop backward (with its recorded forward) of the 64 -> 128 -> 64 per-token workload."""
    out = {}
    M, T, C, c, d = 256, 32768, 64, 4, 32
    th = torch.rand((M, T), device=dev)
    et = torch.rand((M, T), device=dev)
    al = torch.rand((M, T), device=dev)
    ga = torch.rand((M, T), device=dev)
    cW = torch.empty((M, T), device=dev)
    cS = torch.empty((M, T), device=dev)
    sc = torch.empty((M, T // C, 3), device=dev)
    R = C + c - 1
    oW = torch.empty((M, T // C, R), device=dev)
    oS = torch.empty((M, T // C, R), device=dev)
    NP = 262144
    X = torch.randn((NP, d), device=dev).to(torch.bfloat16).view(torch.int16)
    F = torch.empty((NP, (d + 1) * (d + 2) // 2), device=dev)
    NM = 4096
    G = torch.randn((NM, 128, 64), device=dev)
    Gout = torch.empty_like(G)
    CM, CT, CD, CH = 128, 32768, 64, 16
    KX = torch.randn((CM, CT, CD), device=dev).to(torch.bfloat16).view(torch.int16)
    KO = torch.empty_like(KX)
    Khist = torch.zeros((CM, 3, CD), dtype=torch.int16, device=dev)
    taps = 0.5 * torch.randn((CH, CD, 4), device=dev)
    cbias = 0.1 * torch.randn((CH, CD), device=dev)
    GB, DM = 8, 512
    U = torch.randn((GB, CT, DM), device=dev).to(torch.bfloat16).view(torch.int16)
    Wg = torch.randn((4, CH, DM), device=dev) / DM ** 0.5
    bg = torch.randn((4, CH), device=dev)
    gsc = torch.tensor(synth.GATE_SCALES, device=dev)
    gout = torch.empty((4, GB, CH, CT), device=dev)
    gout_c = torch.empty((3, GB, CH, CT // 128), device=dev)
    FN3, FD = 16384, 32
    F3 = (FD + 1) * (FD + 2) * (FD + 3) // 6
    X3 = torch.randn((FN3, FD), device=dev).to(torch.bfloat16).view(torch.int16)
    F3out = torch.empty((FN3, F3), device=dev)
    FDO = 64
    Pproj = torch.randn((FDO, F.shape[1]), device=dev) / F.shape[1] ** 0.5
    Fproj = torch.empty((NP, FDO), device=dev)
    # outer-loop backward at the 64 -> 128 -> 64 per-token workload's size (forward included)
    bi = synth.make_inputs(1, "stabilised")
    bs = bi.spec
    bmem = am.Memory(_cfg(am, bs), torch.from_numpy(bi.W0).to(dev), torch.from_numpy(bi.S0).to(dev))
    bdev = {k: _dev(torch, getattr(bi, k), dev) for k in ("K", "Q", "V", "theta", "eta", "alpha")}
    BT, BM = bs.T, bs.n_mem
    bws = torch.empty(bmem.backward_workspace_bytes(BT), dtype=torch.uint8, device=dev)
    bz = lambda *shape: torch.zeros(shape, dtype=torch.float32, device=dev)
    bout = dict(dK=bz(BM, BT, bs.d_key), dQ=bz(BM, BT, bs.d_key), dV=bz(BM, BT, bs.d_value), dth=bz(BM, BT),
                det=bz(BM, BT), dal=bz(BM, BT), dW0=bz(BM, bmem.P), dS0=bz(BM, bmem.P))
    bdY = torch.randn((BM, BT, bs.d_value), device=dev)
    W0d, S0d = torch.from_numpy(bi.W0).to(dev), torch.from_numpy(bi.S0).to(dev)

    def backward_call():
        bmem.set_state(W0d, S0d)
        bmem.update_backward(bdev["K"], bdev["Q"], bdev["V"], bdev["theta"], bdev["eta"], bdev["alpha"], BT, bdY,
                             bout["dK"], bout["dQ"], bout["dV"], bout["dth"], bout["det"], bout["dal"], bout["dW0"],
                             bout["dS0"], bws)
    bwork = BM * (BT // bs.chunk) * backward_flops_per_chunk(bs)
    # the same through per-chunk gates and 5 Newton-Schulz steps: every memory of the
    # 8 x 16, 64 -> 128 -> 64, chunk-128 workload over its first 4096 tokens (32 chunks)
    ni = synth.make_inputs(4, "literal", T=4096)
    ns_ = ni.spec
    nmem = am.Memory(_cfg(am, ns_), torch.from_numpy(ni.W0).to(dev), torch.from_numpy(ni.S0).to(dev))
    ndev = {k: _dev(torch, getattr(ni, k), dev) for k in ("K", "Q", "V", "theta", "eta", "alpha")}
    NT, NMm, NG = ns_.T, ns_.n_mem, ni.theta.shape[1]
    nws = torch.empty(nmem.backward_workspace_bytes(NT), dtype=torch.uint8, device=dev)
    nout = [bz(NMm, NT, ns_.d_key), bz(NMm, NT, ns_.d_key), bz(NMm, NT, ns_.d_value), bz(NMm, NG), bz(NMm, NG),
            bz(NMm, NG), bz(NMm, nmem.P), bz(NMm, nmem.P)]
    ndY = torch.randn((NMm, NT, ns_.d_value), device=dev)
    nW0, nS0 = torch.from_numpy(ni.W0).to(dev), torch.from_numpy(ni.S0).to(dev)

    def backward_ns_call():
        nmem.set_state(nW0, nS0)
        nmem.update_backward(ndev["K"], ndev["Q"], ndev["V"], ndev["theta"], ndev["eta"], ndev["alpha"], NT, ndY,
                             *nout, nws)
    nwork = NMm * (NT // ns_.chunk) * backward_flops_per_chunk(ns_)
    cases = [
        ("gate_scan", lambda: am.gate_scan(th, et, al, M, T, C, cW, cS, sc),
         M * T * (12 + 8) + M * (T // C) * 12, "hbm", f"{M} memories x {T} tokens, chunk {C}"),
        ("omega_coeffs", lambda: am.omega_coeffs(cW, cS, ga, None, M, T, C, c, oW, oS),
         M * T * 12 + M * (T // C) * R * 8, "hbm", f"{M} memories x {T} tokens, chunk {C}, window {c}"),
        ("poly_features", lambda: am.poly_features(X, synth.BF16, NP, d, F),
         NP * (2 * d + 4 * F.shape[1]), "hbm", f"{NP} bf16 vectors of width {d} -> {F.shape[1]} fp32"),
        ("newton_schulz", lambda: am.newton_schulz(G, NM, 128, 64, 5, synth.NS_COEFFS, synth.NS_EPS,
                                                   am.PREC_BF16X3, Gout),
         NM * ns_flops_per_matrix(128, 64, 5), "mfma", f"{NM} matrices 128x64, 5 steps, split bf16"),
        ("short_conv", lambda: am.short_conv(KX, synth.BF16, CM, CT, CD, CH, taps, cbias, Khist, True, KO, synth.BF16),
         CM * CT * CD * (2 + 2), "hbm", f"{CM} memories x {CT} tokens x {CD}, bf16 in/out, L2-normalised"),
        ("gates_per_token", lambda: am.gates(U, GB, CT, DM, CH, 4, Wg, bg, gsc, 1, gout),
         GB * CT * DM * 2 + 4 * GB * CH * CT * 4, "hbm", f"{GB} x {CT} inputs of width {DM}, 4 gates x {CH} heads"),
        ("gates_per_chunk", lambda: am.gates(U, GB, CT, DM, CH, 3, Wg[:3], bg[:3], gsc[:3], 128, gout_c),
         GB * CT * DM * 2 + 3 * GB * CH * (CT // 128) * 4, "hbm",
         f"{GB} x {CT} inputs of width {DM}, 3 gates x {CH} heads, pooled per chunk of 128"),
        ("feature_map_deg3", lambda: am.feature_map(X3, synth.BF16, FN3, FD, 3, F3out),
         FN3 * (2 * FD + 4 * F3), "hbm", f"{FN3} bf16 vectors of width {FD} -> {F3} fp32 (degree 3)"),
        ("feature_project_deg2", lambda: am.feature_map(X, synth.BF16, NP, d, 2, Fproj, P=Pproj, d_out=FDO),
         2 * NP * F.shape[1] * FDO, "mfma", f"{NP} bf16 vectors of width {d}: degree-2 features x {FDO}-row projection"),
        ("outer_backward", backward_call, bwork, "mfma",
         f"{bs.name} stabilised: forward with checkpoints and backward, {BM} memories x {BT} tokens",
         lambda: _oracle_backward_sample(synth, bi, 2 * bs.chunk)),
        ("outer_backward_ns5", backward_ns_call, nwork, "mfma",
         f"64 -> 128 -> 64 memory, chunk 128, per-chunk gates, 5 Newton-Schulz steps, forward with checkpoints "
         f"and backward, "
         f"{NMm} memories x {NT} tokens", lambda: _oracle_backward_sample(synth, ni, ns_.chunk)),
    ]
    # the memory variants and the general per-chunk path at the Newton-Schulz workload's shape
    # (128 memories, 64 -> 128 -> 64, chunk 128, 5 steps), over the first 4096 tokens
    def update_case(spec_over, flags, label, flops_fn):
        vi = synth.make_inputs(4, "literal", T=4096, **spec_over)
        vs = vi.spec
        vcfg = am.make_config(kind=vs.kind, batch=vs.batch, heads=vs.heads, d_key=vs.d_key, d_value=vs.d_value,
                              d_hidden=vs.d_hidden, poly_degree=vs.poly_degree, chunk=vs.chunk,
                              omega_window=vs.omega_window, gate_mode=vs.gate_mode, ns_steps=vs.ns_steps,
                              input_dtype=vs.input_dtype, flags=flags)
        W0v, S0v = torch.from_numpy(vi.W0).to(dev), torch.from_numpy(vi.S0).to(dev)
        vm = am.Memory(vcfg, W0v, S0v)
        vd = {k: _dev(torch, getattr(vi, k), dev) for k in ("K", "Q", "V", "theta", "eta", "alpha")}
        Yv = torch.empty((vs.n_mem, vs.T, vs.d_value), dtype=torch.float32, device=dev)

        def call():
            vm.set_state(W0v, S0v)
            vm.update_chunked(vd["K"], vd["Q"], vd["V"], vd["theta"], vd["eta"], vd["alpha"], None, vs.T, Yv)
        work = vs.n_mem * (vs.T // vs.chunk) * sum(flops_fn(vs).values())

        def sample():
            import oracle
            oracle.run_inputs(vi, mems=[0], T=2 * vs.chunk)
            return 2 * vs.chunk
        return (call, work, f"{label}: {vs.n_mem} memories x {vs.T} tokens, 64 -> 128 -> 64, chunk {vs.chunk}, "
                            f"{vs.ns_steps} Newton-Schulz steps", sample)
    if only is None or only in ("update_general_ns5", "update_residual_ns5", "update_gated_ns5"):
        ug = update_case({}, am.FLAG_NO_FUSED, "general per-chunk path (fused kernel off)", mlp_flops_per_chunk)
        ur = update_case(dict(kind=synth.MLP2_SILU_RESIDUAL), 0, "residual memory", mlp_flops_per_chunk)
        ugt = update_case(dict(kind=synth.MLP2_GATED), 0, "gated memory (W1, W3, W2)", gated_flops_per_chunk)
        cases += [("update_general_ns5",) + ug[:2] + ("mfma",) + ug[2:],
                  ("update_residual_ns5",) + ur[:2] + ("mfma",) + ur[2:],
                  ("update_gated_ns5",) + ugt[:2] + ("mfma",) + ugt[2:]]
    # the short convolution of K, Q, V before the update: three stand-alone convolutions writing the
    # convolved rows, then the update reading them, against the update that convolves while it
    # stages its operands (atlasmem_update_chunked_conv), both on the general per-product path, at
    # the Newton-Schulz workload's shape over 4096 tokens (keys and queries L2-normalised)
    if only is None or only in ("conv_then_update", "conv_folded_update"):
        ci = synth.make_inputs(4, "literal", T=4096, norm_k=False)
        cs = ci.spec
        ctaps, cvbias = synth.make_conv_params(4, cs.heads, cs.d_key, cs.d_value)
        ccfg = am.make_config(kind=cs.kind, batch=cs.batch, heads=cs.heads, d_key=cs.d_key, d_value=cs.d_value,
                              d_hidden=cs.d_hidden, chunk=cs.chunk, gate_mode=cs.gate_mode, ns_steps=cs.ns_steps,
                              input_dtype=cs.input_dtype, flags=am.FLAG_NO_FUSED)
        W0c, S0c = torch.from_numpy(ci.W0).to(dev), torch.from_numpy(ci.S0).to(dev)
        cmem = am.Memory(ccfg, W0c, S0c)
        cd = {k: _dev(torch, getattr(ci, k), dev) for k in ("K", "Q", "V", "theta", "eta", "alpha")}
        ctd = [torch.from_numpy(t).to(dev) for t in ctaps]
        cbd = [torch.from_numpy(b).to(dev) for b in cvbias]
        cconv = [torch.empty_like(cd[k]) for k in ("K", "Q", "V")]
        Yc = torch.empty((cs.n_mem, cs.T, cs.d_value), dtype=torch.float32, device=dev)
        ntok = cs.n_mem * cs.T

        def conv_then_update():
            cmem.set_state(W0c, S0c)
            cmem.reset_history()
            for x, o, tp, bs, d, l2 in ((cd["K"], cconv[0], ctd[0], cbd[0], cs.d_key, True),
                                         (cd["Q"], cconv[1], ctd[1], cbd[1], cs.d_key, True),
                                         (cd["V"], cconv[2], ctd[2], cbd[2], cs.d_value, False)):
                am.short_conv(x, synth.BF16, cs.n_mem, cs.T, d, cs.heads, tp, bs, None, l2, o, synth.BF16)
            cmem.update_chunked(cconv[0], cconv[1], cconv[2], cd["theta"], cd["eta"], cd["alpha"], None, cs.T, Yc)

        def conv_folded_update():
            cmem.set_state(W0c, S0c)
            cmem.reset_history()
            cmem.update_chunked_conv(cd["K"], cd["Q"], cd["V"], ctd, cbd, (True, True), cd["theta"], cd["eta"],
                                     cd["alpha"], None, cs.T, Yc)
        cwork = cs.n_mem * (cs.T // cs.chunk) * sum(mlp_flops_per_chunk(cs).values())
        row = 2 * (2 * cs.d_key + cs.d_value)  # bf16 bytes of one token's K, Q, V rows
        cases += [("conv_then_update", conv_then_update, cwork, "mfma",
                   f"short convolution of K, Q, V (three launches, convolved rows written: {3 * ntok * row / 1e9:.3f} "
                   f"GB of row traffic) then the update on the general path, {cs.n_mem} memories x {cs.T} tokens"),
                  ("conv_folded_update", conv_folded_update, cwork, "mfma",
                   f"the update convolving its K, Q, V rows while staging them (raw rows read by the update, "
                   f"{ntok * row / 1e9:.3f} GB, plus 8 B of inverse norms per token; {2 * ntok * row / 1e9:.3f} GB of "
                   f"row traffic saved), {cs.n_mem} memories x {cs.T} tokens")]
    # per-token retrieval at the per-token workload's shape (8 memories x 4096 tokens, chunk 64)
    if only is None or only == "update_per_token_retrieve":
        pi = synth.make_inputs(1, "stabilised", per_token_retrieve=True)
        ps = pi.spec
        pcfg = am.make_config(kind=ps.kind, batch=ps.batch, heads=ps.heads, d_key=ps.d_key, d_value=ps.d_value,
                              d_hidden=ps.d_hidden, chunk=ps.chunk, gate_mode=ps.gate_mode,
                              input_dtype=ps.input_dtype, flags=am.FLAG_PER_TOKEN_RETRIEVE)
        W0p, S0p = torch.from_numpy(pi.W0).to(dev), torch.from_numpy(pi.S0).to(dev)
        pm = am.Memory(pcfg, W0p, S0p)
        pd = {k: _dev(torch, getattr(pi, k), dev) for k in ("K", "Q", "V", "theta", "eta", "alpha")}
        Yp = torch.empty((ps.n_mem, ps.T, ps.d_value), dtype=torch.float32, device=dev)

        def ptr_call():
            pm.set_state(W0p, S0p)
            pm.update_chunked(pd["K"], pd["Q"], pd["V"], pd["theta"], pd["eta"], pd["alpha"], None, ps.T, Yp)
        def ptr_sample():
            import oracle
            oracle.run_inputs(pi, mems=[0], T=2 * ps.chunk)
            return 2 * ps.chunk
        cases.append(("update_per_token_retrieve", ptr_call,
                      ps.n_mem * (ps.T // ps.chunk) * sum(ptr_flops_per_chunk(ps).values()), "mfma",
                      f"{ps.name}: queries read the state after their own token, {ps.n_mem} memories x {ps.T} tokens",
                      ptr_sample))
    # decoding: one token per call through the streaming path (the chunk's update runs on the
    # call that completes it), 128 memories of the Newton-Schulz workload over two chunks.  Its
    # algorithmic bytes per call: every memory's weights read for the query (fp32), the token's
    # bf16 key, query and value, its fp32 output row.
    if only is None or only == "decode_one_token_calls":
        di = synth.make_inputs(4, "literal", T=256)
        ds = di.spec
        dm = am.Memory(_cfg(am, ds), torch.from_numpy(di.W0).to(dev), torch.from_numpy(di.S0).to(dev))
        W0d2, S0d2 = torch.from_numpy(di.W0).to(dev), torch.from_numpy(di.S0).to(dev)
        toks = []
        for t in range(ds.T):
            g0, g1 = t // ds.chunk, (t + 1) // ds.chunk
            toks.append(dict(K=_dev(torch, di.K[:, t:t + 1], dev), Q=_dev(torch, di.Q[:, t:t + 1], dev),
                             V=_dev(torch, di.V[:, t:t + 1], dev), th=_dev(torch, di.theta[:, g0:g1], dev),
                             et=_dev(torch, di.eta[:, g0:g1], dev), al=_dev(torch, di.alpha[:, g0:g1], dev)))
        Yd = torch.empty((ds.n_mem, 1, ds.d_value), dtype=torch.float32, device=dev)

        def decode_call():
            dm.set_state(W0d2, S0d2)
            for tk in toks:
                dm.update_chunked(tk["K"], tk["Q"], tk["V"], tk["th"], tk["et"], tk["al"], None, 1, Yd)
        dbytes = ds.T * ds.n_mem * (dm.P * 4 + (2 * ds.d_key + ds.d_value) * 2 + ds.d_value * 4)
        def decode_sample():
            import oracle
            oracle.run_inputs(di, mems=[0], T=ds.T)
            return ds.T
        cases.append(("decode_one_token_calls", decode_call, dbytes, "hbm",
                      f"{ds.n_mem} memories x {ds.T} tokens, one token per call (two chunks of {ds.chunk}), "
                      f"64 -> 128 -> 64, 5 Newton-Schulz steps", decode_sample))
    for case in cases:
        name, fn, work, bound, shape = case[:5]
        if only is not None and name != only:
            continue
        for _ in range(3):
            fn()
        t = event_ms(fn, 20, stream)
        if bound == "hbm":
            ach = work / (t * 1e-3) / 1e9
            out[name] = dict(bound="hbm", achieved=round(ach, 1), peak=PEAK_HBM_GBS, unit="GB/s",
                             frac=round(ach / PEAK_HBM_GBS, 4), algorithmic_bytes=int(work), ms=round(t, 5), shape=shape)
        else:
            ach = work / (t * 1e-3) / 1e12
            out[name] = dict(bound="mfma", achieved=round(ach, 2), peak=PEAK_BF16_TFLOPS, unit="TFLOP/s",
                             frac=round(ach / PEAK_BF16_TFLOPS, 5), algorithmic_flops=int(work), ms=round(t, 5),
                             shape=shape)
        if cpu and len(case) > 5:
            # the fp64 oracle on a small sample of the same workload, one process, for context
            # (repeated until half a second has passed, for a steadier rate)
            t0 = time.perf_counter()
            ntok, reps = 0, 0
            with np.errstate(all="ignore"):
                while reps == 0 or time.perf_counter() - t0 < 0.5:
                    ntok += case[5]()
                    reps += 1
            dt = time.perf_counter() - t0
            out[name]["cpu_oracle"] = dict(tokens_per_s=round(ntok / dt, 1), cores=1, kind="oracle",
                                           sample=f"memory 0, first {ntok // reps} tokens, {reps} runs, {dt:.2f} s")
    return out


def cpu_baseline(inp, seconds_target: float, cores: int):
    """The fp64 oracle, as it stands, on a bounded sample: `n` memories over their first T_s tokens,
    one memory per process."""
    import multiprocessing as mp

    import oracle
    s = inp.spec
    # probe the cost of one chunk of one memory (over four chunks)
    probe_chunks = min(4, s.T // s.chunk)
    t0 = time.perf_counter()
    with np.errstate(all="ignore"):
        oracle.run_inputs(inp, mems=[0], T=probe_chunks * s.chunk)
    one = max((time.perf_counter() - t0) / probe_chunks, 1e-4)
    chunks_per_mem = s.T // s.chunk
    n_mem = min(s.n_mem, cores)
    budget_chunks = max(1, int(seconds_target * cores / one / n_mem))
    n_chunks = min(chunks_per_mem, budget_chunks)
    Ts = n_chunks * s.chunk
    mems = list(range(n_mem))
    global _CPU_INPUTS
    _CPU_INPUTS = inp          # inherited by the forked workers, not pickled
    ctx = mp.get_context("fork")
    t0 = time.perf_counter()
    with ctx.Pool(cores, initializer=_limit_threads) as pool:
        pool.map(_oracle_one, [(m, Ts) for m in mems], chunksize=1)
    wall = time.perf_counter() - t0
    return dict(value=n_mem * Ts / wall, unit="tokens/s", cores=cores, kind="oracle", cpu_model=cpu_model(),
                sample=f"{n_mem} memories x first {Ts} tokens ({n_chunks} of {chunks_per_mem} chunks) of "
                       f"{s.name}, fp64 NumPy, one memory per process, {wall:.1f} s wall")


def _limit_threads():
    try:
        from threadpoolctl import threadpool_limits
        threadpool_limits(1)
    except Exception:
        pass


_CPU_INPUTS = None


def _oracle_one(args):
    import oracle
    m, Ts = args
    with np.errstate(all="ignore"):
        oracle.run_inputs(_CPU_INPUTS, mems=[m], T=Ts)
    return m


def config_lines(torch, am, synth, dev, stream, steps=5, warmup=2) -> dict:
    """Every smaller workload's whole update call timed like the main line (state restored before
    each step, inputs resident): tokens/s and, for the MLP memories, algorithmic TFLOP/s against
    the bf16 matrix peak.  Workloads 1-3 run their stabilised inputs (the literal ones overflow
    fp32, which leaves nothing meaningful to time); workload 0 is the literal linear memory."""
    out = {}
    for idx, variant in ((0, "literal"), (1, "stabilised"), (2, "stabilised"), (3, "stabilised")):
        inp = synth.make_inputs(idx, variant)
        s = inp.spec
        K, Q, V = (_dev(torch, a, dev) for a in (inp.K, inp.Q, inp.V))
        th, et, al = (_dev(torch, a, dev) for a in (inp.theta, inp.eta, inp.alpha))
        ga = None if inp.gamma is None else _dev(torch, inp.gamma, dev)
        W0, S0 = _dev(torch, inp.W0, dev), _dev(torch, inp.S0, dev)
        mem = am.Memory(_cfg(am, s), W0, S0)
        Y = torch.empty((s.n_mem, s.T, s.d_value), dtype=torch.float32, device=dev)

        def step():
            mem.set_state(W0, S0)
            mem.reset_history()
            mem.update_chunked(K, Q, V, th, et, al, ga, s.T, Y)

        for _ in range(warmup):
            step()
        torch.cuda.synchronize()
        ms = event_ms(step, steps, stream)
        tokens = s.n_mem * s.T
        line = dict(workload=s.name, variant=variant, ms=round(ms, 4), tokens_per_s=round(tokens / (ms * 1e-3), 1))
        if s.kind == synth.LINEAR:
            line["path"] = "lin_kernel (one launch, sequential over tokens)"
        else:
            line["path"] = {1: "fused_pt_kernel (one launch per block of chunks, one workgroup per memory)",
                            2: "general path (per-product launches, split-K)",
                            3: "hsplit_kernel (one launch per chunk, 8 workgroups per memory)"}[idx]
            fl = sum(mlp_flops_per_chunk(s).values()) * (s.T // s.chunk) * s.n_mem
            tf = fl / (ms * 1e-3) / 1e12
            line.update(tflops=round(tf, 3), frac_bf16_peak=round(tf / PEAK_BF16_TFLOPS, 6))
        out[f"workload_{idx}"] = line
        mem.close()
        del K, Q, V, th, et, al, ga, W0, S0, Y
    return out


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", type=int, default=4)
    ap.add_argument("--variant", default="literal")
    ap.add_argument("--precision", type=int, default=0, help="0 auto (split bf16), 1 bf16, 2 split bf16, 3 fp32 operands")
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=15.0)
    ap.add_argument("--no-check", action="store_true")
    ap.add_argument("--no-stages", action="store_true", help="skip the stand-alone stage rooflines")
    ap.add_argument("--no-fused", action="store_true",
                    help="time the general per-product path (ATLASMEM_FLAG_NO_FUSED) for the workload")
    ap.add_argument("--only-stage", default=None,
                    help="time only this stand-alone stage (for profiling) and print its JSON object")
    ap.add_argument("--copy-calibration", type=int, default=0,
                    help="also run one device-to-device copy of this many MiB (counter calibration)")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: the memories shard over (batch, head) with no exchange, "
              "and this build runs and reports the single-GPU share. Use --gpus 1.", file=sys.stderr)
        sys.exit(2)

    import torch

    from test_learned_neural_amd import atlasmem as am
    from test_learned_neural_amd import synth

    torch.cuda.set_device(0)
    dev = "cuda:0"
    stream = torch.cuda.current_stream()
    if args.only_stage:
        st = stage_rooflines(torch, am, synth, dev, stream, only=args.only_stage)
        if not st:
            print(f"no stage named {args.only_stage}", file=sys.stderr)
            sys.exit(2)
        print(json.dumps(st))
        return
    inp = synth.make_inputs(args.workload, args.variant)
    s = inp.spec

    def t(a):
        if a.dtype == np.uint16:
            a = a.view(np.int16)
        return torch.from_numpy(np.ascontiguousarray(a)).to(dev)

    K, Q, V = t(inp.K), t(inp.Q), t(inp.V)
    th, et, al = t(inp.theta), t(inp.eta), t(inp.alpha)
    ga = None if inp.gamma is None else t(inp.gamma)
    W0, S0 = t(inp.W0), t(inp.S0)
    cfg = am.make_config(kind=s.kind, batch=s.batch, heads=s.heads, d_key=s.d_key, d_value=s.d_value,
                         d_hidden=s.d_hidden, poly_degree=s.poly_degree, chunk=s.chunk, omega_window=s.omega_window,
                         gate_mode=s.gate_mode, ns_steps=s.ns_steps, input_dtype=s.input_dtype,
                         precision=args.precision, flags=am.FLAG_NO_FUSED if args.no_fused else 0)
    mem = am.Memory(cfg, W0, S0)
    Y = torch.empty((s.n_mem, s.T, s.d_value), dtype=torch.float32, device=dev)
    if args.copy_calibration:
        n = args.copy_calibration << 20
        src = torch.ones(n // 4, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        am.calibrate_copy(src, dst, n, stream)
        torch.cuda.synchronize()
        del src, dst

    upd_start = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps)]
    upd_end = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps)]

    def step(i=None):
        mem.set_state(W0, S0)
        mem.reset_history()
        if i is not None:
            upd_start[i].record(stream)
        mem.update_chunked(K, Q, V, th, et, al, ga, s.T, Y)
        if i is not None:
            upd_end[i].record(stream)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    start.record(stream)
    for i in range(args.steps):
        step(i)
    end.record(stream)
    end.synchronize()
    ms = start.elapsed_time(end) / args.steps
    wall_ms = (time.perf_counter() - t0) * 1e3 / args.steps
    upd_ms = sum(a.elapsed_time(b) for a, b in zip(upd_start, upd_end)) / args.steps
    tokens = s.n_mem * s.T
    value = tokens / (ms * 1e-3)

    # algorithmic FLOPs of the whole step and per stage
    nchunks = s.T // s.chunk
    per_chunk = mlp_flops_per_chunk(s)
    step_flops = sum(per_chunk.values()) * nchunks * s.n_mem
    path_tflops = step_flops / (ms * 1e-3) / 1e12

    # dominant kernel: the update call.  On the fused path it is one launch of the whole-call
    # kernel; on the general path it is the whole per-chunk launch sequence.
    fused = (s.kind == synth.MLP2_SILU and s.gate_mode == synth.PER_CHUNK and s.ns_steps > 0 and s.d_key == 64
             and s.d_value == 64 and s.d_hidden == 128 and s.chunk % 64 == 0 and args.precision in (am.PREC_AUTO, am.PREC_BF16X3, am.PREC_BF16)
             and not args.no_fused)
    ach = step_flops / (upd_ms * 1e-3) / 1e12
    roof = dict(bound="mfma", achieved=round(ach, 2), peak=PEAK_BF16_TFLOPS, unit="TFLOP/s",
                frac=round(ach / PEAK_BF16_TFLOPS, 5),
                traffic=(measured_traffic() if fused and s.T == 32768 and s.n_mem == 128 else None),
                kernel="am::fz::fused_ns_kernel" if fused else "update_chunked launch sequence",
                launch=((f"{16 * ((s.n_mem + 7) // 8)} workgroups x 256 threads, two per memory (one per row set, "
                         f"on two CUs of one XCD), cooperative, all {nchunks} chunks" if s.n_mem <= 128 else
                         f"{s.n_mem} workgroups x 512 threads, one memory each, all {nchunks} chunks")
                        if fused else "per-chunk launches"),
                avg_launch_ms=round(upd_ms, 5),
                algorithmic_flops_per_launch=int(step_flops))

    calib = None if args.no_stages else calibration(torch, am, dev, stream)
    if calib:
        roof["peak_measured"] = calib["mfma_bf16_tflops"]
        roof["frac_of_measured_peak"] = round(ach / calib["mfma_bf16_tflops"], 5)
    if fused and s.T == 32768 and s.n_mem == 128:
        rp = rocprof_kernel_ms()
        roof["kernel_sources_sha256_16"] = sources_sha16()
        roof["rocprof_avg_launch_ms"] = None if rp is None else round(rp, 5)
        roof["frac_rocprof"] = None if rp is None else round(step_flops / (rp * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 5)

    check = None
    if not args.no_check:
        import oracle
        Wg = torch.empty((s.n_mem, mem.P), dtype=torch.float32, device=dev)
        Sg = torch.empty_like(Wg)
        st = mem.get_state(Wg, Sg)
        m = s.n_mem // 2
        Yr, Wr, Sr = oracle.run_inputs(inp, mems=[m])

        def rel(x, r):
            return float(np.abs(x - r).max() / np.abs(r).max())
        check = dict(memory=m, status=st, Y=rel(Y[m].cpu().numpy(), Yr[0]), W=rel(Wg[m].cpu().numpy(), Wr[0]),
                     S=rel(Sg[m].cpu().numpy(), Sr[0]))

    stages = None if args.no_stages else stage_rooflines(torch, am, synth, dev, stream, cpu=not args.no_cpu)
    if calib and stages:
        for v in stages.values():  # HBM-bound stages also against the copy rate this chip reaches
            if v.get("bound") == "hbm":
                v["frac_of_measured_copy"] = round(v["achieved"] / calib["copy_gbs"], 4)
    configs = None if args.no_stages else config_lines(torch, am, synth, dev, stream)

    cpu = None
    if not args.no_cpu:
        cores = min(os.cpu_count() or 1, 16)
        cpu = cpu_baseline(inp, args.cpu_seconds, cores)

    out = {
        "metric": METRIC,
        "value": round(value, 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": {1: "bf16", 3: "f32"}.get(args.precision, "bf16x3"),
        "data": "synthetic (seeded, generator inputs resident in HBM)",
        "config": {"workload": s.name, "batch": s.batch, "heads": s.heads, "T": s.T, "chunk": s.chunk,
                   "d_key": s.d_key, "d_hidden": s.d_hidden, "d_value": s.d_value, "ns_steps": s.ns_steps,
                   "gate_mode": "per_chunk" if s.gate_mode else "per_token", "variant": args.variant,
                   "key_norm": "l2" if s.norm_k else "none", "query_norm": "l2" if s.norm_q else "none",
                   "value_norm": "l2" if s.norm_v else "none",
                   "tokens_per_step": tokens, "parallelism": "single GPU; memories spread over workgroups",
                   **({"path": "general (fused kernels off)"} if args.no_fused else {})},
        "path_tflops": round(path_tflops, 2),
        "path_frac_bf16_peak": round(path_tflops / PEAK_BF16_TFLOPS, 5),
        "wall_ms_per_step": round(wall_ms, 4),
        "roofline": roof,
        "cpu_baseline": cpu,
        "check": check,
        "calibration": calib,
        "configs": configs,
        "stages": stages,
    }
    print(json.dumps(out))


if __name__ == "__main__":
    main()
