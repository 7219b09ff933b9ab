"""Shared helpers of the GPU tests: generator inputs on the device, one library run, error metric."""

from __future__ import annotations

import sys

import numpy as np

import oracle
from test_learned_neural_amd import atlasmem as am
from test_learned_neural_amd import synth

DEV = "cuda:0"
BF16_TOL = 2e-2   # max relative error for bf16-input workloads (Y, W, S)
F32_TOL = 1e-4    # max relative error for fp32 workloads


def log(msg: str):
    print(msg, flush=True)
    sys.stdout.flush()


def maxrel(x, r) -> float:
    """max |x - r| / max |r| over a whole tensor (every memory at once)."""
    x = np.asarray(x, dtype=np.float64)
    r = np.asarray(r, dtype=np.float64)
    den = float(np.max(np.abs(r))) if r.size else 0.0
    if den == 0.0:
        return float(np.max(np.abs(x))) if x.size else 0.0
    return float(np.max(np.abs(x - r)) / den)


def config_for(spec, precision=am.PREC_AUTO, output_dtype=am.F32, flags=0):
    if getattr(spec, "per_token_retrieve", False):
        flags |= am.FLAG_PER_TOKEN_RETRIEVE
    return am.make_config(kind=spec.kind, batch=spec.batch, heads=spec.heads, d_key=spec.d_key,
                          d_value=spec.d_value, d_hidden=spec.d_hidden, poly_degree=spec.poly_degree,
                          chunk=spec.chunk, omega_window=spec.omega_window, gate_mode=spec.gate_mode,
                          ns_steps=spec.ns_steps, input_dtype=spec.input_dtype, output_dtype=output_dtype,
                          precision=precision, flags=flags)


def to_dev(a: np.ndarray):
    import torch
    if a.dtype == np.uint16:
        a = a.view(np.int16)
    return torch.from_numpy(np.ascontiguousarray(a)).to(DEV)


def segment(inp, t0: int, t1: int):
    """Device tensors of the inputs for tokens [t0, t1) of every memory."""
    s = inp.spec
    g0, g1 = (t0, t1) if s.gate_mode == synth.PER_TOKEN else (t0 // s.chunk, t1 // s.chunk)
    out = dict(K=to_dev(inp.K[:, t0:t1]), Q=to_dev(inp.Q[:, t0:t1]), V=to_dev(inp.V[:, t0:t1]),
               theta=to_dev(inp.theta[:, g0:g1]), eta=to_dev(inp.eta[:, g0:g1]), alpha=to_dev(inp.alpha[:, g0:g1]),
               gamma=None if inp.gamma is None else to_dev(inp.gamma[:, t0:t1]))
    return out


def y_to_np(Y):
    import torch
    if Y.dtype == torch.int16:
        u = Y.cpu().numpy().view(np.uint16)
        return synth.bf16_bits_to_f32(u).astype(np.float64)
    return Y.cpu().numpy().astype(np.float64)


def run_gpu(inp, splits=None, precision=am.PREC_AUTO, output_dtype=am.F32, with_y=True, W0=None, S0=None, flags=0):
    """Run the library over the generator inputs, one update call per segment in `splits`
    (token boundaries, default one call over all of T).  Returns (Y, W, S, status) as float64."""
    import torch
    s = inp.spec
    T = s.T
    splits = [0, T] if splits is None else splits
    cfg = config_for(s, precision, output_dtype, flags)
    W0 = to_dev(inp.W0 if W0 is None else W0)
    S0 = to_dev(inp.S0 if S0 is None else S0)
    mem = am.Memory(cfg, W0, S0)
    if output_dtype == am.BF16:
        Y = torch.zeros((s.n_mem, T, s.d_value), dtype=torch.int16, device=DEV)
    else:
        Y = torch.full((s.n_mem, T, s.d_value), float("nan"), dtype=torch.float32, device=DEV)
    for a, b in zip(splits[:-1], splits[1:]):
        seg = segment(inp, a, b)
        y = torch.empty((s.n_mem, b - a, s.d_value), dtype=Y.dtype, device=DEV) if with_y else None
        mem.update_chunked(seg["K"], seg["Q"], seg["V"], seg["theta"], seg["eta"], seg["alpha"], seg["gamma"],
                           b - a, y)
        if with_y:
            Y[:, a:b] = y
    W = torch.empty((s.n_mem, mem.P), dtype=torch.float32, device=DEV)
    S = torch.empty_like(W)
    status = mem.get_state(W, S)
    torch.cuda.synchronize()
    mem.close()
    return y_to_np(Y), W.cpu().numpy().astype(np.float64), S.cpu().numpy().astype(np.float64), status


def split_params(spec, flat):
    """[..., P] -> list of per-matrix arrays [..., n_i] (W1, W2 or W)."""
    if spec.kind == synth.LINEAR:
        return [flat]
    n1 = spec.d_hidden * spec.d_in
    if spec.kind == synth.MLP2_GATED:
        return [flat[..., :n1], flat[..., n1:2 * n1], flat[..., 2 * n1:]]
    return [flat[..., :n1], flat[..., n1:]]


def compare(name, spec, got, ref, tol, check_state=True):
    """Print and return the max relative errors of Y and of every weight / momentum matrix."""
    Yg, Wg, Sg = got[:3]
    Yr, Wr, Sr = ref[:3]
    errs = {"Y": maxrel(Yg, Yr)}
    names = ["1", "3", "2"] if spec.kind == synth.MLP2_GATED else ["1", "2"]  # storage order of the matrices
    if check_state:
        for i, (a, b) in enumerate(zip(split_params(spec, Wg), split_params(spec, Wr))):
            errs[f"W{names[i]}"] = maxrel(a, b)
        for i, (a, b) in enumerate(zip(split_params(spec, Sg), split_params(spec, Sr))):
            errs[f"S{names[i]}"] = maxrel(a, b)
    log(f"PARITY {name}: " + " ".join(f"{k}={v:.3e}" for k, v in errs.items()) + f" (tol {tol:g})")
    return errs


def oracle_run(inp, mems=None, T=None, processes=1):
    with np.errstate(all="ignore"):
        return oracle.run_inputs(inp, mems=mems, T=T, processes=processes)


# ----------------------------------------------------------------------------- per-chunk parity
#
# The stabilised workloads' state shrinks geometrically (W = 0 attracts under the forgetting gate),
# so a whole-tensor max|x - r| / max|r| is set by the first chunks and cannot see the late ones.
# These checks scale every chunk of every memory by its own magnitude, down to FLOOR: a million
# times fp32's smallest normal (1.2e-38), so that even the low halves of the split products
# (2^-8 of the high ones) stay normal and the relative error still means something.

FLOOR = 1e-32


def per_chunk_y_errors(Yg, Yr, chunk, floor=FLOOR):
    """Per memory and chunk k: max|Yg - Yr| / max|Yr| over the chunk's rows, for every chunk whose
    reference magnitude is at least `floor`.  Yg, Yr: [m, T, d_v].  Returns (worst error, number of
    chunks checked per memory, the last chunk checked per memory)."""
    Yg = np.asarray(Yg, dtype=np.float64)
    Yr = np.asarray(Yr, dtype=np.float64)
    m, T = Yr.shape[:2]
    worst, counts, last = 0.0, [], []
    for i in range(m):
        n, lk = 0, -1
        for k, s in enumerate(range(0, T, chunk)):
            r = Yr[i, s:s + chunk]
            scale = float(np.max(np.abs(r)))
            if not scale >= floor:
                continue
            g = Yg[i, s:s + chunk]
            err = float(np.max(np.abs(g - r))) / scale if np.all(np.isfinite(g)) else float("inf")
            worst = max(worst, err)
            n += 1
            lk = k
        counts.append(n)
        last.append(lk)
    return worst, counts, last


def oracle_boundaries(inp, mems, T=None):
    """The oracle's Y and its (W, S) at every chunk boundary (flat [P] vectors) of each memory."""
    cfg = oracle.config_from(inp.spec)
    s = inp.spec
    T = s.T if T is None else T
    ng = T if s.gate_mode == synth.PER_TOKEN else -(-T // s.chunk)
    out = []
    with np.errstate(all="ignore"):
        for m in mems:
            r = oracle.run_memory(cfg, oracle.unflatten(cfg, inp.W0[m]), oracle.unflatten(cfg, inp.S0[m]),
                                  inp.values("K", [m])[0, :T], inp.values("Q", [m])[0, :T],
                                  inp.values("V", [m])[0, :T], inp.values("theta", [m])[0, :ng],
                                  inp.values("eta", [m])[0, :ng], inp.values("alpha", [m])[0, :ng],
                                  None if inp.gamma is None else inp.values("gamma", [m])[0, :T],
                                  keep_boundaries=True)
            bounds = [(oracle.flatten(w), oracle.flatten(sm)) for w, sm in r.boundary_states]
            out.append((r.Y, bounds))
    return out


def boundary_state_errors(spec, got_states, ref_bounds, chunk_ids, floor=FLOOR):
    """Relative error of every weight and momentum matrix at the given chunk boundaries, each matrix
    scaled by its own reference magnitude, where that magnitude is at least `floor`.
    got_states[j] = (W [P], S [P]) at boundary chunk_ids[j] of one memory; ref_bounds[k] = the
    oracle's (W, S) at boundary k.  Returns (worst error, last boundary checked)."""
    worst, last = 0.0, -1
    for (Wg, Sg), k in zip(got_states, chunk_ids):
        Wr, Sr = ref_bounds[k]
        for a, b in list(zip(split_params(spec, Wg), split_params(spec, Wr))) + \
                list(zip(split_params(spec, Sg), split_params(spec, Sr))):
            scale = float(np.max(np.abs(b)))
            if not scale >= floor:
                continue
            err = float(np.max(np.abs(np.asarray(a, dtype=np.float64) - b))) / scale
            worst = max(worst, err if np.isfinite(err) else float("inf"))
            last = max(last, k)
    return worst, last


def run_gpu_states(inp, mems, calls, chunks_per_call, precision=am.PREC_AUTO, flags=0):
    """The library over the given memories only (their inputs sliced out, so the handle holds just
    them), in `calls` update calls of `chunks_per_call` chunks each, with the state read after every
    call.  Returns (Y [m, T, d_v], [(W [m, P], S [m, P]) after each call])."""
    import dataclasses
    import torch
    s = inp.spec
    sub = dataclasses.replace(inp, spec=dataclasses.replace(s, batch=1, heads=len(mems)),
                              **{k: (None if getattr(inp, k) is None else getattr(inp, k)[np.asarray(mems)])
                                 for k in ("K", "Q", "V", "theta", "eta", "alpha", "gamma", "W0", "S0")})
    ss = sub.spec
    cfg = config_for(ss, precision, am.F32, flags)
    mem = am.Memory(cfg, to_dev(sub.W0), to_dev(sub.S0))
    T = calls * chunks_per_call * ss.chunk
    Y = torch.full((ss.n_mem, T, ss.d_value), float("nan"), dtype=torch.float32, device=DEV)
    W = torch.empty((ss.n_mem, mem.P), dtype=torch.float32, device=DEV)
    S = torch.empty_like(W)
    states = []
    step = chunks_per_call * ss.chunk
    for j in range(calls):
        a, b = j * step, (j + 1) * step
        seg = segment(sub, a, b)
        y = torch.empty((ss.n_mem, b - a, ss.d_value), dtype=torch.float32, device=DEV)
        mem.update_chunked(seg["K"], seg["Q"], seg["V"], seg["theta"], seg["eta"], seg["alpha"], seg["gamma"],
                           b - a, y)
        Y[:, a:b] = y
        st = mem.get_state(W, S)
        assert st == am.OK, st
        states.append((W.cpu().numpy().astype(np.float64), S.cpu().numpy().astype(np.float64)))
    torch.cuda.synchronize()
    mem.close()
    return y_to_np(Y), states


def handle_update_run(inp):
    """One update_chunked call on a handle over the whole input (fp32 output): (Y, W, S) on the host."""
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


def static_update_run(inp):
    """The allocation-free update (one workgroup per memory) over the whole input: (Y, W, S)."""
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
