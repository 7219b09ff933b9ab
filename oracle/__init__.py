"""fp64 CPU oracle of the neural-memory update (test infrastructure only).

Only the test suite, the smoke check and the benchmark's CPU-baseline leg may
import this package; the library itself never does.
"""

from .neural_memory import (  # noqa: F401
    LINEAR, MLP2_SILU, MLP2_SILU_RESIDUAL, MLP2_GATED, PER_TOKEN, PER_CHUNK, MemoryConfig, MemoryResult, flatten, loss, loss_grad,
    memory_apply, newton_schulz, poly_feature_count, poly_features, run_many, run_memory, silu,
    silu_prime, unflatten,
)


def config_from(spec) -> MemoryConfig:
    """MemoryConfig from any object carrying the workload fields (kind, d_key, ...)."""
    return MemoryConfig(kind=spec.kind, d_key=spec.d_key, d_value=spec.d_value, d_hidden=spec.d_hidden,
                        poly_degree=spec.poly_degree, chunk=spec.chunk, omega_window=spec.omega_window,
                        gate_mode=spec.gate_mode, ns_steps=spec.ns_steps,
                        per_token_retrieve=getattr(spec, "per_token_retrieve", False))


def run_inputs(inputs, mems=None, T=None, processes: int = 1):
    """Run the oracle on a generated input set (optionally a subset of memories / a prefix of T).

    Returns (Y [m, T, d_v], W [m, P], S [m, P]) in float64."""
    import numpy as np
    s = inputs.spec
    cfg = config_from(s)
    mems = list(range(s.n_mem)) if mems is None else list(mems)
    T = s.T if T is None else T
    ng = T if s.gate_mode == PER_TOKEN else -(-T // s.chunk)
    K = inputs.values("K", mems)[:, :T]
    Q = inputs.values("Q", mems)[:, :T]
    V = inputs.values("V", mems)[:, :T]
    th = inputs.values("theta", mems)[:, :ng]
    et = inputs.values("eta", mems)[:, :ng]
    al = inputs.values("alpha", mems)[:, :ng]
    ga = None if inputs.gamma is None else inputs.values("gamma", mems)[:, :T]
    W0 = inputs.W0[np.asarray(mems)].astype(np.float64)
    S0 = inputs.S0[np.asarray(mems)].astype(np.float64)
    return run_many(cfg, W0, S0, K, Q, V, th, et, al, ga, processes=processes)
