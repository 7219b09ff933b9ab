"""Thin ctypes binding of libatlasmem.so (argument marshalling only).

Every function takes torch tensors (or raw integer device pointers) and passes
their device addresses to the C ABI of the same name; all computation happens
in the library's HIP kernels.  The library must have been built
(`python -m test_learned_neural_amd.build`); loading raises if it is missing.
"""

from __future__ import annotations

import ctypes
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libatlasmem.so")

OK, E_INVALID, E_SHAPE, E_UNSUPPORTED, E_DEVICE, E_NOMEM, E_NONFINITE = range(7)
LINEAR, MLP2_SILU, MLP2_SILU_RESIDUAL, MLP2_GATED = 0, 1, 2, 3
PER_TOKEN, PER_CHUNK = 0, 1
F32, BF16 = 0, 1
PREC_AUTO, PREC_BF16, PREC_BF16X3, PREC_F32 = 0, 1, 2, 3
FLAG_NO_FUSED = 1
FLAG_PER_TOKEN_RETRIEVE = 2
FLAG_NO_CHUNK_LOOP = 4
FLAG_NO_SPLIT_K = 8
ABI_VERSION = 2

EXPORTS = (
    "atlasmem_abi_version", "atlasmem_status_string", "atlasmem_param_count", "atlasmem_create",
    "atlasmem_update_chunked", "atlasmem_flush", "atlasmem_pending", "atlasmem_retrieve", "atlasmem_get_state",
    "atlasmem_set_state",
    "atlasmem_reset_history", "atlasmem_destroy", "atlasmem_gate_scan", "atlasmem_omega_coeffs",
    "atlasmem_poly_features", "atlasmem_newton_schulz", "atlasmem_short_conv", "atlasmem_gates",
    "atlasmem_feature_map", "atlasmem_backward_workspace_bytes", "atlasmem_update_backward",
    "atlasmem_calibrate_mfma", "atlasmem_calibrate_copy", "atlasmem_update_chunked_static",
    "atlasmem_update_chunked_conv",
)
STATIC_MAX_MEMORIES = 128


class Config(ctypes.Structure):
    _fields_ = [
        ("abi_version", ctypes.c_int32), ("memory_kind", ctypes.c_int32), ("batch", ctypes.c_int32),
        ("heads", ctypes.c_int32), ("d_key", ctypes.c_int32), ("d_value", ctypes.c_int32),
        ("d_hidden", ctypes.c_int32), ("poly_degree", ctypes.c_int32), ("chunk", ctypes.c_int32),
        ("omega_window", ctypes.c_int32), ("gate_mode", ctypes.c_int32), ("ns_steps", ctypes.c_int32),
        ("ns_a", ctypes.c_float), ("ns_b", ctypes.c_float), ("ns_c", ctypes.c_float), ("ns_eps", ctypes.c_float),
        ("input_dtype", ctypes.c_int32), ("output_dtype", ctypes.c_int32), ("precision", ctypes.c_int32),
        ("flags", ctypes.c_int32),
    ]


class ConvParams(ctypes.Structure):
    _fields_ = [("taps_k", ctypes.c_void_p), ("taps_q", ctypes.c_void_p), ("taps_v", ctypes.c_void_p),
                ("bias_k", ctypes.c_void_p), ("bias_q", ctypes.c_void_p), ("bias_v", ctypes.c_void_p),
                ("l2norm_k", ctypes.c_int32), ("l2norm_q", ctypes.c_int32)]


class AtlasMemError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {status_string(status)} (status {status})")


_lib = None
_vp = ctypes.c_void_p
_i64 = ctypes.c_int64
_i32 = ctypes.c_int32
_f = ctypes.c_float


def load():
    """Load the HIP library (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is missing: build it with `python -m test_learned_neural_amd.build`")
    lib = ctypes.CDLL(LIB_PATH)
    sig = {
        "atlasmem_abi_version": ([], ctypes.c_int),
        "atlasmem_status_string": ([ctypes.c_int], ctypes.c_char_p),
        "atlasmem_param_count": ([ctypes.POINTER(Config)], _i64),
        "atlasmem_create": ([ctypes.POINTER(Config), _vp, _vp, _vp, ctypes.POINTER(_vp)], ctypes.c_int),
        "atlasmem_update_chunked": ([_vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _i64, _vp, _vp], ctypes.c_int),
        "atlasmem_flush": ([_vp, _vp, _vp, _vp, _vp], ctypes.c_int),
        "atlasmem_pending": ([_vp], _i64),
        "atlasmem_retrieve": ([_vp, _vp, _i64, _vp, _vp], ctypes.c_int),
        "atlasmem_get_state": ([_vp, _vp, _vp, _vp], ctypes.c_int),
        "atlasmem_set_state": ([_vp, _vp, _vp, _vp], ctypes.c_int),
        "atlasmem_reset_history": ([_vp, _vp], ctypes.c_int),
        "atlasmem_destroy": ([_vp], None),
        "atlasmem_gate_scan": ([_vp, _vp, _vp, _i64, _i64, _i32, _vp, _vp, _vp, _vp], ctypes.c_int),
        "atlasmem_omega_coeffs": ([_vp, _vp, _vp, _vp, _i64, _i64, _i32, _i32, _vp, _vp, _vp], ctypes.c_int),
        "atlasmem_poly_features": ([_vp, _i32, _i64, _i32, _vp, _vp], ctypes.c_int),
        "atlasmem_newton_schulz": ([_vp, _i64, _i32, _i32, _i32, _f, _f, _f, _f, _i32, _vp, _vp], ctypes.c_int),
        "atlasmem_short_conv": ([_vp, _i32, _i64, _i64, _i32, _i32, _vp, _vp, _vp, _i32, _vp, _i32, _vp, _vp],
                                ctypes.c_int),
        "atlasmem_gates": ([_vp, _i64, _i64, _i32, _i32, _i32, _vp, _vp, _vp, _i32, _vp, _vp], ctypes.c_int),
        "atlasmem_feature_map": ([_vp, _i32, _i64, _i32, _i32, _vp, _vp, _i32, _vp, _vp], ctypes.c_int),
        "atlasmem_backward_workspace_bytes": ([_vp, _i64], _i64),
        "atlasmem_update_backward": ([_vp] * 8 + [_i64] + [_vp] * 5 + [_i64] + [_vp] * 10, ctypes.c_int),
        "atlasmem_calibrate_mfma": ([_i64, _i32, _vp, _vp], ctypes.c_int),
        "atlasmem_calibrate_copy": ([_vp, _vp, _i64, _vp], ctypes.c_int),
        "atlasmem_update_chunked_static": ([ctypes.POINTER(Config)] + [_vp] * 6 + [_i64] + [_vp] * 5, ctypes.c_int),
        "atlasmem_update_chunked_conv": ([_vp, _vp, _vp, _vp, ctypes.POINTER(ConvParams), _vp, _vp, _vp, _vp, _i64, _vp,
                                          _vp], ctypes.c_int),
    }
    for name, (args, res) in sig.items():
        fn = getattr(lib, name)
        fn.argtypes = args
        fn.restype = res
    _lib = lib
    return lib


def status_string(status: int) -> str:
    return load().atlasmem_status_string(int(status)).decode()


def _ptr(x):
    """Device address of a tensor (or an int address, or None -> NULL)."""
    if x is None:
        return None
    if isinstance(x, int):
        return x
    return x.data_ptr()


def _stream(stream):
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def _check(status: int, where: str) -> int:
    if status != OK:
        raise AtlasMemError(status, where)
    return status


def make_config(kind, batch, heads, d_key, d_value, d_hidden=0, poly_degree=1, chunk=1, omega_window=1,
                gate_mode=PER_TOKEN, ns_steps=0, ns_coeffs=(3.4445, -4.7750, 2.0315), ns_eps=1e-7,
                input_dtype=BF16, output_dtype=F32, precision=PREC_AUTO, flags=0) -> Config:
    return Config(ABI_VERSION, kind, batch, heads, d_key, d_value, d_hidden, poly_degree, chunk, omega_window,
                  gate_mode, ns_steps, ns_coeffs[0], ns_coeffs[1], ns_coeffs[2], ns_eps, input_dtype, output_dtype,
                  precision, flags)


def abi_version() -> int:
    return load().atlasmem_abi_version()


def param_count(cfg: Config) -> int:
    return load().atlasmem_param_count(ctypes.byref(cfg))


class Memory:
    """An atlasmem handle: state, momentum and window history of B*H memories on one device."""

    def __init__(self, cfg: Config, W0=None, S0=None, stream=None):
        lib = load()
        self.cfg = cfg
        self.P = lib.atlasmem_param_count(ctypes.byref(cfg))
        h = _vp()
        _check(lib.atlasmem_create(ctypes.byref(cfg), _ptr(W0), _ptr(S0), _stream(stream), ctypes.byref(h)),
               "atlasmem_create")
        self._h = h

    def update_chunked(self, K, Q, V, theta, eta, alpha, gamma, T: int, Y=None, stream=None):
        _check(load().atlasmem_update_chunked(self._h, _ptr(K), _ptr(Q), _ptr(V), _ptr(theta), _ptr(eta),
                                              _ptr(alpha), _ptr(gamma), int(T), _ptr(Y), _stream(stream)),
               "atlasmem_update_chunked")

    def update_chunked_conv(self, K, Q, V, taps, bias, l2norm, theta, eta, alpha, gamma, T: int, Y=None,
                            stream=None):
        """K, Q, V raw rows; taps = (taps_k, taps_q, taps_v) [heads, d, 4]; bias = (bias_k, bias_q,
        bias_v) or None entries; l2norm = (keys, queries)."""
        bias = bias or (None, None, None)
        p = ConvParams(_ptr(taps[0]), _ptr(taps[1]), _ptr(taps[2]), _ptr(bias[0]), _ptr(bias[1]), _ptr(bias[2]),
                       int(bool(l2norm[0])), int(bool(l2norm[1])))
        _check(load().atlasmem_update_chunked_conv(self._h, _ptr(K), _ptr(Q), _ptr(V), ctypes.byref(p), _ptr(theta),
                                                   _ptr(eta), _ptr(alpha), _ptr(gamma), int(T), _ptr(Y),
                                                   _stream(stream)), "atlasmem_update_chunked_conv")

    def flush(self, theta=None, eta=None, alpha=None, stream=None):
        _check(load().atlasmem_flush(self._h, _ptr(theta), _ptr(eta), _ptr(alpha), _stream(stream)), "atlasmem_flush")

    @property
    def pending(self) -> int:
        return int(load().atlasmem_pending(self._h))

    def backward_workspace_bytes(self, T: int) -> int:
        return int(load().atlasmem_backward_workspace_bytes(self._h, int(T)))

    def update_backward(self, K, Q, V, theta, eta, alpha, T: int, dY, dK, dQ, dV, dtheta, deta, dalpha, dW0, dS0,
                        workspace, Y=None, dW_T=None, dS_T=None, gamma=None, dgamma=None, stream=None):
        _check(load().atlasmem_update_backward(
            self._h, _ptr(K), _ptr(Q), _ptr(V), _ptr(theta), _ptr(eta), _ptr(alpha), _ptr(gamma), int(T), _ptr(Y),
            _ptr(dY), _ptr(dW_T), _ptr(dS_T), _ptr(workspace), int(workspace.numel() * workspace.element_size()),
            _ptr(dK), _ptr(dQ), _ptr(dV), _ptr(dtheta), _ptr(deta), _ptr(dalpha), _ptr(dgamma), _ptr(dW0), _ptr(dS0),
            _stream(stream)),
            "atlasmem_update_backward")

    def retrieve(self, Q, T: int, Y, stream=None):
        _check(load().atlasmem_retrieve(self._h, _ptr(Q), int(T), _ptr(Y), _stream(stream)), "atlasmem_retrieve")

    def get_state(self, W=None, S=None, stream=None) -> int:
        """Copies the state out; returns OK or E_NONFINITE (raises on other errors)."""
        st = load().atlasmem_get_state(self._h, _ptr(W), _ptr(S), _stream(stream))
        if st not in (OK, E_NONFINITE):
            raise AtlasMemError(st, "atlasmem_get_state")
        return st

    def set_state(self, W=None, S=None, stream=None):
        _check(load().atlasmem_set_state(self._h, _ptr(W), _ptr(S), _stream(stream)), "atlasmem_set_state")

    def reset_history(self, stream=None):
        _check(load().atlasmem_reset_history(self._h, _stream(stream)), "atlasmem_reset_history")

    def close(self):
        if getattr(self, "_h", None):
            load().atlasmem_destroy(self._h)
            self._h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


def gate_scan(theta, eta, alpha, M: int, T: int, chunk: int, cW, cS, chunk_scalars, stream=None):
    _check(load().atlasmem_gate_scan(_ptr(theta), _ptr(eta), _ptr(alpha), M, T, chunk, _ptr(cW), _ptr(cS),
                                     _ptr(chunk_scalars), _stream(stream)), "atlasmem_gate_scan")


def omega_coeffs(cW, cS, gamma, gamma_hist, M: int, T: int, chunk: int, window: int, oW, oS, stream=None):
    _check(load().atlasmem_omega_coeffs(_ptr(cW), _ptr(cS), _ptr(gamma), _ptr(gamma_hist), M, T, chunk, window,
                                        _ptr(oW), _ptr(oS), _stream(stream)), "atlasmem_omega_coeffs")


def poly_features(X, in_dtype: int, n: int, d: int, F, stream=None):
    _check(load().atlasmem_poly_features(_ptr(X), in_dtype, n, d, _ptr(F), _stream(stream)),
           "atlasmem_poly_features")


def newton_schulz(G, n_mat: int, rows: int, cols: int, steps: int, coeffs, eps: float, precision: int, out,
                  stream=None):
    a, b, c = coeffs
    _check(load().atlasmem_newton_schulz(_ptr(G), n_mat, rows, cols, steps, a, b, c, eps, precision, _ptr(out),
                                         _stream(stream)), "atlasmem_newton_schulz")


def update_chunked_static(cfg: Config, K, Q, V, theta, eta, alpha, T: int, W, S, Y=None, nonfinite=None,
                          stream=None):
    """The allocation-free update (no handle): W, S updated in place; returns the status."""
    return _check(load().atlasmem_update_chunked_static(ctypes.byref(cfg), _ptr(K), _ptr(Q), _ptr(V), _ptr(theta),
                                                        _ptr(eta), _ptr(alpha), T, _ptr(W), _ptr(S), _ptr(Y),
                                                        _ptr(nonfinite), _stream(stream)),
                  "atlasmem_update_chunked_static")


def calibrate_mfma(iters: int, n_workgroups: int, sink, stream=None):
    """FLOPs of the call: n_workgroups * 8 * iters * 8 * 32768."""
    _check(load().atlasmem_calibrate_mfma(iters, n_workgroups, _ptr(sink), _stream(stream)), "atlasmem_calibrate_mfma")


def calibrate_copy(src, dst, nbytes: int, stream=None):
    _check(load().atlasmem_calibrate_copy(_ptr(src), _ptr(dst), nbytes, _stream(stream)), "atlasmem_calibrate_copy")


def short_conv(X, in_dtype: int, M: int, T: int, d: int, heads: int, taps, bias, hist, l2norm: bool, out,
               out_dtype: int, hist_out=None, stream=None):
    _check(load().atlasmem_short_conv(_ptr(X), in_dtype, M, T, d, heads, _ptr(taps), _ptr(bias), _ptr(hist),
                                      int(l2norm), _ptr(out), out_dtype, _ptr(hist_out), _stream(stream)),
           "atlasmem_short_conv")


def gates(U, B: int, T: int, d_model: int, heads: int, n_gates: int, Wg, bg, scale, chunk: int, out, stream=None):
    _check(load().atlasmem_gates(_ptr(U), B, T, d_model, heads, n_gates, _ptr(Wg), _ptr(bg), _ptr(scale), chunk,
                                 _ptr(out), _stream(stream)), "atlasmem_gates")


def feature_map(X, in_dtype: int, n: int, d: int, degree: int, out, coeffs=None, P=None, d_out: int = 0,
                stream=None):
    """coeffs: a host sequence of degree + 1 floats (None: 1/k!)."""
    arr = None if coeffs is None else (ctypes.c_float * (degree + 1))(*[float(v) for v in coeffs])
    c = None if arr is None else ctypes.cast(arr, ctypes.c_void_p)
    _check(load().atlasmem_feature_map(_ptr(X), in_dtype, n, d, degree, c, _ptr(P), d_out, _ptr(out),
                                       _stream(stream)), "atlasmem_feature_map")

