"""CPU fp64 oracle for the Mamba-2 mixer layer (test infrastructure).

Only the tests, ``__graft_entry__.smoke()`` and ``bench.py``'s cpu_baseline leg
may import this package. It wraps ``liboracle_m2.so`` (plain C, built with gcc
from ``m2_oracle.c``; see that file's header for the definition it follows and
the passages of the pages it rests on). It shares no code with the HIP library.

Arrays are numpy. Weights are passed in their stored form (float32, bf16 bit
patterns as uint16, int8 with float16 scales, or packed 4- or 3-bit codes as uint8
rows with float16 (scale, bias) pairs); the oracle decodes them itself.
States are float64 and are updated in place.
"""
from __future__ import annotations

import ctypes as C
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "m2_oracle.c")
_HDR = os.path.join(_HERE, "m2_oracle.h")
LIB_PATH = os.path.join(_HERE, "liboracle_m2.so")

_WT = {"f32": 0, "bf16": 1, "int8g": 2, "int4g": 3, "int3g": 4}
_BITS = {"int4g": 4, "int3g": 3}


def build(force: bool = False) -> str:
    """Compile the oracle with gcc (-O2, no fast-math: summation order stays as written)."""
    stale = (not os.path.exists(LIB_PATH)) or any(
        os.path.getmtime(p) > os.path.getmtime(LIB_PATH) for p in (_SRC, _HDR))
    if force or stale:
        tmp = LIB_PATH + ".tmp%d" % os.getpid()
        subprocess.check_call(["gcc", "-O2", "-std=c11", "-fopenmp", "-fPIC", "-shared",
                               "-Wall", "-Werror", _SRC, "-o", tmp, "-lm"])
        os.replace(tmp, LIB_PATH)
    return LIB_PATH


class _Cfg(C.Structure):
    _fields_ = [("d_model", C.c_int32), ("n_heads", C.c_int32), ("head_dim", C.c_int32),
                ("d_state", C.c_int32), ("n_groups", C.c_int32), ("d_conv", C.c_int32),
                ("norm_group", C.c_int32), ("norm_eps", C.c_double), ("wtype", C.c_int32),
                ("q_group", C.c_int32), ("q_gamma_in", C.c_double), ("q_gamma_out", C.c_double)]


class _Weights(C.Structure):
    _fields_ = [("w_in", C.c_void_p), ("s_in", C.c_void_p), ("w_out", C.c_void_p),
                ("s_out", C.c_void_p), ("conv_w", C.c_void_p), ("conv_b", C.c_void_p),
                ("dt_bias", C.c_void_p), ("A_log", C.c_void_p), ("D", C.c_void_p),
                ("norm_w", C.c_void_p)]


class _Trace(C.Structure):
    _fields_ = [(n, C.c_void_p) for n in ("zxbcdt", "xconv", "dt", "y", "v", "yn", "out")]


_lib = None


def lib():
    """The oracle's C library; M2_ORACLE_LIB names another build of the same source (the
    sanitizer tests load one built with AddressSanitizer and UBSan)."""
    global _lib
    if _lib is None:
        _lib = C.CDLL(os.environ.get("M2_ORACLE_LIB") or build())
        P = C.c_void_p
        i32 = C.c_int32
        _lib.orc_step.argtypes = [P, P, P, P, i32, P, P, i32, P, i32, P]
        _lib.orc_step.restype = C.c_int
        _lib.orc_prefill.argtypes = [P, P, P, P, i32, P, P, i32, i32, P, i32]
        _lib.orc_prefill.restype = C.c_int
        _lib.orc_ssd_recurrent.argtypes = [i32] * 5 + [P] * 8
        _lib.orc_ssd_recurrent.restype = None
        _lib.orc_ssd_quadratic.argtypes = [i32] * 5 + [P] * 9
        _lib.orc_ssd_quadratic.restype = None
        for f in ("orc_bf16_to_double", "orc_fp16_to_double"):
            getattr(_lib, f).argtypes = [C.c_uint16]
            getattr(_lib, f).restype = C.c_double
        _lib.orc_lowbit_code.argtypes = [i32, P, C.c_int64, C.c_int64, C.c_int64]
        _lib.orc_lowbit_code.restype = C.c_int32
        for f in ("orc_softplus", "orc_silu"):
            getattr(_lib, f).argtypes = [C.c_double]
            getattr(_lib, f).restype = C.c_double
        _lib.orc_num_threads.restype = C.c_int
        _lib.orc_set_num_threads.argtypes = [C.c_int]
        _lib.orc_set_num_threads.restype = None
        _lib.orc_head_argmax.argtypes = [i32, i32, C.c_double, C.c_int64, C.c_int64, P, P, P, i32, P, P]
        _lib.orc_head_argmax.restype = C.c_int
        _lib.orc_attn_step.argtypes = [P, P, P, P, P, P, P, P, i32, P, P, i32, P, i32, P, P]
        _lib.orc_attn_step.restype = C.c_int
        _lib.orc_double_to_bf16.argtypes = [C.c_double]
        _lib.orc_double_to_bf16.restype = C.c_uint16
    return _lib


def num_threads() -> int:
    return int(lib().orc_num_threads())


def set_num_threads(n: int) -> None:
    """Threads of the oracle's parallel loops from now on (timing on one core)."""
    lib().orc_set_num_threads(int(n))


def _ptr(a):
    return None if a is None else a.ctypes.data


def _f64(a, shape=None):
    out = np.ascontiguousarray(a, dtype=np.float64)
    if shape is not None and out.shape != tuple(shape):
        raise ValueError("shape %s, expected %s" % (out.shape, tuple(shape)))
    return out


class Layer:
    """One mixer layer's configuration and weights, held for the C oracle.

    ``dims`` is any object with the attributes d_model, n_heads, head_dim,
    d_state, n_groups, d_conv, rms_group, norm_eps, wtype, q_group, q_gamma_in,
    q_gamma_out, d_inner, conv_dim, d_in_proj. ``w`` maps the parameter names
    (w_in, s_in, w_out, s_out, conv_w, conv_b, dt_bias, A_log, D, norm_w) to
    numpy arrays in their stored dtypes.
    """

    def __init__(self, dims, w):
        self.dims = dims
        d = dims
        self.cfg = _Cfg(d.d_model, d.n_heads, d.head_dim, d.d_state, d.n_groups, d.d_conv,
                        d.rms_group, float(d.norm_eps), _WT[d.wtype], d.q_group,
                        float(d.q_gamma_in), float(d.q_gamma_out))
        keep = {}
        for k in ("w_in", "w_out"):
            want = {"f32": np.float32, "bf16": np.uint16, "int8g": np.int8, "int4g": np.uint8,
                    "int3g": np.uint8}[d.wtype]
            keep[k] = np.ascontiguousarray(w[k], dtype=want)
        for k in ("s_in", "s_out"):
            keep[k] = None if w.get(k) is None else np.ascontiguousarray(w[k], dtype=np.float16).view(np.uint16)
        for k in ("conv_w", "conv_b", "dt_bias", "A_log", "D", "norm_w"):
            keep[k] = np.ascontiguousarray(w[k], dtype=np.float32)
        bits = _BITS.get(d.wtype)
        cols = (lambda K: K) if bits is None else (lambda K: K * bits // 8)   # packed bytes per row
        if keep["w_in"].shape != (d.d_in_proj, cols(d.d_model)) or keep["w_out"].shape != (d.d_model, cols(d.d_inner)):
            raise ValueError("weight shapes do not match the dimensions")
        if keep["conv_w"].shape != (d.conv_dim, d.d_conv):
            raise ValueError("conv_w shape")
        if d.wtype in ("int8g", "int4g", "int3g") and (keep["s_in"] is None or keep["s_out"] is None):
            raise ValueError("quantized weights need scales")
        self._keep = keep
        self.w = _Weights(*[_ptr(keep[k]) for k in ("w_in", "s_in", "w_out", "s_out", "conv_w",
                                                     "conv_b", "dt_bias", "A_log", "D", "norm_w")])

    def new_state(self, n_slots, ssm0=None, conv0=None):
        d = self.dims
        ssm = np.zeros((n_slots, d.n_heads, d.head_dim, d.d_state)) if ssm0 is None else _f64(ssm0).copy()
        conv = np.zeros((n_slots, d.d_conv - 1, d.conv_dim)) if conv0 is None else _f64(conv0).copy()
        return ssm, conv

    def step(self, ssm, conv, x, slot_ids=None, residual=False, trace=False):
        """One token for x.shape[0] sessions; ssm and conv (float64) are updated in place."""
        d = self.dims
        x = _f64(x)
        B = x.shape[0]
        if x.shape != (B, d.d_model):
            raise ValueError("x shape")
        _check_state(d, ssm, conv)
        y = np.empty((B, d.d_model))
        sl = None if slot_ids is None else np.ascontiguousarray(slot_ids, dtype=np.int32)
        tr = None
        bufs = None
        if trace:
            bufs = {"zxbcdt": np.empty((B, d.d_in_proj)), "xconv": np.empty((B, d.conv_dim)),
                    "dt": np.empty((B, d.n_heads)), "y": np.empty((B, d.d_inner)),
                    "v": np.empty((B, d.d_inner)), "yn": np.empty((B, d.d_inner)),
                    "out": np.empty((B, d.d_model))}
            tr = _Trace(*[_ptr(bufs[k]) for k in ("zxbcdt", "xconv", "dt", "y", "v", "yn", "out")])
        rc = lib().orc_step(C.byref(self.cfg), C.byref(self.w), _ptr(ssm), _ptr(conv), ssm.shape[0],
                            _ptr(x), _ptr(y), B, _ptr(sl), int(bool(residual)),
                            None if tr is None else C.byref(tr))
        if rc != 0:
            raise ValueError("orc_step rejected its arguments")
        return (y, bufs) if trace else y

    def prefill(self, ssm, conv, x, slot_ids=None, residual=False):
        """x [B][T][d_model]: T recurrent steps; returns y [B][T][d_model]."""
        d = self.dims
        x = _f64(x)
        B, T = x.shape[0], x.shape[1]
        if x.shape != (B, T, d.d_model):
            raise ValueError("x shape")
        _check_state(d, ssm, conv)
        y = np.empty((B, T, d.d_model))
        sl = None if slot_ids is None else np.ascontiguousarray(slot_ids, dtype=np.int32)
        rc = lib().orc_prefill(C.byref(self.cfg), C.byref(self.w), _ptr(ssm), _ptr(conv), ssm.shape[0],
                               _ptr(x), _ptr(y), B, T, _ptr(sl), int(bool(residual)))
        if rc != 0:
            raise ValueError("orc_prefill rejected its arguments")
        return y


def _check_state(d, ssm, conv):
    if ssm.dtype != np.float64 or conv.dtype != np.float64:
        raise TypeError("oracle states are float64")
    if not (ssm.flags.c_contiguous and conv.flags.c_contiguous):
        raise ValueError("oracle states must be contiguous")
    n = ssm.shape[0]
    if ssm.shape != (n, d.n_heads, d.head_dim, d.d_state) or conv.shape != (n, d.d_conv - 1, d.conv_dim):
        raise ValueError("state shapes")


def ssd_recurrent(x, Bm, Cm, dt, A, D, S):
    """Steps 5-7 token by token. x [T][H][P], Bm/Cm [T][G][N], dt [T][H], A/D [H];
    S [H][P][N] float64 updated in place. Returns y [T][H][P]."""
    x, Bm, Cm, dt, A, D = (_f64(a) for a in (x, Bm, Cm, dt, A, D))
    T, H, P = x.shape
    G, N = Bm.shape[1], Bm.shape[2]
    assert S.dtype == np.float64 and S.shape == (H, P, N) and S.flags.c_contiguous
    y = np.empty((T, H, P))
    lib().orc_ssd_recurrent(T, H, P, N, G, _ptr(x), _ptr(Bm), _ptr(Cm), _ptr(dt), _ptr(A), _ptr(D),
                            _ptr(S), _ptr(y))
    return y


def ssd_quadratic(x, Bm, Cm, dt, A, D, S0):
    """The materialised quadratic form of the same map. Returns (y [T][H][P], S_final [H][P][N])."""
    x, Bm, Cm, dt, A, D, S0 = (_f64(a) for a in (x, Bm, Cm, dt, A, D, S0))
    T, H, P = x.shape
    G, N = Bm.shape[1], Bm.shape[2]
    y = np.empty((T, H, P))
    Sf = np.empty((H, P, N))
    lib().orc_ssd_quadratic(T, H, P, N, G, _ptr(x), _ptr(Bm), _ptr(Cm), _ptr(dt), _ptr(A), _ptr(D),
                            _ptr(S0), _ptr(y), _ptr(Sf))
    return y, Sf


def bf16_to_double(bits: int) -> float:
    return lib().orc_bf16_to_double(bits)


def fp16_to_double(bits: int) -> float:
    return lib().orc_fp16_to_double(bits)


def softplus(x: float) -> float:
    return lib().orc_softplus(x)


def silu(x: float) -> float:
    return lib().orc_silu(x)


def lowbit_code(wtype: str, w: np.ndarray, row: int, k: int) -> int:
    """Code k of row `row` of packed low-bit weights w [rows][packed bytes] (the oracle's decoder)."""
    w = np.ascontiguousarray(w, dtype=np.uint8)
    K = w.shape[1] * 8 // _BITS[wtype]
    return int(lib().orc_lowbit_code(_WT[wtype], _ptr(w), row, K, k))


def head_argmax(wtype: str, w: np.ndarray, h, scales=None, q_group: int = 0, gamma: float = 1.0):
    """Output head: (logits [B][vocab] fp64, greedy tokens [B] int32) of W h for w in the
    layer's storage formats (bf16 as uint16 bits, low-bit as packed codes [vocab][bytes])."""
    h = _f64(h)
    if h.ndim == 1:
        h = h[None]
    B, K = h.shape
    w = np.ascontiguousarray(w)
    vocab = w.shape[0]
    s = None if scales is None else np.ascontiguousarray(scales).view(np.uint16)
    logits = np.zeros((B, vocab), np.float64)
    token = np.zeros(B, np.int32)
    rc = lib().orc_head_argmax(_WT[wtype], q_group, float(gamma), vocab, K, _ptr(w), _ptr(s), _ptr(h), B,
                               _ptr(logits), _ptr(token))
    if rc != 0:
        raise ValueError("orc_head_argmax: bad arguments")
    return logits, token


class _AttnCfg(C.Structure):
    _fields_ = [("d_model", C.c_int32), ("n_q", C.c_int32), ("n_kv", C.c_int32), ("head_dim", C.c_int32),
                ("max_len", C.c_int32), ("wtype", C.c_int32), ("q_group", C.c_int32),
                ("q_gamma_qkv", C.c_double), ("q_gamma_o", C.c_double)]


class AttnLayer:
    """The attention decode step (orc_attn_step) over host copies of the weights."""

    def __init__(self, dims, weights):
        self.dims = d = dims
        self.cfg = _AttnCfg(d.d_model, d.n_q, d.n_kv, d.head_dim, d.max_len, _WT[d.wtype], d.q_group,
                            float(np.float32(d.q_gamma_qkv)), float(np.float32(d.q_gamma_o)))
        self.w = {k: (None if v is None else np.ascontiguousarray(v)) for k, v in weights.items()}
        for k in ("s_qkv", "s_o"):
            if self.w.get(k) is not None:
                self.w[k] = self.w[k].view(np.uint16)

    def step(self, kc, vc, pos, x, slot_ids=None, residual=False, trace=False):
        """One token for x [B][d_model]; kc, vc (uint16 bf16 bits) and pos (int32) are
        updated in place. Returns y [B][d_model] (and the qkv and o intermediates)."""
        d = self.dims
        x = _f64(x)
        if x.ndim == 1:
            x = x[None]
        B = x.shape[0]
        for a, dt in ((kc, np.uint16), (vc, np.uint16), (pos, np.int32)):
            if a.dtype != dt or not a.flags.c_contiguous:
                raise ValueError("kv cache must be contiguous uint16, pos contiguous int32")
        n_slots = pos.shape[0]
        if kc.shape != (n_slots, d.n_kv, d.max_len, d.head_dim) or vc.shape != kc.shape:
            raise ValueError("kv cache shape")
        sl = None if slot_ids is None else np.ascontiguousarray(slot_ids, np.int32)
        y = np.zeros((B, d.d_model))
        qkv = np.zeros((B, d.qkv_rows)) if trace else None
        o = np.zeros((B, d.o_dim)) if trace else None
        rc = lib().orc_attn_step(C.byref(self.cfg), _ptr(self.w["w_qkv"]), _ptr(self.w.get("s_qkv")),
                                 _ptr(self.w["w_o"]), _ptr(self.w.get("s_o")), _ptr(kc), _ptr(vc), _ptr(pos),
                                 n_slots, _ptr(x), _ptr(y), B, _ptr(sl), int(bool(residual)), _ptr(qkv), _ptr(o))
        if rc != 0:
            raise ValueError("orc_attn_step: bad arguments")
        return (y, {"qkv": qkv, "o": o}) if trace else y


def double_to_bf16(v: float) -> int:
    return int(lib().orc_double_to_bf16(float(v)))


def stack_step(entries, x, slot_ids=None):
    """A hybrid stack's step as the residual chain u_{l+1} = u_l + layer_l(u_l): entries are
    (Layer, (ssm, conv)) or (AttnLayer, (kc, vc, pos)), their states updated in place."""
    u = _f64(x)
    for lay, st in entries:
        if isinstance(lay, AttnLayer):
            u = lay.step(st[0], st[1], st[2], u, slot_ids=slot_ids, residual=True)
        else:
            u = lay.step(st[0], st[1], u, slot_ids=slot_ids, residual=True)
    return u
