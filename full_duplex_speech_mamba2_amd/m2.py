"""Thin ctypes binding of libm2.so (argument marshalling only).

Every step of the layer runs in the HIP library; this module only moves
arguments across the C ABI declared in include/m2.h. PyTorch supplies device
memory (tensors) and the stream (torch's current stream). torch is imported
before the library is loaded so that the process maps a single HIP runtime
(torch's bundled libamdhip64.so.7 satisfies libm2.so's dependency).

Importing this module raises ImportError if libm2.so has not been built: there
is no CPU fallback.
"""
from __future__ import annotations

import ctypes as C
import os
from typing import Dict, Optional

import numpy as np
import torch

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libm2.so")
if not os.path.exists(LIB_PATH):
    raise ImportError("libm2.so is not built (python -m full_duplex_speech_mamba2_amd.build)")

_lib = C.CDLL(LIB_PATH)

M2_OK, M2_ERR_NULL, M2_ERR_SHAPE, M2_ERR_DTYPE, M2_ERR_ALIGN = 0, -1, -2, -3, -4
M2_ERR_WORKSPACE, M2_ERR_SLOT, M2_ERR_UNSUPPORTED, M2_ERR_HIP = -5, -6, -7, -8
M2_RESIDUAL = 1
M2_PERSISTENT = 2
WTYPE = {"f32": 0, "bf16": 1, "int8g": 2, "int4g": 3, "int3g": 4}


class Config(C.Structure):
    _fields_ = [("d_model", C.c_int32), ("n_heads", C.c_int32), ("head_dim", C.c_int32),
                ("d_state", C.c_int32), ("n_groups", C.c_int32), ("d_conv", C.c_int32),
                ("norm_group", C.c_int32), ("norm_eps", C.c_float), ("wtype", C.c_int32),
                ("q_group", C.c_int32), ("q_gamma_in", C.c_float), ("q_gamma_out", C.c_float)]


class HeadConfig(C.Structure):
    _fields_ = [("d_model", C.c_int32), ("vocab", C.c_int32), ("wtype", C.c_int32),
                ("q_group", C.c_int32), ("q_gamma", C.c_float)]


class AttnConfig(C.Structure):
    _fields_ = [("d_model", C.c_int32), ("n_q", C.c_int32), ("n_kv", C.c_int32), ("head_dim", C.c_int32),
                ("max_len", C.c_int32), ("wtype", C.c_int32), ("q_group", C.c_int32),
                ("q_gamma_qkv", C.c_float), ("q_gamma_o", C.c_float)]


class AttnWeights(C.Structure):
    _fields_ = [(n, C.c_void_p) for n in ("w_qkv", "s_qkv", "w_o", "s_o")]


class Weights(C.Structure):
    _fields_ = [(n, C.c_void_p) for n in ("w_in", "s_in", "w_out", "s_out", "conv_w", "conv_b",
                                          "dt_bias", "A_log", "D", "norm_w", "w_in_panels",
                                          "w_out_panels")]


_P = C.c_void_p
_i32 = C.c_int32
_lib.m2_abi_version.restype = C.c_int
_lib.m2_last_error.restype = C.c_char_p
_lib.m2_layer_create.argtypes = [_P, _P, _P]
_lib.m2_panels_bytes.argtypes = [_i32, _i32, _i32]
_lib.m2_panels_bytes.restype = C.c_size_t
_lib.m2_pack_panels.argtypes = [_i32, _P, _i32, _i32, _P, _P]
_lib.m2_layer_destroy.argtypes = [_P]
_lib.m2_layer_destroy.restype = None
_lib.m2_state_sizes.argtypes = [_P, _i32, _P, _P]
_lib.m2_state_create.argtypes = [_P, _i32, _P, _P, _P]
_lib.m2_state_destroy.argtypes = [_P]
_lib.m2_state_destroy.restype = None
_lib.m2_state_zero.argtypes = [_P, _P, _i32, _P]
_lib.m2_step_workspace.argtypes = [_P, _i32]
_lib.m2_step_workspace.restype = C.c_size_t
_lib.m2_step.argtypes = [_P, _P, _P, _P, _i32, _P, _i32, _P, C.c_size_t, _P]
_lib.m2_step_timed.argtypes = [_P, _P, _P, _P, _i32, _P, _i32, _P, C.c_size_t, _P, _P]
_lib.m2_step_noalloc.argtypes = [_P, _P, _P, _P, _i32, _P, _i32, _P]
_lib.m2_step_noalloc.restype = C.c_int
_lib.m2_noalloc_scratch_bytes.restype = C.c_size_t
_lib.m2_step_plan.argtypes = [_P, _i32]
_lib.m2_step_plan.restype = C.c_int
_lib.m2_step_plan_flags.argtypes = [_P, _i32, _i32]
_lib.m2_step_plan_flags.restype = C.c_int
_lib.m2_prefill_workspace.argtypes = [_P, _i32, _i32, _i32]
_lib.m2_prefill_workspace.restype = C.c_size_t
_lib.m2_prefill.argtypes = [_P, _P, _P, _P, _i32, _i32, _i32, _P, _i32, _P, C.c_size_t, _P]
_lib.m2_head_workspace.argtypes = [_P, _i32]
_lib.m2_head_workspace.restype = C.c_size_t
_lib.m2_head_argmax.argtypes = [_P, _P, _P, _P, _i32, _P, _P, _P, C.c_size_t, _P]
_lib.m2_head_argmax_timed.argtypes = [_P, _P, _P, _P, _i32, _P, _P, _P, C.c_size_t, _P, _P]
_lib.m2_attn_create.argtypes = [_P, _P, _P]
_lib.m2_attn_destroy.argtypes = [_P]
_lib.m2_attn_destroy.restype = None
_lib.m2_attn_workspace.argtypes = [_P, _i32]
_lib.m2_attn_workspace.restype = C.c_size_t
_lib.m2_attn_step.argtypes = [_P, _P, _P, _P, _i32, _P, _P, _i32, _P, _i32, _P, C.c_size_t, _P]
_lib.m2_attn_step_timed.argtypes = [_P, _P, _P, _P, _i32, _P, _P, _i32, _P, _i32, _P, C.c_size_t, _P, _P]
_lib.m2_stack_create.argtypes = [_P, _i32, _i32, _P]
_lib.m2_stack_destroy.argtypes = [_P]
_lib.m2_stack_destroy.restype = None
_lib.m2_stack_workspace.argtypes = [_P, _i32]
_lib.m2_stack_workspace.restype = C.c_size_t
_lib.m2_stack_step.argtypes = [_P, _P, _P, _i32, _P, _P, C.c_size_t, _P]
_lib.m2_stack_workspace_flags.argtypes = [_P, _i32, _i32]
_lib.m2_stack_workspace_flags.restype = C.c_size_t
_lib.m2_stack_step_flags.argtypes = [_P, _P, _P, _i32, _P, _i32, _P, C.c_size_t, _P]
_lib.m2_stack_persistent_runs.argtypes = [_P, _i32, _i32]
for _f in ("m2_attn_create", "m2_attn_step", "m2_attn_step_timed", "m2_stack_create", "m2_stack_step",
           "m2_stack_step_flags", "m2_stack_persistent_runs"):
    getattr(_lib, _f).restype = C.c_int
for _f in ("m2_layer_create", "m2_state_sizes", "m2_state_create", "m2_state_zero", "m2_step",
           "m2_step_timed", "m2_prefill", "m2_head_argmax", "m2_head_argmax_timed"):
    getattr(_lib, _f).restype = C.c_int


class M2Error(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__("m2 status %d: %s" % (status, msg))
        self.status = status


def _check(rc: int):
    if rc != M2_OK:
        raise M2Error(rc, _lib.m2_last_error().decode())


def lib():
    return _lib


def abi_version() -> int:
    return _lib.m2_abi_version()


def config_from_dims(dims) -> Config:
    return Config(dims.d_model, dims.n_heads, dims.head_dim, dims.d_state, dims.n_groups, dims.d_conv,
                  dims.norm_group, float(dims.norm_eps), WTYPE[dims.wtype], dims.q_group,
                  float(dims.q_gamma_in), float(dims.q_gamma_out))


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else t.data_ptr()


def _stream(stream) -> Optional[int]:
    if stream is None:
        stream = torch.cuda.current_stream()
    return stream.cuda_stream or None


def to_device(a, device="cuda") -> Optional[torch.Tensor]:
    """numpy (float32, uint16 bf16 bits, int8, float16) or tensor -> contiguous device tensor."""
    if a is None:
        return None
    if isinstance(a, torch.Tensor):
        return a.to(device).contiguous()
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        a = a.view(np.int16)
    return torch.from_numpy(a).to(device)


def panels_bytes(wtype: str, rows: int, k: int) -> int:
    """Bytes of the 16-row panel copy of a [rows][k] matrix (m2_panels_bytes; 0 if none)."""
    return int(_lib.m2_panels_bytes(WTYPE[wtype], rows, k))


def pack_panels(wtype: str, w: torch.Tensor, rows: int, k: int) -> torch.Tensor:
    """The 16-row panel copy of the device row-major matrix w, written by m2_pack_panels on
    the current stream (a uint8 tensor of panels_bytes)."""
    n = panels_bytes(wtype, rows, k)
    out = torch.empty(n, dtype=torch.uint8, device=w.device)
    _check(_lib.m2_pack_panels(WTYPE[wtype], _ptr(w), rows, k, _ptr(out),
                               C.c_void_p(torch.cuda.current_stream(w.device).cuda_stream)))
    return out


class Layer:
    """A mixer layer handle over device copies of its weights (the handle borrows them).

    With panels (the default, bf16 and int8 weights only) the layer also holds the 16-row
    panel copies of W_in and W_out (m2_pack_panels), which the batched decode step's
    matrix-core GEMVs and the bf16 prefill GEMMs read; panels=False leaves them out (those
    kernels then read the row-major weights)."""

    def __init__(self, dims, weights: Dict[str, object], device="cuda", panels: bool = True):
        self.dims = dims
        self.device = torch.device(device)
        self.tensors = {k: to_device(v, self.device) for k, v in weights.items()}
        self.cfg = config_from_dims(dims)
        if panels and dims.wtype in ("bf16", "int8g"):
            d_inner = dims.n_heads * dims.head_dim
            d_in_proj = 2 * d_inner + 2 * dims.n_groups * dims.d_state + dims.n_heads
            for name, rows, k in (("w_in", d_in_proj, dims.d_model), ("w_out", dims.d_model, d_inner)):
                self.tensors[name + "_panels"] = pack_panels(dims.wtype, self.tensors[name], rows, k)
            torch.cuda.current_stream(self.device).synchronize()
        self.wstruct = Weights(*[_ptr(self.tensors.get(k)) for k in
                                 ("w_in", "s_in", "w_out", "s_out", "conv_w", "conv_b", "dt_bias",
                                  "A_log", "D", "norm_w", "w_in_panels", "w_out_panels")])
        h = C.c_void_p()
        _check(_lib.m2_layer_create(C.byref(self.cfg), C.byref(self.wstruct), C.byref(h)))
        self.handle = h
        self._ws: Dict[tuple, torch.Tensor] = {}

    def __del__(self):
        h = getattr(self, "handle", None)
        if h:
            _lib.m2_layer_destroy(h)
            self.handle = None

    def step_workspace_bytes(self, batch: int) -> int:
        return int(_lib.m2_step_workspace(self.handle, batch))

    def step_plan(self, batch: int, persistent: bool = False) -> int:
        """0: VALU GEMVs; 1: MFMA GEMVs around the SSD kernel; 2: in_proj GEMV, then the
        persistent SSD + out_proj kernel (only with persistent=True) (m2_step_plan_flags)."""
        return int(_lib.m2_step_plan_flags(self.handle, batch, _flags(False, persistent)))

    def prefill_workspace_bytes(self, batch: int, seqlen: int, chunk: int) -> int:
        return int(_lib.m2_prefill_workspace(self.handle, batch, seqlen, chunk))

    def workspace(self, kind: str, *args) -> torch.Tensor:
        """A cached device workspace for step(batch) or prefill(batch, seqlen, chunk)."""
        key = (kind,) + tuple(args)
        ws = self._ws.get(key)
        if ws is None:
            n = self.step_workspace_bytes(*args) if kind == "step" else self.prefill_workspace_bytes(*args)
            if n == 0:
                raise M2Error(M2_ERR_UNSUPPORTED, "no workspace size for %s%s" % (kind, args))
            ws = torch.empty(n, dtype=torch.uint8, device=self.device)
            self._ws[key] = ws
        return ws


class State:
    """Per-layer session state: ssm [n_slots][H][P][N] and conv [n_slots][d_conv-1][conv_dim], fp32."""

    def __init__(self, layer: Layer, n_slots: int, ssm: Optional[torch.Tensor] = None,
                 conv: Optional[torch.Tensor] = None):
        d = layer.dims
        self.layer = layer
        self.n_slots = n_slots
        self.ssm = ssm if ssm is not None else torch.zeros(
            (n_slots, d.n_heads, d.head_dim, d.d_state), dtype=torch.float32, device=layer.device)
        self.conv = conv if conv is not None else torch.zeros(
            (n_slots, d.d_conv - 1, d.conv_dim), dtype=torch.float32, device=layer.device)
        for t in (self.ssm, self.conv):
            if t.dtype != torch.float32 or not t.is_contiguous():
                raise ValueError("state tensors must be contiguous float32")
        h = C.c_void_p()
        _check(_lib.m2_state_create(layer.handle, n_slots, _ptr(self.ssm), _ptr(self.conv), C.byref(h)))
        self.handle = h

    def __del__(self):
        h = getattr(self, "handle", None)
        if h:
            _lib.m2_state_destroy(h)
            self.handle = None

    def zero(self, slot_ids: Optional[torch.Tensor] = None, stream=None):
        n = 0 if slot_ids is None else int(slot_ids.numel())
        _check(_lib.m2_state_zero(self.handle, _ptr(slot_ids), n, _stream(stream)))


def _act(t: torch.Tensor, shape) -> torch.Tensor:
    if t.dtype != torch.float32 or not t.is_contiguous() or tuple(t.shape) != tuple(shape):
        raise ValueError("expected a contiguous float32 tensor of shape %s, got %s %s"
                         % (tuple(shape), t.dtype, tuple(t.shape)))
    return t


def _tokens(t: torch.Tensor, n: int) -> torch.Tensor:
    if t.dtype != torch.int32 or not t.is_contiguous() or t.numel() != n:
        raise ValueError("expected a contiguous int32 tensor of %d tokens, got %s %s" % (n, t.dtype, tuple(t.shape)))
    return t


def _flags(residual: bool, persistent: bool = False) -> int:
    return (M2_RESIDUAL if residual else 0) | (M2_PERSISTENT if persistent else 0)


def step(layer: Layer, state: State, x: torch.Tensor, y: Optional[torch.Tensor] = None,
         slot_ids: Optional[torch.Tensor] = None, residual: bool = False,
         ws: Optional[torch.Tensor] = None, stream=None, persistent: bool = False) -> torch.Tensor:
    """One decode token for x.shape[0] sessions; returns y [B][d_model]. persistent: plan 2
    (the persistent SSD + out_proj kernel) where it applies."""
    B = x.shape[0]
    _act(x, (B, layer.dims.d_model))
    if y is None:
        y = torch.empty_like(x)
    _act(y, x.shape)
    if ws is None:
        ws = layer.workspace("step", B)
    _check(_lib.m2_step(layer.handle, state.handle, _ptr(x), _ptr(y), B, _ptr(slot_ids),
                        _flags(residual, persistent), _ptr(ws), ws.numel(), _stream(stream)))
    return y


def step_noalloc(layer: Layer, state: State, x: torch.Tensor, y: Optional[torch.Tensor] = None,
                 slot_ids: Optional[torch.Tensor] = None, residual: bool = False, stream=None) -> torch.Tensor:
    """step() through m2_step_noalloc: the library's static per-GPU scratch serves as the
    workspace (no workspace tensor); returns y [B][d_model]."""
    B = x.shape[0]
    _act(x, (B, layer.dims.d_model))
    if y is None:
        y = torch.empty_like(x)
    _act(y, x.shape)
    _check(_lib.m2_step_noalloc(layer.handle, state.handle, _ptr(x), _ptr(y), B, _ptr(slot_ids),
                                M2_RESIDUAL if residual else 0, _stream(stream)))
    return y


def noalloc_scratch_bytes() -> int:
    return int(_lib.m2_noalloc_scratch_bytes())


def step_timed(layer: Layer, state: State, x: torch.Tensor, y: torch.Tensor, events,
               slot_ids: Optional[torch.Tensor] = None, residual: bool = False,
               ws: Optional[torch.Tensor] = None, stream=None, persistent: bool = False) -> torch.Tensor:
    """step() that records the four events in `events` around its three kernels. Each is a
    raw hipEvent_t handle (int) or a torch.cuda.Event that has been recorded once (so that
    its HIP event exists)."""
    B = x.shape[0]
    _act(x, (B, layer.dims.d_model))
    _act(y, x.shape)
    if ws is None:
        ws = layer.workspace("step", B)
    ev = (C.c_void_p * 4)(*[getattr(e, "cuda_event", e) for e in events])
    _check(_lib.m2_step_timed(layer.handle, state.handle, _ptr(x), _ptr(y), B, _ptr(slot_ids),
                              _flags(residual, persistent), _ptr(ws), ws.numel(), _stream(stream), ev))
    return y


def prefill(layer: Layer, state: State, x: torch.Tensor, y: Optional[torch.Tensor] = None,
            chunk: int = 256, slot_ids: Optional[torch.Tensor] = None, residual: bool = False,
            ws: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """Chunked prefill of x [B][T][d_model]; returns y [B][T][d_model]."""
    B, T = x.shape[0], x.shape[1]
    _act(x, (B, T, layer.dims.d_model))
    if y is None:
        y = torch.empty_like(x)
    _act(y, x.shape)
    if ws is None:
        ws = layer.workspace("prefill", B, T, chunk)
    _check(_lib.m2_prefill(layer.handle, state.handle, _ptr(x), _ptr(y), B, T, chunk, _ptr(slot_ids),
                           M2_RESIDUAL if residual else 0, _ptr(ws), ws.numel(), _stream(stream)))
    return y


class Head:
    """An output head (m2_head_argmax) over device copies of its matrix and scales."""

    def __init__(self, d_model: int, vocab: int, w, scales=None, wtype: str = "bf16", q_group: int = 0,
                 q_gamma: float = 1.0, device="cuda"):
        self.cfg = HeadConfig(d_model, vocab, WTYPE[wtype], q_group, float(q_gamma))
        self.w = to_device(w, device)
        self.s = to_device(scales, device)
        self._ws: Dict[int, torch.Tensor] = {}

    def workspace(self, batch: int) -> torch.Tensor:
        n = _lib.m2_head_workspace(C.byref(self.cfg), batch)
        if n == 0:
            raise M2Error(M2_ERR_SHAPE, "invalid head configuration")
        if n not in self._ws:
            self._ws[n] = torch.empty(n, dtype=torch.uint8, device=self.w.device)
        return self._ws[n]

    def argmax(self, h: torch.Tensor, token: Optional[torch.Tensor] = None, logits: Optional[torch.Tensor] = None,
               stream=None) -> torch.Tensor:
        """Greedy token of each session of h [B][d_model] (device fp32); logits, if given,
        [B][vocab] fp32, receive W h."""
        B = h.shape[0]
        _act(h, (B, self.cfg.d_model))
        if logits is not None:
            _act(logits, (B, self.cfg.vocab))
        if token is None:
            token = torch.empty(B, dtype=torch.int32, device=h.device)
        _tokens(token, B)
        ws = self.workspace(B)
        _check(_lib.m2_head_argmax(C.byref(self.cfg), _ptr(self.w), _ptr(self.s), _ptr(h), B, _ptr(token),
                                   _ptr(logits), _ptr(ws), ws.numel(), _stream(stream)))
        return token

    def argmax_timed(self, h: torch.Tensor, token: torch.Tensor, events, stream=None) -> torch.Tensor:
        """argmax (no logits) recording three hipEvent_t handles: before the GEMV kernel,
        between it and the reduction, after the reduction. At most 4 sessions."""
        B = h.shape[0]
        _act(h, (B, self.cfg.d_model))
        _tokens(token, B)
        ws = self.workspace(B)
        ev = (C.c_void_p * 3)(*[getattr(e, "cuda_event", e) for e in events])
        _check(_lib.m2_head_argmax_timed(C.byref(self.cfg), _ptr(self.w), _ptr(self.s), _ptr(h), B, _ptr(token),
                                         None, _ptr(ws), ws.numel(), _stream(stream), ev))
        return token


def attn_config(dims) -> AttnConfig:
    return AttnConfig(dims.d_model, dims.n_q, dims.n_kv, dims.head_dim, dims.max_len, WTYPE[dims.wtype],
                      dims.q_group, float(dims.q_gamma_qkv), float(dims.q_gamma_o))


class Attn:
    """An attention-layer handle (m2_attn) over device copies of W_qkv and W_o."""

    def __init__(self, dims, weights: Dict[str, object], device="cuda"):
        self.dims = dims
        self.device = torch.device(device)
        self.tensors = {k: to_device(v, self.device) for k, v in weights.items()}
        self.cfg = attn_config(dims)
        self.wstruct = AttnWeights(*[_ptr(self.tensors.get(k)) for k in ("w_qkv", "s_qkv", "w_o", "s_o")])
        h = C.c_void_p()
        _check(_lib.m2_attn_create(C.byref(self.cfg), C.byref(self.wstruct), C.byref(h)))
        self.handle = h
        self._ws: Dict[int, torch.Tensor] = {}

    def __del__(self):
        h = getattr(self, "handle", None)
        if h:
            _lib.m2_attn_destroy(h)
            self.handle = None

    def workspace(self, batch: int) -> torch.Tensor:
        ws = self._ws.get(batch)
        if ws is None:
            n = int(_lib.m2_attn_workspace(self.handle, batch))
            if n == 0:
                raise M2Error(M2_ERR_SHAPE, "no workspace size for batch %d" % batch)
            ws = self._ws[batch] = torch.empty(n, dtype=torch.uint8, device=self.device)
        return ws

    def new_cache(self, n_slots: int):
        """Zeroed device caches k, v (bf16 bits as int16) [n_slots][n_kv][max_len][D] and pos."""
        d = self.dims
        shape = (n_slots, d.n_kv, d.max_len, d.head_dim)
        return (torch.zeros(shape, dtype=torch.int16, device=self.device),
                torch.zeros(shape, dtype=torch.int16, device=self.device),
                torch.zeros(n_slots, dtype=torch.int32, device=self.device))

    def _args(self, kc, vc, pos, x, y, slot_ids, residual, ws, stream):
        d = self.dims
        B = x.shape[0]
        _act(x, (B, d.d_model))
        _act(y, x.shape)
        n_slots = pos.numel()
        shape = (n_slots, d.n_kv, d.max_len, d.head_dim)
        for c in (kc, vc):
            if c.dtype not in (torch.int16, torch.bfloat16) or not c.is_contiguous() or tuple(c.shape) != shape:
                raise ValueError("kv cache must be a contiguous 16-bit tensor of shape %s" % (shape,))
        _tokens(pos, n_slots)
        if slot_ids is not None:
            _tokens(slot_ids, B)
        if ws is None:
            ws = self.workspace(B)
        return (self.handle, _ptr(kc), _ptr(vc), _ptr(pos), n_slots, _ptr(x), _ptr(y), B, _ptr(slot_ids),
                M2_RESIDUAL if residual else 0, _ptr(ws), ws.numel(), _stream(stream))

    def step(self, kc, vc, pos, x, y=None, slot_ids=None, residual=False, ws=None, stream=None):
        """One token for x [B][d_model]; appends to the caches and advances pos in place."""
        if y is None:
            y = torch.empty_like(x)
        _check(_lib.m2_attn_step(*self._args(kc, vc, pos, x, y, slot_ids, residual, ws, stream)))
        return y

    def step_timed(self, kc, vc, pos, x, y, events, slot_ids=None, residual=False, ws=None, stream=None):
        """step() recording five events: before, and after each of its four kernels."""
        ev = (C.c_void_p * 5)(*[getattr(e, "cuda_event", e) for e in events])
        _check(_lib.m2_attn_step_timed(*self._args(kc, vc, pos, x, y, slot_ids, residual, ws, stream), ev))
        return y


M2_LAYER_MIXER, M2_LAYER_ATTN = 0, 1


class StackLayer(C.Structure):
    _fields_ = [("kind", C.c_int32), ("layer", C.c_void_p), ("state", C.c_void_p), ("k_cache", C.c_void_p),
                ("v_cache", C.c_void_p), ("pos", C.c_void_p)]


class Stack:
    """A hybrid layer stack (m2_stack) stepped by one call. entries: (Layer, State) for a
    mixer, (Attn, (k_cache, v_cache, pos)) for an attention layer; references are kept."""

    def __init__(self, entries, n_slots: int):
        self.entries = list(entries)
        table = (StackLayer * len(self.entries))()
        d_model = None
        for i, (lay, st) in enumerate(self.entries):
            if isinstance(lay, Layer):
                table[i] = StackLayer(M2_LAYER_MIXER, lay.handle.value, st.handle.value, None, None, None)
            else:
                kc, vc, pos = st
                table[i] = StackLayer(M2_LAYER_ATTN, lay.handle.value, None, _ptr(kc), _ptr(vc), _ptr(pos))
            d_model = lay.dims.d_model
        self.d_model = d_model
        self.device = self.entries[0][0].device
        h = C.c_void_p()
        _check(_lib.m2_stack_create(table, len(self.entries), n_slots, C.byref(h)))
        self.handle = h
        self._ws: Dict[int, torch.Tensor] = {}

    def __del__(self):
        h = getattr(self, "handle", None)
        if h:
            _lib.m2_stack_destroy(h)
            self.handle = None

    def workspace(self, batch: int, persistent: bool = False) -> torch.Tensor:
        key = (batch, persistent)
        ws = self._ws.get(key)
        if ws is None:
            n = int(_lib.m2_stack_workspace_flags(self.handle, batch, M2_PERSISTENT if persistent else 0))
            if n == 0:
                raise M2Error(M2_ERR_SHAPE, "no workspace size for batch %d" % batch)
            ws = self._ws[key] = torch.empty(n, dtype=torch.uint8, device=self.device)
        return ws

    def persistent_runs(self, batch: int) -> int:
        """Persistent launches per step with M2_PERSISTENT (m2_stack_persistent_runs)."""
        return int(_lib.m2_stack_persistent_runs(self.handle, batch, M2_PERSISTENT))

    def step(self, x: torch.Tensor, y: Optional[torch.Tensor] = None, slot_ids: Optional[torch.Tensor] = None,
             ws: Optional[torch.Tensor] = None, stream=None, persistent: bool = False) -> torch.Tensor:
        """One token through every layer (residual chain); returns y [B][d_model].
        persistent: each run of mixer layers in one persistent launch where that applies."""
        B = x.shape[0]
        _act(x, (B, self.d_model))
        if y is None:
            y = torch.empty_like(x)
        _act(y, x.shape)
        if slot_ids is not None:
            _tokens(slot_ids, B)
        if ws is None:
            ws = self.workspace(B, persistent)
        _check(_lib.m2_stack_step_flags(self.handle, _ptr(x), _ptr(y), B, _ptr(slot_ids),
                                        M2_PERSISTENT if persistent else 0, _ptr(ws), ws.numel(), _stream(stream)))
        return y
