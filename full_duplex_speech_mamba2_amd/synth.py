"""Seeded synthetic inputs for the Mamba-2 mixer layer (data only).

This module draws weights, per-frame inputs and initial states. It holds none
of the mixer's arithmetic: both the HIP path and the CPU oracle take what it
produces as plain arrays.

Workload shapes follow the backbone the pages describe: a Nemotron-Nano-9B-v2
hybrid Mamba-2/attention LLM (page "NemotronLabs VoiceChat 11B: GPTQ 3-bit LLM,
MLX", introduction) that advances one token per 80 ms frame (page
"NemotronLabs VoiceChat" of the SGLang-Omni cookbook, introduction and "Request
parameters"), after a system-prompt prefill (same GPTQ page, "Recipe"). The
pages give no layer dimensions; the 9B-shaped dimensions and the distributions
below are the stated workload configurations of this library.

Random streams: numpy PCG64 seeded by SeedSequence([seed, layer, tag]) per tensor,
and by SeedSequence([seed, layer, tag, block]) per block of 512 rows of the two
projection matrices (drawn on a small thread pool), so every tensor is
reproducible on its own.

Distributions (variance reading of "N(0, v)"):
  W_in ~ N(0, 1/d_model), W_out ~ N(0, 1/d_inner)   (bf16: rounded to nearest even)
  int8 weights: q ~ U{-127..127}, fp16 scales ~ U[0.5, 2]/127 per (row, K-group)
  4- and 3-bit weights: the fp32 N(0, 1/K) matrix quantized per (row, group of
    q_group columns) to nearest with the group's min and max: scale =
    fp16((max - min) / (2^bits - 1)), bias = fp16(min), code = clip(rint((w - bias) /
    scale)), so w ~ scale code + bias; packed as the library and the oracle read them
    (4-bit: two codes per byte, the even one in the low nibble; 3-bit: 32 codes in 12
    bytes, code i at bits 3i..3i+2 of the little-endian 96-bit run)
  conv_w, conv_b ~ N(0, 1/4); norm_w ~ U[0.5, 1.5]; D ~ N(0, 1)
  A_log ~ U[0, ln 16]  (so A = -exp(A_log) lies in [-16, -1])
  dt_bias = softplus^-1(dt0), dt0 = exp(U[ln 1e-3, ln 0.1])
  per-frame inputs x ~ N(0, 1) fp32
  output heads [vocab][d_model] as W_in (tags text_head, func_head); head inputs h ~ N(0, 1)
  attention layers: W_qkv ~ N(0, 1/d_model), W_o ~ N(0, 1/(n_q head_dim)) in the same
    formats; cached keys and values ~ N(0, 1) rounded to bf16 below each session's
    position and NaN at and above it (so that any read past the position shows)
"""
from __future__ import annotations

import dataclasses
import math
from typing import Dict, Optional

import numpy as np

WTYPES = ("f32", "bf16", "int8g", "int4g", "int3g")
LOWBIT = {"int4g": 4, "int3g": 3}

# one integer tag per tensor: the third word of the SeedSequence
_TAGS = {
    "w_in": 1, "s_in": 2, "w_out": 3, "s_out": 4, "conv_w": 5, "conv_b": 6,
    "dt_bias": 7, "A_log": 8, "D": 9, "norm_w": 10,
    "x": 20, "prompt": 21, "ssm0": 22, "conv0": 23,
    "text_head": 30, "text_head_s": 31, "func_head": 32, "func_head_s": 33, "head_h": 34,
    "w_qkv": 40, "s_qkv": 41, "w_o": 42, "s_o": 43, "kv_k": 44, "kv_v": 45, "attn_x": 46,
}


@dataclasses.dataclass(frozen=True)
class MixerDims:
    d_model: int
    n_heads: int
    head_dim: int
    d_state: int
    n_groups: int
    d_conv: int = 4
    norm_group: int = 0          # channels per RMS group; 0 means d_inner / n_groups
    norm_eps: float = 1e-5
    wtype: str = "bf16"
    q_group: int = 128
    q_gamma_in: float = 1.0      # per-tensor dequant multiplier (quantized weights)
    q_gamma_out: float = 1.0

    @property
    def d_inner(self) -> int:
        return self.n_heads * self.head_dim

    @property
    def conv_dim(self) -> int:
        return self.d_inner + 2 * self.n_groups * self.d_state

    @property
    def d_in_proj(self) -> int:
        return 2 * self.d_inner + 2 * self.n_groups * self.d_state + self.n_heads

    @property
    def rms_group(self) -> int:
        return self.norm_group if self.norm_group > 0 else self.d_inner // self.n_groups

    def replace(self, **kw) -> "MixerDims":
        return dataclasses.replace(self, **kw)


TINY = MixerDims(d_model=256, n_heads=8, head_dim=32, d_state=16, n_groups=1,
                 d_conv=4, wtype="f32")
NINE_B = MixerDims(d_model=4480, n_heads=128, head_dim=80, d_state=128, n_groups=8,
                   d_conv=4, wtype="bf16")
NINE_B_INT8 = NINE_B.replace(wtype="int8g", q_group=128,
                             q_gamma_in=float(np.float32(1.0 / math.sqrt(4480))),
                             q_gamma_out=float(np.float32(1.0 / math.sqrt(10240))))
NINE_B_INT4 = NINE_B.replace(wtype="int4g", q_group=64)
NINE_B_INT3 = NINE_B.replace(wtype="int3g", q_group=64)


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    dims: MixerDims
    batch: int
    steps: int
    layers: int = 1
    prefill: int = 0             # prompt length before decode (0: none)
    chunk: int = 256
    weight_seed: int = 0
    seed: int = 0
    state_var: float = 0.0       # variance of the initial state and conv cache (0: zeros)


WORKLOADS: Dict[int, Workload] = {
    0: Workload("tiny_fp32_b1_16steps", TINY, batch=1, steps=16, weight_seed=0, seed=0),
    1: Workload("mamba2_9b_bf16_b1_decode750", NINE_B, batch=1, steps=750,
                weight_seed=1, seed=1),
    2: Workload("mamba2_9b_bf16_b32_decode200", NINE_B, batch=32, steps=200,
                weight_seed=1, seed=2, state_var=0.1),
    3: Workload("mamba2_9b_int8g128_27layers_b8_decode100", NINE_B_INT8, batch=8,
                steps=100, layers=27, weight_seed=3, seed=3),
    4: Workload("mamba2_9b_bf16_b4_prefill2048_decode750", NINE_B, batch=4, steps=750,
                prefill=2048, chunk=256, weight_seed=1, seed=4),
    5: Workload("mamba2_9b_int4g64_b1_decode750", NINE_B_INT4, batch=1, steps=750,
                weight_seed=5, seed=5),
    6: Workload("mamba2_9b_int3g64_b1_decode750", NINE_B_INT3, batch=1, steps=750,
                weight_seed=6, seed=6),
}


@dataclasses.dataclass(frozen=True)
class AttnDims:
    """An attention layer of the hybrid backbone: n_q query heads sharing n_kv key/value
    heads of head_dim, a bf16 KV cache of max_len positions per session."""
    d_model: int
    n_q: int
    n_kv: int
    head_dim: int
    max_len: int
    wtype: str = "bf16"
    q_group: int = 128
    q_gamma_qkv: float = 1.0
    q_gamma_o: float = 1.0

    @property
    def qkv_rows(self) -> int:
        return (self.n_q + 2 * self.n_kv) * self.head_dim

    @property
    def o_dim(self) -> int:
        return self.n_q * self.head_dim

    def replace(self, **kw) -> "AttnDims":
        return dataclasses.replace(self, **kw)


# The pages give no attention shapes: a 9B-class grouped-query layout (40 query heads, 8
# key/value heads of 128) is a configured reading; 1500 positions = the 2-minute context
# at one token per 80 ms frame.
ATTN_9B = AttnDims(d_model=4480, n_q=40, n_kv=8, head_dim=128, max_len=1500)


@dataclasses.dataclass(frozen=True)
class HeadWorkload:
    """Per-frame greedy decode of the output heads: `heads` matrices of [vocab][d_model]
    (the text head, then the function head) over `batch` sessions' final hidden states."""
    name: str
    d_model: int
    vocab: int
    heads: int
    wtype: str
    batch: int
    steps: int
    q_group: int = 0
    seed: int = 0


@dataclasses.dataclass(frozen=True)
class AttnWorkload:
    """Attention-layer decode for `batch` sessions whose caches hold `start_pos` positions
    when timing starts; consecutive steps take consecutive sets of sessions (slot_sets
    disjoint sets, so every set's cache advances once per slot_sets steps)."""
    name: str
    dims: AttnDims
    batch: int
    steps: int
    start_pos: int
    slot_sets: int
    seed: int = 0


ATTN_WORKLOADS: Dict[int, AttnWorkload] = {
    8: AttnWorkload("attn_9b_bf16_b1_ctx1000_decode", ATTN_9B, batch=1, steps=750, start_pos=1000,
                    slot_sets=8, seed=8),
    10: AttnWorkload("attn_9b_bf16_b32_ctx1000_decode", ATTN_9B, batch=32, steps=100, start_pos=1000,
                     slot_sets=8, seed=10),
}


@dataclasses.dataclass(frozen=True)
class StackWorkload:
    """A hybrid stack stepped as one call: `pattern` lists the layers in order (M: Mamba-2
    mixer, A: attention); attention caches hold `start_pos` positions when timing starts and
    consecutive steps take consecutive sets of sessions (slot_sets sets)."""
    name: str
    mixer: MixerDims
    attn: AttnDims
    pattern: str
    batch: int
    steps: int
    start_pos: int
    slot_sets: int
    seed: int = 0


# 27 Mamba-2 mixers and 4 attention layers spread through the stack: a configured reading of
# the 9B hybrid backbone (its MLP layers are not part of this path).
HYBRID_9B_PATTERN = "MMMMMMMAMMMMMMMAMMMMMMMAMMMMMMA"

STACK_WORKLOADS: Dict[int, StackWorkload] = {
    9: StackWorkload("hybrid_27m4a_9b_bf16_b1_decode", NINE_B, ATTN_9B, HYBRID_9B_PATTERN, batch=1, steps=750,
                     start_pos=1000, slot_sets=8, seed=9),
}


# The pages give no vocabulary size: 131072 rows per head is a configured reading, with the
# function head taken to be a second head of the text head's shape.
HEAD_WORKLOADS: Dict[int, HeadWorkload] = {
    7: HeadWorkload("heads_2x131072x4480_bf16_b1_decode750", d_model=4480, vocab=131072, heads=2,
                    wtype="bf16", batch=1, steps=750, seed=7),
}


def _rng(seed: int, layer: int, tag: str, block: int = -1) -> np.random.Generator:
    words = [seed, layer, _TAGS[tag]] + ([block] if block >= 0 else [])
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence(words)))


def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """Round finite float32 values to bfloat16 (nearest, ties to even); return uint16 bit patterns."""
    u = np.array(a, dtype=np.float32, copy=True).view(np.uint32)
    lsb = (u >> 16) & 1
    u += np.uint32(0x7FFF)
    u += lsb
    return (u >> 16).astype(np.uint16)


_ROW_BLOCK = 512          # rows per independent random stream of a weight matrix


def _blocked(rows, fill):
    """Run fill(block_index, row0, row1) over row blocks on a small thread pool."""
    import concurrent.futures as cf
    import os
    blocks = [(i, r, min(rows, r + _ROW_BLOCK)) for i, r in enumerate(range(0, rows, _ROW_BLOCK))]
    workers = max(1, min(16, len(os.sched_getaffinity(0)) if hasattr(os, "sched_getaffinity") else 4))
    with cf.ThreadPoolExecutor(workers) as ex:
        list(ex.map(lambda b: fill(*b), blocks))


def _normal(seed, layer, tag, shape, std, wtype):
    rows, k = shape
    out = np.empty(shape, np.uint16 if wtype == "bf16" else np.float32)

    def fill(i, r0, r1):
        w = _rng(seed, layer, tag, i).standard_normal((r1 - r0, k), dtype=np.float32)
        w *= np.float32(std)
        out[r0:r1] = f32_to_bf16_bits(w) if wtype == "bf16" else w
    _blocked(rows, fill)
    return out


def _int8(seed, layer, tq, ts, rows, k, group):
    q = np.empty((rows, k), np.int8)
    s = np.empty((rows, k // group), np.float16)

    def fill(i, r0, r1):
        q[r0:r1] = _rng(seed, layer, tq, i).integers(-127, 128, size=(r1 - r0, k), dtype=np.int8)
        s[r0:r1] = (_rng(seed, layer, ts, i).uniform(0.5, 2.0, size=(r1 - r0, k // group)) / 127.0
                    ).astype(np.float16)
    _blocked(rows, fill)
    return q, s


def pack_codes(q: np.ndarray, bits: int) -> np.ndarray:
    """Unsigned codes q [rows][K] (values < 2^bits) -> packed uint8 rows [rows][K bits / 8]."""
    q = np.ascontiguousarray(q, dtype=np.uint8)
    rows, K = q.shape
    if bits == 4:
        return (q[:, 0::2] | (q[:, 1::2] << 4)).astype(np.uint8)
    runs = q.reshape(rows, K // 32, 32).astype(np.uint64)
    lo = np.zeros((rows, K // 32), np.uint64)      # bits 0..63 of each 96-bit run
    hi = np.zeros((rows, K // 32), np.uint64)      # bits 64..95
    for i in range(32):
        b = 3 * i
        if b + 3 <= 64:
            lo |= runs[..., i] << np.uint64(b)
        elif b >= 64:
            hi |= runs[..., i] << np.uint64(b - 64)
        else:                                      # straddles bit 64
            lo |= (runs[..., i] << np.uint64(b)) & np.uint64(0xFFFFFFFFFFFFFFFF)
            hi |= runs[..., i] >> np.uint64(64 - b)
    out = np.empty((rows, K // 32, 12), np.uint8)
    out[..., :8] = lo[..., None].view(np.uint8).reshape(rows, K // 32, 8)
    out[..., 8:] = hi[..., None].view(np.uint8).reshape(rows, K // 32, 8)[..., :4]
    return out.reshape(rows, K // 32 * 12)


def _lowbit(seed, layer, tq, rows, k, group, bits, std):
    packed = np.empty((rows, k * bits // 8), np.uint8)
    sb = np.empty((rows, k // group, 2), np.float16)
    top = float(2 ** bits - 1)

    def fill(i, r0, r1):
        w = _rng(seed, layer, tq, i).standard_normal((r1 - r0, k), dtype=np.float32) * np.float32(std)
        g = w.reshape(r1 - r0, k // group, group)
        mn, mx = g.min(axis=2), g.max(axis=2)
        sc = ((mx - mn) / np.float32(top)).astype(np.float16)
        bi = mn.astype(np.float16)
        scf = np.maximum(sc.astype(np.float32), np.float32(1e-7))
        q = np.clip(np.rint((g - bi.astype(np.float32)[..., None]) / scf[..., None]), 0, top).astype(np.uint8)
        packed[r0:r1] = pack_codes(q.reshape(r1 - r0, k), bits)
        sb[r0:r1, :, 0] = sc
        sb[r0:r1, :, 1] = bi
    _blocked(rows, fill)
    return packed, sb


def make_layer_weights(dims: MixerDims, seed: int, layer: int = 0) -> Dict[str, Optional[np.ndarray]]:
    """All parameters of one mixer layer.

    w_in [d_in_proj][d_model] and w_out [d_model][d_inner] are row-major with K
    contiguous: float32 (wtype f32), uint16 bf16 bits (bf16) or int8 (int8g, with
    float16 scales s_in [d_in_proj][d_model/q_group], s_out [d_model][d_inner/q_group]),
    or packed 4/3-bit codes as uint8 [rows][K bits/8] (int4g, int3g) with float16
    (scale, bias) pairs s_in [d_in_proj][d_model/q_group][2], s_out [d_model][d_inner/q_group][2].
    conv_w is [conv_dim][d_conv] with tap d_conv-1 multiplying the newest input.
    """
    d = dims
    w: Dict[str, Optional[np.ndarray]] = {"s_in": None, "s_out": None}
    if d.wtype == "int8g":
        w["w_in"], w["s_in"] = _int8(seed, layer, "w_in", "s_in", d.d_in_proj, d.d_model, d.q_group)
        w["w_out"], w["s_out"] = _int8(seed, layer, "w_out", "s_out", d.d_model, d.d_inner, d.q_group)
    elif d.wtype in LOWBIT:
        b = LOWBIT[d.wtype]
        w["w_in"], w["s_in"] = _lowbit(seed, layer, "w_in", d.d_in_proj, d.d_model, d.q_group, b,
                                       1.0 / math.sqrt(d.d_model))
        w["w_out"], w["s_out"] = _lowbit(seed, layer, "w_out", d.d_model, d.d_inner, d.q_group, b,
                                         1.0 / math.sqrt(d.d_inner))
    else:
        w["w_in"] = _normal(seed, layer, "w_in", (d.d_in_proj, d.d_model),
                            1.0 / math.sqrt(d.d_model), d.wtype)
        w["w_out"] = _normal(seed, layer, "w_out", (d.d_model, d.d_inner),
                             1.0 / math.sqrt(d.d_inner), d.wtype)
    w["conv_w"] = (_rng(seed, layer, "conv_w").standard_normal((d.conv_dim, d.d_conv)) * 0.5).astype(np.float32)
    w["conv_b"] = (_rng(seed, layer, "conv_b").standard_normal(d.conv_dim) * 0.5).astype(np.float32)
    dt0 = np.exp(_rng(seed, layer, "dt_bias").uniform(math.log(1e-3), math.log(0.1), d.n_heads))
    w["dt_bias"] = np.log(np.expm1(dt0)).astype(np.float32)          # inverse softplus of dt0
    w["A_log"] = _rng(seed, layer, "A_log").uniform(0.0, math.log(16.0), d.n_heads).astype(np.float32)
    w["D"] = _rng(seed, layer, "D").standard_normal(d.n_heads).astype(np.float32)
    w["norm_w"] = _rng(seed, layer, "norm_w").uniform(0.5, 1.5, d.d_inner).astype(np.float32)
    return w


def make_inputs(dims: MixerDims, seed: int, steps: int, batch: int, tag: str = "x") -> np.ndarray:
    """Per-frame fused embeddings x[steps][batch][d_model] ~ N(0, 1), float32."""
    return _rng(seed, 0, tag).standard_normal((steps, batch, dims.d_model), dtype=np.float32)


def make_prompt(dims: MixerDims, seed: int, batch: int, seqlen: int) -> np.ndarray:
    """Prompt embeddings x[batch][seqlen][d_model] ~ N(0, 1), float32."""
    return _rng(seed, 0, "prompt").standard_normal((batch, seqlen, dims.d_model), dtype=np.float32)


def make_state(dims: MixerDims, seed: int, n_slots: int, var: float, layer: int = 0):
    """Initial SSM state [slots][H][P][N] and conv cache [slots][d_conv-1][conv_dim], float32."""
    d = dims
    ssm_shape = (n_slots, d.n_heads, d.head_dim, d.d_state)
    conv_shape = (n_slots, d.d_conv - 1, d.conv_dim)
    if var == 0.0:
        return np.zeros(ssm_shape, np.float32), np.zeros(conv_shape, np.float32)
    std = np.float32(math.sqrt(var))
    ssm = _rng(seed, layer, "ssm0").standard_normal(ssm_shape, dtype=np.float32) * std
    conv = _rng(seed, layer, "conv0").standard_normal(conv_shape, dtype=np.float32) * std
    return ssm, conv


def workload(i: int) -> Workload:
    return WORKLOADS[i]


def make_head_weights(vocab: int, d_model: int, wtype: str, q_group: int, seed: int,
                      tag: str = "text_head"):
    """An output head [vocab][d_model] in the layer matrices' storage formats, W ~ N(0, 1/d_model)
    (int8g: uniform codes with scales as for w_in); returns (w, scales or None)."""
    if wtype == "int8g":
        return _int8(seed, 0, tag, tag + "_s", vocab, d_model, q_group)
    if wtype in LOWBIT:
        return _lowbit(seed, 0, tag, vocab, d_model, q_group, LOWBIT[wtype], 1.0 / math.sqrt(d_model))
    return _normal(seed, 0, tag, (vocab, d_model), 1.0 / math.sqrt(d_model), wtype), None


def make_head_states(d_model: int, batch: int, seed: int, tag: str = "head_h") -> np.ndarray:
    """Final hidden states h[batch][d_model] ~ N(0, 1), float32, fed to the output heads."""
    return _rng(seed, 0, tag).standard_normal((batch, d_model), dtype=np.float32)


def make_attn_weights(dims: AttnDims, seed: int, layer: int = 0) -> Dict[str, Optional[np.ndarray]]:
    """W_qkv [(n_q + 2 n_kv) head_dim][d_model] and W_o [d_model][n_q head_dim] in the layer
    matrices' storage formats, with scales s_qkv, s_o for the quantized ones."""
    d = dims
    w: Dict[str, Optional[np.ndarray]] = {"s_qkv": None, "s_o": None}
    for wn, sn, rows, k in (("w_qkv", "s_qkv", d.qkv_rows, d.d_model), ("w_o", "s_o", d.d_model, d.o_dim)):
        if d.wtype == "int8g":
            w[wn], w[sn] = _int8(seed, layer, wn, sn, rows, k, d.q_group)
        elif d.wtype in LOWBIT:
            w[wn], w[sn] = _lowbit(seed, layer, wn, rows, k, d.q_group, LOWBIT[d.wtype], 1.0 / math.sqrt(k))
        else:
            w[wn] = _normal(seed, layer, wn, (rows, k), 1.0 / math.sqrt(k), d.wtype)
    return w


def make_kv_cache(dims: AttnDims, seed: int, pos, layer: int = 0):
    """bf16 bits k, v [n_slots][n_kv][max_len][head_dim] for sessions at positions pos
    [n_slots]: N(0, 1) entries below pos[s], NaN (0x7FC0) from pos[s] on."""
    pos = np.asarray(pos, np.int32)
    shape = (len(pos), dims.n_kv, dims.max_len, dims.head_dim)
    out = []
    for tag in ("kv_k", "kv_v"):
        c = f32_to_bf16_bits(_rng(seed, layer, tag).standard_normal(shape, dtype=np.float32))
        for s_, p in enumerate(pos):
            c[s_, :, p:, :] = 0x7FC0
        out.append(c)
    return out[0], out[1]


def make_attn_inputs(dims: AttnDims, seed: int, steps: int, batch: int) -> np.ndarray:
    """Per-frame attention-layer inputs u[steps][batch][d_model] ~ N(0, 1), float32."""
    return _rng(seed, 0, "attn_x").standard_normal((steps, batch, dims.d_model), dtype=np.float32)
