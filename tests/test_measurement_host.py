"""The measurement's accounting on the CPU: the algorithmic bytes per step that every bench
line's GB/s and roofline rest on, against figures derived from the layer shapes alone (the
weights a step must stream once, the state read and written once), and the weight rotation
that keeps the last-level cache from serving a step."""
import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

import bench  # noqa: E402
from full_duplex_speech_mamba2_amd import synth  # noqa: E402

MB = 1e6


def _weights(d):
    """Stored bytes of W_in and W_out from the shapes: rows z | x | B | C | dt of d_model, and
    d_model rows of d_inner, at the format's width, plus its per-group scale words."""
    d_inner = d.n_heads * d.head_dim
    rows_in = 2 * d_inner + 2 * d.n_groups * d.d_state + d.n_heads
    width = {"f32": 4.0, "bf16": 2.0, "int8g": 1.0, "int4g": 0.5, "int3g": 0.375}[d.wtype]
    scale = {"int8g": 2, "int4g": 4, "int3g": 4}.get(d.wtype, 0)
    w_in = rows_in * d.d_model * width + (rows_in * (d.d_model // d.q_group) * scale if scale else 0)
    w_out = d.d_model * d_inner * width + (d.d_model * (d_inner // d.q_group) * scale if scale else 0)
    return w_in, w_out


@pytest.mark.parametrize("config,step_mb", [(1, 305.9), (2, 641.2), (3, 236.5), (4, 338.3)])
def test_step_bytes_match_the_workload_table(config, step_mb):
    """The per-layer step bytes of the four decode workloads as the workload table states them
    (9B shapes: 294.75 MB of bf16 weights, 10.49 MB of state per session read and written)."""
    wl = synth.workload(config)
    kb = bench.kernel_bytes(wl.dims, wl.batch)
    assert abs(kb["step"] / MB - step_mb) < 0.05


@pytest.mark.parametrize("config", [1, 2, 3, 4, 5, 6])
def test_phase_bytes_are_weights_plus_small_terms(config):
    """Each GEMV phase moves its matrix once plus activations; the SSD phase the state once in
    and once out plus the conv inputs; the phases together cover the step."""
    wl = synth.workload(config)
    d, B = wl.dims, wl.batch
    kb = bench.kernel_bytes(d, B)
    w_in, w_out = _weights(d)
    state = 2 * B * d.n_heads * d.head_dim * d.d_state * 4
    assert 0 <= kb["gemv_in"] - w_in < 1.0 * MB * max(1, B)
    assert 0 <= kb["gemv_out"] - w_out < 0.5 * MB * max(1, B)
    assert 0 <= kb["ssd_step"] - state < 0.6 * MB * max(1, B)
    # the step counts each byte once; the phases double-count only the hand-offs between them
    assert kb["step"] <= kb["gemv_in"] + kb["ssd_step"] + kb["gemv_out"]
    assert kb["step"] >= w_in + w_out + state


def test_head_and_attention_bytes():
    """A 131072 x 4480 bf16 head streams 1,174.4 MB per launch; the 9B-shaped attention layer
    moves its QKV (7168 x 4480) and O (4480 x 5120) weights plus the cache rows attended."""
    h = synth.HEAD_WORKLOADS[7]
    assert bench.head_bytes(h)["head_wave"] == 131072 * 4480 * 2 + h.batch * 4480 * 4
    a = synth.ATTN_WORKLOADS[8]
    ab = bench.attn_bytes(a, 1188.0)
    assert abs(ab["qkv_gemv"] / MB - 64.27) < 0.01 and abs(ab["o_gemv"] / MB - 45.93) < 0.01
    cache = 2 * a.batch * a.dims.n_kv * 1188 * a.dims.head_dim * 2
    assert abs(ab["step"] - (7168 * 4480 * 2 + 4480 * 5120 * 2 + cache)) < 0.1 * MB


@pytest.mark.parametrize("config", [1, 2, 4, 5, 6])
def test_weight_rotation_exceeds_the_last_level_cache(config):
    """The single-layer workloads rotate enough identical weight copies that at least 2.5 GB
    (about ten times the 256 MB last-level cache) stream through between two reads of a copy,
    even counting only W_out, the matrix read with cache-allocating loads before."""
    wl = synth.workload(config)
    kb = bench.kernel_bytes(wl.dims, 1)
    per = kb["gemv_in"] + kb["gemv_out"]
    copies = max(2, -(-bench.ROTATION_BYTES // per))
    assert copies * per >= 2.5e9
    assert copies * kb["gemv_out"] > 2 * 256 * 2 ** 20


def test_bench_refuses_more_than_one_gpu():
    """The library runs on one GPU: asked for several, the bench exits with status 2 and a
    message saying so, before touching a device."""
    import subprocess
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
