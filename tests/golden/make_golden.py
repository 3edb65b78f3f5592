"""Write the oracle's expected values for the two full-size workloads that are too slow
to recompute inside a GPU test (the 27-layer int8 stack and the 2048-token prefill
followed by 750 decode steps).

Calls only the CPU oracle (oracle/) and the seeded input generator; no value here
comes from the HIP path. Sessions are independent, so the oracle runs a subset of
each workload's sessions; the GPU test runs every session and compares the subset.

    python tests/golden/make_golden.py [stack|prefill|all]

Stored per workload (float64 unless noted):
  y at sampled steps / tokens for the sampled sessions (float32),
  per-(layer, session, head) max |S| of the state and the state at 4096 sampled
  (head, p, n) positions, per-(layer, session) max |cache| of the conv cache and
  the cache at 4096 sampled (tap, channel) positions.
"""
import os
import sys
import time

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
sys.path.insert(0, ROOT)

import oracle  # noqa: E402
from full_duplex_speech_mamba2_amd import synth  # noqa: E402

N_STATE_SAMPLES = 4096


def state_positions(dims, seed):
    r = np.random.default_rng(seed)
    h = r.integers(0, dims.n_heads, N_STATE_SAMPLES)
    p = r.integers(0, dims.head_dim, N_STATE_SAMPLES)
    n = r.integers(0, dims.d_state, N_STATE_SAMPLES)
    return np.stack([h, p, n]).astype(np.int32)


def conv_positions(dims, seed):
    r = np.random.default_rng(seed)
    k = r.integers(0, dims.d_conv - 1, N_STATE_SAMPLES)
    c = r.integers(0, dims.conv_dim, N_STATE_SAMPLES)
    return np.stack([k, c]).astype(np.int32)


def state_record(ssm, conv, pos, cpos):
    """ssm [S][H][P][N], conv [S][K-1][C] (sampled sessions) -> (head max, samples,
    cache max, cache samples)."""
    hmax = np.max(np.abs(ssm), axis=(2, 3))
    samp = ssm[:, pos[0], pos[1], pos[2]]
    cmax = np.max(np.abs(conv), axis=(1, 2))
    csamp = conv[:, cpos[0], cpos[1]]
    return hmax, samp, cmax, csamp


def make_stack():
    wl = synth.workload(3)
    d = wl.dims
    sessions = np.array([0, 5], np.int32)
    steps_kept = np.array([0, 1, 4, 19, 39, 59, 79, 99], np.int32)
    t0 = time.time()
    layers = [oracle.Layer(d, synth.make_layer_weights(d, wl.weight_seed, l)) for l in range(wl.layers)]
    print("weights %.1f s" % (time.time() - t0), flush=True)
    xs = synth.make_inputs(d, wl.seed, wl.steps, wl.batch)[:, sessions].astype(np.float64)
    states = [lay.new_state(len(sessions)) for lay in layers]
    ys = []
    for t in range(wl.steps):
        u = xs[t]
        for lay, (s, c) in zip(layers, states):
            u = lay.step(s, c, u, residual=True)
        if t in steps_kept:
            ys.append(u.astype(np.float32))
        if t % 10 == 0:
            print("step %d %.1f s" % (t, time.time() - t0), flush=True)
    pos, cpos = state_positions(d, 303), conv_positions(d, 304)
    recs = [state_record(s, c, pos, cpos) for s, c in states]
    np.savez_compressed(os.path.join(HERE, "stack_int8_27layers_b8_100steps.npz"),
                        sessions=sessions, steps=steps_kept, y=np.array(ys), pos=pos, cpos=cpos,
                        hmax=np.array([r[0] for r in recs]), samples=np.array([r[1] for r in recs]),
                        cmax=np.array([r[2] for r in recs]), csamples=np.array([r[3] for r in recs]))
    print("stack done %.1f s" % (time.time() - t0), flush=True)


def make_prefill():
    wl = synth.workload(4)
    d = wl.dims
    sessions = np.array([0, 3], np.int32)
    tok_kept = np.array([0, 1, 2, 255, 256, 257, 1023, 1536, 2046, 2047], np.int32)
    steps_kept = np.array([0, 1, 99, 374, 749], np.int32)
    t0 = time.time()
    lay = oracle.Layer(d, synth.make_layer_weights(d, wl.weight_seed))
    prompt = synth.make_prompt(d, wl.seed, wl.batch, wl.prefill)[sessions].astype(np.float64)
    xs = synth.make_inputs(d, wl.seed, wl.steps, wl.batch)[:, sessions].astype(np.float64)
    s, c = lay.new_state(len(sessions))
    ypf = lay.prefill(s, c, prompt)
    print("prefill %.1f s" % (time.time() - t0), flush=True)
    pos, cpos = state_positions(d, 404), conv_positions(d, 405)
    after_prefill = state_record(s, c, pos, cpos)
    ys = []
    for t in range(wl.steps):
        y = lay.step(s, c, xs[t])
        if t in steps_kept:
            ys.append(y.astype(np.float32))
    after_decode = state_record(s, c, pos, cpos)
    np.savez_compressed(os.path.join(HERE, "prefill2048_decode750_bf16_b4.npz"),
                        sessions=sessions, tokens=tok_kept, y_prefill=ypf[:, tok_kept].astype(np.float32),
                        steps=steps_kept, y_decode=np.array(ys), pos=pos, cpos=cpos,
                        hmax_prefill=after_prefill[0], samples_prefill=after_prefill[1],
                        cmax_prefill=after_prefill[2], csamples_prefill=after_prefill[3],
                        hmax_decode=after_decode[0], samples_decode=after_decode[1],
                        cmax_decode=after_decode[2], csamples_decode=after_decode[3])
    print("prefill+decode done %.1f s" % (time.time() - t0), flush=True)


if __name__ == "__main__":
    which = sys.argv[1] if len(sys.argv) > 1 else "all"
    if which in ("stack", "all"):
        make_stack()
    if which in ("prefill", "all"):
        make_prefill()
