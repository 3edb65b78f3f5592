"""Parity of the HIP path with the fp64 oracle on the full-size workloads, in the
launch configurations the bench times (m2_step / m2_prefill through the C ABI):

  9B-shaped layer, bf16, 1 session, 750 steps       oracle run live on the session
  9B-shaped layer, bf16, 32 sessions, 200 steps     oracle run live on 3 of the sessions
  27-layer int8 (g128) residual stack, 8 sessions   oracle run live on one session (every
      x 100 steps                                   step's output, every layer's whole state
                                                    and cache); stored oracle values
                                                    (tests/golden/make_golden.py) for two
                                                    more sessions, sampled
  bf16, 4 sessions, 2048-token chunked prefill      oracle run live on one session (every
      then 750 decode steps                         prompt token and step, whole state and
                                                    cache); stored values for two more
  int4 g64 and int3 g64 weights, 1 session,         oracle run live
      750 steps
  one int8 g128 layer with the stated scales and    oracle run live (1 and 8 sessions)
      no per-tensor gamma (gamma = 1)

The tiny fp32 workload runs in test_decode_gpu.py. Sessions are independent, so
checking a subset of them checks the batched kernels on those sessions; against the
stored values the state is compared at 4096 sampled (head, p, n) positions per layer
and session against the oracle's per-head maximum (the normwise measure of parity.py).
"""
import os

import numpy as np
import pytest

from full_duplex_speech_mamba2_amd import synth
from parity import TOL_OUT, TOL_STATE, e_conv, e_out, e_state, gpu_decode, oracle_decode

pytestmark = pytest.mark.gpu

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _report(tag, **errs):
    print("[parity] %s %s" % (tag, " ".join("%s=%.3e" % kv for kv in errs.items())), flush=True)


def e_state_sampled(S, pos, samples, hmax):
    """S [H][P][N] of one session (GPU), the oracle's values at pos = [h, p, n] and its
    per-head max |S|: max over sampled positions of |S - So| / max(hmax[h], 1e-6 max hmax)."""
    if not np.all(np.isfinite(S)):
        return float("inf")
    h = pos[0]
    floor = 1e-6 * max(float(np.max(hmax)), 1e-30)
    d = np.abs(S[pos[0], pos[1], pos[2]].astype(np.float64) - samples)
    return float(np.max(d / np.maximum(hmax[h], floor)))


def e_conv_sampled(C, cpos, csamples, cmax):
    """C [K-1][conv_dim] of one session against the oracle at cpos = [k, c]."""
    if not np.all(np.isfinite(C)):
        return float("inf")
    d = np.abs(C[cpos[0], cpos[1]].astype(np.float64) - csamples)
    return float(np.max(d / max(float(cmax), 1e-30)))


@pytest.mark.parametrize("persistent", [False, True])
def test_9b_bf16_single_session_750_steps(persistent):
    """The headline workload on the three-kernel plan (as timed) and on plan 2."""
    wl = synth.workload(1)
    w = synth.make_layer_weights(wl.dims, wl.weight_seed)
    xs = synth.make_inputs(wl.dims, wl.seed, wl.steps, wl.batch)
    ssm0, conv0 = synth.make_state(wl.dims, wl.seed, wl.batch, wl.state_var)
    yg, sg, cg = gpu_decode(wl.dims, w, xs, ssm0, conv0, persistent=persistent)
    yo, so, co = oracle_decode(wl.dims, w, xs, ssm0, conv0)
    eo, es, ec = e_out(yg, yo), e_state(sg, so), e_conv(cg, co)
    _report(wl.name + (" persistent" if persistent else ""), e_out=eo, e_state=es, e_conv=ec)
    assert eo <= TOL_OUT and es <= TOL_STATE and ec <= TOL_STATE


@pytest.mark.parametrize("config", [5, 6])
def test_9b_lowbit_single_session_750_steps(config):
    """The 9B-shaped layer with 4-bit and 3-bit group-64 weights, oracle run live."""
    wl = synth.workload(config)
    w = synth.make_layer_weights(wl.dims, wl.weight_seed)
    xs = synth.make_inputs(wl.dims, wl.seed, wl.steps, wl.batch)
    ssm0, conv0 = synth.make_state(wl.dims, wl.seed, wl.batch, wl.state_var)
    yg, sg, cg = gpu_decode(wl.dims, w, xs, ssm0, conv0)
    yo, so, co = oracle_decode(wl.dims, w, xs, ssm0, conv0)
    eo, es, ec = e_out(yg, yo), e_state(sg, so), e_conv(cg, co)
    _report(wl.name, e_out=eo, e_state=es, e_conv=ec)
    assert eo <= TOL_OUT and es <= TOL_STATE and ec <= TOL_STATE


def test_9b_bf16_32_sessions_200_steps():
    wl = synth.workload(2)
    w = synth.make_layer_weights(wl.dims, wl.weight_seed)
    xs = synth.make_inputs(wl.dims, wl.seed, wl.steps, wl.batch)
    ssm0, conv0 = synth.make_state(wl.dims, wl.seed, wl.batch, wl.state_var)
    sessions = [0, 17, 31]
    yg, sg, cg = gpu_decode(wl.dims, w, xs, ssm0, conv0)
    yo, so, co = oracle_decode(wl.dims, w, xs, ssm0, conv0, sessions=sessions)
    eo = e_out(yg[:, sessions], yo)
    es, ec = e_state(sg[sessions], so[sessions]), e_conv(cg[sessions], co[sessions])
    _report(wl.name, e_out=eo, e_state=es, e_conv=ec)
    assert eo <= TOL_OUT and es <= TOL_STATE and ec <= TOL_STATE


def test_int8_27_layer_stack_100_steps():
    import torch
    from full_duplex_speech_mamba2_amd import m2
    g = np.load(os.path.join(GOLDEN, "stack_int8_27layers_b8_100steps.npz"))
    wl = synth.workload(3)
    d = wl.dims
    layers, states = [], []
    for l in range(wl.layers):
        lay = m2.Layer(d, synth.make_layer_weights(d, wl.weight_seed, l))
        layers.append(lay)
        states.append(m2.State(lay, wl.batch))
    xs = torch.from_numpy(synth.make_inputs(d, wl.seed, wl.steps, wl.batch)).cuda()
    kept = {int(t): i for i, t in enumerate(g["steps"])}
    sessions = g["sessions"]
    live = LIVE_STACK_SESSION
    assert live not in sessions
    eo = 0.0
    y_live = np.empty((wl.steps, d.d_model), np.float32)
    for t in range(wl.steps):
        u = xs[t].clone()
        for lay, st in zip(layers, states):
            m2.step(lay, st, u, u, residual=True)      # y aliases x under M2_RESIDUAL
        uh = u.cpu().numpy()
        y_live[t] = uh[live]
        if t in kept:
            eo = max(eo, e_out(uh[sessions], g["y"][kept[t]]))
    torch.cuda.synchronize()
    _live_stack_check(wl, [st.ssm.cpu().numpy()[live] for st in states],
                      [st.conv.cpu().numpy()[live] for st in states], y_live, live)
    es = ec = 0.0
    for l, st in enumerate(states):
        S = st.ssm.cpu().numpy()
        C = st.conv.cpu().numpy()
        for j, s in enumerate(sessions):
            es = max(es, e_state_sampled(S[s], g["pos"], g["samples"][l, j], g["hmax"][l, j]))
            ec = max(ec, e_conv_sampled(C[s], g["cpos"], g["csamples"][l, j], g["cmax"][l, j]))
    _report(wl.name, e_out=eo, e_state=es, e_conv=ec)
    assert eo <= TOL_OUT and es <= TOL_STATE and ec <= TOL_STATE


LIVE_STACK_SESSION = 2
LIVE_PREFILL_SESSION = 1


def _live_stack_check(wl, S_gpu, C_gpu, y_gpu, b):
    """The oracle's 27-layer chain for session b alone, every step: each step's output and,
    after the last step, every layer's whole state and conv cache."""
    import oracle
    d = wl.dims
    xs = synth.make_inputs(d, wl.seed, wl.steps, wl.batch)[:, b:b + 1]
    lays = [oracle.Layer(d, synth.make_layer_weights(d, wl.weight_seed, l)) for l in range(wl.layers)]
    sts = [lay.new_state(1) for lay in lays]
    yo = np.empty((wl.steps, d.d_model))
    for t in range(wl.steps):
        u = xs[t].astype(np.float64)
        for lay, (so, co) in zip(lays, sts):
            u = lay.step(so, co, u, residual=True)
        yo[t] = u[0]
    eo = e_out(y_gpu, yo)
    es = max(e_state(S_gpu[l][None], sts[l][0]) for l in range(wl.layers))
    ec = max(e_conv(C_gpu[l][None], sts[l][1]) for l in range(wl.layers))
    _report(wl.name + " live session %d" % b, e_out=eo, e_state=es, e_conv=ec)
    assert eo <= TOL_OUT and es <= TOL_STATE and ec <= TOL_STATE


def test_bf16_prefill_2048_then_750_steps():
    import torch
    from full_duplex_speech_mamba2_amd import m2
    g = np.load(os.path.join(GOLDEN, "prefill2048_decode750_bf16_b4.npz"))
    wl = synth.workload(4)
    d = wl.dims
    lay = m2.Layer(d, synth.make_layer_weights(d, wl.weight_seed))
    st = m2.State(lay, wl.batch)
    prompt = torch.from_numpy(synth.make_prompt(d, wl.seed, wl.batch, wl.prefill)).cuda()
    sessions = g["sessions"]
    ypf = m2.prefill(lay, st, prompt, chunk=wl.chunk)
    torch.cuda.synchronize()
    live = LIVE_PREFILL_SESSION
    assert live not in sessions
    ypf_h = ypf.cpu().numpy()
    eo_pf = e_out(ypf_h[sessions][:, g["tokens"]], g["y_prefill"])
    S, C = st.ssm.cpu().numpy(), st.conv.cpu().numpy()
    live_pf = (ypf_h[live], S[live], C[live])
    es_pf = max(e_state_sampled(S[s], g["pos"], g["samples_prefill"][j], g["hmax_prefill"][j])
                for j, s in enumerate(sessions))
    ec_pf = max(e_conv_sampled(C[s], g["cpos"], g["csamples_prefill"][j], g["cmax_prefill"][j])
                for j, s in enumerate(sessions))
    xs = torch.from_numpy(synth.make_inputs(d, wl.seed, wl.steps, wl.batch)).cuda()
    ys = torch.empty_like(xs)
    for t in range(wl.steps):
        m2.step(lay, st, xs[t], ys[t])
    torch.cuda.synchronize()
    ys_h = ys.cpu().numpy()
    eo_dec = e_out(ys_h[g["steps"]][:, sessions], g["y_decode"])
    S, C = st.ssm.cpu().numpy(), st.conv.cpu().numpy()
    _live_prefill_check(wl, live, live_pf, (ys_h[:, live], S[live], C[live]))
    es_dec = max(e_state_sampled(S[s], g["pos"], g["samples_decode"][j], g["hmax_decode"][j])
                 for j, s in enumerate(sessions))
    ec_dec = max(e_conv_sampled(C[s], g["cpos"], g["csamples_decode"][j], g["cmax_decode"][j])
                 for j, s in enumerate(sessions))
    _report(wl.name, e_out_prefill=eo_pf, e_state_prefill=es_pf, e_conv_prefill=ec_pf,
            e_out_decode=eo_dec, e_state_decode=es_dec, e_conv_decode=ec_dec)
    assert eo_pf <= TOL_OUT and es_pf <= TOL_STATE and ec_pf <= TOL_STATE
    assert eo_dec <= TOL_OUT and es_dec <= TOL_STATE and ec_dec <= TOL_STATE


def _live_prefill_check(wl, b, after_prefill, after_decode):
    """The oracle for session b alone: the prompt as 2048 recurrent steps, then the 750
    decode steps; every prompt token's and every step's output, and the whole state and
    conv cache after the prefill and after the last step."""
    import oracle
    d = wl.dims
    lay = oracle.Layer(d, synth.make_layer_weights(d, wl.weight_seed))
    so, co = lay.new_state(1)
    prompt = synth.make_prompt(d, wl.seed, wl.batch, wl.prefill)[b:b + 1]
    ypo = lay.prefill(so, co, prompt.astype(np.float64))
    y_pf, S_pf, C_pf = after_prefill
    eo_pf = e_out(y_pf, ypo[0])
    es_pf, ec_pf = e_state(S_pf[None], so), e_conv(C_pf[None], co)
    xs = synth.make_inputs(d, wl.seed, wl.steps, wl.batch)[:, b:b + 1]
    yo = np.empty((wl.steps, d.d_model))
    for t in range(wl.steps):
        yo[t] = lay.step(so, co, xs[t].astype(np.float64))[0]
    y_dec, S_dec, C_dec = after_decode
    eo_dec = e_out(y_dec, yo)
    es_dec, ec_dec = e_state(S_dec[None], so), e_conv(C_dec[None], co)
    _report(wl.name + " live session %d" % b, e_out_prefill=eo_pf, e_state_prefill=es_pf, e_conv_prefill=ec_pf,
            e_out_decode=eo_dec, e_state_decode=es_dec, e_conv_decode=ec_dec)
    assert eo_pf <= TOL_OUT and es_pf <= TOL_STATE and ec_pf <= TOL_STATE
    assert eo_dec <= TOL_OUT and es_dec <= TOL_STATE and ec_dec <= TOL_STATE


@pytest.mark.parametrize("batch", [1, 8])
def test_int8_literal_scales_gamma_one(batch):
    """One 9B-shaped int8 g128 layer with the int8 values and fp16 scales U[0.5, 2]/127 of
    the stack workload taken literally: no per-tensor gamma (gamma = 1), so the dequantized
    weights are O(1) and every GEMV output is about 50-80 times larger than with unit-variance
    weights (dt saturates, states and sums of squares grow by orders of magnitude). A dequant
    stress test in fp32 against the fp64 oracle: 1 session (VALU GEMVs) and 8 (MFMA GEMVs)."""
    wl = synth.workload(3)
    d = wl.dims.replace(q_gamma_in=1.0, q_gamma_out=1.0)
    w = synth.make_layer_weights(d, wl.weight_seed, 0)
    xs = synth.make_inputs(d, wl.seed, 6, batch)
    ssm0, conv0 = synth.make_state(d, wl.seed, batch, 0.0)
    yg, sg, cg = gpu_decode(d, w, xs, ssm0, conv0, residual=True)
    yo, so, co = oracle_decode(d, w, xs, ssm0, conv0, residual=True)
    eo, es, ec = e_out(yg, yo), e_state(sg, so), e_conv(cg, co)
    _report("int8-literal-gamma1-b%d" % batch, e_out=eo, e_state=es, e_conv=ec,
            y_max=float(np.max(np.abs(yo))), s_max=float(np.max(np.abs(so))))
    assert eo <= TOL_OUT and es <= TOL_STATE and ec <= TOL_STATE
