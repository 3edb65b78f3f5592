"""Plan 2 of the decode step (M2_PERSISTENT: one session, bf16 weights; the in_proj GEMV,
then the SSD and out_proj in one persistent kernel with a grid barrier) through the C ABI:
against the fp64 oracle and against the three-kernel plan of the same step, with slots and
the residual, an out-of-range slot, the dt = 0 and A -> -inf limits, shapes whose rows,
chunks and head ranges leave parts of the grid idle, run-to-run determinism and HIP-graph
replays."""
import numpy as np
import pytest

from full_duplex_speech_mamba2_amd import synth
from parity import TOL_OUT, TOL_STATE, e_conv, e_out, e_state, oracle_decode

pytestmark = pytest.mark.gpu

MID = synth.MixerDims(d_model=512, n_heads=16, head_dim=32, d_state=64, n_groups=4, wtype="bf16")
RAGGED = synth.MixerDims(d_model=272, n_heads=6, head_dim=24, d_state=32, n_groups=2, d_conv=4, wtype="bf16")


def _run(dims, w, xs, ssm0, conv0, slot=None, residual=False, persistent=True):
    import torch
    from full_duplex_speech_mamba2_amd import m2
    lay = m2.Layer(dims, w)
    st = m2.State(lay, ssm0.shape[0], torch.from_numpy(np.ascontiguousarray(ssm0)).cuda(),
                  torch.from_numpy(np.ascontiguousarray(conv0)).cuda())
    xd = torch.from_numpy(np.ascontiguousarray(xs)).cuda()
    yd = torch.empty_like(xd)
    sl = None if slot is None else torch.tensor([slot], dtype=torch.int32, device="cuda")
    for t in range(xs.shape[0]):
        m2.step(lay, st, xd[t], yd[t], slot_ids=sl, residual=residual, persistent=persistent)
    torch.cuda.synchronize()
    return lay, yd.cpu().numpy(), st.ssm.cpu().numpy(), st.conv.cpu().numpy()


@pytest.mark.parametrize("dims,variant", [(MID, "plain"), (MID, "slot_residual"), (RAGGED, "plain"),
                                          (RAGGED.replace(norm_group=24, d_conv=5), "slot_residual"),
                                          (synth.MixerDims(d_model=128, n_heads=4, head_dim=8, d_state=256,
                                                           n_groups=2, wtype="bf16"), "plain")])
def test_fused_matches_oracle_and_three_kernel_plan(dims, variant):
    w = synth.make_layer_weights(dims, 201)
    xs = synth.make_inputs(dims, 202, 9, 1)
    n_slots = 4 if variant == "slot_residual" else 1
    slot = 2 if variant == "slot_residual" else None
    residual = variant == "slot_residual"
    ssm0, conv0 = synth.make_state(dims, 203, n_slots, 0.1)
    lay, yf, sf, cf = _run(dims, w, xs, ssm0, conv0, slot, residual)
    assert lay.step_plan(1, persistent=True) == 2, "plan 2 should apply to this shape"
    _, yu, su, cu = _run(dims, w, xs, ssm0, conv0, slot, residual, persistent=False)
    used = [slot if slot is not None else 0]
    yo, so, co = oracle_decode(dims, w, xs, ssm0, conv0, slot_ids=None if slot is None else [slot],
                               residual=residual)
    eo, es, ec = e_out(yf, yo), e_state(sf[used], so[used]), e_conv(cf[used], co[used])
    eu = e_out(yf, yu)
    print("[parity] persistent %s d_model=%d e_out=%.3e e_state=%.3e e_conv=%.3e vs-three-kernel=%.3e"
          % (variant, dims.d_model, eo, es, ec, eu), flush=True)
    assert eo <= TOL_OUT and es <= TOL_STATE and ec <= TOL_STATE
    # the other slots are untouched
    others = [i for i in range(n_slots) if i not in used]
    assert np.array_equal(sf[others], ssm0[others]) and np.array_equal(cf[others], conv0[others])
    # in_proj sums in the same order on both plans and the SSD code is shared, so the state
    # and conv cache agree bitwise; only out_proj's order of sums differs
    assert np.array_equal(cf, cu) and np.array_equal(sf, su)


def test_fused_out_of_range_slot_gives_nan_and_touches_nothing():
    dims = MID
    w = synth.make_layer_weights(dims, 211)
    xs = synth.make_inputs(dims, 212, 2, 1)
    ssm0, conv0 = synth.make_state(dims, 213, 2, 0.1)
    lay, y, s, c = _run(dims, w, xs, ssm0, conv0, slot=5)
    assert lay.step_plan(1, persistent=True) == 2
    assert np.all(np.isnan(y))
    assert np.array_equal(s, ssm0) and np.array_equal(c, conv0)


def test_fused_dt_zero_keeps_state_and_A_to_minus_inf_resets_it():
    dims = MID
    w = synth.make_layer_weights(dims, 221)
    w["dt_bias"] = np.full(dims.n_heads, -1e4, np.float32)
    xs = synth.make_inputs(dims, 222, 1, 1)
    ssm0, conv0 = synth.make_state(dims, 223, 1, 0.1)
    lay, y, s, c = _run(dims, w, xs, ssm0, conv0)
    assert lay.step_plan(1, persistent=True) == 2
    assert np.array_equal(s, ssm0)
    w2 = synth.make_layer_weights(dims, 221)
    w2["A_log"] = np.full(dims.n_heads, np.log(1e30), np.float32)
    _, y2, s2, _ = _run(dims, w2, xs, ssm0, conv0)
    yo, so, _ = oracle_decode(dims, w2, xs, ssm0, conv0)
    assert e_state(s2, so) <= 1e-5 and e_out(y2, yo) <= TOL_OUT


def test_fused_run_twice_bitwise_and_graph_replays():
    """Two runs give identical bits; a captured graph of the step (the barrier clear and the
    persistent kernel), replayed three times with eager steps between, matches eager steps."""
    import torch
    from full_duplex_speech_mamba2_amd import m2
    dims = MID
    w = synth.make_layer_weights(dims, 231)
    xs = synth.make_inputs(dims, 232, 6, 1)
    ssm0, conv0 = synth.make_state(dims, 233, 1, 0.1)
    a = _run(dims, w, xs, ssm0, conv0)[1:]
    b = _run(dims, w, xs, ssm0, conv0)[1:]
    for u, v in zip(a, b):
        assert np.array_equal(u, v)
    lay = m2.Layer(dims, w)
    st_e = m2.State(lay, 1, torch.from_numpy(ssm0).cuda(), torch.from_numpy(conv0).cuda())
    st_g = m2.State(lay, 1, torch.from_numpy(ssm0).cuda(), torch.from_numpy(conv0).cuda())
    xd = torch.from_numpy(xs).cuda()
    ws = lay.workspace("step", 1)
    yg = torch.zeros(1, dims.d_model, device="cuda")
    g = torch.cuda.CUDAGraph()
    sgr = torch.cuda.Stream()
    sgr.wait_stream(torch.cuda.current_stream())
    xin = xd[0].clone()
    with torch.cuda.stream(sgr):
        with torch.cuda.graph(g, stream=sgr):
            m2.step(lay, st_g, xin, yg, ws=ws, persistent=True)
    torch.cuda.current_stream().wait_stream(sgr)
    torch.cuda.synchronize()
    # capturing does not run the step: the graph's state is still the initial one
    assert torch.equal(st_g.ssm, st_e.ssm)
    ye = torch.empty_like(yg)
    for t in range(3):
        xin.copy_(xd[t])
        g.replay()
        m2.step(lay, st_e, xd[t], ye, persistent=True)
        torch.cuda.synchronize()
        assert torch.equal(yg, ye), "replay %d" % t
        assert torch.equal(st_g.ssm, st_e.ssm) and torch.equal(st_g.conv, st_e.conv)
