"""Parity of the HIP decode step (m2_step through the C ABI) with the fp64 oracle."""
import numpy as np
import pytest

from full_duplex_speech_mamba2_amd import synth
from parity import (TOL_OUT, TOL_STATE, e_conv, e_out, e_state, gpu_decode, oracle_decode)

pytestmark = pytest.mark.gpu


def _report(tag, eo, es, ec):
    print("[parity] %s e_out=%.3e e_state=%.3e e_conv=%.3e" % (tag, eo, es, ec), flush=True)


def _check(tag, dims, w, xs, ssm0, conv0, slot_ids=None, residual=False, sessions=None, panels=True):
    yg, sg, cg = gpu_decode(dims, w, xs, ssm0, conv0, slot_ids=slot_ids, residual=residual, panels=panels)
    yo, so, co = oracle_decode(dims, w, xs, ssm0, conv0, slot_ids=slot_ids, residual=residual,
                               sessions=sessions)
    if sessions is not None:
        used = np.asarray(sessions) if slot_ids is None else np.asarray(slot_ids)[sessions]
        yg = yg[:, sessions]
    else:
        used = np.arange(xs.shape[1]) if slot_ids is None else np.asarray(slot_ids)
    eo, es, ec = e_out(yg, yo), e_state(sg[used], so[used]), e_conv(cg[used], co[used])
    _report(tag, eo, es, ec)
    assert eo <= TOL_OUT and es <= TOL_STATE and ec <= TOL_STATE
    return yg, sg, cg


def test_tiny_fp32_16_steps():
    wl = synth.workload(0)
    w = synth.make_layer_weights(wl.dims, wl.weight_seed)
    xs = synth.make_inputs(wl.dims, wl.seed, wl.steps, wl.batch)
    ssm0, conv0 = synth.make_state(wl.dims, wl.seed, wl.batch, wl.state_var)
    _check("tiny", wl.dims, w, xs, ssm0, conv0)


RAGGED = synth.MixerDims(d_model=272, n_heads=6, head_dim=24, d_state=32, n_groups=2, d_conv=4)


@pytest.mark.parametrize("batch", [1, 2, 3])
@pytest.mark.parametrize("wtype", ["f32", "bf16", "int8g"])
@pytest.mark.parametrize("variant", ["plain", "slots_residual", "norm_all", "conv2", "conv5_n64"])
def test_ragged_shapes(wtype, variant, batch):
    """Batches of 1 and 2 take the one-wave-per-row VALU GEMVs; 3 takes the MFMA GEMVs
    (bf16 and int8 g16 here: int8 at q_group 16 stays on the tiled VALU GEMV)."""
    dims = RAGGED.replace(wtype=wtype, q_group=16, q_gamma_in=0.0625, q_gamma_out=0.1)
    B, slots, n_slots, residual, steps = batch, None, batch, False, 9
    if variant == "slots_residual":
        n_slots, slots, residual = 5, np.array([4, 0, 2][:batch], np.int32), True
    elif variant == "norm_all":
        dims = dims.replace(norm_group=dims.d_inner)
    elif variant == "conv2":
        dims = dims.replace(d_conv=2, norm_group=48)
    elif variant == "conv5_n64":
        dims = dims.replace(d_conv=5, d_state=64, n_groups=3, norm_group=24)
    w = synth.make_layer_weights(dims, 31)
    xs = synth.make_inputs(dims, 32, steps, B)
    ssm0, conv0 = synth.make_state(dims, 33, n_slots, 0.1)
    _check("ragged-%s-%s-b%d" % (wtype, variant, batch), dims, w, xs, ssm0, conv0, slot_ids=slots,
           residual=residual)


@pytest.mark.parametrize("batch", [1, 2, 4, 8, 17])
@pytest.mark.parametrize("norm_group", [0, 20])
def test_doubled_ssd_range(batch, norm_group):
    """The 9B SSD item shape at 1-17 sessions: head_dim 80 gives 20-row ranges, which the
    step doubles to 40-row items with one sum of squares each (10 waves x 2 state slices of a
    128-wide state row at 1-2 sessions, 4 x 5 at 4 and 2 x 10 at 8 and 17, where the GEMVs
    are the MFMA plan's); with RMS groups of 20 channels a doubled range would straddle two groups, so
    the layer's 20-row items stay. Slots and the residual on; outputs, states and conv caches
    against the oracle."""
    dims = synth.MixerDims(d_model=256, n_heads=4, head_dim=80, d_state=128, n_groups=2, wtype="bf16",
                           norm_group=norm_group)
    w = synth.make_layer_weights(dims, 91)
    xs = synth.make_inputs(dims, 92, 7, batch)
    ssm0, conv0 = synth.make_state(dims, 93, 20, 0.1)
    slots = np.array([3, 1, 9, 0, 5, 7, 2, 8, 19, 11, 4, 16, 6, 13, 10, 18, 12][:batch], np.int32)
    _check("doubled-range-b%d-ng%s" % (batch, norm_group), dims, w, xs, ssm0, conv0, slot_ids=slots, residual=True)


@pytest.mark.parametrize("batch", [1, 2, 5, 8, 17, 40])
def test_batch_sizes_bf16(batch):
    """1-2 sessions: one-wave-per-row GEMVs; 3-32: MFMA GEMVs; 40: the tiled VALU GEMVs."""
    dims = synth.MixerDims(d_model=512, n_heads=16, head_dim=32, d_state=64, n_groups=4, wtype="bf16")
    w = synth.make_layer_weights(dims, 41)
    xs = synth.make_inputs(dims, 42, 5, batch)
    ssm0, conv0 = synth.make_state(dims, 43, batch, 0.1)
    _check("batch%d" % batch, dims, w, xs, ssm0, conv0)


def test_dt_zero_keeps_state_and_A_to_minus_inf_resets_it():
    import torch
    from full_duplex_speech_mamba2_amd import m2
    dims = synth.MixerDims(d_model=256, n_heads=8, head_dim=32, d_state=16, n_groups=2, wtype="bf16")
    w = synth.make_layer_weights(dims, 51)
    w["dt_bias"] = np.full(dims.n_heads, -1e4, np.float32)       # softplus underflows to 0
    ssm0, conv0 = synth.make_state(dims, 52, 1, 0.1)
    lay = m2.Layer(dims, w)
    st = m2.State(lay, 1, torch.from_numpy(ssm0).cuda(), torch.from_numpy(conv0).cuda())
    x = torch.from_numpy(synth.make_inputs(dims, 53, 1, 1)[0]).cuda()
    m2.step(lay, st, x)
    torch.cuda.synchronize()
    assert np.array_equal(st.ssm.cpu().numpy(), ssm0)             # bitwise unchanged

    w2 = synth.make_layer_weights(dims, 51)
    w2["A_log"] = np.full(dims.n_heads, np.log(1e30), np.float32)  # exp(dt A) = 0
    lay2 = m2.Layer(dims, w2)
    st2 = m2.State(lay2, 1, torch.from_numpy(ssm0).cuda(), torch.from_numpy(conv0).cuda())
    m2.step(lay2, st2, x)
    torch.cuda.synchronize()
    lo = __import__("oracle").Layer(dims, w2)
    so, co = lo.new_state(1, ssm0, conv0)
    _, tr = lo.step(so, co, x.cpu().numpy().astype(np.float64), trace=True)
    # the reset state is dt x B^T: no trace of the random initial state remains
    assert e_state(st2.ssm.cpu().numpy(), so) <= 1e-5


def test_run_twice_bitwise_equal():
    dims = synth.MixerDims(d_model=512, n_heads=16, head_dim=32, d_state=64, n_groups=4, wtype="bf16")
    w = synth.make_layer_weights(dims, 61)
    xs = synth.make_inputs(dims, 62, 4, 6)
    ssm0, conv0 = synth.make_state(dims, 63, 6, 0.1)
    a = gpu_decode(dims, w, xs, ssm0, conv0)
    b = gpu_decode(dims, w, xs, ssm0, conv0)
    for u, v in zip(a, b):
        assert np.array_equal(u, v)


def test_out_of_range_slot_gives_nan_and_touches_nothing():
    import torch
    from full_duplex_speech_mamba2_amd import m2
    dims = synth.MixerDims(d_model=256, n_heads=8, head_dim=32, d_state=16, n_groups=2, wtype="bf16")
    w = synth.make_layer_weights(dims, 71)
    ssm0, conv0 = synth.make_state(dims, 72, 2, 0.1)
    lay = m2.Layer(dims, w)
    st = m2.State(lay, 2, torch.from_numpy(ssm0).cuda(), torch.from_numpy(conv0).cuda())
    x = torch.from_numpy(synth.make_inputs(dims, 73, 1, 2)[0]).cuda()
    y = m2.step(lay, st, x, slot_ids=torch.tensor([1, 7], dtype=torch.int32, device="cuda"))
    torch.cuda.synchronize()
    yh = y.cpu().numpy()
    assert np.all(np.isfinite(yh[0])) and np.all(np.isnan(yh[1]))
    assert np.array_equal(st.ssm.cpu().numpy()[0], ssm0[0])
    assert np.array_equal(st.conv.cpu().numpy()[0], conv0[0])


@pytest.mark.parametrize("wtype", ["bf16", "int8g"])
def test_mfma_bad_slot_leaves_neighbours_finite(wtype):
    """bf16, 3 sessions: the MFMA plan with K = d_inner = 144, not a multiple of the 256-wide tile:
    the out_proj activations past K are zero and their RMS factor must come from the same
    session. A session on an out-of-range slot has NaN factors; its neighbours' outputs
    stay finite and match the oracle, and its own are all NaN."""
    import torch
    from full_duplex_speech_mamba2_amd import m2
    dims = RAGGED.replace(wtype=wtype, q_group=16)     # int8 g16: the tiled VALU GEMVs
    w = synth.make_layer_weights(dims, 151)
    xs = synth.make_inputs(dims, 152, 3, 3)
    ssm0, conv0 = synth.make_state(dims, 153, 3, 0.1)
    lay = m2.Layer(dims, w)
    st = m2.State(lay, 3, torch.from_numpy(ssm0).cuda(), torch.from_numpy(conv0).cuda())
    slots = np.array([0, 9, 1], np.int32)
    sd = torch.from_numpy(slots).cuda()
    xd = torch.from_numpy(xs).cuda()
    yd = torch.empty_like(xd)
    for t in range(xs.shape[0]):
        m2.step(lay, st, xd[t], yd[t], slot_ids=sd)
    torch.cuda.synchronize()
    yg = yd.cpu().numpy()
    assert np.all(np.isnan(yg[:, 1]))
    good = [0, 2]
    assert np.all(np.isfinite(yg[:, good]))
    yo, so, co = oracle_decode(dims, w, xs, ssm0, conv0, slot_ids=slots, sessions=good)
    eo = e_out(yg[:, good], yo)
    es = e_state(st.ssm.cpu().numpy()[[0, 1]], so[[0, 1]])
    print("[parity] mfma-bad-slot-%s plan=%d e_out=%.3e e_state=%.3e" % (wtype, lay.step_plan(3), eo, es), flush=True)
    assert eo <= TOL_OUT and es <= TOL_STATE


def test_state_zero_selected_slots():
    import torch
    from full_duplex_speech_mamba2_amd import m2
    dims = synth.MixerDims(d_model=256, n_heads=8, head_dim=32, d_state=16, n_groups=2, wtype="bf16")
    w = synth.make_layer_weights(dims, 81)
    ssm0, conv0 = synth.make_state(dims, 82, 4, 0.1)
    lay = m2.Layer(dims, w)
    st = m2.State(lay, 4, torch.from_numpy(ssm0).cuda(), torch.from_numpy(conv0).cuda())
    st.zero(torch.tensor([2, 0], dtype=torch.int32, device="cuda"))
    torch.cuda.synchronize()
    s, c = st.ssm.cpu().numpy(), st.conv.cpu().numpy()
    assert np.all(s[[0, 2]] == 0) and np.all(c[[0, 2]] == 0)
    assert np.array_equal(s[[1, 3]], ssm0[[1, 3]]) and np.array_equal(c[[1, 3]], conv0[[1, 3]])
    st.zero()
    torch.cuda.synchronize()
    assert not st.ssm.any() and not st.conv.any()


MID = synth.MixerDims(d_model=512, n_heads=16, head_dim=32, d_state=64, n_groups=4, wtype="bf16")


@pytest.mark.parametrize("panels", [True, False])
@pytest.mark.parametrize("wtype", ["bf16", "int8g"])
@pytest.mark.parametrize("batch", [3, 8, 32])
def test_mfma_batched_gemv(wtype, batch, panels):
    """The stream-K MFMA GEMVs from the 16-row panel copies and from the row-major weights."""
    dims = MID.replace(wtype=wtype, q_group=128, q_gamma_in=float(np.float32(1 / np.sqrt(512))),
                       q_gamma_out=float(np.float32(1 / np.sqrt(512))))
    w = synth.make_layer_weights(dims, 91)
    xs = synth.make_inputs(dims, 92, 6, batch)
    n_slots = batch + 3
    ssm0, conv0 = synth.make_state(dims, 93, n_slots, 0.1)
    slots = np.random.default_rng(94).permutation(n_slots)[:batch].astype(np.int32)
    _check("mfma-%s-b%d-%s" % (wtype, batch, "panels" if panels else "rows"), dims, w, xs, ssm0, conv0,
           slot_ids=slots, residual=True, panels=panels)


@pytest.mark.parametrize("panels", [True, False])
@pytest.mark.parametrize("wtype", ["bf16", "int8g"])
def test_mfma_ragged_rows_and_k(wtype, panels):
    """Rows and K not multiples of the 128-row block, the 16-row panel or the 256-wide k
    tile: bf16 in_proj 326 x 336 (K not a multiple of the 32-wide k-step either) and
    out_proj 336 x 96; int8 (groups of 128) in_proj 908 x 384 and out_proj 384 x 384, whose
    last k tile holds one whole scale group."""
    if wtype == "bf16":
        dims = synth.MixerDims(d_model=336, n_heads=6, head_dim=16, d_state=32, n_groups=2, wtype=wtype)
    else:
        dims = synth.MixerDims(d_model=384, n_heads=12, head_dim=32, d_state=32, n_groups=2, wtype=wtype,
                               q_group=128, q_gamma_in=0.0625, q_gamma_out=0.1)
    w = synth.make_layer_weights(dims, 95)
    xs = synth.make_inputs(dims, 96, 4, 5)
    ssm0, conv0 = synth.make_state(dims, 97, 5, 0.1)
    _check("mfma-ragged-%s-%s" % (wtype, "panels" if panels else "rows"), dims, w, xs, ssm0, conv0,
           panels=panels)


@pytest.mark.parametrize("d_state", [4, 256])
@pytest.mark.parametrize("batch", [1, 3])
def test_state_size_extremes(d_state, batch):
    """The smallest and largest d_state: one lane per state row (64 rows per wave
    instruction) and 64 lanes per row (more conv channels than some item shapes have
    threads)."""
    dims = synth.MixerDims(d_model=128, n_heads=4, head_dim=8, d_state=d_state, n_groups=2, wtype="bf16")
    w = synth.make_layer_weights(dims, 141)
    xs = synth.make_inputs(dims, 142, 6, batch)
    ssm0, conv0 = synth.make_state(dims, 143, batch, 0.1)
    _check("dstate%d-b%d" % (d_state, batch), dims, w, xs, ssm0, conv0)


LOWBIT = synth.MixerDims(d_model=512, n_heads=8, head_dim=32, d_state=32, n_groups=2, d_conv=4)


@pytest.mark.parametrize("batch", [1, 2, 5])
@pytest.mark.parametrize("wtype,q_group", [("int4g", 64), ("int3g", 64), ("int4g", 32), ("int3g", 256)])
def test_lowbit_weights(wtype, q_group, batch):
    """4- and 3-bit codes with (scale, bias) groups: 1-2 sessions take the wave GEMVs,
    5 the tiled GEMVs; one case with slots, residual and per-tensor gammas."""
    dims = LOWBIT.replace(wtype=wtype, q_group=q_group)
    slots, n_slots, residual = None, batch, False
    if q_group == 32:
        dims = dims.replace(q_gamma_in=0.5, q_gamma_out=2.0)
        n_slots, slots, residual = 6, np.array([5, 0, 3, 1, 2][:batch], np.int32), True
    w = synth.make_layer_weights(dims, 51)
    xs = synth.make_inputs(dims, 52, 7, batch)
    ssm0, conv0 = synth.make_state(dims, 53, n_slots, 0.1)
    _check("lowbit-%s-g%d-b%d" % (wtype, q_group, batch), dims, w, xs, ssm0, conv0, slot_ids=slots,
           residual=residual)


@pytest.mark.parametrize("batch", [1, 2])
@pytest.mark.parametrize("wtype,q_group,d_model", [("int4g", 32, 544), ("int3g", 32, 544), ("int4g", 64, 576)])
def test_lowbit_ragged_k(wtype, q_group, d_model, batch):
    """in_proj K of 17 or 18 chunks of 32 codes (a partial 128-code block), rows not a
    multiple of 16; out_proj K = 384."""
    dims = synth.MixerDims(d_model=d_model, n_heads=6, head_dim=64, d_state=32, n_groups=2, d_conv=4,
                           wtype=wtype, q_group=q_group)
    w = synth.make_layer_weights(dims, 61)
    xs = synth.make_inputs(dims, 62, 6, batch)
    ssm0, conv0 = synth.make_state(dims, 63, batch, 0.1)
    _check("lowbit-ragged-%s-g%d-k%d-b%d" % (wtype, q_group, d_model, batch), dims, w, xs, ssm0, conv0)


@pytest.mark.parametrize("batch,panels", [(5, True), (17, False)])
def test_mfma_whole_row_block_in_proj(batch, panels):
    """bf16 in_proj of at least 160 row blocks: one workgroup per 128-row block applies the
    row epilogue itself (no partial sums). 20714 rows (161 whole blocks and one of 106 rows,
    which holds the dt rows) x 336 (K not a multiple of the 32-wide k-step); one and two
    16-session MFMA tiles; slots permuted, residual on."""
    dims = synth.MixerDims(d_model=336, n_heads=106, head_dim=96, d_state=64, n_groups=2, wtype="bf16")
    assert dims.d_in_proj == 20714
    w = synth.make_layer_weights(dims, 181)
    xs = synth.make_inputs(dims, 182, 4, batch)
    n_slots = batch + 2
    ssm0, conv0 = synth.make_state(dims, 183, n_slots, 0.1)
    slots = np.random.default_rng(184).permutation(n_slots)[:batch].astype(np.int32)
    _check("mfma-whole-b%d-%s" % (batch, "panels" if panels else "rows"), dims, w, xs, ssm0, conv0,
           slot_ids=slots, residual=True, panels=panels)


@pytest.mark.parametrize("wtype,batch", [("bf16", 8), ("int8g", 5), ("bf16", 32)])
def test_mfma_plan_graph_replays_match_eager_steps(wtype, batch):
    """A captured step of the MFMA plan (GEMV + reduction kernels around the SSD kernel),
    replayed three times with eager work between replays, gives the same bits as eager
    steps from the same state."""
    import torch
    from full_duplex_speech_mamba2_amd import m2
    dims = MID.replace(wtype=wtype, q_group=128, q_gamma_in=0.0625, q_gamma_out=0.0625)
    w = synth.make_layer_weights(dims, 171)
    xs = torch.from_numpy(synth.make_inputs(dims, 172, 3, batch)).cuda()
    ssm0, conv0 = synth.make_state(dims, 173, batch, 0.1)
    lay = m2.Layer(dims, w)
    assert lay.step_plan(batch) == 1
    runs = []
    for graph in (False, True):
        st = m2.State(lay, batch, torch.from_numpy(ssm0).cuda(), torch.from_numpy(conv0).cuda())
        ws = torch.empty(lay.step_workspace_bytes(batch), dtype=torch.uint8, device="cuda")
        xin, y = xs[0].clone(), torch.empty_like(xs[0])
        if graph:
            g = torch.cuda.CUDAGraph()
            s = torch.cuda.Stream()
            s.wait_stream(torch.cuda.current_stream())
            with torch.cuda.stream(s):
                with torch.cuda.graph(g, stream=s):
                    m2.step(lay, st, xin, y, ws=ws)
            torch.cuda.current_stream().wait_stream(s)
        res = []
        for t in range(3):
            xin.copy_(xs[t])
            if graph:
                g.replay()
            else:
                m2.step(lay, st, xin, y, ws=ws)
            torch.cuda.synchronize()
            res.append(y.clone())
            _ = (xs * 2).sum().item()
        runs.append(res + [st.ssm.clone(), st.conv.clone()])
    assert all(torch.equal(a, b) for a, b in zip(*runs))
