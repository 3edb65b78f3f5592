"""Parity of the chunked HIP prefill (m2_prefill through the C ABI) with the oracle's
T recurrent steps, and of prefill followed by decode steps."""
import numpy as np
import pytest

from full_duplex_speech_mamba2_amd import synth
from parity import TOL_OUT, TOL_STATE, e_conv, e_out, e_state

pytestmark = pytest.mark.gpu


def gpu_prefill(dims, w, x, ssm0, conv0, chunk, slot_ids=None, residual=False):
    import torch
    from full_duplex_speech_mamba2_amd import m2
    lay = m2.Layer(dims, w)
    st = m2.State(lay, ssm0.shape[0], torch.from_numpy(np.ascontiguousarray(ssm0, np.float32)).cuda(),
                  torch.from_numpy(np.ascontiguousarray(conv0, np.float32)).cuda())
    xd = torch.from_numpy(np.ascontiguousarray(x, np.float32)).cuda()
    sl = None if slot_ids is None else torch.from_numpy(np.asarray(slot_ids, np.int32)).cuda()
    y = m2.prefill(lay, st, xd, chunk=chunk, slot_ids=sl, residual=residual)
    torch.cuda.synchronize()
    return y.cpu().numpy(), st.ssm.cpu().numpy(), st.conv.cpu().numpy(), (lay, st)


def oracle_prefill(dims, w, x, ssm0, conv0, slot_ids=None, residual=False):
    import oracle
    lay = oracle.Layer(dims, w)
    s, c = lay.new_state(ssm0.shape[0], ssm0, conv0)
    y = lay.prefill(s, c, x, slot_ids=slot_ids, residual=residual)
    return y, s, c


def _check(tag, dims, w, x, ssm0, conv0, chunk, slot_ids=None, residual=False):
    yg, sg, cg, handles = gpu_prefill(dims, w, x, ssm0, conv0, chunk, slot_ids, residual)
    yo, so, co = oracle_prefill(dims, w, x, ssm0, conv0, slot_ids, residual)
    used = np.arange(x.shape[0]) if slot_ids is None else np.asarray(slot_ids)
    eo = e_out(yg, yo)
    es, ec = e_state(sg[used], so[used]), e_conv(cg[used], co[used])
    print("[parity] prefill %s e_out=%.3e e_state=%.3e e_conv=%.3e" % (tag, eo, es, ec), flush=True)
    assert eo <= TOL_OUT and es <= TOL_STATE and ec <= TOL_STATE
    return handles, so, co


SMALL = synth.MixerDims(d_model=272, n_heads=4, head_dim=32, d_state=32, n_groups=2, wtype="bf16")


@pytest.mark.parametrize("T,chunk", [(1, 16), (2, 16), (3, 32), (16, 16), (37, 16), (100, 32), (130, 64)])
def test_small_bf16_ragged_lengths(T, chunk):
    w = synth.make_layer_weights(SMALL, 101)
    x = synth.make_prompt(SMALL, 102, 2, T)
    ssm0, conv0 = synth.make_state(SMALL, 103, 2, 0.1)
    _check("small-T%d-c%d" % (T, chunk), SMALL, w, x, ssm0, conv0, chunk)


def test_panel_and_row_major_weights_give_identical_prefill():
    """The bf16 projection GEMMs read W from the 16-row panel copies when the layer holds
    them, row-major otherwise: the same products in the same order, so bitwise-equal outputs,
    states and conv caches (K = 272, half a 32-wide k-step past the last whole one; in_proj
    N = 388, out_proj N = 272: ragged column tiles)."""
    import torch
    from full_duplex_speech_mamba2_amd import m2
    w = synth.make_layer_weights(SMALL, 121)
    x = synth.make_prompt(SMALL, 122, 2, 70)
    ssm0, conv0 = synth.make_state(SMALL, 123, 2, 0.1)
    outs = []
    for panels in (True, False):
        lay = m2.Layer(SMALL, w, panels=panels)
        assert (lay.tensors.get("w_in_panels") is not None) == panels
        st = m2.State(lay, 2, torch.from_numpy(ssm0).cuda(), torch.from_numpy(conv0).cuda())
        y = m2.prefill(lay, st, torch.from_numpy(x).cuda(), chunk=32)
        torch.cuda.synchronize()
        outs.append((y.cpu().numpy(), st.ssm.cpu().numpy(), st.conv.cpu().numpy()))
    for a, b in zip(*outs):
        assert np.array_equal(a, b)


def test_small_slots_residual_and_all_weight_types():
    for wtype in ("f32", "bf16", "int8g"):
        dims = SMALL.replace(wtype=wtype, q_group=16, q_gamma_in=0.0625, q_gamma_out=0.1)
        w = synth.make_layer_weights(dims, 111)
        x = synth.make_prompt(dims, 112, 3, 45)
        ssm0, conv0 = synth.make_state(dims, 113, 5, 0.1)
        _check("small-%s-slots" % wtype, dims, w, x, ssm0, conv0, 16, slot_ids=np.array([4, 1, 2], np.int32),
               residual=True)


def test_tiny_fp32_prefill():
    wl = synth.workload(0)
    w = synth.make_layer_weights(wl.dims, wl.weight_seed)
    x = synth.make_prompt(wl.dims, 7, 2, 70)
    ssm0, conv0 = synth.make_state(wl.dims, 8, 2, 0.0)
    _check("tiny", wl.dims, w, x, ssm0, conv0, 32)


def test_prefill_then_decode_equals_steps():
    """A prefill followed by decode steps on the GPU against T + k oracle steps."""
    import torch
    from full_duplex_speech_mamba2_amd import m2
    import oracle
    dims = SMALL
    w = synth.make_layer_weights(dims, 121)
    x = synth.make_prompt(dims, 122, 2, 50)
    xs = synth.make_inputs(dims, 123, 6, 2)
    ssm0, conv0 = synth.make_state(dims, 124, 2, 0.0)
    (lay, st), so, co = _check("then-decode", dims, w, x, ssm0, conv0, 32)
    ol = oracle.Layer(dims, w)
    for t in range(xs.shape[0]):
        yg = m2.step(lay, st, torch.from_numpy(xs[t]).cuda())
        yo = ol.step(so, co, xs[t])
        torch.cuda.synchronize()
        assert e_out(yg.cpu().numpy(), yo) <= TOL_OUT
    assert e_state(st.ssm.cpu().numpy(), so) <= TOL_STATE


def test_9b_shape_short_prompt():
    """The 9B-shaped layer (bf16) with 2 sessions and a 300-token prompt: two chunks of 256, the
    second partial."""
    dims = synth.NINE_B
    w = synth.make_layer_weights(dims, 1)
    x = synth.make_prompt(dims, 131, 2, 300)
    ssm0, conv0 = synth.make_state(dims, 132, 2, 0.1)
    _check("9b-T300", dims, w, x, ssm0, conv0, 256)


def test_many_heads_per_group_uses_per_head_chunk_states():
    """64 heads in one group at chunk 256: the group's B chunk (135 KB) and the 64 heads'
    weights (64 KB) exceed LDS, so the chunk states are formed per head instead of per group."""
    dims = synth.MixerDims(d_model=256, n_heads=64, head_dim=16, d_state=128, n_groups=1, wtype="bf16")
    w = synth.make_layer_weights(dims, 141)
    x = synth.make_prompt(dims, 142, 2, 300)
    ssm0, conv0 = synth.make_state(dims, 143, 2, 0.1)
    _check("hpg64-c256", dims, w, x, ssm0, conv0, 256)


@pytest.mark.parametrize("wtype", ["int4g", "int3g"])
def test_lowbit_prefill(wtype):
    dims = synth.MixerDims(d_model=256, n_heads=4, head_dim=32, d_state=32, n_groups=2, wtype=wtype, q_group=64)
    w = synth.make_layer_weights(dims, 151)
    x = synth.make_prompt(dims, 152, 2, 70)
    ssm0, conv0 = synth.make_state(dims, 153, 2, 0.1)
    _check("lowbit-%s" % wtype, dims, w, x, ssm0, conv0, 32)


def test_prefill_dt_zero_keeps_state_and_A_to_minus_inf_resets_it():
    """The chunked scan's limits through m2_prefill (37 tokens, chunks of 16, the last
    partial), from a random state: dt = 0 (softplus underflows) makes every decay exp(0) = 1
    and every input term 0, so the state is bitwise unchanged and y = C.S + D x; A -> -inf
    makes every decay across tokens 0, so the final state is dt x B^T of the last token
    alone, with no trace of the initial state or of earlier tokens."""
    dims = SMALL
    x = synth.make_prompt(dims, 161, 2, 37)
    ssm0, conv0 = synth.make_state(dims, 162, 2, 0.1)
    w = synth.make_layer_weights(dims, 163)
    w["dt_bias"] = np.full(dims.n_heads, -1e4, np.float32)
    yg, sg, cg, _ = gpu_prefill(dims, w, x, ssm0, conv0, 16)
    assert np.array_equal(sg, ssm0)
    yo, so, co = oracle_prefill(dims, w, x, ssm0, conv0)
    eo, ec = e_out(yg, yo), e_conv(cg, co)
    print("[parity] prefill dt=0 e_out=%.3e e_conv=%.3e" % (eo, ec), flush=True)
    assert eo <= TOL_OUT and ec <= TOL_STATE

    w2 = synth.make_layer_weights(dims, 163)
    w2["A_log"] = np.full(dims.n_heads, np.log(1e30), np.float32)
    yg2, sg2, cg2, _ = gpu_prefill(dims, w2, x, ssm0, conv0, 16)
    yo2, so2, co2 = oracle_prefill(dims, w2, x, ssm0, conv0)
    # the last token alone, from a zero state with the conv cache the first 36 tokens left,
    # gives the same final state: nothing of the initial state or earlier tokens remains
    cache36 = oracle_prefill(dims, w2, x[:, :-1], ssm0, conv0)[2]
    _, so_last, _ = oracle_prefill(dims, w2, x[:, -1:], np.zeros_like(ssm0), cache36)
    eo2, es2 = e_out(yg2, yo2), e_state(sg2, so2)
    print("[parity] prefill A->-inf e_out=%.3e e_state=%.3e" % (eo2, es2), flush=True)
    assert eo2 <= TOL_OUT and es2 <= 1e-5
    assert e_state(so2, so_last) <= 1e-12


@pytest.mark.parametrize("T", [255, 256, 257])
def test_9b_prefill_chunk_edges_from_random_state(T):
    """The 9B-shaped layer at one token short of, exactly at, and one past the 256-token
    chunk, 2 sessions from random states and caches; every state element compared."""
    dims = synth.NINE_B
    w = synth.make_layer_weights(dims, 1)
    x = synth.make_prompt(dims, 170 + T, 2, T)
    ssm0, conv0 = synth.make_state(dims, 171, 2, 0.1)
    _check("9b-T%d" % T, dims, w, x, ssm0, conv0, 256)
