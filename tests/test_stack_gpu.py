"""Parity of the hybrid stack step (m2_stack_step through the C ABI): against the oracle's
residual chain of the same layers (outputs normwise within 2e-3, mixer states within 1e-3,
attention positions exact), bitwise against the same layers stepped one call at a time, and
bitwise between graph replays and eager steps."""
import numpy as np
import pytest

import oracle
from full_duplex_speech_mamba2_amd import synth

pytestmark = pytest.mark.gpu

MIX = synth.MixerDims(d_model=256, n_heads=8, head_dim=32, d_state=16, n_groups=2, wtype="bf16")
ATT = synth.AttnDims(d_model=256, n_q=4, n_kv=2, head_dim=64, max_len=80)
PATTERN = "MAMMA"
N_SLOTS = 3
POS0 = np.array([5, 0, 20], np.int32)


def _host_layers(pattern=PATTERN):
    out = []
    for i, k in enumerate(pattern):
        if k == "M":
            w = synth.make_layer_weights(MIX, 60, layer=i)
            ssm, conv = synth.make_state(MIX, 61, N_SLOTS, 0.1, layer=i)
            out.append(("M", w, (ssm, conv)))
        else:
            w = synth.make_attn_weights(ATT, 62, layer=i)
            kc, vc = synth.make_kv_cache(ATT, 63, POS0, layer=i)
            out.append(("A", w, (kc, vc, POS0.copy())))
    return out


def _gpu_entries(host):
    import torch
    from full_duplex_speech_mamba2_amd import m2
    entries = []
    for k, w, st in host:
        if k == "M":
            lay = m2.Layer(MIX, w)
            entries.append((lay, m2.State(lay, N_SLOTS, torch.from_numpy(st[0]).cuda(), torch.from_numpy(st[1]).cuda())))
        else:
            at = m2.Attn(ATT, w)
            entries.append((at, (torch.from_numpy(st[0].view(np.int16).copy()).cuda(),
                                 torch.from_numpy(st[1].view(np.int16).copy()).cuda(),
                                 torch.from_numpy(st[2].copy()).cuda())))
    return entries


def _rel(a, b):
    return float(np.max(np.max(np.abs(a - b), axis=-1) / np.max(np.abs(b), axis=-1)))


def test_stack_matches_oracle_chain_and_per_layer_calls():
    import torch
    from full_duplex_speech_mamba2_amd import m2
    host = _host_layers()
    xs = synth.make_inputs(MIX, 64, 6, 3)
    slots = np.array([2, 0, 1], np.int32)
    sd = torch.from_numpy(slots).cuda()

    ents = _gpu_entries(host)
    stack = m2.Stack(ents, N_SLOTS)
    ys = [stack.step(torch.from_numpy(xs[t]).cuda(), slot_ids=sd).cpu().numpy() for t in range(xs.shape[0])]

    ents2 = _gpu_entries(host)                              # the same layers, one call each
    ys2 = []
    for t in range(xs.shape[0]):
        u = torch.from_numpy(xs[t]).cuda()
        for lay, st in ents2:
            if isinstance(lay, m2.Layer):
                m2.step(lay, st, u, u, slot_ids=sd, residual=True)
            else:
                lay.step(st[0], st[1], st[2], u, u, slot_ids=sd, residual=True)
        ys2.append(u.cpu().numpy())
    torch.cuda.synchronize()
    assert all(np.array_equal(a, b) for a, b in zip(ys, ys2))
    for (l1, s1), (l2, s2) in zip(ents, ents2):
        if isinstance(l1, m2.Layer):
            assert torch.equal(s1.ssm, s2.ssm) and torch.equal(s1.conv, s2.conv)
        else:
            assert all(torch.equal(a, b) for a, b in zip(s1, s2))

    olay = []
    for k, w, st in host:
        if k == "M":
            ol = oracle.Layer(MIX, w)
            olay.append((ol, ol.new_state(N_SLOTS, st[0], st[1])))
        else:
            olay.append((oracle.AttnLayer(ATT, w), (st[0].copy(), st[1].copy(), st[2].copy())))
    yo = [oracle.stack_step(olay, xs[t], slot_ids=slots) for t in range(xs.shape[0])]
    e = max(_rel(a, b) for a, b in zip(ys, yo))
    print("[stack] e_out=%.3e" % e, flush=True)
    assert e <= 2e-3
    for (l1, s1), (lo, so) in zip(ents, olay):
        if isinstance(l1, m2.Layer):
            S, So = s1.ssm.cpu().numpy().astype(np.float64), so[0]
            assert np.max(np.abs(S - So)) <= 1e-3 * np.max(np.abs(So))
        else:
            assert np.array_equal(s1[2].cpu().numpy(), so[2])
            assert np.array_equal(so[2], POS0 + 6)


def test_stack_graph_replays_match_eager_steps():
    import torch
    from full_duplex_speech_mamba2_amd import m2
    host = _host_layers("MAM")
    xs = torch.from_numpy(synth.make_inputs(MIX, 65, 1, 3)[0]).cuda()
    outs = []
    for graph in (False, True):
        ents = _gpu_entries(host)
        stack = m2.Stack(ents, N_SLOTS)
        y = torch.empty_like(xs)
        ws = stack.workspace(3)
        res = []
        if graph:
            g = torch.cuda.CUDAGraph()
            s = torch.cuda.Stream()
            s.wait_stream(torch.cuda.current_stream())
            with torch.cuda.stream(s):
                with torch.cuda.graph(g, stream=s):
                    stack.step(xs, y, ws=ws)
            torch.cuda.current_stream().wait_stream(s)
        for _ in range(3):
            if graph:
                g.replay()
            else:
                stack.step(xs, y, ws=ws)
            torch.cuda.synchronize()
            res.append(y.clone())
            _ = (xs * 2).sum().item()                       # eager work between replays
        outs.append(res + [ents[1][1][2].clone()])
    assert all(torch.equal(a, b) for a, b in zip(*outs))


def test_stack_of_quantized_layers_matches_oracle_chain():
    """int8 g64 mixers and 4-bit g32 attention layers in one stack (slots, 4 steps)."""
    import torch
    from full_duplex_speech_mamba2_amd import m2
    mix = MIX.replace(wtype="int8g", q_group=64, q_gamma_in=0.0625, q_gamma_out=0.0625)
    att = ATT.replace(wtype="int4g", q_group=32)
    host, ents, olay = [], [], []
    for i, k in enumerate("MAM"):
        if k == "M":
            w = synth.make_layer_weights(mix, 70, layer=i)
            ssm, conv = synth.make_state(mix, 71, N_SLOTS, 0.1, layer=i)
            lay = m2.Layer(mix, w)
            ents.append((lay, m2.State(lay, N_SLOTS, torch.from_numpy(ssm).cuda(), torch.from_numpy(conv).cuda())))
            ol = oracle.Layer(mix, w)
            olay.append((ol, ol.new_state(N_SLOTS, ssm, conv)))
        else:
            w = synth.make_attn_weights(att, 72, layer=i)
            kc, vc = synth.make_kv_cache(att, 73, POS0, layer=i)
            ents.append((m2.Attn(att, w), (torch.from_numpy(kc.view(np.int16).copy()).cuda(),
                                           torch.from_numpy(vc.view(np.int16).copy()).cuda(),
                                           torch.from_numpy(POS0.copy()).cuda())))
            olay.append((oracle.AttnLayer(att, w), (kc.copy(), vc.copy(), POS0.copy())))
    stack = m2.Stack(ents, N_SLOTS)
    xs = synth.make_inputs(mix, 74, 4, 2)
    slots = np.array([1, 2], np.int32)
    sd = torch.from_numpy(slots).cuda()
    ys = [stack.step(torch.from_numpy(xs[t]).cuda(), slot_ids=sd).cpu().numpy() for t in range(xs.shape[0])]
    yo = [oracle.stack_step(olay, xs[t], slot_ids=slots) for t in range(xs.shape[0])]
    e = max(_rel(a, b) for a, b in zip(ys, yo))
    print("[stack] quantized e_out=%.3e" % e, flush=True)
    assert e <= 2e-3
