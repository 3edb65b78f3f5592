"""The persistent stack step (m2_stack_step_flags with M2_PERSISTENT: each run of
consecutive mixer layers in one launch, grid barriers between the in_proj, SSD and out_proj
phases of every layer) through the C ABI: bitwise against the same layers stepped one
m2_step call at a time with plan 2 (the arithmetic the persistent kernel shares), within
tolerance of the oracle's residual chain, in hybrid tables with attention layers between
the runs, on shapes that leave parts of the grid idle, with an out-of-range slot, over HIP
graph replays, and falling back to the per-layer kernels where the path does not apply."""
import numpy as np
import pytest

import oracle
from full_duplex_speech_mamba2_amd import synth

pytestmark = pytest.mark.gpu

MIX = synth.MixerDims(d_model=256, n_heads=8, head_dim=32, d_state=16, n_groups=2, wtype="bf16")
RAGGED = synth.MixerDims(d_model=272, n_heads=6, head_dim=24, d_state=32, n_groups=2, d_conv=4, wtype="bf16")
ATT = synth.AttnDims(d_model=256, n_q=4, n_kv=2, head_dim=64, max_len=80)
N_SLOTS = 3
POS0 = np.array([5, 0, 20], np.int32)


def _host_layers(pattern, mix, seed):
    out = []
    for i, k in enumerate(pattern):
        if k == "M":
            w = synth.make_layer_weights(mix, seed, layer=i)
            ssm, conv = synth.make_state(mix, seed + 1, N_SLOTS, 0.1, layer=i)
            out.append(("M", w, (ssm, conv)))
        else:
            att = ATT.replace(d_model=mix.d_model)
            w = synth.make_attn_weights(att, seed + 2, layer=i)
            kc, vc = synth.make_kv_cache(att, seed + 3, POS0, layer=i)
            out.append(("A", w, (kc, vc, POS0.copy()), att))
    return out


def _gpu_entries(host, mix):
    import torch
    from full_duplex_speech_mamba2_amd import m2
    entries = []
    for h in host:
        if h[0] == "M":
            _, w, st = h
            lay = m2.Layer(mix, w)
            entries.append((lay, m2.State(lay, N_SLOTS, torch.from_numpy(st[0]).cuda(),
                                          torch.from_numpy(st[1]).cuda())))
        else:
            _, w, st, att = h
            entries.append((m2.Attn(att, w), (torch.from_numpy(st[0].view(np.int16).copy()).cuda(),
                                              torch.from_numpy(st[1].view(np.int16).copy()).cuda(),
                                              torch.from_numpy(st[2].copy()).cuda())))
    return entries


def _per_layer(ents, xs, sd):
    """The same chain, one m2_step (plan 2) or m2_attn_step call per layer."""
    import torch
    from full_duplex_speech_mamba2_amd import m2
    ys = []
    for t in range(xs.shape[0]):
        u = torch.from_numpy(xs[t]).cuda()
        for lay, st in ents:
            if isinstance(lay, m2.Layer):
                m2.step(lay, st, u, u, slot_ids=sd, residual=True, persistent=True)
            else:
                lay.step(st[0], st[1], st[2], u, u, slot_ids=sd, residual=True)
        ys.append(u.cpu().numpy())
    torch.cuda.synchronize()
    return ys


def _rel(a, b):
    return float(np.max(np.max(np.abs(a - b), axis=-1) / np.max(np.abs(b), axis=-1)))


def _same_states(ents_a, ents_b):
    import torch
    from full_duplex_speech_mamba2_amd import m2
    for (l1, s1), (_, s2) in zip(ents_a, ents_b):
        if isinstance(l1, m2.Layer):
            if not (torch.equal(s1.ssm, s2.ssm) and torch.equal(s1.conv, s2.conv)):
                return False
        elif not all(torch.equal(a, b) for a, b in zip(s1, s2)):
            return False
    return True


@pytest.mark.parametrize("pattern,mix,slot,runs", [("MMAMMM", MIX, 2, 2), ("MMM", RAGGED, None, 1),
                                                   ("AMA", MIX, 1, 1),
                                                   ("MM", RAGGED.replace(norm_group=24, d_conv=5), 0, 1)])
def test_persistent_stack_matches_per_layer_plan2_and_oracle(pattern, mix, slot, runs):
    import torch
    from full_duplex_speech_mamba2_amd import m2
    assert m2.Layer(mix, synth.make_layer_weights(mix, 1)).step_plan(1, persistent=True) == 2
    host = _host_layers(pattern, mix, 80)
    steps = 5
    xs = synth.make_inputs(mix, 84, steps, 1)
    slots = None if slot is None else np.array([slot], np.int32)
    sd = None if slots is None else torch.from_numpy(slots).cuda()

    ents = _gpu_entries(host, mix)
    stack = m2.Stack(ents, N_SLOTS)
    assert stack.persistent_runs(1) == runs
    ys = [stack.step(torch.from_numpy(xs[t]).cuda(), slot_ids=sd, persistent=True).cpu().numpy()
          for t in range(steps)]
    torch.cuda.synchronize()

    ents2 = _gpu_entries(host, mix)
    ys2 = _per_layer(ents2, xs, sd)
    assert all(np.array_equal(a, b) for a, b in zip(ys, ys2)), "persistent stack differs from per-layer plan 2"
    assert _same_states(ents, ents2)

    olay = []
    for h in host:
        if h[0] == "M":
            ol = oracle.Layer(mix, h[1])
            olay.append((ol, ol.new_state(N_SLOTS, h[2][0], h[2][1])))
        else:
            olay.append((oracle.AttnLayer(h[3], h[1]), (h[2][0].copy(), h[2][1].copy(), h[2][2].copy())))
    yo = [oracle.stack_step(olay, xs[t], slot_ids=slots) for t in range(steps)]
    e = max(_rel(a, b) for a, b in zip(ys, yo))
    es = 0.0
    for (l1, s1), (_, so) in zip(ents, olay):
        if isinstance(l1, m2.Layer):
            S, So = s1.ssm.cpu().numpy().astype(np.float64), so[0]
            es = max(es, float(np.max(np.abs(S - So)) / np.max(np.abs(So))))
    print("[stack-persistent] %s d_model=%d runs=%d e_out=%.3e e_state=%.3e" % (pattern, mix.d_model, runs, e, es),
          flush=True)
    assert e <= 2e-3 and es <= 1e-3


def test_persistent_stack_bad_slot_and_fallback():
    """An out-of-range slot gives NaN outputs and leaves every state as it was, as the
    per-layer calls do; at two sessions the path does not apply and the step is
    m2_stack_step's, bit for bit."""
    import torch
    from full_duplex_speech_mamba2_amd import m2
    host = _host_layers("MAM", MIX, 90)
    xs = synth.make_inputs(MIX, 94, 2, 2)
    ents = _gpu_entries(host, MIX)
    stack = m2.Stack(ents, N_SLOTS)
    before = [(s.ssm.clone(), s.conv.clone()) for l, s in ents if isinstance(l, m2.Layer)]
    y = stack.step(torch.from_numpy(xs[0][:1]).cuda(), slot_ids=torch.tensor([7], dtype=torch.int32).cuda(),
                   persistent=True)
    torch.cuda.synchronize()
    assert torch.isnan(y).all()
    after = [(s.ssm, s.conv) for l, s in ents if isinstance(l, m2.Layer)]
    assert all(torch.equal(a[0], b[0]) and torch.equal(a[1], b[1]) for a, b in zip(before, after))

    assert stack.persistent_runs(2) == 0
    ents_p, ents_q = _gpu_entries(host, MIX), _gpu_entries(host, MIX)
    sp, sq = m2.Stack(ents_p, N_SLOTS), m2.Stack(ents_q, N_SLOTS)
    sd = torch.tensor([2, 0], dtype=torch.int32).cuda()
    for t in range(2):
        a = sp.step(torch.from_numpy(xs[t]).cuda(), slot_ids=sd, persistent=True)
        b = sq.step(torch.from_numpy(xs[t]).cuda(), slot_ids=sd)
        torch.cuda.synchronize()
        assert torch.equal(a, b)
    assert _same_states(ents_p, ents_q)


def test_persistent_stack_graph_replays_match_eager_steps():
    import torch
    from full_duplex_speech_mamba2_amd import m2
    host = _host_layers("MMAM", MIX, 100)
    x = torch.from_numpy(synth.make_inputs(MIX, 104, 1, 1)[0]).cuda()
    outs = []
    for graph in (False, True):
        ents = _gpu_entries(host, MIX)
        stack = m2.Stack(ents, N_SLOTS)
        y = torch.empty_like(x)
        ws = stack.workspace(1, persistent=True)
        res = []
        if graph:
            g = torch.cuda.CUDAGraph()
            s = torch.cuda.Stream()
            s.wait_stream(torch.cuda.current_stream())
            with torch.cuda.stream(s):
                with torch.cuda.graph(g, stream=s):
                    stack.step(x, y, ws=ws, persistent=True)
            torch.cuda.current_stream().wait_stream(s)
        for _ in range(3):
            if graph:
                g.replay()
            else:
                stack.step(x, y, ws=ws, persistent=True)
            torch.cuda.synchronize()
            res.append(y.clone())
            _ = (x * 2).sum().item()                        # eager work between replays
        outs.append(res + [ents[0][1].ssm.clone(), ents[3][1].conv.clone()])
    assert all(torch.equal(a, b) for a, b in zip(*outs))
