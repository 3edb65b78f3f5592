"""m2_step_noalloc (the library's static per-GPU scratch as the workspace) against m2_step
with a caller workspace, through the C ABI: two calls in a row, the second with fewer
sessions (and another kernel plan), on identical copies of the state. The kernels are the
same, so outputs, states and conv caches must agree bitwise."""
import numpy as np
import pytest

from full_duplex_speech_mamba2_amd import synth

pytestmark = pytest.mark.gpu

MID = synth.MixerDims(d_model=512, n_heads=16, head_dim=32, d_state=64, n_groups=4, wtype="bf16")


def test_step_noalloc_matches_step_twice_second_smaller():
    import torch
    from full_duplex_speech_mamba2_amd import m2
    dims = MID
    w = synth.make_layer_weights(dims, 171)
    n_slots = 10
    ssm0, conv0 = synth.make_state(dims, 172, n_slots, 0.1)
    lay = m2.Layer(dims, w)
    sa = m2.State(lay, n_slots, torch.from_numpy(ssm0).cuda(), torch.from_numpy(conv0).cuda())
    sb = m2.State(lay, n_slots, torch.from_numpy(ssm0).cuda(), torch.from_numpy(conv0).cuda())
    assert lay.step_plan(8) == 1 and lay.step_plan(2) == 0
    for call, (batch, slots) in enumerate([(8, [9, 0, 3, 5, 1, 8, 2, 6]), (2, [4, 9])]):
        x = torch.from_numpy(synth.make_inputs(dims, 173 + call, 1, batch)[0]).cuda()
        sl = torch.tensor(slots, dtype=torch.int32, device="cuda")
        assert lay.step_workspace_bytes(batch) <= m2.noalloc_scratch_bytes()
        ya = m2.step(lay, sa, x, slot_ids=sl, residual=True)
        yb = m2.step_noalloc(lay, sb, x, slot_ids=sl, residual=True)
        torch.cuda.synchronize()
        print("[no-alloc] call %d batch %d plan %d max|dy| %.3e" % (
            call, batch, lay.step_plan(batch), float((ya - yb).abs().max())), flush=True)
        assert torch.isfinite(yb).all()
        assert torch.equal(ya, yb)
        assert torch.equal(sa.ssm, sb.ssm) and torch.equal(sa.conv, sb.conv)


def test_step_noalloc_whole_row_block_in_proj_twice_second_smaller():
    """The same on a layer whose bf16 in_proj has 162 row blocks (20714 rows), so that the
    in_proj GEMV runs one workgroup per row block with its epilogue in the kernel (no partial
    sums in the workspace): 17 sessions (two 16-session MFMA tiles), then 5."""
    import torch
    from full_duplex_speech_mamba2_amd import m2
    dims = synth.MixerDims(d_model=336, n_heads=106, head_dim=96, d_state=64, n_groups=2, wtype="bf16")
    w = synth.make_layer_weights(dims, 181)
    n_slots = 20
    ssm0, conv0 = synth.make_state(dims, 182, n_slots, 0.1)
    lay = m2.Layer(dims, w)
    sa = m2.State(lay, n_slots, torch.from_numpy(ssm0).cuda(), torch.from_numpy(conv0).cuda())
    sb = m2.State(lay, n_slots, torch.from_numpy(ssm0).cuda(), torch.from_numpy(conv0).cuda())
    assert lay.step_plan(17) == 1 and lay.step_plan(5) == 1
    perm = np.random.default_rng(183).permutation(n_slots).astype(np.int32)
    for call, (batch, slots) in enumerate([(17, perm[:17]), (5, perm[3:8])]):
        x = torch.from_numpy(synth.make_inputs(dims, 184 + call, 1, batch)[0]).cuda()
        sl = torch.from_numpy(np.ascontiguousarray(slots)).cuda()
        assert lay.step_workspace_bytes(batch) <= m2.noalloc_scratch_bytes()
        ya = m2.step(lay, sa, x, slot_ids=sl, residual=True)
        yb = m2.step_noalloc(lay, sb, x, slot_ids=sl, residual=True)
        torch.cuda.synchronize()
        print("[no-alloc] whole call %d batch %d max|dy| %.3e" % (call, batch, float((ya - yb).abs().max())), flush=True)
        assert torch.isfinite(yb).all()
        assert torch.equal(ya, yb)
        assert torch.equal(sa.ssm, sb.ssm) and torch.equal(sa.conv, sb.conv)
