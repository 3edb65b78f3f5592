"""Parity of the attention decode step (m2_attn_step through the C ABI) with the fp64 oracle.

Outputs: normwise per token and session, max_i |y - yo| / max_i |yo| <= 1e-3 (fp32 GEMVs and
attention against fp64; the bf16 rounding of a new key or value can differ by one step
where the fp32 and fp64 values straddle a rounding midpoint, which moves an output by
~1e-5). Caches: the oracle's bits, except at most 1 % of elements that are one bf16 step
apart or within the fp32 error of the projection (an entry that is a sum with
cancellation, as the 4- and 3-bit GEMV's scale * sum(code x) + bias * sum(x) can be).
Positions: exact. Caches start NaN at and past each
session's position, so a read past the last position shows as NaN.
"""
import numpy as np
import pytest

import oracle
from full_duplex_speech_mamba2_amd import synth

pytestmark = pytest.mark.gpu

TOL = 1e-3


def _gpu(dims, w, kc, vc, pos, xs, slots=None, residual=False):
    import torch
    from full_duplex_speech_mamba2_amd import m2
    at = m2.Attn(dims, w)
    kd = torch.from_numpy(kc.view(np.int16).copy()).cuda()
    vd = torch.from_numpy(vc.view(np.int16).copy()).cuda()
    pd = torch.from_numpy(pos.copy()).cuda()
    sd = None if slots is None else torch.from_numpy(np.asarray(slots, np.int32)).cuda()
    ys = []
    for t in range(xs.shape[0]):
        x = torch.from_numpy(xs[t]).cuda()
        ys.append(at.step(kd, vd, pd, x, slot_ids=sd, residual=residual))
    torch.cuda.synchronize()
    return (np.stack([y.cpu().numpy() for y in ys]), kd.cpu().numpy().view(np.uint16),
            vd.cpu().numpy().view(np.uint16), pd.cpu().numpy())


def _oracle(dims, w, kc, vc, pos, xs, slots=None, residual=False):
    lay = oracle.AttnLayer(dims, w)
    kc, vc, pos = kc.copy(), vc.copy(), pos.copy()
    ys = [lay.step(kc, vc, pos, xs[t], slot_ids=slots, residual=residual) for t in range(xs.shape[0])]
    return np.stack(ys), kc, vc, pos


def _cache_ok(g, o):
    """Equal bits, except where the fp32 and fp64 projections round to neighbouring bf16
    values or differ by the fp32 error of the projection (1e-5 of the largest entry, for
    entries that are sums with cancellation); NaN (unwritten rows) in the same places."""
    if np.array_equal(g, o):
        return True
    a = (g.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    b = (o.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    if not np.array_equal(np.isnan(a), np.isnan(b)):
        return False
    diff = (g != o) & ~np.isnan(b)
    big = float(np.max(np.abs(b[~np.isnan(b)])))
    close = np.abs(a[diff] - b[diff]) <= 2.0 ** -7 * np.maximum(np.abs(a[diff]), np.abs(b[diff])) + 1e-5 * big
    print("[attn] cache: %d elements differ, largest gap %.3e (entries up to %.3e), all within bound: %s"
          % (diff.sum(), float(np.max(np.abs(a[diff] - b[diff]))), big, bool(np.all(close))), flush=True)
    return bool(np.all(close)) and diff.sum() <= max(1, g.size // 100)


def _check(tag, dims, w, kc, vc, pos, xs, slots=None, residual=False):
    print("[attn] %s wtype=%s Hq=%d Hk=%d D=%d B=%d pos=%s" % (tag, dims.wtype, dims.n_q, dims.n_kv, dims.head_dim,
                                                               xs.shape[1], pos.tolist()[:8]), flush=True)
    yg, kg, vg, pg = _gpu(dims, w, kc, vc, pos, xs, slots, residual)
    yo, ko, vo, po = _oracle(dims, w, kc, vc, pos, xs, slots, residual)
    assert np.array_equal(pg, po)
    dead = np.all(np.isnan(yo), axis=-1)
    assert np.array_equal(np.all(np.isnan(yg), axis=-1), dead)
    live = ~dead
    err = 0.0
    if live.any():
        d = np.max(np.abs(yg - yo), axis=-1)[live]
        m = np.max(np.abs(yo), axis=-1)[live]
        assert np.all(np.isfinite(yg[live]))
        err = float(np.max(d / m))
    print("[attn] %s e_out=%.3e" % (tag, err), flush=True)
    assert err <= TOL
    assert _cache_ok(kg, ko) and _cache_ok(vg, vo)
    return yg


SMALL = synth.AttnDims(d_model=256, n_q=4, n_kv=2, head_dim=64, max_len=200)


@pytest.mark.parametrize("batch", [1, 2, 3, 5])
@pytest.mark.parametrize("wtype,q_group,gamma", [("f32", 16, 1.0), ("bf16", 16, 1.0), ("int8g", 64, 0.0625),
                                                 ("int8g", 128, 0.0625), ("int4g", 32, 1.0), ("int3g", 64, 1.0)])
def test_attn_formats_and_chunk_edges(wtype, q_group, gamma, batch):
    """Positions at and across the 64-position chunk edges (0, 1, 63, 64, 130); 3 steps. From
    3 sessions, bf16 and int8 g128 projections take the MFMA GEMV."""
    d = SMALL.replace(wtype=wtype, q_group=q_group, q_gamma_qkv=gamma, q_gamma_o=gamma)
    pos = np.array([0, 63, 1, 130, 64][:batch], np.int32)
    w = synth.make_attn_weights(d, 21)
    kc, vc = synth.make_kv_cache(d, 22, pos)
    xs = synth.make_attn_inputs(d, 23, 3, batch)
    _check("formats", d, w, kc, vc, pos, xs)


@pytest.mark.parametrize("n_q,n_kv", [(8, 8), (6, 2), (16, 2), (10, 2)])
def test_attn_group_sizes_d128(n_q, n_kv):
    d = synth.AttnDims(d_model=512, n_q=n_q, n_kv=n_kv, head_dim=128, max_len=300)
    pos = np.array([5, 299, 128], np.int32)
    w = synth.make_attn_weights(d, 24)
    kc, vc = synth.make_kv_cache(d, 25, pos)
    xs = synth.make_attn_inputs(d, 26, 2, 3)
    _check("groups", d, w, kc, vc, pos, xs)


def test_attn_slots_residual_full_cache_and_bad_slots():
    d = SMALL.replace(max_len=100)
    pos = np.array([10, 99, 0, 50, 100], np.int32)          # slot 1 fills on the first step; slot 4 is full
    w = synth.make_attn_weights(d, 27)
    kc, vc = synth.make_kv_cache(d, 28, pos)
    xs = synth.make_attn_inputs(d, 29, 3, 5)
    yg = _check("slots", d, w, kc, vc, pos, xs, slots=[3, 1, 7, 4, 0], residual=True)
    assert np.all(np.isnan(yg[:, 2])) and np.all(np.isnan(yg[:, 3])) and np.all(np.isnan(yg[1:, 1]))


@pytest.mark.parametrize("batch,pos", [(1, [1499]), (4, [0, 700, 1100, 1499]), (2, [1000, 64])])
def test_attn_9b_shapes(batch, pos):
    """40 query heads over 8 key/value heads of 128, 1500 positions (the 2-minute context)."""
    d = synth.ATTN_9B
    pos = np.array(pos, np.int32)
    w = synth.make_attn_weights(d, 30)
    kc, vc = synth.make_kv_cache(d, 31, pos)
    xs = synth.make_attn_inputs(d, 32, 2, batch)
    _check("9b", d, w, kc, vc, pos, xs, residual=True)


def test_attn_9b_32_sessions():
    d = synth.ATTN_9B
    pos = np.random.default_rng(33).integers(0, 1500, 32).astype(np.int32)
    w = synth.make_attn_weights(d, 34)
    kc, vc = synth.make_kv_cache(d, 35, pos)
    xs = synth.make_attn_inputs(d, 36, 1, 32)
    _check("9b-b32", d, w, kc, vc, pos, xs)


def test_attn_timed_step_matches():
    import torch
    from full_duplex_speech_mamba2_amd import m2
    d = SMALL
    pos = np.array([17, 90], np.int32)
    w = synth.make_attn_weights(d, 37)
    kc, vc = synth.make_kv_cache(d, 38, pos)
    x = torch.from_numpy(synth.make_attn_inputs(d, 39, 1, 2)[0]).cuda()
    at = m2.Attn(d, w)
    outs = []
    for timed in (False, True):
        kd = torch.from_numpy(kc.view(np.int16).copy()).cuda()
        vd = torch.from_numpy(vc.view(np.int16).copy()).cuda()
        pd = torch.from_numpy(pos.copy()).cuda()
        y = torch.empty_like(x)
        if timed:
            ev = [torch.cuda.Event(enable_timing=True) for _ in range(5)]
            for e in ev:
                e.record()
            at.step_timed(kd, vd, pd, x, y, ev)
        else:
            at.step(kd, vd, pd, x, y)
        torch.cuda.synchronize()
        outs.append((y.cpu(), kd.cpu(), pd.cpu()))
    assert all(torch.equal(a, b) for a, b in zip(*outs))
    assert all(ev[i].elapsed_time(ev[i + 1]) > 0 for i in range(4))


@pytest.mark.parametrize("batch", [1, 3])
def test_attn_long_cache_combines_more_than_32_chunks(batch):
    """3000 positions = 47 chunks: the combine takes two passes of 32 chunks."""
    d = synth.AttnDims(d_model=256, n_q=4, n_kv=1, head_dim=128, max_len=3000)
    pos = np.array([2999, 2100, 40][:batch], np.int32)
    w = synth.make_attn_weights(d, 40)
    kc, vc = synth.make_kv_cache(d, 41, pos)
    xs = synth.make_attn_inputs(d, 42, 2, batch)
    _check("long", d, w, kc, vc, pos, xs)


@pytest.mark.parametrize("n_q,n_kv", [(4, 4), (16, 2)])
def test_attn_group_sizes_d64(n_q, n_kv):
    """head_dim 64: 8 lanes share a cache row (the half-row reductions), 1 and 8 query heads per group."""
    d = synth.AttnDims(d_model=256, n_q=n_q, n_kv=n_kv, head_dim=64, max_len=200)
    pos = np.array([0, 199, 64, 127], np.int32)
    w = synth.make_attn_weights(d, 43)
    kc, vc = synth.make_kv_cache(d, 44, pos)
    xs = synth.make_attn_inputs(d, 45, 2, 4)
    _check("d64", d, w, kc, vc, pos, xs)
