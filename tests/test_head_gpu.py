"""Parity of the output-head kernels (m2_head_argmax through the C ABI) with the fp64 oracle.

Logits: element by element within the a-priori bound of fp32 accumulation,
|g - o| <= (K/64 + 16) 2^-24 sum_k |w~_vk| |h_k|, where the kernel sums K/64 terms per
lane, then 6 shuffle levels, and |w~| bounds a decoded weight (|w| for f32 and bf16,
|q| s gamma for int8, ((2^bits - 1) s + |b|) gamma for the 4- and 3-bit codes).
Tokens: where the oracle's best logit leads the next by more than twice the largest
bound the token is the oracle's; elsewhere it must be a row whose oracle logit lies
within that margin of the maximum. Exact ties (bitwise equal rows give bitwise equal
sums on both sides) must give the lowest index; a NaN logit is never the token.
"""
import functools

import numpy as np
import pytest

import oracle
from full_duplex_speech_mamba2_amd import synth

pytestmark = pytest.mark.gpu

U = 2.0 ** -24


def _abs_weight_bound(wtype, w, s, q_group, gamma):
    if wtype == "f32":
        return np.abs(w.astype(np.float64))
    if wtype == "bf16":
        return np.abs((w.astype(np.uint32) << 16).view(np.float32).astype(np.float64))
    if wtype == "int8g":
        return np.abs(w.astype(np.float64)) * np.repeat(np.abs(s.astype(np.float64)), q_group, axis=1) * gamma
    top = 2.0 ** synth.LOWBIT[wtype] - 1.0
    s = np.abs(s.astype(np.float64))
    return np.repeat(top * s[..., 0] + s[..., 1], q_group, axis=1) * gamma


def _run(wtype, w, s, h, q_group=0, gamma=1.0, with_logits=True):
    import torch
    from full_duplex_speech_mamba2_amd import m2
    V, K = w.shape[0], h.shape[1]
    head = m2.Head(K, V, w, s, wtype=wtype, q_group=q_group, q_gamma=gamma)
    hd = torch.from_numpy(np.ascontiguousarray(h, np.float32)).cuda()
    logits = torch.full((h.shape[0], V), float("nan"), device="cuda") if with_logits else None
    tok = head.argmax(hd, logits=logits)
    torch.cuda.synchronize()
    return tok.cpu().numpy(), None if logits is None else logits.cpu().numpy()


def _check(tag, wtype, w, s, h, q_group=0, gamma=1.0):
    V, K = w.shape[0], h.shape[1]
    print("[head] %s wtype=%s V=%d K=%d B=%d" % (tag, wtype, V, K, h.shape[0]), flush=True)
    tok, lg = _run(wtype, w, s, h, q_group, gamma)
    tok2, _ = _run(wtype, w, s, h, q_group, gamma, with_logits=False)
    lo, to = oracle.head_argmax(wtype, w, h, s, q_group, gamma if wtype not in ("f32", "bf16") else 1.0)
    ah = np.abs(h.astype(np.float64))
    bound = np.empty((h.shape[0], V))
    for r0 in range(0, V, 4096):                          # in row blocks: the 9B head is 587M weights
        r1 = min(V, r0 + 4096)
        wb = _abs_weight_bound(wtype, w[r0:r1], None if s is None else s[r0:r1], q_group, gamma)
        bound[:, r0:r1] = (K / 64 + 16) * U * (ah @ wb.T)
    err = np.abs(lg - lo)
    print("[head] %s max |g-o| = %.3e, max bound %.3e, max |o| %.3e" % (tag, err.max(), bound.max(),
                                                                         np.abs(lo).max()), flush=True)
    assert np.all(err <= bound)
    assert np.array_equal(tok, tok2)
    for b in range(h.shape[0]):
        margin = 2 * bound[b].max()
        order = np.argsort(-lo[b], kind="stable")
        assert 0 <= tok[b] < V
        assert lo[b, tok[b]] >= lo[b, order[0]] - margin
        if V == 1 or lo[b, order[0]] - lo[b, order[1]] > margin:
            assert tok[b] == to[b]
    return tok, lg, lo


@pytest.mark.parametrize("batch", [1, 2, 3, 5])
@pytest.mark.parametrize("wtype,q_group,gamma", [("f32", 0, 1.0), ("bf16", 0, 1.0), ("int8g", 64, 0.5),
                                                 ("int4g", 32, 1.0), ("int3g", 64, 2.0)])
def test_head_ragged_vocab(wtype, q_group, gamma, batch):
    """1003 rows: the last workgroup holds 3 rows; K = 320 leaves most lanes of the chunk loop idle."""
    w, s = synth.make_head_weights(1003, 320, wtype, q_group, seed=61)
    h = synth.make_head_states(320, batch, seed=62)
    _check("ragged", wtype, w, s, h, q_group, gamma)


@pytest.mark.parametrize("V", [1, 8, 9, 4099])
def test_head_vocab_edges_bf16(V):
    w, _ = synth.make_head_weights(V, 4480, "bf16", 0, seed=63)
    h = synth.make_head_states(4480, 4, seed=64)
    tok, _, _ = _check("edges", "bf16", w, None, h)
    if V == 1:
        assert np.array_equal(tok, [0, 0, 0, 0])


def test_head_exact_ties_take_the_lowest_index():
    V, K = 2051, 512
    w, _ = synth.make_head_weights(V, K, "bf16", 0, seed=65)
    h = synth.make_head_states(K, 3, seed=66)
    h[1] = h[0]
    big = synth.f32_to_bf16_bits((np.sign(h[0]) * 0.05).astype(np.float32))
    for r in (1900, 333, 334, 12, 1024):                  # other workgroups, one workgroup, first and last
        w[r] = big
    tok, lg, _ = _check("ties", "bf16", w, None, h)
    assert tok[0] == 12 and tok[1] == 12
    assert np.all(lg[0, [1900, 333, 334, 1024]] == lg[0, 12])
    tok, lg, _ = _check("zeros", "bf16", np.zeros((V, K), np.uint16), None, h)
    assert np.array_equal(tok, [0, 0, 0]) and not np.any(lg)


def test_head_nan_never_wins():
    import torch  # noqa: F401
    V, K = 700, 256
    rng = np.random.default_rng(67)
    w = (rng.standard_normal((V, K)) / 16).astype(np.float32)
    h = np.abs(rng.standard_normal((3, K)).astype(np.float32)) + 0.5
    w[3, 0] = np.nan                                          # NaN logit in every session
    w[650] = 1.0                                              # the maximum in every session
    h[2, 7] = np.nan                                          # session 2: every logit NaN
    tok, lg = _run("f32", w, None, h)
    lo, to = oracle.head_argmax("f32", w, h)
    assert np.array_equal(tok, [650, 650, -1]) and np.array_equal(to, tok)
    assert np.isnan(lg[0, 3]) and np.all(np.isnan(lg[2]))
    w[:] = -np.inf                                            # every logit -inf: the lowest index
    tok, _ = _run("f32", w, None, h[:2])
    assert np.array_equal(tok, [0, 0])


@functools.lru_cache(maxsize=1)
def _text_head_9b():
    return synth.make_head_weights(131072, 4480, "bf16", 0, seed=71)


@pytest.mark.parametrize("batch", [1, 2, 4])
def test_head_9b_text_head_bf16(batch):
    """The 131072 x 4480 bf16 head of the per-frame workload (one row per wave, 16384 workgroups)."""
    w, _ = _text_head_9b()
    h = synth.make_head_states(4480, batch, seed=72)
    _check("9b", "bf16", w, None, h)


@pytest.mark.parametrize("wtype,q_group", [("int4g", 64), ("int3g", 64), ("int8g", 128)])
def test_head_9b_quantized(wtype, q_group):
    w, s = synth.make_head_weights(32768, 4480, wtype, q_group, seed=73)
    h = synth.make_head_states(4480, 2, seed=74)
    _check("9b-q", wtype, w, s, h, q_group, 1.0)


def test_head_timed_call_matches_and_times_both_kernels():
    import torch
    from full_duplex_speech_mamba2_amd import m2
    w, _ = synth.make_head_weights(4099, 4480, "bf16", 0, seed=75)
    h = torch.from_numpy(synth.make_head_states(4480, 3, seed=76)).cuda()
    head = m2.Head(4480, 4099, w)
    ref = head.argmax(h)
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(3)]
    for e in ev:
        e.record()
    tok = torch.empty(3, dtype=torch.int32, device="cuda")
    head.argmax_timed(h, tok, ev)
    torch.cuda.synchronize()
    assert torch.equal(tok, ref)
    assert ev[0].elapsed_time(ev[1]) > 0 and ev[1].elapsed_time(ev[2]) > 0
    with pytest.raises(m2.M2Error):
        head.argmax_timed(torch.zeros((5, 4480), device="cuda"), torch.empty(5, dtype=torch.int32, device="cuda"),
                          ev)
