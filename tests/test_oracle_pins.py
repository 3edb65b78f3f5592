"""Pins of the CPU oracle against facts that do not come from the oracle itself.

Each test checks the fp64 oracle against mathematics or a library routine: the
materialised quadratic form of the SSD map, closed forms, special cases that
reduce to a plain contraction or to numpy, and invariants. Together they are
chosen so that a plausible slip in the oracle (a dropped term, a wrong index,
sign or tap order, a swapped B/C, a transposed weight) fails at least one.

The pages print no numeric example of the mixer, so there are no page values
to store under tests/golden/.
"""
import math

import numpy as np
import pytest

import oracle
from full_duplex_speech_mamba2_amd import synth

RTOL = 1e-12


def rel(a, b):
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    return float(np.max(np.abs(a - b)) / max(np.max(np.abs(b)), 1e-300))


SMALL_G2 = synth.MixerDims(d_model=64, n_heads=4, head_dim=8, d_state=16, n_groups=2,
                           d_conv=4, wtype="f32")


def codes_from_bytes(row_bytes, bits):
    """Codes of one packed row, decoded here from the stated format with Python integers:
    4-bit, the even code in the low nibble; 3-bit, each 12-byte run is a little-endian
    96-bit integer holding code i at bits 3i .. 3i+2."""
    b = bytes(np.asarray(row_bytes, np.uint8))
    if bits == 4:
        return [c for byte in b for c in (byte & 15, byte >> 4)]
    out = []
    for r in range(0, len(b), 12):
        v = int.from_bytes(b[r:r + 12], "little")
        out += [(v >> (3 * i)) & 7 for i in range(32)]
    return out


def decoded(dims, w, which):
    """Dequantised weight matrix via numpy (float32 view of bf16 bits, int8 * fp16 * gamma,
    low-bit (scale code + bias) * gamma with codes from codes_from_bytes)."""
    m = w[which]
    if dims.wtype == "f32":
        return m.astype(np.float64)
    if dims.wtype == "bf16":
        return (m.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    s = w["s_in" if which == "w_in" else "s_out"].astype(np.float64)
    gamma = dims.q_gamma_in if which == "w_in" else dims.q_gamma_out
    if dims.wtype in synth.LOWBIT:
        q = np.array([codes_from_bytes(r, synth.LOWBIT[dims.wtype]) for r in m], np.float64)
        return (q * np.repeat(s[..., 0], dims.q_group, axis=1) + np.repeat(s[..., 1], dims.q_group, axis=1)) * gamma
    return m.astype(np.float64) * np.repeat(s, dims.q_group, axis=1) * gamma


def split(dims, v):
    """Split a conv-output vector into x [H][P], B [G][N], C [G][N] by the declared layout."""
    di, G, N = dims.d_inner, dims.n_groups, dims.d_state
    x = v[..., :di].reshape(v.shape[:-1] + (dims.n_heads, dims.head_dim))
    Bm = v[..., di:di + G * N].reshape(v.shape[:-1] + (G, N))
    Cm = v[..., di + G * N:di + 2 * G * N].reshape(v.shape[:-1] + (G, N))
    return x, Bm, Cm


# ---------------------------------------------------------------- element decoders

def test_fp16_decoder_matches_numpy_for_every_pattern():
    bits = np.arange(65536, dtype=np.uint16)
    ref = bits.view(np.float16).astype(np.float64)
    got = np.array([oracle.fp16_to_double(int(b)) for b in bits])
    finite = np.isfinite(ref)
    assert np.array_equal(got[finite], ref[finite])
    assert np.all(np.isnan(got[np.isnan(ref)]))
    assert np.array_equal(got[np.isinf(ref)], ref[np.isinf(ref)])


def test_bf16_decoder_is_top_half_of_binary32():
    assert oracle.bf16_to_double(0x3F80) == 1.0
    assert oracle.bf16_to_double(0xC000) == -2.0
    assert oracle.bf16_to_double(0x0001) == 2.0 ** -133
    rng = np.random.default_rng(5)
    for b in rng.integers(0, 0x7F80, 200):
        ref = np.array([int(b) << 16], np.uint32).view(np.float32)[0]
        assert oracle.bf16_to_double(int(b)) == float(ref)


def test_lowbit_decoder_against_hand_packed_bytes():
    # 4-bit: byte 0x21 holds codes 1 (low nibble, even k) then 2
    row = np.array([[0x21, 0x43, 0xF0, 0x0E] + [0] * 28], np.uint8)
    got = [oracle.lowbit_code("int4g", row, 0, k) for k in range(8)]
    assert got == [1, 2, 3, 4, 0, 15, 14, 0]
    # 3-bit: two rows of two 32-code runs built as 96-bit integers here
    rng = np.random.default_rng(5)
    codes = rng.integers(0, 8, size=(2, 64))
    packed = np.zeros((2, 24), np.uint8)
    for r in range(2):
        for run in range(2):
            v = sum(int(c) << (3 * i) for i, c in enumerate(codes[r, 32 * run:32 * run + 32]))
            packed[r, 12 * run:12 * run + 12] = np.frombuffer(v.to_bytes(12, "little"), np.uint8)
    for r in range(2):
        assert [oracle.lowbit_code("int3g", packed, r, k) for k in range(64)] == list(codes[r])
    # the generator's packer agrees with both
    for bits, wt in ((4, "int4g"), (3, "int3g")):
        q = rng.integers(0, 2 ** bits, size=(3, 128)).astype(np.uint8)
        pk = synth.pack_codes(q, bits)
        assert [codes_from_bytes(r, bits) for r in pk] == q.tolist()
        assert [oracle.lowbit_code(wt, pk, 2, k) for k in range(128)] == q[2].tolist()


def test_bf16_rounding_of_generator_is_nearest_even():
    # 1 + 2^-8 lies exactly between bf16 neighbours 1 and 1 + 2^-7: ties go to the even one (1.0)
    vals = np.array([1.0 + 2.0 ** -8, 1.0 + 3 * 2.0 ** -8, 1.0 + 2.0 ** -9], np.float32)
    bits = synth.f32_to_bf16_bits(vals)
    assert [oracle.bf16_to_double(int(b)) for b in bits] == [1.0, 1.0 + 2 ** -6, 1.0]


# ---------------------------------------------------------------- scalar functions

def test_softplus_against_logaddexp_and_limits():
    xs = np.concatenate([np.linspace(-40, 40, 801), [-1e4, -800.0, 800.0, 1e4]])
    got = np.array([oracle.softplus(float(x)) for x in xs])
    assert rel(got, np.logaddexp(0.0, xs)) < 1e-15
    assert oracle.softplus(0.0) == pytest.approx(math.log(2.0), rel=1e-16)
    assert oracle.softplus(-1e4) == 0.0          # underflows to exactly 0: the dt = 0 case
    assert oracle.softplus(1e4) == 1e4


def test_silu_against_logistic():
    from scipy.special import expit
    xs = np.linspace(-30, 30, 601)
    got = np.array([oracle.silu(float(x)) for x in xs])
    assert rel(got, xs * expit(xs)) < 1e-15
    assert oracle.silu(0.0) == 0.0


# ---------------------------------------------------------------- SSD core: two definitions

def _ssd_inputs(T, H, P, N, G, seed, s0=True):
    r = np.random.default_rng(seed)
    x = r.standard_normal((T, H, P))
    Bm = r.standard_normal((T, G, N))
    Cm = r.standard_normal((T, G, N))
    dt = np.exp(r.uniform(math.log(1e-3), math.log(0.5), (T, H)))
    A = -np.exp(r.uniform(0, math.log(16), H))
    D = r.standard_normal(H)
    S0 = r.standard_normal((H, P, N)) if s0 else np.zeros((H, P, N))
    return x, Bm, Cm, dt, A, D, S0


@pytest.mark.parametrize("T,H,P,N,G", [(37, 4, 3, 5, 2), (64, 8, 4, 16, 1), (1, 2, 2, 3, 2), (20, 6, 5, 7, 3)])
def test_recurrence_equals_quadratic_form(T, H, P, N, G):
    x, Bm, Cm, dt, A, D, S0 = _ssd_inputs(T, H, P, N, G, seed=T * 7 + H)
    S = S0.copy()
    y_rec = oracle.ssd_recurrent(x, Bm, Cm, dt, A, D, S)
    y_q, S_q = oracle.ssd_quadratic(x, Bm, Cm, dt, A, D, S0)
    assert rel(y_rec, y_q) < RTOL
    assert rel(S, S_q) < RTOL


def test_scalar_geometric_closed_form():
    # H = P = N = G = 1, constant dt, A, x, B = C = 1, S0 = 0, D = 0:
    # S_t = dt x (1 - a^(t+1)) / (1 - a) with a = exp(dt A), and y_t = S_t.
    T, dtv, Av, xv = 50, 0.07, -3.0, 1.7
    a = math.exp(dtv * Av)
    S = np.zeros((1, 1, 1))
    y = oracle.ssd_recurrent(np.full((T, 1, 1), xv), np.ones((T, 1, 1)), np.ones((T, 1, 1)),
                             np.full((T, 1), dtv), np.array([Av]), np.array([0.0]), S)
    ref = np.array([dtv * xv * (1 - a ** (t + 1)) / (1 - a) for t in range(T)])
    assert rel(y[:, 0, 0], ref) < 1e-14
    assert S[0, 0, 0] == pytest.approx(ref[-1], rel=1e-14)


def test_d_skip_only_when_C_is_zero():
    x, Bm, Cm, dt, A, D, S0 = _ssd_inputs(9, 4, 3, 5, 2, seed=3)
    S = S0.copy()
    y = oracle.ssd_recurrent(x, Bm, np.zeros_like(Cm), dt, A, D, S)
    assert np.array_equal(y, D[None, :, None] * x)


# ---------------------------------------------------------------- the full step

def _layer(dims, seed=0, **override):
    w = synth.make_layer_weights(dims, seed)
    w.update(override)
    return oracle.Layer(dims, w), w


def test_in_and_out_projection_match_numpy_matmul():
    for dims in (SMALL_G2, synth.TINY.replace(wtype="bf16"),
                 synth.TINY.replace(wtype="int8g", q_group=128, q_gamma_in=0.0625, q_gamma_out=0.0625),
                 synth.TINY.replace(wtype="int4g", q_group=64),
                 synth.TINY.replace(wtype="int3g", q_group=32, q_gamma_in=0.5, q_gamma_out=2.0),
                 synth.TINY.replace(wtype="int3g", q_group=128)):
        lay, w = _layer(dims, seed=11)
        ssm, conv = lay.new_state(2)
        x = np.random.default_rng(1).standard_normal((2, dims.d_model))
        y, tr = lay.step(ssm, conv, x, trace=True)
        assert rel(tr["zxbcdt"], x @ decoded(dims, w, "w_in").T) < RTOL
        assert rel(tr["out"], tr["yn"] @ decoded(dims, w, "w_out").T) < RTOL
        assert np.array_equal(y, tr["out"])


def test_step_ssd_wiring_matches_quadratic_form_over_a_sequence():
    # run T steps through orc_step, take the conv outputs and dt it traced, split them by
    # the declared layout and recompute every readout with the quadratic form
    dims = SMALL_G2
    lay, w = _layer(dims, seed=2)
    T = 12
    ssm, conv = lay.new_state(1, ssm0=np.random.default_rng(4).standard_normal((1, 4, 8, 16)))
    S0 = ssm[0].copy()
    xs = np.random.default_rng(3).standard_normal((T, 1, dims.d_model))
    xc, dts, ys = [], [], []
    for t in range(T):
        _, tr = lay.step(ssm, conv, xs[t], trace=True)
        xc.append(tr["xconv"][0]); dts.append(tr["dt"][0]); ys.append(tr["y"][0])
    xh, Bm, Cm = split(dims, np.array(xc))
    A = -np.exp(w["A_log"].astype(np.float64))
    yq, Sq = oracle.ssd_quadratic(xh, Bm, Cm, np.array(dts), A, w["D"].astype(np.float64), S0)
    assert rel(np.array(ys), yq.reshape(T, -1)) < RTOL
    assert rel(ssm[0], Sq) < RTOL


def test_dt_zero_leaves_state_bitwise_unchanged():
    dims = SMALL_G2
    lay, w = _layer(dims, seed=3, dt_bias=np.full(dims.n_heads, -1e4, np.float32))
    ssm, conv = lay.new_state(1, ssm0=np.random.default_rng(6).standard_normal((1, 4, 8, 16)))
    before = ssm.copy()
    x = np.random.default_rng(7).standard_normal((1, dims.d_model))
    _, tr = lay.step(ssm, conv, x, trace=True)
    assert np.all(tr["dt"] == 0.0)
    assert np.array_equal(ssm, before)
    xh, Bm, Cm = split(dims, tr["xconv"][0])
    g = np.arange(dims.n_heads) // (dims.n_heads // dims.n_groups)
    ref = np.einsum("hpn,hn->hp", before[0], Cm[g]) + w["D"][:, None] * xh
    assert rel(tr["y"][0], ref.reshape(-1)) < RTOL


def test_very_negative_A_resets_state_to_input_outer_product():
    dims = SMALL_G2
    lay, w = _layer(dims, seed=4, A_log=np.full(dims.n_heads, math.log(1e30), np.float32))
    ssm, conv = lay.new_state(1, ssm0=np.random.default_rng(8).standard_normal((1, 4, 8, 16)))
    x = np.random.default_rng(9).standard_normal((1, dims.d_model))
    _, tr = lay.step(ssm, conv, x, trace=True)
    xh, Bm, Cm = split(dims, tr["xconv"][0])
    g = np.arange(dims.n_heads) // (dims.n_heads // dims.n_groups)
    dt = tr["dt"][0]
    S_ref = dt[:, None, None] * xh[:, :, None] * Bm[g][:, None, :]
    assert np.array_equal(ssm[0], S_ref)
    y_ref = dt[:, None] * np.sum(Cm[g] * Bm[g], axis=1)[:, None] * xh + w["D"][:, None] * xh
    assert rel(tr["y"][0], y_ref.reshape(-1)) < RTOL


def test_dt_rows_are_last_and_softplus_inverts_bias():
    # zero dt rows of W_in: dt_raw = 0, so dt = softplus(dt_bias) = dt0 of the generator
    dims = SMALL_G2
    w = synth.make_layer_weights(dims, 5)
    w["w_in"] = w["w_in"].copy()
    w["w_in"][-dims.n_heads:, :] = 0.0
    lay = oracle.Layer(dims, w)
    ssm, conv = lay.new_state(1)
    _, tr = lay.step(ssm, conv, np.ones((1, dims.d_model)), trace=True)
    assert np.all(tr["zxbcdt"][0, -dims.n_heads:] == 0.0)
    dt0 = np.log1p(np.exp(w["dt_bias"].astype(np.float64)))
    assert rel(tr["dt"][0], dt0) < 1e-15
    assert np.all((tr["dt"][0] > 0.9e-3) & (tr["dt"][0] < 0.11))


def test_zero_gate_rows_give_zero_output():
    # z occupies the first d_inner rows: with them zero, v = y * SiLU(0) = 0, so out = 0
    dims = SMALL_G2
    w = synth.make_layer_weights(dims, 6)
    w["w_in"] = w["w_in"].copy()
    w["w_in"][:dims.d_inner, :] = 0.0
    lay = oracle.Layer(dims, w)
    ssm, conv = lay.new_state(1)
    x = np.random.default_rng(2).standard_normal((1, dims.d_model))
    y = lay.step(ssm, conv, x)
    assert np.all(y == 0.0)
    assert np.any(ssm != 0.0)                       # the state still advanced
    yr = lay.step(ssm, conv, x, residual=True)
    assert np.array_equal(yr, x)                    # residual: y = x + 0


def test_large_gate_is_identity():
    # z >> 0 makes SiLU(z) = z to double precision, so v = y * z
    dims = SMALL_G2
    w = synth.make_layer_weights(dims, 7)
    w["w_in"] = w["w_in"].copy()
    w["w_in"][:dims.d_inner, :] = 0.0
    w["w_in"][:dims.d_inner, 0] = 100.0
    lay = oracle.Layer(dims, w)
    ssm, conv = lay.new_state(1)
    x = np.zeros((1, dims.d_model)); x[0, 0] = 1.0; x[0, 1] = 0.5
    _, tr = lay.step(ssm, conv, x, trace=True)
    assert rel(tr["v"], tr["y"] * 100.0) < 1e-15


def test_group_map_is_consecutive_heads():
    # B rows and conv bias of group 1 zero: heads of group 1 (the last H/G) get no input
    dims = SMALL_G2
    di, N = dims.d_inner, dims.d_state
    w = synth.make_layer_weights(dims, 8)
    w["w_in"] = w["w_in"].copy(); w["conv_b"] = w["conv_b"].copy()
    w["w_in"][di + di + N:di + di + 2 * N, :] = 0.0      # z | x | B(g0) | B(g1) ...
    w["conv_b"][di + N:di + 2 * N] = 0.0
    lay = oracle.Layer(dims, w)
    ssm, conv = lay.new_state(1)
    for t in range(3):
        lay.step(ssm, conv, np.random.default_rng(t).standard_normal((1, dims.d_model)))
    assert np.all(ssm[0, 2:] == 0.0)
    assert np.all(np.abs(ssm[0, :2]).max(axis=(1, 2)) > 0.0)


def test_conv_identity_tap_and_cache_shift():
    dims = SMALL_G2
    K = dims.d_conv
    cw = np.zeros((dims.conv_dim, K), np.float32); cw[:, K - 1] = 1.0
    lay, _ = _layer(dims, seed=9, conv_w=cw, conv_b=np.zeros(dims.conv_dim, np.float32))
    ssm, conv = lay.new_state(1)
    raws = []
    for t in range(5):
        x = np.random.default_rng(20 + t).standard_normal((1, dims.d_model))
        _, tr = lay.step(ssm, conv, x, trace=True)
        raw = tr["zxbcdt"][0, dims.d_inner:dims.d_inner + dims.conv_dim]
        raws.append(raw)
        from scipy.special import expit
        assert rel(tr["xconv"][0], raw * expit(raw)) < 1e-15
    # after >= d_conv - 1 steps the cache holds the last d_conv - 1 raw inputs, oldest first
    assert np.array_equal(conv[0], np.array(raws[-(K - 1):]))


def test_conv_oldest_tap_is_a_three_step_delay():
    dims = SMALL_G2
    K = dims.d_conv
    cw = np.zeros((dims.conv_dim, K), np.float32); cw[:, 0] = 1.0
    lay, _ = _layer(dims, seed=10, conv_w=cw, conv_b=np.zeros(dims.conv_dim, np.float32))
    ssm, conv = lay.new_state(1)
    raws, outs = [], []
    from scipy.special import expit
    for t in range(7):
        x = np.random.default_rng(40 + t).standard_normal((1, dims.d_model))
        _, tr = lay.step(ssm, conv, x, trace=True)
        raws.append(tr["zxbcdt"][0, dims.d_inner:dims.d_inner + dims.conv_dim])
        outs.append(tr["xconv"][0])
    for t in range(7):
        ref = raws[t - (K - 1)] if t >= K - 1 else np.zeros(dims.conv_dim)
        assert rel(outs[t], ref * expit(ref)) < 1e-15 if t >= K - 1 else np.all(outs[t] == 0.0)


def test_grouped_rmsnorm_invariants():
    # per RMS group: yn / norm_w is parallel to v and has RMS sqrt(ms / (ms + eps))
    for dims in (SMALL_G2, SMALL_G2.replace(norm_group=SMALL_G2.d_inner), SMALL_G2.replace(norm_group=8)):
        lay, w = _layer(dims, seed=12)
        ssm, conv = lay.new_state(1)
        _, tr = lay.step(ssm, conv, np.random.default_rng(1).standard_normal((1, dims.d_model)), trace=True)
        gs = dims.rms_group
        v = tr["v"][0].reshape(-1, gs)
        u = (tr["yn"][0] / w["norm_w"]).reshape(-1, gs)
        ms = np.mean(v * v, axis=1)
        assert rel(np.sqrt(np.mean(u * u, axis=1)), np.sqrt(ms / (ms + dims.norm_eps))) < 1e-13
        ratio = u / v
        assert np.max(np.abs(ratio - ratio[:, :1])) / np.max(np.abs(ratio)) < 1e-13


def test_constant_vector_rmsnorm_closed_form():
    # with W_out = I-like selection we can read yn; use the trace: a group whose v is constant c
    # normalises to sign(c) * norm_w * |c| / sqrt(c^2 + eps). Build it with y = D x only (C = 0)
    # and x constant per head (conv identity tap, x rows selecting one input coordinate).
    dims = synth.MixerDims(d_model=16, n_heads=4, head_dim=4, d_state=8, n_groups=2, wtype="f32")
    di, G, N, K = dims.d_inner, dims.n_groups, dims.d_state, dims.d_conv
    w = synth.make_layer_weights(dims, 13)
    win = np.zeros((dims.d_in_proj, dims.d_model), np.float32)
    win[:di, 0] = 50.0                       # z = 50 * u0: SiLU(z) = z to double precision
    win[di:2 * di, 1] = 1.0                  # x = u1 on every channel
    w["w_in"] = win
    cw = np.zeros((dims.conv_dim, K), np.float32); cw[:, K - 1] = 1.0
    w["conv_w"] = cw
    w["conv_b"] = np.zeros(dims.conv_dim, np.float32)
    w["D"] = np.array([0.5, 0.5, -1.0, -1.0], np.float32)   # one value per RMS group of 8 channels
    lay = oracle.Layer(dims, w)
    ssm, conv = lay.new_state(1)
    u = np.zeros((1, dims.d_model)); u[0, 0] = 1.0; u[0, 1] = 2.0
    _, tr = lay.step(ssm, conv, u, trace=True)
    from scipy.special import expit
    xv = 2.0 * expit(2.0)
    for j, dval in enumerate([0.5, -1.0]):
        c = dval * xv * 50.0
        sl = slice(j * 8, (j + 1) * 8)
        assert np.allclose(tr["v"][0, sl], c, rtol=1e-15, atol=0)
        ref = np.sign(c) * w["norm_w"][sl] * abs(c) / math.sqrt(c * c + dims.norm_eps)
        assert rel(tr["yn"][0, sl], ref) < 1e-15


def test_batch_sessions_are_independent_and_slots_permute():
    dims = SMALL_G2
    lay, _ = _layer(dims, seed=14)
    r = np.random.default_rng(15)
    ssm0 = r.standard_normal((3, 4, 8, 16)); conv0 = r.standard_normal((3, 3, dims.conv_dim))
    x = r.standard_normal((3, dims.d_model))
    ssm, conv = lay.new_state(3, ssm0, conv0)
    y = lay.step(ssm, conv, x)
    for b in range(3):
        s1, c1 = lay.new_state(1, ssm0[b:b + 1], conv0[b:b + 1])
        y1 = lay.step(s1, c1, x[b:b + 1])
        assert np.array_equal(y1[0], y[b])
        assert np.array_equal(s1[0], ssm[b])
    perm = np.array([2, 0, 1], np.int32)
    ssm_p, conv_p = lay.new_state(3, ssm0, conv0)
    # session b now lives in slot perm[b] and feeds the input that slot's session fed before
    yp = lay.step(ssm_p, conv_p, x[perm], slot_ids=perm)
    assert np.array_equal(yp, y[perm])
    assert np.array_equal(ssm_p, ssm) and np.array_equal(conv_p, conv)
    with pytest.raises(ValueError):
        lay.step(ssm_p, conv_p, x, slot_ids=np.array([0, 0, 1], np.int32))


def test_prefill_is_the_step_loop():
    dims = SMALL_G2
    lay, _ = _layer(dims, seed=16)
    x = np.random.default_rng(17).standard_normal((2, 9, dims.d_model))
    s1, c1 = lay.new_state(2)
    yp = lay.prefill(s1, c1, x)
    s2, c2 = lay.new_state(2)
    for t in range(9):
        yt = lay.step(s2, c2, x[:, t])
        assert np.array_equal(yp[:, t], yt)
    assert np.array_equal(s1, s2) and np.array_equal(c1, c2)


def test_tiny_workload_runs_and_stays_bounded():
    wl = synth.workload(0)
    lay, _ = _layer(wl.dims, seed=wl.weight_seed)
    ssm, conv = lay.new_state(wl.batch)
    xs = synth.make_inputs(wl.dims, wl.seed, wl.steps, wl.batch)
    for t in range(wl.steps):
        y = lay.step(ssm, conv, xs[t])
        assert np.all(np.isfinite(y)) and np.max(np.abs(y)) < 50


# ---- output heads: logits W h and the greedy token ----

def _head_decoded(wtype, w, s, q_group, gamma):
    """The head matrix as fp64 via the same numpy decoding as `decoded`."""
    dims = synth.TINY.replace(wtype=wtype, q_group=q_group or 1, q_gamma_in=gamma)
    return decoded(dims, {"w_in": w, "s_in": s}, "w_in")


@pytest.mark.parametrize("wtype,q_group,gamma", [("f32", 0, 1.0), ("bf16", 0, 1.0), ("int8g", 64, 0.5),
                                                 ("int4g", 32, 1.0), ("int3g", 64, 2.0)])
def test_head_logits_match_numpy_matmul_and_argmax(wtype, q_group, gamma):
    V, K, B = 333, 256, 3
    w, s = synth.make_head_weights(V, K, wtype, q_group, seed=7)
    h = synth.make_head_states(K, B, seed=8)
    logits, token = oracle.head_argmax(wtype, w, h, s, q_group, gamma)
    ref = h.astype(np.float64) @ _head_decoded(wtype, w, s, q_group, gamma).T
    assert rel(logits, ref) < RTOL
    assert np.array_equal(token, np.argmax(ref, axis=1))
    assert logits.shape == (B, V) and token.dtype == np.int32


def test_head_ties_take_the_lowest_index():
    rng = np.random.default_rng(3)
    V, K = 40, 32
    w = rng.standard_normal((V, K)).astype(np.float32)
    h = rng.standard_normal((2, K))
    w[[29, 11, 36]] = 10.0 * np.sign(h[0]).astype(np.float32)   # three equal rows, far above the rest
    _, token = oracle.head_argmax("f32", w, h)
    assert token[0] == 11
    w2 = np.zeros((V, K), np.float32)                            # every logit exactly 0
    _, token = oracle.head_argmax("f32", w2, h)
    assert np.array_equal(token, [0, 0])


def test_head_nan_is_never_chosen_and_infinities_order():
    rng = np.random.default_rng(4)
    V, K = 12, 16
    h = np.abs(rng.standard_normal((1, K))) + 0.5                # every entry positive
    w = rng.standard_normal((V, K)).astype(np.float32)
    w[2, 5] = np.nan                                             # NaN logit
    w[6, 0] = -np.inf                                            # -inf logit
    w[9, 3] = np.inf                                             # +inf logit: the maximum
    logits, token = oracle.head_argmax("f32", w, h)
    assert np.isnan(logits[0, 2]) and logits[0, 6] == -np.inf and logits[0, 9] == np.inf
    assert token[0] == 9
    w[9, 3] = 0.0
    _, token = oracle.head_argmax("f32", w, h)
    with np.errstate(invalid="ignore"):
        ref = h @ w.astype(np.float64).T                         # NaN and -inf carry through
    assert token[0] == int(np.nanargmax(ref[0])) and token[0] not in (2, 6)
    w[:] = -np.inf                                               # every logit -inf: the lowest index
    _, token = oracle.head_argmax("f32", w, h)
    assert token[0] == 0
    w[:] = np.nan                                                # every logit NaN: no token
    _, token = oracle.head_argmax("f32", w, h)
    assert token[0] == -1


def test_head_single_row_and_sessions_are_independent():
    w, _ = synth.make_head_weights(1, 64, "bf16", 0, seed=2)
    h = synth.make_head_states(64, 4, seed=3)
    logits, token = oracle.head_argmax("bf16", w, h)
    assert np.array_equal(token, [0, 0, 0, 0])
    w, _ = synth.make_head_weights(50, 64, "bf16", 0, seed=2)
    full, tok = oracle.head_argmax("bf16", w, h)
    for b in range(4):
        one, t1 = oracle.head_argmax("bf16", w, h[b])
        assert np.array_equal(one[0], full[b]) and t1[0] == tok[b]


# ---- attention decode step ----

def test_double_to_bf16_rounding_against_hand_values_and_the_generator():
    cases = {1.0: 0x3F80, 1 + 2 ** -8: 0x3F80, 1 + 3 * 2 ** -8: 0x3F82, -2.0: 0xC000, -0.0: 0x8000,
             2.0 ** -133: 0x0001, 2.0 ** -134: 0x0000, 3 * 2.0 ** -134: 0x0002, 3.3895e38: 0x7F7F,
             3.3962e38: 0x7F80, -1e39: 0xFF80, float("inf"): 0x7F80}
    for v, bits in cases.items():
        assert oracle.double_to_bf16(v) == bits, (v, hex(oracle.double_to_bf16(v)))
    assert oracle.double_to_bf16(float("nan")) == 0x7FC0
    vals = np.random.default_rng(5).standard_normal(4000).astype(np.float32) * np.float32(37.0)
    ref = synth.f32_to_bf16_bits(vals)
    assert all(oracle.double_to_bf16(float(v)) == int(r) for v, r in zip(vals, ref))


ATT = synth.AttnDims(d_model=64, n_q=6, n_kv=2, head_dim=16, max_len=12, wtype="f32")


def _attn(dims, pos, seed=3, w=None, slots=None):
    w = w if w is not None else synth.make_attn_weights(dims, seed)
    kc, vc = synth.make_kv_cache(dims, seed + 1, pos)
    return oracle.AttnLayer(dims, w), w, kc, vc, np.array(pos, np.int32)


def _bf(bits):
    return (np.asarray(bits, np.uint16).astype(np.uint32) << 16).view(np.float32).astype(np.float64)


@pytest.mark.parametrize("wtype,q_group,gamma", [("f32", 16, 1.0), ("bf16", 16, 1.0), ("int8g", 16, 0.25),
                                                 ("int4g", 32, 1.0), ("int3g", 32, 0.5)])
def test_attn_projections_match_numpy_matmul(wtype, q_group, gamma):
    d = ATT.replace(d_model=128, head_dim=32, wtype=wtype, q_group=q_group, q_gamma_qkv=gamma, q_gamma_o=gamma)
    lay, w, kc, vc, pos = _attn(d, [5, 0, 11])
    x = np.random.default_rng(2).standard_normal((3, d.d_model))
    y, tr = lay.step(kc, vc, pos, x, trace=True)
    dims = synth.TINY.replace(wtype=wtype, q_group=q_group, q_gamma_in=gamma, q_gamma_out=gamma)
    Wqkv = decoded(dims, {"w_in": w["w_qkv"], "s_in": w["s_qkv"]}, "w_in")
    Wo = decoded(dims, {"w_out": w["w_o"], "s_out": w["s_o"]}, "w_out")
    assert rel(tr["qkv"], x @ Wqkv.T) < RTOL
    assert rel(y, tr["o"] @ Wo.T) < RTOL


def test_attn_first_position_returns_the_rounded_new_value():
    lay, w, kc, vc, pos = _attn(ATT, [0, 0])
    x = np.random.default_rng(4).standard_normal((2, ATT.d_model))
    _, tr = lay.step(kc, vc, pos, x, trace=True)
    D, Hq, Hk = ATT.head_dim, ATT.n_q, ATT.n_kv
    for b in range(2):
        v_new = tr["qkv"][b, (Hq + Hk) * D:]
        k_new = tr["qkv"][b, Hq * D:(Hq + Hk) * D]
        for h in range(Hq):
            g = h // (Hq // Hk)
            expect = _bf(synth.f32_to_bf16_bits(v_new[g * D:(g + 1) * D].astype(np.float32)))
            assert np.array_equal(tr["o"][b, h * D:(h + 1) * D], expect)
        assert np.array_equal(_bf(kc[b, :, 0, :]).ravel(), _bf(synth.f32_to_bf16_bits(k_new.astype(np.float32))))
    assert np.array_equal(pos, [1, 1])


def test_attn_zero_queries_average_every_value_up_to_the_new_one():
    w = synth.make_attn_weights(ATT, 3)
    w["w_qkv"] = w["w_qkv"].copy()
    w["w_qkv"][:ATT.n_q * ATT.head_dim] = 0.0                  # q = 0: all scores 0
    lay, _, kc, vc, pos = _attn(ATT, [7, 3, 11], w=w)
    x = np.random.default_rng(6).standard_normal((3, ATT.d_model))
    _, tr = lay.step(kc, vc, pos, x, trace=True)
    D, Hq, Hk = ATT.head_dim, ATT.n_q, ATT.n_kv
    for b, t in enumerate([7, 3, 11]):
        for h in range(Hq):
            g = h // (Hq // Hk)
            V = _bf(vc[b, g, :t + 1, :])                        # includes the entry just written
            assert rel(tr["o"][b, h * D:(h + 1) * D], V.mean(axis=0)) < RTOL


def test_attn_dominant_key_selects_its_value():
    d = ATT.replace(n_q=2, n_kv=2)                               # one query head per key head
    lay, w, kc, vc, pos = _attn(d, [9])
    x = np.random.default_rng(7).standard_normal((1, d.d_model))
    q = x @ np.asarray(w["w_qkv"], np.float64)[:d.n_q * d.head_dim].T
    D = d.head_dim
    for g, j in ((0, 4), (1, 0)):
        qg = q[0, g * D:(g + 1) * D]
        kc[0, g, j] = synth.f32_to_bf16_bits((60.0 * qg / np.linalg.norm(qg)).astype(np.float32))
    _, tr = lay.step(kc, vc, pos, x, trace=True)
    for g, j in ((0, 4), (1, 0)):
        assert rel(tr["o"][0, g * D:(g + 1) * D], _bf(vc[0, g, j])) < 1e-9


def test_attn_is_invariant_to_permuting_cached_positions_and_shares_kv_within_a_group():
    w = synth.make_attn_weights(ATT, 8)
    w["w_qkv"] = w["w_qkv"].copy()
    D = ATT.head_dim
    w["w_qkv"][1 * D:2 * D] = w["w_qkv"][0:D]                    # heads 0 and 1 (group 0): same q
    w["w_qkv"][3 * D:4 * D] = w["w_qkv"][0:D]                    # head 3 (group 1): same q, other K/V
    lay, _, kc, vc, pos = _attn(ATT, [10], w=w)
    x = np.random.default_rng(9).standard_normal((1, ATT.d_model))
    perm = np.random.default_rng(10).permutation(10)
    kc2, vc2, pos2 = kc.copy(), vc.copy(), pos.copy()
    kc2[0, :, :10] = kc[0][:, perm]
    vc2[0, :, :10] = vc[0][:, perm]
    _, t1 = lay.step(kc, vc, pos, x, trace=True)
    _, t2 = lay.step(kc2, vc2, pos2, x, trace=True)
    assert rel(t2["o"], t1["o"]) < 1e-13
    o = t1["o"][0]
    assert np.array_equal(o[0:D], o[D:2 * D])
    assert rel(o[3 * D:4 * D], o[0:D]) > 1e-3


def test_attn_two_positions_is_a_logistic_mix():
    from scipy.special import expit
    lay, w, kc, vc, pos = _attn(ATT, [1])
    x = np.random.default_rng(11).standard_normal((1, ATT.d_model))
    _, tr = lay.step(kc, vc, pos, x, trace=True)
    D = ATT.head_dim
    for h in range(ATT.n_q):
        g = h // (ATT.n_q // ATT.n_kv)
        q = tr["qkv"][0, h * D:(h + 1) * D]
        s0, s1 = (_bf(kc[0, g, j]) @ q / math.sqrt(D) for j in (0, 1))
        expect = expit(s0 - s1) * _bf(vc[0, g, 0]) + expit(s1 - s0) * _bf(vc[0, g, 1])
        assert rel(tr["o"][0, h * D:(h + 1) * D], expect) < 1e-12


def test_attn_residual_full_cache_and_bad_slots():
    lay, w, kc, vc, pos = _attn(ATT, [4, ATT.max_len, 2])
    x = np.random.default_rng(12).standard_normal((4, ATT.d_model))
    k0, v0 = kc.copy(), vc.copy()
    y = lay.step(kc, vc, pos, x, slot_ids=[0, 1, 7, 2], residual=True)
    assert np.all(np.isnan(y[1])) and np.all(np.isnan(y[2]))        # full cache, slot out of range
    assert np.array_equal(pos, [5, ATT.max_len, 3])
    assert np.array_equal(kc[1], k0[1]) and np.array_equal(vc[1], v0[1])
    changed = np.argwhere(kc != k0)
    assert set(map(tuple, changed[:, [0, 2]])) <= {(0, 4), (2, 2)}
    lay2, _, kc2, vc2, pos2 = _attn(ATT, [4, ATT.max_len, 2])
    y2 = lay2.step(kc2, vc2, pos2, x[[0, 3]], slot_ids=[0, 2])
    assert rel(y[[0, 3]] - x[[0, 3]], y2) < 1e-13


# ---------------------------------------------------------------- the hybrid stack

def _stack_parts(seed):
    """An M-A-M chain on d_model 64: two mixers with their own weights and states, one
    attention layer with its cache; 3 session slots, random states and caches."""
    r = np.random.default_rng(seed)
    m0, _ = _layer(SMALL_G2, seed=seed)
    m2_, _ = _layer(SMALL_G2, seed=seed + 1)
    att = oracle.AttnLayer(ATT, synth.make_attn_weights(ATT, seed + 2))
    st0 = m0.new_state(3, r.standard_normal((3, 4, 8, 16)), r.standard_normal((3, 3, SMALL_G2.conv_dim)))
    st2 = m2_.new_state(3, r.standard_normal((3, 4, 8, 16)), r.standard_normal((3, 3, SMALL_G2.conv_dim)))
    kc, vc = synth.make_kv_cache(ATT, seed + 3, np.array([3, 0, 7], np.int32))
    return [(m0, st0), (att, (kc, vc, np.array([3, 0, 7], np.int32))), (m2_, st2)]


def _copy_parts(parts):
    return [(lay, tuple(a.copy() for a in st)) for lay, st in parts]


def test_stack_step_is_the_residual_chain_of_its_layers():
    """oracle.stack_step against the chain written out: u1 = x + M0(x), u2 = u1 + A(u1),
    y = u2 + M2(u2), each layer called on its own without the residual flag. The layers
    differ, so a dropped residual or a permuted order gives another result (checked)."""
    x = np.random.default_rng(40).standard_normal((3, SMALL_G2.d_model))
    slots = np.array([1, 2, 0], np.int32)
    parts = _stack_parts(41)
    ref = _copy_parts(parts)
    (m0, s0), (att, sa), (m2_, s2) = ref
    u1 = x + m0.step(s0[0], s0[1], x, slot_ids=slots)
    u2 = u1 + att.step(sa[0], sa[1], sa[2], u1, slot_ids=slots)
    y_ref = u2 + m2_.step(s2[0], s2[1], u2, slot_ids=slots)
    got = _copy_parts(parts)
    y = oracle.stack_step(got, x, slot_ids=slots)
    assert rel(y, y_ref) < 1e-14
    for (_, a), (_, b) in zip(got, ref):            # every layer's state advanced the same way
        for u, v in zip(a, b):
            assert np.array_equal(u, v)
    # the same layers without residuals, or in another order, give something else
    alt = _copy_parts(parts)
    (n0, t0), (nat, ta), (n2, t2) = alt
    v = n0.step(t0[0], t0[1], x, slot_ids=slots)
    v = nat.step(ta[0], ta[1], ta[2], v, slot_ids=slots)
    v = n2.step(t2[0], t2[1], v, slot_ids=slots)
    assert rel(v, y_ref) > 1e-2
    rev = _copy_parts(parts)
    assert rel(oracle.stack_step(rev[::-1], x, slot_ids=slots), y_ref) > 1e-2


def test_stack_step_follows_the_slot_ids():
    """Session b on slot perm[b] through every layer: permuting the sessions' inputs and
    slot ids together permutes the outputs and leaves every state and cache the same."""
    x = np.random.default_rng(42).standard_normal((3, SMALL_G2.d_model))
    parts = _stack_parts(43)
    a = _copy_parts(parts)
    ya = oracle.stack_step(a, x)                     # identity slots
    perm = np.array([2, 0, 1], np.int32)
    b = _copy_parts(parts)
    yb = oracle.stack_step(b, x[perm], slot_ids=perm)
    assert np.array_equal(yb, ya[perm])
    for (_, u), (_, v) in zip(a, b):
        for p, q in zip(u, v):
            assert np.array_equal(p, q)
    # a slot id forwarded to one layer only (the others on identity) breaks the equality
    c = _copy_parts(parts)
    (m0, s0), (att, sa), (m2_, s2) = c
    u = x[perm] + m0.step(s0[0], s0[1], x[perm], slot_ids=perm)
    u = u + att.step(sa[0], sa[1], sa[2], u)
    u = u + m2_.step(s2[0], s2[1], u, slot_ids=perm)
    assert rel(u, ya[perm]) > 1e-2
