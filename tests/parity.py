"""Shared helpers of the parity tests: run the HIP path and the oracle on the same
seeded inputs and measure the normwise errors.

Error measures (fp32 accumulate on the GPU, fp64 in the oracle):
  e_out   = max over tokens and sessions of  max_i |y_i - yo_i| / max_i |yo_i|
  e_state = max over sessions and heads of   max_{p,n} |S - So| / max(max_{p,n} |So|, 1e-6 max_all |So|)
  e_conv  = max over sessions of             max |c - co| / max(max |co|, 1e-30)
Bars: e_out <= 2e-3, e_state <= 1e-3 (and e_conv <= 1e-3).
"""
from __future__ import annotations

import numpy as np

TOL_OUT = 2e-3
TOL_STATE = 1e-3


def e_out(y, yo):
    y = np.asarray(y, np.float64)
    yo = np.asarray(yo, np.float64)
    d = np.max(np.abs(y - yo), axis=-1)
    m = np.max(np.abs(yo), axis=-1)
    if np.any(~np.isfinite(y)):
        return float("inf")
    return float(np.max(d / np.maximum(m, 1e-30)))


def e_state(S, So):
    S = np.asarray(S, np.float64)
    So = np.asarray(So, np.float64)
    if np.any(~np.isfinite(S)):
        return float("inf")
    floor = 1e-6 * max(float(np.max(np.abs(So))), 1e-30)
    d = np.max(np.abs(S - So), axis=(-2, -1))
    m = np.maximum(np.max(np.abs(So), axis=(-2, -1)), floor)
    return float(np.max(d / m))


def e_conv(c, co):
    c = np.asarray(c, np.float64)
    co = np.asarray(co, np.float64)
    if np.any(~np.isfinite(c)):
        return float("inf")
    axes = tuple(range(1, c.ndim))
    d = np.max(np.abs(c - co), axis=axes)
    m = np.maximum(np.max(np.abs(co), axis=axes), 1e-30)
    return float(np.max(d / m))


def oracle_decode(dims, weights, xs, ssm0, conv0, slot_ids=None, residual=False, sessions=None):
    """Run the oracle for xs [steps][B][d_model]; sessions selects a subset (independent sessions)."""
    import oracle
    lay = oracle.Layer(dims, weights)
    if sessions is not None:
        xs = xs[:, sessions]
        sl = None if slot_ids is None else np.asarray(slot_ids)[sessions]
    else:
        sl = slot_ids
    ssm, conv = lay.new_state(ssm0.shape[0], ssm0, conv0)
    ys = np.empty(xs.shape, np.float64)
    if sessions is not None and sl is None:
        sl = np.asarray(sessions, np.int32)
    for t in range(xs.shape[0]):
        ys[t] = lay.step(ssm, conv, xs[t], slot_ids=sl, residual=residual)
    return ys, ssm, conv


def gpu_decode(dims, weights, xs, ssm0, conv0, slot_ids=None, residual=False, graph=False, persistent=False,
               panels=True):
    """Run m2_step over xs [steps][B][d_model] on cuda:0; returns numpy ys, ssm, conv
    (persistent: plan 2, the persistent SSD + out_proj kernel, where it applies; panels:
    the layer holds the 16-row panel copies the batched GEMVs read)."""
    import torch
    from full_duplex_speech_mamba2_amd import m2
    lay = m2.Layer(dims, weights, panels=panels)
    st = m2.State(lay, ssm0.shape[0], torch.from_numpy(np.ascontiguousarray(ssm0, np.float32)).cuda(),
                  torch.from_numpy(np.ascontiguousarray(conv0, np.float32)).cuda())
    xd = torch.from_numpy(np.ascontiguousarray(xs, np.float32)).cuda()
    yd = torch.empty_like(xd)
    sl = None if slot_ids is None else torch.from_numpy(np.asarray(slot_ids, np.int32)).cuda()
    for t in range(xs.shape[0]):
        m2.step(lay, st, xd[t], yd[t], slot_ids=sl, residual=residual, persistent=persistent)
    torch.cuda.synchronize()
    return yd.cpu().numpy(), st.ssm.cpu().numpy(), st.conv.cpu().numpy()
