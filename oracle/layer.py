"""Float64 oracle of one Mamba-1 decode layer and its two building blocks
(linear projection, RMSNorm).

TEST INFRASTRUCTURE ONLY, like the rest of oracle/: used by tests/ and never
by the product package; it shares no code with the HIP path.  numpy float64
throughout; the conv and the state update are the C oracle's
(oracle.causal_conv1d, oracle.state_update).

The layer is the one the Mamba-2.8B model of "feat(llama.cu): 适配 mamba 模型"
(InfiniLM-Rust PR #48, sections 2.1-2.2) runs around its conv and scan
operators.  The pages name the model and those operators but do not write the
layer out; it is taken as the standard Mamba-1 residual block:
    hn = rmsnorm(hidden) ; x|z = hn in_proj^T ; u = silu(conv(x)) ;
    dt_low|B|C = u x_proj^T ; dt = dt_low dt_proj^T ;
    y = state_update(u, dt, A, B, C, D, z, dt_bias, softplus) ;
    hidden + y out_proj^T
Each function returns the result and a magnitude ("scale") of the same shape
that bounds the terms a float32 implementation rounds (see tests/_parity.py).
"""
from __future__ import annotations

import numpy as np

from . import causal_conv1d, round_to, state_update


def linear(x, weight, residual=None):
    """out = x . weight^T (+ residual), x [M, K], weight [N, K]: the plain
    definition of a linear projection.  Scale: |x| . |weight|^T (+|residual|)."""
    x = np.asarray(x, dtype=np.float64)
    w = np.asarray(weight, dtype=np.float64)
    out = x @ w.T
    scale = np.abs(x) @ np.abs(w).T
    if residual is not None:
        r = np.asarray(residual, dtype=np.float64)
        out = out + r
        scale = scale + np.abs(r)
    return out, scale


def rmsnorm(x, weight, eps):
    """out[m] = x[m] / sqrt(mean(x[m]^2) + eps) * weight (root-mean-square
    normalisation of each row).  Scale: |out|."""
    x = np.asarray(x, dtype=np.float64)
    w = np.asarray(weight, dtype=np.float64)
    inv = 1.0 / np.sqrt(np.mean(x * x, axis=-1, keepdims=True) + eps)
    out = x * inv * w
    return out, np.abs(out)


def mamba1_decode_layer(w: dict, hidden, conv_state, ssm_state, slot_idx=None, eps=1e-5,
                        round_kind=None, stages=None):
    """One decode token per request through the layer.  w: float64 arrays
    (norm_weight, in_proj, conv_weight, conv_bias, x_proj, dt_proj, dt_bias,
    A, D, out_proj); hidden [batch, d_model]; conv_state [S, d_inner, W-1];
    ssm_state [S, d_inner, 1, d_state].  round_kind (F16/BF16) rounds every
    intermediate that a stored implementation keeps in that dtype (the
    layer's io dtype), None keeps float64 throughout.  stages, if a dict,
    receives each intermediate.  Returns (hidden_out, scale, conv_state,
    ssm_state, ssm_state_scale)."""
    rnd = (lambda a: round_to(a, round_kind)) if round_kind is not None else (lambda a: a)
    hidden = np.asarray(hidden, dtype=np.float64)
    batch = hidden.shape[0]
    d_inner = w["in_proj"].shape[0] // 2
    d_state = w["A"].shape[1]
    R = w["dt_proj"].shape[1]
    st = {} if stages is None else stages
    st["hn"] = rnd(rmsnorm(hidden, w["norm_weight"], eps)[0])
    xz = linear(st["hn"], w["in_proj"])[0]
    st["x"], st["z"] = rnd(xz[:, :d_inner]), rnd(xz[:, d_inner:])
    u, _, cs = causal_conv1d(st["x"][:, :, None], w["conv_weight"], w.get("conv_bias"), conv_state,
                             slot_idx, has_initial_state=True, apply_silu=True)
    st["u"] = rnd(u[:, :, 0])
    dbc = linear(st["u"], w["x_proj"])[0]
    st["dt_low"] = rnd(dbc[:, :R])
    st["B"], st["C"] = rnd(dbc[:, R:R + d_state]), rnd(dbc[:, R + d_state:])
    st["dt"] = rnd(linear(st["dt_low"], w["dt_proj"])[0])
    y, ys, ss, sss = state_update(ssm_state, st["u"][:, :, None], st["dt"], w["A"],
                                  st["B"][:, None, :], st["C"][:, None, :], D=w.get("D"),
                                  z=st["z"][:, :, None], dt_bias=w.get("dt_bias"),
                                  slot_idx=slot_idx)
    st["y"] = rnd(y[:, :, 0])
    out, scale = linear(st["y"], w["out_proj"], residual=hidden)
    if slot_idx is not None:
        pad = np.asarray(slot_idx) < 0
        out[pad] = hidden[pad]
        scale[pad] = 0.0
    return out, scale, cs, ss, sss
