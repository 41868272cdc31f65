"""GPU parity through strided views.  The boundary takes every tensor with its
element strides (innermost dimension contiguous), so a caller passes the
views its own layers produce: the x and z halves of one in_proj output, B and
C sliced out of an x_proj output, a state cache whose rows are padded, output
written into a slice of a larger buffer.  Each case runs the HIP path on the
views and the float64 oracle on dense copies of the same values, to the
bar of tests/_parity.py; bytes outside the views must not change.
"""
import numpy as np
import pytest
import torch

import workloads as W
from tests._parity import RTOL, check, to_f64 as f

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import state_space_model_causal_amd as ssm

    ssm.load_library()
    return torch.device("cuda:0")


@pytest.fixture(scope="module")
def ssm():
    import state_space_model_causal_amd as m

    return m


def embed(t, dim, before, after, fill=3.0):
    """t placed inside a buffer that is larger along `dim` (before / after
    extra entries): returns (buffer, view of t's place in it)."""
    shape = list(t.shape)
    shape[dim] += before + after
    buf = torch.full(shape, fill, dtype=t.dtype, device=t.device)
    view = buf.narrow(dim, before, t.shape[dim])
    view.copy_(t)
    return buf, view


SCAN_CASES = [
    # (label, spec kwargs, chunked form)
    ("m1_f16_L256", dict(io="f16", seqlen=256, nheads=48, batch=2, index_sensitive=True), False),
    ("m1_f16_L300", dict(io="f16", seqlen=300, nheads=40, batch=2, index_sensitive=True), False),
    ("m1_f32_L96", dict(io="f32", seqlen=96, nheads=20, batch=3, index_sensitive=True), False),
    ("m2_bf16_chunked", dict(io="bf16", state="f32", seqlen=192, nheads=2, headdim=64, dstate=128,
                             a_per_state=False, index_sensitive=True, batch=2), True),
    ("m2_bf16_recurrent", dict(io="bf16", state="bf16", seqlen=136, nheads=4, headdim=8, dstate=32,
                               ngroups=2, a_per_state=False, index_sensitive=True, batch=2), False),
]


@pytest.mark.parametrize("label,kw,chunked", SCAN_CASES, ids=[c[0] for c in SCAN_CASES])
def test_scan_on_projection_views(dev, ssm, oracle, label, kw, chunked):
    """u and z are the two halves of one [batch, 2*channels, seqlen]
    projection output; B and C are slices of one [batch, ngroups, 2*dstate
    + 8, seqlen] buffer; out is written into the middle of a wider buffer;
    the final state goes to a cache whose slots are padded."""
    spec = W.tiny(nslots=5, random_slots=True, **kw)
    t = W.make(spec, dev)
    Bt, Cn, L, N, G = spec.batch, spec.channels, spec.seqlen, spec.dstate, spec.ngroups
    xz = torch.cat([t["x"], t["z"]], dim=1)           # [Bt, 2 Cn, L]
    u, z = xz[:, :Cn], xz[:, Cn:]
    bc = torch.cat([t["B"], t["C"], torch.zeros_like(t["B"][:, :, :8])], dim=2)
    Bv, Cv = bc[:, :, :N], bc[:, :, N:2 * N]
    obuf = torch.full((Bt, Cn + 24, L), 5.0, dtype=t["x"].dtype, device=dev)
    out = obuf[:, 8:8 + Cn]
    sbuf, state = embed(t["ssm_state"], 3, 0, 8)       # [S, H, P, N + 8]
    state0 = state.clone()
    ssm.selective_scan(u, t["dt"], t["A"], Bv, Cv, D=t["D"], z=z, dt_bias=t["dt_bias"],
                       ssm_state=state, slot_idx=t["slot_idx"], has_initial_state=True, out=out,
                       algo=ssm.SCAN_CHUNKED if chunked else None)
    torch.cuda.synchronize()
    o, s, st, sts = oracle.selective_scan(f(u), f(t["dt"]), f(t["A"]), f(Bv), f(Cv), D=f(t["D"]),
                                          z=f(z), dt_bias=f(t["dt_bias"]), state=f(state0),
                                          slot_idx=t["slot_idx"].cpu().numpy(), has_initial_state=True)
    check(out, o, s, RTOL[spec.io], spec.io, f"strided scan {label} out")
    idx = t["slot_idx"].cpu().numpy()
    check(state[idx], st[idx], sts[idx], RTOL[spec.io], spec.state, f"strided scan {label} state")
    # nothing outside the views moved: the output buffer's margins and the
    # state rows' padding, and the slots not named
    assert torch.all(obuf[:, :8] == 5.0) and torch.all(obuf[:, 8 + Cn:] == 5.0)
    assert torch.all(sbuf[..., N:] == 3.0)
    others = np.setdiff1d(np.arange(spec.slots), idx)
    np.testing.assert_array_equal(f(state[others]), f(state0[others]))


CONV_CASES = [
    ("f16_L256", dict(io="f16", seqlen=256, nheads=40, batch=3, nslots=5, random_slots=True)),
    ("bf16_L77", dict(io="bf16", seqlen=77, nheads=24, batch=2, nslots=4, random_slots=True)),
    ("f16_L1_decode", dict(io="f16", seqlen=1, nheads=64, batch=6, nslots=9, random_slots=True)),
]


@pytest.mark.parametrize("label,kw", CONV_CASES, ids=[c[0] for c in CONV_CASES])
def test_conv1d_on_projection_views(dev, ssm, oracle, label, kw):
    """x is the first half of a [batch, 2*channels, seqlen] projection output,
    the output goes into a slice of a wider buffer, the conv cache rows are
    padded ([nslots, channels, width] with width-1 used) and the taps come
    from a padded weight matrix."""
    spec = W.tiny(**kw)
    t = W.make(spec, dev)
    Bt, Cn, L = spec.batch, spec.channels, spec.seqlen
    x3 = t["x"].view(Bt, Cn, L)
    xz = torch.cat([x3, torch.zeros_like(x3)], dim=1)
    x = xz[:, :Cn]
    obuf = torch.full((Bt, Cn + 16, L), 5.0, dtype=x3.dtype, device=dev)
    out = obuf[:, 16:]
    cbuf, cs = embed(t["conv_state"], 2, 0, 1)          # [S, Cn, 4], 3 used
    wbuf, w = embed(t["conv_w"], 1, 0, 4)               # [Cn, 8], 4 used
    cs0 = cs.clone()
    ssm.causal_conv1d(x, w, t["conv_b"], conv_state=cs, slot_idx=t["slot_idx"], out=out,
                      has_initial_state=True)
    torch.cuda.synchronize()
    idx = t["slot_idx"].cpu().numpy()
    o, s, cs_o = oracle.causal_conv1d(f(x), f(w), f(t["conv_b"]), f(cs0), idx, has_initial_state=True)
    check(out, o, s, RTOL[spec.io], spec.io, f"strided conv {label} out")
    np.testing.assert_array_equal(f(cs), cs_o)
    assert torch.all(obuf[:, :16] == 5.0)
    assert torch.all(cbuf[..., 3:] == 3.0)


SSU_CASES = [
    # (label, spec kwargs, state row padding): padded rows take the blocked
    # lane map; dense rows with padded slots at >= 2^18 rows the interleaved one
    ("m2_f16_hd64_pad_rows", dict(batch=6, nslots=9, random_slots=True, nheads=8, headdim=64,
                                  dstate=128, io="f16", state="f16", a_per_state=False,
                                  index_sensitive=True, ngroups=2), (0, 8)),
    ("m1_f32_ilv_pad_slots", dict(batch=64, nslots=70, random_slots=True, nheads=4096, headdim=1,
                                  dstate=16, io="f16", state="f32", index_sensitive=True), (64, 0)),
    ("m2_bf16_hd128_pad_slots", dict(batch=3, nslots=4, random_slots=True, nheads=4, headdim=128,
                                     dstate=256, io="bf16", state="bf16", a_per_state=False,
                                     index_sensitive=True), (256, 0)),
]


@pytest.mark.parametrize("label,kw,pad", SSU_CASES, ids=[c[0] for c in SSU_CASES])
def test_state_update_on_views(dev, ssm, oracle, label, kw, pad):
    """x and z are the halves of one [batch, 2*nheads*headdim] projection
    output viewed per head, dt and B/C are slices of one x_proj-like row,
    out goes into a wider buffer; the state cache has padded slots and/or
    padded rows."""
    spec = W.decode(seqlen=1, width=0, has_initial_state=True, seed=17, **kw)
    t = W.make(spec, dev)
    Bt, H, P, N, G = spec.batch, spec.nheads, spec.headdim, spec.dstate, spec.ngroups
    HP = H * P
    xz = torch.cat([t["x"].reshape(Bt, HP), t["z"].reshape(Bt, HP)], dim=1)
    x, z = xz[:, :HP].view(Bt, H, P), xz[:, HP:].view(Bt, H, P)
    row = torch.cat([t["dt"], t["B"].reshape(Bt, G * N), t["C"].reshape(Bt, G * N)], dim=1)
    dt = row[:, :H]
    Bv = row[:, H:H + G * N].view(Bt, G, N)
    Cv = row[:, H + G * N:].view(Bt, G, N)
    obuf = torch.full((Bt, HP + 64), 5.0, dtype=t["x"].dtype, device=dev)
    out = obuf[:, 32:32 + HP].view(Bt, H, P)
    slot_pad, row_pad = pad
    S = spec.slots
    st = t["ssm_state"]
    big = torch.full((S, HP * (N + row_pad) + slot_pad), 3.0, dtype=st.dtype, device=dev)
    state = big[:, :HP * (N + row_pad)].view(S, H, P, N + row_pad)[..., :N]
    state.copy_(st)
    state0 = state.clone()
    ssm.state_update(state, x, dt, t["A"], Bv, Cv, D=t["D"], z=z, dt_bias=t["dt_bias"],
                     slot_idx=t["slot_idx"], out=out)
    torch.cuda.synchronize()
    idx = t["slot_idx"].cpu().numpy()
    o, s, so, sso = oracle.state_update(f(state0), f(x), f(dt), f(t["A"]), f(Bv), f(Cv), D=f(t["D"]),
                                        z=f(z), dt_bias=f(t["dt_bias"]), slot_idx=idx)
    check(out, o, s, RTOL[spec.io], spec.io, f"strided ssu {label} out")
    check(state[idx], so[idx], sso[idx], RTOL[spec.io], spec.state, f"strided ssu {label} state")
    assert torch.all(obuf[:, :32] == 5.0) and torch.all(obuf[:, 32 + HP:] == 5.0)
    pads = torch.ones_like(big, dtype=torch.bool)
    pads[:, :HP * (N + row_pad)].view(S, H, P, N + row_pad)[..., :N] = False
    assert torch.all(big[pads] == 3.0)
    others = np.setdiff1d(np.arange(S), idx)
    np.testing.assert_array_equal(f(state[others]), f(state0[others]))


@pytest.mark.parametrize("batch,H", [(5, 256), (64, 4096)], ids=["blocked", "interleaved"])
def test_decode_step_on_views(dev, ssm, oracle, batch, H):
    """The fused decode step with x and z halves of one projection output,
    a conv cache of padded rows and a state cache of padded slots."""
    spec = W.decode(batch=batch, nslots=batch + 4, nheads=H, seed=23, index_sensitive=True)
    t = W.make(spec, dev)
    Bt, N = spec.batch, spec.dstate
    xz = torch.cat([t["x"].reshape(Bt, H), t["z"].reshape(Bt, H)], dim=1)
    x, z = xz[:, :H].view(Bt, H, 1), xz[:, H:].view(Bt, H, 1)
    cbuf, cs = embed(t["conv_state"], 2, 0, 1)                   # [S, Cn, 4], 3 used
    sbig = torch.full((spec.slots, H * N + 32), 3.0, dtype=t["ssm_state"].dtype, device=dev)
    state = sbig[:, :H * N].view(spec.slots, H, 1, N)
    state.copy_(t["ssm_state"])
    cs0, st0 = cs.clone(), state.clone()
    u_out = torch.empty((Bt, H, 1), dtype=x.dtype, device=dev)
    out = ssm.decode_step(state, cs, x, t["conv_w"], t["dt"], t["A"], t["B"], t["C"],
                          conv_bias=t["conv_b"], D=t["D"], z=z, dt_bias=t["dt_bias"],
                          slot_idx=t["slot_idx"], u_out=u_out)
    torch.cuda.synchronize()
    idx = t["slot_idx"].cpu().numpy()
    uo, uso, cso = oracle.causal_conv1d(f(x).reshape(Bt, H, 1), f(t["conv_w"]), f(t["conv_b"]),
                                        f(cs0), idx, has_initial_state=True)
    np.testing.assert_array_equal(f(cs), cso)
    check(u_out, uo, uso, 3e-3, "f16", "strided decode step u")
    # the fused step hands the float32 conv output to the update; its scales
    # take the conv's term magnitude in place of |u| (as for the dense step)
    args = (f(t["dt"]), f(t["A"]), f(t["B"]), f(t["C"]))
    kw = dict(D=f(t["D"]), z=f(z), dt_bias=f(t["dt_bias"]), slot_idx=idx)
    o, _, so, _ = oracle.state_update(f(st0), uo, *args, **kw)
    _, os_, _, sos = oracle.state_update(f(st0), uso, *args, **kw)
    check(out, o, os_, 3e-3, "f16", "strided decode step out")
    check(state[idx], so[idx], sos[idx], 3e-3, "f32", "strided decode step state")
    assert torch.all(cbuf[..., 3:] == 3.0)
    assert torch.all(sbig[:, H * N:] == 3.0)
