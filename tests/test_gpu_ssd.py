"""GPU parity of the chunked (matrix-core) Mamba-2 prefill against the float64
oracle's recurrence, and against the step-by-step kernel on the same inputs.

The chunked form applies to one decay per head, f16 or bf16 I/O, dstate
64/128/256, headdim a multiple of 64 and seqlen a multiple of 8.  Cases span
one chunk and many, a ragged last chunk (seqlen not a multiple of 64), several
workgroups per head (headdim 128), groups, initial states in every cache
dtype, padded requests and the optional arguments, each with both I/O types;
with f16 I/O also a carried state beyond f16's range and values far below 1
(the f16 parts of the state and the weighted u are taken under per-row
power-of-two scales).  Tolerance: the 16-bit I/O bar of tests/_parity.py
(3e-3 of the magnitude scale plus half an ulp).
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


SSD_CASES = [
    # (label, spec kwargs, options)
    ("N64_L8", dict(seqlen=8, nheads=2, headdim=64, dstate=64), {}),
    ("N64_L64", dict(seqlen=64, nheads=2, headdim=64, dstate=64, batch=2), dict(init=True)),
    ("N128_L200_G2", dict(seqlen=200, nheads=4, headdim=64, dstate=128, ngroups=2, batch=2,
                          nslots=5, random_slots=True), dict(init=True, pad=2)),
    ("N256_P128_L520", dict(seqlen=520, nheads=2, headdim=128, dstate=256, state="bf16",
                            nslots=3, random_slots=True), dict(init=True)),
    ("N256_L1024_f16state", dict(seqlen=1024, nheads=1, headdim=64, dstate=256, state="f16"),
     dict(init=True)),
    ("N128_noz_noD_nobias", dict(seqlen=136, nheads=2, headdim=64, dstate=128),
     dict(z=False, D=False, bias=False)),
    ("N64_no_softplus", dict(seqlen=96, nheads=2, headdim=64, dstate=64), dict(softplus=False)),
    ("N256_G4_L2048", dict(seqlen=2048, nheads=4, headdim=64, dstate=256, ngroups=4), {}),
    # magnitudes: a carried state of up to ~10^5 (its f16 parts need the
    # scale) with u x 100 and C x 10^-2 (so that the outputs stay within
    # f16); then values around 10^-3 and a state around 10^-6
    ("N128_large_state", dict(seqlen=256, nheads=2, headdim=64, dstate=128),
     dict(init=True, state_scale=3e4, x_scale=100.0, c_scale=1e-2)),
    ("N64_small_values", dict(seqlen=128, nheads=2, headdim=64, dstate=64),
     dict(init=True, state_scale=1e-6, x_scale=1e-3)),
]


def _run(ssm, oracle, dev, spec, opts, label, algo):
    t = W.make(spec, dev)
    if not opts.get("softplus", True):
        t["dt"].abs_().add_(0.01)
    if opts.get("state_scale"):
        t["ssm_state"].mul_(opts["state_scale"])
    if opts.get("x_scale"):
        t["x"].mul_(opts["x_scale"])
    if opts.get("c_scale"):
        t["C"].mul_(opts["c_scale"])
    u = t["x"]
    z = t["z"] if opts.get("z", True) else None
    D = t["D"] if opts.get("D", True) else None
    bias = t["dt_bias"] if opts.get("bias", True) and opts.get("softplus", True) else None
    sp = opts.get("softplus", True)
    init = opts.get("init", False)
    idx = t["slot_idx"].clone()
    if opts.get("pad"):
        idx[::opts["pad"]] = -1
    st0 = t["ssm_state"].clone()
    out0 = torch.full_like(u, 5.0)
    out = ssm.selective_scan(u, t["dt"], t["A"], t["B"], t["C"], D=D, z=z, dt_bias=bias,
                             dt_softplus=sp, ssm_state=t["ssm_state"], slot_idx=idx,
                             has_initial_state=init, out=out0.clone(), algo=algo)
    torch.cuda.synchronize()
    idx_np = idx.cpu().numpy()
    o, s, st, sts = oracle.selective_scan(
        f(u), f(t["dt"]), f(t["A"]), f(t["B"]), f(t["C"]), D=None if D is None else f(D),
        z=None if z is None else f(z), dt_bias=None if bias is None else f(bias),
        dt_softplus=sp, state=f(st0), slot_idx=idx_np, has_initial_state=init, out=f(out0))
    check(out, o, s, RTOL[spec.io], spec.io, f"chunked scan {label} out")
    named = idx_np[idx_np >= 0]
    gst = f(t["ssm_state"])
    check(gst[named], st[named], sts[named], RTOL[spec.io], spec.state,
          f"chunked scan {label} state")
    others = np.setdiff1d(np.arange(spec.slots), named)
    np.testing.assert_array_equal(gst[others], f(st0)[others])
    return out, t["ssm_state"]


@pytest.mark.parametrize("io", ["bf16", "f16"])
@pytest.mark.parametrize("label,kw,opts", SSD_CASES, ids=[c[0] for c in SSD_CASES])
def test_chunked_scan_parity(dev, ssm, oracle, label, kw, opts, io):
    spec = W.tiny(io=io, a_per_state=False, index_sensitive=True,
                  **{**dict(state="f32"), **kw})
    _run(ssm, oracle, dev, spec, opts, f"{label} {io}", ssm.SCAN_CHUNKED)


@pytest.mark.parametrize("io", ["bf16", "f16"])
def test_auto_takes_the_chunked_form(dev, ssm, io):
    # the library's choice for a supported shape equals the explicit request,
    # bit for bit (same kernel)
    spec = W.tiny(io=io, a_per_state=False, seqlen=128, nheads=2, headdim=64, dstate=128,
                  index_sensitive=True)
    t = W.make(spec, dev)
    outs = []
    for algo in (None, ssm.SCAN_CHUNKED):
        st = t["ssm_state"].clone()
        outs.append((ssm.selective_scan(t["x"], t["dt"], t["A"], t["B"], t["C"], D=t["D"],
                                        z=t["z"], dt_bias=t["dt_bias"], ssm_state=st,
                                        algo=algo), st))
    torch.cuda.synchronize()
    assert torch.equal(outs[0][0], outs[1][0]) and torch.equal(outs[0][1], outs[1][1])


@pytest.mark.parametrize("io", ["bf16", "f16"])
def test_chunked_and_recurrent_agree(dev, ssm, io):
    # the two algorithms on the same inputs: within the 16-bit I/O bar of
    # each other
    spec = W.tiny(io=io, a_per_state=False, seqlen=640, nheads=2, headdim=128, dstate=256,
                  index_sensitive=True, state="f32")
    t = W.make(spec, dev)
    res = {}
    for algo in (ssm.SCAN_RECURRENT, ssm.SCAN_CHUNKED):
        st = t["ssm_state"].clone()
        o = ssm.selective_scan(t["x"], t["dt"], t["A"], t["B"], t["C"], D=t["D"], z=t["z"],
                               dt_bias=t["dt_bias"], ssm_state=st, has_initial_state=True,
                               algo=algo)
        res[algo] = (f(o), f(st))
    torch.cuda.synchronize()
    a, b = res[ssm.SCAN_RECURRENT], res[ssm.SCAN_CHUNKED]
    scale = np.abs(a[0]).max()
    assert np.abs(a[0] - b[0]).max() <= 2e-2 * scale
    assert np.abs(a[1] - b[1]).max() <= 1e-3 * np.abs(a[1]).max()
