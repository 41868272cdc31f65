"""GPU parity at the full workload sizes, in the launch configuration the
benchmark times.  The HIP path runs the whole workload; the float64 oracle
recomputes a sample of whole channels / rows / requests (they are independent
in the method), and the rest is checked through properties that hold at any
size (untouched cache slots bit-exact, every output finite).

Workloads: Mamba-1 2.8B layer prefill (batch 4, L 2048, d_inner 5120,
d_state 16, conv 4, f16 I/O, f32 state) and decode (245 requests from a
512-slot cache); Mamba-2 state update (headdim 64, dstate 128, 80 heads,
ngroups 1 and 8, batch 1024, f16 and f32 cache; headdim 128, dstate 256,
64 heads, batch 512 from a 1024-slot cache, bf16 and f32 cache) and the
matching Mamba-2 prefill (batch 2, L 4096).
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


def test_mamba1_prefill_full(dev, ssm, oracle):
    spec = W.prefill()
    t = W.make(spec, dev)
    st0 = t["ssm_state"].clone()
    u = ssm.causal_conv1d(t["x"], t["conv_w"], t["conv_b"], conv_state=t["conv_state"],
                          slot_idx=t["slot_idx"], has_initial_state=False)
    out = ssm.selective_scan(u, t["dt"], t["A"], t["B"], t["C"], D=t["D"], z=t["z"],
                             dt_bias=t["dt_bias"], ssm_state=t["ssm_state"],
                             slot_idx=t["slot_idx"], has_initial_state=False)
    torch.cuda.synchronize()
    assert torch.isfinite(out).all()
    rng = np.random.default_rng(11)
    chans = np.unique(np.concatenate([[0, 1, 15, 16, 5119], rng.choice(5120, 11, replace=False)]))
    ci = torch.as_tensor(chans, device=dev)
    for b in range(spec.batch):
        x = f(t["x"][b:b + 1, ci])
        uo, uso, _ = oracle.causal_conv1d(x, f(t["conv_w"][ci]), f(t["conv_b"][ci]), None, None)
        check(u[b:b + 1, ci], uo, uso, RTOL["f16"], "f16", f"prefill conv b={b}")
        uo = oracle.round_to(uo, oracle.F16)  # the scan reads u stored in f16
        o, so, st, sts = oracle.selective_scan(
            uo, f(t["dt"][b:b + 1, ci]), f(t["A"][ci]), f(t["B"][b:b + 1]), f(t["C"][b:b + 1]),
            D=f(t["D"][ci]), z=f(t["z"][b:b + 1, ci]), dt_bias=f(t["dt_bias"][ci]),
            state=np.zeros((1, len(chans), 1, 16)))
        check(out[b:b + 1, ci], o, so, RTOL["f16"], "f16", f"prefill scan out b={b}")
        slot = int(t["slot_idx"][b])
        check(t["ssm_state"][slot, ci], st[0], sts[0], RTOL["f16"], "f32", f"prefill state b={b}")
        # conv tail: the last 3 inputs, bit-exact
        np.testing.assert_array_equal(f(t["conv_state"][slot, ci]), x[0, :, -3:])


def test_mamba1_decode_full(dev, ssm, oracle):
    spec = W.decode()
    t = W.make(spec, dev)
    cs0, ss0 = t["conv_state"].clone(), t["ssm_state"].clone()
    x3 = t["x"].view(245, 5120, 1)
    u = ssm.causal_conv1d(x3, t["conv_w"], t["conv_b"], conv_state=t["conv_state"],
                          slot_idx=t["slot_idx"], has_initial_state=True)
    y = ssm.state_update(t["ssm_state"], u.view(245, 5120, 1), t["dt"], t["A"], t["B"], t["C"],
                         D=t["D"], z=t["z"], dt_bias=t["dt_bias"], slot_idx=t["slot_idx"])
    torch.cuda.synchronize()
    idx = t["slot_idx"].cpu().numpy()
    for b in (0, 1, 100, 244):
        s = int(idx[b])
        uo, uso, cso = oracle.causal_conv1d(f(x3[b:b + 1]), f(t["conv_w"]), f(t["conv_b"]),
                                            f(cs0[s:s + 1]), np.array([0], np.int32),
                                            has_initial_state=True)
        check(u[b:b + 1], uo, uso, RTOL["f16"], "f16", f"decode conv b={b}")
        np.testing.assert_array_equal(f(t["conv_state"][s:s + 1]), cso)
        uo = oracle.round_to(uo, oracle.F16)
        o, so, st, sts = oracle.state_update(
            f(ss0[s:s + 1]), uo.reshape(1, 5120, 1), f(t["dt"][b:b + 1]), f(t["A"]),
            f(t["B"][b:b + 1]), f(t["C"][b:b + 1]), D=f(t["D"]), z=f(t["z"][b:b + 1]),
            dt_bias=f(t["dt_bias"]), slot_idx=np.array([0], np.int32))
        check(y[b:b + 1], o, so, RTOL["f16"], "f16", f"decode ssu out b={b}")
        check(t["ssm_state"][s:s + 1], st, sts, RTOL["f16"], "f32", f"decode ssu state b={b}")
    others = np.setdiff1d(np.arange(512), idx)
    oi = torch.as_tensor(others, device=dev)
    assert torch.equal(t["ssm_state"][oi], ss0[oi])
    assert torch.equal(t["conv_state"][oi], cs0[oi])


def _ssu_full(ssm, oracle, dev, spec, sample):
    t = W.make(spec, dev)
    idx_t = t["slot_idx"]
    idx = idx_t.cpu().numpy()
    si = torch.as_tensor(idx[list(sample)], device=dev, dtype=torch.int64)
    st0_sample = t["ssm_state"][si].clone()
    untouched = np.setdiff1d(np.arange(spec.slots), idx)[:64]
    ui = torch.as_tensor(untouched, device=dev, dtype=torch.int64)
    st0_untouched = t["ssm_state"][ui].clone() if len(untouched) else None
    y = ssm.state_update(t["ssm_state"], t["x"], t["dt"], t["A"], t["B"], t["C"], D=t["D"],
                         z=t["z"], dt_bias=t["dt_bias"], slot_idx=idx_t)
    torch.cuda.synchronize()
    assert torch.isfinite(y).all()
    bi = torch.as_tensor(list(sample), device=dev)
    o, so, st, sts = oracle.state_update(
        f(st0_sample), f(t["x"][bi]), f(t["dt"][bi]), f(t["A"]), f(t["B"][bi]), f(t["C"][bi]),
        D=f(t["D"]), z=f(t["z"][bi]), dt_bias=f(t["dt_bias"]),
        slot_idx=np.arange(len(sample), dtype=np.int32))
    check(y[bi], o, so, RTOL[spec.io], spec.io, f"ssu out {spec}")
    check(t["ssm_state"][si], st, sts, RTOL[spec.io], spec.state, f"ssu state {spec}")
    if st0_untouched is not None:
        assert torch.equal(t["ssm_state"][ui], st0_untouched)


@pytest.mark.parametrize("ngroups", [1, 8])
@pytest.mark.parametrize("state", ["f16", "f32"])
def test_mamba2_ssu_hd64_full(dev, ssm, oracle, ngroups, state):
    _ssu_full(ssm, oracle, dev, W.m2_ssu_64(batch=1024, ngroups=ngroups, state=state),
              sample=(0, 1, 511, 1023))


@pytest.mark.parametrize("state", ["bf16", "f32"])
def test_mamba2_ssu_hd128_full(dev, ssm, oracle, state):
    _ssu_full(ssm, oracle, dev, W.m2_ssu_128(batch=512, state=state), sample=(0, 255, 511))


@pytest.mark.parametrize("batch", [1, 8, 64])
def test_mamba2_ssu_hd128_batches(dev, ssm, oracle, batch):
    _ssu_full(ssm, oracle, dev, W.m2_ssu_128(batch=batch, state="bf16"),
              sample=tuple(sorted({0, batch - 1})))


@pytest.mark.parametrize("batch", [1, 16, 256])
def test_mamba2_ssu_hd64_batches(dev, ssm, oracle, batch):
    _ssu_full(ssm, oracle, dev, W.m2_ssu_64(batch=batch, state="f16"),
              sample=tuple(sorted({0, batch - 1})))


@pytest.mark.parametrize("io,state", [("bf16", "bf16"), ("bf16", "f32"), ("f16", "f32")])
def test_mamba2_prefill_full(dev, ssm, oracle, io, state):
    # the chunked form at the full hd128/N256, L 4096, batch 2 size, with
    # bf16 and f16 I/O: sampled heads and rows against the oracle
    spec = W.m2_prefill(state=state, io=io)
    t = W.make(spec, dev)
    out = ssm.selective_scan(t["x"], t["dt"], t["A"], t["B"], t["C"], D=t["D"], z=t["z"],
                             dt_bias=t["dt_bias"], ssm_state=t["ssm_state"],
                             slot_idx=t["slot_idx"], has_initial_state=False)
    torch.cuda.synchronize()
    assert torch.isfinite(out).all()
    heads, rows = [0, 37, 63], [0, 1, 77, 127]
    P = spec.headdim
    ch = torch.as_tensor([h * P + p for h in heads for p in rows], device=dev)
    hi = torch.as_tensor(heads, device=dev)
    pi = torch.as_tensor(rows, device=dev)
    for b in range(spec.batch):
        o, so, st, sts = oracle.selective_scan(
            f(t["x"][b:b + 1, ch]), f(t["dt"][b:b + 1, hi]), f(t["A"][hi]), f(t["B"][b:b + 1]),
            f(t["C"][b:b + 1]), D=f(t["D"][hi]), z=f(t["z"][b:b + 1, ch]),
            dt_bias=f(t["dt_bias"][hi]), state=np.zeros((1, len(heads), len(rows), spec.dstate)))
        check(out[b:b + 1, ch], o, so, RTOL[spec.io], spec.io, f"m2 prefill {io} out b={b}")
        slot = int(t["slot_idx"][b])
        gst = t["ssm_state"][slot][hi][:, pi]
        check(gst, st[0], sts[0], RTOL[spec.io], spec.state, f"m2 prefill {io} state b={b}")


def test_mamba1_decode_step_fused_full(dev, ssm, oracle):
    """The decode workload through the fused conv-update + state-update entry
    point (the configuration the benchmark times)."""
    spec = W.decode()
    t = W.make(spec, dev)
    cs0, ss0 = t["conv_state"].clone(), t["ssm_state"].clone()
    y = ssm.decode_step(t["ssm_state"], t["conv_state"], t["x"], t["conv_w"], t["dt"], t["A"],
                        t["B"], t["C"], conv_bias=t["conv_b"], D=t["D"], z=t["z"],
                        dt_bias=t["dt_bias"], slot_idx=t["slot_idx"])
    torch.cuda.synchronize()
    idx = t["slot_idx"].cpu().numpy()
    for b in (0, 3, 128, 244):
        s = int(idx[b])
        uo, _, cso = oracle.causal_conv1d(f(t["x"][b:b + 1]).reshape(1, 5120, 1), f(t["conv_w"]),
                                          f(t["conv_b"]), f(cs0[s:s + 1]),
                                          np.array([0], np.int32), has_initial_state=True)
        np.testing.assert_array_equal(f(t["conv_state"][s:s + 1]), cso)
        o, so, st, sts = oracle.state_update(
            f(ss0[s:s + 1]), uo.reshape(1, 5120, 1), f(t["dt"][b:b + 1]), f(t["A"]),
            f(t["B"][b:b + 1]), f(t["C"][b:b + 1]), D=f(t["D"]), z=f(t["z"][b:b + 1]),
            dt_bias=f(t["dt_bias"]), slot_idx=np.array([0], np.int32))
        check(y[b:b + 1], o, so, RTOL["f16"], "f16", f"fused decode out b={b}")
        check(t["ssm_state"][s:s + 1], st, sts, RTOL["f16"], "f32", f"fused decode state b={b}")
    others = torch.as_tensor(np.setdiff1d(np.arange(512), idx), device=dev)
    assert torch.equal(t["ssm_state"][others], ss0[others])
    assert torch.equal(t["conv_state"][others], cs0[others])
