"""GPU parity: the HIP path (through the C ABI) against the float64 oracle,
element by element, on the same seeded inputs.  Sizes keep the oracle to
seconds while spanning several workgroups, several 256-step tiles and ragged
tails; the full-size workloads are in test_gpu_fullsize.py.

Output tolerance: |g - o| <= rtol * s + ulp/2 (tests/_parity.py), rtol 1e-5
for float32 I/O and 3e-3 for float16/bfloat16 I/O.  Cache rows: same metric in
the cache dtype; unnamed slots, padded requests and conv tails bit-exact.
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

    ssm.load_library()  # fail loudly if the HIP library is missing
    return torch.device("cuda:0")


@pytest.fixture(scope="module")
def ssm():
    import state_space_model_causal_amd as m

    return m


def _pad(idx: torch.Tensor, every: int) -> torch.Tensor:
    idx = idx.clone()
    if every:
        idx[::every] = -1
    return idx


def _named(idx_np):
    return idx_np[idx_np >= 0]


# ------------------------------------------------------------------ conv1d
CONV_CASES = [
    # (label, spec kwargs, has_initial_state, pad_every)
    ("tiny_f32", dict(), False, 0),
    ("tiny_f32_init", dict(), True, 0),
    ("f16_L1_decode_like", dict(seqlen=1, io="f16", nheads=300, batch=5, nslots=9,
                                random_slots=True), True, 2),
    ("f16_L3", dict(seqlen=3, io="f16", nheads=40, batch=3, nslots=5, random_slots=True), True, 0),
    ("bf16_L7", dict(seqlen=7, io="bf16", nheads=33, batch=2), True, 0),
    ("f16_L65_w2", dict(seqlen=65, io="f16", nheads=17, width=2, batch=2), False, 0),
    ("f32_L513_w3", dict(seqlen=513, io="f32", nheads=9, width=3, batch=3, nslots=4,
                         random_slots=True), True, 3),
    ("f16_L2048", dict(seqlen=2048, io="f16", nheads=24, batch=2), False, 0),
    ("bf16_L2049_w1", dict(seqlen=2049, io="bf16", nheads=5, width=1, batch=2), True, 0),
    ("f16_L4104", dict(seqlen=4104, io="f16", nheads=6, batch=1), True, 0),
    # 16-byte rows (seqlen % 8 == 0): two rows per workgroup, an odd row count,
    # padded requests, history through every width, several tiles
    ("f16_L1024_odd_rows_pad", dict(seqlen=1024, io="f16", nheads=7, batch=3, nslots=6,
                                    random_slots=True), True, 2),
    ("bf16_L256_w2", dict(seqlen=256, io="bf16", nheads=10, width=2, batch=2), True, 0),
    ("f32_L4096_init", dict(seqlen=4096, io="f32", nheads=3, batch=2, nslots=3,
                            random_slots=True), True, 0),
    ("bf16_L16_w1", dict(seqlen=16, io="bf16", nheads=9, width=1, batch=2), True, 0),
    # decode through the 8-channels-per-lane vector kernel (channels % 8 == 0)
    ("f16_L1_vec", dict(seqlen=1, io="f16", nheads=512, batch=7, nslots=11, random_slots=True),
     True, 3),
    ("bf16_L1_vec_w2", dict(seqlen=1, io="bf16", nheads=64, width=2, batch=6, nslots=9,
                            random_slots=True), True, 2),
    ("f32_L1_vec_w3_noinit", dict(seqlen=1, io="f32", nheads=40, width=3, batch=3), False, 0),
    ("f16_L1_vec_w1", dict(seqlen=1, io="f16", nheads=16, width=1, batch=2), True, 0),
]


@pytest.mark.parametrize("label,kw,init,pad", CONV_CASES, ids=[c[0] for c in CONV_CASES])
def test_conv1d_parity(dev, ssm, oracle, label, kw, init, pad):
    spec = W.tiny(**kw)
    t = W.make(spec, dev)
    x = t["x"].view(spec.batch, spec.channels, spec.seqlen)
    idx = _pad(t["slot_idx"], pad)
    cs0 = t["conv_state"].clone()
    out0 = torch.full_like(x, 7.0)
    out = ssm.causal_conv1d(x, t["conv_w"], t["conv_b"], conv_state=t["conv_state"], slot_idx=idx,
                            out=out0.clone(), has_initial_state=init)
    torch.cuda.synchronize()
    idx_np = idx.cpu().numpy()
    o, s, cs = oracle.causal_conv1d(f(x), f(t["conv_w"]), f(t["conv_b"]), f(cs0), idx_np,
                                    has_initial_state=init, out=f(out0))
    check(out, o, s, RTOL[spec.io], spec.io, f"conv {label} out")
    # cache: tails are exact copies, other slots untouched
    np.testing.assert_array_equal(f(t["conv_state"]), cs)


def test_conv1d_no_bias_no_silu(dev, ssm, oracle):
    spec = W.tiny(seqlen=100, io="f32", nheads=20)
    t = W.make(spec, dev)
    out = ssm.causal_conv1d(t["x"], t["conv_w"], None, apply_silu=False)
    torch.cuda.synchronize()
    o, s, _ = oracle.causal_conv1d(f(t["x"]), f(t["conv_w"]), None, None, None, apply_silu=False)
    check(out, o, s, 1e-5, "f32", "conv no bias/silu")


# ------------------------------------------------------------------- scan
SCAN_CASES = [
    # (label, spec kwargs, options)
    ("tiny_f32", dict(), {}),
    ("tiny_f32_idx", dict(index_sensitive=True), {}),
    ("tiny_f32_init_state", dict(index_sensitive=True, nslots=3, random_slots=True),
     dict(init=True)),
    ("m1_f16_L1", dict(io="f16", seqlen=1, nheads=40, batch=2), dict(init=True)),
    ("m1_f16_L3", dict(io="f16", seqlen=3, nheads=40, batch=2), {}),
    ("m1_bf16_L7", dict(io="bf16", seqlen=7, nheads=24, batch=2, index_sensitive=True), {}),
    ("m1_f16_L65", dict(io="f16", seqlen=65, nheads=40, batch=2, index_sensitive=True), {}),
    ("m1_f32_L513", dict(io="f32", seqlen=513, nheads=20, batch=2, index_sensitive=True,
                         nslots=5, random_slots=True), dict(init=True, pad=2)),
    ("m1_f16_L2049", dict(io="f16", seqlen=2049, nheads=18, batch=1, index_sensitive=True), {}),
    ("m1_f16_L2048_stf16", dict(io="f16", state="f16", seqlen=2048, nheads=32, batch=2,
                                index_sensitive=True), dict(init=True)),
    ("m1_f32_N5", dict(io="f32", seqlen=100, nheads=12, dstate=5, index_sensitive=True),
     dict(init=True)),
    ("m1_f32_N20", dict(io="f32", seqlen=77, nheads=12, dstate=20, index_sensitive=True), {}),
    ("m1_hd4", dict(io="f32", seqlen=50, nheads=6, headdim=4, index_sensitive=True), {}),
    ("m1_noz_noD_nobias", dict(io="f32", seqlen=300, nheads=16, index_sensitive=True),
     dict(z=False, D=False, bias=False)),
    ("m1_no_softplus", dict(io="f32", seqlen=64, nheads=16, index_sensitive=True),
     dict(softplus=False, bias=False)),
    ("m2_bf16_N256", dict(io="bf16", state="bf16", seqlen=300, nheads=2, headdim=64,
                          dstate=256, a_per_state=False, index_sensitive=True), dict(init=True)),
    ("m2_f16_N128_G8", dict(io="f16", state="f32", seqlen=129, nheads=16, headdim=4,
                            dstate=128, ngroups=8, a_per_state=False, index_sensitive=True,
                            batch=2), {}),
    ("m2_f32_N16_G2", dict(io="f32", state="f32", seqlen=258, nheads=4, headdim=8, dstate=16,
                           ngroups=2, a_per_state=False, index_sensitive=True, nslots=4,
                           random_slots=True, batch=3), dict(init=True, pad=3)),
    ("m2_bf16_L4096_N256", dict(io="bf16", state="f32", seqlen=4096, nheads=1, headdim=16,
                                dstate=256, a_per_state=False, index_sensitive=True), {}),
    # 16-byte rows whose length is not a multiple of 256 end in 8- and 4-step
    # tiles (64-bit loads and stores for 2-byte types)
    ("m1_f16_L264_vec_ladder", dict(io="f16", seqlen=264, nheads=24, batch=2, index_sensitive=True,
                                    nslots=3, random_slots=True), dict(init=True)),
    ("m1_bf16_L136_vec_ladder", dict(io="bf16", seqlen=136, nheads=16, batch=2, index_sensitive=True), {}),
    ("m1_f32_L40_vec_ladder", dict(io="f32", seqlen=40, nheads=12, batch=3, index_sensitive=True), {}),
    ("m2_f16_L408_vec_ladder", dict(io="f16", state="f32", seqlen=408, nheads=4, headdim=8, dstate=16,
                                    ngroups=2, a_per_state=False, index_sensitive=True), {}),
]


def run_scan(ssm, oracle, dev, spec, opts, label, t=None):
    t = t or W.make(spec, dev)
    u = t["x"].view(spec.batch, spec.channels, spec.seqlen)
    dt = t["dt"].view(spec.batch, spec.nheads, spec.seqlen)
    Bm = t["B"].view(spec.batch, spec.ngroups, spec.dstate, spec.seqlen)
    Cm = t["C"].view(spec.batch, spec.ngroups, spec.dstate, spec.seqlen)
    z = t["z"].view(spec.batch, spec.channels, spec.seqlen) if opts.get("z", True) else None
    D = t["D"] if opts.get("D", True) else None
    bias = t["dt_bias"] if opts.get("bias", True) else None
    sp = opts.get("softplus", True)
    init = opts.get("init", False)
    idx = _pad(t["slot_idx"], opts.get("pad", 0))
    st0 = t["ssm_state"].clone()
    out0 = torch.full_like(u, 5.0)
    out = ssm.selective_scan(u, dt, t["A"], Bm, Cm, D=D, z=z, dt_bias=bias, dt_softplus=sp,
                             ssm_state=t["ssm_state"], slot_idx=idx, has_initial_state=init,
                             out=out0.clone())
    torch.cuda.synchronize()
    idx_np = idx.cpu().numpy()
    o, s, st, sts = oracle.selective_scan(
        f(u), f(dt), f(t["A"]), f(Bm), f(Cm), D=None if D is None else f(D),
        z=None if z is None else f(z), dt_bias=None if bias is None else f(bias),
        dt_softplus=sp, state=f(st0), slot_idx=idx_np, has_initial_state=init, out=f(out0))
    check(out, o, s, RTOL[spec.io], spec.io, f"scan {label} out")
    named = _named(idx_np)
    gst = f(t["ssm_state"])
    check(gst[named], st[named], sts[named], RTOL[spec.io], spec.state, f"scan {label} state")
    others = np.setdiff1d(np.arange(spec.slots), named)
    np.testing.assert_array_equal(gst[others], f(st0)[others])
    return t, out


@pytest.mark.parametrize("label,kw,opts", SCAN_CASES, ids=[c[0] for c in SCAN_CASES])
def test_selective_scan_parity(dev, ssm, oracle, label, kw, opts):
    spec = W.tiny(**kw)
    t = W.make(spec, dev)
    if not opts.get("softplus", True):
        # raw steps (no softplus, no bias): keep them positive, |dt| + 0.01
        t["dt"].abs_().add_(0.01)
    run_scan(ssm, oracle, dev, spec, opts, label, t=t)


def test_scan_no_state_cache(dev, ssm, oracle):
    spec = W.tiny(io="f16", seqlen=200, nheads=16, index_sensitive=True)
    t = W.make(spec, dev)
    out = ssm.selective_scan(t["x"], t["dt"], t["A"], t["B"], t["C"], D=t["D"], z=t["z"],
                             dt_bias=t["dt_bias"])
    torch.cuda.synchronize()
    o, s, _, _ = oracle.selective_scan(f(t["x"]), f(t["dt"]), f(t["A"]), f(t["B"]), f(t["C"]),
                                       D=f(t["D"]), z=f(t["z"]), dt_bias=f(t["dt_bias"]))
    check(out, o, s, 3e-3, "f16", "scan without cache")


# -------------------------------------------------------------------- SSU
SSU_CASES = [
    # (label, spec kwargs, options)
    ("m1_N16_f32", dict(seqlen=1, nheads=300, dstate=16, io="f16", state="f32", batch=7,
                        nslots=20, random_slots=True, index_sensitive=True), dict(pad=3)),
    ("m1_N16_f16", dict(seqlen=1, nheads=64, dstate=16, io="f16", state="f16", batch=5,
                        nslots=6, random_slots=True, index_sensitive=True), {}),
    # batch >= 8 with one channel per head: two requests per lane, an odd
    # batch leaving the last lane's second request empty, padded requests
    ("m1_N16_f32_two_per_lane", dict(seqlen=1, nheads=96, dstate=16, io="f16", state="f32",
                                     batch=9, nslots=24, random_slots=True,
                                     index_sensitive=True), dict(pad=4)),
    ("m1_N16_bf16_two_per_lane", dict(seqlen=1, nheads=64, dstate=16, io="bf16", state="bf16",
                                      batch=8, nslots=8, random_slots=True,
                                      index_sensitive=True), {}),
    ("m2_hd64_N128_f16", dict(seqlen=1, nheads=80, headdim=64, dstate=128, io="f16", state="f16",
                              a_per_state=False, batch=3, index_sensitive=True), {}),
    ("m2_hd64_N128_G8_f32", dict(seqlen=1, nheads=80, headdim=64, dstate=128, ngroups=8, io="f16",
                                 state="f32", a_per_state=False, batch=2, index_sensitive=True),
     {}),
    ("m2_hd128_N256_bf16", dict(seqlen=1, nheads=8, headdim=128, dstate=256, io="bf16",
                                state="bf16", a_per_state=False, batch=3, nslots=11,
                                random_slots=True, index_sensitive=True), dict(pad=2)),
    ("m2_hd128_N256_f32io", dict(seqlen=1, nheads=4, headdim=128, dstate=256, io="f32",
                                 state="f32", a_per_state=False, batch=2, index_sensitive=True),
     {}),
    ("N5_scalar_path", dict(seqlen=1, nheads=6, headdim=3, dstate=5, io="f32", state="f32",
                            a_per_state=False, batch=2, index_sensitive=True), {}),
    ("N24_pad_lanes", dict(seqlen=1, nheads=6, headdim=3, dstate=24, io="f32", state="f16",
                           a_per_state=True, batch=2, index_sensitive=True), {}),
    ("N512", dict(seqlen=1, nheads=2, headdim=4, dstate=512, io="bf16", state="f32",
                  a_per_state=False, batch=2, index_sensitive=True), {}),
    ("hd1_noz_noD", dict(seqlen=1, nheads=50, dstate=16, io="f32", state="f32", batch=3,
                         index_sensitive=True), dict(z=False, D=False, bias=False)),
    # interleaved lane map (32 bytes of state per lane, power-of-two rows,
    # >= 2^18 (request, row) pairs): 2, 16, 32 and 64 lanes per row, groups,
    # two requests per lane with an odd batch, padded requests, a workgroup
    # whose last wave lies past the last row
    ("ilv_m1_N16_f32", dict(seqlen=1, nheads=2048, dstate=16, io="f16", state="f32", batch=129,
                            nslots=140, random_slots=True, index_sensitive=True), dict(pad=5)),
    ("ilv_m1_N16_past_last_row", dict(seqlen=1, nheads=96, dstate=16, io="f16", state="f32",
                                      batch=2731, index_sensitive=True), dict(pad=2)),
    ("ilv_m1_N16_f32io_noz_noD", dict(seqlen=1, nheads=2048, dstate=16, io="f32", state="f32",
                                      batch=128, index_sensitive=True),
     dict(z=False, D=False, bias=False)),
    ("ilv_m2_hd64_N128_G8_f16", dict(seqlen=1, nheads=80, headdim=64, dstate=128, ngroups=8,
                                     io="f16", state="f16", a_per_state=False, batch=52,
                                     nslots=60, random_slots=True, index_sensitive=True),
     dict(pad=3)),
    ("ilv_m2_hd128_N256_bf16", dict(seqlen=1, nheads=64, headdim=128, dstate=256, io="bf16",
                                    state="bf16", a_per_state=False, batch=33, nslots=36,
                                    random_slots=True, index_sensitive=True), {}),
    ("ilv_N256_f32_1KB_rows", dict(seqlen=1, nheads=16, headdim=64, dstate=256, io="f16",
                                   state="f32", a_per_state=False, batch=257,
                                   index_sensitive=True), {}),
    ("ilv_N8_f32_2_lanes_per_row", dict(seqlen=1, nheads=64, headdim=64, dstate=8, io="f16",
                                        state="f32", a_per_state=False, batch=65,
                                        index_sensitive=True), {}),
    ("ilv_N64_f16_8_lanes_per_row", dict(seqlen=1, nheads=32, headdim=64, dstate=64, io="bf16",
                                         state="f16", a_per_state=True, batch=129,
                                         index_sensitive=True), dict(pad=1)),
    # as many (request, row) pairs, but groups of 10 rows do not hold whole
    # 32-row wave blocks: the blocked map
    ("blocked_groups_not_wave_aligned", dict(seqlen=1, nheads=80, dstate=16, ngroups=8, io="f16",
                                             state="f32", batch=3300, index_sensitive=True), {}),
]


def run_ssu(ssm, oracle, dev, spec, opts, label, t=None):
    t = t or W.make(spec, dev)
    z = t["z"] if opts.get("z", True) else None
    D = t["D"] if opts.get("D", True) else None
    bias = t["dt_bias"] if opts.get("bias", True) else None
    idx = _pad(t["slot_idx"], opts.get("pad", 0))
    st0 = t["ssm_state"].clone()
    out0 = torch.full_like(t["x"], 3.0)
    # without a table the slot of request b is b (the arange the oracle takes)
    out = ssm.state_update(t["ssm_state"], t["x"], t["dt"], t["A"], t["B"], t["C"], D=D, z=z,
                           dt_bias=bias, slot_idx=None if opts.get("no_table") else idx,
                           out=out0.clone())
    torch.cuda.synchronize()
    idx_np = idx.cpu().numpy()
    o, s, st, sts = oracle.state_update(
        f(st0), f(t["x"]), f(t["dt"]), f(t["A"]), f(t["B"]), f(t["C"]),
        D=None if D is None else f(D), z=None if z is None else f(z),
        dt_bias=None if bias is None else f(bias), slot_idx=idx_np, out=f(out0))
    check(out, o, s, RTOL[spec.io], spec.io, f"ssu {label} out")
    named = _named(idx_np)
    gst = f(t["ssm_state"])
    check(gst[named], st[named], sts[named], RTOL[spec.io], spec.state, f"ssu {label} state")
    others = np.setdiff1d(np.arange(spec.slots), named)
    np.testing.assert_array_equal(gst[others], f(st0)[others])


@pytest.mark.parametrize("label,kw,opts", SSU_CASES, ids=[c[0] for c in SSU_CASES])
def test_state_update_parity(dev, ssm, oracle, label, kw, opts):
    run_ssu(ssm, oracle, dev, W.tiny(**kw), opts, label)


# ------------------------------------------------------------- invariants
def test_scan_equals_chained_gpu_updates(dev, ssm):
    """A GPU scan over L tokens equals L chained GPU state updates (float32
    state, float32 I/O): both from the same cached initial state."""
    spec = W.tiny(io="f32", state="f32", seqlen=37, nheads=4, headdim=8, dstate=32,
                  a_per_state=False, index_sensitive=True, batch=2, nslots=3, random_slots=True)
    t = W.make(spec, dev)
    st_chain = t["ssm_state"].clone()
    out = ssm.selective_scan(t["x"], t["dt"], t["A"], t["B"], t["C"], D=t["D"], z=t["z"],
                             dt_bias=t["dt_bias"], ssm_state=t["ssm_state"],
                             slot_idx=t["slot_idx"], has_initial_state=True)
    outs = []
    for s in range(spec.seqlen):
        x = t["x"][:, :, s].contiguous().view(2, 4, 8)
        z = t["z"][:, :, s].contiguous().view(2, 4, 8)
        y = ssm.state_update(st_chain, x, t["dt"][:, :, s].contiguous(), t["A"],
                             t["B"][..., s].contiguous(), t["C"][..., s].contiguous(), D=t["D"],
                             z=z, dt_bias=t["dt_bias"], slot_idx=t["slot_idx"])
        outs.append(y.view(2, 32))
    torch.cuda.synchronize()
    chain = torch.stack(outs, dim=2)
    err = (chain - out).abs().max().item()
    scale = out.abs().max().item()
    assert err <= 2e-5 * scale, (err, scale)
    serr = (st_chain - t["ssm_state"]).abs().max().item()
    assert serr <= 2e-5 * t["ssm_state"].abs().max().item()


def test_prefill_then_decode_resumes(dev, ssm, oracle):
    """Prefill writes the final state and conv tail to the slot; decode steps
    continue from them (checked against one oracle pass over the whole
    sequence)."""
    L1, L2 = 40, 3
    spec = W.tiny(io="f32", seqlen=L1 + L2, nheads=24, index_sensitive=True, nslots=4,
                  random_slots=True, batch=2)
    t = W.make(spec, dev)
    x = t["x"]
    cs, ss = t["conv_state"], t["ssm_state"]
    idx = t["slot_idx"]
    u1 = ssm.causal_conv1d(x[..., :L1].contiguous(), t["conv_w"], t["conv_b"], conv_state=cs,
                           slot_idx=idx, has_initial_state=False)
    y1 = ssm.selective_scan(u1, t["dt"][..., :L1].contiguous(), t["A"],
                            t["B"][..., :L1].contiguous(), t["C"][..., :L1].contiguous(),
                            D=t["D"], z=t["z"][..., :L1].contiguous(), dt_bias=t["dt_bias"],
                            ssm_state=ss, slot_idx=idx, has_initial_state=False)
    ys = []
    for s in range(L1, L1 + L2):
        u = ssm.causal_conv1d(x[..., s:s + 1].contiguous(), t["conv_w"], t["conv_b"],
                              conv_state=cs, slot_idx=idx, has_initial_state=True)
        y = ssm.state_update(ss, u.view(2, 24, 1), t["dt"][..., s].contiguous(), t["A"],
                             t["B"][..., s].contiguous(), t["C"][..., s].contiguous(), D=t["D"],
                             z=t["z"][..., s].contiguous().view(2, 24, 1), dt_bias=t["dt_bias"],
                             slot_idx=idx)
        ys.append(y.view(2, 24, 1))
    torch.cuda.synchronize()
    got = torch.cat([y1] + ys, dim=2)
    uo, _, _ = oracle.causal_conv1d(f(x), f(t["conv_w"]), f(t["conv_b"]), None, None)
    o, sc, _, _ = oracle.selective_scan(uo, f(t["dt"]), f(t["A"]), f(t["B"]), f(t["C"]),
                                        D=f(t["D"]), z=f(t["z"]), dt_bias=f(t["dt_bias"]))
    check(got, o, sc, 1e-5, "f32", "prefill+decode resume")


def test_graph_replay_matches_eager(dev, ssm):
    """The entry points are capturable: a HIP graph of conv + scan + update,
    replayed several times with eager work in between, matches eager runs."""
    spec = W.tiny(io="f16", seqlen=128, nheads=32, index_sensitive=True)
    t = W.make(spec, dev)
    d = W.make(W.decode(batch=3, nslots=5, nheads=64, seed=21), dev)
    out_u = torch.empty_like(t["x"])
    out_y = torch.empty_like(t["x"])
    out_d = torch.empty_like(d["x"])

    def body():
        ssm.causal_conv1d(t["x"], t["conv_w"], t["conv_b"], out=out_u)
        ssm.selective_scan(out_u, t["dt"], t["A"], t["B"], t["C"], D=t["D"], z=t["z"],
                           dt_bias=t["dt_bias"], out=out_y)
        ssm.state_update(d["ssm_state"], d["x"], d["dt"], d["A"], d["B"], d["C"], D=d["D"],
                         z=d["z"], dt_bias=d["dt_bias"], slot_idx=d["slot_idx"], out=out_d)

    st_init = d["ssm_state"].clone()
    refs = []
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        for _ in range(3):
            body()
            refs.append((out_y.clone(), out_d.clone(), d["ssm_state"].clone()))
    torch.cuda.current_stream().wait_stream(s)
    d["ssm_state"].copy_(st_init)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        body()
    d["ssm_state"].copy_(st_init)
    for k in range(3):
        out_y.fill_(0)
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out_y, refs[k][0])
        assert torch.equal(out_d, refs[k][1])
        assert torch.equal(d["ssm_state"], refs[k][2])
        _ = (t["x"].float() * 2).sum().item()  # eager work between replays


@pytest.mark.parametrize("io", ["f32", "bf16"])
def test_softplus_step_accuracy(dev, ssm, oracle, io):
    """The step size alone: a one-step scan with B = C = u = 1, D = 0, no gate
    and a single state returns delta = softplus(dt + bias) itself, over raw
    values from -30 to 25 (both exp tails and the log1p-sensitive middle)."""
    nv = 2048
    v = torch.linspace(-30.0, 25.0, nv, dtype=torch.float64)
    dtype = W.DTYPES[io]
    dt = v.to(dtype).view(1, nv, 1).to(dev)
    one = torch.ones(1, nv, 1, dtype=dtype, device=dev)
    Bm = torch.ones(1, 1, 1, 1, dtype=dtype, device=dev)
    A = -torch.ones(nv, 1, dtype=torch.float32, device=dev)
    out = ssm.selective_scan(one, dt, A, Bm, Bm.clone(), D=None, z=None, dt_bias=None)
    torch.cuda.synchronize()
    want = np.array([oracle.softplus(x) for x in f(dt).ravel()])
    got = f(out).ravel()
    # float32: a few ulp, plus the rounding of the exponent argument |v|*log2(e)
    # (about |v| * 6e-8 relative); the bf16 store adds half an ulp
    x = np.abs(f(dt).ravel())
    tol = (4e-7 + 1e-7 * x) * np.abs(want) + (0.5 * 2.0 ** -7 * np.abs(want) if io == "bf16" else 0.0)
    bad = np.abs(got - want) > tol
    assert not bad.any(), (f(dt).ravel()[bad][:5], got[bad][:5], want[bad][:5])


def _bf16_rounding_cases(rng, n):
    """float32 bit patterns that exercise round-to-nearest-even into bfloat16:
    exact ties (odd and even), one below and one above a tie, subnormals,
    values that round up to infinity, random patterns, and +-inf and NaN."""
    top = rng.integers(0, 1 << 16, n, dtype=np.uint64)
    top = np.where((top & 0x7f80) == 0x7f80, top & 0x807f, top)  # finite
    low = np.array([0x8000, 0x7fff, 0x8001, 0x0000], dtype=np.uint64)[np.arange(n) % 4]
    bits = (top << 16) | low
    sub = rng.integers(1, 1 << 23, n // 8, dtype=np.uint64)  # float32 subnormals
    bits[: n // 8] = sub | (np.uint64(0x80000000) * (sub & 1))
    bits[n // 8: n // 4] = rng.integers(0, 0x7f800000, n // 8, dtype=np.uint64)
    bits[-6:] = [0x7f7fffff, 0xff7f8000, 0x7f800000, 0xff800000, 0x7fc00001, 0xffa00000]
    return bits.astype(np.uint32).view(np.float32)


def test_bf16_state_rounding_is_rne(dev, ssm, oracle):
    """The stored bfloat16 state is the float32 state rounded to nearest even,
    bit for bit.  A one-step scan with step size 1, B = 1 and a decay of 0
    (A = -1e30) leaves exactly u in the state, so the cache holds
    round(u) over the crafted patterns; NaN stays NaN."""
    n, N = 4096, 16
    u_np = _bf16_rounding_cases(np.random.default_rng(5), n)
    u = torch.from_numpy(u_np.copy()).view(1, n, 1).to(dev)
    dt = torch.ones(1, n, 1, dtype=torch.float32, device=dev)
    A = torch.full((n, N), -1e30, dtype=torch.float32, device=dev)
    Bm = torch.ones(1, 1, N, 1, dtype=torch.float32, device=dev)
    Cm = torch.zeros(1, 1, N, 1, dtype=torch.float32, device=dev)
    state = torch.zeros(1, n, 1, N, dtype=torch.bfloat16, device=dev)
    slot = torch.zeros(1, dtype=torch.int32, device=dev)
    ssm.selective_scan(u, dt, A, Bm, Cm, dt_softplus=False, ssm_state=state, slot_idx=slot)
    torch.cuda.synchronize()
    got = state.float().cpu().numpy().reshape(n, N).astype(np.float64)
    want = oracle.round_to(u_np.astype(np.float64), 2)
    nan = np.isnan(want)
    assert (np.isnan(got[nan]).all()), "NaN not kept"
    ok = got[~nan] == want[~nan][:, None]
    assert ok.all(), (u_np[~nan][~ok.all(1)][:5], got[~nan][~ok.all(1)][:5, 0], want[~nan][~ok.all(1)][:5])


# ------------------------------------------------------- fused decode step
DECODE_CASES = [
    ("m1_f16_f32state", dict(seqlen=1, nheads=300, dstate=16, io="f16", state="f32", batch=7,
                             nslots=20, random_slots=True, index_sensitive=True), dict(pad=3)),
    ("m1_bf16_bf16state", dict(seqlen=1, nheads=64, dstate=16, io="bf16", state="bf16", batch=5,
                               nslots=6, random_slots=True, index_sensitive=True), {}),
    # two requests per lane (batch >= 8), odd batch, padded requests
    ("m1_f16_two_per_lane", dict(seqlen=1, nheads=160, dstate=16, io="f16", state="f32", batch=11,
                                 nslots=30, random_slots=True, index_sensitive=True), dict(pad=3)),
    ("m1_f32_noz_noD", dict(seqlen=1, nheads=40, dstate=16, io="f32", state="f32", batch=3,
                            index_sensitive=True), dict(z=False, D=False, bias=False)),
    ("m2_hd64_N128_G8", dict(seqlen=1, nheads=16, headdim=64, dstate=128, ngroups=8, io="f16",
                             state="f16", a_per_state=False, batch=3, index_sensitive=True), {}),
    ("m2_hd128_N256_bf16", dict(seqlen=1, nheads=4, headdim=128, dstate=256, io="bf16",
                                state="f32", a_per_state=False, batch=2, nslots=5,
                                random_slots=True, index_sensitive=True), dict(pad=2)),
    # interleaved lane map (>= 2^18 (request, channel) pairs)
    ("ilv_m1_f16_f32state", dict(seqlen=1, nheads=2048, dstate=16, io="f16", state="f32",
                                 batch=129, nslots=140, random_slots=True, index_sensitive=True),
     dict(pad=5)),
    ("ilv_m1_f32_noz_noD", dict(seqlen=1, nheads=2048, dstate=16, io="f32", state="f32", batch=128,
                                index_sensitive=True), dict(z=False, D=False, bias=False)),
    # the quad-shared conv with 16 lanes per row (every quad of a row computes
    # it, the first one writes the window), and the per-lane conv at 2 lanes
    # per row
    ("ilv_m2_hd64_N128_f16_conv_16_lanes", dict(seqlen=1, nheads=64, headdim=64, dstate=128, io="f16",
                                                state="f16", a_per_state=False, batch=65, nslots=70,
                                                random_slots=True, index_sensitive=True), dict(pad=2)),
    ("ilv_N8_f32_conv_2_lanes", dict(seqlen=1, nheads=2048, headdim=2, dstate=8, io="bf16", state="f32",
                                     batch=65, index_sensitive=True), {}),
]


def run_decode_step(ssm, oracle, spec, t, opts, label):
    z = t["z"] if opts.get("z", True) else None
    D = t["D"] if opts.get("D", True) else None
    bias = t["dt_bias"] if opts.get("bias", True) else None
    idx = _pad(t["slot_idx"], opts.get("pad", 0))
    st0, cs0 = t["ssm_state"].clone(), t["conv_state"].clone()
    out0 = torch.full_like(t["x"], 3.0)
    u_out = torch.full_like(t["x"], 9.0)
    out = ssm.decode_step(t["ssm_state"], t["conv_state"], t["x"], t["conv_w"], t["dt"], t["A"],
                          t["B"], t["C"], conv_bias=t["conv_b"], D=D, z=z, dt_bias=bias,
                          slot_idx=None if opts.get("no_table") else idx, out=out0.clone(),
                          u_out=u_out)
    torch.cuda.synchronize()
    idx_np = idx.cpu().numpy()
    Bt, Cn = spec.batch, spec.channels
    x3 = f(t["x"]).reshape(Bt, Cn, 1)
    uo, uso, cso = oracle.causal_conv1d(x3, f(t["conv_w"]), f(t["conv_b"]), f(cs0), idx_np,
                                        has_initial_state=True, out=f(u_out).reshape(Bt, Cn, 1))
    shp = (Bt, spec.nheads, spec.headdim)
    # the fused step hands the float32 conv output to the update (no rounding)
    o, so, st, sts = oracle.state_update(
        f(st0), uo.reshape(shp), f(t["dt"]), f(t["A"]), f(t["B"]), f(t["C"]),
        D=None if D is None else f(D), z=None if z is None else f(z),
        dt_bias=None if bias is None else f(bias), slot_idx=idx_np, out=f(out0))
    # That conv output carries the rounding of the conv's own terms (scale
    # uso >= |u|), which a near-cancelling conv leaves large next to |u|: the
    # update's scales are taken with uso in place of |u|.
    _, so, _, sts = oracle.state_update(
        f(st0), uso.reshape(shp), f(t["dt"]), f(t["A"]), f(t["B"]), f(t["C"]),
        D=None if D is None else f(D), z=None if z is None else f(z),
        dt_bias=None if bias is None else f(bias), slot_idx=idx_np, out=f(out0))
    check(out, o, so, RTOL[spec.io], spec.io, f"decode_step {label} out")
    check(u_out.reshape(Bt, Cn, 1), uo, uso, RTOL[spec.io], spec.io, f"decode_step {label} u")
    np.testing.assert_array_equal(f(t["conv_state"]), cso)
    named = _named(idx_np)
    gst = f(t["ssm_state"])
    check(gst[named], st[named], sts[named], RTOL[spec.io], spec.state, f"decode_step {label} state")
    others = np.setdiff1d(np.arange(spec.slots), named)
    np.testing.assert_array_equal(gst[others], f(st0)[others])


@pytest.mark.parametrize("label,kw,opts", DECODE_CASES, ids=[c[0] for c in DECODE_CASES])
def test_decode_step_parity(dev, ssm, oracle, label, kw, opts):
    spec = W.tiny(**kw)
    run_decode_step(ssm, oracle, spec, W.make(spec, dev), opts, label)


# Batches whose request groups (one or two requests per lane) exceed the
# grid's y dimension (65535): the update is launched in parts of that many
# groups; without a slot table each part's state and conv-cache rows start at
# its first request.
BIG_BATCH_CASES = [
    ("m1_two_per_lane_table", dict(seqlen=1, nheads=2, dstate=16, io="f16", state="f32",
                                   batch=140001, nslots=140007, random_slots=True,
                                   index_sensitive=True), dict(pad=7)),
    ("m1_two_per_lane_no_table", dict(seqlen=1, nheads=2, dstate=16, io="f32", state="f32",
                                      batch=131075, index_sensitive=True), dict(no_table=True)),
    ("m2_one_per_lane_no_table", dict(seqlen=1, nheads=1, headdim=4, dstate=16, io="bf16",
                                      state="bf16", a_per_state=False, batch=65539,
                                      index_sensitive=True), dict(no_table=True)),
]


@pytest.mark.parametrize("label,kw,opts", BIG_BATCH_CASES, ids=[c[0] for c in BIG_BATCH_CASES])
def test_state_update_and_decode_step_past_grid_limit(dev, ssm, oracle, label, kw, opts):
    spec = W.tiny(**kw)
    run_ssu(ssm, oracle, dev, spec, opts, label + " ssu")
    run_decode_step(ssm, oracle, spec, W.make(spec, dev), opts, label + " decode")


def test_decode_step_chain_matches_prefill(dev, ssm, oracle):
    """Prefill the first tokens, then run fused decode steps: the outputs
    continue the one-pass oracle sequence (conv tail and state from slots)."""
    L1, L2 = 30, 4
    spec = W.tiny(io="f32", seqlen=L1 + L2, nheads=24, index_sensitive=True, nslots=4,
                  random_slots=True, batch=2)
    t = W.make(spec, dev)
    idx = t["slot_idx"]
    u1 = ssm.causal_conv1d(t["x"][..., :L1].contiguous(), t["conv_w"], t["conv_b"],
                           conv_state=t["conv_state"], slot_idx=idx)
    y1 = ssm.selective_scan(u1, t["dt"][..., :L1].contiguous(), t["A"],
                            t["B"][..., :L1].contiguous(), t["C"][..., :L1].contiguous(),
                            D=t["D"], z=t["z"][..., :L1].contiguous(), dt_bias=t["dt_bias"],
                            ssm_state=t["ssm_state"], slot_idx=idx)
    ys = [y1]
    for s in range(L1, L1 + L2):
        y = ssm.decode_step(t["ssm_state"], t["conv_state"],
                            t["x"][..., s].contiguous().view(2, 24, 1), t["conv_w"],
                            t["dt"][..., s].contiguous(), t["A"], t["B"][..., s].contiguous(),
                            t["C"][..., s].contiguous(), conv_bias=t["conv_b"], D=t["D"],
                            z=t["z"][..., s].contiguous().view(2, 24, 1), dt_bias=t["dt_bias"],
                            slot_idx=idx)
        ys.append(y.view(2, 24, 1))
    torch.cuda.synchronize()
    uo, _, _ = oracle.causal_conv1d(f(t["x"]), f(t["conv_w"]), f(t["conv_b"]), None, None)
    o, sc, _, _ = oracle.selective_scan(uo, f(t["dt"]), f(t["A"]), f(t["B"]), f(t["C"]),
                                        D=f(t["D"]), z=f(t["z"]), dt_bias=f(t["dt_bias"]))
    check(torch.cat(ys, dim=2), o, sc, 1e-5, "f32", "prefill + fused decode")


# ------------------------------------------------- state-update geometries
GEOMETRY_SHAPES = [
    # (label, spec kwargs): row widths that exercise 1 to 64 lanes per row,
    # partial lanes (dstate 24) and the scalar path (dstate 20 with 16 per lane)
    ("m1_N16", dict(seqlen=1, nheads=96, dstate=16, io="f16", state="f32", batch=5, nslots=9,
                    random_slots=True, index_sensitive=True)),
    ("hd3_N24", dict(seqlen=1, nheads=6, headdim=3, dstate=24, io="f32", state="f16",
                     a_per_state=True, batch=3, index_sensitive=True)),
    ("hd4_N20", dict(seqlen=1, nheads=4, headdim=4, dstate=20, io="f32", state="f32",
                     a_per_state=False, batch=2, index_sensitive=True)),
    ("hd64_N128", dict(seqlen=1, nheads=16, headdim=64, dstate=128, io="f16", state="f16",
                       a_per_state=False, ngroups=4, batch=3, index_sensitive=True)),
    ("hd8_N512", dict(seqlen=1, nheads=2, headdim=8, dstate=512, io="bf16", state="f32",
                      a_per_state=False, batch=2, index_sensitive=True)),
]


@pytest.mark.parametrize("label,kw", GEOMETRY_SHAPES, ids=[g[0] for g in GEOMETRY_SHAPES])
def test_state_update_every_geometry(dev, ssm, oracle, label, kw):
    # every geometry the override accepts meets the parity bar, and all of
    # them leave the same cache bytes (the update of a state does not depend
    # on how states are spread over lanes)
    spec = W.tiny(**kw)
    t = W.make(spec, dev)
    st0 = t["ssm_state"].clone()
    idx = t["slot_idx"]
    idx_np = idx.cpu().numpy()
    o, s, st, sts = oracle.state_update(f(st0), f(t["x"]), f(t["dt"]), f(t["A"]), f(t["B"]),
                                        f(t["C"]), D=f(t["D"]), z=f(t["z"]),
                                        dt_bias=f(t["dt_bias"]), slot_idx=idx_np)
    first = None
    for v in ((4, 8, 16) if spec.state == "f32" and spec.dstate <= 256 else (8, 16)):
        for b in (64, 128, 256, 512):
            state = st0.clone()
            out = ssm.state_update(state, t["x"], t["dt"], t["A"], t["B"], t["C"], D=t["D"],
                                   z=t["z"], dt_bias=t["dt_bias"], slot_idx=idx, config=(v, b))
            torch.cuda.synchronize()
            check(out, o, s, RTOL[spec.io], spec.io, f"ssu {label} {v}x{b} out")
            if first is None:
                first = state
                gst = f(state)
                named = _named(idx_np)
                check(gst[named], st[named], sts[named], RTOL[spec.io], spec.state,
                      f"ssu {label} state")
            else:
                assert torch.equal(state, first), f"{label} {v}x{b}: cache bytes differ"
