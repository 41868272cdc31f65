"""GPU parity of the decode layer around the path: the projection kernel
(ssm_linear), the RMSNorm (ssm_rmsnorm) and one whole Mamba-1 decode layer
(ssm_mamba1_decode_layer) against the float64 oracle (oracle/layer.py).

Projections: f16 and bf16, shapes from one row to more rows than a
workgroup covers, narrow outputs (split over K), K not a multiple of the MFMA
step, a residual.  Layer: the oracle rounds each intermediate to the io dtype
as the library stores it; tolerance the f16/bf16 bar of tests/_parity.py.
"""
import numpy as np
import pytest
import torch

import workloads as W
from tests._parity import check, to_f64 as f

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


LINEAR_CASES = [
    # (M, N, K, dtype, residual)
    (1, 64, 32, torch.float16, False),
    (7, 100, 40, torch.bfloat16, True),
    (245, 192, 5120, torch.float16, False),   # split over K
    (245, 5120, 160, torch.bfloat16, False),
    (300, 130, 264, torch.float16, True),     # two row blocks, ragged N
    (245, 2560, 5120, torch.bfloat16, True),  # out_proj shape, split over K
    (33, 70, 24, torch.float16, True),        # N % 4 != 0, K not split: stores in the reduce pass
    (300, 128, 64, torch.bfloat16, True),     # two row blocks, outputs stored by the main kernel
]


@pytest.mark.parametrize("M,N,K,dt,res", LINEAR_CASES,
                         ids=[f"{c[0]}x{c[1]}x{c[2]}_{str(c[3])[6:]}{'_res' if c[4] else ''}"
                              for c in LINEAR_CASES])
def test_linear_parity(dev, ssm, M, N, K, dt, res):
    from oracle import layer

    g = torch.Generator(device=dev).manual_seed(M * 7 + N)
    x = torch.randn(M, K, generator=g, device=dev).to(dt)
    w = (torch.randn(N, K, generator=g, device=dev) / K ** 0.5).to(dt)
    r = torch.randn(M, N, generator=g, device=dev).to(dt) if res else None
    out = ssm.linear(x, w, residual=r)
    torch.cuda.synchronize()
    o, s = layer.linear(f(x), f(w), residual=None if r is None else f(r))
    check(out, o, s, 3e-3, "f16" if dt == torch.float16 else "bf16", f"linear {M}x{N}x{K}")


# every plan the product kernel takes: rows per wave x columns per workgroup
# x splits (partials added by the reduce kernel); ragged rows and columns,
# N % 4 != 0
PLAN_SHAPES = [(245, 10240, 2560), (245, 2560, 5120), (77, 200, 1000), (130, 70, 512)]
PLANS = [(wr, c, sp) for wr in (16, 32, 64) for c in (64, 128) for sp in (1, 3, 8)]


@pytest.mark.parametrize("M,N,K", PLAN_SHAPES, ids=[f"{m}x{n}x{k}" for m, n, k in PLAN_SHAPES])
def test_linear_every_plan(dev, ssm, M, N, K):
    """Each plan against the oracle on the same inputs, twice (bit-identical)."""
    from oracle import layer

    lib = ssm.load_library()
    g = torch.Generator(device=dev).manual_seed(M + N + K)
    x = torch.randn(M, K, generator=g, device=dev).to(torch.float16)
    w = (torch.randn(N, K, generator=g, device=dev) / K ** 0.5).to(torch.float16)
    r = torch.randn(M, N, generator=g, device=dev).to(torch.float16)
    o, s = layer.linear(f(x), f(w), residual=f(r))
    for wr, c, sp in PLANS:
        need = lib.ssm_linear_workspace_ex(M, N, K, wr, c, sp)
        ws = torch.full((max(need, 16) // 4,), -1, dtype=torch.int32, device=dev)
        outs = []
        for rep in range(2):
            outs.append(ssm.linear(x, w, residual=r, workspace=ws, rows_per_wave=wr, cols=c, splits=sp))
            torch.cuda.synchronize()
            check(outs[-1], o, s, 3e-3, "f16", f"linear {M}x{N}x{K} wr={wr} cols={c} splits={sp} call {rep}")
        assert torch.equal(outs[0], outs[1]), f"wr={wr} cols={c} splits={sp}: repeated call differs"


def test_linear_plan_validation(dev, ssm):
    lib = ssm.load_library()
    assert lib.ssm_linear_workspace_ex(245, 2560, 5120, 128, 0, 0) == 0
    assert lib.ssm_linear_workspace_ex(245, 2560, 5120, 48, 0, 0) == 0
    assert lib.ssm_linear_workspace_ex(245, 2560, 5120, 0, 96, 0) == 0
    assert lib.ssm_linear_workspace_ex(245, 2560, 5120, 0, 0, 81) == 0  # more splits than 64-k batches
    x = torch.zeros(8, 64, dtype=torch.float16, device=dev)
    w = torch.zeros(16, 64, dtype=torch.float16, device=dev)
    out = torch.zeros(8, 16, dtype=torch.float16, device=dev)
    T = ssm._tensor
    code = {v: k for k, v in ssm.STATUS.items()}
    call = lambda wr, c, sp: lib.ssm_linear_ex(T(x, "x"), T(w, "w"), T(None, "r"), T(out, "o"), 8, 16, 64,
                                               wr, c, sp, None, 0, None)
    assert call(128, 0, 0) == code["SSM_ERR_OUT_OF_RESOURCES"]
    assert call(0, 256, 0) == code["SSM_ERR_OUT_OF_RESOURCES"]
    assert call(16, 64, 2) == code["SSM_ERR_SHAPE"]  # more splits than the one 64-k batch


@pytest.mark.parametrize("dt", [torch.float16, torch.bfloat16])
def test_linear_unaligned_output(dev, ssm, dt):
    """An output (and residual) only 2-byte aligned: the main kernel's stores
    fall back from 8-byte to element stores."""
    from oracle import layer

    M, N, K = 40, 96, 136
    g = torch.Generator(device=dev).manual_seed(11)
    x = torch.randn(M, K, generator=g, device=dev).to(dt)
    w = (torch.randn(N, K, generator=g, device=dev) / K ** 0.5).to(dt)
    rbuf = torch.randn(M * N + 1, generator=g, device=dev).to(dt)
    r = rbuf[1:].view(M, N)
    obuf = torch.zeros(M * N + 1, device=dev, dtype=dt)
    out = obuf[1:].view(M, N)
    ssm.linear(x, w, residual=r, out=out)
    torch.cuda.synchronize()
    assert obuf[0].item() == 0.0
    o, s = layer.linear(f(x), f(w), residual=f(r))
    check(out, o, s, 3e-3, "f16" if dt == torch.float16 else "bf16", "linear unaligned")


# widths: one round of 128-bit loads per lane (520: a partial second round),
# the 2.8B model's 2560, the largest vector width, and widths that take the
# element-wise kernel (not a multiple of 8; past the vector form's limit)
@pytest.mark.parametrize("D", [520, 2560, 8192, 100, 8200])
@pytest.mark.parametrize("dt", [torch.float16, torch.bfloat16])
def test_rmsnorm_parity(dev, ssm, dt, D):
    from oracle import layer

    g = torch.Generator(device=dev).manual_seed(3)
    x = (torch.randn(37, D, generator=g, device=dev) * 3).to(dt)
    w = torch.rand(D, generator=g, device=dev) + 0.5
    out = ssm.rmsnorm(x, w, eps=1e-5)
    torch.cuda.synchronize()
    o, s = layer.rmsnorm(f(x), f(w), 1e-5)
    check(out, o, s, 3e-3, "f16" if dt == torch.float16 else "bf16", f"rmsnorm D={D}")


def test_rmsnorm_strided_rows(dev, ssm):
    """Rows 4 elements apart from 8-aligned (the element-wise kernel) and a
    view of every other row (the vector kernel), against the oracle."""
    from oracle import layer

    g = torch.Generator(device=dev).manual_seed(4)
    w = torch.rand(512, generator=g, device=dev) + 0.5
    for ld, rows in ((516, slice(None)), (1024, slice(None, None, 2))):
        base = (torch.randn(21, ld, generator=g, device=dev) * 2).to(torch.float16)
        x = base[:, :512] if rows == slice(None) else base.view(-1, 512)[rows]
        out = ssm.rmsnorm(x, w, eps=1e-6)
        torch.cuda.synchronize()
        o, s = layer.rmsnorm(f(x), f(w), 1e-6)
        check(out, o, s, 3e-3, "f16", f"rmsnorm ld={ld}")


LAYER_CASES = [
    # (label, mamba1_layer kwargs, pad every)
    ("small_f16", dict(d_model=256, d_inner=512, d_state=16, dt_rank=32, batch=5, nslots=9,
                       io="f16", state="f32"), 0),
    ("small_bf16_pad", dict(d_model=128, d_inner=256, d_state=16, dt_rank=16, batch=6, nslots=8,
                            io="bf16", state="bf16"), 3),
    ("mamba1_2.8b_b16", dict(batch=16, nslots=20, io="f16", state="f32"), 5),
]


@pytest.mark.parametrize("label,kw,pad", LAYER_CASES, ids=[c[0] for c in LAYER_CASES])
def test_decode_layer_parity(dev, ssm, oracle, label, kw, pad):
    from oracle import layer

    t = W.mamba1_layer(seed=11, device=dev, **kw)
    idx = t["slot_idx"].clone()
    if pad:
        idx[::pad] = -1
    h0, cs0, ss0 = t["hidden"].clone(), t["conv_state"].clone(), t["ssm_state"].clone()
    desc = ssm.mamba1_layer(t["w"], eps=1e-5)
    ssm.mamba1_decode_layer(desc, t["hidden"], t["conv_state"], t["ssm_state"], slot_idx=idx)
    torch.cuda.synchronize()
    kind = oracle.F16 if kw["io"] == "f16" else oracle.BF16
    wf = {k: f(v) for k, v in t["w"].items()}
    idx_np = idx.cpu().numpy()
    stages = {}
    o, s, cs, ss, sss = layer.mamba1_decode_layer(wf, f(h0), f(cs0), f(ss0), idx_np, eps=1e-5,
                                                  round_kind=kind, stages=stages)
    check(t["hidden"], o, s, 3e-3, kw["io"], f"layer {label} hidden")
    named = idx_np[idx_np >= 0]
    check(f(t["ssm_state"])[named], ss[named], sss[named], 3e-3, kw["state"], f"layer {label} state")
    others = np.setdiff1d(np.arange(cs0.shape[0]), named)
    np.testing.assert_array_equal(f(t["conv_state"])[others], f(cs0)[others])
    np.testing.assert_array_equal(f(t["ssm_state"])[others], f(ss0)[others])
    # conv windows: the old samples shift by one exactly; the newest is this
    # step's x (a projection output, compared at the projection's tolerance)
    gcs = f(t["conv_state"])[named]
    np.testing.assert_array_equal(gcs[:, :, :-1], f(cs0)[named][:, :, 1:])
    live = idx_np >= 0
    _, xs = layer.linear(stages["hn"], wf["in_proj"])
    d_inner = wf["in_proj"].shape[0] // 2
    check(gcs[:, :, -1], stages["x"][live], xs[live][:, :d_inner], 3e-3, kw["io"],
          f"layer {label} conv window")


def test_decode_layer_batch245_sampled_rows(dev, ssm, oracle):
    """The layer at the size the benchmark runs (Mamba-2.8B dimensions, 245
    requests from a 512-slot cache, f16 I/O, f32 state), every fifth request
    padded.  The requests are independent, so the oracle runs only a sample
    of them (with their slots) and each sampled row is compared in full."""
    from oracle import layer

    t = W.mamba1_layer(seed=13, device=dev, batch=245, nslots=512, io="f16", state="f32")
    idx = t["slot_idx"].clone()
    idx[::5] = -1
    h0, cs0, ss0 = t["hidden"].clone(), t["conv_state"].clone(), t["ssm_state"].clone()
    desc = ssm.mamba1_layer(t["w"], eps=1e-5)
    ssm.mamba1_decode_layer(desc, t["hidden"], t["conv_state"], t["ssm_state"], slot_idx=idx)
    torch.cuda.synchronize()
    idx_np = idx.cpu().numpy()
    rows = np.array([0, 1, 2, 77, 128, 200, 243, 244])  # 0 and 200 are padded
    wf = {k: f(v) for k, v in t["w"].items()}
    o, s, cs, ss, sss = layer.mamba1_decode_layer(wf, f(h0)[rows], f(cs0), f(ss0), idx_np[rows],
                                                  eps=1e-5, round_kind=oracle.F16)
    check(f(t["hidden"])[rows], o, s, 3e-3, "f16", "layer b245 hidden (sampled rows)")
    named = idx_np[rows][idx_np[rows] >= 0]
    check(f(t["ssm_state"])[named], ss[named], sss[named], 3e-3, "f32", "layer b245 state (sampled slots)")
    np.testing.assert_array_equal(f(t["conv_state"])[named][:, :, :-1], f(cs0)[named][:, :, 1:])
    # padded requests: hidden rows untouched
    pad = np.nonzero(idx_np < 0)[0]
    np.testing.assert_array_equal(f(t["hidden"])[pad], f(h0)[pad])
    # slots no request names: untouched
    others = np.setdiff1d(np.arange(512), idx_np[idx_np >= 0])
    np.testing.assert_array_equal(f(t["ssm_state"])[others], f(ss0)[others])
    np.testing.assert_array_equal(f(t["conv_state"])[others], f(cs0)[others])
