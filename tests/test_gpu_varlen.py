"""GPU parity of the packed variable-length prefill (ssm_causal_conv1d_varlen,
ssm_selective_scan_varlen) against the float64 oracle, whose varlen entries
run each sequence as an independent dense call.

Length mixes include empty sequences, sequences shorter than the conv window,
sequences straddling 256-step tiles, starts at every offset within a 128-bit
vector (packed totals that are multiples of 8 take the vector path, the others
the scalar path), padded sequences, and a mix of sequences that continue from
their slot and fresh ones.  Tolerances as in test_gpu_parity.py; conv tails,
unnamed slots and padded sequences' columns bit-exact.
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


VARLEN_CASES = [
    # (label, spec kwargs, lengths, padded sequence index (or list) or None)
    ("m1_f16_vec_mix", dict(io="f16", state="f32", nheads=64, nslots=16, seed=11),
     [0, 1, 2, 3, 5, 17, 255, 256, 257, 700], 4),                     # total 1496 (vec)
    ("m1_f16_scalar_mix", dict(io="f16", state="f16", nheads=40, nslots=8, seed=12),
     [3, 100, 901], None),                                           # total 1004
    ("m1_bf16_w2", dict(io="bf16", state="bf16", nheads=24, width=2, nslots=9, seed=13),
     [513, 7, 1, 0, 129, 30], 1),                                     # total 680 (vec)
    ("m1_f32_w3_N20", dict(io="f32", state="f32", nheads=20, dstate=20, width=3, nslots=6,
                           seed=14), [9, 600, 31, 2], None),          # total 642
    ("m1_f32_vec_w1", dict(io="f32", state="f32", nheads=16, width=1, nslots=5, seed=15),
     [4, 8, 300, 1, 39], None),                                       # total 352 (vec)
    ("m2_f32_G2_N64", dict(io="f32", state="f32", nheads=4, headdim=16, dstate=64, ngroups=2,
                           a_per_state=False, nslots=7, seed=16), [40, 300, 1, 83], 2),  # 424
    ("m2_bf16_N128", dict(io="bf16", state="f32", nheads=2, headdim=32, dstate=128,
                          a_per_state=False, nslots=4, seed=17), [261, 0, 6, 3], None),  # 270
    ("m2_f16_N16_G4", dict(io="f16", state="bf16", nheads=8, headdim=4, dstate=16, ngroups=4,
                           a_per_state=False, nslots=6, seed=18), [1, 1, 510, 8], 0),   # 520
    # plain tables (no padded sequence, vector totals): the conv runs the dense
    # kernel over the packed rows, and the tail pass redoes each sequence's
    # first width-1 outputs from its history, here for sequences shorter
    # than the window too
    ("m1_f16_vec_mix_plain", dict(io="f16", state="f32", nheads=64, nslots=16, seed=21),
     [0, 1, 2, 3, 5, 17, 255, 256, 257, 700], None),                  # total 1496 (vec)
    ("m1_f32_w3_plain", dict(io="f32", state="f32", nheads=20, dstate=20, width=3, nslots=8,
                             seed=22), [9, 600, 31, 0, 2, 6], None),  # total 648 (vec)
    # a padded sequence in packed rows of several conv tiles (2048 f16 or 1024
    # f32 columns): the dense walk stores around the padded columns
    # (a padded first sequence: m2_f16_N16_G4)
    ("m1_f16_padded_3_tiles", dict(io="f16", state="f32", nheads=8, nslots=8, seed=23),
     [1500, 3, 2000, 1497], 1),                                      # total 5000 (vec)
    ("m1_f32_w2_padded_3_tiles", dict(io="f32", state="f32", nheads=6, width=2, nslots=8,
                                      seed=24), [700, 900, 5, 795], 3),  # total 2400 (vec)
    # more than 8 padded sequences: the row kernel walks each row tile by
    # tile with the start-aware code, a barrier between tiles
    ("m1_f16_10_padded_3_tiles", dict(io="f16", state="f32", nheads=8, nslots=24, seed=26),
     W.varlen_lengths(26, 20, 5000), [0, 2, 3, 4, 6, 8, 10, 12, 16, 18]),  # total 5000 (vec)
    # packed rows of several conv tiles (2048 f16 or 1024 f32 columns):
    # sequences that start one or two columns before a tile's end, so that
    # their first width-1 outputs span two tiles, with and without a
    # history; one that starts on a tile boundary; and a padded sequence
    # next to them
    ("m1_f16_starts_at_tile_edges", dict(io="f16", state="f32", nheads=8, nslots=8, seed=28),
     [5, 2042, 3, 1, 2045, 8], None),                                # total 4104 (vec)
    ("m1_f16_start_before_edge_padded", dict(io="f16", state="f16", nheads=6, nslots=8, seed=29),
     [6, 2040, 700, 6], 3),                                          # total 2752 (vec)
    ("m1_f32_start_at_tile_edge", dict(io="f32", state="f32", nheads=6, nslots=8, seed=30),
     [1021, 1, 4, 900, 2], None),                                    # total 1928 (vec)
    ("m1_bf16_w2_start_at_tile_edge", dict(io="bf16", state="f32", nheads=4, width=2, nslots=8, seed=31),
     [2047, 2, 7, 2000], 0),                                         # total 4056 (vec)
    # Mamba-2 shapes that take the chunked matrix form (16-bit I/O, headdim a
    # multiple of 64, dstate 64/128/256): sequences shorter than a chunk, a
    # vector or a step, starting mid-vector, padded and empty ones
    ("m2_bf16_hd64_N128_chunked", dict(io="bf16", state="f32", nheads=2, headdim=64, dstate=128,
                                       a_per_state=False, nslots=8, seed=32),
     [100, 3, 0, 517, 64, 9, 307], 1),                                 # total 1000 (vec)
    ("m2_f16_hd128_N256_chunked", dict(io="f16", state="bf16", nheads=1, headdim=128, dstate=256,
                                       a_per_state=False, nslots=6, seed=33),
     [1, 130, 64, 7, 598], None),                                      # total 800 (vec)
    ("m2_f16_hd64_N64_G2_chunked", dict(io="f16", state="f16", nheads=4, headdim=64, dstate=64,
                                        ngroups=2, a_per_state=False, nslots=9, seed=34),
     [65, 0, 2, 127, 8, 70], 2),                                       # total 272 (vec)
    # more sequences than the conv kernel stages in LDS (its global-table path)
    ("m1_f16_300_seqs", dict(io="f16", state="f32", nheads=8, nslots=320, seed=19),
     [0, 3] + W.varlen_lengths(19, 298, 2395), None),                    # total 2398
    # many sequences, none padded: every tile takes the staged path
    ("m1_bf16_200_seqs", dict(io="bf16", state="f32", nheads=8, nslots=210, seed=20),
     W.varlen_lengths(20, 200, 3000), None),                             # total 3000 (vec)
]


def _run(ssm, oracle, dev, spec, lengths, pad, init_every=2):
    t = W.make_varlen(spec, lengths, dev, init_every=init_every)
    if pad is not None:
        t["slot_idx"][pad] = -1
    idx_np = t["slot_idx"].cpu().numpy()
    hin = t["has_init"].cpu().numpy()
    cu = t["cu_seqlens"]
    cs0, st0 = t["conv_state"].clone(), t["ssm_state"].clone()
    u0 = torch.full_like(t["x"], 7.0)
    out0 = torch.full_like(t["x"], 5.0)
    u = ssm.causal_conv1d_varlen(t["x"], t["conv_w"], cu, bias=t["conv_b"],
                                 conv_state=t["conv_state"], slot_idx=t["slot_idx"],
                                 has_initial_state=t["has_init"], out=u0.clone())
    out = ssm.selective_scan_varlen(u, t["dt"], t["A"], t["B"], t["C"], cu, D=t["D"], z=t["z"],
                                    dt_bias=t["dt_bias"], ssm_state=t["ssm_state"],
                                    slot_idx=t["slot_idx"], has_initial_state=t["has_init"],
                                    out=out0.clone())
    torch.cuda.synchronize()
    return t, u, out, dict(idx=idx_np, hin=hin, cu=cu.cpu().numpy(), cs0=cs0, st0=st0, u0=u0,
                           out0=out0)


@pytest.mark.parametrize("label,kw,lengths,pad", VARLEN_CASES, ids=[c[0] for c in VARLEN_CASES])
def test_varlen_prefill_parity(dev, ssm, oracle, label, kw, lengths, pad):
    spec = W.tiny(**kw)
    t, u, out, r = _run(ssm, oracle, dev, spec, lengths, pad)
    # conv against the oracle on the same inputs
    uo, us, cs = oracle.causal_conv1d_varlen(f(t["x"]), f(t["conv_w"]), r["cu"], f(t["conv_b"]),
                                             f(r["cs0"]), r["idx"], r["hin"], out=f(r["u0"]))
    check(u, uo, us, RTOL[spec.io], spec.io, f"varlen conv {label}")
    np.testing.assert_array_equal(f(t["conv_state"]), cs)
    # scan on the GPU's own conv output (the stored u), so the two stages are
    # checked separately
    o, s, st, sts = oracle.selective_scan_varlen(
        f(u), f(t["dt"]), f(t["A"]), f(t["B"]), f(t["C"]), r["cu"], D=f(t["D"]), z=f(t["z"]),
        dt_bias=f(t["dt_bias"]), state=f(r["st0"]), slot_idx=r["idx"], has_initial_state=r["hin"],
        out=f(r["out0"]))
    check(out, o, s, RTOL[spec.io], spec.io, f"varlen scan {label}")
    lens = np.diff(r["cu"])
    named = np.array([sl for sl, n in zip(r["idx"], lens) if sl >= 0 and n > 0], dtype=np.int64)
    gst = f(t["ssm_state"])
    if named.size:
        check(gst[named], st[named], sts[named], RTOL[spec.io], spec.state, f"varlen state {label}")
    others = np.setdiff1d(np.arange(gst.shape[0]), named)
    np.testing.assert_array_equal(gst[others], f(r["st0"])[others])


@pytest.mark.parametrize("io", ["f16", "f32"])
def test_varlen_equal_lengths_match_dense_kernels(dev, ssm, io):
    # sequences of one length packed side by side give the dense call's
    # results: the conv's bits, and the scan's up to the order of its sums
    # (the packed scan walks 8 steps per lane, the dense one 16), within the
    # parity tolerance of the io dtype; both are checked against the oracle
    # elsewhere
    spec = W.tiny(io=io, state="f32", nheads=48, nslots=6, seed=21)
    L, nseq = 264, 3
    t = W.make_varlen(spec, [L] * nseq, dev, init_every=1)
    cu, idx = t["cu_seqlens"], t["slot_idx"]
    cs_v, st_v = t["conv_state"].clone(), t["ssm_state"].clone()
    cs_d, st_d = t["conv_state"].clone(), t["ssm_state"].clone()
    u_v = ssm.causal_conv1d_varlen(t["x"], t["conv_w"], cu, bias=t["conv_b"], conv_state=cs_v,
                                   slot_idx=idx, has_initial_state=t["has_init"])
    o_v = ssm.selective_scan_varlen(u_v, t["dt"], t["A"], t["B"], t["C"], cu, D=t["D"], z=t["z"],
                                    dt_bias=t["dt_bias"], ssm_state=st_v, slot_idx=idx,
                                    has_initial_state=t["has_init"])

    def dense(a):  # [rows..., nseq*L] -> [nseq, rows..., L]
        return torch.stack(a.split(L, dim=-1)).contiguous()

    u_d = ssm.causal_conv1d(dense(t["x"]), t["conv_w"], t["conv_b"], conv_state=cs_d,
                            slot_idx=idx, has_initial_state=True)
    o_d = ssm.selective_scan(u_d, dense(t["dt"]), t["A"], dense(t["B"]), dense(t["C"]), D=t["D"],
                             z=dense(t["z"]), dt_bias=t["dt_bias"], ssm_state=st_d, slot_idx=idx,
                             has_initial_state=True)
    torch.cuda.synchronize()
    assert torch.equal(dense(u_v), u_d)
    assert torch.equal(cs_v, cs_d)
    rtol = RTOL[io]
    ov, od = dense(o_v).double(), o_d.double()
    # |difference| <= rtol * max|o| + half an ulp of the io dtype at |o|
    tol = rtol * od.abs().max() + 0.5 * od.abs() * (2.0 ** -10 if io == "f16" else 2.0 ** -23)
    assert bool(((ov - od).abs() <= tol).all())
    sv, sd = st_v.double(), st_d.double()
    assert bool(((sv - sd).abs() <= 1e-5 * sd.abs().max()).all())


@pytest.mark.parametrize("io", ["bf16", "f16"])
def test_varlen_mamba2_chunked_matches_dense(dev, ssm, io):
    # packed sequences of one length (a multiple of 8, so every sequence
    # starts on a vector) walk the same chunks as the dense call: the chunked
    # Mamba-2 scan gives the same bits either way
    spec = W.tiny(io=io, state="f32", nheads=2, headdim=64, dstate=128, a_per_state=False,
                  nslots=6, seed=35)
    L, nseq = 264, 3
    t = W.make_varlen(spec, [L] * nseq, dev, init_every=1)
    cu, idx = t["cu_seqlens"], t["slot_idx"]
    st_v, st_d = t["ssm_state"].clone(), t["ssm_state"].clone()
    o_v = ssm.selective_scan_varlen(t["x"], t["dt"], t["A"], t["B"], t["C"], cu, D=t["D"], z=t["z"],
                                    dt_bias=t["dt_bias"], ssm_state=st_v, slot_idx=idx,
                                    has_initial_state=t["has_init"])

    def dense(a):  # [rows..., nseq*L] -> [nseq, rows..., L]
        return torch.stack(a.split(L, dim=-1)).contiguous()

    o_d = ssm.selective_scan(dense(t["x"]), dense(t["dt"]), t["A"], dense(t["B"]), dense(t["C"]),
                             D=t["D"], z=dense(t["z"]), dt_bias=t["dt_bias"], ssm_state=st_d,
                             slot_idx=idx, has_initial_state=True, algo=ssm.SCAN_CHUNKED)
    torch.cuda.synchronize()
    assert torch.equal(dense(o_v), o_d)
    assert torch.equal(st_v, st_d)


def test_varlen_all_empty_is_noop(dev, ssm):
    spec = W.tiny(io="f16", nheads=16, nslots=3, seed=22)
    t = W.make_varlen(spec, [5, 3], dev)
    cu = torch.zeros(3, dtype=torch.int32, device=dev)  # every sequence empty
    cs0, st0 = t["conv_state"].clone(), t["ssm_state"].clone()
    u = torch.full_like(t["x"], 3.0)
    ssm.causal_conv1d_varlen(t["x"], t["conv_w"], cu, bias=t["conv_b"], conv_state=t["conv_state"],
                             slot_idx=t["slot_idx"], has_initial_state=t["has_init"], out=u)
    out = torch.full_like(t["x"], 3.0)
    ssm.selective_scan_varlen(t["x"], t["dt"], t["A"], t["B"], t["C"], cu, D=t["D"],
                              ssm_state=t["ssm_state"], slot_idx=t["slot_idx"],
                              has_initial_state=t["has_init"], out=out)
    torch.cuda.synchronize()
    assert bool((u == 3.0).all()) and bool((out == 3.0).all())
    assert torch.equal(t["conv_state"], cs0) and torch.equal(t["ssm_state"], st0)


def test_varlen_then_decode_continues(dev, ssm, oracle):
    # continuous batching: a packed prefill leaves each sequence's conv window
    # and state in its slot; one fused decode step then continues every
    # sequence exactly as the oracle's prefill over length+1 would
    spec = W.tiny(io="f32", state="f32", nheads=32, nslots=8, seed=23)
    lengths = [1, 2, 130, 57]
    t = W.make_varlen(spec, lengths, dev, init_every=0)
    cu = t["cu_seqlens"]
    u = ssm.causal_conv1d_varlen(t["x"], t["conv_w"], cu, bias=t["conv_b"],
                                 conv_state=t["conv_state"], slot_idx=t["slot_idx"])
    ssm.selective_scan_varlen(u, t["dt"], t["A"], t["B"], t["C"], cu, D=t["D"], z=t["z"],
                              dt_bias=t["dt_bias"], ssm_state=t["ssm_state"], slot_idx=t["slot_idx"])
    g = torch.Generator(device=dev).manual_seed(5)
    nseq, H = len(lengths), spec.nheads
    xd = torch.randn(nseq, H, 1, generator=g, device=dev)
    zd = torch.randn(nseq, H, 1, generator=g, device=dev)
    dtd = torch.randn(nseq, H, generator=g, device=dev)
    Bd = torch.randn(nseq, 1, spec.dstate, generator=g, device=dev)
    Cd = torch.randn(nseq, 1, spec.dstate, generator=g, device=dev)
    yd = ssm.decode_step(t["ssm_state"], t["conv_state"], xd, t["conv_w"], dtd, t["A"], Bd, Cd,
                         conv_bias=t["conv_b"], D=t["D"], z=zd, dt_bias=t["dt_bias"],
                         slot_idx=t["slot_idx"])
    torch.cuda.synchronize()
    x, z, dt, B, C = (f(t[k]) for k in ("x", "z", "dt", "B", "C"))
    cuv = cu.cpu().numpy()
    for s in range(nseq):
        tb, te = cuv[s], cuv[s + 1]
        xs = np.concatenate([x[:, tb:te], f(xd)[s].reshape(H, 1)], axis=1)[None]
        uo, _, _ = oracle.causal_conv1d(xs, f(t["conv_w"]), f(t["conv_b"]))
        o, sc, _, _ = oracle.selective_scan(
            uo, np.concatenate([dt[:, tb:te], f(dtd)[s][:, None]], axis=1)[None], f(t["A"]),
            np.concatenate([B[:, :, tb:te], f(Bd)[s][:, :, None]], axis=2)[None],
            np.concatenate([C[:, :, tb:te], f(Cd)[s][:, :, None]], axis=2)[None], D=f(t["D"]),
            z=np.concatenate([z[:, tb:te], f(zd)[s].reshape(H, 1)], axis=1)[None],
            dt_bias=f(t["dt_bias"]))
        # the last step of the long prefill is the decode token; the GPU's
        # decode reads u in float32, as does this float64 chain
        check(yd[s].reshape(H), o[0, :, -1], sc[0, :, -1], 1e-5, "f32", f"decode after varlen {s}")


@pytest.mark.parametrize("io,silu", [("f16", True), ("f32", False)])
def test_varlen_conv_without_cache(dev, ssm, oracle, io, silu):
    """No conv cache, no slot table, no bias: every sequence starts from zeros
    (the row kernel's start fix-up with an empty history), with and without
    the SiLU."""
    spec = W.tiny(io=io, state="f32", nheads=16, nslots=8, seed=25)
    lengths = [3, 1, 700, 0, 2, 90, 4]  # total 800 (vector rows)
    t = W.make_varlen(spec, lengths, dev)
    cu = t["cu_seqlens"]
    u = ssm.causal_conv1d_varlen(t["x"], t["conv_w"], cu, apply_silu=silu)
    torch.cuda.synchronize()
    uo, us, _ = oracle.causal_conv1d_varlen(f(t["x"]), f(t["conv_w"]), cu.cpu().numpy(),
                                            apply_silu=silu)
    check(u, uo, us, RTOL[io], io, f"varlen conv without cache {io}")
