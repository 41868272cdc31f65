"""Pins for the float64 oracle: every check here compares the oracle with
something other than itself -- closed forms, textbook special cases, brute
force on tiny inputs, and invariants between independent oracle loops (the
scan and the single-token update are separate functions).  CPU only.

Each case says which mistake it is there to catch.
"""
import math

import numpy as np
import pytest


def rng(seed):
    return np.random.default_rng(seed)


# ----------------------------------------------------------------- scalar maps
def test_softplus_special_values(oracle):
    # softplus(0) = ln 2; softplus(v) - softplus(-v) = v for every v (a dropped
    # max(v,0) term or a sign slip breaks it); far tails: e^v and v.
    assert oracle.softplus(0.0) == pytest.approx(math.log(2.0), rel=1e-15)
    for v in np.linspace(-30, 30, 61):
        assert oracle.softplus(v) - oracle.softplus(-v) == pytest.approx(v, abs=1e-12)
    # (absolute tolerance 0: the naive log(1 + e^v) returns 0 at v = -40)
    assert oracle.softplus(-40.0) == pytest.approx(math.exp(-40.0), rel=1e-15, abs=0)
    assert oracle.softplus(-12.0) == pytest.approx(math.exp(-12.0) - math.exp(-24.0) / 2
                                                   + math.exp(-36.0) / 3, rel=1e-15, abs=0)
    for v in (-25.0, -18.0, -9.5):
        assert oracle.softplus(v) == pytest.approx(math.log1p(math.exp(v)), rel=1e-15, abs=0)
    assert oracle.softplus(700.0) == 700.0
    assert oracle.softplus(710.0) == 710.0


def test_silu_special_values(oracle):
    assert oracle.silu(0.0) == 0.0
    # silu(v) - silu(-v) = v, silu(v) -> v for large v, -> 0 for very negative
    for v in np.linspace(-20, 20, 41):
        assert oracle.silu(v) - oracle.silu(-v) == pytest.approx(v, abs=1e-12)
    assert oracle.silu(1.0) == pytest.approx(1.0 / (1.0 + math.exp(-1.0)), rel=1e-15)
    assert oracle.silu(50.0) == pytest.approx(50.0, rel=1e-15)
    assert abs(oracle.silu(-50.0)) < 1e-19
    assert oracle.silu(-30.0) == pytest.approx(-30.0 * math.exp(-30.0), rel=1e-12, abs=0)


# ----------------------------------------------------------- rounding helpers
def _wide_sample(seed, n=20000):
    r = rng(seed)
    mant = r.uniform(-2, 2, n)
    ex = r.integers(-160, 140, n)
    v = mant * np.exp2(ex.astype(np.float64))
    # exact ties and near-ties in the f16/bf16 grids
    ties = (np.arange(1, 200) + 0.5) * 2.0 ** -10
    return np.concatenate([v, ties, -ties, [0.0, -0.0, 65504.0, 65520.0, 65519.99, 6e-8, 3e-8]])


def test_round_f16_matches_numpy(oracle):
    v = _wide_sample(1)
    got = oracle.round_to(v, oracle.F16)
    with np.errstate(over="ignore"):
        want = v.astype(np.float16).astype(np.float64)
    np.testing.assert_array_equal(got, want)


def test_round_f32_matches_numpy(oracle):
    v = _wide_sample(2)
    got = oracle.round_to(v, oracle.F32)
    with np.errstate(over="ignore"):
        want = v.astype(np.float32).astype(np.float64)
    np.testing.assert_array_equal(got, want)


def _bf16_brute(v):
    """Nearest bfloat16 by enumerating the two neighbours in float32 bit space;
    ties go to the even bit pattern."""
    out = np.empty_like(v)
    for i, x in enumerate(v):
        if x == 0 or not np.isfinite(x):
            out[i] = x
            continue
        f = np.float32(x)  # only to find the binade; neighbours are exact below
        bits = int(np.array([f], dtype=np.float32).view(np.uint32)[0]) & 0xFFFF0000
        cands = []
        for db in (-0x10000, 0, 0x10000):
            b = (bits + db) & 0xFFFFFFFF
            c = float(np.array([b], dtype=np.uint32).view(np.float32)[0])
            if np.isfinite(c):
                cands.append((abs(c - x), (b >> 16) & 1, c))
        cands.sort()
        best = cands[0]
        if len(cands) > 1 and cands[1][0] == best[0] and best[1] == 1:
            best = cands[1]
        out[i] = best[2]
    return out


def test_round_bf16_brute_force(oracle):
    v = _wide_sample(3, n=3000)
    v = v[(np.abs(v) < 3e38) & ((np.abs(v) > 1e-36) | (v == 0))]
    got = oracle.round_to(v, oracle.BF16)
    want = _bf16_brute(v)
    np.testing.assert_array_equal(got, want)


# ---------------------------------------------------------------------- conv
def _conv_case(seed, batch=2, channels=5, seqlen=13, width=4):
    r = rng(seed)
    x = r.standard_normal((batch, channels, seqlen))
    w = r.uniform(-0.5, 0.5, (channels, width))
    b = r.uniform(-0.5, 0.5, channels)
    cs = r.standard_normal((batch + 2, channels, width - 1))
    return x, w, b, cs


@pytest.mark.parametrize("width", [1, 2, 4])
@pytest.mark.parametrize("init", [False, True])
def test_conv_matches_numpy_convolve(oracle, width, init):
    # brute force: direct correlation of the left-extended row with the taps
    # (catches a reversed tap order, an off-by-one in the history window, a
    # dropped bias, a missing SiLU)
    x, w, b, cs = _conv_case(10 + width, width=width)
    idx = np.array([3, 0], dtype=np.int32)
    out, sc, cs_new = oracle.causal_conv1d(x, w, b, cs, idx, has_initial_state=init,
                                           apply_silu=True)
    for bi in range(x.shape[0]):
        s = idx[bi]
        for c in range(x.shape[1]):
            hist = cs[s, c] if init else np.zeros(width - 1)
            ext = np.concatenate([hist, x[bi, c]])
            acc = np.convolve(ext, w[c][::-1], mode="valid") + b[c]
            np.testing.assert_allclose(out[bi, c], acc / (1 + np.exp(-acc)), rtol=1e-13, atol=1e-14)
            assert np.all(sc[bi, c] >= np.abs(out[bi, c]) - 1e-12)
            # tail: last W-1 of the extended row, copied exactly
            np.testing.assert_array_equal(cs_new[s, c], ext[len(ext) - (width - 1):])
    # slots not named are untouched, bit for bit
    for s in (1, 2):
        np.testing.assert_array_equal(cs_new[s], cs[s])


def test_conv_short_sequence_tail(oracle):
    # L < W-1: the tail mixes old history and new samples
    x, w, b, cs = _conv_case(20, seqlen=2, width=4)
    out, _, cs_new = oracle.causal_conv1d(x, w, b, cs, None, has_initial_state=True)
    for bi in range(2):
        for c in range(5):
            ext = np.concatenate([cs[bi, c], x[bi, c]])
            np.testing.assert_array_equal(cs_new[bi, c], ext[-3:])


def test_conv_prefill_equals_chained_decode(oracle):
    # invariant: one prefill over L tokens == L single-token updates from the
    # same history (outputs to rounding, cache bit-exact)
    x, w, b, cs = _conv_case(30, seqlen=9)
    out_p, _, cs_p = oracle.causal_conv1d(x, w, b, cs, None, has_initial_state=True)
    cs_d = cs.copy()
    outs = []
    for t in range(x.shape[2]):
        o, _, cs_d = oracle.causal_conv1d(x[:, :, t:t + 1], w, b, cs_d, None,
                                          has_initial_state=True)
        outs.append(o)
    np.testing.assert_allclose(np.concatenate(outs, axis=2), out_p, rtol=1e-14, atol=1e-15)
    np.testing.assert_array_equal(cs_d, cs_p)


def test_conv_padded_request_untouched(oracle):
    x, w, b, cs = _conv_case(40)
    idx = np.array([-1, 2], dtype=np.int32)
    init_out = np.full(x.shape, 7.0)
    out, _, cs_new = oracle.causal_conv1d(x, w, b, cs, idx, has_initial_state=True, out=init_out)
    np.testing.assert_array_equal(out[0], init_out[0])
    for s in (0, 1, 3):
        np.testing.assert_array_equal(cs_new[s], cs[s])


# ---------------------------------------------------------------------- scan
def _scan_case(seed, batch=2, seqlen=17, nheads=3, headdim=1, dstate=4, ngroups=1,
               a_per_state=True):
    r = rng(seed)
    Cn = nheads * headdim
    u = r.standard_normal((batch, Cn, seqlen))
    z = r.standard_normal((batch, Cn, seqlen))
    dt = r.standard_normal((batch, nheads, seqlen))
    dt_bias = r.uniform(math.log(1e-3), math.log(1e-1), nheads)
    A = -r.uniform(0.5, 4.0, (nheads, dstate)) if a_per_state else -r.uniform(1, 16, nheads)
    B = r.standard_normal((batch, ngroups, dstate, seqlen))
    C = r.standard_normal((batch, ngroups, dstate, seqlen))
    D = r.uniform(0.5, 1.5, nheads)
    state = r.standard_normal((batch + 1, nheads, headdim, dstate))
    return dict(u=u, z=z, dt=dt, dt_bias=dt_bias, A=A, B=B, C=C, D=D, state=state)


def _softplus(v):
    return np.maximum(v, 0) + np.log1p(np.exp(-np.abs(v)))


def test_scan_geometric_series(oracle):
    # constant delta, B, u, C: h_t = b(1 - a^{t+1})/(1 - a) from h_{-1} = 0,
    # a = exp(delta A), b = delta B u; y_t = sum_n C h_t[n] + D u
    # (catches an exponent sign error, a missing delta in either term, an
    # off-by-one in the first step)
    L, N = 40, 3
    delta_raw, bias = 0.3, -1.0
    delta = math.log1p(math.exp(delta_raw + bias))
    A = np.array([[-0.5, -1.5, -3.0]])
    Bv = np.array([0.7, -1.1, 0.4])
    Cv = np.array([1.3, 0.2, -0.8])
    u0, D = 0.9, 0.6
    u = np.full((1, 1, L), u0)
    dt = np.full((1, 1, L), delta_raw)
    B = np.repeat(Bv[None, None, :, None], L, axis=3)
    C = np.repeat(Cv[None, None, :, None], L, axis=3)
    out, _, st, _ = oracle.selective_scan(u, dt, A, B, C, D=np.array([D]), z=None,
                                          dt_bias=np.array([bias]),
                                          state=np.zeros((1, 1, 1, N)))
    a = np.exp(delta * A[0])
    b = delta * Bv * u0
    t = np.arange(L)[:, None]
    h = b * (1 - a ** (t + 1)) / (1 - a)
    y = h @ Cv + D * u0
    np.testing.assert_allclose(out[0, 0], y, rtol=1e-12)
    np.testing.assert_allclose(st[0, 0, 0], h[-1], rtol=1e-12)


def test_scan_zero_A_is_prefix_sum(oracle):
    # A = 0 => abar = 1 exactly => h is the running sum of delta*B*u
    c = _scan_case(1, a_per_state=True)
    c["A"] = np.zeros_like(c["A"])
    out, _, st, _ = oracle.selective_scan(c["u"], c["dt"], c["A"], c["B"], c["C"], D=None,
                                          z=None, dt_bias=c["dt_bias"], state=c["state"],
                                          has_initial_state=False)
    delta = _softplus(c["dt"] + c["dt_bias"][None, :, None])          # [b, h, t]
    bx = delta[:, :, None, :] * c["B"][:, 0][:, None] * c["u"][:, :, None, :]  # [b,h,n,t]
    h = np.cumsum(bx, axis=3)
    y = np.einsum("bnt,bhnt->bht", c["C"][:, 0], h)
    np.testing.assert_allclose(out, y, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(st[:2, :, 0, :], h[:, :, :, -1], rtol=1e-12)


def test_scan_zero_B_is_skip_and_gate(oracle):
    # B = 0 and zero initial state => out = D u silu(z)
    c = _scan_case(2)
    c["B"] = np.zeros_like(c["B"])
    out, _, _, _ = oracle.selective_scan(c["u"], c["dt"], c["A"], c["B"], c["C"], D=c["D"],
                                         z=c["z"], dt_bias=c["dt_bias"])
    want = c["D"][None, :, None] * c["u"] * c["z"] / (1 + np.exp(-c["z"]))
    np.testing.assert_allclose(out, want, rtol=1e-13, atol=1e-15)


def test_scan_infinite_decay_is_memoryless(oracle):
    # A = -inf => abar = 0 => h_t = delta_t B_t u_t (no memory at all)
    c = _scan_case(3)
    A = np.full_like(c["A"], -np.inf)
    out, _, _, _ = oracle.selective_scan(c["u"], c["dt"], A, c["B"], c["C"], D=c["D"], z=None,
                                         dt_bias=c["dt_bias"], state=c["state"],
                                         has_initial_state=True)
    delta = _softplus(c["dt"] + c["dt_bias"][None, :, None])
    y = (np.einsum("bnt,bnt->bt", c["C"][:, 0], c["B"][:, 0])[:, None, :] * delta * c["u"]
         + c["D"][None, :, None] * c["u"])
    np.testing.assert_allclose(out, y, rtol=1e-12, atol=1e-13)


@pytest.mark.parametrize("a_per_state", [True, False])
def test_scan_matches_unrolled_quadratic_form(oracle, a_per_state):
    # brute force: y_t = sum_{s<=t} sum_n C_t[n] (prod_{s<i<=t} abar_i[n]) delta_s B_s[n] u_s
    #              + C_t . (prod_{i<=t} abar_i) h_init + D u_t, then the gate
    c = _scan_case(4, batch=1, seqlen=12, nheads=2, headdim=2, dstate=3, ngroups=2,
                   a_per_state=a_per_state)
    out, _, st, _ = oracle.selective_scan(c["u"], c["dt"], c["A"], c["B"], c["C"], D=c["D"],
                                          z=c["z"], dt_bias=c["dt_bias"], state=c["state"],
                                          has_initial_state=True)
    L, H, P, N = 12, 2, 2, 3
    delta = _softplus(c["dt"] + c["dt_bias"][None, :, None])[0]  # [h, t]
    for h in range(H):
        g = h  # 2 heads, 2 groups
        Ah = c["A"][h] if a_per_state else np.full(N, c["A"][h])
        abar = np.exp(delta[h][:, None] * Ah[None, :])           # [t, n]
        for p in range(P):
            ch = h * P + p
            u = c["u"][0, ch]
            for t in range(L):
                y = 0.0
                for n in range(N):
                    Ct = c["C"][0, g, n, t]
                    y += Ct * np.prod(abar[:t + 1, n]) * c["state"][0, h, p, n]
                    for s in range(t + 1):
                        y += Ct * np.prod(abar[s + 1:t + 1, n]) * delta[h, s] * c["B"][0, g, n, s] * u[s]
                y += c["D"][h] * u[t]
                zt = c["z"][0, ch, t]
                assert out[0, ch, t] == pytest.approx(y * zt / (1 + np.exp(-zt)), rel=1e-11, abs=1e-13)


def test_scan_linear_in_u(oracle):
    # for fixed delta, B, C and no gate, out is linear in u (D term included)
    c = _scan_case(5)
    u2 = rng(55).standard_normal(c["u"].shape)
    kw = dict(D=c["D"], z=None, dt_bias=c["dt_bias"])
    o1 = oracle.selective_scan(c["u"], c["dt"], c["A"], c["B"], c["C"], **kw)[0]
    o2 = oracle.selective_scan(u2, c["dt"], c["A"], c["B"], c["C"], **kw)[0]
    o3 = oracle.selective_scan(2.5 * c["u"] - 0.5 * u2, c["dt"], c["A"], c["B"], c["C"], **kw)[0]
    np.testing.assert_allclose(o3, 2.5 * o1 - 0.5 * o2, rtol=1e-11, atol=1e-12)


@pytest.mark.parametrize("a_per_state,headdim,ngroups", [(True, 1, 1), (False, 2, 3)])
def test_scan_equals_chained_state_updates(oracle, a_per_state, headdim, ngroups):
    # invariant between two independent loops: a scan over L tokens == L
    # single-token updates on the slot cache (catches a wrong time index in
    # either, a state not carried, a head/group mix-up in one of them)
    c = _scan_case(6, batch=2, seqlen=11, nheads=3, headdim=headdim, dstate=5, ngroups=ngroups,
                   a_per_state=a_per_state)
    idx = np.array([2, 0], dtype=np.int32)
    out_s, _, st_s, _ = oracle.selective_scan(c["u"], c["dt"], c["A"], c["B"], c["C"], D=c["D"],
                                              z=c["z"], dt_bias=c["dt_bias"], state=c["state"],
                                              slot_idx=idx, has_initial_state=True)
    st = c["state"].copy()
    H, P = 3, headdim
    for t in range(11):
        x = c["u"][:, :, t].reshape(2, H, P)
        z = c["z"][:, :, t].reshape(2, H, P)
        o, _, st, _ = oracle.state_update(st, x, c["dt"][:, :, t], c["A"], c["B"][..., t],
                                          c["C"][..., t], D=c["D"], z=z, dt_bias=c["dt_bias"],
                                          slot_idx=idx)
        np.testing.assert_allclose(o.reshape(2, H * P), out_s[:, :, t], rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(st, st_s, rtol=1e-12, atol=1e-13)
    np.testing.assert_array_equal(st[1], c["state"][1])  # unnamed slot untouched


def test_scan_resume_from_slot(oracle):
    # prefill(L1) then prefill(L2 | cached state) == prefill(L1 + L2)
    c = _scan_case(7, seqlen=20, headdim=2, a_per_state=False)
    full = oracle.selective_scan(c["u"], c["dt"], c["A"], c["B"], c["C"], D=c["D"], z=c["z"],
                                 dt_bias=c["dt_bias"], state=c["state"], has_initial_state=False)
    cut = 7
    p1 = oracle.selective_scan(c["u"][..., :cut], c["dt"][..., :cut], c["A"], c["B"][..., :cut],
                               c["C"][..., :cut], D=c["D"], z=c["z"][..., :cut],
                               dt_bias=c["dt_bias"], state=c["state"], has_initial_state=False)
    p2 = oracle.selective_scan(c["u"][..., cut:], c["dt"][..., cut:], c["A"], c["B"][..., cut:],
                               c["C"][..., cut:], D=c["D"], z=c["z"][..., cut:],
                               dt_bias=c["dt_bias"], state=p1[2], has_initial_state=True)
    np.testing.assert_allclose(np.concatenate([p1[0], p2[0]], axis=2), full[0], rtol=1e-12,
                               atol=1e-13)
    np.testing.assert_allclose(p2[2], full[2], rtol=1e-12, atol=1e-13)


def test_mamba2_equals_per_channel_expansion(oracle):
    # Mamba-2 (scalar A per head, headdim rows per head, groups shared by
    # nheads/ngroups consecutive heads) == Mamba-1 on the expanded problem
    # where every channel carries its head's dt/A/D and its group's B/C.
    H, P, N, G, L, Bt = 4, 3, 5, 2, 9, 2
    c = _scan_case(8, batch=Bt, seqlen=L, nheads=H, headdim=P, dstate=N, ngroups=G,
                   a_per_state=False)
    out2, _, st2, _ = oracle.selective_scan(c["u"], c["dt"], c["A"], c["B"], c["C"], D=c["D"],
                                            z=c["z"], dt_bias=c["dt_bias"], state=c["state"],
                                            has_initial_state=True)
    head = np.repeat(np.arange(H), P)               # channel -> head
    grp = head // (H // G)                          # channel -> group
    Cn = H * P
    B1 = np.stack([c["B"][:, g] for g in grp], axis=1)   # [Bt, Cn, N, L] per channel
    C1 = np.stack([c["C"][:, g] for g in grp], axis=1)
    out1 = np.empty_like(out2)
    for ch in range(Cn):
        o, _, _, _ = oracle.selective_scan(
            c["u"][:, ch:ch + 1], c["dt"][:, head[ch]:head[ch] + 1],
            np.full((1, N), c["A"][head[ch]]), B1[:, ch:ch + 1], C1[:, ch:ch + 1],
            D=c["D"][head[ch]:head[ch] + 1], z=c["z"][:, ch:ch + 1],
            dt_bias=c["dt_bias"][head[ch]:head[ch] + 1],
            state=c["state"][:, head[ch], ch % P][:, None, None, :], has_initial_state=True)
        out1[:, ch] = o[:, 0]
    np.testing.assert_allclose(out2, out1, rtol=1e-13, atol=1e-14)


def test_scan_scale_bounds_output(oracle):
    c = _scan_case(9, headdim=2, a_per_state=False)
    out, sc, st, sts = oracle.selective_scan(c["u"], c["dt"], c["A"], c["B"], c["C"], D=c["D"],
                                             z=c["z"], dt_bias=c["dt_bias"], state=c["state"],
                                             has_initial_state=True)
    assert np.all(sc >= np.abs(out) * (1 - 1e-12))
    assert np.all(sts[:2] >= np.abs(st[:2]) * (1 - 1e-12))


def test_scan_padded_and_unnamed_slots_untouched(oracle):
    c = _scan_case(10)
    idx = np.array([-1, 1], dtype=np.int32)
    init_out = np.full(c["u"].shape, 3.0)
    out, _, st, _ = oracle.selective_scan(c["u"], c["dt"], c["A"], c["B"], c["C"], D=c["D"],
                                          z=c["z"], dt_bias=c["dt_bias"], state=c["state"],
                                          slot_idx=idx, has_initial_state=True, out=init_out)
    np.testing.assert_array_equal(out[0], init_out[0])
    np.testing.assert_array_equal(st[0], c["state"][0])
    np.testing.assert_array_equal(st[2], c["state"][2])
    assert not np.array_equal(st[1], c["state"][1])


def test_state_update_gathers_named_slot(oracle):
    # the update reads the named slot: permuting the cache rows and the slot
    # indices together gives the same outputs
    c = _scan_case(11, batch=3, seqlen=1, nheads=2, headdim=3, dstate=4, a_per_state=False)
    r = rng(111)
    st = r.standard_normal((6, 2, 3, 4))
    idx = np.array([4, 1, 5], dtype=np.int32)
    x = c["u"][:, :, 0].reshape(3, 2, 3)
    args = (x, c["dt"][:, :, 0], c["A"], c["B"][..., 0], c["C"][..., 0])
    o1, _, s1, _ = oracle.state_update(st, *args, D=c["D"], dt_bias=c["dt_bias"], slot_idx=idx)
    perm = r.permutation(6)
    inv = np.argsort(perm)
    st_p = st[perm]                        # row j of st_p is row perm[j] of st
    o2, _, s2, _ = oracle.state_update(st_p, *args, D=c["D"], dt_bias=c["dt_bias"],
                                       slot_idx=inv[idx].astype(np.int32))
    np.testing.assert_array_equal(o1, o2)
    np.testing.assert_array_equal(s1, s2[inv])


# ------------------------------------------------------ packed variable length
def _pack(a):
    # dense [batch, rows..., L] -> packed [rows..., batch*L] (sequence b at
    # columns [b*L, (b+1)*L)), written with explicit loops
    batch, L = a.shape[0], a.shape[-1]
    out = np.zeros(a.shape[1:-1] + (batch * L,))
    for b in range(batch):
        for t in range(L):
            out[..., b * L + t] = a[b, ..., t]
    return out


def test_varlen_equal_lengths_equals_dense(oracle):
    # sequences of one length packed side by side == the dense batch call
    # (catches a wrong column slice, a wrong slot or a dropped initial state)
    c = _scan_case(60, batch=3, seqlen=11, nheads=4, headdim=2, dstate=3, ngroups=2,
                   a_per_state=False)
    idx = np.array([3, 0, 2], dtype=np.int32)
    cu = np.array([0, 11, 22, 33], dtype=np.int32)
    dense = oracle.selective_scan(c["u"], c["dt"], c["A"], c["B"], c["C"], D=c["D"], z=c["z"],
                                  dt_bias=c["dt_bias"], state=c["state"], slot_idx=idx,
                                  has_initial_state=True)
    packed = oracle.selective_scan_varlen(
        _pack(c["u"]), _pack(c["dt"]), c["A"], _pack(c["B"]), _pack(c["C"]), cu, D=c["D"],
        z=_pack(c["z"]), dt_bias=c["dt_bias"], state=c["state"], slot_idx=idx,
        has_initial_state=np.ones(3, dtype=np.int32))
    np.testing.assert_array_equal(packed[0], _pack(dense[0]))
    np.testing.assert_array_equal(packed[2], dense[2])
    x, w, b, cs = _conv_case(61, batch=3, seqlen=11)
    cs = np.concatenate([cs, cs[:1] + 1.0])  # 4 slots
    dense = oracle.causal_conv1d(x, w, b, cs, idx, has_initial_state=True)
    packed = oracle.causal_conv1d_varlen(_pack(x), w, cu, b, cs, idx,
                                         has_initial_state=np.ones(3, dtype=np.int32))
    np.testing.assert_array_equal(packed[0], _pack(dense[0]))
    np.testing.assert_array_equal(packed[2], dense[2])


def test_varlen_split_sequence_resumes(oracle):
    # a sequence cut across two packed calls (the second continuing from the
    # slot) == one dense call over the whole sequence; the other sequences of
    # the calls do not disturb it (catches a flag applied to the wrong
    # sequence or a state written to the wrong slot)
    r = rng(62)
    H, N, L1, L2 = 3, 4, 6, 9
    c = _scan_case(63, batch=1, seqlen=L1 + L2, nheads=H, dstate=N)
    state0 = np.zeros((4, H, 1, N))
    full = oracle.selective_scan(c["u"], c["dt"], c["A"], c["B"], c["C"], D=c["D"], z=c["z"],
                                 dt_bias=c["dt_bias"], state=state0, slot_idx=[2])

    def packed_call(cols, other_len, init, state):
        # the piece of sequence 0 as the second of two packed sequences; the
        # first is unrelated data of other_len steps bound to slot 1
        o = {k: r.standard_normal(c[k].shape[1:-1] + (other_len,)) for k in ("u", "z", "dt", "B", "C")}
        cat = {k: np.concatenate([o[k], c[k][0][..., cols]], axis=-1) for k in o}
        cu = np.array([0, other_len, other_len + cols.stop - cols.start], np.int32)
        res = oracle.selective_scan_varlen(cat["u"], cat["dt"], c["A"], cat["B"], cat["C"], cu,
                                           D=c["D"], z=cat["z"], dt_bias=c["dt_bias"],
                                           state=state, slot_idx=np.array([1, 2], np.int32),
                                           has_initial_state=np.array([1, init], np.int32))
        return res[0][:, other_len:], res[2]

    y1, st1 = packed_call(slice(0, L1), 5, 0, state0)
    y2, st2 = packed_call(slice(L1, L1 + L2), 3, 1, st1)
    np.testing.assert_allclose(np.concatenate([y1, y2], axis=1), full[0][0], rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(st2[2], full[2][2], rtol=1e-12, atol=1e-13)


def test_varlen_padded_and_empty_sequences(oracle):
    # a padded sequence leaves its columns and every slot alone; an empty
    # sequence leaves its slot alone
    x, w, b, cs = _conv_case(64, batch=1, seqlen=10)
    cs = np.concatenate([cs, cs + 1.0, cs + 2.0])  # 3 slots
    packed = x[0]
    cu = np.array([0, 4, 4, 10], dtype=np.int32)   # lengths 4, 0, 6
    idx = np.array([0, 1, -1], dtype=np.int32)
    sentinel = np.full(packed.shape, 5.0)
    out, _, cs_new = oracle.causal_conv1d_varlen(packed, w, cu, b, cs, idx,
                                                 has_initial_state=np.array([1, 1, 1], np.int32),
                                                 out=sentinel)
    np.testing.assert_array_equal(out[:, 4:], sentinel[:, 4:])
    np.testing.assert_array_equal(cs_new[1], cs[1])
    np.testing.assert_array_equal(cs_new[2], cs[2])
    assert not np.array_equal(cs_new[0], cs[0])


# ----------------------------------------------------- decode layer around it
def test_linear_matches_explicit_loops():
    # brute force: out[m, n] = sum_k x[m, k] w[n, k] (catches a transposed weight)
    from oracle import layer

    r = rng(70)
    x, w, res = r.standard_normal((3, 5)), r.standard_normal((4, 5)), r.standard_normal((3, 4))
    out, scale = layer.linear(x, w, residual=res)
    for m in range(3):
        for n in range(4):
            s = sum(x[m, k] * w[n, k] for k in range(5))
            assert abs(out[m, n] - (s + res[m, n])) < 1e-12
            assert scale[m, n] >= abs(out[m, n]) - 1e-12


def test_rmsnorm_closed_forms():
    from oracle import layer

    # a constant row c maps to sign(c) * w * |c| / sqrt(c^2 + eps)
    w = np.array([1.0, 2.0, -0.5])
    out, _ = layer.rmsnorm(np.full((1, 3), -3.0), w, 1e-5)
    np.testing.assert_allclose(out[0], -w * 3.0 / math.sqrt(9.0 + 1e-5), rtol=1e-14)
    # without eps the result does not depend on the row's scale, and the
    # normalised row has mean square 1 (weight 1)
    x = rng(71).standard_normal((2, 7))
    a, _ = layer.rmsnorm(x, np.ones(7), 0.0)
    b, _ = layer.rmsnorm(x * 37.5, np.ones(7), 0.0)
    np.testing.assert_allclose(a, b, rtol=1e-13)
    np.testing.assert_allclose(np.mean(a * a, axis=1), 1.0, rtol=1e-13)


def test_decode_layer_matches_explicit_loops(oracle):
    # the layer's wiring (split of x|z and of dt_low|B|C, conv window, softplus
    # of dt + bias, D skip, z gate, residual, slots) against a per-request,
    # per-channel loop written out here without the oracle's functions
    from oracle import layer

    r = rng(72)
    Dm, Di, N, R, W, S, batch = 8, 6, 4, 3, 4, 5, 2
    w = {"norm_weight": r.uniform(0.5, 1.5, Dm), "in_proj": r.standard_normal((2 * Di, Dm)) * 0.3,
         "conv_weight": r.uniform(-0.5, 0.5, (Di, W)), "conv_bias": r.uniform(-0.5, 0.5, Di),
         "x_proj": r.standard_normal((R + 2 * N, Di)) * 0.3,
         "dt_proj": r.standard_normal((Di, R)) * 0.3, "dt_bias": r.uniform(-3, -1, Di),
         "A": -r.uniform(0.5, 4.0, (Di, N)), "D": r.uniform(0.5, 1.5, Di),
         "out_proj": r.standard_normal((Dm, Di)) * 0.3}
    hidden = r.standard_normal((batch, Dm))
    cs = r.standard_normal((S, Di, W - 1))
    ss = r.standard_normal((S, Di, 1, N))
    idx = np.array([3, 1], dtype=np.int32)
    out, _, cs_o, ss_o, _ = layer.mamba1_decode_layer(w, hidden, cs, ss, idx, eps=1e-5)

    sig = lambda v: 1.0 / (1.0 + math.exp(-v))
    want = hidden.copy()
    cs_w, ss_w = cs.copy(), ss.copy()
    for b in range(batch):
        s = idx[b]
        ms = sum(v * v for v in hidden[b]) / Dm
        hn = [hidden[b, i] / math.sqrt(ms + 1e-5) * w["norm_weight"][i] for i in range(Dm)]
        xz = [sum(w["in_proj"][j, i] * hn[i] for i in range(Dm)) for j in range(2 * Di)]
        u = []
        for c in range(Di):
            win = list(cs[s, c]) + [xz[c]]
            a = w["conv_bias"][c] + sum(w["conv_weight"][c, k] * win[k] for k in range(W))
            u.append(a * sig(a))
            cs_w[s, c] = win[1:]
        dbc = [sum(w["x_proj"][j, c] * u[c] for c in range(Di)) for j in range(R + 2 * N)]
        y = []
        for c in range(Di):
            v = sum(w["dt_proj"][c, k] * dbc[k] for k in range(R)) + w["dt_bias"][c]
            d = math.log1p(math.exp(v))
            acc = 0.0
            for n in range(N):
                h = math.exp(d * w["A"][c, n]) * ss[s, c, 0, n] + d * dbc[R + n] * u[c]
                ss_w[s, c, 0, n] = h
                acc += dbc[R + N + n] * h
            zc = xz[Di + c]
            y.append((acc + w["D"][c] * u[c]) * zc * sig(zc))
        for i in range(Dm):
            want[b, i] += sum(w["out_proj"][i, c] * y[c] for c in range(Di))
    np.testing.assert_allclose(out, want, rtol=1e-11, atol=1e-12)
    np.testing.assert_allclose(cs_o, cs_w, rtol=1e-13, atol=1e-14)  # x is a computed sum
    np.testing.assert_allclose(ss_o, ss_w, rtol=1e-11, atol=1e-12)
