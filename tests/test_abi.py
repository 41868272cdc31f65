"""C-ABI library checks that need no GPU: the library loads, exports every
function include/ssm.h declares, and rejects bad arguments on the host before
anything is enqueued (fake device pointers are never dereferenced: every call
here fails validation or is a documented no-op)."""
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "ssm.h")


@pytest.fixture(scope="module")
def lib():
    import state_space_model_causal_amd as ssm

    if not os.path.exists(ssm.LIB_PATH):
        from state_space_model_causal_amd import build

        build.build()
    return ssm.load_library()


def header_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(ssm_[a-z0-9_]+)\s*\(", text)))


def test_header_declares_the_entry_points():
    names = header_functions()
    for n in ("ssm_causal_conv1d", "ssm_selective_scan", "ssm_state_update"):
        assert n in names


def test_library_exports_every_declared_symbol(lib):
    import state_space_model_causal_amd as ssm

    for name in header_functions():
        assert hasattr(lib, name), name
    assert set(ssm.EXPORTED) <= set(header_functions())


def test_abi_version_matches_header(lib):
    m = re.search(r"#define SSM_ABI_VERSION (\d+)", open(HEADER).read())
    assert lib.ssm_abi_version() == int(m.group(1))


def test_status_strings(lib):
    for code in range(9):
        assert lib.ssm_status_string(code)
    assert lib.ssm_status_string(99) == b"unknown status"


FAKE = 0x10000  # aligned, never dereferenced
F32, F16, BF16 = 0, 1, 2
NULL, SHAPE, DTYPE, ALIGN, UNSUP, HIP, LAYOUT, OOR = 1, 2, 3, 4, 5, 6, 7, 8


def T(ptr, dtype, shape, strides=None):
    """An ssm_tensor: dense strides of `shape` unless given (ptr None = absent)."""
    import state_space_model_causal_amd as ssm

    if ptr is None:
        return ssm.Tensor()
    if strides is None:
        strides, acc = [], 1
        for n in reversed(shape):
            strides.insert(0, acc)
            acc *= n
    st = list(strides) + [0] * (4 - len(strides))
    t = ssm.Tensor()
    t.data, t.dtype = ptr, dtype
    for i in range(4):
        t.stride[i] = st[i]
    return t


def conv(lib, **kw):
    a = dict(x=FAKE, w=FAKE, b=None, cs=None, idx=None, out=FAKE, batch=2, ch=8, L=16, W=4,
             S=0, dt=F16, wdt=F32, odt=None, init=0, silu=1, xs=None, os=None)
    a.update(kw)
    sh = (a["batch"], a["ch"], a["L"])
    return lib.ssm_causal_conv1d(
        T(a["x"], a["dt"], sh, a["xs"]), T(a["w"], a["wdt"], (a["ch"], a["W"])),
        T(a["b"], F32, (a["ch"],)), T(a["cs"], a["dt"], (a["S"], a["ch"], a["W"] - 1)), a["idx"],
        T(a["out"], a["dt"] if a["odt"] is None else a["odt"], sh, a["os"]), a["batch"], a["ch"],
        a["L"], a["W"], a["S"], a["init"], a["silu"], None)


def scan(lib, **kw):
    a = dict(u=FAKE, dt=FAKE, bias=None, A=FAKE, B=FAKE, C=FAKE, D=None, z=None, st=None,
             idx=None, out=FAKE, batch=2, L=16, H=8, P=1, N=16, G=1, S=0, io=F16, sd=F32, bio=None,
             aps=1, sp=1, init=0, Bs=None, us=None)
    a.update(kw)
    Bt, L, H, P, N, G, io = a["batch"], a["L"], a["H"], a["P"], a["N"], a["G"], a["io"]
    bio = io if a["bio"] is None else a["bio"]
    return lib.ssm_selective_scan(
        T(a["u"], io, (Bt, H * P, L), a["us"]), T(a["dt"], io, (Bt, H, L)),
        T(a["bias"], F32, (H,)), T(a["A"], F32, (H, N) if a["aps"] else (H,)),
        T(a["B"], bio, (Bt, G, N, L), a["Bs"]), T(a["C"], io, (Bt, G, N, L)), T(a["D"], F32, (H,)),
        T(a["z"], io, (Bt, H * P, L)), T(a["st"], a["sd"], (a["S"], H, P, N)), a["idx"],
        T(a["out"], io, (Bt, H * P, L)), Bt, L, H, P, N, G, a["S"], a["aps"], a["sp"], a["init"],
        None)


def _ssu_args(a):
    Bt, H, P, N, G, io = a["batch"], a["H"], a["P"], a["N"], a["G"], a["io"]
    return (T(a["st"], a["sd"], (a["S"], H, P, N), a["sts"]), a["idx"], T(a["x"], io, (Bt, H, P), a["xs"]),
            T(a["dt"], io, (Bt, H)), T(a["bias"], F32, (H,)), T(a["A"], F32, (H, N) if a["aps"] else (H,)),
            T(a["B"], io, (Bt, G, N)), T(a["C"], io, (Bt, G, N)), T(a["D"], F32, (H,)),
            T(a["z"], io, (Bt, H, P)), T(a["out"], io, (Bt, H, P)), Bt, H, P, N, G, a["S"], a["aps"],
            a["sp"])


SSU = dict(st=FAKE, idx=None, x=FAKE, dt=FAKE, bias=None, A=FAKE, B=FAKE, C=FAKE, D=None, z=None,
           out=FAKE, batch=2, H=8, P=4, N=16, G=1, S=2, io=F16, sd=F32, aps=0, sp=1, sts=None, xs=None)


def ssu(lib, **kw):
    a = dict(SSU)
    a.update(kw)
    return lib.ssm_state_update(*_ssu_args(a), None)


@pytest.mark.parametrize("kw,code", [
    (dict(x=None), NULL), (dict(w=None), NULL), (dict(out=None), NULL),
    (dict(dt=7), DTYPE), (dict(wdt=F16), DTYPE), (dict(odt=BF16), DTYPE),
    (dict(batch=-1), SHAPE), (dict(ch=0), SHAPE), (dict(W=0), SHAPE),
    (dict(W=5), UNSUP), (dict(cs=FAKE, S=0), SHAPE), (dict(cs=FAKE, S=1, batch=2), SHAPE),
    (dict(x=FAKE + 1), ALIGN), (dict(w=FAKE + 2), ALIGN), (dict(idx=FAKE + 2), ALIGN),
    (dict(xs=(256, 32, 2)), LAYOUT), (dict(os=(-128, 16, 1)), LAYOUT),
    (dict(batch=0), 0), (dict(L=0), 0), (dict(batch=0, xs=(512, 32, 1)), 0),
])
def test_conv_validation(lib, kw, code):
    assert conv(lib, **kw) == code


@pytest.mark.parametrize("kw,code", [
    (dict(u=None), NULL), (dict(A=None), NULL), (dict(B=None), NULL), (dict(out=None), NULL),
    (dict(io=3), DTYPE), (dict(sd=-1, st=FAKE, S=4), DTYPE), (dict(bio=BF16), DTYPE),
    (dict(H=6, G=4), SHAPE), (dict(N=0), SHAPE), (dict(P=0), SHAPE), (dict(st=FAKE, S=1), SHAPE),
    (dict(N=257), OOR),
    (dict(u=FAKE + 1), ALIGN), (dict(st=FAKE + 2, S=4, sd=F32), ALIGN), (dict(A=FAKE + 1), ALIGN),
    (dict(Bs=(256, 256, 16, 3)), LAYOUT), (dict(us=(128, -16, 1)), LAYOUT),
    (dict(batch=0), 0), (dict(L=0), 0),
])
def test_scan_validation(lib, kw, code):
    assert scan(lib, **kw) == code


@pytest.mark.parametrize("kw,code", [
    (dict(st=None), NULL), (dict(x=None), NULL), (dict(C=None), NULL),
    (dict(io=9), DTYPE), (dict(H=8, G=3), SHAPE), (dict(N=513), OOR), (dict(S=1), SHAPE),
    (dict(S=0, idx=FAKE), SHAPE), (dict(x=FAKE + 1), ALIGN), (dict(st=FAKE + 2, sd=F32), ALIGN),
    (dict(sts=(512, 64, 16, 2)), LAYOUT), (dict(xs=(32, 4, 3)), LAYOUT),
    (dict(batch=0), 0),
])
def test_ssu_validation(lib, kw, code):
    assert ssu(lib, **kw) == code


def test_binding_refuses_cpu_tensors(lib):
    import torch
    import state_space_model_causal_amd as ssm

    x = torch.zeros(1, 4, 8)
    with pytest.raises(ValueError, match="GPU"):
        ssm.causal_conv1d(x, torch.zeros(4, 4))


def dstep(lib, **kw):
    a = dict(SSU)
    a.update(cs=FAKE, w=FAKE, cb=None, W=4, uo=None, csdt=None)
    a.update(kw)
    Cn = a["H"] * a["P"]
    args = list(_ssu_args(a))
    st, idx, x = args[0], args[1], args[2]
    rest = args[3:11]
    return lib.ssm_decode_step(
        st, T(a["cs"], a["io"] if a["csdt"] is None else a["csdt"], (a["S"], Cn, a["W"] - 1)), idx, x,
        T(a["w"], F32, (Cn, a["W"])), T(a["cb"], F32, (Cn,)), a["W"], *rest,
        T(a["uo"], a["io"], (a["batch"], a["H"], a["P"])), *args[11:], None)


@pytest.mark.parametrize("kw,code", [
    (dict(cs=None), NULL), (dict(w=None), NULL), (dict(st=None), NULL), (dict(W=3), UNSUP),
    (dict(W=0), SHAPE), (dict(N=513), OOR), (dict(cs=FAKE + 1), ALIGN),
    (dict(uo=FAKE + 1), ALIGN), (dict(w=FAKE + 2), ALIGN), (dict(H=8, G=3), SHAPE),
    (dict(csdt=F32), DTYPE), (dict(batch=0), 0),
])
def test_decode_step_validation(lib, kw, code):
    assert dstep(lib, **kw) == code


def ssu_ex(lib, cfg, **kw):
    import ctypes
    import state_space_model_causal_amd as ssm

    a = dict(SSU)
    a.update(kw)
    c = None if cfg is None else ctypes.byref(ssm.LaunchConfig(*cfg))
    return lib.ssm_state_update_ex(*_ssu_args(a), c, None)


@pytest.mark.parametrize("cfg,kw", [
    ((4, 256), dict(sd=F16)),  # 4 states per lane only for a 4-byte cache
    ((8, 32), {}), ((8, 96), {}), ((0, 0), {}), ((12, 256), {}), ((8, 320), {}),
])
def test_state_update_ex_rejects_bad_geometry(lib, cfg, kw):
    assert ssu_ex(lib, cfg, **kw) == SHAPE


@pytest.mark.parametrize("cfg,kw", [
    ((32, 256), {}),           # more states per lane than the kernels hold in registers
    ((16, 1024), {}),          # more lanes than the kernels' launch bound
    ((4, 256), dict(N=512)),   # a row of 128 lanes would not fit in a wave
])
def test_state_update_ex_out_of_resources(lib, cfg, kw):
    assert ssu_ex(lib, cfg, **kw) == OOR


def test_state_update_ex_validates_like_the_plain_call(lib):
    # the override does not bypass the argument checks (none of these launch)
    assert ssu_ex(lib, (8, 256), st=None) == NULL
    assert ssu_ex(lib, (8, 256), N=513) == OOR
    assert ssu_ex(lib, (16, 64), batch=0) == 0


def test_state_update_config_choices(lib):
    import torch
    import state_space_model_causal_amd as ssm

    for batch, H, P, N, io, st in [(245, 5120, 1, 16, torch.float16, torch.float32),
                                   (1, 80, 64, 128, torch.float16, torch.float16),
                                   (1024, 80, 64, 128, torch.float16, torch.float32),
                                   (8, 64, 128, 256, torch.bfloat16, torch.bfloat16),
                                   (3, 7, 3, 24, torch.float32, torch.float32)]:
        v, b, from_table = ssm.state_update_config(batch, H, P, N, io, st)
        assert v in (4, 8, 16) and b in (64, 128, 256, 512)
        if not from_table:  # the documented heuristic: 32 bytes of state per lane
            two = st in (torch.float16, torch.bfloat16)
            assert (v, b) == ((16 if two and N % 16 == 0 and N >= 32 else 8), 256)
    with pytest.raises(ssm.SsmError):
        ssm.state_update_config(1, 8, 4, 513, torch.float16, torch.float16)


def test_tuned_table_entries_are_valid():
    # every line of the compiled-in table names a legal geometry and a
    # non-empty effective-batch range
    import re

    path = os.path.join(ROOT, "state_space_model_causal_amd", "csrc", "ssu_table_gfx950.inc")
    for line in open(path):
        line = line.split("//")[0].strip()
        if not line:
            continue
        vals = [int(v) for v in re.findall(r"-?\d+", line)]
        assert len(vals) == 8, line
        P, N, io, st, lo, hi, v, b = vals
        assert P >= 1 and 1 <= N <= 512 and io in (0, 1, 2) and st in (0, 1, 2)
        assert 0 <= lo < hi and b in (64, 128, 256, 512)
        # 4 states per lane only for a float32 cache, with the row within a wave
        assert v in (8, 16) or (v == 4 and st == 0), line
        assert (N + v - 1) // v <= 64, line


def scan_ex(lib, algo, **kw):
    a = dict(u=FAKE, dt=FAKE, bias=None, A=FAKE, B=FAKE, C=FAKE, D=None, z=None, st=None,
             idx=None, out=FAKE, batch=2, L=64, H=4, P=64, N=128, G=1, S=0, io=BF16, sd=F32, aps=0,
             sp=1, init=0, bs=None)
    a.update(kw)
    Bt, L, H, P, N, G, io = a["batch"], a["L"], a["H"], a["P"], a["N"], a["G"], a["io"]
    return lib.ssm_selective_scan_ex(
        T(a["u"], io, (Bt, H * P, L)), T(a["dt"], io, (Bt, H, L)), T(a["bias"], F32, (H,)),
        T(a["A"], F32, (H, N) if a["aps"] else (H,)), T(a["B"], io, (Bt, G, N, L), a["bs"]),
        T(a["C"], io, (Bt, G, N, L)), T(a["D"], F32, (H,)), T(a["z"], io, (Bt, H * P, L)),
        T(a["st"], a["sd"], (a["S"], H, P, N)), a["idx"], T(a["out"], io, (Bt, H * P, L)), Bt, L,
        H, P, N, G, a["S"], a["aps"], a["sp"], a["init"], algo, None)


# (the last case: B's states 2^25 elements apart, so a (request, group) plane
# spans more than the chunked kernel's 32-bit byte offsets reach)
@pytest.mark.parametrize("kw", [dict(aps=1, N=16), dict(io=F32), dict(N=96),
                                dict(P=32), dict(L=60), dict(u=FAKE + 2),
                                dict(bs=(128 << 25, 128 << 25, 1 << 25, 1))])
def test_scan_chunked_refuses_unsupported_shapes(lib, kw):
    # the chunked form is asked for explicitly where it does not apply: the
    # call fails before anything is launched (fake pointers are never touched)
    assert scan_ex(lib, 2, **kw) == UNSUP


def test_scan_ex_rejects_unknown_algorithm(lib):
    assert scan_ex(lib, 7) == SHAPE
    assert scan_ex(lib, 2, batch=0) == 0


def layer_desc(**kw):
    import state_space_model_causal_amd as ssm

    a = dict(d_model=64, d_inner=128, d_state=16, dt_rank=8, conv_width=4, norm_eps=1e-5,
             norm_weight=FAKE, in_proj=FAKE, conv_weight=FAKE, conv_bias=None, x_proj=FAKE,
             dt_proj=FAKE, dt_bias=None, A=FAKE, D=None, out_proj=FAKE)
    a.update(kw)
    return ssm.Mamba1Layer(*[a[f] for f, _ in ssm.Mamba1Layer._fields_])


def layer(lib, desc=None, **kw):
    import ctypes

    a = dict(hidden=FAKE, cs=FAKE, st=FAKE, idx=None, batch=4, S=8, io=F16, sd=F32, hs=None,
             sts=None, ws=FAKE, wsb=1 << 30)
    a.update(kw)
    desc = desc or layer_desc()
    return lib.ssm_mamba1_decode_layer(
        ctypes.byref(desc), T(a["hidden"], a["io"], (a["batch"], desc.d_model), a["hs"]),
        T(a["cs"], a["io"], (a["S"], desc.d_inner, desc.conv_width - 1)),
        T(a["st"], a["sd"], (a["S"], desc.d_inner, 1, desc.d_state), a["sts"]), a["idx"],
        a["batch"], a["S"], a["ws"], a["wsb"], None)


@pytest.mark.parametrize("kw,code", [
    (dict(st=FAKE + 2), ALIGN),               # misaligned f32 state: the last step's check
    (dict(S=2), SHAPE),                       # implicit slots need nslots >= batch
    (dict(sts=(2048, 16, 16, 2)), LAYOUT),    # state with a non-unit inner stride
    (dict(sd=9), DTYPE), (dict(io=F32), UNSUP), (dict(hs=(64, 2)), LAYOUT),
    (dict(ws=FAKE + 16), ALIGN), (dict(wsb=64), SHAPE),
])
def test_layer_checks_every_step_before_launching(lib, kw, code):
    # Every step's arguments are checked before the first launch: with fake
    # pointers and no GPU, any launch would come back as SSM_ERR_HIP (or
    # fault), so the validation code itself shows that nothing ran and the
    # conv cache (shifted by step 3) is untouched.
    assert layer(lib, **kw) == code


def test_layer_batch_zero_is_a_noop(lib):
    assert layer(lib, batch=0) == 0


def test_linear_and_rmsnorm_validation(lib):
    f = lambda x=FAKE, w=FAKE, o=FAKE, M=4, N=16, K=32, xs=None, dt=F16: lib.ssm_linear(
        T(x, dt, (M, K), xs), T(w, dt, (N, K)), T(None, dt, (M, N)), T(o, dt, (M, N)), M, N, K,
        None, 0, None)
    assert f(x=None) == NULL
    assert f(dt=F32) == UNSUP
    assert f(K=12) == SHAPE
    assert f(xs=(36, 1)) == ALIGN      # rows of 72 bytes are not 16-byte multiples
    assert f(xs=(64, 2)) == LAYOUT
    assert f(M=0) == 0
    g = lambda x=FAKE, o=FAKE, M=4, D=64, os=None: lib.ssm_rmsnorm(
        T(x, F16, (M, D)), T(FAKE, F32, (D,)), T(o, F16, (M, D), os), M, D, 1e-5, None)
    assert g(o=None) == NULL
    assert g(os=(64, 3)) == LAYOUT
    assert g(M=0) == 0


def test_linear_plan_query(lib):
    # the plan ssm_linear takes, reported on the host; its workspace is the
    # one ssm_linear asks for, and every reported plan is one ssm_linear_ex takes
    import ctypes

    import state_space_model_causal_amd as ssm

    for M, N, K in ((245, 10240, 2560), (245, 192, 5120), (245, 5120, 160), (245, 2560, 5120),
                    (1, 64, 32), (7, 100, 40), (300, 130, 264)):
        wr, c, sp = ssm.linear_plan(M, N, K)
        assert wr in (16, 32, 64) and c in (64, 128) and 1 <= sp <= min(32, (K + 63) // 64)
        assert lib.ssm_linear_workspace_ex(M, N, K, wr, c, sp) == lib.ssm_linear_workspace(M, N, K)
    out = ctypes.c_int()
    assert lib.ssm_linear_plan(0, 64, 32, None, None, None) == SHAPE
    assert lib.ssm_linear_plan(4, 64, 4, ctypes.byref(out), None, None) == SHAPE


def test_noalloc_layer_scratch_limit(lib):
    # the documented limit: the Mamba-2.8B layer's workspace fits the 64 MiB
    # array up to 687 requests; beyond, the call is refused before any HIP call
    import ctypes

    desc = layer_desc(d_model=2560, d_inner=5120, d_state=16, dt_rank=160)
    ws = lambda b: lib.ssm_mamba1_decode_layer_workspace(ctypes.byref(desc), b)
    assert max(ws(b) for b in range(1, 688)) <= 64 << 20 < ws(688)
    assert lib.ssm_mamba1_decode_layer_noalloc(
        ctypes.byref(desc), T(FAKE, F16, (688, 2560)), T(FAKE, F16, (700, 5120, 3)),
        T(FAKE, F32, (700, 5120, 1, 16)), None, 688, 700, None) == OOR
    assert lib.ssm_mamba1_decode_layer_noalloc(
        ctypes.byref(desc), T(FAKE, F16, (4, 2560)), T(FAKE, F16, (8, 5120, 3)),
        T(FAKE, F32, (8, 5120, 1, 16)), None, 0, 8, None) == 0


def test_launch_group_state_errors(lib):
    # host-side only: no device call is made by begin, or by an end with
    # nothing held
    s, other = 0x1000, 0x2000  # stream handles are only compared
    assert lib.ssm_group_end(s) == 5            # no open group: SSM_ERR_UNSUPPORTED
    assert lib.ssm_group_begin(s) == 0
    assert lib.ssm_group_begin(s) == 5          # groups do not nest
    assert lib.ssm_group_end(other) == 5        # the group's stream only
    assert lib.ssm_group_end(s) == 0
    assert lib.ssm_group_end(s) == 5            # closed
