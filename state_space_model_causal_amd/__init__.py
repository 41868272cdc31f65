"""Python binding of the gfx950 causal selective-SSM library (libssm_hip.so).

Argument marshalling only: every step of the computation runs in the HIP
kernels behind the C ABI of ``include/ssm.h``.  PyTorch supplies device memory
(tensors are passed as raw pointers) and the current stream.  There is no CPU
fallback: if the library is missing or the tensors are not on the GPU the
calls raise.

Tensors are passed with their strides (views such as the x and z halves of a
projection output are taken as they are); the innermost dimension must be
contiguous.  Layouts (time innermost for prefill):
    prefill  u/x/z/out [batch, channels, seqlen], dt [batch, nheads, seqlen],
             B/C [batch, ngroups, dstate, seqlen]
    decode   x/z/out [batch, nheads, headdim], dt [batch, nheads],
             B/C [batch, ngroups, dstate]
    varlen   sequences packed along time: x/u/z/out [channels, total_len],
             dt [nheads, total_len], B/C [ngroups, dstate, total_len];
             cu_seqlens int32 [nseq+1] on the GPU
    caches   conv_state [nslots, channels, width-1], ssm_state
             [nslots, nheads, headdim, dstate]
    params   A [nheads, dstate] (one decay per channel and state) or [nheads]
             (one decay per head), D/dt_bias [nheads], conv weight
             [channels, width], conv bias [channels] -- all float32
"""
from __future__ import annotations

import contextlib
import ctypes
import os

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libssm_hip.so")

SSM_F32, SSM_F16, SSM_BF16 = 0, 1, 2
SCAN_AUTO, SCAN_RECURRENT, SCAN_CHUNKED = 0, 1, 2
_DTYPE_CODE = {torch.float32: SSM_F32, torch.float16: SSM_F16, torch.bfloat16: SSM_BF16}

EXPORTED = ("ssm_causal_conv1d", "ssm_selective_scan", "ssm_selective_scan_ex", "ssm_state_update",
            "ssm_state_update_ex", "ssm_state_update_config",
            "ssm_decode_step", "ssm_causal_conv1d_varlen", "ssm_selective_scan_varlen",
            "ssm_linear", "ssm_linear_workspace", "ssm_linear_ex", "ssm_linear_workspace_ex", "ssm_linear_plan",
            "ssm_rmsnorm", "ssm_mamba1_decode_layer",
            "ssm_mamba1_decode_layer_workspace", "ssm_mamba1_decode_layer_noalloc",
            "ssm_group_begin", "ssm_group_end",
            "ssm_status_string", "ssm_abi_version")


class Tensor(ctypes.Structure):
    """ssm_tensor: device pointer, dtype code and element strides (outermost
    first).  data = NULL marks an absent optional tensor."""
    _fields_ = [("data", ctypes.c_void_p), ("dtype", ctypes.c_int32), ("reserved", ctypes.c_int32),
                ("stride", ctypes.c_int64 * 4)]


class Mamba1Layer(ctypes.Structure):
    """ssm_mamba1_layer: dimensions and device pointers of one layer's weights."""
    _fields_ = [("d_model", ctypes.c_int), ("d_inner", ctypes.c_int), ("d_state", ctypes.c_int),
                ("dt_rank", ctypes.c_int), ("conv_width", ctypes.c_int),
                ("norm_eps", ctypes.c_float), ("norm_weight", ctypes.c_void_p),
                ("in_proj", ctypes.c_void_p), ("conv_weight", ctypes.c_void_p),
                ("conv_bias", ctypes.c_void_p), ("x_proj", ctypes.c_void_p),
                ("dt_proj", ctypes.c_void_p), ("dt_bias", ctypes.c_void_p), ("A", ctypes.c_void_p),
                ("D", ctypes.c_void_p), ("out_proj", ctypes.c_void_p)]


class LaunchConfig(ctypes.Structure):
    """ssm_launch_config: the state update's geometry."""
    _fields_ = [("states_per_lane", ctypes.c_int), ("block_threads", ctypes.c_int)]

STATUS = {0: "SSM_OK", 1: "SSM_ERR_NULL_ARG", 2: "SSM_ERR_SHAPE", 3: "SSM_ERR_DTYPE",
          4: "SSM_ERR_ALIGN", 5: "SSM_ERR_UNSUPPORTED", 6: "SSM_ERR_HIP", 7: "SSM_ERR_LAYOUT",
          8: "SSM_ERR_OUT_OF_RESOURCES"}


class SsmError(RuntimeError):
    def __init__(self, fn: str, status: int, text: str):
        super().__init__(f"{fn} failed: {STATUS.get(status, status)} ({text})")
        self.status = status


_lib = None


def load_library(path: str = LIB_PATH) -> ctypes.CDLL:
    """dlopen the HIP library and declare the C signatures (no device call)."""
    global _lib
    if _lib is not None and path == LIB_PATH:
        return _lib
    if not os.path.exists(path):
        raise ImportError(
            f"{path} is missing: the HIP extension has not been built "
            "(run __graft_entry__.build() or python state_space_model_causal_amd/build.py)")
    lib = ctypes.CDLL(path)
    P, I, T = ctypes.c_void_p, ctypes.c_int, Tensor
    lib.ssm_causal_conv1d.argtypes = [T, T, T, T, P, T, I, I, I, I, I, I, I, P]
    lib.ssm_causal_conv1d.restype = I
    lib.ssm_selective_scan.argtypes = [T, T, T, T, T, T, T, T, T, P, T,
                                       I, I, I, I, I, I, I, I, I, I, P]
    lib.ssm_selective_scan.restype = I
    lib.ssm_selective_scan_ex.argtypes = [T, T, T, T, T, T, T, T, T, P, T,
                                          I, I, I, I, I, I, I, I, I, I, I, P]
    lib.ssm_selective_scan_ex.restype = I
    lib.ssm_state_update.argtypes = [T, P, T, T, T, T, T, T, T, T, T,
                                     I, I, I, I, I, I, I, I, P]
    lib.ssm_state_update.restype = I
    lib.ssm_state_update_ex.argtypes = [T, P, T, T, T, T, T, T, T, T, T,
                                        I, I, I, I, I, I, I, I, P, P]
    lib.ssm_state_update_ex.restype = I
    lib.ssm_state_update_config.argtypes = [I, I, I, I, I, I, P, P]
    lib.ssm_state_update_config.restype = I
    lib.ssm_decode_step.argtypes = [T, T, P, T, T, T, I, T, T, T, T, T, T, T, T, T,
                                    I, I, I, I, I, I, I, I, P]
    lib.ssm_decode_step.restype = I
    lib.ssm_causal_conv1d_varlen.argtypes = [T, T, T, T, P, P, P, T, I, I, I, I, I, I, P]
    lib.ssm_causal_conv1d_varlen.restype = I
    lib.ssm_selective_scan_varlen.argtypes = [T, T, T, T, T, T, T, T, T, P, P, P, T,
                                              I, I, I, I, I, I, I, I, I, P]
    lib.ssm_selective_scan_varlen.restype = I
    Z = ctypes.c_size_t
    lib.ssm_linear_workspace.argtypes = [I, I, I]
    lib.ssm_linear_workspace.restype = Z
    lib.ssm_linear.argtypes = [T, T, T, T, I, I, I, P, Z, P]
    lib.ssm_linear.restype = I
    lib.ssm_linear_workspace_ex.argtypes = [I, I, I, I, I, I]
    lib.ssm_linear_workspace_ex.restype = Z
    lib.ssm_linear_ex.argtypes = [T, T, T, T, I, I, I, I, I, I, P, Z, P]
    lib.ssm_linear_ex.restype = I
    IP = ctypes.POINTER(ctypes.c_int)
    lib.ssm_linear_plan.argtypes = [I, I, I, IP, IP, IP]
    lib.ssm_linear_plan.restype = I
    lib.ssm_rmsnorm.argtypes = [T, T, T, I, I, ctypes.c_float, P]
    lib.ssm_rmsnorm.restype = I
    lib.ssm_mamba1_decode_layer_workspace.argtypes = [P, I]
    lib.ssm_mamba1_decode_layer_workspace.restype = Z
    lib.ssm_mamba1_decode_layer.argtypes = [P, T, T, T, P, I, I, P, Z, P]
    lib.ssm_mamba1_decode_layer.restype = I
    lib.ssm_mamba1_decode_layer_noalloc.argtypes = [P, T, T, T, P, I, I, P]
    lib.ssm_mamba1_decode_layer_noalloc.restype = I
    lib.ssm_group_begin.argtypes = [P]
    lib.ssm_group_begin.restype = I
    lib.ssm_group_end.argtypes = [P]
    lib.ssm_group_end.restype = I
    lib.ssm_status_string.argtypes = [I]
    lib.ssm_status_string.restype = ctypes.c_char_p
    lib.ssm_abi_version.argtypes = []
    lib.ssm_abi_version.restype = I
    if path == LIB_PATH:
        _lib = lib
    return lib


def _check(fn: str, status: int):
    if status != 0:
        raise SsmError(fn, status, load_library().ssm_status_string(status).decode())


def _gpu(t, name, dtype=None):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must live on the GPU (got {t.device})")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype} (got {t.dtype})")


def _ptr(t, name, dtype=None):
    """Raw device pointer of a dense tensor (index tables, layer weights)."""
    if t is None:
        return None
    _gpu(t, name, dtype)
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return t.data_ptr()


def _tensor(t, name, dtype=None):
    """ssm_tensor of a torch tensor: its pointer, dtype code and strides as
    they are (views included); an empty Tensor for None."""
    if t is None:
        return Tensor()
    _gpu(t, name, dtype)
    if t.dim() > 4:
        raise ValueError(f"{name} has more than 4 dimensions")
    st = (ctypes.c_int64 * 4)(*(list(t.stride()) + [0] * (4 - t.dim())))
    return Tensor(t.data_ptr(), _code(t, name), 0, st)


def _code(t, name):
    try:
        return _DTYPE_CODE[t.dtype]
    except KeyError:
        raise TypeError(f"{name}: unsupported dtype {t.dtype}") from None


def _stream(stream):
    if stream is None:
        stream = torch.cuda.current_stream()
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)


def _new_like(t):
    # a dense output of t's shape and dtype
    return torch.empty(t.shape, dtype=t.dtype, device=t.device)


def causal_conv1d(x, weight, bias=None, conv_state=None, slot_idx=None, out=None,
                  has_initial_state=False, apply_silu=True, stream=None):
    """ssm_causal_conv1d: x [batch, channels, seqlen] -> out (same shape/dtype)."""
    batch, channels, seqlen = x.shape
    width = weight.shape[1]
    if out is None:
        out = _new_like(x)
    nslots = conv_state.shape[0] if conv_state is not None else 0
    st = load_library().ssm_causal_conv1d(
        _tensor(x, "x"), _tensor(weight, "weight"), _tensor(bias, "bias"),
        _tensor(conv_state, "conv_state"), _ptr(slot_idx, "slot_idx", torch.int32),
        _tensor(out, "out"), batch, channels, seqlen, width, nslots, int(bool(has_initial_state)),
        int(bool(apply_silu)), _stream(stream))
    _check("ssm_causal_conv1d", st)
    return out


def selective_scan(u, dt, A, B, C, D=None, z=None, dt_bias=None, dt_softplus=True,
                   ssm_state=None, slot_idx=None, has_initial_state=False, out=None,
                   stream=None, algo=None):
    """ssm_selective_scan: u [batch, nheads*headdim, seqlen] -> out.
    algo: None (the library's choice), SCAN_RECURRENT or SCAN_CHUNKED
    (ssm_selective_scan_ex)."""
    batch, channels, seqlen = u.shape
    nheads = dt.shape[1]
    headdim = channels // nheads
    ngroups, dstate = B.shape[1], B.shape[2]
    a_per_state = 1 if A.dim() == 2 else 0
    if out is None:
        out = _new_like(u)
    nslots = ssm_state.shape[0] if ssm_state is not None else 0
    args = (_tensor(u, "u"), _tensor(dt, "dt"), _tensor(dt_bias, "dt_bias"), _tensor(A, "A"),
            _tensor(B, "B"), _tensor(C, "C"), _tensor(D, "D"), _tensor(z, "z"),
            _tensor(ssm_state, "ssm_state"), _ptr(slot_idx, "slot_idx", torch.int32),
            _tensor(out, "out"), batch, seqlen, nheads, headdim, dstate, ngroups, nslots,
            a_per_state, int(bool(dt_softplus)), int(bool(has_initial_state)))
    if algo is None:
        st = load_library().ssm_selective_scan(*args, _stream(stream))
        _check("ssm_selective_scan", st)
    else:
        st = load_library().ssm_selective_scan_ex(*args, int(algo), _stream(stream))
        _check("ssm_selective_scan_ex", st)
    return out


def state_update(state, x, dt, A, B, C, D=None, z=None, dt_bias=None, dt_softplus=True,
                 slot_idx=None, out=None, stream=None, config=None):
    """ssm_state_update: one token per request, state cache updated in place.
    config: (states_per_lane, block_threads) to override the library's launch
    geometry (ssm_state_update_ex), or None."""
    nslots, nheads, headdim, dstate = state.shape
    batch = x.shape[0]
    ngroups = B.shape[1]
    a_per_state = 1 if A.dim() == 2 else 0
    if out is None:
        out = _new_like(x)
    args = (_tensor(state, "state"), _ptr(slot_idx, "slot_idx", torch.int32), _tensor(x, "x"),
            _tensor(dt, "dt"), _tensor(dt_bias, "dt_bias"), _tensor(A, "A"), _tensor(B, "B"),
            _tensor(C, "C"), _tensor(D, "D"), _tensor(z, "z"), _tensor(out, "out"), batch,
            nheads, headdim, dstate, ngroups, nslots, a_per_state, int(bool(dt_softplus)))
    if config is None:
        st = load_library().ssm_state_update(*args, _stream(stream))
        _check("ssm_state_update", st)
    else:
        cfg = LaunchConfig(*config)
        st = load_library().ssm_state_update_ex(*args, ctypes.byref(cfg), _stream(stream))
        _check("ssm_state_update_ex", st)
    return out


def state_update_config(batch, nheads, headdim, dstate, io_dtype, state_dtype):
    """ssm_state_update_config: the geometry the library picks for a shape,
    as (states_per_lane, block_threads, from_table).  Dtypes are torch dtypes."""
    cfg = LaunchConfig()
    ft = ctypes.c_int(0)
    st = load_library().ssm_state_update_config(batch, nheads, headdim, dstate,
                                                _DTYPE_CODE[io_dtype], _DTYPE_CODE[state_dtype],
                                                ctypes.byref(cfg), ctypes.byref(ft))
    _check("ssm_state_update_config", st)
    return cfg.states_per_lane, cfg.block_threads, bool(ft.value)


def decode_step(state, conv_state, x, conv_weight, dt, A, B, C, conv_bias=None, D=None, z=None,
                dt_bias=None, dt_softplus=True, slot_idx=None, out=None, u_out=None,
                stream=None):
    """ssm_decode_step: conv update + state update for one token per request.
    x [batch, nheads, headdim] is the conv input; returns out."""
    nslots, nheads, headdim, dstate = state.shape
    batch = x.shape[0]
    ngroups = B.shape[1]
    a_per_state = 1 if A.dim() == 2 else 0
    if out is None:
        out = _new_like(x)
    st = load_library().ssm_decode_step(
        _tensor(state, "state"), _tensor(conv_state, "conv_state"),
        _ptr(slot_idx, "slot_idx", torch.int32), _tensor(x, "x"),
        _tensor(conv_weight, "conv_weight"), _tensor(conv_bias, "conv_bias"),
        conv_weight.shape[1], _tensor(dt, "dt"), _tensor(dt_bias, "dt_bias"), _tensor(A, "A"),
        _tensor(B, "B"), _tensor(C, "C"), _tensor(D, "D"), _tensor(z, "z"), _tensor(out, "out"),
        _tensor(u_out, "u_out"), batch, nheads, headdim, dstate, ngroups, nslots, a_per_state,
        int(bool(dt_softplus)), _stream(stream))
    _check("ssm_decode_step", st)
    return out


@contextlib.contextmanager
def launch_group(stream=None):
    """ssm_group_begin / ssm_group_end around a block of independent calls on
    `stream` (default: the current stream): a Mamba-1 prefill scan and a
    fused decode step of the kinds ssm.h lists run as one launch, with the
    same results as the calls made one after the other.  Buffers of the calls
    must stay alive until the block has ended."""
    s = _stream(stream)
    _check("ssm_group_begin", load_library().ssm_group_begin(s))
    try:
        yield
    finally:
        st = load_library().ssm_group_end(s)
    _check("ssm_group_end", st)


def causal_conv1d_varlen(x, weight, cu_seqlens, bias=None, conv_state=None, slot_idx=None,
                         has_initial_state=None, out=None, apply_silu=True, stream=None):
    """ssm_causal_conv1d_varlen: x [channels, total_len] holding len(cu_seqlens)-1
    sequences; has_initial_state int32 [nseq] (on the GPU) or None."""
    channels, total_len = x.shape
    nseq = cu_seqlens.shape[0] - 1
    width = weight.shape[1]
    if out is None:
        out = _new_like(x)
    nslots = conv_state.shape[0] if conv_state is not None else 0
    st = load_library().ssm_causal_conv1d_varlen(
        _tensor(x, "x"), _tensor(weight, "weight"), _tensor(bias, "bias"),
        _tensor(conv_state, "conv_state"), _ptr(slot_idx, "slot_idx", torch.int32),
        _ptr(has_initial_state, "has_initial_state", torch.int32),
        _ptr(cu_seqlens, "cu_seqlens", torch.int32), _tensor(out, "out"), nseq, channels,
        total_len, width, nslots, int(bool(apply_silu)), _stream(stream))
    _check("ssm_causal_conv1d_varlen", st)
    return out


def selective_scan_varlen(u, dt, A, B, C, cu_seqlens, D=None, z=None, dt_bias=None,
                          dt_softplus=True, ssm_state=None, slot_idx=None,
                          has_initial_state=None, out=None, stream=None):
    """ssm_selective_scan_varlen: u [nheads*headdim, total_len] holding
    len(cu_seqlens)-1 sequences -> out."""
    channels, total_len = u.shape
    nheads = dt.shape[0]
    headdim = channels // nheads
    ngroups, dstate = B.shape[0], B.shape[1]
    nseq = cu_seqlens.shape[0] - 1
    a_per_state = 1 if A.dim() == 2 else 0
    if out is None:
        out = _new_like(u)
    nslots = ssm_state.shape[0] if ssm_state is not None else 0
    st = load_library().ssm_selective_scan_varlen(
        _tensor(u, "u"), _tensor(dt, "dt"), _tensor(dt_bias, "dt_bias"), _tensor(A, "A"),
        _tensor(B, "B"), _tensor(C, "C"), _tensor(D, "D"), _tensor(z, "z"),
        _tensor(ssm_state, "ssm_state"), _ptr(slot_idx, "slot_idx", torch.int32),
        _ptr(has_initial_state, "has_initial_state", torch.int32),
        _ptr(cu_seqlens, "cu_seqlens", torch.int32), _tensor(out, "out"), nseq, total_len, nheads,
        headdim, dstate, ngroups, nslots, a_per_state, int(bool(dt_softplus)), _stream(stream))
    _check("ssm_selective_scan_varlen", st)
    return out


def _workspace(nbytes, device):
    # caller-side allocation of a library workspace (the library allocates nothing)
    if nbytes == 0:
        return None
    return torch.empty(nbytes, dtype=torch.uint8, device=device)


def linear(x, weight, residual=None, out=None, workspace=None, stream=None, rows_per_wave=0, cols=0,
           splits=0):
    """ssm_linear: out[M, N] = x[M, K] . weight[N, K]^T (+ residual).  With
    rows_per_wave / cols / splits (0: the library's choice) the plan is given
    (ssm_linear_ex)."""
    M, K = x.shape
    N = weight.shape[0]
    if out is None:
        out = torch.empty(M, N, dtype=x.dtype, device=x.device)
    lib = load_library()
    if workspace is None:
        need = lib.ssm_linear_workspace_ex(M, N, K, int(rows_per_wave), int(cols), int(splits))
        workspace = _workspace(need, x.device)
    st = lib.ssm_linear_ex(
        _tensor(x, "x"), _tensor(weight, "weight"), _tensor(residual, "residual"),
        _tensor(out, "out"), M, N, K, int(rows_per_wave), int(cols), int(splits), _ptr(workspace, "workspace"),
        0 if workspace is None else workspace.numel() * workspace.element_size(), _stream(stream))
    _check("ssm_linear_ex", st)
    return out


def linear_plan(M, N, K):
    """ssm_linear_plan: (rows per wave, columns per workgroup, splits) that
    ssm_linear takes for the shape."""
    r, c, s = ctypes.c_int(), ctypes.c_int(), ctypes.c_int()
    _check("ssm_linear_plan", load_library().ssm_linear_plan(M, N, K, ctypes.byref(r), ctypes.byref(c),
                                                             ctypes.byref(s)))
    return r.value, c.value, s.value


def rmsnorm(x, weight, eps=1e-5, out=None, stream=None):
    """ssm_rmsnorm over the last dimension of x [M, D]."""
    M, D = x.shape
    if out is None:
        out = _new_like(x)
    st = load_library().ssm_rmsnorm(_tensor(x, "x"), _tensor(weight, "weight"), _tensor(out, "out"),
                                    M, D, float(eps), _stream(stream))
    _check("ssm_rmsnorm", st)
    return out


def mamba1_layer(weights: dict, eps=1e-5):
    """Build the ssm_mamba1_layer descriptor from a dict of GPU tensors (keys:
    norm_weight, in_proj, conv_weight, conv_bias, x_proj, dt_proj, dt_bias, A,
    D, out_proj).  The tensors must outlive the descriptor."""
    w = weights
    d_inner, d_model = w["in_proj"].shape[0] // 2, w["in_proj"].shape[1]
    d_state = w["A"].shape[1]
    dt_rank = w["dt_proj"].shape[1]
    f32 = torch.float32
    return Mamba1Layer(d_model, d_inner, d_state, dt_rank, w["conv_weight"].shape[1], float(eps),
                       _ptr(w["norm_weight"], "norm_weight", f32), _ptr(w["in_proj"], "in_proj"),
                       _ptr(w["conv_weight"], "conv_weight", f32),
                       _ptr(w.get("conv_bias"), "conv_bias", f32), _ptr(w["x_proj"], "x_proj"),
                       _ptr(w["dt_proj"], "dt_proj"), _ptr(w.get("dt_bias"), "dt_bias", f32),
                       _ptr(w["A"], "A", f32), _ptr(w.get("D"), "D", f32),
                       _ptr(w["out_proj"], "out_proj"))


def mamba1_decode_layer(layer, hidden, conv_state, ssm_state, slot_idx=None, workspace=None,
                        stream=None):
    """ssm_mamba1_decode_layer: hidden [batch, d_model] updated in place."""
    batch = hidden.shape[0]
    lib = load_library()
    need = lib.ssm_mamba1_decode_layer_workspace(ctypes.byref(layer), batch)
    if workspace is None:
        workspace = _workspace(need, hidden.device)
    st = lib.ssm_mamba1_decode_layer(
        ctypes.byref(layer), _tensor(hidden, "hidden"), _tensor(conv_state, "conv_state"),
        _tensor(ssm_state, "ssm_state"), _ptr(slot_idx, "slot_idx", torch.int32), batch,
        conv_state.shape[0], _ptr(workspace, "workspace"),
        0 if workspace is None else workspace.numel() * workspace.element_size(), _stream(stream))
    _check("ssm_mamba1_decode_layer", st)
    return hidden


def mamba1_decode_layer_noalloc(layer, hidden, conv_state, ssm_state, slot_idx=None, stream=None):
    """ssm_mamba1_decode_layer_noalloc: the decode layer with its workspace in
    the library's per-GPU device array (no allocation by caller or library);
    hidden [batch, d_model] updated in place."""
    st = load_library().ssm_mamba1_decode_layer_noalloc(
        ctypes.byref(layer), _tensor(hidden, "hidden"), _tensor(conv_state, "conv_state"),
        _tensor(ssm_state, "ssm_state"), _ptr(slot_idx, "slot_idx", torch.int32), hidden.shape[0],
        conv_state.shape[0], _stream(stream))
    _check("ssm_mamba1_decode_layer_noalloc", st)
    return hidden


__all__ = ["Tensor", "linear", "linear_plan", "mamba1_decode_layer_noalloc", "rmsnorm", "mamba1_layer", "mamba1_decode_layer", "Mamba1Layer",
           "causal_conv1d", "selective_scan", "state_update", "state_update_config",
           "LaunchConfig", "decode_step", "SCAN_AUTO", "SCAN_RECURRENT", "SCAN_CHUNKED",
           "causal_conv1d_varlen", "selective_scan_varlen", "load_library",
           "SsmError",
           "SSM_F32", "SSM_F16", "SSM_BF16", "EXPORTED", "LIB_PATH"]
