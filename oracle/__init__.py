"""Float64 CPU oracle for the causal selective-SSM hot path.

TEST INFRASTRUCTURE ONLY: imported by ``tests/``, by ``__graft_entry__.smoke()``
and by the CPU-baseline leg of ``bench.py``; never by the product package.  It
shares no code with the HIP path.  The arithmetic lives in ``ssm_oracle.c``
(plain sequential C, double precision); this module only compiles it with gcc
and marshals numpy arrays in and out.

What it computes (equations, layouts, slot convention) is documented at the top
of ``ssm_oracle.c``; each entry below names the passage it follows.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "ssm_oracle.c")
# SSM_ORACLE_LIB points the wrapper at another build of ssm_oracle.c (the
# mutation test uses it to check that the pins reject planted mistakes).
_LIB = os.environ.get("SSM_ORACLE_LIB") or os.path.join(_HERE, "libssm_oracle.so")
_lib = None

F32, F16, BF16 = 0, 1, 2  # rounding kinds of oracle_round


def build(force: bool = True) -> str:
    """Compile ssm_oracle.c into libssm_oracle.so with gcc (plain -O2, IEEE)."""
    global _lib
    if force or not os.path.exists(_LIB):
        tmp = _LIB + ".tmp"
        subprocess.check_call(
            ["gcc", "-O2", "-std=c99", "-fPIC", "-shared", "-Wall", "-Wextra",
             "-o", tmp, _SRC, "-lm"])
        os.replace(tmp, _LIB)
        _lib = None
    return _LIB


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB):
        build(force=True)
    lib = ctypes.CDLL(_LIB)
    dp = ctypes.POINTER(ctypes.c_double)
    ip = ctypes.POINTER(ctypes.c_int32)
    I = ctypes.c_int
    lib.oracle_softplus.argtypes = [ctypes.c_double]
    lib.oracle_softplus.restype = ctypes.c_double
    lib.oracle_silu.argtypes = [ctypes.c_double]
    lib.oracle_silu.restype = ctypes.c_double
    lib.oracle_round.argtypes = [ctypes.c_double, I]
    lib.oracle_round.restype = ctypes.c_double
    lib.oracle_round_array.argtypes = [dp, ctypes.c_size_t, I]
    lib.oracle_round_array.restype = None
    lib.oracle_causal_conv1d.argtypes = [I, I, I, I, dp, dp, dp, dp, ip, I, I, I, dp, dp]
    lib.oracle_causal_conv1d.restype = I
    lib.oracle_selective_scan.argtypes = [I, I, I, I, I, I, dp, dp, dp, I, dp, I, dp, dp, dp,
                                          dp, dp, ip, I, I, dp, dp, dp]
    lib.oracle_selective_scan.restype = I
    lib.oracle_state_update.argtypes = [I, I, I, I, I, dp, ip, I, dp, dp, dp, I, dp, I, dp, dp,
                                        dp, dp, dp, dp, dp]
    lib.oracle_state_update.restype = I
    _lib = lib
    return lib


def _f64(a):
    return None if a is None else np.ascontiguousarray(a, dtype=np.float64)


def _dp(a):
    if a is None:
        return None
    return a.ctypes.data_as(ctypes.POINTER(ctypes.c_double))


def _ip(a):
    if a is None:
        return None
    return a.ctypes.data_as(ctypes.POINTER(ctypes.c_int32))


def _idx(a):
    return None if a is None else np.ascontiguousarray(a, dtype=np.int32)


def softplus(v: float) -> float:
    """log(1 + e^v) in double (the dt preprocessing named by dt_softplus=True
    in the decode call of the vLLM PR #50534 report, "关键源码片段")."""
    return _load().oracle_softplus(float(v))


def silu(v: float) -> float:
    """v * sigmoid(v) (the silu operator of InfiniLM-Rust PR #48, section 2.1)."""
    return _load().oracle_silu(float(v))


def round_to(a, kind: int) -> np.ndarray:
    """Round a float64 array to binary32 / binary16 / bfloat16 (RNE), result
    kept in float64."""
    out = np.array(a, dtype=np.float64, copy=True, order="C")
    _load().oracle_round_array(_dp(out), out.size, int(kind))
    return out


def causal_conv1d(x, weight, bias=None, conv_state=None, slot_idx=None,
                  has_initial_state=False, apply_silu=True, out=None):
    """Causal depthwise conv1d + optional SiLU with an optional conv cache
    (causal-conv1d and silu of InfiniLM-Rust PR #48 section 2.1; cache reads
    and writes at the conv operator, section 3.1).

    x: [batch, channels, seqlen]; weight: [channels, width]; bias: [channels];
    conv_state: [nslots, channels, width-1] (copied, the updated copy is
    returned); slot_idx: int32 [batch] or None.
    Returns (out, out_scale, conv_state_after).
    """
    x = _f64(x)
    weight = _f64(weight)
    bias = _f64(bias)
    batch, channels, seqlen = x.shape
    width = weight.shape[1]
    cs = None if conv_state is None else np.array(conv_state, dtype=np.float64, copy=True, order="C")
    nslots = 0 if cs is None else cs.shape[0]
    idx = _idx(slot_idx)
    o = np.zeros_like(x) if out is None else np.array(out, dtype=np.float64, copy=True, order="C")
    sc = np.zeros_like(x)
    rc = _load().oracle_causal_conv1d(batch, channels, seqlen, width, _dp(x), _dp(weight),
                                      _dp(bias), _dp(cs), _ip(idx), nslots,
                                      int(bool(has_initial_state)), int(bool(apply_silu)),
                                      _dp(o), _dp(sc))
    if rc != 0:
        raise ValueError("oracle_causal_conv1d rejected its arguments")
    return o, sc, cs


def selective_scan(u, dt, A, B, C, D=None, z=None, dt_bias=None, dt_softplus=True,
                   state=None, slot_idx=None, has_initial_state=False, out=None):
    """Selective scan over a sequence (selective-scan of InfiniLM-Rust PR #48
    section 2.1, with the element-mul gate by silu(z)); final state written to
    the request's slot (section 3.1).

    u, z: [batch, nheads*headdim, seqlen]; dt: [batch, nheads, seqlen];
    A: [nheads, dstate] (per state) or [nheads] (scalar per head);
    B, C: [batch, ngroups, dstate, seqlen]; D, dt_bias: [nheads];
    state: [nslots, nheads, headdim, dstate] (copied; updated copy returned).
    Returns (out, out_scale, state_after, state_scale).
    """
    u, dt, A, B, C = _f64(u), _f64(dt), _f64(A), _f64(B), _f64(C)
    D, z, dt_bias = _f64(D), _f64(z), _f64(dt_bias)
    batch, channels, seqlen = u.shape
    nheads = dt.shape[1]
    headdim = channels // nheads
    ngroups, dstate = B.shape[1], B.shape[2]
    a_per_state = 1 if A.ndim == 2 else 0
    st = None if state is None else np.array(state, dtype=np.float64, copy=True, order="C")
    nslots = 0 if st is None else st.shape[0]
    sts = None if st is None else np.zeros_like(st)
    idx = _idx(slot_idx)
    o = np.zeros_like(u) if out is None else np.array(out, dtype=np.float64, copy=True, order="C")
    sc = np.zeros_like(u)
    rc = _load().oracle_selective_scan(batch, seqlen, nheads, headdim, dstate, ngroups,
                                       _dp(u), _dp(dt), _dp(dt_bias), int(bool(dt_softplus)),
                                       _dp(A), a_per_state, _dp(B), _dp(C), _dp(D), _dp(z),
                                       _dp(st), _ip(idx), nslots, int(bool(has_initial_state)),
                                       _dp(o), _dp(sc), _dp(sts))
    if rc != 0:
        raise ValueError("oracle_selective_scan rejected its arguments")
    return o, sc, st, sts


def state_update(state, x, dt, A, B, C, D=None, z=None, dt_bias=None, dt_softplus=True,
                 slot_idx=None, out=None):
    """One-token selective state update, in place on a slot-indexed cache (the
    selective_state_update(state, x, dt, A, B, C, D=D, z=None, dt_bias=dt_bias,
    dt_softplus=True, out=out) call of the vLLM PR #50534 report,
    "关键源码片段").

    state: [nslots, nheads, headdim, dstate] (copied; updated copy returned);
    x, z: [batch, nheads, headdim]; dt: [batch, nheads]; B, C: [batch, ngroups,
    dstate]; A: [nheads, dstate] or [nheads].
    Returns (out, out_scale, state_after, state_scale).
    """
    x, dt, A, B, C = _f64(x), _f64(dt), _f64(A), _f64(B), _f64(C)
    D, z, dt_bias = _f64(D), _f64(z), _f64(dt_bias)
    st = np.array(state, dtype=np.float64, copy=True, order="C")
    nslots, nheads, headdim, dstate = st.shape
    batch = x.shape[0]
    ngroups = B.shape[1]
    a_per_state = 1 if A.ndim == 2 else 0
    idx = _idx(slot_idx)
    o = np.zeros_like(x) if out is None else np.array(out, dtype=np.float64, copy=True, order="C")
    sc = np.zeros_like(x)
    sts = np.zeros_like(st)
    rc = _load().oracle_state_update(batch, nheads, headdim, dstate, ngroups, _dp(st), _ip(idx),
                                     nslots, _dp(x), _dp(dt), _dp(dt_bias), int(bool(dt_softplus)),
                                     _dp(A), a_per_state, _dp(B), _dp(C), _dp(D), _dp(z),
                                     _dp(o), _dp(sc), _dp(sts))
    if rc != 0:
        raise ValueError("oracle_state_update rejected its arguments")
    return o, sc, st, sts


def _seq_bounds(cu_seqlens):
    cu = [int(v) for v in np.asarray(cu_seqlens).reshape(-1)]
    return [(cu[s], cu[s + 1]) for s in range(len(cu) - 1)]


def causal_conv1d_varlen(x, weight, cu_seqlens, bias=None, conv_state=None, slot_idx=None,
                         has_initial_state=None, apply_silu=True, out=None):
    """Packed variable-length batch of the conv: x [channels, total_len] holds
    the sequences at columns [cu_seqlens[s], cu_seqlens[s+1]).  By definition
    each sequence is one independent dense call (batch 1) on its own columns,
    with its own slot and initial-state flag (one mamba cache per request,
    InfiniLM-Rust PR #48 section 3.1); padded (slot < 0) and empty sequences
    are skipped.  No arithmetic of its own: it slices and calls
    causal_conv1d.  Returns (out, out_scale, conv_state_after)."""
    x = _f64(x)
    cs = None if conv_state is None else np.array(conv_state, dtype=np.float64, copy=True, order="C")
    o = np.zeros_like(x) if out is None else np.array(out, dtype=np.float64, copy=True, order="C")
    sc = np.zeros_like(x)
    for s, (tb, te) in enumerate(_seq_bounds(cu_seqlens)):
        slot = s if slot_idx is None else int(slot_idx[s])
        if slot < 0 or te == tb:
            continue
        init = bool(has_initial_state[s]) if has_initial_state is not None else False
        os_, ss_, cs = causal_conv1d(x[None, :, tb:te], weight, bias, conv_state=cs,
                                     slot_idx=None if cs is None else [slot],
                                     has_initial_state=init, apply_silu=apply_silu)
        o[:, tb:te] = os_[0]
        sc[:, tb:te] = ss_[0]
    return o, sc, cs


def selective_scan_varlen(u, dt, A, B, C, cu_seqlens, D=None, z=None, dt_bias=None,
                          dt_softplus=True, state=None, slot_idx=None, has_initial_state=None,
                          out=None):
    """Packed variable-length batch of the scan: u, z [nheads*headdim,
    total_len], dt [nheads, total_len], B, C [ngroups, dstate, total_len].
    Each sequence is one independent dense call (batch 1) on its columns,
    starting from its slot's state when its flag is set and leaving its final
    state in the slot; padded and empty sequences are skipped.  No arithmetic
    of its own: it slices and calls selective_scan.
    Returns (out, out_scale, state_after, state_scale)."""
    u, dt, B, C = _f64(u), _f64(dt), _f64(B), _f64(C)
    z = _f64(z)
    st = None if state is None else np.array(state, dtype=np.float64, copy=True, order="C")
    sts = None if st is None else np.zeros_like(st)
    o = np.zeros_like(u) if out is None else np.array(out, dtype=np.float64, copy=True, order="C")
    sc = np.zeros_like(u)
    for s, (tb, te) in enumerate(_seq_bounds(cu_seqlens)):
        slot = s if slot_idx is None else int(slot_idx[s])
        if slot < 0 or te == tb:
            continue
        init = bool(has_initial_state[s]) if has_initial_state is not None else False
        os_, ss_, st_new, sts_new = selective_scan(
            u[None, :, tb:te], dt[None, :, tb:te], A, B[None, :, :, tb:te], C[None, :, :, tb:te],
            D=D, z=None if z is None else z[None, :, tb:te], dt_bias=dt_bias,
            dt_softplus=dt_softplus, state=st, slot_idx=None if st is None else [slot],
            has_initial_state=init)
        o[:, tb:te] = os_[0]
        sc[:, tb:te] = ss_[0]
        if st is not None:
            st = st_new
            sts[slot] = sts_new[slot]
    return o, sc, st, sts
