"""Seeded synthetic inputs for the causal selective-SSM hot path.

This module only draws random tensors; it holds none of the method's
arithmetic.  The same tensors (the same bytes) feed the HIP path and the
float64 oracle: tensors are drawn with a seeded ``torch.Generator`` on the
device that will use them, rounded once (round-to-nearest-even, by torch's
dtype conversion) to their storage dtype, and the oracle receives exact float64
widenings of those stored values.

Workloads (shapes from the Mamba-2.8B layer and the Mamba-2 / Falcon-H1 decode
shapes the pages measure on; the pages' trained weights and datasets are not
available, so seeded synthetic tensors of the same shapes stand in for them):

* ``tiny``        Mamba-1, fp32: batch 1, L=64, d_inner=128, d_state=16, conv 4.
* ``prefill``     Mamba-1 2.8B layer prefill: batch 4, L=2048, d_inner=5120,
                  d_state=16, conv 4, fp16 I/O, fp32 A/D/state.
* ``decode``      Mamba-1 2.8B decode step: 245 requests gathered from a
                  512-slot cache, conv cache fp16 [512,5120,3], SSM cache fp32
                  [512,5120,16], one fp16 token per request.
* ``m2_ssu_64``   Mamba-2 SSU, headdim 64, dstate 128, 80 heads, ngroups 1 or 8.
* ``m2_ssu_128``  Mamba-2 SSU, headdim 128, dstate 256, 64 heads, ngroups 1,
                  random slots in a 1024-slot cache.
* ``m2_prefill``  Mamba-2 prefill scan, L=4096, batch 2, headdim 128,
                  dstate 256, 64 heads.

Distributions: x, z ~ N(0,1); dt = N(0,1) raw values plus a per-head bias
~ U(ln 1e-3, ln 1e-1) that the kernels add before softplus; Mamba-1
A[c,n] = -(n+1) (S4D-real) and Mamba-2 A_h = -U(1,16); B, C ~ N(0,1) per
(batch, group, state, time); D = 1; conv weight and bias ~ U(-1/2, 1/2); cache
contents ~ N(0,1).  ``index_sensitive=True`` replaces the structured A, D and
the bias with per-channel / per-head random values so that a wrong channel or
head index cannot hide behind identical parameters.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, replace

import numpy as np
import torch

DTYPES = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16}


@dataclass(frozen=True)
class Spec:
    batch: int
    seqlen: int              # 1 for decode
    nheads: int
    headdim: int
    dstate: int
    ngroups: int = 1
    width: int = 4           # conv width; 0 = no conv in this workload
    io: str = "f32"          # dtype of x, dt, B, C, z, out, conv cache
    state: str = "f32"       # dtype of the SSM state cache
    a_per_state: bool = True  # Mamba-1 A[h, n]; False: Mamba-2 scalar A[h]
    nslots: int = 0          # 0: nslots = batch, slot = b
    random_slots: bool = False  # slot_idx = first batch entries of a permutation
    has_initial_state: bool = False
    index_sensitive: bool = False
    seed: int = 0

    @property
    def channels(self) -> int:
        return self.nheads * self.headdim

    @property
    def slots(self) -> int:
        return self.nslots if self.nslots else self.batch


def tiny(**kw) -> Spec:
    return replace(Spec(batch=1, seqlen=64, nheads=128, headdim=1, dstate=16, width=4,
                        io="f32", state="f32", seed=0), **kw)


def prefill(**kw) -> Spec:
    return replace(Spec(batch=4, seqlen=2048, nheads=5120, headdim=1, dstate=16, width=4,
                        io="f16", state="f32", seed=1), **kw)


def decode(**kw) -> Spec:
    return replace(Spec(batch=245, seqlen=1, nheads=5120, headdim=1, dstate=16, width=4,
                        io="f16", state="f32", nslots=512, random_slots=True,
                        has_initial_state=True, seed=2), **kw)


def m2_ssu_64(batch=1024, ngroups=1, state="f16", **kw) -> Spec:
    return replace(Spec(batch=batch, seqlen=1, nheads=80, headdim=64, dstate=128,
                        ngroups=ngroups, width=0, io="f16", state=state, a_per_state=False,
                        has_initial_state=True, seed=3), **kw)


def m2_ssu_128(batch=512, state="bf16", **kw) -> Spec:
    return replace(Spec(batch=batch, seqlen=1, nheads=64, headdim=128, dstate=256,
                        ngroups=1, width=0, io="bf16", state=state, a_per_state=False,
                        nslots=1024, random_slots=True, has_initial_state=True,
                        seed=4), **kw)


def m2_prefill(state="bf16", **kw) -> Spec:
    return replace(Spec(batch=2, seqlen=4096, nheads=64, headdim=128, dstate=256,
                        ngroups=1, width=0, io="bf16", state=state, a_per_state=False,
                        nslots=1024, random_slots=True, seed=4), **kw)


class _Draw:
    """One seeded generator per tensor, in a fixed order, on one device."""

    def __init__(self, seed: int, device):
        self.seed = int(seed)
        self.device = torch.device(device)
        self.k = 0

    def gen(self) -> torch.Generator:
        g = torch.Generator(device=self.device)
        g.manual_seed(self.seed * 1_000_003 + 7919 * self.k)
        self.k += 1
        return g

    def normal(self, shape, dtype):
        t = torch.randn(shape, generator=self.gen(), device=self.device, dtype=torch.float32)
        return t.to(dtype)

    def uniform(self, shape, lo, hi, dtype=torch.float32):
        t = torch.rand(shape, generator=self.gen(), device=self.device, dtype=torch.float32)
        return (lo + (hi - lo) * t).to(dtype)

    def perm(self, n):
        return torch.randperm(n, generator=self.gen(), device=self.device, dtype=torch.int64)


def make(spec: Spec, device="cpu") -> dict:
    """Draw every tensor of a workload.  Prefill layouts are channel-major,
    time innermost; decode tensors are the seqlen == 1 case of the same layout
    (x/z/out [batch, nheads, headdim], dt [batch, nheads], B/C [batch, ngroups,
    dstate])."""
    io = DTYPES[spec.io]
    st = DTYPES[spec.state]
    d = _Draw(spec.seed, device)
    Bt, L, H, P, N, G = spec.batch, spec.seqlen, spec.nheads, spec.headdim, spec.dstate, spec.ngroups
    Cn, S = spec.channels, spec.slots
    t = {}
    # fixed draw order: x, z, dt, dt_bias, A, B, C, D, conv_w, conv_b, conv_state,
    # ssm_state, slot_idx
    t["x"] = d.normal((Bt, Cn, L), io)
    t["z"] = d.normal((Bt, Cn, L), io)
    t["dt"] = d.normal((Bt, H, L), io)
    t["dt_bias"] = d.uniform((H,), math.log(1e-3), math.log(1e-1))
    if spec.a_per_state:
        if spec.index_sensitive:
            t["A"] = -d.uniform((H, N), 0.5, N + 0.5)
        else:
            d.gen()
            t["A"] = -torch.arange(1, N + 1, dtype=torch.float32, device=d.device).repeat(H, 1)
    else:
        t["A"] = -d.uniform((H,), 1.0, 16.0)
    t["B"] = d.normal((Bt, G, N, L), io)
    t["C"] = d.normal((Bt, G, N, L), io)
    if spec.index_sensitive:
        t["D"] = d.uniform((H,), 0.5, 1.5)
    else:
        d.gen()
        t["D"] = torch.ones((H,), dtype=torch.float32, device=d.device)
    if spec.width > 0:
        t["conv_w"] = d.uniform((Cn, spec.width), -0.5, 0.5)
        t["conv_b"] = d.uniform((Cn,), -0.5, 0.5)
        t["conv_state"] = d.normal((S, Cn, spec.width - 1), io)
    else:
        d.gen(); d.gen(); d.gen()
    t["ssm_state"] = d.normal((S, H, P, N), st)
    if spec.random_slots:
        t["slot_idx"] = d.perm(S)[:Bt].to(torch.int32).contiguous()
    else:
        d.gen()
        t["slot_idx"] = torch.arange(Bt, dtype=torch.int32, device=d.device)
    if L == 1:
        # decode views: same memory, decode shapes
        t["x"] = t["x"].view(Bt, H, P)
        t["z"] = t["z"].view(Bt, H, P)
        t["dt"] = t["dt"].view(Bt, H)
        t["B"] = t["B"].view(Bt, G, N)
        t["C"] = t["C"].view(Bt, G, N)
    return t


def varlen_lengths(seed: int, nseq: int, total: int, lo: int = 1) -> list:
    """A seeded mix of nseq sequence lengths summing to total: log-uniform
    draws between lo and total (short requests next to long ones, as in a
    continuous-batching prefill), rescaled to the total.  Lengths are not
    rounded to any multiple."""
    g = torch.Generator().manual_seed(int(seed) * 7_368_787 + 11)
    u = torch.rand(nseq, generator=g, dtype=torch.float64)
    raw = torch.exp(math.log(lo) + u * (math.log(max(total, lo + 1)) - math.log(lo)))
    lens = [max(lo, int(v)) for v in (raw / raw.sum() * total)]
    lens[int(torch.argmax(raw))] += total - sum(lens)
    return lens


def make_varlen(spec: Spec, lengths, device="cpu", init_every: int = 2) -> dict:
    """Draw a packed variable-length prefill: the sequences of `lengths`
    concatenated along time, x/z [channels, T], dt [nheads, T], B/C [ngroups,
    dstate, T] (T = sum of lengths), with the parameters and caches of `spec`
    (spec.batch is ignored: one sequence per length).  Every init_every-th
    sequence (from the first) continues from its slot's state; slots are the
    first len(lengths) entries of a permutation of the cache."""
    io = DTYPES[spec.io]
    st = DTYPES[spec.state]
    d = _Draw(spec.seed, device)
    H, P, N, G = spec.nheads, spec.headdim, spec.dstate, spec.ngroups
    Cn, nseq = spec.channels, len(lengths)
    S = max(spec.nslots, nseq)
    T = int(sum(lengths))
    t = {}
    t["x"] = d.normal((Cn, T), io)
    t["z"] = d.normal((Cn, T), io)
    t["dt"] = d.normal((H, T), io)
    t["dt_bias"] = d.uniform((H,), math.log(1e-3), math.log(1e-1))
    if spec.a_per_state:
        t["A"] = -d.uniform((H, N), 0.5, N + 0.5)
    else:
        t["A"] = -d.uniform((H,), 1.0, 16.0)
    t["B"] = d.normal((G, N, T), io)
    t["C"] = d.normal((G, N, T), io)
    t["D"] = d.uniform((H,), 0.5, 1.5)
    t["conv_w"] = d.uniform((Cn, spec.width), -0.5, 0.5)
    t["conv_b"] = d.uniform((Cn,), -0.5, 0.5)
    t["conv_state"] = d.normal((S, Cn, spec.width - 1), io)
    t["ssm_state"] = d.normal((S, H, P, N), st)
    t["slot_idx"] = d.perm(S)[:nseq].to(torch.int32).contiguous()
    cu = [0]
    for n in lengths:
        cu.append(cu[-1] + int(n))
    t["cu_seqlens"] = torch.tensor(cu, dtype=torch.int32, device=d.device)
    t["has_init"] = torch.tensor([1 if (init_every and s % init_every == 0) else 0
                                  for s in range(nseq)], dtype=torch.int32, device=d.device)
    return t


def varlen_bytes(spec: Spec, lengths, n_init: int) -> dict:
    """Algorithmic bytes of a packed prefill: the dense formula with the
    token count T in place of batch x seqlen, plus each sequence's cache
    rows (read when it continues from its slot, always written)."""
    isz = {"f32": 4, "f16": 2, "bf16": 2}
    io, st = isz[spec.io], isz[spec.state]
    T, nseq = int(sum(lengths)), len(lengths)
    H, P, N, G, W = spec.nheads, spec.headdim, spec.dstate, spec.ngroups, spec.width
    Cn = H * P
    conv = 2 * Cn * T * io + Cn * W * 4 + Cn * 4 + (nseq + n_init) * Cn * (W - 1) * io + (nseq + 1) * 4
    scan = (2 * Cn * T * io + H * T * io + 2 * G * N * T * io + Cn * T * io
            + (H * N if spec.a_per_state else H) * 4 + 2 * H * 4
            + (nseq + n_init) * H * P * N * st + (nseq + 1) * 4)
    return {"conv": conv, "scan": scan}


def mamba1_layer(d_model=2560, d_inner=5120, d_state=16, dt_rank=160, width=4, batch=245,
                 nslots=512, io="f16", state="f32", seed=7, device="cpu") -> dict:
    """Random weights and decode inputs of one Mamba-1 layer (Mamba-2.8B
    sizes by default): projections ~ N(0, 1/fan_in) in the io dtype, RMSNorm
    weight ~ U(0.5, 1.5), conv taps and bias ~ U(-1/2, 1/2), dt bias such
    that softplus(bias) is log-uniform in [1e-3, 1e-1], A[c, n] = -(n+1),
    D = 1; hidden ~ N(0, 1), caches ~ N(0, 1); slots = the first `batch`
    entries of a permutation of the cache."""
    io_t, st_t = DTYPES[io], DTYPES[state]
    d = _Draw(seed, device)

    def proj(n_out, n_in):
        return (d.normal((n_out, n_in), torch.float32) / math.sqrt(n_in)).to(io_t)

    w = {
        "norm_weight": d.uniform((d_model,), 0.5, 1.5),
        "in_proj": proj(2 * d_inner, d_model),
        "conv_weight": d.uniform((d_inner, width), -0.5, 0.5),
        "conv_bias": d.uniform((d_inner,), -0.5, 0.5),
        "x_proj": proj(dt_rank + 2 * d_state, d_inner),
        "dt_proj": proj(d_inner, dt_rank),
    }
    dtv = torch.exp(d.uniform((d_inner,), math.log(1e-3), math.log(1e-1)))
    w["dt_bias"] = dtv + torch.log(-torch.expm1(-dtv))  # softplus^-1
    w["A"] = -torch.arange(1, d_state + 1, dtype=torch.float32, device=d.device).repeat(d_inner, 1)
    w["D"] = torch.ones(d_inner, dtype=torch.float32, device=d.device)
    w["out_proj"] = proj(d_model, d_inner)
    t = {"w": w,
         "hidden": d.normal((batch, d_model), io_t),
         "conv_state": d.normal((nslots, d_inner, width - 1), io_t),
         "ssm_state": d.normal((nslots, d_inner, 1, d_state), st_t),
         "slot_idx": d.perm(nslots)[:batch].to(torch.int32).contiguous()}
    return t


def layer_bytes(d_model, d_inner, d_state, dt_rank, width, batch, io="f16", state="f32") -> dict:
    """Bytes one decode layer must move: every weight once, the state and
    conv window of each request read and written, the hidden rows read and
    written, and each intermediate written and read once."""
    isz = {"f32": 4, "f16": 2, "bf16": 2}
    io_b, st_b = isz[io], isz[state]
    weights = (2 * d_inner * d_model + (dt_rank + 2 * d_state) * d_inner + d_inner * dt_rank
               + d_model * d_inner) * io_b + (d_model + d_inner * (width + 3 + d_state)) * 4
    caches = batch * d_inner * (2 * (width - 1) * io_b + 2 * d_state * st_b)
    acts = batch * io_b * (2 * d_model + 2 * (d_model + 5 * d_inner + dt_rank + 2 * d_state
                                              + d_inner))
    return {"weights": weights, "caches": caches, "activations": acts,
            "total": weights + caches + acts}


def to_f64(a) -> np.ndarray:
    """Exact float64 widening of a stored tensor (any of f32/f16/bf16/ints)."""
    if a is None:
        return None
    if isinstance(a, torch.Tensor):
        a = a.detach().cpu()
        if a.dtype in (torch.float16, torch.bfloat16):
            a = a.to(torch.float32)
        return a.numpy().astype(np.float64)
    return np.asarray(a, dtype=np.float64)


def algorithmic_bytes(spec: Spec) -> dict:
    """Bytes the method must move (each input read once, each output written
    once), per kernel, for a workload."""
    isz = {"f32": 4, "f16": 2, "bf16": 2}
    io, st = isz[spec.io], isz[spec.state]
    Bt, L, H, P, N, G = spec.batch, spec.seqlen, spec.nheads, spec.headdim, spec.dstate, spec.ngroups
    Cn, W = spec.channels, spec.width
    out = {}
    if L > 1:
        if W:
            out["conv"] = (2 * Bt * Cn * L * io + Cn * W * 4 + Cn * 4 + Bt * Cn * (W - 1) * io
                           * (2 if spec.has_initial_state else 1))
        scan = (2 * Bt * Cn * L * io          # u, z
                + Bt * H * L * io             # dt
                + 2 * Bt * G * N * L * io     # B, C
                + Bt * Cn * L * io            # out
                + (H * N if spec.a_per_state else H) * 4 + 2 * H * 4   # A, D, dt_bias
                + Bt * H * P * N * st * (2 if spec.has_initial_state else 1))
        out["scan"] = scan
    else:
        if W:
            out["conv"] = 2 * Bt * Cn * (W - 1) * io + 2 * Bt * Cn * io + Cn * W * 4 + Cn * 4
        out["ssu"] = (2 * Bt * H * P * N * st          # state read + write
                      + 3 * Bt * H * P * io            # x, z, out
                      + Bt * H * io                    # dt
                      + 2 * Bt * G * N * io            # B, C
                      + (H * N if spec.a_per_state else H) * 4 + 2 * H * 4
                      + Bt * 4)                        # slot_idx
    return out


def algorithmic_flops(spec: Spec) -> float:
    """Floating-point operations the recurrence needs, counting an exponential
    as one operation and an FMA as two: per (batch, channel, time, state)
    element, Mamba-1 takes delta*A (1), exp (1), (delta*u)*B (1), the state FMA
    (2) and the readout FMA (2); Mamba-2 shares delta*A and exp across states
    (per head and time: 2) and keeps 5 per element.  Per (batch, channel, time)
    another 14: softplus (6), delta*u (1), D*u plus add (2), SiLU (4), gate (1).
    """
    Bt, L, H, P, N = spec.batch, spec.seqlen, spec.nheads, spec.headdim, spec.dstate
    Cn = H * P
    per_elem = 7 if spec.a_per_state else 5
    flops = Bt * Cn * L * N * per_elem + Bt * Cn * L * 14
    if not spec.a_per_state:
        flops += Bt * H * L * 2
    return float(flops)


def chunked_mfma_flops(spec: Spec, chunk: int = 64) -> float:
    """Dense matrix work of the chunked (SSD) form of a Mamba-2 prefill, per
    (request, head, chunk of Q steps): C B^T (Q x Q x N), its masked product
    with X (Q x Q x P), the readout of the carried state C h (Q x N x P) and
    the state update B^T X (N x Q x P), two flops per multiply-add.  Counts
    full Q x Q products (no saving from the causal mask) and operands at
    their own precision (no split-operand passes)."""
    Bt, L, H, P, N = spec.batch, spec.seqlen, spec.nheads, spec.headdim, spec.dstate
    Q = chunk
    nchunks = (L + Q - 1) // Q
    per = 2 * Q * (Q * N + Q * P + 2 * N * P)
    return float(Bt * H * nchunks * per)
