// ssu.hip -- single-token selective state update (decode) on gfx950.
//
// Operation: the selective_state_update call described in "[XPU] Add tuned
// Mamba SSU configs for Intel Arc Pro B70" (vLLM PR #50534 report, section
// "关键源码片段"): for every request b with slot s = slot_idx[b] >= 0, head h,
// row p and state n,
//     delta = softplus(dt[b,h] + dt_bias[h])
//     h'    = exp(delta * A[h,n]) * state[s,h,p,n] + delta * B[b,g,n] * x[b,h,p]
//     out   = (sum_n C[b,g,n] * h' + D[h] * x[b,h,p]) * silu(z[b,h,p])
// with h' written back to state[s,h,p,n] in the cache dtype.
//
// Design: the kernel is bound by streaming the state cache once (read +
// write).  One lane owns V (8 or 16) consecutive states of one (b,h,p) row, so
// a row of dstate states is dstate/V lanes (rounded up to a power of two that
// divides 64) and a wave covers 64*V consecutive states of the cache, read and
// written with 128-bit accesses.  The readout sum over states is a butterfly
// across the row's lanes.  No LDS, no barriers.  V and the workgroup size
// (64 to 512 lanes) are chosen per shape on the host, from a table tuned on
// gfx950 or a heuristic, or given by the caller.
#include "ssm_device.hpp"
#include "ssm_kernels.hpp"

namespace ssm {

// What one lane holds for its (h,p) row and state range that does not depend
// on the request: loaded once and used for each of the lane's requests.
template <int V, int CW>
struct SsuParams {
    float an[V];                      // A[h, n] * log2(e) (per-state decays)
    float a2;                         // A[h] * log2(e) (one decay per head)
    float tap[CW > 0 ? CW : 1];
    float cbias, dtb, Dh;
    int64_t hp;                       // h * headdim + p
    int h, n0;
    bool in;                          // the lane has a row and a state range
};

// What one lane holds for one request between issuing its loads and storing
// its results.
template <typename TS, typename TI, int V, int CW>
struct SsuReq {
    float hs[V], bv[V], cv[V];
    // the row's values as stored (loaded by its first lane; widened when used,
    // so that no load waits inside the branch that issues it)
    TI dt_raw, x_raw, z_raw;
    TI win_raw[CW > 1 ? CW - 1 : 1];
    float delta, xv, zv;
    int64_t bh;                       // b * nheads + h
    TS *sp;
    TI *cw;
    int64_t row;                      // (b * nheads + h) * headdim + p
    bool live;
};

template <bool A_PER_STATE, bool VEC, int V, int CW>
__device__ __forceinline__ void ssu_params(const SsuArgs &a, int64_t hp, int j, SsuParams<V, CW> &q)
{
    const int64_t HP = (int64_t)a.nheads * a.headdim;
    const int n0 = j * V;
    q.in = hp < HP && n0 < a.dstate;
    q.hp = hp < HP ? hp : 0;
    q.h = (int)(q.hp / a.headdim);
    q.n0 = n0 < a.dstate ? n0 : 0;
    if constexpr (A_PER_STATE) {
        const float *Ap = a.A + (int64_t)q.h * a.dstate + q.n0;
        if constexpr (VEC) {
            load_vec_cached<float, V>(Ap, q.an);
        } else {
#pragma unroll
            for (int i = 0; i < V; ++i) {
                const bool ok = q.n0 + i < a.dstate;
                const float av = Ap[ok ? i : 0];
                q.an[i] = ok ? av : 0.0f;
            }
        }
#pragma unroll
        for (int i = 0; i < V; ++i)
            q.an[i] *= kLog2e;
        q.a2 = 0.0f;
    } else {
        q.a2 = a.A[q.h] * kLog2e;
    }
    // the row's first lane takes the step size, the conv and the readout's
    // D term: only it needs dt_bias, D and the conv taps
    q.dtb = q.Dh = q.cbias = 0.0f;
#pragma unroll
    for (int k = 0; k < (CW > 0 ? CW : 1); ++k)
        q.tap[k] = 0.0f;
    if (j == 0) {
        q.dtb = a.dt_bias ? a.dt_bias[q.h] : 0.0f;
        q.Dh = a.D ? a.D[q.h] : 0.0f;
        if constexpr (CW > 0) {
#pragma unroll
            for (int k = 0; k < CW; ++k)
                q.tap[k] = a.conv_weight[q.hp * CW + k];
            q.cbias = a.conv_bias ? a.conv_bias[q.hp] : 0.0f;
        }
    }
}

// Phase 1 for one request: resolve its slot and issue all of its loads.
template <typename TS, typename TI, bool VEC, int V, int CW>
__device__ __forceinline__ void ssu_load(const SsuArgs &a, int b, int j, const SsuParams<V, CW> &q,
                                         SsuReq<TS, TI, V, CW> &r)
{
    const bool bin = b < a.batch;
    const int bb = bin ? b : 0;
    const int slot = a.slot_idx ? a.slot_idx[bb] : bb;  // uniform over the workgroup
    r.live = q.in && bin && slot >= 0;  // padded: loads from slot 0, discarded
    const int s = slot >= 0 ? slot : 0;
    r.row = (int64_t)bb * a.nheads * a.headdim + q.hp;
    const int64_t bh = (int64_t)bb * a.nheads + q.h;
    const int g = q.h / a.heads_per_group;
    r.sp = static_cast<TS *>(a.state) + (((int64_t)s * a.nheads * a.headdim + q.hp) * a.dstate + q.n0);
    const int64_t bc_off = ((int64_t)bb * a.ngroups + g) * a.dstate + q.n0;
    const TI *Bp = static_cast<const TI *>(a.B) + bc_off;
    const TI *Cp = static_cast<const TI *>(a.C) + bc_off;
    r.dt_raw = r.x_raw = r.z_raw = TI{};
    r.bh = bh;
    if constexpr (CW > 0) {
        r.cw = static_cast<TI *>(a.conv_state) + ((int64_t)s * a.nheads * a.headdim + q.hp) * (CW - 1);
#pragma unroll
        for (int k = 0; k < CW - 1; ++k)
            r.win_raw[k] = TI{};
    }
    if constexpr (VEC) {
        load_vec_cached<TS, V>(r.sp, r.hs);
        if constexpr (V * StorageSize<TI>::value >= 16) {
            load_vec_cached<TI, V>(Bp, r.bv);
            load_vec_cached<TI, V>(Cp, r.cv);
        } else {
#pragma unroll
            for (int i = 0; i < V; ++i) {
                r.bv[i] = to_f32(Bp[i]);
                r.cv[i] = to_f32(Cp[i]);
            }
        }
    } else {
#pragma unroll
        for (int i = 0; i < V; ++i) {
            const bool ok = q.n0 + i < a.dstate;
            const int ii = ok ? i : 0;
            const float hv = to_f32(r.sp[ii]), bvv = to_f32(Bp[ii]), cvv = to_f32(Cp[ii]);
            r.hs[i] = ok ? hv : 0.0f;
            r.bv[i] = ok ? bvv : 0.0f;
            r.cv[i] = ok ? cvv : 0.0f;
        }
    }
}

// Phase 1b: the row's values (dt, x, z, the conv window), loaded by the row's
// first lane only, after every lane's state loads have been issued (a wait
// for these then covers all of them at once).
template <typename TS, typename TI, int V, int CW>
__device__ __forceinline__ void ssu_load_row(const SsuArgs &a, SsuReq<TS, TI, V, CW> &r)
{
    r.dt_raw = static_cast<const TI *>(a.dt)[r.bh];
    r.x_raw = static_cast<const TI *>(a.x)[r.row];
    if (a.z)
        r.z_raw = static_cast<const TI *>(a.z)[r.row];
    if constexpr (CW > 0) {
#pragma unroll
        for (int k = 0; k < CW - 1; ++k)
            r.win_raw[k] = r.cw[k];
    }
}

// Phase 2 for one request: (fused conv), state update, store, partial readout.
template <typename TS, typename TI, bool A_PER_STATE, bool VEC, int V, int CW>
__device__ __forceinline__ float ssu_compute(const SsuArgs &a, int j, const SsuParams<V, CW> &q,
                                             SsuReq<TS, TI, V, CW> &r)
{
    // the row's first lane holds dt, x, z and the window: it takes the step
    // size and the conv, then shares both with the row's other lanes
    float xv = to_f32(r.x_raw);
    r.zv = to_f32(r.z_raw);
    if constexpr (CW > 0) {
        // fused conv update of channel hp; the first lane also shifts the
        // cached window (its stored values depend on the window loads, so
        // the read has returned first)
        constexpr int HW = CW - 1;
        float acc = q.cbias;
#pragma unroll
        for (int k = 0; k < HW; ++k)
            acc = fmaf(q.tap[k], to_f32(r.win_raw[k]), acc);
        acc = fmaf(q.tap[HW], xv, acc);
        const float u = silu_f32(acc);
        if (r.live && j == 0) {
#pragma unroll
            for (int k = 0; k + 1 < HW; ++k)
                r.cw[k] = r.win_raw[k + 1];
            if (HW > 0)
                r.cw[HW - 1] = r.x_raw;
            if (a.u_out)
                static_cast<TI *>(a.u_out)[r.row] = from_f32<TI>(u);
        }
        xv = u;  // the update reads the float32 conv output
    }
    const float v = to_f32(r.dt_raw) + q.dtb;
    float delta = a.dt_softplus ? softplus_f32(v) : v;
    // rows of 2 or 4 lanes: a quad permutation (a VALU move); wider rows: the
    // LDS crossbar
    if (a.lanes_per_row_log2 == 1) {
        delta = dpp_move_zero<DPP_QUAD_BCAST2>(delta);
        xv = dpp_move_zero<DPP_QUAD_BCAST2>(xv);
    } else if (a.lanes_per_row_log2 == 2) {
        delta = dpp_move_zero<DPP_QUAD_BCAST4>(delta);
        xv = dpp_move_zero<DPP_QUAD_BCAST4>(xv);
    } else if (a.lanes_per_row_log2 > 2) {
        const int lead = (int)(threadIdx.x & 63) & ~((1 << a.lanes_per_row_log2) - 1);
        delta = __shfl(delta, lead, 64);
        xv = __shfl(xv, lead, 64);
    }
    r.delta = delta;
    r.xv = xv;
    const float dx = r.delta * xv;
    float y = 0.0f;
    if constexpr (A_PER_STATE) {
#pragma unroll
        for (int i = 0; i < V; ++i) {
            const float dA = exp2_hw(r.delta * q.an[i]);
            r.hs[i] = fmaf(dA, r.hs[i], dx * r.bv[i]);
            y = fmaf(r.cv[i], r.hs[i], y);
        }
    } else {
        const float dA = exp2_hw(r.delta * q.a2);
#pragma unroll
        for (int i = 0; i < V; ++i) {
            r.hs[i] = fmaf(dA, r.hs[i], dx * r.bv[i]);
            y = fmaf(r.cv[i], r.hs[i], y);
        }
    }
    if (r.live) {
        if constexpr (VEC) {
            store_vec_cached<TS, V>(r.sp, r.hs);
        } else {
#pragma unroll
            for (int i = 0; i < V; ++i)
                if (q.n0 + i < a.dstate)
                    r.sp[i] = from_f32<TS>(r.hs[i]);
        }
    }
    return r.live ? y : 0.0f;
}

// Lanes: 2^lanes_per_row_log2 per (h,p) row, each owning V consecutive
// states (blockIdx.x covers the rows of one request); blockIdx.y picks RB
// consecutive requests, which every lane takes in turn with the same
// parameters.  All loads of the RB requests are issued before any
// arithmetic.  A wave covers 64*V consecutive states of one request's slot.
template <typename TS, typename TI, bool A_PER_STATE, bool VEC, int V, int CW, int RB>
__global__ __launch_bounds__(512) void ssu_kernel(SsuArgs a)
{
    const int lpr_log2 = a.lanes_per_row_log2;
    const int64_t gid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    const int64_t hp = gid >> lpr_log2;
    const int j = (int)(gid & ((1 << lpr_log2) - 1));  // lane within the row
    SsuParams<V, CW> q;
    ssu_params<A_PER_STATE, VEC, V, CW>(a, hp, j, q);
    SsuReq<TS, TI, V, CW> r[RB];
#pragma unroll
    for (int k = 0; k < RB; ++k)
        ssu_load<TS, TI, VEC, V, CW>(a, (int)blockIdx.y * RB + k, j, q, r[k]);
    if (j == 0) {
#pragma unroll
        for (int k = 0; k < RB; ++k)
            ssu_load_row<TS, TI, V, CW>(a, r[k]);
    }
#pragma unroll
    for (int k = 0; k < RB; ++k) {
        float y = ssu_compute<TS, TI, A_PER_STATE, VEC, V, CW>(a, j, q, r[k]);
        // sum over the row's lanes (butterfly; lanes of one row are contiguous)
        for (int o = (1 << lpr_log2) >> 1; o > 0; o >>= 1)
            y += __shfl_xor(y, o, 64);
        if (j == 0 && r[k].live) {
            if (a.D)
                y = fmaf(q.Dh, r[k].xv, y);
            if (a.z)
                y *= silu_f32(r[k].zv);
            static_cast<TI *>(a.out)[r[k].row] = from_f32<TI>(y);
        }
    }
}

template <typename TS, typename TI, bool APS, bool VEC, int V, int CW>
static void launch_ssu_rb(const SsuArgs &a, hipStream_t stream)
{
    const int64_t lanes = ((int64_t)a.nheads * a.headdim) << a.lanes_per_row_log2;
    const int rb = a.requests_per_lane;
    const dim3 grid((unsigned)((lanes + a.block_threads - 1) / a.block_threads), (unsigned)((a.batch + rb - 1) / rb));
    if (rb == 4)
        hipLaunchKernelGGL((ssu_kernel<TS, TI, APS, VEC, V, CW, 4>), grid, dim3(a.block_threads), 0, stream, a);
    else if (rb == 2)
        hipLaunchKernelGGL((ssu_kernel<TS, TI, APS, VEC, V, CW, 2>), grid, dim3(a.block_threads), 0, stream, a);
    else
        hipLaunchKernelGGL((ssu_kernel<TS, TI, APS, VEC, V, CW, 1>), grid, dim3(a.block_threads), 0, stream, a);
}

template <typename TS, typename TI, bool APS, bool VEC, int V>
static void launch_ssu_v(const SsuArgs &a, hipStream_t stream)
{
    if (a.conv_width == kFusedConvWidth)
        launch_ssu_rb<TS, TI, APS, VEC, V, kFusedConvWidth>(a, stream);
    else
        launch_ssu_rb<TS, TI, APS, VEC, V, 0>(a, stream);
}

template <typename TS, typename TI>
static hipError_t launch_ssu_t(const SsuArgs &a, hipStream_t stream)
{
    if (a.states_per_lane == 4) {
        // one 16-byte vector of a 4-byte cache per lane
        if constexpr (StorageSize<TS>::value == 4) {
            if (a.a_per_state) {
                if (a.vec) launch_ssu_v<TS, TI, true, true, 4>(a, stream);
                else launch_ssu_v<TS, TI, true, false, 4>(a, stream);
            } else {
                if (a.vec) launch_ssu_v<TS, TI, false, true, 4>(a, stream);
                else launch_ssu_v<TS, TI, false, false, 4>(a, stream);
            }
        } else {
            return hipErrorInvalidValue;
        }
    } else if (a.states_per_lane == 16) {
        if (a.a_per_state) {
            if (a.vec) launch_ssu_v<TS, TI, true, true, 16>(a, stream);
            else launch_ssu_v<TS, TI, true, false, 16>(a, stream);
        } else {
            if (a.vec) launch_ssu_v<TS, TI, false, true, 16>(a, stream);
            else launch_ssu_v<TS, TI, false, false, 16>(a, stream);
        }
    } else {
        if (a.a_per_state) {
            if (a.vec) launch_ssu_v<TS, TI, true, true, 8>(a, stream);
            else launch_ssu_v<TS, TI, true, false, 8>(a, stream);
        } else {
            if (a.vec) launch_ssu_v<TS, TI, false, true, 8>(a, stream);
            else launch_ssu_v<TS, TI, false, false, 8>(a, stream);
        }
    }
    return hipGetLastError();
}

template <typename TS>
static hipError_t launch_ssu_s(const SsuArgs &a, hipStream_t stream)
{
    switch (a.io_dtype) {
    case 0: return launch_ssu_t<TS, float>(a, stream);
    case 1: return launch_ssu_t<TS, f16>(a, stream);
    default: return launch_ssu_t<TS, bf16>(a, stream);
    }
}

hipError_t launch_ssu(const SsuArgs &a, hipStream_t stream)
{
    switch (a.state_dtype) {
    case 0: return launch_ssu_s<float>(a, stream);
    case 1: return launch_ssu_s<f16>(a, stream);
    default: return launch_ssu_s<bf16>(a, stream);
    }
}

} // namespace ssm
