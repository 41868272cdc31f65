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

// Everything one lane holds for one (b,h,p) row between issuing its loads and
// storing its results.
template <typename TS, typename TI, int V, int CW>
struct SsuRow {
    float hs[V], bv[V], cv[V], an[V];
    float win[CW > 1 ? CW - 1 : 1];
    float tap[CW > 0 ? CW : 1];
    float cbias;
    float delta, xv;
    TS *sp;
    TI *cw;
    int64_t row, bh;
    int h;
    bool live;
};

// Phase 1: resolve the row's slot and issue all of its loads.
template <typename TS, typename TI, bool A_PER_STATE, bool VEC, int V, bool WAVE_REQ, int CW>
__device__ __forceinline__ void ssu_load(const SsuArgs &a, int64_t row, int j, SsuRow<TS, TI, V, CW> &r)
{
    const bool in = row < a.nrows;
    const int64_t rr = in ? row : 0;
    const int p = (int)(rr % a.headdim);
    const int64_t bh = rr / a.headdim;
    const int h = (int)(bh % a.nheads);
    int b = (int)(bh / a.nheads);
    if constexpr (WAVE_REQ)
        b = __builtin_amdgcn_readfirstlane(b);  // one request per wave: scalar slot load
    const int slot = a.slot_idx ? a.slot_idx[b] : b;
    const int n0 = j * V;
    r.live = in && slot >= 0 && n0 < a.dstate;  // padded: loads from slot 0, discarded
    r.row = rr;
    r.bh = bh;
    r.h = h;
    const int s = slot >= 0 ? slot : 0;
    const int nc = n0 < a.dstate ? n0 : 0;
    const int g = h / a.heads_per_group;
    r.sp = static_cast<TS *>(a.state) + ((((int64_t)s * a.nheads + h) * a.headdim + p) * a.dstate + nc);
    const int64_t bc_off = ((int64_t)b * a.ngroups + g) * a.dstate + nc;
    const TI *Bp = static_cast<const TI *>(a.B) + bc_off;
    const TI *Cp = static_cast<const TI *>(a.C) + bc_off;
    const float *Ap = a.A + (int64_t)h * a.dstate + nc;
    if constexpr (VEC) {
        load_vec_cached<TS, V>(r.sp, r.hs);
        load_vec_cached<TI, V>(Bp, r.bv);
        load_vec_cached<TI, V>(Cp, r.cv);
        if constexpr (A_PER_STATE)
            load_vec_cached<float, V>(Ap, r.an);
    } else {
#pragma unroll
        for (int i = 0; i < V; ++i) {
            const bool ok = nc + i < a.dstate;
            const int ii = ok ? i : 0;
            const float hv = to_f32(r.sp[ii]), bvv = to_f32(Bp[ii]), cvv = to_f32(Cp[ii]);
            r.hs[i] = ok ? hv : 0.0f;
            r.bv[i] = ok ? bvv : 0.0f;
            r.cv[i] = ok ? cvv : 0.0f;
            if constexpr (A_PER_STATE) {
                const float av = Ap[ii];
                r.an[i] = ok ? av : 0.0f;
            }
        }
    }
    const float v = to_f32(static_cast<const TI *>(a.dt)[bh]) + (a.dt_bias ? a.dt_bias[h] : 0.0f);
    r.delta = a.dt_softplus ? softplus_f32(v) : v;
    r.xv = to_f32(static_cast<const TI *>(a.x)[rr]);
    if constexpr (CW > 0) {
        constexpr int HW = CW - 1;
        const int64_t c = (int64_t)h * a.headdim + p;
        r.cw = static_cast<TI *>(a.conv_state) + ((int64_t)s * a.nheads * a.headdim + c) * HW;
#pragma unroll
        for (int k = 0; k < HW; ++k)
            r.win[k] = to_f32(r.cw[k]);
#pragma unroll
        for (int k = 0; k < CW; ++k)
            r.tap[k] = a.conv_weight[c * CW + k];
        r.cbias = a.conv_bias ? a.conv_bias[c] : 0.0f;
    }
}

// Phase 2: (fused conv), state update, store, partial readout.
template <typename TS, typename TI, bool A_PER_STATE, bool VEC, int V, int CW>
__device__ __forceinline__ float ssu_compute(const SsuArgs &a, int j, SsuRow<TS, TI, V, CW> &r)
{
    float xv = r.xv;
    if constexpr (CW > 0) {
        // fused conv update of channel c: every lane of the row computes the
        // (cheap) conv; lane 0 shifts the cached window, whose stored values
        // depend on the window loads, so every lane's read has returned first
        constexpr int HW = CW - 1;
        float acc = r.cbias;
#pragma unroll
        for (int k = 0; k < HW; ++k)
            acc = fmaf(r.tap[k], r.win[k], acc);
        acc = fmaf(r.tap[HW], xv, acc);
        const float u = silu_f32(acc);
        if (r.live && j == 0) {
#pragma unroll
            for (int k = 0; k + 1 < HW; ++k)
                r.cw[k] = from_f32<TI>(r.win[k + 1]);
            if (HW > 0)
                r.cw[HW - 1] = static_cast<const TI *>(a.x)[r.row];
            if (a.u_out)
                static_cast<TI *>(a.u_out)[r.row] = from_f32<TI>(u);
        }
        xv = u;  // the update reads the float32 conv output
    }
    r.xv = xv;
    const float dx = r.delta * xv;
    float y = 0.0f;
    if constexpr (A_PER_STATE) {
#pragma unroll
        for (int i = 0; i < V; ++i) {
            const float dA = exp2_hw(r.delta * (r.an[i] * kLog2e));
            r.hs[i] = fmaf(dA, r.hs[i], dx * r.bv[i]);
            y = fmaf(r.cv[i], r.hs[i], y);
        }
    } else {
        const float dA = exp2_hw(r.delta * (a.A[r.h] * kLog2e));
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
                if (j * V + i < a.dstate)
                    r.sp[i] = from_f32<TS>(r.hs[i]);
        }
    }
    return r.live ? y : 0.0f;
}

// One (b,h,p) row per group of 2^lanes_per_row_log2 lanes, each lane owning V
// consecutive states; all of a lane's loads are issued before any arithmetic.
template <typename TS, typename TI, bool A_PER_STATE, bool VEC, int V, bool WAVE_REQ, int CW>
__global__ __launch_bounds__(512) void ssu_kernel(SsuArgs a)
{
    const int lpr_log2 = a.lanes_per_row_log2;
    const int64_t gtid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    const int64_t row = gtid >> lpr_log2;                // (b*H + h)*P + p
    const int j = (int)(gtid & ((1 << lpr_log2) - 1));   // lane within the row
    SsuRow<TS, TI, V, CW> r;
    ssu_load<TS, TI, A_PER_STATE, VEC, V, WAVE_REQ, CW>(a, row, j, r);
    float y = ssu_compute<TS, TI, A_PER_STATE, VEC, V, CW>(a, j, r);
    // sum over the row's lanes (butterfly; lanes of one row are contiguous)
    for (int o = (1 << lpr_log2) >> 1; o > 0; o >>= 1)
        y += __shfl_xor(y, o, 64);
    if (j == 0 && r.live) {
        if (a.D)
            y = fmaf(a.D[r.h], r.xv, y);
        if (a.z)
            y *= silu_f32(to_f32(static_cast<const TI *>(a.z)[row]));
        static_cast<TI *>(a.out)[row] = from_f32<TI>(y);
    }
}

template <typename TS, typename TI, bool APS, bool VEC, int V, bool WREQ>
static void launch_ssu_cw(const SsuArgs &a, dim3 grid, hipStream_t stream)
{
    if (a.conv_width == kFusedConvWidth)
        hipLaunchKernelGGL((ssu_kernel<TS, TI, APS, VEC, V, WREQ, kFusedConvWidth>), grid, dim3(a.block_threads), 0,
                           stream, a);
    else
        hipLaunchKernelGGL((ssu_kernel<TS, TI, APS, VEC, V, WREQ, 0>), grid, dim3(a.block_threads), 0, stream, a);
}

template <typename TS, typename TI, bool APS, bool VEC, int V>
static void launch_ssu_v(const SsuArgs &a, dim3 grid, hipStream_t stream)
{
    if (a.wave_per_request)
        launch_ssu_cw<TS, TI, APS, VEC, V, true>(a, grid, stream);
    else
        launch_ssu_cw<TS, TI, APS, VEC, V, false>(a, grid, stream);
}

template <typename TS, typename TI>
static hipError_t launch_ssu_t(const SsuArgs &a, hipStream_t stream)
{
    const int64_t threads = a.nrows << a.lanes_per_row_log2;
    const dim3 grid((unsigned)((threads + a.block_threads - 1) / a.block_threads));
    if (a.states_per_lane == 16) {
        if (a.a_per_state) {
            if (a.vec) launch_ssu_v<TS, TI, true, true, 16>(a, grid, stream);
            else launch_ssu_v<TS, TI, true, false, 16>(a, grid, stream);
        } else {
            if (a.vec) launch_ssu_v<TS, TI, false, true, 16>(a, grid, stream);
            else launch_ssu_v<TS, TI, false, false, 16>(a, grid, stream);
        }
    } else {
        if (a.a_per_state) {
            if (a.vec) launch_ssu_v<TS, TI, true, true, 8>(a, grid, stream);
            else launch_ssu_v<TS, TI, true, false, 8>(a, grid, stream);
        } else {
            if (a.vec) launch_ssu_v<TS, TI, false, true, 8>(a, grid, stream);
            else launch_ssu_v<TS, TI, false, false, 8>(a, grid, stream);
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
