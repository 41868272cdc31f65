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
// across the row's lanes.  No LDS, no barriers.
#include "ssm_device.hpp"
#include "ssm_kernels.hpp"

namespace ssm {

template <typename TS, typename TI, bool A_PER_STATE, bool VEC, int V, bool WAVE_REQ, int CW>
__global__ __launch_bounds__(256) void ssu_kernel(SsuArgs a)
{
    const int lpr_log2 = a.lanes_per_row_log2;
    const int64_t gtid = (int64_t)blockIdx.x * 256 + threadIdx.x;
    const int64_t row = gtid >> lpr_log2;               // (b*H + h)*P + p
    const int j = (int)(gtid & ((1 << lpr_log2) - 1));  // lane within the row
    if (row >= a.nrows)
        return;  // whole rows leave together: lanes_per_row divides 64
    const int p = (int)(row % a.headdim);
    const int64_t bh = row / a.headdim;
    const int h = (int)(bh % a.nheads);
    int b = (int)(bh / a.nheads);
    if constexpr (WAVE_REQ)
        b = __builtin_amdgcn_readfirstlane(b);  // one request per wave: scalar slot load
    const int slot = a.slot_idx ? a.slot_idx[b] : b;
    if (slot < 0)
        return;  // padded request: nothing read or written
    const int g = h / a.heads_per_group;
    const int n0 = j * V;

    const TI *dtp = static_cast<const TI *>(a.dt);
    const TI *xp = static_cast<const TI *>(a.x);
    float v = to_f32(dtp[bh]) + (a.dt_bias ? a.dt_bias[h] : 0.0f);
    const float delta = a.dt_softplus ? softplus_f32(v) : v;
    float xv = to_f32(xp[row]);
    if constexpr (CW > 0) {
        // fused conv update of channel c: every lane of the row computes the
        // (cheap) conv; lane 0 shifts the cached window after its own loads
        // of the old window have returned (the stored values depend on them)
        constexpr int HW = CW - 1;
        const int64_t c = (int64_t)h * a.headdim + p;
        TI *cw = static_cast<TI *>(a.conv_state) + ((int64_t)slot * a.nheads * a.headdim + c) * HW;
        float acc = a.conv_bias ? a.conv_bias[c] : 0.0f;
        float win[HW > 0 ? HW : 1];
#pragma unroll
        for (int k = 0; k < HW; ++k) {
            win[k] = to_f32(cw[k]);
            acc = fmaf(a.conv_weight[c * CW + k], win[k], acc);
        }
        acc = fmaf(a.conv_weight[c * CW + HW], xv, acc);
        const float u = silu_f32(acc);
        if (j == 0) {
#pragma unroll
            for (int k = 0; k + 1 < HW; ++k)
                cw[k] = from_f32<TI>(win[k + 1]);
            if (HW > 0)
                cw[HW - 1] = xp[row];
            if (a.u_out)
                static_cast<TI *>(a.u_out)[row] = from_f32<TI>(u);
        }
        xv = u;  // the update reads the float32 conv output
    }
    const float dx = delta * xv;

    float y = 0.0f;
    if (n0 < a.dstate) {
        TS *sp = static_cast<TS *>(a.state) + ((((int64_t)slot * a.nheads + h) * a.headdim + p) * a.dstate + n0);
        const int64_t bc_off = ((int64_t)b * a.ngroups + g) * a.dstate + n0;
        const TI *Bp = static_cast<const TI *>(a.B) + bc_off;
        const TI *Cp = static_cast<const TI *>(a.C) + bc_off;
        float hs[V], bv[V], cv[V];
        if constexpr (VEC) {
            load_vec_cached<TS, V>(sp, hs);
            load_vec_cached<TI, V>(Bp, bv);
            load_vec_cached<TI, V>(Cp, cv);
        } else {
#pragma unroll
            for (int i = 0; i < V; ++i) {
                const bool ok = n0 + i < a.dstate;
                hs[i] = ok ? to_f32(sp[i]) : 0.0f;
                bv[i] = ok ? to_f32(Bp[i]) : 0.0f;
                cv[i] = ok ? to_f32(Cp[i]) : 0.0f;
            }
        }
        if constexpr (A_PER_STATE) {
            float an[V];
            const float *Ap = a.A + (int64_t)h * a.dstate + n0;
            if constexpr (VEC) {
                load_vec_cached<float, V>(Ap, an);
            } else {
#pragma unroll
                for (int i = 0; i < V; ++i)
                    an[i] = (n0 + i < a.dstate) ? Ap[i] : 0.0f;
            }
#pragma unroll
            for (int i = 0; i < V; ++i) {
                const float dA = exp2_hw(delta * (an[i] * kLog2e));
                hs[i] = fmaf(dA, hs[i], dx * bv[i]);
                y = fmaf(cv[i], hs[i], y);
            }
        } else {
            const float dA = exp2_hw(delta * (a.A[h] * kLog2e));
#pragma unroll
            for (int i = 0; i < V; ++i) {
                hs[i] = fmaf(dA, hs[i], dx * bv[i]);
                y = fmaf(cv[i], hs[i], y);
            }
        }
        if constexpr (VEC) {
            store_vec_cached<TS, V>(sp, hs);
        } else {
#pragma unroll
            for (int i = 0; i < V; ++i)
                if (n0 + i < a.dstate)
                    sp[i] = from_f32<TS>(hs[i]);
        }
    }
    // sum over the row's lanes (butterfly; lanes of one row are contiguous)
    for (int o = (1 << lpr_log2) >> 1; o > 0; o >>= 1)
        y += __shfl_xor(y, o, 64);
    if (j == 0) {
        if (a.D)
            y = fmaf(a.D[h], xv, y);
        if (a.z)
            y *= silu_f32(to_f32(static_cast<const TI *>(a.z)[row]));
        static_cast<TI *>(a.out)[row] = from_f32<TI>(y);
    }
}

template <typename TS, typename TI>
static hipError_t launch_ssu_t(const SsuArgs &a, hipStream_t stream)
{
    const int64_t threads = a.nrows << a.lanes_per_row_log2;
    const dim3 grid((unsigned)((threads + 255) / 256));
#define SSU_LAUNCH_CW(APS, VEC, V, CW)                                                             \
    do {                                                                                           \
        if (a.wave_per_request)                                                                    \
            hipLaunchKernelGGL((ssu_kernel<TS, TI, APS, VEC, V, true, CW>), grid, dim3(256), 0, stream, a);  \
        else                                                                                       \
            hipLaunchKernelGGL((ssu_kernel<TS, TI, APS, VEC, V, false, CW>), grid, dim3(256), 0, stream, a); \
    } while (0)
#define SSU_LAUNCH(APS, VEC, V)                                                                    \
    do {                                                                                           \
        if (a.conv_width == kFusedConvWidth)                                                       \
            SSU_LAUNCH_CW(APS, VEC, V, kFusedConvWidth);                                           \
        else                                                                                       \
            SSU_LAUNCH_CW(APS, VEC, V, 0);                                                         \
    } while (0)
    if (a.states_per_lane == 16) {
        if (a.a_per_state) {
            if (a.vec) SSU_LAUNCH(true, true, 16); else SSU_LAUNCH(true, false, 16);
        } else {
            if (a.vec) SSU_LAUNCH(false, true, 16); else SSU_LAUNCH(false, false, 16);
        }
    } else {
        if (a.a_per_state) {
            if (a.vec) SSU_LAUNCH(true, true, 8); else SSU_LAUNCH(true, false, 8);
        } else {
            if (a.vec) SSU_LAUNCH(false, true, 8); else SSU_LAUNCH(false, false, 8);
        }
    }
#undef SSU_LAUNCH
#undef SSU_LAUNCH_CW
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
