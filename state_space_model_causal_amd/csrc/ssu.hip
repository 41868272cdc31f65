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
// write).  Each lane holds V states (V*sizeof(state) = 16, 32 or 64 bytes) of
// every request it takes, and a wave covers 64*V consecutive states of the
// cache, read and written with 128-bit accesses.  Two lane maps:
//  - blocked (ssu_kernel): a lane owns V consecutive states of one (b,h,p)
//    row, a row is dstate/V lanes (rounded up to a power of two dividing 64);
//  - interleaved (ssu_ilv_kernel, 32 bytes per lane, power-of-two rows of at
//    most 1 KB, large batches): the k-th access of a wave reads the k-th
//    contiguous kilobyte of its block, lane L the 16 bytes at 16L.  Every
//    access instruction then fills whole cache lines, where the blocked map
//    touches twice the lines per instruction, half of each.
// The readout sum over states is a butterfly across a row's lanes.  No LDS,
// no barriers.  V and the workgroup size (64 to 512 lanes) are chosen per
// shape on the host, from a table tuned on gfx950 or a heuristic, or given by
// the caller.
#include "scan_body.hpp"
#include "ssu_body.hpp"

namespace ssm {

// The interleaved map for a launch, if it applies: 32 bytes of state per lane
// (two kilobyte accesses per wave), aligned 128-bit vectors, dense (head,
// row) rows within a slot, rows of power-of-two size from 32 bytes to 1 KB,
// every wave's block inside one group, and at least kIlvMinRows (request,
// row) pairs.  Below that the launch
// is latency-bound and the blocked map, with half the rows per lane, was 4-5%
// faster (Mamba-2 shapes at batch 8-16).  Returns log2(lanes per row), or -1.
constexpr int64_t kIlvMinRows = int64_t(1) << 18;
template <typename TS>
static int ilv_lanes_log2(const SsuArgs &a)
{
    const int rowbytes = a.dstate * StorageSize<TS>::value;
    if (!a.vec || a.states_per_lane * StorageSize<TS>::value != 32 || (rowbytes & (rowbytes - 1)) != 0 ||
        rowbytes < 32 || rowbytes > 1024 || a.st_sp != a.dstate || a.st_sh != (int64_t)a.headdim * a.dstate)
        return -1;
    int lg = 0;
    while ((16 << lg) < rowbytes)
        ++lg;
    const int64_t rows_per_wave = 2 * (64 >> lg);
    if (((int64_t)a.heads_per_group * a.headdim) % rows_per_wave != 0 ||
        (int64_t)a.batch * a.nheads * a.headdim < kIlvMinRows)
        return -1;
    return lg;
}

template <typename TS, typename TI, bool APS, int CW, bool COOP>
static void launch_ssu_ilv_c(const SsuArgs &a, hipStream_t stream)
{
    constexpr int NCH = 2;
    const int64_t rows_per_wave = NCH * (64 >> a.lanes_per_row_log2);
    const int64_t lanes = ((int64_t)a.nheads * a.headdim + rows_per_wave - 1) / rows_per_wave * 64;
    const int rb = a.requests_per_lane;
    const dim3 grid((unsigned)((lanes + a.block_threads - 1) / a.block_threads), (unsigned)((a.batch + rb - 1) / rb));
    if (rb == 2)
        hipLaunchKernelGGL((ssu_ilv_kernel<TS, TI, APS, CW, 2, NCH, COOP>), grid, dim3(a.block_threads), 0, stream, a);
    else
        hipLaunchKernelGGL((ssu_ilv_kernel<TS, TI, APS, CW, 1, NCH, COOP>), grid, dim3(a.block_threads), 0, stream, a);
}

template <typename TS, typename TI, bool APS, int CW>
static void launch_ssu_ilv(const SsuArgs &a0, int lg, hipStream_t stream)
{
    SsuArgs a = a0;
    a.lanes_per_row_log2 = lg;
    if constexpr (CW == 4) {
        if (lg >= 2) {  // rows of at least 4 lanes share the conv
            launch_ssu_ilv_c<TS, TI, APS, CW, true>(a, stream);
            return;
        }
    }
    launch_ssu_ilv_c<TS, TI, APS, CW, false>(a, stream);
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
    if constexpr (VEC && V * StorageSize<TS>::value == 32) {
        const int lg = ilv_lanes_log2<TS>(a);
        if (lg >= 0) {
            if (a.conv_width == kFusedConvWidth)
                launch_ssu_ilv<TS, TI, APS, kFusedConvWidth>(a, lg, stream);
            else
                launch_ssu_ilv<TS, TI, APS, 0>(a, lg, stream);
            return;
        }
    }
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

static hipError_t launch_ssu_one(const SsuArgs &a, hipStream_t stream)
{
    switch (a.state_dtype) {
    case 0: return launch_ssu_s<float>(a, stream);
    case 1: return launch_ssu_s<f16>(a, stream);
    default: return launch_ssu_s<bf16>(a, stream);
    }
}

// ---- the mixed launch: a prefill scan and an independent decode step ----
//
// One grid runs both: its first `nscan` workgroups are the scan's (in the
// scan's own XCD-aware order), the rest are the decode step's interleaved
// map, 256 lanes (four waves) per workgroup, request group by request group.
// Workgroups are dispatched in index order, so the decode's start only once
// every scan workgroup has started.  The scan's 1280 workgroups of the
// Mamba-2.8B prefill (batch 4) fill its 768 resident slots (3 per CU) and
// then run a second round of 2 per CU; the decode's workgroups take the slot
// that round leaves free, and its HBM-bound work runs beside the scan's
// VALU-bound tiles instead of after them.  The two halves share no memory.

bool mixed_scan_ok(const ScanArgs &s)
{
    return (s.io_dtype == 1 || s.io_dtype == 2) && s.state_dtype == 0 && s.a_per_state && s.vec &&
           s.dstate <= NC;
}

bool mixed_decode_ok(const SsuArgs &d)
{
    return (d.io_dtype == 1 || d.io_dtype == 2) && d.state_dtype == 0 && d.a_per_state && d.vec &&
           d.conv_width == kFusedConvWidth && d.states_per_lane == 8 && d.requests_per_lane == 2 &&
           d.batch <= 65535 * 2 && ilv_lanes_log2<float>(d) >= 2;
}

template <typename TI, int WALK>
__global__ __launch_bounds__(256)
__attribute__((amdgpu_waves_per_eu(scan_waves_per_simd<TI, true, true, true>())))
void mixed_kernel(ScanArgs s, SsuArgs d, uint32_t nscan, uint32_t dx)
{
    if (blockIdx.x < nscan) {
        scan_body<TI, float, true, true, true, WALK>(s, blockIdx.x, nscan);
        return;
    }
    const uint32_t w = blockIdx.x - nscan;  // uniform: the request group and wave block
    ssu_ilv_body<float, TI, true, kFusedConvWidth, 2, 2, true>(
        d, ((int64_t)(w % dx) * 256 + threadIdx.x) >> 6, (int)(w / dx));
}

bool mixed_pair_ok(const ScanArgs &s, const SsuArgs &d)
{
    if (!mixed_scan_ok(s) || !mixed_decode_ok(d) || s.io_dtype != d.io_dtype)
        return false;
    const int cpg = s.heads_per_group * s.headdim;
    const int64_t nscan = (int64_t)s.batch * s.ngroups * ((cpg + CPB - 1) / CPB);
    const int64_t rows_per_wave = 2 * (64 >> ilv_lanes_log2<float>(d));
    const int64_t lanes = ((int64_t)d.nheads * d.headdim + rows_per_wave - 1) / rows_per_wave * 64;
    const int64_t ndec = (lanes + 255) / 256 * ((d.batch + 1) / 2);
    return nscan + ndec <= 0x7fffffff;
}

hipError_t launch_mixed(const ScanArgs &s, const SsuArgs &d0, hipStream_t stream)
{
    SsuArgs d = d0;
    d.lanes_per_row_log2 = ilv_lanes_log2<float>(d);
    const int64_t rows_per_wave = 2 * (64 >> d.lanes_per_row_log2);
    const int64_t lanes = ((int64_t)d.nheads * d.headdim + rows_per_wave - 1) / rows_per_wave * 64;
    const uint32_t dx = (uint32_t)((lanes + 255) / 256);
    const uint32_t dy = (uint32_t)((d.batch + 1) / 2);
    const int cpg = s.heads_per_group * s.headdim;
    const uint32_t nscan = (uint32_t)((int64_t)s.batch * s.ngroups * ((cpg + CPB - 1) / CPB));
    const dim3 grid(nscan + dx * dy);
    // the scan's walk as in its own launch: the ladder of shorter end tiles
    // for packed batches and rows of other lengths
    const bool ladder = s.cu_seqlens || s.seqlen % (R * KD) != 0;
    if (s.io_dtype == 1) {
        if (ladder)
            hipLaunchKernelGGL((mixed_kernel<f16, WALK_LADDER>), grid, dim3(256), 0, stream, s, d, nscan, dx);
        else
            hipLaunchKernelGGL((mixed_kernel<f16, WALK_DENSE>), grid, dim3(256), 0, stream, s, d, nscan, dx);
    } else {
        if (ladder)
            hipLaunchKernelGGL((mixed_kernel<bf16, WALK_LADDER>), grid, dim3(256), 0, stream, s, d, nscan, dx);
        else
            hipLaunchKernelGGL((mixed_kernel<bf16, WALK_DENSE>), grid, dim3(256), 0, stream, s, d, nscan, dx);
    }
    return hipGetLastError();
}

template <typename P>
static P *advance(P *p, int64_t elems, int elem_bytes)
{
    using C = typename std::conditional<std::is_const<P>::value, const char, char>::type;
    return p ? reinterpret_cast<P *>(reinterpret_cast<C *>(p) + elems * elem_bytes) : p;
}

// The request groups of a launch sit on the grid's y dimension (at most
// 65535 of them); a larger batch is launched in consecutive parts of that
// many groups, each with its request rows, and (without a slot table) its
// state and conv-cache rows, offset to its first request.
hipError_t launch_ssu(const SsuArgs &a, hipStream_t stream)
{
    const int64_t per = (int64_t)65535 * a.requests_per_lane;
    if (a.batch <= per)
        return launch_ssu_one(a, stream);
    const int io = a.io_dtype == 0 ? 4 : 2, sd = a.state_dtype == 0 ? 4 : 2;
    for (int64_t b0 = 0; b0 < a.batch; b0 += per) {
        SsuArgs c = a;
        c.batch = (int)std::min<int64_t>(per, a.batch - b0);
        c.nrows = (int64_t)c.batch * a.nheads * a.headdim;
        c.x = advance(a.x, b0 * a.x_sb, io);
        c.dt = advance(a.dt, b0 * a.dt_sb, io);
        c.B = advance(a.B, b0 * a.B_sb, io);
        c.C = advance(a.C, b0 * a.C_sb, io);
        c.z = advance(a.z, b0 * a.z_sb, io);
        c.out = advance(a.out, b0 * a.o_sb, io);
        c.u_out = advance(a.u_out, b0 * a.u_sb, io);
        if (a.slot_idx) {
            c.slot_idx = a.slot_idx + b0;
        } else {  // slot = request
            c.state = advance(a.state, b0 * a.st_ss, sd);
            c.conv_state = advance(a.conv_state, b0 * a.cs_ss, io);
        }
        const hipError_t e = launch_ssu_one(c, stream);
        if (e != hipSuccess)
            return e;
    }
    return hipSuccess;
}

} // namespace ssm
