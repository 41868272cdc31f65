// scan.hip -- chunked selective scan (prefill) on gfx950.
//
// Operation: the selective-scan operator of "feat(llama.cu): 适配 mamba 模型"
// (InfiniLM-Rust PR #48, section 2.1) with its silu(z) element-mul gate, and
// the final state stored to the request's cache slot (section 3.1):
//     delta_t = softplus(dt_t + dt_bias)
//     h_t[n]  = exp(delta_t A[n]) h_{t-1}[n] + delta_t B_t[n] u_t
//     out_t   = (sum_n C_t[n] h_t[n] + D u_t) * silu(z_t)
//
// Work decomposition
//   * Workgroup = 256 lanes = 16 channels x 16 lanes ("a row": one DPP row).
//     All 16 channels belong to one (request, group), so they share one B/C
//     stream, which is staged once per tile in LDS and read by all of them.
//   * The sequence is walked in tiles of 16 K timesteps; lane r of a channel
//     owns timesteps [K r, K r + K) of the tile (K = 16: 128-bit loads of u,
//     dt and z).  In packed batches, and in dense rows whose length is not
//     a multiple of 256, each sequence ends in shorter tiles (K = 8, then at
//     most one each of K = 4, 2 and 1, with 8-, 4- and 2-byte loads for
//     2-byte types), so that it pads its last tile by fewer than 16 steps.
//   * For each state n, every lane reduces its K steps to one affine map
//     h -> a*h + b (a = product of decays, b = local state from zero), the 16
//     maps of a row are combined by an inclusive Hillis-Steele scan with DPP
//     row shifts (4 steps), and each lane then re-runs its K steps from the
//     exact incoming state, accumulating C_t[n] h_t[n] into its outputs.  The
//     tile-end state of each channel (lane 15's scan result, rotated into lane
//     0) carries to the next tile in registers (through LDS when dstate > 16).
//   * Mamba-2 (one decay per head, a_per_state == 0): the decays and their
//     row scan are state-independent and are computed once per tile.
// All arithmetic is float32; the state never leaves the chip until the final
// write to the cache slot.
#include "scan_body.hpp"

namespace ssm {

template <typename TI, typename TS, bool A_PER_STATE, bool VEC, int WALK>
static void launch_scan_w(const ScanArgs &a, dim3 grid, hipStream_t stream)
{
    if (a.dstate <= NC)
        hipLaunchKernelGGL((scan_kernel<TI, TS, A_PER_STATE, VEC, true, WALK>), grid, dim3(256), 0, stream, a);
    else
        hipLaunchKernelGGL((scan_kernel<TI, TS, A_PER_STATE, VEC, false, WALK>), grid, dim3(256), 0, stream, a);
}

template <typename TI, typename TS, bool A_PER_STATE, bool VEC>
static void launch_scan_v(const ScanArgs &a, dim3 grid, hipStream_t stream)
{
    if (a.cu_seqlens || a.seqlen % (R * KD) != 0)
        launch_scan_w<TI, TS, A_PER_STATE, VEC, WALK_LADDER>(a, grid, stream);
    else
        launch_scan_w<TI, TS, A_PER_STATE, VEC, WALK_DENSE>(a, grid, stream);
}

template <typename TI, typename TS>
static hipError_t launch_scan_ts(const ScanArgs &a, hipStream_t stream)
{
    const int cpg = a.heads_per_group * a.headdim;
    const int64_t nblocks = (int64_t)a.batch * a.ngroups * ((cpg + CPB - 1) / CPB);
    const dim3 grid((unsigned)nblocks);
    if (a.a_per_state) {
        if (a.vec) launch_scan_v<TI, TS, true, true>(a, grid, stream);
        else launch_scan_v<TI, TS, true, false>(a, grid, stream);
    } else {
        if (a.vec) launch_scan_v<TI, TS, false, true>(a, grid, stream);
        else launch_scan_v<TI, TS, false, false>(a, grid, stream);
    }
    return hipGetLastError();
}

template <typename TI>
static hipError_t launch_scan_t(const ScanArgs &a, hipStream_t stream)
{
    switch (a.state_dtype) {
    case 0: return launch_scan_ts<TI, float>(a, stream);
    case 1: return launch_scan_ts<TI, f16>(a, stream);
    default: return launch_scan_ts<TI, bf16>(a, stream);
    }
}

hipError_t launch_scan(const ScanArgs &a, hipStream_t stream)
{
    switch (a.io_dtype) {
    case 0: return launch_scan_t<float>(a, stream);
    case 1: return launch_scan_t<f16>(a, stream);
    default: return launch_scan_t<bf16>(a, stream);
    }
}

} // namespace ssm
