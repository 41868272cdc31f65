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
//     owns timesteps [K r, K r + K) of the tile (K = 16 for dense batches,
//     8 for packed ones; one to four 128-bit loads of u, dt and z).
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
#include "ssm_device.hpp"
#include "ssm_kernels.hpp"

#include <type_traits>

namespace ssm {

namespace {
constexpr int R = 16;        // lanes per channel
constexpr int KD = 16;       // timesteps per lane per tile: dense batches
constexpr int KP = 8;        // packed batches (half the padding at each sequence's last tile)
constexpr int CPB = 256 / R; // channels per workgroup
constexpr int NC = 16;       // states per LDS chunk of B/C
} // namespace

// Columns of a row: the walk over a sequence covers columns [0, hi) of its
// rows, the sequence itself being columns [lo, hi) (lo > 0 only when a vector
// row starts the sequence in the middle of a 128-bit vector).

// Load columns [tl, tl+K) of one row, zeros outside [lo, hi).  Every load is
// issued unconditionally from a clamped, in-bounds address and the
// out-of-range values are replaced afterwards, so all loads of a lane are in
// flight together instead of each waiting behind its own branch.
template <typename TI, bool VEC, int K>
__device__ __forceinline__ void load_steps(const TI *__restrict__ row, int tl, int lo, int hi, float (&dst)[K])
{
    constexpr int E = 16 / StorageSize<TI>::value;
    if constexpr (VEC) {
        // a vector that starts before hi ends inside the row (rows are a
        // multiple of 8 long and 16-byte aligned), and column 0 is a valid vector
#pragma unroll
        for (int v = 0; v < K / E; ++v) {
            const int off = tl + v * E;
            float part[E];
            load_vec_cached<TI, E>(row + (off < hi ? off : 0), part);
#pragma unroll
            for (int e = 0; e < E; ++e)
                dst[v * E + e] = (off + e >= lo && off + e < hi) ? part[e] : 0.0f;
        }
    } else {
#pragma unroll
        for (int i = 0; i < K; ++i) {
            const bool ok = tl + i >= lo && tl + i < hi;
            const float x = to_f32(row[ok ? tl + i : lo]);
            dst[i] = ok ? x : 0.0f;
        }
    }
}

// Raw 128-bit loads of timesteps [tl, tl+K) of one row (VEC rows only),
// issued back to back; widen() converts them once they are needed.
template <typename TI, int K>
struct RawSteps {
    static constexpr int E = 16 / StorageSize<TI>::value;
    static constexpr int NV = K / E;
    u32x4 w[NV];
    bool ok[NV];
};

template <typename TI, int K>
__device__ __forceinline__ void load_raw(RawSteps<TI, K> &r, const TI *__restrict__ row, int tl, int hi)
{
#pragma unroll
    for (int v = 0; v < RawSteps<TI, K>::NV; ++v) {
        const int off = tl + v * RawSteps<TI, K>::E;
        r.ok[v] = off < hi;
        r.w[v] = *reinterpret_cast<const u32x4 *>(row + (r.ok[v] ? off : 0));
    }
}

// Values outside the sequence are not masked here: they came from clamped
// in-bounds addresses, and the caller zeroes the step size and the input of
// those columns, which makes them identity steps (decay 1, input 0) whose
// outputs are never stored.
template <typename TI, int K>
__device__ __forceinline__ void widen(const RawSteps<TI, K> &r, float (&dst)[K])
{
    constexpr int E = RawSteps<TI, K>::E, PW = PerWord<TI>::value;
#pragma unroll
    for (int v = 0; v < RawSteps<TI, K>::NV; ++v) {
        float part[E];
        unpack_word(r.w[v].x, &part[0 * PW], TI{});
        unpack_word(r.w[v].y, &part[1 * PW], TI{});
        unpack_word(r.w[v].z, &part[2 * PW], TI{});
        unpack_word(r.w[v].w, &part[3 * PW], TI{});
#pragma unroll
        for (int e = 0; e < E; ++e)
            dst[v * E + e] = part[e];
    }
}

// Store columns [tl, tl+K) that lie in [lo, hi): whole vectors where the
// sequence covers them, single elements at its two ends (the neighbouring
// columns belong to other sequences).
template <typename TI, bool VEC, int K>
__device__ __forceinline__ void store_steps(TI *__restrict__ row, int tl, int lo, int hi, const float (&src)[K])
{
    constexpr int E = 16 / StorageSize<TI>::value;
    if constexpr (VEC) {
#pragma unroll
        for (int v = 0; v < K / E; ++v) {
            const int off = tl + v * E;
            if (off >= lo && off + E <= hi) {
                float part[E];
#pragma unroll
                for (int e = 0; e < E; ++e)
                    part[e] = src[v * E + e];
                store_vec_cached<TI, E>(row + off, part);
            } else if (off + E > lo && off < hi) {
#pragma unroll
                for (int e = 0; e < E; ++e)
                    if (off + e >= lo && off + e < hi)
                        row[off + e] = from_f32<TI>(src[v * E + e]);
            }
        }
    } else {
#pragma unroll
        for (int i = 0; i < K; ++i)
            if (tl + i >= lo && tl + i < hi)
                row[tl + i] = from_f32<TI>(src[i]);
    }
}

// Register budget: with 16 steps per lane the float16 vector paths (except
// per-state decays over several state chunks) fit three waves per SIMD (at
// most 168 VGPRs) without spilling, and the other variants are allowed two;
// 8 steps per lane take about half the registers of the per-step arrays.
template <typename TI, bool VEC, bool A_PER_STATE, bool ONE_CHUNK, int K>
constexpr int scan_waves_per_simd()
{
    return (std::is_same<TI, f16>::value && VEC && (ONE_CHUNK || !A_PER_STATE)) ? (K == KP ? 5 : 3)
                                                                                    : (K == KP ? 3 : 2);
}

// Packed batches of at most 256 sequences: the sequence of rank r when the
// sequences are sorted by length, longest first (ties by index).  Every
// workgroup derives the same order from the table, so the ranks form a
// permutation whatever the table holds.  Call from every lane.
__device__ __forceinline__ int packed_seq_of_rank(const int32_t *__restrict__ cu, int nseq, int L, int r)
{
    __shared__ int s_len[256];
    __shared__ int s_pick;
    const int tid = threadIdx.x;
    int len = 0;
    if (tid < nseq) {
        const int lo = min(max(cu[tid], 0), L);
        len = min(max(cu[tid + 1], lo), L) - lo;
        s_len[tid] = len;
    }
    __syncthreads();
    if (tid < nseq) {
        int rank = 0;
        for (int j = 0; j < nseq; ++j) {
            const int lj = s_len[j];
            rank += (lj > len || (lj == len && j < tid)) ? 1 : 0;
        }
        if (rank == r)
            s_pick = tid;
    }
    __syncthreads();
    return s_pick;
}

template <typename TI, typename TS, bool A_PER_STATE, bool VEC, bool ONE_CHUNK, int K>
__global__ __launch_bounds__(256)
__attribute__((amdgpu_waves_per_eu(scan_waves_per_simd<TI, VEC, A_PER_STATE, ONE_CHUNK, K>())))
void scan_kernel(ScanArgs a)
{
    constexpr int T = R * K;  // timesteps per tile
    constexpr int E = 16 / StorageSize<TI>::value;
    // B/C chunk in a lane-interleaved layout: the float4 holding timesteps
    // [16r + 4q, 16r + 4q + 4) of local state nl sits at (nl*(K/4) + q)*R + r,
    // so the 16 lanes of a row read 16 consecutive float4s (no bank conflict).
    __shared__ float4 lds_b[NC * T / 4];
    __shared__ float4 lds_c[NC * T / 4];
    // per channel and state: the state entering the current tile (the carry)
    // and A*log2(e); lane 0 of the row reads and rewrites the carry once per
    // tile, all 16 lanes read A*log2(e) (an LDS broadcast)
    constexpr int NCAP = ONE_CHUNK ? NC : kMaxScanDstate;
    __shared__ float lds_carry[CPB][NCAP];
    __shared__ float lds_a2[A_PER_STATE ? CPB : 1][A_PER_STATE ? NCAP : 1];

    const int L = a.seqlen, N = a.dstate, P = a.headdim;  // L: row length
    const int cpg = a.heads_per_group * P;  // channels per group (contiguous)
    const int nblk_g = (cpg + CPB - 1) / CPB;
    // Dense batches: consecutive blocks (one request's channels, sharing its
    // B/C) stay on one XCD.  Packed batches keep the hardware order, which
    // spreads every sequence over all XCDs: there the longest sequence is the
    // critical path and must not be confined to an eighth of the chip.
    const uint32_t lb = a.cu_seqlens ? blockIdx.x : xcd_block_order(blockIdx.x, gridDim.x);
    const int cb = (int)(lb % nblk_g);
    const int bg = (int)(lb / nblk_g);
    const int g = bg % a.ngroups;
    int b = bg / a.ngroups;
    if constexpr (K == KP) {
        // packed batches (the only ones with 8 steps per lane): the longest
        // sequences' workgroups start first, so the longest walks do not
        // begin late and leave the chip idle at the end
        if (a.batch <= 256)
            b = packed_seq_of_rank(a.cu_seqlens, a.batch, L, b);
    }
    const SeqSpan sp = seq_span(a.cu_seqlens, a.has_init_seq, b, L, a.has_initial_state);
    const int slot = a.slot_idx ? a.slot_idx[b] : b;
    if (slot < 0 || sp.len == 0)
        return;  // padded or empty sequence (uniform over the workgroup)
    // the walk starts at the 128-bit vector holding the sequence's first step
    // (every row of the sequence starts at the same offset within a vector)
    const int lo = VEC ? sp.begin % E : 0, hi = lo + sp.len;
    const int64_t col0 = sp.begin - lo;

    const int tid = threadIdx.x, ch = tid / R, r = tid % R;
    const int cig = cb * CPB + ch;
    const bool active = cig < cpg;
    const int c = g * cpg + (active ? cig : 0);  // inactive lanes shadow a valid channel
    const int h = c / P, p = c % P;
    const int Cn = a.nheads * P;

    const int64_t blk = sp.block;
    const TI *urow = static_cast<const TI *>(a.u) + (blk * Cn + c) * L + col0;
    const TI *dtrow = static_cast<const TI *>(a.dt) + (blk * a.nheads + h) * L + col0;
    const TI *zrow = a.z ? static_cast<const TI *>(a.z) + (blk * Cn + c) * L + col0 : nullptr;
    TI *orow = static_cast<TI *>(a.out) + (blk * Cn + c) * L + col0;
    const TI *Bg = static_cast<const TI *>(a.B) + (blk * a.ngroups + g) * N * L + col0;
    const TI *Cg = static_cast<const TI *>(a.C) + (blk * a.ngroups + g) * N * L + col0;
    TS *srow = a.state ? static_cast<TS *>(a.state) + (((int64_t)slot * a.nheads + h) * P + p) * N : nullptr;
    const bool load_init = srow && sp.init;

    const float bias_h = a.dt_bias ? a.dt_bias[h] : 0.0f;
    const float D_h = a.D ? a.D[h] : 0.0f;
    const float A2_h = A_PER_STATE ? 0.0f : a.A[h] * kLog2e;

    for (int n = r; n < N; n += R) {
        lds_carry[ch][n] = load_init ? to_f32(srow[n]) : 0.0f;
        if constexpr (A_PER_STATE)
            lds_a2[ch][n] = a.A[(int64_t)h * N + n] * kLog2e;
    }

    for (int t0 = 0; t0 < hi; t0 += T) {
        const int tl = t0 + r * K;
        float dl[K], du[K], y[K];
        RawSteps<TI, K> rz;  // the gate's loads are issued with the others
        {
            float uu[K], dd[K];
            if constexpr (VEC) {
                RawSteps<TI, K> ru, rd;
                load_raw(ru, urow, tl, hi);
                load_raw(rd, dtrow, tl, hi);
                // 2-byte gates are fetched early (8 VGPRs); 4-byte ones at the end
                if (zrow && StorageSize<TI>::value == 2)
                    load_raw(rz, zrow, tl, hi);
                widen(ru, uu);
                widen(rd, dd);
            } else {
                load_steps<TI, VEC, K>(urow, tl, lo, hi, uu);
                load_steps<TI, VEC, K>(dtrow, tl, lo, hi, dd);
            }
#pragma unroll
            for (int i = 0; i < K; ++i) {
                const float v = dd[i] + bias_h;
                const float spv = softplus_f32(v);
                const bool in = tl + i >= lo && tl + i < hi;
                // identity step outside the sequence (decay 1, input 0)
                const float d = in ? (a.dt_softplus ? spv : v) : 0.0f;
                const float uv = in ? uu[i] : 0.0f;
                dl[i] = d;
                du[i] = d * uv;
                y[i] = D_h * uv;
            }
        }
        float sdl = 0.0f;
#pragma unroll
        for (int i = 0; i < K; ++i)
            sdl += dl[i];

        // Mamba-2: decays and their row scan do not depend on the state.
        float am[A_PER_STATE ? 1 : K];
        float acum[A_PER_STATE ? 1 : 4];
        if constexpr (!A_PER_STATE) {
#pragma unroll
            for (int i = 0; i < K; ++i)
                am[i] = exp2_hw(dl[i] * A2_h);
            float ag = exp2_hw(sdl * A2_h);
            acum[0] = ag;
            ag *= dpp_move_zero<DPP_ROW_SHR1>(ag);
            acum[1] = ag;
            ag *= dpp_move_zero<DPP_ROW_SHR2>(ag);
            acum[2] = ag;
            ag *= dpp_move_zero<DPP_ROW_SHR4>(ag);
            acum[3] = ag;
        }

        for (int n0 = 0; n0 < N; n0 += NC) {
            __syncthreads();  // previous chunk's readers are done with the LDS tiles
            for (int m = tid; m < NC * T / E; m += 256) {
                const int nl = m / (T / E), tc = (m % (T / E)) * E;
                const int n = n0 + nl, t = t0 + tc;
                float vb[E], vc[E];
                if constexpr (VEC) {
                    // clamped address, unconditional load, then select
                    const bool ok = n < N && t < hi;
                    const int64_t off = ok ? (int64_t)n * L + t : 0;
                    load_vec_cached<TI, E>(Bg + off, vb);
                    load_vec_cached<TI, E>(Cg + off, vc);
#pragma unroll
                    for (int e = 0; e < E; ++e) {
                        const bool in = ok && t + e >= lo && t + e < hi;
                        vb[e] = in ? vb[e] : 0.0f;
                        vc[e] = in ? vc[e] : 0.0f;
                    }
                } else {
#pragma unroll
                    for (int e = 0; e < E; ++e) {
                        const bool ok = n < N && t + e >= lo && t + e < hi;
                        const int64_t off = ok ? (int64_t)n * L + t + e : lo;
                        const float xb = to_f32(Bg[off]), xc = to_f32(Cg[off]);
                        vb[e] = ok ? xb : 0.0f;
                        vc[e] = ok ? xc : 0.0f;
                    }
                }
#pragma unroll
                for (int e4 = 0; e4 < E / 4; ++e4) {
                    const int tt = tc + 4 * e4;
                    const int idx = (nl * (K / 4) + (tt % K) / 4) * R + tt / K;
                    lds_b[idx] = make_float4(vb[4 * e4], vb[4 * e4 + 1], vb[4 * e4 + 2], vb[4 * e4 + 3]);
                    lds_c[idx] = make_float4(vc[4 * e4], vc[4 * e4 + 1], vc[4 * e4 + 2], vc[4 * e4 + 3]);
                }
            }
            __syncthreads();
#pragma unroll 1
            for (int nl = 0; nl < NC; ++nl) {
                if (n0 + nl >= N)
                    break;
                const int n = n0 + nl;
                float Bv[K], Cv[K];
#pragma unroll
                for (int q = 0; q < K / 4; ++q) {
                    const float4 vb = lds_b[(nl * (K / 4) + q) * R + r];
                    const float4 vc = lds_c[(nl * (K / 4) + q) * R + r];
                    Bv[4 * q] = vb.x; Bv[4 * q + 1] = vb.y; Bv[4 * q + 2] = vb.z; Bv[4 * q + 3] = vb.w;
                    Cv[4 * q] = vc.x; Cv[4 * q + 1] = vc.y; Cv[4 * q + 2] = vc.z; Cv[4 * q + 3] = vc.w;
                }
                const float cin = lds_carry[ch][n];
                const float carry = (r == 0) ? cin : 0.0f;
                float av[K], bx[K];
                float aagg, bagg;
                if constexpr (A_PER_STATE) {
                    const float A2 = lds_a2[ch][n];
#pragma unroll
                    for (int i = 0; i < K; ++i)
                        av[i] = exp2_hw(dl[i] * A2);
                    aagg = exp2_hw(sdl * A2);
                } else {
#pragma unroll
                    for (int i = 0; i < K; ++i)
                        av[i] = am[i];
                    aagg = acum[0];
                }
#pragma unroll
                for (int i = 0; i < K; ++i) {
                    bx[i] = du[i] * Bv[i];
                    bagg = (i == 0) ? bx[0] : fmaf(av[i], bagg, bx[i]);
                }
                bagg = fmaf(aagg, carry, bagg);  // lane 0 starts from the incoming state
                // inclusive scan of the affine maps over the 16 lanes of the row.
                // Lanes whose source lies before lane 0 read 0: the b term then
                // adds nothing, and the decay products they corrupt belong to
                // segments that start at lane 0, which no later step multiplies
                // into a valid combine (nothing precedes lane 0).
                if constexpr (A_PER_STATE) {
                    bagg = fmaf(aagg, dpp_move_zero<DPP_ROW_SHR1>(bagg), bagg);
                    aagg *= dpp_move_zero<DPP_ROW_SHR1>(aagg);
                    bagg = fmaf(aagg, dpp_move_zero<DPP_ROW_SHR2>(bagg), bagg);
                    aagg *= dpp_move_zero<DPP_ROW_SHR2>(aagg);
                    bagg = fmaf(aagg, dpp_move_zero<DPP_ROW_SHR4>(bagg), bagg);
                    aagg *= dpp_move_zero<DPP_ROW_SHR4>(aagg);
                    bagg = fmaf(aagg, dpp_move_zero<DPP_ROW_SHR8>(bagg), bagg);
                } else {
                    bagg = fmaf(acum[0], dpp_move_zero<DPP_ROW_SHR1>(bagg), bagg);
                    bagg = fmaf(acum[1], dpp_move_zero<DPP_ROW_SHR2>(bagg), bagg);
                    bagg = fmaf(acum[2], dpp_move_zero<DPP_ROW_SHR4>(bagg), bagg);
                    bagg = fmaf(acum[3], dpp_move_zero<DPP_ROW_SHR8>(bagg), bagg);
                }
                // lane r >= 1 starts from lane r-1's end state; lane 0 from the
                // carry, and receives lane 15's end state as the next carry
                const float rot = dpp_move_zero<DPP_ROW_ROR1>(bagg);
                float hh = (r == 0) ? carry : rot;
                if (r == 0)
                    lds_carry[ch][n] = rot;
#pragma unroll
                for (int i = 0; i < K; ++i) {
                    hh = fmaf(av[i], hh, bx[i]);
                    y[i] = fmaf(Cv[i], hh, y[i]);
                }
            }
        }
        if (zrow) {
            float zz[K];
            if constexpr (VEC && StorageSize<TI>::value == 2)
                widen(rz, zz);
            else
                load_steps<TI, VEC, K>(zrow, tl, lo, hi, zz);
#pragma unroll
            for (int i = 0; i < K; ++i)
                y[i] *= silu_f32(zz[i]);
        }
        if (active)
            store_steps<TI, VEC, K>(orow, tl, lo, hi, y);
    }
    __syncthreads();
    if (srow && active)
        for (int n = r; n < N; n += R)
            srow[n] = from_f32<TS>(lds_carry[ch][n]);
}

template <typename TI, typename TS, bool A_PER_STATE, bool VEC>
static void launch_scan_v(const ScanArgs &a, dim3 grid, hipStream_t stream)
{
    // Packed batches take 8 steps per lane: each sequence pads its last tile
    // to a tile boundary, and halving the tile halves that waste (packed
    // 16-sequence Mamba-1 prefill 281 -> 261 us).  Dense batches keep 16,
    // whose lane scan costs less per step (227 vs 238 us).
    if (a.cu_seqlens) {
        if (a.dstate <= NC)
            hipLaunchKernelGGL((scan_kernel<TI, TS, A_PER_STATE, VEC, true, KP>), grid, dim3(256), 0, stream, a);
        else
            hipLaunchKernelGGL((scan_kernel<TI, TS, A_PER_STATE, VEC, false, KP>), grid, dim3(256), 0, stream, a);
    } else {
        if (a.dstate <= NC)
            hipLaunchKernelGGL((scan_kernel<TI, TS, A_PER_STATE, VEC, true, KD>), grid, dim3(256), 0, stream, a);
        else
            hipLaunchKernelGGL((scan_kernel<TI, TS, A_PER_STATE, VEC, false, KD>), grid, dim3(256), 0, stream, a);
    }
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
