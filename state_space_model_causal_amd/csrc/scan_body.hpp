// scan_body.hpp -- device code of the chunked selective scan (the work
// decomposition is described in scan.hip), shared by its own kernel and
// by the mixed prefill + decode launch.
#pragma once
#include "ssm_device.hpp"
#include "ssm_kernels.hpp"

#include <type_traits>

namespace ssm {

namespace {
constexpr int R = 16;        // lanes per channel
constexpr int KD = 16;       // timesteps per lane per tile (the last tiles of a packed sequence: 8, 4)
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
    if constexpr (VEC && K >= E) {
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

// Raw vector loads of timesteps [tl, tl+K) of one row (VEC rows only),
// issued back to back; widen() converts them once they are needed.  A lane's
// K steps are 128-bit vectors, or one narrower vector (8, 4 or 2 bytes) when
// they take less than 16 bytes.
template <typename TI, int K>
struct RawSteps {
    static constexpr int VB = K * StorageSize<TI>::value >= 16 ? 16 : K * StorageSize<TI>::value;
    static constexpr int E = VB / StorageSize<TI>::value;  // elements per vector
    static constexpr int NV = K / E;
    u32x4 w[NV];  // a 64-bit vector in .x and .y
    bool ok[NV];
};

template <typename TI, int K>
__device__ __forceinline__ void load_raw(RawSteps<TI, K> &r, const TI *__restrict__ row, int tl, int hi)
{
#pragma unroll
    for (int v = 0; v < RawSteps<TI, K>::NV; ++v) {
        const int off = tl + v * RawSteps<TI, K>::E;
        r.ok[v] = off < hi;
        const TI *p = row + (r.ok[v] ? off : 0);
        if constexpr (RawSteps<TI, K>::VB == 16) {
            r.w[v] = *reinterpret_cast<const u32x4 *>(p);
        } else if constexpr (RawSteps<TI, K>::VB == 8) {
            const uint2 q = *reinterpret_cast<const uint2 *>(p);
            r.w[v] = u32x4{q.x, q.y, 0u, 0u};
        } else if constexpr (RawSteps<TI, K>::VB == 4) {
            r.w[v] = u32x4{*reinterpret_cast<const uint32_t *>(p), 0u, 0u, 0u};
        } else {
            r.w[v] = u32x4{(uint32_t)*reinterpret_cast<const uint16_t *>(p), 0u, 0u, 0u};
        }
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
        float part[4 * PW];
        unpack_word(r.w[v].x, &part[0 * PW], TI{});
        if constexpr (RawSteps<TI, K>::VB >= 8)
            unpack_word(r.w[v].y, &part[1 * PW], TI{});
        if constexpr (RawSteps<TI, K>::VB == 16) {
            unpack_word(r.w[v].z, &part[2 * PW], TI{});
            unpack_word(r.w[v].w, &part[3 * PW], TI{});
        }
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
    if constexpr (VEC) {
        constexpr int E = RawSteps<TI, K>::E, PW = PerWord<TI>::value;
#pragma unroll
        for (int v = 0; v < K / E; ++v) {
            const int off = tl + v * E;
            if (off >= lo && off + E <= hi) {
                float part[E < PW ? PW : E];
#pragma unroll
                for (int e = 0; e < E; ++e)
                    part[e] = src[v * E + e];
                if constexpr (RawSteps<TI, K>::VB == 16)
                    store_vec_cached<TI, E>(row + off, part);
                else if constexpr (RawSteps<TI, K>::VB == 8)
                    *reinterpret_cast<uint2 *>(row + off) = uint2{pack_word(&part[0], TI{}), pack_word(&part[PW], TI{})};
                else if constexpr (RawSteps<TI, K>::VB == 4)
                    *reinterpret_cast<uint32_t *>(row + off) = pack_word(&part[0], TI{});
                else
                    row[off] = from_f32<TI>(part[0]);
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
// most 168 VGPRs) without spilling, and the other variants are allowed two.
template <typename TI, bool VEC, bool A_PER_STATE, bool ONE_CHUNK>
constexpr int scan_waves_per_simd()
{
    return (std::is_same<TI, f16>::value && VEC && (ONE_CHUNK || !A_PER_STATE)) ? 3 : 2;
}

// Walks: WALK_DENSE, tiles of 16 steps per lane; WALK_LADDER, the same
// ending in tiles of 8, 4, 2 and 1 steps per lane, for packed batches (their
// sequences handed out longest first) and for dense rows whose length is not
// a multiple of 256.
enum { WALK_DENSE = 0, WALK_LADDER = 1 };

// The scan of workgroup `bid` of a grid of `nbid` scan workgroups.
template <typename TI, typename TS, bool A_PER_STATE, bool VEC, bool ONE_CHUNK, int WALK>
__device__ __forceinline__ void scan_body(const ScanArgs &a, uint32_t bid, uint32_t nbid)
{
    constexpr int E = 16 / StorageSize<TI>::value;  // elements per 128-bit vector
    // B/C chunk in a lane-interleaved layout: the float4 holding timesteps
    // [K r + 4q, K r + 4q + 4) of local state nl sits at (nl*(K/4) + q)*R + r,
    // so the 16 lanes of a row read 16 consecutive float4s (no bank conflict).
    __shared__ float4 lds_b[NC * R * KD / 4];
    __shared__ float4 lds_c[NC * R * KD / 4];
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
    const uint32_t lb = a.cu_seqlens ? bid : xcd_block_order(bid, nbid);
    const int cb = (int)(lb % nblk_g);
    const int bg = (int)(lb / nblk_g);
    const int g = bg % a.ngroups;
    int b = bg / a.ngroups;
    if constexpr (WALK == WALK_LADDER) {
        // packed batches: the longest sequences' workgroups start first, so
        // the longest walks do not begin late and leave the chip idle at the
        // end
        if (a.cu_seqlens && a.batch <= 256)
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

    const int64_t blk = sp.block;
    const TI *urow = static_cast<const TI *>(a.u) + blk * a.u_sb + c * a.u_sc + col0;
    const TI *dtrow = static_cast<const TI *>(a.dt) + blk * a.dt_sb + h * a.dt_sh + col0;
    const TI *zrow = a.z ? static_cast<const TI *>(a.z) + blk * a.z_sb + c * a.z_sc + col0 : nullptr;
    TI *orow = static_cast<TI *>(a.out) + blk * a.o_sb + c * a.o_sc + col0;
    const TI *Bg = static_cast<const TI *>(a.B) + blk * a.B_sb + g * a.B_sg + col0;
    const TI *Cg = static_cast<const TI *>(a.C) + blk * a.C_sb + g * a.C_sg + col0;
    TS *srow = a.state ? static_cast<TS *>(a.state) + slot * a.st_ss + h * a.st_sh + p * a.st_sp : nullptr;
    const bool load_init = srow && sp.init;

    const float bias_h = a.dt_bias ? a.dt_bias[h] : 0.0f;
    const float D_h = a.D ? a.D[h] : 0.0f;
    const float A2_h = A_PER_STATE ? 0.0f : a.A[h] * kLog2e;

    for (int n = r; n < N; n += R) {
        lds_carry[ch][n] = load_init ? to_f32(srow[n]) : 0.0f;
        if constexpr (A_PER_STATE)
            lds_a2[ch][n] = a.A[h * a.A_sh + n] * kLog2e;
    }

    // One tile: 16 lanes x K steps per channel, starting at column t0.
    auto tile = [&](auto kc, const int t0) {
        constexpr int K = decltype(kc)::value;
        constexpr int T = R * K;  // timesteps per tile
        const int tl = t0 + r * K;
        // a tile whose every step lies in the sequence needs no masking
        // (uniform over the workgroup; most tiles of a dense batch)
        const bool full = t0 >= lo && t0 + T <= hi;
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
            auto steps = [&](auto all_in) {
#pragma unroll
                for (int i = 0; i < K; ++i) {
                    const float v = dd[i] + bias_h;
                    const float spv = softplus_f32(v);
                    float d = a.dt_softplus ? spv : v, uv = uu[i];
                    if constexpr (!decltype(all_in)::value) {
                        // identity step outside the sequence (decay 1, input 0)
                        const bool in = tl + i >= lo && tl + i < hi;
                        d = in ? d : 0.0f;
                        uv = in ? uv : 0.0f;
                    }
                    dl[i] = d;
                    du[i] = d * uv;
                    y[i] = D_h * uv;
                }
            };
            if (full)
                steps(std::true_type{});
            else
                steps(std::false_type{});
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
            const bool bc_full = full && n0 + NC <= N;  // no state or step out of range
            for (int m = tid; m < NC * T / E; m += 256) {
                const int nl = m / (T / E), tc = (m % (T / E)) * E;
                const int n = n0 + nl, t = t0 + tc;
                float vb[E], vc[E];
                if constexpr (VEC) {
                    if (bc_full) {
                        load_vec_cached<TI, E>(Bg + n * a.B_sn + t, vb);
                        load_vec_cached<TI, E>(Cg + n * a.C_sn + t, vc);
                    } else {
                        // clamped address, unconditional load, then select
                        const bool ok = n < N && t < hi;
                        load_vec_cached<TI, E>(Bg + (ok ? n * a.B_sn + t : 0), vb);
                        load_vec_cached<TI, E>(Cg + (ok ? n * a.C_sn + t : 0), vc);
#pragma unroll
                        for (int e = 0; e < E; ++e) {
                            const bool in = ok && t + e >= lo && t + e < hi;
                            vb[e] = in ? vb[e] : 0.0f;
                            vc[e] = in ? vc[e] : 0.0f;
                        }
                    }
                } else {
#pragma unroll
                    for (int e = 0; e < E; ++e) {
                        const bool ok = n < N && t + e >= lo && t + e < hi;
                        const float xb = to_f32(Bg[ok ? n * a.B_sn + t + e : lo]);
                        const float xc = to_f32(Cg[ok ? n * a.C_sn + t + e : lo]);
                        vb[e] = ok ? xb : 0.0f;
                        vc[e] = ok ? xc : 0.0f;
                    }
                }
#pragma unroll
                for (int e4 = 0; e4 < E / 4; ++e4) {
                    const int tt = tc + 4 * e4;
                    // tiles of fewer than 4 steps per lane: the state's T steps
                    // in order (a lane reads its K consecutive floats)
                    const int idx = K >= 4 ? (nl * (K / 4) + (tt % K) / 4) * R + tt / K : (nl * T + tt) / 4;
                    lds_b[idx] = make_float4(vb[4 * e4], vb[4 * e4 + 1], vb[4 * e4 + 2], vb[4 * e4 + 3]);
                    lds_c[idx] = make_float4(vc[4 * e4], vc[4 * e4 + 1], vc[4 * e4 + 2], vc[4 * e4 + 3]);
                }
            }
            __syncthreads();
            // four states per pass: 196.6 against 199.1 us one at a time
            // (2: 197.2, 8: 198.0) on the Mamba-1 2.8B prefill
#pragma unroll 4
            for (int nl = 0; nl < NC; ++nl) {
                if (n0 + nl >= N)
                    break;
                const int n = n0 + nl;
                float Bv[K], Cv[K];
                if constexpr (K >= 4) {
#pragma unroll
                    for (int q = 0; q < K / 4; ++q) {
                        const float4 vb = lds_b[(nl * (K / 4) + q) * R + r];
                        const float4 vc = lds_c[(nl * (K / 4) + q) * R + r];
                        Bv[4 * q] = vb.x; Bv[4 * q + 1] = vb.y; Bv[4 * q + 2] = vb.z; Bv[4 * q + 3] = vb.w;
                        Cv[4 * q] = vc.x; Cv[4 * q + 1] = vc.y; Cv[4 * q + 2] = vc.z; Cv[4 * q + 3] = vc.w;
                    }
                } else {
                    const float *fb = reinterpret_cast<const float *>(lds_b) + nl * T + r * K;
                    const float *fc = reinterpret_cast<const float *>(lds_c) + nl * T + r * K;
#pragma unroll
                    for (int i = 0; i < K; ++i) {
                        Bv[i] = fb[i];
                        Cv[i] = fc[i];
                    }
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
    };
    if constexpr (WALK != WALK_DENSE) {
        // Each sequence pads its last tile to a tile boundary.  Tiles of 16
        // steps per lane while more than 3/4 of one remains, then of 8 while
        // more than 64 steps remain, then at most one each of 4, 2 and 1
        // (64, 32 and 16 steps), each taken while more than half of it
        // remains: under 16 padded steps per sequence, and the dense
        // per-step cost for the rest.
        int t0 = 0;
        for (; hi - t0 > 3 * R * KD / 4; t0 += R * KD)
            tile(std::integral_constant<int, KD>{}, t0);
        for (; hi - t0 > R * 4; t0 += R * 8)
            tile(std::integral_constant<int, 8>{}, t0);
        if (hi - t0 > R * 2) {
            tile(std::integral_constant<int, 4>{}, t0);
            t0 += R * 4;
        }
        if (hi - t0 > R) {
            tile(std::integral_constant<int, 2>{}, t0);
            t0 += R * 2;
        }
        if (t0 < hi)
            tile(std::integral_constant<int, 1>{}, t0);
    } else {
        for (int t0 = 0; t0 < hi; t0 += R * KD)
            tile(std::integral_constant<int, KD>{}, t0);
    }
    __syncthreads();
    if (srow && active)
        for (int n = r; n < N; n += R)
            srow[n] = from_f32<TS>(lds_carry[ch][n]);
}

template <typename TI, typename TS, bool A_PER_STATE, bool VEC, bool ONE_CHUNK, int WALK>
__global__ __launch_bounds__(256)
__attribute__((amdgpu_waves_per_eu(scan_waves_per_simd<TI, VEC, A_PER_STATE, ONE_CHUNK>())))
void scan_kernel(ScanArgs a)
{
    scan_body<TI, TS, A_PER_STATE, VEC, ONE_CHUNK, WALK>(a, blockIdx.x, gridDim.x);
}

} // namespace ssm
