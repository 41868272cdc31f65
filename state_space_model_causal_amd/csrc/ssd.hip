// ssd.hip -- Mamba-2 prefill (one decay per head) in chunked matrix form on
// the gfx950 matrix cores.
//
// Operation: the same selective scan as scan.hip (the selective-scan operator
// of "feat(llama.cu): 适配 mamba 模型", InfiniLM-Rust PR #48, section 2.1, with
// its silu(z) gate and the final state to the request's slot, section 3.1),
// for the case where the decay exp(delta_t * A_h) is one scalar per head and
// step.  The result is the recurrence's, up to rounding; only the order of
// the arithmetic changes.
//
// With a scalar decay the recurrence over a chunk of Q steps is a product of
// small dense matrices.  For head h, rows p (headdim) and states n, with the
// chunk's cumulative log-decay L_s = sum_{i<=s} delta_i A_h:
//     Y[s,p]  = sum_{r<=s} C_s.B_r exp(L_s - L_r) delta_r X[r,p]     (within)
//             + exp(L_s) sum_n C_s[n] H[p,n]                           (carried)
//     H'[p,n] = exp(L_Q-1) H[p,n] + sum_r exp(L_Q-1 - L_r) delta_r B_r[n] X[r,p]
// where H is the state entering the chunk.  The four contractions (C^T B over
// states, the masked decay matrix times X, C times H^T, and B times the
// weighted X) run on the 16x16x32 matrix instructions with float32
// accumulation, each product keeping one operand exact:
//   * bf16 I/O: all on v_mfma_f32_16x16x32_bf16; B, C and X are exact, and
//     the float32 operand (the masked decay matrix, the carried state, the
//     weighted X) is split into a bf16 high part and a bf16 remainder (about
//     16 significant bits per product).
//   * f16 I/O: C^T B on v_mfma_f32_16x16x32_f16 (exact products); X split
//     exactly into two bf16 parts against the bf16 decay matrix; C and B as
//     stored on the f16 instruction against the carried state and the
//     weighted X, split into f16 parts under a power-of-two scale per row p
//     (no part overflows; about 22 significant bits), scaled back afterwards.
//
// Work decomposition: one 512-lane workgroup per (request, head, 64 rows of
// headdim); in a packed batch the request is a sequence, walked from the
// 16-byte vector holding its first column, its neighbours' columns being
// identity steps (zero step size), the longest sequences first.  Each wave owns 16 rows and half of the states: its part of the
// state (dstate/2 x 16, float32) stays in MFMA accumulators for the whole
// sequence, which is walked in chunks of 64 steps.  Per chunk the workgroup
// stages B and C in LDS as stored ([state][step]; the operands that need them
// transposed use gfx950's transpose reads), builds the masked decay matrix
// once for all waves, then every wave computes its share of the outputs and
// updates its part of the state.  Two waves per SIMD let one wave's vector
// work overlap the other's matrix work.  The next chunk's loads are issued in
// three parts between the phases, and two barriers per chunk suffice (the
// staged tiles' last readers precede the second).  HBM traffic: u, dt, z, B,
// C read once (B and C from L2 for every head of a group), out written once,
// the state read and written once.
#include <algorithm>
#include <type_traits>

#include "ssm_device.hpp"
#include "ssm_kernels.hpp"

namespace ssm {

namespace {
constexpr int SQ = 64;   // chunk length (steps)
constexpr int SPB = 64;  // headdim rows per workgroup (4 row tiles of 16)
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
} // namespace

__device__ __forceinline__ f32x4_t mma(bf16x8_t a, bf16x8_t b, f32x4_t c)
{
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// a = ha + la and b = hb + lb with the four parts in bfloat16 (relative
// error of a pair ~2^-16): the high parts are a and b rounded (one packed
// conversion), the remainders are exact in float32 before their own rounding
__device__ __forceinline__ void split_pair(float a, float b, uint32_t &hi, uint32_t &lo)
{
    hi = pk_bf16(a, b);
    // the low half moved up by a byte permute (a shift there is rewritten
    // into a second conversion of a alone)
    const float ha = __uint_as_float(__builtin_amdgcn_perm(0u, hi, 0x01000c0cu));
    lo = pk_bf16(a - ha, b - __uint_as_float(hi & 0xffff0000u));
}

__device__ __forceinline__ void split_bf16(const float (&x)[8], bf16x8_t &hi, bf16x8_t &lo)
{
    uint32_t h[4], l[4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
        split_pair(x[2 * i], x[2 * i + 1], h[i], l[i]);
    hi = __builtin_bit_cast(bf16x8_t, u32x4{h[0], h[1], h[2], h[3]});
    lo = __builtin_bit_cast(bf16x8_t, u32x4{l[0], l[1], l[2], l[3]});
}

__device__ __forceinline__ bf16x8_t as_bf16x8(u32x4 w) { return __builtin_bit_cast(bf16x8_t, w); }

// f16 I/O: the f16 matrix instruction of the same shape and lane layout
typedef _Float16 f16x8_t __attribute__((ext_vector_type(8)));
__device__ __forceinline__ f16x8_t as_f16x8(u32x4 w) { return __builtin_bit_cast(f16x8_t, w); }
__device__ __forceinline__ f32x4_t mma16(f16x8_t a, f16x8_t b, f32x4_t c)
{
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}

// The product of two operands exact in the I/O type (B and C as stored).
template <typename TI>
__device__ __forceinline__ f32x4_t mma_io(u32x4 a, u32x4 b, f32x4_t c)
{
    if constexpr (std::is_same<TI, f16>::value)
        return mma16(as_f16x8(a), as_f16x8(b), c);
    else
        return mma(as_bf16x8(a), as_bf16x8(b), c);
}

// 8 values of the I/O type (raw bits) as floats
template <typename TI>
__device__ __forceinline__ void widen8(u32x4 w, float (&x)[8])
{
    unpack_word(w.x, &x[0], TI{});
    unpack_word(w.y, &x[2], TI{});
    unpack_word(w.z, &x[4], TI{});
    unpack_word(w.w, &x[6], TI{});
}

// A power of two s, and 1/s, that bring m (>= 0) into [2^13, 2^14): the
// scale under which float32 values of magnitude <= m split into f16 high and
// low parts without overflow, with 22 significant bits for the largest
// (exponents clamped to the normal range; a zero m gives the largest s).
__device__ __forceinline__ void pow2_scale(float m, float &s, float &inv)
{
    const int be = (__float_as_int(m) >> 23) & 0xff;  // m = f 2^(be-126), f in [0.5, 1)
    int k = 14 - (be - 126);
    k = k < -126 ? -126 : (k > 126 ? 126 : k);
    s = __int_as_float((k + 127) << 23);
    inv = __int_as_float((127 - k) << 23);
}

// x s = hi + lo with hi and lo in f16 (|x s| <= 2^14)
__device__ __forceinline__ void split_f16(const float (&x)[8], float s, f16x8_t &hi, f16x8_t &lo)
{
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const float v = x[i] * s;
        const _Float16 h = (_Float16)v;
        hi[i] = h;
        lo[i] = (_Float16)(v - (float)h);
    }
}

// the largest value over the 4 lanes that share lane % 16 (the lanes that
// hold one column of an MFMA operand or result)
__device__ __forceinline__ float col_max4(float m)
{
    m = fmaxf(m, __shfl_xor(m, 16));
    return fmaxf(m, __shfl_xor(m, 32));
}

typedef short s16x4_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4_t lds_s16x4_t;

// gfx950 transpose read (ds_read_b64_tr_b16).  Within each 16-lane group,
// lane 4i + a supplies the address of 4 consecutive 16-bit elements; lane
// 4a + b receives element b of lanes a, 4 + a, 8 + a, 12 + a.  So if lane
// 4i + a points at row n0 + i, columns c0 + 4a .. +3 of a row-major tile, lane
// d = 4a + b receives column c0 + d of rows n0 .. n0 + 3: a column of the
// tile, as an MFMA operand holds it.
__device__ __forceinline__ uint2 ds_read_tr(const __bf16 *p)
{
    const s16x4_t v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_t *)(p));
    return __builtin_bit_cast(uint2, v);
}

// 8 consecutive rows n0 .. n0 + 7 (read as rows n0 + i and n0 + 4 + i) of
// column c0 + (lane % 16) of a row-major LDS tile with row stride ld: the
// k-operand of one lane of v_mfma_f32_16x16x32_bf16 from the natural layout.
// n0 and c0 may differ between the lane's 16-lane groups.
__device__ __forceinline__ u32x4 col8_tr(const __bf16 *tile, int ld, int n0, int n0b, int c0, int l16)
{
    const int i = l16 >> 2, a = l16 & 3;
    const uint2 lo = ds_read_tr(tile + (n0 + i) * ld + c0 + 4 * a);
    const uint2 hi = ds_read_tr(tile + (n0b + i) * ld + c0 + 4 * a);
    return u32x4{lo.x, lo.y, hi.x, hi.y};
}

constexpr int SNW = 8;           // waves per workgroup
constexpr int STHREADS = 64 * SNW;

// Global data of one chunk, loaded a chunk ahead (registers) so that the
// loads of chunk c+1 are in flight while chunk c is computed.
template <typename TI, int N>
struct ChunkLoads {
    static constexpr int NUNITS = (N / 2) * (SQ / 8);  // (pair of states, 8 steps)
    static constexpr int UNITS = (NUNITS + STHREADS - 1) / STHREADS;
    u32x4 b0[UNITS], b1[UNITS], c0[UNITS], c1[UNITS];
    u32x4 x[2];          // X[p][t0 + 32 kk + 8 lq .. +8)
    uint2 xo[2], zo[2];  // u and z at steps t0 + 16 st + 4 lq .. +4, this wave's 2 row tiles
    TI dt;               // dt of step t0 + lane, as stored (wave 0 widens it when staging)
};

// The B (or C) part of a chunk's loads: unit u of the chunk is a pair of
// states and 8 steps.
template <typename TI, int N>
__device__ __forceinline__ void load_pairs(u32x4 (&v0)[(ChunkLoads<TI, N>::UNITS)], u32x4 (&v1)[(ChunkLoads<TI, N>::UNITS)],
                                           int t0, int L, const TI *G, int64_t sn, int tid)
{
#pragma unroll
    for (int k = 0; k < ChunkLoads<TI, N>::UNITS; ++k) {
        const int u = min(tid + STHREADS * k, ChunkLoads<TI, N>::NUNITS - 1);
        const int n = 2 * (u >> 3), tv = u & 7;
        const int t = t0 + 8 * tv;
        const int tc = t < L ? t : 0;  // clamped; zeroed when staged
        // byte offsets from the workgroup's base (32-bit: the host checks the
        // extent), so that the loads take the scalar base + vector offset form
        const uint32_t o0 = 2u * (uint32_t)(n * (int)sn + tc), o1 = o0 + 2u * (uint32_t)sn;
        const char *g = reinterpret_cast<const char *>(G);
        v0[k] = *reinterpret_cast<const u32x4 *>(g + o0);
        v1[k] = *reinterpret_cast<const u32x4 *>(g + o1);
    }
}

// The rest of a chunk's loads: u, z and dt.
template <typename TI, int N>
__device__ __forceinline__ void load_rows(ChunkLoads<TI, N> &c, int t0, int L, const TI *urow, const TI *zrow,
                                          const TI *dtrow, int l, int lq, int nh)
{
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
        const int t = t0 + 32 * kk + 8 * lq;
        c.x[kk] = *reinterpret_cast<const u32x4 *>(urow + (t < L ? t : 0));
    }
    // No load below sits under a branch or next to a select on its value:
    // the compiler would wait for it there, and that wait would also cover
    // every load issued before it (the whole chunk).  Without a gate the z
    // load reads u, and the value goes unused; every wave loads dt (wave 0
    // uses it).
    const TI *zsrc = zrow ? zrow : urow;
#pragma unroll
    for (int i = 0; i < 2; ++i) {
        const int t = t0 + 16 * (2 * nh + i) + 4 * lq;
        const int tc = t < L ? t : 0;
        c.xo[i] = *reinterpret_cast<const uint2 *>(urow + tc);
        c.zo[i] = *reinterpret_cast<const uint2 *>(zsrc + tc);
    }
    {
        const int t = t0 + l;
        c.dt = dtrow[t < L ? t : t0];
    }
}

template <typename TI, int N>
__device__ __forceinline__ void load_chunk(ChunkLoads<TI, N> &c, int t0, int L, const TI *Bg, const TI *Cg,
                                           int64_t bsn, int64_t csn, const TI *urow, const TI *zrow,
                                           const TI *dtrow, int tid, int l, int lq, int nh)
{
    load_pairs<TI, N>(c.b0, c.b1, t0, L, Bg, bsn, tid);
    load_pairs<TI, N>(c.c0, c.c1, t0, L, Cg, csn, tid);
    load_rows<TI, N>(c, t0, L, urow, zrow, dtrow, l, lq, nh);
}

__device__ __forceinline__ float bf_lo(uint32_t v) { return __uint_as_float(v << 16); }
__device__ __forceinline__ float bf_hi(uint32_t v) { return __uint_as_float(v & 0xffff0000u); }

// Eight waves: wave w owns headdim rows 16 (w%4) .. +16 of the workgroup's 64
// and half of the states, n-tiles [NT/2 (w/4), NT/2 (w/4 + 1)); the two
// waves of a row block exchange their halves of C.H through LDS and each
// writes half of the chunk's output rows (row tiles 2 (w/4) and 2 (w/4) + 1).
template <typename TI, typename TS, int N>
__global__ __launch_bounds__(STHREADS) void ssd_kernel(ScanArgs a)
{
    constexpr int LDQ = SQ + 8;  // row stride of the natural B and C tiles and of M
    constexpr int NT = N / 16;   // 16-state tiles of the state
    constexpr int NTH = NT / 2;  // tiles per wave
    // B and C of the chunk as stored, [n][r] and [n][s]; the operands that
    // need them transposed read them with transpose reads
    __shared__ __align__(16) __bf16 s_bn[N * LDQ];
    __shared__ __align__(16) __bf16 s_cn[N * LDQ];
    __shared__ __align__(16) __bf16 s_mh[SQ * LDQ];  // masked decay matrix M[s][r], high part
    __shared__ __align__(16) __bf16 s_ml[SQ * LDQ];  // and remainder
    __shared__ __align__(16) float s_x[SNW][2][64][4];  // C.H halves for the partner wave
    // e^{L} is read after the second barrier, by the outputs; it is kept per
    // chunk parity so that the next chunk's staging (which no barrier
    // separates from this chunk's outputs) does not overwrite it
    __shared__ float s_d[SQ], s_L[SQ], s_eL[2][SQ], s_w[SQ], s_etot[1];

    const int P = a.headdim, H = a.nheads;
    const int npb = P / SPB;
    const int pb = blockIdx.x % npb;
    const int bh = blockIdx.x / npb;
    const int h = bh % H;
    int b = bh / H;
    // packed batches: the longest sequences' workgroups start first
    if (a.cu_seqlens && a.batch <= 256)
        b = packed_seq_of_rank(a.cu_seqlens, a.batch, a.seqlen, b);
    const int g = h / a.heads_per_group;
    const int slot = a.slot_idx ? a.slot_idx[b] : b;
    if (slot < 0)
        return;  // padded request (uniform over the workgroup)
    // the request's columns: the whole rows of a dense batch; in a packed
    // batch the sequence's columns, walked from the 16-byte vector holding
    // its first one, with the columns of its neighbours as identity steps
    const SeqSpan sp = seq_span(a.cu_seqlens, a.has_init_seq, b, a.seqlen, a.has_initial_state);
    if (sp.len == 0)
        return;
    const int lo = sp.begin % 8, hi = lo + sp.len;  // the walk covers columns [0, hi), the sequence [lo, hi)
    const int64_t col0 = sp.begin - lo, blk = sp.block;

    const int tid = threadIdx.x, w = tid >> 6, l = tid & 63;
    const int l16 = l & 15, lq = l >> 4;
    const int pw = w & 3, nh = w >> 2;        // row tile, state half
    const int partner = pw + 4 * (1 - nh);
    const int p = pb * SPB + 16 * pw + l16;   // this lane's row of headdim
    const int64_t c = (int64_t)h * P + p;  // channel
    constexpr bool F16 = std::is_same<TI, f16>::value;
    const TI *urow = static_cast<const TI *>(a.u) + blk * a.u_sb + c * a.u_sc + col0;
    const TI *zrow = a.z ? static_cast<const TI *>(a.z) + blk * a.z_sb + c * a.z_sc + col0 : nullptr;
    TI *orow = static_cast<TI *>(a.out) + blk * a.o_sb + c * a.o_sc + col0;
    const TI *dtrow = static_cast<const TI *>(a.dt) + blk * a.dt_sb + h * a.dt_sh + col0;
    const TI *Bg = static_cast<const TI *>(a.B) + blk * a.B_sb + g * a.B_sg + col0;
    const TI *Cg = static_cast<const TI *>(a.C) + blk * a.C_sb + g * a.C_sg + col0;
    TS *srow = a.state ? static_cast<TS *>(a.state) + slot * a.st_ss + h * a.st_sh + p * a.st_sp : nullptr;

    const float bias = a.dt_bias ? a.dt_bias[h] : 0.0f;
    const float Dh = a.D ? a.D[h] : 0.0f;
    const float A2 = a.A[h] * kLog2e;

    // this wave's state^T tiles: hacc[q][j] = H[p][16 (NTH nh + q) + 4 lq + j]
    f32x4_t hacc[NTH];
#pragma unroll
    for (int q = 0; q < NTH; ++q) {
        f32x4_t v = {0.0f, 0.0f, 0.0f, 0.0f};
        if (srow && sp.init) {
#pragma unroll
            for (int j = 0; j < 4; ++j)
                v[j] = to_f32(srow[16 * (NTH * nh + q) + 4 * lq + j]);
        }
        hacc[q] = v;
    }

    // the two upper tiles of M that the outputs read, (0, 1) and (2, 3), stay
    // zero; every other tile they read is computed in each chunk
    {
        const int tile = tid >> 8, e = tid & 255;
        const int s = 32 * tile + (e >> 4), r = 32 * tile + 16 + (e & 15);
        s_mh[s * LDQ + r] = (__bf16)0.0f;
        s_ml[s * LDQ + r] = (__bf16)0.0f;
    }

    ChunkLoads<TI, N> cur;
    load_chunk<TI, N>(cur, 0, hi, Bg, Cg, a.B_sn, a.C_sn, urow, zrow, dtrow, tid, l, lq, nh);

    for (int t0 = 0; t0 < hi; t0 += SQ) {
        const int par = (t0 / SQ) & 1;
        // ---- stage the chunk (its loads were issued one chunk earlier).
        // The previous chunk's readers of the staged B, C, delta, L and w
        // all sit before its second barrier, so no barrier is needed here.
        if (w == 0) {
            const bool ok = t0 + l >= lo && t0 + l < hi;
            const float v = to_f32(cur.dt) + bias;
            const float sp = softplus_f32(v);
            const float d = ok ? (a.dt_softplus ? sp : v) : 0.0f;  // identity step past the end
            // log2 of the decay over the chunk's steps up to this one
            const float cum = wave_prefix_sum(d * A2);
            const float tot = lane_value(cum, 63);
            s_d[l] = d;
            s_L[l] = cum;
            s_eL[par][l] = exp2_hw(cum);
            s_w[l] = exp2_hw(tot - cum) * d;
            if (l == 0)
                s_etot[0] = exp2_hw(tot);
        }
#pragma unroll
        for (int k = 0; k < ChunkLoads<TI, N>::UNITS; ++k) {
            const int u = tid + STHREADS * k;
            if (u < ChunkLoads<TI, N>::NUNITS) {
                const int n = 2 * (u >> 3), tv = u & 7;
                // a vector past the end is zeroed (rows are a multiple of 8
                // long); the steps of the first vector before the sequence
                // take a zero step size (no decay, no input)
                const bool ok = t0 + 8 * tv < hi;
                const u32x4 z4 = {0u, 0u, 0u, 0u};
                const u32x4 b0 = ok ? cur.b0[k] : z4, b1 = ok ? cur.b1[k] : z4;
                const u32x4 c0 = ok ? cur.c0[k] : z4, c1 = ok ? cur.c1[k] : z4;
                *reinterpret_cast<u32x4 *>(&s_bn[n * LDQ + 8 * tv]) = b0;
                *reinterpret_cast<u32x4 *>(&s_bn[(n + 1) * LDQ + 8 * tv]) = b1;
                *reinterpret_cast<u32x4 *>(&s_cn[n * LDQ + 8 * tv]) = c0;
                *reinterpret_cast<u32x4 *>(&s_cn[(n + 1) * LDQ + 8 * tv]) = c1;
            }
        }
        u32x4 xk[2];
#pragma unroll
        for (int kk = 0; kk < 2; ++kk)
            xk[kk] = t0 + 32 * kk + 8 * lq < hi ? cur.x[kk] : u32x4{0u, 0u, 0u, 0u};
        const uint2 xo[2] = {cur.xo[0], cur.xo[1]}, zo[2] = {cur.zo[0], cur.zo[1]};
        // f16 I/O: X as the sum of two bf16 parts (exact: an f16 value's 11
        // significant bits fit in a rounded bf16 and its remainder), the
        // operand the bf16 decay matrix multiplies
        bf16x8_t xkh[2], xkl[2];
        if constexpr (F16) {
#pragma unroll
            for (int kk = 0; kk < 2; ++kk) {
                float xf[8];
                widen8<TI>(xk[kk], xf);
                split_bf16(xf, xkh[kk], xkl[kk]);
            }
        }
        __syncthreads();

        // ---- the next chunk's loads, in flight during this chunk's work;
        // issued in three parts between the phases below, so that no wave
        // stalls on a full load queue for the whole chunk's worth at once
        const bool more = t0 + SQ < hi;
        if (more)
            load_pairs<TI, N>(cur.c0, cur.c1, t0 + SQ, hi, Cg, a.C_sn, tid);

        // ---- carried state over this wave's half of the states:
        // yc[k] = sum_{n in half} C_s[n] H[p][n] over the steps s of row tile
        // st = (k + 2 (1 - nh)) % 4: the partner's two output tiles first
        // (k = 0, 1), then this wave's own (k = 2, 3); the state as MFMA
        // operands (high and low parts) in the order the accumulators hold it
        f32x4_t yc[4];
        {
            if constexpr (F16) {
                // the f16 instruction takes C as stored; the state is split
                // into f16 parts under a power-of-two scale per row p (this
                // lane's column of every state tile), so no part overflows,
                // and the products are scaled back
                float m = 0.0f;
#pragma unroll
                for (int q = 0; q < NTH; ++q)
#pragma unroll
                    for (int i = 0; i < 4; ++i)
                        m = fmaxf(m, fabsf(hacc[q][i]));
                float hsc, hinv;
                pow2_scale(col_max4(m), hsc, hinv);
                f16x8_t hh[NTH / 2], hl[NTH / 2];
#pragma unroll
                for (int q2 = 0; q2 < NTH / 2; ++q2) {
                    float hv[8];
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        hv[i] = hacc[2 * q2][i];
                        hv[4 + i] = hacc[2 * q2 + 1][i];
                    }
                    split_f16(hv, hsc, hh[q2], hl[q2]);
                }
#pragma unroll
                for (int k = 0; k < 4; ++k) {
                    const int st = (k + 2 * (1 - nh)) & 3;
                    f32x4_t acc = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
                    for (int q2 = 0; q2 < NTH / 2; ++q2) {
                        const int kk = (NTH / 2) * nh + q2;
                        const int nc = 32 * kk + 4 * lq;
                        const f16x8_t cv = as_f16x8(col8_tr(s_cn, LDQ, nc, nc + 16, 16 * st, l16));
                        acc = mma16(cv, hh[q2], acc);
                        acc = mma16(cv, hl[q2], acc);
                    }
                    yc[k] = acc * hinv;
                }
            } else {
                bf16x8_t hh[NTH / 2], hl[NTH / 2];
#pragma unroll
                for (int q2 = 0; q2 < NTH / 2; ++q2) {
                    float hv[8];
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        hv[i] = hacc[2 * q2][i];
                        hv[4 + i] = hacc[2 * q2 + 1][i];
                    }
                    split_bf16(hv, hh[q2], hl[q2]);
                }
#pragma unroll
                for (int k = 0; k < 4; ++k) {
                    const int st = (k + 2 * (1 - nh)) & 3;
                    f32x4_t acc = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
                    for (int q2 = 0; q2 < NTH / 2; ++q2) {
                        const int kk = (NTH / 2) * nh + q2;  // 32-state step
                        // C_s[n] for s = 16 st + l16 and the states of hh's order:
                        // n = 32 kk + 4 lq + i and 32 kk + 16 + 4 lq + i
                        const int nc = 32 * kk + 4 * lq;
                        const bf16x8_t cv = as_bf16x8(col8_tr(s_cn, LDQ, nc, nc + 16, 16 * st, l16));
                        acc = mma(cv, hh[q2], acc);
                        acc = mma(cv, hl[q2], acc);
                    }
                    yc[k] = acc;
                }
            }
            // the partner needs this half for its output row tiles
            *reinterpret_cast<f32x4_t *>(&s_x[partner][0][l][0]) = yc[0];
            *reinterpret_cast<f32x4_t *>(&s_x[partner][1][l][0]) = yc[1];
        }

        // the gate of this wave's outputs, computed here where the matrix
        // work of the other waves hides it (1 without z)
        float gz[2][4];
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            float zv[4];
            unpack_word(zo[i].x, &zv[0], TI{});
            unpack_word(zo[i].y, &zv[2], TI{});
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                gz[i][j] = zrow ? silu_f32(zv[j]) : 1.0f;
                // pinned here: left alone, the compiler sinks the gate into
                // the output phase, where nothing overlaps it
                asm volatile("" ::"v"(gz[i][j]));
            }
        }

        if (more)
            load_pairs<TI, N>(cur.b0, cur.b1, t0 + SQ, hi, Bg, a.B_sn, tid);

        // ---- masked decay matrix M[s][r] = (C_s.B_r) exp(L_s - L_r) delta_r
        // for r <= s, over its 10 lower-triangle 16 x 16 tiles (st, rt).  The
        // tiles are dealt so that waves w and w + 4 (which share a SIMD) hold
        // at most 3 between them: one byte per (wave, tile), st in the high
        // nibble and rt in the low one, 0xff for none
        {
            const uint64_t deal = w < 4 ? 0xff22ff2011103300ull : 0xff32ff21ff31ff30ull;
#pragma unroll
            for (int i = 0; i < 2; ++i) {
                const int code = (int)((deal >> (8 * (2 * pw + i))) & 0xffu);
                if (code != 0xff) {
                    const int st = code >> 4, rt = code & 15;
                    const int s = 16 * st + l16;
                    f32x4_t acc = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
                    for (int kk = 0; kk < N / 32; ++kk) {
                        const int nb = 32 * kk + 8 * lq;
                        const u32x4 av = col8_tr(s_bn, LDQ, nb, nb + 4, 16 * rt, l16);
                        const u32x4 bv = col8_tr(s_cn, LDQ, nb, nb + 4, 16 * st, l16);
                        acc = mma_io<TI>(av, bv, acc);
                    }
                    const float Ls = s_L[s];
                    const int r0 = 16 * rt + 4 * lq;
                    const float4 Lr = *reinterpret_cast<const float4 *>(&s_L[r0]);
                    const float4 dr = *reinterpret_cast<const float4 *>(&s_d[r0]);
                    const float lr[4] = {Lr.x, Lr.y, Lr.z, Lr.w}, dv[4] = {dr.x, dr.y, dr.z, dr.w};
                    float m[4];
#pragma unroll
                    for (int j = 0; j < 4; ++j)
                        m[j] = (r0 + j <= s) ? acc[j] * exp2_hw(Ls - lr[j]) * dv[j] : 0.0f;
                    uint32_t mh[2], ml[2];
                    split_pair(m[0], m[1], mh[0], ml[0]);
                    split_pair(m[2], m[3], mh[1], ml[1]);
                    *reinterpret_cast<uint2 *>(&s_mh[s * LDQ + r0]) = uint2{mh[0], mh[1]};
                    *reinterpret_cast<uint2 *>(&s_ml[s * LDQ + r0]) = uint2{ml[0], ml[1]};
                }
            }
        }

        if (more)
            load_rows<TI, N>(cur, t0 + SQ, hi, urow, zrow, dtrow, l, lq, nh);

        // ---- state update of this wave's half: H <- exp(L_last) H +
        // sum_r B_r (w_r X_r)^T, w_r = exp(L_last - L_r) delta_r on this
        // lane's X (exact B is the other operand)
        {
            const float etot = s_etot[0];
            float xw[2][8];
#pragma unroll
            for (int kk = 0; kk < 2; ++kk) {
                const float4 w0 = *reinterpret_cast<const float4 *>(&s_w[32 * kk + 8 * lq]);
                const float4 w1 = *reinterpret_cast<const float4 *>(&s_w[32 * kk + 8 * lq + 4]);
                const float wv[8] = {w0.x, w0.y, w0.z, w0.w, w1.x, w1.y, w1.z, w1.w};
                float xf[8];
                widen8<TI>(xk[kk], xf);
#pragma unroll
                for (int i = 0; i < 8; ++i)
                    xw[kk][i] = xf[i] * wv[i];
            }
            if constexpr (F16) {
                // B as stored on the f16 instruction; the weighted X split into
                // f16 parts under a power-of-two scale per row p (this lane's
                // column), the products scaled back as they join the state
                float m = 0.0f;
#pragma unroll
                for (int kk = 0; kk < 2; ++kk)
#pragma unroll
                    for (int i = 0; i < 8; ++i)
                        m = fmaxf(m, fabsf(xw[kk][i]));
                float wsc, winv;
                pow2_scale(col_max4(m), wsc, winv);
                f16x8_t xwh[2], xwl[2];
#pragma unroll
                for (int kk = 0; kk < 2; ++kk)
                    split_f16(xw[kk], wsc, xwh[kk], xwl[kk]);
#pragma unroll
                for (int q = 0; q < NTH; ++q) {
                    const int nt = NTH * nh + q;
                    f32x4_t acc = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
                    for (int kk = 0; kk < 2; ++kk) {
                        const f16x8_t braw = as_f16x8(*reinterpret_cast<const u32x4 *>(
                            &s_bn[(16 * nt + l16) * LDQ + 32 * kk + 8 * lq]));
                        acc = mma16(braw, xwh[kk], acc);
                        acc = mma16(braw, xwl[kk], acc);
                    }
                    hacc[q] = hacc[q] * etot + acc * winv;
                }
            } else {
                bf16x8_t xwh[2], xwl[2];
#pragma unroll
                for (int kk = 0; kk < 2; ++kk)
                    split_bf16(xw[kk], xwh[kk], xwl[kk]);
#pragma unroll
                for (int q = 0; q < NTH; ++q) {
                    const int nt = NTH * nh + q;
                    f32x4_t acc = hacc[q] * etot;
#pragma unroll
                    for (int kk = 0; kk < 2; ++kk) {
                        const bf16x8_t braw = *reinterpret_cast<const bf16x8_t *>(
                            &s_bn[(16 * nt + l16) * LDQ + 32 * kk + 8 * lq]);
                        acc = mma(braw, xwh[kk], acc);
                        acc = mma(braw, xwl[kk], acc);
                    }
                    hacc[q] = acc;
                }
            }
        }
        __syncthreads();  // M and the C.H halves visible

        // ---- outputs: row tiles st = 2 nh + i, rows s = 16 st + 4 lq + j
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            const int st = 2 * nh + i;
            f32x4_t y = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
            for (int kk = 0; kk <= nh; ++kk) {  // r < 16 st + 16 <= 32 (nh + 1)
                const bf16x8_t mh = *reinterpret_cast<const bf16x8_t *>(
                    &s_mh[(16 * st + l16) * LDQ + 32 * kk + 8 * lq]);
                const bf16x8_t ml = *reinterpret_cast<const bf16x8_t *>(
                    &s_ml[(16 * st + l16) * LDQ + 32 * kk + 8 * lq]);
                if constexpr (F16) {
                    y = mma(mh, xkh[kk], y);
                    y = mma(mh, xkl[kk], y);
                    y = mma(ml, xkh[kk], y);
                } else {
                    y = mma(mh, as_bf16x8(xk[kk]), y);
                    y = mma(ml, as_bf16x8(xk[kk]), y);
                }
            }
            const f32x4_t other = *reinterpret_cast<const f32x4_t *>(&s_x[w][i][l][0]);
            const int s0 = 16 * st + 4 * lq;
            const int t = t0 + s0;
            if (t + 4 > lo && t < hi) {  // some of the 4 steps lie in the sequence
                const float4 eL = *reinterpret_cast<const float4 *>(&s_eL[par][s0]);
                const float el[4] = {eL.x, eL.y, eL.z, eL.w};
                float xv[4];
                unpack_word(xo[i].x, &xv[0], TI{});
                unpack_word(xo[i].y, &xv[2], TI{});
                float o[4];
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const f32x4_t mine = yc[2 + i];
                    const float v = y[j] + el[j] * (mine[j] + other[j]) + Dh * xv[j];
                    o[j] = v * gz[i][j];
                }
                if (t >= lo && t + 4 <= hi) {
                    *reinterpret_cast<uint2 *>(orow + t) = uint2{pack_word(&o[0], TI{}), pack_word(&o[2], TI{})};
                } else {  // a sequence's end: its own columns only
#pragma unroll
                    for (int j = 0; j < 4; ++j)
                        if (t + j >= lo && t + j < hi)
                            orow[t + j] = from_f32<TI>(o[j]);
                }
            }
        }
    }

    if (srow) {
#pragma unroll
        for (int q = 0; q < NTH; ++q)
#pragma unroll
            for (int j = 0; j < 4; ++j)
                srow[16 * (NTH * nh + q) + 4 * lq + j] = from_f32<TS>(hacc[q][j]);
    }
}

template <typename TI, typename TS>
static hipError_t launch_ssd_ts(const ScanArgs &a, hipStream_t stream)
{
    const dim3 grid((unsigned)((int64_t)a.batch * a.nheads * (a.headdim / SPB)));
    switch (a.dstate) {
    case 64: hipLaunchKernelGGL((ssd_kernel<TI, TS, 64>), grid, dim3(STHREADS), 0, stream, a); break;
    case 128: hipLaunchKernelGGL((ssd_kernel<TI, TS, 128>), grid, dim3(STHREADS), 0, stream, a); break;
    default: hipLaunchKernelGGL((ssd_kernel<TI, TS, 256>), grid, dim3(STHREADS), 0, stream, a); break;
    }
    return hipGetLastError();
}

template <typename TI>
static hipError_t launch_ssd_t(const ScanArgs &a, hipStream_t stream)
{
    switch (a.state_dtype) {
    case 0: return launch_ssd_ts<TI, float>(a, stream);
    case 1: return launch_ssd_ts<TI, f16>(a, stream);
    default: return launch_ssd_ts<TI, bf16>(a, stream);
    }
}

bool ssd_supported(const ScanArgs &a)
{
    // B and C are addressed by 32-bit byte offsets from each (request, group)
    // base
    const int64_t span = (int64_t)2 * ((int64_t)(a.dstate - 1) * std::max(a.B_sn, a.C_sn) + a.seqlen);
    return !a.a_per_state && (a.io_dtype == 1 || a.io_dtype == 2) && a.vec &&
           (a.dstate == 64 || a.dstate == 128 || a.dstate == 256) && a.headdim % SPB == 0 &&
           span < ((int64_t)1 << 32);
}

hipError_t launch_ssd(const ScanArgs &a, hipStream_t stream)
{
    return a.io_dtype == 1 ? launch_ssd_t<f16>(a, stream) : launch_ssd_t<bf16>(a, stream);
}

} // namespace ssm
