// ssm_device.hpp -- device-side helpers shared by the gfx950 kernels:
// storage conversions, 128-bit vector access, the float32 transcendental
// pieces of the selective SSM (softplus of the step size, SiLU gate, exp of
// the decay), DPP lane moves and the XCD-aware block order.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace ssm {

// ---------------------------------------------------------------- storage
// Three storage formats; arithmetic is always float32.
using f16 = _Float16;
struct bf16 {
    uint16_t bits;
};

template <typename T> struct StorageSize;
template <> struct StorageSize<float> { static constexpr int value = 4; };
template <> struct StorageSize<f16> { static constexpr int value = 2; };
template <> struct StorageSize<bf16> { static constexpr int value = 2; };

__device__ __forceinline__ float to_f32(float v) { return v; }
__device__ __forceinline__ float to_f32(f16 v) { return (float)v; }
__device__ __forceinline__ float to_f32(bf16 v) { return __uint_as_float((uint32_t)v.bits << 16); }

template <typename T> __device__ __forceinline__ T from_f32(float v);
template <> __device__ __forceinline__ float from_f32<float>(float v) { return v; }
// v_cvt_f16_f32 rounds to nearest even in the default mode.
template <> __device__ __forceinline__ f16 from_f32<f16>(float v) { return (f16)v; }
// Round to nearest even: gfx950 converts in hardware (v_cvt_pk_bf16_f32,
// which keeps NaNs NaN and, with float32 denormals on, rounds denormals too).
template <> __device__ __forceinline__ bf16 from_f32<bf16>(float v)
{
    bf16 r;
    r.bits = __builtin_bit_cast(uint16_t, (__bf16)v);
    return r;
}

// Two floats rounded to bf16 in one conversion, a in the low half.
__device__ __forceinline__ uint32_t pk_bf16(float a, float b)
{
    typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
    const bf16x2_t v = {(__bf16)a, (__bf16)b};
    return __builtin_bit_cast(uint32_t, v);
}

// Unpack one 32-bit word holding 1 (f32) or 2 (f16/bf16) elements.
__device__ __forceinline__ void unpack_word(uint32_t w, float *dst, float) { dst[0] = __uint_as_float(w); }
__device__ __forceinline__ void unpack_word(uint32_t w, float *dst, f16)
{
    union { uint32_t u; f16 h[2]; } c;
    c.u = w;
    dst[0] = (float)c.h[0];
    dst[1] = (float)c.h[1];
}
__device__ __forceinline__ void unpack_word(uint32_t w, float *dst, bf16)
{
    dst[0] = __uint_as_float(w << 16);
    dst[1] = __uint_as_float(w & 0xffff0000u);
}

__device__ __forceinline__ uint32_t pack_word(const float *src, float) { return __float_as_uint(src[0]); }
__device__ __forceinline__ uint32_t pack_word(const float *src, f16)
{
    union { uint32_t u; f16 h[2]; } c;
    c.h[0] = (f16)src[0];
    c.h[1] = (f16)src[1];
    return c.u;
}
__device__ __forceinline__ uint32_t pack_word(const float *src, bf16) { return pk_bf16(src[0], src[1]); }

template <typename T> struct PerWord { static constexpr int value = 4 / StorageSize<T>::value; };

// 128-bit access unit (a native vector type, usable with the nontemporal
// builtins).
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// Load K consecutive elements (K * sizeof(T) a multiple of 16 bytes, p 16-byte
// aligned) with 128-bit loads and widen them to float.
template <typename T, int K>
__device__ __forceinline__ void load_vec(const T *__restrict__ p, float (&dst)[K])
{
    constexpr int PW = PerWord<T>::value;
    constexpr int NV = K * StorageSize<T>::value / 16;
    static_assert(NV * 16 == K * StorageSize<T>::value, "K elements must fill whole 16-byte vectors");
    const u32x4 *q = reinterpret_cast<const u32x4 *>(p);
#pragma unroll
    for (int v = 0; v < NV; ++v) {
        u32x4 w = __builtin_nontemporal_load(q + v);
        unpack_word(w.x, &dst[(4 * v + 0) * PW], T{});
        unpack_word(w.y, &dst[(4 * v + 1) * PW], T{});
        unpack_word(w.z, &dst[(4 * v + 2) * PW], T{});
        unpack_word(w.w, &dst[(4 * v + 3) * PW], T{});
    }
}

// Same, with ordinary (cached) loads: for data read by several workgroups.
template <typename T, int K>
__device__ __forceinline__ void load_vec_cached(const T *__restrict__ p, float (&dst)[K])
{
    constexpr int PW = PerWord<T>::value;
    constexpr int NV = K * StorageSize<T>::value / 16;
    static_assert(NV * 16 == K * StorageSize<T>::value, "K elements must fill whole 16-byte vectors");
    const u32x4 *q = reinterpret_cast<const u32x4 *>(p);
#pragma unroll
    for (int v = 0; v < NV; ++v) {
        u32x4 w = q[v];
        unpack_word(w.x, &dst[(4 * v + 0) * PW], T{});
        unpack_word(w.y, &dst[(4 * v + 1) * PW], T{});
        unpack_word(w.z, &dst[(4 * v + 2) * PW], T{});
        unpack_word(w.w, &dst[(4 * v + 3) * PW], T{});
    }
}

template <typename T, int K>
__device__ __forceinline__ void store_vec(T *__restrict__ p, const float (&src)[K])
{
    constexpr int PW = PerWord<T>::value;
    constexpr int NV = K * StorageSize<T>::value / 16;
    static_assert(NV * 16 == K * StorageSize<T>::value, "K elements must fill whole 16-byte vectors");
    u32x4 *q = reinterpret_cast<u32x4 *>(p);
#pragma unroll
    for (int v = 0; v < NV; ++v) {
        u32x4 w;
        w.x = pack_word(&src[(4 * v + 0) * PW], T{});
        w.y = pack_word(&src[(4 * v + 1) * PW], T{});
        w.z = pack_word(&src[(4 * v + 2) * PW], T{});
        w.w = pack_word(&src[(4 * v + 3) * PW], T{});
        __builtin_nontemporal_store(w, q + v);
    }
}

template <typename T, int K>
__device__ __forceinline__ void store_vec_cached(T *__restrict__ p, const float (&src)[K])
{
    constexpr int PW = PerWord<T>::value;
    constexpr int NV = K * StorageSize<T>::value / 16;
    static_assert(NV * 16 == K * StorageSize<T>::value, "K elements must fill whole 16-byte vectors");
    u32x4 *q = reinterpret_cast<u32x4 *>(p);
#pragma unroll
    for (int v = 0; v < NV; ++v) {
        u32x4 w;
        w.x = pack_word(&src[(4 * v + 0) * PW], T{});
        w.y = pack_word(&src[(4 * v + 1) * PW], T{});
        w.z = pack_word(&src[(4 * v + 2) * PW], T{});
        w.w = pack_word(&src[(4 * v + 3) * PW], T{});
        q[v] = w;
    }
}

// ------------------------------------------------------------ math pieces
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// 2^x on the hardware exponential unit (v_exp_f32).
__device__ __forceinline__ float exp2_hw(float x) { return __builtin_amdgcn_exp2f(x); }
// log2(x) on the hardware unit (v_log_f32).
__device__ __forceinline__ float log2_hw(float x) { return __builtin_amdgcn_logf(x); }
__device__ __forceinline__ float rcp_hw(float x) { return __builtin_amdgcn_rcpf(x); }

// log1p(e) for e in [0, 1], accurate to a few ulp.  w = 1 + e is rounded and
// c = e - (w - 1) is its rounding error, exactly (Dekker's Fast2Sum, 1971:
// 1 >= e).  Then log1p(e) = log(w) + log(1 + c/w), and since |c| <= 2^-24
// and w is in [1, 2], log(1 + c/w) = c up to 2^-24 * e, about an ulp of the
// result at most.  When w rounds to 1 the result is c = e.  One
// transcendental, no division.
__device__ __forceinline__ float log1p_unit(float e)
{
    const float w = 1.0f + e;
    const float c = e - (w - 1.0f);
    return fmaf(log2_hw(w), kLn2, c);
}

// softplus(v) = log(1 + e^v) = max(v, 0) + log1p(e^{-|v|}).  Branch-free
// and without a cutoff: for v > 16.7 the second term is below half an ulp of
// v, so the sum rounds to v by itself; v = +inf gives inf, v = -inf gives 0.
__device__ __forceinline__ float softplus_f32(float v)
{
    const float e = exp2_hw(-fabsf(v) * kLog2e);
    return fmaxf(v, 0.0f) + log1p_unit(e);
}

// SiLU(v) = v / (1 + e^{-v}).
__device__ __forceinline__ float silu_f32(float v)
{
    return v * rcp_hw(1.0f + exp2_hw(-v * kLog2e));
}

// ---------------------------------------------------------------- lane moves
// DPP controls (GCN/CDNA encoding).
enum : int {
    DPP_ROW_SHR1 = 0x111,
    DPP_ROW_SHR2 = 0x112,
    DPP_ROW_SHR4 = 0x114,
    DPP_ROW_SHR8 = 0x118,
    DPP_ROW_ROR1 = 0x121,
    DPP_QUAD_XOR1 = 0xB1,  // quad_perm [1,0,3,2]
    DPP_QUAD_XOR2 = 0x4E,  // quad_perm [2,3,0,1]
    DPP_QUAD_NEXT = 0xF9,  // quad_perm [1,2,3,3]: lane i of a quad reads lane min(i+1, 3)
    DPP_ROW_BCAST15 = 0x142,  // lane 15 of each row to every lane of the next row
    DPP_ROW_BCAST31 = 0x143,  // lane 31 to every lane of rows 2 and 3
    DPP_WAVE_SHR1 = 0x138,    // lane i reads lane i-1 of the wave (lane 0: bound_ctrl)
};

// Read `src` from another lane of the same 16-lane row; lanes whose source
// falls outside the row receive `old`.
template <int CTRL>
__device__ __forceinline__ float dpp_move(float old, float src)
{
    return __int_as_float(__builtin_amdgcn_update_dpp(__float_as_int(old), __float_as_int(src), CTRL,
                                                      0xf, 0xf, false));
}

// Same, but lanes whose source falls outside the row read 0 (bound_ctrl).  No
// "old" operand has to be materialised, so the move can fold into the VALU
// instruction that consumes it.
template <int CTRL>
__device__ __forceinline__ float dpp_move_zero(float src)
{
    return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(src), CTRL, 0xf, 0xf, true));
}

// Same, on raw 32-bit values.
template <int CTRL>
__device__ __forceinline__ uint32_t dpp_move_bits(uint32_t src)
{
    return (uint32_t)__builtin_amdgcn_mov_dpp((int)src, CTRL, 0xf, 0xf, true);
}

// Inclusive prefix sum over the 64 lanes of a wave: a Hillis-Steele scan in
// each 16-lane row, then the row totals added by the two row broadcasts
// (rows 1 and 3 take the total of the row before; rows 2 and 3 that of
// rows 0-1).  No LDS round trip.
__device__ __forceinline__ float wave_prefix_sum(float v)
{
    v += dpp_move_zero<DPP_ROW_SHR1>(v);
    v += dpp_move_zero<DPP_ROW_SHR2>(v);
    v += dpp_move_zero<DPP_ROW_SHR4>(v);
    v += dpp_move_zero<DPP_ROW_SHR8>(v);
    v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), DPP_ROW_BCAST15, 0xa, 0xf, false));
    v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), DPP_ROW_BCAST31, 0xc, 0xf, false));
    return v;
}

__device__ __forceinline__ float lane_value(float v, int lane)
{
    return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), lane));
}

// ---------------------------------------------------------------- block order
// MI355X hands consecutive workgroups to its 8 XCDs round-robin.  Renumber so
// that each XCD receives one contiguous range of logical blocks: neighbours
// that share operands (B/C of one request, one head's parameters) then share
// one XCD's L2.
__device__ __forceinline__ uint32_t xcd_block_order(uint32_t i, uint32_t nblocks)
{
    constexpr uint32_t kXcd = 8;
    const uint32_t xcd = i % kXcd, local = i / kXcd;
    const uint32_t per = nblocks / kXcd, rem = nblocks % kXcd;
    return xcd < rem ? xcd * (per + 1) + local : rem * (per + 1) + (xcd - rem) * per + local;
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

} // namespace ssm
