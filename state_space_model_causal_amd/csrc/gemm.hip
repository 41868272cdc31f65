// gemm.hip -- the projections around the selective SSM in one Mamba-1 decode
// layer, and its RMSNorm, on gfx950.
//
// The Mamba-2.8B model of "feat(llama.cu): 适配 mamba 模型" (InfiniLM-Rust PR
// #48, sections 2.1-2.2) runs the conv and scan operators between linear
// projections of each token's hidden state.  At decode every projection is a
// skinny product: out[M, N] = act[M, K] . W[N, K]^T with M = the number of
// requests (245 on the pages' concurrency test), K and N the layer widths.
//
// Kernel: one 256-lane workgroup per (64 output columns, slice of K, 256
// rows).  Wave w owns rows [64 w, 64 w + 64) of the block and all 64
// columns: 4 x 4 tiles of v_mfma_f32_16x16x32_{f16,bf16}, float32
// accumulation.  K is walked in batches of 64: each batch's activation tile
// (256 rows x 64 k) and weight tile (64 rows x 64 k) are loaded once per
// workgroup with coalesced 128-bit loads (consecutive lanes, consecutive 16
// bytes of a row) and staged in LDS, from where each wave reads its MFMA
// operands (8 consecutive k of one row: row-major, k innermost is the operand
// order).  The next batch's loads are in flight during the current batch's
// MFMAs.  The weights, the dominant traffic, stream from
// HBM once per row block (the activations, 2.6 MB at most, stay in L2).
// Narrow outputs split K over several workgroups, whose float32 partial sums
// a second kernel adds.
//
// Epilogue: output columns go to up to three destinations (column segments,
// e.g. the x and z halves of in_proj), optionally added to a residual, rows
// of padded requests left untouched.
#include "ssm_device.hpp"
#include "ssm_kernels.hpp"

namespace ssm {

namespace {
typedef __bf16 bf16x8_g __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8_g __attribute__((ext_vector_type(8)));
typedef float f32x4_g __attribute__((ext_vector_type(4)));
constexpr int GM = 256;  // rows per workgroup
constexpr int GN = 64;   // columns per workgroup
constexpr int GK = 32;   // k per MFMA step

template <typename T> struct Mfma;
template <> struct Mfma<f16> {
    static __device__ __forceinline__ f32x4_g run(u32x4 a, u32x4 b, f32x4_g c)
    {
        return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8_g, a),
                                                     __builtin_bit_cast(f16x8_g, b), c, 0, 0, 0);
    }
};
template <> struct Mfma<bf16> {
    static __device__ __forceinline__ f32x4_g run(u32x4 a, u32x4 b, f32x4_g c)
    {
        return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_g, a),
                                                      __builtin_bit_cast(bf16x8_g, b), c, 0, 0, 0);
    }
};
} // namespace

// value of output (row, col) to its destination (the general path)
template <typename T>
__device__ __forceinline__ void gemm_store(const GemmArgs &a, int row, int col, float v)
{
    if (col >= a.N)
        return;
#pragma unroll
    for (int sgi = 0; sgi < 3; ++sgi) {
        if (sgi < a.nseg && col >= a.seg[sgi].col0 && col < a.seg[sgi].col0 + a.seg[sgi].ncols) {
            T *dst = static_cast<T *>(a.seg[sgi].ptr) + (int64_t)row * a.seg[sgi].ld + (col - a.seg[sgi].col0);
            if (a.residual)
                v += to_f32(static_cast<const T *>(a.residual)[(int64_t)row * a.ld_residual + col]);
            *dst = from_f32<T>(v);
        }
    }
}

// outputs (row, col .. col + 3) to their destination: one 8-byte store (and
// one 8-byte residual load) when the four columns share a segment and the
// addresses are aligned, else element by element.  Rows of padded requests
// are left untouched.
template <typename T>
__device__ __forceinline__ void gemm_store4(const GemmArgs &a, int row, int col, f32x4_g v)
{
    if (row >= a.M || col >= a.N)
        return;
    if (a.row_slot && a.row_slot[row] < 0)
        return;
#pragma unroll
    for (int sgi = 0; sgi < 3; ++sgi) {
        const GemmSeg &sg = a.seg[sgi];
        if (sgi < a.nseg && col >= sg.col0 && col + 3 < sg.col0 + sg.ncols) {
            T *dst = static_cast<T *>(sg.ptr) + (int64_t)row * sg.ld + (col - sg.col0);
            const T *res = a.residual ? static_cast<const T *>(a.residual) + (int64_t)row * a.ld_residual + col
                                      : nullptr;
            if (((reinterpret_cast<uintptr_t>(dst) | reinterpret_cast<uintptr_t>(res)) & 7) == 0) {
                float x[4] = {v[0], v[1], v[2], v[3]};
                if (res) {
                    const uint2 r = *reinterpret_cast<const uint2 *>(res);
                    float rf[4];
                    unpack_word(r.x, rf, T{});
                    unpack_word(r.y, rf + 2, T{});
#pragma unroll
                    for (int e = 0; e < 4; ++e)
                        x[e] += rf[e];
                }
                *reinterpret_cast<uint2 *>(dst) = uint2{pack_word(x, T{}), pack_word(x + 2, T{})};
                return;
            }
        }
    }
#pragma unroll
    for (int e = 0; e < 4; ++e)
        gemm_store<T>(a, row, col + e, v[e]);
}

template <typename T>
__global__ __launch_bounds__(256) void gemm_kernel(GemmArgs a)
{
    // one k batch of both operands in LDS: the activation tile (GM rows) and
    // the weight tile (GN rows), KBK k each, row stride padded by 16 B
    constexpr int KB = 2;            // MFMA k-steps per batch
    constexpr int KBK = KB * GK;     // k per batch
    constexpr int LDK = KBK + 8;     // elements per LDS row
    constexpr int CPR = KBK / 8;     // 16-byte chunks per row
    constexpr int ACH = GM * CPR / 256, WCH = GN * CPR / 256;  // chunks per thread
    __shared__ __align__(16) T s_a[GM * LDK];
    __shared__ __align__(16) T s_w[GN * LDK];

    const int nb = blockIdx.x, ks = blockIdx.y, mb = blockIdx.z;
    const int tid = threadIdx.x, w = tid >> 6, l = tid & 63;
    const int l16 = l & 15, lq = l >> 4;
    const int K = a.K;
    const int nbatch = (K + KBK - 1) / KBK;
    const int b0 = (int)((int64_t)nbatch * ks / a.splits), b1 = (int)((int64_t)nbatch * (ks + 1) / a.splits);

    // chunk c = tid + 256 q of a tile: row c / CPR, k offset 8 (c % CPR);
    // consecutive threads read consecutive 16 B of a row
    const T *asrc[ACH];
    const T *wsrc[WCH];
    int adst[ACH], wdst[WCH];
    const int kofs = 8 * (tid % CPR);  // the same for every chunk of this thread
#pragma unroll
    for (int q = 0; q < ACH; ++q) {
        const int c = tid + 256 * q, r = c / CPR;
        const int m = min(mb * GM + r, a.M - 1);  // clamped rows are never stored
        asrc[q] = static_cast<const T *>(a.A) + (int64_t)m * a.lda + kofs;
        adst[q] = r * LDK + kofs;
    }
#pragma unroll
    for (int q = 0; q < WCH; ++q) {
        const int c = tid + 256 * q, r = c / CPR;
        const int n = min(nb * GN + r, a.N - 1);
        wsrc[q] = static_cast<const T *>(a.W) + (int64_t)n * a.ldw + kofs;
        wdst[q] = r * LDK + kofs;
    }

    f32x4_g acc[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j)
            acc[i][j] = f32x4_g{0.0f, 0.0f, 0.0f, 0.0f};

    // K % 8 == 0: an 8-element chunk is all in or all out; out of range it
    // is loaded from the row's first chunk (in bounds) and zeroed when it is
    // staged.  Zeroing at staging time, not right after the load, keeps the
    // loads in flight during the MFMAs of the batch before.
    u32x4 ar[ACH], wr[WCH];
    bool in_range = true;
    auto load = [&](int batch) {
        in_range = batch * KBK + kofs < K;
        const int off = in_range ? batch * KBK : -kofs;
#pragma unroll
        for (int q = 0; q < ACH; ++q)
            ar[q] = *reinterpret_cast<const u32x4 *>(asrc[q] + off);
#pragma unroll
        for (int q = 0; q < WCH; ++q)
            wr[q] = *reinterpret_cast<const u32x4 *>(wsrc[q] + off);
    };
    auto stage = [&]() {
        const u32x4 zero{0u, 0u, 0u, 0u};
#pragma unroll
        for (int q = 0; q < ACH; ++q)
            *reinterpret_cast<u32x4 *>(&s_a[adst[q]]) = in_range ? ar[q] : zero;
#pragma unroll
        for (int q = 0; q < WCH; ++q)
            *reinterpret_cast<u32x4 *>(&s_w[wdst[q]]) = in_range ? wr[q] : zero;
    };

    if (b0 < b1)
        load(b0);
    for (int bt = b0; bt < b1; ++bt) {
        stage();
        __syncthreads();
        if (bt + 1 < b1)
            load(bt + 1);  // in flight during this batch's MFMAs
#pragma unroll
        for (int q = 0; q < KB; ++q) {
            u32x4 av[4], bv[4];
#pragma unroll
            for (int i = 0; i < 4; ++i)
                av[i] = *reinterpret_cast<const u32x4 *>(&s_a[(64 * w + 16 * i + l16) * LDK + q * GK + 8 * lq]);
#pragma unroll
            for (int j = 0; j < 4; ++j)
                bv[j] = *reinterpret_cast<const u32x4 *>(&s_w[(16 * j + l16) * LDK + q * GK + 8 * lq]);
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int j = 0; j < 4; ++j)
                    acc[i][j] = Mfma<T>::run(bv[j], av[i], acc[i][j]);
        }
        __syncthreads();  // the tiles are restaged next batch
    }

    // The products are taken as W . act^T, so acc[i][j][e] is output row
    // mb*GM + 64 w + 16 i + l16, column nb*GN + 16 j + 4 lq + e: each lane
    // holds four consecutive columns of one row.
    const int col0 = nb * GN + 4 * lq;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int row = mb * GM + 64 * w + 16 * i + l16;
        if (a.splits == 1) {
#pragma unroll
            for (int j = 0; j < 4; ++j)
                gemm_store4<T>(a, row, col0 + 16 * j, acc[i][j]);
        } else if (row < a.M) {
            // float32 partials, row-major per split: 16-byte stores when N
            // keeps them aligned
            float *prow = a.partial + ((int64_t)ks * a.M + row) * a.N;
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int col = col0 + 16 * j;
                if ((a.N & 3) == 0 && col < a.N) {
                    *reinterpret_cast<f32x4_g *>(prow + col) = acc[i][j];
                } else {
#pragma unroll
                    for (int e = 0; e < 4; ++e)
                        if (col + e < a.N)
                            prow[col + e] = acc[i][j][e];
                }
            }
        }
    }
}

// sum of the split-K partials, then the epilogue: each thread takes four
// consecutive columns of one row (N is padded to a multiple of 4 in the
// indexing; columns past N are not read)
template <typename T>
__global__ __launch_bounds__(256) void gemm_reduce_kernel(GemmArgs a)
{
    const int nq = (a.N + 3) >> 2;  // column quads per row
    const int64_t q = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (q >= (int64_t)a.M * nq)
        return;
    const int row = (int)(q / nq), col = 4 * (int)(q % nq);
    const int64_t stride = (int64_t)a.M * a.N;
    const float *p = a.partial + (int64_t)row * a.N + col;
    f32x4_g v{0.0f, 0.0f, 0.0f, 0.0f};
    if ((a.N & 3) == 0) {
        // the partials' loads are independent: issue them in groups of 4
        int s = 0;
        for (; s + 4 <= a.splits; s += 4) {
            f32x4_g t[4];
#pragma unroll
            for (int u = 0; u < 4; ++u)
                t[u] = *reinterpret_cast<const f32x4_g *>(p + (s + u) * stride);
#pragma unroll
            for (int u = 0; u < 4; ++u)
                v += t[u];
        }
        for (; s < a.splits; ++s)
            v += *reinterpret_cast<const f32x4_g *>(p + s * stride);
    } else {
        for (int s = 0; s < a.splits; ++s)
#pragma unroll
            for (int e = 0; e < 4; ++e)
                if (col + e < a.N)
                    v[e] += p[s * stride + e];
    }
    gemm_store4<T>(a, row, col, v);
}

template <typename T>
static hipError_t launch_gemm_t(const GemmArgs &a, hipStream_t stream)
{
    const dim3 grid((unsigned)((a.N + GN - 1) / GN), (unsigned)a.splits, (unsigned)((a.M + GM - 1) / GM));
    hipLaunchKernelGGL((gemm_kernel<T>), grid, dim3(256), 0, stream, a);
    if (a.splits > 1) {
        const int64_t n = (int64_t)a.M * ((a.N + 3) / 4);
        hipLaunchKernelGGL((gemm_reduce_kernel<T>), dim3((unsigned)((n + 255) / 256)), dim3(256), 0, stream, a);
    }
    return hipGetLastError();
}

hipError_t launch_gemm(const GemmArgs &a, hipStream_t stream)
{
    return a.dtype == 1 ? launch_gemm_t<f16>(a, stream) : launch_gemm_t<bf16>(a, stream);
}

// RMSNorm of each row: out = x / sqrt(mean(x^2) + eps) * weight (weight in
// float32), one workgroup per row.
template <typename T>
__global__ __launch_bounds__(256) void rmsnorm_kernel(const T *__restrict__ x, int64_t ldx,
                                                      const float *__restrict__ wt, T *__restrict__ out,
                                                      int64_t ldo, int M, int D, float eps)
{
    __shared__ float red[4];
    const int row = blockIdx.x, tid = threadIdx.x;
    const T *xr = x + row * ldx;
    float ss = 0.0f;
    for (int i = tid; i < D; i += 256) {
        const float v = to_f32(xr[i]);
        ss = fmaf(v, v, ss);
    }
    for (int o = 32; o > 0; o >>= 1)
        ss += __shfl_xor(ss, o, 64);
    if ((tid & 63) == 0)
        red[tid >> 6] = ss;
    __syncthreads();
    const float tot = red[0] + red[1] + red[2] + red[3];
    const float inv = 1.0f / sqrtf(tot / (float)D + eps);
    for (int i = tid; i < D; i += 256)
        out[row * ldo + i] = from_f32<T>(to_f32(xr[i]) * inv * wt[i]);
}

hipError_t launch_rmsnorm(const void *x, int64_t ldx, const float *w, void *out, int64_t ldo, int M, int D,
                          float eps, int dtype, hipStream_t stream)
{
    if (dtype == 1)
        hipLaunchKernelGGL((rmsnorm_kernel<f16>), dim3(M), dim3(256), 0, stream, static_cast<const f16 *>(x), ldx,
                           w, static_cast<f16 *>(out), ldo, M, D, eps);
    else
        hipLaunchKernelGGL((rmsnorm_kernel<bf16>), dim3(M), dim3(256), 0, stream, static_cast<const bf16 *>(x),
                           ldx, w, static_cast<bf16 *>(out), ldo, M, D, eps);
    return hipGetLastError();
}

} // namespace ssm
