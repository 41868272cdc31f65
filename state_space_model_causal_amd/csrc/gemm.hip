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
// accumulation.  Both operands are read straight from global memory with
// 128-bit loads: a lane's A operand is 8 consecutive k of one activation row
// and its B operand 8 consecutive k of one weight row, which is how both
// tensors are stored (row-major, k innermost), so no LDS staging is needed;
// the next k step's loads are issued before the current step's MFMAs.  The
// weights, the dominant traffic, stream from HBM once per row block (the
// activations, 2.6 MB at most, stay in L2).  Narrow outputs split K over
// several workgroups, whose float32 partial sums a second kernel adds.
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

// value of output (row, col) to its destination
template <typename T>
__device__ __forceinline__ void gemm_store(const GemmArgs &a, int row, int col, float v)
{
    if (row >= a.M || col >= a.N)
        return;
    if (a.row_slot && a.row_slot[row] < 0)
        return;  // padded request
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

template <typename T>
__global__ __launch_bounds__(256) void gemm_kernel(GemmArgs a)
{
    const int nb = blockIdx.x, ks = blockIdx.y, mb = blockIdx.z;
    const int tid = threadIdx.x, w = tid >> 6, l = tid & 63;
    const int l16 = l & 15, lq = l >> 4;
    const int K = a.K;
    const int nsteps = (K + GK - 1) / GK;
    const int s0 = (int)((int64_t)nsteps * ks / a.splits), s1 = (int)((int64_t)nsteps * (ks + 1) / a.splits);

    // operand rows: activations (clamped to the last row; never stored) and
    // weights (clamped to the last column)
    const T *arow[4];
    const T *wrow[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int m = min(mb * GM + 64 * w + 16 * i + l16, a.M - 1);
        const int n = min(nb * GN + 16 * i + l16, a.N - 1);
        arow[i] = static_cast<const T *>(a.A) + (int64_t)m * a.lda;
        wrow[i] = static_cast<const T *>(a.W) + (int64_t)n * K;
    }
    f32x4_g acc[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j)
            acc[i][j] = f32x4_g{0.0f, 0.0f, 0.0f, 0.0f};

    // Loads go out in batches of GB k-steps, one batch ahead of the MFMAs
    // that use them (the L2 latency is several times one step's MFMA time).
    // K % 8 == 0: a lane's 8 k are all in or all out.
    constexpr int GB = 2;
    auto load = [&](int step, u32x4 (&av)[GB][4], u32x4 (&wv)[GB][4]) {
#pragma unroll
        for (int q = 0; q < GB; ++q) {
            const int k = (step + q) * GK + 8 * lq;
            const bool ok = step + q < s1 && k < K;
            const int kc = ok ? k : 0;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                av[q][i] = *reinterpret_cast<const u32x4 *>(arow[i] + kc);
                wv[q][i] = *reinterpret_cast<const u32x4 *>(wrow[i] + kc);
                if (!ok) {
                    av[q][i] = u32x4{0u, 0u, 0u, 0u};
                    wv[q][i] = u32x4{0u, 0u, 0u, 0u};
                }
            }
        }
    };
    u32x4 av[GB][4], wv[GB][4], an[GB][4], wn[GB][4];
    if (s0 < s1)
        load(s0, av, wv);
    for (int st = s0; st < s1; st += GB) {
        if (st + GB < s1)
            load(st + GB, an, wn);
#pragma unroll
        for (int q = 0; q < GB; ++q)
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int j = 0; j < 4; ++j)
                    acc[i][j] = Mfma<T>::run(av[q][i], wv[q][j], acc[i][j]);
#pragma unroll
        for (int q = 0; q < GB; ++q)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                av[q][i] = an[q][i];
                wv[q][i] = wn[q][i];
            }
    }

    // acc[i][j][e]: row mb*GM + 64 w + 16 i + 4 lq + e, column nb*GN + 16 j + l16
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int row = mb * GM + 64 * w + 16 * i + 4 * lq + e;
                const int col = nb * GN + 16 * j + l16;
                if (a.splits == 1) {
                    gemm_store<T>(a, row, col, acc[i][j][e]);
                } else if (row < a.M && col < a.N) {
                    a.partial[((int64_t)ks * a.M + row) * a.N + col] = acc[i][j][e];
                }
            }
}

// sum of the split-K partials, then the epilogue
template <typename T>
__global__ __launch_bounds__(256) void gemm_reduce_kernel(GemmArgs a)
{
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (i >= (int64_t)a.M * a.N)
        return;
    const int row = (int)(i / a.N), col = (int)(i % a.N);
    const int64_t stride = (int64_t)a.M * a.N;
    // the partials' loads are independent: issue them in groups of 8
    float v = 0.0f;
    int s = 0;
    for (; s + 8 <= a.splits; s += 8) {
        float p[8];
#pragma unroll
        for (int q = 0; q < 8; ++q)
            p[q] = a.partial[(s + q) * stride + i];
#pragma unroll
        for (int q = 0; q < 8; ++q)
            v += p[q];
    }
    for (; s < a.splits; ++s)
        v += a.partial[s * stride + i];
    gemm_store<T>(a, row, col, v);
}

template <typename T>
static hipError_t launch_gemm_t(const GemmArgs &a, hipStream_t stream)
{
    const dim3 grid((unsigned)((a.N + GN - 1) / GN), (unsigned)a.splits, (unsigned)((a.M + GM - 1) / GM));
    hipLaunchKernelGGL((gemm_kernel<T>), grid, dim3(256), 0, stream, a);
    if (a.splits > 1) {
        const int64_t n = (int64_t)a.M * a.N;
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
__global__ __launch_bounds__(256) void rmsnorm_kernel(const T *__restrict__ x, const float *__restrict__ wt,
                                                      T *__restrict__ out, int M, int D, float eps)
{
    __shared__ float red[4];
    const int row = blockIdx.x, tid = threadIdx.x;
    const T *xr = x + (int64_t)row * D;
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
        out[(int64_t)row * D + i] = from_f32<T>(to_f32(xr[i]) * inv * wt[i]);
}

hipError_t launch_rmsnorm(const void *x, const float *w, void *out, int M, int D, float eps, int dtype,
                          hipStream_t stream)
{
    if (dtype == 1)
        hipLaunchKernelGGL((rmsnorm_kernel<f16>), dim3(M), dim3(256), 0, stream, static_cast<const f16 *>(x), w,
                           static_cast<f16 *>(out), M, D, eps);
    else
        hipLaunchKernelGGL((rmsnorm_kernel<bf16>), dim3(M), dim3(256), 0, stream, static_cast<const bf16 *>(x), w,
                           static_cast<bf16 *>(out), M, D, eps);
    return hipGetLastError();
}

} // namespace ssm
