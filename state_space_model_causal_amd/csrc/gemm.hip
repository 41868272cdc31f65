// gemm.hip -- the projections around the selective SSM in one Mamba-1 decode
// layer, and its RMSNorm, on gfx950.
//
// The Mamba-2.8B model of "feat(llama.cu): 适配 mamba 模型" (InfiniLM-Rust PR
// #48, sections 2.1-2.2) runs the conv and scan operators between linear
// projections of each token's hidden state.  At decode every projection is a
// skinny product: out[M, N] = act[M, K] . W[N, K]^T with M = the number of
// requests (245 on the pages' concurrency test), K and N the layer widths.
//
// Kernel: one workgroup of 4 CW waves per (64 CW output columns, 4 WR rows,
// slice of K), WR = 64, 32 or 16 rows per wave and CW = 1 or 2 column groups.
// Wave w owns rows [WR (w % 4), + WR) of the block and the 64 columns of
// group w / 4: WR/16 x 4 tiles of v_mfma_f32_16x16x32_{f16,bf16}, float32
// accumulation.  K is walked in batches of 64: each batch's activation tile
// (4 WR rows x 64 k) and weight tile (64 CW rows x 64 k) are copied once per
// workgroup from global memory straight into LDS by global_load_lds_dwordx4
// (each wave instruction fills 1 KB, 8 rows of 128 bytes), from where each
// wave reads its MFMA operands (8 consecutive k of one row: row-major, k
// innermost is the operand order).  A ring of three LDS stages keeps two
// batches in flight during the MFMAs.  A wave reads all of a batch's operands
// before it issues the next copy: the compiler waits for every copy in flight
// before an LDS read that may touch one, and only for copies into other
// stages can it tell that none does.  The weights,
// the dominant traffic, stream from HBM once (the row blocks of one column
// tile run on one XCD and share its L2; the activations, 2.6 MB at most, stay
// in L2).
// Narrow outputs split K over several workgroups, whose float32 partial sums
// a second kernel adds.  The plan (rows per wave, columns per workgroup,
// splits) comes from plan_gemm's traffic model.
//
// Epilogue: output columns go to up to three destinations (column segments,
// e.g. the x and z halves of in_proj), optionally added to a residual, rows
// of padded requests left untouched.
#include <algorithm>
#include <cmath>
#include <type_traits>

#include "ssm_device.hpp"
#include "ssm_kernels.hpp"

namespace ssm {

namespace {
typedef __bf16 bf16x8_g __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8_g __attribute__((ext_vector_type(8)));
typedef float f32x4_g __attribute__((ext_vector_type(4)));
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

// Workgroup of 4 x CW waves for a tile of 4 WR rows x 64 CW columns and one
// slice of K; wave w owns rows [WR (w % 4), + WR) and columns
// [64 (w / 4), + 64).  Each batch of 64 k is copied from global memory
// straight into LDS (global_load_lds_dwordx4: no registers, no LDS stores
// of its own), in a ring of three stages so that two batches are in flight
// while one is multiplied.  A row of a stage is 128 bytes, its 16-byte
// chunk c stored at position c ^ (row & 7): an operand read (one chunk of 16
// consecutive rows) spreads over eight bank groups instead of one.
typedef __attribute__((address_space(3))) void lds_void_t;
template <typename T, int WR, int CW>
__global__ __launch_bounds__(256 * CW) void gemm_kernel(GemmArgs a)
{
    constexpr int NW = 4 * CW;       // waves
    constexpr int GMR = 4 * WR;      // rows per workgroup
    constexpr int GNC = GN * CW;     // columns per workgroup
    constexpr int RT = WR / 16;      // 16-row MFMA tiles per wave
    constexpr int KB = 2;            // MFMA k-steps per batch
    constexpr int KBK = KB * GK;     // k per batch (64)
    constexpr int ABLK = GMR * 8 / 64, WBLK = GNC * 8 / 64;  // 1 KB blocks per tile
    constexpr int AJ = ABLK / NW, WJ = WBLK / NW;             // DMA instructions per wave and tile
    static_assert(AJ * NW == ABLK && WJ * NW == WBLK, "tiles must split evenly over the waves");
    static_assert(sizeof(T) == 2, "2-byte operands");
    __shared__ __align__(16) T sA0[GMR * KBK];
    __shared__ __align__(16) T sA1[GMR * KBK];
    __shared__ __align__(16) T sA2[GMR * KBK];
    __shared__ __align__(16) T sW0[GNC * KBK];
    __shared__ __align__(16) T sW1[GNC * KBK];
    __shared__ __align__(16) T sW2[GNC * KBK];

    const int ncol = (a.N + GNC - 1) / GNC, nrow = (a.M + GMR - 1) / GMR;
    const uint32_t lb = xcd_block_order(blockIdx.x, gridDim.x);
    const int ks = (int)(lb % (uint32_t)a.splits);
    const int mb = (int)((lb / (uint32_t)a.splits) % (uint32_t)nrow);
    const int nb = (int)(lb / ((uint32_t)a.splits * (uint32_t)nrow));
    if (nb >= ncol)
        return;
    const int tid = threadIdx.x, w = tid >> 6, l = tid & 63;
    const int wm = w & 3, wn = w >> 2;
    const int l16 = l & 15, lq = l >> 4;
    const int K = a.K;
    const int nbatch = (K + KBK - 1) / KBK;
    const int b0 = (int)((int64_t)nbatch * ks / a.splits), b1 = (int)((int64_t)nbatch * (ks + 1) / a.splits);

    // lane l of DMA block bI: row bI*8 + l/8, stored chunk position l%8,
    // which holds global chunk (l%8) ^ (row & 7)
    const T *asrc[AJ];
    const T *wsrc[WJ];
    int achk[AJ], wchk[WJ];
#pragma unroll
    for (int j = 0; j < AJ; ++j) {
        const int r = (j * NW + w) * 8 + (l >> 3);
        achk[j] = 8 * ((l & 7) ^ (r & 7));
        asrc[j] = static_cast<const T *>(a.A) + (int64_t)min(mb * GMR + r, a.M - 1) * a.lda;
    }
#pragma unroll
    for (int j = 0; j < WJ; ++j) {
        const int r = (j * NW + w) * 8 + (l >> 3);
        wchk[j] = 8 * ((l & 7) ^ (r & 7));
        wsrc[j] = static_cast<const T *>(a.W) + (int64_t)min(nb * GNC + r, a.N - 1) * a.ldw;
    }
    // the DMA written out: the compiler then does not count it among the LDS
    // writes it must drain before every LDS read; its completion is waited
    // for explicitly (vmcnt) before each batch's barrier
    auto dma16 = [&](const T *g, T *ldst) {
        __builtin_amdgcn_global_load_lds((const void *)g, (lds_void_t *)ldst, 16, 0, 0);
    };
    auto issue = [&](int batch, T *sA, T *sW) {
#pragma unroll
        for (int j = 0; j < AJ; ++j) {
            const int k = batch * KBK + achk[j];
            dma16(asrc[j] + (k < K ? k : 0), sA + (j * NW + w) * 512);
        }
#pragma unroll
        for (int j = 0; j < WJ; ++j) {
            const int k = batch * KBK + wchk[j];
            dma16(wsrc[j] + (k < K ? k : 0), sW + (j * NW + w) * 512);
        }
    };

    f32x4_g acc[RT][4];
#pragma unroll
    for (int i = 0; i < RT; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j)
            acc[i][j] = f32x4_g{0.0f, 0.0f, 0.0f, 0.0f};

    auto step = [&](int bt, const T *sA, const T *sW, T *nA, T *nW) {
        if (bt + 1 < b1)
            __builtin_amdgcn_s_waitcnt(0x0F70 | (AJ + WJ));  // batch bt has landed (bt + 1 may be in flight)
        else
            __builtin_amdgcn_s_waitcnt(0x0F70);
        __builtin_amdgcn_s_barrier();
        // every operand of this batch read out of LDS before the DMA of batch
        // bt + 2 is issued: the compiler then finds no DMA in flight to an
        // LDS array these reads may touch, and adds no wait of its own
        const bool partial = (bt + 1) * KBK > K;
        const u32x4 zero{0u, 0u, 0u, 0u};
        u32x4 av[KB][RT], bv[KB][4];
#pragma unroll
        for (int q = 0; q < KB; ++q) {
            const int kc = 4 * q + lq;  // 16-byte chunk of the batch
            const bool kin = !partial || bt * KBK + 8 * kc < K;
#pragma unroll
            for (int i = 0; i < RT; ++i) {
                const int row = WR * wm + 16 * i + l16;
                av[q][i] = *reinterpret_cast<const u32x4 *>(&sA[row * KBK + 8 * (kc ^ (row & 7))]);
                if (partial)
                    av[q][i] = kin ? av[q][i] : zero;
            }
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int row = GN * wn + 16 * j + l16;
                bv[q][j] = *reinterpret_cast<const u32x4 *>(&sW[row * KBK + 8 * (kc ^ (row & 7))]);
                if (partial)
                    bv[q][j] = kin ? bv[q][j] : zero;
            }
        }
        if (bt + 2 < b1)
            issue(bt + 2, nA, nW);
#pragma unroll
        for (int q = 0; q < KB; ++q)
#pragma unroll
            for (int i = 0; i < RT; ++i)
#pragma unroll
                for (int j = 0; j < 4; ++j)
                    acc[i][j] = Mfma<T>::run(bv[q][j], av[q][i], acc[i][j]);
    };

    if (b0 < b1)
        issue(b0, sA0, sW0);
    if (b0 + 1 < b1)
        issue(b0 + 1, sA1, sW1);
    for (int bt = b0; bt < b1; bt += 3) {
        step(bt, sA0, sW0, sA2, sW2);
        if (bt + 1 < b1)
            step(bt + 1, sA1, sW1, sA0, sW0);
        if (bt + 2 < b1)
            step(bt + 2, sA2, sW2, sA1, sW1);
    }

    // The products are taken as W . act^T, so acc[i][j][e] is output row
    // mb*GMR + WR wm + 16 i + l16, column nb*GNC + 64 wn + 16 j + 4 lq + e:
    // each lane holds four consecutive columns of one row.
    const int col0 = nb * GNC + GN * wn + 4 * lq;
#pragma unroll
    for (int i = 0; i < RT; ++i) {
        const int row = mb * GMR + WR * wm + 16 * i + l16;
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

template <typename T, int WR, int CW>
static void launch_gemm_wr(const GemmArgs &a, hipStream_t stream)
{
    const int64_t ncol = (a.N + GN * CW - 1) / (GN * CW), nrow = (a.M + 4 * WR - 1) / (4 * WR);
    const dim3 grid((unsigned)(ncol * nrow * a.splits));
    hipLaunchKernelGGL((gemm_kernel<T, WR, CW>), grid, dim3(256 * CW), 0, stream, a);
}

template <typename T, int CW>
static void launch_gemm_cw(const GemmArgs &a, hipStream_t stream)
{
    switch (a.wr) {
    case 16: launch_gemm_wr<T, 16, CW>(a, stream); break;
    case 32: launch_gemm_wr<T, 32, CW>(a, stream); break;
    default: launch_gemm_wr<T, 64, CW>(a, stream); break;
    }
}

template <typename T>
static hipError_t launch_gemm_t(const GemmArgs &a, hipStream_t stream)
{
    if (a.cw == 2)
        launch_gemm_cw<T, 2>(a, stream);
    else
        launch_gemm_cw<T, 1>(a, stream);
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

// How a product is laid over the chip (see GemmPlan): the plan of least
// modelled time among rows per wave {16, 32, 64} x column groups {1, 2} x
// splits 1 .. min(32, K / 64) (those the caller fixed, fixed).  The model,
// fitted to measured sweeps on gfx950: a compute unit takes its operand tiles
// in through its L1 at about 38 GB/s, one workgroup after another (the
// activation tile is re-read by every column tile, the weight tile by every
// row block); a split also writes its float32 partial sums, and the second
// kernel's round trip through HBM plus its launch (about 3 us) is added.
GemmPlan plan_gemm(int M, int N, int K, int rows_per_wave, int cols, int splits)
{
    const int nbatch = (K + 63) / 64;
    GemmPlan best{64, 1, 1};
    double tbest = 1e300;
    for (int wr : {16, 32, 64}) {
        if (rows_per_wave && wr != rows_per_wave)
            continue;
        for (int cw : {1, 2}) {
            if (cols && cw * GN != cols)
                continue;
            const int s0 = splits ? splits : 1, s1 = splits ? splits : (nbatch < 32 ? nbatch : 32);
            for (int s = s0; s <= s1; ++s) {
                const double rows = 4.0 * wr, c = (double)GN * cw;
                const double tiles = std::ceil(N / c) * std::ceil(M / rows);
                const double ks = 64.0 * std::ceil((double)nbatch / s);
                const double bytes = ks * 2.0 * (std::min(rows, (double)M) + c) + (s > 1 ? rows * c * 4.0 : 0.0);
                double t = bytes * std::ceil(tiles * s / 256.0) / 38.4e9;
                if (s > 1)
                    t += (double)s * M * N * 8.0 / 8e12 + 3e-6;
                if (t < tbest) {
                    tbest = t;
                    best = GemmPlan{wr, cw, s};
                }
            }
        }
    }
    return best;
}

// RMSNorm of each row: out = x / sqrt(mean(x^2) + eps) * weight (weight in
// float32).  One wave per row: the row is read once into registers with
// 128-bit loads (8 elements per lane and round, C rounds), its sum of squares
// reduced across the wave, then scaled and written with 128-bit stores.
template <typename T, int C>
__global__ __launch_bounds__(256) void rmsnorm_rows_kernel(const T *__restrict__ x, int64_t ldx,
                                                           const float *__restrict__ wt, T *__restrict__ out,
                                                           int64_t ldo, int M, int D, float eps)
{
    const int row = (int)blockIdx.x * 4 + (int)(threadIdx.x >> 6);
    const int lane = threadIdx.x & 63;
    if (row >= M)
        return;  // the whole wave
    const T *xr = x + row * ldx;
    u32x4 v[C];
    float ss = 0.0f;
#pragma unroll
    for (int c = 0; c < C; ++c) {
        const int e = 512 * c + 8 * lane;
        if (e < D) {
            v[c] = *reinterpret_cast<const u32x4 *>(xr + e);
            float f[8];
            unpack_word(v[c].x, f, T{});
            unpack_word(v[c].y, f + 2, T{});
            unpack_word(v[c].z, f + 4, T{});
            unpack_word(v[c].w, f + 6, T{});
#pragma unroll
            for (int i = 0; i < 8; ++i)
                ss = fmaf(f[i], f[i], ss);
        }
    }
    for (int o = 32; o > 0; o >>= 1)
        ss += __shfl_xor(ss, o, 64);
    const float inv = 1.0f / sqrtf(ss / (float)D + eps);
    T *orow = out + row * ldo;
#pragma unroll
    for (int c = 0; c < C; ++c) {
        const int e = 512 * c + 8 * lane;
        if (e < D) {
            float f[8];
            unpack_word(v[c].x, f, T{});
            unpack_word(v[c].y, f + 2, T{});
            unpack_word(v[c].z, f + 4, T{});
            unpack_word(v[c].w, f + 6, T{});
            const float4 w0 = *reinterpret_cast<const float4 *>(wt + e);
            const float4 w1 = *reinterpret_cast<const float4 *>(wt + e + 4);
            const float wv[8] = {w0.x, w0.y, w0.z, w0.w, w1.x, w1.y, w1.z, w1.w};
#pragma unroll
            for (int i = 0; i < 8; ++i)
                f[i] = f[i] * inv * wv[i];
            u32x4 o;
            o.x = pack_word(f, T{});
            o.y = pack_word(f + 2, T{});
            o.z = pack_word(f + 4, T{});
            o.w = pack_word(f + 6, T{});
            *reinterpret_cast<u32x4 *>(orow + e) = o;
        }
    }
}

// Rows whose width or alignment does not allow the vector form: one
// workgroup per row, element by element.
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

template <typename T, int C>
static void launch_rmsnorm_rows(const T *x, int64_t ldx, const float *w, T *out, int64_t ldo, int M, int D,
                                float eps, hipStream_t stream)
{
    hipLaunchKernelGGL((rmsnorm_rows_kernel<T, C>), dim3((unsigned)((M + 3) / 4)), dim3(256), 0, stream, x, ldx, w,
                       out, ldo, M, D, eps);
}

template <typename T>
static void launch_rmsnorm_t(const T *x, int64_t ldx, const float *w, T *out, int64_t ldo, int M, int D,
                             float eps, hipStream_t stream)
{
    const bool vec = D % 8 == 0 && ldx % 8 == 0 && ldo % 8 == 0 &&
                     ((reinterpret_cast<uintptr_t>(x) | reinterpret_cast<uintptr_t>(out)) & 15) == 0 &&
                     (reinterpret_cast<uintptr_t>(w) & 15) == 0;
    if (vec && D <= 1024)
        launch_rmsnorm_rows<T, 2>(x, ldx, w, out, ldo, M, D, eps, stream);
    else if (vec && D <= 4096)
        launch_rmsnorm_rows<T, 8>(x, ldx, w, out, ldo, M, D, eps, stream);
    else if (vec && D <= 8192)
        launch_rmsnorm_rows<T, 16>(x, ldx, w, out, ldo, M, D, eps, stream);
    else
        hipLaunchKernelGGL((rmsnorm_kernel<T>), dim3(M), dim3(256), 0, stream, x, ldx, w, out, ldo, M, D, eps);
}

hipError_t launch_rmsnorm(const void *x, int64_t ldx, const float *w, void *out, int64_t ldo, int M, int D,
                          float eps, int dtype, hipStream_t stream)
{
    if (dtype == 1)
        launch_rmsnorm_t<f16>(static_cast<const f16 *>(x), ldx, w, static_cast<f16 *>(out), ldo, M, D, eps, stream);
    else
        launch_rmsnorm_t<bf16>(static_cast<const bf16 *>(x), ldx, w, static_cast<bf16 *>(out), ldo, M, D, eps,
                               stream);
    return hipGetLastError();
}

} // namespace ssm
