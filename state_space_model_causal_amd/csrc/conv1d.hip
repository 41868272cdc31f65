// conv1d.hip -- causal depthwise conv1d + bias + SiLU with a per-request conv
// cache, on gfx950.
//
// Operation: the causal-conv1d and silu operators of "feat(llama.cu): 适配
// mamba 模型" (InfiniLM-Rust PR #48, section 2.1), with the cache handling of
// section 3.1 (the conv operator reads the request's cached history and leaves
// the newest width-1 samples behind for the next call):
//     out[b,c,t] = silu(bias[c] + sum_{k<W} w[c,k] * xh[b,c,t-W+1+k])
// where xh is x preceded by the cached history (or zeros).
//
// Prefill kernel: one 256-lane workgroup per (sequence, channel) row walks
// the row in tiles of 256*E samples (E = one 128-bit load per lane).  The tile
// plus its W-1 history is staged in LDS so each lane reads its neighbours'
// samples without re-fetching them from memory; the history of the next tile
// is kept in LDS, and the sequence's final W-1 samples go to the cache at the
// end.  The same kernel serves a dense batch and a packed variable-length
// batch (sequences of different lengths concatenated along time, each with
// its own slot and initial-state flag); the tiles are aligned to 128-bit
// vectors whatever column a sequence starts at.  HBM traffic: x read once,
// out written once.
//
// Decode kernels (seqlen == 1): gather the window from the slot, one output,
// shift the window by one in place.  The vector kernel gives each lane 8
// channels with 128-bit accesses; the scalar kernel (any channel count or
// alignment) gives each lane one channel.
#include "ssm_device.hpp"
#include "ssm_kernels.hpp"

namespace ssm {

template <typename T, int W, bool VEC>
__global__ __launch_bounds__(256) void conv_prefill_kernel(ConvArgs a)
{
    constexpr int E = 16 / StorageSize<T>::value;  // samples per 128-bit access
    constexpr int TILE = 256 * E;
    constexpr int H = W - 1;
    constexpr int OFF = 4;                          // history sits in xs[OFF-H, OFF)
    __shared__ float xs[OFF + TILE];
    __shared__ float hist[4];   // the H samples in front of the current tile
    __shared__ float init[4];   // the sequence's history (cache or zeros)

    const int64_t row = xcd_block_order(blockIdx.x, gridDim.x);  // b*channels + c
    const int b = (int)(row / a.channels), c = (int)(row % a.channels);
    const SeqSpan sp = seq_span(a.cu_seqlens, a.has_init_seq, b, a.seqlen, a.has_initial_state);
    const int slot = a.slot_idx ? a.slot_idx[b] : b;
    if (slot < 0 || sp.len == 0)
        return;  // padded or empty sequence (uniform over the workgroup)
    const int tid = threadIdx.x;
    const int len = sp.len;

    float w[W];
#pragma unroll
    for (int k = 0; k < W; ++k)
        w[k] = a.weight[(int64_t)c * W + k];
    const float bias = a.bias ? a.bias[c] : 0.0f;

    T *cs = a.conv_state ? static_cast<T *>(a.conv_state) + ((int64_t)slot * a.channels + c) * H : nullptr;
    if (tid < H)
        init[tid] = (sp.init && cs) ? to_f32(cs[tid]) : 0.0f;

    // The row is walked in tiles aligned to 128-bit vectors: column j of the
    // walk is sequence step j - m, where m places the sequence's first sample
    // inside its vector.  Samples outside the sequence are replaced by the
    // history (before it) or by zeros (after it) and never stored.
    const int64_t first = (sp.block * a.channels + c) * a.seqlen + sp.begin;
    const int m = VEC ? (int)(first % E) : 0;
    const T *xr = static_cast<const T *>(a.x) + (first - m);
    T *orow = static_cast<T *>(a.out) + (first - m);
    const int64_t room = a.x_elems - (first - m);  // elements of x from xr on

    __syncthreads();  // init visible
    if (tid < H) {
        // columns -H..-1 of the first tile are steps -m-H..-m-1
        const int tau = tid - H - m;
        hist[tid] = tau >= -H ? init[H + tau] : 0.0f;
    }
    for (int t0 = 0; t0 < m + len; t0 += TILE) {
        const int t = t0 + tid * E;
        float v[E];
        if (VEC && t < m + len && t + E <= room) {
            load_vec<T, E>(xr + t, v);
        } else {
#pragma unroll
            for (int i = 0; i < E; ++i) {
                const int j = t + i;
                v[i] = (j >= m && j < m + len) ? to_f32(xr[j]) : 0.0f;
            }
        }
#pragma unroll
        for (int i = 0; i < E; ++i) {
            const int tau = t + i - m;
            if (tau < 0)
                v[i] = tau >= -H ? init[H + tau] : 0.0f;
            else if (tau >= len)
                v[i] = 0.0f;
        }
        __syncthreads();  // hist written / previous tile's readers finished
#pragma unroll
        for (int i = 0; i < E; ++i)
            xs[OFF + tid * E + i] = v[i];
        if (tid < H)
            xs[OFF - H + tid] = hist[tid];
        __syncthreads();
        float o[E];
#pragma unroll
        for (int i = 0; i < E; ++i) {
            float acc = bias;
#pragma unroll
            for (int k = 0; k < W; ++k)
                acc = fmaf(w[k], xs[OFF + tid * E + i - H + k], acc);
            o[i] = a.apply_silu ? silu_f32(acc) : acc;
        }
        if (VEC && t >= m && t + E <= m + len) {
            store_vec<T, E>(orow + t, o);
        } else {
#pragma unroll
            for (int i = 0; i < E; ++i)
                if (t + i >= m && t + i < m + len)
                    orow[t + i] = from_f32<T>(o[i]);
        }
        if (tid < H)
            hist[tid] = xs[OFF + TILE - H + tid];
    }
    __syncthreads();  // every lane has read init and the cache row
    if (cs && tid < H) {
        // the new tail: the last H samples of history || sequence, copied
        const int tau = len - H + tid;
        cs[tid] = tau >= 0 ? xr[m + tau] : from_f32<T>(init[H + tau]);
    }
}

template <typename T, int W>
__global__ __launch_bounds__(256) void conv_decode_kernel(ConvArgs a)
{
    constexpr int H = W - 1;
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (i >= (int64_t)a.batch * a.channels)
        return;
    const int b = (int)(i / a.channels), c = (int)(i % a.channels);
    const int slot = a.slot_idx ? a.slot_idx[b] : b;
    if (slot < 0)
        return;
    T *cs = a.conv_state ? static_cast<T *>(a.conv_state) + ((int64_t)slot * a.channels + c) * H : nullptr;
    const T xv_raw = static_cast<const T *>(a.x)[i];
    T win[H > 0 ? H : 1];
    float acc = a.bias ? a.bias[c] : 0.0f;
#pragma unroll
    for (int k = 0; k < H; ++k) {
        win[k] = cs ? cs[k] : T{};
        const float hv = (a.has_initial_state && cs) ? to_f32(win[k]) : 0.0f;
        acc = fmaf(a.weight[(int64_t)c * W + k], hv, acc);
    }
    acc = fmaf(a.weight[(int64_t)c * W + H], to_f32(xv_raw), acc);
    static_cast<T *>(a.out)[i] = from_f32<T>(a.apply_silu ? silu_f32(acc) : acc);
    if (cs) {
        // shift the window by one; without an initial state the history is
        // zeros, so the new window is (0, ..., 0, x)
#pragma unroll
        for (int k = 0; k + 1 < H; ++k)
            cs[k] = a.has_initial_state ? win[k + 1] : from_f32<T>(0.0f);
        if (H > 0)
            cs[H - 1] = xv_raw;
    }
}

// Decode with 128-bit accesses: one lane per 8 consecutive channels of one
// request (channels % 8 == 0, 16-byte aligned tensors).  The 8 windows of
// width-1 samples are contiguous in the cache row, so a lane reads and writes
// them as whole vectors; the window values pass through float32 unchanged.
template <typename T, int W>
__global__ __launch_bounds__(256) void conv_decode_vec_kernel(ConvArgs a)
{
    constexpr int H = W - 1, G = 8;
    const int groups = a.channels / G;
    const int64_t gi = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (gi >= (int64_t)a.batch * groups)
        return;
    const int b = (int)(gi / groups), c0 = (int)(gi % groups) * G;
    const int slot = a.slot_idx ? a.slot_idx[b] : b;
    if (slot < 0)
        return;
    const int64_t xo = (int64_t)b * a.channels + c0;
    float xv[G], w[G * W], bias[G];
    load_vec_cached<T, G>(static_cast<const T *>(a.x) + xo, xv);
    load_vec_cached<float, G * W>(a.weight + (int64_t)c0 * W, w);
    if (a.bias)
        load_vec_cached<float, G>(a.bias + c0, bias);
    else
#pragma unroll
        for (int g = 0; g < G; ++g)
            bias[g] = 0.0f;
    T *cs = a.conv_state ? static_cast<T *>(a.conv_state) + ((int64_t)slot * a.channels + c0) * H : nullptr;
    float win[G * H > 0 ? G * H : 1];
    if constexpr (H > 0) {
        if (cs && a.has_initial_state)
            load_vec_cached<T, G * H>(cs, win);
        else
#pragma unroll
            for (int k = 0; k < G * H; ++k)
                win[k] = 0.0f;
    }
    float o[G];
#pragma unroll
    for (int g = 0; g < G; ++g) {
        float acc = bias[g];
#pragma unroll
        for (int k = 0; k < H; ++k)
            acc = fmaf(w[g * W + k], win[g * H + k], acc);
        acc = fmaf(w[g * W + H], xv[g], acc);
        o[g] = a.apply_silu ? silu_f32(acc) : acc;
    }
    store_vec_cached<T, G>(static_cast<T *>(a.out) + xo, o);
    if constexpr (H > 0) {
        if (cs) {
            float nw[G * H];
#pragma unroll
            for (int g = 0; g < G; ++g) {
#pragma unroll
                for (int k = 0; k + 1 < H; ++k)
                    nw[g * H + k] = win[g * H + k + 1];
                nw[g * H + H - 1] = xv[g];
            }
            store_vec_cached<T, G * H>(cs, nw);
        }
    }
}

template <typename T, int W>
static hipError_t launch_conv_tw(const ConvArgs &a, hipStream_t stream)
{
    if (!a.cu_seqlens && a.seqlen == 1 && a.vec_decode) {
        const int64_t n = (int64_t)a.batch * (a.channels / 8);
        hipLaunchKernelGGL((conv_decode_vec_kernel<T, W>), dim3((unsigned)((n + 255) / 256)), dim3(256), 0,
                           stream, a);
    } else if (!a.cu_seqlens && a.seqlen == 1) {
        const int64_t n = (int64_t)a.batch * a.channels;
        hipLaunchKernelGGL((conv_decode_kernel<T, W>), dim3((unsigned)((n + 255) / 256)), dim3(256), 0,
                           stream, a);
    } else {
        const dim3 grid((unsigned)((int64_t)a.batch * a.channels));
        if (a.vec)
            hipLaunchKernelGGL((conv_prefill_kernel<T, W, true>), grid, dim3(256), 0, stream, a);
        else
            hipLaunchKernelGGL((conv_prefill_kernel<T, W, false>), grid, dim3(256), 0, stream, a);
    }
    return hipGetLastError();
}

template <typename T>
static hipError_t launch_conv_t(const ConvArgs &a, hipStream_t stream)
{
    switch (a.width) {
    case 1: return launch_conv_tw<T, 1>(a, stream);
    case 2: return launch_conv_tw<T, 2>(a, stream);
    case 3: return launch_conv_tw<T, 3>(a, stream);
    default: return launch_conv_tw<T, 4>(a, stream);
    }
}

hipError_t launch_conv(const ConvArgs &a, hipStream_t stream)
{
    switch (a.dtype) {
    case 0: return launch_conv_t<float>(a, stream);
    case 1: return launch_conv_t<f16>(a, stream);
    default: return launch_conv_t<bf16>(a, stream);
    }
}

} // namespace ssm
