// ssm_kernels.hpp -- argument blocks and launchers of the gfx950 kernels.
// The C-ABI layer (ssm_api.hip) validates the caller's arguments, fills one
// of these blocks (pointers + sizes, already checked) and calls a launcher.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace ssm {

struct ConvArgs {
    const void *x;
    const float *weight;
    const float *bias;        // may be null
    void *conv_state;         // may be null
    const int32_t *slot_idx;  // may be null
    void *out;
    // Packed variable-length batch: sequence b occupies columns
    // [cu_seqlens[b], cu_seqlens[b+1]) of every channel row of length seqlen
    // (the packed token count); null = dense batch [batch, channels, seqlen].
    const int32_t *cu_seqlens;
    const int32_t *has_init_seq;  // varlen: per-sequence flag, null = none
    int batch, channels, seqlen, width, nslots;
    int dtype;                // 0 f32, 1 f16, 2 bf16
    int has_initial_state, apply_silu;
    int vec;                  // x and out 16-byte aligned (dense: and seqlen % 8 == 0)
    int vec_decode;           // seqlen 1, channels % 8 == 0, 16-byte aligned tensors
};

struct ScanArgs {
    const void *u, *dt, *B, *C, *z;  // z may be null
    const float *dt_bias, *A, *D;    // dt_bias, D may be null
    void *state;                     // may be null
    const int32_t *slot_idx;         // may be null
    void *out;
    // varlen as in ConvArgs: sequence b is columns [cu_seqlens[b],
    // cu_seqlens[b+1]) of rows of length seqlen; null = dense batch
    const int32_t *cu_seqlens;
    const int32_t *has_init_seq;     // varlen: per-sequence flag, null = none
    int batch, seqlen, nheads, headdim, dstate, ngroups, nslots;
    int heads_per_group;
    int io_dtype, state_dtype;
    int a_per_state, dt_softplus, has_initial_state;
    int vec;                         // 16-byte aligned bases and seqlen a multiple of 8
};

// Where sequence b lies: columns [begin, begin+len) of the rows of row block
// `block` (b for a dense batch, 0 for a packed one, whose sequences share
// rows), rows being seqlen long.
struct SeqSpan {
    int64_t block;
    int begin, len;
    bool init;
};

__device__ __forceinline__ SeqSpan seq_span(const int32_t *cu, const int32_t *has_init_seq, int b,
                                            int seqlen, int dense_init)
{
    SeqSpan sp;
    if (cu) {
        // clamped: a malformed table cannot address columns outside the rows
        const int tb = min(max(cu[b], 0), seqlen);
        const int te = min(max(cu[b + 1], tb), seqlen);
        sp.block = 0;
        sp.begin = tb;
        sp.len = te - tb;
        sp.init = has_init_seq ? has_init_seq[b] != 0 : false;
    } else {
        sp.block = b;
        sp.begin = 0;
        sp.len = seqlen;
        sp.init = dense_init != 0;
    }
    return sp;
}

struct SsuArgs {
    void *state;
    const int32_t *slot_idx;         // may be null
    const void *x, *dt, *B, *C, *z;  // z may be null
    const float *dt_bias, *A, *D;    // dt_bias, D may be null
    void *out;
    int64_t nrows;                   // batch * nheads * headdim
    int batch, nheads, headdim, dstate, ngroups, nslots;
    int heads_per_group;
    int lanes_per_row_log2;          // lanes per (b,h,p) row = 2^this
    int states_per_lane;             // 8 or 16
    int block_threads;               // 64, 128, 256 or 512 lanes per workgroup
    int io_dtype, state_dtype;
    int a_per_state, dt_softplus;
    int vec;                         // dstate % 8 == 0 and 16-byte aligned bases
    int requests_per_lane;           // 1, 2 or 4 requests taken in turn by each lane
    // fused decode step (conv update in front of the state update); width 0 = none
    void *conv_state;                // [nslots, nheads*headdim, width-1], io dtype
    const float *conv_weight;        // [nheads*headdim, width]
    const float *conv_bias;          // [nheads*headdim] or null
    void *u_out;                     // optional: the conv output, io dtype
    int conv_width;
};

// out[M, N] = A[M, K] . W[N, K]^T (f16 or bf16, float32 accumulation)
struct GemmSeg {
    void *ptr;   // destination of output columns [col0, col0 + ncols)
    int ld;      // its row stride (elements)
    int col0, ncols;
};
struct GemmArgs {
    const void *A;           // [M, lda]
    const void *W;           // [N, K], row-major
    int lda, M, N, K;
    int dtype;               // 1 f16, 2 bf16
    int splits;              // K split over this many workgroups
    float *partial;          // [splits, M, N] float32 when splits > 1
    GemmSeg seg[3];
    int nseg;
    const void *residual;    // optional: added to the output, [M, ld_residual]
    int ld_residual;
    const int32_t *row_slot; // optional: rows with a negative entry are not written
};
hipError_t launch_gemm(const GemmArgs &a, hipStream_t stream);
hipError_t launch_rmsnorm(const void *x, const float *w, void *out, int M, int D, float eps, int dtype,
                          hipStream_t stream);

hipError_t launch_conv(const ConvArgs &a, hipStream_t stream);
hipError_t launch_scan(const ScanArgs &a, hipStream_t stream);
// Mamba-2 prefill in chunked matrix form on the matrix cores (dense batches,
// bf16 I/O, one decay per head, dstate 64/128/256, headdim a multiple of 64)
bool ssd_supported(const ScanArgs &a);
hipError_t launch_ssd(const ScanArgs &a, hipStream_t stream);
hipError_t launch_ssu(const SsuArgs &a, hipStream_t stream);

// Limits the kernels are built for.
constexpr int kMaxConvWidth = 4;
constexpr int kMaxScanDstate = 256;
constexpr int kMaxSsuDstate = 512;
constexpr int kFusedConvWidth = 4;  // the conv width the fused decode step is built for

} // namespace ssm
