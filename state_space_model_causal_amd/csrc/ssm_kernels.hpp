// ssm_kernels.hpp -- argument blocks and launchers of the gfx950 kernels.
// The C-ABI layer (ssm_api.hip) validates the caller's arguments, fills one
// of these blocks (pointers + sizes, already checked) and calls a launcher.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "ssm.h"

namespace ssm {

// Element strides: every tensor's innermost dimension is contiguous (checked
// on the host); the outer strides below are free.  A packed (varlen) batch
// has no batch dimension: its batch strides are 0.
struct ConvArgs {
    const void *x;
    const float *weight;
    const float *bias;        // may be null; dense
    void *conv_state;         // may be null
    const int32_t *slot_idx;  // may be null
    void *out;
    int64_t x_sb, x_sc;       // x [batch, channels, seqlen]
    int64_t o_sb, o_sc;       // out, same shape
    int64_t cs_ss, cs_sc;     // conv_state [nslots, channels, width-1]
    int64_t w_sc;             // weight [channels, width]
    // Packed variable-length batch: sequence b occupies columns
    // [cu_seqlens[b], cu_seqlens[b+1]) of every channel row of length seqlen
    // (the packed token count); null = dense batch [batch, channels, seqlen].
    const int32_t *cu_seqlens;
    const int32_t *has_init_seq;  // varlen: per-sequence flag, null = none
    int batch, channels, seqlen, width, nslots;
    int dtype;                // 0 f32, 1 f16, 2 bf16
    int has_initial_state, apply_silu;
    int vec;                  // dense: x and out rows 16-byte aligned (base and outer
                              // strides), seqlen a multiple of a vector; packed: 16-byte
                              // aligned bases, rows all aligned or sharing one stride
    int rows16;               // x and out rows 16-byte aligned, seqlen a multiple of a vector
    int vec_decode;           // seqlen 1, 8 channels per 128-bit access: x, out, cache and
                              // weight contiguous over channels, 16-byte aligned
};

struct ScanArgs {
    const void *u, *dt, *B, *C, *z;  // z may be null
    const float *dt_bias, *A, *D;    // dt_bias, D may be null
    void *state;                     // may be null
    const int32_t *slot_idx;         // may be null
    void *out;
    int64_t u_sb, u_sc, z_sb, z_sc, o_sb, o_sc;  // [batch, channels, seqlen]
    int64_t dt_sb, dt_sh;            // dt [batch, nheads, seqlen]
    int64_t B_sb, B_sg, B_sn;        // B [batch, ngroups, dstate, seqlen]
    int64_t C_sb, C_sg, C_sn;        // C, same shape
    int64_t A_sh;                    // A [nheads, dstate] (per-state decays)
    int64_t st_ss, st_sh, st_sp;     // state [nslots, nheads, headdim, dstate]
    // varlen as in ConvArgs: sequence b is columns [cu_seqlens[b],
    // cu_seqlens[b+1]) of rows of length seqlen; null = dense batch
    const int32_t *cu_seqlens;
    const int32_t *has_init_seq;     // varlen: per-sequence flag, null = none
    int batch, seqlen, nheads, headdim, dstate, ngroups, nslots;
    int heads_per_group;
    int io_dtype, state_dtype;
    int a_per_state, dt_softplus, has_initial_state;
    int vec;                         // 16-byte aligned rows (bases and outer strides) and
                                     // seqlen a multiple of a vector
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
    int64_t x_sb, x_sh, z_sb, z_sh, o_sb, o_sh;  // [batch, nheads, headdim]
    int64_t dt_sb;                   // dt [batch, nheads]
    int64_t B_sb, B_sg, C_sb, C_sg;  // B, C [batch, ngroups, dstate]
    int64_t A_sh;                    // A [nheads, dstate] (per-state decays)
    int64_t st_ss, st_sh, st_sp;     // state [nslots, nheads, headdim, dstate]
    int64_t nrows;                   // batch * nheads * headdim
    int batch, nheads, headdim, dstate, ngroups, nslots;
    int heads_per_group;
    int lanes_per_row_log2;          // lanes per (b,h,p) row = 2^this
    int states_per_lane;             // 8 or 16
    int block_threads;               // 64, 128, 256 or 512 lanes per workgroup
    int io_dtype, state_dtype;
    int a_per_state, dt_softplus;
    int vec;                         // dstate % V == 0, 16-byte aligned state / B / C / A rows
    int requests_per_lane;           // 1, 2 or 4 requests taken in turn by each lane
    // fused decode step (conv update in front of the state update); width 0 = none
    void *conv_state;                // [nslots, nheads*headdim, width-1], io dtype
    const float *conv_weight;        // [nheads*headdim, width]
    const float *conv_bias;          // [nheads*headdim] or null; dense
    void *u_out;                     // optional: the conv output, io dtype [batch, nheads, headdim]
    int64_t cs_ss, cs_sc, cw_sc, u_sb, u_sh;
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
    const void *W;           // [N, ldw], row-major
    int lda, ldw, M, N, K;
    int dtype;               // 1 f16, 2 bf16
    int wr;                  // rows per wave: 16, 32 or 64
    int cw;                  // column groups of 64 per workgroup (1 or 2; 4 waves each)
    int splits;              // K split over this many workgroups
    float *partial;          // [splits, M, N] float32 when splits > 1
    GemmSeg seg[3];
    int nseg;
    const void *residual;    // optional: added to the output, [M, ld_residual]
    int ld_residual;
    const int32_t *row_slot; // optional: rows with a negative entry are not written
};
// How a product is laid over the chip: rows per wave, column groups of 64
// (a workgroup of 4 cw waves takes 4 wr rows x 64 cw columns) and K splits
// (their float32 partial sums added by a second kernel).
struct GemmPlan {
    int wr, cw, splits;
};
// (rows_per_wave, cols, splits: 0 for the library's choice)
GemmPlan plan_gemm(int M, int N, int K, int rows_per_wave = 0, int cols = 0, int splits = 0);
hipError_t launch_gemm(const GemmArgs &a, hipStream_t stream);
hipError_t launch_rmsnorm(const void *x, int64_t ldx, const float *w, void *out, int64_t ldo, int M, int D,
                          float eps, int dtype, hipStream_t stream);

hipError_t launch_conv(const ConvArgs &a, hipStream_t stream);
hipError_t launch_scan(const ScanArgs &a, hipStream_t stream);
// Mamba-2 prefill in chunked matrix form on the matrix cores (dense batches,
// bf16 I/O, one decay per head, dstate 64/128/256, headdim a multiple of 64)
bool ssd_supported(const ScanArgs &a);
hipError_t launch_ssd(const ScanArgs &a, hipStream_t stream);
hipError_t launch_ssu(const SsuArgs &a, hipStream_t stream);

// Host-side validation of the C entry points (ssm_api.hip): each fills an
// argument block and returns SSM_OK, or an ssm_status, without any HIP call,
// so a caller that chains several steps can check all of them first.
int prepare_conv(ConvArgs &a, const ssm_tensor &x, const ssm_tensor &weight, const ssm_tensor &bias,
                 const ssm_tensor &conv_state, const int32_t *slot_idx, const int32_t *cu_seqlens,
                 const int32_t *has_init_seq, const ssm_tensor &out, int batch, int channels, int seqlen,
                 int width, int nslots, int has_initial_state, int apply_silu);
int prepare_scan(ScanArgs &a, const ssm_tensor &u, const ssm_tensor &dt, const ssm_tensor &dt_bias,
                 const ssm_tensor &A, const ssm_tensor &B, const ssm_tensor &C, const ssm_tensor &D,
                 const ssm_tensor &z, const ssm_tensor &ssm_state, const int32_t *slot_idx,
                 const int32_t *cu_seqlens, const int32_t *has_init_seq, const ssm_tensor &out, int batch,
                 int seqlen, int nheads, int headdim, int dstate, int ngroups, int nslots, int a_per_state,
                 int dt_softplus, int has_initial_state);
int prepare_ssu(SsuArgs &a, const ssm_tensor &state, const int32_t *slot_idx, const ssm_tensor &x,
                const ssm_tensor &dt, const ssm_tensor &dt_bias, const ssm_tensor &A, const ssm_tensor &B,
                const ssm_tensor &C, const ssm_tensor &D, const ssm_tensor &z, const ssm_tensor &out,
                int batch, int nheads, int headdim, int dstate, int ngroups, int nslots, int a_per_state,
                int dt_softplus, const ssm_launch_config *cfg);
int prepare_decode_conv(SsuArgs &a, const ssm_tensor &conv_state, const ssm_tensor &conv_weight,
                        const ssm_tensor &conv_bias, const ssm_tensor &u_out, int conv_width);
int status_of(hipError_t e);

// The mixed launch (ssu.hip): a prefill scan and an independent fused
// decode step in one grid.  mixed_scan_ok / mixed_decode_ok: the kinds it is
// built for (f16 or bf16 I/O, f32 state, per-state decays, 128-bit rows; a
// Mamba-1 scan of dstate <= 16, dense or packed; the
// decode step's interleaved map with the shared conv, two requests per lane);
// mixed_pair_ok: both, with one io dtype, within one grid.
bool mixed_scan_ok(const ScanArgs &s);
bool mixed_decode_ok(const SsuArgs &d);
bool mixed_pair_ok(const ScanArgs &s, const SsuArgs &d);
hipError_t launch_mixed(const ScanArgs &s, const SsuArgs &d, hipStream_t stream);

// Limits the kernels are built for.
constexpr int kMaxConvWidth = 4;
constexpr int kMaxScanDstate = 256;
constexpr int kMaxSsuDstate = 512;
constexpr int kFusedConvWidth = 4;  // the conv width the fused decode step is built for

} // namespace ssm
