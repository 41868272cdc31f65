/*
 * ssm.h -- C ABI of the MI355X (gfx950) causal selective-SSM hot path.
 *
 * Three operations, named after the operators of the Mamba adaptation in
 * "feat(llama.cu): 适配 mamba 模型" (InfiniLM-Rust PR #48, section 2.1 lists
 * causal-conv1d, selective-scan, silu and element-mul; section 3.1 places the
 * per-request mamba-cache reads and writes at the conv and scan operators) and
 * after the decode call of "[XPU] Add tuned Mamba SSU configs for Intel Arc Pro
 * B70" (vLLM PR #50534 report, section "关键源码片段": a selective state
 * update taking the state cache, x, dt, A, B, C, optional D and z gate, a dt
 * bias with softplus, and a caller-provided out).  The pages name the
 * operators without writing their equations; the equations below are the
 * standard selective SSM that those operator names and arguments describe.
 *
 * Common conventions
 * ------------------
 *  - Every tensor is an ssm_tensor: a pointer to DEVICE memory owned by the
 *    caller, its dtype code, and the element strides of its dimensions in the
 *    order of the shape given per call (outermost first; entries past the
 *    tensor's rank are ignored).  data == NULL marks an optional tensor as
 *    absent.  The library allocates nothing, frees nothing, keeps no state
 *    between calls and never synchronises: each call validates its arguments
 *    on the host, enqueues its kernels on `stream` (a hipStream_t; NULL = the
 *    null stream) and returns.  Calls can be captured into a HIP graph.
 *  - Layout rules: the innermost dimension must have stride 1 (a dimension of
 *    size 1 may have any stride), every stride must be >= 0, and data must be
 *    aligned to the element size; otherwise SSM_ERR_LAYOUT / SSM_ERR_ALIGN.
 *    Outer strides are free, so views such as the x and z halves of a
 *    [batch, 2*channels, seqlen] projection output are taken as they are.
 *    The 128-bit vector paths are used when the base pointer and every outer
 *    stride are 16-byte multiples; other layouts take element-wise paths with
 *    the same results.  Outputs must not overlap inputs or one another.
 *  - dtype codes (ssm_dtype): SSM_F32, SSM_F16 (IEEE binary16), SSM_BF16.
 *    "io dtype" covers x/u, dt, B, C, z, out and the conv cache, which must
 *    all have the same dtype; A, D, dt_bias, conv weight and conv bias are
 *    always float32.  The state cache's dtype is its own.  All arithmetic is
 *    float32; narrowing to f16/bf16 rounds to nearest, ties to even.
 *  - Slots: slot_idx (int32 [batch], device memory, may be NULL) maps request
 *    b to cache row slot_idx[b]; NULL means slot b.  A negative index marks a
 *    padded request: nothing is written for it (its out rows keep their
 *    contents) and its inputs affect no output.  Non-negative indices must be
 *    < nslots and distinct within a call (duplicates race; this is not
 *    checked on the device).
 *  - batch == 0 or seqlen == 0 is a no-op returning SSM_OK.
 *  - Errors are returned synchronously, before anything is enqueued, as
 *    ssm_status codes; asynchronous device faults surface at the caller's
 *    next synchronisation, as with any HIP launch.  Nothing is thrown.
 */
#ifndef SSM_H
#define SSM_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define SSM_ABI_VERSION 3

typedef enum ssm_dtype {
    SSM_F32 = 0,
    SSM_F16 = 1,
    SSM_BF16 = 2
} ssm_dtype;

typedef enum ssm_status {
    SSM_OK = 0,
    SSM_ERR_NULL_ARG = 1,         /* a required tensor or pointer is NULL              */
    SSM_ERR_SHAPE = 2,            /* a size is out of range or sizes disagree          */
    SSM_ERR_DTYPE = 3,            /* unknown dtype code, or dtypes that must agree don't */
    SSM_ERR_ALIGN = 4,            /* a pointer is not aligned to its element size      */
    SSM_ERR_UNSUPPORTED = 5,      /* a size or variant the kernels are not built for   */
    SSM_ERR_HIP = 6,              /* the HIP runtime refused a launch                  */
    SSM_ERR_LAYOUT = 7,           /* an innermost stride is not 1, or a stride is < 0  */
    SSM_ERR_OUT_OF_RESOURCES = 8  /* a launch geometry beyond the kernels' register,
                                     LDS or workgroup-size budget                     */
} ssm_status;

typedef struct ssm_tensor {
    void *data;         /* device memory; NULL = absent                              */
    int32_t dtype;      /* ssm_dtype                                                  */
    int32_t reserved;   /* 0                                                          */
    int64_t stride[4];  /* element strides, outermost dimension first                 */
} ssm_tensor;

/*
 * ssm_causal_conv1d -- causal depthwise conv1d + bias + optional SiLU, with an
 * optional per-request conv cache (the causal-conv1d and silu operators and
 * the cache of InfiniLM-Rust PR #48, sections 2.1 and 3.1).
 *
 *   x, out      io dtype [batch, channels, seqlen]   (time innermost)
 *   weight      f32 [channels, width]; tap width-1 multiplies the newest sample
 *   bias        f32 [channels] or absent
 *   conv_state  io dtype [nslots, channels, width-1] or absent; oldest sample
 *               first.  In: the history before x[...,0] when
 *               has_initial_state (else the history is zeros).  Out: the last
 *               width-1 samples of history||x, copied bit-exactly.
 *
 *   out[b,c,t] = act(bias[c] + sum_{k<width} weight[c,k] * xh(t-width+1+k))
 *   xh(s) = x[b,c,s] for s >= 0, history for s < 0; act = SiLU or identity.
 *
 * seqlen == 1 with has_initial_state is the decode update (one output, window
 * shifted by one); prefill writes the tail a later decode step starts from.
 * Limits: 1 <= width <= 4 and batch*channels <= 2^31-1 (else
 * SSM_ERR_UNSUPPORTED).
 */
int ssm_causal_conv1d(ssm_tensor x, ssm_tensor weight, ssm_tensor bias, ssm_tensor conv_state,
                      const int32_t *slot_idx, ssm_tensor out, int batch, int channels,
                      int seqlen, int width, int nslots, int has_initial_state, int apply_silu,
                      void *stream);

/*
 * ssm_selective_scan -- selective scan over a whole sequence (prefill): the
 * selective-scan operator with its silu(z) element-mul gate (InfiniLM-Rust PR
 * #48, section 2.1), final state stored to the request's cache slot (3.1).
 *
 *   u, z, out   io dtype [batch, nheads*headdim, seqlen]; z may be absent
 *   dt          io dtype [batch, nheads, seqlen]
 *   dt_bias, D  f32 [nheads] or absent
 *   A           f32 [nheads, dstate] when a_per_state (Mamba-1: one decay per
 *               channel and state, headdim 1), else f32 [nheads] (Mamba-2:
 *               one decay per head)
 *   B, C        io dtype [batch, ngroups, dstate, seqlen]; head h reads group
 *               h / (nheads/ngroups)
 *   ssm_state   state dtype [nslots, nheads, headdim, dstate] or absent; in:
 *               the initial state when has_initial_state (else zeros); out:
 *               the state after the last token
 *
 *   delta_t = softplus(dt_t + dt_bias) (or dt_t + dt_bias if !dt_softplus)
 *   h_t[n]  = exp(delta_t*A[n]) * h_{t-1}[n] + delta_t * B_t[n] * u_t
 *   out_t   = (sum_n C_t[n] h_t[n] + D u_t) * silu(z_t)
 *
 * Limits: nheads % ngroups == 0; 1 <= dstate <= 256 (the carried states of
 * a workgroup's channels are held in LDS; larger: SSM_ERR_OUT_OF_RESOURCES).
 */
int ssm_selective_scan(ssm_tensor u, ssm_tensor dt, ssm_tensor dt_bias, ssm_tensor A,
                       ssm_tensor B, ssm_tensor C, ssm_tensor D, ssm_tensor z,
                       ssm_tensor ssm_state, const int32_t *slot_idx, ssm_tensor out, int batch,
                       int seqlen, int nheads, int headdim, int dstate, int ngroups, int nslots,
                       int a_per_state, int dt_softplus, int has_initial_state, void *stream);

/*
 * ssm_selective_scan_ex -- ssm_selective_scan with a choice of algorithm.
 *   algo  SSM_SCAN_AUTO: the library's choice;
 *         SSM_SCAN_RECURRENT: the step-by-step recurrence (any shape);
 *         SSM_SCAN_CHUNKED: the chunked matrix form on the matrix cores.
 * The chunked form needs one decay per head (a_per_state == 0), f16 or bf16 I/O,
 * dstate 64, 128 or 256, headdim a multiple of 64, seqlen a multiple of 8,
 * 16-byte aligned rows, B and C (request, group) planes spanning less than
 * 4 GiB, and a dense [.., headdim, dstate] state slot;
 * otherwise SSM_SCAN_CHUNKED returns SSM_ERR_UNSUPPORTED.  SSM_SCAN_AUTO
 * takes it whenever it applies.  The chunked form computes the same
 * recurrence: over a chunk of steps with one scalar decay per step, the state
 * recursion unrolls into products of small matrices (decay-weighted C.B^T
 * within the chunk, C times the carried state, and the decay-weighted B
 * times u for the next state), which run on MFMA with float32 accumulation.
 * With bf16 I/O, operands that are not exact in bf16 are split into two bf16
 * parts (about 16 significant bits per product).  With f16 I/O, C.B^T runs on
 * the f16 instruction, u is split exactly into two bf16 parts for the bf16
 * decay matrix, and the carried state and the weighted u are split into two
 * f16 parts under a power-of-two scale per row (about 22 bits).  Other
 * arguments as in ssm_selective_scan.
 */
#define SSM_SCAN_AUTO 0
#define SSM_SCAN_RECURRENT 1
#define SSM_SCAN_CHUNKED 2
int ssm_selective_scan_ex(ssm_tensor u, ssm_tensor dt, ssm_tensor dt_bias, ssm_tensor A,
                          ssm_tensor B, ssm_tensor C, ssm_tensor D, ssm_tensor z,
                          ssm_tensor ssm_state, const int32_t *slot_idx, ssm_tensor out,
                          int batch, int seqlen, int nheads, int headdim, int dstate,
                          int ngroups, int nslots, int a_per_state, int dt_softplus,
                          int has_initial_state, int algo, void *stream);

/*
 * ssm_state_update -- one-token selective state update (decode) in place on a
 * slot-indexed state cache: the selective state update of the vLLM PR #50534
 * report ("关键源码片段"), same argument set.
 *
 *   state       state dtype [nslots, nheads, headdim, dstate], read-modify-
 *               written in place for the named slots only
 *   x, z, out   io dtype [batch, nheads, headdim]; z may be absent
 *   dt          io dtype [batch, nheads]
 *   dt_bias, D  f32 [nheads] or absent
 *   A           f32 [nheads, dstate] (a_per_state) or f32 [nheads]
 *   B, C        io dtype [batch, ngroups, dstate]
 *
 *   h' = exp(delta*A) * h + delta * B * x;  out = (C.h' + D x) * silu(z)
 * The readout uses the float32 h'; the cache receives h' rounded to the state
 * dtype.  Limits: nheads % ngroups == 0; 1 <= dstate <= 512 (a row spans at
 * most one wave; larger: SSM_ERR_OUT_OF_RESOURCES).
 */
int ssm_state_update(ssm_tensor state, const int32_t *slot_idx, ssm_tensor x, ssm_tensor dt,
                     ssm_tensor dt_bias, ssm_tensor A, ssm_tensor B, ssm_tensor C, ssm_tensor D,
                     ssm_tensor z, ssm_tensor out, int batch, int nheads, int headdim,
                     int dstate, int ngroups, int nslots, int a_per_state, int dt_softplus,
                     void *stream);

/*
 * Launch geometry of the state update.  "[XPU] Add tuned Mamba SSU configs for
 * Intel Arc Pro B70" (vLLM PR #50534 report, section "实现拆解", steps 2-3)
 * tunes the update's launch configuration per device over a grid of
 * effective batches (batch x nheads) for each (headdim, dstate, dtype) key and
 * keeps a tuned entry only where it beats the heuristic.  Here the
 * geometry is the number of consecutive states each lane owns (4, 8 or 16;
 * 4 only for a 4-byte cache, and a row of dstate states must span at most 64
 * lanes) and the workgroup size (64, 128, 256 or 512 lanes); the library
 * carries a table tuned on gfx950 and falls back to a heuristic for other
 * shapes: 32 bytes of state per lane (16 states of a 2-byte cache for rows of
 * >= 32 states that are a multiple of 16, else 8) in 256-lane workgroups.
 * Independently of the geometry, with one channel per head (headdim 1) and
 * at least 8 requests each lane updates its states for two requests in
 * turn.  With 32 bytes of state per lane, rows of a power-of-two size up to
 * 1 KB, dense state slots and at least 2^18 (request, row) pairs, the lanes
 * take the same number of states in an interleaved order instead (each
 * 128-bit access of a wave covers a contiguous kilobyte of the cache); the
 * cache bytes written are the same.
 */
typedef struct ssm_launch_config {
    int states_per_lane; /* 4, 8 or 16             */
    int block_threads;   /* 64, 128, 256 or 512    */
} ssm_launch_config;

/*
 * ssm_state_update_config -- the geometry ssm_state_update would use for a
 * shape (no device call).  *from_table (may be NULL) is set to 1 when the
 * tuned table supplied it, 0 for the heuristic.
 */
int ssm_state_update_config(int batch, int nheads, int headdim, int dstate,
                            int io_dtype, int state_dtype,
                            ssm_launch_config *config, int *from_table);

/*
 * ssm_state_update_ex -- ssm_state_update with the caller's geometry (the
 * override hook of the tuning method); config NULL = the library's choice.
 * Every geometry computes the same values: the cache bytes are identical, the
 * outputs differ only in the summation order of the readout.  A geometry
 * past what the kernels are built for returns SSM_ERR_OUT_OF_RESOURCES
 * (more than 16 states per lane: the registers of the state arrays; more than
 * 512 lanes per workgroup: the kernels' launch bound; a row of more than 64
 * lanes: the readout sums within one wave), the analogue of the skipped
 * out-of-resources configurations of the vLLM tuning benchmark; any other
 * invalid geometry (states per lane or workgroup size not one of the listed
 * values, 4 states per lane with a 2-byte cache) returns SSM_ERR_SHAPE.
 */
int ssm_state_update_ex(ssm_tensor state, const int32_t *slot_idx, ssm_tensor x,
                        ssm_tensor dt, ssm_tensor dt_bias, ssm_tensor A, ssm_tensor B,
                        ssm_tensor C, ssm_tensor D, ssm_tensor z, ssm_tensor out, int batch,
                        int nheads, int headdim, int dstate, int ngroups, int nslots,
                        int a_per_state, int dt_softplus, const ssm_launch_config *config,
                        void *stream);

/*
 * ssm_decode_step -- one decode token per request: the conv update followed by
 * the state update, in one kernel (the causal-conv1d and silu operators of
 * InfiniLM-Rust PR #48 section 2.1 at seqlen 1, feeding the selective state
 * update of the vLLM PR #50534 report).
 *
 *   x           io dtype [batch, nheads, headdim]: the token's input to the
 *               conv (channel c = h*headdim + p)
 *   conv_state  io dtype [nslots, nheads*headdim, conv_width-1], in/out: the
 *               window before the token, shifted by one on return
 *   conv_weight f32 [nheads*headdim, conv_width]; conv_bias f32 or absent
 *   u_out       io dtype [batch, nheads, headdim] or absent: the conv output
 *   every other argument as in ssm_state_update
 *
 *   u = silu(conv_bias + sum_k conv_weight[c,k] * window_k (newest = x))
 *   then ssm_state_update with x := u.
 * Equals ssm_causal_conv1d (seqlen 1, has_initial_state) followed by
 * ssm_state_update, except that u is passed to the update in float32 instead
 * of being rounded to the io dtype in between.  Limits: conv_width == 4, plus
 * those of ssm_state_update.
 */
int ssm_decode_step(ssm_tensor state, ssm_tensor conv_state, const int32_t *slot_idx,
                    ssm_tensor x, ssm_tensor conv_weight, ssm_tensor conv_bias, int conv_width,
                    ssm_tensor dt, ssm_tensor dt_bias, ssm_tensor A, ssm_tensor B, ssm_tensor C,
                    ssm_tensor D, ssm_tensor z, ssm_tensor out, ssm_tensor u_out, int batch,
                    int nheads, int headdim, int dstate, int ngroups, int nslots,
                    int a_per_state, int dt_softplus, void *stream);

/*
 * Packed variable-length batches (continuous batching).  Several sequences of
 * different lengths are prefilled in one call, each with its own cache slot
 * and its own initial-state flag: the serving pattern of InfiniLM-Rust PR #48
 * (section 3.1 keeps one mamba cache per request; section 4.2, Fig. 2, serves
 * 245 concurrent requests), where requests that already hold a state continue
 * from it.  The pages describe no varlen kernel; the packing is this
 * library's.  The sequences are concatenated along time:
 *
 *   cu_seqlens  int32 [nseq+1], DEVICE memory: sequence s is columns
 *               [cu_seqlens[s], cu_seqlens[s+1]) of every row; the table must
 *               be non-decreasing from 0 to total_len (entries are clamped to
 *               [0, total_len] on the device, so a bad table cannot address
 *               outside the tensors, but overlapping sequences race).  A
 *               sequence of length 0 reads and writes nothing.
 *   slot_idx    int32 [nseq] or NULL (slot s); negative = padded sequence
 *   has_initial_state  int32 [nseq], DEVICE memory, or NULL (none): nonzero =
 *               the sequence continues from the state in its slot
 *
 * Each sequence gives exactly the result of the dense call on that sequence
 * alone (batch 1, seqlen = its length, has_initial_state = its flag).
 */

/*
 * ssm_causal_conv1d_varlen -- ssm_causal_conv1d over a packed batch.
 *   x, out      io dtype [channels, total_len]
 *   other arguments as in ssm_causal_conv1d; the conv cache of each sequence
 *   receives the last width-1 samples of its history || its samples.
 *   Limit: channels <= 65535 (else SSM_ERR_UNSUPPORTED).
 */
int ssm_causal_conv1d_varlen(ssm_tensor x, ssm_tensor weight, ssm_tensor bias,
                             ssm_tensor conv_state, const int32_t *slot_idx,
                             const int32_t *has_initial_state, const int32_t *cu_seqlens,
                             ssm_tensor out, int nseq, int channels, int total_len, int width,
                             int nslots, int apply_silu, void *stream);

/*
 * ssm_selective_scan_varlen -- ssm_selective_scan over a packed batch.
 *   u, z, out   io dtype [nheads*headdim, total_len]
 *   dt          io dtype [nheads, total_len]
 *   B, C        io dtype [ngroups, dstate, total_len]
 *   other arguments as in ssm_selective_scan; each sequence's final state goes
 *   to its slot.  A sequence is walked from the 16-byte vector that holds its
 *   first column, and the neighbouring columns it meets there and in its
 *   last vector enter as identity steps (zero step size, zero-weighted
 *   products): they must hold finite values.  Mamba-2 shapes with f16 or
 *   bf16 I/O take the chunked form (as in ssm_selective_scan_ex).
 */
int ssm_selective_scan_varlen(ssm_tensor u, ssm_tensor dt, ssm_tensor dt_bias, ssm_tensor A,
                              ssm_tensor B, ssm_tensor C, ssm_tensor D, ssm_tensor z,
                              ssm_tensor ssm_state, const int32_t *slot_idx,
                              const int32_t *has_initial_state, const int32_t *cu_seqlens,
                              ssm_tensor out, int nseq, int total_len, int nheads, int headdim,
                              int dstate, int ngroups, int nslots, int a_per_state,
                              int dt_softplus, void *stream);

/*
 * One whole Mamba-1 decode layer around the path, and its two building
 * blocks.  The Mamba-2.8B model of InfiniLM-Rust PR #48 (sections 2.1-2.2)
 * runs its conv and scan operators inside residual layers whose other steps
 * are linear projections and a normalisation; the pages do not spell the
 * layer out, so it is taken as the standard Mamba-1 block (the reading is
 * documented with the tests):
 *   hn        = RMSNorm(hidden) * norm_weight
 *   x | z     = hn . in_proj^T                 in_proj  [2 d_inner, d_model]
 *   u         = silu(conv1d update of x)       (ssm_causal_conv1d, seqlen 1)
 *   dt_low | B | C = u . x_proj^T              x_proj   [dt_rank + 2 d_state, d_inner]
 *   dt        = dt_low . dt_proj^T             dt_proj  [d_inner, dt_rank]
 *   y         = ssm_state_update(u, dt + dt_bias through softplus, A, B, C, D, z)
 *   hidden   += y . out_proj^T                 out_proj [d_model, d_inner]
 * Weights are dense row-major in the io dtype (f16 or bf16; the products run
 * on the matrix cores with float32 accumulation); norm weight, conv weight
 * and bias, dt_bias, A and D are dense float32.  Intermediates between steps
 * are stored in the io dtype in a caller-provided workspace.
 */

/*
 * ssm_linear -- out[M, N] = x[M, K] . weight[N, K]^T (+ residual[M, N]).
 * f16 or bf16 (f32 returns SSM_ERR_UNSUPPORTED); K a multiple of 8; x and
 * weight rows 16-byte aligned (base and row stride); out and residual may be
 * strided views with unit inner stride.  workspace: ssm_linear_workspace(M,
 * N, K) bytes (may be 0 and NULL) of device memory for split-K partial sums;
 * its contents need not be preserved between calls.
 *
 * ssm_linear_ex -- the same with the launch plan given: rows_per_wave (16,
 * 32 or 64), cols_per_workgroup (64 or 128: a workgroup of 4 waves per 64
 * columns takes 4 x rows_per_wave rows) and splits (1 .. min(64, ceil(K /
 * 64)) workgroups along K, partial sums added by a second kernel); 0 for the
 * library's choice of each.  A power of two above 64 rows per wave or 128
 * columns returns SSM_ERR_OUT_OF_RESOURCES (past a wave's accumulator
 * registers or a workgroup's threads), other values SSM_ERR_SHAPE.  Its
 * workspace is ssm_linear_workspace_ex of the same plan (0 for an invalid
 * plan).  For tuning sweeps.
 */
size_t ssm_linear_workspace(int M, int N, int K);
int ssm_linear(ssm_tensor x, ssm_tensor weight, ssm_tensor residual, ssm_tensor out, int M,
               int N, int K, void *workspace, size_t workspace_bytes, void *stream);
size_t ssm_linear_workspace_ex(int M, int N, int K, int rows_per_wave, int cols_per_workgroup,
                               int splits);
/* The plan ssm_linear takes for a shape (each output may be NULL);
 * SSM_ERR_SHAPE for M, N < 1 or K < 8. */
int ssm_linear_plan(int M, int N, int K, int *rows_per_wave, int *cols_per_workgroup,
                    int *splits);
int ssm_linear_ex(ssm_tensor x, ssm_tensor weight, ssm_tensor residual, ssm_tensor out, int M,
                  int N, int K, int rows_per_wave, int cols_per_workgroup, int splits,
                  void *workspace, size_t workspace_bytes, void *stream);

/* ssm_rmsnorm -- out[m, :] = x[m, :] / sqrt(mean(x[m, :]^2) + eps) * weight
 * (weight float32 [D], dense; x, out f16 or bf16 [M, D]). */
int ssm_rmsnorm(ssm_tensor x, ssm_tensor weight, ssm_tensor out, int M, int D, float eps,
                void *stream);

typedef struct ssm_mamba1_layer {
    int d_model, d_inner, d_state, dt_rank, conv_width;
    float norm_eps;
    const float *norm_weight;  /* [d_model]                          */
    const void *in_proj;       /* [2 d_inner, d_model], io dtype     */
    const float *conv_weight;  /* [d_inner, conv_width]              */
    const float *conv_bias;    /* [d_inner] or NULL                  */
    const void *x_proj;        /* [dt_rank + 2 d_state, d_inner]     */
    const void *dt_proj;       /* [d_inner, dt_rank]                 */
    const float *dt_bias;      /* [d_inner] or NULL                  */
    const float *A;            /* [d_inner, d_state]                 */
    const float *D;            /* [d_inner] or NULL                  */
    const void *out_proj;      /* [d_model, d_inner]                 */
} ssm_mamba1_layer;

/* Bytes of workspace ssm_mamba1_decode_layer needs for `batch` requests. */
size_t ssm_mamba1_decode_layer_workspace(const ssm_mamba1_layer *layer,
                                         int batch);

/*
 * ssm_mamba1_decode_layer -- one decode token per request through the whole
 * layer.  hidden [batch, d_model] io dtype (f16 or bf16), updated in place
 * (rows of padded requests, slot < 0, are left as they are); conv_state
 * [nslots, d_inner, conv_width-1] io dtype and ssm_state [nslots, d_inner, 1,
 * d_state] state dtype, read and updated for the named slots.  d_model,
 * d_inner, dt_rank, d_state multiples of 8; conv_width <= 4; d_state <= 512.
 * Every argument of every step is checked before the first launch, so an
 * error leaves hidden and both caches untouched.
 */
int ssm_mamba1_decode_layer(const ssm_mamba1_layer *layer, ssm_tensor hidden,
                            ssm_tensor conv_state, ssm_tensor ssm_state,
                            const int32_t *slot_idx, int batch, int nslots, void *workspace,
                            size_t workspace_bytes, void *stream);

/*
 * ssm_mamba1_decode_layer_noalloc -- ssm_mamba1_decode_layer for callers that
 * cannot allocate device memory (code under HIP graph capture, tight serving
 * loops, harnesses that forbid allocation): the same layer, the same kernels
 * and the same results, with the workspace taken from a device array inside
 * the library instead of a caller buffer.  The array is
 * SSM_LAYER_SCRATCH_BYTES (64 MiB) per GPU, held from the first call on that
 * GPU until the process ends; a layer and batch whose workspace
 * (ssm_mamba1_decode_layer_workspace) exceeds it return
 * SSM_ERR_OUT_OF_RESOURCES before anything is enqueued (the Mamba-2.8B layer
 * fits for up to 687 requests).  Nothing is allocated, by this call or by
 * the library: the first call on a GPU looks up that GPU's copy of the array
 * (an SSM_ERR_HIP if the runtime cannot), later calls reuse it.  Every byte a
 * call reads from the array was written earlier in the same call, so nothing
 * needs clearing between calls; but all calls on one GPU share the one array,
 * so calls that may overlap on a GPU (on different streams, or from several
 * threads) race and must be serialised by the caller.  Other arguments and
 * errors as in ssm_mamba1_decode_layer.
 */
#define SSM_LAYER_SCRATCH_BYTES (64 << 20)
int ssm_mamba1_decode_layer_noalloc(const ssm_mamba1_layer *layer, ssm_tensor hidden,
                                    ssm_tensor conv_state, ssm_tensor ssm_state,
                                    const int32_t *slot_idx, int batch, int nslots,
                                    void *stream);

/*
 * ssm_group_begin / ssm_group_end -- a launch group: calls made between the
 * two on `stream` by this host thread are declared independent of each other
 * (no call reads or writes what another writes), so the library may run them
 * together.  This is the serving step of a batch that holds requests in
 * prefill and requests in decode, each with its own cache slot (the
 * per-request state cache of InfiniLM-Rust PR #48, section 3.1, under the
 * concurrent requests of its section 4.2): one prefill scan and one decode
 * step of the kinds below go out as ONE kernel launch, the decode step's
 * workgroups after the scan's, so that they run in the slots the scan's last
 * round of workgroups leaves free.
 *
 *   Taken together: an ssm_selective_scan or ssm_selective_scan_varlen
 *   that takes the recurrence, with f16 or bf16 io, an f32 state cache,
 *   per-state decays (Mamba-1) and dstate <= 16; and an
 *   ssm_decode_step with the same io dtype, an f32 state cache, per-state
 *   decays and conv_width 4 whose state rows the interleaved map takes
 *   (dstate 8 to 256 in powers of two, at least 2^18 (request, channel)
 *   rows, two requests per lane).  Such a call is validated when made (its
 *   errors are returned then) and held until its partner arrives or the
 *   group ends; every other call launches at once.  A held call's launch
 *   status is returned by the call or ssm_group_end that launches it.  The
 *   values computed are the same, bit for bit, as those of the calls made
 *   outside a group.
 *
 *   The caller keeps every buffer of a held call alive and unchanged until
 *   ssm_group_end has returned (pointers are held, not contents).  Groups do
 *   not nest: ssm_group_begin with a group open, and ssm_group_end without
 *   one or with another stream, return SSM_ERR_UNSUPPORTED.  Host-side only:
 *   the group allocates nothing and is usable under stream capture.
 */
int ssm_group_begin(void *stream);
int ssm_group_end(void *stream);

/* Human-readable text for a status code (static storage; never NULL). */
const char *ssm_status_string(int status);

/* SSM_ABI_VERSION of the built library. */
int ssm_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* SSM_H */
