// ssm_api.hip -- the C ABI declared in include/ssm.h: host-side argument
// validation, launch-geometry choice and dispatch to the gfx950 kernels.
// Everything here runs on the host before any HIP call; a rejected call
// enqueues nothing.
#include "ssm.h"
#include "ssm_kernels.hpp"

#include <stdint.h>

namespace {

bool valid_dtype(int d) { return d == SSM_F32 || d == SSM_F16 || d == SSM_BF16; }
int dtype_size(int d) { return d == SSM_F32 ? 4 : 2; }

bool aligned(const void *p, uintptr_t n) { return p == nullptr || (reinterpret_cast<uintptr_t>(p) % n) == 0; }

int status_of(hipError_t e) { return e == hipSuccess ? SSM_OK : SSM_ERR_HIP; }

// Slot arguments: with a cache, explicit indices need nslots >= 1; implicit
// (slot = b) needs nslots >= batch.
bool slots_ok(const void *cache, const int32_t *slot_idx, int nslots, int batch)
{
    if (!cache)
        return true;
    if (nslots < 1)
        return false;
    return slot_idx != nullptr || nslots >= batch;
}

// Dense batch (cu_seqlens null): x [batch, channels, seqlen].  Packed batch:
// x [channels, seqlen] holding batch sequences at the columns cu_seqlens gives.
int conv_call(const void *x, const float *weight, const float *bias, void *conv_state,
              const int32_t *slot_idx, const int32_t *cu_seqlens, const int32_t *has_init_seq,
              void *out, int batch, int channels, int seqlen, int width, int nslots, int dtype,
              int has_initial_state, int apply_silu, void *stream)
{
    if (!x || !weight || !out)
        return SSM_ERR_NULL_ARG;
    if (!valid_dtype(dtype))
        return SSM_ERR_DTYPE;
    if (batch < 0 || seqlen < 0 || channels < 1 || width < 1)
        return SSM_ERR_SHAPE;
    if (width > ssm::kMaxConvWidth)
        return SSM_ERR_UNSUPPORTED;
    if (!slots_ok(conv_state, slot_idx, nslots, batch))
        return SSM_ERR_SHAPE;
    const int es = dtype_size(dtype);
    if (!aligned(x, es) || !aligned(out, es) || !aligned(conv_state, es) || !aligned(weight, 4) ||
        !aligned(bias, 4) || !aligned(slot_idx, 4) || !aligned(cu_seqlens, 4) ||
        !aligned(has_init_seq, 4))
        return SSM_ERR_ALIGN;
    if ((int64_t)batch * channels > INT32_MAX)
        return SSM_ERR_UNSUPPORTED;
    if (cu_seqlens && channels > 65535)  // packed rows index the grid's y dimension
        return SSM_ERR_UNSUPPORTED;
    if (batch == 0 || seqlen == 0)
        return SSM_OK;
    ssm::ConvArgs a;
    a.x = x;
    a.weight = weight;
    a.bias = bias;
    a.conv_state = conv_state;
    a.slot_idx = slot_idx;
    a.out = out;
    a.cu_seqlens = cu_seqlens;
    a.has_init_seq = has_init_seq;
    a.batch = batch;
    a.channels = channels;
    a.seqlen = seqlen;
    a.width = width;
    a.nslots = nslots;
    a.dtype = dtype;
    a.has_initial_state = has_initial_state ? 1 : 0;
    a.apply_silu = apply_silu ? 1 : 0;
    // dense rows need a length that keeps every row 16-byte aligned; the
    // packed kernel aligns its tiles to each row itself
    a.vec = aligned(x, 16) && aligned(out, 16) && (cu_seqlens || seqlen % 8 == 0);
    a.vec_decode = (seqlen == 1) && (channels % 8 == 0) && aligned(x, 16) && aligned(out, 16) &&
                   aligned(conv_state, 16) && aligned(weight, 16) && aligned(bias, 16);
    return status_of(ssm::launch_conv(a, static_cast<hipStream_t>(stream)));
}

// Dense batch (cu_seqlens null) or packed batch, as for conv_call.
int scan_call(const void *u, const void *dt, const float *dt_bias, const float *A, const void *B,
              const void *C, const float *D, const void *z, void *ssm_state,
              const int32_t *slot_idx, const int32_t *cu_seqlens, const int32_t *has_init_seq,
              void *out, int batch, int seqlen, int nheads, int headdim, int dstate, int ngroups,
              int nslots, int io_dtype, int state_dtype, int a_per_state, int dt_softplus,
              int has_initial_state, void *stream, int algo = SSM_SCAN_AUTO)
{
    if (algo != SSM_SCAN_AUTO && algo != SSM_SCAN_RECURRENT && algo != SSM_SCAN_CHUNKED)
        return SSM_ERR_SHAPE;
    if (!u || !dt || !A || !B || !C || !out)
        return SSM_ERR_NULL_ARG;
    if (!valid_dtype(io_dtype) || !valid_dtype(state_dtype))
        return SSM_ERR_DTYPE;
    if (batch < 0 || seqlen < 0 || nheads < 1 || headdim < 1 || dstate < 1 || ngroups < 1 ||
        nheads % ngroups != 0)
        return SSM_ERR_SHAPE;
    if (dstate > ssm::kMaxScanDstate)
        return SSM_ERR_UNSUPPORTED;
    if (!slots_ok(ssm_state, slot_idx, nslots, batch))
        return SSM_ERR_SHAPE;
    const int es = dtype_size(io_dtype);
    if (!aligned(u, es) || !aligned(dt, es) || !aligned(B, es) || !aligned(C, es) ||
        !aligned(z, es) || !aligned(out, es) || !aligned(ssm_state, dtype_size(state_dtype)) ||
        !aligned(A, 4) || !aligned(D, 4) || !aligned(dt_bias, 4) || !aligned(slot_idx, 4) ||
        !aligned(cu_seqlens, 4) || !aligned(has_init_seq, 4))
        return SSM_ERR_ALIGN;
    const int64_t channels = (int64_t)nheads * headdim;
    const int64_t cpg = channels / ngroups;
    const int64_t nblocks = (int64_t)batch * ngroups * ((cpg + 15) / 16);
    if (channels > INT32_MAX || nblocks > INT32_MAX)
        return SSM_ERR_UNSUPPORTED;
    if (batch == 0 || seqlen == 0)
        return SSM_OK;
    ssm::ScanArgs a;
    a.u = u;
    a.dt = dt;
    a.B = B;
    a.C = C;
    a.z = z;
    a.dt_bias = dt_bias;
    a.A = A;
    a.D = D;
    a.state = ssm_state;
    a.slot_idx = slot_idx;
    a.out = out;
    a.cu_seqlens = cu_seqlens;
    a.has_init_seq = has_init_seq;
    a.batch = batch;
    a.seqlen = seqlen;
    a.nheads = nheads;
    a.headdim = headdim;
    a.dstate = dstate;
    a.ngroups = ngroups;
    a.nslots = nslots;
    a.heads_per_group = nheads / ngroups;
    a.io_dtype = io_dtype;
    a.state_dtype = state_dtype;
    a.a_per_state = a_per_state ? 1 : 0;
    a.dt_softplus = dt_softplus ? 1 : 0;
    a.has_initial_state = has_initial_state ? 1 : 0;
    a.vec = (seqlen % 8 == 0) && aligned(u, 16) && aligned(dt, 16) && aligned(B, 16) &&
            aligned(C, 16) && aligned(z, 16) && aligned(out, 16);
    const bool chunked = ssm::ssd_supported(a);
    if (algo == SSM_SCAN_CHUNKED && !chunked)
        return SSM_ERR_UNSUPPORTED;
    if (chunked && algo != SSM_SCAN_RECURRENT)
        return status_of(ssm::launch_ssd(a, static_cast<hipStream_t>(stream)));
    return status_of(ssm::launch_scan(a, static_cast<hipStream_t>(stream)));
}

} // namespace

extern "C" {

int ssm_abi_version(void) { return SSM_ABI_VERSION; }

const char *ssm_status_string(int status)
{
    switch (status) {
    case SSM_OK: return "ok";
    case SSM_ERR_NULL_ARG: return "a required pointer is NULL";
    case SSM_ERR_SHAPE: return "a size is out of range or sizes disagree";
    case SSM_ERR_DTYPE: return "unknown dtype code";
    case SSM_ERR_ALIGN: return "a pointer is not aligned to its element size";
    case SSM_ERR_UNSUPPORTED: return "a size beyond what the kernels are built for";
    case SSM_ERR_HIP: return "the HIP runtime refused a launch";
    default: return "unknown status";
    }
}

int ssm_causal_conv1d(const void *x, const float *weight, const float *bias, void *conv_state,
                      const int32_t *slot_idx, void *out, int batch, int channels, int seqlen,
                      int width, int nslots, int dtype, int has_initial_state, int apply_silu,
                      void *stream)
{
    return conv_call(x, weight, bias, conv_state, slot_idx, nullptr, nullptr, out, batch, channels,
                     seqlen, width, nslots, dtype, has_initial_state, apply_silu, stream);
}

int ssm_causal_conv1d_varlen(const void *x, const float *weight, const float *bias,
                             void *conv_state, const int32_t *slot_idx,
                             const int32_t *has_initial_state, const int32_t *cu_seqlens,
                             void *out, int nseq, int channels, int total_len, int width,
                             int nslots, int dtype, int apply_silu, void *stream)
{
    if (!cu_seqlens)
        return SSM_ERR_NULL_ARG;
    return conv_call(x, weight, bias, conv_state, slot_idx, cu_seqlens, has_initial_state, out,
                     nseq, channels, total_len, width, nslots, dtype, 0, apply_silu, stream);
}

int ssm_selective_scan(const void *u, const void *dt, const float *dt_bias, const float *A,
                       const void *B, const void *C, const float *D, const void *z, void *ssm_state,
                       const int32_t *slot_idx, void *out, int batch, int seqlen, int nheads,
                       int headdim, int dstate, int ngroups, int nslots, int io_dtype,
                       int state_dtype, int a_per_state, int dt_softplus, int has_initial_state,
                       void *stream)
{
    return scan_call(u, dt, dt_bias, A, B, C, D, z, ssm_state, slot_idx, nullptr, nullptr, out,
                     batch, seqlen, nheads, headdim, dstate, ngroups, nslots, io_dtype,
                     state_dtype, a_per_state, dt_softplus, has_initial_state, stream);
}

int ssm_selective_scan_ex(const void *u, const void *dt, const float *dt_bias, const float *A,
                          const void *B, const void *C, const float *D, const void *z,
                          void *ssm_state, const int32_t *slot_idx, void *out, int batch,
                          int seqlen, int nheads, int headdim, int dstate, int ngroups, int nslots,
                          int io_dtype, int state_dtype, int a_per_state, int dt_softplus,
                          int has_initial_state, int algo, void *stream)
{
    return scan_call(u, dt, dt_bias, A, B, C, D, z, ssm_state, slot_idx, nullptr, nullptr, out,
                     batch, seqlen, nheads, headdim, dstate, ngroups, nslots, io_dtype,
                     state_dtype, a_per_state, dt_softplus, has_initial_state, stream, algo);
}

int ssm_selective_scan_varlen(const void *u, const void *dt, const float *dt_bias,
                              const float *A, const void *B, const void *C, const float *D,
                              const void *z, void *ssm_state, const int32_t *slot_idx,
                              const int32_t *has_initial_state, const int32_t *cu_seqlens,
                              void *out, int nseq, int total_len, int nheads, int headdim,
                              int dstate, int ngroups, int nslots, int io_dtype, int state_dtype,
                              int a_per_state, int dt_softplus, void *stream)
{
    if (!cu_seqlens)
        return SSM_ERR_NULL_ARG;
    return scan_call(u, dt, dt_bias, A, B, C, D, z, ssm_state, slot_idx, cu_seqlens,
                     has_initial_state, out, nseq, total_len, nheads, headdim, dstate, ngroups,
                     nslots, io_dtype, state_dtype, a_per_state, dt_softplus, 0, stream);
}

} // extern "C"

namespace {

// ----------------------------------------------------------- SSU geometry
// One tuned entry: for the key (headdim, dstate, io dtype, cache dtype) and
// effective batches (batch x nheads) in (eff_lo, eff_hi], use this geometry.
struct SsuTableEntry {
    int headdim, dstate, io_dtype, state_dtype;
    int64_t eff_lo, eff_hi;
    int states_per_lane, block_threads;
};

// The gfx950 table, written by state_space_model_causal_amd/tune_ssu.py from
// measurements on an MI355X; only entries that beat the heuristic are kept.
const SsuTableEntry kSsuTable[] = {
#include "ssu_table_gfx950.inc"
    {0, 0, 0, 0, 0, 0, 0, 0}  // end marker
};

bool valid_ssu_config(int V, int block, int state_dtype, int dstate)
{
    // 4 states per lane only for a 4-byte cache (one 16-byte vector); a row's
    // lanes must fit in one wave (the readout sum is a butterfly within it)
    return (V == 8 || V == 16 || (V == 4 && dtype_size(state_dtype) == 4)) && (dstate + V - 1) / V <= 64 &&
           (block == 64 || block == 128 || block == 256 || block == 512);
}

// The library's choice: the table entry covering the shape, else the
// heuristic: 32 bytes of state per lane (16 states of a 2-byte cache, for rows
// of >= 32 states that are a multiple of 16; else 8 states) in 256-lane
// workgroups.
void choose_ssu(int batch, int nheads, int headdim, int dstate, int io_dtype, int state_dtype,
                int &V, int &block, int &from_table)
{
    const int64_t eff = (int64_t)batch * nheads;
    for (const SsuTableEntry *e = kSsuTable; e->headdim != 0; ++e) {
        if (e->headdim == headdim && e->dstate == dstate && e->io_dtype == io_dtype &&
            e->state_dtype == state_dtype && eff > e->eff_lo && eff <= e->eff_hi &&
            valid_ssu_config(e->states_per_lane, e->block_threads, state_dtype, dstate)) {
            V = e->states_per_lane;
            block = e->block_threads;
            from_table = 1;
            return;
        }
    }
    V = (dtype_size(state_dtype) == 2 && dstate % 16 == 0 && dstate >= 32) ? 16 : 8;
    block = 256;
    from_table = 0;
}

// Requests each lane takes in turn.  With one channel per head (headdim 1)
// a row is only dstate states, so the row's parameters (A, D, dt_bias, the
// conv taps) cost as much to fetch as its state: two requests per lane fetch
// them once for both (7% faster on the 245-request Mamba-1 2.8B decode step).
// Wider heads keep one request per lane (two were 2-5% slower there).
int ssu_requests_per_lane(int batch, int headdim)
{
    return (headdim == 1 && batch >= 8) ? 2 : 1;
}

// Validation and launch geometry shared by ssm_state_update(_ex) and
// ssm_decode_step; fills `a` and returns SSM_OK, or an error status.
// cfg: the caller's geometry, or null for the library's choice.
int prepare_ssu(ssm::SsuArgs &a, void *state, const int32_t *slot_idx, const void *x,
                const void *dt, const float *dt_bias, const float *A, const void *B,
                const void *C, const float *D, const void *z, void *out, int batch, int nheads,
                int headdim, int dstate, int ngroups, int nslots, int io_dtype, int state_dtype,
                int a_per_state, int dt_softplus, const ssm_launch_config *cfg = nullptr)
{
    if (!state || !x || !dt || !A || !B || !C || !out)
        return SSM_ERR_NULL_ARG;
    if (!valid_dtype(io_dtype) || !valid_dtype(state_dtype))
        return SSM_ERR_DTYPE;
    if (batch < 0 || nheads < 1 || headdim < 1 || dstate < 1 || ngroups < 1 ||
        nheads % ngroups != 0)
        return SSM_ERR_SHAPE;
    if (dstate > ssm::kMaxSsuDstate)
        return SSM_ERR_UNSUPPORTED;
    if (!slots_ok(state, slot_idx, nslots, batch))
        return SSM_ERR_SHAPE;
    const int es = dtype_size(io_dtype), ss = dtype_size(state_dtype);
    if (!aligned(state, ss) || !aligned(x, es) || !aligned(dt, es) || !aligned(B, es) ||
        !aligned(C, es) || !aligned(z, es) || !aligned(out, es) || !aligned(A, 4) ||
        !aligned(D, 4) || !aligned(dt_bias, 4) || !aligned(slot_idx, 4))
        return SSM_ERR_ALIGN;
    int V, block, from_table;
    if (cfg) {
        if (!valid_ssu_config(cfg->states_per_lane, cfg->block_threads, state_dtype, dstate))
            return SSM_ERR_SHAPE;
        V = cfg->states_per_lane;
        block = cfg->block_threads;
    } else {
        choose_ssu(batch, nheads, headdim, dstate, io_dtype, state_dtype, V, block, from_table);
    }
    // lanes per (b,h,p) row: ceil(dstate/V) rounded up to a power of two (<= 64)
    int lanes = (dstate + V - 1) / V, lg = 0;
    while ((1 << lg) < lanes)
        ++lg;
    const int64_t nrows = (int64_t)batch * nheads * headdim;
    const int rb = ssu_requests_per_lane(batch, headdim);
    if (((((int64_t)nheads * headdim) << lg) + 63) / 64 > INT32_MAX || (batch + rb - 1) / rb > 65535)
        return SSM_ERR_UNSUPPORTED;
    a = ssm::SsuArgs{};
    a.state = state;
    a.slot_idx = slot_idx;
    a.x = x;
    a.dt = dt;
    a.B = B;
    a.C = C;
    a.z = z;
    a.dt_bias = dt_bias;
    a.A = A;
    a.D = D;
    a.out = out;
    a.nrows = nrows;
    a.batch = batch;
    a.nheads = nheads;
    a.headdim = headdim;
    a.dstate = dstate;
    a.ngroups = ngroups;
    a.nslots = nslots;
    a.heads_per_group = nheads / ngroups;
    a.lanes_per_row_log2 = lg;
    a.states_per_lane = V;
    a.block_threads = block;
    a.io_dtype = io_dtype;
    a.state_dtype = state_dtype;
    a.a_per_state = a_per_state ? 1 : 0;
    a.dt_softplus = dt_softplus ? 1 : 0;
    a.vec = (dstate % V == 0) && aligned(state, 16) && aligned(B, 16) && aligned(C, 16) &&
            aligned(A, 16);
    a.requests_per_lane = rb;
    a.conv_width = 0;
    return SSM_OK;
}

} // namespace

extern "C" {

int ssm_state_update(void *state, const int32_t *slot_idx, const void *x, const void *dt,
                     const float *dt_bias, const float *A, const void *B, const void *C,
                     const float *D, const void *z, void *out, int batch, int nheads, int headdim,
                     int dstate, int ngroups, int nslots, int io_dtype, int state_dtype,
                     int a_per_state, int dt_softplus, void *stream)
{
    ssm::SsuArgs a;
    const int st = prepare_ssu(a, state, slot_idx, x, dt, dt_bias, A, B, C, D, z, out, batch,
                               nheads, headdim, dstate, ngroups, nslots, io_dtype, state_dtype,
                               a_per_state, dt_softplus);
    if (st != SSM_OK)
        return st;
    if (batch == 0)
        return SSM_OK;
    return status_of(ssm::launch_ssu(a, static_cast<hipStream_t>(stream)));
}

int ssm_state_update_ex(void *state, const int32_t *slot_idx, const void *x, const void *dt,
                        const float *dt_bias, const float *A, const void *B, const void *C,
                        const float *D, const void *z, void *out, int batch, int nheads,
                        int headdim, int dstate, int ngroups, int nslots, int io_dtype,
                        int state_dtype, int a_per_state, int dt_softplus,
                        const ssm_launch_config *config, void *stream)
{
    ssm::SsuArgs a;
    const int st = prepare_ssu(a, state, slot_idx, x, dt, dt_bias, A, B, C, D, z, out, batch,
                               nheads, headdim, dstate, ngroups, nslots, io_dtype, state_dtype,
                               a_per_state, dt_softplus, config);
    if (st != SSM_OK)
        return st;
    if (batch == 0)
        return SSM_OK;
    return status_of(ssm::launch_ssu(a, static_cast<hipStream_t>(stream)));
}

int ssm_state_update_config(int batch, int nheads, int headdim, int dstate, int io_dtype,
                            int state_dtype, ssm_launch_config *config, int *from_table)
{
    if (!config)
        return SSM_ERR_NULL_ARG;
    if (!valid_dtype(io_dtype) || !valid_dtype(state_dtype))
        return SSM_ERR_DTYPE;
    if (batch < 0 || nheads < 1 || headdim < 1 || dstate < 1)
        return SSM_ERR_SHAPE;
    if (dstate > ssm::kMaxSsuDstate)
        return SSM_ERR_UNSUPPORTED;
    int V, block, ft;
    choose_ssu(batch, nheads, headdim, dstate, io_dtype, state_dtype, V, block, ft);
    config->states_per_lane = V;
    config->block_threads = block;
    if (from_table)
        *from_table = ft;
    return SSM_OK;
}

int ssm_decode_step(void *state, void *conv_state, const int32_t *slot_idx, const void *x,
                    const float *conv_weight, const float *conv_bias, int conv_width,
                    const void *dt, const float *dt_bias, const float *A, const void *B,
                    const void *C, const float *D, const void *z, void *out, void *u_out,
                    int batch, int nheads, int headdim, int dstate, int ngroups, int nslots,
                    int io_dtype, int state_dtype, int a_per_state, int dt_softplus, void *stream)
{
    ssm::SsuArgs a;
    const int st = prepare_ssu(a, state, slot_idx, x, dt, dt_bias, A, B, C, D, z, out, batch,
                               nheads, headdim, dstate, ngroups, nslots, io_dtype, state_dtype,
                               a_per_state, dt_softplus);
    if (st != SSM_OK)
        return st;
    if (!conv_state || !conv_weight)
        return SSM_ERR_NULL_ARG;
    if (conv_width < 1)
        return SSM_ERR_SHAPE;
    if (conv_width != ssm::kFusedConvWidth)
        return SSM_ERR_UNSUPPORTED;
    const int es = dtype_size(io_dtype);
    if (!aligned(conv_state, es) || !aligned(u_out, es) || !aligned(conv_weight, 4) ||
        !aligned(conv_bias, 4))
        return SSM_ERR_ALIGN;
    if (batch == 0)
        return SSM_OK;
    a.conv_state = conv_state;
    a.conv_weight = conv_weight;
    a.conv_bias = conv_bias;
    a.u_out = u_out;
    a.conv_width = conv_width;
    return status_of(ssm::launch_ssu(a, static_cast<hipStream_t>(stream)));
}

} // extern "C"
