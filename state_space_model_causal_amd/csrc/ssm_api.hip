// ssm_api.hip -- the C ABI declared in include/ssm.h: host-side argument
// validation, launch-geometry choice and dispatch to the gfx950 kernels.
// Everything here runs on the host before any HIP call; a rejected call
// enqueues nothing.
#include "ssm.h"
#include "ssm_kernels.hpp"

#include <stdint.h>

namespace ssm {

namespace {

bool valid_dtype(int d) { return d == SSM_F32 || d == SSM_F16 || d == SSM_BF16; }
int dtype_size(int d) { return d == SSM_F32 ? 4 : 2; }
bool present(const ssm_tensor &t) { return t.data != nullptr; }
bool aligned(const void *p, uintptr_t n) { return p == nullptr || (reinterpret_cast<uintptr_t>(p) % n) == 0; }

// One tensor argument against its documented shape: dtype, layout and
// alignment.  `want` is the dtype it must have (-1: any valid io dtype, the
// caller compares io tensors with one another).  A dimension of size 1 may
// have any stride; the innermost one of any larger size must be contiguous.
int check_tensor(const ssm_tensor &t, int rank, const int64_t *size, int want)
{
    if (!present(t))
        return SSM_OK;
    if (!valid_dtype(t.dtype) || (want >= 0 && t.dtype != want))
        return SSM_ERR_DTYPE;
    for (int i = 0; i < rank; ++i)
        if (t.stride[i] < 0)
            return SSM_ERR_LAYOUT;
    if (rank > 0 && size[rank - 1] > 1 && t.stride[rank - 1] != 1)
        return SSM_ERR_LAYOUT;
    if (!aligned(t.data, dtype_size(t.dtype)))
        return SSM_ERR_ALIGN;
    return SSM_OK;
}

// Rows of 16-byte vectors: the base and every outer stride (of a dimension
// of size > 1) a multiple of 16 bytes.
bool rows16(const ssm_tensor &t, int rank, const int64_t *size)
{
    if (!present(t))
        return true;
    if (!aligned(t.data, 16))
        return false;
    const int es = dtype_size(t.dtype);
    for (int i = 0; i + 1 < rank; ++i)
        if (size[i] > 1 && (t.stride[i] * es) % 16 != 0)
            return false;
    return true;
}

// Stride of dimension i, or 0 for an absent tensor.
int64_t st(const ssm_tensor &t, int i) { return present(t) ? t.stride[i] : 0; }

// The first non-OK status of a list of checks.
#define SSM_TRY(expr)                 \
    do {                              \
        const int st_ = (expr);       \
        if (st_ != SSM_OK)            \
            return st_;               \
    } while (0)

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

} // namespace

int status_of(hipError_t e) { return e == hipSuccess ? SSM_OK : SSM_ERR_HIP; }

// Dense batch (cu_seqlens null): x [batch, channels, seqlen].  Packed batch:
// x [channels, seqlen] holding batch sequences at the columns cu_seqlens gives.
int prepare_conv(ConvArgs &a, const ssm_tensor &x, const ssm_tensor &weight, const ssm_tensor &bias,
                 const ssm_tensor &conv_state, const int32_t *slot_idx, const int32_t *cu_seqlens,
                 const int32_t *has_init_seq, const ssm_tensor &out, int batch, int channels, int seqlen,
                 int width, int nslots, int has_initial_state, int apply_silu)
{
    if (!present(x) || !present(weight) || !present(out))
        return SSM_ERR_NULL_ARG;
    if (batch < 0 || seqlen < 0 || channels < 1 || width < 1)
        return SSM_ERR_SHAPE;
    if (width > kMaxConvWidth)
        return SSM_ERR_UNSUPPORTED;
    if (!slots_ok(conv_state.data, slot_idx, nslots, batch))
        return SSM_ERR_SHAPE;
    const bool packed = cu_seqlens != nullptr;
    const int dtype = x.dtype;
    // x, out: [batch, channels, seqlen], or [channels, seqlen] packed
    const int64_t xs3[3] = {batch, channels, seqlen}, xs2[2] = {channels, seqlen};
    const int xr = packed ? 2 : 3;
    const int64_t *xs = packed ? xs2 : xs3;
    const int64_t ws[2] = {channels, width}, bs[1] = {channels};
    const int64_t cs[3] = {nslots, channels, width - 1};
    SSM_TRY(check_tensor(x, xr, xs, -1));
    SSM_TRY(check_tensor(out, xr, xs, dtype));
    SSM_TRY(check_tensor(conv_state, 3, cs, dtype));
    SSM_TRY(check_tensor(weight, 2, ws, SSM_F32));
    SSM_TRY(check_tensor(bias, 1, bs, SSM_F32));
    if (!aligned(slot_idx, 4) || !aligned(cu_seqlens, 4) || !aligned(has_init_seq, 4))
        return SSM_ERR_ALIGN;
    if ((int64_t)batch * channels > INT32_MAX)
        return SSM_ERR_UNSUPPORTED;
    if (packed && channels > 65535)  // packed rows index the grid's y dimension
        return SSM_ERR_UNSUPPORTED;
    a = ConvArgs{};
    a.x = x.data;
    a.weight = static_cast<const float *>(weight.data);
    a.bias = static_cast<const float *>(bias.data);
    a.conv_state = conv_state.data;
    a.slot_idx = slot_idx;
    a.out = out.data;
    a.x_sb = packed ? 0 : x.stride[0];
    a.x_sc = x.stride[packed ? 0 : 1];
    a.o_sb = packed ? 0 : out.stride[0];
    a.o_sc = out.stride[packed ? 0 : 1];
    a.cs_ss = st(conv_state, 0);
    a.cs_sc = st(conv_state, 1);
    a.w_sc = weight.stride[0];
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
    const int es = dtype_size(dtype), E = 16 / es;
    const bool r16 = rows16(x, xr, xs) && rows16(out, xr, xs);
    a.rows16 = r16 && seqlen % E == 0;
    if (packed) {
        // the packed walks shift every row by its start's offset within a
        // vector, which must be the same for x and out
        a.vec = r16 || (aligned(x.data, 16) && aligned(out.data, 16) && a.x_sc == a.o_sc);
    } else {
        // dense rows need a length that keeps every row 16-byte aligned
        a.vec = r16 && seqlen % E == 0;
    }
    // decode: 8 consecutive channels per 128-bit access of x, out, the
    // window rows and the taps
    const int H = width - 1;
    a.vec_decode = !packed && seqlen == 1 && channels % 8 == 0 && aligned(x.data, 16) &&
                   aligned(out.data, 16) && (channels == 1 || (a.x_sc == 1 && a.o_sc == 1)) &&
                   (a.x_sb * es) % 16 == 0 && (a.o_sb * es) % 16 == 0 && a.w_sc == width &&
                   aligned(weight.data, 16) && aligned(bias.data, 16) &&
                   (!present(conv_state) || (aligned(conv_state.data, 16) && (H == 0 || a.cs_sc == H) &&
                                             (a.cs_ss * es) % 16 == 0));
    return SSM_OK;
}

// Dense batch (cu_seqlens null) or packed batch, as for prepare_conv.
int prepare_scan(ScanArgs &a, const ssm_tensor &u, const ssm_tensor &dt, const ssm_tensor &dt_bias,
                 const ssm_tensor &A, const ssm_tensor &B, const ssm_tensor &C, const ssm_tensor &D,
                 const ssm_tensor &z, const ssm_tensor &ssm_state, const int32_t *slot_idx,
                 const int32_t *cu_seqlens, const int32_t *has_init_seq, const ssm_tensor &out, int batch,
                 int seqlen, int nheads, int headdim, int dstate, int ngroups, int nslots, int a_per_state,
                 int dt_softplus, int has_initial_state)
{
    if (!present(u) || !present(dt) || !present(A) || !present(B) || !present(C) || !present(out))
        return SSM_ERR_NULL_ARG;
    if (batch < 0 || seqlen < 0 || nheads < 1 || headdim < 1 || dstate < 1 || ngroups < 1 ||
        nheads % ngroups != 0)
        return SSM_ERR_SHAPE;
    if (dstate > kMaxScanDstate)
        return SSM_ERR_OUT_OF_RESOURCES;  // the carried states live in LDS
    if (!slots_ok(ssm_state.data, slot_idx, nslots, batch))
        return SSM_ERR_SHAPE;
    const bool packed = cu_seqlens != nullptr;
    const int io = u.dtype;
    const int64_t Cn = (int64_t)nheads * headdim;
    // dense shapes, or the packed ones (no batch dimension)
    const int64_t us3[3] = {batch, Cn, seqlen}, us2[2] = {Cn, seqlen};
    const int64_t ds3[3] = {batch, nheads, seqlen}, ds2[2] = {nheads, seqlen};
    const int64_t bs4[4] = {batch, ngroups, dstate, seqlen}, bs3[3] = {ngroups, dstate, seqlen};
    const int o = packed ? 1 : 0;  // rank offset
    const int64_t as2[2] = {nheads, dstate}, as1[1] = {nheads};
    const int64_t ss[4] = {nslots, nheads, headdim, dstate};
    SSM_TRY(check_tensor(u, 3 - o, packed ? us2 : us3, -1));
    SSM_TRY(check_tensor(z, 3 - o, packed ? us2 : us3, io));
    SSM_TRY(check_tensor(out, 3 - o, packed ? us2 : us3, io));
    SSM_TRY(check_tensor(dt, 3 - o, packed ? ds2 : ds3, io));
    SSM_TRY(check_tensor(B, 4 - o, packed ? bs3 : bs4, io));
    SSM_TRY(check_tensor(C, 4 - o, packed ? bs3 : bs4, io));
    SSM_TRY(check_tensor(A, a_per_state ? 2 : 1, a_per_state ? as2 : as1, SSM_F32));
    SSM_TRY(check_tensor(D, 1, as1, SSM_F32));
    SSM_TRY(check_tensor(dt_bias, 1, as1, SSM_F32));
    SSM_TRY(check_tensor(ssm_state, 4, ss, -1));
    if (!aligned(slot_idx, 4) || !aligned(cu_seqlens, 4) || !aligned(has_init_seq, 4))
        return SSM_ERR_ALIGN;
    const int64_t cpg = Cn / ngroups;
    const int64_t nblocks = (int64_t)batch * ngroups * ((cpg + 15) / 16);
    if (Cn > INT32_MAX || nblocks > INT32_MAX)
        return SSM_ERR_UNSUPPORTED;
    a = ScanArgs{};
    a.u = u.data;
    a.dt = dt.data;
    a.B = B.data;
    a.C = C.data;
    a.z = z.data;
    a.dt_bias = static_cast<const float *>(dt_bias.data);
    a.A = static_cast<const float *>(A.data);
    a.D = static_cast<const float *>(D.data);
    a.state = ssm_state.data;
    a.slot_idx = slot_idx;
    a.out = out.data;
    a.u_sb = packed ? 0 : u.stride[0];
    a.u_sc = u.stride[1 - o];
    a.z_sb = packed ? 0 : st(z, 0);
    a.z_sc = st(z, 1 - o);
    a.o_sb = packed ? 0 : out.stride[0];
    a.o_sc = out.stride[1 - o];
    a.dt_sb = packed ? 0 : dt.stride[0];
    a.dt_sh = dt.stride[1 - o];
    a.B_sb = packed ? 0 : B.stride[0];
    a.B_sg = B.stride[1 - o];
    a.B_sn = B.stride[2 - o];
    a.C_sb = packed ? 0 : C.stride[0];
    a.C_sg = C.stride[1 - o];
    a.C_sn = C.stride[2 - o];
    a.A_sh = a_per_state ? A.stride[0] : 1;
    a.st_ss = st(ssm_state, 0);
    a.st_sh = st(ssm_state, 1);
    a.st_sp = st(ssm_state, 2);
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
    a.io_dtype = io;
    a.state_dtype = present(ssm_state) ? ssm_state.dtype : SSM_F32;
    a.a_per_state = a_per_state ? 1 : 0;
    a.dt_softplus = dt_softplus ? 1 : 0;
    a.has_initial_state = has_initial_state ? 1 : 0;
    const int E = 16 / dtype_size(io);
    const int ur = 3 - o, br = 4 - o;
    const int64_t *usz = packed ? us2 : us3, *dsz = packed ? ds2 : ds3, *bsz = packed ? bs3 : bs4;
    a.vec = (seqlen % E == 0) && rows16(u, ur, usz) && rows16(z, ur, usz) && rows16(out, ur, usz) &&
            rows16(dt, ur, dsz) && rows16(B, br, bsz) && rows16(C, br, bsz);
    return SSM_OK;
}

} // namespace ssm

namespace {

using ssm::prepare_conv;
using ssm::prepare_scan;
using ssm::status_of;

int conv_call(const ssm_tensor &x, const ssm_tensor &weight, const ssm_tensor &bias,
              const ssm_tensor &conv_state, const int32_t *slot_idx, const int32_t *cu_seqlens,
              const int32_t *has_init_seq, const ssm_tensor &out, int batch, int channels, int seqlen,
              int width, int nslots, int has_initial_state, int apply_silu, void *stream)
{
    ssm::ConvArgs a;
    SSM_TRY(prepare_conv(a, x, weight, bias, conv_state, slot_idx, cu_seqlens, has_init_seq, out, batch,
                         channels, seqlen, width, nslots, has_initial_state, apply_silu));
    if (batch == 0 || seqlen == 0)
        return SSM_OK;
    return status_of(ssm::launch_conv(a, static_cast<hipStream_t>(stream)));
}

// The open launch group of this host thread (ssm_group_begin / _end): at
// most one held scan and one held decode step of the kinds the mixed kernel
// takes; a held pair goes out as one mixed launch as soon as both are there.
struct LaunchGroup {
    bool open = false;
    void *stream = nullptr;
    bool has_scan = false, has_decode = false;
    ssm::ScanArgs scan;
    ssm::SsuArgs decode;
};
thread_local LaunchGroup g_group;

// A scan handed to the open group: true when the group now holds it or has
// launched it with its held decode step (*st = that launch's status); false
// when the caller launches it itself.
bool group_take_scan(const ssm::ScanArgs &a, void *stream, int *st)
{
    LaunchGroup &g = g_group;
    if (!g.open || g.stream != stream || !ssm::mixed_scan_ok(a))
        return false;
    if (g.has_decode && ssm::mixed_pair_ok(a, g.decode)) {
        g.has_decode = false;
        *st = status_of(ssm::launch_mixed(a, g.decode, static_cast<hipStream_t>(stream)));
        return true;
    }
    if (g.has_scan)
        return false;
    g.scan = a;
    g.has_scan = true;
    *st = SSM_OK;
    return true;
}

bool group_take_decode(const ssm::SsuArgs &a, void *stream, int *st)
{
    LaunchGroup &g = g_group;
    if (!g.open || g.stream != stream || !ssm::mixed_decode_ok(a))
        return false;
    if (g.has_scan && ssm::mixed_pair_ok(g.scan, a)) {
        g.has_scan = false;
        *st = status_of(ssm::launch_mixed(g.scan, a, static_cast<hipStream_t>(stream)));
        return true;
    }
    if (g.has_decode)
        return false;
    g.decode = a;
    g.has_decode = true;
    *st = SSM_OK;
    return true;
}

int scan_call(const ssm_tensor &u, const ssm_tensor &dt, const ssm_tensor &dt_bias, const ssm_tensor &A,
              const ssm_tensor &B, const ssm_tensor &C, const ssm_tensor &D, const ssm_tensor &z,
              const ssm_tensor &ssm_state, const int32_t *slot_idx, const int32_t *cu_seqlens,
              const int32_t *has_init_seq, const ssm_tensor &out, int batch, int seqlen, int nheads,
              int headdim, int dstate, int ngroups, int nslots, int a_per_state, int dt_softplus,
              int has_initial_state, void *stream, int algo = SSM_SCAN_AUTO)
{
    if (algo != SSM_SCAN_AUTO && algo != SSM_SCAN_RECURRENT && algo != SSM_SCAN_CHUNKED)
        return SSM_ERR_SHAPE;
    ssm::ScanArgs a;
    SSM_TRY(prepare_scan(a, u, dt, dt_bias, A, B, C, D, z, ssm_state, slot_idx, cu_seqlens, has_init_seq,
                         out, batch, seqlen, nheads, headdim, dstate, ngroups, nslots, a_per_state,
                         dt_softplus, has_initial_state));
    const bool chunked = ssm::ssd_supported(a);
    if (algo == SSM_SCAN_CHUNKED && !chunked)
        return SSM_ERR_UNSUPPORTED;
    if (batch == 0 || seqlen == 0)
        return SSM_OK;
    if (chunked && algo != SSM_SCAN_RECURRENT)
        return status_of(ssm::launch_ssd(a, static_cast<hipStream_t>(stream)));
    int st;
    if (group_take_scan(a, stream, &st))
        return st;
    return status_of(ssm::launch_scan(a, static_cast<hipStream_t>(stream)));
}

} // namespace

extern "C" {

int ssm_abi_version(void) { return SSM_ABI_VERSION; }

const char *ssm_status_string(int status)
{
    switch (status) {
    case SSM_OK: return "ok";
    case SSM_ERR_NULL_ARG: return "a required tensor or pointer is NULL";
    case SSM_ERR_SHAPE: return "a size is out of range or sizes disagree";
    case SSM_ERR_DTYPE: return "unknown dtype code, or dtypes that must agree differ";
    case SSM_ERR_ALIGN: return "a pointer is not aligned to its element size";
    case SSM_ERR_UNSUPPORTED: return "a size or variant the kernels are not built for";
    case SSM_ERR_HIP: return "the HIP runtime refused a launch";
    case SSM_ERR_LAYOUT: return "an innermost stride is not 1, or a stride is negative";
    case SSM_ERR_OUT_OF_RESOURCES:
        return "a launch geometry beyond the kernels' register, LDS or workgroup-size budget";
    default: return "unknown status";
    }
}

int ssm_causal_conv1d(ssm_tensor x, ssm_tensor weight, ssm_tensor bias, ssm_tensor conv_state,
                      const int32_t *slot_idx, ssm_tensor out, int batch, int channels, int seqlen,
                      int width, int nslots, int has_initial_state, int apply_silu, void *stream)
{
    return conv_call(x, weight, bias, conv_state, slot_idx, nullptr, nullptr, out, batch, channels,
                     seqlen, width, nslots, has_initial_state, apply_silu, stream);
}

int ssm_causal_conv1d_varlen(ssm_tensor x, ssm_tensor weight, ssm_tensor bias, ssm_tensor conv_state,
                             const int32_t *slot_idx, const int32_t *has_initial_state,
                             const int32_t *cu_seqlens, ssm_tensor out, int nseq, int channels,
                             int total_len, int width, int nslots, int apply_silu, void *stream)
{
    if (!cu_seqlens)
        return SSM_ERR_NULL_ARG;
    return conv_call(x, weight, bias, conv_state, slot_idx, cu_seqlens, has_initial_state, out, nseq,
                     channels, total_len, width, nslots, 0, apply_silu, stream);
}

int ssm_selective_scan(ssm_tensor u, ssm_tensor dt, ssm_tensor dt_bias, ssm_tensor A, ssm_tensor B,
                       ssm_tensor C, ssm_tensor D, ssm_tensor z, ssm_tensor ssm_state,
                       const int32_t *slot_idx, ssm_tensor out, int batch, int seqlen, int nheads,
                       int headdim, int dstate, int ngroups, int nslots, int a_per_state,
                       int dt_softplus, int has_initial_state, void *stream)
{
    return scan_call(u, dt, dt_bias, A, B, C, D, z, ssm_state, slot_idx, nullptr, nullptr, out, batch,
                     seqlen, nheads, headdim, dstate, ngroups, nslots, a_per_state, dt_softplus,
                     has_initial_state, stream);
}

int ssm_selective_scan_ex(ssm_tensor u, ssm_tensor dt, ssm_tensor dt_bias, ssm_tensor A, ssm_tensor B,
                          ssm_tensor C, ssm_tensor D, ssm_tensor z, ssm_tensor ssm_state,
                          const int32_t *slot_idx, ssm_tensor out, int batch, int seqlen, int nheads,
                          int headdim, int dstate, int ngroups, int nslots, int a_per_state,
                          int dt_softplus, int has_initial_state, int algo, void *stream)
{
    return scan_call(u, dt, dt_bias, A, B, C, D, z, ssm_state, slot_idx, nullptr, nullptr, out, batch,
                     seqlen, nheads, headdim, dstate, ngroups, nslots, a_per_state, dt_softplus,
                     has_initial_state, stream, algo);
}

int ssm_selective_scan_varlen(ssm_tensor u, ssm_tensor dt, ssm_tensor dt_bias, ssm_tensor A,
                              ssm_tensor B, ssm_tensor C, ssm_tensor D, ssm_tensor z,
                              ssm_tensor ssm_state, const int32_t *slot_idx,
                              const int32_t *has_initial_state, const int32_t *cu_seqlens,
                              ssm_tensor out, int nseq, int total_len, int nheads, int headdim,
                              int dstate, int ngroups, int nslots, int a_per_state, int dt_softplus,
                              void *stream)
{
    if (!cu_seqlens)
        return SSM_ERR_NULL_ARG;
    return scan_call(u, dt, dt_bias, A, B, C, D, z, ssm_state, slot_idx, cu_seqlens, has_initial_state,
                     out, nseq, total_len, nheads, headdim, dstate, ngroups, nslots, a_per_state,
                     dt_softplus, 0, stream);
}

} // extern "C"

namespace {

using ssm::dtype_size;

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

// A caller's geometry: SSM_OK, SSM_ERR_OUT_OF_RESOURCES past what the kernels
// are built for (more than 16 states per lane, more than 512 lanes per
// workgroup, a row wider than one wave), else SSM_ERR_SHAPE for values that
// are not one of the listed ones.
int check_ssu_config(int V, int block, int state_dtype, int dstate)
{
    const bool pow2v = V > 0 && (V & (V - 1)) == 0;
    const bool pow2b = block > 0 && (block & (block - 1)) == 0;
    if ((pow2v && V > 16) || (pow2b && block > 512))
        return SSM_ERR_OUT_OF_RESOURCES;
    // 4 states per lane only for a 4-byte cache (one 16-byte vector)
    if (!(V == 8 || V == 16 || (V == 4 && dtype_size(state_dtype) == 4)))
        return SSM_ERR_SHAPE;
    if (!(block == 64 || block == 128 || block == 256 || block == 512))
        return SSM_ERR_SHAPE;
    // a row's lanes must fit in one wave (the readout sum is a butterfly within it)
    if ((dstate + V - 1) / V > 64)
        return SSM_ERR_OUT_OF_RESOURCES;
    return SSM_OK;
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
            check_ssu_config(e->states_per_lane, e->block_threads, state_dtype, dstate) == SSM_OK) {
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

} // namespace

namespace ssm {

// Validation and launch geometry shared by ssm_state_update(_ex),
// ssm_decode_step and the decode layer; fills `a` and returns SSM_OK, or an
// error status.  cfg: the caller's geometry, or null for the library's choice.
int prepare_ssu(SsuArgs &a, const ssm_tensor &state, const int32_t *slot_idx, const ssm_tensor &x,
                const ssm_tensor &dt, const ssm_tensor &dt_bias, const ssm_tensor &A, const ssm_tensor &B,
                const ssm_tensor &C, const ssm_tensor &D, const ssm_tensor &z, const ssm_tensor &out,
                int batch, int nheads, int headdim, int dstate, int ngroups, int nslots, int a_per_state,
                int dt_softplus, const ssm_launch_config *cfg)
{
    if (!present(state) || !present(x) || !present(dt) || !present(A) || !present(B) || !present(C) ||
        !present(out))
        return SSM_ERR_NULL_ARG;
    if (batch < 0 || nheads < 1 || headdim < 1 || dstate < 1 || ngroups < 1 || nheads % ngroups != 0)
        return SSM_ERR_SHAPE;
    if (dstate > kMaxSsuDstate)
        return SSM_ERR_OUT_OF_RESOURCES;  // a row of more than 64 lanes of 8 states
    if (!slots_ok(state.data, slot_idx, nslots, batch))
        return SSM_ERR_SHAPE;
    const int io = x.dtype;
    const int64_t xs[3] = {batch, nheads, headdim}, ds[2] = {batch, nheads};
    const int64_t bs[3] = {batch, ngroups, dstate}, as2[2] = {nheads, dstate}, as1[1] = {nheads};
    const int64_t ss[4] = {nslots, nheads, headdim, dstate};
    SSM_TRY(check_tensor(x, 3, xs, -1));
    SSM_TRY(check_tensor(z, 3, xs, io));
    SSM_TRY(check_tensor(out, 3, xs, io));
    SSM_TRY(check_tensor(dt, 2, ds, io));
    SSM_TRY(check_tensor(B, 3, bs, io));
    SSM_TRY(check_tensor(C, 3, bs, io));
    SSM_TRY(check_tensor(A, a_per_state ? 2 : 1, a_per_state ? as2 : as1, SSM_F32));
    SSM_TRY(check_tensor(D, 1, as1, SSM_F32));
    SSM_TRY(check_tensor(dt_bias, 1, as1, SSM_F32));
    SSM_TRY(check_tensor(state, 4, ss, -1));
    if (!aligned(slot_idx, 4))
        return SSM_ERR_ALIGN;
    const int state_dtype = state.dtype;
    int V, block, from_table;
    if (cfg) {
        SSM_TRY(check_ssu_config(cfg->states_per_lane, cfg->block_threads, state_dtype, dstate));
        V = cfg->states_per_lane;
        block = cfg->block_threads;
    } else {
        choose_ssu(batch, nheads, headdim, dstate, io, state_dtype, V, block, from_table);
    }
    // lanes per (b,h,p) row: ceil(dstate/V) rounded up to a power of two (<= 64)
    int lanes = (dstate + V - 1) / V, lg = 0;
    while ((1 << lg) < lanes)
        ++lg;
    const int64_t nrows = (int64_t)batch * nheads * headdim;
    const int rb = ssu_requests_per_lane(batch, headdim);
    if (((((int64_t)nheads * headdim) << lg) + 63) / 64 > INT32_MAX)
        return SSM_ERR_UNSUPPORTED;
    a = SsuArgs{};
    a.state = state.data;
    a.slot_idx = slot_idx;
    a.x = x.data;
    a.dt = dt.data;
    a.B = B.data;
    a.C = C.data;
    a.z = z.data;
    a.dt_bias = static_cast<const float *>(dt_bias.data);
    a.A = static_cast<const float *>(A.data);
    a.D = static_cast<const float *>(D.data);
    a.out = out.data;
    a.x_sb = x.stride[0];
    a.x_sh = x.stride[1];
    a.z_sb = st(z, 0);
    a.z_sh = st(z, 1);
    a.o_sb = out.stride[0];
    a.o_sh = out.stride[1];
    a.dt_sb = dt.stride[0];
    a.B_sb = B.stride[0];
    a.B_sg = B.stride[1];
    a.C_sb = C.stride[0];
    a.C_sg = C.stride[1];
    a.A_sh = a_per_state ? A.stride[0] : 1;
    a.st_ss = state.stride[0];
    a.st_sh = state.stride[1];
    a.st_sp = state.stride[2];
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
    a.io_dtype = io;
    a.state_dtype = state_dtype;
    a.a_per_state = a_per_state ? 1 : 0;
    a.dt_softplus = dt_softplus ? 1 : 0;
    // 128-bit state, B, C and A vectors: 16-byte aligned rows
    a.vec = (dstate % V == 0) && rows16(state, 4, ss) && rows16(B, 3, bs) && rows16(C, 3, bs) &&
            rows16(A, a_per_state ? 2 : 1, a_per_state ? as2 : as1);
    a.requests_per_lane = rb;
    a.conv_width = 0;
    // a request's x / z / out rows are addressed with 32-bit offsets
    const int64_t hmax = (int64_t)nheads - 1;
    if (hmax * a.x_sh + headdim > INT32_MAX || hmax * a.z_sh + headdim > INT32_MAX ||
        hmax * a.o_sh + headdim > INT32_MAX)
        return SSM_ERR_UNSUPPORTED;
    return SSM_OK;
}

// The fused conv's arguments on top of prepare_ssu's.
int prepare_decode_conv(SsuArgs &a, const ssm_tensor &conv_state, const ssm_tensor &conv_weight,
                        const ssm_tensor &conv_bias, const ssm_tensor &u_out, int conv_width)
{
    if (!present(conv_state) || !present(conv_weight))
        return SSM_ERR_NULL_ARG;
    if (conv_width < 1)
        return SSM_ERR_SHAPE;
    if (conv_width != kFusedConvWidth)
        return SSM_ERR_UNSUPPORTED;
    const int64_t Cn = (int64_t)a.nheads * a.headdim;
    const int64_t cs[3] = {a.nslots, Cn, conv_width - 1}, ws[2] = {Cn, conv_width}, bs[1] = {Cn};
    const int64_t us[3] = {a.batch, a.nheads, a.headdim};
    SSM_TRY(check_tensor(conv_state, 3, cs, a.io_dtype));
    SSM_TRY(check_tensor(conv_weight, 2, ws, SSM_F32));
    SSM_TRY(check_tensor(conv_bias, 1, bs, SSM_F32));
    SSM_TRY(check_tensor(u_out, 3, us, a.io_dtype));
    a.conv_state = conv_state.data;
    a.conv_weight = static_cast<const float *>(conv_weight.data);
    a.conv_bias = static_cast<const float *>(conv_bias.data);
    a.u_out = u_out.data;
    a.cs_ss = conv_state.stride[0];
    a.cs_sc = conv_state.stride[1];
    a.cw_sc = conv_weight.stride[0];
    a.u_sb = st(u_out, 0);
    a.u_sh = st(u_out, 1);
    a.conv_width = conv_width;
    if ((int64_t)(a.nheads - 1) * a.u_sh + a.headdim > INT32_MAX)
        return SSM_ERR_UNSUPPORTED;
    return SSM_OK;
}

} // namespace ssm

extern "C" {

int ssm_state_update(ssm_tensor state, const int32_t *slot_idx, ssm_tensor x, ssm_tensor dt,
                     ssm_tensor dt_bias, ssm_tensor A, ssm_tensor B, ssm_tensor C, ssm_tensor D,
                     ssm_tensor z, ssm_tensor out, int batch, int nheads, int headdim, int dstate,
                     int ngroups, int nslots, int a_per_state, int dt_softplus, void *stream)
{
    return ssm_state_update_ex(state, slot_idx, x, dt, dt_bias, A, B, C, D, z, out, batch, nheads,
                               headdim, dstate, ngroups, nslots, a_per_state, dt_softplus, nullptr,
                               stream);
}

int ssm_state_update_ex(ssm_tensor state, const int32_t *slot_idx, ssm_tensor x, ssm_tensor dt,
                        ssm_tensor dt_bias, ssm_tensor A, ssm_tensor B, ssm_tensor C, ssm_tensor D,
                        ssm_tensor z, ssm_tensor out, int batch, int nheads, int headdim, int dstate,
                        int ngroups, int nslots, int a_per_state, int dt_softplus,
                        const ssm_launch_config *config, void *stream)
{
    ssm::SsuArgs a;
    SSM_TRY(ssm::prepare_ssu(a, state, slot_idx, x, dt, dt_bias, A, B, C, D, z, out, batch, nheads,
                             headdim, dstate, ngroups, nslots, a_per_state, dt_softplus, config));
    if (batch == 0)
        return SSM_OK;
    return status_of(ssm::launch_ssu(a, static_cast<hipStream_t>(stream)));
}

int ssm_state_update_config(int batch, int nheads, int headdim, int dstate, int io_dtype,
                            int state_dtype, ssm_launch_config *config, int *from_table)
{
    if (!config)
        return SSM_ERR_NULL_ARG;
    if (!ssm::valid_dtype(io_dtype) || !ssm::valid_dtype(state_dtype))
        return SSM_ERR_DTYPE;
    if (batch < 0 || nheads < 1 || headdim < 1 || dstate < 1)
        return SSM_ERR_SHAPE;
    if (dstate > ssm::kMaxSsuDstate)
        return SSM_ERR_OUT_OF_RESOURCES;
    int V, block, ft;
    choose_ssu(batch, nheads, headdim, dstate, io_dtype, state_dtype, V, block, ft);
    config->states_per_lane = V;
    config->block_threads = block;
    if (from_table)
        *from_table = ft;
    return SSM_OK;
}

int ssm_decode_step(ssm_tensor state, ssm_tensor conv_state, const int32_t *slot_idx, ssm_tensor x,
                    ssm_tensor conv_weight, ssm_tensor conv_bias, int conv_width, ssm_tensor dt,
                    ssm_tensor dt_bias, ssm_tensor A, ssm_tensor B, ssm_tensor C, ssm_tensor D,
                    ssm_tensor z, ssm_tensor out, ssm_tensor u_out, int batch, int nheads, int headdim,
                    int dstate, int ngroups, int nslots, int a_per_state, int dt_softplus, void *stream)
{
    ssm::SsuArgs a;
    SSM_TRY(ssm::prepare_ssu(a, state, slot_idx, x, dt, dt_bias, A, B, C, D, z, out, batch, nheads,
                             headdim, dstate, ngroups, nslots, a_per_state, dt_softplus, nullptr));
    SSM_TRY(ssm::prepare_decode_conv(a, conv_state, conv_weight, conv_bias, u_out, conv_width));
    if (batch == 0)
        return SSM_OK;
    int st;
    if (group_take_decode(a, stream, &st))
        return st;
    return status_of(ssm::launch_ssu(a, static_cast<hipStream_t>(stream)));
}

int ssm_group_begin(void *stream)
{
    LaunchGroup &g = g_group;
    if (g.open)
        return SSM_ERR_UNSUPPORTED;
    g = LaunchGroup();
    g.open = true;
    g.stream = stream;
    return SSM_OK;
}

int ssm_group_end(void *stream)
{
    LaunchGroup &g = g_group;
    if (!g.open || g.stream != stream)
        return SSM_ERR_UNSUPPORTED;
    int st = SSM_OK;
    if (g.has_scan)
        st = status_of(ssm::launch_scan(g.scan, static_cast<hipStream_t>(stream)));
    if (g.has_decode) {
        const int s2 = status_of(ssm::launch_ssu(g.decode, static_cast<hipStream_t>(stream)));
        if (st == SSM_OK)
            st = s2;
    }
    g = LaunchGroup();
    return st;
}

} // extern "C"
