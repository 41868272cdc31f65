// layer.hip -- C ABI of the projections, the RMSNorm and one whole Mamba-1
// decode layer (include/ssm.h): host-side validation, workspace carving and
// the sequence of launches.  Each step runs in this library's kernels.
#include "ssm.h"
#include "ssm_kernels.hpp"

#include <stddef.h>
#include <stdint.h>

namespace {

bool mfma_dtype(int d) { return d == SSM_F16 || d == SSM_BF16; }
bool valid_dtype_code(int d) { return d == SSM_F32 || d == SSM_F16 || d == SSM_BF16; }
bool al(const void *p, uintptr_t n) { return p == nullptr || (reinterpret_cast<uintptr_t>(p) % n) == 0; }
size_t round_up(size_t v) { return (v + 255) & ~(size_t)255; }
int status_of(hipError_t e) { return e == hipSuccess ? SSM_OK : SSM_ERR_HIP; }

// K split so that a narrow output still spreads over the chip: up to 32
// slices of at least 2 k batches, aiming at ~512 workgroups.
int choose_splits(int M, int N, int K)
{
    const int nsteps = (K + 63) / 64;  // 64-k batches of the projection kernel
    const int64_t blocks = (int64_t)((N + 63) / 64) * ((M + 255) / 256);
    int s = (int)(512 / (blocks > 0 ? blocks : 1));
    if (s > 32)
        s = 32;
    if (s > nsteps / 2)
        s = nsteps / 2;
    return s < 1 ? 1 : s;
}

size_t linear_partial_bytes(int M, int N, int K)
{
    const int s = choose_splits(M, N, K);
    return s > 1 ? round_up((size_t)s * M * N * sizeof(float)) : 0;
}

int check_linear(const void *x, const void *w, const void *out, int M, int N, int K, int dtype)
{
    if (!x || !w || !out)
        return SSM_ERR_NULL_ARG;
    if (!mfma_dtype(dtype))
        return valid_dtype_code(dtype) ? SSM_ERR_UNSUPPORTED : SSM_ERR_DTYPE;
    if (M < 0 || N < 1 || K < 8 || K % 8 != 0)
        return SSM_ERR_SHAPE;
    if (!al(x, 16) || !al(w, 16) || !al(out, 2))
        return SSM_ERR_ALIGN;
    if ((int64_t)M * N > INT32_MAX || (int64_t)N * K > INT32_MAX)
        return SSM_ERR_UNSUPPORTED;
    return SSM_OK;
}

int run_linear(ssm::GemmArgs g, int M, int N, int K, void *ws, hipStream_t stream)
{
    g.M = M;
    g.N = N;
    g.K = K;
    g.splits = choose_splits(M, N, K);
    g.partial = g.splits > 1 ? static_cast<float *>(ws) : nullptr;
    return status_of(ssm::launch_gemm(g, stream));
}

} // namespace

extern "C" {

size_t ssm_linear_workspace(int M, int N, int K)
{
    if (M < 1 || N < 1 || K < 1)
        return 0;
    return linear_partial_bytes(M, N, K);
}

int ssm_linear(const void *x, const void *weight, const void *residual, void *out, int M, int N, int K,
               int dtype, void *workspace, size_t workspace_bytes, void *stream)
{
    const int st = check_linear(x, weight, out, M, N, K, dtype);
    if (st != SSM_OK)
        return st;
    if (!al(residual, 2) || !al(workspace, 16))
        return SSM_ERR_ALIGN;
    if (M == 0)
        return SSM_OK;
    const size_t need = linear_partial_bytes(M, N, K);
    if (need && (!workspace || workspace_bytes < need))
        return SSM_ERR_SHAPE;
    ssm::GemmArgs g{};
    g.A = x;
    g.W = weight;
    g.lda = K;
    g.dtype = dtype;
    g.seg[0] = ssm::GemmSeg{out, N, 0, N};
    g.nseg = 1;
    g.residual = residual;
    g.ld_residual = N;
    return run_linear(g, M, N, K, workspace, static_cast<hipStream_t>(stream));
}

int ssm_rmsnorm(const void *x, const float *weight, void *out, int M, int D, float eps, int dtype,
                void *stream)
{
    if (!x || !weight || !out)
        return SSM_ERR_NULL_ARG;
    if (!mfma_dtype(dtype))
        return valid_dtype_code(dtype) ? SSM_ERR_UNSUPPORTED : SSM_ERR_DTYPE;
    if (M < 0 || D < 1 || !(eps >= 0.0f))
        return SSM_ERR_SHAPE;
    if (!al(x, 2) || !al(out, 2) || !al(weight, 4))
        return SSM_ERR_ALIGN;
    if (M == 0)
        return SSM_OK;
    return status_of(ssm::launch_rmsnorm(x, weight, out, M, D, eps, dtype, static_cast<hipStream_t>(stream)));
}

// Workspace of one decode layer: the intermediates of the batch, each
// 256-byte aligned, then the largest split-K partial buffer.
struct LayerWs {
    size_t hn, x, z, u, dtl, B, C, dt, y, partial, total;
};

static LayerWs layer_ws(const ssm_mamba1_layer *L, int batch)
{
    const size_t e = 2;  // f16 / bf16
    const size_t M = (size_t)batch;
    LayerWs w{};
    size_t o = 0;
    w.hn = o; o += round_up(M * L->d_model * e);
    w.x = o; o += round_up(M * L->d_inner * e);
    w.z = o; o += round_up(M * L->d_inner * e);
    w.u = o; o += round_up(M * L->d_inner * e);
    w.dtl = o; o += round_up(M * L->dt_rank * e);
    w.B = o; o += round_up(M * L->d_state * e);
    w.C = o; o += round_up(M * L->d_state * e);
    w.dt = o; o += round_up(M * L->d_inner * e);
    w.y = o; o += round_up(M * L->d_inner * e);
    w.partial = o;
    size_t p = linear_partial_bytes(batch, 2 * L->d_inner, L->d_model);
    const size_t p2 = linear_partial_bytes(batch, L->dt_rank + 2 * L->d_state, L->d_inner);
    const size_t p3 = linear_partial_bytes(batch, L->d_inner, L->dt_rank);
    const size_t p4 = linear_partial_bytes(batch, L->d_model, L->d_inner);
    if (p2 > p) p = p2;
    if (p3 > p) p = p3;
    if (p4 > p) p = p4;
    w.total = o + p;
    return w;
}

static int check_layer(const ssm_mamba1_layer *L, int batch)
{
    if (!L)
        return SSM_ERR_NULL_ARG;
    if (!L->norm_weight || !L->in_proj || !L->conv_weight || !L->x_proj || !L->dt_proj || !L->A ||
        !L->out_proj)
        return SSM_ERR_NULL_ARG;
    if (batch < 0 || L->d_model < 8 || L->d_inner < 8 || L->d_state < 1 || L->dt_rank < 8 ||
        L->d_model % 8 || L->d_inner % 8 || L->dt_rank % 8 || L->d_state % 8 || !(L->norm_eps >= 0.0f))
        return SSM_ERR_SHAPE;
    if (L->conv_width < 1 || L->conv_width > 4 || L->d_state > 512)
        return SSM_ERR_UNSUPPORTED;
    return SSM_OK;
}

size_t ssm_mamba1_decode_layer_workspace(const ssm_mamba1_layer *layer, int batch)
{
    if (check_layer(layer, batch) != SSM_OK || batch < 1)
        return 0;
    return layer_ws(layer, batch).total;
}

int ssm_mamba1_decode_layer(const ssm_mamba1_layer *L, void *hidden, void *conv_state, void *ssm_state,
                            const int32_t *slot_idx, int batch, int nslots, int io_dtype, int state_dtype,
                            void *workspace, size_t workspace_bytes, void *stream)
{
    int st = check_layer(L, batch);
    if (st != SSM_OK)
        return st;
    if (!hidden || !conv_state || !ssm_state)
        return SSM_ERR_NULL_ARG;
    if (!mfma_dtype(io_dtype))
        return valid_dtype_code(io_dtype) ? SSM_ERR_UNSUPPORTED : SSM_ERR_DTYPE;
    if (!valid_dtype_code(state_dtype))
        return SSM_ERR_DTYPE;
    if (!al(hidden, 16) || !al(L->in_proj, 16) || !al(L->x_proj, 16) || !al(L->dt_proj, 16) ||
        !al(L->out_proj, 16) || !al(workspace, 256))
        return SSM_ERR_ALIGN;
    if (batch == 0)
        return SSM_OK;
    const LayerWs w = layer_ws(L, batch);
    if (!workspace || workspace_bytes < w.total)
        return SSM_ERR_SHAPE;
    char *ws = static_cast<char *>(workspace);
    void *hn = ws + w.hn, *x = ws + w.x, *z = ws + w.z, *u = ws + w.u, *dtl = ws + w.dtl;
    void *Bm = ws + w.B, *Cm = ws + w.C, *dt = ws + w.dt, *y = ws + w.y, *part = ws + w.partial;
    const int M = batch, Dm = L->d_model, Di = L->d_inner, N = L->d_state, R = L->dt_rank;
    hipStream_t s = static_cast<hipStream_t>(stream);

    // 1. normalised hidden state
    st = status_of(ssm::launch_rmsnorm(hidden, L->norm_weight, hn, M, Dm, L->norm_eps, io_dtype, s));
    if (st != SSM_OK)
        return st;
    // 2. in_proj -> x | z
    ssm::GemmArgs g{};
    g.dtype = io_dtype;
    g.A = hn;
    g.lda = Dm;
    g.W = L->in_proj;
    g.seg[0] = ssm::GemmSeg{x, Di, 0, Di};
    g.seg[1] = ssm::GemmSeg{z, Di, Di, Di};
    g.nseg = 2;
    if ((st = run_linear(g, M, 2 * Di, Dm, part, s)) != SSM_OK)
        return st;
    // 3. conv update + SiLU of x (the request's window in its slot)
    st = ssm_causal_conv1d(x, L->conv_weight, L->conv_bias, conv_state, slot_idx, u, M, Di, 1,
                           L->conv_width, nslots, io_dtype, 1, 1, stream);
    if (st != SSM_OK)
        return st;
    // 4. x_proj -> dt_low | B | C
    g = ssm::GemmArgs{};
    g.dtype = io_dtype;
    g.A = u;
    g.lda = Di;
    g.W = L->x_proj;
    g.seg[0] = ssm::GemmSeg{dtl, R, 0, R};
    g.seg[1] = ssm::GemmSeg{Bm, N, R, N};
    g.seg[2] = ssm::GemmSeg{Cm, N, R + N, N};
    g.nseg = 3;
    if ((st = run_linear(g, M, R + 2 * N, Di, part, s)) != SSM_OK)
        return st;
    // 5. dt_proj -> dt (its bias goes in with the softplus of the update)
    g = ssm::GemmArgs{};
    g.dtype = io_dtype;
    g.A = dtl;
    g.lda = R;
    g.W = L->dt_proj;
    g.seg[0] = ssm::GemmSeg{dt, Di, 0, Di};
    g.nseg = 1;
    if ((st = run_linear(g, M, Di, R, part, s)) != SSM_OK)
        return st;
    // 6. selective state update (one channel per head: headdim 1)
    st = ssm_state_update(ssm_state, slot_idx, u, dt, L->dt_bias, L->A, Bm, Cm, L->D, z, y, M, Di, 1, N, 1,
                          nslots, io_dtype, state_dtype, 1, 1, stream);
    if (st != SSM_OK)
        return st;
    // 7. out_proj + residual, in place on hidden (rows of padded requests kept)
    g = ssm::GemmArgs{};
    g.dtype = io_dtype;
    g.A = y;
    g.lda = Di;
    g.W = L->out_proj;
    g.seg[0] = ssm::GemmSeg{hidden, Dm, 0, Dm};
    g.nseg = 1;
    g.residual = hidden;
    g.ld_residual = Dm;
    g.row_slot = slot_idx;
    return run_linear(g, M, Dm, Di, part, s);
}

} // extern "C"
