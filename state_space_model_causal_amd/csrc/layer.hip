// layer.hip -- C ABI of the projections, the RMSNorm and one whole Mamba-1
// decode layer (include/ssm.h): host-side validation, workspace carving and
// the sequence of launches.  Each step runs in this library's kernels.
#include "ssm.h"
#include "ssm_kernels.hpp"

#include <stddef.h>
#include <stdint.h>

#include <mutex>

// Device memory of ssm_mamba1_decode_layer_noalloc: its workspace (the
// layer's intermediates and split-K partial sums) lives here instead of in a
// caller buffer.  Each GPU the library runs on holds its own copy, from the
// first call on that GPU until the process ends.  Host code never uses this
// name as an address: it looks up the device's copy with
// hipGetSymbolAddress and keeps that pointer per device.
static __device__ __align__(256) unsigned char scratch[SSM_LAYER_SCRATCH_BYTES];

namespace {

bool mfma_dtype(int d) { return d == SSM_F16 || d == SSM_BF16; }
bool valid_dtype_code(int d) { return d == SSM_F32 || d == SSM_F16 || d == SSM_BF16; }
bool al(const void *p, uintptr_t n) { return p == nullptr || (reinterpret_cast<uintptr_t>(p) % n) == 0; }
size_t round_up(size_t v) { return (v + 255) & ~(size_t)255; }
using ssm::status_of;

// Workspace of one product: the float32 partial sums of a K split.
struct LinearWs {
    ssm::GemmPlan plan;
    size_t total;
};

LinearWs linear_ws(int M, int N, const ssm::GemmPlan &plan)
{
    LinearWs w{};
    w.plan = plan;
    w.total = plan.splits > 1 ? round_up((size_t)plan.splits * M * N * sizeof(float)) : 0;
    return w;
}

// The plan as given (0: the library's choice of that part); status of values
// the product kernel does not take
int plan_of(int M, int N, int K, int rows_per_wave, int cols, int splits, ssm::GemmPlan &plan)
{
    const bool pow2 = (rows_per_wave & (rows_per_wave - 1)) == 0 && (cols & (cols - 1)) == 0;
    if (pow2 && (rows_per_wave > 64 || cols > 128))
        return SSM_ERR_OUT_OF_RESOURCES;  // past a wave's accumulators / a workgroup's threads
    if ((rows_per_wave != 0 && rows_per_wave != 16 && rows_per_wave != 32 && rows_per_wave != 64) ||
        (cols != 0 && cols != 64 && cols != 128) || splits < 0 || splits > (K + 63) / 64 || splits > 64)
        return SSM_ERR_SHAPE;
    plan = ssm::plan_gemm(M, N, K, rows_per_wave, cols, splits);
    return SSM_OK;
}

ssm_tensor dense(const void *p, int dtype, int64_t s0, int64_t s1 = 1, int64_t s2 = 1)
{
    ssm_tensor t{};
    t.data = const_cast<void *>(p);
    t.dtype = dtype;
    t.stride[0] = s0;
    t.stride[1] = s1;
    t.stride[2] = s2;
    t.stride[3] = 1;
    return t;
}

// A [rows, cols] operand of the projections: f16/bf16 of the given dtype,
// unit inner stride, non-negative row stride that fits the kernels' int.
int check_matrix(const ssm_tensor &t, int rows, int cols, int dtype, bool rows16)
{
    if (!t.data)
        return SSM_OK;
    if (!valid_dtype_code(t.dtype) || t.dtype != dtype)
        return SSM_ERR_DTYPE;
    if (t.stride[0] < 0 || t.stride[1] < 0 || (cols > 1 && t.stride[1] != 1))
        return SSM_ERR_LAYOUT;
    if (t.stride[0] > INT32_MAX)
        return SSM_ERR_UNSUPPORTED;
    if (!al(t.data, 2))
        return SSM_ERR_ALIGN;
    if (rows16 && (!al(t.data, 16) || (rows > 1 && (t.stride[0] * 2) % 16 != 0)))
        return SSM_ERR_ALIGN;
    return SSM_OK;
}

int check_linear(const ssm_tensor &x, const ssm_tensor &w, const ssm_tensor &res, const ssm_tensor &out, int M,
                 int N, int K)
{
    if (!x.data || !w.data || !out.data)
        return SSM_ERR_NULL_ARG;
    if (!mfma_dtype(x.dtype))
        return valid_dtype_code(x.dtype) ? SSM_ERR_UNSUPPORTED : SSM_ERR_DTYPE;
    if (M < 0 || N < 1 || K < 8 || K % 8 != 0)
        return SSM_ERR_SHAPE;
    int st;
    if ((st = check_matrix(x, M, K, x.dtype, true)) != SSM_OK || (st = check_matrix(w, N, K, x.dtype, true)) != SSM_OK ||
        (st = check_matrix(out, M, N, x.dtype, false)) != SSM_OK ||
        (st = check_matrix(res, M, N, x.dtype, false)) != SSM_OK)
        return st;
    if ((int64_t)M * N > INT32_MAX || (int64_t)N * K > INT32_MAX)
        return SSM_ERR_UNSUPPORTED;
    return SSM_OK;
}

// The product with its plan (partial sums in `partial` when it splits K).
int run_linear(ssm::GemmArgs g, int M, int N, int K, const LinearWs &lw, void *partial, hipStream_t stream)
{
    g.M = M;
    g.N = N;
    g.K = K;
    g.wr = lw.plan.wr;
    g.cw = lw.plan.cw;
    g.splits = lw.plan.splits;
    g.partial = g.splits > 1 ? static_cast<float *>(partial) : nullptr;
    return status_of(ssm::launch_gemm(g, stream));
}

} // namespace

extern "C" {

size_t ssm_linear_workspace_ex(int M, int N, int K, int rows_per_wave, int cols_per_workgroup, int splits)
{
    ssm::GemmPlan plan;
    if (M < 1 || N < 1 || K < 1 || plan_of(M, N, K, rows_per_wave, cols_per_workgroup, splits, plan) != SSM_OK)
        return 0;
    return linear_ws(M, N, plan).total;
}

size_t ssm_linear_workspace(int M, int N, int K) { return ssm_linear_workspace_ex(M, N, K, 0, 0, 0); }

int ssm_linear_plan(int M, int N, int K, int *rows_per_wave, int *cols_per_workgroup, int *splits)
{
    if (M < 1 || N < 1 || K < 8)
        return SSM_ERR_SHAPE;
    const ssm::GemmPlan plan = ssm::plan_gemm(M, N, K);
    if (rows_per_wave)
        *rows_per_wave = plan.wr;
    if (cols_per_workgroup)
        *cols_per_workgroup = 64 * plan.cw;
    if (splits)
        *splits = plan.splits;
    return SSM_OK;
}

int ssm_linear_ex(ssm_tensor x, ssm_tensor weight, ssm_tensor residual, ssm_tensor out, int M, int N, int K,
                  int rows_per_wave, int cols_per_workgroup, int splits, void *workspace, size_t workspace_bytes,
                  void *stream)
{
    int st = check_linear(x, weight, residual, out, M, N, K);
    if (st != SSM_OK)
        return st;
    ssm::GemmPlan plan;
    if ((st = plan_of(M > 0 ? M : 1, N, K, rows_per_wave, cols_per_workgroup, splits, plan)) != SSM_OK)
        return st;
    if (!al(workspace, 16))
        return SSM_ERR_ALIGN;
    if (M == 0)
        return SSM_OK;
    const LinearWs lw = linear_ws(M, N, plan);
    if (lw.total && (!workspace || workspace_bytes < lw.total))
        return SSM_ERR_SHAPE;
    hipStream_t s = static_cast<hipStream_t>(stream);
    ssm::GemmArgs g{};
    g.A = x.data;
    g.lda = (int)x.stride[0];
    g.W = weight.data;
    g.ldw = (int)weight.stride[0];
    g.dtype = x.dtype;
    g.seg[0] = ssm::GemmSeg{out.data, (int)out.stride[0], 0, N};
    g.nseg = 1;
    g.residual = residual.data;
    g.ld_residual = residual.data ? (int)residual.stride[0] : 0;
    return run_linear(g, M, N, K, lw, workspace, s);
}

int ssm_linear(ssm_tensor x, ssm_tensor weight, ssm_tensor residual, ssm_tensor out, int M, int N, int K,
               void *workspace, size_t workspace_bytes, void *stream)
{
    return ssm_linear_ex(x, weight, residual, out, M, N, K, 0, 0, 0, workspace, workspace_bytes, stream);
}

int ssm_rmsnorm(ssm_tensor x, ssm_tensor weight, ssm_tensor out, int M, int D, float eps, void *stream)
{
    if (!x.data || !weight.data || !out.data)
        return SSM_ERR_NULL_ARG;
    if (!mfma_dtype(x.dtype))
        return valid_dtype_code(x.dtype) ? SSM_ERR_UNSUPPORTED : SSM_ERR_DTYPE;
    if (weight.dtype != SSM_F32)
        return SSM_ERR_DTYPE;
    if (M < 0 || D < 1 || !(eps >= 0.0f))
        return SSM_ERR_SHAPE;
    int st;
    if ((st = check_matrix(x, M, D, x.dtype, false)) != SSM_OK ||
        (st = check_matrix(out, M, D, x.dtype, false)) != SSM_OK)
        return st;
    if (D > 1 && weight.stride[0] != 1)
        return SSM_ERR_LAYOUT;
    if (!al(weight.data, 4))
        return SSM_ERR_ALIGN;
    if (M == 0)
        return SSM_OK;
    return status_of(ssm::launch_rmsnorm(x.data, x.stride[0], static_cast<const float *>(weight.data), out.data,
                                         out.stride[0], M, D, eps, x.dtype, static_cast<hipStream_t>(stream)));
}

// Workspace of one decode layer: the intermediates of the batch, each
// 256-byte aligned, then the largest split-K partial buffer.
struct LayerWs {
    LinearWs in, xp, dtp, out;  // the four products
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
    const int b = batch, R = L->dt_rank, N2 = L->dt_rank + 2 * L->d_state;
    w.in = linear_ws(b, 2 * L->d_inner, ssm::plan_gemm(b, 2 * L->d_inner, L->d_model));
    w.xp = linear_ws(b, N2, ssm::plan_gemm(b, N2, L->d_inner));
    w.dtp = linear_ws(b, L->d_inner, ssm::plan_gemm(b, L->d_inner, R));
    w.out = linear_ws(b, L->d_model, ssm::plan_gemm(b, L->d_model, L->d_inner));
    size_t p = 0;
    for (const LinearWs *lw : {&w.in, &w.xp, &w.dtp, &w.out})
        p = lw->total > p ? lw->total : p;
    w.partial = o;
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

int ssm_mamba1_decode_layer(const ssm_mamba1_layer *L, ssm_tensor hidden, ssm_tensor conv_state,
                            ssm_tensor ssm_state, const int32_t *slot_idx, int batch, int nslots, void *workspace,
                            size_t workspace_bytes, void *stream)
{
    int st = check_layer(L, batch);
    if (st != SSM_OK)
        return st;
    if (!hidden.data || !conv_state.data || !ssm_state.data)
        return SSM_ERR_NULL_ARG;
    const int io = hidden.dtype;
    if (!mfma_dtype(io))
        return valid_dtype_code(io) ? SSM_ERR_UNSUPPORTED : SSM_ERR_DTYPE;
    const int M = batch, Dm = L->d_model, Di = L->d_inner, N = L->d_state, R = L->dt_rank;
    if ((st = check_matrix(hidden, M, Dm, io, true)) != SSM_OK)
        return st;
    if (!al(L->in_proj, 16) || !al(L->x_proj, 16) || !al(L->dt_proj, 16) || !al(L->out_proj, 16) ||
        !al(workspace, 256))
        return SSM_ERR_ALIGN;
    const LayerWs w = layer_ws(L, batch > 0 ? batch : 1);
    if (batch > 0 && (!workspace || workspace_bytes < w.total))
        return SSM_ERR_SHAPE;
    char *ws = static_cast<char *>(workspace);
    void *hn = ws + w.hn, *x = ws + w.x, *z = ws + w.z, *u = ws + w.u, *dtl = ws + w.dtl;
    void *Bm = ws + w.B, *Cm = ws + w.C, *dt = ws + w.dt, *y = ws + w.y, *part = ws + w.partial;

    // every later step's arguments, checked before the first launch so that
    // an error leaves hidden and both caches untouched
    ssm::ConvArgs ca;
    st = ssm::prepare_conv(ca, dense(x, io, Di, 1, 1), dense(L->conv_weight, SSM_F32, L->conv_width),
                           dense(L->conv_bias, SSM_F32, 1), conv_state, slot_idx, nullptr, nullptr,
                           dense(u, io, Di, 1, 1), M, Di, 1, L->conv_width, nslots, 1, 1);
    if (st != SSM_OK)
        return st;
    // the state update: one channel per head (headdim 1)
    ssm::SsuArgs sa;
    st = ssm::prepare_ssu(sa, ssm_state, slot_idx, dense(u, io, Di, 1, 1), dense(dt, io, Di, 1),
                          dense(L->dt_bias, SSM_F32, 1), dense(L->A, SSM_F32, N, 1), dense(Bm, io, N, N, 1),
                          dense(Cm, io, N, N, 1), dense(L->D, SSM_F32, 1), dense(z, io, Di, 1, 1),
                          dense(y, io, Di, 1, 1), M, Di, 1, N, 1, nslots, 1, 1, nullptr);
    if (st != SSM_OK)
        return st;
    if (batch == 0)
        return SSM_OK;
    hipStream_t s = static_cast<hipStream_t>(stream);

    // 1. normalised hidden state
    st = status_of(ssm::launch_rmsnorm(hidden.data, hidden.stride[0], L->norm_weight, hn, Dm, M, Dm, L->norm_eps,
                                       io, s));
    if (st != SSM_OK)
        return st;
    // 2. in_proj -> x | z
    ssm::GemmArgs g{};
    g.dtype = io;
    g.A = hn;
    g.lda = Dm;
    g.W = L->in_proj;
    g.ldw = Dm;
    g.seg[0] = ssm::GemmSeg{x, Di, 0, Di};
    g.seg[1] = ssm::GemmSeg{z, Di, Di, Di};
    g.nseg = 2;
    if ((st = run_linear(g, M, 2 * Di, Dm, w.in, part, s)) != SSM_OK)
        return st;
    // 3. conv update + SiLU of x (the request's window in its slot)
    if ((st = status_of(ssm::launch_conv(ca, s))) != SSM_OK)
        return st;
    // 4. x_proj -> dt_low | B | C
    g = ssm::GemmArgs{};
    g.dtype = io;
    g.A = u;
    g.lda = Di;
    g.W = L->x_proj;
    g.ldw = Di;
    g.seg[0] = ssm::GemmSeg{dtl, R, 0, R};
    g.seg[1] = ssm::GemmSeg{Bm, N, R, N};
    g.seg[2] = ssm::GemmSeg{Cm, N, R + N, N};
    g.nseg = 3;
    if ((st = run_linear(g, M, R + 2 * N, Di, w.xp, part, s)) != SSM_OK)
        return st;
    // 5. dt_proj -> dt (its bias goes in with the softplus of the update)
    g = ssm::GemmArgs{};
    g.dtype = io;
    g.A = dtl;
    g.lda = R;
    g.W = L->dt_proj;
    g.ldw = R;
    g.seg[0] = ssm::GemmSeg{dt, Di, 0, Di};
    g.nseg = 1;
    if ((st = run_linear(g, M, Di, R, w.dtp, part, s)) != SSM_OK)
        return st;
    // 6. selective state update
    if ((st = status_of(ssm::launch_ssu(sa, s))) != SSM_OK)
        return st;
    // 7. out_proj + residual, in place on hidden (rows of padded requests kept)
    g = ssm::GemmArgs{};
    g.dtype = io;
    g.A = y;
    g.lda = Di;
    g.W = L->out_proj;
    g.ldw = Di;
    g.seg[0] = ssm::GemmSeg{hidden.data, (int)hidden.stride[0], 0, Dm};
    g.nseg = 1;
    g.residual = hidden.data;
    g.ld_residual = (int)hidden.stride[0];
    g.row_slot = slot_idx;
    return run_linear(g, M, Dm, Di, w.out, part, s);
}

namespace {

// The scratch array's address on each device, looked up once per device.
constexpr int kMaxDevices = 64;
void *g_scratch[kMaxDevices];
std::mutex g_scratch_mutex;

int scratch_of_current_device(void **ptr)
{
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0)
        return SSM_ERR_HIP;
    if (dev >= kMaxDevices)
        return SSM_ERR_UNSUPPORTED;
    std::lock_guard<std::mutex> lock(g_scratch_mutex);
    if (!g_scratch[dev]) {
        void *p = nullptr;
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p)
            return SSM_ERR_HIP;
        g_scratch[dev] = p;
    }
    *ptr = g_scratch[dev];
    return SSM_OK;
}

} // namespace

int ssm_mamba1_decode_layer_noalloc(const ssm_mamba1_layer *L, ssm_tensor hidden, ssm_tensor conv_state,
                                    ssm_tensor ssm_state, const int32_t *slot_idx, int batch, int nslots,
                                    void *stream)
{
    int st = check_layer(L, batch);
    if (st != SSM_OK)
        return st;
    if (batch == 0)  // validated like the plain call, then a no-op
        return ssm_mamba1_decode_layer(L, hidden, conv_state, ssm_state, slot_idx, 0, nslots, nullptr, 0, stream);
    if (layer_ws(L, batch).total > (size_t)SSM_LAYER_SCRATCH_BYTES)
        return SSM_ERR_OUT_OF_RESOURCES;
    void *ws = nullptr;
    if ((st = scratch_of_current_device(&ws)) != SSM_OK)
        return st;
    return ssm_mamba1_decode_layer(L, hidden, conv_state, ssm_state, slot_idx, batch, nslots, ws,
                                   (size_t)SSM_LAYER_SCRATCH_BYTES, stream);
}

} // extern "C"
