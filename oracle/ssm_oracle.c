/*
 * ssm_oracle.c -- plain, sequential, float64 CPU oracle for the causal
 * selective-SSM (Mamba) hot path: causal depthwise conv1d + SiLU, the
 * selective scan (prefill) and the single-token selective state update.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product library links, loads or
 * calls this file; only the tests, the smoke check and the benchmark's CPU
 * baseline leg do.  It shares no source, header, table or helper with the HIP
 * path.
 *
 * Sources (the pages name the operators and the decode call; they never write
 * the equations, so the plain reading below is the one adopted):
 *  - "feat(llama.cu): 适配 mamba 模型" (InfiniLM-Rust PR #48), section 2.1
 *    "模型适配与功能扩展": the operator set causal-conv1d, selective-scan, silu,
 *    element-mul.  Section 3.1 "高效缓存管理": a per-request mamba cache whose
 *    reads and writes sit at the conv and scan operators.
 *  - "[XPU] Add tuned Mamba SSU configs for Intel Arc Pro B70" (vLLM PR #50534
 *    report), section "关键源码片段": the decode call
 *    selective_state_update(state, x, dt, A, B, C, D=D, z=None,
 *    dt_bias=dt_bias, dt_softplus=True, out=out) -- so dt gets a bias and then
 *    softplus, D and z are optional, and the state is updated in place.
 *
 * The recurrence is the selective SSM with zero-order-hold decay:
 *    delta_t = softplus(dt_t + dt_bias)
 *    h_t[n]  = exp(delta_t * A[n]) * h_{t-1}[n] + delta_t * B_t[n] * u_t
 *    y_t     = sum_n C_t[n] * h_t[n] + D * u_t
 *    out_t   = y_t * silu(z_t)            (no gate when z is absent)
 *
 * Layouts (element offsets, all row-major, time innermost for prefill):
 *    u, z, out : [batch, nheads*headdim, seqlen]     (channel c = h*headdim + p)
 *    dt        : [batch, nheads, seqlen]
 *    B, C      : [batch, ngroups, dstate, seqlen]    (head h uses group
 *                h / (nheads/ngroups))
 *    A         : [nheads, dstate] when a_per_state, else [nheads]
 *    D, dt_bias: [nheads]
 *    state     : [nslots, nheads, headdim, dstate]
 *    conv x/out: [batch, channels, seqlen]; weight [channels, width];
 *    conv_state: [nslots, channels, width-1], oldest sample first.
 *    Decode tensors are the seqlen == 1 case of the same layouts.
 *
 * Slot convention: slot_idx == NULL means request b uses slot b; a negative
 * index marks a padded request, whose outputs and cache rows are untouched.
 *
 * Every function also returns a "scale" per output: the same loops run on
 * absolute values, giving s >= |o|.  The parity metric uses it as the
 * magnitude that rounding errors of a correct implementation are relative to.
 *
 * Return value: 0 on success, -1 on an inconsistent argument.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#include "ssm_oracle.h"

/* softplus(v) = log(1 + e^v), written in the form that is exact in double
 * for every v: max(v, 0) + log1p(e^{-|v|}). */
double oracle_softplus(double v)
{
    return (v > 0.0 ? v : 0.0) + log1p(exp(-fabs(v)));
}

/* SiLU(v) = v * sigmoid(v) = v / (1 + e^{-v}). */
double oracle_silu(double v)
{
    return v / (1.0 + exp(-v));
}

static int slot_of(const int32_t *slot_idx, int b)
{
    return slot_idx ? (int)slot_idx[b] : b;
}

/* ---------------------------------------------------------------------------
 * Causal depthwise conv1d (+ bias, + optional SiLU), with optional conv cache.
 *
 *   acc[b,c,t] = bias[c] + sum_{k<W} w[c,k] * xt(b,c,t-W+1+k)
 *   out[b,c,t] = silu(acc) if apply_silu else acc
 * where xt(s) = x[b,c,s] for s >= 0 and, for -(W-1) <= s < 0, the cached
 * history conv_state[slot,c,W-1+s] when has_initial_state, else 0.
 * When conv_state is given, its row for the request's slot is replaced by the
 * last W-1 samples of xt (an exact copy).  With seqlen == 1 and
 * has_initial_state this is the decode update: one output, window shifted by
 * one.
 * ------------------------------------------------------------------------- */
int oracle_causal_conv1d(int batch, int channels, int seqlen, int width,
                         const double *x, const double *weight,
                         const double *bias, double *conv_state,
                         const int32_t *slot_idx, int nslots,
                         int has_initial_state, int apply_silu, double *out,
                         double *out_scale)
{
    if (batch < 0 || channels < 0 || seqlen < 0 || width < 1)
        return -1;
    const int hist = width - 1;
    double *tail = (double *)malloc(sizeof(double) * (size_t)(hist > 0 ? hist : 1));
    if (!tail)
        return -1;
    for (int b = 0; b < batch; ++b) {
        const int slot = slot_of(slot_idx, b);
        if (slot < 0)
            continue; /* padded request */
        if (conv_state && slot >= nslots) {
            free(tail);
            return -1;
        }
        for (int c = 0; c < channels; ++c) {
            const double *xr = x + ((size_t)b * channels + c) * (size_t)seqlen;
            double *cs = conv_state ? conv_state + ((size_t)slot * channels + c) * (size_t)hist : NULL;
            /* xt(s) for s in [-(W-1), seqlen-1] */
#define XT(s) ((s) >= 0 ? xr[(s)] : ((has_initial_state && cs) ? cs[hist + (s)] : 0.0))
            for (int t = 0; t < seqlen; ++t) {
                double acc = bias ? bias[c] : 0.0;
                double mag = bias ? fabs(bias[c]) : 0.0;
                for (int k = 0; k < width; ++k) {
                    const double v = weight[(size_t)c * width + k] * XT(t - hist + k);
                    acc += v;
                    mag += fabs(v);
                }
                const size_t o = ((size_t)b * channels + c) * (size_t)seqlen + t;
                out[o] = apply_silu ? oracle_silu(acc) : acc;
                if (out_scale)
                    out_scale[o] = mag;
            }
            if (cs) {
                for (int j = 0; j < hist; ++j)
                    tail[j] = XT(seqlen - hist + j);
                for (int j = 0; j < hist; ++j)
                    cs[j] = tail[j];
            }
#undef XT
        }
    }
    free(tail);
    return 0;
}

/* ---------------------------------------------------------------------------
 * Selective scan over a whole sequence (prefill).  Sequential in time, one
 * (batch, head, row) at a time, all dstate states in a plain array.
 * ------------------------------------------------------------------------- */
int oracle_selective_scan(int batch, int seqlen, int nheads, int headdim,
                          int dstate, int ngroups, const double *u,
                          const double *dt, const double *dt_bias,
                          int dt_softplus, const double *A, int a_per_state,
                          const double *B, const double *C, const double *D,
                          const double *z, double *state,
                          const int32_t *slot_idx, int nslots,
                          int has_initial_state, double *out, double *out_scale,
                          double *state_scale)
{
    if (batch < 0 || seqlen < 0 || nheads < 1 || headdim < 1 || dstate < 1 ||
        ngroups < 1 || nheads % ngroups != 0)
        return -1;
    const int heads_per_group = nheads / ngroups;
    const int channels = nheads * headdim;
    double *h = (double *)malloc(sizeof(double) * (size_t)dstate);
    double *hm = (double *)malloc(sizeof(double) * (size_t)dstate);
    if (!h || !hm) {
        free(h);
        free(hm);
        return -1;
    }
    for (int b = 0; b < batch; ++b) {
        const int slot = slot_of(slot_idx, b);
        if (slot < 0)
            continue;
        if (state && slot >= nslots) {
            free(h);
            free(hm);
            return -1;
        }
        for (int hd = 0; hd < nheads; ++hd) {
            const int g = hd / heads_per_group;
            const double *dtr = dt + ((size_t)b * nheads + hd) * (size_t)seqlen;
            const double *Br = B + ((size_t)b * ngroups + g) * (size_t)dstate * seqlen;
            const double *Cr = C + ((size_t)b * ngroups + g) * (size_t)dstate * seqlen;
            for (int p = 0; p < headdim; ++p) {
                const int c = hd * headdim + p;
                const double *ur = u + ((size_t)b * channels + c) * (size_t)seqlen;
                const double *zr = z ? z + ((size_t)b * channels + c) * (size_t)seqlen : NULL;
                double *st = state ? state + (((size_t)slot * nheads + hd) * headdim + p) * (size_t)dstate : NULL;
                for (int n = 0; n < dstate; ++n) {
                    h[n] = (st && has_initial_state) ? st[n] : 0.0;
                    hm[n] = fabs(h[n]);
                }
                for (int t = 0; t < seqlen; ++t) {
                    const double v = dtr[t] + (dt_bias ? dt_bias[hd] : 0.0);
                    const double delta = dt_softplus ? oracle_softplus(v) : v;
                    const double ut = ur[t];
                    double y = 0.0, ym = 0.0;
                    for (int n = 0; n < dstate; ++n) {
                        const double a = a_per_state ? A[(size_t)hd * dstate + n] : A[hd];
                        const double abar = exp(delta * a);
                        const double bx = delta * Br[(size_t)n * seqlen + t] * ut;
                        h[n] = abar * h[n] + bx;
                        hm[n] = abar * hm[n] + fabs(bx);
                        y += Cr[(size_t)n * seqlen + t] * h[n];
                        ym += fabs(Cr[(size_t)n * seqlen + t]) * hm[n];
                    }
                    if (D) {
                        y += D[hd] * ut;
                        ym += fabs(D[hd] * ut);
                    }
                    double gate = 1.0;
                    if (zr)
                        gate = oracle_silu(zr[t]);
                    const size_t o = ((size_t)b * channels + c) * (size_t)seqlen + t;
                    out[o] = y * gate;
                    if (out_scale)
                        out_scale[o] = ym * fabs(gate);
                }
                if (st) {
                    for (int n = 0; n < dstate; ++n) {
                        st[n] = h[n];
                        if (state_scale)
                            state_scale[(((size_t)slot * nheads + hd) * headdim + p) * (size_t)dstate + n] = hm[n];
                    }
                }
            }
        }
    }
    free(h);
    free(hm);
    return 0;
}

/* ---------------------------------------------------------------------------
 * Single-token selective state update (decode), in place on the state cache.
 *   x, z, out: [batch, nheads, headdim]; dt: [batch, nheads];
 *   B, C: [batch, ngroups, dstate]; state: [nslots, nheads, headdim, dstate].
 * Written on its own (not through the scan) so that "a scan of L tokens equals
 * L chained updates" is a check between two independent loops.
 * ------------------------------------------------------------------------- */
int oracle_state_update(int batch, int nheads, int headdim, int dstate,
                        int ngroups, double *state, const int32_t *slot_idx,
                        int nslots, const double *x, const double *dt,
                        const double *dt_bias, int dt_softplus, const double *A,
                        int a_per_state, const double *B, const double *C,
                        const double *D, const double *z, double *out,
                        double *out_scale, double *state_scale)
{
    if (batch < 0 || nheads < 1 || headdim < 1 || dstate < 1 || ngroups < 1 ||
        nheads % ngroups != 0)
        return -1;
    const int heads_per_group = nheads / ngroups;
    for (int b = 0; b < batch; ++b) {
        const int slot = slot_of(slot_idx, b);
        if (slot < 0)
            continue;
        if (slot >= nslots)
            return -1;
        for (int hd = 0; hd < nheads; ++hd) {
            const int g = hd / heads_per_group;
            const double v = dt[(size_t)b * nheads + hd] + (dt_bias ? dt_bias[hd] : 0.0);
            const double delta = dt_softplus ? oracle_softplus(v) : v;
            const double *Bv = B + ((size_t)b * ngroups + g) * (size_t)dstate;
            const double *Cv = C + ((size_t)b * ngroups + g) * (size_t)dstate;
            for (int p = 0; p < headdim; ++p) {
                const size_t io = ((size_t)b * nheads + hd) * headdim + p;
                const size_t so = (((size_t)slot * nheads + hd) * headdim + p) * (size_t)dstate;
                const double xv = x[io];
                double y = 0.0, ym = 0.0;
                for (int n = 0; n < dstate; ++n) {
                    const double a = a_per_state ? A[(size_t)hd * dstate + n] : A[hd];
                    const double abar = exp(delta * a);
                    const double bx = delta * Bv[n] * xv;
                    const double hn = abar * state[so + n] + bx;
                    const double hmag = abar * fabs(state[so + n]) + fabs(bx);
                    state[so + n] = hn;
                    if (state_scale)
                        state_scale[so + n] = hmag;
                    y += Cv[n] * hn;
                    ym += fabs(Cv[n]) * hmag;
                }
                if (D) {
                    y += D[hd] * xv;
                    ym += fabs(D[hd] * xv);
                }
                double gate = 1.0;
                if (z)
                    gate = oracle_silu(z[io]);
                out[io] = y * gate;
                if (out_scale)
                    out_scale[io] = ym * fabs(gate);
            }
        }
    }
    return 0;
}

/* ---------------------------------------------------------------------------
 * Round-to-nearest-even from double straight to a narrower binary format
 * (no intermediate float), used when the tests emulate a narrow cache between
 * chained steps.  kind: 0 = binary32, 1 = binary16, 2 = bfloat16.
 * Method: scale by the format's quantum at the value's binade (a power of two,
 * so exact), round to an integer with rint() in the default ties-to-even mode,
 * scale back; values whose rounded magnitude reaches 2^(emax+1) become inf.
 * ------------------------------------------------------------------------- */
double oracle_round(double v, int kind)
{
    int prec, emin, emax_plus1;
    switch (kind) {
    case 0: prec = 24; emin = -125; emax_plus1 = 128; break; /* binary32 */
    case 1: prec = 11; emin = -13; emax_plus1 = 16; break;   /* binary16 */
    case 2: prec = 8; emin = -125; emax_plus1 = 128; break;  /* bfloat16 */
    default: return NAN;
    }
    if (v == 0.0 || isnan(v) || isinf(v))
        return v;
    int e;
    (void)frexp(v, &e); /* v = m * 2^e with 0.5 <= |m| < 1 */
    if (e < emin)
        e = emin; /* subnormal range: fixed quantum */
    const double q = ldexp(1.0, e - prec);
    const double r = rint(v / q) * q;
    if (fabs(r) >= ldexp(1.0, emax_plus1))
        return r > 0 ? INFINITY : -INFINITY;
    return r;
}

void oracle_round_array(double *v, size_t n, int kind)
{
    for (size_t i = 0; i < n; ++i)
        v[i] = oracle_round(v[i], kind);
}
