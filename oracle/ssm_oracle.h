/*
 * ssm_oracle.h -- declarations of the float64 CPU oracle (test infrastructure
 * only; see ssm_oracle.c for the definitions, layouts and sources).
 */
#ifndef SSM_ORACLE_H
#define SSM_ORACLE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

double oracle_softplus(double v);
double oracle_silu(double v);

int oracle_causal_conv1d(int batch, int channels, int seqlen, int width,
                         const double *x, const double *weight,
                         const double *bias, double *conv_state,
                         const int32_t *slot_idx, int nslots,
                         int has_initial_state, int apply_silu, double *out,
                         double *out_scale);

int oracle_selective_scan(int batch, int seqlen, int nheads, int headdim,
                          int dstate, int ngroups, const double *u,
                          const double *dt, const double *dt_bias,
                          int dt_softplus, const double *A, int a_per_state,
                          const double *B, const double *C, const double *D,
                          const double *z, double *state,
                          const int32_t *slot_idx, int nslots,
                          int has_initial_state, double *out, double *out_scale,
                          double *state_scale);

int oracle_state_update(int batch, int nheads, int headdim, int dstate,
                        int ngroups, double *state, const int32_t *slot_idx,
                        int nslots, const double *x, const double *dt,
                        const double *dt_bias, int dt_softplus, const double *A,
                        int a_per_state, const double *B, const double *C,
                        const double *D, const double *z, double *out,
                        double *out_scale, double *state_scale);

double oracle_round(double v, int kind);
void oracle_round_array(double *v, size_t n, int kind);

#ifdef __cplusplus
}
#endif

#endif
