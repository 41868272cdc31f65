// ssu_body.hpp -- device code of the selective state update (the maps are
// described in ssu.hip), shared by its own kernels and by the mixed
// prefill + decode launch.
#pragma once
#include <algorithm>
#include <type_traits>

#include "ssm_device.hpp"
#include "ssm_kernels.hpp"

namespace ssm {

// What one lane holds for its (h,p) row and state range that does not depend
// on the request: loaded once and used for each of the lane's requests.
template <int V, int CW>
struct SsuParams {
    float an[V];                      // A[h, n] * log2(e) (per-state decays)
    float a2;                         // A[h] * log2(e) (one decay per head)
    float tap[CW > 0 ? CW : 1];
    float cbias, dtb, Dh;
    int64_t hp;                       // h * headdim + p
    int h, p, n0;
    bool in;                          // the lane has a row and a state range
};

// What one lane holds for one request between issuing its loads and storing
// its results.
template <typename TS, typename TI, int V, int CW>
struct SsuReq {
    float hs[V], bv[V], cv[V];
    // the row's values as stored (widened when used, after every load of the
    // lane has been issued)
    TI dt_raw, x_raw, z_raw;
    TI win_raw[CW > 1 ? CW - 1 : 1];
    float delta, xv, zv;
    TS *sp;
    TI *cw;
    int64_t x_off, z_off, o_off, u_off, dt_off;  // element offsets of the row's values
    bool live;
};

template <bool A_PER_STATE, bool VEC, int V, int CW>
__device__ __forceinline__ void ssu_params(const SsuArgs &a, int64_t hp, int j, SsuParams<V, CW> &q)
{
    const int64_t HP = (int64_t)a.nheads * a.headdim;
    const int n0 = j * V;
    q.in = hp < HP && n0 < a.dstate;
    q.hp = hp < HP ? hp : 0;
    q.h = (int)(q.hp / a.headdim);
    q.p = (int)(q.hp - (int64_t)q.h * a.headdim);
    q.n0 = n0 < a.dstate ? n0 : 0;
    if constexpr (A_PER_STATE) {
        const float *Ap = a.A + q.h * a.A_sh + q.n0;
        if constexpr (VEC) {
            load_vec_cached<float, V>(Ap, q.an);
        } else {
#pragma unroll
            for (int i = 0; i < V; ++i) {
                const bool ok = q.n0 + i < a.dstate;
                const float av = Ap[ok ? i : 0];
                q.an[i] = ok ? av : 0.0f;
            }
        }
#pragma unroll
        for (int i = 0; i < V; ++i)
            q.an[i] *= kLog2e;
        q.a2 = 0.0f;
    } else {
        q.a2 = a.A[q.h] * kLog2e;
    }
    // every lane of the row takes the step size, the conv and the readout's
    // D term itself (same addresses within a wave: one access per row)
    q.dtb = a.dt_bias ? a.dt_bias[q.h] : 0.0f;
    q.Dh = a.D ? a.D[q.h] : 0.0f;
    q.cbias = 0.0f;
    if constexpr (CW > 0) {
#pragma unroll
        for (int k = 0; k < CW; ++k)
            q.tap[k] = a.conv_weight[q.hp * a.cw_sc + k];
        q.cbias = a.conv_bias ? a.conv_bias[q.hp] : 0.0f;
    } else {
        q.tap[0] = 0.0f;
    }
}

// Phase 1 for one request: resolve its slot and issue all of its loads.
template <typename TS, typename TI, bool VEC, int V, int CW>
__device__ __forceinline__ void ssu_load(const SsuArgs &a, int b, int j, const SsuParams<V, CW> &q,
                                         SsuReq<TS, TI, V, CW> &r)
{
    const bool bin = b < a.batch;
    const int bb = bin ? b : 0;
    const int slot = a.slot_idx ? a.slot_idx[bb] : bb;  // uniform over the workgroup
    r.live = q.in && bin && slot >= 0;  // padded: loads from slot 0, discarded
    const int s = slot >= 0 ? slot : 0;
    r.x_off = bb * a.x_sb + q.h * a.x_sh + q.p;
    r.z_off = bb * a.z_sb + q.h * a.z_sh + q.p;
    r.o_off = bb * a.o_sb + q.h * a.o_sh + q.p;
    r.u_off = bb * a.u_sb + q.h * a.u_sh + q.p;
    r.dt_off = bb * a.dt_sb + q.h;
    const int g = q.h / a.heads_per_group;
    r.sp = static_cast<TS *>(a.state) + s * a.st_ss + q.h * a.st_sh + q.p * a.st_sp + q.n0;
    const TI *Bp = static_cast<const TI *>(a.B) + bb * a.B_sb + g * a.B_sg + q.n0;
    const TI *Cp = static_cast<const TI *>(a.C) + bb * a.C_sb + g * a.C_sg + q.n0;
    r.dt_raw = r.x_raw = r.z_raw = TI{};
    if constexpr (CW > 0) {
        r.cw = static_cast<TI *>(a.conv_state) + s * a.cs_ss + q.hp * a.cs_sc;
#pragma unroll
        for (int k = 0; k < CW - 1; ++k)
            r.win_raw[k] = TI{};
    }
    if constexpr (VEC) {
        load_vec_cached<TS, V>(r.sp, r.hs);
        if constexpr (V * StorageSize<TI>::value >= 16) {
            load_vec_cached<TI, V>(Bp, r.bv);
            load_vec_cached<TI, V>(Cp, r.cv);
        } else {
#pragma unroll
            for (int i = 0; i < V; ++i) {
                r.bv[i] = to_f32(Bp[i]);
                r.cv[i] = to_f32(Cp[i]);
            }
        }
    } else {
#pragma unroll
        for (int i = 0; i < V; ++i) {
            const bool ok = q.n0 + i < a.dstate;
            const int ii = ok ? i : 0;
            const float hv = to_f32(r.sp[ii]), bvv = to_f32(Bp[ii]), cvv = to_f32(Cp[ii]);
            r.hs[i] = ok ? hv : 0.0f;
            r.bv[i] = ok ? bvv : 0.0f;
            r.cv[i] = ok ? cvv : 0.0f;
        }
    }
}

// Phase 1b: the row's values (dt, x, z, the conv window), loaded by every lane
// of the row after all state loads have been issued, with no branch around
// them: a conversion inside a branch would be placed right after its load, and
// the wait for it would also cover every load issued before.
template <typename TS, typename TI, int V, int CW>
__device__ __forceinline__ void ssu_load_row(const SsuArgs &a, SsuReq<TS, TI, V, CW> &r)
{
    r.dt_raw = static_cast<const TI *>(a.dt)[r.dt_off];
    r.x_raw = static_cast<const TI *>(a.x)[r.x_off];
    // without a gate this reads x, and the value goes unused
    r.z_raw = a.z ? static_cast<const TI *>(a.z)[r.z_off] : static_cast<const TI *>(a.x)[r.x_off];
    if constexpr (CW > 0) {
#pragma unroll
        for (int k = 0; k < CW - 1; ++k)
            r.win_raw[k] = r.cw[k];
    }
}

// Phase 2 for one request: (fused conv), state update, store, partial readout.
template <typename TS, typename TI, bool A_PER_STATE, bool VEC, int V, int CW>
__device__ __forceinline__ float ssu_compute(const SsuArgs &a, int j, const SsuParams<V, CW> &q,
                                             SsuReq<TS, TI, V, CW> &r)
{
    float xv = to_f32(r.x_raw);
    r.zv = to_f32(r.z_raw);
    if constexpr (CW > 0) {
        // fused conv update of channel hp; the row's first lane also shifts
        // the cached window (its stored values depend on the window loads,
        // so the read has returned first)
        constexpr int HW = CW - 1;
        float acc = q.cbias;
#pragma unroll
        for (int k = 0; k < HW; ++k)
            acc = fmaf(q.tap[k], to_f32(r.win_raw[k]), acc);
        acc = fmaf(q.tap[HW], xv, acc);
        const float u = silu_f32(acc);
        if (r.live && j == 0) {
#pragma unroll
            for (int k = 0; k + 1 < HW; ++k)
                r.cw[k] = r.win_raw[k + 1];
            if (HW > 0)
                r.cw[HW - 1] = r.x_raw;
            if (a.u_out)
                static_cast<TI *>(a.u_out)[r.u_off] = from_f32<TI>(u);
        }
        xv = u;  // the update reads the float32 conv output
    }
    const float v = to_f32(r.dt_raw) + q.dtb;
    r.delta = a.dt_softplus ? softplus_f32(v) : v;
    r.xv = xv;
    const float dx = r.delta * xv;
    float y = 0.0f;
    if constexpr (A_PER_STATE) {
#pragma unroll
        for (int i = 0; i < V; ++i) {
            const float dA = exp2_hw(r.delta * q.an[i]);
            r.hs[i] = fmaf(dA, r.hs[i], dx * r.bv[i]);
            y = fmaf(r.cv[i], r.hs[i], y);
        }
    } else {
        const float dA = exp2_hw(r.delta * q.a2);
#pragma unroll
        for (int i = 0; i < V; ++i) {
            r.hs[i] = fmaf(dA, r.hs[i], dx * r.bv[i]);
            y = fmaf(r.cv[i], r.hs[i], y);
        }
    }
    if (r.live) {
        if constexpr (VEC) {
            store_vec_cached<TS, V>(r.sp, r.hs);
        } else {
#pragma unroll
            for (int i = 0; i < V; ++i)
                if (q.n0 + i < a.dstate)
                    r.sp[i] = from_f32<TS>(r.hs[i]);
        }
    }
    return r.live ? y : 0.0f;
}

// Lanes: 2^lanes_per_row_log2 per (h,p) row, each owning V consecutive
// states (blockIdx.x covers the rows of one request); blockIdx.y picks RB
// consecutive requests, which every lane takes in turn with the same
// parameters.  All loads of the RB requests are issued before any
// arithmetic.  A wave covers 64*V consecutive states of one request's slot.
template <typename TS, typename TI, bool A_PER_STATE, bool VEC, int V, int CW, int RB>
__global__ __launch_bounds__(512) void ssu_kernel(SsuArgs a)
{
    const int lpr_log2 = a.lanes_per_row_log2;
    const int64_t gid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    const int64_t hp = gid >> lpr_log2;
    const int j = (int)(gid & ((1 << lpr_log2) - 1));  // lane within the row
    SsuParams<V, CW> q;
    ssu_params<A_PER_STATE, VEC, V, CW>(a, hp, j, q);
    SsuReq<TS, TI, V, CW> r[RB];
#pragma unroll
    for (int k = 0; k < RB; ++k)
        ssu_load<TS, TI, VEC, V, CW>(a, (int)blockIdx.y * RB + k, j, q, r[k]);
#pragma unroll
    for (int k = 0; k < RB; ++k)
        ssu_load_row<TS, TI, V, CW>(a, r[k]);
    // keep the scheduler from moving arithmetic (and the waits it needs) in
    // between the loads above
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int k = 0; k < RB; ++k) {
        float y = ssu_compute<TS, TI, A_PER_STATE, VEC, V, CW>(a, j, q, r[k]);
        // sum over the row's lanes (butterfly; lanes of one row are contiguous)
        for (int o = (1 << lpr_log2) >> 1; o > 0; o >>= 1)
            y += __shfl_xor(y, o, 64);
        if (j == 0 && r[k].live) {
            if (a.D)
                y = fmaf(q.Dh, r[k].xv, y);
            if (a.z)
                y *= silu_f32(r[k].zv);
            static_cast<TI *>(a.out)[r[k].o_off] = from_f32<TI>(y);
        }
    }
}

// A stored element's bits in a 32-bit register and back (for lane moves).
__device__ __forceinline__ uint32_t raw_bits(float v) { return __float_as_uint(v); }
__device__ __forceinline__ uint32_t raw_bits(f16 v) { return __builtin_bit_cast(uint16_t, v); }
__device__ __forceinline__ uint32_t raw_bits(bf16 v) { return v.bits; }
template <typename T> __device__ __forceinline__ T from_bits(uint32_t b);
template <> __device__ __forceinline__ float from_bits<float>(uint32_t b) { return __uint_as_float(b); }
template <> __device__ __forceinline__ f16 from_bits<f16>(uint32_t b) { return __builtin_bit_cast(f16, (uint16_t)b); }
template <> __device__ __forceinline__ bf16 from_bits<bf16>(uint32_t b) { bf16 r; r.bits = (uint16_t)b; return r; }

// E elements of B or C at p (E * sizeof(T) is 8 bytes or a multiple of 16;
// p aligned to 16 bytes, or to 8 for an 8-byte read).
template <typename T, int E>
__device__ __forceinline__ void load_bc(const T *p, float (&dst)[E])
{
    if constexpr (E * StorageSize<T>::value >= 16) {
        load_vec_cached<T, E>(p, dst);
    } else {
        static_assert(E * StorageSize<T>::value == 8, "8-byte access");
        const uint2 w = *reinterpret_cast<const uint2 *>(p);
        unpack_word(w.x, &dst[0], T{});
        unpack_word(w.y, &dst[PerWord<T>::value], T{});
    }
}

// Interleaved lane map (same operation as ssu_kernel).  A wave's block is
// NCH kilobytes of one request's slot: NCH * RPC consecutive (h,p) rows of
// rowbytes = dstate * sizeof(state) each, RPC = 1024 / rowbytes.  Access k
// reads kilobyte k, lane L its 16 bytes at 16L: row k*RPC + L/LPR of the
// block, states (L % LPR)*E .. +E-1, with LPR = rowbytes / 16 lanes per row
// and E = 16 / sizeof(state).  Every lane holds all values of each of its NCH
// rows (step size, x, z, conv window) itself, so no lane waits on another.
// The host takes this map only when every wave's block lies in one group of
// heads (its B and C are shared by the block).
//
// Fused conv with rows of at least 4 lanes (COOP): the first 4 lanes of a row
// (and every further quad of it, redundantly) share the conv.  Lane v of the
// quad loads one value (window sample v for v < 3, x for v = 3) and its tap,
// the 4 products are summed across the quad, and lane v < 3 writes the
// shifted window's sample v (the quad neighbour's value), so each value is
// loaded and stored by one lane.  Without it every lane loads the whole
// window and x, and the row's first lane shifts the window.
// The interleaved map's work for wave `wave` (its rows) and request group
// `rg` (requests [rg RB, rg RB + RB)); waves are independent of each other.
template <typename TS, typename TI, bool A_PER_STATE, int CW, int RB, int NCH, bool COOP>
__device__ __forceinline__ void ssu_ilv_body(const SsuArgs &a, int64_t wave, int rg)
{
    static_assert(!COOP || CW == 4, "the quad conv takes 4 taps");
    constexpr int E = 16 / StorageSize<TS>::value;
    constexpr int HW = CW > 1 ? CW - 1 : 1;  // cached window length
    const int lg = a.lanes_per_row_log2;       // log2(LPR)
    const int lpr = 1 << lg, rpc = 64 >> lg;
    const int lane = (int)(threadIdx.x & 63);
    const int64_t HP = (int64_t)a.nheads * a.headdim;
    const int N = a.dstate;
    const int jl = lane & (lpr - 1);  // lane within its row
    const int n0 = jl * E;

    // request-independent values of the lane's NCH rows
    int64_t hp[NCH];
    int hh[NCH], pp[NCH];
    bool in[NCH];
    float an[NCH][A_PER_STATE ? E : 1], a2[NCH], dtb[NCH], Dh[NCH], cbias[NCH], tap[NCH][CW > 0 ? CW : 1];
#pragma unroll
    for (int k = 0; k < NCH; ++k) {
        const int64_t row = (wave * NCH + k) * rpc + (lane >> lg);
        in[k] = row < HP;
        hp[k] = in[k] ? row : 0;  // a wave past the last row reads row 0 and stores nothing
        hh[k] = (int)(hp[k] / a.headdim);
        pp[k] = (int)(hp[k] - (int64_t)hh[k] * a.headdim);
        if constexpr (A_PER_STATE) {
            load_vec_cached<float, E>(a.A + hh[k] * a.A_sh + n0, an[k]);
#pragma unroll
            for (int i = 0; i < E; ++i)
                an[k][i] *= kLog2e;
            a2[k] = 0.0f;
        } else {
            a2[k] = a.A[hh[k]] * kLog2e;
        }
        dtb[k] = a.dt_bias ? a.dt_bias[hh[k]] : 0.0f;
        Dh[k] = a.D ? a.D[hh[k]] : 0.0f;
        cbias[k] = 0.0f;
        tap[k][0] = 0.0f;
        if constexpr (COOP) {
            tap[k][0] = a.conv_weight[hp[k] * a.cw_sc + (jl & 3)];  // this lane's tap
            cbias[k] = a.conv_bias ? a.conv_bias[hp[k]] : 0.0f;
        } else if constexpr (CW > 0) {
#pragma unroll
            for (int c = 0; c < CW; ++c)
                tap[k][c] = a.conv_weight[hp[k] * a.cw_sc + c];
            cbias[k] = a.conv_bias ? a.conv_bias[hp[k]] : 0.0f;
        }
    }
    const int g = hh[0] / a.heads_per_group;

    // phase 1: every load of the RB requests (state and B/C first, then the
    // rows' values), before any arithmetic
    float hs[RB][NCH][E], bv[RB][E], cv[RB][E];
    TI dt_raw[RB][NCH], x_raw[RB][NCH], z_raw[RB][NCH], win[RB][NCH][HW];
    bool live[RB];
    TS *sp[RB];
    TI *cwp[RB];
    int64_t bb64[RB];
    // the row's element offset within a request's x / z / out / u_out rows
    // (32-bit: the host checks that a request's rows fit), formed where used
    auto rowoff = [&](int k, int64_t sh) { return hh[k] * (int)sh + pp[k]; };
#pragma unroll
    for (int q = 0; q < RB; ++q) {
        const int b = rg * RB + q;
        const bool bin = b < a.batch;
        const int bb = bin ? b : 0;
        const int slot = a.slot_idx ? a.slot_idx[bb] : bb;  // uniform over the workgroup
        live[q] = bin && slot >= 0;                         // padded: loads from slot 0, discarded
        const int s = slot >= 0 ? slot : 0;
        // the slot's (head, row) rows are dense: row hp at hp * N
        sp[q] = static_cast<TS *>(a.state) + s * a.st_ss + n0;
        cwp[q] = CW > 0 ? static_cast<TI *>(a.conv_state) + s * a.cs_ss : nullptr;
        bb64[q] = bb;
#pragma unroll
        for (int k = 0; k < NCH; ++k)
            load_vec<TS, E>(sp[q] + hp[k] * N, hs[q][k]);
        load_bc<TI, E>(static_cast<const TI *>(a.B) + bb * a.B_sb + g * a.B_sg + n0, bv[q]);
        load_bc<TI, E>(static_cast<const TI *>(a.C) + bb * a.C_sb + g * a.C_sg + n0, cv[q]);
    }
#pragma unroll
    for (int q = 0; q < RB; ++q) {
#pragma unroll
        for (int k = 0; k < NCH; ++k) {
            const TI *xq = static_cast<const TI *>(a.x) + bb64[q] * a.x_sb;  // uniform
            dt_raw[q][k] = (static_cast<const TI *>(a.dt) + bb64[q] * a.dt_sb)[hh[k]];
            // without a gate this reads x, and the value goes unused
            z_raw[q][k] = a.z ? (static_cast<const TI *>(a.z) + bb64[q] * a.z_sb)[rowoff(k, a.z_sh)] : xq[rowoff(k, a.x_sh)];
            if constexpr (COOP) {
                // window sample v of the row, or x for v = 3
                const int v = jl & 3;
                const TI *src = v < 3 ? cwp[q] + hp[k] * a.cs_sc + v : xq + rowoff(k, a.x_sh);
                x_raw[q][k] = *src;
            } else {
                x_raw[q][k] = xq[rowoff(k, a.x_sh)];
                if constexpr (CW > 1) {
#pragma unroll
                    for (int c = 0; c < HW; ++c)
                        win[q][k][c] = cwp[q][hp[k] * a.cs_sc + c];
                }
            }
        }
    }
    __builtin_amdgcn_sched_barrier(0);

    // phase 2: (fused conv), update, store, readout
#pragma unroll
    for (int q = 0; q < RB; ++q) {
#pragma unroll
        for (int k = 0; k < NCH; ++k) {
            const bool ok = live[q] && in[k];
            float xv = to_f32(x_raw[q][k]);
            if constexpr (COOP) {
                float acc = tap[k][0] * xv;
                acc += dpp_move_zero<DPP_QUAD_XOR1>(acc);
                acc += dpp_move_zero<DPP_QUAD_XOR2>(acc);
                acc += cbias[k];
                const float u = silu_f32(acc);
                // lane v < 3 of the row's first quad writes the shifted
                // window's sample v: the value lane v + 1 loaded
                const uint32_t nb = dpp_move_bits<DPP_QUAD_NEXT>(raw_bits(x_raw[q][k]));
                if (ok && jl < 3)
                    cwp[q][hp[k] * a.cs_sc + jl] = from_bits<TI>(nb);
                if (ok && jl == 0 && a.u_out)
                    (static_cast<TI *>(a.u_out) + bb64[q] * a.u_sb)[rowoff(k, a.u_sh)] = from_f32<TI>(u);
                xv = u;
            } else if constexpr (CW > 0) {
                float acc = cbias[k];
#pragma unroll
                for (int c = 0; c < CW - 1; ++c)
                    acc = fmaf(tap[k][c], to_f32(win[q][k][c]), acc);
                acc = fmaf(tap[k][CW - 1], xv, acc);
                const float u = silu_f32(acc);
                if (ok && jl == 0) {  // the row's first lane shifts the window
                    TI *w = cwp[q] + hp[k] * a.cs_sc;
#pragma unroll
                    for (int c = 0; c + 1 < CW - 1; ++c)
                        w[c] = win[q][k][c + 1];
                    if (CW > 1)
                        w[CW - 2] = x_raw[q][k];
                    if (a.u_out)
                        (static_cast<TI *>(a.u_out) + bb64[q] * a.u_sb)[rowoff(k, a.u_sh)] = from_f32<TI>(u);
                }
                xv = u;  // the update reads the float32 conv output
            }
            const float v = to_f32(dt_raw[q][k]) + dtb[k];
            const float delta = a.dt_softplus ? softplus_f32(v) : v;
            const float dx = delta * xv;
            float hn[E];
            float y = 0.0f;
            if constexpr (A_PER_STATE) {
#pragma unroll
                for (int i = 0; i < E; ++i) {
                    hn[i] = fmaf(exp2_hw(delta * an[k][i]), hs[q][k][i], dx * bv[q][i]);
                    y = fmaf(cv[q][i], hn[i], y);
                }
            } else {
                const float dA = exp2_hw(delta * a2[k]);
#pragma unroll
                for (int i = 0; i < E; ++i) {
                    hn[i] = fmaf(dA, hs[q][k][i], dx * bv[q][i]);
                    y = fmaf(cv[q][i], hn[i], y);
                }
            }
            if (ok)
                store_vec<TS, E>(sp[q] + hp[k] * N, hn);
            for (int o = lpr >> 1; o > 0; o >>= 1)
                y += __shfl_xor(y, o, 64);
            if (ok && jl == 0) {
                if (a.D)
                    y = fmaf(Dh[k], xv, y);
                if (a.z)
                    y *= silu_f32(to_f32(z_raw[q][k]));
                (static_cast<TI *>(a.out) + bb64[q] * a.o_sb)[rowoff(k, a.o_sh)] = from_f32<TI>(y);
            }
        }
    }
}

template <typename TS, typename TI, bool A_PER_STATE, int CW, int RB, int NCH, bool COOP>
__global__ __launch_bounds__(512) void ssu_ilv_kernel(SsuArgs a)
{
    ssu_ilv_body<TS, TI, A_PER_STATE, CW, RB, NCH, COOP>(
        a, ((int64_t)blockIdx.x * blockDim.x + threadIdx.x) >> 6, (int)blockIdx.y);
}

} // namespace ssm
