// conv1d.hip -- causal depthwise conv1d + bias + SiLU with a per-request conv
// cache, on gfx950.
//
// Operation: the causal-conv1d and silu operators of "feat(llama.cu): 适配
// mamba 模型" (InfiniLM-Rust PR #48, section 2.1), with the cache handling of
// section 3.1 (the conv operator reads the request's cached history and leaves
// the newest width-1 samples behind for the next call):
//     out[b,c,t] = silu(bias[c] + sum_{k<W} w[c,k] * xh[b,c,t-W+1+k])
// where xh is x preceded by the cached history (or zeros).
//
// Dense prefill, 16-byte aligned rows (the common case): two rows per
// 256-lane workgroup, each lane one 128-bit chunk of each row per tile plus
// the few samples in front of it (from the previous lane, by DPP), no LDS
// and no barriers (conv_rows_kernel).  The first tile's loads are issued
// before the rows' parameters are fetched.
// Other dense rows: one workgroup per (b, c) row walks the row in tiles of
// 256*E samples staged in LDS with their W-1 history (conv_prefill_kernel).
// Either way HBM traffic is x read once, out written once, and the row's
// final W-1 samples go to the cache at the end.
//
// Packed variable-length batches (sequences of different lengths side by side
// along time, each with its own slot and initial-state flag), when the packed
// rows suit the dense row kernel: each workgroup owns whole channel rows.
// With a sequence table that covers the columns exactly (and at most 8 padded
// sequences, whose columns it stores around) it runs the dense conv of each
// packed row and then redoes the first W-1 outputs of every sequence from the
// sequence's own history; with any other table it walks the rows tile by
// tile with start-aware code.  Either way it
// writes the rows' new cache tails last.  Other packed rows (unaligned, or
// more than 255 sequences) take the tiled code with one workgroup per tile
// and a separate pass for the caches.
//
// Decode kernels (seqlen == 1): gather the window from the slot, one output,
// shift the window by one in place.  The vector kernel gives each lane 8
// channels of two requests with 128-bit accesses (the taps loaded once for
// both); the scalar kernel (any channel count or alignment) gives each lane
// one channel.
#include "ssm_device.hpp"
#include "ssm_kernels.hpp"

#include <type_traits>

namespace ssm {

template <typename T, int W, bool VEC>
__global__ __launch_bounds__(256) void conv_prefill_kernel(ConvArgs a)
{
    constexpr int E = 16 / StorageSize<T>::value;  // samples per 128-bit access
    constexpr int TILE = 256 * E;
    constexpr int H = W - 1;
    constexpr int OFF = 4;                          // history sits in xs[OFF-H, OFF)
    __shared__ float xs[OFF + TILE];
    __shared__ float hist[4];

    const int64_t row = xcd_block_order(blockIdx.x, gridDim.x);  // b*channels + c
    const int b = (int)(row / a.channels), c = (int)(row % a.channels);
    const int slot = a.slot_idx ? a.slot_idx[b] : b;
    if (slot < 0)
        return;  // padded request (uniform over the workgroup)
    const int tid = threadIdx.x;

    float w[W];
#pragma unroll
    for (int k = 0; k < W; ++k)
        w[k] = a.weight[c * a.w_sc + k];
    const float bias = a.bias ? a.bias[c] : 0.0f;

    T *cs = a.conv_state ? static_cast<T *>(a.conv_state) + slot * a.cs_ss + c * a.cs_sc : nullptr;
    if (tid < H)
        hist[tid] = (a.has_initial_state && cs) ? to_f32(cs[tid]) : 0.0f;

    const T *xr = static_cast<const T *>(a.x) + b * a.x_sb + c * a.x_sc;
    T *orow = static_cast<T *>(a.out) + b * a.o_sb + c * a.o_sc;

    for (int t0 = 0; t0 < a.seqlen; t0 += TILE) {
        const int t = t0 + tid * E;
        const int len = min(TILE, a.seqlen - t0);
        float v[E];
        if (VEC && t + E <= a.seqlen) {
            load_vec<T, E>(xr + t, v);
        } else {
#pragma unroll
            for (int i = 0; i < E; ++i)
                v[i] = (t + i < a.seqlen) ? to_f32(xr[t + i]) : 0.0f;
        }
        __syncthreads();  // hist written / previous tile's readers finished
#pragma unroll
        for (int i = 0; i < E; ++i)
            xs[OFF + tid * E + i] = v[i];
        if (tid < H)
            xs[OFF - H + tid] = hist[tid];
        __syncthreads();
        float o[E];
#pragma unroll
        for (int i = 0; i < E; ++i) {
            float acc = bias;
#pragma unroll
            for (int k = 0; k < W; ++k)
                acc = fmaf(w[k], xs[OFF + tid * E + i - H + k], acc);
            o[i] = a.apply_silu ? silu_f32(acc) : acc;
        }
        if (VEC && t + E <= a.seqlen) {
            store_vec<T, E>(orow + t, o);
        } else {
#pragma unroll
            for (int i = 0; i < E; ++i)
                if (t + i < a.seqlen)
                    orow[t + i] = from_f32<T>(o[i]);
        }
        // history of the next tile: the last H samples of history||tile
        if (tid < H)
            hist[tid] = xs[OFF + len - H + tid];
    }
    __syncthreads();
    if (cs && tid < H)
        cs[tid] = from_f32<T>(hist[tid]);  // exact: the values came from T
}

// The rows of a workgroup's walk and the loads of their current tile, from
// the first loads (rows_begin, which a caller can issue early) to the
// compute (conv_rows_walk).
template <typename T, int RPW>
struct RowTiles {
    static constexpr int E = 16 / StorageSize<T>::value;  // samples per 128-bit access
    static constexpr int PW = 4;                          // samples loaded in front of a chunk (>= W-1)
    static constexpr int PB = PW * StorageSize<T>::value;  // their bytes: 8 or 16
    using Prev = typename std::conditional<PB == 16, u32x4, uint2>::type;
    const T *xr[RPW];
    int64_t rb[RPW];
    int rc[RPW];
    u32x4 raw[RPW];
    Prev praw[RPW];
};

// Issue the loads of tile t0 of the rows.  The samples in front of a chunk
// are the end of the previous lane's chunk, moved from it within the wave
// (conv_rows_walk); the first lane of a wave loads them (they belong to the
// previous wave or tile).
template <typename T, int RPW>
__device__ __forceinline__ void rows_issue(RowTiles<T, RPW> &rt, int L, int t0)
{
    using RT = RowTiles<T, RPW>;
    const int tid = threadIdx.x;
    const int t = t0 + tid * RT::E;
    const int tc = t < L ? t : 0;
    const int tp = tc > 0 ? tc - RT::PW : 0;  // clamped; sample 0 takes the history
#pragma unroll
    for (int r = 0; r < RPW; ++r) {
        // x is streamed once: non-temporal (41.9 -> 35.7 us per call on
        // the 4 x 5120 x 2048 f16 prefill)
        rt.raw[r] = __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(rt.xr[r] + tc));
        if ((tid & 63) == 0)
            rt.praw[r] = *reinterpret_cast<const typename RT::Prev *>(rt.xr[r] + tp);
    }
}

// The rows row0 .. row0 + RPW - 1 (row = b*channels + c, uniform over the
// workgroup) and the loads of their first tile, requested before anything
// else: the addresses need only the kernel arguments, while the slot, the
// taps and the history are further loads, whose latency then overlaps the
// tile's.  One division for the first row (32-bit where the rows allow: a
// 64-bit one is a long scalar sequence in front of every load), the next
// rows by stepping c.
template <typename T, int RPW>
__device__ __forceinline__ void rows_begin(RowTiles<T, RPW> &rt, const ConvArgs &a, const int64_t row0)
{
    const int64_t nrows = (int64_t)a.batch * a.channels;
    int64_t b0 = 0;
    int c0 = 0;
    if (row0 < nrows) {
        if (nrows <= (int64_t)UINT32_MAX) {
            const uint32_t q = (uint32_t)row0 / (uint32_t)a.channels;
            b0 = q;
            c0 = (int)((uint32_t)row0 - q * (uint32_t)a.channels);
        } else {
            b0 = row0 / a.channels;
            c0 = (int)(row0 % a.channels);
        }
    }
#pragma unroll
    for (int r = 0; r < RPW; ++r) {
        int64_t b = 0;
        int c = 0;
        if (row0 + r < nrows) {  // rows past the end read row 0 and store nothing
            b = b0;
            c = c0 + r;
            for (; c >= a.channels; c -= a.channels)
                ++b;
        }
        rt.rb[r] = b;
        rt.rc[r] = c;
        rt.xr[r] = static_cast<const T *>(a.x) + b * a.x_sb + c * a.x_sc;
    }
    rows_issue<T, RPW>(rt, a.seqlen, 0);
}

// Dense prefill with rows of whole 16-byte vectors: no LDS and no
// barriers.  A workgroup takes RPW rows (rows_begin has issued their first
// tile); per tile, each lane takes E samples of each of its rows (one
// 128-bit load per row, all issued before any arithmetic, so RPW loads are
// in flight per lane) and, for the taps that reach in front of them, the 4
// samples before: the end of the previous lane's chunk, moved by a DPP wave
// shift (the first lane of each wave loads them).  The first chunk of a row
// takes the row's history instead (the slot's cache or zeros).  Lane 0
// reads the histories before its first chunk and writes the rows' new tails
// after the walk, so the two accesses to a cache slot are ordered within
// one lane.
template <typename T, int W, int RPW, bool MASKED = false>
__device__ __forceinline__ void conv_rows_walk(RowTiles<T, RPW> &rt, const ConvArgs &a, const int64_t row0,
                                               const int *pads = nullptr, int npad = 0)
{
    using RT = RowTiles<T, RPW>;
    constexpr int E = RT::E;
    constexpr int H = W - 1;
    constexpr int PW = RT::PW;
    constexpr int PB = RT::PB;
    using Prev = typename RT::Prev;
    const int64_t nrows = (int64_t)a.batch * a.channels;
    const int tid = threadIdx.x, L = a.seqlen;
    const bool first = (tid & 63) == 0;
    const T *const *xr = rt.xr;
    u32x4 *raw = rt.raw;
    Prev *praw = rt.praw;

    float w[RPW][W], bias[RPW], hist[RPW][PW];
    bool live[RPW];
    T *orow[RPW];
    T *cs[RPW];
#pragma unroll
    for (int r = 0; r < RPW; ++r) {
        const int64_t b = rt.rb[r];
        const int c = rt.rc[r];
        const int slot = a.slot_idx ? a.slot_idx[b] : (int)b;
        live[r] = row0 + r < nrows && slot >= 0;  // padded request: untouched
#pragma unroll
        for (int k = 0; k < W; ++k)
            w[r][k] = a.weight[c * a.w_sc + k];
        bias[r] = a.bias ? a.bias[c] : 0.0f;
        orow[r] = static_cast<T *>(a.out) + b * a.o_sb + c * a.o_sc;
        cs[r] = (a.conv_state && slot >= 0) ? static_cast<T *>(a.conv_state) + slot * a.cs_ss + c * a.cs_sc
                                            : nullptr;
        // history in front of sample 0 (only lane 0 uses it)
#pragma unroll
        for (int k = 0; k < PW; ++k)
            hist[r][k] = 0.0f;
        if (tid == 0 && live[r] && a.has_initial_state && cs[r]) {
#pragma unroll
            for (int k = 0; k < H; ++k)
                hist[r][PW - H + k] = to_f32(cs[r][k]);
        }
    }

    for (int t0 = 0; t0 < L; t0 += 256 * E) {
        const int t = t0 + tid * E;
        const bool tin = t < L;  // L % E == 0: a chunk is all in or all out
        const int tc = tin ? t : 0;
        if (t0 > 0)
            rows_issue<T, RPW>(rt, L, t0);
#pragma unroll
        for (int r = 0; r < RPW; ++r) {
            Prev nb;
            if constexpr (PB == 16) {
                nb = u32x4{dpp_move_bits<DPP_WAVE_SHR1>(raw[r].x), dpp_move_bits<DPP_WAVE_SHR1>(raw[r].y),
                           dpp_move_bits<DPP_WAVE_SHR1>(raw[r].z), dpp_move_bits<DPP_WAVE_SHR1>(raw[r].w)};
            } else {
                nb = uint2{dpp_move_bits<DPP_WAVE_SHR1>(raw[r].z), dpp_move_bits<DPP_WAVE_SHR1>(raw[r].w)};
            }
            if (!first)
                praw[r] = nb;
        }
#pragma unroll
        for (int r = 0; r < RPW; ++r) {
            if (!(live[r] && tin))
                continue;
            float xw[PW + E];
            const uint32_t *pw = reinterpret_cast<const uint32_t *>(&praw[r]);
#pragma unroll
            for (int q = 0; q < PB / 4; ++q)
                unpack_word(pw[q], &xw[q * PerWord<T>::value], T{});
            if (tc == 0) {
#pragma unroll
                for (int k = 0; k < PW; ++k)
                    xw[k] = hist[r][k];
            }
            unpack_word(raw[r].x, &xw[PW + 0 * PerWord<T>::value], T{});
            unpack_word(raw[r].y, &xw[PW + 1 * PerWord<T>::value], T{});
            unpack_word(raw[r].z, &xw[PW + 2 * PerWord<T>::value], T{});
            unpack_word(raw[r].w, &xw[PW + 3 * PerWord<T>::value], T{});
            float o[E];
#pragma unroll
            for (int i = 0; i < E; ++i) {
                float acc = bias[r];
#pragma unroll
                for (int k = 0; k < W; ++k)
                    acc = fmaf(w[r][k], xw[PW - H + i + k], acc);
                o[i] = a.apply_silu ? silu_f32(acc) : acc;
            }
            if constexpr (MASKED) {
                // column ranges [pads[2j], pads[2j+1]) of padded sequences
                // stay untouched: a chunk meeting one stores around it
                bool hit = false;
                for (int j = 0; j < npad; ++j)
                    hit = hit || (tc < pads[2 * j + 1] && tc + E > pads[2 * j]);
                if (hit) {
#pragma unroll
                    for (int i = 0; i < E; ++i) {
                        bool pad = false;
                        for (int j = 0; j < npad; ++j)
                            pad = pad || (tc + i >= pads[2 * j] && tc + i < pads[2 * j + 1]);
                        if (!pad)
                            orow[r][tc + i] = from_f32<T>(o[i]);
                    }
                    continue;
                }
            }
            store_vec<T, E>(orow[r] + tc, o);
        }
    }
    // the new cache tail: the last H samples of history || x
    if (tid == 0) {
#pragma unroll
        for (int r = 0; r < RPW; ++r) {
            if (!live[r] || !cs[r])
                continue;
#pragma unroll
            for (int k = 0; k < H; ++k) {
                const int s = L - H + k;  // position in x (negative: in the history)
                cs[r][k] = s >= 0 ? xr[r][s] : from_f32<T>(hist[r][PW + s]);
            }
        }
    }
}

// Packed variable-length batch: x [channels, T] holds the sequences side by
// side.  One workgroup per (tile of a packed row, channel): every tile is the
// same amount of work whatever the mix of lengths.
//
// Away from sequence starts an output is the dense conv of the packed row.
// The taps of the first W-1 columns of a sequence reach in front of it and
// read its history instead (the slot's cache when the sequence continues from
// it, else zeros).  The workgroup therefore stages in LDS, besides the tile, a
// bitmask of the columns where a sequence starts, the sequence table and the
// history of each sequence starting in the tile.  A lane whose taps meet no
// start (two 32-bit LDS reads tell) computes the dense conv; the few others
// find the sequence and its history in LDS.  Tiles that hold columns of a
// padded sequence (which must be left untouched) or columns outside every
// sequence, and tables of more than kSeqCap sequences, take a
// column-by-column path that reads the table from global memory.
//
// The caches are not written here: they are written after every tile of a
// channel has read its histories (by conv_varlen_tail_kernel when each tile
// is its own workgroup, at the end of the row kernel when one workgroup
// walks all tiles of its channels).
constexpr int kSeqCap = 255;

__device__ __forceinline__ int cu_at(const int32_t *__restrict__ cu, int i, int T)
{
    return min(max(cu[i], 0), T);
}

template <typename T, int W, bool VEC>
__device__ __forceinline__ void conv_varlen_tile(const ConvArgs &a, const int k, const int c)
{
    constexpr int E = 16 / StorageSize<T>::value;
    constexpr int TILE = 256 * E;
    constexpr int H = W - 1;
    constexpr int HS = H > 0 ? H : 1;
    constexpr int OFF = 4;
    constexpr int NW = TILE / 32 + 1;   // start bits: bit o is column j0 - 32 + o
    __shared__ float xs[OFF + TILE];
    __shared__ uint32_t sbits[NW];
    __shared__ unsigned char sseq[TILE + 32];  // at a start column: the sequence starting there
    __shared__ float lhist[kSeqCap][HS];       // history of each sequence starting in the tile

    const int Tn = a.seqlen, tid = threadIdx.x, nseq = a.batch;
    // vector alignment of the row (x and out rows share it: same row stride,
    // or rows that are whole vectors)
    const int m = VEC ? (int)((c * a.x_sc) % E) : 0;
    const T *xr = static_cast<const T *>(a.x) + c * a.x_sc;  // column 0 of row c
    T *orow = static_cast<T *>(a.out) + c * a.o_sc;
    const int j0 = k * TILE - m;               // first packed column of the tile
    const int jend = min(j0 + TILE, Tn);       // end of the tile's columns in the row
    const bool staged = nseq <= kSeqCap;

    int need_slow = staged ? 0 : 1;
    // stage columns [j0 - H, j0 + TILE) of the row (zeros outside [0, T));
    // all loads from clamped addresses, issued together
    {
        const int j = j0 + tid * E;
        float v[E];
        if (VEC && j >= 0 && j + E <= Tn) {
            load_vec<T, E>(xr + j, v);
        } else {
#pragma unroll
            for (int i = 0; i < E; ++i) {
                const bool ok = j + i >= 0 && j + i < Tn;
                const float xv = to_f32(xr[ok ? j + i : 0]);
                v[i] = ok ? xv : 0.0f;
            }
        }
        const int q = j0 - H + (tid < H ? tid : 0);
        const bool qok = tid < H && q >= 0 && q < Tn;
        const float hv = to_f32(xr[qok ? q : 0]);
#pragma unroll
        for (int i = 0; i < E; ++i)
            xs[OFF + tid * E + i] = v[i];
        if (tid < H)
            xs[OFF - H + tid] = qok ? hv : 0.0f;
        if (tid < NW)
            sbits[tid] = 0u;
    }
    // one lane per sequence: its start, its history, whether it pads this tile
    int my_start = -1;
    if (staged && tid <= nseq) {
        const int ts = min(tid, nseq - 1);
        const int tb = cu_at(a.cu_seqlens, tid, Tn);
        const int te = tid < nseq ? max(cu_at(a.cu_seqlens, tid + 1, Tn), tb) : tb;
        const int slot = a.slot_idx ? a.slot_idx[ts] : ts;
        const bool init = a.has_init_seq && a.has_init_seq[ts] != 0;
        const bool touches = te > tb && tb < jend && te > max(j0, 0);
        if (touches && slot < 0)
            need_slow = 1;  // a padded sequence's columns must stay untouched
        if (te > tb && slot >= 0 && tb > j0 - H && tb < jend) {
            my_start = tb;
            const T *cs = (init && a.conv_state)
                              ? static_cast<const T *>(a.conv_state) + slot * a.cs_ss + c * a.cs_sc
                              : nullptr;
#pragma unroll
            for (int h = 0; h < H; ++h)
                lhist[tid][h] = cs ? to_f32(cs[h]) : 0.0f;
        }
        if (tid == 0 || tid == nseq) {
            // columns in front of the first sequence or after the last one
            const int lo0 = max(j0, 0);
            if ((tid == 0 && tb > lo0 && lo0 < jend) || (tid == nseq && tb < jend))
                need_slow = 1;
        }
    }
    float w[W];
#pragma unroll
    for (int kk = 0; kk < W; ++kk)
        w[kk] = a.weight[c * a.w_sc + kk];
    const float bias = a.bias ? a.bias[c] : 0.0f;
    const bool slow = __syncthreads_or(need_slow) != 0;  // tile, table, histories, cleared bits
    if (my_start >= 0) {
        const int o = my_start - j0 + 32;
        atomicOr(&sbits[o >> 5], 1u << (o & 31));
        sseq[o] = (unsigned char)tid;  // read only where the bit is set
    }
    __syncthreads();

    const int jl = j0 + tid * E;  // the lane's first column
    if (!slow) {
        // starts among columns jl-H+1 .. jl+E-1 (the ones that can cut a tap)
        const int olo = tid * E + 32 - H + 1, ohi = tid * E + 32 + E - 1;
        const uint64_t win = (uint64_t)sbits[olo >> 5] | ((uint64_t)sbits[ohi >> 5] << 32);
        const int base = olo & ~31;  // bit 0 of win is bit `base`
        const uint64_t lanebits = (win >> (olo - base)) & ((1ull << (ohi - olo + 1)) - 1);
        float o_[E];
        if (lanebits == 0) {
            // no sequence starts among the lane's taps: the dense conv
#pragma unroll
            for (int i = 0; i < E; ++i) {
                float acc = bias;
#pragma unroll
                for (int kk = 0; kk < W; ++kk)
                    acc = fmaf(w[kk], xs[OFF + tid * E + i - H + kk], acc);
                o_[i] = a.apply_silu ? silu_f32(acc) : acc;
            }
        } else {
#pragma unroll
            for (int i = 0; i < E; ++i) {
                // latest start b in (j-H, j]: bit (i + H - 1 - d) of lanebits is column j - d
                int b = INT32_MIN / 2;
#pragma unroll
                for (int d = H - 1; d >= 0; --d)
                    if ((lanebits >> (i + H - 1 - d)) & 1ull)
                        b = jl + i - d;
                const bool has_b = b != INT32_MIN / 2;
                const int sq = sseq[has_b ? b - j0 + 32 : 32];  // meaningful when has_b
                float acc = bias;
#pragma unroll
                for (int kk = 0; kk < W; ++kk) {
                    const int q = jl + i - H + kk;  // tap column
                    const bool use_h = has_b && q < b;
                    const float xv = xs[OFF + tid * E + i - H + kk];
                    const float hv = lhist[use_h ? sq : 0][use_h ? H + q - b : 0];
                    acc = fmaf(w[kk], use_h ? hv : xv, acc);
                }
                o_[i] = a.apply_silu ? silu_f32(acc) : acc;
            }
        }
        bool all = true;
#pragma unroll
        for (int i = 0; i < E; ++i)
            all = all && (jl + i >= 0 && jl + i < Tn);
        if (VEC && all) {
            store_vec<T, E>(orow + jl, o_);
        } else {
#pragma unroll
            for (int i = 0; i < E; ++i)
                if (jl + i >= 0 && jl + i < Tn)
                    orow[jl + i] = from_f32<T>(o_[i]);
        }
        return;
    }

    // column by column, the table read from global memory
    int s = 0;
    {
        const int jc = max(min(jl, Tn - 1), 0);
        int lo = 0, hi = nseq;  // the last s with cu[s] <= jc
        while (hi - lo > 1) {
            const int mid = (lo + hi) >> 1;
            if (cu_at(a.cu_seqlens, mid, Tn) <= jc)
                lo = mid;
            else
                hi = mid;
        }
        s = lo;
    }
    int cur = -1, tb = 0, te = 0, slot = -1;
    const T *hist = nullptr;  // the sequence's cached history, or null (zeros)
    for (int i = 0; i < E; ++i) {
        const int j = jl + i;
        if (j < 0 || j >= Tn)
            continue;
        // advance to the sequence holding column j (skipping empty ones)
        while (s + 1 < nseq && cu_at(a.cu_seqlens, s + 1, Tn) <= j)
            ++s;
        if (s != cur) {
            cur = s;
            tb = cu_at(a.cu_seqlens, s, Tn);
            te = max(cu_at(a.cu_seqlens, s + 1, Tn), tb);
            slot = a.slot_idx ? a.slot_idx[s] : s;
            const bool init = a.has_init_seq && a.has_init_seq[s] != 0;
            hist = (init && a.conv_state && slot >= 0)
                       ? static_cast<const T *>(a.conv_state) + slot * a.cs_ss + c * a.cs_sc
                       : nullptr;
        }
        if (slot < 0 || j < tb || j >= te)
            continue;
        float acc = bias;
#pragma unroll
        for (int kk = 0; kk < W; ++kk) {
            const int q = j - H + kk;  // tap column
            float xv;
            if (q >= tb)
                xv = xs[OFF + tid * E + i - H + kk];
            else
                xv = hist ? to_f32(hist[H + q - tb]) : 0.0f;
            acc = fmaf(w[kk], xv, acc);
        }
        orow[j] = from_f32<T>(a.apply_silu ? silu_f32(acc) : acc);
    }
}

template <typename T, int W, bool VEC>
__global__ __launch_bounds__(256) void conv_varlen_kernel(ConvArgs a)
{
    conv_varlen_tile<T, W, VEC>(a, blockIdx.x, blockIdx.y);  // tile, channel
}

// A packed batch over the dense row kernel's grid: the workgroup owns its
// channel rows for every sequence, so it alone reads and rewrites those rows'
// caches and no separate cache pass is needed.
//
// Table covering the packed row (cu_seqlens rising from 0 to the packed
// length) with at most 8 padded sequences: the dense conv of each packed
// channel row as one request with no history, storing around the padded
// sequences' columns; then one lane per (sequence, row) redoes the
// sequence's first W-1 outputs, whose taps in front of the start read the
// previous sequence's samples, from the sequence's own history (its slot's
// cache, or zeros), summing the taps in the dense order.  Any other table:
// the start-aware tiled code over the rows.  Either way the same lanes then
// write each sequence's new cache tail, the last W-1 samples of history ||
// sequence.
template <typename T, int W, int RPW>
__device__ __forceinline__ void conv_rows_packed(ConvArgs a, const int64_t row0)
{
    constexpr int H = W - 1;
    constexpr int HS = H > 0 ? H : 1;
    const int tid = threadIdx.x, nseq = a.batch, Tn = a.seqlen;
    const ConvArgs pa = a;  // the packed-batch arguments
    // the dense walk's view: each packed channel row as one request with no
    // history; its first tile is requested before the table is read (if the
    // table turns out not to suit the walk, those values go unused)
    ConvArgs da = a;
    da.batch = 1;
    da.slot_idx = nullptr;
    da.conv_state = nullptr;
    da.has_initial_state = 0;
    RowTiles<T, RPW> rt;
    rows_begin<T, RPW>(rt, da, row0);
    // lane t <= nseq: entry t of the table (lane t < nseq: sequence t)
    constexpr int kPadCap = 8;  // padded sequences the dense walk stores around
    __shared__ int s_pads[2 * kPadCap];
    __shared__ int s_npad;
    int cb = 0, ce = 0, slot = -1, bad = 0, padded = 0;
    bool init = false;
    if (tid == 0)
        s_npad = 0;
    if (tid <= nseq) {
        cb = a.cu_seqlens[tid];
        ce = a.cu_seqlens[tid < nseq ? tid + 1 : tid];
        slot = tid < nseq ? (a.slot_idx ? a.slot_idx[tid] : tid) : -1;
        init = tid < nseq && a.has_init_seq && a.has_init_seq[tid] != 0;
        bad = ce < cb || (tid == 0 && cb != 0) || (tid == nseq && cb != Tn);
        padded = tid < nseq && slot < 0 && ce > cb;
    }
    // the table covers the packed row exactly; with no padded sequence the
    // dense walk stores every column, with a few it stores around them
    const bool covered = __syncthreads_or(bad) == 0;
    const int npad = __syncthreads_count(padded);
    const bool plain = covered && npad == 0;
    const bool masked = covered && npad > 0 && npad <= kPadCap;
    if (masked) {
        if (padded) {
            const int j = atomicAdd(&s_npad, 1);
            s_pads[2 * j] = cb;
            s_pads[2 * j + 1] = ce;
        }
        __syncthreads();
    }

    // One lane per (sequence, row) then redoes the sequence's first W-1
    // outputs and writes its cache tail.  Its inputs (the cached history,
    // the first and the last H samples) do not depend on the walk's outputs:
    // they are requested now, so their latency overlaps the walk's.
    const int tb = min(max(cb, 0), Tn);
    const int te = min(max(ce, tb), Tn);
    const int len = te - tb;
    const bool fix = H > 0 && tid < nseq && slot >= 0 && len > 0;
    T hraw[RPW][HS], xb[RPW][HS], xe[RPW][HS];
    if (fix) {
#pragma unroll
        for (int r = 0; r < RPW; ++r) {
            const int64_t c = min(row0 + r, (int64_t)pa.channels - 1);  // rows past the end: unused
            const T *cs = pa.conv_state ? static_cast<const T *>(pa.conv_state) + slot * pa.cs_ss + c * pa.cs_sc
                                        : nullptr;
            const T *xr = static_cast<const T *>(pa.x) + c * pa.x_sc + tb;
            // every sample from an in-bounds address, issued together
#pragma unroll
            for (int k = 0; k < H; ++k) {
                hraw[r][k] = cs ? cs[k] : from_f32<T>(0.0f);
                xb[r][k] = xr[min(k, len - 1)];
                xe[r][k] = xr[max(len - H + k, 0)];
            }
        }
    }

    if (plain) {
        conv_rows_walk<T, W, RPW>(rt, da, row0);
    } else if (masked) {
        conv_rows_walk<T, W, RPW, true>(rt, da, row0, s_pads, npad);
    } else {
        constexpr int E = 16 / StorageSize<T>::value;
        constexpr int TILE = 256 * E;
        const int ntiles = (Tn + TILE - 1) / TILE;
        for (int r = 0; r < RPW; ++r) {
            const int64_t c = row0 + r;
            if (c >= pa.channels)
                break;
            for (int k = 0; k < ntiles; ++k) {
                __syncthreads();  // the previous tile's LDS is free
                conv_varlen_tile<T, W, true>(pa, k, (int)c);
            }
        }
    }
    if (H == 0)
        return;
    // every wave's stores of the rows' outputs have completed (reached the
    // L2, which all waves of the workgroup write through) before any lane
    // rewrites a start: vmcnt(0), expcnt and lgkmcnt left free
    __builtin_amdgcn_s_waitcnt(0x0F70);
    __syncthreads();
    if (!fix)
        return;
#pragma unroll
    for (int r = 0; r < RPW; ++r) {
        const int64_t c = row0 + r;
        if (c >= pa.channels)
            break;
        T *cs = pa.conv_state ? static_cast<T *>(pa.conv_state) + slot * pa.cs_ss + c * pa.cs_sc : nullptr;
        if (plain || masked) {
            float hx[2 * HS];  // history || the first H samples (zeros past the end)
#pragma unroll
            for (int k = 0; k < H; ++k) {
                hx[k] = init ? to_f32(hraw[r][k]) : 0.0f;
                hx[H + k] = k < len ? to_f32(xb[r][k]) : 0.0f;
            }
            float w[W];
#pragma unroll
            for (int kk = 0; kk < W; ++kk)
                w[kk] = pa.weight[c * pa.w_sc + kk];
            const float bias = pa.bias ? pa.bias[c] : 0.0f;
            T *orow = static_cast<T *>(pa.out) + c * pa.o_sc + tb;
#pragma unroll
            for (int j = 0; j < H; ++j) {
                if (j >= len)
                    break;
                float acc = bias;
#pragma unroll
                for (int kk = 0; kk < W; ++kk)
                    acc = fmaf(w[kk], hx[j + kk], acc);
                orow[j] = from_f32<T>(pa.apply_silu ? silu_f32(acc) : acc);
            }
        }
        if (cs) {
#pragma unroll
            for (int k = 0; k < H; ++k) {
                const int tau = len - H + k;  // step of the k-th kept sample
                T v = from_f32<T>(0.0f);      // before the sequence, with no history
                if (tau >= 0) {
                    v = xe[r][k];
                } else if (init) {
#pragma unroll
                    for (int m = 0; m < H; ++m)
                        if (m == H + tau)
                            v = hraw[r][m];
                }
                cs[k] = v;
            }
        }
    }
}

template <typename T, int W, int RPW, bool VARLEN>
__global__ __launch_bounds__(256) void conv_rows_kernel(ConvArgs a)
{
    const int64_t row0 = (int64_t)xcd_block_order(blockIdx.x, gridDim.x) * RPW;
    if constexpr (VARLEN) {
        conv_rows_packed<T, W, RPW>(a, row0);
    } else {
        RowTiles<T, RPW> rt;
        rows_begin<T, RPW>(rt, a, row0);
        conv_rows_walk<T, W, RPW>(rt, a, row0);
    }
}


// Conv caches of a packed batch, after conv_varlen_kernel: one lane per
// (sequence, channel) copies the last W-1 samples of history || sequence
// into the slot.  Each lane reads only the cache row it writes.
template <typename T, int W>
__global__ __launch_bounds__(256) void conv_varlen_tail_kernel(ConvArgs a)
{
    constexpr int H = W - 1;
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (i >= (int64_t)a.batch * a.channels)
        return;
    const int s = (int)(i / a.channels), c = (int)(i % a.channels);
    const int Tn = a.seqlen;
    const int tb = min(max(a.cu_seqlens[s], 0), Tn);
    const int te = min(max(a.cu_seqlens[s + 1], tb), Tn);
    const int slot = a.slot_idx ? a.slot_idx[s] : s;
    if (slot < 0 || te == tb)
        return;
    const bool init = a.has_init_seq && a.has_init_seq[s] != 0;
    T *cs = static_cast<T *>(a.conv_state) + slot * a.cs_ss + c * a.cs_sc;
    const T *xr = static_cast<const T *>(a.x) + c * a.x_sc + tb;
    const int len = te - tb;
    T v[H > 0 ? H : 1];
#pragma unroll
    for (int k = 0; k < H; ++k) {
        const int tau = len - H + k;  // step of the k-th kept sample
        v[k] = tau >= 0 ? xr[tau] : (init ? cs[H + tau] : from_f32<T>(0.0f));
    }
#pragma unroll
    for (int k = 0; k < H; ++k)
        cs[k] = v[k];
}

template <typename T, int W>
__global__ __launch_bounds__(256) void conv_decode_kernel(ConvArgs a)
{
    constexpr int H = W - 1;
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (i >= (int64_t)a.batch * a.channels)
        return;
    const int b = (int)(i / a.channels), c = (int)(i % a.channels);
    const int slot = a.slot_idx ? a.slot_idx[b] : b;
    if (slot < 0)
        return;
    T *cs = a.conv_state ? static_cast<T *>(a.conv_state) + slot * a.cs_ss + c * a.cs_sc : nullptr;
    const T xv_raw = static_cast<const T *>(a.x)[b * a.x_sb + c * a.x_sc];
    T win[H > 0 ? H : 1];
    float acc = a.bias ? a.bias[c] : 0.0f;
#pragma unroll
    for (int k = 0; k < H; ++k) {
        win[k] = cs ? cs[k] : T{};
        const float hv = (a.has_initial_state && cs) ? to_f32(win[k]) : 0.0f;
        acc = fmaf(a.weight[c * a.w_sc + k], hv, acc);
    }
    acc = fmaf(a.weight[c * a.w_sc + H], to_f32(xv_raw), acc);
    static_cast<T *>(a.out)[b * a.o_sb + c * a.o_sc] = from_f32<T>(a.apply_silu ? silu_f32(acc) : acc);
    if (cs) {
        // shift the window by one; without an initial state the history is
        // zeros, so the new window is (0, ..., 0, x)
#pragma unroll
        for (int k = 0; k + 1 < H; ++k)
            cs[k] = a.has_initial_state ? win[k + 1] : from_f32<T>(0.0f);
        if (H > 0)
            cs[H - 1] = xv_raw;
    }
}

// Decode with 128-bit accesses: one lane per 8 consecutive channels of one
// request (channels % 8 == 0; x, out, the cache rows and the taps contiguous
// over channels and 16-byte aligned).  The 8 windows of width-1 samples are
// contiguous in the cache row, so a lane reads and writes them as whole
// vectors; the window values pass through float32 unchanged.
template <typename T, int W, int RB>
__global__ __launch_bounds__(256) void conv_decode_vec_kernel(ConvArgs a)
{
    // blockIdx.x: groups of G channels; blockIdx.y: RB consecutive requests,
    // which each lane takes in turn with the same taps and bias (loaded once)
    constexpr int H = W - 1, G = 8;
    const int groups = a.channels / G;
    const int gi = (int)(blockIdx.x * blockDim.x + threadIdx.x);
    if (gi >= groups)
        return;
    const int c0 = gi * G;
    float w[G * W], bias[G];
    load_vec_cached<float, G * W>(a.weight + (int64_t)c0 * W, w);
    if (a.bias)
        load_vec_cached<float, G>(a.bias + c0, bias);
    else
#pragma unroll
        for (int g = 0; g < G; ++g)
            bias[g] = 0.0f;
    // every request's loads are issued before any arithmetic, with no
    // branch or select around them: widening a value inside a branch makes
    // the compiler wait for it there, and that wait covers every load issued
    // before (the next request's loads would start a second round trip)
    constexpr int NWV = H > 0 ? G * H * (int)sizeof(T) / 16 : 1;  // window vectors
    static_assert(H == 0 || NWV * 16 == G * H * (int)sizeof(T), "G*H samples fill whole vectors");
    float xv[RB][G];
    u32x4 wraw[RB][NWV];
    T *cs[RB];
    bool live[RB];
    const bool init = a.conv_state && a.has_initial_state;
#pragma unroll
    for (int k = 0; k < RB; ++k) {
        const int b = (int)blockIdx.y * RB + k;  // uniform over the workgroup
        const int bb = b < a.batch ? b : 0;
        const int slot = a.slot_idx ? a.slot_idx[bb] : bb;
        live[k] = b < a.batch && slot >= 0;  // padded request: untouched
        const int s = slot >= 0 ? slot : 0;
        load_vec_cached<T, G>(static_cast<const T *>(a.x) + bb * a.x_sb + c0, xv[k]);
        cs[k] = a.conv_state ? static_cast<T *>(a.conv_state) + s * a.cs_ss + (int64_t)c0 * H : nullptr;
        if constexpr (H > 0) {
            // without a cache (or its history) the weights are read instead
            // and the values replaced by zeros below
            const u32x4 *src = reinterpret_cast<const u32x4 *>(
                init ? static_cast<const void *>(cs[k]) : static_cast<const void *>(a.weight));
#pragma unroll
            for (int v = 0; v < NWV; ++v)
                wraw[k][v] = src[v];
        }
    }
#pragma unroll
    for (int k = 0; k < RB; ++k) {
        if (!live[k])
            continue;
        const int b = (int)blockIdx.y * RB + k;
        float win[G * H > 0 ? G * H : 1];
        if constexpr (H > 0) {
            constexpr int PW = PerWord<T>::value;
#pragma unroll
            for (int v = 0; v < NWV; ++v) {
                unpack_word(wraw[k][v].x, &win[(4 * v + 0) * PW], T{});
                unpack_word(wraw[k][v].y, &win[(4 * v + 1) * PW], T{});
                unpack_word(wraw[k][v].z, &win[(4 * v + 2) * PW], T{});
                unpack_word(wraw[k][v].w, &win[(4 * v + 3) * PW], T{});
            }
#pragma unroll
            for (int q = 0; q < G * H; ++q)
                win[q] = init ? win[q] : 0.0f;
        }
        float o[G];
#pragma unroll
        for (int g = 0; g < G; ++g) {
            float acc = bias[g];
#pragma unroll
            for (int q = 0; q < H; ++q)
                acc = fmaf(w[g * W + q], win[g * H + q], acc);
            acc = fmaf(w[g * W + H], xv[k][g], acc);
            o[g] = a.apply_silu ? silu_f32(acc) : acc;
        }
        store_vec_cached<T, G>(static_cast<T *>(a.out) + b * a.o_sb + c0, o);
        if constexpr (H > 0) {
            if (cs[k]) {
                float nw[G * H];
#pragma unroll
                for (int g = 0; g < G; ++g) {
#pragma unroll
                    for (int q = 0; q + 1 < H; ++q)
                        nw[g * H + q] = win[g * H + q + 1];
                    nw[g * H + H - 1] = xv[k][g];
                }
                store_vec_cached<T, G * H>(cs[k], nw);
            }
        }
    }
}

template <typename T, int W>
static hipError_t launch_conv_tw(const ConvArgs &a, hipStream_t stream)
{
    // decode: two requests per lane in 64-lane workgroups (8.3 -> 7.0 us on
    // the 245-request Mamba-1 2.8B step; four per lane, or wider workgroups,
    // leave too few workgroups to fill the chip)
    if (!a.cu_seqlens && a.seqlen == 1 && a.vec_decode && (a.batch + 1) / 2 <= 65535) {
        constexpr int RB = 2;   // requests per lane (grid y = request groups)
        constexpr int BT = 64;  // lanes per workgroup
        const dim3 grid((unsigned)((a.channels / 8 + BT - 1) / BT), (unsigned)((a.batch + RB - 1) / RB));
        hipLaunchKernelGGL((conv_decode_vec_kernel<T, W, RB>), grid, dim3(BT), 0, stream, a);
    } else if (!a.cu_seqlens && a.seqlen == 1) {
        const int64_t n = (int64_t)a.batch * a.channels;
        hipLaunchKernelGGL((conv_decode_kernel<T, W>), dim3((unsigned)((n + 255) / 256)), dim3(256), 0,
                           stream, a);
    } else if (a.cu_seqlens && a.rows16 && a.batch <= 255) {
        // packed batch whose rows the dense kernel can walk: the dense walk
        // (storing around up to 8 padded sequences), else the tiled code;
        // then the starts and the caches, in one launch
        constexpr int RPW = 2;
        const dim3 grid((unsigned)((a.channels + RPW - 1) / RPW));
        hipLaunchKernelGGL((conv_rows_kernel<T, W, RPW, true>), grid, dim3(256), 0, stream, a);
    } else if (a.cu_seqlens) {
        constexpr int E = 16 / StorageSize<T>::value;
        // rows start inside a vector only when the row stride or the packed
        // length is not a multiple of E; then one more tile covers the
        // shifted walk
        const bool shifted = (a.x_sc % E) != 0 || (a.seqlen % E) != 0;
        const int ntiles = (a.seqlen + (shifted ? E - 1 : 0) + 256 * E - 1) / (256 * E);
        const dim3 grid((unsigned)ntiles, (unsigned)a.channels);
        if (a.vec)
            hipLaunchKernelGGL((conv_varlen_kernel<T, W, true>), grid, dim3(256), 0, stream, a);
        else
            hipLaunchKernelGGL((conv_varlen_kernel<T, W, false>), grid, dim3(256), 0, stream, a);
        if (a.conv_state && W > 1) {  // the caches, once every tile has read them
            const int64_t n = (int64_t)a.batch * a.channels;
            hipLaunchKernelGGL((conv_varlen_tail_kernel<T, W>), dim3((unsigned)((n + 255) / 256)), dim3(256),
                               0, stream, a);
        }
    } else if (a.vec) {
        constexpr int RPW = 2;  // rows per workgroup
        const dim3 grid((unsigned)(((int64_t)a.batch * a.channels + RPW - 1) / RPW));
        hipLaunchKernelGGL((conv_rows_kernel<T, W, RPW, false>), grid, dim3(256), 0, stream, a);
    } else {
        const dim3 grid((unsigned)((int64_t)a.batch * a.channels));
        hipLaunchKernelGGL((conv_prefill_kernel<T, W, false>), grid, dim3(256), 0, stream, a);
    }
    return hipGetLastError();
}

template <typename T>
static hipError_t launch_conv_t(const ConvArgs &a, hipStream_t stream)
{
    switch (a.width) {
    case 1: return launch_conv_tw<T, 1>(a, stream);
    case 2: return launch_conv_tw<T, 2>(a, stream);
    case 3: return launch_conv_tw<T, 3>(a, stream);
    default: return launch_conv_tw<T, 4>(a, stream);
    }
}

hipError_t launch_conv(const ConvArgs &a, hipStream_t stream)
{
    switch (a.dtype) {
    case 0: return launch_conv_t<float>(a, stream);
    case 1: return launch_conv_t<f16>(a, stream);
    default: return launch_conv_t<bf16>(a, stream);
    }
}

} // namespace ssm
