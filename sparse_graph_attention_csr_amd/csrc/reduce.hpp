// Min/max reduction aggregation over a CSR neighbourhood (gfx950, wave64).
//
// out[i,f] = min (or max) over the in-edges e of row i of X[colidx[e], f]; the
// winner is the first CSR position attaining it, arg[i,f] = that position
// (reduction-based aggregation family: IO-aware layers abstract; min/max
// pooling: Yandex Research blog, paragraph on aggregation layers). Heavy rows
// arrive split into chunks by the plan's degree-aware work list and their
// partial (value, position) pairs are merged in chunk order.
//
// Lane geometry. A node row of F features is F / VEC fragments of 16 bytes.
// One edge occupies LPE lanes (the smallest power of two covering the row,
// at most 64); a lane holds NF fragments, k * LPE + pos for k < NF; a wave
// takes EPW = 64 / LPE edges of the same row side by side. Every comparison
// is exact (bf16 widens to fp32 exactly), so any processing order that keeps
// the (value, position) order gives the same bits: inside a lane group edges
// come in increasing position, and groups and chunks combine
// lexicographically.
#pragma once

#include "device.hpp"

namespace sgat {

constexpr int32_t kNoEdge = 0x7fffffff;   // position of a lane group that saw no edge

template <bool MAX>
__device__ __forceinline__ bool beats(float x, float cur) { return MAX ? x > cur : x < cur; }

// (v2, p2) precedes (v1, p1): a strictly better value, or an equal one at a
// lower position.
template <bool MAX>
__device__ __forceinline__ bool precedes(float v2, int32_t p2, float v1, int32_t p1)
{
    return beats<MAX>(v2, v1) || (v2 == v1 && p2 < p1);
}

// The exact element bits of a value that was widened from type DT.
template <int DT>
__device__ __forceinline__ void stg_exact(void* base, int64_t elem, const float (&x)[Elem<DT>::VEC])
{
    uint4 v;
    if constexpr (DT == SGAT_F32) {
        v = make_uint4(__float_as_uint(x[0]), __float_as_uint(x[1]), __float_as_uint(x[2]),
                       __float_as_uint(x[3]));
    } else {
        uint32_t w[4];
#pragma unroll
        for (int k = 0; k < 4; ++k)
            w[k] = (__float_as_uint(x[2 * k]) >> 16) | (__float_as_uint(x[2 * k + 1]) & 0xffff0000u);
        v = make_uint4(w[0], w[1], w[2], w[3]);
    }
    *reinterpret_cast<uint4*>(static_cast<char*>(base) + elem * Elem<DT>::BYTES) = v;
}

template <int N>
__device__ __forceinline__ void st_i32(int32_t* p, const int32_t (&x)[N])
{
    static_assert(N % 4 == 0, "");
#pragma unroll
    for (int k = 0; k < N; k += 4)
        *reinterpret_cast<int4*>(p + k) = make_int4(x[k], x[k + 1], x[k + 2], x[k + 3]);
}

template <int N>
__device__ __forceinline__ void ld_i32(const int32_t* p, int32_t (&x)[N])
{
#pragma unroll
    for (int k = 0; k < N; k += 4) {
        const int4 v = *reinterpret_cast<const int4*>(p + k);
        x[k] = v.x; x[k + 1] = v.y; x[k + 2] = v.z; x[k + 3] = v.w;
    }
}

struct ReduceFwdArgs {
    const sgat_work_item* items;
    int64_t n_items;
    int F;
    const int32_t* colidx;
    const void* X;
    void* out;
    int32_t* arg;          // may be null: no winners written
    float* part_val;       // [row_slots][F]
    int32_t* part_pos;     // [row_slots][F]
};

template <int DT, int LPE, int NF, bool MAX, int U>
__global__ __launch_bounds__(kBlock) void reduce_fwd_rows(ReduceFwdArgs a)
{
    constexpr int VEC = Elem<DT>::VEC;
    constexpr int EPW = kWave / LPE;
    const int64_t unit = logical_block() * kWavesPerBlock + wave_id();
    if (unit >= a.n_items) return;
    const sgat_work_item it = a.items[unit];
    const int lane = threadIdx.x & 63, sub = lane / LPE, pos = lane % LPE;
    const int64_t F = a.F;
    bool fv[NF];
#pragma unroll
    for (int k = 0; k < NF; ++k) fv[k] = (k * LPE + pos) * VEC < F;

    float cur[NF][VEC];
    int32_t at[NF][VEC];
#pragma unroll
    for (int k = 0; k < NF; ++k)
#pragma unroll
        for (int v = 0; v < VEC; ++v) {
            cur[k][v] = MAX ? -__builtin_inff() : __builtin_inff();
            at[k][v] = kNoEdge;
        }

    const int32_t* ci = a.colidx + it.begin;
    const int32_t first = static_cast<int32_t>(it.begin);
    for (int base = 0; base < it.len; base += kWave) {
        const int nb = min(kWave, it.len - base);
        const int cj = lane < nb ? ci[base + lane] : 0;
        for (int t = 0; t < nb; t += EPW * U) {
            Frag xf[U][NF];
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const int e = t + u * EPW + sub;
                const int64_t j = bcast<EPW>(cj, e);
#pragma unroll
                for (int k = 0; k < NF; ++k) {
                    xf[u][k] = frag_zero();
                    if (e < nb && fv[k]) xf[u][k] = ldg<DT>(a.X, j * F + (k * LPE + pos) * VEC);
                }
            }
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const int e = t + u * EPW + sub;
                const bool ok = e < nb;
                const int32_t p = first + base + e;
#pragma unroll
                for (int k = 0; k < NF; ++k) {
                    float x[VEC];
                    to_f32<DT>(xf[u][k], x);
#pragma unroll
                    for (int v = 0; v < VEC; ++v)
                        if (ok && beats<MAX>(x[v], cur[k][v])) { cur[k][v] = x[v]; at[k][v] = p; }
                }
            }
        }
    }
    // A group whose values never beat the start value (all +inf for min, all
    // -inf for max) still has a winner: its first edge, of that value.
    if (sub < it.len) {
#pragma unroll
        for (int k = 0; k < NF; ++k)
#pragma unroll
            for (int v = 0; v < VEC; ++v)
                if (at[k][v] == kNoEdge) at[k][v] = first + sub;
    }
    if constexpr (EPW > 1) {
#pragma unroll
        for (int off = LPE; off < kWave; off <<= 1)
#pragma unroll
            for (int k = 0; k < NF; ++k)
#pragma unroll
                for (int v = 0; v < VEC; ++v) {
                    const float v2 = __shfl_xor(cur[k][v], off);
                    const int32_t p2 = __shfl_xor(at[k][v], off);
                    if (precedes<MAX>(v2, p2, cur[k][v], at[k][v])) { cur[k][v] = v2; at[k][v] = p2; }
                }
    }
    if (sub != 0) return;
#pragma unroll
    for (int k = 0; k < NF; ++k) {
        if (!fv[k]) continue;
        const int64_t col = (k * LPE + pos) * VEC;
        if (it.slot < 0) {
            float o[VEC];
            int32_t w[VEC];
#pragma unroll
            for (int v = 0; v < VEC; ++v) {
                const bool none = at[k][v] == kNoEdge;
                o[v] = none ? 0.f : cur[k][v];
                w[v] = none ? -1 : at[k][v];
            }
            stg_exact<DT>(a.out, static_cast<int64_t>(it.row) * F + col, o);
            if (a.arg) st_i32<VEC>(a.arg + static_cast<int64_t>(it.row) * F + col, w);
        } else {
            st_f32<VEC>(a.part_val + static_cast<int64_t>(it.slot) * F + col, cur[k]);
            st_i32<VEC>(a.part_pos + static_cast<int64_t>(it.slot) * F + col, at[k]);
        }
    }
}

// Chunks of a split row, combined in chunk order: one thread per feature.
struct ReduceMergeArgs {
    const sgat_split* splits;
    int F;
    const float* part_val;
    const int32_t* part_pos;
    void* out;
    int32_t* arg;
};

template <int DT, bool MAX>
__global__ __launch_bounds__(kBlock) void reduce_merge(ReduceMergeArgs a)
{
    const sgat_split sp = a.splits[blockIdx.x];
    const int f = blockIdx.y * kBlock + threadIdx.x;
    if (f >= a.F) return;
    const int64_t F = a.F;
    const float* pv = a.part_val + static_cast<int64_t>(sp.first_slot) * F + f;
    const int32_t* pp = a.part_pos + static_cast<int64_t>(sp.first_slot) * F + f;
    float cur = pv[0];
    int32_t at = pp[0];
    for (int s = 1; s < sp.nslots; ++s) {
        const float v2 = pv[s * F];
        const int32_t p2 = pp[s * F];
        if (precedes<MAX>(v2, p2, cur, at)) { cur = v2; at = p2; }
    }
    const int64_t oi = static_cast<int64_t>(sp.row) * F + f;
    if constexpr (DT == SGAT_F32) static_cast<float*>(a.out)[oi] = cur;
    else static_cast<uint16_t*>(a.out)[oi] = static_cast<uint16_t>(__float_as_uint(cur) >> 16);
    if (a.arg) a.arg[oi] = at;
}

// Backward over the transposed CSR: for source j and each of its out-edges
// e = (j -> i), feature f of dX[j] takes dout[i,f] where arg[i,f] == e. The
// winners are read once per edge; dout only where an edge won. Sums run in
// transposed-CSR order (lane groups and chunks in fixed order).
struct ReduceBwdArgs {
    const sgat_work_item* items;
    int64_t n_items;
    int F;
    const int32_t* rowidx;
    const int32_t* col_edge;
    const int32_t* arg;
    const void* dO;
    void* dX;
    float* part;           // [col_slots][F]
};

template <int DT, int LPE, int NF, int U>
__global__ __launch_bounds__(kBlock) void reduce_bwd_cols(ReduceBwdArgs a)
{
    constexpr int VEC = Elem<DT>::VEC;
    constexpr int EPW = kWave / LPE;
    const int64_t unit = logical_block() * kWavesPerBlock + wave_id();
    if (unit >= a.n_items) return;
    const sgat_work_item it = a.items[unit];
    const int lane = threadIdx.x & 63, sub = lane / LPE, pos = lane % LPE;
    const int64_t F = a.F;
    bool fv[NF];
#pragma unroll
    for (int k = 0; k < NF; ++k) fv[k] = (k * LPE + pos) * VEC < F;

    float acc[NF][VEC];
#pragma unroll
    for (int k = 0; k < NF; ++k)
#pragma unroll
        for (int v = 0; v < VEC; ++v) acc[k][v] = 0.f;

    const int32_t* ri = a.rowidx + it.begin;
    const int32_t* ce = a.col_edge + it.begin;
    for (int base = 0; base < it.len; base += kWave) {
        const int nb = min(kWave, it.len - base);
        const int li = lane < nb ? ri[base + lane] : 0;
        const int le = lane < nb ? ce[base + lane] : -1;
        for (int t = 0; t < nb; t += EPW * U) {
            int32_t w[U][NF][VEC];
            int32_t eid[U];
            int64_t row[U];
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const int e = t + u * EPW + sub;
                // both cross-lane reads run on every lane (a read from a lane
                // that is switched off returns garbage); the select comes after
                row[u] = bcast<EPW>(li, e);
                const int32_t ev = bcast<EPW>(le, e);
                eid[u] = e < nb ? ev : -2;
#pragma unroll
                for (int k = 0; k < NF; ++k) {
#pragma unroll
                    for (int v = 0; v < VEC; ++v) w[u][k][v] = -1;
                    if (e < nb && fv[k]) ld_i32<VEC>(a.arg + row[u] * F + (k * LPE + pos) * VEC, w[u][k]);
                }
            }
#pragma unroll
            for (int u = 0; u < U; ++u)
#pragma unroll
                for (int k = 0; k < NF; ++k) {
                    bool any = false;
#pragma unroll
                    for (int v = 0; v < VEC; ++v) any |= w[u][k][v] == eid[u];
                    if (any) {
                        float d[VEC];
                        to_f32<DT>(ldg<DT>(a.dO, row[u] * F + (k * LPE + pos) * VEC), d);
#pragma unroll
                        for (int v = 0; v < VEC; ++v)
                            if (w[u][k][v] == eid[u]) acc[k][v] += d[v];
                    }
                }
        }
    }
    if constexpr (EPW > 1) {
#pragma unroll
        for (int off = LPE; off < kWave; off <<= 1)
#pragma unroll
            for (int k = 0; k < NF; ++k)
#pragma unroll
                for (int v = 0; v < VEC; ++v) acc[k][v] += __shfl_xor(acc[k][v], off);
    }
    if (sub != 0) return;
#pragma unroll
    for (int k = 0; k < NF; ++k) {
        if (!fv[k]) continue;
        const int64_t col = (k * LPE + pos) * VEC;
        if (it.slot < 0) stg<DT>(a.dX, static_cast<int64_t>(it.row) * F + col, acc[k]);
        else st_f32<VEC>(a.part + static_cast<int64_t>(it.slot) * F + col, acc[k]);
    }
}

}  // namespace sgat
