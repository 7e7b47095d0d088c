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
    const u32x4_t nv = {v.x, v.y, v.z, v.w};   // written once: non-temporal
    __builtin_nontemporal_store(nv, reinterpret_cast<u32x4_t*>(static_cast<char*>(base) +
                                                               elem * Elem<DT>::BYTES));
}

template <int N>
__device__ __forceinline__ void st_i32(int32_t* p, const int32_t (&x)[N])
{
    static_assert(N % 4 == 0, "");
#pragma unroll
    for (int k = 0; k < N; k += 4) {   // written once: non-temporal
        const u32x4_t v = {static_cast<uint32_t>(x[k]), static_cast<uint32_t>(x[k + 1]),
                           static_cast<uint32_t>(x[k + 2]), static_cast<uint32_t>(x[k + 3])};
        __builtin_nontemporal_store(v, reinterpret_cast<u32x4_t*>(p + k));
    }
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

// Backward, in two passes. dX[j,f] is the sum of dout[i,f] over the (i, f)
// whose winner is an edge j -> i. Reading each edge's winners from the
// transposed side would fetch a whole row of arg per edge and scatter
// 16-byte reads of dout; instead the contributions are first regrouped by
// edge on the destination side, where arg_i and dout_i are read once each.
//
// Route (one wave per destination row): count the row's F winners per edge
// in an LDS histogram (over windows of the row's edges, so any degree fits),
// turn the counts into starts by a wave scan, write every edge's
// (start, count) inside the row's block of F entries, and place each feature
// f at its edge's next free slot as the pair (f, dout[i,f]). The order of the
// pairs inside one edge's range does not matter: they name distinct features.
//
// Gather (one wave per transposed-CSR work item): for each out-edge of the
// source, in transposed-CSR order, add its pairs into an LDS accumulator of F
// values; one edge's pairs name distinct features, so lanes never collide,
// and a feature receives the edges' contributions in a fixed order.
constexpr int kRouteWindow = 512;         // histogram bins per wave

template <int DT> struct RouteEntry;      // (feature, dout) pair of one winner
template <> struct RouteEntry<SGAT_BF16> { using T = uint32_t; };   // f | bf16 bits << 16
template <> struct RouteEntry<SGAT_F32> { using T = uint2; };       // (f, fp32 bits)

struct ReduceRouteArgs {
    const sgat_work_item* items;   // the CSR work list (a split row's first chunk stands for it)
    int64_t n_items;
    int F;
    const int64_t* rowptr;
    const int32_t* arg;
    const void* dO;
    uint32_t* sc;                  // [nnz] start | count << 16
    void* entries;                 // [n][F] RouteEntry, grouped by winning edge per row
};

__device__ __forceinline__ int wave_inclusive_scan(int x)
{
    const int lane = threadIdx.x & 63;
#pragma unroll
    for (int o = 1; o < kWave; o <<= 1) {
        const int t = __shfl_up(x, o);
        if (lane >= o) x += t;
    }
    return x;
}

template <int DT, int NR>
__global__ __launch_bounds__(kBlock) void reduce_bwd_route(ReduceRouteArgs a)
{
    constexpr int VEC = Elem<DT>::VEC;
    // the window's counters, then one spare counter per lane that entries
    // outside the window update (so the atomics need no lane-dependent branch)
    __shared__ int32_t hist_all[kWavesPerBlock][kRouteWindow + kWave];
    // Where a row's pairs fit 4 KB, they are placed at their slots in LDS and
    // written out with contiguous stores once per window, instead of one
    // scattered 4- or 8-byte store per feature.
    using E = typename RouteEntry<DT>::T;
    constexpr int kRowPairs = NR * kWave * VEC;
    constexpr bool kStage = kRowPairs * sizeof(E) <= 4096;
    __shared__ E stage_all[kWavesPerBlock][kStage ? kRowPairs : 1];
    const int64_t unit = logical_block() * kWavesPerBlock + wave_id();
    if (unit >= a.n_items) return;
    const sgat_work_item it = a.items[unit];
    if (it.slot >= 0 && !(it.flags & 1)) return;
    const int64_t r0 = a.rowptr[it.row];
    const int64_t d = a.rowptr[it.row + 1] - r0;
    if (d == 0) return;
    const int lane = threadIdx.x & 63;
    int32_t* hist = hist_all[wave_id()];
    const int64_t F = a.F;
    const int64_t rowF = static_cast<int64_t>(it.row) * F;

    bool fv[NR];
    int32_t q[NR][VEC];            // winner as an edge index inside the row (nnz < 2^31)
    float dv[NR][VEC];
#pragma unroll
    for (int k = 0; k < NR; ++k) {
        const int64_t c = (k * kWave + lane) * VEC;
        fv[k] = c < F;
        int32_t w[VEC];
#pragma unroll
        for (int v = 0; v < VEC; ++v) { w[v] = -1; dv[k][v] = 0.f; }
        if (fv[k]) {
            ld_i32<VEC>(a.arg + rowF + c, w);
            to_f32<DT>(ldg<DT>(a.dO, rowF + c), dv[k]);
        }
#pragma unroll
        for (int v = 0; v < VEC; ++v) q[k][v] = w[v] - static_cast<int32_t>(r0);
    }

    E* ent = static_cast<E*>(a.entries) + rowF;
    E* stage = stage_all[wave_id()];
    int total = 0;
    for (int32_t w0 = 0; w0 < d; w0 += kRouteWindow) {
        const int nb = static_cast<int>(d - w0 < kRouteWindow ? d - w0 : kRouteWindow);
        for (int b = lane; b < nb; b += kWave) hist[b] = 0;
        wave_lds_fence();
        const int spare = kRouteWindow + lane;
#pragma unroll
        for (int k = 0; k < NR; ++k)
#pragma unroll
            for (int v = 0; v < VEC; ++v) {
                const int32_t b = q[k][v] - w0;
                atomicAdd(&hist[fv[k] && b >= 0 && b < nb ? b : spare], 1);
            }
        wave_lds_fence();
        const int win_lo = total;   // this window's pairs take slots [win_lo, total)
        for (int b0 = 0; b0 < nb; b0 += kWave) {
            const int b = b0 + lane;
            const int c = b < nb ? hist[b] : 0;
            const int incl = wave_inclusive_scan(c);
            const int st = total + incl - c;
            if (b < nb) {
                hist[b] = st;
                a.sc[r0 + w0 + b] = static_cast<uint32_t>(st) | (static_cast<uint32_t>(c) << 16);
            }
            total += __builtin_amdgcn_readlane(incl, 63);
        }
        wave_lds_fence();
        // all slots first (the atomics issue back to back), then the stores
        int slot[NR][VEC];
#pragma unroll
        for (int k = 0; k < NR; ++k)
#pragma unroll
            for (int v = 0; v < VEC; ++v) {
                const int32_t b = q[k][v] - w0;
                slot[k][v] = atomicAdd(&hist[fv[k] && b >= 0 && b < nb ? b : spare], 1);
            }
#pragma unroll
        for (int k = 0; k < NR; ++k)
#pragma unroll
            for (int v = 0; v < VEC; ++v) {
                const int32_t b = q[k][v] - w0;
                if (fv[k] && b >= 0 && b < nb) {
                    const uint32_t f = static_cast<uint32_t>((k * kWave + lane) * VEC + v);
                    E x;
                    if constexpr (DT == SGAT_BF16)
                        x = f | (__float_as_uint(dv[k][v]) & 0xffff0000u);
                    else
                        x = make_uint2(f, __float_as_uint(dv[k][v]));
                    if constexpr (kStage)
                        stage[slot[k][v]] = x;   // slots are below F <= kRowPairs
                    else
                        ent[slot[k][v]] = x;
                }
            }
        wave_lds_fence();
        if constexpr (kStage) {
            for (int sl = win_lo + lane; sl < total; sl += kWave) ent[sl] = stage[sl];
            wave_lds_fence();
        }
    }
}

template <int DT>
__device__ __forceinline__ int route_feature(typename RouteEntry<DT>::T x)
{
    if constexpr (DT == SGAT_BF16) return static_cast<int>(x & 0xffffu);
    else return static_cast<int>(x.x);
}

template <int DT>
__device__ __forceinline__ float route_value(typename RouteEntry<DT>::T x)
{
    if constexpr (DT == SGAT_BF16) return __uint_as_float(x & 0xffff0000u);
    else return __uint_as_float(x.y);
}

struct ReduceGatherArgs {
    const sgat_work_item* items;   // the transposed-CSR work list
    int64_t n_items;
    int F;
    const int32_t* rowidx;
    const int32_t* col_edge;
    const uint32_t* sc;
    const void* entries;
    void* dX;
    float* part;                   // [col_slots][F]
};

template <int DT, int NR, int U>
__global__ __launch_bounds__(kBlock) void reduce_bwd_gather(ReduceGatherArgs a)
{
    constexpr int VEC = Elem<DT>::VEC;
    constexpr int ACC = NR * kWave * VEC;
    // F accumulators, then one spare slot per lane that idle lanes update
    __shared__ float acc_all[kWavesPerBlock][ACC + kWave];
    const int64_t unit = logical_block() * kWavesPerBlock + wave_id();
    if (unit >= a.n_items) return;
    const sgat_work_item it = a.items[unit];
    const int lane = threadIdx.x & 63;
    float* acc = acc_all[wave_id()];
    const int64_t F = a.F;
    for (int b = lane; b < ACC + kWave; b += kWave) acc[b] = 0.f;
    const int spare = ACC + lane;
    wave_lds_fence();

    using E = typename RouteEntry<DT>::T;
    const E* ent = static_cast<const E*>(a.entries);
    const int32_t* ri = a.rowidx + it.begin;
    const int32_t* ce = a.col_edge + it.begin;
    // Every load below is unconditional; only the LDS update is masked. (A
    // load under a lane-dependent branch is waited for inside that branch,
    // which would serialise the edges.) Lanes past an edge's count load the
    // edge's last pair again (index clamped to the slice, and to the row's F
    // pairs), so they fetch no memory beyond the slice.
    for (int base = 0; base < it.len; base += kWave) {
        const int nb = min(kWave, it.len - base);
        const int lc = min(lane, nb - 1);
        const int li = ri[base + lc];
        const uint32_t ls = a.sc[ce[base + lc]];
        for (int t = 0; t < nb; t += U) {
            E x[U];
            uint32_t cnt[U], st[U];
            int64_t row[U];
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const int e = t + u < nb ? t + u : nb - 1;
                const uint32_t sv = __builtin_amdgcn_readlane(ls, e);
                row[u] = __builtin_amdgcn_readlane(li, e);
                cnt[u] = t + u < nb ? sv >> 16 : 0u;
                st[u] = sv & 0xffffu;
                const uint32_t last = cnt[u] > 0 ? cnt[u] - 1 : 0u;
                const int64_t k = min(static_cast<int64_t>(st[u] + min(static_cast<uint32_t>(lane), last)), F - 1);
                x[u] = ent[row[u] * F + k];
            }
            // pairs inside [start, start + count) were written by this call's
            // route pass, with features below F. Lanes past the count update
            // their spare slot with value * 0: the product needs the loaded
            // value on every lane, so the compiler cannot move a load under a
            // lane-dependent branch (a select of 0 would let it).
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const bool live = static_cast<uint32_t>(lane) < cnt[u];
                acc[live ? route_feature<DT>(x[u]) : spare] += route_value<DT>(x[u]) * (live ? 1.f : 0.f);
            }
            // edges that won more than 64 features of their row
#pragma unroll
            for (int u = 0; u < U; ++u)
                for (uint32_t c0 = kWave; c0 < cnt[u]; c0 += kWave) {
                    const uint32_t o = min(c0 + static_cast<uint32_t>(lane), cnt[u] - 1);
                    const int64_t k = min(static_cast<int64_t>(st[u] + o), F - 1);
                    const E y = ent[row[u] * F + k];
                    const bool live = c0 + lane < cnt[u];
                    acc[live ? route_feature<DT>(y) : spare] += route_value<DT>(y) * (live ? 1.f : 0.f);
                }
        }
    }
    wave_lds_fence();
#pragma unroll
    for (int k = 0; k < NR; ++k) {
        const int64_t c = (k * kWave + lane) * VEC;
        if (c >= F) continue;
        float x[VEC];
#pragma unroll
        for (int q = 0; q < VEC; ++q) x[q] = acc[c + q];
        if (it.slot < 0) stg<DT>(a.dX, static_cast<int64_t>(it.row) * F + c, x);
        else st_f32<VEC>(a.part + static_cast<int64_t>(it.slot) * F + c, x);
    }
}

}  // namespace sgat
