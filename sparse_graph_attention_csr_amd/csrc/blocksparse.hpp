// Block-sparse Graph Transformer kernels: 16x16 adjacency tiles on bf16 MFMA.
//
// A block-sparse representation of the graph lets dense matrix units do the
// score and aggregation products where the graph is locally dense (Yandex
// Research blog "On efficient scaling of GNNs via IO-aware layer
// implementations", paragraph on attention-based architectures; IO-Aware
// Layers paper, Abstract: block-sparse variants on locally dense graphs).
//
// One workgroup owns a tile row (16 destination rows); each wave owns one head
// at a time. Per tile (16 source columns) and head:
//   S^T = K_t Q_t^T   v_mfma_f32_16x16x32_bf16, K over D in steps of 32
//   masked online softmax over the row's tiles, in registers
//   O^T += V_t^T P^T  v_mfma_f32_16x16x16_bf16 per 16-channel block
// Computing S^T rather than S leaves every lane with four scores of one row
// (row l%16, columns 4(l/16)..+3), which is exactly the B operand layout of the
// second product, so P never moves between lanes; only V is transposed,
// through a per-wave LDS tile. Edges outside dense tiles (the residual CSR)
// are packed 16 at a time into gathered "pseudo-tiles" whose column c is one
// residual edge, so they go through the same softmax.
#pragma once

#include "gather.hpp"

namespace sgat {

constexpr int kTileDim = 16;

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef short s16x4_t __attribute__((ext_vector_type(4)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

__device__ __forceinline__ bf16x8_t ld_bf16x8(const void* base, int64_t elem)
{
    return __builtin_bit_cast(bf16x8_t, *reinterpret_cast<const uint4*>(
                                            static_cast<const uint16_t*>(base) + elem));
}

__device__ __forceinline__ short bf16_bits(float x)
{
    return __builtin_bit_cast(short, static_cast<__bf16>(x));
}

struct BsFwdArgs {
    int64_t n, n_tile_rows;
    int H;
    const int64_t* tile_rowptr;
    const int32_t* tile_col;
    const uint16_t* tile_mask;
    const int64_t* res_rowptr;
    const int32_t* res_colidx;
    const void *Q, *K, *V;
    void* out;
    float* lse;
    float scale2;   // log2(e) / sqrt(D)
};

template <int D>
struct TileFwd {
    static constexpr int KS = D / 32;     // k-steps of the score product
    static constexpr int NB = D / 16;     // 16-channel output blocks
    static constexpr int SPL = D / 32;    // 16-byte V segments per lane
    static constexpr int LDW = D + 16;    // LDS row stride (elements): 4 rows hit distinct banks

    // One tile of 16 columns for one head. `base` is the element offset of the
    // (node, head) row of column l%16; `valid` holds the edge bits of this
    // lane's entries (row l%16, columns 4g..4g+3).
    static __device__ __forceinline__ void step(int64_t base, uint32_t valid,
                                                const bf16x8_t (&qf)[KS], float& m, float& lsum,
                                                f32x4_t (&acc)[NB], const void* K, const void* V,
                                                uint16_t* vs, float scale2, int i, int g)
    {
        Frag kf[KS];
        uint4 vr[SPL];
#pragma unroll
        for (int s = 0; s < KS; ++s) kf[s] = ldg<SGAT_BF16>(K, base + 32 * s + 8 * g);
#pragma unroll
        for (int q = 0; q < SPL; ++q)
            vr[q] = *reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(V) + base +
                                                    8 * (g + 4 * q));
        f32x4_t st = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int s = 0; s < KS; ++s)
            st = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, kf[s]),
                                                         qf[s], st, 0, 0, 0);
#pragma unroll
        for (int q = 0; q < SPL; ++q)
            *reinterpret_cast<uint4*>(vs + i * LDW + 8 * (g + 4 * q)) = vr[q];

        float sv[4];
        float rmax = kNegInf;
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            sv[k] = ((valid >> k) & 1u) ? st[k] * scale2 : kNegInf;
            rmax = fmaxf(rmax, sv[k]);
        }
        rmax = fmaxf(rmax, __shfl_xor(rmax, 16));
        rmax = fmaxf(rmax, __shfl_xor(rmax, 32));
        const float mn = fmaxf(m, rmax);
        const float corr = mn == kNegInf ? 1.f : fast_exp2(m - mn);
        float p[4], ps = 0.f;
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            p[k] = ((valid >> k) & 1u) ? fast_exp2(sv[k] - mn) : 0.f;
            ps += p[k];
        }
        ps += __shfl_xor(ps, 16);
        ps += __shfl_xor(ps, 32);
        lsum = lsum * corr + ps;
        m = mn;
        const s16x4_t pb = {bf16_bits(p[0]), bf16_bits(p[1]), bf16_bits(p[2]), bf16_bits(p[3])};
        __builtin_amdgcn_wave_barrier();
#pragma unroll
        for (int s = 0; s < NB; ++s) {
            s16x4_t va;
#pragma unroll
            for (int kk = 0; kk < 4; ++kk)
                va[kk] = static_cast<short>(vs[(4 * g + kk) * LDW + 16 * s + i]);
            acc[s] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(va, pb, acc[s] * corr, 0, 0, 0);
        }
        __builtin_amdgcn_wave_barrier();
    }
};

template <int D>
__global__ __launch_bounds__(kBlock) void gt_bs_fwd(BsFwdArgs a)
{
    using T = TileFwd<D>;
    __shared__ __attribute__((aligned(16))) uint16_t vs_all[kWavesPerBlock][16 * T::LDW];
    const int64_t br = logical_block();
    if (br >= a.n_tile_rows) return;          // the whole workgroup leaves; no barrier follows
    const int w = wave_id();
    const int l = threadIdx.x & 63, i = l & 15, g = l >> 4;
    const int64_t HD = static_cast<int64_t>(a.H) * D;
    const int64_t r_lo = br * kTileDim;
    const int64_t r_hi = r_lo + kTileDim < a.n ? r_lo + kTileDim : a.n;
    const int64_t row = r_lo + i;
    const bool row_ok = row < a.n;
    const int64_t tb = a.tile_rowptr[br], te = a.tile_rowptr[br + 1];
    const int64_t rb = a.res_rowptr[r_lo], re = a.res_rowptr[r_hi];
    uint16_t* vs = vs_all[w];

    for (int h = w; h < a.H; h += kWavesPerBlock) {
        const int64_t hoff = static_cast<int64_t>(h) * D;
        bf16x8_t qf[T::KS];
#pragma unroll
        for (int s = 0; s < T::KS; ++s) {
            qf[s] = bf16x8_t{};
            if (row_ok) qf[s] = ld_bf16x8(a.Q, row * HD + hoff + 32 * s + 8 * g);
        }
        float m = kNegInf, lsum = 0.f;
        f32x4_t acc[T::NB];
#pragma unroll
        for (int s = 0; s < T::NB; ++s) acc[s] = f32x4_t{0.f, 0.f, 0.f, 0.f};

        for (int64_t t = tb; t < te; ++t) {
            const int64_t src = min(static_cast<int64_t>(a.tile_col[t]) * kTileDim + i, a.n - 1);
            const uint32_t valid = (static_cast<uint32_t>(a.tile_mask[t * kTileDim + i]) >> (4 * g)) & 0xFu;
            T::step(src * HD + hoff, valid, qf, m, lsum, acc, a.K, a.V, vs, a.scale2, i, g);
        }
        for (int64_t e0 = rb; e0 < re; e0 += 16) {
            const int64_t e = e0 + i;       // column i of this pseudo-tile is residual edge e
            int rr = -1;
            int64_t src = 0;
            if (e < re) {
                src = a.res_colidx[e];
                rr = 0;
                for (int r = 1; r < kTileDim; ++r) {
                    const int64_t q = r_lo + r < r_hi ? r_lo + r : r_hi;
                    rr += a.res_rowptr[q] <= e ? 1 : 0;
                }
            }
            uint32_t valid = 0;
#pragma unroll
            for (int k = 0; k < 4; ++k)
                valid |= (__shfl(rr, 4 * g + k) == i ? 1u : 0u) << k;
            T::step(src * HD + hoff, valid, qf, m, lsum, acc, a.K, a.V, vs, a.scale2, i, g);
        }

        if (row_ok) {
            const float inv = lsum > 0.f ? 1.f / lsum : 0.f;
#pragma unroll
            for (int s = 0; s < T::NB; ++s) {
                uint2 v;
                v.x = pack_bf16x2(acc[s][0] * inv, acc[s][1] * inv);
                v.y = pack_bf16x2(acc[s][2] * inv, acc[s][3] * inv);
                *reinterpret_cast<uint2*>(static_cast<uint16_t*>(a.out) + row * HD + hoff + 16 * s +
                                          4 * g) = v;
            }
            if (g == 0)
                a.lse[row * a.H + h] = lsum > 0.f ? (m + __log2f(lsum)) * kLn2 : kNegInf;
        }
    }
}

// ---------------------------------------------------------------------------
// backward: recompute S and dP per tile from the forward's lse, no stored
// edge values; dQ per tile row, dK and dV per tile column, no atomics
// ---------------------------------------------------------------------------

struct BsBwdArgs {
    int64_t n, n_blocks;   // 16-node blocks (tile rows or tile columns)
    int H;
    const int64_t* tile_rowptr;
    const int32_t* tile_col;
    const uint16_t* tile_mask;
    const int32_t* tile_row;
    const int64_t* tile_colptr;
    const int32_t* tile_bycol;
    const int64_t* res_rowptr;
    const int32_t* res_colidx;
    const int64_t* res_colptr;
    const int32_t* res_rowidx;
    const void *Q, *K, *V, *O, *dO;
    const float* lse;
    RowStat* stats;
    void *dQ, *dK, *dV;
    float scale2, oscale;
};

template <int D>
struct TileBwd {
    static constexpr int KS = D / 32;
    static constexpr int NB = D / 16;
    static constexpr int LDW = D + 16;

    // Tile-row step: rows i = l%16 of the block, columns c = 4g..4g+3 in this
    // lane. `base` = element offset of (source of column l%16, head).
    static __device__ __forceinline__ void row_step(int64_t base, uint32_t valid,
                                                    const bf16x8_t (&qf)[KS],
                                                    const bf16x8_t (&df)[KS], float lse2,
                                                    float delta, f32x4_t (&acc)[NB],
                                                    const void* K, const void* V, uint16_t* ks,
                                                    float scale2, int i, int g)
    {
        Frag kf[KS], vf[KS];
#pragma unroll
        for (int s = 0; s < KS; ++s) {
            kf[s] = ldg<SGAT_BF16>(K, base + 32 * s + 8 * g);
            vf[s] = ldg<SGAT_BF16>(V, base + 32 * s + 8 * g);
        }
        f32x4_t st = {0.f, 0.f, 0.f, 0.f}, dp = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int s = 0; s < KS; ++s) {
            st = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, kf[s]), qf[s],
                                                         st, 0, 0, 0);
            dp = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, vf[s]), df[s],
                                                         dp, 0, 0, 0);
        }
#pragma unroll
        for (int s = 0; s < KS; ++s)
            *reinterpret_cast<Frag*>(ks + i * LDW + 32 * s + 8 * g) = kf[s];
        short dsb[4];
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            const float p = ((valid >> k) & 1u) ? fast_exp2(st[k] * scale2 - lse2) : 0.f;
            dsb[k] = bf16_bits(p * (dp[k] - delta));
        }
        const s16x4_t b = {dsb[0], dsb[1], dsb[2], dsb[3]};
        __builtin_amdgcn_wave_barrier();
#pragma unroll
        for (int s = 0; s < NB; ++s) {
            s16x4_t ka;
#pragma unroll
            for (int kk = 0; kk < 4; ++kk)
                ka[kk] = static_cast<short>(ks[(4 * g + kk) * LDW + 16 * s + i]);
            acc[s] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(ka, b, acc[s], 0, 0, 0);
        }
        __builtin_amdgcn_wave_barrier();
    }

    // Tile-column step: columns c = l%16 (sources of the block), rows
    // 4g..4g+3 of the tile in this lane. `qbase` = element offset of (the
    // destination of tile row l%16, head); st[k] = statistics of row 4g+k.
    static __device__ __forceinline__ void col_step(int64_t qbase, const RowStat (&st)[4],
                                                    uint32_t valid, const bf16x8_t (&kf)[KS],
                                                    const bf16x8_t (&vf)[KS], f32x4_t (&dk)[NB],
                                                    f32x4_t (&dv)[NB], const void* Q,
                                                    const void* dO, uint16_t* qs, uint16_t* os,
                                                    float scale2, int c, int g)
    {
        Frag qa[KS], oa[KS];
#pragma unroll
        for (int s = 0; s < KS; ++s) {
            qa[s] = ldg<SGAT_BF16>(Q, qbase + 32 * s + 8 * g);
            oa[s] = ldg<SGAT_BF16>(dO, qbase + 32 * s + 8 * g);
        }
        f32x4_t sc = {0.f, 0.f, 0.f, 0.f}, dp = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int s = 0; s < KS; ++s) {
            sc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, qa[s]), kf[s],
                                                         sc, 0, 0, 0);
            dp = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, oa[s]), vf[s],
                                                         dp, 0, 0, 0);
        }
#pragma unroll
        for (int s = 0; s < KS; ++s) {
            *reinterpret_cast<Frag*>(qs + c * LDW + 32 * s + 8 * g) = qa[s];
            *reinterpret_cast<Frag*>(os + c * LDW + 32 * s + 8 * g) = oa[s];
        }
        short pb[4], db[4];
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            const float p = ((valid >> k) & 1u) ? fast_exp2(sc[k] * scale2 - st[k].lse2) : 0.f;
            pb[k] = bf16_bits(p);
            db[k] = bf16_bits(p * (dp[k] - st[k].delta));
        }
        const s16x4_t P = {pb[0], pb[1], pb[2], pb[3]};
        const s16x4_t S = {db[0], db[1], db[2], db[3]};
        __builtin_amdgcn_wave_barrier();
#pragma unroll
        for (int s = 0; s < NB; ++s) {
            s16x4_t qt, ot;
#pragma unroll
            for (int kk = 0; kk < 4; ++kk) {
                qt[kk] = static_cast<short>(qs[(4 * g + kk) * LDW + 16 * s + c]);
                ot[kk] = static_cast<short>(os[(4 * g + kk) * LDW + 16 * s + c]);
            }
            dk[s] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(qt, S, dk[s], 0, 0, 0);
            dv[s] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(ot, P, dv[s], 0, 0, 0);
        }
        __builtin_amdgcn_wave_barrier();
    }
};

__device__ __forceinline__ void store_tile_rows(void* dst, int64_t off, const f32x4_t& v, float sc)
{
    uint2 w;
    w.x = pack_bf16x2(v[0] * sc, v[1] * sc);
    w.y = pack_bf16x2(v[2] * sc, v[3] * sc);
    *reinterpret_cast<uint2*>(static_cast<uint16_t*>(dst) + off) = w;
}

// Position of edge e among the 16 rows of a block, from the block's pointers.
__device__ __forceinline__ int row_in_block(const int64_t* ptr, int64_t lo, int64_t hi, int64_t e)
{
    int r = 0;
    for (int q = 1; q < kTileDim; ++q) {
        const int64_t x = lo + q < hi ? lo + q : hi;
        r += ptr[x] <= e ? 1 : 0;
    }
    return r;
}

template <int D>
__global__ __launch_bounds__(kBlock) void gt_bs_bwd_rows(BsBwdArgs a)
{
    using T = TileBwd<D>;
    __shared__ __attribute__((aligned(16))) uint16_t ks_all[kWavesPerBlock][16 * T::LDW];
    const int64_t br = logical_block();
    if (br >= a.n_blocks) return;
    const int w = wave_id();
    const int l = threadIdx.x & 63, i = l & 15, g = l >> 4;
    const int64_t HD = static_cast<int64_t>(a.H) * D;
    const int64_t r_lo = br * kTileDim;
    const int64_t r_hi = r_lo + kTileDim < a.n ? r_lo + kTileDim : a.n;
    const int64_t row = r_lo + i;
    const bool row_ok = row < a.n;
    const int64_t tb = a.tile_rowptr[br], te = a.tile_rowptr[br + 1];
    const int64_t rb = a.res_rowptr[r_lo], re = a.res_rowptr[r_hi];
    uint16_t* ks = ks_all[w];

    for (int h = w; h < a.H; h += kWavesPerBlock) {
        const int64_t hoff = static_cast<int64_t>(h) * D;
        bf16x8_t qf[T::KS], df[T::KS];
        float dsum = 0.f, lse2 = 0.f;
#pragma unroll
        for (int s = 0; s < T::KS; ++s) {
            qf[s] = bf16x8_t{};
            df[s] = bf16x8_t{};
            if (row_ok) {
                const int64_t o = row * HD + hoff + 32 * s + 8 * g;
                qf[s] = ld_bf16x8(a.Q, o);
                const Frag d = ldg<SGAT_BF16>(a.dO, o);
                df[s] = __builtin_bit_cast(bf16x8_t, d);
                dsum += dot<SGAT_BF16>(d, ldg<SGAT_BF16>(a.O, o));
            }
        }
        dsum += __shfl_xor(dsum, 16);
        dsum += __shfl_xor(dsum, 32);
        if (row_ok) lse2 = a.lse[row * a.H + h] * kLog2e;
        if (row_ok && g == 0) a.stats[row * a.H + h] = RowStat{lse2, dsum};
        f32x4_t acc[T::NB];
#pragma unroll
        for (int s = 0; s < T::NB; ++s) acc[s] = f32x4_t{0.f, 0.f, 0.f, 0.f};

        for (int64_t t = tb; t < te; ++t) {
            const int64_t src = min(static_cast<int64_t>(a.tile_col[t]) * kTileDim + i, a.n - 1);
            const uint32_t valid = (static_cast<uint32_t>(a.tile_mask[t * kTileDim + i]) >> (4 * g)) & 0xFu;
            T::row_step(src * HD + hoff, valid, qf, df, lse2, dsum, acc, a.K, a.V, ks, a.scale2, i, g);
        }
        for (int64_t e0 = rb; e0 < re; e0 += 16) {
            const int64_t e = e0 + i;
            int rr = -1;
            int64_t src = 0;
            if (e < re) {
                src = a.res_colidx[e];
                rr = row_in_block(a.res_rowptr, r_lo, r_hi, e);
            }
            uint32_t valid = 0;
#pragma unroll
            for (int k = 0; k < 4; ++k) valid |= (__shfl(rr, 4 * g + k) == i ? 1u : 0u) << k;
            T::row_step(src * HD + hoff, valid, qf, df, lse2, dsum, acc, a.K, a.V, ks, a.scale2, i, g);
        }
        if (row_ok) {
#pragma unroll
            for (int s = 0; s < T::NB; ++s)
                store_tile_rows(a.dQ, row * HD + hoff + 16 * s + 4 * g, acc[s], a.oscale);
        }
    }
}

template <int D>
__global__ __launch_bounds__(kBlock) void gt_bs_bwd_cols(BsBwdArgs a)
{
    using T = TileBwd<D>;
    __shared__ __attribute__((aligned(16))) uint16_t qs_all[kWavesPerBlock][16 * T::LDW];
    __shared__ __attribute__((aligned(16))) uint16_t os_all[kWavesPerBlock][16 * T::LDW];
    const int64_t bc = logical_block();
    if (bc >= a.n_blocks) return;
    const int w = wave_id();
    const int l = threadIdx.x & 63, c = l & 15, g = l >> 4;
    const int64_t HD = static_cast<int64_t>(a.H) * D;
    const int64_t c_lo = bc * kTileDim;
    const int64_t c_hi = c_lo + kTileDim < a.n ? c_lo + kTileDim : a.n;
    const int64_t j = c_lo + c;
    const bool j_ok = j < a.n;
    const int64_t tcb = a.tile_colptr[bc], tce = a.tile_colptr[bc + 1];
    const int64_t rcb = a.res_colptr[c_lo], rce = a.res_colptr[c_hi];
    uint16_t* qs = qs_all[w];
    uint16_t* os = os_all[w];

    for (int h = w; h < a.H; h += kWavesPerBlock) {
        const int64_t hoff = static_cast<int64_t>(h) * D;
        bf16x8_t kf[T::KS], vf[T::KS];
#pragma unroll
        for (int s = 0; s < T::KS; ++s) {
            kf[s] = bf16x8_t{};
            vf[s] = bf16x8_t{};
            if (j_ok) {
                kf[s] = ld_bf16x8(a.K, j * HD + hoff + 32 * s + 8 * g);
                vf[s] = ld_bf16x8(a.V, j * HD + hoff + 32 * s + 8 * g);
            }
        }
        f32x4_t dk[T::NB], dv[T::NB];
#pragma unroll
        for (int s = 0; s < T::NB; ++s) {
            dk[s] = f32x4_t{0.f, 0.f, 0.f, 0.f};
            dv[s] = f32x4_t{0.f, 0.f, 0.f, 0.f};
        }
        for (int64_t q = tcb; q < tce; ++q) {
            const int64_t t = a.tile_bycol[q];
            const int64_t r0 = static_cast<int64_t>(a.tile_row[t]) * kTileDim;
            const int64_t arow = min(r0 + c, a.n - 1);    // tile row l%16, as the A operand row
            RowStat st[4];
            uint32_t valid = 0;
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                const int64_t rk = r0 + 4 * g + k;
                const uint32_t bit = (static_cast<uint32_t>(a.tile_mask[t * kTileDim + 4 * g + k]) >> c) & 1u;
                valid |= bit << k;
                st[k] = RowStat{0.f, 0.f};
                if (bit) st[k] = a.stats[rk * a.H + h];
            }
            T::col_step(arow * HD + hoff, st, valid, kf, vf, dk, dv, a.Q, a.dO, qs, os, a.scale2, c, g);
        }
        for (int64_t e0 = rcb; e0 < rce; e0 += 16) {
            const int64_t e = e0 + c;          // row l%16 of this pseudo-tile is residual edge e
            int cc = -1;
            int64_t dst = 0;
            if (e < rce) {
                dst = a.res_rowidx[e];
                cc = row_in_block(a.res_colptr, c_lo, c_hi, e);
            }
            RowStat st[4];
            uint32_t valid = 0;
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                const int lk = 4 * g + k;
                const bool bit = __shfl(cc, lk) == c;
                const int64_t dk_row = __shfl(static_cast<int>(dst), lk);
                valid |= (bit ? 1u : 0u) << k;
                st[k] = RowStat{0.f, 0.f};
                if (bit) st[k] = a.stats[dk_row * a.H + h];
            }
            T::col_step(dst * HD + hoff, st, valid, kf, vf, dk, dv, a.Q, a.dO, qs, os, a.scale2, c, g);
        }
        if (j_ok) {
#pragma unroll
            for (int s = 0; s < T::NB; ++s) {
                store_tile_rows(a.dK, j * HD + hoff + 16 * s + 4 * g, dk[s], a.oscale);
                store_tile_rows(a.dV, j * HD + hoff + 16 * s + 4 * g, dv[s], 1.f);
            }
        }
    }
}

}  // namespace sgat
