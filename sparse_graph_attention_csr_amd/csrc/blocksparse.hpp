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
//
// Every kernel walks its tiles software-pipelined with one set of tile
// registers: a tile's first phase consumes them (the score products, and the
// operand that is transposed goes to LDS), the loads of the next tile refill
// them at once, and they arrive while the second phase (softmax, the
// LDS-fed products) runs. Tile descriptions are fetched two tiles ahead.
#pragma once

#include "gather.hpp"

namespace sgat {

constexpr int kTileDim = 16;
constexpr float kRescaleLog2 = 8.f;   // tile forward: weights stay below 2^8 (see fwd_phase_b)

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
struct Shape {
    static constexpr int KS = D / 32;     // k-steps of a 16x16xD score product
    static constexpr int NB = D / 16;     // 16-channel output blocks
    static constexpr int SPL = D / 32;    // 16-byte segments of a 16-row tile per lane
    // LDS row stride (elements) of tiles read back with ds_read_b64_tr_b16.
    // Measured on gfx950 (SQ_LDS_BANK_CONFLICT per LDS instruction, community
    // workload): D + 8, D + 24 and D + 40 give the fewest conflicts, D + 16
    // twice as many, D + 32 seven times as many; kernel times are the same
    // within 1 % for all but D + 32, so LDS is not what bounds these kernels.
    static constexpr int LDV = D + 8;
};

// Transposed 4 x 16-bit LDS read (gfx950 ds_read_b64_tr_b16). Within each
// group of 16 lanes, lane j receives element j % 4 of the 64-bit word that
// lane 4k + j / 4 addressed, in slot k.
__device__ __forceinline__ s16x4_t lds_read_tr16(const uint16_t* p)
{
    return __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (__attribute__((address_space(3))) s16x4_t*)(p));
}

// V tile lanes: lane l loads and stores row vrow(l) = l % 8 + 8 * (l / 32),
// 16-byte chunk vchunk(l) = (l / 8) % 4 of each 32-channel slab (the V tile
// goes only through LDS, so any assignment of its chunks to lanes works; this
// one has every 16 lanes store 8 rows x 2 chunks).
__device__ __forceinline__ int vrow(int l) { return (l & 7) + 8 * (l >> 5); }
__device__ __forceinline__ int vchunk(int l) { return (l >> 3) & 3; }

// Tiles whose lanes are fixed by the MFMA operand layout (lane (i, g) holds
// row i, 16-byte chunk 4s + g of every 32-channel slab s) are stored at row
// stride LDV with the chunks of rows 8..15 swapped in pairs (chunk ^ 1), so
// that rows i and i + 8, stored by the same instruction, start on different
// banks.
template <int D>
__device__ __forceinline__ void store_operand_tile(uint16_t* t, const Frag (&f)[Shape<D>::KS],
                                                   int i, int g)
{
    uint16_t* row = t + i * Shape<D>::LDV + 8 * (g ^ ((i >> 3) & 1));
#pragma unroll
    for (int s = 0; s < Shape<D>::KS; ++s) *reinterpret_cast<Frag*>(row + 32 * s) = f[s];
}

// Base address of lane (i, g)'s transposed reads of such a tile: block s
// (channels 16s..16s+15, rows 4g..4g+3 into the MFMA A operand) is at + 16 s.
// Lane i of the group addresses row 4g + i/4, channels 16s + 4(i%4).
template <int D>
__device__ __forceinline__ const uint16_t* operand_tr_base(const uint16_t* t, int i, int g)
{
    return t + (4 * g + (i >> 2)) * Shape<D>::LDV + 8 * (((i >> 1) & 1) ^ (g >> 1)) + 4 * (i & 1);
}

// Start offsets of rows 1..15 of a 16-row (or 16-source) block in a pointer
// array, loaded once per block (rows past the end start at ptr[hi]).
struct BlockStarts {
    int64_t v[kTileDim];
    __device__ __forceinline__ void load(const int64_t* ptr, int64_t lo, int64_t hi)
    {
#pragma unroll
        for (int q = 1; q < kTileDim; ++q) v[q] = ptr[lo + q < hi ? lo + q : hi];
    }
    // position of edge e among the block's rows
    __device__ __forceinline__ int row_of(int64_t e) const
    {
        int r = 0;
#pragma unroll
        for (int q = 1; q < kTileDim; ++q) r += v[q] <= e ? 1 : 0;
        return r;
    }
};

// Tiles of one 16-row block, in order: its dense tiles, then its residual
// edges in pseudo-tiles of 16. Tile k is described by a RowRef: the node of
// column l%16 and this lane's 4 edge bits (row l%16, columns 4g..4g+3).
// fetch() issues the raw loads of a description, decode() builds it; k is
// uniform across the wave.
struct RowRef {
    int64_t src;
    uint32_t valid;
};

struct RowTiles {
    int64_t n, tb, nd, rb, re;
    const int32_t* tile_col;
    const uint16_t* tile_mask;
    const int32_t* res_colidx;
    BlockStarts starts;

    __device__ __forceinline__ int64_t count() const { return nd + (re - rb + 15) / 16; }

    __device__ __forceinline__ void fetch(int64_t k, int i, int32_t& col, uint32_t& word) const
    {
        if (k < nd) {
            const int64_t t = tb + k;
            col = tile_col[t];
            word = tile_mask[t * kTileDim + i];
        } else {
            const int64_t e = rb + (k - nd) * 16 + i;
            col = e < re ? res_colidx[e] : 0;
            word = 0;
        }
    }

    __device__ __forceinline__ RowRef decode(int64_t k, int i, int g, int32_t col, uint32_t word) const
    {
        RowRef r;
        if (k < nd) {
            r.src = min(static_cast<int64_t>(col) * kTileDim + i, n - 1);
            r.valid = (word >> (4 * g)) & 0xFu;
        } else {
            const int64_t e = rb + (k - nd) * 16 + i;   // column i is residual edge e
            const int rr = e < re ? starts.row_of(e) : -1;
            r.src = col;
            r.valid = 0;
#pragma unroll
            for (int q = 0; q < 4; ++q) r.valid |= (__shfl(rr, 4 * g + q) == i ? 1u : 0u) << q;
        }
        return r;
    }
};

template <int D>
struct FwdTile {
    Frag kf[Shape<D>::KS];
    uint4 vr[Shape<D>::SPL];
    // kbase: row l%16's node row (K, MFMA operand layout); vbase: row
    // vrow(l)'s node row (V, staged through LDS)
    __device__ __forceinline__ void load(const void* K, const void* V, int64_t kbase,
                                         int64_t vbase, int g, int l)
    {
#pragma unroll
        for (int s = 0; s < Shape<D>::KS; ++s) kf[s] = ldg<SGAT_BF16>(K, kbase + 32 * s + 8 * g);
#pragma unroll
        for (int q = 0; q < Shape<D>::SPL; ++q)
            vr[q] = *reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(V) + vbase +
                                                    32 * q + 8 * vchunk(l));
    }
};

// One forward tile for one head, in two phases. Phase A consumes the tile's
// registers (S^T = K Q^T, V into LDS), so the next tile's loads can refill
// them before phase B: the masked online-softmax update of (m, lsum) and
// O^T += V^T P^T from LDS.
template <int D>
__device__ __forceinline__ f32x4_t fwd_phase_a(const FwdTile<D>& tl,
                                               const bf16x8_t (&qf)[Shape<D>::KS], uint16_t* vs,
                                               int l)
{
    using S = Shape<D>;
    f32x4_t st = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s = 0; s < S::KS; ++s)
        st = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, tl.kf[s]), qf[s],
                                                     st, 0, 0, 0);
#pragma unroll
    for (int q = 0; q < S::SPL; ++q)
        *reinterpret_cast<uint4*>(vs + vrow(l) * S::LDV + 32 * q + 8 * vchunk(l)) = tl.vr[q];
    return st;
}

template <int D>
__device__ __forceinline__ void fwd_phase_b(const f32x4_t& st, uint32_t valid, float& m,
                                            float& lsum, f32x4_t (&acc)[Shape<D>::NB],
                                            const uint16_t* vs, float scale2, int i, int g)
{
    using S = Shape<D>;
    float sv[4];
    float rmax = kNegInf;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        sv[k] = ((valid >> k) & 1u) ? st[k] * scale2 : kNegInf;
        rmax = fmaxf(rmax, sv[k]);
    }
    rmax = fmaxf(rmax, __shfl_xor(rmax, 16));
    rmax = fmaxf(rmax, __shfl_xor(rmax, 32));
    // Lazy rescaling: m is a reference maximum, moved (and O, lsum rescaled)
    // only when a row's score passes it by more than 2^kRescaleLog2, so the
    // weights exp2(s - m) stay below 2^kRescaleLog2 and the common tile leaves
    // the accumulators untouched in the matrix registers. out = O / lsum and
    // lse = m + log2(lsum) hold for any reference m.
    const bool raise = rmax > m + kRescaleLog2;   // never for a row that has no score yet
    if (__any(raise)) {
        const float corr = raise ? fast_exp2(m - rmax) : 1.f;   // m = -inf gives 0
        if (raise) m = rmax;
        lsum *= corr;
#pragma unroll
        for (int s = 0; s < S::NB; ++s) acc[s] *= corr;
    }
    float p[4], ps = 0.f;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        p[k] = ((valid >> k) & 1u) ? fast_exp2(sv[k] - m) : 0.f;
        ps += p[k];
    }
    ps += __shfl_xor(ps, 16);
    ps += __shfl_xor(ps, 32);
    lsum += ps;
    const s16x4_t pb = {bf16_bits(p[0]), bf16_bits(p[1]), bf16_bits(p[2]), bf16_bits(p[3])};
    __builtin_amdgcn_wave_barrier();
    // A operand of block s: V[4g + kk][16s + i] for kk = 0..3, one transposed
    // read (lane 4k + j/4 of the group addresses row 4g + k, channels 16s + 4(j%4))
    const uint16_t* vt = vs + (4 * g + (i >> 2)) * S::LDV + 4 * (i & 3);
#pragma unroll
    for (int s = 0; s < S::NB; ++s) {
        const s16x4_t va = lds_read_tr16(vt + 16 * s);
        acc[s] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(va, pb, acc[s], 0, 0, 0);
    }
    __builtin_amdgcn_wave_barrier();
}

__device__ __forceinline__ void store_tile_rows(void* dst, int64_t off, const f32x4_t& v, float sc)
{
    uint2 w;
    w.x = pack_bf16x2(v[0] * sc, v[1] * sc);
    w.y = pack_bf16x2(v[2] * sc, v[3] * sc);
    *reinterpret_cast<uint2*>(static_cast<uint16_t*>(dst) + off) = w;
}

// At least 3 waves per SIMD: at D = 128 the compiler would otherwise keep
// the accumulators twice (VGPR copies of MFMA results in AGPRs) and stop at 2;
// with the target it keeps them in VGPRs only, without spilling.
template <int D>
__global__ __launch_bounds__(kBlock) __attribute__((amdgpu_waves_per_eu(3))) void gt_bs_fwd(BsFwdArgs a)
{
    using S = Shape<D>;
    __shared__ __attribute__((aligned(16))) uint16_t vs_all[kWavesPerBlock][16 * S::LDV];
    const int64_t br = logical_block();
    if (br >= a.n_tile_rows) return;          // the whole workgroup leaves; no barrier follows
    const int w = wave_id();
    const int l = threadIdx.x & 63, i = l & 15, g = l >> 4;
    const int64_t HD = static_cast<int64_t>(a.H) * D;
    RowTiles tiles;
    const int64_t r_lo = br * kTileDim;
    const int64_t r_hi = r_lo + kTileDim < a.n ? r_lo + kTileDim : a.n;
    tiles.n = a.n;
    tiles.tb = a.tile_rowptr[br];
    tiles.nd = a.tile_rowptr[br + 1] - tiles.tb;
    tiles.rb = a.res_rowptr[r_lo];
    tiles.re = a.res_rowptr[r_hi];
    tiles.tile_col = a.tile_col;
    tiles.tile_mask = a.tile_mask;
    tiles.res_colidx = a.res_colidx;
    tiles.starts.load(a.res_rowptr, r_lo, r_hi);
    const int64_t nt = tiles.count();
    const int64_t row = r_lo + i;
    const bool row_ok = row < a.n;
    uint16_t* vs = vs_all[w];

    for (int h = w; h < a.H; h += kWavesPerBlock) {
        const int64_t hoff = static_cast<int64_t>(h) * D;
        bf16x8_t qf[S::KS];
#pragma unroll
        for (int s = 0; s < S::KS; ++s) {
            qf[s] = bf16x8_t{};
            if (row_ok) qf[s] = ld_bf16x8(a.Q, row * HD + hoff + 32 * s + 8 * g);
        }
        float m = kNegInf, lsum = 0.f;
        f32x4_t acc[S::NB];
#pragma unroll
        for (int s = 0; s < S::NB; ++s) acc[s] = f32x4_t{0.f, 0.f, 0.f, 0.f};

        // pipeline: descriptions two tiles ahead; the data of tile k+1 is
        // loaded into the tile registers as soon as phase A of tile k has
        // consumed them, and arrives during phase B
        FwdTile<D> tile;
        RowRef rnext{0, 0};
        int32_t col2 = 0;
        uint32_t word2 = 0;
        if (nt > 0) {
            int32_t c0;
            uint32_t w0;
            tiles.fetch(0, i, c0, w0);
            rnext = tiles.decode(0, i, g, c0, w0);
            tile.load(a.K, a.V, rnext.src * HD + hoff, __shfl(rnext.src, vrow(l)) * HD + hoff, g, l);
        }
        if (nt > 1) tiles.fetch(1, i, col2, word2);
        for (int64_t k = 0; k < nt; ++k) {
            const uint32_t valid = rnext.valid;
            const f32x4_t st = fwd_phase_a<D>(tile, qf, vs, l);
            if (k + 1 < nt) {
                rnext = tiles.decode(k + 1, i, g, col2, word2);
                if (k + 2 < nt) tiles.fetch(k + 2, i, col2, word2);
                tile.load(a.K, a.V, rnext.src * HD + hoff, __shfl(rnext.src, vrow(l)) * HD + hoff,
                          g, l);
            }
            fwd_phase_b<D>(st, valid, m, lsum, acc, vs, a.scale2, i, g);
        }

        if (row_ok) {
            const float inv = lsum > 0.f ? 1.f / lsum : 0.f;
#pragma unroll
            for (int s = 0; s < S::NB; ++s)
                store_tile_rows(a.out, row * HD + hoff + 16 * s + 4 * g, acc[s], inv);
            if (g == 0)
                a.lse[row * a.H + h] = lsum > 0.f ? (m + __log2f(lsum)) * kLn2 : kNegInf;
        }
    }
}

// ---------------------------------------------------------------------------
// backward: the tile-row pass recomputes S and dP per tile from the forward's
// lse (nothing per edge is kept from the forward), accumulates dQ and hands P
// and dS of every edge to the tile-column pass, which accumulates dK and dV;
// no atomics
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
    const int32_t* res_col_edge;
    const void *Q, *K, *V, *O, *dO;
    const float* lse;
    // weights and dS of every edge, from the tile-row pass to the tile-column
    // pass: per (dense tile, head) the P^T and dS^T operand fragments of the
    // 64 lanes (8 bytes each), per (residual edge, head) one word (bf16 P low,
    // bf16 dS high)
    uint2* tile_pd;      // [tiles][H][2][64]
    uint32_t* res_pd;    // [residual_edges][H]
    void *dQ, *dK, *dV;
    float scale2, oscale;
};

template <int D>
struct RowBwdTile {
    Frag kf[Shape<D>::KS], vf[Shape<D>::KS];
    __device__ __forceinline__ void load(const void* K, const void* V, int64_t base, int g)
    {
#pragma unroll
        for (int s = 0; s < Shape<D>::KS; ++s) {
            kf[s] = ldg<SGAT_BF16>(K, base + 32 * s + 8 * g);
            vf[s] = ldg<SGAT_BF16>(V, base + 32 * s + 8 * g);
        }
    }
};

// Tile-row step: rows i = l%16, columns 4g..4g+3 in this lane;
// dS = P (dP - Delta_i) and dQ^T += K^T dS^T (K transposed through LDS).
// Phase A consumes the tile registers (S, dP; K into LDS); phase B forms dS
// and accumulates from LDS, while the next tile's loads refill the registers.
template <int D>
__device__ __forceinline__ void row_bwd_phase_a(const RowBwdTile<D>& tl,
                                                const bf16x8_t (&qf)[Shape<D>::KS],
                                                const bf16x8_t (&df)[Shape<D>::KS], f32x4_t& st,
                                                f32x4_t& dp, uint16_t* ks, int i, int g)
{
    using S = Shape<D>;
    st = f32x4_t{0.f, 0.f, 0.f, 0.f};
    dp = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s = 0; s < S::KS; ++s) {
        st = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, tl.kf[s]), qf[s],
                                                     st, 0, 0, 0);
        dp = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, tl.vf[s]), df[s],
                                                     dp, 0, 0, 0);
    }
    store_operand_tile<D>(ks, tl.kf, i, g);
}

// Tile-row step, phase B: P and dS of the lane's four entries (also staged
// row-major in the wave's LDS tiles pt, for hand_off()), dQ^T += K^T dS^T from
// LDS.
template <int D>
__device__ __forceinline__ void row_bwd_phase_b(const f32x4_t& st, const f32x4_t& dp,
                                                uint32_t valid, float lse2, float delta,
                                                f32x4_t (&acc)[Shape<D>::NB], const uint16_t* ks,
                                                float scale2, int i, int g,
                                                uint16_t (*pt)[kTileDim * kTileDim])
{
    using S = Shape<D>;
    short pb[4], dsb[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        const float p = ((valid >> k) & 1u) ? fast_exp2(st[k] * scale2 - lse2) : 0.f;
        pb[k] = bf16_bits(p);
        dsb[k] = bf16_bits(p * (dp[k] - delta));
    }
    const s16x4_t b = {dsb[0], dsb[1], dsb[2], dsb[3]};
    *reinterpret_cast<s16x4_t*>(&pt[0][i * kTileDim + 4 * g]) = s16x4_t{pb[0], pb[1], pb[2], pb[3]};
    *reinterpret_cast<s16x4_t*>(&pt[1][i * kTileDim + 4 * g]) = b;
    __builtin_amdgcn_wave_barrier();
    const uint16_t* kt = operand_tr_base<D>(ks, i, g);
#pragma unroll
    for (int s = 0; s < S::NB; ++s) {
        const s16x4_t ka = lds_read_tr16(kt + 16 * s);   // K[4g + kk][16s + i], kk = 0..3
        acc[s] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(ka, b, acc[s], 0, 0, 0);
    }
    __builtin_amdgcn_wave_barrier();
}

// Hands tile k's P and dS, staged row-major in pt by phase B, to the
// tile-column pass. Dense tile: read back with the transposing read so that
// lane (c, g) holds rows 4g..4g+3 of column c (the column pass's B operand),
// and stored as that lane's 8 bytes. Residual pseudo-tile: lane c < 16 stores
// the pair of its column's edge e (at the edge's row) as one word.
__device__ __forceinline__ void hand_off(const BsBwdArgs& a, const RowTiles& tiles, int64_t k,
                                         int h, uint16_t (*pt)[kTileDim * kTileDim], int l,
                                         int i, int g)
{
    if (k < tiles.nd) {
        // lane m of a 16-lane group addresses row 4g + m / 4, columns 4 (m % 4)..+3
        const int off = (4 * g + i / 4) * kTileDim + 4 * (i % 4);
        uint2* dst = a.tile_pd + (static_cast<int64_t>(tiles.tb + k) * a.H + h) * 2 * kWave;
        dst[l] = __builtin_bit_cast(uint2, lds_read_tr16(&pt[0][off]));
        dst[kWave + l] = __builtin_bit_cast(uint2, lds_read_tr16(&pt[1][off]));
    } else {
        const int64_t e = tiles.rb + (k - tiles.nd) * 16 + l;   // column l is residual edge e
        if (l < kTileDim && e < tiles.re) {
            const int r = tiles.starts.row_of(e);
            a.res_pd[e * a.H + h] = static_cast<uint32_t>(pt[0][r * kTileDim + l]) |
                                    (static_cast<uint32_t>(pt[1][r * kTileDim + l]) << 16);
        }
    }
    __builtin_amdgcn_wave_barrier();
}

template <int D>
__global__ __launch_bounds__(kBlock) __attribute__((amdgpu_waves_per_eu(3))) void gt_bs_bwd_rows(BsBwdArgs a)
{
    using S = Shape<D>;
    __shared__ __attribute__((aligned(16))) uint16_t ks_all[kWavesPerBlock][16 * S::LDV];
    // one 16x16 bf16 tile of P and one of dS, row-major, to transpose them
    __shared__ __attribute__((aligned(16))) uint16_t pt_all[kWavesPerBlock][2][kTileDim * kTileDim];
    const int64_t br = logical_block();
    if (br >= a.n_blocks) return;
    const int w = wave_id();
    const int l = threadIdx.x & 63, i = l & 15, g = l >> 4;
    const int64_t HD = static_cast<int64_t>(a.H) * D;
    RowTiles tiles;
    const int64_t r_lo = br * kTileDim;
    const int64_t r_hi = r_lo + kTileDim < a.n ? r_lo + kTileDim : a.n;
    tiles.n = a.n;
    tiles.tb = a.tile_rowptr[br];
    tiles.nd = a.tile_rowptr[br + 1] - tiles.tb;
    tiles.rb = a.res_rowptr[r_lo];
    tiles.re = a.res_rowptr[r_hi];
    tiles.tile_col = a.tile_col;
    tiles.tile_mask = a.tile_mask;
    tiles.res_colidx = a.res_colidx;
    tiles.starts.load(a.res_rowptr, r_lo, r_hi);
    const int64_t nt = tiles.count();
    const int64_t row = r_lo + i;
    const bool row_ok = row < a.n;
    uint16_t* ks = ks_all[w];

    for (int h = w; h < a.H; h += kWavesPerBlock) {
        const int64_t hoff = static_cast<int64_t>(h) * D;
        bf16x8_t qf[S::KS], df[S::KS];
        float dsum = 0.f, lse2 = 0.f;
#pragma unroll
        for (int s = 0; s < S::KS; ++s) {
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
        f32x4_t acc[S::NB];
#pragma unroll
        for (int s = 0; s < S::NB; ++s) acc[s] = f32x4_t{0.f, 0.f, 0.f, 0.f};

        // pipeline: descriptions two tiles ahead; tile k+1's data refills the
        // tile registers once phase A of tile k has consumed them
        RowBwdTile<D> tile;
        RowRef rnext{0, 0};
        int32_t col2 = 0;
        uint32_t word2 = 0;
        if (nt > 0) {
            int32_t c0;
            uint32_t w0;
            tiles.fetch(0, i, c0, w0);
            rnext = tiles.decode(0, i, g, c0, w0);
            tile.load(a.K, a.V, rnext.src * HD + hoff, g);
        }
        if (nt > 1) tiles.fetch(1, i, col2, word2);
        for (int64_t k = 0; k < nt; ++k) {
            const uint32_t valid = rnext.valid;
            f32x4_t st, dp;
            row_bwd_phase_a<D>(tile, qf, df, st, dp, ks, i, g);
            if (k + 1 < nt) {
                rnext = tiles.decode(k + 1, i, g, col2, word2);
                if (k + 2 < nt) tiles.fetch(k + 2, i, col2, word2);
                tile.load(a.K, a.V, rnext.src * HD + hoff, g);
            }
            row_bwd_phase_b<D>(st, dp, valid, lse2, dsum, acc, ks, a.scale2, i, g, pt_all[w]);
            hand_off(a, tiles, k, h, pt_all[w], l, i, g);
        }
        if (row_ok) {
#pragma unroll
            for (int s = 0; s < S::NB; ++s)
                store_tile_rows(a.dQ, row * HD + hoff + 16 * s + 4 * g, acc[s], a.oscale);
        }
    }
}

// Tiles of one 16-source block, in order: its dense tiles (by block row),
// then its residual edges (by source) in pseudo-tiles of 16. The lane's A
// operand row is tile row l%16; its four entries are rows 4g..4g+3 of
// column l%16. fetch() issues the raw description loads of a tile (used two
// tiles later), ColBwdTile::load() its data (used one tile later).
struct ColTiles {
    int64_t n, tcb, nd, rcb, rce;
    int H, h;
    const int32_t* tile_bycol;
    const int32_t* tile_row;
    const int32_t* res_rowidx;
    const int32_t* res_col_edge;
    const uint2* tile_pd;
    const uint32_t* res_pd;
    BlockStarts starts;

    __device__ __forceinline__ int64_t count() const { return nd + (rce - rcb + 15) / 16; }

    // dense tile: t = tile id; residual pseudo-tile: dst = destination of row
    // l%16 and re = its residual-CSR edge id
    __device__ __forceinline__ void fetch(int64_t k, int c, int32_t& t, int32_t& dst,
                                          int32_t& re) const
    {
        if (k < nd) {
            t = tile_bycol[tcb + k];
            dst = 0;
            re = 0;
        } else {
            const int64_t e = rcb + (k - nd) * 16 + c;
            t = 0;
            dst = e < rce ? res_rowidx[e] : 0;
            re = e < rce ? res_col_edge[e] : -1;
        }
    }
};

// One tile of the column pass: the Q and dO rows of its 16 destinations (A
// operand layout) and this lane's P^T and dS^T fragments (rows 4g..4g+3 of
// column l%16), both left by the tile-row pass.
template <int D>
struct ColBwdTile {
    Frag qa[Shape<D>::KS], oa[Shape<D>::KS];
    s16x4_t pt, dt;

    __device__ __forceinline__ void load(const ColTiles& T, int64_t k, int32_t t, int32_t dst,
                                         int32_t re, const void* Q, const void* dO, int64_t HD,
                                         int64_t hoff, int l, int c, int g)
    {
        int64_t arow = 0;
        if (k < T.nd) {
            arow = min(static_cast<int64_t>(T.tile_row[t]) * kTileDim + c, T.n - 1);
            const uint2* f = T.tile_pd + (static_cast<int64_t>(t) * T.H + T.h) * 2 * kWave;
            pt = __builtin_bit_cast(s16x4_t, f[l]);
            dt = __builtin_bit_cast(s16x4_t, f[kWave + l]);
        } else {
            const int64_t e = T.rcb + (k - T.nd) * 16 + c;   // row c of this pseudo-tile is edge e
            const int cc = e < T.rce ? T.starts.row_of(e) : -1;
            const uint32_t w = re >= 0 ? T.res_pd[static_cast<int64_t>(re) * T.H + T.h] : 0u;
            arow = dst;
            short pb[4], db[4];
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const int lq = 4 * g + q;   // entry (row 4g + q, column c)
                const bool bit = __shfl(cc, lq) == c;
                const uint32_t wq = __shfl(w, lq);
                pb[q] = static_cast<short>(bit ? (wq & 0xffffu) : 0u);
                db[q] = static_cast<short>(bit ? (wq >> 16) : 0u);
            }
            pt = s16x4_t{pb[0], pb[1], pb[2], pb[3]};
            dt = s16x4_t{db[0], db[1], db[2], db[3]};
        }
        const int64_t qbase = arow * HD + hoff;
#pragma unroll
        for (int s = 0; s < Shape<D>::KS; ++s) {
            qa[s] = ldg<SGAT_BF16>(Q, qbase + 32 * s + 8 * g);
            oa[s] = ldg<SGAT_BF16>(dO, qbase + 32 * s + 8 * g);
        }
    }
};

// Tile-column step: dK^T += Q^T dS, dV^T += dO^T P, Q and dO transposed
// through LDS. Phase A stores the tile's Q and dO rows (so the next tile's
// loads can refill the registers), phase B accumulates from LDS.
template <int D>
__device__ __forceinline__ void col_bwd_phase_b(const s16x4_t& pt, const s16x4_t& dt,
                                                f32x4_t (&dk)[Shape<D>::NB],
                                                f32x4_t (&dv)[Shape<D>::NB], const uint16_t* qs,
                                                const uint16_t* os, int c, int g)
{
    using S = Shape<D>;
    __builtin_amdgcn_wave_barrier();
    const uint16_t* qt = operand_tr_base<D>(qs, c, g);
    const uint16_t* ot = operand_tr_base<D>(os, c, g);
#pragma unroll
    for (int s = 0; s < S::NB; ++s) {
        // Q[4g + kk][16s + c] and dO[4g + kk][16s + c], kk = 0..3
        dk[s] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(lds_read_tr16(qt + 16 * s), dt, dk[s],
                                                          0, 0, 0);
        dv[s] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(lds_read_tr16(ot + 16 * s), pt, dv[s],
                                                          0, 0, 0);
    }
    __builtin_amdgcn_wave_barrier();
}

template <int D>
__global__ __launch_bounds__(kBlock) __attribute__((amdgpu_waves_per_eu(3))) void gt_bs_bwd_cols(BsBwdArgs a)
{
    using S = Shape<D>;
    __shared__ __attribute__((aligned(16))) uint16_t qs_all[kWavesPerBlock][16 * S::LDV];
    __shared__ __attribute__((aligned(16))) uint16_t os_all[kWavesPerBlock][16 * S::LDV];
    const int64_t bc = logical_block();
    if (bc >= a.n_blocks) return;
    const int w = wave_id();
    const int l = threadIdx.x & 63, c = l & 15, g = l >> 4;
    const int64_t HD = static_cast<int64_t>(a.H) * D;
    ColTiles T;
    const int64_t c_lo = bc * kTileDim;
    const int64_t c_hi = c_lo + kTileDim < a.n ? c_lo + kTileDim : a.n;
    T.n = a.n;
    T.tcb = a.tile_colptr[bc];
    T.nd = a.tile_colptr[bc + 1] - T.tcb;
    T.rcb = a.res_colptr[c_lo];
    T.rce = a.res_colptr[c_hi];
    T.H = a.H;
    T.tile_bycol = a.tile_bycol;
    T.tile_row = a.tile_row;
    T.res_rowidx = a.res_rowidx;
    T.res_col_edge = a.res_col_edge;
    T.tile_pd = a.tile_pd;
    T.res_pd = a.res_pd;
    T.starts.load(a.res_colptr, c_lo, c_hi);
    const int64_t nt = T.count();
    const int64_t j = c_lo + c;
    const bool j_ok = j < a.n;
    uint16_t* qs = qs_all[w];
    uint16_t* os = os_all[w];

    for (int h = w; h < a.H; h += kWavesPerBlock) {
        T.h = h;
        const int64_t hoff = static_cast<int64_t>(h) * D;
        f32x4_t dk[S::NB], dv[S::NB];
#pragma unroll
        for (int s = 0; s < S::NB; ++s) {
            dk[s] = f32x4_t{0.f, 0.f, 0.f, 0.f};
            dv[s] = f32x4_t{0.f, 0.f, 0.f, 0.f};
        }
        // pipeline: descriptions two tiles ahead; tile k+1's data refills the
        // tile registers once phase A of tile k has put them into LDS
        ColBwdTile<D> tile;
        int32_t t2 = 0, d2 = 0, r2 = 0;
        if (nt > 0) {
            int32_t t0, d0, r0;
            T.fetch(0, c, t0, d0, r0);
            tile.load(T, 0, t0, d0, r0, a.Q, a.dO, HD, hoff, l, c, g);
        }
        if (nt > 1) T.fetch(1, c, t2, d2, r2);
        for (int64_t k = 0; k < nt; ++k) {
            const s16x4_t pt = tile.pt, dt = tile.dt;
            store_operand_tile<D>(qs, tile.qa, c, g);
            store_operand_tile<D>(os, tile.oa, c, g);
            if (k + 1 < nt) {
                const int32_t t1 = t2, d1 = d2, r1 = r2;
                if (k + 2 < nt) T.fetch(k + 2, c, t2, d2, r2);
                tile.load(T, k + 1, t1, d1, r1, a.Q, a.dO, HD, hoff, l, c, g);
            }
            col_bwd_phase_b<D>(pt, dt, dk, dv, qs, os, c, g);
        }
        if (j_ok) {
#pragma unroll
            for (int s = 0; s < S::NB; ++s) {
                store_tile_rows(a.dK, j * HD + hoff + 16 * s + 4 * g, dk[s], a.oscale);
                store_tile_rows(a.dV, j * HD + hoff + 16 * s + 4 * g, dv[s], 1.f);
            }
        }
    }
}

}  // namespace sgat
