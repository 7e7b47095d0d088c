// Block-sparse Graph Transformer kernels: 16x16 adjacency tiles on bf16 MFMA.
//
// A block-sparse representation of the graph lets dense matrix units do the
// score and aggregation products where the graph is locally dense (Yandex
// Research blog "On efficient scaling of GNNs via IO-aware layer
// implementations", paragraph on attention-based architectures; IO-Aware
// Layers paper, Abstract: block-sparse variants on locally dense graphs).
//
// One wave owns one head of a tile row (16 destination rows); a tile row's H
// heads go to ceil(H / 4) workgroups of four waves. Per tile (16 source
// columns) and head:
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
    const int32_t* res_row;      // destination of each residual edge
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

// x of this lane and of lane l ^ 16 (R = 16) or l ^ 32 (R = 32), combined
// with a commutative op, in every lane. gfx950's row swaps (v_permlane16_swap
// exchanges the odd 16-lane rows of its first operand with the even rows of
// its second, v_permlane32_swap the upper half with the lower half) are VALU
// instructions: given x twice, one result holds this lane's value and the
// other its partner's, in an order that depends on the row, which a
// commutative op does not see. Bitwise equal to op(x, __shfl_xor(x, R)),
// without the LDS round trip of a permute. All 64 lanes must be active.
// (The results are copied out of the returned pair as scalars: a bit cast
// applied to an element of it directly read element 0 for both.)
template <int R>
__device__ __forceinline__ void row_swap(float x, float& a, float& b)
{
    static_assert(R == 16 || R == 32, "");
    const uint32_t u = __builtin_bit_cast(uint32_t, x);
    uint32_t r0, r1;
    if constexpr (R == 16) {
        const auto r = __builtin_amdgcn_permlane16_swap(u, u, false, false);
        r0 = r[0];
        r1 = r[1];
    } else {
        const auto r = __builtin_amdgcn_permlane32_swap(u, u, false, false);
        r0 = r[0];
        r1 = r[1];
    }
    a = __builtin_bit_cast(float, r0);
    b = __builtin_bit_cast(float, r1);
}

// Sum (max) over the four lanes l, l ^ 16, l ^ 32, l ^ 48, in the order
// (x_l + x_{l^16}) + (x_{l^32} + x_{l^48}).
__device__ __forceinline__ float sum_rows4(float x)
{
    float a, b;
    row_swap<16>(x, a, b);
    row_swap<32>(a + b, a, b);
    return a + b;
}

__device__ __forceinline__ float max_rows4(float x)
{
    float a, b;
    row_swap<16>(x, a, b);
    row_swap<32>(fmaxf(a, b), a, b);
    return fmaxf(a, b);
}

// Transposed 4 x 16-bit LDS read (gfx950 ds_read_b64_tr_b16). Within each
// group of 16 lanes, lane j receives element j % 4 of the 64-bit word that
// lane 4k + j / 4 addressed, in slot k.
__device__ __forceinline__ s16x4_t lds_read_tr16(const uint16_t* p)
{
    return __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (__attribute__((address_space(3))) s16x4_t*)(p));
}

// Base of lane (i, g)'s transposed reads of a row-major LDS tile: block s
// (channels 16s..16s+15 of rows 4g..4g+3) is at + 16 s; lane i of the group
// addresses row 4g + i/4, channels 4(i%4)..+3.
template <int D>
__device__ __forceinline__ const uint16_t* tr_base(const uint16_t* t, int i, int g)
{
    return t + (4 * g + (i >> 2)) * Shape<D>::LDV + 4 * (i & 3);
}

// ---------------------------------------------------------------------------
// the tiles of one 16-node block
// ---------------------------------------------------------------------------

// Workgroups per 16-node block: one wave per head, four waves per workgroup.
__device__ __host__ __forceinline__ int64_t head_groups(int H)
{
    return (H + kWavesPerBlock - 1) / kWavesPerBlock;
}

// A workgroup owns one block of 16 nodes (a tile row, or a tile column in the
// column pass): its dense tiles [tb, tb + nd) of the tile list, then its
// residual entries [rb, re) in pseudo-tiles of 16; lo is its first node.
// (Walking several blocks per workgroup, with the tile pipeline running on
// across block boundaries so that a block's first loads overlap the previous
// block's last tiles, was measured slower twice: consecutive blocks, 1, 2, 4
// and 8 per workgroup, gave 1.67, 1.72, 1.84 and 1.88 ms per community-graph
// step; with whole-line loads, blocks strided by the grid, 1, 2, 4, 8 and 16
// per workgroup gave 1.55, 1.54, 1.54, 1.55 and 1.63 ms, against 1.49 ms for
// one block per workgroup: the stream's three block descriptors cost the row
// pass registers (it spilled), and the forward did not gain.)
struct Blk {
    int64_t tb, nd, rb, re, lo;

    __device__ __forceinline__ void load(const int64_t* tile_ptr, const int64_t* res_ptr,
                                         int64_t b, int64_t n)
    {
        lo = b * kTileDim;
        const int64_t hi = lo + kTileDim < n ? lo + kTileDim : n;
        tb = tile_ptr[b];
        nd = tile_ptr[b + 1] - tb;
        rb = res_ptr[lo];
        re = res_ptr[hi];
    }
    __device__ __forceinline__ int64_t count() const { return nd + (re - rb + 15) / 16; }
};

// What a lane needs of a tile of a row block, loaded two tiles ahead. Dense
// tile: its block column and the lane's row mask word (row i; bit c = edge
// from column c). Pseudo-tile: the source of its column i (residual entry i
// of the tile) and that edge's row within the block (-1 past the block's
// residual entries).
struct RowDesc {
    int32_t col, aux;
};

template <class A>
__device__ __forceinline__ RowDesc row_fetch(const A& a, const Blk& B, int64_t k, int i)
{
    RowDesc d;
    if (k < B.nd) {
        const int64_t t = B.tb + k;
        d.col = a.tile_col[t];
        d.aux = a.tile_mask[t * kTileDim + i];
    } else {
        const int64_t e = B.rb + (k - B.nd) * kTileDim + i;
        d.col = e < B.re ? a.res_colidx[e] : 0;
        d.aux = e < B.re ? a.res_row[e] - static_cast<int32_t>(B.lo) : -1;
    }
    return d;
}

// The source node of the lane's operand row i and its four edge bits (row i,
// columns 4g..4g+3).
struct RowRef {
    int64_t src;
    uint32_t valid;
};

__device__ __forceinline__ RowRef row_decode(const Blk& B, int64_t k, const RowDesc& d, int i,
                                             int g, int64_t n)
{
    RowRef r;
    if (k < B.nd) {
        r.src = min(static_cast<int64_t>(d.col) * kTileDim + i, n - 1);
        r.valid = (static_cast<uint32_t>(d.aux) >> (4 * g)) & 0xFu;
    } else {
        r.src = d.col;
        r.valid = 0;
#pragma unroll
        for (int q = 0; q < 4; ++q) r.valid |= (__shfl(d.aux, 4 * g + q) == i ? 1u : 0u) << q;
    }
    return r;
}

// Whole-line tile loads. In the MFMA operand layout one load instruction
// reads 64 bytes of each of 16 rows (lane l: row l % 16), so it touches 16
// cache lines and uses half of each, and the L1 keeps twice the outstanding
// lines per byte; the TA then waits on the L1 for a large share of the time.
// Instead, instruction j reads rows [j*RPI, (j+1)*RPI) whole: the LPR lanes of
// a row read its 2D-byte head slice contiguously (4 rows x 256 bytes, 8 full
// lines, at D = 128). The rows go to LDS, and the MFMA operands are read
// back from there.
template <int D>
struct TileRows {
    static constexpr int LPR = 2 * D / 16;          // lanes per row
    static constexpr int RPI = kWave / LPR;         // rows per load instruction
    static constexpr int NI = kTileDim / RPI;       // load instructions per tile
    static_assert(NI * RPI == kTileDim, "");
    Frag r[NI];

    // src: this lane's tile row node (row l % 16, in lanes 0..15 of each group)
    __device__ __forceinline__ void load(const void* X, int64_t src, int64_t HD, int64_t hoff,
                                         int l)
    {
#pragma unroll
        for (int j = 0; j < NI; ++j) {
            const int64_t node = __shfl(src, j * RPI + l / LPR);
            r[j] = ldg<SGAT_BF16>(X, node * HD + hoff + 8 * (l % LPR));
        }
    }
    // into an LDS tile of 16 rows at stride Shape<D>::LDV
    __device__ __forceinline__ void store(uint16_t* t, int l) const
    {
#pragma unroll
        for (int j = 0; j < NI; ++j)
            *reinterpret_cast<Frag*>(t + (j * RPI + l / LPR) * Shape<D>::LDV + 8 * (l % LPR)) = r[j];
    }
};

// The MFMA A operand of an LDS tile for k-step s: lane (i, g) holds row i,
// channels 32s + 8g .. +7.
template <int D>
__device__ __forceinline__ bf16x8_t lds_operand(const uint16_t* t, int s, int i, int g)
{
    return *reinterpret_cast<const bf16x8_t*>(t + i * Shape<D>::LDV + 32 * s + 8 * g);
}

template <int D>
struct FwdTile {
    TileRows<D> k, v;
    __device__ __forceinline__ void load(const void* K, const void* V, int64_t src, int64_t HD,
                                         int64_t hoff, int l)
    {
        k.load(K, src, HD, hoff, l);
        v.load(V, src, HD, hoff, l);
    }
};

// One forward tile for one head, in two phases. Phase A consumes the tile's
// registers (K and V rows into LDS, S^T = K Q^T with K read back in operand
// layout), so the next tile's loads can refill them before phase B: the
// masked online-softmax update of (m, lsum) and O^T += V^T P^T from LDS.
template <int D>
__device__ __forceinline__ f32x4_t fwd_phase_a(const FwdTile<D>& tl,
                                               const bf16x8_t (&qf)[Shape<D>::KS], uint16_t* ks,
                                               uint16_t* vs, int l, int i, int g)
{
    using S = Shape<D>;
    tl.k.store(ks, l);
    tl.v.store(vs, l);
    __builtin_amdgcn_wave_barrier();
    f32x4_t st = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s = 0; s < S::KS; ++s)
        st = __builtin_amdgcn_mfma_f32_16x16x32_bf16(lds_operand<D>(ks, s, i, g), qf[s], st, 0, 0, 0);
    __builtin_amdgcn_wave_barrier();
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
    rmax = max_rows4(rmax);
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
    ps = sum_rows4(ps);
    lsum += ps;
    const s16x4_t pb = {bf16_bits(p[0]), bf16_bits(p[1]), bf16_bits(p[2]), bf16_bits(p[3])};
    __builtin_amdgcn_wave_barrier();
    // A operand of block s: V[4g + kk][16s + i] for kk = 0..3, one transposed
    // read (lane 4k + j/4 of the group addresses row 4g + k, channels 16s + 4(j%4))
    const uint16_t* vt = tr_base<D>(vs, i, g);
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

// Rows of a finished row block, head h: out = O / lsum and lse (rows without
// edges: 0 and -inf).
template <int D>
__device__ __forceinline__ void fwd_finish(const BsFwdArgs& a, int64_t lo, int h, int64_t HD,
                                           float m, float lsum, const f32x4_t (&acc)[Shape<D>::NB],
                                           int i, int g)
{
    const int64_t row = lo + i;
    if (row >= a.n) return;
    const int64_t hoff = static_cast<int64_t>(h) * D;
    const float inv = lsum > 0.f ? 1.f / lsum : 0.f;
#pragma unroll
    for (int s = 0; s < Shape<D>::NB; ++s)
        store_tile_rows(a.out, row * HD + hoff + 16 * s + 4 * g, acc[s], inv);
    if (g == 0) a.lse[row * a.H + h] = lsum > 0.f ? (m + __log2f(lsum)) * kLn2 : kNegInf;
}

// Q rows of a row block for head h (A operand of S^T = K Q^T): lane (i, g)
// holds row lo + i, chunk 8g of each 32-channel slab.
template <int D>
__device__ __forceinline__ void load_block_rows(const void* X, int64_t lo, int64_t n, int64_t HD,
                                                int64_t hoff, int i, int g,
                                                bf16x8_t (&x)[Shape<D>::KS])
{
    const int64_t row = lo + i;
#pragma unroll
    for (int s = 0; s < Shape<D>::KS; ++s) {
        x[s] = bf16x8_t{};
        if (row < n) x[s] = ld_bf16x8(X, row * HD + hoff + 32 * s + 8 * g);
    }
}

// At least 3 waves per SIMD: at D = 128 the compiler would otherwise keep
// the accumulators twice (VGPR copies of MFMA results in AGPRs) and stop at 2;
// with the target it keeps them in VGPRs only, without spilling. (Asking for
// 4 fits it in 126 VGPRs, also without spilling, and measured the same.)
template <int D>
__global__ __launch_bounds__(kBlock) __attribute__((amdgpu_waves_per_eu(3))) void gt_bs_fwd(BsFwdArgs a)
{
    using S = Shape<D>;
    __shared__ __attribute__((aligned(16))) uint16_t ks_all[kWavesPerBlock][16 * S::LDV];
    __shared__ __attribute__((aligned(16))) uint16_t vs_all[kWavesPerBlock][16 * S::LDV];
    const int64_t per_block = head_groups(a.H);
    const int64_t lb = logical_block();
    const int64_t br = lb / per_block;
    if (br >= a.n_tile_rows) return;          // the whole workgroup leaves; no barrier follows
    const int w = wave_id();
    const int h = static_cast<int>(lb - br * per_block) * kWavesPerBlock + w;
    if (h >= a.H) return;                     // one head per wave; waves past H idle
    const int l = threadIdx.x & 63, i = l & 15, g = l >> 4;
    const int64_t HD = static_cast<int64_t>(a.H) * D;
    Blk B;
    B.load(a.tile_rowptr, a.res_rowptr, br, a.n);
    const int64_t nt = B.count();
    uint16_t* ks = ks_all[w];
    uint16_t* vs = vs_all[w];
    const int64_t hoff = static_cast<int64_t>(h) * D;
    bf16x8_t qf[S::KS];
    load_block_rows<D>(a.Q, B.lo, a.n, HD, hoff, i, g, qf);
    float m = kNegInf, lsum = 0.f;
    f32x4_t acc[S::NB];
#pragma unroll
    for (int s = 0; s < S::NB; ++s) acc[s] = f32x4_t{0.f, 0.f, 0.f, 0.f};

    // pipeline: descriptions two tiles ahead; the data of tile k+1 is
    // loaded into the tile registers as soon as phase A of tile k has
    // consumed them, and arrives during phase B
    FwdTile<D> tile;
    RowRef rnext{0, 0};
    RowDesc d2{0, -1};
    if (nt > 0) {
        rnext = row_decode(B, 0, row_fetch(a, B, 0, i), i, g, a.n);
        tile.load(a.K, a.V, rnext.src, HD, hoff, l);
    }
    if (nt > 1) d2 = row_fetch(a, B, 1, i);
    for (int64_t k = 0; k < nt; ++k) {
        const uint32_t valid = rnext.valid;
        const f32x4_t st = fwd_phase_a<D>(tile, qf, ks, vs, l, i, g);
        if (k + 1 < nt) {
            rnext = row_decode(B, k + 1, d2, i, g, a.n);
            if (k + 2 < nt) d2 = row_fetch(a, B, k + 2, i);
            tile.load(a.K, a.V, rnext.src, HD, hoff, l);
        }
        fwd_phase_b<D>(st, valid, m, lsum, acc, vs, a.scale2, i, g);
    }
    fwd_finish<D>(a, B.lo, h, HD, m, lsum, acc, i, g);
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
    const int64_t* tile_colptr;
    const int32_t* tile_bycol;
    const int64_t* res_rowptr;
    const int32_t* res_colidx;
    const int64_t* res_colptr;
    const int32_t* res_rowidx;
    const int32_t* res_col_edge;
    const int32_t* res_row;         // destination of each residual edge
    const int32_t* res_colsrc;      // source of each transposed residual entry
    const int32_t* tile_row_bycol;  // block row of each tile, in tile_bycol order
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
    TileRows<D> k, v;
    __device__ __forceinline__ void load(const void* K, const void* V, int64_t src, int64_t HD,
                                         int64_t hoff, int l)
    {
        k.load(K, src, HD, hoff, l);
        v.load(V, src, HD, hoff, l);
    }
};

// Tile-row step: rows i = l%16, columns 4g..4g+3 in this lane;
// dS = P (dP - Delta_i) and dQ^T += K^T dS^T (K read transposed from LDS).
// Phase A consumes the tile registers (K and V rows into LDS; S and dP with
// the operands read back); phase B forms dS and accumulates from LDS, while
// the next tile's loads refill the registers.
template <int D>
__device__ __forceinline__ void row_bwd_phase_a(const RowBwdTile<D>& tl,
                                                const bf16x8_t (&qf)[Shape<D>::KS],
                                                const bf16x8_t (&df)[Shape<D>::KS], f32x4_t& st,
                                                f32x4_t& dp, uint16_t* ks, uint16_t* vs, int l,
                                                int i, int g)
{
    using S = Shape<D>;
    tl.k.store(ks, l);
    tl.v.store(vs, l);
    __builtin_amdgcn_wave_barrier();
    st = f32x4_t{0.f, 0.f, 0.f, 0.f};
    dp = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s = 0; s < S::KS; ++s) {
        st = __builtin_amdgcn_mfma_f32_16x16x32_bf16(lds_operand<D>(ks, s, i, g), qf[s], st, 0, 0, 0);
        dp = __builtin_amdgcn_mfma_f32_16x16x32_bf16(lds_operand<D>(vs, s, i, g), df[s], dp, 0, 0, 0);
    }
    __builtin_amdgcn_wave_barrier();
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
    const uint16_t* kt = tr_base<D>(ks, i, g);
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
// and stored as that lane's 8 bytes. Residual pseudo-tile: lane c < 16
// stores the pair of its column's edge e at the edge's row `aux` as one word.
__device__ __forceinline__ void hand_off(const BsBwdArgs& a, const Blk& B, int64_t k, int32_t aux,
                                         int h, uint16_t (*pt)[kTileDim * kTileDim], int l, int i,
                                         int g)
{
    if (k < B.nd) {
        // lane m of a 16-lane group addresses row 4g + m / 4, columns 4 (m % 4)..+3
        const int off = (4 * g + i / 4) * kTileDim + 4 * (i % 4);
        uint2* dst = a.tile_pd + (static_cast<int64_t>(B.tb + k) * a.H + h) * 2 * kWave;
        dst[l] = __builtin_bit_cast(uint2, lds_read_tr16(&pt[0][off]));
        dst[kWave + l] = __builtin_bit_cast(uint2, lds_read_tr16(&pt[1][off]));
    } else {
        const int64_t e = B.rb + (k - B.nd) * kTileDim + l;   // column l is residual edge e
        if (l < kTileDim && e < B.re) {
            a.res_pd[e * a.H + h] = static_cast<uint32_t>(pt[0][aux * kTileDim + l]) |
                                    (static_cast<uint32_t>(pt[1][aux * kTileDim + l]) << 16);
        }
    }
    __builtin_amdgcn_wave_barrier();
}

// The per-row operands of a row block for head h: Q and dO (A operands of S
// and dP), O (for Delta) and lse.
template <int D>
struct RowBlockRows {
    bf16x8_t qf[Shape<D>::KS], df[Shape<D>::KS];
    Frag of[Shape<D>::KS];
    float lse;

    __device__ __forceinline__ void load(const BsBwdArgs& a, int64_t lo, int64_t HD, int64_t hoff,
                                         int h, int i, int g)
    {
        const int64_t row = lo + i;
        lse = 0.f;
#pragma unroll
        for (int s = 0; s < Shape<D>::KS; ++s) {
            qf[s] = bf16x8_t{};
            df[s] = bf16x8_t{};
            of[s] = frag_zero();
            if (row < a.n) {
                const int64_t o = row * HD + hoff + 32 * s + 8 * g;
                qf[s] = ld_bf16x8(a.Q, o);
                df[s] = __builtin_bit_cast(bf16x8_t, ldg<SGAT_BF16>(a.dO, o));
                of[s] = ldg<SGAT_BF16>(a.O, o);
            }
        }
        if (row < a.n) lse = a.lse[row * a.H + h];
    }
    // Delta of row i (the four lanes of the row hold its D channels) and lse
    // in base 2
    __device__ __forceinline__ void stats(float& delta, float& lse2) const
    {
        float d = 0.f;
#pragma unroll
        for (int s = 0; s < Shape<D>::KS; ++s)
            d += dot<SGAT_BF16>(__builtin_bit_cast(Frag, df[s]), of[s]);
        d = sum_rows4(d);
        delta = d;
        lse2 = lse * kLog2e;
    }
};

template <int D>
__device__ __forceinline__ void store_block_rows(void* dst, int64_t n, int64_t lo, int64_t HD,
                                                 int64_t hoff, const f32x4_t (&acc)[Shape<D>::NB],
                                                 float sc, int i, int g)
{
    const int64_t row = lo + i;
    if (row >= n) return;
#pragma unroll
    for (int s = 0; s < Shape<D>::NB; ++s)
        store_tile_rows(dst, row * HD + hoff + 16 * s + 4 * g, acc[s], sc);
}

template <int D>
__global__ __launch_bounds__(kBlock) __attribute__((amdgpu_waves_per_eu(3))) void gt_bs_bwd_rows(BsBwdArgs a)
{
    using S = Shape<D>;
    __shared__ __attribute__((aligned(16))) uint16_t ks_all[kWavesPerBlock][16 * S::LDV];
    __shared__ __attribute__((aligned(16))) uint16_t vs_all[kWavesPerBlock][16 * S::LDV];
    // one 16x16 bf16 tile of P and one of dS, row-major, to transpose them
    __shared__ __attribute__((aligned(16))) uint16_t pt_all[kWavesPerBlock][2][kTileDim * kTileDim];
    const int64_t per_block = head_groups(a.H);
    const int64_t lb = logical_block();
    const int64_t br = lb / per_block;
    if (br >= a.n_blocks) return;
    const int w = wave_id();
    const int h = static_cast<int>(lb - br * per_block) * kWavesPerBlock + w;
    if (h >= a.H) return;                     // one head per wave; waves past H idle
    const int l = threadIdx.x & 63, i = l & 15, g = l >> 4;
    const int64_t HD = static_cast<int64_t>(a.H) * D;
    Blk B;
    B.load(a.tile_rowptr, a.res_rowptr, br, a.n);
    const int64_t nt = B.count();
    uint16_t* ks = ks_all[w];
    uint16_t* vs = vs_all[w];
    const int64_t hoff = static_cast<int64_t>(h) * D;
    RowBlockRows<D> rows;
    rows.load(a, B.lo, HD, hoff, h, i, g);
    f32x4_t acc[S::NB];
#pragma unroll
    for (int s = 0; s < S::NB; ++s) acc[s] = f32x4_t{0.f, 0.f, 0.f, 0.f};

    // pipeline: descriptions two tiles ahead; tile k+1's data refills the
    // tile registers once phase A of tile k has consumed them
    RowBwdTile<D> tile;
    RowRef rnext{0, 0};
    int32_t auxn = -1;
    RowDesc d2{0, -1};
    if (nt > 0) {
        const RowDesc d0 = row_fetch(a, B, 0, i);
        rnext = row_decode(B, 0, d0, i, g, a.n);
        auxn = d0.aux;
        tile.load(a.K, a.V, rnext.src, HD, hoff, l);
    }
    if (nt > 1) d2 = row_fetch(a, B, 1, i);
    float delta, lse2;
    rows.stats(delta, lse2);
    for (int64_t k = 0; k < nt; ++k) {
        const uint32_t valid = rnext.valid;
        const int32_t aux = auxn;
        f32x4_t st, dpv;
        row_bwd_phase_a<D>(tile, rows.qf, rows.df, st, dpv, ks, vs, l, i, g);
        if (k + 1 < nt) {
            rnext = row_decode(B, k + 1, d2, i, g, a.n);
            auxn = d2.aux;
            if (k + 2 < nt) d2 = row_fetch(a, B, k + 2, i);
            tile.load(a.K, a.V, rnext.src, HD, hoff, l);
        }
        row_bwd_phase_b<D>(st, dpv, valid, lse2, delta, acc, ks, a.scale2, i, g, pt_all[w]);
        hand_off(a, B, k, aux, h, pt_all[w], l, i, g);
    }
    store_block_rows<D>(a.dQ, a.n, B.lo, HD, hoff, acc, a.oscale, i, g);
}

// What a lane needs of a tile of a column block (16 sources), loaded two
// tiles ahead. Dense tile (the column's tiles by block row): its tile id (for
// its P and dS) and the destination of the lane's operand row c. Pseudo-tile
// (residual entries by source, 16 at a time): the destination of entry c, its
// residual edge id (-1 past the block's entries) and its source's column
// within the block.
struct ColDesc {
    int32_t t, dst, re, cc;
};

__device__ __forceinline__ ColDesc col_fetch(const BsBwdArgs& a, const Blk& B, int64_t k, int c)
{
    ColDesc d;
    if (k < B.nd) {
        const int64_t x = B.tb + k;
        d.t = a.tile_bycol[x];
        d.dst = static_cast<int32_t>(min(static_cast<int64_t>(a.tile_row_bycol[x]) * kTileDim + c,
                                         a.n - 1));
        d.re = 0;
        d.cc = 0;
    } else {
        const int64_t e = B.rb + (k - B.nd) * kTileDim + c;
        const bool ok = e < B.re;
        d.t = 0;
        d.dst = ok ? a.res_rowidx[e] : 0;
        d.re = ok ? a.res_col_edge[e] : -1;
        d.cc = ok ? a.res_colsrc[e] - static_cast<int32_t>(B.lo) : -1;
    }
    return d;
}

// One tile of the column pass: the Q and dO rows of its 16 destinations (A
// operand layout) and the raw P, dS the tile-row pass left: a dense tile's
// two 8-byte fragments of this lane, or a pseudo-tile's word (bf16 P, bf16
// dS) of entry c with its column cc. The B operands are formed when the tile
// is computed (pt_dt), so that no load waits inside load().
template <int D>
struct ColBwdTile {
    TileRows<D> q, o;
    uint2 praw, draw;

    __device__ __forceinline__ void load(const BsBwdArgs& a, bool dense, const ColDesc& d, int h,
                                         int64_t HD, int64_t hoff, int l)
    {
        if (dense) {
            const uint2* f = a.tile_pd + (static_cast<int64_t>(d.t) * a.H + h) * 2 * kWave;
            praw = f[l];
            draw = f[kWave + l];
        } else {
            praw.x = d.re >= 0 ? a.res_pd[static_cast<int64_t>(d.re) * a.H + h] : 0u;
            praw.y = static_cast<uint32_t>(d.cc);
            draw = make_uint2(0u, 0u);
        }
        q.load(a.Q, d.dst, HD, hoff, l);
        o.load(a.dO, d.dst, HD, hoff, l);
    }

    // P^T and dS^T B operands: rows 4g..4g+3 of column c
    __device__ __forceinline__ void pt_dt(bool dense, int c, int g, s16x4_t& pt, s16x4_t& dt) const
    {
        if (dense) {
            pt = __builtin_bit_cast(s16x4_t, praw);
            dt = __builtin_bit_cast(s16x4_t, draw);
            return;
        }
        short pb[4], db[4];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const int lq = 4 * g + q;   // entry (row 4g + q, column c)
            const bool bit = __shfl(static_cast<int>(praw.y), lq) == c;
            const uint32_t wq = static_cast<uint32_t>(__shfl(static_cast<int>(praw.x), lq));
            pb[q] = static_cast<short>(bit ? (wq & 0xffffu) : 0u);
            db[q] = static_cast<short>(bit ? (wq >> 16) : 0u);
        }
        pt = s16x4_t{pb[0], pb[1], pb[2], pb[3]};
        dt = s16x4_t{db[0], db[1], db[2], db[3]};
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
    const uint16_t* qt = tr_base<D>(qs, c, g);
    const uint16_t* ot = tr_base<D>(os, c, g);
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

// One head per wave: a block's H heads go to ceil(H / 4) consecutive
// workgroups (waves past H idle). (Splitting each head's channels over two
// waves, which halves a wave's accumulators and tile registers and fits 5
// waves per SIMD, was measured slower: 0.567 against 0.513 ms on the
// community graph, from twice the workgroup starts and hand-off reads.)
template <int D>
__global__ __launch_bounds__(kBlock) __attribute__((amdgpu_waves_per_eu(3))) void gt_bs_bwd_cols(BsBwdArgs a)
{
    using S = Shape<D>;
    __shared__ __attribute__((aligned(16))) uint16_t qs_all[kWavesPerBlock][16 * S::LDV];
    __shared__ __attribute__((aligned(16))) uint16_t os_all[kWavesPerBlock][16 * S::LDV];
    const int64_t per_block = head_groups(a.H);
    const int64_t lb = logical_block();
    const int64_t bc = lb / per_block;
    if (bc >= a.n_blocks) return;
    const int w = wave_id();
    const int h = static_cast<int>(lb - bc * per_block) * kWavesPerBlock + w;
    if (h >= a.H) return;                    // no workgroup barrier follows
    const int l = threadIdx.x & 63, c = l & 15, g = l >> 4;
    const int64_t HD = static_cast<int64_t>(a.H) * D;
    const int64_t hoff = static_cast<int64_t>(h) * D;
    Blk B;
    B.load(a.tile_colptr, a.res_colptr, bc, a.n);
    const int64_t nt = B.count();
    uint16_t* qs = qs_all[w];
    uint16_t* os = os_all[w];

    f32x4_t dk[S::NB], dv[S::NB];
#pragma unroll
    for (int s = 0; s < S::NB; ++s) {
        dk[s] = f32x4_t{0.f, 0.f, 0.f, 0.f};
        dv[s] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    }
    // pipeline: descriptions two tiles ahead; tile k+1's data refills the
    // tile registers once tile k's rows are in LDS
    ColBwdTile<D> tile;
    ColDesc d2{0, 0, -1, -1};
    if (nt > 0) tile.load(a, B.nd > 0, col_fetch(a, B, 0, c), h, HD, hoff, l);
    if (nt > 1) d2 = col_fetch(a, B, 1, c);
    for (int64_t k = 0; k < nt; ++k) {
        s16x4_t pt, dt;
        tile.pt_dt(k < B.nd, c, g, pt, dt);
        tile.q.store(qs, l);
        tile.o.store(os, l);
        if (k + 1 < nt) {
            const ColDesc d1 = d2;
            if (k + 2 < nt) d2 = col_fetch(a, B, k + 2, c);
            tile.load(a, k + 1 < B.nd, d1, h, HD, hoff, l);
        }
        col_bwd_phase_b<D>(pt, dt, dk, dv, qs, os, c, g);
    }
    store_block_rows<D>(a.dK, a.n, B.lo, HD, hoff, dk, a.oscale, c, g);
    store_block_rows<D>(a.dV, a.n, B.lo, HD, hoff, dv, 1.f, c, g);
}

}  // namespace sgat
