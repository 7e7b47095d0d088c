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

}  // namespace sgat
