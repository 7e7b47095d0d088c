// Device helpers shared by the gather-path kernels (gfx950, wave64).
//
// Lane geometry. Every lane owns one 16-byte fragment of a node's feature row:
// VEC = 4 fp32 or 8 bf16 channels. A head of D channels spans SPH = D / VEC
// lanes, one edge's head group spans LPE = 64 / EPW lanes, and a wavefront
// processes EPW edges of the same row side by side. Reductions over a head are
// cross-lane sums inside aligned groups of SPH lanes, done with DPP moves.
#pragma once

#include <hip/hip_runtime.h>
#include <cstdint>

#include "sgattn.h"

namespace sgat {

constexpr int kWave = 64;
constexpr int kBlock = 256;
constexpr int kWavesPerBlock = kBlock / kWave;
constexpr int kXcds = 8;         // MI355X: 8 accelerator complex dies, one L2 each
constexpr int kXcdWindow = 16;   // consecutive logical blocks kept on one XCD
constexpr int kGridQuantum = kXcds * kXcdWindow;
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

template <int DT> struct Elem;
template <> struct Elem<SGAT_F32> { static constexpr int VEC = 4; static constexpr int BYTES = 4; };
template <> struct Elem<SGAT_BF16> { static constexpr int VEC = 8; static constexpr int BYTES = 2; };

struct Frag { uint32_t w[4]; };

__device__ __forceinline__ Frag frag_zero() { return Frag{{0u, 0u, 0u, 0u}}; }

template <int DT>
__device__ __forceinline__ Frag ldg(const void* base, int64_t elem)
{
    const uint4 v = *reinterpret_cast<const uint4*>(
        static_cast<const char*>(base) + elem * Elem<DT>::BYTES);
    return Frag{{v.x, v.y, v.z, v.w}};
}

// A row read once per kernel (the item's own row): marked non-temporal so it
// does not displace gathered rows that other waves will read again.
// A lane's 16 bytes of row `row` of a row-major [N][H*D] array: lane_base is
// the array plus the lane's column offset, row_bytes the row pitch. One
// 32 x 32 + 64-bit multiply-add forms the address (rows and pitches fit 32
// bits) instead of 64-bit index arithmetic.
__device__ __forceinline__ Frag ldg_row(const char* lane_base, uint32_t row, uint32_t row_bytes)
{
    const uint4 v = *reinterpret_cast<const uint4*>(
        lane_base + static_cast<uint64_t>(row) * row_bytes);
    return Frag{{v.x, v.y, v.z, v.w}};
}

// ldg_row for element `col` of row `row` of an [N][H*D] array of DT
template <int DT>
__device__ __forceinline__ Frag ldg_nbr(const void* base, uint32_t row, int col, int64_t HD)
{
    return ldg_row(static_cast<const char*>(base) + col * Elem<DT>::BYTES, row,
                   static_cast<uint32_t>(HD) * Elem<DT>::BYTES);
}

typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

template <int DT>
__device__ __forceinline__ Frag ldg_once(const void* base, int64_t elem)
{
    const u32x4_t v = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(
        static_cast<const char*>(base) + elem * Elem<DT>::BYTES));
    return Frag{{v.x, v.y, v.z, v.w}};
}

template <int DT>
__device__ __forceinline__ void to_f32(const Frag& f, float (&x)[Elem<DT>::VEC])
{
    if constexpr (DT == SGAT_F32) {
#pragma unroll
        for (int k = 0; k < 4; ++k) x[k] = __uint_as_float(f.w[k]);
    } else {
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            x[2 * k] = __uint_as_float(f.w[k] << 16);
            x[2 * k + 1] = __uint_as_float(f.w[k] & 0xffff0000u);
        }
    }
}

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

// Partial dot product of two fragments (this lane's channels only).
template <int DT>
__device__ __forceinline__ float dot(const Frag& a, const Frag& b)
{
    float s = 0.f;
    if constexpr (DT == SGAT_F32) {
#pragma unroll
        for (int k = 0; k < 4; ++k) s = fmaf(__uint_as_float(a.w[k]), __uint_as_float(b.w[k]), s);
    } else {
#pragma unroll
        for (int k = 0; k < 4; ++k)
            s = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a.w[k]),
                                                __builtin_bit_cast(bf16x2_t, b.w[k]), s, false);
    }
    return s;
}

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi)
{
    bf16x2_t v = {static_cast<__bf16>(lo), static_cast<__bf16>(hi)};   // round to nearest even
    return __builtin_bit_cast(uint32_t, v);
}

template <int DT>
__device__ __forceinline__ void stg(void* base, int64_t elem, const float (&x)[Elem<DT>::VEC])
{
    uint4 v;
    if constexpr (DT == SGAT_F32) {
        v = make_uint4(__float_as_uint(x[0]), __float_as_uint(x[1]), __float_as_uint(x[2]),
                       __float_as_uint(x[3]));
    } else {
        v = make_uint4(pack_bf16x2(x[0], x[1]), pack_bf16x2(x[2], x[3]), pack_bf16x2(x[4], x[5]),
                       pack_bf16x2(x[6], x[7]));
    }
    const u32x4_t w = {v.x, v.y, v.z, v.w};
    __builtin_nontemporal_store(w, reinterpret_cast<u32x4_t*>(static_cast<char*>(base) +
                                                              elem * Elem<DT>::BYTES));
}

template <int N>
__device__ __forceinline__ void st_f32(float* p, const float (&x)[N])
{
    static_assert(N % 4 == 0, "");
#pragma unroll
    for (int k = 0; k < N; k += 4)
        *reinterpret_cast<float4*>(p + k) = make_float4(x[k], x[k + 1], x[k + 2], x[k + 3]);
}

template <int N>
__device__ __forceinline__ void ld_f32(const float* p, float (&x)[N])
{
#pragma unroll
    for (int k = 0; k < N; k += 4) {
        const float4 v = *reinterpret_cast<const float4*>(p + k);
        x[k] = v.x; x[k + 1] = v.y; x[k + 2] = v.z; x[k + 3] = v.w;
    }
}

template <int CTRL>
__device__ __forceinline__ float dpp(float x)
{
    return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x),
                                                                  CTRL, 0xF, 0xF, true));
}

// Sum over each aligned group of SPH lanes; every lane of the group gets it.
// All 64 lanes must be active.
template <int SPH>
__device__ __forceinline__ float head_sum(float x)
{
    static_assert(SPH == 4 || SPH == 8 || SPH == 16 || SPH == 32, "");
    x += dpp<0xB1>(x);                               // quad_perm [1,0,3,2]: lane ^ 1
    x += dpp<0x4E>(x);                               // quad_perm [2,3,0,1]: lane ^ 2
    if constexpr (SPH >= 8) x += dpp<0x141>(x);      // row_half_mirror: the other quad
    if constexpr (SPH >= 16) x += dpp<0x140>(x);     // row_mirror: the other half-row
    if constexpr (SPH >= 32) x += __shfl_xor(x, 16);
    return x;
}

// Value of `v` held by lane `src` (same for all lanes when EPW == 1).
template <int EPW>
__device__ __forceinline__ int bcast(int v, int src)
{
    if constexpr (EPW == 1) return __builtin_amdgcn_readlane(v, src & 63);
    else return __shfl(v, src & 63);
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Wave index inside the block as a uniform (scalar) value.
__device__ __forceinline__ int wave_id() { return __builtin_amdgcn_readfirstlane(threadIdx.x >> 6); }

// LDS traffic of one wave stays in issue order; this keeps the compiler from
// moving accesses across the phase boundaries either.
__device__ __forceinline__ void wave_lds_fence()
{
    __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
    __builtin_amdgcn_wave_barrier();
}

// Logical block index. Hardware hands consecutive workgroups to the XCDs in
// turn; remap so that each XCD receives runs of kXcdWindow consecutive logical
// blocks (neighbouring rows share K/V rows in its L2). The grid is a multiple
// of kGridQuantum, so the map is a bijection.
__device__ __forceinline__ int64_t logical_block()
{
    const int64_t b = blockIdx.x;
    const int64_t win = b / kGridQuantum, r = b - win * kGridQuantum;
    return win * kGridQuantum + (r % kXcds) * kXcdWindow + r / kXcds;
}

// Geometry of a lane for element type DT, head dim D, EPW edges per wave.
template <int DT, int D, int EPW>
struct Geo {
    static constexpr int VEC = Elem<DT>::VEC;
    static constexpr int SPH = D / VEC;
    static constexpr int LPE = kWave / EPW;
    static constexpr int HG = LPE / SPH;
    static_assert(HG >= 1, "edge group narrower than one head");
    int lane, sub, pos, head, col;
    bool hvalid, leader;
    __device__ __forceinline__ Geo(int hg, int H)
    {
        lane = threadIdx.x & 63;
        sub = lane / LPE;
        pos = lane % LPE;
        head = hg * HG + pos / SPH;
        hvalid = head < H;
        col = head * D + (pos % SPH) * VEC;
        leader = (pos % SPH) == 0;
    }
};

}  // namespace sgat
