// Gather-path kernels: one wavefront per work item (a whole row, or one chunk
// of a split row; in the GATv2 kernels short items go several to a wavefront,
// one per edge group), neighbour rows gathered straight from HBM in 16-byte
// lane fragments, scores and weights kept in registers.
//
// The fused forward computes, per destination i and head h, the scores of its
// in-edges, an online softmax and the weighted sum of neighbour rows in one
// pass, so no edge-level value reaches device memory (Yandex Research blog "On
// efficient scaling of GNNs via IO-aware layer implementations", paragraph on
// attention-based architectures). Scores are kept in base 2: s2 = s * log2(e).
//
// The backward recomputes alpha_ij = exp(s_ij - lse_i) from the forward's
// per-(node, head) log-sum-exp (same paragraph: recomputation from compact
// statistics), with Delta_i = dout_i . out_i. Gradients that belong to a
// destination are summed over the CSR, those that belong to a source over the
// transposed CSR, so no atomics are needed. Graph Transformer: the
// transposed-CSR pass runs first; it holds K_j and V_j of its source, gathers
// Q_i and dout_i, forms dS_ij and writes it (H floats per edge) for the CSR
// pass, which then gathers only K_j for dQ. GATv2: the CSR pass (dXs, da,
// Delta) runs first and leaves per edge p_ij, dE_ij and the signs of z_ij, so
// the transposed pass (dXt) gathers only dout_i.
#pragma once

#include "device.hpp"

namespace sgat {

constexpr float kNegInf = -__builtin_huge_valf();

struct RowStat { float lse2; float delta; };   // lse * log2(e), Delta

// ---------------------------------------------------------------------------
// forward: online softmax over one row (or chunk)
// ---------------------------------------------------------------------------

// a running maximum moves only when passed by more than 2^kLazyLog2 (the
// weights then stay below 2^8: no overflow risk in fp32 sums)
constexpr float kLazyLog2 = 8.f;

// Online-softmax state of one lane: reference maximum m (base 2; the running
// maximum, or in the GATv2 step within 2^kLazyLog2 below it), sum l of
// exp2(s - m) and the weighted accumulator of this lane's VEC channels.
template <int VEC>
struct Online {
    float m = kNegInf, l = 0.f;
    float acc[VEC] = {};
};

// Merge the states of the EPW edge groups of a wave (log-sum-exp merge).
template <int VEC, int LPE>
__device__ __forceinline__ void merge_groups(Online<VEC>& s)
{
#pragma unroll
    for (int off = LPE; off < kWave; off <<= 1) {
        const float m2 = __shfl_xor(s.m, off);
        const float l2 = __shfl_xor(s.l, off);
        const float mn = fmaxf(s.m, m2);
        const float c1 = s.m == kNegInf ? 0.f : fast_exp2(s.m - mn);
        const float c2 = m2 == kNegInf ? 0.f : fast_exp2(m2 - mn);
        s.l = s.l * c1 + l2 * c2;
#pragma unroll
        for (int k = 0; k < VEC; ++k) s.acc[k] = s.acc[k] * c1 + __shfl_xor(s.acc[k], off) * c2;
        s.m = mn;
    }
}

template <int VEC, int LPE>
__device__ __forceinline__ void sum_groups(float (&x)[VEC])
{
#pragma unroll
    for (int off = LPE; off < kWave; off <<= 1)
#pragma unroll
        for (int k = 0; k < VEC; ++k) x[k] += __shfl_xor(x[k], off);
}

// Write a finished row (slot < 0) or a chunk's partial state (slot >= 0).
template <int DT, int VEC>
__device__ __forceinline__ void fwd_store(const Online<VEC>& s, const sgat_work_item& it,
                                          int64_t HD, int H, int head, int col, bool leader,
                                          void* out, float* lse, float* part_acc, float* part_ml)
{
    if (it.slot < 0) {
        const float inv = s.l > 0.f ? 1.f / s.l : 0.f;
        float o[VEC];
#pragma unroll
        for (int k = 0; k < VEC; ++k) o[k] = s.acc[k] * inv;
        stg<DT>(out, static_cast<int64_t>(it.row) * HD + col, o);
        if (leader)
            lse[static_cast<int64_t>(it.row) * H + head] =
                s.l > 0.f ? (s.m + __log2f(s.l)) * kLn2 : kNegInf;
    } else {
        st_f32<VEC>(part_acc + static_cast<int64_t>(it.slot) * HD + col, s.acc);
        if (leader) {
            float2* ml = reinterpret_cast<float2*>(part_ml) + static_cast<int64_t>(it.slot) * H + head;
            *ml = make_float2(s.m, s.l);
        }
    }
}

struct GtFwdArgs {
    const sgat_work_item* items;
    int64_t n_units;
    int n_hg, H;
    const int32_t* colidx;
    const void *Q, *K, *V;
    void* out;
    float* lse;
    float *part_acc, *part_ml;
    float scale2;   // log2(e) / sqrt(D)
};

template <int DT, int D, int EPW, int U>
__global__ __launch_bounds__(kBlock) void gt_fwd_rows(GtFwdArgs a)
{
    using G = Geo<DT, D, EPW>;
    constexpr int VEC = G::VEC;
    const int64_t unit = logical_block() * kWavesPerBlock + wave_id();
    if (unit >= a.n_units) return;
    const int64_t ii = unit / a.n_hg;
    const int hg = static_cast<int>(unit - ii * a.n_hg);
    const sgat_work_item it = a.items[ii];
    const G g(hg, a.H);
    const int64_t HD = static_cast<int64_t>(a.H) * D;

    Frag q = frag_zero();
    if (g.hvalid) q = ldg_once<DT>(a.Q, static_cast<int64_t>(it.row) * HD + g.col);
    Online<VEC> st;
    const int32_t* ci = a.colidx + it.begin;
    for (int base = 0; base < it.len; base += kWave) {
        const int nb = min(kWave, it.len - base);
        const int cj = g.lane < nb ? ci[base + g.lane] : 0;
        for (int t = 0; t < nb; t += EPW * U) {
            Frag kf[U], vf[U];
            bool ok[U];
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const int e = t + u * EPW + g.sub;
                ok[u] = e < nb;
                const int64_t j = bcast<EPW>(cj, e);
                kf[u] = frag_zero();
                vf[u] = frag_zero();
                if (ok[u] && g.hvalid) {
                    kf[u] = ldg_nbr<DT>(a.K, static_cast<uint32_t>(j), g.col, HD);
                    vf[u] = ldg_nbr<DT>(a.V, static_cast<uint32_t>(j), g.col, HD);
                }
            }
            float s[U];
            float mb = kNegInf;
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const float hs = head_sum<G::SPH>(dot<DT>(q, kf[u])) * a.scale2;
                s[u] = ok[u] ? hs : kNegInf;
                mb = fmaxf(mb, s[u]);
            }
            const float mn = fmaxf(st.m, mb);
            const float corr = mn == kNegInf ? 1.f : fast_exp2(st.m - mn);
            st.l *= corr;
#pragma unroll
            for (int k = 0; k < VEC; ++k) st.acc[k] *= corr;
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const float p = ok[u] ? fast_exp2(s[u] - mn) : 0.f;
                st.l += p;
                float v[VEC];
                to_f32<DT>(vf[u], v);
#pragma unroll
                for (int k = 0; k < VEC; ++k) st.acc[k] = fmaf(p, v[k], st.acc[k]);
            }
            st.m = mn;
        }
    }
    if constexpr (EPW > 1) merge_groups<VEC, G::LPE>(st);
    if (g.sub == 0 && g.hvalid)
        fwd_store<DT, VEC>(st, it, HD, a.H, g.head, g.col, g.leader, a.out, a.lse, a.part_acc,
                           a.part_ml);
}

// Work items [0, n_single) get one wavefront each (head group per unit as
// usual); the rest, all short, come EPW to a wavefront: edge group q of the
// wave owns item n_single + EPW*k + q and walks its edges U at a time, so the
// dependent chain of one short row (item, colidx, gathers) overlaps with the
// other rows of the wave instead of running alone.
struct GatFwdArgs {
    const sgat_work_item* items;
    int64_t n_units;
    int64_t n_items, n_single;
    int n_hg, H;
    const int32_t* colidx;
    const void *Xs, *Xt;
    const float* att;
    float slope;
    void* out;
    float* lse;
    float *part_acc, *part_ml;
};

// One GATv2 online-softmax step over U gathered neighbour rows (rows with
// ok == false take no part). a LeakyReLU(z) = c1 z + c2 |z| with
// c1 = a (1 + slope) / 2 and c2 = a (1 - slope) / 2 (both sides agree for
// z > 0, z < 0 and z = 0), two multiply-adds per channel with |z| an operand
// modifier instead of a compare, a select and a multiply-add; c1 and c2 are
// scaled by log2(e).
template <int DT, int VEC, int SPH, int U>
__device__ __forceinline__ void gat_online_step(Online<VEC>& st, const Frag (&xf)[U],
                                                const bool (&ok)[U], const float (&xs)[VEC],
                                                const float (&c1)[VEC], const float (&c2)[VEC])
{
    float s[U];
    float mb = kNegInf;
#pragma unroll
    for (int u = 0; u < U; ++u) {
        float x[VEC];
        to_f32<DT>(xf[u], x);
        float part = 0.f;
#pragma unroll
        for (int k = 0; k < VEC; ++k) {
            const float z = xs[k] + x[k];
            part = fmaf(c2[k], fabsf(z), fmaf(c1[k], z, part));
        }
        const float hs = head_sum<SPH>(part);
        s[u] = ok[u] ? hs : kNegInf;
        mb = fmaxf(mb, s[u]);
    }
    // Lazy rescaling: m is a reference maximum, moved (and l, acc rescaled)
    // only when a score passes it by more than 2^kLazyLog2, so the weights
    // exp2(s - m) stay below 2^kLazyLog2 and most steps skip the rescale;
    // out = acc / l and lse = m + log2(l) hold for any reference m (while m
    // is -inf, l and acc are 0 and the factor exp2(-inf) = 0 keeps them so).
    if (mb > st.m + kLazyLog2) {
        const float corr = fast_exp2(st.m - mb);
        st.l *= corr;
#pragma unroll
        for (int k = 0; k < VEC; ++k) st.acc[k] *= corr;
        st.m = mb;
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
        const float p = ok[u] ? fast_exp2(s[u] - st.m) : 0.f;
        st.l += p;
        float x[VEC];
        to_f32<DT>(xf[u], x);
#pragma unroll
        for (int k = 0; k < VEC; ++k) st.acc[k] = fmaf(p, x[k], st.acc[k]);
    }
}

template <int DT, int D, int EPW>
__device__ __forceinline__ void gat_fwd_prologue(const GatFwdArgs& a, const Geo<DT, D, EPW>& g,
                                                 const sgat_work_item& it, bool has, int64_t HD,
                                                 float (&xs)[Elem<DT>::VEC], float (&c1)[Elem<DT>::VEC],
                                                 float (&c2)[Elem<DT>::VEC])
{
    constexpr int VEC = Elem<DT>::VEC;
    float at[VEC];
#pragma unroll
    for (int k = 0; k < VEC; ++k) xs[k] = at[k] = 0.f;
    if (g.hvalid) {
        if (has) to_f32<DT>(ldg_once<DT>(a.Xs, static_cast<int64_t>(it.row) * HD + g.col), xs);
        ld_f32<VEC>(a.att + g.col, at);
    }
    const float h1 = 0.5f * (1.f + a.slope) * kLog2e, h2 = 0.5f * (1.f - a.slope) * kLog2e;
#pragma unroll
    for (int k = 0; k < VEC; ++k) {
        c1[k] = at[k] * h1;
        c2[k] = at[k] * h2;
    }
}

template <int DT, int D, int EPW, int U>
__device__ __forceinline__ void gat_fwd_one(const GatFwdArgs& a, int64_t ii, int hg)
{
    using G = Geo<DT, D, EPW>;
    constexpr int VEC = G::VEC;
    const sgat_work_item it = a.items[ii];
    const G g(hg, a.H);
    const int64_t HD = static_cast<int64_t>(a.H) * D;
    float xs[VEC], c1[VEC], c2[VEC];
    gat_fwd_prologue<DT, D, EPW>(a, g, it, true, HD, xs, c1, c2);
    Online<VEC> st;
    const int32_t* ci = a.colidx + it.begin;
    for (int base = 0; base < it.len; base += kWave) {
        const int nb = min(kWave, it.len - base);
        const int cj = g.lane < nb ? ci[base + g.lane] : 0;
        for (int t = 0; t < nb; t += EPW * U) {
            Frag xf[U];
            bool ok[U];
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const int e = t + u * EPW + g.sub;
                ok[u] = e < nb;
                const int64_t j = bcast<EPW>(cj, e);
                xf[u] = frag_zero();
                if (ok[u] && g.hvalid) xf[u] = ldg_nbr<DT>(a.Xt, static_cast<uint32_t>(j), g.col, HD);
            }
            gat_online_step<DT, VEC, G::SPH, U>(st, xf, ok, xs, c1, c2);
        }
    }
    if constexpr (EPW > 1) merge_groups<VEC, G::LPE>(st);
    if (g.sub == 0 && g.hvalid)
        fwd_store<DT, VEC>(st, it, HD, a.H, g.head, g.col, g.leader, a.out, a.lse, a.part_acc,
                           a.part_ml);
}

// EPW short items per wave, one per edge group (all lanes of a group share
// the group's trip counts, so the in-group shuffles read active lanes only).
template <int DT, int D, int EPW, int U>
__device__ __forceinline__ void gat_fwd_multi(const GatFwdArgs& a, int64_t first, int hg)
{
    using G = Geo<DT, D, EPW>;
    constexpr int VEC = G::VEC;
    static_assert(G::LPE % U == 0, "a step must not cross the group's index block");
    const G g(hg, a.H);
    const int64_t HD = static_cast<int64_t>(a.H) * D;
    const int64_t idx = first + g.sub;
    const bool has = idx < a.n_items;
    sgat_work_item it{0, 0, 0, -1, 0};
    if (has) it = a.items[idx];
    float xs[VEC], c1[VEC], c2[VEC];
    gat_fwd_prologue<DT, D, EPW>(a, g, it, has, HD, xs, c1, c2);
    Online<VEC> st;
    const int32_t* ci = a.colidx + it.begin;
    const int lead = g.sub * G::LPE;
    for (int base = 0; base < it.len; base += G::LPE) {
        const int nb = min(G::LPE, it.len - base);
        const int cj = g.pos < nb ? ci[base + g.pos] : 0;
        for (int t = 0; t < nb; t += U) {
            Frag xf[U];
            bool ok[U];
#pragma unroll
            for (int u = 0; u < U; ++u) {
                ok[u] = t + u < nb;
                const int64_t j = __shfl(cj, lead + t + u);
                xf[u] = frag_zero();
                if (ok[u] && g.hvalid) xf[u] = ldg_nbr<DT>(a.Xt, static_cast<uint32_t>(j), g.col, HD);
            }
            gat_online_step<DT, VEC, G::SPH, U>(st, xf, ok, xs, c1, c2);
        }
    }
    if (has && g.hvalid)
        fwd_store<DT, VEC>(st, it, HD, a.H, g.head, g.col, g.leader, a.out, a.lse, a.part_acc,
                           a.part_ml);
}

template <int DT, int D, int EPW, int U, int UM>
__global__ __launch_bounds__(kBlock) void gat_fwd_rows(GatFwdArgs a)
{
    const int64_t unit = logical_block() * kWavesPerBlock + wave_id();
    if (unit >= a.n_units) return;
    const int64_t wi = unit / a.n_hg;
    const int hg = static_cast<int>(unit - wi * a.n_hg);
    if (EPW == 1 || wi < a.n_single)
        gat_fwd_one<DT, D, EPW, U>(a, wi, hg);
    else if constexpr (EPW > 1)
        gat_fwd_multi<DT, D, EPW, (UM < Geo<DT, D, EPW>::LPE ? UM : Geo<DT, D, EPW>::LPE)>(
            a, a.n_single + (wi - a.n_single) * EPW, hg);
}

// Merges of split rows. Grid: (split, block of channels). A block covers EB =
// min(H*D, 256) channels with G = 256 / EB groups of threads; group q takes
// chunks q, q+G, q+2G, ... in order, and group 0 combines the G group results
// in group order, so the result is fixed for a given plan.
__device__ __forceinline__ void merge_geometry(int HD, int& eb, int& grp, int& e)
{
    eb = HD < kBlock ? HD : kBlock;
    grp = threadIdx.x / eb;
    e = blockIdx.y * eb + static_cast<int>(threadIdx.x) % eb;
}

// Log-sum-exp merge of the chunks of split rows (forward).
struct LseMergeArgs {
    const sgat_split* splits;
    int H, D;
    const float *part_acc, *part_ml;
    void* out;
    float* lse;
};

template <int DT>
__global__ __launch_bounds__(kBlock) void lse_merge(LseMergeArgs a)
{
    __shared__ float red[3][kBlock];
    const sgat_split sp = a.splits[blockIdx.x];
    const int HD = a.H * a.D;
    int eb, grp, e;
    merge_geometry(HD, eb, grp, e);
    const int G = kBlock / eb;
    const bool live = e < HD && grp < G;
    const int h = live ? e / a.D : 0;
    const float2* ml = reinterpret_cast<const float2*>(a.part_ml) + static_cast<int64_t>(sp.first_slot) * a.H + h;
    const float* pa = a.part_acc + static_cast<int64_t>(sp.first_slot) * HD + (live ? e : 0);
    float M = kNegInf, L = 0.f, A = 0.f;
    if (live) {
        int k0 = grp;
        for (; k0 + 7 * G < sp.nslots; k0 += 8 * G) {
            float x[8];
#pragma unroll
            for (int u = 0; u < 8; ++u) x[u] = ml[static_cast<int64_t>(k0 + u * G) * a.H].x;
#pragma unroll
            for (int u = 0; u < 8; ++u) M = fmaxf(M, x[u]);
        }
        for (; k0 < sp.nslots; k0 += G) M = fmaxf(M, ml[static_cast<int64_t>(k0) * a.H].x);
        if (M != kNegInf) {
            int k = grp;
            for (; k + 7 * G < sp.nslots; k += 8 * G) {
                float2 v[8];
                float x[8];
#pragma unroll
                for (int u = 0; u < 8; ++u) {
                    v[u] = ml[static_cast<int64_t>(k + u * G) * a.H];
                    x[u] = pa[static_cast<int64_t>(k + u * G) * HD];
                }
#pragma unroll
                for (int u = 0; u < 8; ++u) {
                    const float c = v[u].x == kNegInf ? 0.f : fast_exp2(v[u].x - M);
                    L = fmaf(v[u].y, c, L);
                    A = fmaf(x[u], c, A);
                }
            }
            for (; k < sp.nslots; k += G) {
                const float2 v = ml[static_cast<int64_t>(k) * a.H];
                const float c = v.x == kNegInf ? 0.f : fast_exp2(v.x - M);
                L = fmaf(v.y, c, L);
                A = fmaf(pa[static_cast<int64_t>(k) * HD], c, A);
            }
        }
    }
    red[0][threadIdx.x] = M;
    red[1][threadIdx.x] = L;
    red[2][threadIdx.x] = A;
    __syncthreads();
    if (!live || grp != 0) return;
    float Mt = kNegInf;
    for (int q = 0; q < G; ++q) Mt = fmaxf(Mt, red[0][q * eb + threadIdx.x]);
    float Lt = 0.f, At = 0.f;
    if (Mt != kNegInf) {
        for (int q = 0; q < G; ++q) {
            const float mq = red[0][q * eb + threadIdx.x];
            const float c = mq == kNegInf ? 0.f : fast_exp2(mq - Mt);
            Lt = fmaf(red[1][q * eb + threadIdx.x], c, Lt);
            At = fmaf(red[2][q * eb + threadIdx.x], c, At);
        }
    }
    const float o = Lt > 0.f ? At / Lt : 0.f;
    const int64_t oi = static_cast<int64_t>(sp.row) * HD + e;
    if constexpr (DT == SGAT_F32) static_cast<float*>(a.out)[oi] = o;
    else static_cast<__bf16*>(a.out)[oi] = static_cast<__bf16>(o);
    if (e % a.D == 0)
        a.lse[static_cast<int64_t>(sp.row) * a.H + h] = Lt > 0.f ? (Mt + __log2f(Lt)) * kLn2 : kNegInf;
}

// Fixed-order sum of the partial gradients of split rows (or sources), for
// one or two gradient tensors sharing the split list.
struct SumMergeArgs {
    const sgat_split* splits;
    int HD;
    const float* part[2];
    float scale[2];
    void* out[2];
    int n_out;
};

template <int DT>
__global__ __launch_bounds__(kBlock) void sum_merge(SumMergeArgs a)
{
    __shared__ float red[kBlock];
    const sgat_split sp = a.splits[blockIdx.x];
    int eb, grp, e;
    merge_geometry(a.HD, eb, grp, e);
    const int G = kBlock / eb;
    const bool live = e < a.HD && grp < G;
    for (int o = 0; o < a.n_out; ++o) {
        float s = 0.f;
        if (live) {
            const float* p = a.part[o] + static_cast<int64_t>(sp.first_slot) * a.HD + e;
            int k = grp;
            for (; k + 7 * G < sp.nslots; k += 8 * G) {
                float x[8];
#pragma unroll
                for (int u = 0; u < 8; ++u) x[u] = p[static_cast<int64_t>(k + u * G) * a.HD];
#pragma unroll
                for (int u = 0; u < 8; ++u) s += x[u];
            }
            for (; k < sp.nslots; k += G) s += p[static_cast<int64_t>(k) * a.HD];
        }
        red[threadIdx.x] = s;
        __syncthreads();
        if (live && grp == 0) {
            float t = 0.f;
            for (int q = 0; q < G; ++q) t += red[q * eb + threadIdx.x];
            t *= a.scale[o];
            const int64_t oi = static_cast<int64_t>(sp.row) * a.HD + e;
            if constexpr (DT == SGAT_F32) static_cast<float*>(a.out[o])[oi] = t;
            else static_cast<__bf16*>(a.out[o])[oi] = static_cast<__bf16>(t);
        }
        __syncthreads();
    }
}

// ---------------------------------------------------------------------------
// backward, CSR pass
// ---------------------------------------------------------------------------

template <int DT, int VEC>
__device__ __forceinline__ void grad_store(const float (&x)[VEC], float scale,
                                           const sgat_work_item& it, int64_t HD, int col,
                                           void* out, float* part)
{
    if (it.slot < 0) {
        float o[VEC];
#pragma unroll
        for (int k = 0; k < VEC; ++k) o[k] = x[k] * scale;
        stg<DT>(out, static_cast<int64_t>(it.row) * HD + col, o);
    } else {
        st_f32<VEC>(part + static_cast<int64_t>(it.slot) * HD + col, x);
    }
}

// Delta pre-pass of the Graph Transformer backward: (lse * log2 e, Delta) per
// (node, head); EPW consecutive nodes per wave.
struct DeltaArgs {
    int64_t n_units, n;
    int n_hg, H;
    const void *O, *dO;
    const float* lse;
    RowStat* stats;
};

template <int DT, int D, int EPW>
__global__ __launch_bounds__(kBlock) void bwd_delta(DeltaArgs a)
{
    using G = Geo<DT, D, EPW>;
    const int64_t unit = logical_block() * kWavesPerBlock + wave_id();
    if (unit >= a.n_units) return;
    const int64_t ng = unit / a.n_hg;
    const int hg = static_cast<int>(unit - ng * a.n_hg);
    const G g(hg, a.H);
    const int64_t node = ng * EPW + g.sub;
    const bool ok = node < a.n && g.hvalid;
    const int64_t HD = static_cast<int64_t>(a.H) * D;
    Frag of = frag_zero(), dof = frag_zero();
    if (ok) {
        of = ldg_once<DT>(a.O, node * HD + g.col);
        dof = ldg<DT>(a.dO, node * HD + g.col);
    }
    const float delta = head_sum<G::SPH>(dot<DT>(dof, of));
    if (ok && g.leader) {
        const int64_t k = node * a.H + g.head;
        a.stats[k] = RowStat{a.lse[k] * kLog2e, delta};
    }
}

// Graph Transformer CSR pass: dQ_i = (1/sqrt(D)) sum_j dS_ij K_j, with dS read
// from the transposed pass's per-edge output (CSR edge order, [E][H]).
struct GtBwdRowArgs {
    const sgat_work_item* items;
    int64_t n_units;
    int n_hg, H;
    const int32_t* colidx;
    const int32_t* tpos;   // TPOS: transposed position of each CSR edge (where its dS is)
    const void* K;
    const float* ds;
    void* dQ;
    float* part;
    float oscale;   // 1 / sqrt(D)
};

// TPOS = false: dS is in CSR edge order, read contiguously; true: it is in
// transposed order and each edge's H floats are found through tpos.
template <int DT, int D, int EPW, int U, bool TPOS>
__global__ __launch_bounds__(kBlock) void gt_bwd_rows(GtBwdRowArgs a)
{
    using G = Geo<DT, D, EPW>;
    constexpr int VEC = G::VEC;
    const int64_t unit = logical_block() * kWavesPerBlock + wave_id();
    if (unit >= a.n_units) return;
    const int64_t ii = unit / a.n_hg;
    const int hg = static_cast<int>(unit - ii * a.n_hg);
    const sgat_work_item it = a.items[ii];
    const G g(hg, a.H);
    const int64_t HD = static_cast<int64_t>(a.H) * D;

    float dq[VEC] = {};
    const int32_t* ci = a.colidx + it.begin;
    const float* dsr = a.ds + (TPOS ? 0 : it.begin * a.H) + g.head;
    for (int base = 0; base < it.len; base += kWave) {
        const int nb = min(kWave, it.len - base);
        const int cj = g.lane < nb ? ci[base + g.lane] : 0;
        const int tq = TPOS && g.lane < nb ? a.tpos[it.begin + base + g.lane] : 0;
        for (int t = 0; t < nb; t += EPW * U) {
            Frag kf[U];
            float d[U];
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const int e = t + u * EPW + g.sub;
                const int64_t j = bcast<EPW>(cj, e);
                const int64_t q = TPOS ? static_cast<int64_t>(bcast<EPW>(tq, e)) : base + e;
                kf[u] = frag_zero();
                d[u] = 0.f;
                if (e < nb && g.hvalid) {
                    kf[u] = ldg_nbr<DT>(a.K, static_cast<uint32_t>(j), g.col, HD);
                    d[u] = __builtin_nontemporal_load(dsr + q * a.H);
                }
            }
#pragma unroll
            for (int u = 0; u < U; ++u) {
                float kx[VEC];
                to_f32<DT>(kf[u], kx);
#pragma unroll
                for (int k = 0; k < VEC; ++k) dq[k] = fmaf(d[u], kx[k], dq[k]);
            }
        }
    }
    if constexpr (EPW > 1) sum_groups<VEC, G::LPE>(dq);
    if (g.sub == 0 && g.hvalid) grad_store<DT, VEC>(dq, a.oscale, it, HD, g.col, a.dQ, a.part);
}

// GATv2 CSR pass: dXs and the da partials. Grid-stride over items with a
// fixed grid so the da partials are one per workgroup; blockIdx.y = head group.
// It also leaves one record per (head group, edge) with what the transposed
// pass needs of the edge, so that pass gathers neither Xs_i nor row
// statistics: for head h of the group the weight p and dE (float2 at dword
// 2h), then from byte 8*hg on one byte per lane of the edge group (lane
// position q covers channels q*VEC .. q*VEC+VEC-1 of the group's hg*D), bit k
// set where z > 0 on channel q*VEC + k. Records of head group g start at
// g * nnz records; each is an even number of dwords.
__host__ __device__ constexpr int gat_rec_dwords(int hg, int lanes)
{
    return 2 * hg + ((lanes / 4 + 1) & ~1);
}

struct GatBwdRowArgs {
    const sgat_work_item* items;
    int64_t n_items, n_single;   // items [n_single, n_items) come EPW to a wave, as in the forward
    int H;
    const int32_t* colidx;
    const void *Xs, *Xt, *O, *dO;
    const float* att;
    float slope;
    const float* lse;
    uint32_t* edge_rec;   // [n_hg][nnz][gat_rec_dwords]
    int64_t nnz;
    void* dXs;
    float* part;
    float* da_part;   // [gridDim.x][H*D]
};

// Per-destination state of the GATv2 CSR backward pass.
template <int VEC>
struct GatRowState {
    float xs[VEC];
    Frag dof;
    float lse2, delta;
};

template <int DT, int D, int EPW>
__device__ __forceinline__ GatRowState<Elem<DT>::VEC> gat_row_state(const GatBwdRowArgs& a,
                                                                     const Geo<DT, D, EPW>& g,
                                                                     const sgat_work_item& it,
                                                                     bool load)
{
    constexpr int VEC = Elem<DT>::VEC;
    GatRowState<VEC> r;
    const int64_t ro = static_cast<int64_t>(it.row) * a.H * D + g.col;
    Frag of = frag_zero();
    r.dof = frag_zero();
    r.lse2 = 0.f;
#pragma unroll
    for (int k = 0; k < VEC; ++k) r.xs[k] = 0.f;
    if (load && g.hvalid) {
        to_f32<DT>(ldg_once<DT>(a.Xs, ro), r.xs);
        r.dof = ldg<DT>(a.dO, ro);   // gathered again by the transposed pass
        of = ldg_once<DT>(a.O, ro);
        r.lse2 = a.lse[static_cast<int64_t>(it.row) * a.H + g.head] * kLog2e;
    }
    r.delta = head_sum<Geo<DT, D, EPW>::SPH>(dot<DT>(r.dof, of));
    return r;
}

// da without a per-edge term. a LeakyReLU(z) = a (z s) with s = 1 for z > 0
// and the slope otherwise, and z_ij = Xs_i + Xt_j, so
//   da = sum_ij dE_ij LeakyReLU(z_ij) = sum_i Xs_i . T_i + sum_j Xt_j . U_j
// with T_i = sum_j dE_ij s_ij (the CSR pass; dXs_i = a . T_i) and U_j =
// sum_i dE_ij s_ij (the transposed pass; its share of dXt_j is a . U_j), all
// per channel. Each pass adds its per-row terms, once per item, into per-lane
// LDS slots, and sums them per workgroup at its end in fixed order (waves,
// then edge groups).
template <int VEC>
__device__ __forceinline__ void da_add(float* slot, const float (&x)[VEC], const float (&t)[VEC])
{
#pragma unroll
    for (int k = 0; k < VEC; ++k) slot[k] = fmaf(x[k], t[k], slot[k]);
}

template <int VEC, int LPE, int HG, int D>
__device__ __forceinline__ void da_block_partial(const float (*dal)[kWave * VEC], int hg, int H,
                                                 float* da_part_block)
{
    constexpr int W = LPE * VEC;        // HG heads * D channels
    constexpr int EPW = kWave / LPE;
    __syncthreads();
    for (int t = threadIdx.x; t < W; t += kBlock) {
        const int head = hg * HG + t / D;
        if (head >= H) continue;
        float s = 0.f;
#pragma unroll
        for (int w = 0; w < kWavesPerBlock; ++w)
#pragma unroll
            for (int q = 0; q < EPW; ++q) s += dal[w][q * W + t];   // lane q*LPE + t/VEC
        da_part_block[head * D + (t % D)] = s;
    }
}

// One edge (i, j) for the lane's channels: p = exp(e_ij - lse_i), dE =
// p (dO_i . Xt_j - Delta_i); adds dE s to T (s = 1 for z > 0, the slope
// otherwise; dXs = a . T) and stages (p, dE) and the signs of z in the edge's
// LDS record. The score: a LeakyReLU(z) = h1 (a z) + h2 (a |z|) summed over
// the channels, with h1 = (1 + slope) / 2 and h2 = (1 - slope) / 2 (here
// also scaled by log2(e)): two multiply-adds per channel on a alone.
template <int DT, int D, int EPW>
__device__ __forceinline__ void gat_bwd_edge(const Geo<DT, D, EPW>& g, const Frag& xf, bool ok,
                                             const GatRowState<Elem<DT>::VEC>& r,
                                             const float (&at)[Elem<DT>::VEC], float h1, float h2,
                                             float slope, float (&tsum)[Elem<DT>::VEC],
                                             uint32_t* lr)
{
    using G = Geo<DT, D, EPW>;
    constexpr int VEC = G::VEC;
    float x[VEC], z[VEC];
    to_f32<DT>(xf, x);
    float p1 = 0.f, p2 = 0.f;
#pragma unroll
    for (int k = 0; k < VEC; ++k) {
        z[k] = r.xs[k] + x[k];
        p1 = fmaf(at[k], z[k], p1);
        p2 = fmaf(at[k], fabsf(z[k]), p2);
    }
    const float e2 = head_sum<G::SPH>(fmaf(h1, p1, h2 * p2));
    const float dp = head_sum<G::SPH>(dot<DT>(r.dof, xf));
    const float p = ok ? fast_exp2(e2 - r.lse2) : 0.f;
    const float dE = p * (dp - r.delta);
    const float dEs = dE * slope;
    uint32_t zbits = 0;
#pragma unroll
    for (int k = 0; k < VEC; ++k) {
        tsum[k] += z[k] > 0.f ? dE : dEs;
        zbits |= (z[k] > 0.f ? 1u : 0u) << k;
    }
    reinterpret_cast<uint8_t*>(lr + 2 * G::HG)[g.pos] = static_cast<uint8_t>(zbits);
    if (g.leader) {
        const int hl = g.pos / G::SPH;   // head within the group
        lr[2 * hl] = __float_as_uint(p);
        lr[2 * hl + 1] = __float_as_uint(dE);
    }
}

// 8 bytes of an edge record, read once by the transposed pass (non-temporal)
__device__ __forceinline__ void rec_store(uint2* dst, uint2 v)
{
    typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));
    const u32x2_t w = {v.x, v.y};
    __builtin_nontemporal_store(w, reinterpret_cast<u32x2_t*>(dst));
}

// SHORT = false: the items [0, n_single), one wave each; SHORT = true: the
// items [n_single, n_items), EPW to a wave. Each launch writes one da
// partial per workgroup into its own da_part.
// Waves per SIMD asked of the short-item instance: 6 for the bf16 layouts
// whose short path fits 80 VGPRs without spilling (D = 64, and D = 128 with 4
// edge groups); the others keep the compiler's choice.
constexpr int gat_short_rows_waves(int dt, int D, int epw)
{
    return dt == SGAT_BF16 && (D == 64 || (D == 128 && epw == 4)) ? 6 : 1;
}

template <int DT, int D, int EPW, int U, bool SHORT>
__global__ __launch_bounds__(kBlock)
__attribute__((amdgpu_waves_per_eu(SHORT ? gat_short_rows_waves(DT, D, EPW) : 1)))
void gat_bwd_rows(GatBwdRowArgs a)
{
    using G = Geo<DT, D, EPW>;
    constexpr int VEC = G::VEC;
    constexpr int RS = gat_rec_dwords(G::HG, G::LPE);
    __shared__ float dal[kWavesPerBlock][kWave * VEC];  // per-lane da sums
    // records of one block of edges (64 for a single item, LPE per group for
    // short items), written out contiguously once per block: per-edge global
    // stores inside the loop would make each wait for the next loads also
    // wait for them
    __shared__ __align__(16) uint32_t recbuf[kWavesPerBlock][kWave * RS];
    const int hg = blockIdx.y;
    const G g(hg, a.H);
    const int64_t HD = static_cast<int64_t>(a.H) * D;
    const int wid = wave_id();
    uint32_t* const lrec = recbuf[wid];
    float* const myda = &dal[wid][g.lane * VEC];
#pragma unroll
    for (int k = 0; k < VEC; ++k) myda[k] = 0.f;

    float at[VEC] = {};
    if (g.hvalid) ld_f32<VEC>(a.att + g.col, at);
    const float h1 = 0.5f * (1.f + a.slope) * kLog2e, h2 = 0.5f * (1.f - a.slope) * kLog2e;
    // neighbour rows: a padded head's lanes read row 0, column 0
    const char* const xt_lane =
        static_cast<const char*>(a.Xt) + (g.hvalid ? g.col * Elem<DT>::BYTES : 0);
    const uint32_t row_bytes = static_cast<uint32_t>(HD * Elem<DT>::BYTES);

    const int64_t n_wunits = SHORT ? (a.n_items - a.n_single + EPW - 1) / EPW : a.n_single;
    const int64_t stride = static_cast<int64_t>(gridDim.x) * kWavesPerBlock;
    for (int64_t wi = static_cast<int64_t>(blockIdx.x) * kWavesPerBlock + wid; wi < n_wunits;
         wi += stride) {
        if constexpr (!SHORT) {
            // one item for the whole wave, EPW edges side by side
            const sgat_work_item it = a.items[wi];
            const GatRowState<VEC> r = gat_row_state<DT, D, EPW>(a, g, it, true);
            float ts[VEC] = {};
            const int32_t* ci = a.colidx + it.begin;
            uint32_t* rec = a.edge_rec + (static_cast<int64_t>(hg) * a.nnz + it.begin) * RS;
            for (int base = 0; base < it.len; base += kWave) {
                const int nb = min(kWave, it.len - base);
                const int cj = g.lane < nb ? ci[base + g.lane] : 0;
                // steps of EPW*U edges over two register buffers: the next
                // step's rows are in flight while a step is processed (the
                // short-item loop below explains the unconditional loads)
                auto fetch = [&](int t, Frag (&xf)[U]) {
#pragma unroll
                    for (int u = 0; u < U; ++u) {
                        const int e = t + u * EPW + g.sub;
                        const uint32_t j = bcast<EPW>(cj, e < nb ? e : nb - 1);
                        xf[u] = ldg_row(xt_lane, g.hvalid ? j : 0u, row_bytes);
                    }
                };
                auto step = [&](int t, const Frag (&xf)[U]) {
#pragma unroll
                    for (int u = 0; u < U; ++u) {   // t + u*EPW + sub < 64: EPW*U divides 64
                        const int e = t + u * EPW + g.sub;
                        gat_bwd_edge<DT, D, EPW>(g, xf[u], e < nb, r, at, h1, h2, a.slope, ts,
                                                 lrec + e * RS);
                    }
                };
                Frag xa[U], xb[U];
                fetch(0, xa);
                for (int t = 0; t < nb; t += 2 * EPW * U) {
                    fetch(t + EPW * U, xb);
                    step(t, xa);
                    fetch(t + 2 * EPW * U, xa);
                    if (t + EPW * U < nb) step(t + EPW * U, xb);   // uniform over the wave
                }
                wave_lds_fence();
                {
                    uint2* dst = reinterpret_cast<uint2*>(rec + static_cast<int64_t>(base) * RS);
                    const uint2* src = reinterpret_cast<const uint2*>(lrec);
                    for (int w = g.lane; w < nb * (RS / 2); w += kWave) rec_store(dst + w, src[w]);
                }
                wave_lds_fence();
            }
            if constexpr (EPW > 1) sum_groups<VEC, G::LPE>(ts);
            if (g.sub == 0 && g.hvalid) {
                float dxs[VEC];
#pragma unroll
                for (int k = 0; k < VEC; ++k) dxs[k] = at[k] * ts[k];
                grad_store<DT, VEC>(dxs, 1.f, it, HD, g.col, a.dXs, a.part);
                da_add<VEC>(myda, r.xs, ts);
            }
        } else {
            // EPW short items, one per edge group; all lanes of a group share
            // its trip counts, so the in-group shuffles read active lanes only
            static_assert(EPW > 1, "short items need several edge groups per wave");
            const int64_t idx = a.n_single + wi * EPW + g.sub;
            const bool has = idx < a.n_items;
            sgat_work_item it{0, 0, 0, -1, 0};
            if (has) it = a.items[idx];
            const GatRowState<VEC> r = gat_row_state<DT, D, EPW>(a, g, it, has);
            float ts[VEC] = {};
            const int32_t* ci = a.colidx + it.begin;
            uint32_t* rec = a.edge_rec + (static_cast<int64_t>(hg) * a.nnz + it.begin) * RS;
            uint32_t* const grec = lrec + g.sub * G::LPE * RS;   // the group's LPE records
            const int lead = g.sub * G::LPE;
            for (int base = 0; base < it.len; base += G::LPE) {
                const int nb = min(G::LPE, it.len - base);
                const int cj = g.pos < nb ? ci[base + g.pos] : 0;
                // rolling prefetch over two buffers: the next edge's row is in
                // flight while an edge is processed, and each load refills the
                // buffer just consumed (no register copy that would wait for
                // it). The loads are unconditional (a padded head's lanes read
                // row 0; past the last edge the last one is read again), so
                // each wait needs only the older of two loads.
                auto fetch = [&](int t) {
                    const uint32_t j = __shfl(cj, lead + (t < nb ? t : nb - 1));
                    return ldg_row(xt_lane, g.hvalid ? j : 0u, row_bytes);
                };
                Frag xa = fetch(0);
                for (int t = 0; t < nb; t += 2) {
                    const Frag xb = fetch(t + 1);
                    gat_bwd_edge<DT, D, EPW>(g, xa, true, r, at, h1, h2, a.slope, ts,
                                             grec + t * RS);
                    xa = fetch(t + 2);
                    if (t + 1 < nb)   // the same for the whole group
                        gat_bwd_edge<DT, D, EPW>(g, xb, true, r, at, h1, h2, a.slope, ts,
                                                 grec + (t + 1) * RS);
                }
                wave_lds_fence();
                {
                    uint2* dst = reinterpret_cast<uint2*>(rec + static_cast<int64_t>(base) * RS);
                    const uint2* src = reinterpret_cast<const uint2*>(grec);
                    for (int w = g.pos; w < nb * (RS / 2); w += G::LPE) rec_store(dst + w, src[w]);
                }
                wave_lds_fence();
            }
            if (has && g.hvalid) {
                float dxs[VEC];
#pragma unroll
                for (int k = 0; k < VEC; ++k) dxs[k] = at[k] * ts[k];
                grad_store<DT, VEC>(dxs, 1.f, it, HD, g.col, a.dXs, a.part);
                da_add<VEC>(myda, r.xs, ts);
            }
        }
    }
    da_block_partial<VEC, G::LPE, G::HG, D>(dal, hg, a.H,
                                            a.da_part + static_cast<int64_t>(blockIdx.x) * HD);
}

struct DaReduceArgs {
    const float* da_part;
    int G, HD;
    float* da;
};

// ---------------------------------------------------------------------------
// backward, transposed-CSR pass (one wave per source or source chunk)
// ---------------------------------------------------------------------------

struct GtBwdColArgs {
    const sgat_work_item* items;
    int64_t n_units;
    int n_hg, H;
    const int32_t* rowidx;
    const int32_t* col_edge;   // CSR edge id of each transposed entry
    const void *Q, *K, *V, *dO;
    const RowStat* stats;
    void *dK, *dV;
    float *part_k, *part_v;
    float* ds;                 // out: dS per (CSR edge, head)
    float scale2, oscale;
};

// dS of a block of 64 edges is collected in LDS (one float per edge and head
// of the group) and written once the block's gathers are done: loads and
// stores share one outstanding-memory counter, so a store issued inside the
// gather loop would make every later wait for gathered rows wait for it too.
// TPOS = false: each edge's H floats go to its CSR position (col_edge), a
// scattered partial-line write per edge; true: to its transposed position,
// so a block's values are one contiguous span.
template <int DT, int D, int EPW, int U, bool TPOS>
__global__ __launch_bounds__(kBlock) void gt_bwd_cols(GtBwdColArgs a)
{
    using G = Geo<DT, D, EPW>;
    constexpr int VEC = G::VEC;
    __shared__ float dsl[kWavesPerBlock][kWave * G::HG];
    const int64_t unit = logical_block() * kWavesPerBlock + wave_id();
    if (unit >= a.n_units) return;
    float* my_ds = dsl[wave_id()];
    const int64_t ii = unit / a.n_hg;
    const int hg = static_cast<int>(unit - ii * a.n_hg);
    const sgat_work_item it = a.items[ii];
    const G g(hg, a.H);
    const int64_t HD = static_cast<int64_t>(a.H) * D;

    Frag kj = frag_zero(), vj = frag_zero();
    if (g.hvalid) {
        kj = ldg_once<DT>(a.K, static_cast<int64_t>(it.row) * HD + g.col);
        vj = ldg_once<DT>(a.V, static_cast<int64_t>(it.row) * HD + g.col);
    }
    float dk[VEC] = {}, dv[VEC] = {};
    const int32_t* ri = a.rowidx + it.begin;
    const int32_t* re = a.col_edge + it.begin;
    for (int base = 0; base < it.len; base += kWave) {
        const int nb = min(kWave, it.len - base);
        const int ci = g.lane < nb ? ri[base + g.lane] : 0;
        const int ce = !TPOS && g.lane < nb ? re[base + g.lane] : 0;
        for (int t = 0; t < nb; t += EPW * U) {
            Frag qf[U], df[U];
            RowStat rs[U];
            bool ok[U];
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const int e = t + u * EPW + g.sub;
                ok[u] = e < nb;
                const int64_t i = bcast<EPW>(ci, e);
                qf[u] = frag_zero();
                df[u] = frag_zero();
                rs[u] = RowStat{0.f, 0.f};
                if (ok[u] && g.hvalid) {
                    qf[u] = ldg_nbr<DT>(a.Q, static_cast<uint32_t>(i), g.col, HD);
                    df[u] = ldg_nbr<DT>(a.dO, static_cast<uint32_t>(i), g.col, HD);
                    rs[u] = a.stats[i * a.H + g.head];
                }
            }
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const float s2 = head_sum<G::SPH>(dot<DT>(kj, qf[u])) * a.scale2;
                const float dp = head_sum<G::SPH>(dot<DT>(df[u], vj));
                const float p = ok[u] ? fast_exp2(s2 - rs[u].lse2) : 0.f;
                const float ds = p * (dp - rs[u].delta);
                if (ok[u] && g.leader) my_ds[(t + u * EPW + g.sub) * G::HG + g.pos / G::SPH] = ds;
                float qx[VEC], dx[VEC];
                to_f32<DT>(qf[u], qx);
                to_f32<DT>(df[u], dx);
#pragma unroll
                for (int k = 0; k < VEC; ++k) {
                    dv[k] = fmaf(p, dx[k], dv[k]);
                    dk[k] = fmaf(ds, qx[k], dk[k]);
                }
            }
        }
        // the block's dS: value k*64 + lane is edge (k*64 + lane) / HG, head
        // (k*64 + lane) % HG of the group, so HG consecutive lanes write one
        // edge's HG floats
        wave_lds_fence();
#pragma unroll 1
        for (int k = 0; k < G::HG; ++k) {
            const int v = k * kWave + g.lane;
            const int e = v / G::HG;
            const int head = hg * G::HG + v % G::HG;
            const int64_t eid = TPOS ? it.begin + base + e : __shfl(ce, e);
            if (e < nb && head < a.H)
                __builtin_nontemporal_store(my_ds[v], a.ds + eid * a.H + head);
        }
        wave_lds_fence();
    }
    if constexpr (EPW > 1) {
        sum_groups<VEC, G::LPE>(dk);
        sum_groups<VEC, G::LPE>(dv);
    }
    if (g.sub == 0 && g.hvalid) {
        grad_store<DT, VEC>(dk, a.oscale, it, HD, g.col, a.dK, a.part_k);
        grad_store<DT, VEC>(dv, 1.f, it, HD, g.col, a.dV, a.part_v);
    }
}

struct GatBwdColArgs {
    const sgat_work_item* items;
    int64_t n_items, n_single;   // items [n_single, n_items) come EPW to a wave
    int H;
    const int32_t* rowidx;
    const int32_t* col_edge;    // CSR edge id of each transposed entry
    const void *Xt, *dO;        // Xt: the sources' own rows, for their da terms
    const float* att;
    float slope;
    const uint32_t* edge_rec;   // written by the CSR pass
    int64_t nnz;
    void* dXt;
    float* part;
    float* da_part;             // [gridDim.x][H*D]
};

// (p, dE) of one head from an edge record, read once (non-temporal)
__device__ __forceinline__ float2 rec_pd(const uint32_t* r)
{
    typedef float f32x2_t __attribute__((ext_vector_type(2)));
    const f32x2_t v = __builtin_nontemporal_load(reinterpret_cast<const f32x2_t*>(r));
    return make_float2(v.x, v.y);
}

// Adds U edges (ok == false: no edge) to pacc += p dO_i and uacc += dE s,
// s from the sign bits of the edge record (1 for z > 0, the slope otherwise).
template <int DT, int VEC, int U>
__device__ __forceinline__ void gat_col_step(float (&pacc)[VEC], float (&uacc)[VEC],
                                             const Frag (&df)[U], const float2 (&pd)[U],
                                             const uint32_t (&zb)[U], float slope)
{
#pragma unroll
    for (int u = 0; u < U; ++u) {
        float dx[VEC];
        to_f32<DT>(df[u], dx);
        const float dEs = pd[u].y * slope;
#pragma unroll
        for (int k = 0; k < VEC; ++k) {
            pacc[k] = fmaf(pd[u].x, dx[k], pacc[k]);
            uacc[k] += (zb[u] >> k) & 1u ? pd[u].y : dEs;
        }
    }
}

// dXt_j = sum over i of p_ij dO_i + a . U_j (U_j = sum_i dE_ij s_ij): the
// per-edge p, dE and signs of z come from the CSR pass; only dO_i is
// gathered. Grid-stride over the items with a fixed grid (blockIdx.y = head
// group), so the da partials are one per workgroup.
template <int DT, int D, int EPW, int U, int UM>
__global__ __launch_bounds__(kBlock) void gat_bwd_cols(GatBwdColArgs a)
{
    using G = Geo<DT, D, EPW>;
    constexpr int VEC = G::VEC;
    __shared__ float dal[kWavesPerBlock][kWave * VEC];   // per-lane da sums
    const int hg = blockIdx.y;
    const G g(hg, a.H);
    const int64_t HD = static_cast<int64_t>(a.H) * D;
    const int wid = wave_id();
    constexpr int RS = gat_rec_dwords(G::HG, G::LPE);
    const uint32_t* const rbase = a.edge_rec + static_cast<int64_t>(hg) * a.nnz * RS;
    const int hl = g.pos / G::SPH;
    const int zl = 2 * G::HG + g.pos / 4, zsh = 8 * (g.pos % 4);   // the lane's sign byte
    float* const myda = &dal[wid][g.lane * VEC];
#pragma unroll
    for (int k = 0; k < VEC; ++k) myda[k] = 0.f;

    const int64_t n_wunits =
        EPW == 1 ? a.n_items : a.n_single + (a.n_items - a.n_single + EPW - 1) / EPW;
    // logical_block() keeps runs of consecutive units on one XCD (the grid is
    // a multiple of the remap's quantum)
    const int64_t stride = static_cast<int64_t>(gridDim.x) * kWavesPerBlock;
    for (int64_t wi = logical_block() * kWavesPerBlock + wid; wi < n_wunits; wi += stride) {
        float pacc[VEC] = {}, uacc[VEC] = {};
        if (EPW == 1 || wi < a.n_single) {
            const sgat_work_item it = a.items[wi];
            const int32_t* ri = a.rowidx + it.begin;
            const int32_t* re = a.col_edge + it.begin;
            for (int base = 0; base < it.len; base += kWave) {
                const int nb = min(kWave, it.len - base);
                const int ci = g.lane < nb ? ri[base + g.lane] : 0;
                const int ce = g.lane < nb ? re[base + g.lane] : 0;
                for (int t = 0; t < nb; t += EPW * U) {
                    Frag df[U];
                    float2 pd[U];
                    uint32_t zb[U];
#pragma unroll
                    for (int u = 0; u < U; ++u) {
                        const int e = t + u * EPW + g.sub;
                        const int64_t i = bcast<EPW>(ci, e);
                        const int64_t eid = bcast<EPW>(ce, e);
                        df[u] = frag_zero();
                        pd[u] = make_float2(0.f, 0.f);
                        zb[u] = 0;
                        if (e < nb && g.hvalid) {
                            const uint32_t* r = rbase + eid * RS;
                            df[u] = ldg<DT>(a.dO, i * HD + g.col);   // keeps 7 waves per SIMD
                            pd[u] = rec_pd(r + 2 * hl);
                            zb[u] = __builtin_nontemporal_load(r + zl) >> zsh;
                        }
                    }
                    gat_col_step<DT, VEC, U>(pacc, uacc, df, pd, zb, a.slope);
                }
            }
            if constexpr (EPW > 1) {
                sum_groups<VEC, G::LPE>(pacc);
                sum_groups<VEC, G::LPE>(uacc);
            }
            if (g.sub == 0 && g.hvalid) {
                float dxt[VEC], xt[VEC], at[VEC];
                ld_f32<VEC>(a.att + g.col, at);   // a is read per item, not held
#pragma unroll
                for (int k = 0; k < VEC; ++k) dxt[k] = fmaf(at[k], uacc[k], pacc[k]);
                grad_store<DT, VEC>(dxt, 1.f, it, HD, g.col, a.dXt, a.part);
                to_f32<DT>(ldg_once<DT>(a.Xt, static_cast<int64_t>(it.row) * HD + g.col), xt);
                da_add<VEC>(myda, xt, uacc);
            }
        } else if constexpr (EPW > 1) {
            // EPW short items, one per edge group (in-group shuffles only)
            constexpr int V = UM < G::LPE ? UM : G::LPE;
            const int64_t idx = a.n_single + (wi - a.n_single) * EPW + g.sub;
            const bool has = idx < a.n_items;
            sgat_work_item it{0, 0, 0, -1, 0};
            if (has) it = a.items[idx];
            const int32_t* ri = a.rowidx + it.begin;
            const int32_t* re = a.col_edge + it.begin;
            const int lead = g.sub * G::LPE;
            for (int base = 0; base < it.len; base += G::LPE) {
                const int nb = min(G::LPE, it.len - base);
                const int ci = g.pos < nb ? ri[base + g.pos] : 0;
                const int ce = g.pos < nb ? re[base + g.pos] : 0;
                for (int t = 0; t < nb; t += V) {
                    Frag df[V];
                    float2 pd[V];
                    uint32_t zb[V];
#pragma unroll
                    for (int u = 0; u < V; ++u) {
                        const int64_t i = __shfl(ci, lead + t + u);
                        const int64_t eid = __shfl(ce, lead + t + u);
                        df[u] = frag_zero();
                        pd[u] = make_float2(0.f, 0.f);
                        zb[u] = 0;
                        if (t + u < nb && g.hvalid) {
                            const uint32_t* r = rbase + eid * RS;
                            df[u] = ldg<DT>(a.dO, i * HD + g.col);   // keeps 7 waves per SIMD
                            pd[u] = rec_pd(r + 2 * hl);
                            zb[u] = __builtin_nontemporal_load(r + zl) >> zsh;
                        }
                    }
                    gat_col_step<DT, VEC, V>(pacc, uacc, df, pd, zb, a.slope);
                }
            }
            if (has && g.hvalid) {
                float dxt[VEC], xt[VEC], at[VEC];
                ld_f32<VEC>(a.att + g.col, at);   // a is read per item, not held
#pragma unroll
                for (int k = 0; k < VEC; ++k) dxt[k] = fmaf(at[k], uacc[k], pacc[k]);
                grad_store<DT, VEC>(dxt, 1.f, it, HD, g.col, a.dXt, a.part);
                to_f32<DT>(ldg_once<DT>(a.Xt, static_cast<int64_t>(it.row) * HD + g.col), xt);
                da_add<VEC>(myda, xt, uacc);
            }
        }
    }
    da_block_partial<VEC, G::LPE, G::HG, D>(dal, hg, a.H,
                                            a.da_part + static_cast<int64_t>(blockIdx.x) * HD);
}

}  // namespace sgat
