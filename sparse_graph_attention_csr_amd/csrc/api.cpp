// C ABI of the fused graph-attention library: argument checks, workspace
// layout, plan upload, kernel-timing trace, dispatch to the launchers.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstring>
#include <mutex>
#include <string>
#include <vector>

#include "launch.hpp"
#include "plan.hpp"

namespace sgat {

Decomp decompose(int dt, int D, int H)
{
    Decomp d{};
    d.vec = dt == SGAT_F32 ? 4 : 8;
    d.sph = D / d.vec;
    const int hg_max = 64 / d.sph;
    const int want = std::min(H, hg_max);
    int hg = 1;
    while (hg < want) hg <<= 1;
    d.hg = hg;
    d.epw = 64 / (hg * d.sph);
    d.n_hg = (H + hg - 1) / hg;
    return d;
}

int64_t wave_grid(int64_t units)
{
    const int64_t blocks = (units + kWavesPerBlock - 1) / kWavesPerBlock;
    return (blocks + kGridQuantum - 1) / kGridQuantum * kGridQuantum;
}

// ---------------------------------------------------------------------------
// trace
// ---------------------------------------------------------------------------

namespace {
struct TraceRec {
    std::string name;
    hipEvent_t start = nullptr, stop = nullptr;
};
bool g_trace = false;
std::string g_trace_only;   // empty: every kernel
std::vector<TraceRec> g_recs;
size_t g_used = 0;
}  // namespace

int launch(const char* name, const void* fn, dim3 grid, dim3 block, void* arg, hipStream_t s)
{
    void* args[] = {arg};
    TraceRec* rec = nullptr;
    if (g_trace && (g_trace_only.empty() || g_trace_only == name)) {
        if (g_used == g_recs.size()) {
            TraceRec r;
            if (hipEventCreate(&r.start) != hipSuccess || hipEventCreate(&r.stop) != hipSuccess)
                return SGAT_HIP_ERROR;
            g_recs.push_back(r);
        }
        rec = &g_recs[g_used++];
        rec->name = name;
        if (hipEventRecord(rec->start, s) != hipSuccess) return SGAT_HIP_ERROR;
    }
    hipError_t e = hipLaunchKernel(fn, grid, block, args, 0, s);
    if (e != hipSuccess) return SGAT_HIP_ERROR;
    if (rec && hipEventRecord(rec->stop, s) != hipSuccess) return SGAT_HIP_ERROR;
    return SGAT_OK;
}

// ---------------------------------------------------------------------------
// argument checks and workspace layout
// ---------------------------------------------------------------------------

namespace {

bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

int check_common(const sgat_plan* plan, int64_t n, int64_t nnz, const int64_t* rowptr,
                 const int32_t* colidx, int H, int D, int dt)
{
    if (!plan) return SGAT_INVALID_ARGUMENT;
    if (H < 1 || H > 16 || (D != 32 && D != 64 && D != 128)) return SGAT_INVALID_ARGUMENT;
    if (dt != SGAT_F32 && dt != SGAT_BF16) return SGAT_INVALID_ARGUMENT;
    if (n != plan->p.n || nnz != plan->p.nnz) return SGAT_PLAN_MISMATCH;
    if (!plan->p.uploaded) return SGAT_NOT_UPLOADED;
    if (!rowptr || (nnz > 0 && !colidx)) return SGAT_INVALID_ARGUMENT;
    return SGAT_OK;
}

int check_reduce(const sgat_plan* plan, int64_t n, int64_t nnz, const int64_t* rowptr,
                 const int32_t* colidx, int F, int dt)
{
    if (!plan) return SGAT_INVALID_ARGUMENT;
    if (!reduce_supported(dt, F)) return SGAT_INVALID_ARGUMENT;
    if (n != plan->p.n || nnz != plan->p.nnz) return SGAT_PLAN_MISMATCH;
    if (!plan->p.uploaded) return SGAT_NOT_UPLOADED;
    if (!rowptr || (nnz > 0 && !colidx)) return SGAT_INVALID_ARGUMENT;
    return SGAT_OK;
}

int check_tensor(const void* p, int64_t n)
{
    if (n == 0) return SGAT_OK;
    if (!p || !aligned(p, 16)) return SGAT_INVALID_ARGUMENT;
    return SGAT_OK;
}

struct Layout {
    size_t off[8] = {};
    size_t total = 0;
};

// Regions, each 256-byte aligned, in this order.
Layout ws_layout(const Plan& p, int op, int H, int D, int dt)
{
    const size_t HD = static_cast<size_t>(H) * D;
    size_t sz[8] = {};
    switch (op) {
    case SGAT_OP_GT_FWD:
    case SGAT_OP_GAT_FWD:
        sz[0] = static_cast<size_t>(p.row_slots) * HD * 4;          // part_acc
        sz[1] = static_cast<size_t>(p.row_slots) * H * 8;           // part_ml
        break;
    case SGAT_OP_GT_BWD:
        sz[0] = static_cast<size_t>(p.n) * H * 8;                   // stats
        sz[1] = static_cast<size_t>(p.row_slots) * HD * 4;          // dQ partials
        sz[2] = static_cast<size_t>(p.col_slots) * HD * 4;          // dK partials
        sz[3] = static_cast<size_t>(p.col_slots) * HD * 4;          // dV partials
        sz[4] = static_cast<size_t>(p.nnz) * H * 4;                 // dS per edge
        if (p.block_sparse) {   // the tile path's edge weights (P, dS)
            sz[6] = static_cast<size_t>(p.tile_col.size()) * H * 2 * 64 * 8;   // per tile, head
            sz[7] = static_cast<size_t>(p.res_colidx.size()) * H * 4;         // per residual edge, head
        }
        break;
    case SGAT_OP_GAT_BWD:
        sz[0] = static_cast<size_t>(p.nnz) * gat_edge_record_dwords(dt, D, H) * 4; // edge records
        sz[1] = static_cast<size_t>(p.row_slots) * HD * 4;          // dXs partials
        sz[2] = static_cast<size_t>(p.col_slots) * HD * 4;          // dXt partials
        {
            const GatRowGrid gx = gat_bwd_row_grid(p, dt, D, H);
            sz[4] = static_cast<size_t>(gat_da_part_rows(gx)) * HD * 4;   // da partials
        }
        break;
    case SGAT_OP_REDUCE_FWD:                                        // H = 1, D = F
        sz[0] = static_cast<size_t>(p.row_slots) * HD * 4;          // partial values
        sz[1] = static_cast<size_t>(p.row_slots) * HD * 4;          // partial winners
        break;
    case SGAT_OP_REDUCE_BWD:
        sz[0] = static_cast<size_t>(p.col_slots) * HD * 4;          // dX partials
        sz[1] = static_cast<size_t>(p.nnz) * 4;                     // (start, count) per edge
        sz[2] = static_cast<size_t>(p.n) * HD * (dt == SGAT_BF16 ? 4 : 8);   // routed pairs
        break;
    default:
        break;
    }
    Layout L;
    size_t off = 0;
    for (int r = 0; r < 8; ++r) {
        L.off[r] = off;
        off = align_up(off + sz[r]);
    }
    L.total = off;
    return L;
}

template <class T>
T* at(void* ws, size_t off) { return reinterpret_cast<T*>(static_cast<char*>(ws) + off); }

int check_ws(const Plan& p, int op, int H, int D, int dt, const void* ws, size_t ws_bytes,
             Layout& L)
{
    L = ws_layout(p, op, H, D, dt);
    if (ws_bytes < L.total) return SGAT_WORKSPACE_TOO_SMALL;
    if (L.total > 0 && (!ws || !aligned(ws, 256))) return SGAT_INVALID_ARGUMENT;
    return SGAT_OK;
}

}  // namespace
}  // namespace sgat

// Static scratch of gt_fwd_noalloc: one copy per GPU, held until the process
// ends. In host code `scratch` is only a handle for the symbol lookup below;
// kernels receive the per-device address that hipGetSymbolAddress returns.
static __device__ __align__(256) unsigned char scratch[SGAT_NOALLOC_SCRATCH_BYTES];

namespace sgat {
namespace {

constexpr int kMaxDevices = 256;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// Address of the scratch array on the device that `s` launches on, looked up
// once per device with that device current (the caller's current device is
// restored).
int scratch_address(hipStream_t s, void** out)
{
    int dev = -1;
    if (hipStreamGetDevice(s, &dev) != hipSuccess || dev < 0 || dev >= kMaxDevices)
        return SGAT_HIP_ERROR;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        int cur = -1;
        if (hipGetDevice(&cur) != hipSuccess) return SGAT_HIP_ERROR;
        if (cur != dev && hipSetDevice(dev) != hipSuccess) return SGAT_HIP_ERROR;
        void* p = nullptr;
        const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (cur != dev && hipSetDevice(cur) != hipSuccess) return SGAT_HIP_ERROR;
        if (e != hipSuccess || !p) return SGAT_HIP_ERROR;
        g_scratch_ptr[dev] = p;
    }
    *out = g_scratch_ptr[dev];
    return SGAT_OK;
}

// gt_fwd with the workspace given as a pointer and size (a caller's buffer,
// or the static scratch; `noalloc` selects the error for a short one).
int gt_fwd_impl(const sgat_plan* plan, int64_t n, int64_t nnz, const int64_t* rowptr,
                const int32_t* colidx, int H, int D, int dtype, const void* Q, const void* K,
                const void* V, void* out, float* lse, void* ws, size_t ws_bytes, bool noalloc,
                int use_tiles, hipStream_t stream)
{
    int rc = check_common(plan, n, nnz, rowptr, colidx, H, D, dtype);
    if (rc) return rc;
    for (const void* t : {Q, K, V, static_cast<const void*>(out)})
        if ((rc = check_tensor(t, n))) return rc;
    if (n > 0 && (!lse || !aligned(lse, 4))) return SGAT_INVALID_ARGUMENT;
    if (use_tiles != 0 && use_tiles != 1) return SGAT_INVALID_ARGUMENT;
    if (use_tiles && (!plan->p.block_sparse || dtype != SGAT_BF16)) return SGAT_UNSUPPORTED;
    Layout L;
    if (noalloc) {
        L = ws_layout(plan->p, SGAT_OP_GT_FWD, H, D, dtype);
        if (L.total > SGAT_NOALLOC_SCRATCH_BYTES) return SGAT_SCRATCH_LIMIT;
        if (n == 0 || use_tiles || L.total == 0) ws = nullptr;   // nothing to look up
        else if ((rc = scratch_address(stream, &ws))) return rc;
    } else if ((rc = check_ws(plan->p, SGAT_OP_GT_FWD, H, D, dtype, ws, ws_bytes, L))) {
        return rc;
    }
    if (n == 0) return SGAT_OK;
    if (use_tiles) return launch_gt_bs_fwd(plan->p, H, D, Q, K, V, out, lse, stream);
    FwdWs w{at<float>(ws, L.off[0]), at<float>(ws, L.off[1])};
    return launch_gt_fwd(plan->p, H, D, dtype, colidx, Q, K, V, out, lse, w, stream);
}

}  // namespace
}  // namespace sgat

using namespace sgat;

extern "C" {

const char* sgat_status_string(int st)
{
    switch (st) {
    case SGAT_OK: return "ok";
    case SGAT_INVALID_ARGUMENT: return "invalid argument";
    case SGAT_INVALID_CSR: return "invalid CSR";
    case SGAT_WORKSPACE_TOO_SMALL: return "workspace or buffer too small";
    case SGAT_PLAN_MISMATCH: return "n or nnz differs from the plan";
    case SGAT_HIP_ERROR: return "HIP error";
    case SGAT_NOT_UPLOADED: return "plan not uploaded";
    case SGAT_OUT_OF_HOST_MEMORY: return "out of host memory";
    case SGAT_UNSUPPORTED: return "unsupported for this plan";
    case SGAT_SCRATCH_LIMIT: return "needs more than the static scratch (SGAT_NOALLOC_SCRATCH_BYTES)";
    default: return "unknown status";
    }
}

int sgat_plan_upload(sgat_plan* plan, void* dev_buf, size_t bytes, void* stream)
{
    if (!plan || !dev_buf) return SGAT_INVALID_ARGUMENT;
    Plan& p = plan->p;
    if (bytes < p.device_bytes) return SGAT_WORKSPACE_TOO_SMALL;
    if (!aligned(dev_buf, kAlign)) return SGAT_INVALID_ARGUMENT;
    hipStream_t s = static_cast<hipStream_t>(stream);
    for (int a = 0; a < SGAT_ARR_COUNT; ++a) {
        if (p.bytes[a] == 0) continue;
        // pageable source: the copy has read it by the time the call returns
        if (hipMemcpyAsync(static_cast<char*>(dev_buf) + p.offset[a], p.host_array(a), p.bytes[a],
                           hipMemcpyHostToDevice, s) != hipSuccess)
            return SGAT_HIP_ERROR;
    }
    p.dev = static_cast<const unsigned char*>(dev_buf);
    p.uploaded = true;
    return SGAT_OK;
}

int sgat_workspace_bytes(const sgat_plan* plan, int op, int H, int D, int dtype, size_t* bytes)
{
    if (!plan || !bytes) return SGAT_INVALID_ARGUMENT;
    if (op < SGAT_OP_GT_FWD || op > SGAT_OP_REDUCE_BWD) return SGAT_INVALID_ARGUMENT;
    if (op >= SGAT_OP_REDUCE_FWD) {
        if (H != 1 || !reduce_supported(dtype, D)) return SGAT_INVALID_ARGUMENT;
    } else {
        if (H < 1 || H > 16 || (D != 32 && D != 64 && D != 128)) return SGAT_INVALID_ARGUMENT;
        if (dtype != SGAT_F32 && dtype != SGAT_BF16) return SGAT_INVALID_ARGUMENT;
    }
    *bytes = ws_layout(plan->p, op, H, D, dtype).total;
    return SGAT_OK;
}

int gt_fwd(const sgat_plan* plan, int64_t n, int64_t nnz, const int64_t* rowptr,
           const int32_t* colidx, int H, int D, int dtype, const void* Q, const void* K,
           const void* V, void* out, float* lse, void* ws, size_t ws_bytes, int use_tiles,
           void* stream)
{
    return gt_fwd_impl(plan, n, nnz, rowptr, colidx, H, D, dtype, Q, K, V, out, lse, ws,
                       ws_bytes, false, use_tiles, static_cast<hipStream_t>(stream));
}

int gt_fwd_noalloc(const sgat_plan* plan, int64_t n, int64_t nnz, const int64_t* rowptr,
                   const int32_t* colidx, int H, int D, int dtype, const void* Q, const void* K,
                   const void* V, void* out, float* lse, int use_tiles, void* stream)
{
    return gt_fwd_impl(plan, n, nnz, rowptr, colidx, H, D, dtype, Q, K, V, out, lse, nullptr,
                       0, true, use_tiles, static_cast<hipStream_t>(stream));
}

int gt_bwd(const sgat_plan* plan, int64_t n, int64_t nnz, const int64_t* rowptr,
           const int32_t* colidx, int H, int D, int dtype, const void* Q, const void* K,
           const void* V, const void* out, const float* lse, const void* dout, void* dQ, void* dK,
           void* dV, void* ws, size_t ws_bytes, int use_tiles, void* stream)
{
    int rc = check_common(plan, n, nnz, rowptr, colidx, H, D, dtype);
    if (rc) return rc;
    for (const void* t : {Q, K, V, out, dout, static_cast<const void*>(dQ),
                          static_cast<const void*>(dK), static_cast<const void*>(dV)})
        if ((rc = check_tensor(t, n))) return rc;
    if (n > 0 && (!lse || !aligned(lse, 4))) return SGAT_INVALID_ARGUMENT;
    if (use_tiles != 0 && use_tiles != 1) return SGAT_INVALID_ARGUMENT;
    if (use_tiles && (!plan->p.block_sparse || dtype != SGAT_BF16)) return SGAT_UNSUPPORTED;
    Layout L;
    if ((rc = check_ws(plan->p, SGAT_OP_GT_BWD, H, D, dtype, ws, ws_bytes, L))) return rc;
    if (n == 0) return SGAT_OK;
    if (use_tiles)
        return launch_gt_bs_bwd(plan->p, H, D, Q, K, V, out, lse, dout, dQ, dK, dV,
                                at<void>(ws, L.off[6]), at<void>(ws, L.off[7]),
                                static_cast<hipStream_t>(stream));
    BwdWs w{at<void>(ws, L.off[0]), at<float>(ws, L.off[1]), at<float>(ws, L.off[2]),
            at<float>(ws, L.off[3]), nullptr, at<float>(ws, L.off[4]), nullptr};
    return launch_gt_bwd(plan->p, H, D, dtype, colidx, Q, K, V, out, lse, dout, dQ, dK, dV, w,
                         static_cast<hipStream_t>(stream));
}

int gat_fwd(const sgat_plan* plan, int64_t n, int64_t nnz, const int64_t* rowptr,
            const int32_t* colidx, int H, int D, int dtype, const void* x_dst, const void* x_nbr,
            const float* a, float negative_slope, void* out, float* lse, void* ws,
            size_t ws_bytes, void* stream)
{
    int rc = check_common(plan, n, nnz, rowptr, colidx, H, D, dtype);
    if (rc) return rc;
    for (const void* t : {x_dst, x_nbr, static_cast<const void*>(out)})
        if ((rc = check_tensor(t, n))) return rc;
    if (n > 0 && (!lse || !aligned(lse, 4) || !a || !aligned(a, 16))) return SGAT_INVALID_ARGUMENT;
    if (!(negative_slope == negative_slope)) return SGAT_INVALID_ARGUMENT;   // NaN
    Layout L;
    if ((rc = check_ws(plan->p, SGAT_OP_GAT_FWD, H, D, dtype, ws, ws_bytes, L))) return rc;
    if (n == 0) return SGAT_OK;
    FwdWs w{at<float>(ws, L.off[0]), at<float>(ws, L.off[1])};
    return launch_gat_fwd(plan->p, H, D, dtype, colidx, x_dst, x_nbr, a, negative_slope, out,
                          lse, w, static_cast<hipStream_t>(stream));
}

int gat_bwd(const sgat_plan* plan, int64_t n, int64_t nnz, const int64_t* rowptr,
            const int32_t* colidx, int H, int D, int dtype, const void* x_dst, const void* x_nbr,
            const float* a, float negative_slope, const void* out, const float* lse,
            const void* dout, void* dx_dst, void* dx_nbr, float* da, void* ws, size_t ws_bytes,
            void* stream)
{
    int rc = check_common(plan, n, nnz, rowptr, colidx, H, D, dtype);
    if (rc) return rc;
    for (const void* t : {x_dst, x_nbr, out, dout, static_cast<const void*>(dx_dst),
                          static_cast<const void*>(dx_nbr)})
        if ((rc = check_tensor(t, n))) return rc;
    if (!da || !aligned(da, 4)) return SGAT_INVALID_ARGUMENT;
    if (n > 0 && (!lse || !aligned(lse, 4) || !a || !aligned(a, 16))) return SGAT_INVALID_ARGUMENT;
    if (!(negative_slope == negative_slope)) return SGAT_INVALID_ARGUMENT;
    Layout L;
    if ((rc = check_ws(plan->p, SGAT_OP_GAT_BWD, H, D, dtype, ws, ws_bytes, L))) return rc;
    if (n == 0) return launch_da_zero(da, H * D, static_cast<hipStream_t>(stream));
    BwdWs w{nullptr, at<float>(ws, L.off[1]), at<float>(ws, L.off[2]), nullptr,
            at<float>(ws, L.off[4]), nullptr, at<void>(ws, L.off[0])};
    return launch_gat_bwd(plan->p, H, D, dtype, colidx, x_dst, x_nbr, a, negative_slope, out, lse,
                          dout, dx_dst, dx_nbr, da, w, static_cast<hipStream_t>(stream));
}

int reduce_fwd(const sgat_plan* plan, int64_t n, int64_t nnz, const int64_t* rowptr,
               const int32_t* colidx, int F, int dtype, int op, const void* X, void* out,
               int32_t* arg, void* ws, size_t ws_bytes, void* stream)
{
    int rc = check_reduce(plan, n, nnz, rowptr, colidx, F, dtype);
    if (rc) return rc;
    if (op != SGAT_REDUCE_MIN && op != SGAT_REDUCE_MAX) return SGAT_INVALID_ARGUMENT;
    for (const void* t : {X, static_cast<const void*>(out)})
        if ((rc = check_tensor(t, n))) return rc;
    if (arg && !aligned(arg, 16)) return SGAT_INVALID_ARGUMENT;
    Layout L;
    if ((rc = check_ws(plan->p, SGAT_OP_REDUCE_FWD, 1, F, dtype, ws, ws_bytes, L))) return rc;
    if (n == 0) return SGAT_OK;
    return launch_reduce_fwd(plan->p, F, dtype, op, colidx, X, out, arg, at<float>(ws, L.off[0]),
                             at<int32_t>(ws, L.off[1]), static_cast<hipStream_t>(stream));
}

int reduce_bwd(const sgat_plan* plan, int64_t n, int64_t nnz, const int64_t* rowptr,
               const int32_t* colidx, int F, int dtype, const int32_t* arg, const void* dout,
               void* dX, void* ws, size_t ws_bytes, void* stream)
{
    int rc = check_reduce(plan, n, nnz, rowptr, colidx, F, dtype);
    if (rc) return rc;
    for (const void* t : {static_cast<const void*>(arg), dout, static_cast<const void*>(dX)})
        if ((rc = check_tensor(t, n))) return rc;
    Layout L;
    if ((rc = check_ws(plan->p, SGAT_OP_REDUCE_BWD, 1, F, dtype, ws, ws_bytes, L))) return rc;
    if (n == 0) return SGAT_OK;
    return launch_reduce_bwd(plan->p, F, dtype, rowptr, arg, dout, dX, at<float>(ws, L.off[0]),
                             at<uint32_t>(ws, L.off[1]), at<void>(ws, L.off[2]),
                             static_cast<hipStream_t>(stream));
}

int sgat_trace_enable(int on)
{
    g_trace = on != 0;
    return SGAT_OK;
}

int sgat_trace_only(const char* name)
{
    g_trace_only = name ? name : "";
    return SGAT_OK;
}

int sgat_trace_clear(void)
{
    g_used = 0;
    return SGAT_OK;
}

int sgat_trace_count(void) { return static_cast<int>(g_used); }

int sgat_trace_get(int index, char* name, size_t name_len, float* ms)
{
    if (index < 0 || static_cast<size_t>(index) >= g_used) return SGAT_INVALID_ARGUMENT;
    const TraceRec& r = g_recs[static_cast<size_t>(index)];
    if (name && name_len > 0) {
        std::strncpy(name, r.name.c_str(), name_len - 1);
        name[name_len - 1] = '\0';
    }
    if (ms) {
        float t = 0.f;
        if (hipEventElapsedTime(&t, r.start, r.stop) != hipSuccess) return SGAT_HIP_ERROR;
        *ms = t;
    }
    return SGAT_OK;
}

}  // extern "C"
