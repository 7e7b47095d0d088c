/*
 * sgattn.h - fused sparse graph attention on AMD MI355X (gfx950), C ABI.
 *
 * The library computes the two attention-GNN layers named by
 *   "On Efficient Scaling of GNNs via IO-Aware Layers Implementations"
 *   (arXiv 2605.31500), Abstract: the attention-based layer family,
 *   GATv2 and Graph Transformer;
 * and by "DF-GNN: Dynamic Fusion Framework for Attention Graph Neural
 *   Networks on GPUs" (arXiv 2411.16127), Abstract: GAT and Graph Transformer
 *   executed as one fused kernel instead of separate kernels with heavy data
 *   movement between them.
 *
 * Each layer is edge scores (SDDMM), a per-destination softmax over the
 * in-neighbours, and an alpha-weighted aggregation of neighbour rows (SpMM),
 * evaluated in one pass with an online softmax so that no edge-level score or
 * weight is written to device memory; the backward recomputes the weights
 * from one log-sum-exp value per (node, head) (Yandex Research blog "On
 * efficient scaling of GNNs via IO-aware layer implementations", paragraph on
 * attention-based architectures). It also computes the reduction-based
 * aggregation family of the IO-aware layers paper (Abstract): min or max
 * pooling of the neighbour rows, reduce_fwd / reduce_bwd below.
 *
 * Conventions for every entry point:
 *   - Graph: CSR by destination. Row i holds edges e in [rowptr[i],
 *     rowptr[i+1]); colidx[e] = j is the source of the edge j -> i. rowptr is
 *     int64 [n+1], colidx int32 [nnz]. Repeated edges are separate softmax
 *     terms. Rows may be empty: their output is 0 and their lse is -inf.
 *   - Features: [n, H, D] row-major (node, head, channel), element type fp32
 *     or bf16, base address 16-byte aligned. H in 1..16, D in {32, 64, 128}.
 *     Accumulation is fp32; outputs and gradients are written in the input
 *     type, rounded to nearest even. lse is fp32 [n, H], natural log. (The
 *     aggregation takes [n, F] rows instead; see reduce_fwd.)
 *   - Graph capture: the compute calls allocate nothing, synchronise nothing
 *     and issue no memset, so a sequence of them can be captured into a HIP
 *     graph and replayed (same buffers, same plan).
 *   - Memory: every tensor, plan buffer and workspace pointer is a device
 *     pointer owned by the caller. The library never allocates or frees device
 *     memory. Host arrays given to sgat_plan_create are copied.
 *   - Streams: `stream` is a hipStream_t passed as void* (NULL = the default
 *     stream). All device work is enqueued on it; the library never
 *     synchronises. Device faults surface at the caller's next sync.
 *   - Every compute call repeats n and nnz; they must equal the plan's
 *     (SGAT_PLAN_MISMATCH otherwise). rowptr/colidx are the device copies of
 *     the arrays the plan was built from; their content is not re-checked.
 *   - Errors: every function returns an sgat_status. Arguments are checked on
 *     the host before any launch; on a non-zero status nothing was enqueued,
 *     except SGAT_HIP_ERROR, which reports a failed launch. No C++ exception
 *     crosses this interface.
 *   - Determinism: no floating-point atomics are used; for a fixed plan every
 *     output is bitwise reproducible run to run.
 *   - Concurrency: a plan is read-only after upload. Calls may share a plan
 *     on different streams if each has its own workspace and outputs.
 */
#ifndef SGATTN_H
#define SGATTN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum sgat_status {
    SGAT_OK = 0,
    SGAT_INVALID_ARGUMENT = 1,    /* null pointer, H/D/dtype unsupported, misaligned tensor */
    SGAT_INVALID_CSR = 2,         /* rowptr[0] != 0, rowptr not monotone, rowptr[n] != nnz,
                                     colidx outside [0, n) */
    SGAT_WORKSPACE_TOO_SMALL = 3, /* workspace or plan buffer smaller than required */
    SGAT_PLAN_MISMATCH = 4,       /* n or nnz differs from the plan's */
    SGAT_HIP_ERROR = 5,           /* a HIP call or kernel launch failed */
    SGAT_NOT_UPLOADED = 6,        /* plan used before sgat_plan_upload */
    SGAT_OUT_OF_HOST_MEMORY = 7,  /* host allocation inside sgat_plan_create failed */
    SGAT_UNSUPPORTED = 8,         /* option not available for this plan (e.g. no tiles built) */
    SGAT_SCRATCH_LIMIT = 9        /* gt_fwd_noalloc: the call needs more scratch than the
                                     library's static array holds */
} sgat_status;

typedef enum sgat_dtype { SGAT_F32 = 0, SGAT_BF16 = 1 } sgat_dtype;

typedef enum sgat_op {
    SGAT_OP_GT_FWD = 0,
    SGAT_OP_GT_BWD = 1,
    SGAT_OP_GAT_FWD = 2,
    SGAT_OP_GAT_BWD = 3,
    SGAT_OP_REDUCE_FWD = 4,   /* workspace queries pass H = 1 and D = F */
    SGAT_OP_REDUCE_BWD = 5
} sgat_op;

typedef enum sgat_reduce { SGAT_REDUCE_MIN = 0, SGAT_REDUCE_MAX = 1 } sgat_reduce;

/* Preprocessing options (0 selects the default for every field). */
typedef struct sgat_plan_opts {
    int64_t chunk;        /* A row (or, in the transposed CSR, a source) with more
                             than `chunk` edges is split into chunks of `chunk`
                             edges, each processed by its own wavefront and merged
                             afterwards in fixed order. Default 1024. */
    int32_t tile_min_nnz; /* A 16x16 block of the adjacency with at least this many
                             distinct edges becomes a dense tile. Default 32. */
    int32_t block_sparse; /* 1: also build the 16x16 tile layout and residual CSR. */
    int32_t locality;     /* 0: rows of a degree bin in ascending id; 1: in Cuthill-McKee
                             order of the undirected graph, so rows that share
                             neighbours run close together in time (more L2 reuse
                             of gathered rows). Results are the same up to rounding. */
    int32_t edge_order;   /* Where the Graph Transformer backward (gather path) keeps the
                             dS values its transposed-CSR pass hands to its CSR pass:
                             1 = CSR edge order (each edge's H floats written at its CSR
                             position: scattered small writes, contiguous reads);
                             2 = transposed order (written contiguously, read through
                             SGAT_ARR_ROW_TPOS); 0 = automatic: transposed when
                             nnz * H * 4 bytes exceed 128 MiB, about half the 256 MB
                             Infinity Cache, beyond which the scattered partial-line
                             writes reach HBM; CSR order otherwise. Results are bitwise
                             the same either way. */
} sgat_plan_opts;

/* Summary of a plan (all counts are exact). */
typedef struct sgat_plan_stats {
    int64_t n, nnz;
    int64_t chunk;
    int64_t max_in_degree, max_out_degree;
    int64_t row_items, row_splits, row_slots;   /* CSR work list                    */
    int64_t col_items, col_splits, col_slots;   /* transposed-CSR work list         */
    int64_t tiles, tile_edges, residual_edges;  /* block-sparse layout (0 if off)   */
    int64_t device_bytes;                       /* size of the uploaded plan buffer */
} sgat_plan_stats;

/* Arrays of a plan, for sgat_plan_array_bytes / sgat_plan_export. */
typedef enum sgat_array {
    SGAT_ARR_ROW_ITEMS = 0,   /* sgat_work_item[row_items]                              */
    SGAT_ARR_ROW_SPLITS = 1,  /* sgat_split[row_splits]                                 */
    SGAT_ARR_COLPTR = 2,      /* int64 [n+1]: transposed CSR (edges grouped by source)  */
    SGAT_ARR_ROWIDX = 3,      /* int32 [nnz]: destination of each edge, by source       */
    SGAT_ARR_COL_ITEMS = 4,   /* sgat_work_item[col_items]                              */
    SGAT_ARR_COL_SPLITS = 5,  /* sgat_split[col_splits]                                 */
    SGAT_ARR_TILE_ROWPTR = 6, /* int64 [ceil(n/16)+1]                                   */
    SGAT_ARR_TILE_COL = 7,    /* int32 [tiles]: 16-column block index of each tile      */
    SGAT_ARR_TILE_MASK = 8,   /* uint16 [tiles][16]: bit c of word r = edge
                                 (16*col+c) -> (16*row+r)                               */
    SGAT_ARR_RES_ROWPTR = 9,  /* int64 [n+1]: edges not covered by a dense tile         */
    SGAT_ARR_RES_COLIDX = 10, /* int32 [residual_edges]                                 */
    SGAT_ARR_TILE_ROW = 11,   /* int32 [tiles]: 16-row block index of each tile         */
    SGAT_ARR_TILE_COLPTR = 12,/* int64 [ceil(n/16)+1]: tiles grouped by block column    */
    SGAT_ARR_TILE_BYCOL = 13, /* int32 [tiles]: tile ids by block column, then row      */
    SGAT_ARR_RES_COLPTR = 14, /* int64 [n+1]: residual edges grouped by source          */
    SGAT_ARR_RES_ROWIDX = 15, /* int32 [residual_edges]: their destinations             */
    SGAT_ARR_COL_EDGE = 16,   /* int32 [nnz]: CSR edge id of each transposed-CSR entry  */
    SGAT_ARR_RES_COL_EDGE = 17,/* int32 [residual_edges]: residual-CSR edge id of each
                                 transposed residual entry                              */
    SGAT_ARR_ROW_TPOS = 18,   /* int32 [nnz]: transposed-CSR position of each CSR edge
                                 (the inverse of SGAT_ARR_COL_EDGE); built for
                                 edge_order 2, and for 0 when nnz > 2^21; else empty     */
    SGAT_ARR_RES_ROW = 19,    /* int32 [residual_edges]: destination of each residual edge */
    SGAT_ARR_RES_COLSRC = 20, /* int32 [residual_edges]: source of each transposed
                                 residual entry                                         */
    SGAT_ARR_TILE_ROW_BYCOL = 21,/* int32 [tiles]: block row of the tiles in
                                 SGAT_ARR_TILE_BYCOL order                              */
    SGAT_ARR_COUNT = 22
} sgat_array;

/* One unit of work of the gather kernels: `len` consecutive edges starting at
 * edge offset `begin` of row (or source) `row`. slot < 0: the item covers the
 * whole row and writes the final result; slot >= 0: the row is split and the
 * item writes partial state into workspace slot `slot`. flags bit 0: first
 * chunk of its row. */
typedef struct sgat_work_item {
    int64_t begin;
    int32_t len;
    int32_t row;
    int32_t slot;
    int32_t flags;
} sgat_work_item;

/* A split row: its chunks own slots [first_slot, first_slot + nslots). */
typedef struct sgat_split {
    int32_t row;
    int32_t first_slot;
    int32_t nslots;
    int32_t reserved;
} sgat_split;

typedef struct sgat_plan sgat_plan;

/* ---- plan: preprocessing on the host (integer only, deterministic) -------- */

/* Validate the CSR (n >= 0, nnz >= 0, n < 2^31, nnz < 2^31 (edge positions
 * are stored as int32), rowptr[0] = 0, rowptr monotone,
 * rowptr[n] = nnz, 0 <= colidx < n) and build the plan: degree-binned work
 * lists for the CSR and for its transpose, with heavy rows and heavy sources
 * split into chunks (degree-aware parallelisation of high-degree nodes: Yandex
 * Research blog, paragraph on aggregation layers; super nodes: DF-GNN,
 * Abstract), the transposed CSR itself, and with opts->block_sparse the 16x16
 * tile layout plus residual CSR (block-sparse representation for locally dense
 * graphs: blog, paragraph on attention-based architectures). `opts` may be
 * NULL. On success *out owns a host copy of everything; no HIP call is made.
 * Returns SGAT_INVALID_ARGUMENT (null pointer, bad option), SGAT_INVALID_CSR or
 * SGAT_OUT_OF_HOST_MEMORY; *out is then NULL. */
int sgat_plan_create(int64_t n, int64_t nnz, const int64_t* rowptr, const int32_t* colidx,
                     const sgat_plan_opts* opts, sgat_plan** out);

/* Bytes of device memory the caller must provide to sgat_plan_upload. */
int sgat_plan_device_bytes(const sgat_plan* plan, size_t* bytes);

/* Copy the plan's arrays into the caller-owned device buffer `dev_buf` (256-byte
 * aligned, at least sgat_plan_device_bytes) on `stream`. The buffer must stay
 * alive and unmodified for as long as the plan is used. */
int sgat_plan_upload(sgat_plan* plan, void* dev_buf, size_t bytes, void* stream);

int sgat_plan_stats_get(const sgat_plan* plan, sgat_plan_stats* stats);

/* Size in bytes of one plan array, and a host copy of it (for tests). */
int sgat_plan_array_bytes(const sgat_plan* plan, int array_id, size_t* bytes);
int sgat_plan_export(const sgat_plan* plan, int array_id, void* host_dst, size_t bytes);

/* Frees the host side of the plan (never the caller's device buffer). NULL is a no-op. */
void sgat_plan_destroy(sgat_plan* plan);

/* Workspace bytes that `op` needs for this plan, H, D and dtype (for the
 * reduction ops H = 1 and D = F). */
int sgat_workspace_bytes(const sgat_plan* plan, int op, int H, int D, int dtype, size_t* bytes);

/* ---- Graph Transformer: score s_ij = <Q_i, K_j> / sqrt(D) ------------------- */

/* Forward: out_i = sum_j alpha_ij V_j with alpha = softmax over the in-edges
 * of i of s_ij; lse_i = ln sum_j exp(s_ij). One fused pass with an online
 * softmax; rows longer than the plan's chunk are split across wavefronts and
 * their partial (max, sum, accumulator) merged by log-sum-exp in fixed order.
 * Q, K, V, out: [n,H,D]; lse: fp32 [n,H]. With use_tiles = 1 (plan built with
 * block_sparse) the dense 16x16 tiles run on bf16 matrix cores and the rest on
 * the gather path; requires dtype = bf16. */
int gt_fwd(const sgat_plan* plan, int64_t n, int64_t nnz,
           const int64_t* rowptr, const int32_t* colidx,
           int H, int D, int dtype, const void* Q, const void* K, const void* V,
           void* out, float* lse, void* ws, size_t ws_bytes, int use_tiles, void* stream);

/* gt_fwd without a workspace argument, for callers that cannot allocate
 * device memory (code under HIP graph capture, tight serving loops, harnesses
 * that forbid hipMalloc). It runs the same kernels as gt_fwd, with the
 * partial results of split rows in a static device array of
 * SGAT_NOALLOC_SCRATCH_BYTES that the library owns; each GPU the library runs
 * on holds one such array until the process ends. The first call on a device
 * looks the array's address up there (hipGetSymbolAddress, no allocation);
 * no call allocates or frees anything. Every call on one GPU shares that GPU's
 * array, so calls that overlap in time on one GPU (on different streams, or
 * from several threads) race on it and must be serialised by the caller. No
 * region of it needs to start at zero (each chunk writes its own slot before
 * the merge reads it). Arguments and results are those of gt_fwd; a call
 * whose gt_fwd workspace (sgat_workspace_bytes, SGAT_OP_GT_FWD) would exceed
 * SGAT_NOALLOC_SCRATCH_BYTES returns SGAT_SCRATCH_LIMIT and enqueues nothing. */
#define SGAT_NOALLOC_SCRATCH_BYTES ((size_t)32 << 20)
int gt_fwd_noalloc(const sgat_plan* plan, int64_t n, int64_t nnz,
                   const int64_t* rowptr, const int32_t* colidx,
                   int H, int D, int dtype, const void* Q, const void* K, const void* V,
                   void* out, float* lse, int use_tiles, void* stream);

/* Backward of L = sum(out * dout): dQ, dK, dV. Recomputes alpha_ij from lse
 * (the forward's output); nothing per edge is kept from the forward.
 * Delta_i = dout_i . out_i per head; dS_ij = alpha_ij (dout_i . V_j - Delta_i).
 * The transposed-CSR pass computes dK, dV and dS, leaving dS per (edge, head)
 * in the workspace; the CSR pass then accumulates dQ from it, so no atomics are
 * needed. With use_tiles = 1 the order is reversed: the tile-row pass computes
 * dQ and leaves P and dS per edge for the tile-column pass (dK, dV).
 * All gradients are overwritten (not accumulated into). */
int gt_bwd(const sgat_plan* plan, int64_t n, int64_t nnz,
           const int64_t* rowptr, const int32_t* colidx,
           int H, int D, int dtype, const void* Q, const void* K, const void* V,
           const void* out, const float* lse, const void* dout,
           void* dQ, void* dK, void* dV, void* ws, size_t ws_bytes, int use_tiles, void* stream);

/* ---- GATv2: score e_ij = sum_d a[h,d] LeakyReLU(x_dst[i,h,d] + x_nbr[j,h,d]) -- */

/* Forward: out_i = sum_j alpha_ij x_nbr[j], softmax over the in-edges of i.
 * x_dst is indexed by the destination i, x_nbr gathered by the neighbour j
 * (read once per edge for both score and value). a: fp32 [H,D].
 * negative_slope: LeakyReLU slope for z <= 0 (0.2 in GATv2). */
int gat_fwd(const sgat_plan* plan, int64_t n, int64_t nnz,
            const int64_t* rowptr, const int32_t* colidx,
            int H, int D, int dtype, const void* x_dst, const void* x_nbr,
            const float* a, float negative_slope,
            void* out, float* lse, void* ws, size_t ws_bytes, void* stream);

/* Backward of L = sum(out * dout): dx_dst, dx_nbr (input dtype, [n,H,D]) and
 * da (fp32 [H,D]), all overwritten. The CSR pass recomputes alpha_ij from lse,
 * accumulates dx_dst, and leaves per edge the weight, dE_ij = alpha_ij
 * (dout_i . x_nbr[j] - Delta_i) and the signs of z in the workspace; the
 * transposed-CSR pass reads them and gathers only dout_i for dx_nbr. da splits
 * into per-node terms (sum_i x_dst[i] . T_i + sum_j x_nbr[j] . U_j, T and U the
 * sums of dE times LeakyReLU'(z) the two passes form anyway); both passes write
 * them as per-workgroup partials, reduced in fixed order. */
int gat_bwd(const sgat_plan* plan, int64_t n, int64_t nnz,
            const int64_t* rowptr, const int32_t* colidx,
            int H, int D, int dtype, const void* x_dst, const void* x_nbr,
            const float* a, float negative_slope,
            const void* out, const float* lse, const void* dout,
            void* dx_dst, void* dx_nbr, float* da, void* ws, size_t ws_bytes, void* stream);

/* ---- min/max aggregation: out[i,f] = min or max over edges j -> i of X[j,f] -- */

/* Reduction-based aggregation (IO-aware layers abstract: the reduction kernel
 * family; Yandex Research blog, paragraph on aggregation layers: min/max
 * pooling, with degree-aware parallelisation of high-degree nodes). The
 * message of edge j -> i is the source row X[j]; op = SGAT_REDUCE_MIN or
 * SGAT_REDUCE_MAX. X and out: [n, F] row-major, fp32 or bf16, 16-byte aligned;
 * F a multiple of 4 (fp32) or 8 (bf16), at most 2048. Comparisons are exact,
 * so out holds the input bits of the winning edge: the first CSR position of
 * the row attaining the extreme (ties go to the lowest position). arg, if not
 * NULL: int32 [n, F], 16-byte aligned, receives that position, -1 for empty
 * rows (whose out is 0). Rows longer than the plan's chunk are split across
 * wavefronts and their partial winners combined in chunk order. NaN inputs
 * give unspecified results. */
int reduce_fwd(const sgat_plan* plan, int64_t n, int64_t nnz,
               const int64_t* rowptr, const int32_t* colidx,
               int F, int dtype, int op, const void* X, void* out, int32_t* arg,
               void* ws, size_t ws_bytes, void* stream);

/* Backward of L = sum(out * dout): dX[j,f] = sum of dout[i,f] over the (i, f)
 * whose winner arg[i,f] is an edge j -> i. arg is the reduce_fwd output for
 * this plan and F (its content is not re-checked); dout and dX [n, F] in the
 * dtype, dX overwritten. Accumulated over the transposed CSR in fixed order
 * (sources with many out-edges split and summed in chunk order), so no
 * atomics are used. */
int reduce_bwd(const sgat_plan* plan, int64_t n, int64_t nnz,
               const int64_t* rowptr, const int32_t* colidx,
               int F, int dtype, const int32_t* arg, const void* dout, void* dX,
               void* ws, size_t ws_bytes, void* stream);

/* ---- diagnostics ----------------------------------------------------------- */

const char* sgat_status_string(int status);

/* Kernel timing trace. While enabled, every kernel the library launches is
 * bracketed by two HIP events recorded on the launch stream. After the caller
 * has synchronised the stream, sgat_trace_count / sgat_trace_get return the
 * kernel names and elapsed milliseconds in launch order. Off by default;
 * enabling it changes no result, but each event pair adds a few microseconds
 * between kernels. sgat_trace_only(name) restricts the trace to the kernels
 * of that name (as sgat_trace_get reports it; the string is copied), and
 * sgat_trace_only(NULL) or "" restores every kernel. Not thread-safe. */
int sgat_trace_enable(int on);
int sgat_trace_only(const char* name);
int sgat_trace_clear(void);
int sgat_trace_count(void);
int sgat_trace_get(int index, char* name, size_t name_len, float* ms);

/* Bandwidth probes (measurement only; they compute nothing of the layers).
 * sgat_probe_read streams `bytes` (a multiple of 16, src 16-byte aligned) of
 * device memory with `blocks` workgroups of 256 lanes, each lane reading 16
 * bytes per access. sgat_probe_gather reads whole rows of a row-major table of
 * `rows` rows of `row_bytes` bytes (256, 512 or 1024; table 16-byte aligned) at
 * the n_idx row indices idx (device int32; indices outside [0, rows) read
 * nothing), 16 KiB in flight per wave like the attention forward's neighbour
 * gathers. `sink` is a device uint32 that the probes leave unwritten in
 * practice (a data-dependent store keeps the loads from being removed). Both
 * launch through the timing trace as "probe_read" / "probe_gather", so the
 * achieved rate is bytes / traced time. */
int sgat_probe_read(const void* src, size_t bytes, uint32_t* sink, int blocks, void* stream);
int sgat_probe_gather(const void* table, int64_t rows, int row_bytes, const int32_t* idx,
                      int64_t n_idx, uint32_t* sink, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* SGATTN_H */
