/*
 * velox.h — C ABI of the routed block-sparse history attention library
 * (libvelox.so, HIP for gfx950 / MI355X).
 *
 * The method: "Velox: Spatial Memory Makes World Models Efficient". Pages:
 *   [digest]  paper digest (paper.rainbus.top): Prerequisites, Core method,
 *             Method steps (eq. 9-15).
 *   [project] project page "Velox: Spatial Memory Makes Long-context World
 *             Models Efficient" (velox-world.com/velox): 02 · Method.
 *   [onedev]  Korean summary (onedev.kr): "What differs", "How to use".
 *
 * One attention call of one layer, per head h and query block i of the
 * current chunk:
 *   1. importance p[h][i][r] over the M visible history blocks   (route_scores)
 *   2. fused, coverage-gated route with reservation + safeguards (route_select)
 *   3. attention over the routed history tiles + current chunk    (sparse_attn)
 * plus a dense baseline over every tile (dense_attn) and the block-mean
 * helper that fills the per-block key-mean cache (block_mean).
 *
 * Conventions for every entry point:
 *   - A block is VELOX_BLOCK = 128 consecutive tokens; it is both the routing
 *     unit and the attention tile ([project] "Why the route is a block").
 *   - Block ids are the global (Gilbert) order of the KV cache: history blocks
 *     are 0 .. M-1, the current chunk's N blocks are M .. M+N-1, stored in the
 *     same k / v tensors ([onedev] "How to use": KV stored in the routes'
 *     global Gilbert order).
 *   - Pointers are DEVICE pointers unless stated; the caller owns all memory.
 *     The library allocates nothing, keeps no state between calls and is
 *     reentrant. Every call is asynchronous on `stream` (a hipStream_t; NULL is
 *     the default stream).
 *   - Row-major layouts; "ld_*_h" is a head stride in ELEMENTS; token rows are
 *     contiguous with d elements each.
 *   - Arguments are checked on the host before any launch. A failed check
 *     returns VELOX_ERR_INVALID (or VELOX_ERR_UNSUPPORTED for a valid request
 *     outside the supported envelope) and launches nothing; the message is
 *     available from velox_last_error(). Launch failures return
 *     VELOX_ERR_LAUNCH. No C++ exception crosses this interface.
 *   - Supported: d in {64, 128}; dtype VELOX_F32 or VELOX_BF16 (bf16 storage,
 *     fp32 accumulation and softmax); M <= VELOX_MAX_HISTORY.
 */
#ifndef VELOX_H
#define VELOX_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define VELOX_BLOCK 128
#define VELOX_MAX_HISTORY 16384

typedef enum {
  VELOX_OK = 0,
  VELOX_ERR_INVALID = 1,
  VELOX_ERR_UNSUPPORTED = 2,
  VELOX_ERR_LAUNCH = 3
} velox_status_t;

typedef enum { VELOX_F32 = 0, VELOX_BF16 = 1 } velox_dtype_t;

/* Router settings (host struct). Defaults from the pages ([digest] Core method;
 * [onedev] "What differs"): tau 0.1, g_ref 0.2, lambda 2, eta_cov 0.9,
 * K_cov 80, K_unc 150. */
typedef struct {
  float tau;        /* overlap noise threshold: ghat = 0 unless g > tau           */
  float g_ref;      /* overlap normaliser: ghat = min(g / g_ref, 1), g_ref > 0    */
  float lambda;     /* fusion strength, 0 <= lambda <= 14: w = p * (1 + lambda*ghat) */
  float eta_cov;    /* coverage gate: row i is covered iff rho[i] >= eta_cov      */
  float theta_cov;  /* mass threshold of covered rows; >= 1 disables the cut      */
  float theta_unc;  /* mass threshold of uncovered rows; >= 1 disables the cut    */
  int32_t K_cov;    /* cap of covered rows (>= 0), reservation included          */
  int32_t K_unc;    /* cap of uncovered rows (>= 0), reservation included        */
  int32_t n_prev;   /* history ids M-n_prev .. M-1 are always kept (0..M)         */
  int32_t neigh26;  /* 1: add history blocks at Chebyshev distance 1 from the
                       query block in the coord grid, outside the budget          */
  const int32_t* ref_ids; /* DEVICE, n_ref extra always-added ids (outside the
                             budget); ids outside [0, M) are ignored; may be NULL
                             when n_ref == 0                                        */
  int32_t n_ref;
  int32_t mode;     /* weights of a COVERED row (uncovered rows always use p):
                       VELOX_ROUTE_FUSED (0, the method), VELOX_ROUTE_MODEL_ONLY
                       (1, w = p with the same budgets: the matched model-only
                       block-sparse route), VELOX_ROUTE_GEOMETRY_ONLY (2, w = g,
                       plain top-K_cov with no mass cut: hard geometric top-K) */
  int32_t* status;  /* DEVICE int32[2] or NULL: input report of velox_route_select
                       (see there); status[0] = rows with bad inputs, status[1] =
                       the smallest such row h*N + i, or H*N when there is none */
} velox_route_params_t;

#define VELOX_ROUTE_FUSED 0
#define VELOX_ROUTE_MODEL_ONLY 1
#define VELOX_ROUTE_GEOMETRY_ONLY 2

/* Message for the last non-OK status returned on this host thread. */
const char* velox_last_error(void);

/* Library version: major * 10000 + minor * 100 + patch. */
int velox_version(void);

/*
 * velox_block_mean — xbar[h][b][:] = mean of tokens b*128 .. b*128+127 of x[h].
 * The per-block means of the pages' importance ([digest] Method steps, step 4,
 * eq. 9: mean query and mean key of a block). Used to fill the key-mean cache
 * when a chunk joins the history (a finished chunk's keys never change).
 *   x     [H][nblk*128][d], dtype dt, head stride ld_x_h (>= nblk*128*d);
 *         x and ld_x_h in bytes must be multiples of 16
 *   xbar  [H][nblk][d] fp32, head stride ld_bar_h (>= nblk*d)
 * nblk >= 0 (0: no-op).
 */
velox_status_t velox_block_mean(const void* x, velox_dtype_t dt, int64_t ld_x_h, int H,
                                int nblk, int d, float* xbar, int64_t ld_bar_h,
                                void* stream);

/*
 * velox_route_scores — block importance ([digest] Method steps, step 4, eq. 9;
 * [onedev] "What differs": softmax of the mean query . mean key inner product).
 *   p[h][i][r] = softmax_r( scale * qbar[h][i] . kbar[h][r] ),  r in [0, M)
 * with qbar the block means of q computed inside the call (fp32 accumulation).
 *   q     [H][N*128][d], dtype dt, head stride ld_q_h (>= N*128*d)
 *   kbar  [H][>=M][d] fp32 key-mean cache, head stride ld_kbar_h (>= M*d)
 *         q, kbar and both head strides in bytes must be multiples of 16
 *   p     [H][N][M] fp32, contiguous (output)
 * scale is normally 1/sqrt(d). M == 0 writes nothing.
 */
velox_status_t velox_route_scores(const void* q, velox_dtype_t dt, int64_t ld_q_h,
                                  const float* kbar, int64_t ld_kbar_h, int H, int N,
                                  int M, int d, float scale, float* p, void* stream);

/*
 * velox_route_scores_shared — one importance per layer instead of per head
 * ([digest] Method steps, step 4 and [onedev] "What differs" index the
 * importance p^l by layer only): p[i][r] = softmax over r of the mean over
 * heads of scale * qbar_h . kbar_h (the head-mean of velox_route_scores'
 * logits; ascending heads, then one division by H).
 *   logits  [H][N][M] fp32 workspace, overwritten with the per-head scaled
 *           logits (caller-owned)
 *   p       [N][M] fp32 (output)
 * Other arguments as velox_route_scores. Feed p to velox_route_select with
 * H = 1 and the routes to velox_sparse_attn_shared.
 */
velox_status_t velox_route_scores_shared(const void* q, velox_dtype_t dt, int64_t ld_q_h,
                                         const float* kbar, int64_t ld_kbar_h, int H, int N, int M,
                                         int d, float scale, float* logits, float* p,
                                         void* stream);

/*
 * velox_route_select — route materialisation ([project] 02 · Method, fusion
 * formula and "Covered and uncovered blocks"; [digest] Core method and Method
 * steps, step 4, eq. 10-14; [onedev] "What differs").
 * Per (h, i), in IEEE fp32 without contraction:
 *   ghat = (g > tau) ? min(g / g_ref, 1) : 0
 *   w    = (rho[i] >= eta_cov) ? p * (1 + lambda * ghat) : p
 * (covered rows under prm->mode = VELOX_ROUTE_MODEL_ONLY take w = p, under
 * VELOX_ROUTE_GEOMETRY_ONLY w = g with no mass cut; [project] 03 · Results
 * compares the method with a matched model-only block-sparse route, and
 * [digest] Prerequisites contrasts soft fusion with hard geometric top-K)
 * Mass in fixed point: W = floor(w * 2^60), Z = sum_r W.
 * Route = reserved {M-n_prev .. M-1}, then the other blocks in order of w
 * (descending; equal w by ascending id) while |route| < K and, if theta < 1,
 * while  m * 2^24 < floor(theta * 2^24) * Z  (m = mass of the route so far);
 * K, theta are the covered or uncovered values. Safeguards (neighbours, ref
 * ids) are then added outside the budget; ids are emitted ascending.
 *   p         [H][N][M] fp32 (normally route_scores' output)
 *   g         [N][M] fp32 overlaps, shared by heads
 *   rho       [N] fp32 coverage
 *   coord     [M+N][3] int32 (t, h, w) block-grid cells; may be NULL unless
 *             prm->neigh26. Cells should be distinct.
 *   prm       HOST pointer
 *   route_ids [H][N][L] int32 (output), unused slots = -1
 *   route_len [H][N] int32 (output)
 * L must be >= min(M, max(K_cov, K_unc, n_prev) + 26*neigh26 + n_ref) and >= 1.
 * (With duplicated cells a row could exceed this; it is then cut to its L
 * smallest ids.)
 * Input preconditions, checked on the device per row: every p entry finite and
 * >= 0, every g entry in [0, 1], and, on a row with a mass cut (theta < 1),
 * a fixed-point total Z < 2^64 (guaranteed when the row of p sums to at most
 * 1 + 2^-10, since lambda <= 14). A row that breaks one is counted in
 * prm->status when that pointer is non-NULL (the call clears it first, with a
 * launch of its own); its route is still ascending, unique and in [0, M), but
 * computed from saturated masses, so it carries no meaning. The call itself
 * returns VELOX_OK: the check runs asynchronously on the device.
 */
velox_status_t velox_route_select(const float* p, const float* g, const float* rho,
                                  const int32_t* coord, int H, int N, int M,
                                  const velox_route_params_t* prm, int L,
                                  int32_t* route_ids, int32_t* route_len, void* stream);

/*
 * velox_route_check — checks what the attention calls assume of a route
 * ([digest] Method steps, step 4: a route is a set of history block ids,
 * emitted ascending): for every row, 0 <= route_len <= L and the first
 * route_len ids strictly ascending and in [0, M). The attention kernels do
 * not check this (they clamp ids into range); this call is the check for
 * routes built outside velox_route_select. Asynchronous on `stream`.
 *   route_ids [rows][L], route_len [rows] int32 (rows = H*N, or N for shared
 *             routes)
 *   bad       device int32[2] (output): bad[0] = number of invalid rows,
 *             bad[1] = smallest invalid row index, or rows when none
 */
velox_status_t velox_route_check(const int32_t* route_ids, const int32_t* route_len, int rows,
                                 int M, int L, int32_t* bad, void* stream);

/*
 * velox_sparse_attn — indexed block-sparse attention ([digest] Core method,
 * eq. 15; Prerequisites: skipping a tile skips both its QK^T product and its
 * K/V load). For each (h, i) and each query row a of block i:
 *   o[h][i*128+a] = softmax_b( scale * q_a . k_b ) v_b
 * over the tokens b of the routed history tiles route_ids[h][i][0 .. len-1]
 * (len = clamp(route_len[h][i], 0, L)) followed, if include_current, by the
 * current chunk's tiles M .. M+N-1. Route ids must be ascending, unique and
 * in [0, M) (velox_route_select emits them so); the kernels do not check
 * this, but clamp an id outside [0, M) into that range so that no load leaves
 * the history (such an id then names the nearest valid tile).
 *   q        [H][N*128][d], head stride ld_q_h
 *   k, v     [H][>=(M+N)*128][d], head stride ld_kv_h
 *   o        [H][N*128][d] dtype dt, contiguous (output)
 *   lse      [H][N*128] fp32 natural-log sum of exp of the scaled logits
 *            (output, may be NULL)
 * A row with no tile at all gets o = 0 and lse = -inf.
 *   workspace  device buffer of at least velox_sparse_attn_workspace_size(H, N,
 *              L, d) bytes, 16-byte aligned, caller-owned, contents undefined
 *              on return; the call writes its unit schedule there (which pairs
 *              of rows share a workgroup and in which order the workgroups take
 *              them: rows of a head ranked by route length, each XCD's units
 *              longest first), computed on the device by a first launch. NULL
 *              is accepted: every workgroup then ranks the units itself
 *              (slower start). Only the d = 128 bf16 kernel reads it. Two calls
 *              that share a workspace must not overlap in time.
 */
velox_status_t velox_sparse_attn(const void* q, const void* k, const void* v,
                                 velox_dtype_t dt, int64_t ld_q_h, int64_t ld_kv_h, int H,
                                 int N, int M, int d, float scale, const int32_t* route_ids,
                                 const int32_t* route_len, int L, int include_current,
                                 void* o, float* lse, void* workspace, void* stream);

/* Bytes of the workspace of velox_sparse_attn: 16 per (head, pair of query
 * blocks), i.e. 16 * H * ceil(N / 2); 0 for H < 1, N < 1, L < 1 or d < 1. */
size_t velox_sparse_attn_workspace_size(int H, int N, int L, int d);

/*
 * velox_sparse_attn_noalloc — velox_sparse_attn for callers that cannot
 * allocate device memory: code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc. Same arguments and results as
 * velox_sparse_attn without the workspace: the unit schedule goes to a fixed
 * array in the library's device memory (VELOX_NOALLOC_MAX_UNITS entries of 16
 * bytes = 1 MiB per device, held until the process ends; its address is
 * resolved once per device, on the first call with that device current).
 * The call allocates nothing and calls no allocating routine.
 * Limit: H * ceil(N / 2) <= VELOX_NOALLOC_MAX_UNITS, else VELOX_ERR_UNSUPPORTED
 * (checked on the host, nothing launched). Every call on a device shares that
 * device's array: two calls on one device that overlap in time (different
 * streams, or host threads) race and must not be issued. Nothing in the
 * array needs clearing: each call writes every entry it reads.
 */
#define VELOX_NOALLOC_MAX_UNITS 65536
velox_status_t velox_sparse_attn_noalloc(const void* q, const void* k, const void* v,
                                         velox_dtype_t dt, int64_t ld_q_h, int64_t ld_kv_h, int H,
                                         int N, int M, int d, float scale,
                                         const int32_t* route_ids, const int32_t* route_len,
                                         int L, int include_current, void* o, float* lse,
                                         void* stream);

/*
 * velox_dense_attn — the dense baseline ([digest] Prerequisites: dense
 * FlashAttention schedules every current-history tile pair). Same as
 * velox_sparse_attn with every history tile routed and include_current = 1.
 */
velox_status_t velox_dense_attn(const void* q, const void* k, const void* v,
                                velox_dtype_t dt, int64_t ld_q_h, int64_t ld_kv_h, int H,
                                int N, int M, int d, float scale, void* o, float* lse,
                                void* stream);

/*
 * Split rows: velox_sparse_attn_split and velox_dense_attn_split compute the
 * same attention as velox_sparse_attn / velox_dense_attn ([digest] Core
 * method, eq. 15); the difference is only the work distribution. The tile list
 * of every query row (current chunk, then the routed tiles) is cut into
 * consecutive ranges, each handled by its own workgroup; the ranges'
 * unnormalised outputs and softmax (max, sum) go to the workspace and a second
 * kernel merges them (softmax is associative under rescaling). The dense call
 * cuts every row into n_split ranges. The sparse call cuts each pair of rows
 * that share a workgroup into at most n_split ranges, as many as the pairs of
 * an XCD need to fill one round of its 32 CUs with ranges of about equal
 * length (decided on the device from route_len, in the unit schedule); when an
 * XCD has more pairs than CUs nothing is cut. Meant for shapes with few rows
 * per GPU, e.g. one GPU's share of the heads (5 heads x 36 query blocks = 180
 * rows for 256 CUs). Results equal the unsplit call's up to float rounding.
 *   n_split          1 .. VELOX_MAX_SPLIT; 1 is the unsplit call
 *   workspace        device buffer, 16-byte aligned, of at least
 *                    velox_attn_split_workspace_size(H, N, n_split) bytes
 *                    (partial outputs, then, for routed calls, the unit
 *                    schedule as in velox_sparse_attn), caller-owned; contents
 *                    undefined on return; may be NULL when n_split = 1
 *   workspace_bytes  its size
 * Other arguments as for the unsplit calls. Rows are split only by the d = 128
 * bf16 kernel with routes of at most 2048 tiles; other shapes run unsplit and
 * leave the workspace untouched. Two calls that share a workspace must not
 * overlap in time.
 */
#define VELOX_MAX_SPLIT 16
size_t velox_attn_split_workspace_size(int H, int N, int n_split);
velox_status_t velox_sparse_attn_split(const void* q, const void* k, const void* v,
                                       velox_dtype_t dt, int64_t ld_q_h, int64_t ld_kv_h, int H,
                                       int N, int M, int d, float scale,
                                       const int32_t* route_ids, const int32_t* route_len, int L,
                                       int include_current, int n_split, void* workspace,
                                       size_t workspace_bytes, void* o, float* lse, void* stream);
velox_status_t velox_dense_attn_split(const void* q, const void* k, const void* v,
                                      velox_dtype_t dt, int64_t ld_q_h, int64_t ld_kv_h, int H,
                                      int N, int M, int d, float scale, int n_split,
                                      void* workspace, size_t workspace_bytes, void* o,
                                      float* lse, void* stream);

/*
 * velox_sparse_attn_shared — velox_sparse_attn with one route per query block
 * shared by every head (routes of velox_route_scores_shared):
 *   route_ids  [N][L] int32, route_len [N] int32
 * Everything else as velox_sparse_attn.
 */
velox_status_t velox_sparse_attn_shared(const void* q, const void* k, const void* v,
                                        velox_dtype_t dt, int64_t ld_q_h, int64_t ld_kv_h, int H,
                                        int N, int M, int d, float scale,
                                        const int32_t* route_ids, const int32_t* route_len, int L,
                                        int include_current, void* o, float* lse, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* VELOX_H */
