/*
 * velox_geometry.h — C ABI of the geometry scorer in libvelox.so: the slab
 * overlaps g and the coverage rho that the router consumes (velox.h,
 * velox_route_select).
 *
 * The method: "Velox: Spatial Memory Makes World Models Efficient". Pages:
 *   [digest]  paper digest (paper.rainbus.top): Prerequisites "frustum slab and
 *             OBB overlap"; Method steps, step 3 (eq. 7-8).
 *   [project] project page (velox-world.com/velox): 02 · Method, "What the
 *             router sees" (g is a world-space IoU of slabs).
 *   [onedev]  Korean summary (onedev.kr): "How it works" (OBB IoU first, then
 *             coverage from warped token depths; trust geometry at >= 90%).
 *
 * A slab — a block's token rectangle with its percentile depth interval — is
 * approximated by a camera-facing oriented box (OBB), passed as a float32
 * record of 16 words:
 *   [0..2]  centre (world)
 *   [3..5]  half-extents e0, e1, e2 along the box axes
 *   [6..14] axes, row-major 3x3: axis j (a world-space unit vector) is column j
 *   [15]    unused
 * A box is valid iff e0, e1, e2 > 0; an invalid box overlaps nothing and
 * covers nothing (a history block without reliable depth).
 *
 * Conventions are those of velox.h: device pointers, caller-owned memory, no
 * allocation, asynchronous on `stream`, host-side argument checks that return
 * VELOX_ERR_INVALID before any launch, VELOX_ERR_LAUNCH on launch failure.
 */
#ifndef VELOX_GEOMETRY_H
#define VELOX_GEOMETRY_H

#include "velox.h"

#ifdef __cplusplus
extern "C" {
#endif

#define VELOX_OBB_WORDS 16
#define VELOX_MAX_LATTICE 16

/*
 * velox_slab_overlap — g[i][r] = IoU of query box i with history box r
 * ([digest] Method steps, step 3, eq. 7; [project] "What the router sees").
 * The intersection volume is approximated on the n^3 cell-centre lattice of
 * the query box: lattice point (k0, k1, k2) sits at local offsets
 * e_j ((2 k_j + 1) / n - 1); I = vol(A) * (points inside B) / n^3 and
 * g = I / (vol(A) + vol(B) - I), g = 0 when no point is inside. Computed in
 * float32 with one rounding per operation in a fixed order, so the result is
 * a deterministic function of the records:
 *   world point   p = c_A + ((R_A[.,0] u0 + R_A[.,1] u1) + R_A[.,2] u2)
 *   local coord   l_j = (R_B[0,j] d0 + R_B[1,j] d1) + R_B[2,j] d2,  d = p - c_B
 *   inside        |l_j| <= e_B,j for j = 0, 1, 2
 *   volume        ((8 e0) e1) e2
 *   q_obb   [N][16] query-block boxes (current chunk)
 *   h_obb   [M][16] history-block boxes
 *   lattice n, 1 <= n <= VELOX_MAX_LATTICE (the pages' grid; 8 is the usual)
 *   g       [N][M] float32 (output), in [0, 1]
 * N, M >= 0 (nothing is launched when either is 0), N <= 65535.
 */
velox_status_t velox_slab_overlap(const float* q_obb, const float* h_obb, int N, int M,
                                  int lattice, float* g, void* stream);

/*
 * velox_slab_coverage — rho[i] = (tokens of query block i whose world point
 * lies inside at least one valid history box) / 128 ([digest] Method steps,
 * step 3, eq. 8; [onedev] "How it works"). The point of a token is its
 * multiwarp depth back-projected through the target camera; a token without
 * depth is passed as NaN and is never covered. The inside test is the one of
 * velox_slab_overlap (closed box, float32, same operation order).
 *   q_pts       [N][128][3] float32 token world points
 *   h_obb       [M][16] history-block boxes
 *   token_mask  [N][4] uint32 (output): bit (a % 32) of word a / 32 is set
 *               iff token a is covered
 *   rho         [N] float32 (output), a multiple of 1/128
 * N, M >= 0 (M = 0 gives rho = 0), N <= 65535.
 */
velox_status_t velox_slab_coverage(const float* q_pts, const float* h_obb, int N, int M,
                                   uint32_t* token_mask, float* rho, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* VELOX_GEOMETRY_H */
