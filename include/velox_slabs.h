/*
 * velox_slabs.h — C ABI of the slab table and the recency-priority multiwarp
 * in libvelox.so: the geometry that turns reconstructed depth into the boxes
 * and token points the overlap scorer (velox_geometry.h) consumes.
 *
 * The method: "Velox: Spatial Memory Makes World Models Efficient". Pages:
 *   [digest]  paper digest (paper.rainbus.top): Prerequisites ("frustum slab",
 *             "recency-priority multiwarp"); Method steps 1-2 (eq. 4-6).
 *   [onedev]  Korean summary (onedev.kr): "How it works" (percentile depth
 *             interval per block fragment; warped first/last-frame depths;
 *             median of the newest frame whose sample count clears the bound).
 *
 * Camera model (pinhole in token units; both the latent camera of a chunk and
 * the cached depth frames use it): a camera is float32[12], R row-major (9)
 * then centre c (3), with world = c + R * camera; camera axes x right, y up,
 * z forward. Token cell (col, row) has centre (col + 0.5, row + 0.5); the ray
 * through (u, v) is ((u - cx) / f, (cy - v) / f, 1). A depth is reliable iff
 * it is finite and > 0. Every decision and output is float32 with one
 * rounding per operation in this order:
 *   point       X_r = c_r + ((R_r0 (z rx) + R_r1 (z ry)) + R_r2 z)
 *   projection  d = X - c_t;  p_j = (R_0j d0 + R_1j d1) + R_2j d2;
 *               u' = (f p0) / p2 + cx,  v' = cy - (f p1) / p2
 *   percentile  h = (n - 1) p, i = floor(h), q = x_i + (h - i)(x_{i+1} - x_i)
 *   box         centre = point of the rectangle centre at zm = (zlo + zhi) / 2,
 *               e0 = (zm (u1 - u0)) / (2 f), e1 = (zm (v1 - v0)) / (2 f),
 *               e2 = (zhi - zlo) / 2, axes = the camera axes
 * Conventions otherwise as velox.h.
 */
#ifndef VELOX_SLABS_H
#define VELOX_SLABS_H

#include "velox.h"

#ifdef __cplusplus
extern "C" {
#endif

/*
 * velox_slab_table — one slab and its box per block ([digest] Method steps,
 * step 1, eq. 4-5; Prerequisites, "frustum slab"). Block b owns samples
 * 128 b .. 128 b + 127 (its tokens in global order, each with the depth
 * bucketed to it).
 *   cells         [nblk*128][2] int32 (col, row) token cells in the block's
 *                 latent camera
 *   depth         [nblk*128] fp32 (unreliable: not finite or <= 0)
 *   cams          [ncam][12] fp32, cam_of_block [nblk] int32 (clamped)
 *   slabs         [nblk][8] fp32 (output): u0, u1, v0, v1 (the cells of the
 *                 reliable samples: [min col, max col + 1] x [min row,
 *                 max row + 1]), zlo = Q10, zhi = Q90 of the reliable depths,
 *                 count, valid (count >= n_min, count >= 1); an invalid slab is
 *                 zero except its count
 *   boxes         [nblk][16] fp32 (output): the camera-facing box, in the
 *                 record layout of velox_geometry.h; zero when invalid
 */
velox_status_t velox_slab_table(const int32_t* cells, const float* depth, const float* cams,
                                const int32_t* cam_of_block, int ncam, int nblk, float f,
                                float cx, float cy, int n_min, float* slabs, float* boxes,
                                void* stream);

/* Workspace bytes velox_multiwarp needs for K source frames of
 * src_width x src_height pixels and a width x height target grid. */
size_t velox_multiwarp_workspace_size(int K, int src_width, int src_height, int width, int height);

/*
 * velox_multiwarp — recency-priority multiwarp ([digest] Prerequisites and
 * Method steps, step 2, eq. 6): every reliable pixel (col, row) of the K cached
 * depth frames is lifted to 3-D through its frame's camera and pinhole (pixel
 * centre (col + 0.5, row + 0.5)) and projected into the target camera; it
 * lands in target token cell (floor(u'), floor(v')) when p2 > 0 and the cell is
 * inside the grid. For each target cell the newest frame (highest index) with
 * at least k_warp samples there is chosen and zq is the median of that frame's
 * samples (mean of the two middle values for an even count); NaN and
 * chosen = -1 when no frame qualifies.
 *   src_depth  [K][src_height*src_width] fp32 depth maps (row-major pixels)
 *   src_cams   [K][12] fp32; (src_f, src_cx, src_cy) their pinhole in pixels
 *   tgt_cam    [12] fp32; (f, cx, cy) the target pinhole in token units
 *   zq         [height*width] fp32 (output); chosen [height*width] int32 (output)
 *   workspace  >= velox_multiwarp_workspace_size(...) bytes, 4-byte aligned,
 *              overwritten; calls sharing it must not overlap
 * 1 <= k_warp; K >= 0 (K = 0 gives NaN everywhere).
 */
velox_status_t velox_multiwarp(const float* src_depth, const float* src_cams, int K, int src_width,
                               int src_height, float src_f, float src_cx, float src_cy,
                               const float* tgt_cam, float f, float cx, float cy, int width,
                               int height, int k_warp, float* zq, int32_t* chosen,
                               void* workspace, size_t workspace_bytes, void* stream);

/*
 * velox_token_points — depth and world point of each token from the warped
 * map ([digest] Method steps, step 2-3: the query side's depth for coverage
 * and for its slabs): depth[s] = zq[cell of token s] (cells clamped into the
 * grid), point = the back-projection of the cell centre at that depth through
 * cam, NaN when the depth is unreliable.
 *   cells [n_tok][2] int32, zq [height*width], cam [12]
 *   depth [n_tok] fp32 (output), pts [n_tok][3] fp32 (output)
 */
velox_status_t velox_token_points(const int32_t* cells, const float* zq, int width, int height,
                                  const float* cam, float f, float cx, float cy, int64_t n_tok,
                                  float* depth, float* pts, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* VELOX_SLABS_H */
