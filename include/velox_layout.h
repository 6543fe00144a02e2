/*
 * velox_layout.h — C ABI of the global-order layout in libvelox.so: the
 * per-chunk generalised-Hilbert ("Gilbert") curve and the append of a new
 * chunk's keys and values into the KV cache in global order, with the
 * key-mean cache update that the importance step (velox.h,
 * velox_route_scores) reads.
 *
 * The method: "Velox: Spatial Memory Makes World Models Efficient". Pages:
 *   [digest]  paper digest (paper.rainbus.top): Prerequisites, "Gilbert
 *             space-filling curve" (one chunk's rank map, horizontal flip of
 *             in-chunk coordinates by chunk parity, concatenation; the order is
 *             the KV layout, the neighbour domain and the block id).
 *   [project] project page (velox-world.com/velox): 02 · Method, "Keeping
 *             neighbours adjacent in the block order", Figures 6-7.
 *   [onedev]  Korean summary (onedev.kr): "How to use" (KV stored in the
 *             routes' global Gilbert order).
 *
 * Token order inside a chunk of T latent frames of height x width tokens:
 * cells follow the curve over the (height, width) grid — mirrored in width on
 * odd chunks — and the T tokens of a cell follow each other in time order.
 * Chunk-local position of token (t, h, w):
 *   rank(h, w') * T + t,   w' = w (even chunk) or width - 1 - w (odd chunk),
 * where rank is the position of a cell along the curve. The last cell of a
 * chunk and the first of the next then coincide, so the seam tokens are
 * consecutive in time.
 *
 * Conventions are those of velox.h.
 */
#ifndef VELOX_LAYOUT_H
#define VELOX_LAYOUT_H

#include "velox.h"

#ifdef __cplusplus
extern "C" {
#endif

#define VELOX_MAX_GRID_CELLS (1 << 24)

/*
 * velox_gilbert_curve — the generalised-Hilbert curve over a width x height
 * grid ([digest] Prerequisites, "Gilbert space-filling curve"): cells[k] =
 * y * width + x of the k-th cell along the curve. The curve starts at (0, 0)
 * and ends at (width-1, 0) when width >= height, else at (0, height-1);
 * consecutive cells are grid neighbours (one diagonal step can occur when the
 * long side is odd). On power-of-two squares it is the Hilbert curve.
 *   cells  [width*height] int32, HOST memory (output)
 * Host-only, synchronous; 1 <= width, height and width*height <=
 * VELOX_MAX_GRID_CELLS.
 */
velox_status_t velox_gilbert_curve(int width, int height, int32_t* cells);

/*
 * velox_kv_append — write one new chunk into the KV cache in global order
 * and refresh the key means of its blocks ([digest] Prerequisites, "Gilbert
 * space-filling curve"; [onedev] "How to use"; key means as in velox.h,
 * velox_block_mean).
 *   k_new, v_new  [H][T*height*width][d] dtype dt, THW-linear token order
 *                 (token (t, h, w) at row (t*height + h)*width + w), head
 *                 stride ld_new_h
 *   cells         [height*width] int32 DEVICE copy of velox_gilbert_curve's
 *                 output for (width, height); entries outside [0, height*width)
 *                 are clamped (the kernel trusts it to be a permutation)
 *   chunk_index   parity selects the mirrored map (odd chunks)
 *   k_cache, v_cache  [H][cap][d] dtype dt, head stride ld_kv_h; rows
 *                 token_offset .. token_offset + T*height*width - 1 are written
 *   kbar          [H][>=token_offset/128 + nblk][d] fp32, head stride
 *                 ld_kbar_h: entries token_offset/128 .. + nblk - 1 are written
 *                 with the mean of each new block's keys; may be NULL
 * T*height*width must be a multiple of 128 (whole blocks; else
 * VELOX_ERR_UNSUPPORTED), token_offset a multiple of 128; every pointer and
 * head stride 16-byte aligned; H <= 65535. Summation order of a key mean: per
 * lane over its rows in ascending order, then over row groups in order.
 */
velox_status_t velox_kv_append(const void* k_new, const void* v_new, velox_dtype_t dt,
                               int64_t ld_new_h, int H, int T, int height, int width, int d,
                               int chunk_index, const int32_t* cells, void* k_cache,
                               void* v_cache, int64_t ld_kv_h, int64_t token_offset,
                               float* kbar, int64_t ld_kbar_h, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* VELOX_LAYOUT_H */
