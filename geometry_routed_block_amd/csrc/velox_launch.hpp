// Internal host-side launch interface between the C ABI layer and the kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace velox {

constexpr size_t kMaxLdsBytes = 160 * 1024;  // LDS per workgroup on gfx950

struct RouteConfig {
  float tau, g_ref, lambda, eta_cov, theta_cov, theta_unc;
  int K_cov, K_unc, n_prev, neigh26, mode;
  const int32_t* ref_ids;
  int n_ref;
  int32_t* status;  // nullable device int32[2]: rows with bad inputs, smallest such row
};

struct AttnConfig {
  const void* q;
  const void* k;
  const void* v;
  bool bf16;
  int64_t ld_q_h, ld_kv_h;
  int H, N, M, d;
  float scale;
  const int32_t* route_ids;  // nullptr: dense (every history tile)
  const int32_t* route_len;
  int L;
  bool shared_routes;        // one route per query block for every head
  int include_current;
  void* o;
  float* lse;
  int n_split;               // > 1: split rows (d = 128 bf16 only), with the two buffers below
  float* part_o;             // [n_split][H][N*128][128] fp32
  float* part_ml;            // [n_split][H][N*128][2] fp32
  void* plan;                // nullable: unit schedule of the routed d = 128 bf16 kernel,
                             // attn_plan_bytes(H, N, n_split) bytes, 16-byte aligned
};

// Bytes of the unit schedule of a routed call (0 when the call needs none).
size_t attn_plan_bytes(int H, int N, int n_split);

hipError_t launch_block_mean(const void* x, bool bf16, int64_t ld_x_h, int H, int nblk, int d,
                             float* xbar, int64_t ld_bar_h, hipStream_t stream);
size_t route_scores_lds_bytes(int qb, int M, int d);
hipError_t launch_route_scores(const void* q, bool bf16, int64_t ld_q_h, const float* kbar,
                               int64_t ld_kbar_h, int H, int N, int M, int d, float scale,
                               float* p, hipStream_t stream);
hipError_t launch_route_scores_shared(const void* q, bool bf16, int64_t ld_q_h, const float* kbar,
                                      int64_t ld_kbar_h, int H, int N, int M, int d, float scale,
                                      float* logits, float* p, hipStream_t stream);
size_t route_select_lds_bytes(int M, int fs);
hipError_t launch_route_select(const float* p, const float* g, const float* rho,
                               const int32_t* coord, int H, int N, int M, const RouteConfig& cfg,
                               int L, int32_t* route_ids, int32_t* route_len, hipStream_t stream);
hipError_t launch_attention(const AttnConfig& cfg, hipStream_t stream);
hipError_t launch_slab_overlap(const float* q_obb, const float* h_obb, int N, int M, int n,
                               float* g, hipStream_t stream);
void gilbert_curve(int width, int height, int32_t* cells);
hipError_t launch_slab_table(const int32_t* cells, const float* depth, const float* cams,
                             const int32_t* cam_of_block, int ncam, int nblk, float f, float cx, float cy,
                             int n_min, float* slabs, float* boxes, hipStream_t stream);
size_t multiwarp_workspace_bytes(int K, int P, int C);
hipError_t launch_multiwarp(const float* src_depth, const float* src_cams, int K, int SW, int SH, float fs,
                            float cxs, float cys, const float* tgt_cam, float ft, float cxt, float cyt, int W,
                            int H, int k_warp, float* zq, int32_t* chosen, void* workspace,
                            hipStream_t stream);
hipError_t launch_token_points(const int32_t* cells, const float* zq, int W, int H, const float* cam,
                               float f, float cx, float cy, int64_t n_tok, float* depth, float* pts,
                               hipStream_t stream);
hipError_t launch_route_check(const int32_t* route_ids, const int32_t* route_len, int rows, int M,
                              int L, int32_t* bad, hipStream_t stream);
hipError_t launch_kv_append(const void* k_new, const void* v_new, bool bf16, int64_t ld_new_h, int H,
                            int T, int height, int width, int d, int chunk_index,
                            const int32_t* cells, void* k_cache, void* v_cache, int64_t ld_kv_h,
                            int64_t token_offset, float* kbar, int64_t ld_kbar_h,
                            hipStream_t stream);
hipError_t launch_slab_coverage(const float* q_pts, const float* h_obb, int N, int M,
                                uint32_t* mask, float* rho, hipStream_t stream);

}  // namespace velox
