// Slab table and recency-priority multiwarp: the geometry that turns
// reconstructed depth into the boxes the overlap scorer consumes.
//
// Paper digest "Velox: Spatial Memory Makes World Models Efficient", Method
// steps 1-2 (eq. 4-6) and Prerequisites ("frustum slab", "recency-priority
// multiwarp"); onedev summary "How it works". A history block's slab is its
// token rectangle in the chunk's latent camera plus the 10/90 percentile
// interval of its reliable depths; a slab is approximated by a camera-facing
// oriented box. The current chunk gets its depth by forward-warping the cached
// first/last frame depths of recent chunks into its camera and taking, per
// token, the median of the newest frame that supplies at least k_warp samples.
//
// Camera model (pinhole in token units): a pose is (R, c) with world =
// c + R * camera; token cell (col, row) has centre (col + 0.5, row + 0.5); the
// ray through (u, v) is ((u - cx) / f, (cy - v) / f, 1). Every decision and
// output is computed in float32 with one rounding per operation (this unit is
// compiled with -ffp-contract=off) in this order:
//   point       X_r = c_r + ((R_r0 (z rx) + R_r1 (z ry)) + R_r2 z)
//   projection  d = X - c_t;  p_j = (R_0j d0 + R_1j d1) + R_2j d2;
//               u' = (f p0) / p2 + cx,  v' = cy - (f p1) / p2
//   percentile  h = (n - 1) p, i = floor(h), q = x_i + (h - i)(x_{i+1} - x_i)
//   box         centre = point of the rectangle centre at zm = (zlo + zhi) / 2,
//               e0 = (zm (u1 - u0)) / (2 f), e1 = (zm (v1 - v0)) / (2 f),
//               e2 = (zhi - zlo) / 2, axes = camera axes

#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include "velox_device.hpp"
#include "velox_launch.hpp"

namespace velox {
namespace {

struct Pinhole {
  float f, cx, cy;
};

__device__ __forceinline__ bool reliable_depth(float z) { return isfinite(z) && z > 0.0f; }

// World point at depth z on the ray through (u, v) of camera cam[12].
__device__ __forceinline__ void world_point(const float* __restrict__ cam, float u, float v, float z,
                                            const Pinhole& k, float (&X)[3]) {
  const float rx = __fdiv_rn(__fsub_rn(u, k.cx), k.f);
  const float ry = __fdiv_rn(__fsub_rn(k.cy, v), k.f);
  const float a = __fmul_rn(z, rx), b = __fmul_rn(z, ry);
#pragma unroll
  for (int r = 0; r < 3; ++r) {
    const float s = __fadd_rn(__fadd_rn(__fmul_rn(cam[3 * r], a), __fmul_rn(cam[3 * r + 1], b)),
                              __fmul_rn(cam[3 * r + 2], z));
    X[r] = __fadd_rn(cam[9 + r], s);
  }
}

constexpr int kSlabThreads = kBlock;   // one thread per sample of the block

// One workgroup per block: count, rectangle and bitonic sort of the reliable
// depths (unreliable ones sort to the end as +inf), then thread 0 writes the
// slab record and its box.
__global__ __launch_bounds__(kSlabThreads) void slab_table_kernel(
    const int32_t* __restrict__ cells, const float* __restrict__ depth, const float* __restrict__ cams,
    const int32_t* __restrict__ cam_of_block, int ncam, Pinhole k, int n_min, float* __restrict__ slabs,
    float* __restrict__ boxes) {
  __shared__ float zs[kBlock];
  const int b = blockIdx.x, t = threadIdx.x;
  const int64_t s = static_cast<int64_t>(b) * kBlock + t;
  const float z = depth[s];
  const bool ok = reliable_depth(z);
  const int col = cells[2 * s], row = cells[2 * s + 1];
  zs[t] = ok ? z : INFINITY;
  // counts and rectangle
  const int lane = t % kWave, w = t / kWave;
  int n = __popcll(__ballot(ok));
  int cmin = ok ? col : INT32_MAX, cmax = ok ? col : INT32_MIN;
  int rmin = ok ? row : INT32_MAX, rmax = ok ? row : INT32_MIN;
  for (int o = kWave / 2; o > 0; o >>= 1) {
    cmin = min(cmin, __shfl_xor(cmin, o));
    cmax = max(cmax, __shfl_xor(cmax, o));
    rmin = min(rmin, __shfl_xor(rmin, o));
    rmax = max(rmax, __shfl_xor(rmax, o));
  }
  __shared__ int rect[2][4];
  __shared__ int cnt[2];
  if (lane == 0) {
    rect[w][0] = cmin;
    rect[w][1] = cmax;
    rect[w][2] = rmin;
    rect[w][3] = rmax;
    cnt[w] = n;
  }
  __syncthreads();
  // bitonic sort of the 128 depths, ascending
  for (int kk = 2; kk <= kBlock; kk <<= 1) {
    for (int j = kk >> 1; j > 0; j >>= 1) {
      const int p = t ^ j;
      if (p > t) {
        const float x = zs[t], y = zs[p];
        const bool up = (t & kk) == 0;
        if ((x > y) == up) {
          zs[t] = y;
          zs[p] = x;
        }
      }
      __syncthreads();
    }
  }
  if (t != 0) return;
  n = cnt[0] + cnt[1];
  float* sl = slabs + static_cast<int64_t>(b) * 8;
  float* bx = boxes + static_cast<int64_t>(b) * 16;
  if (n < n_min || n == 0) {
    for (int e = 0; e < 8; ++e) sl[e] = 0.0f;
    sl[6] = static_cast<float>(n);
    for (int e = 0; e < 16; ++e) bx[e] = 0.0f;
    return;
  }
  const float u0 = static_cast<float>(min(rect[0][0], rect[1][0]));
  const float u1 = static_cast<float>(max(rect[0][1], rect[1][1]) + 1);
  const float v0 = static_cast<float>(min(rect[0][2], rect[1][2]));
  const float v1 = static_cast<float>(max(rect[0][3], rect[1][3]) + 1);
  float q[2];
  const float ps[2] = {0.1f, 0.9f};
  for (int e = 0; e < 2; ++e) {
    const float h = __fmul_rn(static_cast<float>(n - 1), ps[e]);
    const int i = static_cast<int>(floorf(h));
    const float fr = __fsub_rn(h, static_cast<float>(i));
    const float xi = zs[i];
    q[e] = (i + 1 >= n) ? xi : __fadd_rn(xi, __fmul_rn(fr, __fsub_rn(zs[i + 1], xi)));
  }
  const float zlo = q[0], zhi = q[1];
  sl[0] = u0;
  sl[1] = u1;
  sl[2] = v0;
  sl[3] = v1;
  sl[4] = zlo;
  sl[5] = zhi;
  sl[6] = static_cast<float>(n);
  sl[7] = 1.0f;
  const int ci = min(max(cam_of_block[b], 0), ncam - 1);
  const float* cam = cams + 12 * static_cast<int64_t>(ci);
  const float uc = __fmul_rn(__fadd_rn(u0, u1), 0.5f), vc = __fmul_rn(__fadd_rn(v0, v1), 0.5f);
  const float zm = __fmul_rn(__fadd_rn(zlo, zhi), 0.5f);
  float X[3];
  world_point(cam, uc, vc, zm, k, X);
  const float two_f = __fmul_rn(2.0f, k.f);
  bx[0] = X[0];
  bx[1] = X[1];
  bx[2] = X[2];
  bx[3] = __fdiv_rn(__fmul_rn(zm, __fsub_rn(u1, u0)), two_f);
  bx[4] = __fdiv_rn(__fmul_rn(zm, __fsub_rn(v1, v0)), two_f);
  bx[5] = __fmul_rn(__fsub_rn(zhi, zlo), 0.5f);
  for (int e = 0; e < 9; ++e) bx[6 + e] = cam[e];
  bx[15] = 0.0f;
}

// ---------------------------------------------------------------- multiwarp

struct WarpWs {
  int32_t* cell_of;   // [K*P] target cell of each source pixel, -1 if none
  float* dep;         // [K*P] its depth in the target camera
  int32_t* count;     // [C*K] samples per (cell, frame)
  int32_t* need;      // [C] samples of the chosen frame
  int32_t* start;     // [C+1] exclusive scan of need
  int32_t* fill;      // [C] append cursor
  float* buf;         // [K*P] samples of the chosen frames, grouped by cell
};

__global__ void clear_ints_kernel(int32_t* __restrict__ p, int64_t n) {
  const int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (i < n) p[i] = 0;
}

__global__ __launch_bounds__(256) void warp_project_kernel(const float* __restrict__ src_depth,
                                                           const float* __restrict__ src_cams, Pinhole ks,
                                                           int SW, int SH, const float* __restrict__ tgt,
                                                           Pinhole kt, int K, int W, int H, WarpWs ws) {
  const int P = SW * SH;
  const int64_t g = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (g >= static_cast<int64_t>(K) * P) return;
  const int f = static_cast<int>(g / P), pix = static_cast<int>(g % P);
  const float z = src_depth[g];
  int cell = -1;
  float pz = 0.0f;
  if (reliable_depth(z)) {
    const int col = pix % SW, row = pix / SW;
    float X[3];
    world_point(src_cams + 12 * static_cast<int64_t>(f), __fadd_rn(static_cast<float>(col), 0.5f),
                __fadd_rn(static_cast<float>(row), 0.5f), z, ks, X);
    const float d0 = __fsub_rn(X[0], tgt[9]), d1 = __fsub_rn(X[1], tgt[10]), d2 = __fsub_rn(X[2], tgt[11]);
    float p[3];
#pragma unroll
    for (int j = 0; j < 3; ++j)
      p[j] = __fadd_rn(__fadd_rn(__fmul_rn(tgt[j], d0), __fmul_rn(tgt[3 + j], d1)), __fmul_rn(tgt[6 + j], d2));
    if (p[2] > 0.0f) {
      const float u = __fadd_rn(__fdiv_rn(__fmul_rn(kt.f, p[0]), p[2]), kt.cx);
      const float v = __fsub_rn(kt.cy, __fdiv_rn(__fmul_rn(kt.f, p[1]), p[2]));
      const float fu = floorf(u), fv = floorf(v);
      if (fu >= 0.0f && fu < static_cast<float>(W) && fv >= 0.0f && fv < static_cast<float>(H)) {
        cell = static_cast<int>(fv) * W + static_cast<int>(fu);
        pz = p[2];
        atomicAdd(&ws.count[static_cast<int64_t>(cell) * K + f], 1);
      }
    }
  }
  ws.cell_of[g] = cell;
  ws.dep[g] = pz;
}

__global__ __launch_bounds__(256) void warp_choose_kernel(int K, int C, int k_warp, WarpWs ws,
                                                          int32_t* __restrict__ chosen) {
  const int c = blockIdx.x * blockDim.x + threadIdx.x;
  if (c >= C) return;
  int ch = -1, n = 0;
  for (int f = K - 1; f >= 0; --f) {
    const int cn = ws.count[static_cast<int64_t>(c) * K + f];
    if (cn >= k_warp) {
      ch = f;
      n = cn;
      break;
    }
  }
  chosen[c] = ch;
  ws.need[c] = n;
}

// Exclusive scan of need over the cells in one workgroup of 1024 threads.
__global__ __launch_bounds__(1024) void warp_scan_kernel(int C, WarpWs ws) {
  __shared__ int part[1024 / kWave];
  const int t = threadIdx.x, lane = t % kWave, w = t / kWave;
  int carry = 0;
  for (int base = 0; base < C; base += 1024) {
    const int c = base + t;
    const int x = c < C ? ws.need[c] : 0;
    int incl = x;
    for (int o = 1; o < kWave; o <<= 1) {
      const int y = __shfl_up(incl, o);
      if (lane >= o) incl += y;
    }
    if (lane == kWave - 1) part[w] = incl;
    __syncthreads();
    int before = 0, total = 0;
    for (int j = 0; j < 1024 / kWave; ++j) {
      if (j < w) before += part[j];
      total += part[j];
    }
    if (c < C) ws.start[c] = carry + before + incl - x;
    carry += total;
    __syncthreads();
  }
  if (t == 0) ws.start[C] = carry;
}

__global__ __launch_bounds__(256) void warp_gather_kernel(int K, int P, WarpWs ws,
                                                          const int32_t* __restrict__ chosen) {
  const int64_t g = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (g >= static_cast<int64_t>(K) * P) return;
  const int cell = ws.cell_of[g];
  if (cell < 0) return;
  const int f = static_cast<int>(g / P);
  if (chosen[cell] != f) return;
  const int slot = atomicAdd(&ws.fill[cell], 1);
  ws.buf[ws.start[cell] + slot] = ws.dep[g];
}

// One wave per cell: the median by rank counting (order-independent, so the
// arrival order of the gathered samples does not matter).
__global__ __launch_bounds__(kWave) void warp_median_kernel(int C, WarpWs ws, float* __restrict__ zq) {
  __shared__ float mid[2];
  const int c = blockIdx.x, t = threadIdx.x;
  const int n = ws.need[c];
  if (n == 0) {
    if (t == 0) zq[c] = NAN;
    return;
  }
  const float* x = ws.buf + ws.start[c];
  const int lo = (n - 1) / 2, hi = n / 2;
  for (int i = t; i < n; i += kWave) {
    const float xi = x[i];
    int rank = 0;
    for (int j = 0; j < n; ++j) {
      const float xj = x[j];
      rank += (xj < xi) || (xj == xi && j < i);
    }
    if (rank == lo) mid[0] = xi;
    if (rank == hi) mid[1] = xi;
  }
  __syncthreads();
  if (t == 0) zq[c] = (n & 1) ? mid[0] : __fmul_rn(__fadd_rn(mid[0], mid[1]), 0.5f);
}

// Token depth from the warped map and its world point (NaN point without depth).
__global__ __launch_bounds__(256) void token_points_kernel(const int32_t* __restrict__ cells,
                                                           const float* __restrict__ zq, int W, int H,
                                                           const float* __restrict__ cam, Pinhole k,
                                                           int64_t n_tok, float* __restrict__ depth,
                                                           float* __restrict__ pts) {
  const int64_t s = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (s >= n_tok) return;
  const int col = min(max(cells[2 * s], 0), W - 1), row = min(max(cells[2 * s + 1], 0), H - 1);
  const float z = zq[row * W + col];
  float X[3] = {NAN, NAN, NAN};
  if (reliable_depth(z))
    world_point(cam, __fadd_rn(static_cast<float>(col), 0.5f), __fadd_rn(static_cast<float>(row), 0.5f), z,
                k, X);
  depth[s] = z;
  pts[3 * s] = X[0];
  pts[3 * s + 1] = X[1];
  pts[3 * s + 2] = X[2];
}

WarpWs carve(void* workspace, int K, int P, int C) {
  char* p = static_cast<char*>(workspace);
  const size_t kp = static_cast<size_t>(K) * P, kc = static_cast<size_t>(K) * C;
  WarpWs ws;
  ws.cell_of = reinterpret_cast<int32_t*>(p);
  p += kp * 4;
  ws.dep = reinterpret_cast<float*>(p);
  p += kp * 4;
  ws.count = reinterpret_cast<int32_t*>(p);
  p += kc * 4;
  ws.fill = reinterpret_cast<int32_t*>(p);   // adjacent to count: one clear covers both
  p += static_cast<size_t>(C) * 4;
  ws.need = reinterpret_cast<int32_t*>(p);
  p += static_cast<size_t>(C) * 4;
  ws.start = reinterpret_cast<int32_t*>(p);
  p += static_cast<size_t>(C + 1) * 4;
  ws.buf = reinterpret_cast<float*>(p);
  return ws;
}

}  // namespace

size_t multiwarp_workspace_bytes(int K, int P, int C) {
  const size_t kp = static_cast<size_t>(K) * P, kc = static_cast<size_t>(K) * C;
  return 4 * (3 * kp + kc + 3 * static_cast<size_t>(C) + 1);
}

hipError_t launch_slab_table(const int32_t* cells, const float* depth, const float* cams,
                             const int32_t* cam_of_block, int ncam, int nblk, float f, float cx, float cy,
                             int n_min, float* slabs, float* boxes, hipStream_t stream) {
  if (nblk == 0) return hipSuccess;
  hipLaunchKernelGGL(slab_table_kernel, dim3(nblk), dim3(kSlabThreads), 0, stream, cells, depth, cams,
                     cam_of_block, ncam, Pinhole{f, cx, cy}, n_min, slabs, boxes);
  return hipGetLastError();
}

hipError_t launch_multiwarp(const float* src_depth, const float* src_cams, int K, int SW, int SH, float fs,
                            float cxs, float cys, const float* tgt_cam, float ft, float cxt, float cyt, int W,
                            int H, int k_warp, float* zq, int32_t* chosen, void* workspace,
                            hipStream_t stream) {
  const int C = W * H, P = SW * SH;
  WarpWs ws = carve(workspace, K, P, C);
  const int64_t kp = static_cast<int64_t>(K) * P;
  const int64_t nclear = static_cast<int64_t>(K) * C + C;
  hipLaunchKernelGGL(clear_ints_kernel, dim3(static_cast<unsigned>((nclear + 255) / 256)), dim3(256), 0, stream,
                     ws.count, nclear);
  if (kp > 0)
    hipLaunchKernelGGL(warp_project_kernel, dim3(static_cast<unsigned>((kp + 255) / 256)), dim3(256), 0, stream,
                       src_depth, src_cams, Pinhole{fs, cxs, cys}, SW, SH, tgt_cam, Pinhole{ft, cxt, cyt}, K,
                       W, H, ws);
  hipLaunchKernelGGL(warp_choose_kernel, dim3((C + 255) / 256), dim3(256), 0, stream, K, C, k_warp, ws, chosen);
  hipLaunchKernelGGL(warp_scan_kernel, dim3(1), dim3(1024), 0, stream, C, ws);
  if (kp > 0)
    hipLaunchKernelGGL(warp_gather_kernel, dim3(static_cast<unsigned>((kp + 255) / 256)), dim3(256), 0, stream,
                       K, P, ws, chosen);
  hipLaunchKernelGGL(warp_median_kernel, dim3(C), dim3(kWave), 0, stream, C, ws, zq);
  return hipGetLastError();
}

hipError_t launch_token_points(const int32_t* cells, const float* zq, int W, int H, const float* cam,
                               float f, float cx, float cy, int64_t n_tok, float* depth, float* pts,
                               hipStream_t stream) {
  if (n_tok == 0) return hipSuccess;
  hipLaunchKernelGGL(token_points_kernel, dim3(static_cast<unsigned>((n_tok + 255) / 256)), dim3(256), 0,
                     stream, cells, zq, W, H, cam, Pinhole{f, cx, cy}, n_tok, depth, pts);
  return hipGetLastError();
}

}  // namespace velox
