// Geometry scorer: frustum-slab overlaps g and query-block coverage rho.
//
// A slab (a block's token rectangle with its percentile depth interval) is
// approximated by a camera-facing oriented box; blocks correspond by the IoU of
// these boxes in world space, with the intersection volume approximated on a
// grid (paper digest "Velox: Spatial Memory Makes World Models Efficient",
// Prerequisites "frustum slab and OBB overlap" and Method steps, step 3, eq. 7;
// project page "Velox: Spatial Memory Makes Long-context World Models
// Efficient", 02 · Method, "What the router sees"). Coverage is the fraction
// of a query block's tokens whose warped-depth world point lies in a valid
// history slab (same digest step 3, eq. 8; onedev summary "How it works").
//
// Grid: the n^3 cell-centre lattice of the query box A, local offsets
// e_j ((2 k_j + 1) / n - 1); I = vol(A) * inside / n^3, g = I / (vol(A) + vol(B) - I).
// A box is valid iff its three half-extents are > 0. Every decision is taken
// in float32 with one rounding per operation (this unit is compiled with
// -ffp-contract=off) in the order
//   p_x = c_x + ((R00 u0 + R01 u1) + R02 u2),  l_j = (R0j d0 + R1j d1) + R2j d2,
//   inside iff |l_j| <= e_j,  vol = ((8 e0) e1) e2,
//   f = count / n^3,  I = vol_A f,  U = (vol_A + vol_B) - I,  g = I / U.
// Record layout (float32 [16]): centre, half-extents, axes row-major (axis j is
// column j), one unused word.

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "velox_device.hpp"
#include "velox_launch.hpp"

namespace velox {
namespace {

struct Box {
  float c[3], e[3], R[9];
};

__device__ __forceinline__ Box load_box(const float* __restrict__ rec) {
  Box b;
#pragma unroll
  for (int j = 0; j < 3; ++j) {
    b.c[j] = rec[j];
    b.e[j] = rec[3 + j];
  }
#pragma unroll
  for (int j = 0; j < 9; ++j) b.R[j] = rec[6 + j];
  return b;
}

__device__ __forceinline__ bool box_valid(const Box& b) {
  return b.e[0] > 0.0f && b.e[1] > 0.0f && b.e[2] > 0.0f;
}

__device__ __forceinline__ float box_volume(const Box& b) {
  return __fmul_rn(__fmul_rn(__fmul_rn(8.0f, b.e[0]), b.e[1]), b.e[2]);
}

// World point of lattice cell (k0, k1, k2) of box a.
__device__ __forceinline__ void lattice_point(const Box& a, int n, int k0, int k1, int k2,
                                              float (&p)[3]) {
  const float fn = static_cast<float>(n);
  const float t0 = __fsub_rn(__fdiv_rn(static_cast<float>(2 * k0 + 1), fn), 1.0f);
  const float t1 = __fsub_rn(__fdiv_rn(static_cast<float>(2 * k1 + 1), fn), 1.0f);
  const float t2 = __fsub_rn(__fdiv_rn(static_cast<float>(2 * k2 + 1), fn), 1.0f);
  const float u0 = __fmul_rn(a.e[0], t0), u1 = __fmul_rn(a.e[1], t1), u2 = __fmul_rn(a.e[2], t2);
#pragma unroll
  for (int r = 0; r < 3; ++r) {
    const float s = __fadd_rn(__fadd_rn(__fmul_rn(a.R[3 * r], u0), __fmul_rn(a.R[3 * r + 1], u1)),
                              __fmul_rn(a.R[3 * r + 2], u2));
    p[r] = __fadd_rn(a.c[r], s);
  }
}

__device__ __forceinline__ bool point_inside(const Box& b, float px, float py, float pz) {
  const float d0 = __fsub_rn(px, b.c[0]), d1 = __fsub_rn(py, b.c[1]), d2 = __fsub_rn(pz, b.c[2]);
  bool in = true;
#pragma unroll
  for (int j = 0; j < 3; ++j) {
    const float l = __fadd_rn(__fadd_rn(__fmul_rn(b.R[j], d0), __fmul_rn(b.R[3 + j], d1)),
                              __fmul_rn(b.R[6 + j], d2));
    in = in && (fabsf(l) <= b.e[j]);
  }
  return in;
}

constexpr int kOverlapThreads = 256;   // 4 waves
constexpr int kOverlapRows = 64;       // history boxes per workgroup
constexpr int kCachedPoints = 8;       // lattice points cached per lane (n^3 <= 512)

// One workgroup per (query box i, 64 history boxes). Each wave owns the whole
// lattice (lane l holds points l, l + 64, ...) and takes every fourth history
// box of the range; the count is a sum of ballot popcounts, so no barrier.
template <bool kCached>
__global__ __launch_bounds__(kOverlapThreads) void slab_overlap_kernel(
    const float* __restrict__ q_obb, const float* __restrict__ h_obb, int N, int M, int n,
    float* __restrict__ g) {
  const int i = blockIdx.y;
  const int lane = threadIdx.x % kWave;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  const int r0 = blockIdx.x * kOverlapRows;
  const int r1 = min(M, r0 + kOverlapRows);
  const Box a = load_box(q_obb + 16 * static_cast<int64_t>(i));
  float* grow = g + static_cast<int64_t>(i) * M;
  if (!box_valid(a)) {
    for (int r = r0 + threadIdx.x; r < r1; r += kOverlapThreads) grow[r] = 0.0f;
    return;
  }
  const int P = n * n * n;
  const int steps = (P + kWave - 1) / kWave;
  const float va = box_volume(a);
  const float fP = static_cast<float>(P);

  float px[kCachedPoints], py[kCachedPoints], pz[kCachedPoints];
  if (kCached) {
#pragma unroll
    for (int s = 0; s < kCachedPoints; ++s) {
      const int j = lane + s * kWave;
      float p[3] = {0.f, 0.f, 0.f};
      if (j < P) lattice_point(a, n, j / (n * n), (j / n) % n, j % n, p);
      px[s] = p[0];
      py[s] = p[1];
      pz[s] = p[2];
    }
  }

  for (int r = r0 + w; r < r1; r += kOverlapThreads / kWave) {
    const Box b = load_box(h_obb + 16 * static_cast<int64_t>(r));
    int count = 0;
    if (box_valid(b)) {
      if (kCached) {
#pragma unroll
        for (int s = 0; s < kCachedPoints; ++s) {
          const bool in = (lane + s * kWave < P) && point_inside(b, px[s], py[s], pz[s]);
          count += __popcll(__ballot(in));
        }
      } else {
        for (int s = 0; s < steps; ++s) {
          const int j = lane + s * kWave;
          bool in = false;
          if (j < P) {
            float p[3];
            lattice_point(a, n, j / (n * n), (j / n) % n, j % n, p);
            in = point_inside(b, p[0], p[1], p[2]);
          }
          count += __popcll(__ballot(in));
        }
      }
    }
    if (lane == 0) {
      float gv = 0.0f;
      if (count > 0) {
        const float frac = __fdiv_rn(static_cast<float>(count), fP);
        const float inter = __fmul_rn(va, frac);
        const float uni = __fsub_rn(__fadd_rn(va, box_volume(b)), inter);
        gv = __fdiv_rn(inter, uni);
      }
      grow[r] = gv;
    }
  }
}

constexpr int kCoverRows = 64;          // history boxes per coverage workgroup

__global__ void clear_words_kernel(uint32_t* __restrict__ words, int n) {
  const int t = blockIdx.x * blockDim.x + threadIdx.x;
  if (t < n) words[t] = 0u;
}

// One workgroup of 128 threads (one per token) per (query block i, 64
// history boxes); a covered token sets its bit with an atomic OR.
__global__ __launch_bounds__(kBlock) void slab_cover_kernel(const float* __restrict__ q_pts,
                                                           const float* __restrict__ h_obb,
                                                           int M, uint32_t* __restrict__ mask) {
  const int i = blockIdx.y, t = threadIdx.x;
  const int r0 = blockIdx.x * kCoverRows;
  const int r1 = min(M, r0 + kCoverRows);
  const float* pt = q_pts + (static_cast<int64_t>(i) * kBlock + t) * 3;
  const float x = pt[0], y = pt[1], z = pt[2];
  bool cov = false;
  for (int r = r0; r < r1; ++r) {
    const Box b = load_box(h_obb + 16 * static_cast<int64_t>(r));
    if (box_valid(b)) cov = cov || point_inside(b, x, y, z);
  }
  const uint64_t bits = __ballot(cov);
  const int lane = t % kWave;
  if (lane == 0 && (bits & 0xffffffffull)) atomicOr(&mask[i * 4 + (t / 32)], static_cast<uint32_t>(bits));
  if (lane == 32 && (bits >> 32)) atomicOr(&mask[i * 4 + (t / 32)], static_cast<uint32_t>(bits >> 32));
}

__global__ void coverage_rho_kernel(const uint32_t* __restrict__ mask, int N, float* __restrict__ rho) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= N) return;
  int c = 0;
#pragma unroll
  for (int j = 0; j < 4; ++j) c += __popc(mask[i * 4 + j]);
  rho[i] = static_cast<float>(c) * (1.0f / kBlock);  // exact: c <= 128, power-of-two divisor
}

}  // namespace

hipError_t launch_slab_overlap(const float* q_obb, const float* h_obb, int N, int M, int n,
                               float* g, hipStream_t stream) {
  if (N == 0 || M == 0) return hipSuccess;
  dim3 grid((M + kOverlapRows - 1) / kOverlapRows, N);
  if (n * n * n <= kCachedPoints * kWave)
    hipLaunchKernelGGL(slab_overlap_kernel<true>, grid, dim3(kOverlapThreads), 0, stream, q_obb,
                       h_obb, N, M, n, g);
  else
    hipLaunchKernelGGL(slab_overlap_kernel<false>, grid, dim3(kOverlapThreads), 0, stream, q_obb,
                       h_obb, N, M, n, g);
  return hipGetLastError();
}

hipError_t launch_slab_coverage(const float* q_pts, const float* h_obb, int N, int M,
                                uint32_t* mask, float* rho, hipStream_t stream) {
  if (N == 0) return hipSuccess;
  hipLaunchKernelGGL(clear_words_kernel, dim3((4 * N + 255) / 256), dim3(256), 0, stream, mask, 4 * N);
  if (M > 0)
    hipLaunchKernelGGL(slab_cover_kernel, dim3((M + kCoverRows - 1) / kCoverRows, N), dim3(kBlock), 0,
                       stream, q_pts, h_obb, M, mask);
  hipLaunchKernelGGL(coverage_rho_kernel, dim3((N + 255) / 256), dim3(256), 0, stream, mask, N, rho);
  return hipGetLastError();
}

}  // namespace velox
