// Global Gilbert order of the KV cache: the per-chunk curve (host) and the
// append of a new chunk into the cache in that order (device).
//
// The order (paper digest "Velox: Spatial Memory Makes World Models
// Efficient", Prerequisites, "Gilbert space-filling curve"; project page
// "Velox: Spatial Memory Makes Long-context World Models Efficient",
// 02 · Method, "Keeping neighbours adjacent in the block order", Figures 6-7):
// one chunk's cells follow a generalised-Hilbert curve over the latent
// (height, width) grid, alternate chunks use the horizontally mirrored map, and
// chunks are concatenated; the result is at once the KV storage order and the
// block id. A chunk of T latent frames is ordered cell by cell along the
// curve, the T tokens of a cell in time order, so the last cell of a chunk and
// the first cell of the next coincide and the seam tokens are consecutive in
// time.

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <cstdlib>
#include <vector>

#include "velox_device.hpp"
#include "velox_launch.hpp"

namespace velox {

// ------------------------------------------------------------------ the curve
//
// Generalised Hilbert curve for an arbitrary width x height rectangle (the
// published construction): a rectangle is given by its origin cell, a major
// vector a and a minor vector b, and is walked from the origin to the far end
// of a on the same side of b. A one-cell strip is walked directly; a rectangle
// more than 1.5 times longer than wide is cut into two halves along a; any
// other is cut into a U of three pieces (the first half of b walked with a and
// b swapped, the remaining band along a, a returning piece), with half lengths
// moved to even values so that consecutive pieces meet at neighbouring cells.
// Pieces wait on an explicit stack in reverse walking order.

namespace {

struct Piece {
  int x, y, ax, ay, bx, by;
};

inline int sgn(int v) { return (v > 0) - (v < 0); }
inline int half_toward_zero(int v) { return v / 2; }  // C++ division truncates

}  // namespace

void gilbert_curve(int width, int height, int32_t* cells) {
  std::vector<Piece> stack;
  stack.push_back(width >= height ? Piece{0, 0, width, 0, 0, height}
                                  : Piece{0, 0, 0, height, width, 0});
  int k = 0;
  while (!stack.empty()) {
    const Piece p = stack.back();
    stack.pop_back();
    const int la = std::abs(p.ax + p.ay), lb = std::abs(p.bx + p.by);
    const int uax = sgn(p.ax), uay = sgn(p.ay), ubx = sgn(p.bx), uby = sgn(p.by);
    if (lb == 1 || la == 1) {
      const int sx = lb == 1 ? uax : ubx, sy = lb == 1 ? uay : uby, n = lb == 1 ? la : lb;
      for (int s = 0; s < n; ++s) cells[k++] = (p.y + s * sy) * width + (p.x + s * sx);
      continue;
    }
    int hax = half_toward_zero(p.ax), hay = half_toward_zero(p.ay);
    int hbx = half_toward_zero(p.bx), hby = half_toward_zero(p.by);
    if (2 * la > 3 * lb) {
      if (std::abs(hax + hay) % 2 == 1 && la > 2) {
        hax += uax;
        hay += uay;
      }
      stack.push_back(Piece{p.x + hax, p.y + hay, p.ax - hax, p.ay - hay, p.bx, p.by});
      stack.push_back(Piece{p.x, p.y, hax, hay, p.bx, p.by});
      continue;
    }
    if (std::abs(hbx + hby) % 2 == 1 && lb > 2) {
      hbx += ubx;
      hby += uby;
    }
    stack.push_back(Piece{p.x + (p.ax - uax) + (hbx - ubx), p.y + (p.ay - uay) + (hby - uby), -hbx,
                          -hby, -(p.ax - hax), -(p.ay - hay)});
    stack.push_back(Piece{p.x + hbx, p.y + hby, p.ax, p.ay, p.bx - hbx, p.by - hby});
    stack.push_back(Piece{p.x, p.y, hbx, hby, hax, hay});
  }
}

// ------------------------------------------------------------------ append
//
// One workgroup (256 threads) per (destination block, head). Thread groups of
// vpr = d / V lanes (V elements of 16 bytes per lane) move one token row of K
// and of V from its THW-linear source position to its global-order slot, and
// accumulate the block's key sum in fp32 for the key-mean cache (per lane over
// its rows in ascending order, then over row groups in ascending order).

namespace {

struct AppendArgs {
  const void* k_new;
  const void* v_new;
  int64_t ld_new_h;
  int T, height, width, d, odd;
  const int32_t* cells;
  void* k_cache;
  void* v_cache;
  int64_t ld_kv_h, token_offset;
  float* kbar;
  int64_t ld_kbar_h;
};

template <typename T>
__global__ __launch_bounds__(256) void kv_append_kernel(AppendArgs a) {
  constexpr int V = 16 / sizeof(T);
  __shared__ float part[256 * V];
  const int b = blockIdx.x, h = blockIdx.y, t = threadIdx.x;
  const int vpr = a.d / V, groups = 256 / vpr;
  const int cv = t % vpr, grp = t / vpr;
  const int ncell = a.height * a.width;
  const T* kn = static_cast<const T*>(a.k_new) + h * a.ld_new_h + cv * V;
  const T* vn = static_cast<const T*>(a.v_new) + h * a.ld_new_h + cv * V;
  T* kc = static_cast<T*>(a.k_cache) + h * a.ld_kv_h + cv * V;
  T* vc = static_cast<T*>(a.v_cache) + h * a.ld_kv_h + cv * V;
  float acc[V];
#pragma unroll
  for (int e = 0; e < V; ++e) acc[e] = 0.f;
  for (int j = grp; j < kBlock; j += groups) {
    const int rank = b * kBlock + j;
    const int cell_pos = rank / a.T, tt = rank - cell_pos * a.T;
    const int c = min(max(a.cells[cell_pos], 0), ncell - 1);
    const int hh = c / a.width, wq = c - hh * a.width;
    const int ww = a.odd ? a.width - 1 - wq : wq;
    const int64_t src = (static_cast<int64_t>(tt) * a.height + hh) * a.width + ww;
    const int64_t dst = a.token_offset + rank;
    const uint4 ku = *reinterpret_cast<const uint4*>(kn + src * a.d);
    const uint4 vu = *reinterpret_cast<const uint4*>(vn + src * a.d);
    *reinterpret_cast<uint4*>(kc + dst * a.d) = ku;
    *reinterpret_cast<uint4*>(vc + dst * a.d) = vu;
    const uint32_t w[4] = {ku.x, ku.y, ku.z, ku.w};
    if constexpr (V == 8) {
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        acc[2 * q] += __uint_as_float(w[q] << 16);
        acc[2 * q + 1] += __uint_as_float(w[q] & 0xffff0000u);
      }
    } else {
#pragma unroll
      for (int q = 0; q < 4; ++q) acc[q] += __uint_as_float(w[q]);
    }
  }
  if (a.kbar == nullptr) return;  // uniform: every thread takes the same branch
#pragma unroll
  for (int e = 0; e < V; ++e) part[grp * a.d + cv * V + e] = acc[e];
  __syncthreads();
  if (t < a.d) {
    float tot = 0.f;
    for (int g = 0; g < groups; ++g) tot += part[g * a.d + t];
    const int64_t blk = a.token_offset / kBlock + b;
    a.kbar[h * a.ld_kbar_h + blk * a.d + t] = tot * (1.0f / kBlock);
  }
}

}  // namespace

hipError_t launch_kv_append(const void* k_new, const void* v_new, bool bf16, int64_t ld_new_h, int H,
                            int T, int height, int width, int d, int chunk_index,
                            const int32_t* cells, void* k_cache, void* v_cache, int64_t ld_kv_h,
                            int64_t token_offset, float* kbar, int64_t ld_kbar_h,
                            hipStream_t stream) {
  const int nblk = T * height * width / kBlock;
  if (nblk == 0) return hipSuccess;
  AppendArgs a{k_new, v_new, ld_new_h, T, height, width, d, chunk_index & 1, cells,
               k_cache, v_cache, ld_kv_h, token_offset, kbar, ld_kbar_h};
  dim3 grid(nblk, H);
  if (bf16)
    hipLaunchKernelGGL(kv_append_kernel<bf16_t>, grid, dim3(256), 0, stream, a);
  else
    hipLaunchKernelGGL(kv_append_kernel<float>, grid, dim3(256), 0, stream, a);
  return hipGetLastError();
}

}  // namespace velox
