// Router kernels: block means, block importance, route materialisation.
//
// Method: "Velox: Spatial Memory Makes World Models Efficient".
//   importance    — paper digest, Method steps, step 4 (eq. 9); onedev.kr
//                   summary, "What differs": softmax over the mean query . mean
//                   key inner product of a query block and each history block.
//   fusion + gate — project page, 02 · Method, fusion formula
//                   p~ ∝ p (1 + lambda ghat), ghat = 1[g > tau] min(g / g_ref, 1);
//                   covered rows (rho >= eta_cov) fuse, uncovered rows keep p.
//   route         — digest, Core method and Method steps, step 4 (eq. 12-14):
//                   covered rows take the top K_cov, uncovered rows the
//                   cumulative-mass prefix capped at K_unc; previous chunk
//                   reserved inside the budget; neighbours and reference blocks
//                   added outside it (onedev.kr, "What differs").
//
// This translation unit is compiled with -ffp-contract=off: the fused weight
// is a discrete decision (a route), so every float32 operation of the fusion
// is rounded separately, as the formula is written, and the mass is then
// accounted in exact integers (floor(w * 2^60)).

#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include "velox_device.hpp"
#include "velox_launch.hpp"

namespace velox {

// ---------------------------------------------------------------- reductions

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o));
  return v;
}
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
  return v;
}
__device__ __forceinline__ uint64_t wave_sum_u64(uint64_t v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
  return v;
}

// Block-wide max / sum; `red` holds >= blockDim/64 floats. Ends synchronised.
__device__ __forceinline__ float block_max(float v, float* red) {
  const int lane = threadIdx.x % kWave, w = threadIdx.x / kWave, nw = blockDim.x / kWave;
  v = wave_max(v);
  __syncthreads();
  if (lane == 0) red[w] = v;
  __syncthreads();
  float r = red[0];
  for (int j = 1; j < nw; ++j) r = fmaxf(r, red[j]);
  __syncthreads();
  return r;
}
__device__ __forceinline__ float block_sum(float v, float* red) {
  const int lane = threadIdx.x % kWave, w = threadIdx.x / kWave, nw = blockDim.x / kWave;
  v = wave_sum(v);
  __syncthreads();
  if (lane == 0) red[w] = v;
  __syncthreads();
  float r = red[0];
  for (int j = 1; j < nw; ++j) r += red[j];
  __syncthreads();
  return r;
}

// ---------------------------------------------------------------- block means

template <typename T>
__global__ __launch_bounds__(256) void block_mean_kernel(const T* __restrict__ x, int64_t ld_x_h,
                                                         int d, float* __restrict__ xbar,
                                                         int64_t ld_bar_h) {
  __shared__ float part[256];
  const int b = blockIdx.x, h = blockIdx.y, t = threadIdx.x;
  const int parts = 256 / d;  // d in {64, 128}
  const int c = t % d, s = t / d;
  const T* src = x + h * ld_x_h + static_cast<int64_t>(b) * kBlock * d;
  float acc = 0.f;
  for (int a = s; a < kBlock; a += parts) acc += load_f32(src + a * d + c);
  part[t] = acc;
  __syncthreads();
  if (t < d) {
    float tot = 0.f;
    for (int j = 0; j < parts; ++j) tot += part[j * d + t];
    xbar[h * ld_bar_h + static_cast<int64_t>(b) * d + t] = tot * (1.0f / kBlock);
  }
}

// ---------------------------------------------------------------- importance
//
// One workgroup per (group of QB query blocks, head). The query means are
// reduced into LDS, key means stream through LDS 64 blocks at a time, the
// logits of the QB rows stay in LDS, and each row is soft-maxed in place.

constexpr int kScoreTile = 64;

template <typename T, int QB>
__global__ __launch_bounds__(256) void route_scores_kernel(const T* __restrict__ q, int64_t ld_q_h,
                                                           const float* __restrict__ kbar,
                                                           int64_t ld_kbar_h, int N, int M, int d,
                                                           float scale, float* __restrict__ p) {
  extern __shared__ float smem[];
  float* qbar = smem;                              // [QB][d]
  float* ktile = qbar + QB * d;                    // [64][d + 1]
  float* logit = ktile + kScoreTile * (d + 1);     // [QB][M]
  float* red = logit + QB * M;                     // [256]
  const int h = blockIdx.y, i0 = blockIdx.x * QB, t = threadIdx.x;
  const int nq = min(QB, N - i0);

  // 1. query block means
  const int parts = 256 / d, c = t % d, s = t / d;
  for (int qb = 0; qb < nq; ++qb) {
    const T* src = q + h * ld_q_h + static_cast<int64_t>(i0 + qb) * kBlock * d;
    float acc = 0.f;
    for (int a = s; a < kBlock; a += parts) acc += load_f32(src + a * d + c);
    red[t] = acc;
    __syncthreads();
    if (t < d) {
      float tot = 0.f;
      for (int j = 0; j < parts; ++j) tot += red[j * d + t];
      qbar[qb * d + t] = tot * (1.0f / kBlock);
    }
    __syncthreads();
  }

  // 2. logits = scale * qbar . kbar
  const float* kb = kbar + h * ld_kbar_h;
  const int rr = t % kScoreTile, grp = t / kScoreTile;  // grp is the wave index
  for (int r0 = 0; r0 < M; r0 += kScoreTile) {
    const int nr = min(kScoreTile, M - r0);
    for (int e = t; e < nr * d; e += 256) {
      const int er = e / d, ec = e % d;
      ktile[er * (d + 1) + ec] = kb[static_cast<int64_t>(r0 + er) * d + ec];
    }
    __syncthreads();
    if (rr < nr) {
      for (int qb = grp; qb < nq; qb += 4) {
        float acc = 0.f;
        const float* qv = qbar + qb * d;
        const float* kv = ktile + rr * (d + 1);
        for (int cc = 0; cc < d; ++cc) acc = fmaf(qv[cc], kv[cc], acc);
        logit[qb * M + r0 + rr] = acc * scale;
      }
    }
    __syncthreads();
  }

  // 3. softmax over the history blocks of each row
  for (int qb = 0; qb < nq; ++qb) {
    float* lr = logit + qb * M;
    float mx = -INFINITY;
    for (int r = t; r < M; r += 256) mx = fmaxf(mx, lr[r]);
    mx = block_max(mx, red);
    float sum = 0.f;
    for (int r = t; r < M; r += 256) {
      const float e = expf(lr[r] - mx);
      lr[r] = e;
      sum += e;
    }
    sum = block_sum(sum, red);
    float* out = p + (static_cast<int64_t>(h) * N + i0 + qb) * M;
    for (int r = t; r < M; r += 256) out[r] = lr[r] / sum;
  }
}

// ---------------------------------------------------------------- route select
//
// One workgroup (512 threads) per (query block, head).
//  1. fused weight w (fp32, one rounding per operation), fixed-point mass W,
//     total Z and reserved mass; sort key = (~bits(w) << 32) | id so that an
//     ascending sort ranks by w descending, then id ascending (w >= 0).
//  2. bitonic sort of the keys in LDS.
//  3. count c of taken candidates: the cap, or the first prefix whose mass
//     meets the threshold (block-wide scan of the sorted masses).
//  4. route = reserved ∪ first c ∪ safeguards as an LDS bitmask; emit ascending.

struct SelectArgs {
  const float* p;
  const float* g;
  const float* rho;
  const int32_t* coord;
  const int32_t* ref_ids;
  int32_t* route_ids;
  int32_t* route_len;
  int N, M, L, P2, nwords;
  float tau, g_ref, lambda, eta_cov, theta_cov, theta_unc;
  int K_cov, K_unc, n_prev, neigh26, n_ref;
};

constexpr int kSelectThreads = 512;

__device__ __forceinline__ uint64_t fixed_mass(float w) {
  // w * 2^60 is exact in double (24-bit significand, power-of-two scale);
  // conversion truncates, i.e. floors, for w >= 0.
  return static_cast<uint64_t>(static_cast<double>(w) * 0x1p60);
}

__device__ __forceinline__ float key_weight(uint64_t key) {
  return __uint_as_float(~static_cast<uint32_t>(key >> 32));
}

// (m * 2^24 >= thq * Z) in 128-bit integers.
__device__ __forceinline__ bool mass_reached(uint64_t m, uint64_t thq, uint64_t Z) {
  const uint64_t lhs_hi = m >> 40, lhs_lo = m << 24;
  const uint64_t rhs_lo = thq * Z, rhs_hi = __umul64hi(thq, Z);
  return lhs_hi > rhs_hi || (lhs_hi == rhs_hi && lhs_lo >= rhs_lo);
}

__global__ __launch_bounds__(kSelectThreads) void route_select_kernel(SelectArgs a) {
  extern __shared__ uint64_t sel_smem[];
  uint64_t* keys = sel_smem;                                      // [P2]
  uint64_t* red64 = keys + a.P2;                                  // [2 * 8 waves]
  uint32_t* mask = reinterpret_cast<uint32_t*>(red64 + 16);       // [nwords]
  int* wscan = reinterpret_cast<int*>(mask + a.nwords);           // [8 waves + 2]

  const int i = blockIdx.x, h = blockIdx.y, t = threadIdx.x, nt = blockDim.x;
  const int lane = t % kWave, wv = t / kWave, nwv = nt / kWave;
  const int M = a.M;
  const float* prow = a.p + (static_cast<int64_t>(h) * a.N + i) * M;
  const float* grow = a.g + static_cast<int64_t>(i) * M;
  const bool covered = a.rho[i] >= a.eta_cov;
  const int n_res = min(a.n_prev, M);
  const int res0 = M - n_res;

  for (int wd = t; wd < a.nwords; wd += nt) mask[wd] = 0u;

  // 1. weights, masses, keys
  uint64_t zloc = 0, mloc = 0;
  for (int r = t; r < a.P2; r += nt) {
    uint64_t key = ~0ull;
    if (r < M) {
      float w = prow[r];
      if (covered) {
        const float g = grow[r];
        const float gh = (g > a.tau) ? fminf(__fdiv_rn(g, a.g_ref), 1.0f) : 0.0f;
        const float u = __fadd_rn(1.0f, __fmul_rn(a.lambda, gh));
        w = __fmul_rn(w, u);
      }
      const uint64_t W = fixed_mass(w);
      zloc += W;
      if (r >= res0)
        mloc += W;
      else
        key = (static_cast<uint64_t>(~__float_as_uint(w)) << 32) | static_cast<uint32_t>(r);
    }
    keys[r] = key;
  }
  zloc = wave_sum_u64(zloc);
  mloc = wave_sum_u64(mloc);
  if (lane == 0) {
    red64[wv] = zloc;
    red64[8 + wv] = mloc;
  }
  __syncthreads();
  uint64_t Z = 0, m0 = 0;
  for (int j = 0; j < nwv; ++j) {
    Z += red64[j];
    m0 += red64[8 + j];
  }

  // 2. bitonic sort, ascending
  for (int k = 2; k <= a.P2; k <<= 1) {
    for (int j = k >> 1; j > 0; j >>= 1) {
      for (int e = t; e < (a.P2 >> 1); e += nt) {
        const int lo = 2 * e - (e & (j - 1));
        const int hi = lo + j;
        const uint64_t x = keys[lo], y = keys[hi];
        const bool up = (lo & k) == 0;
        if ((x > y) == up) {
          keys[lo] = y;
          keys[hi] = x;
        }
      }
      __syncthreads();
    }
  }

  // 3. number of candidates taken after the reservation
  const int K = covered ? a.K_cov : a.K_unc;
  const float theta = covered ? a.theta_cov : a.theta_unc;
  const int limit = max(0, min(K - n_res, M - n_res));
  int c = limit;
  if (theta < 1.0f && limit > 0) {
    const uint64_t thq = static_cast<uint64_t>(static_cast<double>(theta) * 0x1p24);
    if (t == 0) wscan[nwv] = limit;
    __syncthreads();
    uint64_t carry = m0;
    for (int base = 0; base < limit; base += nt) {
      const int j = base + t;
      const uint64_t Wj = j < limit ? fixed_mass(key_weight(keys[j])) : 0ull;
      // inclusive scan of Wj over the workgroup
      uint64_t incl = Wj;
#pragma unroll
      for (int o = 1; o < kWave; o <<= 1) {
        const uint64_t v = __shfl_up(incl, o);
        if (lane >= o) incl += v;
      }
      if (lane == kWave - 1) red64[wv] = incl;
      __syncthreads();
      uint64_t before = 0, total = 0;
      for (int w2 = 0; w2 < nwv; ++w2) {
        if (w2 < wv) before += red64[w2];
        total += red64[w2];
      }
      const uint64_t mass_before_j = carry + before + incl - Wj;
      if (j < limit && mass_reached(mass_before_j, thq, Z)) atomicMin(&wscan[nwv], j);
      carry += total;
      __syncthreads();
      if (wscan[nwv] < limit) break;  // uniform: read after the barrier
    }
    c = wscan[nwv];
  }

  // 4. bitmask: reserved, selected, safeguards
  for (int r = res0 + t; r < M; r += nt) atomicOr(&mask[r >> 5], 1u << (r & 31));
  for (int j = t; j < c; j += nt) {
    const uint32_t r = static_cast<uint32_t>(keys[j]);
    atomicOr(&mask[r >> 5], 1u << (r & 31));
  }
  if (a.neigh26) {
    const int32_t* qc = a.coord + 3 * static_cast<int64_t>(M + i);
    const int qt = qc[0], qh = qc[1], qw = qc[2];
    for (int r = t; r < M; r += nt) {
      const int32_t* rc = a.coord + 3 * static_cast<int64_t>(r);
      const int dist = max(abs(rc[0] - qt), max(abs(rc[1] - qh), abs(rc[2] - qw)));
      if (dist == 1) atomicOr(&mask[r >> 5], 1u << (r & 31));
    }
  }
  for (int j = t; j < a.n_ref; j += nt) {
    const int r = a.ref_ids[j];
    if (r >= 0 && r < M) atomicOr(&mask[r >> 5], 1u << (r & 31));
  }
  __syncthreads();

  // 5. ascending emission: exclusive scan of per-word popcounts
  int32_t* out = a.route_ids + (static_cast<int64_t>(h) * a.N + i) * a.L;
  int carry_cnt = 0;
  for (int base = 0; base < a.nwords; base += nt) {
    const int wd = base + t;
    const uint32_t bits = wd < a.nwords ? mask[wd] : 0u;
    const int cnt = __popc(bits);
    int incl = cnt;
#pragma unroll
    for (int o = 1; o < kWave; o <<= 1) {
      const int v = __shfl_up(incl, o);
      if (lane >= o) incl += v;
    }
    if (lane == kWave - 1) wscan[wv] = incl;
    __syncthreads();
    int before = 0, total = 0;
    for (int w2 = 0; w2 < nwv; ++w2) {
      if (w2 < wv) before += wscan[w2];
      total += wscan[w2];
    }
    int pos = carry_cnt + before + incl - cnt;
    uint32_t b = bits;
    while (b) {
      const int bit = __ffs(b) - 1;
      b &= b - 1;
      if (pos < a.L) out[pos] = wd * 32 + bit;
      ++pos;
    }
    carry_cnt += total;
    __syncthreads();
  }
  for (int s = carry_cnt + t; s < a.L; s += nt) out[s] = -1;
  if (t == 0) a.route_len[static_cast<int64_t>(h) * a.N + i] = min(carry_cnt, a.L);
}

// ---------------------------------------------------------------- launchers

static int next_pow2(int x) {
  int p = 1;
  while (p < x) p <<= 1;
  return p;
}

hipError_t launch_block_mean(const void* x, bool bf16, int64_t ld_x_h, int H, int nblk, int d,
                             float* xbar, int64_t ld_bar_h, hipStream_t stream) {
  dim3 grid(nblk, H);
  if (bf16)
    hipLaunchKernelGGL(block_mean_kernel<bf16_t>, grid, dim3(256), 0, stream,
                       static_cast<const bf16_t*>(x), ld_x_h, d, xbar, ld_bar_h);
  else
    hipLaunchKernelGGL(block_mean_kernel<float>, grid, dim3(256), 0, stream,
                       static_cast<const float*>(x), ld_x_h, d, xbar, ld_bar_h);
  return hipGetLastError();
}

size_t route_scores_lds_bytes(int qb, int M, int d) {
  return sizeof(float) * (static_cast<size_t>(qb) * d + kScoreTile * (d + 1) +
                          static_cast<size_t>(qb) * M + 256);
}

template <typename T, int QB>
static hipError_t scores_launch(const void* q, int64_t ld_q_h, const float* kbar,
                                int64_t ld_kbar_h, int H, int N, int M, int d, float scale,
                                float* p, hipStream_t stream) {
  const size_t lds = route_scores_lds_bytes(QB, M, d);
  auto kern = route_scores_kernel<T, QB>;
  hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                     hipFuncAttributeMaxDynamicSharedMemorySize,
                                     static_cast<int>(lds));
  if (e != hipSuccess) return e;
  dim3 grid((N + QB - 1) / QB, H);
  hipLaunchKernelGGL(kern, grid, dim3(256), lds, stream, static_cast<const T*>(q), ld_q_h, kbar,
                     ld_kbar_h, N, M, d, scale, p);
  return hipGetLastError();
}

hipError_t launch_route_scores(const void* q, bool bf16, int64_t ld_q_h, const float* kbar,
                               int64_t ld_kbar_h, int H, int N, int M, int d, float scale,
                               float* p, hipStream_t stream) {
  const bool wide = route_scores_lds_bytes(4, M, d) <= kMaxLdsBytes;
  if (bf16)
    return wide ? scores_launch<bf16_t, 4>(q, ld_q_h, kbar, ld_kbar_h, H, N, M, d, scale, p, stream)
                : scores_launch<bf16_t, 1>(q, ld_q_h, kbar, ld_kbar_h, H, N, M, d, scale, p, stream);
  return wide ? scores_launch<float, 4>(q, ld_q_h, kbar, ld_kbar_h, H, N, M, d, scale, p, stream)
              : scores_launch<float, 1>(q, ld_q_h, kbar, ld_kbar_h, H, N, M, d, scale, p, stream);
}

size_t route_select_lds_bytes(int M) {
  const int P2 = next_pow2(M > 0 ? M : 1);
  const int nwords = (M + 31) / 32;
  return sizeof(uint64_t) * (P2 + 16) + sizeof(uint32_t) * nwords + sizeof(int) * 16;
}

hipError_t launch_route_select(const float* p, const float* g, const float* rho,
                               const int32_t* coord, int H, int N, int M, const RouteConfig& cfg,
                               int L, int32_t* route_ids, int32_t* route_len,
                               hipStream_t stream) {
  SelectArgs a;
  a.p = p;
  a.g = g;
  a.rho = rho;
  a.coord = coord;
  a.ref_ids = cfg.ref_ids;
  a.route_ids = route_ids;
  a.route_len = route_len;
  a.N = N;
  a.M = M;
  a.L = L;
  a.P2 = next_pow2(M > 0 ? M : 1);
  a.nwords = (M + 31) / 32;
  a.tau = cfg.tau;
  a.g_ref = cfg.g_ref;
  a.lambda = cfg.lambda;
  a.eta_cov = cfg.eta_cov;
  a.theta_cov = cfg.theta_cov;
  a.theta_unc = cfg.theta_unc;
  a.K_cov = cfg.K_cov;
  a.K_unc = cfg.K_unc;
  a.n_prev = cfg.n_prev;
  a.neigh26 = cfg.neigh26;
  a.n_ref = cfg.n_ref;
  const size_t lds = route_select_lds_bytes(M);
  hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(route_select_kernel),
                                     hipFuncAttributeMaxDynamicSharedMemorySize,
                                     static_cast<int>(lds));
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(route_select_kernel, dim3(N, H), dim3(kSelectThreads), lds, stream, a);
  return hipGetLastError();
}

}  // namespace velox
