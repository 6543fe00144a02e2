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

#include <type_traits>

#include "velox_device.hpp"
#include "velox_launch.hpp"

namespace velox {

// ---------------------------------------------------------------- reductions

// Wave-wide all-reduce without LDS: DPP within quads and 16-lane rows, then
// the row and half-wave swaps (every lane ends with the result). Called with
// all 64 lanes active.
template <typename Op>
__device__ __forceinline__ float wave_allreduce(float v, float identity, Op op) {
  auto dpp = [&](float x, auto ctrl) {
    return __int_as_float(__builtin_amdgcn_update_dpp(__float_as_int(identity), __float_as_int(x),
                                                      decltype(ctrl)::value, 0xf, 0xf, false));
  };
  v = op(v, dpp(v, std::integral_constant<int, 0xB1>{}));   // quad_perm [1, 0, 3, 2]
  v = op(v, dpp(v, std::integral_constant<int, 0x4E>{}));   // quad_perm [2, 3, 0, 1]
  v = op(v, dpp(v, std::integral_constant<int, 0x124>{}));  // row_ror:4
  v = op(v, dpp(v, std::integral_constant<int, 0x128>{}));  // row_ror:8
  const auto r16 = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  v = op(__uint_as_float(r16[0]), __uint_as_float(r16[1]));
  const auto r32 = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return op(__uint_as_float(r32[0]), __uint_as_float(r32[1]));
}
__device__ __forceinline__ float wave_max(float v) {
  return wave_allreduce(v, -INFINITY, [](float a, float b) { return fmaxf(a, b); });
}
__device__ __forceinline__ float wave_sum(float v) {
  return wave_allreduce(v, 0.f, [](float a, float b) { return a + b; });
}
__device__ __forceinline__ uint64_t wave_sum_u64(uint64_t v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
  return v;
}

// Sum over aligned groups of G lanes (G = 16 or 8), every lane receiving its
// group's total: DPP adds within quads, then across quads of the 16-lane row
// (rotations by 4 and 8) or of the 8-lane half row (mirror).
template <int G>
__device__ __forceinline__ float group_sum(float v) {
  static_assert(G == 16 || G == 8, "group of 8 or 16 lanes");
  auto add_dpp = [](float x, auto ctrl) {
    const int y = __builtin_amdgcn_update_dpp(0, __float_as_int(x), decltype(ctrl)::value, 0xf, 0xf, false);
    return x + __int_as_float(y);
  };
  v = add_dpp(v, std::integral_constant<int, 0xB1>{});   // quad_perm [1, 0, 3, 2]
  v = add_dpp(v, std::integral_constant<int, 0x4E>{});   // quad_perm [2, 3, 0, 1]
  if constexpr (G == 16) {
    v = add_dpp(v, std::integral_constant<int, 0x124>{});  // row_ror:4
    v = add_dpp(v, std::integral_constant<int, 0x128>{});  // row_ror:8
  } else {
    v = add_dpp(v, std::integral_constant<int, 0x141>{});  // row_half_mirror
  }
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

// Workgroup barrier that waits only for this wave's LDS (and scalar memory)
// operations: global loads in flight are waited for where their registers are
// used, not at every barrier.
__device__ __forceinline__ void lds_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

// ---------------------------------------------------------------- block means

// One workgroup (256 threads) per (block, head). Each thread reads 16-byte
// vectors of one column group from 128 / (256 / vpr) rows (vpr = vectors per
// row; all of them requested before the first is added), then the row groups
// are summed through LDS. Summation order: per thread over its rows in
// ascending order, then over row groups in ascending order.
template <typename T, int D>
__global__ __launch_bounds__(256) void block_mean_kernel(const T* __restrict__ x, int64_t ld_x_h,
                                                         float* __restrict__ xbar, int64_t ld_bar_h,
                                                         int64_t ld_bar_row) {
  constexpr int V = 16 / sizeof(T);  // elements per 16-byte vector
  constexpr int kVpr = D / V, kGroups = 256 / kVpr, kRows = kBlock / kGroups;
  __shared__ float part[256 * V];
  const int b = blockIdx.x, h = blockIdx.y, t = threadIdx.x;
  const int cv = t % kVpr, g = t / kVpr;
  const T* src = x + h * ld_x_h + static_cast<int64_t>(b) * kBlock * D + cv * V;
  uint4 u[kRows];
#pragma unroll
  for (int k = 0; k < kRows; ++k)
    u[k] = *reinterpret_cast<const uint4*>(src + static_cast<int64_t>(g + k * kGroups) * D);
  float acc[V];
#pragma unroll
  for (int e = 0; e < V; ++e) acc[e] = 0.f;
#pragma unroll
  for (int k = 0; k < kRows; ++k) {
    const uint32_t w[4] = {u[k].x, u[k].y, u[k].z, u[k].w};
    if constexpr (V == 8) {
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        acc[2 * j] += __uint_as_float(w[j] << 16);
        acc[2 * j + 1] += __uint_as_float(w[j] & 0xffff0000u);
      }
    } else {
#pragma unroll
      for (int j = 0; j < 4; ++j) acc[j] += __uint_as_float(w[j]);
    }
  }
#pragma unroll
  for (int e = 0; e < V; ++e) part[g * D + cv * V + e] = acc[e];
  __syncthreads();
  if (t < D) {
    float tot = 0.f;
    for (int j = 0; j < kGroups; ++j) tot += part[j * D + t];
    xbar[h * ld_bar_h + static_cast<int64_t>(b) * ld_bar_row + t] = tot * (1.0f / kBlock);
  }
}

// ---------------------------------------------------------------- importance
//
// One workgroup (512 threads) per (group of QB query blocks, head).
//  1. query block means: 16-byte loads of all QB blocks issued at once, summed
//     per lane, across the row groups of a wave by lane swaps, then across
//     waves in LDS. The first history rows of step 2 are requested before that
//     reduction, so their latency overlaps it.
//  2. logits: a group of 8 lanes shares each history row (each 16-byte load
//     instruction reads whole 128-byte lines of kbar[h][r], the next rows in
//     flight while the current ones are summed); each lane dots its D / 8
//     dims with the QB query means held in registers and DPP adds sum the
//     group. Logits of the QB rows stay in LDS; each lane keeps the running
//     maximum of the logits it wrote. (With M >= D the query means of step 1
//     come from a block-mean launch instead, read back from the output rows.)
//  3. softmax over the history blocks of each row (all QB rows reduced
//     together), written coalesced: exp through the hardware exp2 and one
//     reciprocal per row (within a few float32 ulps of the correctly rounded
//     values).

constexpr int kScoreThreads = 512;

template <typename T>
__device__ __forceinline__ void load8(const T* p, float (&x)[8]);
template <>
__device__ __forceinline__ void load8<bf16_t>(const bf16_t* p, float (&x)[8]) {
  const uint4 u = *reinterpret_cast<const uint4*>(p);
  const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    x[2 * j] = __uint_as_float(w[j] << 16);
    x[2 * j + 1] = __uint_as_float(w[j] & 0xffff0000u);
  }
}
template <>
__device__ __forceinline__ void load8<float>(const float* p, float (&x)[8]) {
  const float4 a = *reinterpret_cast<const float4*>(p);
  const float4 b = *reinterpret_cast<const float4*>(p + 4);
  x[0] = a.x; x[1] = a.y; x[2] = a.z; x[3] = a.w;
  x[4] = b.x; x[5] = b.y; x[6] = b.z; x[7] = b.w;
}

// kRaw: write the scaled logits (no softmax) to p, for the head-shared scores.
// kPre: the query block means were written into the first D floats of every
// output row by a block-mean launch (rows of M >= D floats); the workgroup
// reads them back before it overwrites its rows.
template <typename T, int D, int QB, bool kRaw = false, bool kPre = false>
__global__ __launch_bounds__(kScoreThreads) void route_scores_kernel(
    const T* __restrict__ q, int64_t ld_q_h, const float* __restrict__ kbar, int64_t ld_kbar_h,
    int H, int N, int M, float scale, float* __restrict__ p) {
  constexpr int kCpr = D / 8;                      // 8-element chunks per token row
  constexpr int kGroups = kScoreThreads / kCpr;    // token-row groups
  constexpr int kPasses = kBlock / kGroups;
  constexpr int kWaves = kScoreThreads / kWave;
  extern __shared__ float smem[];
  float* qbar = smem;                              // [QB][D]
  float* red = qbar + QB * D;                      // [kWaves][QB][D] partial sums, then reductions
  float* logit = red + kWaves * QB * D;            // [QB][M]
  // one-dimensional grid of H * groups workgroups, remapped so that the
  // groups of a head share an XCD (its kbar rows are read once into that L2)
  const int groups = (N + QB - 1) / QB;
  const int wg = xcd_remap(blockIdx.x, H * groups);
  const int h = wg / groups, i0 = (wg % groups) * QB, t = threadIdx.x;
  const int nq = min(QB, N - i0);

  // history rows of step 2: a group of kLpr lanes shares a row, each lane
  // holding kDpl dims (d = 128: 8 lanes of 16 dims; d = 64: 8 of 8) as
  // float4 pieces kLpr float4 apart, so that each load instruction reads one
  // whole 128-byte line of every row (dims 4 kLpr c + 4 j8 .. + 3 in piece c)
  constexpr int kDpl = D == 128 ? 16 : 8;
  constexpr int kLpr = D / kDpl, kRpw = kWave / kLpr;
  constexpr int kRowsPerIt = kRpw * (kScoreThreads / kWave);
  constexpr int kBatch = kDpl == 16 ? 2 : 4;  // rows per lane group in flight
  const int lane = t % kWave, wv = t / kWave;
  const int j8 = lane % kLpr, rg = lane / kLpr;
  const float* kb = kbar + h * ld_kbar_h;
  auto load_row = [&](int r, float (&x)[kDpl]) {
    const float4* src =
        reinterpret_cast<const float4*>(kb + static_cast<int64_t>(min(r, M - 1)) * D + j8 * 4);
#pragma unroll
    for (int c = 0; c < kDpl / 4; ++c) {
      const float4 u = src[c * kLpr];
      x[4 * c] = u.x; x[4 * c + 1] = u.y; x[4 * c + 2] = u.z; x[4 * c + 3] = u.w;
    }
  };
  const int r_me = wv * kRpw + rg;
  float kx[kBatch][kDpl];

  if constexpr (kPre) {
    // first history rows, then the precomputed means of the group's rows
    if (M > 0) {
#pragma unroll
      for (int b = 0; b < kBatch; ++b) load_row(r_me + b * kRowsPerIt, kx[b]);
    }
    for (int x = t; x < nq * D; x += kScoreThreads)
      qbar[x] = p[(static_cast<int64_t>(h) * N + i0 + x / D) * M + x % D];
    __syncthreads();
  } else {
    // 1. query block means: 16-byte loads of all QB blocks issued at once, summed
    // per lane, across the row groups of a wave by lane swaps, then across waves
    // in LDS. Blocks past the group's last re-read the last block (no branch
    // around the loads); their sums are not stored.
    float acc[QB][8];
    {
      const int c8 = t % kCpr, grp = t / kCpr;
#pragma unroll
      for (int b = 0; b < QB; ++b) {
        const T* src = q + h * ld_q_h + static_cast<int64_t>(min(i0 + b, N - 1)) * kBlock * D + c8 * 8;
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[b][e] = 0.f;
#pragma unroll
        for (int ps = 0; ps < kPasses; ++ps) {
          float x[8];
          load8<T>(src + (ps * kGroups + grp) * D, x);
#pragma unroll
          for (int e = 0; e < 8; ++e) acc[b][e] += x[e];
        }
      }
    }
    // first history rows of step 2 (rows past the end load the last row; their
    // dot products are not stored)
    if (M > 0) {
#pragma unroll
      for (int b = 0; b < kBatch; ++b) load_row(r_me + b * kRowsPerIt, kx[b]);
    }
    {
      // the lanes of a wave holding the same chunk (lane mod kCpr) differ in
      // bits 3 (D = 64), 4 and 5: swap-and-add over those bits, ascending
      const int c8 = t % kCpr;
#pragma unroll
      for (int b = 0; b < QB; ++b)
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          float v = acc[b][e];
          if constexpr (kCpr == 8) {
            const int y = __builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x128, 0xf, 0xf, false);  // row_ror:8
            v += __int_as_float(y);
          }
          const auto r16 = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
          v = __uint_as_float(r16[0]) + __uint_as_float(r16[1]);
          const auto r32 = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
          v = __uint_as_float(r32[0]) + __uint_as_float(r32[1]);
          acc[b][e] = v;
        }
      if (lane < kCpr) {
#pragma unroll
        for (int b = 0; b < QB; ++b)
#pragma unroll
          for (int e = 0; e < 8; ++e) red[(wv * QB + b) * D + c8 * 8 + e] = acc[b][e];
      }
      __syncthreads();
      for (int x = t; x < nq * D; x += kScoreThreads) {
        const int b = x / D, d = x % D;
        float sum = 0.f;
        for (int w2 = 0; w2 < kWaves; ++w2) sum += red[(w2 * QB + b) * D + d];
        qbar[x] = sum * (1.0f / kBlock);
      }
      __syncthreads();
    }
  }

  // 2. logits. The lanes of a group share one history row: lane j8 loads its
  // kDpl dims (the group reads whole lines of the row) and dots them with the
  // same dims of every query mean, which it keeps in registers; DPP adds then
  // sum the group's partials (every lane ends with the row's dot products). The
  // loads of the next kBatch rows are issued before the arithmetic of the
  // current ones.
  float qv[QB][kDpl];
#pragma unroll
  for (int qb = 0; qb < QB; ++qb)
#pragma unroll
    for (int e = 0; e < kDpl; ++e) qv[qb][e] = qb < nq ? qbar[qb * D + (e / 4) * 4 * kLpr + j8 * 4 + e % 4] : 0.f;
  float lmax = -INFINITY;  // running maximum of the logits this lane stores
  auto dots = [&](int r0, float (&xs)[kBatch][kDpl]) {
#pragma unroll
    for (int b = 0; b < kBatch; ++b) {
      const int r = r0 + b * kRowsPerIt + r_me;
      float mine = 0.f;
#pragma unroll
      for (int qb = 0; qb < QB; ++qb) {
        float acc = 0.f;
#pragma unroll
        for (int e = 0; e < kDpl; ++e) acc = fmaf(qv[qb][e], xs[b][e], acc);
        acc = group_sum<kLpr>(acc);
        if (j8 == qb) mine = acc;
      }
      if (r < M && j8 < nq) {
        logit[j8 * M + r] = mine * scale;
        lmax = fmaxf(lmax, mine * scale);
      }
    }
  };
  // two row buffers used in turn (no register copies between steps)
  constexpr int kStep = kBatch * kRowsPerIt;
  for (int r0 = 0; r0 < M; r0 += 2 * kStep) {
    float nx[kBatch][kDpl];
#pragma unroll
    for (int b = 0; b < kBatch; ++b) load_row(r0 + kStep + b * kRowsPerIt + r_me, nx[b]);
    dots(r0, kx);
    if (r0 + kStep >= M) break;
#pragma unroll
    for (int b = 0; b < kBatch; ++b) load_row(r0 + 2 * kStep + b * kRowsPerIt + r_me, kx[b]);
    dots(r0 + kStep, nx);
  }
  __syncthreads();

  if (kRaw) {
    for (int qb = 0; qb < nq; ++qb) {
      float* out = p + (static_cast<int64_t>(h) * N + i0 + qb) * M;
      for (int r = t; r < M; r += kScoreThreads) out[r] = logit[qb * M + r];
    }
    return;
  }

  // 3. softmax over the history blocks of each row, all rows at once: maxima
  // (lanes j8 of every wave hold partial maxima of row j8), then exponentials
  // and sums, then the normalised values written coalesced (`red` is free
  // again and holds the per-wave partials)
  {
    float v = lmax;
    if constexpr (kRpw == 8) {
      const int y = __builtin_amdgcn_update_dpp(__float_as_int(-INFINITY), __float_as_int(v), 0x128, 0xf, 0xf, false);
      v = fmaxf(v, __int_as_float(y));
    }
    const auto r16 = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    v = fmaxf(__uint_as_float(r16[0]), __uint_as_float(r16[1]));
    const auto r32 = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    v = fmaxf(__uint_as_float(r32[0]), __uint_as_float(r32[1]));
    if (lane < kLpr) red[wv * kLpr + lane] = v;
  }
  __syncthreads();
  float mx[QB];
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    float m = red[qb];
    for (int w2 = 1; w2 < kWaves; ++w2) m = fmaxf(m, red[w2 * kLpr + qb]);
    mx[qb] = m;
  }
  __syncthreads();
  float sm[QB];
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    sm[qb] = 0.f;
    if (qb < nq) {
      float* lr = logit + qb * M;
      for (int r = t; r < M; r += kScoreThreads) {
        const float e = __expf(lr[r] - mx[qb]);
        lr[r] = e;
        sm[qb] += e;
      }
    }
    sm[qb] = wave_sum(sm[qb]);
    if (lane == 0) red[qb * kWaves + wv] = sm[qb];
  }
  __syncthreads();
  for (int qb = 0; qb < nq; ++qb) {
    float sum = red[qb * kWaves];
    for (int w2 = 1; w2 < kWaves; ++w2) sum += red[qb * kWaves + w2];
    const float inv = 1.0f / sum;
    const float* lr = logit + qb * M;
    float* out = p + (static_cast<int64_t>(h) * N + i0 + qb) * M;
    for (int r = t; r < M; r += kScoreThreads) out[r] = lr[r] * inv;
  }
}

// ---------------------------------------------------------------- head-shared importance
//
// One workgroup per query block: the mean over heads (ascending h, then one
// division by H) of the per-head scaled logits, then the softmax over the
// history blocks, as in route_scores_kernel.
__global__ __launch_bounds__(kScoreThreads) void head_mean_softmax_kernel(
    const float* __restrict__ logits, int H, int N, int M, float* __restrict__ p) {
  extern __shared__ float smem[];
  float* red = smem;                 // [kScoreThreads / kWave]
  float* lr = smem + kScoreThreads / kWave;
  const int i = blockIdx.x, t = threadIdx.x;
  const float fH = static_cast<float>(H);
  for (int r = t; r < M; r += kScoreThreads) {
    float s = 0.f;
    for (int h = 0; h < H; ++h) s += logits[(static_cast<int64_t>(h) * N + i) * M + r];
    lr[r] = __fdiv_rn(s, fH);
  }
  __syncthreads();
  float mx = -INFINITY;
  for (int r = t; r < M; r += kScoreThreads) mx = fmaxf(mx, lr[r]);
  mx = block_max(mx, red);
  float sum = 0.f;
  for (int r = t; r < M; r += kScoreThreads) {
    const float e = expf(lr[r] - mx);
    lr[r] = e;
    sum += e;
  }
  sum = block_sum(sum, red);
  float* out = p + static_cast<int64_t>(i) * M;
  for (int r = t; r < M; r += kScoreThreads) out[r] = lr[r] / sum;
}

// ---------------------------------------------------------------- route select
//
// One workgroup (256 threads) per (query block, head); LDS is sized by the
// largest cap of the call, so that all rows of a call fit on the GPU at once.
//  1. fused weight w (fp32, one rounding per operation), fixed-point mass W,
//     total Z and reserved mass; sort key = (~bits(w) << 32) | id so that
//     ascending key order ranks by w descending, then id ascending (w >= 0);
//     the keys are distinct.
//  2. the `limit` smallest keys (limit = the cap): a radix select, 8 bits at a
//     time from the top, finds the bucket of the limit-th smallest key (the
//     first histogram, of the top byte, is made while the keys are built), the
//     keys up to it are gathered and, when a mass cut follows, put in order by
//     counting for each the keys below it. (A cap above kFastSel falls back to
//     a bitonic sort of all keys.)
//  3. count c of taken candidates: the cap, or the first prefix whose mass
//     meets the threshold (block-wide scan of the ordered masses).
//  4. route = reserved ∪ first c ∪ safeguards as an LDS bitmask; emit ascending
//     (every set bit writes its id at its rank among the set bits).
// Inputs outside what the fixed-point mass allows are reported per row in the
// optional status word: an entry of p that is negative, NaN or infinite, an
// entry of g outside [0, 1] (NaN included), or, on a row with a mass cut, a
// total sum_r floor(w_r 2^60) that does not fit in 64 bits (impossible when the
// row's p sums to at most 1 + 2^-10 and lambda <= 14). Such a row still gets
// an in-range ascending route, computed from saturated masses.

struct SelectArgs {
  const float* p;
  const float* g;
  const float* rho;
  const int32_t* coord;
  const int32_t* ref_ids;
  int32_t* route_ids;
  int32_t* route_len;
  int32_t* status;  // nullable: [0] rows with bad inputs, [1] smallest such row
  int N, M, L, P2, nwords;
  int fs;  // capacity of the selected-key buffers: the largest radix-select cap
  int vec;  // rows read as 16-byte vectors: M % 4 == 0, p, g (and coord) 16-byte aligned
  float tau, g_ref, lambda, eta_cov, theta_cov, theta_unc;
  int K_cov, K_unc, n_prev, neigh26, n_ref, mode;
};

// Route modes of a covered row (uncovered rows always use the model's p):
//   0 fused:          w = p (1 + lambda ghat)          (the method)
//   1 model only:     w = p                            (same budgets, no geometry)
//   2 geometry only:  w = g, top-K_cov, no mass cut    (hard geometric top-K)

constexpr int kSelectThreads = 256;
constexpr int kFastSel = 1024;   // largest cap served by the radix select

// Control words of the radix select, in LDS.
struct SelectCtl {
  uint64_t prefix;
  int rank, cnt, n;
};

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

// hist[bin] += number of active lanes with `on` and that bin: one LDS atomic
// per distinct bin of the wave (the top byte of the keys takes few values).
__device__ __forceinline__ void count_by_wave(int* hist, uint32_t bin, bool on) {
  uint64_t pend = __ballot(on);
  while (pend) {
    const int lead = __builtin_ffsll(static_cast<long long>(pend)) - 1;
    const uint32_t b = __builtin_amdgcn_readlane(bin, lead);
    const uint64_t same = __ballot(on && bin == b);
    if (static_cast<int>(threadIdx.x % kWave) == lead) atomicAdd(&hist[b], __popcll(same));
    pend &= ~same;
  }
}

__global__ __launch_bounds__(kSelectThreads) void route_select_kernel(SelectArgs a) {
  extern __shared__ uint64_t sel_smem[];
  const int fs = a.fs;
  uint64_t* keys = sel_smem;                                      // [P2]
  uint64_t* sel = keys + a.P2;                                    // [fs]
  uint64_t* ordered = sel + fs;                                   // [fs]
  uint64_t* red64 = ordered + fs;                                 // [3 * 8 waves + 1]
  SelectCtl* ctl = reinterpret_cast<SelectCtl*>(red64 + 25);
  int* hist = reinterpret_cast<int*>(ctl + 1);                    // [2][256]
  uint32_t* mask = reinterpret_cast<uint32_t*>(hist + 512);       // [nwords]
  int* wscan = reinterpret_cast<int*>(mask + a.nwords);           // [8 waves + 2]

  const int i = blockIdx.x, h = blockIdx.y, t = threadIdx.x, nt = blockDim.x;
  const int lane = t % kWave, wv = t / kWave, nwv = nt / kWave;
  const int M = a.M;
  const float* prow = a.p + (static_cast<int64_t>(h) * a.N + i) * M;
  const float* grow = a.g + static_cast<int64_t>(i) * M;
  const bool covered = a.rho[i] >= a.eta_cov;
  const int n_res = min(a.n_prev, M);
  const int res0 = M - n_res;

  // cleared before any use: route mask, both radix histograms, flag word, gather count
  for (int wd = t; wd < a.nwords; wd += nt) mask[wd] = 0u;
  for (int b = t; b < 512; b += nt) hist[b] = 0;
  if (t == 0) {
    red64[24] = 0;
    ctl->n = 0;
  }
  lds_barrier();

  // 1. weights, masses, keys, and the histogram of the keys' top byte (the
  // radix select's first pass). The loads of kChunk rows per thread are all
  // issued before their arithmetic, with no branch between them (rows past
  // the end re-read the last row). The 26-neighbour test of the same rows is
  // kept in `nbits` (bit k: the k-th row of this thread) and entered in the
  // mask after the next barrier; threads with more than 32 rows test later.
  constexpr int kChunk = 8;
  const bool nb_early = a.neigh26 && a.P2 <= 32 * nt;
  int qt = 0, qh = 0, qw = 0;
  if (a.neigh26) {
    const int32_t* qc = a.coord + 3 * static_cast<int64_t>(M + i);
    qt = qc[0];
    qh = qc[1];
    qw = qc[2];
  }
  // Z is summed as high and low 32-bit halves of each W (neither sum can
  // overflow for M <= 2^16), so that a total of 2^64 or more is detected.
  uint64_t zhi = 0, zlo = 0, mloc = 0;
  bool bad_in = false, big = false;
  uint32_t nbits = 0;
  // key of row r (bit k of nbits marks it a neighbour); also counted into the
  // first histogram
  auto one_key = [&](auto with_nb, int r, float pv, float gv, int cdist, int k) {
    constexpr bool kNb = decltype(with_nb)::value;
    uint64_t key = ~0ull;
    if (r < M) {
      float w = pv;
      bad_in |= !(w >= 0.f && w <= 3.402823466e38f) || !(gv >= 0.f && gv <= 1.f);
      if (covered && a.mode == 0) {
        const float gh = (gv > a.tau) ? fminf(__fdiv_rn(gv, a.g_ref), 1.0f) : 0.0f;
        const float uu = __fadd_rn(1.0f, __fmul_rn(a.lambda, gh));
        w = __fmul_rn(w, uu);
      } else if (covered && a.mode == 2) {
        w = gv;
      }
      const bool fits = w < 16.f;  // else w 2^60 >= 2^64 (NaN fails too)
      big |= !fits;
      const uint64_t W = fits ? fixed_mass(w) : ~0ull;
      zhi += W >> 32;
      zlo += W & 0xffffffffull;
      if (r >= res0)
        mloc += W;
      else
        key = (static_cast<uint64_t>(~__float_as_uint(w)) << 32) | static_cast<uint32_t>(r);
      if (kNb && cdist == 1) nbits |= 1u << k;
    }
    if (r < a.P2) keys[r] = key;
    count_by_wave(hist, static_cast<uint32_t>(key >> 56), r < M);
  };
  auto chebyshev = [&](int ct, int ch, int cw) { return max(abs(ct - qt), max(abs(ch - qh), abs(cw - qw))); };
  // rows t + u nt of each chunk, 4-byte loads (any M, any alignment)
  auto build_keys = [&](auto with_nb) {
    constexpr bool kNb = decltype(with_nb)::value;
    for (int r0 = t, k0 = 0; r0 < a.P2; r0 += kChunk * nt, k0 += kChunk) {
      float pw[kChunk], gw[kChunk];
      int cd[kChunk];  // Chebyshev distance of the row's block to the query block
#pragma unroll
      for (int u = 0; u < kChunk; ++u) {
        const int rr = min(r0 + u * nt, M - 1);
        pw[u] = prow[rr];
        gw[u] = grow[rr];
        cd[u] = 0;
        if constexpr (kNb) {
          const int32_t* rc = a.coord + 3 * static_cast<int64_t>(rr);
          cd[u] = chebyshev(rc[0], rc[1], rc[2]);
        }
      }
#pragma unroll
      for (int u = 0; u < kChunk; ++u) one_key(with_nb, r0 + u * nt, pw[u], gw[u], cd[u], k0 + u);
    }
  };
  // rows 4 t .. 4 t + 3 of each quarter chunk, 16-byte loads (M % 4 == 0,
  // aligned rows); a vector never straddles M, vectors past it re-read the last
  auto build_keys_vec = [&](auto with_nb) {
    constexpr bool kNb = decltype(with_nb)::value;
    constexpr int kVec = kChunk / 4;
    for (int c0 = 0, k0 = 0; c0 < a.P2; c0 += kChunk * nt, k0 += kChunk) {
      float4 pv[kVec], gv[kVec];
      int4 cv[kVec][3];
#pragma unroll
      for (int v = 0; v < kVec; ++v) {
        const int rb = min(c0 + v * 4 * nt + 4 * t, M - 4);
        pv[v] = *reinterpret_cast<const float4*>(prow + rb);
        gv[v] = *reinterpret_cast<const float4*>(grow + rb);
        if constexpr (kNb) {
          const int4* rc = reinterpret_cast<const int4*>(a.coord + 3 * static_cast<int64_t>(rb));
          cv[v][0] = rc[0];
          cv[v][1] = rc[1];
          cv[v][2] = rc[2];
        }
      }
#pragma unroll
      for (int v = 0; v < kVec; ++v) {
        const int r = c0 + v * 4 * nt + 4 * t;
        int cd[4] = {0, 0, 0, 0};
        if constexpr (kNb) {
          cd[0] = chebyshev(cv[v][0].x, cv[v][0].y, cv[v][0].z);
          cd[1] = chebyshev(cv[v][0].w, cv[v][1].x, cv[v][1].y);
          cd[2] = chebyshev(cv[v][1].z, cv[v][1].w, cv[v][2].x);
          cd[3] = chebyshev(cv[v][2].y, cv[v][2].z, cv[v][2].w);
        }
        one_key(with_nb, r, pv[v].x, gv[v].x, cd[0], k0 + 4 * v);
        one_key(with_nb, r + 1, pv[v].y, gv[v].y, cd[1], k0 + 4 * v + 1);
        one_key(with_nb, r + 2, pv[v].z, gv[v].z, cd[2], k0 + 4 * v + 2);
        one_key(with_nb, r + 3, pv[v].w, gv[v].w, cd[3], k0 + 4 * v + 3);
      }
    }
  };
  if (M > 0) {
    if (a.vec) {
      if (nb_early)
        build_keys_vec(std::true_type{});
      else
        build_keys_vec(std::false_type{});
    } else {
      if (nb_early)
        build_keys(std::true_type{});
      else
        build_keys(std::false_type{});
    }
  } else if (t == 0) {
    keys[0] = ~0ull;  // P2 = 1
  }
  zhi = wave_sum_u64(zhi);
  zlo = wave_sum_u64(zlo);
  mloc = wave_sum_u64(mloc);
  const bool wave_bad = __ballot(bad_in) != 0, wave_big = __ballot(big) != 0;
  if (lane == 0) {
    red64[wv] = zhi;
    red64[8 + wv] = mloc;
    red64[16 + wv] = zlo;
    if (wave_bad || wave_big)
      atomicOr(reinterpret_cast<unsigned long long*>(&red64[24]),
               (wave_bad ? 1ull : 0ull) | (wave_big ? 2ull : 0ull));
  }
  lds_barrier();  // keys, masses and the first histogram are complete
  uint64_t zh = 0, zl = 0, m0 = 0;
  for (int j = 0; j < nwv; ++j) {
    zh += red64[j];
    m0 += red64[8 + j];
    zl += red64[16 + j];
  }
  const uint64_t Z = (zh << 32) + zl;  // modulo 2^64
  const bool z_overflow = (red64[24] & 2ull) != 0 || zh + (zl >> 32) >= (1ull << 32);
  const bool input_bad = (red64[24] & 1ull) != 0;
  while (nbits) {
    const int k = __ffs(nbits) - 1;
    nbits &= nbits - 1;
    const int r = a.vec ? (k / kChunk) * kChunk * nt + ((k % kChunk) / 4) * 4 * nt + 4 * t + (k % 4) : t + k * nt;
    atomicOr(&mask[r >> 5], 1u << (r & 31));
  }

  // caps of this row
  const int K = covered ? a.K_cov : a.K_unc;
  // geometry-only rows take the plain top-K (overlaps are not a distribution)
  const float theta = covered ? (a.mode == 2 ? 1.0f : a.theta_cov) : a.theta_unc;
  const int limit = max(0, min(K - n_res, M - n_res));
  const bool cut = theta < 1.0f && limit > 0;
  if (a.status && t == 0 && (input_bad || (cut && z_overflow))) {
    atomicAdd(&a.status[0], 1);
    atomicMin(&a.status[1], h * a.N + i);
  }

  // 2. the `limit` smallest keys, in `top` (ascending when cut)
  const uint64_t* top = keys;
  if (limit <= kFastSel) {
    uint64_t prefix = 0;
    int shift = 64;
    if (limit > 0) {
      int rank = limit - 1;  // rank of the wanted key inside the current bucket
      // pass p counts into hist[p & 1] and clears the other buffer for pass
      // p + 1 (its last reader, the scan of pass p - 1, ended at a barrier)
      for (int pass = 0; pass < 8; ++pass) {
        shift -= 8;
        int* hc = hist + 256 * (pass & 1);
        if (pass > 0) {
          int* hn = hist + 256 * ((pass + 1) & 1);
          for (int b = t; b < 256; b += nt) hn[b] = 0;
          for (int r = t; r < M; r += nt) {
            const uint64_t key = keys[r];
            if ((key >> (shift + 8)) == (prefix >> (shift + 8))) atomicAdd(&hc[(key >> shift) & 255], 1);
          }
          lds_barrier();
        }
        if (wv == 0) {  // lane l scans bins 4 l .. 4 l + 3
          int c4[4], sum = 0;
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            c4[q] = hc[4 * lane + q];
            sum += c4[q];
          }
          int incl = sum;
#pragma unroll
          for (int o = 1; o < kWave; o <<= 1) {
            const int v = __shfl_up(incl, o);
            if (lane >= o) incl += v;
          }
          int before = incl - sum;
          if (before <= rank && rank < incl) {
#pragma unroll
            for (int q = 0; q < 4; ++q) {
              if (rank >= before && rank < before + c4[q]) {
                ctl->prefix = prefix | (static_cast<uint64_t>(4 * lane + q) << shift);
                ctl->rank = rank - before;
                ctl->cnt = c4[q];
              }
              before += c4[q];
            }
          }
        }
        lds_barrier();
        prefix = ctl->prefix;
        rank = ctl->rank;
        if (rank == ctl->cnt - 1) break;  // the whole bucket is taken (uniform)
      }
    }
    // gather the keys whose top 64 - shift bits do not exceed the bucket's:
    // exactly `limit` of them; one slot reservation per wave and row batch
    if (limit > 0) {
      for (int r = t; r < M; r += nt) {
        const uint64_t key = keys[r];
        const bool take = key != ~0ull && (key >> shift) <= (prefix >> shift);
        const uint64_t bal = __ballot(take);
        if (bal != 0) {
          const int lead = __builtin_ffsll(static_cast<long long>(bal)) - 1;
          int base = 0;
          if (lane == lead) base = atomicAdd(&ctl->n, __popcll(bal));
          base = __builtin_amdgcn_readlane(base, lead);
          const int below = __builtin_amdgcn_mbcnt_hi(static_cast<uint32_t>(bal >> 32),
                                                      __builtin_amdgcn_mbcnt_lo(static_cast<uint32_t>(bal), 0));
          if (take) sel[base + below] = key;
        }
      }
    }
    lds_barrier();
    top = sel;
    if (cut) {  // ascending order: each key's position is the number of keys below it
      for (int e = t; e < limit; e += nt) {
        const uint64_t key = sel[e];
        int pos = 0;
        for (int u = 0; u < limit; ++u) pos += sel[u] < key;
        ordered[pos] = key;
      }
      __syncthreads();
      top = ordered;
    }
  } else {
    // all keys in ascending order (bitonic sort)
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
  }

  // 3. number of candidates taken after the reservation
  int c = limit;
  if (cut) {
    const uint64_t thq = static_cast<uint64_t>(static_cast<double>(theta) * 0x1p24);
    if (t == 0) wscan[nwv] = limit;
    __syncthreads();
    uint64_t carry = m0;
    for (int base = 0; base < limit; base += nt) {
      const int j = base + t;
      const float wj = j < limit ? key_weight(top[j]) : 0.f;
      const uint64_t Wj = wj < 16.f ? fixed_mass(wj) : ~0ull;
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
    const uint32_t r = static_cast<uint32_t>(top[j]);
    atomicOr(&mask[r >> 5], 1u << (r & 31));
  }
  if (a.neigh26 && !nb_early) {
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

  // 5. ascending emission: exclusive prefix of the words' popcounts (in the
  // key buffer, free now), then every set bit writes its id at its rank: the
  // prefix of its word plus the set bits below it in the word.
  int32_t* out = a.route_ids + (static_cast<int64_t>(h) * a.N + i) * a.L;
  int* wpre = reinterpret_cast<int*>(keys);  // [nwords]
  int carry_cnt = 0;
  for (int base = 0; base < a.nwords; base += nt) {
    const int wd = base + t;
    const int cnt = wd < a.nwords ? __popc(mask[wd]) : 0;
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
    if (wd < a.nwords) wpre[wd] = carry_cnt + before + incl - cnt;
    carry_cnt += total;
    __syncthreads();
  }
  for (int b = t; b < a.nwords * 32; b += nt) {
    const uint32_t bits = mask[b >> 5];
    if ((bits >> (b & 31)) & 1u) {
      const int sl = wpre[b >> 5] + __popc(bits & ((1u << (b & 31)) - 1u));
      if (sl < a.L) out[sl] = b;
    }
  }
  for (int sl = carry_cnt + t; sl < a.L; sl += nt) out[sl] = -1;
  if (t == 0) a.route_len[static_cast<int64_t>(h) * a.N + i] = min(carry_cnt, a.L);
}

// ---------------------------------------------------------------- route check
//
// One wave per route row: the row is valid when 0 <= len <= L and its first
// len ids are strictly ascending and inside [0, M). bad[0] counts invalid
// rows, bad[1] keeps the smallest invalid row index (h * N + i).

__global__ __launch_bounds__(256) void route_check_init_kernel(int32_t* bad, int rows) {
  if (threadIdx.x == 0 && blockIdx.x == 0) {
    bad[0] = 0;
    bad[1] = rows;
  }
}

__global__ __launch_bounds__(256) void route_check_kernel(const int32_t* __restrict__ ids,
                                                          const int32_t* __restrict__ len, int rows,
                                                          int M, int L, int32_t* bad) {
  const int row = blockIdx.x * (256 / kWave) + threadIdx.x / kWave;
  const int lane = threadIdx.x % kWave;
  if (row >= rows) return;
  const int n = len[row];
  bool ok = n >= 0 && n <= L;
  if (ok) {
    const int32_t* r = ids + static_cast<int64_t>(row) * L;
    for (int j = lane; j < n; j += kWave) {
      const int id = r[j];
      if (id < 0 || id >= M || (j > 0 && r[j - 1] >= id)) ok = false;
    }
  }
  if (__ballot(!ok) != 0 && lane == 0) {
    atomicAdd(&bad[0], 1);
    atomicMin(&bad[1], row);
  }
}

// ---------------------------------------------------------------- launchers

static int next_pow2(int x) {
  int p = 1;
  while (p < x) p <<= 1;
  return p;
}

template <typename T, int D>
static void block_mean_launch(const void* x, int64_t ld_x_h, int H, int nblk, float* xbar,
                              int64_t ld_bar_h, int64_t ld_bar_row, hipStream_t stream) {
  hipLaunchKernelGGL((block_mean_kernel<T, D>), dim3(nblk, H), dim3(256), 0, stream, static_cast<const T*>(x),
                     ld_x_h, xbar, ld_bar_h, ld_bar_row);
}

hipError_t launch_block_mean(const void* x, bool bf16, int64_t ld_x_h, int H, int nblk, int d,
                             float* xbar, int64_t ld_bar_h, hipStream_t stream) {
  if (bf16) {
    if (d == 128)
      block_mean_launch<bf16_t, 128>(x, ld_x_h, H, nblk, xbar, ld_bar_h, d, stream);
    else
      block_mean_launch<bf16_t, 64>(x, ld_x_h, H, nblk, xbar, ld_bar_h, d, stream);
  } else {
    if (d == 128)
      block_mean_launch<float, 128>(x, ld_x_h, H, nblk, xbar, ld_bar_h, d, stream);
    else
      block_mean_launch<float, 64>(x, ld_x_h, H, nblk, xbar, ld_bar_h, d, stream);
  }
  return hipGetLastError();
}

size_t route_scores_lds_bytes(int qb, int M, int d) {
  const int waves = kScoreThreads / kWave;
  return sizeof(float) * (static_cast<size_t>(qb) * d + static_cast<size_t>(waves) * qb * d +
                          static_cast<size_t>(qb) * M);
}

// With M >= d the query block means come from a block-mean launch of their
// own (one workgroup per block: far more loads in flight than the scoring
// workgroups have) that writes them into the first d floats of each output
// row; the scoring workgroup of the row reads them before overwriting it.
template <typename T, int D, int QB, bool kRaw>
static hipError_t scores_launch(const void* q, int64_t ld_q_h, const float* kbar,
                                int64_t ld_kbar_h, int H, int N, int M, float scale, float* p,
                                hipStream_t stream) {
  const size_t lds = route_scores_lds_bytes(QB, M, D);
  const bool pre = M >= D;
  if (pre) {
    block_mean_launch<T, D>(q, ld_q_h, H, N, p, static_cast<int64_t>(N) * M, static_cast<int64_t>(M), stream);
    const hipError_t e0 = hipGetLastError();
    if (e0 != hipSuccess) return e0;
  }
  auto kern = pre ? route_scores_kernel<T, D, QB, kRaw, true> : route_scores_kernel<T, D, QB, kRaw, false>;
  hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                     hipFuncAttributeMaxDynamicSharedMemorySize,
                                     static_cast<int>(lds));
  if (e != hipSuccess) return e;
  dim3 grid(((N + QB - 1) / QB) * H);
  hipLaunchKernelGGL(kern, grid, dim3(kScoreThreads), lds, stream, static_cast<const T*>(q),
                     ld_q_h, kbar, ld_kbar_h, H, N, M, scale, p);
  return hipGetLastError();
}

template <typename T, int D, bool kRaw>
static hipError_t scores_dispatch(const void* q, int64_t ld_q_h, const float* kbar,
                                  int64_t ld_kbar_h, int H, int N, int M, float scale, float* p,
                                  hipStream_t stream) {
  if (route_scores_lds_bytes(6, M, D) <= kMaxLdsBytes)
    return scores_launch<T, D, 6, kRaw>(q, ld_q_h, kbar, ld_kbar_h, H, N, M, scale, p, stream);
  if (route_scores_lds_bytes(3, M, D) <= kMaxLdsBytes)
    return scores_launch<T, D, 3, kRaw>(q, ld_q_h, kbar, ld_kbar_h, H, N, M, scale, p, stream);
  return scores_launch<T, D, 1, kRaw>(q, ld_q_h, kbar, ld_kbar_h, H, N, M, scale, p, stream);
}

template <bool kRaw>
static hipError_t scores_any(const void* q, bool bf16, int64_t ld_q_h, const float* kbar,
                             int64_t ld_kbar_h, int H, int N, int M, int d, float scale, float* p,
                             hipStream_t stream) {
  if (bf16)
    return d == 128 ? scores_dispatch<bf16_t, 128, kRaw>(q, ld_q_h, kbar, ld_kbar_h, H, N, M, scale, p, stream)
                    : scores_dispatch<bf16_t, 64, kRaw>(q, ld_q_h, kbar, ld_kbar_h, H, N, M, scale, p, stream);
  return d == 128 ? scores_dispatch<float, 128, kRaw>(q, ld_q_h, kbar, ld_kbar_h, H, N, M, scale, p, stream)
                  : scores_dispatch<float, 64, kRaw>(q, ld_q_h, kbar, ld_kbar_h, H, N, M, scale, p, stream);
}

hipError_t launch_route_scores(const void* q, bool bf16, int64_t ld_q_h, const float* kbar,
                               int64_t ld_kbar_h, int H, int N, int M, int d, float scale,
                               float* p, hipStream_t stream) {
  return scores_any<false>(q, bf16, ld_q_h, kbar, ld_kbar_h, H, N, M, d, scale, p, stream);
}

size_t head_mean_lds_bytes(int M) {
  return sizeof(float) * (kScoreThreads / kWave + static_cast<size_t>(M));
}

hipError_t launch_route_scores_shared(const void* q, bool bf16, int64_t ld_q_h, const float* kbar,
                                      int64_t ld_kbar_h, int H, int N, int M, int d, float scale,
                                      float* logits, float* p, hipStream_t stream) {
  hipError_t e = scores_any<true>(q, bf16, ld_q_h, kbar, ld_kbar_h, H, N, M, d, scale, logits, stream);
  if (e != hipSuccess) return e;
  const size_t lds = head_mean_lds_bytes(M);
  e = hipFuncSetAttribute(reinterpret_cast<const void*>(head_mean_softmax_kernel),
                          hipFuncAttributeMaxDynamicSharedMemorySize, static_cast<int>(lds));
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(head_mean_softmax_kernel, dim3(N), dim3(kScoreThreads), lds, stream, logits, H,
                     N, M, p);
  return hipGetLastError();
}

// Largest number of keys a row of the call gathers by radix select: the cap
// beyond the reservation, at most M - reserved and kFastSel (larger caps sort).
static int select_capacity(int M, const RouteConfig& cfg) {
  const int n_res = cfg.n_prev < M ? cfg.n_prev : M;
  int cap = cfg.K_cov > cfg.K_unc ? cfg.K_cov : cfg.K_unc;
  cap = cap - n_res < M - n_res ? cap - n_res : M - n_res;
  if (cap > kFastSel) cap = kFastSel;
  return cap > 1 ? cap : 1;
}

size_t route_select_lds_bytes(int M, int fs) {
  const int P2 = next_pow2(M > 0 ? M : 1);
  const int nwords = (M + 31) / 32;
  return sizeof(uint64_t) * (P2 + 2 * fs + 25) + sizeof(SelectCtl) + sizeof(int) * 512 +
         sizeof(uint32_t) * nwords + sizeof(int) * 16;
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
  a.fs = select_capacity(M, cfg);
  auto al16 = [](const void* x) { return reinterpret_cast<uintptr_t>(x) % 16 == 0; };
  a.vec = M % 4 == 0 && al16(p) && al16(g) && (!cfg.neigh26 || al16(coord)) ? 1 : 0;
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
  a.mode = cfg.mode;
  a.status = cfg.status;
  if (a.status) {
    hipLaunchKernelGGL(route_check_init_kernel, dim3(1), dim3(64), 0, stream, a.status, H * N);
    const hipError_t ei = hipGetLastError();
    if (ei != hipSuccess) return ei;
  }
  const size_t lds = route_select_lds_bytes(M, a.fs);
  hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(route_select_kernel),
                                     hipFuncAttributeMaxDynamicSharedMemorySize,
                                     static_cast<int>(lds));
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(route_select_kernel, dim3(N, H), dim3(kSelectThreads), lds, stream, a);
  return hipGetLastError();
}

hipError_t launch_route_check(const int32_t* route_ids, const int32_t* route_len, int rows, int M,
                              int L, int32_t* bad, hipStream_t stream) {
  hipLaunchKernelGGL(route_check_init_kernel, dim3(1), dim3(64), 0, stream, bad, rows);
  if (rows > 0) {
    const int per = 256 / kWave;
    hipLaunchKernelGGL(route_check_kernel, dim3((rows + per - 1) / per), dim3(256), 0, stream, route_ids,
                       route_len, rows, M, L, bad);
  }
  return hipGetLastError();
}

}  // namespace velox
