// Indexed block-sparse attention and the dense baseline (gfx950).
//
// Method: "Velox: Spatial Memory Makes World Models Efficient" — paper digest,
// Core method (eq. 15): attention runs only over the selected 128-token KV
// tiles, so a skipped tile costs neither its QK^T product nor its K/V load
// (digest, Prerequisites; project page, 02 · Method, "Why the route is a
// block"). The current chunk attends to its own tiles after the routed history
// (the digest's "two-phase tile loop", Reproduction assessment). Dense = every
// tile (digest, Prerequisites: dense FlashAttention schedules all N x M_c pairs).
//
// bf16 kernel: one workgroup of 4 waves per (head, query block); each wave owns
// 32 query rows. Per KV tile (128 keys):
//   S^T = K Q^T   on v_mfma_f32_32x32x16_bf16: A = K rows from LDS, B = the
//                 wave's Q rows held in registers; each lane ends up holding
//                 64 scores of ONE query (its lane mod 32), so the softmax row
//                 max / sum need one cross-lane exchange per tile at most.
//   online softmax in the exp2 domain (scale * log2 e folded into one FMA).
//   O^T += V^T P^T: B = P^T straight from the S^T accumulators (a key
//                 permutation inside each 16-key step, applied to both
//                 operands); A = V^T read from the row-major V tile with the
//                 gfx950 LDS transpose read (ds_read_b64_tr_b16).
// K and V tiles are staged global -> registers -> LDS, one tile ahead, so the
// loads of tile j+1 / j+2 overlap the MFMA work of tile j; two workgroups fit
// per CU (70 KB LDS each). Workgroup ids are remapped so that all query blocks
// of one head run on one XCD and share its L2 for the KV tiles they have in
// common.

#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include "velox_device.hpp"
#include "velox_launch.hpp"

namespace velox {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef short s16x4_t __attribute__((ext_vector_type(4)));
typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4_t lds_s16x4_t;

struct AttnArgs {
  const void* q;
  const void* k;
  const void* v;
  int64_t ld_q_h, ld_kv_h;
  int N, M, G;  // G = H * N workgroups
  float scale;
  const int32_t* route_ids;
  const int32_t* route_len;
  int L;
  int include_current;
  void* o;
  float* lse;
};

// Tile id of step j of a row: routed history tiles first, then the current
// chunk. Out-of-range route ids are clamped into [0, M) (never read out of bounds).
template <bool kRouted>
__device__ __forceinline__ int tile_at(const int32_t* route, int rlen, int M, int j) {
  if (kRouted) {
    if (j < rlen) {
      const int id = route[j];
      return min(max(id, 0), M - 1);
    }
    return M + (j - rlen);
  }
  return j;
}

// ---------------------------------------------------------------- bf16 MFMA

template <int D>
struct TileShape {
  static constexpr int kChunksPerRow = D / 8;             // 16-byte chunks per token row
  static constexpr int kRowsPerPass = 256 / kChunksPerRow;
  static constexpr int kPasses = kBlock / kRowsPerPass;
  static constexpr int kLdsStride = D + 8;                 // bf16 elements per LDS row
};

template <int D>
__device__ __forceinline__ void tile_gload(u32x4_t (&r)[TileShape<D>::kPasses],
                                           const bf16_t* __restrict__ src, int t) {
  using S = TileShape<D>;
  const int row = t / S::kChunksPerRow, col = (t % S::kChunksPerRow) * 8;
#pragma unroll
  for (int ps = 0; ps < S::kPasses; ++ps)
    r[ps] = *reinterpret_cast<const u32x4_t*>(src + (ps * S::kRowsPerPass + row) * D + col);
}

template <int D>
__device__ __forceinline__ void tile_lstore(bf16_t* lds, const u32x4_t (&r)[TileShape<D>::kPasses],
                                            int t) {
  using S = TileShape<D>;
  const int row = t / S::kChunksPerRow, col = (t % S::kChunksPerRow) * 8;
#pragma unroll
  for (int ps = 0; ps < S::kPasses; ++ps)
    *reinterpret_cast<u32x4_t*>(lds + (ps * S::kRowsPerPass + row) * S::kLdsStride + col) = r[ps];
}

template <int D, bool kRouted>
__global__ __launch_bounds__(256, 2) void attn_bf16_kernel(AttnArgs a) {
  using S = TileShape<D>;
  constexpr int kDs = D / 16;   // 16-dim MFMA steps of QK^T
  constexpr int kDb = D / 32;   // 32-dim output blocks of PV
  __shared__ __attribute__((aligned(16))) bf16_t k_lds[kBlock * S::kLdsStride];
  __shared__ __attribute__((aligned(16))) bf16_t v_lds[kBlock * S::kLdsStride];

  const int row_id = xcd_remap(blockIdx.x, a.G);
  const int h = row_id / a.N, i = row_id % a.N;
  const int t = threadIdx.x, wv = t / kWave, lane = t % kWave;
  const int l32 = lane % 32, hh = lane / 32;
  const int M = a.M;

  const bf16_t* qh = static_cast<const bf16_t*>(a.q) + h * a.ld_q_h;
  const bf16_t* kh = static_cast<const bf16_t*>(a.k) + h * a.ld_kv_h;
  const bf16_t* vh = static_cast<const bf16_t*>(a.v) + h * a.ld_kv_h;
  const int32_t* route = nullptr;
  int rlen = M;
  if (kRouted) {
    route = a.route_ids + static_cast<int64_t>(row_id) * a.L;
    rlen = min(max(a.route_len[row_id], 0), a.L);
    if (M == 0) rlen = 0;
  }
  const int T = kRouted ? rlen + (a.include_current ? a.N : 0) : M + a.N;

  const int qrow = i * kBlock + wv * 32 + l32;  // this lane's query (token row)
  bf16_t* orow = static_cast<bf16_t*>(a.o) + (static_cast<int64_t>(h) * a.N * kBlock + qrow) * D;

  if (T == 0) {
    for (int db = 0; db < kDb; ++db)
      for (int g4 = 0; g4 < 4; ++g4)
        *reinterpret_cast<uint2*>(orow + db * 32 + g4 * 8 + hh * 4) = make_uint2(0u, 0u);
    if (a.lse && hh == 0) a.lse[static_cast<int64_t>(h) * a.N * kBlock + qrow] = -INFINITY;
    return;
  }

  // Q fragments (B operand of S^T = K Q^T): query l32, dims ds*16 + hh*8 .. +7
  bf16x8_t qf[kDs];
#pragma unroll
  for (int ds = 0; ds < kDs; ++ds)
    qf[ds] = __builtin_bit_cast(
        bf16x8_t, *reinterpret_cast<const u32x4_t*>(qh + static_cast<int64_t>(qrow) * D + ds * 16 + hh * 8));

  f32x16_t o_acc[kDb];
#pragma unroll
  for (int db = 0; db < kDb; ++db) o_acc[db] = f32x16_t{};
  float m_run = -INFINITY;  // running max of scaled logits (log2 units)
  float l_run = 0.f;        // this lane's share of the running sum
  const float sc = a.scale * 1.4426950408889634f;

  {
    u32x4_t kreg[S::kPasses], vreg[S::kPasses];
    const int t0 = tile_at<kRouted>(route, rlen, M, 0);
    tile_gload<D>(kreg, kh + static_cast<int64_t>(t0) * kBlock * D, t);
    tile_gload<D>(vreg, vh + static_cast<int64_t>(t0) * kBlock * D, t);
    tile_lstore<D>(k_lds, kreg, t);
    tile_lstore<D>(v_lds, vreg, t);
  }
  __syncthreads();

  // LDS addresses of this lane's operand fragments
  const bf16_t* k_frag = k_lds + l32 * S::kLdsStride + hh * 8;
  const int grp = lane / 16, gi = lane % 16;
  const bf16_t* v_frag = v_lds + (hh * 4 + gi / 4) * S::kLdsStride + 16 * (grp % 2) + 4 * (gi % 4);

  // Per tile j: the K tile of j+1 is fetched into registers while S(j) is
  // computed and written to LDS once every wave is done with K(j); the V tile
  // of j+1 is fetched during softmax / PV(j) and written after it. The staging
  // registers never live across iterations.
  for (int j = 0; j < T; ++j) {
    const bool more = j + 1 < T;
    // On the last step the loads re-read tile j (always in bounds) and are
    // discarded; loading unconditionally keeps the staging array in registers.
    const int tn = tile_at<kRouted>(route, rlen, M, more ? j + 1 : j);
    u32x4_t kreg[S::kPasses];
    tile_gload<D>(kreg, kh + static_cast<int64_t>(tn) * kBlock * D, t);

    // ---- S^T = K Q^T : 4 key blocks of 32
    f32x16_t s_acc[4];
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) {
      s_acc[kb] = f32x16_t{};
#pragma unroll
      for (int ds = 0; ds < kDs; ++ds) {
        const bf16x8_t kf = __builtin_bit_cast(
            bf16x8_t, *reinterpret_cast<const u32x4_t*>(k_frag + kb * 32 * S::kLdsStride + ds * 16));
        s_acc[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf, qf[ds], s_acc[kb], 0, 0, 0);
      }
    }
    __syncthreads();  // every wave is done with k_lds(j); v_lds(j) is visible
    u32x4_t vreg[S::kPasses];
    if (more) tile_lstore<D>(k_lds, kreg, t);
    tile_gload<D>(vreg, vh + static_cast<int64_t>(tn) * kBlock * D, t);

    // ---- online softmax (this lane: one query, 64 of the tile's 128 keys)
    float mx = s_acc[0][0];
#pragma unroll
    for (int kb = 0; kb < 4; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s_acc[kb][r]);
    mx = fmaxf(mx, __shfl_xor(mx, 32));
    const float m_new = fmaxf(m_run, mx * sc);
    const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
    m_run = m_new;
    float psum = 0.f;
    bf16x8_t pf[8];
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) {
      f32x8_t lo, hi;
#pragma unroll
      for (int r = 0; r < 8; ++r) {
        lo[r] = __builtin_amdgcn_exp2f(fmaf(s_acc[kb][r], sc, -m_new));
        hi[r] = __builtin_amdgcn_exp2f(fmaf(s_acc[kb][8 + r], sc, -m_new));
        psum += lo[r] + hi[r];
      }
      pf[2 * kb] = __builtin_convertvector(lo, bf16x8_t);
      pf[2 * kb + 1] = __builtin_convertvector(hi, bf16x8_t);
    }
    l_run = l_run * alpha + psum;
#pragma unroll
    for (int db = 0; db < kDb; ++db) o_acc[db] *= alpha;

    // ---- O^T += V^T P^T : 8 key steps of 16
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) {
#pragma unroll
      for (int db = 0; db < kDb; ++db) {
        const bf16_t* vp = v_frag + ks * 16 * S::kLdsStride + db * 32;
        const s16x4_t v0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_t*)(vp));
        const s16x4_t v1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_t*)(vp + 8 * S::kLdsStride));
        const bf16x8_t vf = __builtin_bit_cast(
            bf16x8_t, __builtin_shufflevector(v0, v1, 0, 1, 2, 3, 4, 5, 6, 7));
        o_acc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf, pf[ks], o_acc[db], 0, 0, 0);
      }
    }
    __syncthreads();  // every wave is done with v_lds(j); k_lds(j+1) is visible
    if (more) tile_lstore<D>(v_lds, vreg, t);
  }

  // ---- normalise and store
  const float l_tot = l_run + __shfl_xor(l_run, 32);
  const float inv = 1.0f / l_tot;
#pragma unroll
  for (int db = 0; db < kDb; ++db) {
#pragma unroll
    for (int g4 = 0; g4 < 4; ++g4) {
      uint32_t w0 = static_cast<uint32_t>(f32_to_bf16(o_acc[db][g4 * 4 + 0] * inv)) |
                    (static_cast<uint32_t>(f32_to_bf16(o_acc[db][g4 * 4 + 1] * inv)) << 16);
      uint32_t w1 = static_cast<uint32_t>(f32_to_bf16(o_acc[db][g4 * 4 + 2] * inv)) |
                    (static_cast<uint32_t>(f32_to_bf16(o_acc[db][g4 * 4 + 3] * inv)) << 16);
      *reinterpret_cast<uint2*>(orow + db * 32 + g4 * 8 + hh * 4) = make_uint2(w0, w1);
    }
  }
  if (a.lse && hh == 0)
    a.lse[static_cast<int64_t>(h) * a.N * kBlock + qrow] = m_run * 0.6931471805599453f + logf(l_tot);
}

// ---------------------------------------------------------------- fp32
//
// Plain VALU kernel for fp32 storage: one workgroup per (head, query block),
// two threads per query row (each owns half of the head dimensions), K/V tiles
// in LDS, exact expf online softmax key by key.

template <int D, bool kRouted>
__global__ __launch_bounds__(256) void attn_f32_kernel(AttnArgs a) {
  constexpr int kHalf = D / 2;
  __shared__ float k_lds[kBlock * D];
  __shared__ float v_lds[kBlock * D];
  const int row_id = xcd_remap(blockIdx.x, a.G);
  const int h = row_id / a.N, i = row_id % a.N;
  const int t = threadIdx.x, qr = t / 2, half = t % 2;
  const int M = a.M;
  const float* qh = static_cast<const float*>(a.q) + h * a.ld_q_h;
  const float* kh = static_cast<const float*>(a.k) + h * a.ld_kv_h;
  const float* vh = static_cast<const float*>(a.v) + h * a.ld_kv_h;
  const int32_t* route = nullptr;
  int rlen = M;
  if (kRouted) {
    route = a.route_ids + static_cast<int64_t>(row_id) * a.L;
    rlen = min(max(a.route_len[row_id], 0), a.L);
    if (M == 0) rlen = 0;
  }
  const int T = kRouted ? rlen + (a.include_current ? a.N : 0) : M + a.N;
  const int qrow = i * kBlock + qr;

  float qv[kHalf], ov[kHalf];
#pragma unroll
  for (int c = 0; c < kHalf; ++c) {
    qv[c] = qh[static_cast<int64_t>(qrow) * D + half * kHalf + c];
    ov[c] = 0.f;
  }
  float m_run = -INFINITY, l_run = 0.f;
  for (int j = 0; j < T; ++j) {
    const int tile = tile_at<kRouted>(route, rlen, M, j);
    const float4* ks = reinterpret_cast<const float4*>(kh + static_cast<int64_t>(tile) * kBlock * D);
    const float4* vs = reinterpret_cast<const float4*>(vh + static_cast<int64_t>(tile) * kBlock * D);
    __syncthreads();
    for (int e = t; e < kBlock * D / 4; e += 256) {
      reinterpret_cast<float4*>(k_lds)[e] = ks[e];
      reinterpret_cast<float4*>(v_lds)[e] = vs[e];
    }
    __syncthreads();
    for (int key = 0; key < kBlock; ++key) {
      const float* kr = k_lds + key * D + half * kHalf;
      float part = 0.f;
#pragma unroll
      for (int c = 0; c < kHalf; ++c) part = fmaf(qv[c], kr[c], part);
      const float s = (part + __shfl_xor(part, 1)) * a.scale;
      const float m_new = fmaxf(m_run, s);
      const float alpha = expf(m_run - m_new);
      const float pe = expf(s - m_new);
      l_run = l_run * alpha + pe;
      const float* vr = v_lds + key * D + half * kHalf;
#pragma unroll
      for (int c = 0; c < kHalf; ++c) ov[c] = fmaf(pe, vr[c], ov[c] * alpha);
      m_run = m_new;
    }
  }
  float* orow = static_cast<float*>(a.o) + (static_cast<int64_t>(h) * a.N * kBlock + qrow) * D;
  const float inv = T > 0 ? 1.0f / l_run : 0.f;
#pragma unroll
  for (int c = 0; c < kHalf; ++c) orow[half * kHalf + c] = ov[c] * inv;
  if (a.lse && half == 0)
    a.lse[static_cast<int64_t>(h) * a.N * kBlock + qrow] = T > 0 ? m_run + logf(l_run) : -INFINITY;
}

// ---------------------------------------------------------------- launcher

template <int D, bool kRouted>
static hipError_t launch_one(const AttnArgs& args, bool bf16, hipStream_t stream) {
  if (bf16)
    hipLaunchKernelGGL((attn_bf16_kernel<D, kRouted>), dim3(args.G), dim3(256), 0, stream, args);
  else
    hipLaunchKernelGGL((attn_f32_kernel<D, kRouted>), dim3(args.G), dim3(256), 0, stream, args);
  return hipGetLastError();
}

hipError_t launch_attention(const AttnConfig& c, hipStream_t stream) {
  AttnArgs a;
  a.q = c.q;
  a.k = c.k;
  a.v = c.v;
  a.ld_q_h = c.ld_q_h;
  a.ld_kv_h = c.ld_kv_h;
  a.N = c.N;
  a.M = c.M;
  a.G = c.H * c.N;
  a.scale = c.scale;
  a.route_ids = c.route_ids;
  a.route_len = c.route_len;
  a.L = c.L;
  a.include_current = c.include_current;
  a.o = c.o;
  a.lse = c.lse;
  const bool routed = c.route_ids != nullptr;
  if (c.d == 128)
    return routed ? launch_one<128, true>(a, c.bf16, stream) : launch_one<128, false>(a, c.bf16, stream);
  return routed ? launch_one<64, true>(a, c.bf16, stream) : launch_one<64, false>(a, c.bf16, stream);
}

}  // namespace velox
