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

#include <type_traits>

#include "velox_device.hpp"
#include "velox_launch.hpp"

namespace velox {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef short s16x4_t __attribute__((ext_vector_type(4)));
typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4_t lds_s16x4_t;
typedef __attribute__((address_space(3))) u32x4_t lds_u32x4_t;

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
  int route_head_rows;  // route rows between heads: N (per-head routes) or 0 (shared)
  int include_current;
  void* o;
  float* lse;
  // Split rows (d = 128 bf16 kernel only): n_split > 1 cuts the tile list of
  // every row into n_split consecutive ranges, one workgroup each; the ranges
  // leave unnormalised fp32 O in part_o [n_split][H][N*128][128] and the
  // (max, sum) of their softmax in part_ml [n_split][H][N*128][2], which the
  // merge kernel combines.
  int n_split;
  float* part_o;
  float* part_ml;
  // Unit schedule of the routed d = 128 bf16 kernel written by plan_kernel or
  // plan_split_kernel (nullptr: every workgroup ranks the units itself): entry b is the unit of
  // workgroup b, {head, longer row, shorter row or -1, range}.
  const int4* plan;
};

// Route row of (head h, query block i).
__device__ __forceinline__ int64_t route_row(const AttnArgs& a, int h, int i) {
  return static_cast<int64_t>(h) * a.route_head_rows + i;
}

// Tile id of step j of a row. The current chunk's tiles come first (ncur of
// them: N, or 0 without the current chunk): every query block of a head
// visits them, so taking them together at the start lets the blocks of one
// head share them in L2. The routed (or, dense, all) history tiles follow in
// ascending id order. Out-of-range route ids are clamped into [0, M) (never
// read out of bounds).
template <bool kRouted>
__device__ __forceinline__ int tile_at(const int32_t* route, int ncur, int M, int j) {
  if (j < ncur) return M + j;
  j -= ncur;
  if (kRouted) return min(max(route[j], 0), M - 1);
  return j;
}

// ---------------------------------------------------------------- bf16 MFMA

// LDS layout of one 128-token K or V tile (bf16). kSwz (d = 128 only): rows of
// d elements whose 16-byte chunks are XOR-permuted, chunk c of row r stored at
// c ^ (r mod 16) for K and c ^ (4 r mod 16) for V. Those are the permutations
// under which the K fragment reads (16 B per lane, 32 rows x one chunk) and
// the V transpose reads (8 B per lane, 4 rows x two chunks per 16 lanes) hit
// distinct LDS banks. Otherwise rows are padded (K: d + 8, V: d + 32 elements),
// which has the same property at the cost of LDS space.
template <int D, bool kSwz>
struct Layout {
  static_assert(!kSwz || D == 128, "the swizzled layout is defined for d = 128");
  static constexpr int kCpr = D / 8;                         // 16-byte chunks per row
  static constexpr int kKStride = kSwz ? D : D + 8;
  static constexpr int kVStride = kSwz ? D : D + 32;
  static constexpr int kKElems = kBlock * kKStride;
  static constexpr int kVElems = kBlock * kVStride;
  __device__ static __forceinline__ int k_off(int row, int c) {
    return row * kKStride + (kSwz ? ((c ^ (row & 15)) << 3) : (c << 3));
  }
  __device__ static __forceinline__ int v_off(int row, int c) {
    return row * kVStride + (kSwz ? ((c ^ ((row << 2) & 15)) << 3) : (c << 3));
  }
};

// Register-staged tile copy: 256 threads, 16 bytes each per pass.
template <int D>
struct Stage {
  static constexpr int kCpr = D / 8;
  static constexpr int kRowsPerPass = 256 / kCpr;
  static constexpr int kPasses = kBlock / kRowsPerPass;
};

template <int D>
__device__ __forceinline__ void tile_gload(u32x4_t (&r)[Stage<D>::kPasses],
                                           const bf16_t* __restrict__ src, int t) {
  using S = Stage<D>;
  const int row = t / S::kCpr, col = (t % S::kCpr) * 8;
#pragma unroll
  for (int ps = 0; ps < S::kPasses; ++ps)
    r[ps] = *reinterpret_cast<const u32x4_t*>(src + (ps * S::kRowsPerPass + row) * D + col);
}

template <int D, bool kSwz, bool kIsV>
__device__ __forceinline__ void tile_lstore(bf16_t* lds, const u32x4_t (&r)[Stage<D>::kPasses],
                                            int t) {
  using S = Stage<D>;
  using Lay = Layout<D, kSwz>;
  const int row0 = t / S::kCpr, c = t % S::kCpr;
#pragma unroll
  for (int ps = 0; ps < S::kPasses; ++ps) {
    const int row = ps * S::kRowsPerPass + row0;
    const int off = kIsV ? Lay::v_off(row, c) : Lay::k_off(row, c);
    *reinterpret_cast<u32x4_t*>(lds + off) = r[ps];
  }
}

// Direct global -> LDS tile copy (gfx950 global_load_lds_dwordx4): wave w
// fills LDS bytes [w * 8 KiB, (w + 1) * 8 KiB) of the tile, 1 KiB (4 rows) per
// instruction; lane l of instruction i lands at row (8 w + i) * 4 + l / 16,
// physical chunk l % 16, so it fetches the logical chunk that the swizzle puts
// there. d = 128, swizzled layout only.
template <bool kIsV>
__device__ __forceinline__ void tile_dload(bf16_t* lds, const bf16_t* __restrict__ src, int wv,
                                           int lane) {
  constexpr int D = 128;
  const int wu = __builtin_amdgcn_readfirstlane(wv);
  __attribute__((address_space(3))) char* dst =
      (__attribute__((address_space(3))) char*)(lds) + wu * 8192;
  const int p = lane & 15;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int row = (wu * 8 + i) * 4 + (lane >> 4);
    const int c = kIsV ? (p ^ ((row << 2) & 15)) : (p ^ (row & 15));
    __builtin_amdgcn_global_load_lds(src + row * D + c * 8, dst + i * 1024, 16, 0, 0);
  }
}

// Direct global -> LDS copy into the padded layout: the tile's LDS image
// (128 rows of kStride elements) is filled 1 KiB per wave instruction, lane l
// landing at byte 16 l of its instruction's KiB; lanes whose slot falls in a
// row's padding are masked off.
template <int D, int kStride>
__device__ __forceinline__ void tile_dload_pad(bf16_t* lds, const bf16_t* __restrict__ src,
                                               int wv, int lane) {
  constexpr int kRowBytes = D * 2, kStrideBytes = kStride * 2;
  constexpr int kInst = (kBlock * kStrideBytes + 1023) / 1024;
  constexpr int kPerWave = (kInst + 3) / 4;
  const int wu = __builtin_amdgcn_readfirstlane(wv);
  __attribute__((address_space(3))) char* base = (__attribute__((address_space(3))) char*)(lds);
#pragma unroll
  for (int i = 0; i < kPerWave; ++i) {
    const int inst = wu * kPerWave + i;
    if (inst < kInst) {
      const int o = inst * 1024 + lane * 16;
      const int row = o / kStrideBytes, rem = o - row * kStrideBytes;
      if (rem < kRowBytes && row < kBlock)
        __builtin_amdgcn_global_load_lds(src + row * D + rem / 2, base + inst * 1024, 16, 0, 0);
    }
  }
}

__device__ __forceinline__ void wait_vm_all() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N <= 63, "vmcnt range");
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

// The same waits issued through the builtin (gfx9 s_waitcnt encoding: vmcnt in
// bits 3:0 and 15:14, expcnt and lgkmcnt left at their maxima), so that the
// compiler's own wait insertion sees them and adds none of its own.
__device__ __forceinline__ void tracked_wait_vm_all() { __builtin_amdgcn_s_waitcnt((7 << 4) | (15 << 8)); }

template <int N>
__device__ __forceinline__ void tracked_wait_vmcnt() {
  static_assert(N >= 0 && N <= 63, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

// Workgroup barrier without a memory fence: the direct LDS loads are ordered
// with explicit vmcnt waits, and a fence here would drain loads still meant to
// be in flight.
__device__ __forceinline__ void barrier_nofence() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// Direct-LDS instructions each wave issues for one K (kK) or V (kV) tile.
template <int D, bool kSwz>
struct DmaCount {
  static constexpr int kK = kSwz ? 8 : ((kBlock * Layout<D, false>::kKStride * 2 + 1023) / 1024 + 3) / 4;
  static constexpr int kV = kSwz ? 8 : ((kBlock * Layout<D, false>::kVStride * 2 + 1023) / 1024 + 3) / 4;
};

constexpr float kLazyRescale = 8.0f;  // log2 units
constexpr int kMaxRouteLds = 4096;    // route ids staged in LDS by the DMA kernel

template <int D, bool kSwz, bool kIsV>
__device__ __forceinline__ void dload(bf16_t* lds, const bf16_t* __restrict__ src, int wv, int lane) {
  if constexpr (kSwz)
    tile_dload<kIsV>(lds, src, wv, lane);
  else
    tile_dload_pad<D, kIsV ? Layout<D, false>::kVStride : Layout<D, false>::kKStride>(lds, src, wv, lane);
}

template <int D, bool kRouted, bool kSwz, bool kDirect>
__global__ __launch_bounds__(256, 2) void attn_bf16_kernel(AttnArgs a) {
  static_assert(!kDirect || D == 128, "direct LDS loads are written for d = 128");
  using Lay = Layout<D, kSwz>;
  using S = Stage<D>;
  constexpr int kDs = D / 16;   // 16-dim MFMA steps of QK^T
  constexpr int kDb = D / 32;   // 32-dim output blocks of PV
  __shared__ __attribute__((aligned(1024))) bf16_t k_lds[Lay::kKElems];
  __shared__ __attribute__((aligned(1024))) bf16_t v_lds[Lay::kVElems];
  // With direct LDS loads the route is staged in LDS, so reading tile ids
  // never puts a vector load in front of the DMA waits.
  constexpr bool kRouteInLds = kRouted && kDirect;
  __shared__ int route_lds[kRouteInLds ? kMaxRouteLds : 1];

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
    const int64_t rr = route_row(a, h, i);
    route = a.route_ids + rr * a.L;
    rlen = min(max(a.route_len[rr], 0), a.L);
    if (M == 0) rlen = 0;
  }
  const int ncur = (!kRouted || a.include_current) ? a.N : 0;
  const int T = rlen + ncur;

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
  float m_ref = -INFINITY;  // reference max of the scaled logits (log2 units)
  float l_run = 0.f;        // this lane's share of the running sum
  const float sc = a.scale * 1.4426950408889634f;

  // LDS element offsets of this lane's operand fragments.
  //   K (A operand of S^T): row kb*32 + l32, chunk 2 ds + hh.
  //   V (transpose read, A operand of O^T): rows ks*16 + hh*4 + gi/4 (+8),
  //   chunk 4 db + 2 (grp & 1) + (gi & 3) / 2, half-chunk gi & 1.
  const int grp = lane / 16, gi = lane % 16;
  const int vrow = hh * 4 + gi / 4;
  const int vsub = (gi & 1) * 4;

  if constexpr (kRouteInLds) {
    for (int e = t; e < rlen; e += 256) route_lds[e] = min(max(route[e], 0), M - 1);
    __syncthreads();
  }
  auto tile_ptr = [&](const bf16_t* base, int j) {
    int tile;
    if constexpr (kRouteInLds)
      tile = j < ncur ? M + j : route_lds[j - ncur];
    else
      tile = tile_at<kRouted>(route, ncur, M, j);
    return base + static_cast<int64_t>(tile) * kBlock * D;
  };

  {
    if constexpr (kDirect) {
      dload<D, kSwz, false>(k_lds, tile_ptr(kh, 0), wv, lane);
      dload<D, kSwz, true>(v_lds, tile_ptr(vh, 0), wv, lane);
      wait_vm_all();
    } else {
      u32x4_t kreg[S::kPasses], vreg[S::kPasses];
      tile_gload<D>(kreg, tile_ptr(kh, 0), t);
      tile_gload<D>(vreg, tile_ptr(vh, 0), t);
      tile_lstore<D, kSwz, false>(k_lds, kreg, t);
      tile_lstore<D, kSwz, true>(v_lds, vreg, t);
    }
  }
  __syncthreads();

  // Per tile j. Register-staged path: K(j+1) is fetched into registers during
  // S(j) and stored once every wave is done with K(j); V(j+1) is fetched
  // during softmax / PV(j) and stored after it. DMA path: K(j+1) is issued as
  // soon as every wave is done with K(j) and must land before S(j+1); V(j+1)
  // is issued once every wave is done with V(j) and must land before PV(j+1),
  // so each load overlaps about half a tile of MFMA work plus a softmax.
  for (int j = 0; j < T; ++j) {
    const bool more = j + 1 < T;
    // On the last step the staged loads re-read tile j (always in bounds) and
    // are discarded; loading unconditionally keeps the staging in registers.
    const bf16_t* kn = tile_ptr(kh, more ? j + 1 : j);
    const bf16_t* vn = tile_ptr(vh, more ? j + 1 : j);
    u32x4_t kreg[S::kPasses];
    if constexpr (!kDirect) tile_gload<D>(kreg, kn, t);

    // ---- S^T = K Q^T : 4 key blocks of 32
    f32x16_t s_acc[4];
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) {
      s_acc[kb] = f32x16_t{};
#pragma unroll
      for (int ds = 0; ds < kDs; ++ds) {
        const bf16x8_t kf = __builtin_bit_cast(
            bf16x8_t, *reinterpret_cast<const u32x4_t*>(k_lds + Lay::k_off(kb * 32 + l32, 2 * ds + hh)));
        s_acc[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf, qf[ds], s_acc[kb], 0, 0, 0);
      }
    }
    u32x4_t vreg[S::kPasses];
    if constexpr (kDirect) {
      barrier_nofence();  // every wave is done with k_lds(j)
      if (more) dload<D, kSwz, false>(k_lds, kn, wv, lane);
    } else {
      __syncthreads();    // every wave is done with k_lds(j); v_lds(j) is visible
      if (more) tile_lstore<D, kSwz, false>(k_lds, kreg, t);
      tile_gload<D>(vreg, vn, t);
    }

    // ---- online softmax (this lane: one query, 64 of the tile's 128 keys).
    // The reference max only moves when a score exceeds it by more than 2^8
    // (then O and l are rescaled); otherwise every p stays below 2^8 and the
    // final division is unaffected.
    float mk[4];
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) {
      mk[kb] = s_acc[kb][0];
#pragma unroll
      for (int r = 1; r < 16; ++r) mk[kb] = fmaxf(mk[kb], s_acc[kb][r]);
    }
    float mx = fmaxf(fmaxf(mk[0], mk[1]), fmaxf(mk[2], mk[3]));
    mx = fmaxf(mx, __shfl_xor(mx, 32)) * sc;
    if (__ballot(mx > m_ref + kLazyRescale) != 0) {
      const float m_new = fmaxf(m_ref, mx);
      const float alpha = __builtin_amdgcn_exp2f(m_ref - m_new);
      m_ref = m_new;
      l_run *= alpha;
#pragma unroll
      for (int db = 0; db < kDb; ++db) o_acc[db] *= alpha;
    }
    float ps[4];
    bf16x8_t pf[8];
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) {
      f32x8_t lo, hi;
      ps[kb] = 0.f;
#pragma unroll
      for (int r = 0; r < 8; ++r) {
        lo[r] = __builtin_amdgcn_exp2f(fmaf(s_acc[kb][r], sc, -m_ref));
        hi[r] = __builtin_amdgcn_exp2f(fmaf(s_acc[kb][8 + r], sc, -m_ref));
        ps[kb] += lo[r] + hi[r];
      }
      pf[2 * kb] = __builtin_convertvector(lo, bf16x8_t);
      pf[2 * kb + 1] = __builtin_convertvector(hi, bf16x8_t);
    }
    l_run += (ps[0] + ps[1]) + (ps[2] + ps[3]);

    if constexpr (kDirect) {
      // this wave's part of V(j) has landed (K(j+1), issued later, may still fly)
      if (more)
        wait_vmcnt<DmaCount<D, kSwz>::kK>();
      else
        wait_vm_all();
      barrier_nofence();  // v_lds(j) is visible
    }

    // ---- O^T += V^T P^T : 8 key steps of 16
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) {
#pragma unroll
      for (int db = 0; db < kDb; ++db) {
        const int vc = 4 * db + 2 * (grp & 1) + ((gi & 3) >> 1);
        const bf16_t* vp0 = v_lds + Lay::v_off(ks * 16 + vrow, vc) + vsub;
        const bf16_t* vp1 = v_lds + Lay::v_off(ks * 16 + 8 + vrow, vc) + vsub;
        const s16x4_t v0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_t*)(vp0));
        const s16x4_t v1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_t*)(vp1));
        const bf16x8_t vf = __builtin_bit_cast(
            bf16x8_t, __builtin_shufflevector(v0, v1, 0, 1, 2, 3, 4, 5, 6, 7));
        o_acc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf, pf[ks], o_acc[db], 0, 0, 0);
      }
    }
    if constexpr (kDirect) {
      wait_vm_all();      // this wave's part of K(j+1) has landed
      barrier_nofence();  // every wave is done with v_lds(j); k_lds(j+1) is visible
      if (more) dload<D, kSwz, true>(v_lds, vn, wv, lane);
    } else {
      __syncthreads();    // every wave is done with v_lds(j); k_lds(j+1) is visible
      if (more) tile_lstore<D, kSwz, true>(v_lds, vreg, t);
    }
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
    a.lse[static_cast<int64_t>(h) * a.N * kBlock + qrow] = m_ref * 0.6931471805599453f + logf(l_tot);
}


// ---------------------------------------------------------------- bf16, d = 128, ping-pong
//
// Eight waves per workgroup in two teams of four. Each team owns one query
// block (the two blocks of a workgroup belong to one head and are paired by
// route length, so both teams run about the same number of tiles); each wave
// owns 32 query rows of its team's block. Work advances in 64-key half-tiles,
// and for every half-tile j a team runs
//   an MFMA phase:  O += P(j-1) V(j-1)  and  S(j) = K(j) Q^T   (32 MFMAs/wave)
//   a VALU phase:   softmax of S(j) -> P(j)                     (exp, max, sum)
// The two teams are one phase apart, so on every SIMD one wave issues MFMAs
// while the other runs its softmax; a fence-free workgroup barrier separates
// phases. Each team has a two-slot ring for K and one for V (16 KiB slots,
// 128 KiB in all); VALU phase j issues the DMA for V(j+1) at its start and for
// K(j+2) after the softmax, and both must land before MFMA phase j+2 reads them.
// The workgroups of an XCD take their (head, pair) units longest first; with
// split rows a unit is a range of a pair's tile lists and leaves partial
// results for split_merge_kernel.

namespace pp {

constexpr int D = 128;
constexpr int kHalf = 64;                       // keys per half-tile
constexpr int kSlot = kHalf * D * 2;            // 16 KiB: 64 rows of 256 bytes
constexpr int kMaxRoute = 2048;                 // route ids staged in LDS per team
constexpr int kThreads = 512;

typedef __attribute__((address_space(3))) char lds_char_t;
typedef __attribute__((address_space(1))) const char gbl_char_t;

// Slots hold 64 rows of 256 bytes; 16-byte chunk c of row r sits at chunk
// c ^ (r & 15) for K and c ^ (4 r & 15) for V (conflict-free fragment reads).
//
// DMA of a half-tile: 16 instructions of 1 KiB, lane l of instruction n landing
// at row 4 n + l / 16, physical chunk l % 16. Team wave tw issues n = tw + 4 i,
// so n & 3 = tw is constant per wave and the logical chunk each lane fetches,
// (l % 16) ^ ((4 n + l / 16) & 15) for K or (l % 16) ^ (4 (l / 16)) for V,
// does not depend on i: the four instructions use one 32-bit lane offset plus
// 4 KiB per instruction.
__device__ __forceinline__ uint32_t dma_lane_off(int tw, int lane, bool is_v) {
  const int x = lane >> 4, p = lane & 15;
  const int c = is_v ? (p ^ (x << 2)) : (p ^ ((tw << 2) | x));
  return static_cast<uint32_t>(x * 256 + c * 16) + static_cast<uint32_t>(tw * 1024);
}
// The same pointer, held in scalar registers (it is wave-uniform).
__device__ __forceinline__ const bf16_t* uniform_ptr(const bf16_t* p) {
  const uint64_t u = reinterpret_cast<uint64_t>(p);
  const uint32_t lo = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(u));
  const uint32_t hi = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(u >> 32));
  return reinterpret_cast<const bf16_t*>((static_cast<uint64_t>(hi) << 32) | lo);
}

// The four instructions are written in inline assembly so that the compiler
// does not see an LDS DMA in flight: when it does, it treats LDS reads as
// completing out of order and waits for every outstanding LDS read before each
// MFMA, which serialises the fragment loads of the MFMA phases. The kernel
// orders the DMA itself (explicit vmcnt waits, then a workgroup barrier, before
// any wave reads a slot), and no code in it uses M0 otherwise. The leading
// s_nop 4 covers a scalar base freshly computed from a VALU result, each
// s_nop 0 the M0 write before the load that reads it.
// src: wave-uniform global address of the half-tile; m0s[i]: LDS address of
// instruction i (slot + (tw + 4 i) KiB); off[i]: this lane's byte offset.
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
__device__ __forceinline__ void dma_half(gbl_char_t* src, const uint32_t (&m0s)[4], const uint32_t (&off)[4]) {
  asm volatile(
      "s_nop 4\n\t"
      "s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %4, %8\n\t"
      "s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %5, %8\n\t"
      "s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %6, %8\n\t"
      "s_mov_b32 m0, %3\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %7, %8"
      ::"s"(m0s[0]), "s"(m0s[1]), "s"(m0s[2]), "s"(m0s[3]),
        "v"(off[0]), "v"(off[1]), "v"(off[2]), "v"(off[3]), "s"(src)
      : "memory", "m0");
}
#pragma clang diagnostic pop

template <bool kRouted>
__global__ __launch_bounds__(kThreads, 1) void attn_kernel(AttnArgs a) {
  // Four slot arrays (K even/odd half-tile, V even/odd), each holding both
  // teams' 16 KiB slots. With the half-tile loop unrolled by two every LDS
  // access names its array, so the compiler can see that the DMA in flight
  // targets other arrays than the reads of the current phase.
  __shared__ __attribute__((aligned(1024))) char k_even[2 * kSlot];
  __shared__ __attribute__((aligned(1024))) char k_odd[2 * kSlot];
  __shared__ __attribute__((aligned(1024))) char v_even[2 * kSlot];
  __shared__ __attribute__((aligned(1024))) char v_odd[2 * kSlot];
  __shared__ int route_lds[2][kRouted ? kMaxRoute : 1];
  __shared__ int pair_rows[2];
  __shared__ int team_halves[2];

  const int t = threadIdx.x, lane = t % kWave;
  const int wv = __builtin_amdgcn_readfirstlane(t / kWave);
  const int team = wv >> 2, tw = wv & 3;
  const int l32 = lane % 32, hh = lane / 32;
  const int grp = lane / 16, gi = lane % 16;
  const int N = a.N, M = a.M;
  const int pairs = (N + 1) / 2;
  const int nsp = max(a.n_split, 1);
  const int G = (a.G / N) * pairs * nsp;  // work units: (head, pair, range)
  // ---- which (head, pair, range) this workgroup serves. A pair is two rows of one
  // head, ranks 2 pr and 2 pr + 1 of its rows ordered by route length (longest
  // first, ties by index). Each XCD owns a contiguous range of (head, pair) ids
  // (xcd_remap). Routed: the XCD's workgroups, in dispatch order, take that
  // range's pairs longest first (longest-processing-time order, so that the
  // short pairs fill the tail of the grid); the order is computed here from the
  // route lengths, staged in route_lds before the route ids use it.
  int* lens_s = &route_lds[0][0];
  int h, pr, split, n_rng = nsp;  // n_rng: ranges of this unit's rows
  if (t < 2) pair_rows[t] = -1;
  if (kRouted && a.plan) {
    const int4 u = a.plan[blockIdx.x];
    if (u.x < 0) return;  // an empty slot of the plan (the whole workgroup leaves)
    h = u.x;
    split = u.w & 0xff;
    n_rng = max(u.w >> 8, 1);
    pr = 0;
    __syncthreads();
    if (t < 2) pair_rows[t] = t == 0 ? u.y : u.z;
  } else if (kRouted) {
    const int x = blockIdx.x % kXcd, slot = blockIdx.x / kXcd;
    int base, cnt;
    xcd_range(x, G, base, cnt);
    const int h_lo = base / nsp / pairs, nh = (base + cnt - 1) / nsp / pairs - h_lo + 1;
    const int nr = nh * N;
    int* rank_s = lens_s + nr;
    int* cost_s = rank_s + nr;
    int* sorted_s = cost_s + cnt;
    if (3 * nr + cnt <= 2 * kMaxRoute) {
      for (int e = t; e < nr; e += kThreads)
        lens_s[e] = min(max(a.route_len[route_row(a, h_lo + e / N, e % N)], 0), a.L);
      __syncthreads();
      // rank of each row among its head's rows, and of each unit below among
      // the XCD's units: eight LDS reads in flight per wait
      auto rank_of = [](const int* vals, int lo, int hi, int me, int vme) {
        int rank = 0, o = lo;
        for (; o + 8 <= hi; o += 8) {
          int x[8];
#pragma unroll
          for (int u = 0; u < 8; ++u) x[u] = vals[o + u];
#pragma unroll
          for (int u = 0; u < 8; ++u) rank += (x[u] > vme) || (x[u] == vme && o + u < me);
        }
        for (; o < hi; ++o) rank += (vals[o] > vme) || (vals[o] == vme && o < me);
        return rank;
      };
      for (int e = t; e < nr; e += kThreads) {
        const int hb = e - e % N, lr = lens_s[e];
        const int rank = rank_of(lens_s, hb, hb + N, e, lr);
        rank_s[e] = rank;
        sorted_s[hb + rank] = lr;
      }
      __syncthreads();
      for (int w = t; w < cnt; w += kThreads) {
        const int id = (base + w) / nsp;  // (head, pair) of the unit
        cost_s[w] = sorted_s[(id / pairs - h_lo) * N + 2 * (id % pairs)];
      }
      __syncthreads();
      for (int w = t; w < cnt; w += kThreads) {
        const int rank = rank_of(cost_s, 0, cnt, w, cost_s[w]);
        if (rank == slot) pair_rows[0] = base + w;  // the one pair of dispatch rank `slot`
      }
      __syncthreads();
      const int wg = pair_rows[0];
      split = wg % nsp;
      h = wg / nsp / pairs;
      pr = wg / nsp % pairs;
      __syncthreads();
      if (t < 2) pair_rows[t] = -1;
      __syncthreads();
      for (int r = t; r < N; r += kThreads) {
        const int rank = rank_s[(h - h_lo) * N + r];
        if (rank / 2 == pr) pair_rows[rank & 1] = r;
      }
    } else {
      // too many rows to stage: dispatch order of the logical ids
      const int wg = xcd_remap(blockIdx.x, G);
      split = wg % nsp;
      h = wg / nsp / pairs;
      pr = wg / nsp % pairs;
      __syncthreads();
      for (int r = t; r < N; r += kThreads) {
        const int* lens = a.route_len + route_row(a, h, 0);
        const int lr = min(max(lens[r], 0), a.L);
        int rank = 0;
        for (int o = 0; o < N; ++o) {
          const int lo = min(max(lens[o], 0), a.L);
          rank += (lo > lr) || (lo == lr && o < r);
        }
        if (rank / 2 == pr) pair_rows[rank & 1] = r;
      }
    }
  } else {
    const int wg = xcd_remap(blockIdx.x, G);
    split = wg % nsp;
    h = wg / nsp / pairs;
    pr = wg / nsp % pairs;
    __syncthreads();
    for (int r = t; r < N; r += kThreads)
      if (r / 2 == pr) pair_rows[r & 1] = r;
  }
  __syncthreads();
  const int i = pair_rows[team];  // -1: this team has no block (odd N)

  const bf16_t* kh = static_cast<const bf16_t*>(a.k) + h * a.ld_kv_h;
  const bf16_t* vh = static_cast<const bf16_t*>(a.v) + h * a.ld_kv_h;
  int rlen = 0, ncur = 0;
  if (i >= 0) {
    rlen = M;
    if (kRouted) rlen = M == 0 ? 0 : min(max(a.route_len[route_row(a, h, i)], 0), a.L);
    ncur = (!kRouted || a.include_current) ? N : 0;
  }
  // this unit's range [t0, t1) of the row's tile list (the whole list unless
  // rows are split)
  const int t_row = rlen + ncur;
  const int t_chunk = (t_row + n_rng - 1) / n_rng;
  const int t0 = min(t_row, split * t_chunk);
  const int S = 2 * (min(t_row, t0 + t_chunk) - t0);  // half-tiles of this team's range
  if (kRouted && i >= 0) {
    const int32_t* route = a.route_ids + route_row(a, h, i) * a.L;
    for (int e = t - team * 256; e < rlen; e += 256) route_lds[team][e] = min(max(route[e], 0), M - 1);
  }
  if (tw == 0 && lane == 0) team_halves[team] = S;
  __syncthreads();
  // Phases: the lead team (0) runs MFMA(0), VALU(0), ..., MFMA(S), VALU(S);
  // the other team starts one phase later. Both execute the same number of
  // barriers: every wave of the workgroup must reach every barrier.
  const int phases = max(2 * (team_halves[0] + 1), 1 + 2 * (team_halves[1] + 1));


  // slot of half-tile parity P (a compile-time constant at every use)
  auto kslot = [&](auto P) {
    return (lds_char_t*)(decltype(P)::value ? k_odd : k_even) + team * kSlot;
  };
  auto vslot = [&](auto P) {
    return (lds_char_t*)(decltype(P)::value ? v_odd : v_even) + team * kSlot;
  };
  auto kslot_any = [&](int par) { return (lds_char_t*)(par ? k_odd : k_even) + team * kSlot; };
  auto vslot_any = [&](int par) { return (lds_char_t*)(par ? v_odd : v_even) + team * kSlot; };
  using Even = std::integral_constant<int, 0>;
  using Odd = std::integral_constant<int, 1>;
  const uint32_t koff_dma = dma_lane_off(tw, lane, false);
  const uint32_t voff_dma = dma_lane_off(tw, lane, true);

  const int qrow = (i >= 0 ? i : 0) * kBlock + tw * 32 + l32;  // this lane's query row
  const bf16_t* qh = static_cast<const bf16_t*>(a.q) + h * a.ld_q_h;
  // Q fragments, pre-multiplied by scale * log2(e) and rounded to bf16
  // (round to nearest even), so that S = K Q^T comes out in the exp2 domain.
  const float sc = a.scale * 1.4426950408889634f;
  bf16x8_t qf[8];
#pragma unroll
  for (int ds = 0; ds < 8; ++ds) {
    const bf16x8_t raw = __builtin_bit_cast(
        bf16x8_t, *reinterpret_cast<const u32x4_t*>(qh + static_cast<int64_t>(qrow) * D + ds * 16 + hh * 8));
    qf[ds] = __builtin_convertvector(__builtin_convertvector(raw, f32x8_t) * sc, bf16x8_t);
  }

  f32x16_t o_acc[4];
#pragma unroll
  for (int db = 0; db < 4; ++db) o_acc[db] = f32x16_t{};
  f32x16_t s_acc[2];
  bf16x8_t pf[4];
  // m_ref: this lane's query's reference max (exp2 domain); neg_m holds -m_ref
  // in all 16 accumulator slots and is the C operand of the first QK^T MFMA,
  // so each score reaches the softmax as x = s - m_ref.
  float m_ref = 0.f, l_run = 0.f;
  f32x16_t neg_m = f32x16_t{};

  // K fragment (row kb*32 + l32, logical chunk 2 ds + hh) sits at byte
  //   kb*8192 + l32*256 + 16 (hh ^ z0) + 32 (ds ^ z1),  z = l32 & 15.
  const int z = l32 & 15;
  const int kbase = l32 * 256 + ((hh ^ (z & 1)) << 4);
  const int kz1 = (z >> 1) << 5;
  // V fragment (transpose read): row ks*16 + hh*4 + gi/4 (+8), logical chunk
  // 4 db + 2 (grp & 1) + (gi & 3) / 2, half-chunk gi & 1.
  int v_off[4];
#pragma unroll
  for (int db = 0; db < 4; ++db) {
    const int r = hh * 4 + gi / 4, c = 4 * db + 2 * (grp & 1) + ((gi & 3) >> 1);
    v_off[db] = r * 256 + ((c ^ ((r << 2) & 15)) << 4) + (gi & 1) * 8;
  }

  // Byte offset of half-tile j within the head's K or V. The route id of a
  // half-tile is read from LDS one phase ahead, during the MFMA phase, where
  // its latency hides behind the MFMA stream (route_raw; for every j, clamped
  // inside route_lds, so no branch surrounds the read); half_off selects and
  // scales. j may pass the end of the row by two: the result is then unused.
  auto route_raw = [&](int j) {
    const int e = min(max((j >> 1) + t0 - ncur, 0), kMaxRoute - 1);
    return kRouted ? route_lds[team][e] : 0;
  };
  auto half_off = [&](int j, int id) -> uint64_t {
    const int jt = (j >> 1) + t0;
    const int tile = jt < ncur ? M + jt : (kRouted ? id : jt - ncur);
    return static_cast<uint64_t>(static_cast<uint32_t>(tile)) * (kBlock * D * 2) + (j & 1) * (kHalf * D * 2);
  };
  gbl_char_t* const kg = (gbl_char_t*)uniform_ptr(kh);
  gbl_char_t* const vg = (gbl_char_t*)uniform_ptr(vh);
  uint32_t koff[4], voff[4], m0k[2][4], m0v[2][4];
#pragma unroll
  for (int n = 0; n < 4; ++n) {
    koff[n] = koff_dma + n * 4096;
    voff[n] = voff_dma + n * 4096;
#pragma unroll
    for (int par = 0; par < 2; ++par) {
      m0k[par][n] = __builtin_amdgcn_readfirstlane(
          static_cast<uint32_t>(reinterpret_cast<uintptr_t>(kslot_any(par))) + (tw + 4 * n) * 1024);
      m0v[par][n] = __builtin_amdgcn_readfirstlane(
          static_cast<uint32_t>(reinterpret_cast<uintptr_t>(vslot_any(par))) + (tw + 4 * n) * 1024);
    }
  }
  uint64_t hoff_next = 0;  // byte offset of half-tile j + 1 (K(j+1), then V(j+1))
  int id_next = 0;         // route id of half-tile j + 2
  // fragment loads: V^T (ks, db) of the PV product, K (kb, ds) of the QK one
  auto load_v = [&](lds_char_t* vs, int ks, int db) {
    lds_char_t* vp = vs + v_off[db] + ks * 16 * 256;
    const s16x4_t v0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_t*)(vp));
    const s16x4_t v1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_t*)(vp + 8 * 256));
    return __builtin_bit_cast(bf16x8_t, __builtin_shufflevector(v0, v1, 0, 1, 2, 3, 4, 5, 6, 7));
  };
  auto load_k = [&](lds_char_t* ksl, int kb, int ds) {
    return __builtin_bit_cast(bf16x8_t, *(const lds_u32x4_t*)(ksl + kb * 8192 + ((ds << 5) ^ kz1)));
  };
  // Each MFMA phase is two streams of 16 MFMAs (PV(j-1), then K(j) Q^T with
  // the two key blocks alternating, so consecutive MFMAs never depend on each
  // other); every fragment is loaded from LDS kAhead MFMAs before its use.
  // Scheduling fences keep that order: left alone, the compiler waits for
  // each load right after issuing it.
  constexpr int kAhead = 3;
  auto pv_stream = [&](lds_char_t* vs) {
    bf16x8_t fb[16];
#pragma unroll
    for (int u = 0; u < kAhead; ++u) fb[u] = load_v(vs, u >> 2, u & 3);
#pragma unroll
    for (int u = 0; u < 16; ++u) {
      __builtin_amdgcn_sched_barrier(0);
      if (u + kAhead < 16) fb[u + kAhead] = load_v(vs, (u + kAhead) >> 2, (u + kAhead) & 3);
      o_acc[u & 3] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fb[u], pf[u >> 2], o_acc[u & 3], 0, 0, 0);
    }
    __builtin_amdgcn_sched_barrier(0);
  };
  auto qk_stream = [&](lds_char_t* ksl) {
    bf16x8_t fb[16];
#pragma unroll
    for (int u = 0; u < kAhead; ++u) fb[u] = load_k(ksl, u & 1, u >> 1);
#pragma unroll
    for (int u = 0; u < 16; ++u) {
      __builtin_amdgcn_sched_barrier(0);
      if (u + kAhead < 16) fb[u + kAhead] = load_k(ksl, (u + kAhead) & 1, (u + kAhead) >> 1);
      const int kb = u & 1, ds = u >> 1;
      s_acc[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fb[u], qf[ds], ds == 0 ? neg_m : s_acc[kb], 0, 0, 0);
    }
    __builtin_amdgcn_sched_barrier(0);
  };
  // P: parity of j (Even / Odd), Q: the other parity
  // The wave in its MFMA phase gets the higher issue priority, so that the
  // softmax of the other team's wave on the same SIMD fills the gaps between
  // MFMA issues instead of delaying them.
  auto mfma_phase = [&](int j, auto P, auto Q) {
    __builtin_amdgcn_s_setprio(2);
    const int rid = route_raw(j + 2);
    if (j > 0) pv_stream(vslot(Q));             // O += P(j-1) V(j-1)
    if (j < S) qk_stream(kslot(P) + kbase);     // S(j) = K(j) Q^T
    id_next = __builtin_amdgcn_readfirstlane(rid);
  };
  // a workgroup barrier that no instruction is scheduled across
  auto phase_barrier = [] {
    __builtin_amdgcn_sched_barrier(0);
    barrier_nofence();
    __builtin_amdgcn_sched_barrier(0);
  };

  auto valu_phase = [&](int j, auto P, auto Q) {
    // refill the slots MFMA(j) just freed: V(j+1) into V(j-1)'s now, K(j+2)
    // into K(j)'s after the softmax (both orders are correct; this one measured
    // 1-2% faster than issuing both first)
    __builtin_amdgcn_s_setprio(0);
    const bool k_next = j + 2 < S, v_next = j + 1 < S;
    const uint64_t hk = half_off(j + 2, id_next);
    if (v_next) dma_half(vg + hoff_next, m0v[decltype(Q)::value], voff);
    hoff_next = hk;
    // softmax of S(j): p = 2^x with x = s - m_ref straight from the MFMA. The
    // reference moves lazily: on the first half-tile of the range, and when
    // the half-tile's sum of p exceeds 32 * 2^8 (some x above 13; a row of 32
    // values all <= 8 sums to at most that), a wave-uniform slow path takes
    // the query's true maximum x_max (both halves of the row) and, when it is
    // above 8 (always on the first half-tile), moves m_ref up by x_max,
    // rescales O and l by 2^-x_max and recomputes p. Otherwise p <= 2^13.
    f32x8_t e[4];
    auto exps = [&](float shift) {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int r = 0; r < 8; ++r) {
          e[2 * kb][r] = __builtin_amdgcn_exp2f(s_acc[kb][r] - shift);
          e[2 * kb + 1][r] = __builtin_amdgcn_exp2f(s_acc[kb][8 + r] - shift);
        }
    };
    auto row_sum = [&] {  // pairwise tree over the 32 values
      f32x8_t t = (e[0] + e[1]) + (e[2] + e[3]);
      const float a0 = (t[0] + t[1]) + (t[2] + t[3]);
      const float a1 = (t[4] + t[5]) + (t[6] + t[7]);
      return a0 + a1;
    };
    exps(0.f);
    float ps = row_sum();
    if (__ballot(j == 0 || !(ps <= 8192.0f)) != 0) {
      float m0 = fmaxf(fmaxf(s_acc[0][0], s_acc[0][1]), fmaxf(s_acc[1][0], s_acc[1][1]));
#pragma unroll
      for (int r = 2; r < 16; r += 2)
        m0 = fmaxf(m0, fmaxf(fmaxf(s_acc[0][r], s_acc[0][r + 1]), fmaxf(s_acc[1][r], s_acc[1][r + 1])));
      const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(m0), __float_as_uint(m0), false, false);
      const float xmax = fmaxf(__uint_as_float(sw[0]), __uint_as_float(sw[1]));
      const float shift = (j == 0 || xmax > kLazyRescale) ? xmax : 0.f;
      if (j != 0) {
        const float alpha = __builtin_amdgcn_exp2f(-shift);
        l_run *= alpha;
#pragma unroll
        for (int db = 0; db < 4; ++db) o_acc[db] *= alpha;
      }
      m_ref += shift;
#pragma unroll
      for (int r = 0; r < 16; ++r) neg_m[r] = -m_ref;
      exps(shift);
      ps = row_sum();
    }
#pragma unroll
    for (int q4 = 0; q4 < 4; ++q4) pf[q4] = __builtin_convertvector(e[q4], bf16x8_t);
    l_run += ps;
    __builtin_amdgcn_sched_barrier(0);
    if (k_next) dma_half(kg + hk, m0k[decltype(P)::value], koff);
    // K(j+1) and V(j), issued one VALU phase ago, must have landed before the
    // barrier; the four or eight instructions just issued may still fly.
    if (k_next && v_next)
      tracked_wait_vmcnt<8>();
    else if (k_next || v_next)
      tracked_wait_vmcnt<4>();
    else
      tracked_wait_vm_all();
  };

  // The output pointers are not needed before the end, but a scalar load
  // still in flight makes every LDS wait in the loop a wait for all LDS
  // reads (scalar loads return out of order): have them in registers now.
  asm volatile("" ::"s"(a.o), "s"(a.lse));
  // prologue: K(0), K(1), V(0)
  if (S > 0) {  // S >= 2
    const uint64_t h0 = half_off(0, __builtin_amdgcn_readfirstlane(route_raw(0)));
    dma_half(kg + h0, m0k[0], koff);
    dma_half(vg + h0, m0v[0], voff);
    hoff_next = half_off(1, __builtin_amdgcn_readfirstlane(route_raw(1)));
    dma_half(kg + hoff_next, m0k[1], koff);
  }
  tracked_wait_vm_all();
  barrier_nofence();

  int k = 0;
  if (team == 1) {  // the second team starts one phase late
    barrier_nofence();
    ++k;
  }
  auto step = [&](int j, auto P, auto Q) {
    mfma_phase(j, P, Q);
    phase_barrier();
    if (j < S) valu_phase(j, P, Q);
    phase_barrier();
  };
  if (S > 0) {
    for (int j = 0; j <= S; j += 2) {  // S is even
      step(j, Even{}, Odd{});
      if (j + 1 <= S) step(j + 1, Odd{}, Even{});
      k += j + 1 <= S ? 4 : 2;
    }
  }
  for (; k < phases; ++k) barrier_nofence();

  if (i < 0) return;
  if (nsp > 1) {  // split rows: this range's unnormalised O and its (max, sum)
    const float l_tot = l_run + __shfl_xor(l_run, 32);
    const int64_t prow = (static_cast<int64_t>(split) * (a.G / N) + h) * N * kBlock + qrow;
    float* po = a.part_o + prow * D;
#pragma unroll
    for (int db = 0; db < 4; ++db)
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4)
        *reinterpret_cast<float4*>(po + db * 32 + g4 * 8 + hh * 4) =
            S == 0 ? make_float4(0.f, 0.f, 0.f, 0.f)
                   : make_float4(o_acc[db][g4 * 4 + 0], o_acc[db][g4 * 4 + 1], o_acc[db][g4 * 4 + 2],
                                 o_acc[db][g4 * 4 + 3]);
    if (hh == 0) {
      a.part_ml[prow * 2] = S == 0 ? -INFINITY : m_ref;
      a.part_ml[prow * 2 + 1] = S == 0 ? 0.f : l_tot;
    }
    return;
  }
  // ---- normalise and store
  bf16_t* orow = static_cast<bf16_t*>(a.o) + (static_cast<int64_t>(h) * N * kBlock + qrow) * D;
  if (S == 0) {
#pragma unroll
    for (int db = 0; db < 4; ++db)
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4)
        *reinterpret_cast<uint2*>(orow + db * 32 + g4 * 8 + hh * 4) = make_uint2(0u, 0u);
    if (a.lse && hh == 0) a.lse[static_cast<int64_t>(h) * N * kBlock + qrow] = -INFINITY;
    return;
  }
  const float l_tot = l_run + __shfl_xor(l_run, 32);
  const float inv = 1.0f / l_tot;
#pragma unroll
  for (int db = 0; db < 4; ++db) {
#pragma unroll
    for (int g4 = 0; g4 < 4; ++g4) {
      const uint32_t w0 = static_cast<uint32_t>(f32_to_bf16(o_acc[db][g4 * 4 + 0] * inv)) |
                          (static_cast<uint32_t>(f32_to_bf16(o_acc[db][g4 * 4 + 1] * inv)) << 16);
      const uint32_t w1 = static_cast<uint32_t>(f32_to_bf16(o_acc[db][g4 * 4 + 2] * inv)) |
                          (static_cast<uint32_t>(f32_to_bf16(o_acc[db][g4 * 4 + 3] * inv)) << 16);
      *reinterpret_cast<uint2*>(orow + db * 32 + g4 * 8 + hh * 4) = make_uint2(w0, w1);
    }
  }
  if (a.lse && hh == 0)
    a.lse[static_cast<int64_t>(h) * N * kBlock + qrow] = m_ref * 0.6931471805599453f + logf(l_tot);
}


// ---------------------------------------------------------------- unit schedule
//
// plan_kernel (plan_split_kernel for split rows) writes the schedule of the
// routed kernel once per call, so that no attention workgroup spends its start
// ranking units. One workgroup per
// XCD: its contiguous range of (head, pair, range) ids (xcd_range), where a
// pair is ranks 2 pr and 2 pr + 1 of the head's rows ordered by route length
// (longest first, ties by row), and a unit's cost is its longer row's tile
// count. The units are ordered by cost, longest first (ties by id), and unit
// of dispatch rank `slot` on XCD x goes to workgroup slot * 8 + x; the
// hardware dispatches workgroups in id order as CUs free up, which makes the
// launch a longest-processing-time list schedule on every XCD. When the rows
// of an XCD do not fit in LDS, the units keep their id order (ranks are then
// counted in global memory).
struct PlanArgs {
  const int32_t* route_len;
  int route_head_rows;
  int H, N, M, L, include_current, n_split;
  int4* plan;
  float* part_ml;  // split rows: (max, sum) of every range, [n_split][H][N*128][2]
};

constexpr int kPlanThreads = 512;
constexpr int kPlanLdsInts = 12288;
constexpr int kCusPerXcd = 32;  // MI355X: 256 CUs in 8 XCDs

// Rank of value vme at index me among vals[0, n): the count of larger values
// and of equal ones at lower indices (descending order, ties by index). The
// LDS reads go out eight at a time, with one wait per eight.
__device__ __forceinline__ int rank_desc(const int* vals, int n, int me, int vme) {
  int rank = 0, o = 0;
  for (; o + 8 <= n; o += 8) {
    int x[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) x[u] = vals[o + u];
#pragma unroll
    for (int u = 0; u < 8; ++u) rank += (x[u] > vme) || (x[u] == vme && o + u < me);
  }
  for (; o < n; ++o) rank += (vals[o] > vme) || (vals[o] == vme && o < me);
  return rank;
}

// Split rows with a plan: each XCD owns a contiguous range of (head, pair)
// ids. A pair whose cost (its longer row's tiles) is c is cut into
// n = min(ceil(c / tau), n_split) ranges, with tau the smallest value for
// which the XCD's ranges fit one round of its CUs (at most kCusPerXcd units,
// never fewer than one per pair); the ranges of the XCD go longest first to
// its ceil(pairs / 8) * n_split slots, and the slots left over hold empty
// units (head -1), whose workgroups return at once. The ranges a pair does not use get (max, sum) =
// (-inf, 0), which the merge skips. Returns false when the XCD's rows do not
// fit in LDS (the caller then cuts every pair into n_split ranges).
__device__ bool plan_split_adaptive(const PlanArgs& a, int x, int* sh) {
  const int t = threadIdx.x;
  const int N = a.N, pairs = (N + 1) / 2, nsp = a.n_split;
  const int P = a.H * pairs;
  int pbase, pcnt;
  xcd_range(x, P, pbase, pcnt);
  const int slots = (P + kXcd - 1) / kXcd * nsp;  // this XCD's workgroups
  if (pcnt <= 0) {
    for (int s = t; s < slots; s += kPlanThreads) a.plan[s * kXcd + x] = make_int4(-1, -1, -1, 0);
    return true;
  }
  const int h_lo = pbase / pairs, nh = (pbase + pcnt - 1) / pairs - h_lo + 1;
  const int nr = nh * N;
  const int umax = max(pcnt, min(kCusPerXcd, pcnt * nsp));
  if (2 * nr + 4 * pcnt + 3 * umax + 6 > kPlanLdsInts) return false;
  const int ncur = a.include_current ? N : 0;
  int* lens_s = sh;                 // [nr]
  int* row_of = lens_s + nr;        // [nr]: row of rank k in its head
  int* pr_a = row_of + nr;          // [pcnt] longer row of the pair
  int* pr_b = pr_a + pcnt;          // [pcnt] other row or -1
  int* cost_s = pr_b + pcnt;        // [pcnt]
  int* nu_s = cost_s + pcnt;        // [pcnt] ranges of the pair
  int* u_pair = nu_s + pcnt;        // [umax] unit -> pair
  int* u_rng = u_pair + umax;       // [umax] unit -> range
  int* u_size = u_rng + umax;       // [umax] unit -> tiles of its longer range
  int* nunits = u_size + umax;      // [1]
  int* red = nunits + 1;            // [2]: largest cost, smallest fitting tau
  for (int e = t; e < nr; e += kPlanThreads) {
    const int h = h_lo + e / N, r = e % N;
    lens_s[e] = a.M == 0 ? 0 : min(max(a.route_len[static_cast<int64_t>(h) * a.route_head_rows + r], 0), a.L);
  }
  __syncthreads();
  for (int e = t; e < nr; e += kPlanThreads) {
    const int hb = e - e % N, me = e - hb;
    row_of[hb + rank_desc(lens_s + hb, N, me, lens_s[e])] = me;
  }
  __syncthreads();
  if (t == 0) {
    red[0] = 1;
    red[1] = 0x7fffffff;
  }
  __syncthreads();
  for (int w = t; w < pcnt; w += kPlanThreads) {
    const int hp = pbase + w, hb = (hp / pairs - h_lo) * N, pr = hp % pairs;
    const int ra = row_of[hb + 2 * pr];
    pr_a[w] = ra;
    pr_b[w] = 2 * pr + 1 < N ? row_of[hb + 2 * pr + 1] : -1;
    cost_s[w] = lens_s[hb + ra] + ncur;
    atomicMax(&red[0], cost_s[w]);
  }
  __syncthreads();
  // ranges of a pair of cost c for a given tau: min(max(ceil(c / tau), 1),
  // n_split), i.e. one plus the number of k in [1, n_split) with c > k tau
  auto ranges_of = [nsp](int c, int tau) {
    int nu = 1;
    for (int k = 1; k < nsp; ++k) nu += c > k * tau;
    return nu;
  };
  // the smallest tau in [1, largest cost] whose range count fits umax (the
  // largest cost always does: one range per pair), every tau counted by its
  // own thread
  {
    const int cmax = red[0];
    for (int tau = 1 + t; tau <= cmax; tau += kPlanThreads) {
      int cnt = 0, w = 0;
      for (; w + 8 <= pcnt; w += 8) {
        int c[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) c[u] = cost_s[w + u];
#pragma unroll
        for (int u = 0; u < 8; ++u) cnt += ranges_of(c[u], tau);
      }
      for (; w < pcnt; ++w) cnt += ranges_of(cost_s[w], tau);
      if (cnt <= umax) {
        atomicMin(&red[1], tau);
        break;  // larger taus of this thread fit too
      }
    }
  }
  __syncthreads();
  const int lo = red[1];
  for (int w = t; w < pcnt; w += kPlanThreads) nu_s[w] = ranges_of(cost_s[w], lo);
  __syncthreads();
  // units in pair order: pair w's ranges start after those of pairs 0 .. w-1
  for (int w = t; w < pcnt; w += kPlanThreads) {
    int first = 0, o = 0;
    for (; o + 8 <= w; o += 8) {
      int c[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) c[u] = nu_s[o + u];
#pragma unroll
      for (int u = 0; u < 8; ++u) first += c[u];
    }
    for (; o < w; ++o) first += nu_s[o];
    const int nu = nu_s[w], size = (cost_s[w] + nu - 1) / nu;
    for (int r = 0; r < nu; ++r) {
      u_pair[first + r] = w;
      u_rng[first + r] = r;
      u_size[first + r] = size;
    }
    if (w == pcnt - 1) nunits[0] = first + nu;
  }
  __syncthreads();
  const int n = nunits[0];
  // unit of dispatch rank `slot`: sizes descending, ties by unit index
  for (int u = t; u < n; u += kPlanThreads) {
    const int slot = rank_desc(u_size, n, u, u_size[u]);
    const int w = u_pair[u];
    a.plan[slot * kXcd + x] = make_int4((pbase + w) / pairs, pr_a[w], pr_b[w], u_rng[u] | (nu_s[w] << 8));
  }
  for (int s = n + t; s < slots; s += kPlanThreads) a.plan[s * kXcd + x] = make_int4(-1, -1, -1, 0);
  // (max, sum) = (-inf, 0) for the ranges a pair leaves unused: one wave per
  // (pair, range, row) triple writes the 128 queries' pairs (1 KiB, 16 bytes
  // per lane)
  const int64_t rows = static_cast<int64_t>(a.H) * N * kBlock;
  const int lane = t % kWave, wave = t / kWave;
  for (int tr = wave; tr < pcnt * nsp * 2; tr += kPlanThreads / kWave) {
    const int w = tr / (2 * nsp), r = (tr >> 1) % nsp, side = tr & 1;
    const int row = side ? pr_b[w] : pr_a[w];
    if (r < nu_s[w] || row < 0) continue;
    const int h = (pbase + w) / pairs;
    const int64_t idx = static_cast<int64_t>(r) * rows + (static_cast<int64_t>(h) * N + row) * kBlock + 2 * lane;
    *reinterpret_cast<float4*>(a.part_ml + idx * 2) = make_float4(-INFINITY, 0.f, -INFINITY, 0.f);
  }
  return true;
}

// Units of equal ranges (every pair cut into n_split ranges, or none), the
// XCD's share of them longest first.
__device__ void plan_uniform(const PlanArgs& a, int x, int* sh) {
  const int t = threadIdx.x;
  const int N = a.N, pairs = (N + 1) / 2, nsp = max(a.n_split, 1);
  const int G = a.H * pairs * nsp;
  int base, cnt;
  xcd_range(x, G, base, cnt);
  if (nsp > 1) {  // the launch has ceil(pairs / 8) * nsp slots per XCD
    const int slots = (a.H * pairs + kXcd - 1) / kXcd * nsp;
    for (int s = max(cnt, 0) + t; s < slots; s += kPlanThreads) a.plan[s * kXcd + x] = make_int4(-1, -1, -1, 0);
  }
  if (cnt <= 0) return;
  const int h_lo = base / nsp / pairs, nh = (base + cnt - 1) / nsp / pairs - h_lo + 1;
  const int nr = nh * N;
  const int ncur = a.include_current ? N : 0;
  auto row_len = [&](int h, int r) {
    return a.M == 0 ? 0 : min(max(a.route_len[static_cast<int64_t>(h) * a.route_head_rows + r], 0), a.L);
  };
  // the row of rank `rank` in head h, by a scan of the head's lengths
  auto rank_in_head = [](const int* lens, int n, int me, int vme) {
    int rank = 0;
    for (int o = 0; o < n; ++o) rank += (lens[o] > vme) || (lens[o] == vme && o < me);
    return rank;
  };
  if (3 * nr + cnt <= kPlanLdsInts) {
    int* lens_s = sh;              // [nr]
    int* row_of = lens_s + nr;     // [nr]: row of rank k in its head
    int* cost_s = row_of + nr;     // [cnt]
    int* rank_s = cost_s + cnt;    // [nr]
    for (int e = t; e < nr; e += kPlanThreads) lens_s[e] = row_len(h_lo + e / N, e % N);
    __syncthreads();
    for (int e = t; e < nr; e += kPlanThreads) {
      const int hb = e - e % N;
      const int rank = rank_in_head(lens_s + hb, N, e - hb, lens_s[e]);
      rank_s[e] = rank;
      row_of[hb + rank] = e - hb;
    }
    __syncthreads();
    for (int w = t; w < cnt; w += kPlanThreads) {
      const int id = (base + w) / nsp;
      cost_s[w] = lens_s[(id / pairs - h_lo) * N + row_of[(id / pairs - h_lo) * N + 2 * (id % pairs)]] + ncur;
    }
    __syncthreads();
    for (int w = t; w < cnt; w += kPlanThreads) {
      const int cw = cost_s[w];
      int slot = 0;
      for (int o = 0; o < cnt; ++o) slot += (cost_s[o] > cw) || (cost_s[o] == cw && o < w);
      const int id = base + w, hp = id / nsp, h = hp / pairs, pr = hp % pairs;
      const int hb = (h - h_lo) * N;
      const int ra = row_of[hb + 2 * pr];
      const int rb = 2 * pr + 1 < N ? row_of[hb + 2 * pr + 1] : -1;
      a.plan[slot * kXcd + x] = make_int4(h, ra, rb, (id % nsp) | (nsp << 8));
    }
  } else {
    for (int w = t; w < cnt; w += kPlanThreads) {
      const int id = base + w, hp = id / nsp, h = hp / pairs, pr = hp % pairs;
      int ra = -1, rb = -1;
      for (int r = 0; r < N; ++r) {
        const int lr = row_len(h, r);
        int rank = 0;
        for (int o = 0; o < N; ++o) {
          const int lo = row_len(h, o);
          rank += (lo > lr) || (lo == lr && o < r);
        }
        if (rank == 2 * pr) ra = r;
        if (rank == 2 * pr + 1) rb = r;
      }
      a.plan[w * kXcd + x] = make_int4(h, ra, rb, (id % nsp) | (nsp << 8));
    }
  }
}

// One workgroup per XCD writes that XCD's units: plan_kernel for unsplit
// rows, plan_split_kernel for split rows (adaptive ranges, or equal ranges
// when the XCD's rows do not fit in LDS).
__global__ __launch_bounds__(kPlanThreads) void plan_kernel(PlanArgs a) {
  __shared__ int sh[kPlanLdsInts];
  plan_uniform(a, blockIdx.x, sh);
}
__global__ __launch_bounds__(kPlanThreads) void plan_split_kernel(PlanArgs a) {
  __shared__ int sh[kPlanLdsInts];
  if (!(a.part_ml && plan_split_adaptive(a, blockIdx.x, sh))) plan_uniform(a, blockIdx.x, sh);
}

}  // namespace pp

// Combines the n_split ranges of every query row (eight threads per row, 16
// dims each): m = max m_s, l = sum of 2^(m_s - m) l_s, O = sum of
// 2^(m_s - m) O_s / l, lse = m ln 2 + ln l; a row without any tile gets O = 0
// and lse = -inf. rows = H * N * 128, in the layout of o and lse. The maxima of
// all ranges and the partial outputs of the first four are requested together;
// further ranges, four at a time, only up to the row's last range with tiles
// (the ranges a unit plan leaves unused follow the used ones). Each group is
// folded into a running maximum, weight sum and output; a range without tiles
// (maximum -inf; its partial output was never written) is dropped by a
// select, so its memory never enters the sums.
constexpr int kMergeMaxSplit = 16;
__global__ __launch_bounds__(256) void split_merge_kernel(const float* __restrict__ part_o,
                                                          const float* __restrict__ part_ml, int n_split,
                                                          int64_t rows, bf16_t* __restrict__ o,
                                                          float* __restrict__ lse) {
  const int64_t gid = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  const int64_t row = gid >> 3;
  const int eighth = static_cast<int>(gid & 7);
  if (row >= rows) return;
  auto range_row = [&](int s) { return static_cast<int64_t>(min(s, n_split - 1)) * rows + row; };
  float2 ml[kMergeMaxSplit];
#pragma unroll
  for (int s = 0; s < kMergeMaxSplit; ++s) ml[s] = *reinterpret_cast<const float2*>(part_ml + range_row(s) * 2);
  float4 x[4][4];
  auto load_group = [&](int s0) {
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const float4* src = reinterpret_cast<const float4*>(part_o + range_row(s0 + u) * 128 + eighth * 16);
#pragma unroll
      for (int c = 0; c < 4; ++c) x[u][c] = src[c];
    }
  };
  load_group(0);
  int n_used = 0;
#pragma unroll
  for (int s = 0; s < kMergeMaxSplit; ++s)
    if (s < n_split && ml[s].x != -INFINITY) n_used = s + 1;
  float m = -INFINITY, l = 0.f, acc[16];
#pragma unroll
  for (int e = 0; e < 16; ++e) acc[e] = 0.f;
  auto fold = [&](int s0) {
    bool use[4];
    float mc = m;
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      use[u] = s0 + u < n_used && ml[s0 + u].x != -INFINITY;
      if (use[u]) mc = fmaxf(mc, ml[s0 + u].x);
    }
    if (mc == -INFINITY) return;  // no tile in this row so far
    const float a = __builtin_amdgcn_exp2f(m - mc);  // 0 while m is -inf
    l *= a;
#pragma unroll
    for (int e = 0; e < 16; ++e) acc[e] *= a;
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const float w = use[u] ? __builtin_amdgcn_exp2f(ml[s0 + u].x - mc) : 0.f;
      l += use[u] ? w * ml[s0 + u].y : 0.f;
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        acc[4 * c + 0] += use[u] ? w * x[u][c].x : 0.f;
        acc[4 * c + 1] += use[u] ? w * x[u][c].y : 0.f;
        acc[4 * c + 2] += use[u] ? w * x[u][c].z : 0.f;
        acc[4 * c + 3] += use[u] ? w * x[u][c].w : 0.f;
      }
    }
    m = mc;
  };
  fold(0);
#pragma unroll
  for (int s0 = 4; s0 < kMergeMaxSplit; s0 += 4) {
    if (s0 < n_used) {
      load_group(s0);
      fold(s0);
    }
  }
  const float inv = l > 0.f ? 1.0f / l : 0.f;
  uint32_t w[8];
#pragma unroll
  for (int e2 = 0; e2 < 8; ++e2)
    w[e2] = static_cast<uint32_t>(f32_to_bf16(acc[2 * e2] * inv)) |
            (static_cast<uint32_t>(f32_to_bf16(acc[2 * e2 + 1] * inv)) << 16);
  uint4* dst = reinterpret_cast<uint4*>(o + row * 128 + eighth * 16);
  dst[0] = make_uint4(w[0], w[1], w[2], w[3]);
  dst[1] = make_uint4(w[4], w[5], w[6], w[7]);
  if (lse && eighth == 0) lse[row] = l > 0.f ? m * 0.6931471805599453f + logf(l) : -INFINITY;
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
    const int64_t rr = route_row(a, h, i);
    route = a.route_ids + rr * a.L;
    rlen = min(max(a.route_len[rr], 0), a.L);
    if (M == 0) rlen = 0;
  }
  const int ncur = (!kRouted || a.include_current) ? a.N : 0;
  const int T = rlen + ncur;
  const int qrow = i * kBlock + qr;

  float qv[kHalf], ov[kHalf];
#pragma unroll
  for (int c = 0; c < kHalf; ++c) {
    qv[c] = qh[static_cast<int64_t>(qrow) * D + half * kHalf + c];
    ov[c] = 0.f;
  }
  float m_run = -INFINITY, l_run = 0.f;
  for (int j = 0; j < T; ++j) {
    const int tile = tile_at<kRouted>(route, ncur, M, j);
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
  // d = 128: the ping-pong kernel (routes of up to pp::kMaxRoute tiles), else
  // swizzled tiles filled by direct DMA (up to kMaxRouteLds tiles); otherwise
  // padded tiles staged through registers.
  if (bf16 && D == 128 && (!kRouted || args.L <= pp::kMaxRoute)) {
    const int pairs = (args.N + 1) / 2;
    const int nsp = args.n_split > 1 ? args.n_split : 1;
    AttnArgs run = args;
    if (!kRouted) run.plan = nullptr;
    if (kRouted && run.plan) {
      pp::PlanArgs pa{args.route_len, args.route_head_rows, args.G / args.N, args.N, args.M,
                      args.L, args.include_current, nsp, const_cast<int4*>(run.plan),
                      nsp > 1 ? args.part_ml : nullptr};
      if (nsp > 1)
        hipLaunchKernelGGL(pp::plan_split_kernel, dim3(kXcd), dim3(pp::kPlanThreads), 0, stream, pa);
      else
        hipLaunchKernelGGL(pp::plan_kernel, dim3(kXcd), dim3(pp::kPlanThreads), 0, stream, pa);
      const hipError_t e = hipGetLastError();
      if (e != hipSuccess) return e;
    }
    // with a plan, split rows get ceil(pairs / 8) * nsp slots on every XCD
    const int units = (args.G / args.N) * pairs;
    const int grid = kRouted && run.plan && nsp > 1 ? kXcd * ((units + kXcd - 1) / kXcd) * nsp : units * nsp;
    hipLaunchKernelGGL((pp::attn_kernel<kRouted>), dim3(grid), dim3(pp::kThreads), 0, stream, run);
    if (nsp > 1) {
      hipError_t e = hipGetLastError();
      if (e != hipSuccess) return e;
      const int64_t rows = static_cast<int64_t>(args.G) * kBlock;
      hipLaunchKernelGGL(split_merge_kernel, dim3(static_cast<unsigned>((rows * 8 + 255) / 256)), dim3(256), 0,
                         stream, args.part_o, args.part_ml, nsp, rows, static_cast<bf16_t*>(args.o), args.lse);
    }
    return hipGetLastError();
  }
  const bool fast = D == 128 && (!kRouted || args.L <= kMaxRouteLds);
  if (bf16 && fast)
    hipLaunchKernelGGL((attn_bf16_kernel<D, kRouted, D == 128, D == 128>), dim3(args.G), dim3(256),
                       0, stream, args);
  else if (bf16)
    hipLaunchKernelGGL((attn_bf16_kernel<D, kRouted, false, false>), dim3(args.G), dim3(256), 0,
                       stream, args);
  else
    hipLaunchKernelGGL((attn_f32_kernel<D, kRouted>), dim3(args.G), dim3(256), 0, stream, args);
  return hipGetLastError();
}

size_t attn_plan_bytes(int H, int N, int n_split) {
  if (H < 1 || N < 1) return 0;
  const size_t pairs = static_cast<size_t>(H) * ((N + 1) / 2);
  // split rows: every XCD gets ceil(pairs / 8) * n_split slots
  const size_t units = n_split > 1 ? kXcd * ((pairs + kXcd - 1) / kXcd) * n_split : pairs;
  return units * sizeof(int4);
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
  a.route_head_rows = c.shared_routes ? 0 : c.N;
  a.include_current = c.include_current;
  a.o = c.o;
  a.lse = c.lse;
  const bool routed = c.route_ids != nullptr;
  // rows are split only in the d = 128 bf16 kernel; elsewhere n_split is ignored
  const bool pp_path = c.bf16 && c.d == 128 && (!routed || c.L <= pp::kMaxRoute);
  a.n_split = pp_path && c.n_split > 1 ? c.n_split : 1;
  a.part_o = c.part_o;
  a.part_ml = c.part_ml;
  a.plan = pp_path && routed ? static_cast<const int4*>(c.plan) : nullptr;
  if (c.d == 128)
    return routed ? launch_one<128, true>(a, c.bf16, stream) : launch_one<128, false>(a, c.bf16, stream);
  return routed ? launch_one<64, true>(a, c.bf16, stream) : launch_one<64, false>(a, c.bf16, stream);
}

}  // namespace velox
