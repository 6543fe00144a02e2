// Device helpers shared by the library's kernels (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace velox {

constexpr int kBlock = 128;   // tokens per block = attention tile
constexpr int kWave = 64;

typedef uint16_t bf16_t;      // bf16 bit pattern

__device__ __forceinline__ float bf16_to_f32(bf16_t x) {
  return __uint_as_float(static_cast<uint32_t>(x) << 16);
}

// Round-to-nearest-even fp32 -> bf16 (NaN kept quiet).
__device__ __forceinline__ bf16_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return static_cast<bf16_t>((u >> 16) | 0x40u);
  u += 0x7fffu + ((u >> 16) & 1u);
  return static_cast<bf16_t>(u >> 16);
}

template <typename T> __device__ __forceinline__ float load_f32(const T* p);
template <> __device__ __forceinline__ float load_f32<float>(const float* p) { return *p; }
template <> __device__ __forceinline__ float load_f32<bf16_t>(const bf16_t* p) {
  return bf16_to_f32(*p);
}

// Workgroup ids are dispatched round-robin over the 8 XCDs of an MI355X.
// Remap so that consecutive logical ids land on the same XCD (and share its
// L2): XCD x receives a contiguous range of logical ids. Bijective on [0, G).
constexpr int kXcd = 8;
__device__ __forceinline__ int xcd_remap(int b, int G) {
  const int per = G / kXcd, rem = G % kXcd;
  const int x = b % kXcd, slot = b / kXcd;
  return x < rem ? x * (per + 1) + slot : rem * (per + 1) + (x - rem) * per + slot;
}
// The contiguous logical range [base, base + cnt) that xcd_remap gives XCD x.
__device__ __forceinline__ void xcd_range(int x, int G, int& base, int& cnt) {
  const int per = G / kXcd, rem = G % kXcd;
  base = x < rem ? x * (per + 1) : rem * (per + 1) + (x - rem) * per;
  cnt = per + (x < rem ? 1 : 0);
}

}  // namespace velox
