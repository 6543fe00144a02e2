// C ABI of libvelox: argument validation, error reporting and dispatch to the
// kernel launchers. Declarations, layouts and the cited definitions of each
// operation are in include/velox.h, include/velox_geometry.h,
// include/velox_layout.h and include/velox_slabs.h.

#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <mutex>
#include <string>

#include "../../include/velox.h"
#include "../../include/velox_geometry.h"
#include "../../include/velox_layout.h"
#include "../../include/velox_slabs.h"
#include "velox_launch.hpp"

namespace {

thread_local std::string g_last_error;

velox_status_t fail(velox_status_t st, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return st;
}

velox_status_t launched(hipError_t e, const char* what) {
  if (e != hipSuccess) return fail(VELOX_ERR_LAUNCH, "%s: %s", what, hipGetErrorString(e));
  return VELOX_OK;
}

bool dtype_ok(velox_dtype_t dt) { return dt == VELOX_F32 || dt == VELOX_BF16; }
bool dim_ok(int d) { return d == 64 || d == 128; }

#define REQUIRE(cond, ...)                                    \
  do {                                                        \
    if (!(cond)) return fail(VELOX_ERR_INVALID, __VA_ARGS__); \
  } while (0)

velox_status_t check_common(velox_dtype_t dt, int H, int N, int M, int d) {
  REQUIRE(dtype_ok(dt), "dtype must be VELOX_F32 or VELOX_BF16 (got %d)", static_cast<int>(dt));
  REQUIRE(dim_ok(d), "d must be 64 or 128 (got %d)", d);
  REQUIRE(H >= 1 && N >= 1, "H and N must be >= 1 (got H=%d N=%d)", H, N);
  REQUIRE(M >= 0, "M must be >= 0 (got %d)", M);
  if (M > VELOX_MAX_HISTORY)
    return fail(VELOX_ERR_UNSUPPORTED, "M=%d exceeds VELOX_MAX_HISTORY=%d", M, VELOX_MAX_HISTORY);
  return VELOX_OK;
}

velox_status_t check_attn(const void* q, const void* k, const void* v, velox_dtype_t dt,
                          int64_t ld_q_h, int64_t ld_kv_h, int H, int N, int M, int d,
                          float scale, const void* o) {
  velox_status_t st = check_common(dt, H, N, M, d);
  if (st != VELOX_OK) return st;
  REQUIRE(q && k && v && o, "q, k, v and o must be non-NULL");
  REQUIRE(ld_q_h >= static_cast<int64_t>(N) * VELOX_BLOCK * d,
          "ld_q_h=%lld is smaller than N*128*d=%lld", static_cast<long long>(ld_q_h),
          static_cast<long long>(N) * VELOX_BLOCK * d);
  REQUIRE(ld_kv_h >= static_cast<int64_t>(M + N) * VELOX_BLOCK * d,
          "ld_kv_h=%lld is smaller than (M+N)*128*d=%lld", static_cast<long long>(ld_kv_h),
          static_cast<long long>(M + N) * VELOX_BLOCK * d);
  REQUIRE(std::isfinite(scale) && scale > 0.f, "scale must be finite and > 0");
  const size_t align = dt == VELOX_BF16 ? 16 : 16;
  REQUIRE(reinterpret_cast<uintptr_t>(q) % align == 0 && reinterpret_cast<uintptr_t>(k) % align == 0 &&
              reinterpret_cast<uintptr_t>(v) % align == 0 && reinterpret_cast<uintptr_t>(o) % align == 0,
          "q, k, v and o must be 16-byte aligned");
  REQUIRE(ld_q_h % 8 == 0 && ld_kv_h % 8 == 0, "head strides must be multiples of 8 elements");
  return VELOX_OK;
}

}  // namespace

static int64_t elem_bytes(velox_dtype_t dt) { return dt == VELOX_BF16 ? 2 : 4; }

static velox_status_t check_geometry_sizes(int N, int M) {
  REQUIRE(N >= 0 && M >= 0, "N and M must be >= 0 (got N=%d M=%d)", N, M);
  REQUIRE(N <= 65535, "N=%d exceeds 65535", N);
  return VELOX_OK;
}

// ---------------------------------------------------------------- no-allocation entry

// The unit plan of velox_sparse_attn_noalloc: a fixed array in the global
// memory of every device the library runs on, held until the process ends.
// Host code never passes `scratch` itself to a kernel (on the host the name
// stands for a host-side shadow, not a device address); it uses the device
// address resolved once per device below.
static __device__ __align__(256) int4 scratch[VELOX_NOALLOC_MAX_UNITS];

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// Device address of the current device's scratch array (hipGetSymbolAddress
// on the first call on a device, with that device current; cached after).
velox_status_t scratch_address(void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail(VELOX_ERR_LAUNCH, "hipGetDevice: %s", hipGetErrorString(e));
  if (dev < 0 || dev >= kMaxDevices)
    return fail(VELOX_ERR_UNSUPPORTED, "device %d is beyond the %d the library tracks", dev, kMaxDevices);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || p == nullptr)
      return fail(VELOX_ERR_LAUNCH, "hipGetSymbolAddress(scratch) on device %d: %s", dev,
                  e != hipSuccess ? hipGetErrorString(e) : "null address");
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return VELOX_OK;
}

}  // namespace

extern "C" {

const char* velox_last_error(void) { return g_last_error.c_str(); }

int velox_version(void) { return 100; }

velox_status_t velox_block_mean(const void* x, velox_dtype_t dt, int64_t ld_x_h, int H, int nblk,
                                int d, float* xbar, int64_t ld_bar_h, void* stream) {
  REQUIRE(dtype_ok(dt), "dtype must be VELOX_F32 or VELOX_BF16");
  REQUIRE(dim_ok(d), "d must be 64 or 128 (got %d)", d);
  REQUIRE(H >= 1 && nblk >= 0, "need H >= 1 and nblk >= 0 (got H=%d nblk=%d)", H, nblk);
  if (nblk == 0) return VELOX_OK;
  REQUIRE(x && xbar, "x and xbar must be non-NULL");
  REQUIRE(ld_x_h >= static_cast<int64_t>(nblk) * VELOX_BLOCK * d, "ld_x_h too small");
  REQUIRE(ld_bar_h >= static_cast<int64_t>(nblk) * d, "ld_bar_h too small");
  REQUIRE(reinterpret_cast<uintptr_t>(x) % 16 == 0 && (ld_x_h * elem_bytes(dt)) % 16 == 0,
          "x and its head stride must be 16-byte aligned");
  return launched(velox::launch_block_mean(x, dt == VELOX_BF16, ld_x_h, H, nblk, d, xbar, ld_bar_h,
                                           static_cast<hipStream_t>(stream)),
                  "velox_block_mean");
}

velox_status_t velox_route_scores(const void* q, velox_dtype_t dt, int64_t ld_q_h,
                                  const float* kbar, int64_t ld_kbar_h, int H, int N, int M, int d,
                                  float scale, float* p, void* stream) {
  velox_status_t st = check_common(dt, H, N, M, d);
  if (st != VELOX_OK) return st;
  if (M == 0) return VELOX_OK;
  REQUIRE(q && kbar && p, "q, kbar and p must be non-NULL");
  REQUIRE(ld_q_h >= static_cast<int64_t>(N) * VELOX_BLOCK * d, "ld_q_h too small");
  REQUIRE(ld_kbar_h >= static_cast<int64_t>(M) * d, "ld_kbar_h too small");
  REQUIRE(std::isfinite(scale), "scale must be finite");
  REQUIRE(reinterpret_cast<uintptr_t>(q) % 16 == 0 && (ld_q_h * elem_bytes(dt)) % 16 == 0,
          "q and its head stride must be 16-byte aligned");
  REQUIRE(reinterpret_cast<uintptr_t>(kbar) % 16 == 0 && ld_kbar_h % 4 == 0,
          "kbar and its head stride must be 16-byte aligned");
  if (velox::route_scores_lds_bytes(1, M, d) > velox::kMaxLdsBytes)
    return fail(VELOX_ERR_UNSUPPORTED, "M=%d too large for route_scores", M);
  return launched(velox::launch_route_scores(q, dt == VELOX_BF16, ld_q_h, kbar, ld_kbar_h, H, N, M, d,
                                             scale, p, static_cast<hipStream_t>(stream)),
                  "velox_route_scores");
}

velox_status_t velox_route_scores_shared(const void* q, velox_dtype_t dt, int64_t ld_q_h,
                                         const float* kbar, int64_t ld_kbar_h, int H, int N, int M,
                                         int d, float scale, float* logits, float* p,
                                         void* stream) {
  velox_status_t st = check_common(dt, H, N, M, d);
  if (st != VELOX_OK) return st;
  if (M == 0) return VELOX_OK;
  REQUIRE(q && kbar && logits && p, "q, kbar, logits and p must be non-NULL");
  REQUIRE(ld_q_h >= static_cast<int64_t>(N) * VELOX_BLOCK * d, "ld_q_h too small");
  REQUIRE(ld_kbar_h >= static_cast<int64_t>(M) * d, "ld_kbar_h too small");
  REQUIRE(std::isfinite(scale), "scale must be finite");
  REQUIRE(reinterpret_cast<uintptr_t>(q) % 16 == 0 && (ld_q_h * elem_bytes(dt)) % 16 == 0,
          "q and its head stride must be 16-byte aligned");
  REQUIRE(reinterpret_cast<uintptr_t>(kbar) % 16 == 0 && ld_kbar_h % 4 == 0,
          "kbar and its head stride must be 16-byte aligned");
  if (velox::route_scores_lds_bytes(1, M, d) > velox::kMaxLdsBytes)
    return fail(VELOX_ERR_UNSUPPORTED, "M=%d too large for route_scores", M);
  return launched(velox::launch_route_scores_shared(q, dt == VELOX_BF16, ld_q_h, kbar, ld_kbar_h, H, N,
                                                    M, d, scale, logits, p,
                                                    static_cast<hipStream_t>(stream)),
                  "velox_route_scores_shared");
}

velox_status_t velox_route_select(const float* p, const float* g, const float* rho,
                                  const int32_t* coord, int H, int N, int M,
                                  const velox_route_params_t* prm, int L, int32_t* route_ids,
                                  int32_t* route_len, void* stream) {
  REQUIRE(prm, "prm must be non-NULL");
  REQUIRE(H >= 1 && N >= 1 && M >= 0, "need H >= 1, N >= 1, M >= 0 (got H=%d N=%d M=%d)", H, N, M);
  if (M > VELOX_MAX_HISTORY)
    return fail(VELOX_ERR_UNSUPPORTED, "M=%d exceeds VELOX_MAX_HISTORY=%d", M, VELOX_MAX_HISTORY);
  REQUIRE(route_ids && route_len, "route_ids and route_len must be non-NULL");
  REQUIRE(M == 0 || (p && g && rho), "p, g and rho must be non-NULL when M > 0");
  REQUIRE(!prm->neigh26 || coord, "coord must be non-NULL when neigh26 is set");
  REQUIRE(prm->n_ref >= 0 && (prm->n_ref == 0 || prm->ref_ids), "ref_ids must hold n_ref ids");
  REQUIRE(prm->K_cov >= 0 && prm->K_unc >= 0, "K_cov and K_unc must be >= 0");
  REQUIRE(prm->n_prev >= 0 && prm->n_prev <= M, "n_prev must lie in [0, M] (got %d, M=%d)",
          prm->n_prev, M);
  REQUIRE(std::isfinite(prm->tau) && std::isfinite(prm->eta_cov), "tau and eta_cov must be finite");
  REQUIRE(std::isfinite(prm->g_ref) && prm->g_ref > 0.f, "g_ref must be finite and > 0");
  REQUIRE(prm->lambda >= 0.f && prm->lambda <= 14.f, "lambda must lie in [0, 14]");
  REQUIRE(prm->theta_cov > 0.f && prm->theta_unc > 0.f, "theta_cov and theta_unc must be > 0");
  REQUIRE(prm->neigh26 == 0 || prm->neigh26 == 1, "neigh26 must be 0 or 1");
  REQUIRE(prm->mode >= VELOX_ROUTE_FUSED && prm->mode <= VELOX_ROUTE_GEOMETRY_ONLY,
          "mode must be VELOX_ROUTE_FUSED, _MODEL_ONLY or _GEOMETRY_ONLY (got %d)", prm->mode);
  const long long kmax = prm->K_cov > prm->K_unc ? prm->K_cov : prm->K_unc;
  const long long base = kmax > prm->n_prev ? kmax : prm->n_prev;
  long long need = base + 26LL * prm->neigh26 + prm->n_ref;
  if (need > M) need = M;
  if (need < 1) need = 1;
  REQUIRE(L >= need, "L=%d is smaller than the route bound %lld", L, need);
  velox::RouteConfig cfg{prm->tau,       prm->g_ref,     prm->lambda, prm->eta_cov,
                         prm->theta_cov, prm->theta_unc, prm->K_cov,  prm->K_unc,
                         prm->n_prev,    prm->neigh26,   prm->mode,   prm->ref_ids,
                         prm->n_ref,     prm->status};
  return launched(velox::launch_route_select(p, g, rho, coord, H, N, M, cfg, L, route_ids, route_len,
                                             static_cast<hipStream_t>(stream)),
                  "velox_route_select");
}

velox_status_t velox_route_check(const int32_t* route_ids, const int32_t* route_len, int rows,
                                 int M, int L, int32_t* bad, void* stream) {
  REQUIRE(rows >= 0 && M >= 0 && L >= 1, "need rows >= 0, M >= 0, L >= 1 (got %d, %d, %d)", rows, M, L);
  REQUIRE(bad, "bad must be non-NULL");
  REQUIRE(rows == 0 || (route_ids && route_len), "route_ids and route_len must be non-NULL");
  return launched(velox::launch_route_check(route_ids, route_len, rows, M, L, bad,
                                            static_cast<hipStream_t>(stream)),
                  "velox_route_check");
}

size_t velox_attn_split_workspace_size(int H, int N, int n_split) {
  if (H < 1 || N < 1 || n_split < 1) return 0;
  const size_t rows = static_cast<size_t>(n_split) * H * N * VELOX_BLOCK;
  return rows * (128 + 2) * sizeof(float) + velox::attn_plan_bytes(H, N, n_split);
}

size_t velox_sparse_attn_workspace_size(int H, int N, int L, int d) {
  if (L < 1 || d < 1) return 0;
  return velox::attn_plan_bytes(H, N, 1);
}

// split_merge_kernel folds at most 16 ranges per row (kMergeMaxSplit)
static_assert(VELOX_MAX_SPLIT <= 16, "the split-row merge reads at most 16 ranges per row");

// Split settings into the launch config: the workspace holds part_o
// [n_split][rows][128], then part_ml [n_split][rows][2], then the unit plan.
static velox_status_t set_split(velox::AttnConfig& c, int n_split, void* workspace,
                                size_t workspace_bytes) {
  REQUIRE(n_split >= 1 && n_split <= VELOX_MAX_SPLIT, "n_split must be in [1, %d] (got %d)",
          VELOX_MAX_SPLIT, n_split);
  c.n_split = n_split;
  if (n_split == 1) return VELOX_OK;
  const size_t need = velox_attn_split_workspace_size(c.H, c.N, n_split);
  REQUIRE(workspace, "workspace must be non-NULL when n_split > 1");
  REQUIRE(workspace_bytes >= need, "workspace of %zu bytes is smaller than the %zu needed",
          workspace_bytes, need);
  REQUIRE(reinterpret_cast<uintptr_t>(workspace) % 16 == 0, "workspace must be 16-byte aligned");
  const size_t rows = static_cast<size_t>(n_split) * c.H * c.N * VELOX_BLOCK;
  c.part_o = static_cast<float*>(workspace);
  c.part_ml = c.part_o + rows * 128;
  if (c.route_ids) c.plan = c.part_ml + rows * 2;
  return VELOX_OK;
}

static velox_status_t sparse_common(const void* q, const void* k, const void* v, velox_dtype_t dt,
                                    int64_t ld_q_h, int64_t ld_kv_h, int H, int N, int M, int d,
                                    float scale, const int32_t* route_ids, const int32_t* route_len,
                                    int L, int include_current, void* o, float* lse, void* stream,
                                    bool shared, const char* what, int n_split = 1,
                                    void* workspace = nullptr, size_t workspace_bytes = 0,
                                    void* plan = nullptr) {
  velox_status_t st = check_attn(q, k, v, dt, ld_q_h, ld_kv_h, H, N, M, d, scale, o);
  if (st != VELOX_OK) return st;
  REQUIRE(route_ids && route_len, "route_ids and route_len must be non-NULL");
  REQUIRE(L >= 1, "L must be >= 1");
  REQUIRE(include_current == 0 || include_current == 1, "include_current must be 0 or 1");
  REQUIRE(reinterpret_cast<uintptr_t>(plan) % 16 == 0, "workspace must be 16-byte aligned");
  velox::AttnConfig c{q, k, v, dt == VELOX_BF16, ld_q_h, ld_kv_h, H, N, M, d, scale,
                      route_ids, route_len, L, shared, include_current, o, lse};
  c.plan = plan;
  st = set_split(c, n_split, workspace, workspace_bytes);
  if (st != VELOX_OK) return st;
  return launched(velox::launch_attention(c, static_cast<hipStream_t>(stream)), what);
}

velox_status_t velox_sparse_attn(const void* q, const void* k, const void* v, velox_dtype_t dt,
                                 int64_t ld_q_h, int64_t ld_kv_h, int H, int N, int M, int d,
                                 float scale, const int32_t* route_ids, const int32_t* route_len,
                                 int L, int include_current, void* o, float* lse, void* workspace,
                                 void* stream) {
  return sparse_common(q, k, v, dt, ld_q_h, ld_kv_h, H, N, M, d, scale, route_ids, route_len, L,
                       include_current, o, lse, stream, false, "velox_sparse_attn", 1, nullptr, 0,
                       workspace);
}


velox_status_t velox_sparse_attn_noalloc(const void* q, const void* k, const void* v,
                                         velox_dtype_t dt, int64_t ld_q_h, int64_t ld_kv_h, int H,
                                         int N, int M, int d, float scale,
                                         const int32_t* route_ids, const int32_t* route_len,
                                         int L, int include_current, void* o, float* lse,
                                         void* stream) {
  // every check before the first HIP call: a rejected call touches no device
  velox_status_t st = check_attn(q, k, v, dt, ld_q_h, ld_kv_h, H, N, M, d, scale, o);
  if (st != VELOX_OK) return st;
  REQUIRE(route_ids && route_len, "route_ids and route_len must be non-NULL");
  REQUIRE(L >= 1, "L must be >= 1");
  REQUIRE(include_current == 0 || include_current == 1, "include_current must be 0 or 1");
  const size_t need = velox::attn_plan_bytes(H, N, 1);
  if (need > sizeof(scratch))
    return fail(VELOX_ERR_UNSUPPORTED,
                "H * ceil(N / 2) = %zu units exceed the %d of the no-allocation scratch (%zu bytes)",
                need / sizeof(int4), VELOX_NOALLOC_MAX_UNITS, sizeof(scratch));
  void* plan = nullptr;
  st = scratch_address(&plan);
  if (st != VELOX_OK) return st;
  return sparse_common(q, k, v, dt, ld_q_h, ld_kv_h, H, N, M, d, scale, route_ids, route_len, L,
                       include_current, o, lse, stream, false, "velox_sparse_attn_noalloc", 1,
                       nullptr, 0, plan);
}

velox_status_t velox_sparse_attn_shared(const void* q, const void* k, const void* v,
                                        velox_dtype_t dt, int64_t ld_q_h, int64_t ld_kv_h, int H,
                                        int N, int M, int d, float scale,
                                        const int32_t* route_ids, const int32_t* route_len, int L,
                                        int include_current, void* o, float* lse, void* stream) {
  return sparse_common(q, k, v, dt, ld_q_h, ld_kv_h, H, N, M, d, scale, route_ids, route_len, L,
                       include_current, o, lse, stream, true, "velox_sparse_attn_shared");
}

static velox_status_t dense_common(const void* q, const void* k, const void* v, velox_dtype_t dt,
                                   int64_t ld_q_h, int64_t ld_kv_h, int H, int N, int M, int d,
                                   float scale, void* o, float* lse, void* stream, const char* what,
                                   int n_split = 1, void* workspace = nullptr,
                                   size_t workspace_bytes = 0) {
  velox_status_t st = check_attn(q, k, v, dt, ld_q_h, ld_kv_h, H, N, M, d, scale, o);
  if (st != VELOX_OK) return st;
  velox::AttnConfig c{q, k, v, dt == VELOX_BF16, ld_q_h, ld_kv_h, H, N, M, d, scale,
                      nullptr, nullptr, 0, false, 1, o, lse};
  st = set_split(c, n_split, workspace, workspace_bytes);
  if (st != VELOX_OK) return st;
  return launched(velox::launch_attention(c, static_cast<hipStream_t>(stream)), what);
}

velox_status_t velox_dense_attn(const void* q, const void* k, const void* v, velox_dtype_t dt,
                                int64_t ld_q_h, int64_t ld_kv_h, int H, int N, int M, int d,
                                float scale, void* o, float* lse, void* stream) {
  return dense_common(q, k, v, dt, ld_q_h, ld_kv_h, H, N, M, d, scale, o, lse, stream,
                      "velox_dense_attn");
}

velox_status_t velox_sparse_attn_split(const void* q, const void* k, const void* v,
                                       velox_dtype_t dt, int64_t ld_q_h, int64_t ld_kv_h, int H,
                                       int N, int M, int d, float scale,
                                       const int32_t* route_ids, const int32_t* route_len, int L,
                                       int include_current, int n_split, void* workspace,
                                       size_t workspace_bytes, void* o, float* lse, void* stream) {
  return sparse_common(q, k, v, dt, ld_q_h, ld_kv_h, H, N, M, d, scale, route_ids, route_len, L,
                       include_current, o, lse, stream, false, "velox_sparse_attn_split", n_split,
                       workspace, workspace_bytes);
}

velox_status_t velox_dense_attn_split(const void* q, const void* k, const void* v,
                                      velox_dtype_t dt, int64_t ld_q_h, int64_t ld_kv_h, int H,
                                      int N, int M, int d, float scale, int n_split,
                                      void* workspace, size_t workspace_bytes, void* o,
                                      float* lse, void* stream) {
  return dense_common(q, k, v, dt, ld_q_h, ld_kv_h, H, N, M, d, scale, o, lse, stream,
                      "velox_dense_attn_split", n_split, workspace, workspace_bytes);
}

velox_status_t velox_slab_overlap(const float* q_obb, const float* h_obb, int N, int M,
                                  int lattice, float* g, void* stream) {
  velox_status_t st = check_geometry_sizes(N, M);
  if (st != VELOX_OK) return st;
  REQUIRE(lattice >= 1 && lattice <= VELOX_MAX_LATTICE, "lattice must be in [1, %d] (got %d)",
          VELOX_MAX_LATTICE, lattice);
  if (N == 0 || M == 0) return VELOX_OK;
  REQUIRE(q_obb && h_obb && g, "q_obb, h_obb and g must be non-NULL");
  return launched(velox::launch_slab_overlap(q_obb, h_obb, N, M, lattice, g,
                                             static_cast<hipStream_t>(stream)),
                  "velox_slab_overlap");
}

velox_status_t velox_slab_coverage(const float* q_pts, const float* h_obb, int N, int M,
                                   uint32_t* token_mask, float* rho, void* stream) {
  velox_status_t st = check_geometry_sizes(N, M);
  if (st != VELOX_OK) return st;
  if (N == 0) return VELOX_OK;
  REQUIRE(token_mask && rho, "token_mask and rho must be non-NULL");
  REQUIRE(M == 0 || (q_pts && h_obb), "q_pts and h_obb must be non-NULL when M > 0");
  return launched(velox::launch_slab_coverage(q_pts, h_obb, N, M, token_mask, rho,
                                              static_cast<hipStream_t>(stream)),
                  "velox_slab_coverage");
}

velox_status_t velox_gilbert_curve(int width, int height, int32_t* cells) {
  REQUIRE(width >= 1 && height >= 1, "width and height must be >= 1 (got %d x %d)", width, height);
  REQUIRE(static_cast<int64_t>(width) * height <= VELOX_MAX_GRID_CELLS, "grid of %d x %d is too large",
          width, height);
  REQUIRE(cells, "cells must be non-NULL");
  velox::gilbert_curve(width, height, cells);
  return VELOX_OK;
}

velox_status_t velox_kv_append(const void* k_new, const void* v_new, velox_dtype_t dt,
                               int64_t ld_new_h, int H, int T, int height, int width, int d,
                               int chunk_index, const int32_t* cells, void* k_cache,
                               void* v_cache, int64_t ld_kv_h, int64_t token_offset,
                               float* kbar, int64_t ld_kbar_h, void* stream) {
  REQUIRE(dtype_ok(dt), "dtype must be VELOX_F32 or VELOX_BF16");
  REQUIRE(dim_ok(d), "d must be 64 or 128 (got %d)", d);
  REQUIRE(H >= 1 && H <= 65535, "H must be in [1, 65535] (got %d)", H);
  REQUIRE(T >= 1 && height >= 1 && width >= 1, "T, height and width must be >= 1");
  REQUIRE(static_cast<int64_t>(height) * width <= VELOX_MAX_GRID_CELLS, "latent grid too large");
  REQUIRE(chunk_index >= 0, "chunk_index must be >= 0");
  const int64_t n_tok = static_cast<int64_t>(T) * height * width;
  if (n_tok % VELOX_BLOCK != 0 || n_tok > (int64_t{1} << 30))
    return fail(VELOX_ERR_UNSUPPORTED, "T*height*width=%lld is not a whole number of 128-token blocks",
                static_cast<long long>(n_tok));
  REQUIRE(token_offset >= 0 && token_offset % VELOX_BLOCK == 0, "token_offset must be a multiple of 128");
  REQUIRE(k_new && v_new && cells && k_cache && v_cache, "k_new, v_new, cells and the caches must be non-NULL");
  REQUIRE(ld_new_h >= n_tok * d, "ld_new_h too small");
  REQUIRE(ld_kv_h >= (token_offset + n_tok) * d, "ld_kv_h too small for token_offset + chunk");
  const int64_t nblk = n_tok / VELOX_BLOCK;
  if (kbar) REQUIRE(ld_kbar_h >= (token_offset / VELOX_BLOCK + nblk) * d, "ld_kbar_h too small");
  const int64_t eb = elem_bytes(dt);
  REQUIRE(reinterpret_cast<uintptr_t>(k_new) % 16 == 0 && reinterpret_cast<uintptr_t>(v_new) % 16 == 0 &&
              reinterpret_cast<uintptr_t>(k_cache) % 16 == 0 &&
              reinterpret_cast<uintptr_t>(v_cache) % 16 == 0 && (ld_new_h * eb) % 16 == 0 &&
              (ld_kv_h * eb) % 16 == 0,
          "tensors and head strides must be 16-byte aligned");
  return launched(velox::launch_kv_append(k_new, v_new, dt == VELOX_BF16, ld_new_h, H, T, height,
                                          width, d, chunk_index, cells, k_cache, v_cache, ld_kv_h,
                                          token_offset, kbar, ld_kbar_h,
                                          static_cast<hipStream_t>(stream)),
                  "velox_kv_append");
}

static velox_status_t check_pinhole(float f, float cx, float cy) {
  REQUIRE(std::isfinite(f) && f > 0.f && std::isfinite(cx) && std::isfinite(cy),
          "f must be finite and > 0, cx and cy finite");
  return VELOX_OK;
}

velox_status_t velox_slab_table(const int32_t* cells, const float* depth, const float* cams,
                                const int32_t* cam_of_block, int ncam, int nblk, float f,
                                float cx, float cy, int n_min, float* slabs, float* boxes,
                                void* stream) {
  REQUIRE(nblk >= 0 && nblk <= (1 << 24), "nblk must lie in [0, 2^24] (got %d)", nblk);
  if (nblk == 0) return VELOX_OK;
  REQUIRE(ncam >= 1, "ncam must be >= 1");
  REQUIRE(n_min >= 1 && n_min <= VELOX_BLOCK, "n_min must lie in [1, 128]");
  velox_status_t st = check_pinhole(f, cx, cy);
  if (st != VELOX_OK) return st;
  REQUIRE(cells && depth && cams && cam_of_block && slabs && boxes, "pointers must be non-NULL");
  return launched(velox::launch_slab_table(cells, depth, cams, cam_of_block, ncam, nblk, f, cx, cy, n_min,
                                           slabs, boxes, static_cast<hipStream_t>(stream)),
                  "velox_slab_table");
}

size_t velox_multiwarp_workspace_size(int K, int src_width, int src_height, int width, int height) {
  if (K < 0 || src_width < 1 || src_height < 1 || width < 1 || height < 1) return 0;
  return velox::multiwarp_workspace_bytes(K, src_width * src_height, width * height);
}

velox_status_t velox_multiwarp(const float* src_depth, const float* src_cams, int K, int src_width,
                               int src_height, float src_f, float src_cx, float src_cy,
                               const float* tgt_cam, float f, float cx, float cy, int width,
                               int height, int k_warp, float* zq, int32_t* chosen,
                               void* workspace, size_t workspace_bytes, void* stream) {
  REQUIRE(K >= 0 && K <= 4096, "K must lie in [0, 4096] (got %d)", K);
  REQUIRE(width >= 1 && height >= 1 && static_cast<int64_t>(width) * height <= (1 << 22),
          "target grid must be at least 1 x 1 and at most 2^22 cells");
  REQUIRE(src_width >= 1 && src_height >= 1 && static_cast<int64_t>(src_width) * src_height <= (1 << 24),
          "source frames must be at least 1 x 1 and at most 2^24 pixels");
  REQUIRE(static_cast<int64_t>(K) * src_width * src_height <= (int64_t{1} << 30), "K * pixels too large");
  REQUIRE(k_warp >= 1, "k_warp must be >= 1");
  velox_status_t st = check_pinhole(f, cx, cy);
  if (st != VELOX_OK) return st;
  st = check_pinhole(src_f, src_cx, src_cy);
  if (st != VELOX_OK) return st;
  REQUIRE(tgt_cam && zq && chosen && workspace, "tgt_cam, zq, chosen and workspace must be non-NULL");
  REQUIRE(K == 0 || (src_depth && src_cams), "src_depth and src_cams must be non-NULL when K > 0");
  REQUIRE(reinterpret_cast<uintptr_t>(workspace) % 4 == 0, "workspace must be 4-byte aligned");
  const size_t need = velox::multiwarp_workspace_bytes(K, src_width * src_height, width * height);
  REQUIRE(workspace_bytes >= need, "workspace of %zu bytes is smaller than the %zu needed", workspace_bytes,
          need);
  return launched(velox::launch_multiwarp(src_depth, src_cams, K, src_width, src_height, src_f, src_cx, src_cy,
                                          tgt_cam, f, cx, cy, width, height, k_warp, zq, chosen, workspace,
                                          static_cast<hipStream_t>(stream)),
                  "velox_multiwarp");
}

velox_status_t velox_token_points(const int32_t* cells, const float* zq, int width, int height,
                                  const float* cam, float f, float cx, float cy, int64_t n_tok,
                                  float* depth, float* pts, void* stream) {
  REQUIRE(n_tok >= 0 && n_tok <= (int64_t{1} << 30), "n_tok out of range");
  if (n_tok == 0) return VELOX_OK;
  REQUIRE(width >= 1 && height >= 1, "grid must be at least 1 x 1");
  velox_status_t st = check_pinhole(f, cx, cy);
  if (st != VELOX_OK) return st;
  REQUIRE(cells && zq && cam && depth && pts, "pointers must be non-NULL");
  return launched(velox::launch_token_points(cells, zq, width, height, cam, f, cx, cy, n_tok, depth, pts,
                                             static_cast<hipStream_t>(stream)),
                  "velox_token_points");
}

}  // extern "C"
