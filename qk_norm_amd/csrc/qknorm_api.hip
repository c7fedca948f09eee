// C-ABI front end: argument validation (host only, before any HIP call),
// device query, and dispatch to the kernel launchers.
#include <atomic>
#include <cmath>
#include <cstdint>

#include "../../include/qknorm.h"
#include "qknorm_launch.hpp"

namespace {

constexpr int64_t kMaxShards = 1024;
constexpr int64_t kMaxPitchBytes = INT64_C(1) << 26;
constexpr int64_t kMaxHeadIndex = INT64_C(1) << 31;   // T * heads must stay below this
constexpr int64_t kMaxRows = (INT64_C(1) << 31) - (INT64_C(1) << 20);

int esize_of(int32_t dtype) {
  return dtype == QKNORM_F32 ? 4 : (dtype == QKNORM_FP8_E4M3 ? 1 : 2);
}

bool known_dtype(int32_t dtype) {
  return dtype == QKNORM_F32 || dtype == QKNORM_BF16 || dtype == QKNORM_F16 ||
         dtype == QKNORM_FP8_E4M3;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

int check_common(int32_t dtype, float eps, int64_t T, int64_t ld) {
  if (!known_dtype(dtype)) return QKNORM_E_DTYPE;
  if (!std::isfinite(eps) || eps < 0.f) return QKNORM_E_EPS;
  if (T < 0 || ld < 0) return QKNORM_E_SHAPE;
  if (T > kMaxRows) return QKNORM_E_UNSUPPORTED;
  return QKNORM_OK;
}

// Q+K region and row pitch: ld >= wq + wk, pitch a multiple of 16 bytes,
// base 16-byte aligned when anything is touched.
// (ld >= 0 and T <= kMaxRows are checked before; every product below is
// formed only once its factors are bounded, so no input overflows int64.)
int check_region(const void* qkv, int64_t T, int64_t ld, int64_t wq, int64_t wk, int es) {
  if (wq < 0 || wk < 0) return QKNORM_E_SHAPE;
  if (wq > ld || wk > ld - wq) return QKNORM_E_SHAPE;       // ld < wq + wk
  const bool touched = T > 0 && wq + wk > 0;
  if (touched && qkv == nullptr) return QKNORM_E_NULLPTR;
  // rows are addressed with 32-bit buffer offsets: pitch at most 64 MiB
  if (ld > kMaxPitchBytes / es || T * (ld + 1) > (INT64_C(1) << 46)) return QKNORM_E_UNSUPPORTED;
  if (touched && (!aligned16(qkv) || (ld * es) % 16 != 0)) return QKNORM_E_ALIGN;
  if ((wq * es) % 16 != 0 || (wk * es) % 16 != 0) return QKNORM_E_ALIGN;
  return QKNORM_OK;
}

int check_gamma(const void* g, int64_t width, int64_t T) {
  if (width == 0 || T == 0) return QKNORM_OK;
  if (g == nullptr) return QKNORM_E_NULLPTR;
  if (!aligned16(g)) return QKNORM_E_ALIGN;
  return QKNORM_OK;
}

int check_shards(int64_t wq, int64_t wk, int32_t nshards, int es) {
  if (nshards <= 0) return QKNORM_E_SHAPE;
  if (nshards > kMaxShards) return QKNORM_E_UNSUPPORTED;
  if (wq % nshards != 0 || wk % nshards != 0) return QKNORM_E_SHAPE;
  if (((wq / nshards) * es) % 16 != 0 || ((wk / nshards) * es) % 16 != 0) return QKNORM_E_ALIGN;
  return QKNORM_OK;
}

// Compute units of the current device, cached per device.
std::atomic<int> g_cus[256];

int device_cus(int* cus) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return QKNORM_E_HIP;
  if (dev >= 0 && dev < 256) {
    int c = g_cus[dev].load(std::memory_order_relaxed);
    if (c > 0) { *cus = c; return QKNORM_OK; }
  }
  int c = 0;
  if (hipDeviceGetAttribute(&c, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || c <= 0)
    return QKNORM_E_HIP;
  if (dev >= 0 && dev < 256) g_cus[dev].store(c, std::memory_order_relaxed);
  *cus = c;
  return QKNORM_OK;
}

// Everything qknorm_qkv_proj_per_head and its workspace form check before
// any HIP call; on success *a holds the launch arguments and *n the output
// column count N.
int check_proj(const void* x, int64_t ldx, const void* w, int64_t ldw, void* qkv, int64_t ld,
               int64_t T, int64_t hidden, int32_t hq, int32_t hkv, int32_t head_dim,
               const void* gamma_q, const void* gamma_k, float eps, int32_t flags, int32_t dtype,
               qknorm::ProjArgs* a, int64_t* n) {
  int rc = check_common(dtype, eps, T, ld);
  if (rc) return rc;
  if (dtype != QKNORM_BF16 && dtype != QKNORM_F16) return QKNORM_E_UNSUPPORTED;
  if ((flags & ~QKNORM_PROJ_PLAIN) != 0) return QKNORM_E_UNSUPPORTED;
  if (hidden <= 0 || hq < 0 || hkv < 0 || head_dim <= 0 || ldx < hidden || ldw < hidden)
    return QKNORM_E_SHAPE;
  // N of any int32 head counts and head_dim fits 128 bits; N <= ld then fits int64
  const __int128 n_wide = ((__int128)hq + 2 * (__int128)hkv) * head_dim;
  if (n_wide > ld) return QKNORM_E_SHAPE;
  const int64_t N = (int64_t)n_wide;
  const bool norm = (flags & QKNORM_PROJ_PLAIN) == 0;
  const bool touched = T > 0 && N > 0;
  if (touched && (x == nullptr || w == nullptr || qkv == nullptr)) return QKNORM_E_NULLPTR;
  if (norm && (rc = check_gamma(gamma_q, hq, T))) return rc;
  if (norm && (rc = check_gamma(gamma_k, hkv, T))) return rc;
  if (touched && (!aligned16(x) || !aligned16(w) || !aligned16(qkv))) return QKNORM_E_ALIGN;
  // 16-byte row pitches: a multiple of 8 two-byte elements
  if (ldx % 8 != 0 || ldw % 8 != 0 || ld % 8 != 0) return QKNORM_E_ALIGN;
  // every pitch within 64 MiB before any product is formed from it (the
  // kernel's own limits, checked next, are tighter still)
  if (ld > kMaxPitchBytes / 2 || ldx > kMaxPitchBytes / 2 || ldw > kMaxPitchBytes / 2 ||
      T * (ld + 1) > (INT64_C(1) << 46) || N >= (INT64_C(1) << 24))
    return QKNORM_E_UNSUPPORTED;
  *a = qknorm::ProjArgs{x, ldx, w, ldw, qkv, ld, T, hidden, hq, hkv, head_dim, gamma_q, gamma_k,
                        eps, flags, dtype};
  if (!qknorm::proj_shape_ok(*a)) return QKNORM_E_UNSUPPORTED;
  *n = N;
  return QKNORM_OK;
}

int finish(hipError_t e) { return e == hipSuccess ? QKNORM_OK : QKNORM_E_HIP; }

}  // namespace

extern "C" {

int qknorm_abi_version(void) { return QKNORM_ABI_VERSION; }

const char* qknorm_strerror(int code) {
  switch (code) {
    case QKNORM_OK: return "success";
    case QKNORM_E_NULLPTR: return "a required pointer is NULL";
    case QKNORM_E_SHAPE: return "invalid shape (negative size, ld too small, or shards do not divide the width)";
    case QKNORM_E_ALIGN: return "misaligned: base, row pitch, head or shard is not a multiple of 16 bytes";
    case QKNORM_E_DTYPE: return "unknown dtype code";
    case QKNORM_E_UNSUPPORTED: return "unsupported request (head_dim, shard count or size)";
    case QKNORM_E_EPS: return "eps must be finite and non-negative";
    case QKNORM_E_HIP: return "HIP runtime error";
    default: return "unknown error code";
  }
}

int qknorm_per_head(void* qkv, int64_t T, int64_t ld, int32_t hq, int32_t hkv, int32_t head_dim,
                    const void* gamma_q, const void* gamma_k, float eps, int32_t dtype,
                    void* stream) {
  int rc = check_common(dtype, eps, T, ld);
  if (rc) return rc;
  if (hq < 0 || hkv < 0 || head_dim <= 0) return QKNORM_E_SHAPE;
  const int es = esize_of(dtype);
  const int64_t wq = (int64_t)hq * head_dim, wk = (int64_t)hkv * head_dim;
  if ((rc = check_region(qkv, T, ld, wq, wk, es))) return rc;
  if ((rc = check_gamma(gamma_q, wq, T))) return rc;
  if ((rc = check_gamma(gamma_k, wk, T))) return rc;
  // a head is 1..64 vectors of 16 bytes
  const int64_t head_bytes = (int64_t)head_dim * es;
  if (head_bytes % 16 != 0) return QKNORM_E_ALIGN;
  if (head_bytes > 1024) return QKNORM_E_UNSUPPORTED;
  if (T * ((int64_t)hq + hkv) >= kMaxHeadIndex) return QKNORM_E_UNSUPPORTED;
  qknorm::PerHeadArgs a{qkv, T, ld, hq, hkv, head_dim, gamma_q, gamma_k, eps, dtype};
  if (!qknorm::per_head_span_ok(a)) return QKNORM_E_UNSUPPORTED;
  if (T == 0 || hq + hkv == 0) return QKNORM_OK;
  int cus = 0;
  if ((rc = device_cus(&cus))) return rc;
  return finish(qknorm::launch_per_head(a, static_cast<hipStream_t>(stream), cus));
}

int qknorm_layerwise(void* qkv, int64_t T, int64_t ld, int64_t wq, int64_t wk,
                     const void* gamma_q, const void* gamma_k, float eps, int32_t nshards,
                     int32_t dtype, void* stream) {
  int rc = check_common(dtype, eps, T, ld);
  if (rc) return rc;
  const int es = esize_of(dtype);
  if ((rc = check_region(qkv, T, ld, wq, wk, es))) return rc;
  if ((rc = check_shards(wq, wk, nshards, es))) return rc;
  if ((rc = check_gamma(gamma_q, wq, T))) return rc;
  if ((rc = check_gamma(gamma_k, wk, T))) return rc;
  if (T == 0 || wq + wk == 0) return QKNORM_OK;
  int cus = 0;
  if ((rc = device_cus(&cus))) return rc;
  qknorm::LayerwiseArgs a{qkv, T, ld, wq, wk, gamma_q, gamma_k, eps, nshards, dtype};
  return finish(qknorm::launch_layerwise(a, static_cast<hipStream_t>(stream), cus));
}

int qknorm_partial_sumsq(const void* qkv, int64_t T, int64_t ld, int64_t wq, int64_t wk,
                         int32_t nshards, float* part_q, float* part_k, int32_t dtype,
                         void* stream) {
  int rc = check_common(dtype, 0.f, T, ld);
  if (rc) return rc;
  const int es = esize_of(dtype);
  if ((rc = check_region(qkv, T, ld, wq, wk, es))) return rc;
  if ((rc = check_shards(wq, wk, nshards, es))) return rc;
  if (T > 0 && wq > 0 && part_q == nullptr) return QKNORM_E_NULLPTR;
  if (T > 0 && wk > 0 && part_k == nullptr) return QKNORM_E_NULLPTR;
  if ((reinterpret_cast<uintptr_t>(part_q) & 3u) || (reinterpret_cast<uintptr_t>(part_k) & 3u))
    return QKNORM_E_ALIGN;
  if (T == 0 || wq + wk == 0) return QKNORM_OK;
  int cus = 0;
  if ((rc = device_cus(&cus))) return rc;
  qknorm::PartialArgs a{qkv, T, ld, wq, wk, nshards, part_q, part_k, dtype};
  return finish(qknorm::launch_partial_sumsq(a, static_cast<hipStream_t>(stream), cus));
}

int qknorm_apply_scalar(void* qkv, int64_t T, int64_t ld, int64_t wq, int64_t wk,
                        const float* part_q, const float* part_k, int32_t nparts,
                        int64_t norm_wq, int64_t norm_wk, const void* gamma_q,
                        const void* gamma_k, float eps, int32_t dtype, void* stream) {
  int rc = check_common(dtype, eps, T, ld);
  if (rc) return rc;
  const int es = esize_of(dtype);
  if ((rc = check_region(qkv, T, ld, wq, wk, es))) return rc;
  if (nparts <= 0) return QKNORM_E_SHAPE;
  if (nparts > kMaxShards) return QKNORM_E_UNSUPPORTED;
  if (wq > 0 && norm_wq < wq) return QKNORM_E_SHAPE;
  if (wk > 0 && norm_wk < wk) return QKNORM_E_SHAPE;
  if (T > 0 && wq > 0 && part_q == nullptr) return QKNORM_E_NULLPTR;
  if (T > 0 && wk > 0 && part_k == nullptr) return QKNORM_E_NULLPTR;
  if ((reinterpret_cast<uintptr_t>(part_q) & 3u) || (reinterpret_cast<uintptr_t>(part_k) & 3u))
    return QKNORM_E_ALIGN;
  if ((rc = check_gamma(gamma_q, wq, T))) return rc;
  if ((rc = check_gamma(gamma_k, wk, T))) return rc;
  if (T == 0 || wq + wk == 0) return QKNORM_OK;
  int cus = 0;
  if ((rc = device_cus(&cus))) return rc;
  qknorm::ApplyArgs a{qkv, T, ld, wq, wk, part_q, part_k, nparts, norm_wq, norm_wk,
                      gamma_q, gamma_k, eps, dtype};
  return finish(qknorm::launch_apply_scalar(a, static_cast<hipStream_t>(stream), cus));
}

int qknorm_qkv_proj_per_head(const void* x, int64_t ldx, const void* w, int64_t ldw, void* qkv,
                             int64_t ld, int64_t T, int64_t hidden, int32_t hq, int32_t hkv,
                             int32_t head_dim, const void* gamma_q, const void* gamma_k, float eps,
                             int32_t flags, int32_t dtype, void* stream) {
  qknorm::ProjArgs a;
  int64_t N = 0;
  int rc = check_proj(x, ldx, w, ldw, qkv, ld, T, hidden, hq, hkv, head_dim, gamma_q, gamma_k, eps,
                      flags, dtype, &a, &N);
  if (rc) return rc;
  if (T == 0 || N == 0) return QKNORM_OK;
  int cus = 0;
  if ((rc = device_cus(&cus))) return rc;
  return finish(qknorm::launch_qkv_proj(a, static_cast<hipStream_t>(stream), cus));
}

int64_t qknorm_qkv_proj_workspace_bytes(int64_t T, int32_t hq, int32_t hkv, int32_t head_dim) {
  if (T < 0 || hq < 0 || hkv < 0 || head_dim <= 0) return QKNORM_E_SHAPE;
  if (T > kMaxRows) return QKNORM_E_UNSUPPORTED;
  const __int128 n_wide = ((__int128)hq + 2 * (__int128)hkv) * head_dim;
  if (n_wide >= (INT64_C(1) << 24)) return QKNORM_E_UNSUPPORTED;
  return qknorm::proj_workspace_bytes(T, (int64_t)n_wide);
}

int qknorm_qkv_proj_per_head_ws(const void* x, int64_t ldx, const void* w, int64_t ldw, void* qkv,
                                int64_t ld, int64_t T, int64_t hidden, int32_t hq, int32_t hkv,
                                int32_t head_dim, const void* gamma_q, const void* gamma_k,
                                float eps, int32_t flags, int32_t dtype, void* workspace,
                                int64_t workspace_bytes, void* stream) {
  qknorm::ProjArgs a;
  int64_t N = 0;
  int rc = check_proj(x, ldx, w, ldw, qkv, ld, T, hidden, hq, hkv, head_dim, gamma_q, gamma_k, eps,
                      flags, dtype, &a, &N);
  if (rc) return rc;
  if (workspace_bytes < 0) return QKNORM_E_SHAPE;
  const int64_t need = qknorm::proj_workspace_bytes(T, N);
  if (need > 0) {
    if (workspace == nullptr) return QKNORM_E_NULLPTR;
    if (!aligned16(workspace)) return QKNORM_E_ALIGN;
    if (workspace_bytes < need) return QKNORM_E_SHAPE;
  }
  if (T == 0 || N == 0) return QKNORM_OK;
  if (need > 0) return finish(qknorm::launch_qkv_proj_split(a, workspace, static_cast<hipStream_t>(stream)));
  int cus = 0;
  if ((rc = device_cus(&cus))) return rc;
  return finish(qknorm::launch_qkv_proj(a, static_cast<hipStream_t>(stream), cus));
}

int qknorm_qkv_proj_per_head_noalloc(const void* x, int64_t ldx, const void* w, int64_t ldw,
                                     void* qkv, int64_t ld, int64_t T, int64_t hidden, int32_t hq,
                                     int32_t hkv, int32_t head_dim, const void* gamma_q,
                                     const void* gamma_k, float eps, int32_t flags, int32_t dtype,
                                     void* stream) {
  qknorm::ProjArgs a;
  int64_t N = 0;
  int rc = check_proj(x, ldx, w, ldw, qkv, ld, T, hidden, hq, hkv, head_dim, gamma_q, gamma_k, eps,
                      flags, dtype, &a, &N);
  if (rc) return rc;
  const int64_t need = qknorm::proj_workspace_bytes(T, N);
  if (need > qknorm::kProjScratchBytes) return QKNORM_E_UNSUPPORTED;
  if (T == 0 || N == 0) return QKNORM_OK;
  if (need > 0) {
    void* scratch = nullptr;
    if (qknorm::proj_scratch(&scratch) != hipSuccess) return QKNORM_E_HIP;
    return finish(qknorm::launch_qkv_proj_split(a, scratch, static_cast<hipStream_t>(stream)));
  }
  int cus = 0;
  if ((rc = device_cus(&cus))) return rc;
  return finish(qknorm::launch_qkv_proj(a, static_cast<hipStream_t>(stream), cus));
}

}  // extern "C"
