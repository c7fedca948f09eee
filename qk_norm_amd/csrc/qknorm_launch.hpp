// Internal interface between the C-ABI front end and the kernel launchers.
// Arguments reaching these functions have already been validated on the host.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace qknorm {

struct PerHeadArgs {
  void* qkv;
  int64_t T, ld;
  int32_t hq, hkv, head_dim;
  const void* gamma_q;
  const void* gamma_k;
  float eps;
  int32_t dtype;
};

struct LayerwiseArgs {
  void* qkv;
  int64_t T, ld, wq, wk;
  const void* gamma_q;
  const void* gamma_k;
  float eps;
  int32_t nshards, dtype;
};

struct PartialArgs {
  const void* qkv;
  int64_t T, ld, wq, wk;
  int32_t nshards;
  float* part_q;
  float* part_k;
  int32_t dtype;
};

struct ApplyArgs {
  void* qkv;
  int64_t T, ld, wq, wk;
  const float* part_q;
  const float* part_k;
  int32_t nparts;
  int64_t norm_wq, norm_wk;
  const void* gamma_q;
  const void* gamma_k;
  float eps;
  int32_t dtype;
};

struct ProjArgs {
  const void* x;
  int64_t ldx;
  const void* w;
  int64_t ldw;
  void* qkv;
  int64_t ld, T, hidden;
  int32_t hq, hkv, head_dim;
  const void* gamma_q;
  const void* gamma_k;
  float eps;
  int32_t flags;
  int32_t dtype;       // kBF16 or kF16: x, w, gamma and qkv share it
};

// Whether every per-head trip's buffer span stays below 2^31 bytes.
bool per_head_span_ok(const PerHeadArgs& a);
// Whether the projection kernel takes this shape (tile offsets, K step, head_dim).
bool proj_shape_ok(const ProjArgs& a);

// `cus` is the compute-unit count of the current device (grid sizing).
hipError_t launch_per_head(const PerHeadArgs& a, hipStream_t s, int cus);
hipError_t launch_layerwise(const LayerwiseArgs& a, hipStream_t s, int cus);
hipError_t launch_partial_sumsq(const PartialArgs& a, hipStream_t s, int cus);
hipError_t launch_apply_scalar(const ApplyArgs& a, hipStream_t s, int cus);
hipError_t launch_qkv_proj(const ProjArgs& a, hipStream_t s, int cus);

// Token counts up to this take the split projection when the caller gives a
// workspace (or the library's own scratch); larger ones take the tiles.
constexpr int64_t kProjSplitMaxT = 64;
// Bytes of fp32 partials the split projection needs for T tokens and N
// output columns (0 where T is outside 1..kProjSplitMaxT).
int64_t proj_workspace_bytes(int64_t T, int64_t N);
// The split projection: partial sums into `workspace`, then one block per
// head adds them and normalises (two launches on `s`).
hipError_t launch_qkv_proj_split(const ProjArgs& a, void* workspace, hipStream_t s);

// The library's own scratch for the split projection (one array per GPU):
// its size, and its device address on the current device (looked up once per
// device).  Devices numbered kMaxScratchDevices or higher are not served.
constexpr int64_t kProjScratchBytes = INT64_C(8) << 20;
constexpr int kMaxScratchDevices = 64;
hipError_t proj_scratch(void** ptr);

}  // namespace qknorm
