// gfx950 kernels for QK-Norm on fused QKV rows, and their launchers.
//
// All kernels are HBM-bound streams: every Q/K element is read once with a
// 16-byte vector load, reduced in fp32 registers, scaled and written back in
// place with a 16-byte store.  V columns are never addressed.
#include "qknorm_device.hpp"
#include "qknorm_launch.hpp"

#ifndef QKNORM_NT
#define QKNORM_NT 1            // non-temporal loads/stores for the streamed rows
#endif
#ifndef QKNORM_PH_UNROLL
#define QKNORM_PH_UNROLL 4     // heads per 16-lane group per loop trip
#endif
#ifndef QKNORM_PH_BLOCKS_PER_CU
#define QKNORM_PH_BLOCKS_PER_CU 8
#endif
#ifndef QKNORM_LW_WAVES_PER_CU
#define QKNORM_LW_WAVES_PER_CU 32   // grid cap for the row kernels, in waves per CU
#endif

namespace qknorm {

static constexpr bool kNT = QKNORM_NT != 0;

// =================================================================== per head
//
// A head of D values is LPH lanes x 16 bytes (bf16 D=128: 16 lanes, one DPP
// row).  A wave covers 64/LPH consecutive heads per step and U steps per loop
// trip, so each trip streams U contiguous 1 KiB runs (for bf16 D=128) and has
// U independent 16-byte loads in flight per lane.  Heads are numbered
// g = t*H + h over the Q and K heads of every row (H = hq + hkv); head h < hq
// is a Q head with gamma_q, otherwise a K head with gamma_k.  (t, h) are kept
// incrementally so the loop has no integer division.

template <int DT, int LPH, int U>
__global__ __launch_bounds__(256) void per_head_kernel(
    uint8_t* __restrict__ qkv, int64_t ld_bytes, uint32_t T, uint32_t H, uint32_t hq,
    const uint8_t* __restrict__ gamma_q, const uint8_t* __restrict__ gamma_k, float eps,
    float head_dim, uint32_t stride_rows, uint32_t stride_heads) {
  using IO = IoTraits<DT>;
  constexpr int E = IO::kElems;
  constexpr int HPW = 64 / LPH;              // heads per wave step
  constexpr uint32_t CH = HPW * U;           // heads per wave per trip
  const uint32_t lane = threadIdx.x & 63;
  const uint32_t sub = lane % LPH;           // 16-byte slot inside the head
  const uint32_t grp = lane / LPH;           // head slot inside the wave step
  const int64_t head_bytes = (int64_t)LPH * 16;

  // gamma of this lane's columns, kept in registers for the whole kernel
  // (a NULL gamma belongs to a region with no heads and is never applied)
  float gq[E], gk[E];
  unpack<DT>(gamma_q ? load16<false>(gamma_q + sub * 16) : u32x4{0, 0, 0, 0}, gq);
  unpack<DT>(gamma_k ? load16<false>(gamma_k + sub * 16) : u32x4{0, 0, 0, 0}, gk);

  const uint32_t wave = (blockIdx.x * blockDim.x + threadIdx.x) >> 6;
  // first head of this lane: wave*CH + grp
  uint64_t g0 = (uint64_t)wave * CH + grp;
  uint32_t t = (uint32_t)(g0 / H);
  uint32_t h = (uint32_t)(g0 - (uint64_t)t * H);

  while (t < T) {
    u32x4 v[U];
    uint8_t* p[U];
    bool ok[U], isq[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      uint32_t hu = h + u * HPW, tu = t;
      while (hu >= H) { hu -= H; ++tu; }
      ok[u] = tu < T;
      isq[u] = hu < hq;
      p[u] = qkv + (int64_t)tu * ld_bytes + (int64_t)hu * head_bytes + sub * 16;
      if (ok[u]) v[u] = load16<kNT>(p[u]);
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      float x[E];
      unpack<DT>(ok[u] ? v[u] : u32x4{0, 0, 0, 0}, x);
      float s = group_sum<LPH>(vec_sumsq<DT>(x, 0.f));
      float r = rms_scale(s, head_dim, eps);
      float y[E];
#pragma unroll
      for (int e = 0; e < E; ++e) y[e] = (x[e] * (isq[u] ? gq[e] : gk[e])) * r;
      if (ok[u]) store16<kNT>(p[u], pack<DT>(y));
    }
    // advance by the whole grid: stride_rows rows and stride_heads heads
    h += stride_heads;
    t += stride_rows;
    if (h >= H) { h -= H; ++t; }
  }
}

// ================================================================= layerwise
//
// One block of NW waves normalises one row per loop trip (grid-stride over
// rows).  Shard r of Q (and of K) belongs to wave r % NW; inside a shard of
// svecs 16-byte vectors, lane l takes vectors l, l+64, l+128, ... (trips =
// ceil(svecs/64) of them, a zero vector past the end).  The shard partial is
// the lane's fp32 fused-multiply-add chain over those vectors in that order,
// then the 64-lane group_sum.  Every layerwise kernel uses exactly this
// order, so the fused kernel and partial_sumsq + apply_scalar give the same
// bits.  The partials are combined in shard order: ((p0 + p1) + p2) + ...

struct RowGeom {
  int64_t ld_bytes;
  uint32_t T;
  uint32_t q_vecs, k_vecs;      // 16-byte vectors of Q and of K per row
  uint32_t nshards;
  uint32_t q_svecs, k_svecs;    // vectors per shard
  float wq, wk;                 // divisors (full widths)
};

__device__ __forceinline__ float combine(const float* __restrict__ p, uint32_t n, int64_t stride) {
  float s = 0.f;
  for (uint32_t r = 0; r < n; ++r) s += p[(int64_t)r * stride];
  return s;
}

// --- register-resident slots (fused kernel, MODE 0) -------------------------
//
// Slot j of a lane is shard wave + (j / trips)*nw, vector lane + (j % trips)*64.
// The slot loops are fully unrolled so the kept vectors stay in VGPRs.

template <int VPL>
struct Slots {
  u32x4 x[VPL];
  u32x4 g[VPL];
};

template <int DT, int VPL>
__device__ __forceinline__ void slots_load_gamma(const uint8_t* __restrict__ gamma, uint32_t svecs,
                                                 uint32_t R, uint32_t wave, uint32_t nw,
                                                 uint32_t lane, Slots<VPL>& S) {
  const uint32_t trips = (svecs + 63) / 64;
  uint32_t i = 0, k = 0;
#pragma unroll
  for (int j = 0; j < VPL; ++j) {
    const uint32_t r = wave + i * nw, v = lane + k * 64;
    S.g[j] = (r < R && v < svecs) ? load16<false>(gamma + ((int64_t)r * svecs + v) * 16)
                                  : u32x4{0, 0, 0, 0};
    if (++k == trips) { k = 0; ++i; }
  }
}

template <int DT, int VPL>
__device__ __forceinline__ void slots_load(const uint8_t* __restrict__ reg, uint32_t svecs,
                                           uint32_t R, uint32_t wave, uint32_t nw, uint32_t lane,
                                           Slots<VPL>& S) {
  const uint32_t trips = (svecs + 63) / 64;
  uint32_t i = 0, k = 0;
#pragma unroll
  for (int j = 0; j < VPL; ++j) {
    const uint32_t r = wave + i * nw, v = lane + k * 64;
    S.x[j] = (r < R && v < svecs) ? load16<kNT>(reg + ((int64_t)r * svecs + v) * 16)
                                  : u32x4{0, 0, 0, 0};
    if (++k == trips) { k = 0; ++i; }
  }
}

template <int DT, int VPL>
__device__ __forceinline__ void slots_partials(uint32_t svecs, uint32_t R, uint32_t wave,
                                               uint32_t nw, uint32_t lane, const Slots<VPL>& S,
                                               float* __restrict__ part) {
  using IO = IoTraits<DT>;
  const uint32_t trips = (svecs + 63) / 64;
  uint32_t i = 0, k = 0;
  float acc = 0.f;
#pragma unroll
  for (int j = 0; j < VPL; ++j) {
    const uint32_t r = wave + i * nw;
    if (r < R) {
      float x[IO::kElems];
      unpack<DT>(S.x[j], x);
      acc = vec_sumsq<DT>(x, acc);
      if (k + 1 == trips) {
        const float s = group_sum<64>(acc);
        if (lane == 0) part[r] = s;
        acc = 0.f;
      }
    }
    if (++k == trips) { k = 0; ++i; }
  }
}

template <int DT, int VPL>
__device__ __forceinline__ void slots_apply(uint8_t* __restrict__ reg, uint32_t svecs, uint32_t R,
                                            uint32_t wave, uint32_t nw, uint32_t lane,
                                            const Slots<VPL>& S, float scale) {
  using IO = IoTraits<DT>;
  const uint32_t trips = (svecs + 63) / 64;
  uint32_t i = 0, k = 0;
#pragma unroll
  for (int j = 0; j < VPL; ++j) {
    const uint32_t r = wave + i * nw, v = lane + k * 64;
    if (r < R && v < svecs) {
      float x[IO::kElems], g[IO::kElems], y[IO::kElems];
      unpack<DT>(S.x[j], x);
      unpack<DT>(S.g[j], g);
#pragma unroll
      for (int e = 0; e < IO::kElems; ++e) y[e] = (x[e] * g[e]) * scale;
      store16<kNT>(reg + ((int64_t)r * svecs + v) * 16, pack<DT>(y));
    }
    if (++k == trips) { k = 0; ++i; }
  }
}

// --- streamed shards (MODE 1 and 2): same order, dynamic loops ---------------

template <int DT>
__device__ __forceinline__ float shard_sumsq_stream(const uint8_t* __restrict__ sp,
                                                    uint32_t svecs, uint32_t lane) {
  using IO = IoTraits<DT>;
  const uint32_t trips = (svecs + 63) / 64;
  float acc = 0.f;
  for (uint32_t k = 0; k < trips; ++k) {
    const uint32_t v = lane + k * 64;
    float x[IO::kElems];
    unpack<DT>(v < svecs ? load16<kNT>(sp + (int64_t)v * 16) : u32x4{0, 0, 0, 0}, x);
    acc = vec_sumsq<DT>(x, acc);
  }
  return group_sum<64>(acc);
}

template <int DT>
__device__ __forceinline__ void apply_stream(uint8_t* __restrict__ reg,
                                             const uint8_t* __restrict__ gamma, uint32_t nvecs,
                                             uint32_t tid, uint32_t nthreads, float scale) {
  using IO = IoTraits<DT>;
  for (uint32_t v = tid; v < nvecs; v += nthreads) {
    float x[IO::kElems], g[IO::kElems], y[IO::kElems];
    unpack<DT>(load16<kNT>(reg + (int64_t)v * 16), x);
    unpack<DT>(load16<false>(gamma + (int64_t)v * 16), g);
#pragma unroll
    for (int e = 0; e < IO::kElems; ++e) y[e] = (x[e] * g[e]) * scale;
    store16<kNT>(reg + (int64_t)v * 16, pack<DT>(y));
  }
}

// Fused layerwise, row kept in registers (VPL slots per region per lane).
template <int DT, int VPL>
__global__ __launch_bounds__(512) void layerwise_regs_kernel(
    uint8_t* __restrict__ qkv, RowGeom G, const uint8_t* __restrict__ gamma_q,
    const uint8_t* __restrict__ gamma_k, float eps) {
  extern __shared__ float lds[];               // [2 buffers][Q, K][nshards]
  const uint32_t lane = threadIdx.x & 63;
  const uint32_t wave = threadIdx.x >> 6;
  const uint32_t nw = blockDim.x >> 6;
  const uint32_t R = G.nshards;
  const uint32_t Rq = G.q_vecs ? R : 0, Rk = G.k_vecs ? R : 0;
  Slots<VPL> sq, sk;
  slots_load_gamma<DT, VPL>(gamma_q, G.q_svecs, Rq, wave, nw, lane, sq);
  slots_load_gamma<DT, VPL>(gamma_k, G.k_svecs, Rk, wave, nw, lane, sk);
  uint32_t parity = 0;
  for (uint32_t t = blockIdx.x; t < G.T; t += gridDim.x, parity ^= 1) {
    uint8_t* qreg = qkv + (int64_t)t * G.ld_bytes;
    uint8_t* kreg = qreg + (int64_t)G.q_vecs * 16;
    float* pq = lds + parity * 2 * R;
    float* pk = pq + R;
    slots_load<DT, VPL>(qreg, G.q_svecs, Rq, wave, nw, lane, sq);
    slots_load<DT, VPL>(kreg, G.k_svecs, Rk, wave, nw, lane, sk);
    slots_partials<DT, VPL>(G.q_svecs, Rq, wave, nw, lane, sq, pq);
    slots_partials<DT, VPL>(G.k_svecs, Rk, wave, nw, lane, sk, pk);
    __syncthreads();
    // Double-buffered partials: this buffer is next written two trips later,
    // after every thread has passed the next trip's barrier.
    if (Rq) slots_apply<DT, VPL>(qreg, G.q_svecs, Rq, wave, nw, lane, sq,
                                 rms_scale(combine(pq, R, 1), G.wq, eps));
    if (Rk) slots_apply<DT, VPL>(kreg, G.k_svecs, Rk, wave, nw, lane, sk,
                                 rms_scale(combine(pk, R, 1), G.wk, eps));
  }
}

// Fused layerwise for rows too wide for the register slots: partials from a
// first streamed pass, then a second pass re-reads (mostly from L2) and applies.
template <int DT>
__global__ __launch_bounds__(512) void layerwise_stream_kernel(
    uint8_t* __restrict__ qkv, RowGeom G, const uint8_t* __restrict__ gamma_q,
    const uint8_t* __restrict__ gamma_k, float eps) {
  extern __shared__ float lds[];
  const uint32_t lane = threadIdx.x & 63;
  const uint32_t wave = threadIdx.x >> 6;
  const uint32_t nw = blockDim.x >> 6;
  const uint32_t R = G.nshards;
  uint32_t parity = 0;
  for (uint32_t t = blockIdx.x; t < G.T; t += gridDim.x, parity ^= 1) {
    uint8_t* qreg = qkv + (int64_t)t * G.ld_bytes;
    uint8_t* kreg = qreg + (int64_t)G.q_vecs * 16;
    float* pq = lds + parity * 2 * R;
    float* pk = pq + R;
    for (uint32_t r = wave; r < R; r += nw) {
      if (G.q_vecs) {
        const float s = shard_sumsq_stream<DT>(qreg + (int64_t)r * G.q_svecs * 16, G.q_svecs, lane);
        if (lane == 0) pq[r] = s;
      }
      if (G.k_vecs) {
        const float s = shard_sumsq_stream<DT>(kreg + (int64_t)r * G.k_svecs * 16, G.k_svecs, lane);
        if (lane == 0) pk[r] = s;
      }
    }
    __syncthreads();
    if (G.q_vecs)
      apply_stream<DT>(qreg, gamma_q, G.q_vecs, threadIdx.x, blockDim.x,
                       rms_scale(combine(pq, R, 1), G.wq, eps));
    if (G.k_vecs)
      apply_stream<DT>(kreg, gamma_k, G.k_vecs, threadIdx.x, blockDim.x,
                       rms_scale(combine(pk, R, 1), G.wk, eps));
  }
}

// Phase A: one wave per (row, shard) of Q and of K; lane 0 stores the partial
// at part[r*T + t].  Work item i < T*R is Q (row i / R, shard i % R), the
// next T*R items are K.
template <int DT>
__global__ __launch_bounds__(256) void partial_sumsq_kernel(const uint8_t* __restrict__ qkv,
                                                            RowGeom G, float* __restrict__ part_q,
                                                            float* __restrict__ part_k) {
  const uint32_t lane = threadIdx.x & 63;
  const uint64_t nq = G.q_vecs ? (uint64_t)G.T * G.nshards : 0;
  const uint64_t nk = G.k_vecs ? (uint64_t)G.T * G.nshards : 0;
  const uint64_t total = nq + nk;
  const uint64_t nwaves = ((uint64_t)gridDim.x * blockDim.x) >> 6;
  for (uint64_t i = ((uint64_t)blockIdx.x * blockDim.x + threadIdx.x) >> 6; i < total;
       i += nwaves) {
    const bool isk = i >= nq;
    const uint64_t w = isk ? i - nq : i;
    const uint32_t t = (uint32_t)(w / G.nshards), r = (uint32_t)(w % G.nshards);
    const uint32_t svecs = isk ? G.k_svecs : G.q_svecs;
    const uint8_t* sp = qkv + (int64_t)t * G.ld_bytes +
                        (int64_t)((isk ? G.q_vecs : 0) + r * svecs) * 16;
    const float s = shard_sumsq_stream<DT>(sp, svecs, lane);
    if (lane == 0) (isk ? part_k : part_q)[(int64_t)r * G.T + t] = s;
  }
}

// Phase C: one block per row (grid-stride), flat 16-byte vectors over Q then
// K.  scale = rsq((sum over r < nparts of part[r*T + t]) / norm_w + eps).
template <int DT>
__global__ __launch_bounds__(256) void apply_scalar_kernel(
    uint8_t* __restrict__ qkv, int64_t ld_bytes, uint32_t T, uint32_t q_vecs, uint32_t k_vecs,
    const float* __restrict__ part_q, const float* __restrict__ part_k, uint32_t nparts,
    float norm_wq, float norm_wk, const uint8_t* __restrict__ gamma_q,
    const uint8_t* __restrict__ gamma_k, float eps) {
  for (uint32_t t = blockIdx.x; t < T; t += gridDim.x) {
    uint8_t* row = qkv + (int64_t)t * ld_bytes;
    if (q_vecs)
      apply_stream<DT>(row, gamma_q, q_vecs, threadIdx.x, blockDim.x,
                       rms_scale(combine(part_q + t, nparts, T), norm_wq, eps));
    if (k_vecs)
      apply_stream<DT>(row + (int64_t)q_vecs * 16, gamma_k, k_vecs, threadIdx.x, blockDim.x,
                       rms_scale(combine(part_k + t, nparts, T), norm_wk, eps));
  }
}

// ================================================================ launchers

template <int DT, int LPH>
static hipError_t launch_per_head_t(const PerHeadArgs& a, hipStream_t s, int cus) {
  constexpr int U = QKNORM_PH_UNROLL;
  constexpr uint64_t CH = (64 / LPH) * U;
  constexpr int kBlock = 256;
  constexpr uint64_t heads_per_block = CH * (kBlock / 64);
  const uint64_t H = (uint64_t)a.hq + a.hkv;
  const uint64_t total = (uint64_t)a.T * H;
  uint64_t blocks = (total + heads_per_block - 1) / heads_per_block;
  const uint64_t cap = (uint64_t)cus * QKNORM_PH_BLOCKS_PER_CU;
  if (blocks > cap) blocks = cap;
  if (blocks < 1) blocks = 1;
  const uint64_t stride = blocks * heads_per_block;   // heads advanced per trip
  hipLaunchKernelGGL((per_head_kernel<DT, LPH, U>), dim3((uint32_t)blocks), dim3(kBlock), 0, s,
                     (uint8_t*)a.qkv, a.ld * (int64_t)IoTraits<DT>::kBytes, (uint32_t)a.T,
                     (uint32_t)H, (uint32_t)a.hq, (const uint8_t*)a.gamma_q,
                     (const uint8_t*)a.gamma_k, a.eps, (float)a.head_dim,
                     (uint32_t)(stride / H), (uint32_t)(stride % H));
  return hipGetLastError();
}

template <int DT>
static hipError_t launch_per_head_dt(const PerHeadArgs& a, hipStream_t s, int cus) {
  const int lph = a.head_dim * IoTraits<DT>::kBytes / 16;
  switch (lph) {
    case 8: return launch_per_head_t<DT, 8>(a, s, cus);
    case 16: return launch_per_head_t<DT, 16>(a, s, cus);
    case 32: return launch_per_head_t<DT, 32>(a, s, cus);
    case 64: return launch_per_head_t<DT, 64>(a, s, cus);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_per_head(const PerHeadArgs& a, hipStream_t s, int cus) {
  return a.dtype == kBF16 ? launch_per_head_dt<kBF16>(a, s, cus)
                          : launch_per_head_dt<kF32>(a, s, cus);
}

static RowGeom make_geom(int64_t T, int64_t ld, int64_t wq, int64_t wk, int32_t nshards,
                         int esize) {
  RowGeom G;
  G.ld_bytes = ld * esize;
  G.T = (uint32_t)T;
  G.q_vecs = (uint32_t)(wq * esize / 16);
  G.k_vecs = (uint32_t)(wk * esize / 16);
  G.nshards = (uint32_t)nshards;
  G.q_svecs = G.q_vecs / G.nshards;
  G.k_svecs = G.k_vecs / G.nshards;
  G.wq = (float)wq;
  G.wk = (float)wk;
  return G;
}

// Waves per block and register slots per lane for a layerwise geometry.
static void layerwise_shape(const RowGeom& G, uint32_t* nw, uint32_t* vpl) {
  const uint32_t w = G.nshards < 8 ? G.nshards : 8;
  const uint32_t per_wave = (G.nshards + w - 1) / w;
  const uint32_t q = G.q_vecs ? per_wave * ((G.q_svecs + 63) / 64) : 0;
  const uint32_t k = G.k_vecs ? per_wave * ((G.k_svecs + 63) / 64) : 0;
  *nw = w;
  *vpl = q > k ? q : k;
}

static uint32_t row_blocks(uint32_t T, uint32_t nw, int cus) {
  uint64_t cap = (uint64_t)cus * (QKNORM_LW_WAVES_PER_CU / nw);
  if (cap < (uint64_t)cus) cap = cus;
  uint64_t b = T < cap ? T : cap;
  return (uint32_t)(b < 1 ? 1 : b);
}

template <int DT, int VPL>
static hipError_t launch_lw_regs(const RowGeom& G, uint32_t nw, const LayerwiseArgs& a,
                                 hipStream_t s, int cus) {
  hipLaunchKernelGGL((layerwise_regs_kernel<DT, VPL>), dim3(row_blocks(G.T, nw, cus)),
                     dim3(nw * 64), (size_t)4 * G.nshards * sizeof(float), s, (uint8_t*)a.qkv, G,
                     (const uint8_t*)a.gamma_q, (const uint8_t*)a.gamma_k, a.eps);
  return hipGetLastError();
}

template <int DT>
static hipError_t launch_layerwise_dt(const LayerwiseArgs& a, hipStream_t s, int cus) {
  const RowGeom G = make_geom(a.T, a.ld, a.wq, a.wk, a.nshards, IoTraits<DT>::kBytes);
  uint32_t nw, vpl;
  layerwise_shape(G, &nw, &vpl);
  if (vpl <= 1) return launch_lw_regs<DT, 1>(G, nw, a, s, cus);
  if (vpl <= 2) return launch_lw_regs<DT, 2>(G, nw, a, s, cus);
  if (vpl <= 4) return launch_lw_regs<DT, 4>(G, nw, a, s, cus);
  if (vpl <= 8) return launch_lw_regs<DT, 8>(G, nw, a, s, cus);
  hipLaunchKernelGGL((layerwise_stream_kernel<DT>), dim3(row_blocks(G.T, nw, cus)), dim3(nw * 64),
                     (size_t)4 * G.nshards * sizeof(float), s, (uint8_t*)a.qkv, G,
                     (const uint8_t*)a.gamma_q, (const uint8_t*)a.gamma_k, a.eps);
  return hipGetLastError();
}

hipError_t launch_layerwise(const LayerwiseArgs& a, hipStream_t s, int cus) {
  return a.dtype == kBF16 ? launch_layerwise_dt<kBF16>(a, s, cus)
                          : launch_layerwise_dt<kF32>(a, s, cus);
}

template <int DT>
static hipError_t launch_partial_dt(const PartialArgs& a, hipStream_t s, int cus) {
  const RowGeom G = make_geom(a.T, a.ld, a.wq, a.wk, a.nshards, IoTraits<DT>::kBytes);
  const uint64_t items = (uint64_t)a.T * a.nshards * ((a.wq > 0) + (a.wk > 0));
  uint64_t blocks = (items + 3) / 4;
  const uint64_t cap = (uint64_t)cus * 8;
  if (blocks > cap) blocks = cap;
  if (blocks < 1) blocks = 1;
  hipLaunchKernelGGL((partial_sumsq_kernel<DT>), dim3((uint32_t)blocks), dim3(256), 0, s,
                     (const uint8_t*)a.qkv, G, a.part_q, a.part_k);
  return hipGetLastError();
}

hipError_t launch_partial_sumsq(const PartialArgs& a, hipStream_t s, int cus) {
  return a.dtype == kBF16 ? launch_partial_dt<kBF16>(a, s, cus) : launch_partial_dt<kF32>(a, s, cus);
}

template <int DT>
static hipError_t launch_apply_dt(const ApplyArgs& a, hipStream_t s, int cus) {
  const int esize = IoTraits<DT>::kBytes;
  uint64_t blocks = a.T;
  const uint64_t cap = (uint64_t)cus * 8;
  if (blocks > cap) blocks = cap;
  if (blocks < 1) blocks = 1;
  hipLaunchKernelGGL((apply_scalar_kernel<DT>), dim3((uint32_t)blocks), dim3(256), 0, s,
                     (uint8_t*)a.qkv, a.ld * esize, (uint32_t)a.T, (uint32_t)(a.wq * esize / 16),
                     (uint32_t)(a.wk * esize / 16), a.part_q, a.part_k, (uint32_t)a.nparts,
                     (float)a.norm_wq, (float)a.norm_wk, (const uint8_t*)a.gamma_q,
                     (const uint8_t*)a.gamma_k, a.eps);
  return hipGetLastError();
}

hipError_t launch_apply_scalar(const ApplyArgs& a, hipStream_t s, int cus) {
  return a.dtype == kBF16 ? launch_apply_dt<kBF16>(a, s, cus) : launch_apply_dt<kF32>(a, s, cus);
}

}  // namespace qknorm
