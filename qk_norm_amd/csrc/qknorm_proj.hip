// The QKV projection with per-head QK-Norm in its epilogue (gfx950).
//
// qkv[t, n] = sum_k x[t, k] * w[n, k] (x is [T, K], w the projection weight
// [N, K], both K-contiguous: the "NT" product), accumulated in fp32 by MFMA;
// before the result is ever rounded, each Q head and each K head of a row is
// RMS-normalised over its head_dim values and multiplied by its gamma, and
// the V columns are stored as they are.  One pass instead of a projection
// that writes qkv and a normalisation that reads and writes it again.
//
// Tiling: a block of 256 threads (2 x 2 waves) owns a BM x BN = 128 x 128
// output tile; each wave a 64 x 64 quarter, as 2 x 2 v_mfma_f32_32x32x16
// blocks.  K advances in BK = 64 steps through two LDS buffers (rows padded
// to 144 bytes, so the 16-byte fragment reads of 32 consecutive rows hit
// distinct banks): the next step's global loads are in flight in registers
// while the current step's MFMAs run.  Because BN is a multiple of head_dim
// and tiles start at multiples of BN, a tile holds whole heads, and the
// epilogue can normalise them without leaving the block.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "qknorm_device.hpp"
#include "qknorm_launch.hpp"

namespace qknorm {

namespace {

constexpr int kBM = 128, kBN = 128, kBK = 64;
constexpr int kThreads = 256;
constexpr int kLdsRow = kBK + 8;               // bf16 elements per padded LDS row
constexpr int kCRow = kBN + 4;                 // fp32 elements per LDS row of the C tile
constexpr int kTileElems = kBM * kLdsRow;      // one A (or B) buffer, bf16 elements
constexpr int kLdsBytes = 4 * kTileElems * 2;  // A and B, two buffers each
static_assert(kBM * kCRow * 4 <= kLdsBytes, "the C tile reuses the operand buffers");
constexpr int kChunks = kBM * kBK * 2 / 16 / kThreads;   // 16-byte loads per thread per operand

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

// Global -> registers: chunk c = tid + i*256 of the tile is row c/8, columns
// 8*(c%8) .. +8 of this K step.  Rows past the operand's end read zeros (the
// descriptor covers only the valid rows).
__device__ __forceinline__ void load_tile(Rsrc rs, uint32_t pitch_bytes, uint32_t k_bytes,
                                          uint32_t tid, u32x4 (&r)[kChunks]) {
#pragma unroll
  for (int i = 0; i < kChunks; ++i) {
    const uint32_t c = tid + i * kThreads;
    r[i] = __builtin_amdgcn_raw_buffer_load_b128(rs, (c / 8) * pitch_bytes + k_bytes + (c % 8) * 16,
                                                 0, 0);
  }
}

__device__ __forceinline__ void store_tile(__bf16* lds, uint32_t tid, const u32x4 (&r)[kChunks]) {
#pragma unroll
  for (int i = 0; i < kChunks; ++i) {
    const uint32_t c = tid + i * kThreads;
    *reinterpret_cast<u32x4*>(lds + (c / 8) * kLdsRow + (c % 8) * 8) = r[i];
  }
}

__device__ __forceinline__ bf16x8 frag(const __bf16* lds, uint32_t row, uint32_t k) {
  return *reinterpret_cast<const bf16x8*>(lds + row * kLdsRow + k);
}

// Epilogue for one tile: C (fp32, in LDS) -> normalised bf16 rows.  Lane l
// of a wave takes row (step*4 + l/16) of its rows and columns 8*(l%16) ..
// +8, so a head of D columns is D/8 consecutive lanes: its sum of squares is
// the lanes' fma chains, then a D/8-lane reduction.
template <int D>
__device__ __forceinline__ void epilogue(const float* C, uint8_t* __restrict__ out,
                                         uint64_t ld_bytes, uint32_t T, uint32_t N, uint32_t m0,
                                         uint32_t n0, uint32_t hq, uint32_t hkv,
                                         const uint8_t* __restrict__ gamma_q,
                                         const uint8_t* __restrict__ gamma_k, float eps,
                                         float inv_d, bool norm, uint32_t wave, uint32_t lane) {
  constexpr uint32_t LG = D / 8;               // lanes per head
  const uint32_t col = (lane % 16) * 8;        // column inside the tile
  const uint32_t n = n0 + col;                 // global column of this lane's first value
  const uint32_t head = n / D;
  const bool is_q = head < hq, is_k = !is_q && head < hq + hkv;
  const bool normed = norm && (is_q || is_k) && n < N;
  float g[8];
  if (normed) {
    const uint8_t* gp = (is_q ? gamma_q : gamma_k) + (uint64_t)(n % D) * 2;
    unpack<kBF16>(load16(gp), g);
  }
  const uint32_t valid_cols = N - n0 < (uint32_t)kBN ? N - n0 : (uint32_t)kBN;
  for (uint32_t step = 0; step < kBM / 4 / 4; ++step) {   // 4 waves x 4 rows per step
    const uint32_t r = (step * 4 + wave) * 4 + lane / 16;  // row inside the tile
    const uint32_t t = m0 + r;
    float v[8];
    const float4 lo = *reinterpret_cast<const float4*>(C + r * kCRow + col);
    const float4 hi = *reinterpret_cast<const float4*>(C + r * kCRow + col + 4);
    v[0] = lo.x; v[1] = lo.y; v[2] = lo.z; v[3] = lo.w;
    v[4] = hi.x; v[5] = hi.y; v[6] = hi.z; v[7] = hi.w;
    float s = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) s = __builtin_fmaf(v[e], v[e], s);
    s = group_sum<LG>(s);
    if (normed) {
      const float sc = rms_scale(s, inv_d, eps);
#pragma unroll
      for (int e = 0; e < 8; ++e) v[e] = (v[e] * g[e]) * sc;
    }
    // the row's valid columns only; rows past T store nothing
    const Rsrc rs = make_rsrc(out + (uint64_t)(t < T ? t : 0) * ld_bytes + (uint64_t)n0 * 2,
                              t < T ? valid_cols * 2 : 0);
    stream_store(rs, col * 2, pack<kBF16>(v));
  }
}

template <int D>
__global__ __launch_bounds__(kThreads) void qkv_proj_kernel(
    const uint8_t* __restrict__ x, uint32_t ldx_bytes, const uint8_t* __restrict__ w,
    uint32_t ldw_bytes, uint8_t* __restrict__ out, uint64_t ld_bytes, uint32_t T, uint32_t K,
    uint32_t N, uint32_t hq, uint32_t hkv, const uint8_t* __restrict__ gamma_q,
    const uint8_t* __restrict__ gamma_k, float eps, float inv_d, uint32_t norm) {
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
  __bf16* As = reinterpret_cast<__bf16*>(smem);              // [2][BM][kLdsRow]
  __bf16* Bs = As + 2 * kTileElems;                          // [2][BN][kLdsRow]
  const uint32_t tid = threadIdx.x, lane = tid & 63;
  const uint32_t wave = uniform(tid >> 6);
  const uint32_t wm = wave >> 1, wn = wave & 1;              // the wave's 64 x 64 quarter
  const uint32_t n0 = blockIdx.x * kBN, m0 = blockIdx.y * kBM;

  // operand descriptors: the tile's rows that exist
  const uint32_t a_rows = T - m0 < (uint32_t)kBM ? T - m0 : (uint32_t)kBM;
  const uint32_t b_rows = N - n0 < (uint32_t)kBN ? N - n0 : (uint32_t)kBN;
  const Rsrc ra = make_rsrc(x + (uint64_t)m0 * ldx_bytes, (uint64_t)(a_rows - 1) * ldx_bytes + K * 2);
  const Rsrc rb = make_rsrc(w + (uint64_t)n0 * ldw_bytes, (uint64_t)(b_rows - 1) * ldw_bytes + K * 2);

  f32x16 acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.f;

  const uint32_t ksteps = K / kBK;
  u32x4 pa[kChunks], pb[kChunks];
  load_tile(ra, ldx_bytes, 0, tid, pa);
  load_tile(rb, ldw_bytes, 0, tid, pb);
  store_tile(As, tid, pa);
  store_tile(Bs, tid, pb);
  __syncthreads();

  // a lane's fragment: row (lane % 32) of a 32-row block, 8 consecutive k
  // starting at 8*(lane/32) of each 16-wide MFMA step; A and B use the same
  // k order, so the products pair correctly whatever order the hardware sums
  const uint32_t fr = lane % 32, fk = 8 * (lane / 32);
  for (uint32_t ks = 0; ks < ksteps; ++ks) {
    const uint32_t buf = ks & 1;
    const bool more = ks + 1 < ksteps;
    if (more) {
      load_tile(ra, ldx_bytes, (ks + 1) * kBK * 2, tid, pa);
      load_tile(rb, ldw_bytes, (ks + 1) * kBK * 2, tid, pb);
    }
    const __bf16* Ab = As + buf * kTileElems;
    const __bf16* Bb = Bs + buf * kTileElems;
#pragma unroll
    for (uint32_t kk = 0; kk < kBK; kk += 16) {
      bf16x8 a[2], b[2];
#pragma unroll
      for (int i = 0; i < 2; ++i) a[i] = frag(Ab, wm * 64 + i * 32 + fr, kk + fk);
#pragma unroll
      for (int j = 0; j < 2; ++j) b[j] = frag(Bb, wn * 64 + j * 32 + fr, kk + fk);
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[i], b[j], acc[i][j], 0, 0, 0);
    }
    if (more) {
      store_tile(As + (buf ^ 1) * kTileElems, tid, pa);
      store_tile(Bs + (buf ^ 1) * kTileElems, tid, pb);
    }
    __syncthreads();
  }

  // accumulators -> LDS (fp32): block (i, j) of the wave, value e of lane l
  // is row 8*(e/4) + 4*(l/32) + e%4 and column l%32 of that 32 x 32 block
  float* C = reinterpret_cast<float*>(smem);
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const uint32_t r = wm * 64 + i * 32 + 8 * (e / 4) + 4 * (lane / 32) + e % 4;
        const uint32_t c = wn * 64 + j * 32 + lane % 32;
        C[r * kCRow + c] = acc[i][j][e];
      }
  __syncthreads();
  epilogue<D>(C, out, ld_bytes, T, N, m0, n0, hq, hkv, gamma_q, gamma_k, eps, inv_d, norm != 0,
              wave, lane);
}

}  // namespace

bool proj_shape_ok(const ProjArgs& a) {
  // buffer offsets inside one tile's rows stay below 2^31
  const uint64_t es = 2;
  return (uint64_t)kBM * a.ldx * es < (UINT64_C(1) << 31) &&
         (uint64_t)kBN * a.ldw * es < (UINT64_C(1) << 31) && a.hidden % kBK == 0 &&
         (a.head_dim == 64 || a.head_dim == 128);
}

hipError_t launch_qkv_proj(const ProjArgs& a, hipStream_t s) {
  const uint32_t N = (uint32_t)((a.hq + 2 * a.hkv) * a.head_dim);
  const dim3 grid((N + kBN - 1) / kBN, (uint32_t)((a.T + kBM - 1) / kBM));
  auto kern = a.head_dim == 64 ? qkv_proj_kernel<64> : qkv_proj_kernel<128>;
  // more than the default 64 KiB of dynamic LDS (gfx950 has 160 KiB per CU);
  // a host-side attribute, set on every call (no shared state between threads)
  const hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                           hipFuncAttributeMaxDynamicSharedMemorySize, kLdsBytes);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(kern, grid, dim3(kThreads), kLdsBytes, s, (const uint8_t*)a.x,
                     (uint32_t)(a.ldx * 2), (const uint8_t*)a.w, (uint32_t)(a.ldw * 2),
                     (uint8_t*)a.qkv, (uint64_t)a.ld * 2, (uint32_t)a.T, (uint32_t)a.hidden, N,
                     (uint32_t)a.hq, (uint32_t)a.hkv, (const uint8_t*)a.gamma_q,
                     (const uint8_t*)a.gamma_k, a.eps, 1.0f / (float)a.head_dim,
                     (uint32_t)((a.flags & 1) == 0));
  return hipGetLastError();
}

}  // namespace qknorm
