// Device-side building blocks for the gfx950 QK-Norm kernels.
//
// Everything here works on 16-byte vectors (one 16-byte load / store per
// lane): 16 FP8-E4M3 values, 8 bf16 or fp16 values, or 4 fp32 values.  Sums of squares
// are fp32; cross-lane reduction uses DPP row operations inside 16-lane rows
// and the gfx950 permlane swaps across rows, so no LDS is touched.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace qknorm {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));

enum : int { kF32 = 0, kBF16 = 1, kF16 = 2, kFP8 = 3 };

// kGammaDt: the dtype gamma is stored in.  It is the activations' own dtype,
// except that FP8 activations keep bf16 weights.
template <int DT> struct IoTraits;
template <> struct IoTraits<kF32> {
  static constexpr int kElems = 4;   // values per 16-byte vector
  static constexpr int kBytes = 4;
  static constexpr int kGammaDt = kF32;
};
template <> struct IoTraits<kBF16> {
  static constexpr int kElems = 8;
  static constexpr int kBytes = 2;
  static constexpr int kGammaDt = kBF16;
};
template <> struct IoTraits<kF16> {
  static constexpr int kElems = 8;
  static constexpr int kBytes = 2;
  static constexpr int kGammaDt = kF16;
};
template <> struct IoTraits<kFP8> {
  static constexpr int kElems = 16;
  static constexpr int kBytes = 1;
  static constexpr int kGammaDt = kBF16;
};

// The gamma values that pair with one 16-byte activation vector: one 16-byte
// vector, or two when gamma is wider than the activations (FP8 with bf16).
template <int DT>
struct Gam {
  static constexpr int kVecs =
      IoTraits<DT>::kElems * IoTraits<IoTraits<DT>::kGammaDt>::kBytes / 16;
  u32x4 v[kVecs];
};

// ----------------------------------------------------------------- memory --
//
// Streamed rows go through buffer loads/stores so each access carries explicit
// cache-policy bits: "nt sc1" (streaming, no reuse expected) measured best for
// in-place read-modify-write streams on MI355X.  A buffer descriptor must be
// wave-uniform (SGPRs); offsets are 32-bit per lane, and any access past
// num_records reads 0 / is dropped by the hardware range check.

// gfx9-family buffer descriptor word 3 (raw byte addressing).
constexpr int kRsrcWord3 = 0x00020000;
// CPol bits for buffer ops on gfx94x/gfx950: sc0 = 1, nt = 2, sc1 = 16.
#ifndef QKNORM_LOAD_POLICY
#define QKNORM_LOAD_POLICY 18      // nt sc1
#endif
#ifndef QKNORM_STORE_POLICY
#define QKNORM_STORE_POLICY 18     // nt sc1
#endif
constexpr int kLoadPolicy = QKNORM_LOAD_POLICY;
constexpr int kStorePolicy = QKNORM_STORE_POLICY;

typedef __amdgpu_buffer_rsrc_t Rsrc;

__device__ __forceinline__ Rsrc make_rsrc(const void* base, uint64_t bytes) {
  const uint32_t n = bytes > 0xFFFFFFFFull ? 0xFFFFFFFFu : (uint32_t)bytes;
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, n, kRsrcWord3);
}

__device__ __forceinline__ u32x4 stream_load(Rsrc r, uint32_t off) {
  return __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, kLoadPolicy);
}

__device__ __forceinline__ void stream_store(Rsrc r, uint32_t off, u32x4 v) {
  __builtin_amdgcn_raw_buffer_store_b128(v, r, off, 0, kStorePolicy);
}

// Small, reused data (gamma): default policy, kept in the caches.
__device__ __forceinline__ u32x4 cached_load(Rsrc r, uint32_t off) {
  return __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0);
}

__device__ __forceinline__ u32x4 load16(const void* p) {
  return *reinterpret_cast<const u32x4*>(p);
}

// Gamma for activation vector `vec` (gamma element index = activation index).
template <int DT>
__device__ __forceinline__ Gam<DT> load_gamma(const uint8_t* __restrict__ gamma, uint64_t vec) {
  Gam<DT> g;
#pragma unroll
  for (int i = 0; i < Gam<DT>::kVecs; ++i) g.v[i] = load16(gamma + (vec * Gam<DT>::kVecs + i) * 16);
  return g;
}

template <int DT>
__device__ __forceinline__ Gam<DT> zero_gamma() {
  Gam<DT> g;
#pragma unroll
  for (int i = 0; i < Gam<DT>::kVecs; ++i) g.v[i] = u32x4{0, 0, 0, 0};
  return g;
}

// Force a value the compiler cannot prove uniform into an SGPR.
__device__ __forceinline__ uint32_t uniform(uint32_t v) { return __builtin_amdgcn_readfirstlane(v); }

// ------------------------------------------------------------ conversions --

// Widen one 16-byte vector to fp32 (exact for every dtype).
template <int DT>
__device__ __forceinline__ void unpack(u32x4 v, float (&f)[IoTraits<DT>::kElems]) {
  if constexpr (DT == kFP8) {
    // v_cvt_pk_f32_fp8 decodes two OCP E4M3 bytes of a dword (low or high word)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int w = (int)v[i];
      const auto lo = __builtin_amdgcn_cvt_pk_f32_fp8(w, false);
      const auto hi = __builtin_amdgcn_cvt_pk_f32_fp8(w, true);
      f[4 * i] = lo[0];
      f[4 * i + 1] = lo[1];
      f[4 * i + 2] = hi[0];
      f[4 * i + 3] = hi[1];
    }
  } else if constexpr (DT == kBF16) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      f[2 * i] = __uint_as_float(v[i] << 16);
      f[2 * i + 1] = __uint_as_float(v[i] & 0xFFFF0000u);
    }
  } else if constexpr (DT == kF16) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      // copy the element out first: a bit_cast of the vector element itself
      // reads element 0 whatever i is
      const uint32_t w = v[i];
      const f16x2 h = __builtin_bit_cast(f16x2, w);
      f[2 * i] = (float)h[0];
      f[2 * i + 1] = (float)h[1];
    }
  } else {
#pragma unroll
    for (int i = 0; i < 4; ++i) f[i] = __uint_as_float(v[i]);
  }
}

// E4M3 has no infinity and its largest finite value is 448.  The hardware
// conversion rounds nearest-even in range but turns magnitudes that round
// past 448 into NaN; results are saturated to +-448 first instead (a NaN
// fails the comparison and stays NaN).
__device__ __forceinline__ float saturate_e4m3(float x) {
  return __builtin_fabsf(x) > 448.f ? __builtin_copysignf(448.f, x) : x;
}

// Round fp32 to the I/O dtype (bf16: v_cvt_pk_bf16_f32; fp16: v_cvt_f16_f32;
// FP8: v_cvt_pk_fp8_f32, saturated; all nearest-even) and pack.
//
// FP8 `may_exceed`: false only when the caller has shown that no value can
// round past 448 (see e4m3_may_exceed); then the conversion alone already
// gives the saturated result.  Otherwise the vector's largest magnitude is
// tested first and only a vector above 448 takes the saturating selects (a
// NaN is ignored by max, reaches the conversion unchanged and stays NaN).
template <int DT>
__device__ __forceinline__ u32x4 pack(const float (&f)[IoTraits<DT>::kElems],
                                      bool may_exceed = true) {
  u32x4 v;
  if constexpr (DT == kFP8) {
    float g[16];
#pragma unroll
    for (int e = 0; e < 16; ++e) g[e] = f[e];
    if (may_exceed) {
      float m = 0.f;
#pragma unroll
      for (int e = 0; e < 16; ++e) m = __builtin_fmaxf(m, __builtin_fabsf(g[e]));
      if (m > 448.f) {
#pragma unroll
        for (int e = 0; e < 16; ++e) g[e] = saturate_e4m3(g[e]);
      }
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      int w = __builtin_amdgcn_cvt_pk_fp8_f32(g[4 * i], g[4 * i + 1], 0, false);
      w = __builtin_amdgcn_cvt_pk_fp8_f32(g[4 * i + 2], g[4 * i + 3], w, true);
      v[i] = (uint32_t)w;
    }
  } else if constexpr (DT == kBF16) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      bf16x2 h = {(__bf16)f[2 * i], (__bf16)f[2 * i + 1]};
      v[i] = __builtin_bit_cast(uint32_t, h);
    }
  } else if constexpr (DT == kF16) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      f16x2 h = {(_Float16)f[2 * i], (_Float16)f[2 * i + 1]};
      v[i] = __builtin_bit_cast(uint32_t, h);
    }
  } else {
#pragma unroll
    for (int i = 0; i < 4; ++i) v[i] = __float_as_uint(f[i]);
  }
  return v;
}

// Whether any output of this wave could exceed the E4M3 range.  For a group
// of width n normalised with sums computed from its own values,
// |x_j| / sqrt(S/n + eps) <= sqrt(n) because S >= x_j^2, so |y_j| <=
// |gamma_j| sqrt(n); fp32 rounding of the sum, the scale and the two products
// adds at most about (n + 6) * 2^-24 relative (under 1e-3 for n <= 8192).  If
// every gamma of the wave satisfies |gamma| sqrt(n) <= 448 the outputs stay
// below 464, where the conversion rounds to at most 448 by itself.  The test
// is wave-uniform (a ballot), so the saturating path is a scalar branch.
__device__ __forceinline__ bool e4m3_may_exceed(float gmax, float inv_n) {
  const bool mine = gmax * gmax > 200704.f * inv_n;      // 448^2 / n
  return __builtin_amdgcn_ballot_w64(mine) != 0;
}

template <int E>
__device__ __forceinline__ float abs_max(const float (&g)[E], float m) {
#pragma unroll
  for (int e = 0; e < E; ++e) m = __builtin_fmaxf(m, __builtin_fabsf(g[e]));
  return m;
}

// Widen the gamma of one activation vector to fp32.
template <int DT>
__device__ __forceinline__ void unpack_gamma(const Gam<DT>& g, float (&f)[IoTraits<DT>::kElems]) {
  constexpr int GD = IoTraits<DT>::kGammaDt;
  constexpr int P = IoTraits<GD>::kElems;
#pragma unroll
  for (int i = 0; i < Gam<DT>::kVecs; ++i) {
    float t[P];
    unpack<GD>(g.v[i], t);
#pragma unroll
    for (int e = 0; e < P; ++e) f[i * P + e] = t[e];
  }
}

// Sum of squares of one vector, left to right, one fused multiply-add each.
template <int DT>
__device__ __forceinline__ float vec_sumsq(const float (&f)[IoTraits<DT>::kElems], float acc) {
#pragma unroll
  for (int i = 0; i < IoTraits<DT>::kElems; ++i) acc = __builtin_fmaf(f[i], f[i], acc);
  return acc;
}

// ---------------------------------------------------------- lane reduction --
//
// Each stage adds a lane's value to a partner's; fp32 addition commutes, so
// both partners hold the same bits afterwards and, after the last stage,
// every lane of the group holds the identical total.

template <int CTRL>
__device__ __forceinline__ float dpp_add(float v) {
  return v + __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(
                                           0, __builtin_bit_cast(int, v), CTRL, 0xF, 0xF, false));
}

// Sum over aligned groups of LANES consecutive lanes (LANES in 1..64).
template <int LANES>
__device__ __forceinline__ float group_sum(float v) {
  static_assert(LANES == 1 || LANES == 2 || LANES == 4 || LANES == 8 || LANES == 16 ||
                    LANES == 32 || LANES == 64, "group must be a power of two up to the wave");
  if constexpr (LANES == 1) return v;
  v = dpp_add<0xB1>(v);                       // quad_perm [1,0,3,2]: pairs
  if constexpr (LANES >= 4) v = dpp_add<0x4E>(v);   // quad_perm [2,3,0,1]: quads
  if constexpr (LANES >= 8) v = dpp_add<0x141>(v);  // row_half_mirror: half-rows of 8
  if constexpr (LANES >= 16) v = dpp_add<0x140>(v); // row_mirror: rows of 16
  if constexpr (LANES >= 32) {
    // v_permlane16_swap: with both operands v, the two results hold the even
    // and the odd 16-lane row of each 32-lane half, so their sum is the
    // 32-lane total in every lane.
    auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    v = __uint_as_float(r[0]) + __uint_as_float(r[1]);
  }
  if constexpr (LANES >= 64) {
    // v_permlane32_swap: the two results hold the low and the high half.
    auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    v = __uint_as_float(r[0]) + __uint_as_float(r[1]);
  }
  return v;
}

// 1 / sqrt(S/n + eps): the mean square plus eps as one fused multiply-add
// with 1/n (rounded to fp32 on the host, exact for power-of-two widths),
// then v_rsq_f32 (about 1 ulp).
__device__ __forceinline__ float rms_scale(float sumsq, float inv_width, float eps) {
  return __builtin_amdgcn_rsqf(__builtin_fmaf(sumsq, inv_width, eps));
}

}  // namespace qknorm
