// The QKV projection with per-head QK-Norm in its epilogue (gfx950).
//
// qkv[t, n] = sum_k x[t, k] * w[n, k] (x is [T, K], w the projection weight
// [N, K], both K-contiguous: the "NT" product), accumulated in fp32 by MFMA;
// before the result is ever rounded, each Q head and each K head of a row is
// RMS-normalised over its head_dim values and multiplied by its gamma, and
// the V columns are stored as they are.  One pass instead of a projection
// that writes qkv and a normalisation that reads and writes it again.
//
// Tiling: a block of 512 threads (4 x 2 waves, two per SIMD) owns a 256 x 256
// output tile; each wave a 64 x 128 slab of 4 x 8 v_mfma_f32_16x16x32_bf16
// blocks (v_mfma_f32_16x16x32_f16 for fp16, the same layout).  K advances 64
// at a time through a ring of LDS stages (two for these tiles, three or four
// for the smaller ones) filled straight from global memory (buffer loads
// into LDS, no staging registers), with the operand rows XOR-swizzled so that
// fragment reads hit distinct banks.  Where 256 x 256 tiles would leave a
// round of the chip's CUs half empty, the last columns go to 256 x 128 tiles
// of the same launch.  Tiles are ordered so the blocks
// each XCD holds at once share operand panels in its L2.  Because tile widths
// are multiples of head_dim (or one head spans a tile's two column waves)
// and tiles start at multiples of it, a tile holds whole heads, and the
// epilogue normalises them in registers without leaving the block.  The
// MFMAs take the weight's fragment as their first operand, so a lane's
// accumulators are four consecutive columns of one token: one lane swap
// then gives each lane eight consecutive outputs, stored as one 16-byte
// write straight from registers.
//
// Fewer tokens take narrower launches of the same kernel (128-row tiles one
// head wide up to 512 tokens, or on to 1024 while they fit one round of the
// CUs; 64-row tiles from 1 token to 256).  With a workspace, up to 64 tokens
// take two other kernels instead: the weight split over many more blocks
// into fp32 partials, then one block per head adding them and normalising
// (qkv_proj_split_kernel, qkv_proj_split_finish_kernel).
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <atomic>
#include <mutex>
#include <type_traits>

#include "qknorm_device.hpp"
#include "qknorm_launch.hpp"

namespace qknorm {

namespace {

typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

// The 16-bit element type: its 8-element fragment and the 16 x 16 x 32 MFMA
// that takes it (fp32 accumulation, 4 accumulators per lane).
template <int DT>
struct ProjElem;
template <>
struct ProjElem<kBF16> {
  typedef __bf16 T;
  typedef __bf16 V8 __attribute__((ext_vector_type(8)));
  static __device__ __forceinline__ f32x4 mfma(V8 a, V8 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
  }
};
template <>
struct ProjElem<kF16> {
  typedef _Float16 T;
  typedef _Float16 V8 __attribute__((ext_vector_type(8)));
  static __device__ __forceinline__ f32x4 mfma(V8 a, V8 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
  }
};

// Two fp32 values rounded once (to nearest even) to the element type and
// packed into one dword, the first in the low half (the lower address).
template <int DT>
__device__ __forceinline__ uint32_t pack2(float a, float b) {
  typedef typename ProjElem<DT>::T Elem;
  const Elem ea = (Elem)a, eb = (Elem)b;
  return (uint32_t)__builtin_bit_cast(uint16_t, ea) | ((uint32_t)__builtin_bit_cast(uint16_t, eb) << 16);
}

// MFMA block: 16 x 16 outputs, 32 of K per instruction.  Lane l supplies row
// l % 16 of each operand's fragment (8 consecutive k from 8 * (l / 16)), and
// holds accumulator e of the block at row 4 * (l / 16) + e of the first
// operand and row l % 16 of the second.

// Tile geometry.  A block of WM x WN waves owns a BM x BN output tile; each
// wave a (BM/WM) x (BN/WN) slab of MS x MS MFMA blocks; K advances BK at a
// time through S LDS stages.  Operand rows are BK*2 bytes with no padding:
// the 16-byte chunk c of row r sits in slot c ^ ((r / RPB) % CPR) (CPR chunks
// per row, RPB rows per 256 bytes), so the 16 rows read by 16 lanes at once
// land in 16 different 16-byte slots of a 256-byte bank line.  Global loads
// go straight into LDS (buffer_load_dwordx4 ... lds: lane i of a wave writes
// 16 bytes at the instruction's LDS base + 16*i), so lane i of an
// instruction covering rows R .. R+1024/(BK*2)-1 fetches row R + i / CPR and
// the chunk whose slot is i % CPR: no staging registers and no LDS write
// instructions.
template <int BM_, int BN_, int WM_, int WN_, int BK_, int S_>
struct Tile {
  static constexpr int BM = BM_, BN = BN_, WM = WM_, WN = WN_, BK = BK_, S = S_, MS = 16;
  static constexpr int kThreads = 64 * WM * WN, kWaves = WM * WN;
  static constexpr int kWaveM = BM / WM, kWaveN = BN / WN;
  static constexpr int MB = kWaveM / MS, NB = kWaveN / MS;
  static constexpr int KS = 32, KK = BK / KS;                 // K per MFMA, MFMA steps per K step
  typedef f32x4 Acc;
  static constexpr int kRowBytes = BK * 2;
  static constexpr int CPR = kRowBytes / 16, RPB = 256 / kRowBytes;
  static constexpr int kInstRows = 1024 / kRowBytes;         // rows one load instruction fills
  static constexpr int kStageBytes = (BM + BN) * kRowBytes;
  static constexpr int kStagesBytes = S * kStageBytes;
  static constexpr int kAInst = BM / kInstRows / kWaves, kBInst = BN / kInstRows / kWaves;
  static constexpr int kLoads = kAInst + kBInst;              // per wave per K step
  static_assert(BM % (kInstRows * kWaves) == 0 && BN % (kInstRows * kWaves) == 0, "");
  static_assert(RPB * CPR == 16, "a 256-byte line holds 16 chunks");
};

#ifndef QKNORM_PROJ_XCD
#define QKNORM_PROJ_XCD 1
#endif
#ifndef QKNORM_PROJ_MPR
#define QKNORM_PROJ_MPR 1          // MFMAs between the fragment reads of the next sub-step
#endif
#ifndef QKNORM_PROJ_GM
#define QKNORM_PROJ_GM 4
#endif
#ifndef QKNORM_PROJ_STAGGER
#define QKNORM_PROJ_STAGGER 1      // 0: every block walks K from step 0
#endif
constexpr bool kXcdRemap = QKNORM_PROJ_XCD != 0;
constexpr uint32_t kGroupM = QKNORM_PROJ_GM;

template <class G>
__device__ __forceinline__ uint32_t lds_slot(uint32_t row, uint32_t chunk) {
  return chunk ^ ((row / G::RPB) % G::CPR);
}

// Per-lane byte offsets of a wave's operand loads within a K step: A rows in
// off[0..kAInst), B rows after them.  They do not change with the step (the
// step's byte offset travels in the instruction's scalar offset).
template <class G>
struct DmaOffsets {
  uint32_t a[G::kAInst], b[G::kBInst];
};

template <class G>
__device__ __forceinline__ DmaOffsets<G> dma_offsets(uint32_t ldx_bytes, uint32_t ldw_bytes,
                                                     uint32_t wave, uint32_t lane) {
  constexpr uint32_t kRows = G::kInstRows, kBM = G::BM, kCpr = G::CPR, kRpb = G::RPB;
  const uint32_t sub = lane / kCpr, s = lane % kCpr;
  DmaOffsets<G> o;
#pragma unroll
  for (int j = 0; j < G::kAInst; ++j) {
    const uint32_t r = (wave * G::kAInst + j) * kRows + sub;
    o.a[j] = r * ldx_bytes + (s ^ ((r / kRpb) % kCpr)) * 16;
  }
#pragma unroll
  for (int j = 0; j < G::kBInst; ++j) {
    const uint32_t r = (wave * G::kBInst + j) * kRows + sub;
    o.b[j] = r * ldw_bytes + (s ^ (((kBM + r) / kRpb) % kCpr)) * 16;
  }
  return o;
}

// One K step of the block's A and B tiles into a stage, this wave's share.
// Rows past the end of x or w fall outside their descriptors (the row's own
// offset already does, whatever the step's) and arrive as zeros.
template <class G>
__device__ __forceinline__ void dma_tile(Rsrc ra, Rsrc rb, const DmaOffsets<G>& o,
                                         uint32_t k_bytes, uint8_t* stage, uint32_t wave) {
  constexpr uint32_t kRows = G::kInstRows, kRowBytes = G::kRowBytes, kBM = G::BM;
  constexpr int kMax = G::kAInst > G::kBInst ? G::kAInst : G::kBInst;
  // A and B loads alternate while both have some left
#pragma unroll
  for (int j = 0; j < kMax; ++j) {
    if (j < G::kAInst) {
      const uint32_t R = (wave * G::kAInst + j) * kRows;
      const uint32_t va = o.a[j];                // (locals: the host pass rejects members here)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          ra, (__attribute__((address_space(3))) void*)(stage + R * kRowBytes), 16, va, k_bytes,
          0, 0);
    }
    if (j < G::kBInst) {
      const uint32_t R = (wave * G::kBInst + j) * kRows;
      const uint32_t vb = o.b[j];
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          rb, (__attribute__((address_space(3))) void*)(stage + (kBM + R) * kRowBytes), 16, vb,
          k_bytes, 0, 0);
    }
  }
}

template <class G, int DT>
__device__ __forceinline__ typename ProjElem<DT>::V8 sfrag(const uint8_t* base, uint32_t row, uint32_t k) {
  return *reinterpret_cast<const typename ProjElem<DT>::V8*>(base + row * G::kRowBytes +
                                                            lds_slot<G>(row, k / 8) * 16);
}

// Byte offset of the block's K step k (or of its last step for k past it),
// the block's walk through K starting `shift` steps in and wrapping round.
template <class G>
__device__ __forceinline__ uint32_t step_bytes(uint32_t k, uint32_t ksteps, uint32_t shift) {
  uint32_t s = (k < ksteps ? k : ksteps - 1) + shift;
  if (s >= ksteps) s -= ksteps;
  return s * G::BK * 2;
}

// s_waitcnt with vmcnt(N) and the other counters left alone (gfx9 encoding:
// vmcnt bits 3:0 and 15:14, expcnt 6:4, lgkmcnt 11:8).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

// A workgroup barrier that waits for this wave's LDS reads but not for its
// loads into LDS: __syncthreads() would make the compiler wait for every
// outstanding load (vmcnt(0)), including the ones meant to stay in flight.
// The loads that must have landed are waited for explicitly before it.  The
// lgkmcnt(0) matters: a fragment read still in flight at the barrier could
// otherwise meet another wave's refill of the same stage issued after it.
// The "memory" clobber keeps the compiler from moving LDS accesses across it.
__device__ __forceinline__ void stage_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

template <class G, int DT>
__device__ __forceinline__ void read_frags(const uint8_t* st, uint32_t arow, uint32_t brow,
                                           uint32_t k, typename ProjElem<DT>::V8 (&a)[G::MB],
                                           typename ProjElem<DT>::V8 (&b)[G::NB]) {
#pragma unroll
  for (int i = 0; i < G::MB; ++i) a[i] = sfrag<G, DT>(st, arow + i * G::MS, k);
#pragma unroll
  for (int j = 0; j < G::NB; ++j) b[j] = sfrag<G, DT>(st, brow + j * G::MS, k);
}

// One MFMA per block, the weight's fragment first: block (i, j) accumulates
// rows j*16.. of w against rows i*16.. of x, so its lanes hold output
// columns 4*(l/16) + e of token l%16 (the layout the epilogue stores from).
template <class G, int DT>
__device__ __forceinline__ void mfma_step(typename G::Acc (&acc)[G::MB][G::NB],
                                          const typename ProjElem<DT>::V8 (&a)[G::MB],
                                          const typename ProjElem<DT>::V8 (&b)[G::NB]) {
#pragma unroll
  for (int i = 0; i < G::MB; ++i)
#pragma unroll
    for (int j = 0; j < G::NB; ++j) acc[i][j] = ProjElem<DT>::mfma(b[j], a[i], acc[i][j]);
}

// Instruction order for the scheduler (sched_group_barrier masks: 0x008
// MFMA, 0x020 vector memory read, 0x100 LDS read).  One MFMA, then R LDS
// reads and V loads, NP times; then the remaining M MFMAs back to back.  With
// one wave per SIMD nothing else hides a read's latency, so the reads feeding
// the next sub-step go between this sub-step's MFMAs.
template <int NP, int R, int V, int M = 1>
__device__ __forceinline__ void sched_interleave() {
  if constexpr (NP > 0) {
    __builtin_amdgcn_sched_group_barrier(0x008, M, 0);
    if constexpr (R > 0) __builtin_amdgcn_sched_group_barrier(0x100, R, 0);
    if constexpr (V > 0) __builtin_amdgcn_sched_group_barrier(0x020, V, 0);
    sched_interleave<NP - 1, R, V, M>();
  }
}

template <int M>
__device__ __forceinline__ void sched_mfmas() {
  if constexpr (M > 0) __builtin_amdgcn_sched_group_barrier(0x008, M, 0);
}

// Tile order.  Workgroups go to the 8 XCDs round robin (id % 8), each XCD
// with its own L2; the remap gives each XCD a contiguous run of tiles, and
// the runs walk the output in bands of GM tile rows, columns outer, so the
// blocks an XCD holds at once share a few A and B panels in its L2.
// `id` counts the blocks of one tile shape (0 .. count-1); blocks are numbered
// so that id % 8 is the block's XCD.
template <class G>
__device__ __forceinline__ void tile_origin(uint32_t T, uint32_t N, uint32_t id, uint32_t count,
                                            uint32_t* m0, uint32_t* n0) {
  const uint32_t n_tiles = (N + G::BN - 1) / G::BN, m_tiles = (T + G::BM - 1) / G::BM;
  if (kXcdRemap) {
    const uint32_t q = count / 8, r = count % 8, xcd = id % 8;
    id = xcd * q + (xcd < r ? xcd : r) + id / 8;
  }
  const uint32_t band = id / (kGroupM * n_tiles), first_m = band * kGroupM;
  const uint32_t gm = m_tiles - first_m < kGroupM ? m_tiles - first_m : kGroupM;
  const uint32_t within = id - band * kGroupM * n_tiles;
  *n0 = (within / gm) * G::BN;
  *m0 = (first_m + within % gm) * G::BM;
}

// LDS beyond the operand stages: gamma_q and gamma_k as fp32 (head_dim
// values each, at most 256), then the half-head row sums of head_dim 256
// ([2 column waves][256 rows]).
constexpr int kGammaFloats = 2 * 256;
constexpr int kHalfFloats = 2 * 256;

// gamma_q and gamma_k into the block's table, once per block (threads below
// head_dim; a missing gamma reads as 1, and is only used where normalised).
template <int DT, int D>
__device__ __forceinline__ void stage_gamma(float* gtab, const uint8_t* __restrict__ gamma_q,
                                            const uint8_t* __restrict__ gamma_k, uint32_t tid) {
  typedef typename ProjElem<DT>::T Elem;
  if (tid < (uint32_t)D) {
    gtab[tid] = gamma_q ? (float)reinterpret_cast<const Elem*>(gamma_q)[tid] : 1.f;
    gtab[D + tid] = gamma_k ? (float)reinterpret_cast<const Elem*>(gamma_k)[tid] : 1.f;
  }
}

// Sum over the four lanes that hold one token (l, l ^ 16, l ^ 32, l ^ 48):
// every lane gets the same value (each step adds a pair in either order).
__device__ __forceinline__ float token_sum(float v) {
  auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  v = __uint_as_float(r[0]) + __uint_as_float(r[1]);
  auto r2 = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(r2[0]) + __uint_as_float(r2[1]);
}

// Epilogue: per-head QK-Norm on the fp32 accumulators (unless `norm` is 0),
// then 16-byte stores straight from registers.  Block (i, j) of a wave holds
// token i*16 + l%16 of the wave's rows and columns j*16 + 4*(l/16) + e,
// e = 0..3 (the weight's fragment is the MFMA's first operand).  A head of
// D columns is D/16 consecutive blocks j (a wave's columns are whole heads,
// or half of one for head_dim 256): a token's sum of squares is each lane's
// fma chain over its 4 values of each block, then the sum over the 4 lanes
// that hold the token.  For the stores, blocks 2p and 2p+1 are paired: one
// v_permlane16_swap per dword moves the even rows' block-2p+1 values and the
// odd rows' block-2p values across, which leaves each lane 8 consecutive
// columns of its token.
template <class G, int DT, int D>
__device__ __forceinline__ void proj_epilogue(const f32x4 (&acc)[G::MB][G::NB], const float* gtab,
                                              float* half, uint32_t lane, uint32_t wm, uint32_t wn,
                                              uint32_t m0, uint32_t n0, uint32_t a_rows, uint32_t N,
                                              uint32_t hq, uint32_t hkv, float eps, float inv_d,
                                              uint32_t norm, uint8_t* __restrict__ out,
                                              uint64_t ld_bytes) {
  constexpr int MB = G::MB, NB = G::NB;
  constexpr int JH = D / 16;                     // blocks per head
  constexpr int NH = JH <= NB ? NB / JH : 1;     // heads in a wave's columns (or one half-head)
  static_assert(NB % 2 == 0, "blocks are stored in pairs");
  const uint32_t q4 = lane / 16, tl = lane % 16;
  const uint32_t c_wave = n0 + wn * G::kWaveN;   // the wave's first column
  // each block's columns lie in one head, so whether it is normalised (and
  // its gamma table) is the same for the whole block
  bool normed[NB];
  float g[NB][4];
#pragma unroll
  for (int j = 0; j < NB; ++j) {
    const uint32_t nb = c_wave + j * 16;
    const uint32_t head = nb / D;
    normed[j] = norm && head < hq + hkv && nb < N;
    const float4 gv = *reinterpret_cast<const float4*>(gtab + (head < hq ? 0 : D) + nb % D + 4 * q4);
    g[j][0] = gv.x;
    g[j][1] = gv.y;
    g[j][2] = gv.z;
    g[j][3] = gv.w;
  }
  float sc[MB][NH];
  if (norm) {
    if constexpr (JH <= NB) {
      static_assert(NB % JH == 0, "a wave's columns must be whole heads");
#pragma unroll
      for (int h = 0; h < NH; ++h) {
        if (!normed[h * JH]) continue;           // the same for the whole head
#pragma unroll
        for (int i = 0; i < MB; ++i) {
          float s = 0.f;
#pragma unroll
          for (int jj = 0; jj < JH; ++jj)
#pragma unroll
            for (int e = 0; e < 4; ++e) s = __builtin_fmaf(acc[i][h * JH + jj][e], acc[i][h * JH + jj][e], s);
          sc[i][h] = rms_scale(token_sum(s), inv_d, eps);
        }
      }
    } else {
      // a head spans the tile's two column waves (D = 2 * kWaveN): each wave
      // leaves its half-head sums in LDS, and both add the two halves in the
      // same order, so they scale with the same bits
      static_assert(JH == 2 * NB && G::WN == 2 && G::BN == D, "one head across the two column waves");
#pragma unroll
      for (int i = 0; i < MB; ++i) {
        float s = 0.f;
#pragma unroll
        for (int j = 0; j < NB; ++j)
#pragma unroll
          for (int e = 0; e < 4; ++e) s = __builtin_fmaf(acc[i][j][e], acc[i][j][e], s);
        s = token_sum(s);
        if (q4 == 0) half[wn * G::BM + wm * G::kWaveM + i * 16 + tl] = s;
      }
      __syncthreads();
#pragma unroll
      for (int i = 0; i < MB; ++i) {
        const uint32_t r = wm * G::kWaveM + i * 16 + tl;
        sc[i][0] = rms_scale(half[r] + half[G::BM + r], inv_d, eps);
      }
    }
  }
  // one descriptor over the tile's rows (wave-uniform); rows past T and
  // columns past N get an offset outside it
  const uint32_t valid_cols = N - n0 < (uint32_t)G::BN ? N - n0 : (uint32_t)G::BN;
  const Rsrc ro = make_rsrc(out + (uint64_t)m0 * ld_bytes + (uint64_t)n0 * 2,
                            (uint64_t)(a_rows - 1) * ld_bytes + valid_cols * 2);
  auto value = [&](int i, int j, int e) {
    const float v = acc[i][j][e];
    return normed[j] ? (v * g[j][e]) * sc[i][JH <= NB ? j / JH : 0] : v;
  };
#pragma unroll
  for (int i = 0; i < MB; ++i) {
    const uint32_t r = wm * G::kWaveM + i * 16 + tl;
#pragma unroll
    for (int p = 0; p < NB / 2; ++p) {
      const uint32_t a01 = pack2<DT>(value(i, 2 * p, 0), value(i, 2 * p, 1));
      const uint32_t a23 = pack2<DT>(value(i, 2 * p, 2), value(i, 2 * p, 3));
      const uint32_t b01 = pack2<DT>(value(i, 2 * p + 1, 0), value(i, 2 * p + 1, 1));
      const uint32_t b23 = pack2<DT>(value(i, 2 * p + 1, 2), value(i, 2 * p + 1, 3));
      auto s01 = __builtin_amdgcn_permlane16_swap(a01, b01, false, false);
      auto s23 = __builtin_amdgcn_permlane16_swap(a23, b23, false, false);
      // even rows (q4 0, 2): block 2p, columns 4*q4 .. +7; odd rows: block 2p+1,
      // columns 4*(q4-1) .. +7
      const uint32_t c = wn * G::kWaveN + 32 * p + (q4 & 1) * 16 + (q4 >> 1) * 8;
      const u32x4 v = {s01[0], s23[0], s01[1], s23[1]};
      stream_store(ro, r < a_rows && c < valid_cols ? r * (uint32_t)ld_bytes + c * 2 : 0xFFFFFFF0u, v);
    }
  }
}

// The kernel's arguments (one copy for both tile shapes).
struct ProjKArgs {
  const uint8_t* x;
  const uint8_t* w;
  uint8_t* out;
  const uint8_t* gamma_q;
  const uint8_t* gamma_k;
  uint64_t ld_bytes;
  uint32_t ldx_bytes, ldw_bytes, T, K, N, hq, hkv, norm;
  float eps, inv_d;
};

// One output tile of shape G: rows m0 .. m0+BM-1, columns n0 .. n0+BN-1 of
// the column range [n_begin, n_end) this tile shape covers.
template <class G, int DT, int D>
__device__ __forceinline__ void proj_tile(const ProjKArgs& args, uint32_t id, uint32_t count,
                                          uint32_t n_begin, uint32_t n_end, uint8_t* smem,
                                          const float* gtab, float* half) {
  constexpr int MB = G::MB, NB = G::NB, BK = G::BK;
  const uint8_t* __restrict__ x = args.x;
  const uint8_t* __restrict__ w = args.w;
  const uint32_t ldx_bytes = args.ldx_bytes, ldw_bytes = args.ldw_bytes;
  const uint32_t T = args.T, K = args.K;
  const uint32_t tid = threadIdx.x, lane = tid & 63;
  const uint32_t wave = uniform(tid >> 6);
  const uint32_t wm = wave / G::WN, wn = wave % G::WN;
  uint32_t m0, n0;
  tile_origin<G>(T, n_end - n_begin, id, count, &m0, &n0);
  n0 += n_begin;

  const uint32_t a_rows = T - m0 < (uint32_t)G::BM ? T - m0 : (uint32_t)G::BM;
  const uint32_t b_rows = n_end - n0 < (uint32_t)G::BN ? n_end - n0 : (uint32_t)G::BN;
  const Rsrc ra = make_rsrc(x + (uint64_t)m0 * ldx_bytes, (uint64_t)(a_rows - 1) * ldx_bytes + K * 2);
  const Rsrc rb = make_rsrc(w + (uint64_t)n0 * ldw_bytes, (uint64_t)(b_rows - 1) * ldw_bytes + K * 2);

  typename G::Acc acc[MB][NB];
#pragma unroll
  for (int i = 0; i < MB; ++i)
#pragma unroll
    for (int j = 0; j < NB; ++j)
#pragma unroll
      for (int e = 0; e < 4; ++e) acc[i][j][e] = 0.f;

  // S LDS stages in a ring; K step ks computes from stage ks % S.  Fragments
  // are double-buffered in registers: the reads of sub-step kk+1 are issued
  // before the MFMAs of sub-step kk.  Before the last sub-step of a step the
  // wave waits for its loads of step ks+1 (those of steps ks+2 .. ks+S-1 stay
  // in flight: loads into LDS complete in the order they were issued) and
  // meets the barrier; after it, the stage just finished is free (every
  // wave's reads of it have completed), so the loads of step ks+S go there,
  // and the first fragments of step ks+1 are read while the last MFMAs of
  // step ks run.  Loads past the last step fetch the last step again
  // (unused).  More stages keep more of the operands in flight per block,
  // which is what bounds a launch of few blocks reading a cold weight.
  constexpr int S = G::S, KK = G::KK, L = G::kLoads;
  static_assert(S >= 2 && KK % 2 == 0, "two stages or more, an even number of MFMA steps");
  static_assert((S - 1) * L < 64, "the loads in flight fit the vmcnt counter");
  const uint32_t ksteps = K / BK;
  // a lane's fragment: row (lane % MS) of an MS-row block, 8 consecutive k
  // starting at 8*(lane/MS) of each KS-wide MFMA step; A and B use the same
  // k order, so the products pair correctly whatever order the hardware sums
  const uint32_t fr = lane % G::MS, fk = 8 * (lane / G::MS);
  const uint32_t arow = wm * G::kWaveM + fr, brow = G::BM + wn * G::kWaveN + fr;
  uint8_t* const stage0 = smem;
  uint8_t* const stage1 = smem + G::kStageBytes;
  auto stage = [&](uint32_t i) { return smem + i * G::kStageBytes; };

  // The blocks of each XCD start their walk through K at their own eighth of
  // it: blocks on different XCDs that share weight columns then reach each
  // K step at different times, so a step's weight comes from HBM for the
  // first of them only and from the Infinity Cache for the rest.
  const uint32_t shift = QKNORM_PROJ_STAGGER ? uniform(blockIdx.x % 8 * ksteps / 8) : 0;
  const DmaOffsets<G> doff = dma_offsets<G>(ldx_bytes, ldw_bytes, wave, lane);
  if constexpr (S == 2) {
    dma_tile<G>(ra, rb, doff, step_bytes<G>(0, ksteps, shift), stage0, wave);
    wait_vmcnt<0>();
    stage_barrier();
    dma_tile<G>(ra, rb, doff, step_bytes<G>(1, ksteps, shift), stage1, wave);
  } else {
#pragma unroll
    for (int p = 0; p < S; ++p) dma_tile<G>(ra, rb, doff, step_bytes<G>(p, ksteps, shift), stage(p), wave);
    wait_vmcnt<(S - 1) * L>();                 // step 0 has landed (this wave)
    stage_barrier();
  }
  typedef typename ProjElem<DT>::V8 Frag;
  Frag fa[2][MB], fb[2][NB];
  read_frags<G, DT>(stage0, arow, brow, fk, fa[0], fb[0]);

  constexpr int kReads = MB + NB, kMfma = MB * NB;
  // the next sub-step's fragment reads go one after every kMfmaPerRead MFMAs
  // (where there are MFMAs enough), the step's loads between the MFMAs after
  // them; slabs with fewer MFMAs than reads (one 16-row block) leave the
  // order to the compiler
  constexpr bool kSched = kMfma > kReads;
  constexpr int kMfmaPerRead = kSched && QKNORM_PROJ_MPR * kReads < kMfma ? QKNORM_PROJ_MPR : 1;
  constexpr int kFreeMfma = kSched ? kMfma - kReads * kMfmaPerRead : 1;
  constexpr int kLoadsPerMfma = (G::kLoads + kFreeMfma - 1) / kFreeMfma;
  uint32_t cur = 0;                             // the stage of step ks (S > 2)
  for (uint32_t ks = 0; ks < ksteps; ++ks) {
    const uint32_t nxt = cur + 1 == (uint32_t)S ? 0 : cur + 1;
    uint8_t* const st = S == 2 ? ((ks & 1) ? stage1 : stage0) : stage(cur);
    uint8_t* const nx = S == 2 ? ((ks & 1) ? stage0 : stage1) : stage(nxt);
#pragma unroll
    for (int kk = 0; kk < KK - 1; ++kk) {
      read_frags<G, DT>(st, arow, brow, (kk + 1) * G::KS + fk, fa[(kk + 1) & 1], fb[(kk + 1) & 1]);
      mfma_step<G, DT>(acc, fa[kk & 1], fb[kk & 1]);
      if constexpr (kSched) {
        sched_interleave<kReads, 1, 0, kMfmaPerRead>();
        sched_mfmas<kMfma - kReads * kMfmaPerRead>();
      }
      __builtin_amdgcn_sched_barrier(0);
    }
    wait_vmcnt<(S - 2) * L>();                  // step ks+1 has landed (this wave)
    stage_barrier();                            // (and everyone's); stage st is free
    __builtin_amdgcn_sched_barrier(0);
    // the reads come first: the compiler cannot tell that the loads into
    // stage st do not overlap stage nx, so it keeps them in source order
    read_frags<G, DT>(nx, arow, brow, fk, fa[0], fb[0]);
    dma_tile<G>(ra, rb, doff, step_bytes<G>(ks + S, ksteps, shift), st, wave);
    mfma_step<G, DT>(acc, fa[1], fb[1]);
    if constexpr (kSched) {
      sched_interleave<kReads, 1, 0, kMfmaPerRead>();
      sched_interleave<kMfma - kReads * kMfmaPerRead, 0, kLoadsPerMfma>();
    }
    // keeps the reads above in this iteration: without it the compiler merges
    // them with the reads before the loop into one read at the top of the
    // loop, which then waits for its result before the first MFMA
    asm volatile("" ::: "memory");
    cur = nxt;
  }
  // the last step's spare loads into LDS must land before the block ends
  // (its LDS may then go to another block); waiting here, before the
  // stores, leaves the stores out of the wait
  wait_vmcnt<0>();
  proj_epilogue<G, DT, D>(acc, gtab, half, lane, wm, wn, m0, n0, a_rows, n_end, args.hq, args.hkv,
                          args.eps, args.inv_d, args.norm, args.out, args.ld_bytes);
}

// Blocks 0 .. n_full-1 take full tiles (GF) of columns [0, n_split); the rest
// take half-width tiles (GH) of columns [n_split, N).  The half-width tail
// lets a launch fill whole rounds of the chip's CUs where full tiles alone
// would leave a round half empty (384 tiles on 256 CUs at T = 4096).
template <class GF, class GH, int DT, int D>
__global__ __launch_bounds__(GF::kThreads) void qkv_proj_kernel(ProjKArgs args, uint32_t n_full,
                                                                uint32_t n_split) {
  static_assert(GF::kThreads == GH::kThreads, "one block size");
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
  constexpr int kStages = GF::kStagesBytes > GH::kStagesBytes ? GF::kStagesBytes : GH::kStagesBytes;
  float* gtab = reinterpret_cast<float*>(smem + kStages);
  float* half = gtab + kGammaFloats;
  // made visible by the first barrier of the tile's main loop
  stage_gamma<DT, D>(gtab, args.gamma_q, args.gamma_k, threadIdx.x);
  if (blockIdx.x < n_full) {
    proj_tile<GF, DT, D>(args, blockIdx.x, n_full, 0, n_split, smem, gtab, half);
  } else if constexpr (D <= GH::BN) {
    // a half-width tile holds whole heads, or one head across its two column
    // waves (head_dim 128); head_dim 256 never takes this path
    proj_tile<GH, DT, D>(args, blockIdx.x - n_full, gridDim.x - n_full, n_split, args.N, smem, gtab, half);
  }
}

// Small token counts through a workspace (T <= 64).  The tile kernel gives
// a head's D columns (64 rows of them) to one block, so a decode-size launch
// has one block per head (48 on a Qwen3-8B layer), each reading its whole
// weight panel at about 45 GB/s.  Here the weight is cut into 16 * JB columns by KS
// slices of K, one block of 4 waves each for all T tokens (TB blocks of 16),
// so that the whole chip streams it.  Each wave takes a quarter of its
// block's slice with the same MFMA (the weight's fragment first, fragments
// straight from global memory PF - 1 chunks ahead, none past the slice's
// end); the four waves' sums meet in LDS and are added in wave order; the
// block stores them as fp32 partials part[ks][t][n].  A second kernel, one
// block per head and 16 tokens, adds each output's KS partials in slice
// order, normalises the head's rows and stores them.  Rows past T read
// zeros and store nothing.  One kernel in which the last block of a head to
// finish did the norm was measured slower: with agent-scope release fences
// 5-20 times, and with the partials written and read through
// device-coherent stores and loads ahead of a counter still 15-25 %, since
// each block then waits for its writes to reach memory before its CU takes
// the next block.
template <int DT, int D, int KS, int JB, int TB, int PF>
__global__ __launch_bounds__(256) void qkv_proj_split_kernel(ProjKArgs args, float* __restrict__ part) {
  constexpr int CB = 16 * JB;                    // columns per block
  static_assert(D % CB == 0 && PF >= 2 && TB >= 1 && TB <= 4, "");
  __shared__ __attribute__((aligned(16))) float red[4][16 * TB][CB + 4];
  typedef typename ProjElem<DT>::V8 Frag;
  const uint32_t tid = threadIdx.x, lane = tid & 63, wave = uniform(tid >> 6);
  const uint32_t ks = blockIdx.x % KS, n0 = blockIdx.x / KS * CB;
  const uint32_t T = args.T, K = args.K, N = args.N;
  const uint32_t nk = K / 32;                    // 32-wide K chunks; the block takes [b0, b1)
  const uint32_t b0 = ks * nk / KS, b1 = (ks + 1) * nk / KS;
  const uint32_t c0 = b0 + wave * (b1 - b0) / 4, c1 = b0 + (wave + 1) * (b1 - b0) / 4;
  const uint32_t fr = lane % 16, fk = 8 * (lane / 16);
  const Rsrc rw = make_rsrc(args.w + (uint64_t)n0 * args.ldw_bytes, (uint64_t)(CB - 1) * args.ldw_bytes + K * 2);
  const Rsrc rx = make_rsrc(args.x, (uint64_t)(T - 1) * args.ldx_bytes + K * 2);
  const uint32_t wo = fr * args.ldw_bytes + fk * 2, xo = fr * args.ldx_bytes + fk * 2;
  f32x4 acc[TB][JB];
#pragma unroll
  for (int t = 0; t < TB; ++t)
#pragma unroll
    for (int j = 0; j < JB; ++j) acc[t][j] = f32x4{0.f, 0.f, 0.f, 0.f};
  {
    Frag wf[PF][JB], xf[PF][TB];
    auto load = [&](int p, uint32_t c) {
#pragma unroll
      for (int j = 0; j < JB; ++j)
        wf[p][j] = __builtin_bit_cast(
            Frag, __builtin_amdgcn_raw_buffer_load_b128(rw, wo + j * 16 * args.ldw_bytes, c * 64, 0));
#pragma unroll
      for (int t = 0; t < TB; ++t)
        xf[p][t] = __builtin_bit_cast(
            Frag, __builtin_amdgcn_raw_buffer_load_b128(rx, xo + t * 16 * args.ldx_bytes, c * 64, 0));
    };
#pragma unroll
    for (int p = 0; p < PF - 1; ++p)
      if (c0 + p < c1) load(p, c0 + p);
    for (uint32_t c = c0; c < c1; c += PF) {
#pragma unroll
      for (int p = 0; p < PF; ++p) {
        if (c + p + PF - 1 < c1) load((p + PF - 1) % PF, c + p + PF - 1);
        if (c + p < c1) {
#pragma unroll
          for (int t = 0; t < TB; ++t)
#pragma unroll
            for (int j = 0; j < JB; ++j) acc[t][j] = ProjElem<DT>::mfma(wf[p][j], xf[p][t], acc[t][j]);
        }
      }
    }
  }
#pragma unroll
  for (int t = 0; t < TB; ++t)
#pragma unroll
    for (int j = 0; j < JB; ++j)
      *reinterpret_cast<f32x4*>(&red[wave][16 * t + fr][16 * j + 4 * (lane / 16)]) = acc[t][j];
  __syncthreads();
#pragma unroll
  for (int m = 0; m < TB * JB; ++m) {
    const uint32_t i = tid + 256 * m, tok = i / CB, col = i % CB;
    if (tok < T)
      part[((uint64_t)ks * T + tok) * N + n0 + col] =
          ((red[0][tok][col] + red[1][tok][col]) + red[2][tok][col]) + red[3][tok][col];
  }
}

// One block per head and 16 tokens: 16 threads per token, E = D / 16
// consecutive columns each; the KS partials of a column are added in slice order, then the
// token's head is normalised (Q and K heads, unless plain) and stored.
template <int DT, int D, int KS>
__global__ __launch_bounds__(256) void qkv_proj_split_finish_kernel(ProjKArgs args,
                                                                     const float* __restrict__ part) {
  constexpr int E = D / 16;
  typedef typename ProjElem<DT>::T Elem;
  const uint32_t tid = threadIdx.x, head = blockIdx.x, tok = blockIdx.y * 16 + tid / 16, q = tid % 16;
  const uint32_t T = args.T, N = args.N, n = head * D + E * q;
  float v[E];
#pragma unroll
  for (int e = 0; e < E; ++e) v[e] = 0.f;
  if (tok < T) {
#pragma unroll
    for (int s = 0; s < KS; ++s) {
      const float* p = part + ((uint64_t)s * T + tok) * N + n;
#pragma unroll
      for (int e = 0; e < E; e += 4) {
        const f32x4 f = *reinterpret_cast<const f32x4*>(p + e);
#pragma unroll
        for (int i = 0; i < 4; ++i) v[e + i] += f[i];
      }
    }
  }
  if (args.norm && head < args.hq + args.hkv) {
    // every lane of a token's 16 takes part, rows past T with zeros
    const Elem* g = reinterpret_cast<const Elem*>(head < args.hq ? args.gamma_q : args.gamma_k) + E * q;
    float ss = 0.f;
#pragma unroll
    for (int e = 0; e < E; ++e) ss = __builtin_fmaf(v[e], v[e], ss);
    const float sc = rms_scale(group_sum<16>(ss), args.inv_d, args.eps);
#pragma unroll
    for (int e = 0; e < E; ++e) v[e] = (v[e] * (float)g[e]) * sc;
  }
  if (tok < T) {
    const Rsrc ro = make_rsrc(args.out + (uint64_t)head * D * 2, (uint64_t)(T - 1) * args.ld_bytes + D * 2);
    const uint32_t off = tok * (uint32_t)args.ld_bytes + q * E * 2;
    if constexpr (E == 4) {
      typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
      const u32x2 o = {pack2<DT>(v[0], v[1]), pack2<DT>(v[2], v[3])};
      __builtin_amdgcn_raw_buffer_store_b64(o, ro, off, 0, kStorePolicy);
    } else {
#pragma unroll
      for (int e = 0; e < E; e += 8) {
        const u32x4 o = {pack2<DT>(v[e], v[e + 1]), pack2<DT>(v[e + 2], v[e + 3]),
                         pack2<DT>(v[e + 4], v[e + 5]), pack2<DT>(v[e + 6], v[e + 7])};
        __builtin_amdgcn_raw_buffer_store_b128(o, ro, off + e * 2, 0, kStorePolicy);
      }
    }
  }
}

// 256 x 256 tiles of 8 waves (4 along M, 2 along N), each wave 64 x 128 as
// 4 x 8 blocks of 16 x 16: 12 fragment reads per 32 MFMAs and 131 flop per
// byte of operand staged, the best of the shapes measured on MI355X.  The
// others measured: 128 x 128 with 64 x 64 waves; 256 x 128 and 128 x 256
// with 4 waves; 256 x 256 with 4 waves of 128 x 128 (one wave per SIMD, 16
// reads per 64 MFMAs, the accumulators in AGPRs): the same time for the
// plain product and a slower norm epilogue; BK = 32 with three or four
// stages (more barriers outweigh the longer prefetch).  32 x 32 x 16 MFMAs do
// the same work from the same fragments but run the chip at a lower clock
// (about 9 % slower).  An L2 prefetch of later K steps (a 4-byte load per
// operand row) cost about 9 %: it doubles the vector-memory requests per
// step.  Operands staged through registers instead of loaded straight into
// LDS measured 11-17 % slower.  Reading fragments two sub-steps ahead,
// leaving the loads to one wave per SIMD, splitting a step's loads over two
// sub-steps, a persistent grid that loads the next tile during the
// epilogue, or a ping-pong schedule of two wave groups changed the time by
// 3 % or less, or made it slower.  Storing straight from registers (the
// swapped MFMA operands above) instead of through LDS saves about 3 %: the
// LDS round trip of the output tile cost about 6 us of 290 at T = 8192.
#ifndef QKNORM_PROJ_BK
#define QKNORM_PROJ_BK 64
#endif
#ifndef QKNORM_PROJ_SPLIT
#define QKNORM_PROJ_SPLIT 1        // 0: full tiles only
#endif
// Full tiles: 256 x 256, 8 waves of 64 x 128, two LDS stages (128 KiB).
// Half-width tiles: 256 x 128, 8 waves of 64 x 64, three stages (144 KiB, the
// kernel's LDS in either case): where a launch is all or mostly half-width
// tiles (513 to 1280 tokens on a Qwen3-8B layer) the third stage takes a
// quarter to a third off the time with the weight cold (52 against 73-75 us
// at 768 and 1024 tokens).
#ifndef QKNORM_PROJ_STAGES_H
#define QKNORM_PROJ_STAGES_H 3     // LDS stages of the half-width tiles
#endif
using GeoF = Tile<256, 256, 4, 2, QKNORM_PROJ_BK, 2>;
using GeoH = Tile<256, 128, 4, 2, QKNORM_PROJ_BK, QKNORM_PROJ_STAGES_H>;
constexpr bool kSplit = QKNORM_PROJ_SPLIT != 0;
constexpr int kBM = GeoF::BM, kBN = GeoF::BN, kThreads = GeoF::kThreads;
constexpr int kLdsBytes = (GeoF::kStagesBytes > GeoH::kStagesBytes ? GeoF::kStagesBytes : GeoH::kStagesBytes) +
                          (kGammaFloats + kHalfFloats) * 4;
static_assert(kLdsBytes <= 160 * 1024, "the stages fit a CU's 160 KiB of LDS");

}  // namespace

bool proj_shape_ok(const ProjArgs& a) {
  // buffer offsets inside one tile's rows stay below 2^31
  const uint64_t es = 2;
  return (uint64_t)kBM * a.ldx * es < (UINT64_C(1) << 31) &&
         (uint64_t)kBN * a.ldw * es < (UINT64_C(1) << 31) &&
         (uint64_t)kBM * a.ld * es < (UINT64_C(1) << 31) && a.hidden % 64 == 0 &&
         // the tiles (full or half-width) are numbered in one grid
         // dimension, whose size in threads must fit 32 bits
         (uint64_t)((a.T + kBM - 1) / kBM) *
                 (uint64_t)(((a.hq + 2 * a.hkv) * a.head_dim + GeoH::BN - 1) / GeoH::BN) *
                 (uint64_t)kThreads <
             (UINT64_C(1) << 32) &&
         (a.head_dim == 64 || a.head_dim == 128 || a.head_dim == 256);
}

// Where the half-width tail starts: the column n_split (a multiple of 256)
// that minimises the estimated time in rounds of the chip's CUs, a full tile
// costing 1 and a half-width tile kHalfCost; n_split = N means no tail.
// Head dims above 128 never split (a half-width tile would cut a head).
static uint32_t split_column(uint32_t T, uint32_t N, uint32_t head_dim, int cus) {
#ifndef QKNORM_PROJ_HALF_COST
#define QKNORM_PROJ_HALF_COST 0.6
#endif
  constexpr double kHalfCost = QKNORM_PROJ_HALF_COST;
  const uint64_t m_tiles = (T + kBM - 1) / kBM;
  const uint64_t c = cus > 0 ? (uint64_t)cus : 1;
  auto rounds = [&](uint64_t n) { return (double)((n + c - 1) / c); };
  const uint64_t all = m_tiles * ((N + kBN - 1) / kBN);
  uint32_t best = N;
  double best_cost = rounds(all);
  if (!kSplit || head_dim > (uint32_t)GeoH::BN) return best;
  for (uint32_t n1 = 0; n1 < N; n1 += kBN) {
    const uint64_t full = m_tiles * (n1 / kBN);
    const uint64_t half = m_tiles * ((N - n1 + GeoH::BN - 1) / GeoH::BN);
    const double cost = rounds(full) + kHalfCost * rounds(half);
    if (cost < best_cost - 1e-9) { best_cost = cost; best = n1; }
  }
  return best;
}

// The kernel arguments of one call (both kernels take them).
static ProjKArgs kernel_args(const ProjArgs& a) {
  ProjKArgs k;
  k.x = (const uint8_t*)a.x;
  k.w = (const uint8_t*)a.w;
  k.out = (uint8_t*)a.qkv;
  k.gamma_q = (const uint8_t*)a.gamma_q;
  k.gamma_k = (const uint8_t*)a.gamma_k;
  k.ld_bytes = (uint64_t)a.ld * 2;
  k.ldx_bytes = (uint32_t)(a.ldx * 2);
  k.ldw_bytes = (uint32_t)(a.ldw * 2);
  k.T = (uint32_t)a.T;
  k.K = (uint32_t)a.hidden;
  k.N = (uint32_t)((a.hq + 2 * a.hkv) * a.head_dim);
  k.hq = (uint32_t)a.hq;
  k.hkv = (uint32_t)a.hkv;
  k.norm = (uint32_t)((a.flags & 1) == 0);
  k.eps = a.eps;
  k.inv_d = 1.0f / (float)a.head_dim;
  return k;
}

#ifndef QKNORM_PROJ_SMALL_T
#define QKNORM_PROJ_SMALL_T 256    // token counts up to this take 64-row tiles
#endif
// 64-row tiles for small token counts: one head wide (or two heads of 64),
// 8 waves of 16 x 64 (a head of 128 spans the two column waves), or 256
// wide for head_dim 256.  Such a launch has few blocks (96 to 192 on a
// Qwen3-8B layer), each reading a whole weight panel, so what bounds it is
// the operand bytes one block keeps in flight: four LDS stages (96 KiB; three,
// 120 KiB, for head_dim 256) keep three K steps in flight.  With the weight
// cold in the Infinity Cache, 26-28 us from 17 to 256 tokens on that layer,
// against 50-52 us with two stages.
#ifndef QKNORM_PROJ_STAGES_S
#define QKNORM_PROJ_STAGES_S 4     // LDS stages of the 64-row tiles (3 at most for head_dim 256)
#endif
using GeoS = Tile<64, 128, 4, 2, 64, QKNORM_PROJ_STAGES_S>;
using GeoS256 = Tile<64, 256, 4, 2, 64, (QKNORM_PROJ_STAGES_S < 3 ? QKNORM_PROJ_STAGES_S : 3)>;

// One launch of geometry G (G256 for head_dim 256), every block a full tile.
template <class G, class G256>
static hipError_t launch_qkv_proj_tiles(const ProjArgs& a, hipStream_t s) {
  const uint32_t N = (uint32_t)((a.hq + 2 * a.hkv) * a.head_dim);
  const uint32_t m_tiles = (uint32_t)((a.T + G::BM - 1) / G::BM);
  const uint32_t bn = a.head_dim == 256 ? G256::BN : G::BN;
  const uint32_t tiles = m_tiles * ((N + bn - 1) / bn);
  auto kern = a.dtype == kF16
                  ? (a.head_dim == 64    ? qkv_proj_kernel<G, G, kF16, 64>
                     : a.head_dim == 128 ? qkv_proj_kernel<G, G, kF16, 128>
                                         : qkv_proj_kernel<G256, G256, kF16, 256>)
                  : (a.head_dim == 64    ? qkv_proj_kernel<G, G, kBF16, 64>
                     : a.head_dim == 128 ? qkv_proj_kernel<G, G, kBF16, 128>
                                         : qkv_proj_kernel<G256, G256, kBF16, 256>);
  const int lds = (a.head_dim == 256 ? G256::kStagesBytes : G::kStagesBytes) +
                  (kGammaFloats + kHalfFloats) * 4;
  static_assert(G::kStagesBytes + (kGammaFloats + kHalfFloats) * 4 <= 160 * 1024 &&
                    G256::kStagesBytes + (kGammaFloats + kHalfFloats) * 4 <= 160 * 1024,
                "the stages fit a CU's 160 KiB of LDS");
  const hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                           hipFuncAttributeMaxDynamicSharedMemorySize, lds);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(kern, dim3(tiles), dim3(G::kThreads), lds, s, kernel_args(a), tiles, N);
  return hipGetLastError();
}

// 128-row tiles for 257 to 512 tokens (and on while they fit one round of
// the CUs): one head wide, 8 waves of 32 x 64 (a head of 128 across the two
// column waves), or 256 wide for head_dim 256; four LDS stages (128 KiB;
// three, 144 KiB, for head_dim 256).  Weight cold: 36-37 us at 384 and 512
// tokens on the Qwen3-8B layer, against 57-58 us with two stages.
#ifndef QKNORM_PROJ_MID_T
#define QKNORM_PROJ_MID_T 512      // token counts up to this (above the 64-row range) take 128-row tiles
#endif
#ifndef QKNORM_PROJ_STAGES_M
#define QKNORM_PROJ_STAGES_M 4     // LDS stages of the 128-row tiles (3 at most for head_dim 256)
#endif
using GeoM = Tile<128, 128, 4, 2, 64, QKNORM_PROJ_STAGES_M>;
using GeoM256 = Tile<128, 256, 4, 2, 64, (QKNORM_PROJ_STAGES_M < 3 ? QKNORM_PROJ_STAGES_M : 3)>;

// The split geometry for a token count: KS slices of K, blocks of 16 * JB
// columns, TB blocks of 16 tokens.  Up to 8 tokens 16 columns by 4 slices
// (1536 blocks for the Qwen3-8B layer; with the norm kernel 12.1 us per
// call at T = 1 and 14.8 us at T = 8, against 12.2 and 14.9 us with 8
// slices); from 9 tokens 32 columns, which halves the activation fragments
// loaded per weight fragment (17.2 against 18.5 us at T = 16).  From 17
// tokens two or four token blocks share each weight fragment; K slices
// measured with the weight rotating through 6 copies: 8 slices 17.0, 18.0
// and 19.9 us at 17, 24 and 32 tokens (4 slices 17.6, 18.7, 19.8; 16 slices
// 18.2, 20.0, 21.9); 4 slices 23.4 and 25.8 us at 48 and 64 tokens (8
// slices 24.0 and 27.3; 2 slices 26.7 and 30.1).
#ifndef QKNORM_PROJ_SPLIT_KS32
#define QKNORM_PROJ_SPLIT_KS32 8   // K slices for 17 to 32 tokens
#endif
#ifndef QKNORM_PROJ_SPLIT_KS64
#define QKNORM_PROJ_SPLIT_KS64 4   // K slices for 33 to 64 tokens
#endif
struct SplitGeo {
  uint32_t ks, jb, tb;
};
static SplitGeo split_geo(int64_t T) {
  if (T <= 8) return SplitGeo{4, 1, 1};
  if (T <= 16) return SplitGeo{8, 2, 1};
  if (T <= 32) return SplitGeo{QKNORM_PROJ_SPLIT_KS32, 2, 2};
  return SplitGeo{QKNORM_PROJ_SPLIT_KS64, 2, 4};
}

int64_t proj_workspace_bytes(int64_t T, int64_t N) {
  if (T <= 0 || T > kProjSplitMaxT || N <= 0) return 0;
  const int64_t b = (int64_t)split_geo(T).ks * T * N * 4;
  return (b + 255) & ~(int64_t)255;
}

typedef void (*SplitKernel)(ProjKArgs, float*);
typedef void (*FinishKernel)(ProjKArgs, const float*);

template <int DT, int D>
static void split_kernels(const SplitGeo& g, SplitKernel* k1, FinishKernel* k2) {
  constexpr int S32 = QKNORM_PROJ_SPLIT_KS32, S64 = QKNORM_PROJ_SPLIT_KS64;
  if (g.tb == 1 && g.jb == 1) {
    *k1 = qkv_proj_split_kernel<DT, D, 4, 1, 1, 8>;
    *k2 = qkv_proj_split_finish_kernel<DT, D, 4>;
  } else if (g.tb == 1) {
    *k1 = qkv_proj_split_kernel<DT, D, 8, 2, 1, 4>;
    *k2 = qkv_proj_split_finish_kernel<DT, D, 8>;
  } else if (g.tb == 2) {
    *k1 = qkv_proj_split_kernel<DT, D, S32, 2, 2, 4>;
    *k2 = qkv_proj_split_finish_kernel<DT, D, S32>;
  } else {
    *k1 = qkv_proj_split_kernel<DT, D, S64, 2, 4, 4>;
    *k2 = qkv_proj_split_finish_kernel<DT, D, S64>;
  }
}

template <int DT>
static void split_kernels_dt(int head_dim, const SplitGeo& g, SplitKernel* k1, FinishKernel* k2) {
  if (head_dim == 64) split_kernels<DT, 64>(g, k1, k2);
  else if (head_dim == 128) split_kernels<DT, 128>(g, k1, k2);
  else split_kernels<DT, 256>(g, k1, k2);
}

hipError_t launch_qkv_proj_split(const ProjArgs& a, void* workspace, hipStream_t s) {
  const SplitGeo g = split_geo(a.T);
  const uint32_t N = (uint32_t)((a.hq + 2 * a.hkv) * a.head_dim);
  SplitKernel k1;
  FinishKernel k2;
  if (a.dtype == kF16) split_kernels_dt<kF16>(a.head_dim, g, &k1, &k2);
  else split_kernels_dt<kBF16>(a.head_dim, g, &k1, &k2);
  const ProjKArgs k = kernel_args(a);
  float* part = static_cast<float*>(workspace);
  hipLaunchKernelGGL(k1, dim3(N / (16 * g.jb) * g.ks), dim3(256), 0, s, k, part);
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(k2, dim3(N / (uint32_t)a.head_dim, (uint32_t)(a.T + 15) / 16), dim3(256), 0, s, k,
                     (const float*)part);
  return hipGetLastError();
}

// The split projection's partials for callers that cannot allocate a
// workspace: one array per GPU, held from the library's load until the
// process ends.  Host code never passes the array's name to a kernel (on the
// host it names a stand-in, not device memory); the device address comes
// from hipGetSymbolAddress, looked up once per device with that device
// current and kept per device.  Every such call on one GPU shares the array,
// so calls that can overlap on one GPU (different streams) race.  Nothing in
// it needs clearing between calls: the first kernel writes every partial the
// second one reads.
static __device__ __align__(256) uint8_t scratch[kProjScratchBytes];

static std::mutex g_scratch_mu;
static std::atomic<void*> g_scratch_ptr[kMaxScratchDevices];

hipError_t proj_scratch(void** ptr) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxScratchDevices) return hipErrorInvalidDevice;
  void* p = g_scratch_ptr[dev].load(std::memory_order_acquire);
  if (p == nullptr) {
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    p = g_scratch_ptr[dev].load(std::memory_order_relaxed);
    if (p == nullptr) {
      e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
      if (e != hipSuccess || p == nullptr) return e != hipSuccess ? e : hipErrorInvalidSymbol;
      g_scratch_ptr[dev].store(p, std::memory_order_release);
    }
  }
  *ptr = p;
  return hipSuccess;
}

hipError_t launch_qkv_proj(const ProjArgs& a, hipStream_t s, int cus) {
  if (a.T <= QKNORM_PROJ_SMALL_T) return launch_qkv_proj_tiles<GeoS, GeoS256>(a, s);
  const uint32_t N = (uint32_t)((a.hq + 2 * a.hkv) * a.head_dim);
  // 128-row tiles up to 512 tokens, and up to 1024 while they fit one round
  // of the chip's CUs (on a Qwen3-8B layer up to 640 tokens: 36 against 43 us
  // for the 256-row launch at 513 tokens, 60 against 52 us at 768, where a
  // second round would hold 32 tiles)
  const uint64_t bn_m = a.head_dim == 256 ? GeoM256::BN : GeoM::BN;
  const uint64_t m_tiles_m = (uint64_t)(a.T + GeoM::BM - 1) / GeoM::BM;
  if (a.T <= QKNORM_PROJ_MID_T ||
      (a.T <= 2 * QKNORM_PROJ_MID_T && m_tiles_m * ((N + bn_m - 1) / bn_m) <= (uint64_t)(cus > 0 ? cus : 1)))
    return launch_qkv_proj_tiles<GeoM, GeoM256>(a, s);
  const uint32_t T = (uint32_t)a.T;
  const uint32_t n_split = split_column(T, N, (uint32_t)a.head_dim, cus);
  const uint32_t m_tiles = (T + kBM - 1) / kBM;
  const uint32_t n_full = m_tiles * ((n_split + kBN - 1) / kBN);
  const uint32_t n_half = n_split < N ? m_tiles * ((N - n_split + GeoH::BN - 1) / GeoH::BN) : 0;
  auto pick = [&](auto k64, auto k128, auto k256) {
    return a.head_dim == 64 ? k64 : (a.head_dim == 128 ? k128 : k256);
  };
  auto kern = a.dtype == kF16
                  ? pick(qkv_proj_kernel<GeoF, GeoH, kF16, 64>, qkv_proj_kernel<GeoF, GeoH, kF16, 128>,
                         qkv_proj_kernel<GeoF, GeoH, kF16, 256>)
                  : pick(qkv_proj_kernel<GeoF, GeoH, kBF16, 64>, qkv_proj_kernel<GeoF, GeoH, kBF16, 128>,
                         qkv_proj_kernel<GeoF, GeoH, kBF16, 256>);
  // more than the default 64 KiB of dynamic LDS (gfx950 has 160 KiB per CU);
  // a host-side attribute, set on every call (no shared state between threads)
  const hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                           hipFuncAttributeMaxDynamicSharedMemorySize, kLdsBytes);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(kern, dim3(n_full + n_half), dim3(kThreads), kLdsBytes, s, kernel_args(a), n_full,
                     n_split);
  return hipGetLastError();
}

}  // namespace qknorm
