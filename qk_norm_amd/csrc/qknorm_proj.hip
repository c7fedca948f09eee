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
// output tile; each wave a 64 x 128 slab of 2 x 4 v_mfma_f32_32x32x16_bf16
// blocks (v_mfma_f32_32x32x16_f16 for fp16, the same layout).  K advances 64 at a time through two LDS stages filled straight
// from global memory (buffer loads into LDS, no staging registers), with
// the operand rows XOR-swizzled so that fragment reads hit distinct banks.
// Tiles are ordered so the blocks each XCD holds at once share operand
// panels in its L2.  Because the tile width is a multiple of head_dim and
// tiles start at multiples of it, a tile holds whole heads, and the epilogue
// normalises them in registers without leaving the block.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "qknorm_device.hpp"
#include "qknorm_launch.hpp"

namespace qknorm {

namespace {

typedef float f32x16 __attribute__((ext_vector_type(16)));

// The 16-bit element type: its 8-element fragment and the 32 x 32 x 16 MFMA
// that takes it (fp32 accumulation either way).
template <int DT>
struct ProjElem;
template <>
struct ProjElem<kBF16> {
  typedef __bf16 T;
  typedef __bf16 V8 __attribute__((ext_vector_type(8)));
  static __device__ __forceinline__ f32x16 mfma(V8 a, V8 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
  }
};
template <>
struct ProjElem<kF16> {
  typedef _Float16 T;
  typedef _Float16 V8 __attribute__((ext_vector_type(8)));
  static __device__ __forceinline__ f32x16 mfma(V8 a, V8 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
  }
};

// Tile geometry.  A block of WM x WN waves owns a BM x BN output tile; each
// wave a (BM/WM) x (BN/WN) slab of 32 x 32 MFMA blocks; K advances BK at a
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
  static constexpr int BM = BM_, BN = BN_, WM = WM_, WN = WN_, BK = BK_, S = S_;
  static constexpr int kThreads = 64 * WM * WN, kWaves = WM * WN;
  static constexpr int kWaveM = BM / WM, kWaveN = BN / WN;
  static constexpr int MB = kWaveM / 32, NB = kWaveN / 32;
  static constexpr int kRowBytes = BK * 2;
  static constexpr int CPR = kRowBytes / 16, RPB = 256 / kRowBytes;
  static constexpr int kInstRows = 1024 / kRowBytes;         // rows one load instruction fills
  static constexpr int kStageBytes = (BM + BN) * kRowBytes;
  static constexpr int kORow = BN + 8;
  static constexpr int kLdsBytes = S * kStageBytes > BM * kORow * 2 ? S * kStageBytes : BM * kORow * 2;
  static constexpr int kAInst = BM / kInstRows / kWaves, kBInst = BN / kInstRows / kWaves;
  static constexpr int kLoads = kAInst + kBInst;              // per wave per K step
  static_assert(BM % (kInstRows * kWaves) == 0 && BN % (kInstRows * kWaves) == 0, "");
  static_assert(RPB * CPR == 16, "a 256-byte line holds 16 chunks");
};

#ifndef QKNORM_PROJ_XCD
#define QKNORM_PROJ_XCD 1
#endif
#ifndef QKNORM_PROJ_GM
#define QKNORM_PROJ_GM 4
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
  constexpr int kInst = G::kAInst;
  static_assert(G::kAInst == G::kBInst, "as many A as B loads");
  const uint32_t sub = lane / kCpr, s = lane % kCpr;
  DmaOffsets<G> o;
#pragma unroll
  for (int j = 0; j < kInst; ++j) {
    const uint32_t r = (wave * kInst + j) * kRows + sub;
    o.a[j] = r * ldx_bytes + (s ^ ((r / kRpb) % kCpr)) * 16;
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
  constexpr int kInst = G::kAInst;
#pragma unroll
  for (int j = 0; j < kInst; ++j) {
    const uint32_t R = (wave * kInst + j) * kRows;
    const uint32_t va = o.a[j], vb = o.b[j];     // (locals: the host pass rejects members here)
    __builtin_amdgcn_raw_ptr_buffer_load_lds(
        ra, (__attribute__((address_space(3))) void*)(stage + R * kRowBytes), 16, va, k_bytes,
        0, 0);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(
        rb, (__attribute__((address_space(3))) void*)(stage + (kBM + R) * kRowBytes), 16, vb,
        k_bytes, 0, 0);
  }
}

template <class G, int DT>
__device__ __forceinline__ typename ProjElem<DT>::V8 sfrag(const uint8_t* base, uint32_t row, uint32_t k) {
  return *reinterpret_cast<const typename ProjElem<DT>::V8*>(base + row * G::kRowBytes +
                                                            lds_slot<G>(row, k / 8) * 16);
}

// Byte offset of K step k, or of the last step for k past it.
template <class G>
__device__ __forceinline__ uint32_t step_bytes(uint32_t k, uint32_t ksteps) {
  return (k < ksteps ? k : ksteps - 1) * G::BK * 2;
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
  for (int i = 0; i < G::MB; ++i) a[i] = sfrag<G, DT>(st, arow + i * 32, k);
#pragma unroll
  for (int j = 0; j < G::NB; ++j) b[j] = sfrag<G, DT>(st, brow + j * 32, k);
}

template <class G, int DT>
__device__ __forceinline__ void mfma_step(f32x16 (&acc)[G::MB][G::NB],
                                          const typename ProjElem<DT>::V8 (&a)[G::MB],
                                          const typename ProjElem<DT>::V8 (&b)[G::NB]) {
#pragma unroll
  for (int i = 0; i < G::MB; ++i)
#pragma unroll
    for (int j = 0; j < G::NB; ++j) acc[i][j] = ProjElem<DT>::mfma(a[i], b[j], acc[i][j]);
}

// Instruction order for the scheduler (sched_group_barrier masks: 0x008
// MFMA, 0x020 vector memory read, 0x100 LDS read).  One MFMA, then R LDS
// reads and V loads, NP times; then the remaining M MFMAs back to back.  With
// one wave per SIMD nothing else hides a read's latency, so the reads feeding
// the next sub-step go between this sub-step's MFMAs.
template <int NP, int R, int V>
__device__ __forceinline__ void sched_interleave() {
  if constexpr (NP > 0) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
    if constexpr (R > 0) __builtin_amdgcn_sched_group_barrier(0x100, R, 0);
    if constexpr (V > 0) __builtin_amdgcn_sched_group_barrier(0x020, V, 0);
    sched_interleave<NP - 1, R, V>();
  }
}

template <int M>
__device__ __forceinline__ void sched_mfmas() {
  if constexpr (M > 0) __builtin_amdgcn_sched_group_barrier(0x008, M, 0);
}

template <class G, int DT, int D>
__global__ __launch_bounds__(G::kThreads) void qkv_proj_kernel(
    const uint8_t* __restrict__ x, uint32_t ldx_bytes, const uint8_t* __restrict__ w,
    uint32_t ldw_bytes, uint8_t* __restrict__ out, uint64_t ld_bytes, uint32_t T, uint32_t K,
    uint32_t N, uint32_t hq, uint32_t hkv, const uint8_t* __restrict__ gamma_q,
    const uint8_t* __restrict__ gamma_k, float eps, float inv_d, uint32_t norm) {
  constexpr int MB = G::MB, NB = G::NB, BK = G::BK;
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
  const uint32_t tid = threadIdx.x, lane = tid & 63;
  const uint32_t wave = uniform(tid >> 6);
  const uint32_t wm = wave / G::WN, wn = wave % G::WN;
  // Tile order.  Workgroups go to the 8 XCDs round robin (id % 8), each XCD
  // with its own L2; the remap gives each XCD a contiguous run of tiles, and
  // the runs walk the output in bands of GM tile rows, columns outer, so the
  // blocks an XCD holds at once share a few A and B panels in its L2.
  const uint32_t n_tiles = (N + G::BN - 1) / G::BN, m_tiles = (T + G::BM - 1) / G::BM;
  uint32_t id = blockIdx.x;
  if (kXcdRemap) {
    const uint32_t q = gridDim.x / 8, r = gridDim.x % 8, xcd = id % 8;
    id = xcd * q + (xcd < r ? xcd : r) + id / 8;
  }
  const uint32_t band = id / (kGroupM * n_tiles), first_m = band * kGroupM;
  const uint32_t gm = m_tiles - first_m < kGroupM ? m_tiles - first_m : kGroupM;
  const uint32_t within = id - band * kGroupM * n_tiles;
  const uint32_t n0 = (within / gm) * G::BN, m0 = (first_m + within % gm) * G::BM;

  const uint32_t a_rows = T - m0 < (uint32_t)G::BM ? T - m0 : (uint32_t)G::BM;
  const uint32_t b_rows = N - n0 < (uint32_t)G::BN ? N - n0 : (uint32_t)G::BN;
  const Rsrc ra = make_rsrc(x + (uint64_t)m0 * ldx_bytes, (uint64_t)(a_rows - 1) * ldx_bytes + K * 2);
  const Rsrc rb = make_rsrc(w + (uint64_t)n0 * ldw_bytes, (uint64_t)(b_rows - 1) * ldw_bytes + K * 2);

  f32x16 acc[MB][NB];
#pragma unroll
  for (int i = 0; i < MB; ++i)
#pragma unroll
    for (int j = 0; j < NB; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.f;

  // Two LDS stages; K step ks computes from stage ks % 2.  Fragments are
  // double-buffered in registers: the reads of sub-step kk+1 are issued
  // before the MFMAs of sub-step kk.  Before the last sub-step of a step the
  // wave waits for its loads of step ks+1 (into the other stage) and meets
  // the barrier; after it, the stage just finished is free (every wave's
  // reads of it have completed), so the loads of step ks+2 go there, and the
  // first fragments of step ks+1 are read while the last MFMAs of step ks
  // run.  Loads past the last step fetch the last step again (unused).
  static_assert(G::S == 2 && BK % 32 == 0, "two stages, an even number of 16-wide sub-steps");
  constexpr int KK = BK / 16;
  const uint32_t ksteps = K / BK;
  // a lane's fragment: row (lane % 32) of a 32-row block, 8 consecutive k
  // starting at 8*(lane/32) of each 16-wide MFMA step; A and B use the same
  // k order, so the products pair correctly whatever order the hardware sums
  const uint32_t fr = lane % 32, fk = 8 * (lane / 32);
  const uint32_t arow = wm * G::kWaveM + fr, brow = G::BM + wn * G::kWaveN + fr;
  uint8_t* const stage0 = smem;
  uint8_t* const stage1 = smem + G::kStageBytes;

  const DmaOffsets<G> doff = dma_offsets<G>(ldx_bytes, ldw_bytes, wave, lane);
  dma_tile<G>(ra, rb, doff, step_bytes<G>(0, ksteps), stage0, wave);
  wait_vmcnt<0>();
  stage_barrier();
  dma_tile<G>(ra, rb, doff, step_bytes<G>(1, ksteps), stage1, wave);
  typedef typename ProjElem<DT>::V8 Frag;
  typedef typename ProjElem<DT>::T Elem;
  Frag fa[2][MB], fb[2][NB];
  read_frags<G, DT>(stage0, arow, brow, fk, fa[0], fb[0]);

  constexpr int kReads = MB + NB, kMfma = MB * NB;
  static_assert(kMfma > kReads && G::kLoads % (kMfma - kReads) == 0, "");
  for (uint32_t ks = 0; ks < ksteps; ++ks) {
    uint8_t* const st = (ks & 1) ? stage1 : stage0;
    uint8_t* const nx = (ks & 1) ? stage0 : stage1;
#pragma unroll
    for (int kk = 0; kk < KK - 1; ++kk) {
      read_frags<G, DT>(st, arow, brow, (kk + 1) * 16 + fk, fa[(kk + 1) & 1], fb[(kk + 1) & 1]);
      mfma_step<G, DT>(acc, fa[kk & 1], fb[kk & 1]);
      sched_interleave<kReads, 1, 0>();
      sched_mfmas<kMfma - kReads>();
      __builtin_amdgcn_sched_barrier(0);
    }
    wait_vmcnt<0>();                            // step ks+1 has landed (this wave)
    stage_barrier();                            // (and everyone's); stage st is free
    __builtin_amdgcn_sched_barrier(0);
    // the reads come first: the compiler cannot tell that the loads into
    // stage st do not overlap stage nx, so it keeps them in source order
    read_frags<G, DT>(nx, arow, brow, fk, fa[0], fb[0]);
    dma_tile<G>(ra, rb, doff, step_bytes<G>(ks + 2, ksteps), st, wave);
    mfma_step<G, DT>(acc, fa[1], fb[1]);
    sched_interleave<kReads, 1, 0>();
    sched_interleave<kMfma - kReads, 0, G::kLoads / (kMfma - kReads)>();
    // keeps the reads above in this iteration: without it the compiler merges
    // them with the reads before the loop into one read at the top of the
    // loop, which then waits for its result before the first MFMA
    asm volatile("" ::: "memory");
  }
  // the output tile reuses the stages: every load into LDS must be done
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();

  // Epilogue.  Value e of block (i, j) in lane l is row i*32 + 8*(e/4) +
  // 4*(l/32) + e%4 of the wave's slab and column j*32 + l%32.  A head of D
  // columns is D/32 consecutive blocks j (a wave's columns are whole heads):
  // its row sum of squares is the lane's fma chain over those blocks, then
  // the 32-lane sum of the half-wave that holds the row.
  constexpr int JH = D / 32;                    // blocks per head
  if (norm) {
    float g[NB];
    bool normed[NB];
#pragma unroll
    for (int j = 0; j < NB; ++j) {
      const uint32_t n = n0 + wn * G::kWaveN + j * 32 + lane % 32;
      const uint32_t head = n / D;
      const bool is_q = head < hq;
      normed[j] = (is_q || head < hq + hkv) && n < N;
      const Elem* gp = reinterpret_cast<const Elem*>(is_q ? gamma_q : gamma_k);
      g[j] = normed[j] ? (float)gp[n % D] : 1.f;
    }
    if constexpr (JH <= NB) {
      static_assert(NB % JH == 0, "a wave's columns must be whole heads");
#pragma unroll
      for (int i = 0; i < MB; ++i)
#pragma unroll
        for (int h = 0; h < NB / JH; ++h) {
          // the same for every lane and every block of one head (heads lie in
          // one region and the tile's columns past N are whole heads)
          if (!normed[h * JH]) continue;
#pragma unroll
          for (int e = 0; e < 16; ++e) {
            float s = 0.f;
#pragma unroll
            for (int jj = 0; jj < JH; ++jj)
              s = __builtin_fmaf(acc[i][h * JH + jj][e], acc[i][h * JH + jj][e], s);
            s = group_sum<32>(s);
            const float sc = rms_scale(s, inv_d, eps);
#pragma unroll
            for (int jj = 0; jj < JH; ++jj)
              acc[i][h * JH + jj][e] = (acc[i][h * JH + jj][e] * g[h * JH + jj]) * sc;
          }
        }
    } else {
      // a head spans the tile's two column waves (D = 2 * kWaveN): each wave
      // leaves its half-head row sums in LDS (the stages are free), and both
      // add the two halves in the same order, so they scale with the same bits
      static_assert(JH == 2 * NB && G::WN == 2 && G::BN == D, "one head across the two column waves");
      float* half = reinterpret_cast<float*>(smem);   // [WN][BM]
#pragma unroll
      for (int i = 0; i < MB; ++i)
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          float s = 0.f;
#pragma unroll
          for (int j = 0; j < NB; ++j) s = __builtin_fmaf(acc[i][j][e], acc[i][j][e], s);
          s = group_sum<32>(s);
          const uint32_t r = wm * G::kWaveM + i * 32 + 8 * (e / 4) + 4 * (lane / 32) + e % 4;
          if (lane % 32 == 0) half[wn * G::BM + r] = s;
        }
      __syncthreads();
      if (normed[0]) {
#pragma unroll
        for (int i = 0; i < MB; ++i)
#pragma unroll
          for (int e = 0; e < 16; ++e) {
            const uint32_t r = wm * G::kWaveM + i * 32 + 8 * (e / 4) + 4 * (lane / 32) + e % 4;
            const float sc = rms_scale(half[r] + half[G::BM + r], inv_d, eps);
#pragma unroll
            for (int j = 0; j < NB; ++j) acc[i][j][e] = (acc[i][j][e] * g[j]) * sc;
          }
      }
      __syncthreads();                           // the output staging reuses the LDS
    }
  }
  // the bf16 tile goes through LDS (the stages are free after the loop's last
  // barrier) so rows leave as 16-byte stores
  Elem* O = reinterpret_cast<Elem*>(smem);
#pragma unroll
  for (int i = 0; i < MB; ++i)
#pragma unroll
    for (int j = 0; j < NB; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const uint32_t r = wm * G::kWaveM + i * 32 + 8 * (e / 4) + 4 * (lane / 32) + e % 4;
        O[r * G::kORow + wn * G::kWaveN + j * 32 + lane % 32] = (Elem)acc[i][j][e];
      }
  __syncthreads();
  // one descriptor over the tile's rows (wave-uniform); rows past T and
  // columns past N get an offset outside it
  const uint32_t valid_cols = N - n0 < (uint32_t)G::BN ? N - n0 : (uint32_t)G::BN;
  const Rsrc ro = make_rsrc(out + (uint64_t)m0 * ld_bytes + (uint64_t)n0 * 2,
                            (uint64_t)(a_rows - 1) * ld_bytes + valid_cols * 2);
  constexpr uint32_t kCols = G::BN / 8;
  constexpr uint32_t kRowsPerPass = G::kThreads / kCols;
  for (uint32_t r0 = 0; r0 < (uint32_t)G::BM; r0 += kRowsPerPass) {
    const uint32_t r = r0 + tid / kCols, c = (tid % kCols) * 8;
    const u32x4 v = *reinterpret_cast<const u32x4*>(O + r * G::kORow + c);
    stream_store(ro, r < a_rows && c < valid_cols ? r * (uint32_t)ld_bytes + c * 2 : 0xFFFFFFF0u, v);
  }
}

// 256 x 256 tiles of 8 waves (4 along M, 2 along N), each wave 64 x 128:
// 0.75 fragment reads per MFMA and 131 flop per byte of operand staged, the
// best of the shapes measured on MI355X.  The others measured: 128 x 128 with
// 64 x 64 waves; 256 x 128 and 128 x 256 with 4 waves; 256 x 256 with 4
// waves of 128 x 128 (one wave per SIMD, 0.5 reads per MFMA, but about 7 %
// slower: with no second wave on the SIMD every latency shows); BK = 32 with
// three or four stages (more barriers outweigh the longer prefetch).  An L2
// prefetch of later K steps (a 4-byte load per operand row) cost about 9 %:
// it doubles the vector-memory requests per step.  4 waves of 128 x 128 with
// the operands staged through registers (global loads two steps ahead, two
// LDS stages) measured 11-17 % slower than this kernel.  Reading fragments two
// sub-steps ahead, accumulating in AGPRs, leaving the loads to one wave per
// SIMD, splitting a step's loads over two sub-steps (also with 4 waves of
// 128 x 128), an epilogue that stores from registers, or a persistent grid
// that loads the next tile during the epilogue changed the time by 3 % or
// less.
#ifndef QKNORM_PROJ_BK
#define QKNORM_PROJ_BK 64
#endif
#ifndef QKNORM_PROJ_WM
#define QKNORM_PROJ_WM 4
#endif
#ifndef QKNORM_PROJ_WN
#define QKNORM_PROJ_WN 2
#endif
using Geo = Tile<256, 256, QKNORM_PROJ_WM, QKNORM_PROJ_WN, QKNORM_PROJ_BK, 2>;
constexpr int kBM = Geo::BM, kBN = Geo::BN, kThreads = Geo::kThreads;
constexpr int kLdsBytes = Geo::kLdsBytes;

}  // namespace

bool proj_shape_ok(const ProjArgs& a) {
  // buffer offsets inside one tile's rows stay below 2^31
  const uint64_t es = 2;
  return (uint64_t)kBM * a.ldx * es < (UINT64_C(1) << 31) &&
         (uint64_t)kBN * a.ldw * es < (UINT64_C(1) << 31) &&
         (uint64_t)kBM * a.ld * es < (UINT64_C(1) << 31) && a.hidden % 64 == 0 &&
         // the tiles are numbered in one grid dimension, whose size in
         // threads must fit 32 bits
         (uint64_t)((a.T + kBM - 1) / kBM) * (uint64_t)(((a.hq + 2 * a.hkv) * a.head_dim + kBN - 1) / kBN) *
                 (uint64_t)kThreads <
             (UINT64_C(1) << 32) &&
         (a.head_dim == 64 || a.head_dim == 128 || a.head_dim == 256);
}

hipError_t launch_qkv_proj(const ProjArgs& a, hipStream_t s) {
  const uint32_t N = (uint32_t)((a.hq + 2 * a.hkv) * a.head_dim);
  const dim3 grid((uint32_t)(((N + kBN - 1) / kBN) * ((a.T + kBM - 1) / kBM)));
  auto pick = [&](auto k64, auto k128, auto k256) {
    return a.head_dim == 64 ? k64 : (a.head_dim == 128 ? k128 : k256);
  };
  auto kern = a.dtype == kF16 ? pick(qkv_proj_kernel<Geo, kF16, 64>, qkv_proj_kernel<Geo, kF16, 128>,
                                     qkv_proj_kernel<Geo, kF16, 256>)
                              : pick(qkv_proj_kernel<Geo, kBF16, 64>, qkv_proj_kernel<Geo, kBF16, 128>,
                                     qkv_proj_kernel<Geo, kBF16, 256>);
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
