// gfx950 kernels for QK-Norm on fused QKV rows, and their launchers.
//
// All kernels are HBM-bound streams: every Q/K element is read once with a
// 16-byte vector load, reduced in fp32 registers, scaled and written back in
// place with a 16-byte store.  V columns are never addressed.
#include "qknorm_device.hpp"
#include "qknorm_launch.hpp"

#ifndef QKNORM_PH_THREADS
#define QKNORM_PH_THREADS 512      // threads per per-head block (16- and 32-bit heads)
#endif
#ifndef QKNORM_PH_UNROLL
#define QKNORM_PH_UNROLL 2         // heads per lane group per loop trip
#endif
#ifndef QKNORM_PH_BLOCKS_PER_CU
#define QKNORM_PH_BLOCKS_PER_CU 160 // per-head grid cap, blocks per CU (one trip for most sizes)
#endif
#ifndef QKNORM_PH_WAVES_PER_CU_FP8
#define QKNORM_PH_WAVES_PER_CU_FP8 (QKNORM_PH_BLOCKS_PER_CU * QKNORM_PH_THREADS / 64)
#endif
#ifndef QKNORM_LW_WAVES_PER_CU
#define QKNORM_LW_WAVES_PER_CU 512   // layerwise grid cap, waves per CU
#endif

namespace qknorm {

// =================================================================== per head
//
// A head of D values is LPH lanes x 16 bytes (bf16 D=128: 16 lanes, one DPP
// row).  The heads are split into two regions, the Q heads of every row and
// the K heads of every row; a block works in one region only, so each wave
// has a single, uniform gamma.  Inside a region, heads are numbered
// g = t*H + h (H heads per row), a wave covers 64/LPH consecutive heads per
// step and U steps per trip, and (t, h) are kept incrementally, so the loop
// has no integer division.

#ifndef QKNORM_PH_GAMMA_SGPR
#define QKNORM_PH_GAMMA_SGPR 1
#endif
static constexpr bool kGammaSgpr = QKNORM_PH_GAMMA_SGPR != 0;
// FP8 heads do about three times the vector work of bf16 heads per byte, and
// the per-wave gamma hand-out above is a large share of it: FP8 kernels stage
// gamma in LDS instead (scalar loads, one lane per wave, one barrier) and take
// one head per lane group per trip.  On the standalone [4096, 48, 128] FP8
// tensor: 10.24 us with the hand-out and two heads, 9.67 us this way (bf16
// heads measured slower with the LDS staging, 16.95 against 16.53 us).
#ifndef QKNORM_PH_GAMMA_LDS_FP8
#define QKNORM_PH_GAMMA_LDS_FP8 1
#endif
static constexpr bool kFp8GammaLds = QKNORM_PH_GAMMA_LDS_FP8 != 0;
#ifndef QKNORM_PH_UNROLL_FP8
#define QKNORM_PH_UNROLL_FP8 1
#endif
#ifndef QKNORM_PH_THREADS_FP8
#define QKNORM_PH_THREADS_FP8 256  // FP8 heads: smaller blocks measured faster
#endif

// Heads per lane group per loop trip.
template <int DT>
constexpr int ph_unroll() { return DT == kFP8 ? QKNORM_PH_UNROLL_FP8 : QKNORM_PH_UNROLL; }

// Threads per per-head block.
template <int DT>
constexpr int ph_threads() { return DT == kFP8 ? QKNORM_PH_THREADS_FP8 : QKNORM_PH_THREADS; }

// A workgroup barrier after this wave's LDS accesses have completed, with no
// wait for its outstanding vector-memory loads (__syncthreads() would wait for
// every one of them, including the row loads meant to stay in flight).  The
// "memory" clobber keeps the compiler from moving memory accesses across it.
__device__ __forceinline__ void lds_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// The N = 4*GV*LPH gamma dwords of a head (GV 16-byte gamma vectors per
// activation vector), read at uniform addresses (scalar loads); lane group
// `sub` then keeps dwords N/LPH*sub .. N/LPH*(sub+1)-1.  `out` starts at zero.
template <int DT, int LPH>
__device__ __forceinline__ void gamma_to_lanes(const uint32_t* __restrict__ g, uint32_t sub,
                                               Gam<DT>& out) {
  constexpr int GV = Gam<DT>::kVecs;
  uint32_t w[4 * GV * LPH];
#pragma unroll
  for (int k = 0; k < 4 * GV * LPH; ++k) w[k] = g[k];   // all loads first (batched scalar loads)
#pragma unroll
  for (uint32_t j = 0; j < LPH; ++j) {
    const uint32_t mask = 0u - (uint32_t)(sub == j);  // all ones in lane group j
#pragma unroll
    for (int q = 0; q < GV; ++q)
#pragma unroll
      for (int i = 0; i < 4; ++i) out.v[q][i] |= w[(j * GV + q) * 4 + i] & mask;
  }
}

// Division by a divisor d fixed for the launch (1 <= d < 2^31), for
// dividends below 2^31, as a multiply and a shift (Granlund and Montgomery,
// "Division by invariant integers using multiplication", 1994): with
// l = ceil(log2 d) and m = ceil(2^(31+l) / d) (below 2^32),
// floor(n / d) = floor(m * n / 2^(31+l)).  The hardware has no integer
// divide, and the generic sequence sits ahead of every wave's first load.
struct FastDiv {
  uint32_t m, sh;
  __device__ __forceinline__ uint32_t div(uint32_t n) const {
    return (uint32_t)(((uint64_t)m * n) >> sh);
  }
};

static inline FastDiv make_fastdiv(uint32_t d) {
  uint32_t l = 0;
  while ((UINT64_C(1) << l) < d) ++l;
  const uint64_t p = UINT64_C(1) << (31 + l);
  return FastDiv{(uint32_t)((p + d - 1) / d), 31 + l};
}

// The same method for 64-bit dividends below 2^40 (divisor 1 <= d < 2^31):
// m = ceil(2^(40+l) / d) <= 2^41 and floor(n / d) = floor(m * n / 2^(40+l)),
// the product (below 2^81) taken as its high and low 64-bit words.
struct FastDiv40 {
  uint64_t m;
  uint32_t sh;
  __device__ __forceinline__ uint32_t div(uint64_t n) const {
    const uint64_t hi = __umul64hi(m, n), lo = m * n;
    return (uint32_t)(sh >= 64 ? hi >> (sh - 64) : (hi << (64 - sh)) | (lo >> sh));
  }
};

static constexpr uint64_t kFastDiv40Limit = UINT64_C(1) << 40;

static inline FastDiv40 make_fastdiv40(uint32_t d) {
  uint32_t l = 0;
  while ((UINT64_C(1) << l) < d) ++l;
  const unsigned __int128 p = (unsigned __int128)1 << (40 + l);
  return FastDiv40{(uint64_t)((p + d - 1) / d), 40 + l};
}

// One region of heads: H per row, starting `col_bytes` into each row, with
// its gamma; `blocks` blocks of the grid, which advance (stride_rows,
// stride_heads) per trip.
struct PhRegion {
  const uint8_t* gamma;
  uint32_t H;
  uint32_t col_bytes;
  uint32_t blocks;
  uint32_t stride_rows, stride_heads;
  FastDiv byH;              // division by H
};

// Addresses of one trip: U heads per lane group starting at the wave's head
// (tw, hw) of the region.  CONTIG: rows hold just this region's heads, back
// to back, so the heads form one flat array (tw = 0, hw = flat index).
// A head is hv 16-byte vectors (hb = 16*hv bytes); the group has LPH >= hv
// lanes and lanes sub >= hv hold no part of it.
//
// Loads and stores are issued unconditionally (straight-line code, so the
// compiler can keep the next trip's loads in flight while this trip is being
// computed).  The descriptor spans exactly the bytes this trip may touch; a
// lane without a head gets an offset past that span, and a trip past the end
// of the tensor gets an empty descriptor, so the hardware range check turns
// those accesses into no-ops (loads return 0, stores are dropped).  Every
// span is below 2^31 bytes: per_head_span_ok() checks the largest one on the
// host before any launch.
template <int LPH, int U, bool CONTIG>
struct PerHeadTrip {
  Rsrc rs;
  uint32_t off[U];

  static constexpr uint32_t kNoHead = 0xFFFFFFF0u;

  __device__ __forceinline__ void setup(uint8_t* qkv, uint32_t ld_bytes, uint32_t T, uint32_t H,
                                        FastDiv byH, uint32_t col_bytes, bool live, uint32_t tw,
                                        uint32_t hw, uint32_t sub, uint32_t grp, uint32_t hv) {
    constexpr uint32_t HPW = 64 / LPH;
    constexpr uint32_t CH = HPW * U;
    const uint32_t head_bytes = hv * 16;
    const bool mine = sub < hv;              // this lane holds part of its head
    tw = live ? tw : 0;
    hw = live ? hw : 0;
    uint64_t first, rest, span;
    if constexpr (CONTIG) {
      first = (uint64_t)hw * head_bytes;
      rest = ((uint64_t)T * H - hw) * head_bytes;
      span = (uint64_t)CH * head_bytes;
    } else {
      // from the wave's first head to the end of the region in the last row
      first = (uint64_t)tw * ld_bytes + col_bytes;
      rest = (uint64_t)(T - 1 - tw) * ld_bytes + (uint64_t)H * head_bytes;
      span = (uint64_t)byH.div(hw + CH - 1) * ld_bytes + (uint64_t)H * head_bytes;
    }
    rs = make_rsrc(qkv + first, live ? (span < rest ? span : rest) : 0);
#pragma unroll
    for (uint32_t u = 0; u < U; ++u) {
      const uint32_t k = u * HPW + grp;      // head index from the wave's first head
      if constexpr (CONTIG) {
        off[u] = mine && hw + k < T * H ? k * head_bytes + sub * 16 : kNoHead;
      } else {
        uint32_t hu = hw + k, dt = 0;
        if (hu >= H) {                       // wrap into the following row(s)
          dt = byH.div(hu);
          hu -= dt * H;
        }
        off[u] = mine && tw + dt < T ? dt * ld_bytes + hu * head_bytes + sub * 16 : kNoHead;
      }
    }
  }
};

template <int DT, int LPH, int U>
__device__ __forceinline__ void per_head_apply(const u32x4 (&v)[U], const float (&g)[IoTraits<DT>::kElems],
                                               float inv_d, float eps, bool may_exceed, Rsrc rs,
                                               const uint32_t (&off)[U]) {
  using IO = IoTraits<DT>;
  constexpr int E = IO::kElems;
#pragma unroll
  for (uint32_t u = 0; u < U; ++u) {
    float x[E];
    unpack<DT>(v[u], x);
    const float s = group_sum<LPH>(vec_sumsq<DT>(x, 0.f));
    const float r = rms_scale(s, inv_d, eps);
    float y[E];
#pragma unroll
    for (int e = 0; e < E; ++e) y[e] = (x[e] * g[e]) * r;
    stream_store(rs, off[u], pack<DT>(y, may_exceed));
  }
}

// ONE: the grid covers every head in one trip, so there is no loop.
// Otherwise the loop is software-pipelined: the next trip's loads are issued
// before the current trip's reduction and stores.
// EXACT: a head is exactly LPH vectors (a power of two); otherwise it is
// hvec < LPH vectors and the group's last LPH - hvec lanes stay idle.
template <int DT, int LPH, int U, bool CONTIG, bool ONE, bool EXACT, bool TWO>
__global__ __launch_bounds__(ph_threads<DT>()) void per_head_kernel(
    uint8_t* __restrict__ qkv, uint32_t ld_bytes, uint32_t T, PhRegion r0, PhRegion r1, FastDiv40 byN,
    float eps, float inv_d, uint32_t hvec) {
  using IO = IoTraits<DT>;
  using Trip = PerHeadTrip<LPH, U, CONTIG>;
  constexpr int E = IO::kElems;
  constexpr uint32_t CH = (64 / LPH) * U;    // heads per wave per trip
  const uint32_t hv = EXACT ? (uint32_t)LPH : hvec;
  const uint32_t lane = threadIdx.x & 63;
  const uint32_t sub = lane % LPH;           // 16-byte slot inside the head
  const uint32_t grp = lane / LPH;           // head slot inside the wave step

  // This block's region (uniform).  TWO: both regions are present, and
  // their blocks are interleaved in proportion (Bresenham): among blocks
  // 0..b, c(b) = floor((b+1) * blocks1 / N) belong to region 1, so block b is
  // region 1's block c(b-1) when c(b) > c(b-1), else region 0's block
  // b - c(b).  Q and K heads of the same rows then stream at the same time:
  // all Q blocks before all K blocks measured 11 % slower on fused GQA rows.
  // byN.m == 0: the regions' blocks follow one another.
  static_assert(!(CONTIG && TWO), "a flat array of heads is a single region");
  bool second;
  uint32_t lblock;
  // (Single-region kernels keep the run-time test, which they always pass:
  // folding it away at compile time measured 2.7 % slower on the standalone
  // [4096, 48, 128] kernel, with nothing else in the code changed.)
  if (!TWO || byN.m == 0) {
    second = blockIdx.x >= r0.blocks;
    lblock = blockIdx.x - (second ? r0.blocks : 0);
  } else {
    const uint32_t c0 = byN.div((uint64_t)blockIdx.x * r1.blocks);
    const uint32_t c1 = byN.div((uint64_t)(blockIdx.x + 1) * r1.blocks);
    second = c1 > c0;
    lblock = second ? c0 : blockIdx.x - c1;
  }
  const uint8_t* gamma = second ? r1.gamma : r0.gamma;
  const uint32_t H = second ? r1.H : r0.H;
  const uint32_t col = second ? r1.col_bytes : r0.col_bytes;
  const uint32_t stride_rows = second ? r1.stride_rows : r0.stride_rows;
  const uint32_t stride_heads = second ? r1.stride_heads : r0.stride_heads;
  const FastDiv byH = second ? r1.byH : r0.byH;

  // (tw, hw): row and head of the wave's first head this trip (wave-uniform).
  // T*H < 2^31 is checked on the host, so 32-bit arithmetic suffices.
  const uint32_t wave = uniform(lblock * (blockDim.x >> 6) + (threadIdx.x >> 6));
  const uint32_t g0 = wave * CH;
  const bool live = g0 < T * H;
  uint32_t tw = CONTIG || !live ? 0 : byH.div(g0);
  uint32_t hw = CONTIG ? g0 : (live ? g0 - tw * H : 0);

  // first trip's loads go out before any gamma work
  Trip cur;
  u32x4 vc[U];
  cur.setup(qkv, ld_bytes, T, H, byH, col, live, tw, hw, sub, grp, hv);
#pragma unroll
  for (uint32_t u = 0; u < U; ++u) vc[u] = stream_load(cur.rs, cur.off[u]);
  __builtin_amdgcn_sched_barrier(0);           // keep the row loads ahead of the gamma work

  // gamma: a vector load of the same few lines by every wave of the grid
  // makes those lines an L2 hot spot.  Heads with at most 64 dwords of gamma
  // read the region's gamma with scalar loads through the scalar cache and
  // hand each lane its dwords with selects, which run while the row loads are
  // in flight; longer ones, and heads that do not fill their lane group (the
  // scalar loads would read past gamma), stage it once per block in LDS.
  constexpr int GV = Gam<DT>::kVecs;
  float g[E];
  if constexpr (kGammaSgpr && EXACT && 4 * GV * LPH <= 64 && DT == kFP8 && kFp8GammaLds) {
    // the head's LPH*GV 16-byte gamma chunks: chunk c comes from wave
    // c % waves, through its scalar cache and one lane, into LDS
    constexpr uint32_t kChunks = LPH * GV, kWaves = ph_threads<DT>() / 64;
    __shared__ u32x4 g_lds[kChunks];
    const uint32_t wv = threadIdx.x >> 6;
    const uint32_t* g32 = reinterpret_cast<const uint32_t*>(gamma);
#pragma unroll
    for (uint32_t c0 = 0; c0 < kChunks; c0 += kWaves) {
      const uint32_t c = uniform(c0 + wv);
      if (c < kChunks) {
        const u32x4 v = {g32[4 * c], g32[4 * c + 1], g32[4 * c + 2], g32[4 * c + 3]};
        if (lane == 0) g_lds[c] = v;
      }
    }
    lds_barrier();
    Gam<DT> w;
#pragma unroll
    for (int q = 0; q < GV; ++q) w.v[q] = g_lds[sub * GV + q];
    unpack_gamma<DT>(w, g);
  } else if constexpr (kGammaSgpr && EXACT && 4 * GV * LPH <= 64) {
    Gam<DT> w = zero_gamma<DT>();
    gamma_to_lanes<DT, LPH>(reinterpret_cast<const uint32_t*>(gamma), sub, w);
    unpack_gamma<DT>(w, g);
  } else {
    __shared__ u32x4 g_lds[LPH * GV];
    if (threadIdx.x < LPH * GV)
      g_lds[threadIdx.x] = threadIdx.x < hv * GV ? load16(gamma + threadIdx.x * 16)
                                                 : u32x4{0, 0, 0, 0};
    __syncthreads();
    Gam<DT> w;
#pragma unroll
    for (int q = 0; q < GV; ++q) w.v[q] = g_lds[sub * GV + q];
    unpack_gamma<DT>(w, g);
  }
  // FP8: whether this wave's outputs can leave the E4M3 range (all lanes
  // take part in the ballot, so before the early exit)
  bool may_exceed = true;
  if constexpr (DT == kFP8) may_exceed = e4m3_may_exceed(abs_max<E>(g, 0.f), inv_d);
  if (!live) return;

  if constexpr (ONE) {
    per_head_apply<DT, LPH, U>(vc, g, inv_d, eps, may_exceed, cur.rs, cur.off);
    return;
  }
  while (true) {
    // next trip: advance by the region's part of the grid
    uint32_t tn = tw + stride_rows, hn = hw + stride_heads;
    if (!CONTIG && hn >= H) { hn -= H; ++tn; }
    const bool more = CONTIG ? hn < T * H : tn < T;
    Trip nxt;
    u32x4 vn[U];
    nxt.setup(qkv, ld_bytes, T, H, byH, col, more, tn, hn, sub, grp, hv);
#pragma unroll
    for (uint32_t u = 0; u < U; ++u) vn[u] = stream_load(nxt.rs, nxt.off[u]);
    per_head_apply<DT, LPH, U>(vc, g, inv_d, eps, may_exceed, cur.rs, cur.off);
    if (!more) break;
    cur = nxt;
#pragma unroll
    for (uint32_t u = 0; u < U; ++u) vc[u] = vn[u];
    tw = tn;
    hw = hn;
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
  float inv_wq, inv_wk;         // 1 / full widths (fp32)
};

__device__ __forceinline__ float combine(const float* __restrict__ p, uint32_t n, int64_t stride) {
  float s = 0.f;
  for (uint32_t r = 0; r < n; ++r) s += p[(int64_t)r * stride];
  return s;
}

// The same sums for the Q and K partials of one row read from global memory
// (a caller's [nparts][T] arrays, column t): the loads go out eight shards at
// a time for both regions, so a row waits for one memory round trip per
// eight shards instead of one per shard, and the adds still take the shards
// in order, ((p0 + p1) + p2) + ..., the bits of combine().  Both pointers
// must be readable: a caller without one region passes the other's.
__device__ __forceinline__ void combine_cols(const float* __restrict__ p, const float* __restrict__ q,
                                             uint32_t n, int64_t stride, float* sp, float* sq) {
  constexpr uint32_t kBatch = 8;
  float a = 0.f, b = 0.f;
  uint32_t r = 0;
  for (; r + kBatch <= n; r += kBatch) {
    float u[kBatch], v[kBatch];
#pragma unroll
    for (uint32_t i = 0; i < kBatch; ++i) {
      u[i] = p[(int64_t)(r + i) * stride];
      v[i] = q[(int64_t)(r + i) * stride];
    }
#pragma unroll
    for (uint32_t i = 0; i < kBatch; ++i) {
      a += u[i];
      b += v[i];
    }
  }
  for (; r < n; ++r) {
    a += p[(int64_t)r * stride];
    b += q[(int64_t)r * stride];
  }
  *sp = a;
  *sq = b;
}

// Two such sums side by side (the Q and K partials of one row), each in the
// same order as combine(): both regions' reads go out together, so a row
// waits for one round of LDS reads instead of two.
__device__ __forceinline__ void combine2(const float* __restrict__ p, const float* __restrict__ q,
                                         uint32_t n, float* sp, float* sq) {
  float a = 0.f, b = 0.f;
  for (uint32_t r = 0; r < n; ++r) {
    a += p[r];
    b += q[r];
  }
  *sp = a;
  *sq = b;
}

// --- register-resident slots (fused kernel, MODE 0) -------------------------
//
// Slot j of a lane is shard wave + (j / trips)*nw, vector lane + (j % trips)*64.
// The slot loops are fully unrolled so the kept vectors stay in VGPRs.

template <int DT, int VPL>
struct Slots {
  u32x4 x[VPL];
  Gam<DT> g[VPL];
};

constexpr uint32_t kOutOfRange = 0xFFFFFFF0u;

// Straight-line buffer loads (cached policy); an empty slot reads zeros
// through an offset past the descriptor.
template <int DT, int VPL>
__device__ __forceinline__ void slots_load_gamma(const uint8_t* __restrict__ gamma, uint32_t svecs,
                                                 uint32_t R, uint32_t wave, uint32_t nw,
                                                 uint32_t lane, Slots<DT, VPL>& S) {
  constexpr uint32_t GV = Gam<DT>::kVecs;
  const Rsrc gr = make_rsrc(gamma, (uint64_t)R * svecs * GV * 16);
  const uint32_t trips = (svecs + 63) / 64;
  uint32_t i = 0, k = 0;
#pragma unroll
  for (int j = 0; j < VPL; ++j) {
    const uint32_t r = wave + i * nw, v = lane + k * 64;
    const bool ok = r < R && v < svecs;
#pragma unroll
    for (uint32_t q = 0; q < GV; ++q)
      S.g[j].v[q] = cached_load(gr, ok ? ((r * svecs + v) * GV + q) * 16 : kOutOfRange);
    if (++k == trips) { k = 0; ++i; }
  }
}

// Largest |gamma| over a lane's slots (its zero slots included).
template <int DT, int VPL>
__device__ __forceinline__ float slots_gamma_max(const Slots<DT, VPL>& S) {
  float m = 0.f;
#pragma unroll
  for (int j = 0; j < VPL; ++j) {
    float g[IoTraits<DT>::kElems];
    unpack_gamma<DT>(S.g[j], g);
    m = abs_max(g, m);
  }
  return m;
}

// Loads are unconditional (an invalid slot gets an offset past the row's
// descriptor and reads 0), so a whole row's loads can stay in flight while the
// previous row is being reduced.

template <int DT, int VPL>
__device__ __forceinline__ void slots_load(Rsrc rs, uint32_t reg_off, uint32_t svecs, uint32_t R,
                                           uint32_t wave, uint32_t nw, uint32_t lane,
                                           Slots<DT, VPL>& S) {
  const uint32_t trips = (svecs + 63) / 64;
  uint32_t i = 0, k = 0;
#pragma unroll
  for (int j = 0; j < VPL; ++j) {
    const uint32_t r = wave + i * nw, v = lane + k * 64;
    S.x[j] = stream_load(rs, (r < R && v < svecs) ? reg_off + (r * svecs + v) * 16 : kOutOfRange);
    if (++k == trips) { k = 0; ++i; }
  }
}

template <int DT, int VPL>
__device__ __forceinline__ void slots_partials(uint32_t svecs, uint32_t R, uint32_t wave,
                                               uint32_t nw, uint32_t lane, const Slots<DT, VPL>& S,
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
__device__ __forceinline__ void slots_apply(Rsrc rs, uint32_t reg_off, uint32_t svecs, uint32_t R,
                                            uint32_t wave, uint32_t nw, uint32_t lane,
                                            const Slots<DT, VPL>& S, float scale,
                                            bool may_exceed) {
  using IO = IoTraits<DT>;
  const uint32_t trips = (svecs + 63) / 64;
  uint32_t i = 0, k = 0;
#pragma unroll
  for (int j = 0; j < VPL; ++j) {
    const uint32_t r = wave + i * nw, v = lane + k * 64;
    float x[IO::kElems], g[IO::kElems], y[IO::kElems];
    unpack<DT>(S.x[j], x);
    unpack_gamma<DT>(S.g[j], g);
#pragma unroll
    for (int e = 0; e < IO::kElems; ++e) y[e] = (x[e] * g[e]) * scale;
    stream_store(rs, (r < R && v < svecs) ? reg_off + (r * svecs + v) * 16 : kOutOfRange,
                 pack<DT>(y, may_exceed));
    if (++k == trips) { k = 0; ++i; }
  }
}

// --- streamed shards (MODE 1 and 2): same order, dynamic loops ---------------

template <int DT>
__device__ __forceinline__ float shard_sumsq_stream(Rsrc rs, uint32_t shard_off, uint32_t svecs,
                                                    uint32_t lane) {
  using IO = IoTraits<DT>;
  const uint32_t trips = (svecs + 63) / 64;
  float acc = 0.f;
  for (uint32_t k = 0; k < trips; ++k) {
    const uint32_t v = lane + k * 64;
    float x[IO::kElems];
    unpack<DT>(v < svecs ? stream_load(rs, shard_off + v * 16) : u32x4{0, 0, 0, 0}, x);
    acc = vec_sumsq<DT>(x, acc);
  }
  return group_sum<64>(acc);
}

template <int DT>
__device__ __forceinline__ void apply_stream(Rsrc rs, uint32_t reg_off,
                                             const uint8_t* __restrict__ gamma, uint32_t nvecs,
                                             uint32_t tid, uint32_t nthreads, float scale) {
  using IO = IoTraits<DT>;
  for (uint32_t v = tid; v < nvecs; v += nthreads) {
    float x[IO::kElems], g[IO::kElems], y[IO::kElems];
    unpack<DT>(stream_load(rs, reg_off + v * 16), x);
    unpack_gamma<DT>(load_gamma<DT>(gamma, v), g);
#pragma unroll
    for (int e = 0; e < IO::kElems; ++e) y[e] = (x[e] * g[e]) * scale;
    stream_store(rs, reg_off + v * 16, pack<DT>(y));
  }
}

// Descriptor over the Q+K part of row t (wave-uniform).
__device__ __forceinline__ Rsrc row_rsrc(const uint8_t* qkv, uint64_t ld_bytes, uint32_t t,
                                         uint32_t qk_vecs) {
  return make_rsrc(qkv + (uint64_t)t * ld_bytes, (uint64_t)qk_vecs * 16);
}

// Fused layerwise, row kept in registers (VPL slots per region per lane).
// A block walks rows blockIdx.x, +gridDim.x, ...; gamma slots are loaded once
// per block.  Two register sets A and B take alternate rows: while one row is
// reduced, combined and stored, the next row's loads are already in flight in
// the other set (no register copies between them, so nothing forces a wait on
// the previous row's stores).
template <int DT, int QV, int KV>
struct LwRow {
  Slots<DT, QV> q;
  Slots<DT, KV> k;
};

template <int DT, int QV, int KV>
__device__ __forceinline__ void lw_issue(uint8_t* qkv, const RowGeom& G, uint32_t t, bool live,
                                         uint32_t Rq, uint32_t Rk, uint32_t wave, uint32_t nw,
                                         uint32_t lane, Rsrc& rs, LwRow<DT, QV, KV>& row) {
  rs = row_rsrc(qkv, G.ld_bytes, live ? t : 0, live ? G.q_vecs + G.k_vecs : 0);
  slots_load<DT, QV>(rs, 0, G.q_svecs, Rq, wave, nw, lane, row.q);
  slots_load<DT, KV>(rs, G.q_vecs * 16, G.k_svecs, Rk, wave, nw, lane, row.k);
}

template <int DT, int QV, int KV>
__device__ __forceinline__ void lw_finish(const RowGeom& G, Rsrc rs, uint32_t Rq, uint32_t Rk,
                                          uint32_t wave, uint32_t nw, uint32_t lane, float eps,
                                          LwRow<DT, QV, KV>& row, const LwRow<DT, QV, KV>& gam,
                                          bool exceed_q, bool exceed_k, float* __restrict__ part) {
  const uint32_t R = G.nshards;
  float* pq = part;
  float* pk = part + R;
  slots_partials<DT, QV>(G.q_svecs, Rq, wave, nw, lane, row.q, pq);
  slots_partials<DT, KV>(G.k_svecs, Rk, wave, nw, lane, row.k, pk);
  __syncthreads();
#pragma unroll
  for (int j = 0; j < QV; ++j) row.q.g[j] = gam.q.g[j];
#pragma unroll
  for (int j = 0; j < KV; ++j) row.k.g[j] = gam.k.g[j];
  // (a region without vectors reads partials nobody wrote and ignores them)
  float sq, sk;
  combine2(pq, pk, R, &sq, &sk);
  if (Rq) slots_apply<DT, QV>(rs, 0, G.q_svecs, Rq, wave, nw, lane, row.q,
                              rms_scale(sq, G.inv_wq, eps), exceed_q);
  if (Rk) slots_apply<DT, KV>(rs, G.q_vecs * 16, G.k_svecs, Rk, wave, nw, lane, row.k,
                              rms_scale(sk, G.inv_wk, eps), exceed_k);
}

// QV / KV: register slots per lane for Q and for K (a lane's shard vectors).
template <int DT, int QV, int KV>
__global__ __launch_bounds__(512) void layerwise_regs_kernel(
    uint8_t* __restrict__ qkv, RowGeom G, const uint8_t* __restrict__ gamma_q,
    const uint8_t* __restrict__ gamma_k, float eps) {
  extern __shared__ float lds[];               // [2 buffers][Q, K][nshards]
  const uint32_t lane = threadIdx.x & 63;
  const uint32_t wave = uniform(threadIdx.x >> 6);
  const uint32_t nw = blockDim.x >> 6;
  const uint32_t R = G.nshards;
  const uint32_t Rq = G.q_vecs ? R : 0, Rk = G.k_vecs ? R : 0;
  const uint32_t stride = gridDim.x;

  uint32_t t = blockIdx.x;
  if (t >= G.T) return;                        // whole block: no barrier is skipped by part of it
  LwRow<DT, QV, KV> a, b, gam;
  Rsrc ra, rb;
  // gamma first (straight-line loads): the FP8 range test below then waits
  // for gamma only, while the first row's loads stay in flight
  slots_load_gamma<DT, QV>(gamma_q, G.q_svecs, Rq, wave, nw, lane, gam.q);
  slots_load_gamma<DT, KV>(gamma_k, G.k_svecs, Rk, wave, nw, lane, gam.k);
  lw_issue<DT, QV, KV>(qkv, G, t, true, Rq, Rk, wave, nw, lane, ra, a);
  bool exceed_q = true, exceed_k = true;
  if constexpr (DT == kFP8) {
    exceed_q = e4m3_may_exceed(slots_gamma_max(gam.q), G.inv_wq);
    exceed_k = e4m3_may_exceed(slots_gamma_max(gam.k), G.inv_wk);
  }

  // LDS partials alternate between two buffers, one per register set: a
  // buffer is written again only after every thread has passed the barrier of
  // the row in between.
  while (true) {
    const uint32_t t1 = t + stride;
    const bool more1 = t1 < G.T;
    lw_issue<DT, QV, KV>(qkv, G, t1, more1, Rq, Rk, wave, nw, lane, rb, b);
    lw_finish<DT, QV, KV>(G, ra, Rq, Rk, wave, nw, lane, eps, a, gam, exceed_q, exceed_k, lds);
    if (!more1) break;
    const uint32_t t2 = t1 + stride;
    const bool more2 = t2 < G.T;
    lw_issue<DT, QV, KV>(qkv, G, t2, more2, Rq, Rk, wave, nw, lane, ra, a);
    lw_finish<DT, QV, KV>(G, rb, Rq, Rk, wave, nw, lane, eps, b, gam, exceed_q, exceed_k,
                          lds + 2 * R);
    if (!more2) break;
    t = t2;
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
  const uint32_t wave = uniform(threadIdx.x >> 6);
  const uint32_t nw = blockDim.x >> 6;
  const uint32_t R = G.nshards;
  const uint32_t k_off = G.q_vecs * 16;
  uint32_t parity = 0;
  for (uint32_t t = blockIdx.x; t < G.T; t += gridDim.x, parity ^= 1) {
    const Rsrc rs = row_rsrc(qkv, G.ld_bytes, t, G.q_vecs + G.k_vecs);
    float* pq = lds + parity * 2 * R;
    float* pk = pq + R;
    for (uint32_t r = wave; r < R; r += nw) {
      if (G.q_vecs) {
        const float s = shard_sumsq_stream<DT>(rs, r * G.q_svecs * 16, G.q_svecs, lane);
        if (lane == 0) pq[r] = s;
      }
      if (G.k_vecs) {
        const float s = shard_sumsq_stream<DT>(rs, k_off + r * G.k_svecs * 16, G.k_svecs, lane);
        if (lane == 0) pk[r] = s;
      }
    }
    __syncthreads();
    if (G.q_vecs)
      apply_stream<DT>(rs, 0, gamma_q, G.q_vecs, threadIdx.x, blockDim.x,
                       rms_scale(combine(pq, R, 1), G.inv_wq, eps));
    if (G.k_vecs)
      apply_stream<DT>(rs, k_off, gamma_k, G.k_vecs, threadIdx.x, blockDim.x,
                       rms_scale(combine(pk, R, 1), G.inv_wk, eps));
  }
}

// --- one wave per row (fused layerwise, regular shard geometry) -------------
//
// A region of 64*NS vectors is NS slots of 64 consecutive vectors: lane l
// holds vector 64*j + l in slot j, so each slot is one coalesced 1 KiB load.
// A shard of svecs vectors is either a run of m = svecs/64 whole slots, or,
// when svecs divides 64, one of G = 64/svecs lane groups of a slot.  Either
// way the lanes of a shard hold the vectors that lanes 0..svecs-1 hold in the
// block kernel, in the same order, and the reduction is the same tree (a
// narrow shard's group sum is the block kernel's 64-lane sum with zero lanes
// left out), so the partials, their in-order combine and the outputs are the
// same bits.  No barrier and no LDS traffic between waves: gamma is staged
// once per block in LDS and every wave then walks its own rows.

struct WaveShards {
  uint32_t m;       // slots per shard (1 when shards are narrower than a slot)
  uint32_t svecs;   // vectors per shard
  uint32_t G;       // shards per slot (1 when a shard spans whole slots)
};

// Sum over aligned groups of lg lanes, lg = 1, 2, 4, .., 64 (wave-uniform).
__device__ __forceinline__ float group_sum_n(float v, uint32_t lg) {
  switch (lg) {
    case 1: return v;
    case 2: return group_sum<2>(v);
    case 4: return group_sum<4>(v);
    case 8: return group_sum<8>(v);
    case 16: return group_sum<16>(v);
    case 32: return group_sum<32>(v);
    default: return group_sum<64>(v);
  }
}

// The region's sum of squares: shard partials combined in shard order,
// ((p0 + p1) + p2) + ..., wave-uniform.
template <int DT, int NS>
__device__ __forceinline__ float wave_region_sumsq(const u32x4 (&x)[NS], WaveShards w) {
  using IO = IoTraits<DT>;
  const uint32_t lanes = w.svecs < 64 ? w.svecs : 64;
  float s = 0.f, acc = 0.f;
  uint32_t k = 0;                              // slot within the current shard
#pragma unroll
  for (int j = 0; j < NS; ++j) {
    float f[IO::kElems];
    unpack<DT>(x[j], f);
    acc = vec_sumsq<DT>(f, k == 0 ? 0.f : acc);
    if (++k == w.m) {
      const float ps = group_sum_n(acc, lanes);
      for (uint32_t g = 0; g < w.G; ++g)
        s += __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, ps),
                                                                 (int)(g * w.svecs)));
      k = 0;
    }
  }
  return s;
}

// Apply to slot j of the row in `rs` and store it, then load slot j of the
// next row (descriptor `rn`, empty past the last row) into the same registers,
// so the next row's loads go out while this row is still being written.
template <int DT, int NS>
__device__ __forceinline__ void wave_region_apply(Rsrc rs, Rsrc rn, uint32_t reg_off, u32x4 (&x)[NS],
                                                  const u32x4* __restrict__ g_lds, uint32_t lane,
                                                  float scale, bool may_exceed) {
  using IO = IoTraits<DT>;
  constexpr int GV = Gam<DT>::kVecs;
#pragma unroll
  for (int j = 0; j < NS; ++j) {
    const uint32_t v = j * 64 + lane;
    Gam<DT> gw;
#pragma unroll
    for (int q = 0; q < GV; ++q) gw.v[q] = g_lds[v * GV + q];
    float f[IO::kElems], g[IO::kElems], y[IO::kElems];
    unpack<DT>(x[j], f);
    unpack_gamma<DT>(gw, g);
#pragma unroll
    for (int e = 0; e < IO::kElems; ++e) y[e] = (f[e] * g[e]) * scale;
    stream_store(rs, reg_off + v * 16, pack<DT>(y, may_exceed));
    x[j] = stream_load(rn, reg_off + v * 16);
  }
}

// Largest |gamma| over this lane's vectors of a region.
template <int DT, int NS>
__device__ __forceinline__ float wave_gamma_max(const u32x4* __restrict__ g_lds, uint32_t lane) {
  constexpr int GV = Gam<DT>::kVecs;
  float m = 0.f;
#pragma unroll
  for (int j = 0; j < NS; ++j) {
    Gam<DT> gw;
#pragma unroll
    for (int q = 0; q < GV; ++q) gw.v[q] = g_lds[(j * 64 + lane) * GV + q];
    float g[IoTraits<DT>::kElems];
    unpack_gamma<DT>(gw, g);
    m = abs_max(g, m);
  }
  return m;
}

#ifndef QKNORM_LWW_BLOCK
#define QKNORM_LWW_BLOCK 256         // threads per block of the one-wave-per-row kernel
#endif

// NQ, NK: slots of Q and of K (64 vectors each).  Rows: wave w of the grid
// takes rows w, w + (waves in the grid), ...  APPLY: the phase-C form -- each
// row's scale comes from the caller's nparts partials, added in order exactly
// as apply_scalar_kernel adds them (G.inv_wq / G.inv_wk then hold 1 / the
// full widths), and FP8 results are range-checked vector by vector, since a
// caller's scale carries no bound.
template <int DT, int NQ, int NK, bool APPLY>
__global__ __launch_bounds__(QKNORM_LWW_BLOCK) void layerwise_wave_kernel(
    uint8_t* __restrict__ qkv, RowGeom G, WaveShards wq, WaveShards wk,
    const uint8_t* __restrict__ gamma_q, const uint8_t* __restrict__ gamma_k, float eps,
    const float* __restrict__ part_q, const float* __restrict__ part_k, uint32_t nparts) {
  constexpr uint32_t GV = Gam<DT>::kVecs;
  constexpr uint32_t kQg = NQ * 64 * GV, kKg = NK * 64 * GV;   // 16-byte gamma vectors
  extern __shared__ u32x4 g_lds[];             // gamma_q, then gamma_k
  const uint32_t lane = threadIdx.x & 63;
  for (uint32_t i = threadIdx.x; i < kQg; i += blockDim.x) g_lds[i] = load16(gamma_q + i * 16);
  for (uint32_t i = threadIdx.x; i < kKg; i += blockDim.x) g_lds[kQg + i] = load16(gamma_k + i * 16);
  __syncthreads();
  bool exceed_q = true, exceed_k = true;
  if constexpr (DT == kFP8 && !APPLY) {
    exceed_q = e4m3_may_exceed(wave_gamma_max<DT, NQ>(g_lds, lane), G.inv_wq);
    exceed_k = e4m3_may_exceed(wave_gamma_max<DT, NK>(g_lds + kQg, lane), G.inv_wk);
  }
  const uint32_t waves = gridDim.x * (blockDim.x >> 6);
  const uint32_t k_off = G.q_vecs * 16;
  const uint32_t qk_vecs = G.q_vecs + G.k_vecs;
  uint32_t t = uniform(blockIdx.x * (blockDim.x >> 6) + (threadIdx.x >> 6));
  Rsrc rs = row_rsrc(qkv, G.ld_bytes, t < G.T ? t : 0, t < G.T ? qk_vecs : 0);
  u32x4 xq[NQ], xk[NK];
#pragma unroll
  for (int j = 0; j < NQ; ++j) xq[j] = stream_load(rs, (j * 64 + lane) * 16);
#pragma unroll
  for (int j = 0; j < NK; ++j) xk[j] = stream_load(rs, k_off + (j * 64 + lane) * 16);
  for (; t < G.T; t += waves) {
    const uint32_t tn = t + waves;
    const Rsrc rn = row_rsrc(qkv, G.ld_bytes, tn < G.T ? tn : 0, tn < G.T ? qk_vecs : 0);
    float rq, rk;
    if constexpr (APPLY) {
      const float* pq = G.q_vecs ? part_q + t : part_k + t;
      const float* pk = G.k_vecs ? part_k + t : part_q + t;
      float sq, sk;
      combine_cols(pq, pk, nparts, G.T, &sq, &sk);
      rq = rms_scale(sq, G.inv_wq, eps);
      rk = rms_scale(sk, G.inv_wk, eps);
    } else {
      rq = rms_scale(wave_region_sumsq<DT, NQ>(xq, wq), G.inv_wq, eps);
      rk = rms_scale(wave_region_sumsq<DT, NK>(xk, wk), G.inv_wk, eps);
    }
    // keep the row packed between the two passes: without these the compiler
    // reuses the first pass's widened values and holds the whole row in fp32
#pragma unroll
    for (int j = 0; j < NQ; ++j) asm volatile("" : "+v"(xq[j]));
#pragma unroll
    for (int j = 0; j < NK; ++j) asm volatile("" : "+v"(xk[j]));
    wave_region_apply<DT, NQ>(rs, rn, 0, xq, g_lds, lane, rq, exceed_q);
    wave_region_apply<DT, NK>(rs, rn, k_off, xk, g_lds + kQg, lane, rk, exceed_k);
    rs = rn;
  }
}

// Phase A.  A wave takes one shard of one region (Q or K) over a block of 32
// consecutive rows and ends with lane j holding the partial of row t0 + j,
// stored with one coalesced 128-byte write at part[r*T + t0 ...].  (32 rows
// keep the block's descriptor below 2^31 bytes, well under the out-of-range
// offset used for masked lanes.)
//
// A shard of svecs >= 64 vectors is reduced exactly like the fused kernel
// (lane l takes vectors l, l+64, ..., then the 64-lane sum).  A shard of
// fewer vectors uses lane groups of LG = next power of two >= svecs lanes,
// 64/LG rows per step; lane i of a group takes vector i, and the LG-lane sum
// equals the 64-lane sum of the fused kernel bit for bit, because the lanes it
// leaves out hold exact zeros (x + 0 == x).

constexpr uint32_t kRowBlock = 32;

template <int DT>
__global__ __launch_bounds__(256) void partial_sumsq_kernel(const uint8_t* __restrict__ qkv,
                                                            RowGeom G, float* __restrict__ part_q,
                                                            float* __restrict__ part_k) {
  using IO = IoTraits<DT>;
  const uint32_t lane = threadIdx.x & 63;
  const uint32_t R = G.nshards;
  const uint32_t nblk = (G.T + kRowBlock - 1) / kRowBlock;
  const uint32_t nq = G.q_vecs ? R * nblk : 0;
  const uint32_t nk = G.k_vecs ? R * nblk : 0;
  const uint32_t nwaves = (gridDim.x * blockDim.x) >> 6;
  for (uint32_t i = uniform((blockIdx.x * blockDim.x + threadIdx.x) >> 6); i < nq + nk;
       i += nwaves) {
    const bool isk = i >= nq;
    const uint32_t w = isk ? i - nq : i;
    const uint32_t r = w % R, blk = w / R;
    const uint32_t svecs = isk ? G.k_svecs : G.q_svecs;
    const uint32_t shard_off = ((isk ? G.q_vecs : 0) + r * svecs) * 16;
    uint32_t lg = 2;
    while (lg < svecs && lg < 64) lg <<= 1;
    const uint32_t rps = 64 / lg;              // rows per step
    const uint32_t trips = (svecs + lg - 1) / lg;
    const uint32_t grp = lane / lg, li = lane % lg;
    const uint32_t t0 = blk * kRowBlock;
    const uint32_t rows = G.T - t0 < kRowBlock ? G.T - t0 : kRowBlock;
    // descriptor over this block's rows (below 32 rows * 64 MiB = 2^31 bytes)
    const Rsrc rs = make_rsrc(qkv + (uint64_t)t0 * G.ld_bytes,
                              (uint64_t)(rows - 1) * G.ld_bytes + (uint64_t)(G.q_vecs + G.k_vecs) * 16);
    float mine = 0.f;
    for (uint32_t j0 = 0; j0 < rows; j0 += rps) {
      const uint32_t j = j0 + grp;             // this lane group's row in the block
      float acc = 0.f;
      for (uint32_t k = 0; k < trips; ++k) {
        const uint32_t v = li + k * lg;
        float x[IO::kElems];
        unpack<DT>(stream_load(rs, (j < rows && v < svecs)
                                       ? (uint32_t)(j * G.ld_bytes) + shard_off + v * 16
                                       : kOutOfRange), x);
        acc = vec_sumsq<DT>(x, acc);
      }
      const float sum = group_sum_n(acc, lg);
      for (uint32_t g = 0; g < rps; ++g) {
        const float sg = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(sum), g * lg));
        mine = lane == j0 + g ? sg : mine;
      }
    }
    if (lane < rows) (isk ? part_k : part_q)[(uint64_t)r * G.T + t0 + lane] = mine;
  }
}

// Phase C.  A block takes kApplyRows consecutive rows.  First the rows'
// scales: thread i < kApplyRows adds row t0+i's partials in order (r = 0 ..
// nparts-1; each r one contiguous read across those threads), takes
// rsq((sum)/norm_w + eps) and leaves it in LDS.  Then every row is applied
// with flat 16-byte vectors over Q then K; thread tid takes vectors tid,
// tid+nt, ... of every row (nt threads), so its gamma vectors stay in
// registers (VPT of them) for all the block's rows.  The launcher picks VPT
// and nt <= 512 that leave the fewest (thread, vector) slots idle.
#ifndef QKNORM_APPLY_ROWS
#define QKNORM_APPLY_ROWS 2        // rows per phase-C block
#endif
constexpr uint32_t kApplyRows = QKNORM_APPLY_ROWS;

template <int VPT>
__device__ __forceinline__ void apply_rows_load(Rsrc rs, uint32_t tid, uint32_t nt, uint32_t nv,
                                                u32x4 (&x)[VPT]) {
#pragma unroll
  for (int k = 0; k < VPT; ++k) {
    const uint32_t v = tid + k * nt;
    x[k] = stream_load(rs, v < nv ? v * 16 : kOutOfRange);
  }
}

template <int DT, int VPT>
__device__ __forceinline__ void apply_rows_store(Rsrc rs, uint32_t tid, uint32_t nt,
                                                 uint32_t q_vecs, uint32_t nv,
                                                 const u32x4 (&x)[VPT], const Gam<DT> (&g)[VPT],
                                                 float sq, float sk) {
  using IO = IoTraits<DT>;
#pragma unroll
  for (int k = 0; k < VPT; ++k) {
    const uint32_t v = tid + k * nt;
    float xf[IO::kElems], gf[IO::kElems], y[IO::kElems];
    unpack<DT>(x[k], xf);
    unpack_gamma<DT>(g[k], gf);
    const float sc = v < q_vecs ? sq : sk;
#pragma unroll
    for (int e = 0; e < IO::kElems; ++e) y[e] = (xf[e] * gf[e]) * sc;
    stream_store(rs, v < nv ? v * 16 : kOutOfRange, pack<DT>(y));
  }
}

template <int DT, int VPT>
__global__ __launch_bounds__(512) void apply_scalar_kernel(
    uint8_t* __restrict__ qkv, uint64_t ld_bytes, uint32_t T, uint32_t q_vecs, uint32_t k_vecs,
    const float* __restrict__ part_q, const float* __restrict__ part_k, uint32_t nparts,
    float inv_norm_wq, float inv_norm_wk, const uint8_t* __restrict__ gamma_q,
    const uint8_t* __restrict__ gamma_k, float eps) {
  // the rows' scales, two buffers used in turn: a buffer is written again
  // only after every thread has passed the barrier of the rows in between
  __shared__ float scale[2][2][kApplyRows];
  const uint32_t tid = threadIdx.x, nt = blockDim.x;
  const uint32_t nv = q_vecs + k_vecs;
  Gam<DT> g[VPT];
#pragma unroll
  for (int k = 0; k < VPT; ++k) {
    const uint32_t v = tid + k * nt;
    g[k] = v < q_vecs ? load_gamma<DT>(gamma_q, v)
                      : (v < nv ? load_gamma<DT>(gamma_k, v - q_vecs) : zero_gamma<DT>());
  }
  uint32_t buf = 0;
  for (uint32_t t0 = blockIdx.x * kApplyRows; t0 < T; t0 += gridDim.x * kApplyRows, buf ^= 1) {
    const uint32_t rows = T - t0 < kApplyRows ? T - t0 : kApplyRows;
    // the first row's loads go out before the partials are read (they do not
    // need the scales), so the two reads' latencies overlap; the barrier
    // below waits for LDS only, not for these loads
    u32x4 xa[VPT], xb[VPT];
    Rsrc ra = row_rsrc(qkv, ld_bytes, t0, nv), rb;
    apply_rows_load<VPT>(ra, tid, nt, nv, xa);
    float (&sc)[2][kApplyRows] = scale[buf];
    if (tid < rows) {
      float sq, sk;
      combine_cols((q_vecs ? part_q : part_k) + t0 + tid, (k_vecs ? part_k : part_q) + t0 + tid, nparts,
                   T, &sq, &sk);
      sc[0][tid] = rms_scale(sq, inv_norm_wq, eps);   // (a region without vectors never reads its scale)
      sc[1][tid] = rms_scale(sk, inv_norm_wk, eps);
    }
    lds_barrier();
    // rows alternate between two register sets: row j+1's loads are in
    // flight while row j is scaled and stored
    for (uint32_t j = 0; j < rows; j += 2) {
      const bool more1 = j + 1 < rows;
      rb = row_rsrc(qkv, ld_bytes, more1 ? t0 + j + 1 : t0, more1 ? nv : 0);
      apply_rows_load<VPT>(rb, tid, nt, nv, xb);
      apply_rows_store<DT, VPT>(ra, tid, nt, q_vecs, nv, xa, g, sc[0][j], sc[1][j]);
      if (!more1) break;
      const bool more2 = j + 2 < rows;
      ra = row_rsrc(qkv, ld_bytes, more2 ? t0 + j + 2 : t0, more2 ? nv : 0);
      apply_rows_load<VPT>(ra, tid, nt, nv, xa);
      apply_rows_store<DT, VPT>(rb, tid, nt, q_vecs, nv, xb, g, sc[0][j + 1], sc[1][j + 1]);
    }
  }
}

// Phase C for rows wider than 4 vectors per thread: one block per row, gamma
// re-read for each row.
template <int DT>
__global__ __launch_bounds__(256) void apply_scalar_wide_kernel(
    uint8_t* __restrict__ qkv, uint64_t ld_bytes, uint32_t T, uint32_t q_vecs, uint32_t k_vecs,
    const float* __restrict__ part_q, const float* __restrict__ part_k, uint32_t nparts,
    float inv_norm_wq, float inv_norm_wk, const uint8_t* __restrict__ gamma_q,
    const uint8_t* __restrict__ gamma_k, float eps) {
  for (uint32_t t = blockIdx.x; t < T; t += gridDim.x) {
    const Rsrc rs = row_rsrc(qkv, ld_bytes, t, q_vecs + k_vecs);
    float sq, sk;
    combine_cols((q_vecs ? part_q : part_k) + t, (k_vecs ? part_k : part_q) + t, nparts, T, &sq, &sk);
    if (q_vecs)
      apply_stream<DT>(rs, 0, gamma_q, q_vecs, threadIdx.x, blockDim.x, rms_scale(sq, inv_norm_wq, eps));
    if (k_vecs)
      apply_stream<DT>(rs, q_vecs * 16, gamma_k, k_vecs, threadIdx.x, blockDim.x,
                       rms_scale(sk, inv_norm_wk, eps));
  }
}

// ================================================================ launchers

template <int DT, int LPH>
static hipError_t launch_per_head_t(const PerHeadArgs& a, hipStream_t s, int cus) {
  constexpr int U = ph_unroll<DT>();
  constexpr uint64_t CH = (64 / LPH) * U;
  constexpr int kBlock = ph_threads<DT>();
  constexpr uint64_t heads_per_block = CH * (kBlock / 64);
  const int es = IoTraits<DT>::kBytes;
  const uint32_t head_bytes = (uint32_t)(a.head_dim * es);
  const uint32_t hvec = head_bytes / 16;
  const bool exact = hvec == (uint32_t)LPH;
  // the cap in waves is the same for every block size
  const uint64_t cap = DT == kFP8 ? (uint64_t)cus * QKNORM_PH_WAVES_PER_CU_FP8 / (kBlock / 64)
                                  : (uint64_t)cus * QKNORM_PH_BLOCKS_PER_CU * QKNORM_PH_THREADS / kBlock;
  const uint64_t Htot = (uint64_t)a.hq + a.hkv;

  // the non-empty regions, Q first; the grid cap is shared in proportion
  PhRegion reg[2] = {};
  int n = 0;
  bool one = true;
  const uint32_t heads[2] = {(uint32_t)a.hq, (uint32_t)a.hkv};
  const void* gammas[2] = {a.gamma_q, a.gamma_k};
  for (int i = 0; i < 2; ++i) {
    if (heads[i] == 0) continue;
    PhRegion& r = reg[n++];
    r.gamma = (const uint8_t*)gammas[i];
    r.H = heads[i];
    r.col_bytes = i == 0 ? 0u : (uint32_t)a.hq * head_bytes;
    const uint64_t total = (uint64_t)a.T * r.H;
    uint64_t blocks = (total + heads_per_block - 1) / heads_per_block;
    uint64_t rcap = cap * r.H / Htot;
    if (rcap < 1) rcap = 1;
    if (blocks > rcap) blocks = rcap;
    if (blocks < 1) blocks = 1;
    r.blocks = (uint32_t)blocks;
    const uint64_t stride = blocks * heads_per_block;   // heads advanced per trip
    one = one && stride >= total;
    r.stride_rows = (uint32_t)(stride / r.H);
    r.stride_heads = (uint32_t)(stride % r.H);
    r.byH = make_fastdiv(r.H);
  }
  // a single region whose rows hold nothing else: one flat array of heads
  // (heads of a power-of-two size only; others take the row-wise kernel)
  const bool contig = exact && n == 1 && reg[0].col_bytes == 0 &&
                      a.ld == (int64_t)reg[0].H * a.head_dim;
  if (contig) {
    reg[0].stride_heads = reg[0].stride_rows * reg[0].H + reg[0].stride_heads;
    reg[0].stride_rows = 0;
  }
  const bool two = n == 2;
  void (*kern)(uint8_t*, uint32_t, uint32_t, PhRegion, PhRegion, FastDiv40, float, float, uint32_t);
  if (contig)
    kern = one ? per_head_kernel<DT, LPH, U, true, true, true, false>
               : per_head_kernel<DT, LPH, U, true, false, true, false>;
  else if (exact)
    kern = two ? (one ? per_head_kernel<DT, LPH, U, false, true, true, true>
                      : per_head_kernel<DT, LPH, U, false, false, true, true>)
               : (one ? per_head_kernel<DT, LPH, U, false, true, true, false>
                      : per_head_kernel<DT, LPH, U, false, false, true, false>);
  else
    kern = two ? (one ? per_head_kernel<DT, LPH, U, false, true, false, true>
                      : per_head_kernel<DT, LPH, U, false, false, false, true>)
               : (one ? per_head_kernel<DT, LPH, U, false, true, false, false>
                      : per_head_kernel<DT, LPH, U, false, false, false, false>);
  // interleave the two regions' blocks: the largest dividend, N * blocks1,
  // stays far below 2^40 for the capped grids used here (N is at most 320
  // blocks per CU), so the interleave applies to every shape
  const uint64_t N = (uint64_t)reg[0].blocks + reg[1].blocks;
  FastDiv40 byN{0, 0};
  if (reg[1].blocks != 0 && N * reg[1].blocks < kFastDiv40Limit)
    byN = make_fastdiv40((uint32_t)N);
  hipLaunchKernelGGL(kern, dim3((uint32_t)N), dim3(kBlock), 0, s, (uint8_t*)a.qkv,
                     (uint32_t)(a.ld * es), (uint32_t)a.T, reg[0], reg[1], byN, a.eps,
                     1.0f / (float)a.head_dim, hvec);
  return hipGetLastError();
}

// Lanes per head: the head's 16-byte vectors rounded up to a power of two.
static uint32_t lanes_per_head(uint32_t hvec) {
  uint32_t l = 1;
  while (l < hvec) l <<= 1;
  return l;
}

bool per_head_span_ok(const PerHeadArgs& a) {
  // the largest descriptor span of a trip: from a wave's first head (at most
  // H-1 into its row) over CH heads, plus the region, must stay below 2^31
  const int es = a.dtype == kF32 ? 4 : (a.dtype == kFP8 ? 1 : 2);
  const uint64_t hb = (uint64_t)a.head_dim * es;
  const uint64_t ch = (64 / lanes_per_head((uint32_t)(hb / 16))) *
                     (uint64_t)(a.dtype == kFP8 ? ph_unroll<kFP8>() : ph_unroll<kBF16>());
  const uint64_t ld_bytes = (uint64_t)a.ld * es;
  for (int64_t H : {(int64_t)a.hq, (int64_t)a.hkv}) {
    if (H <= 0) continue;
    const uint64_t span = ((uint64_t)H + ch - 2) / (uint64_t)H * ld_bytes + (uint64_t)H * hb;
    if (span >= (UINT64_C(1) << 31)) return false;
  }
  return true;
}

template <int DT>
static hipError_t launch_per_head_dt(const PerHeadArgs& a, hipStream_t s, int cus) {
  switch (lanes_per_head((uint32_t)(a.head_dim * IoTraits<DT>::kBytes / 16))) {
    case 1: return launch_per_head_t<DT, 1>(a, s, cus);
    case 2: return launch_per_head_t<DT, 2>(a, s, cus);
    case 4: return launch_per_head_t<DT, 4>(a, s, cus);
    case 8: return launch_per_head_t<DT, 8>(a, s, cus);
    case 16: return launch_per_head_t<DT, 16>(a, s, cus);
    case 32: return launch_per_head_t<DT, 32>(a, s, cus);
    case 64: return launch_per_head_t<DT, 64>(a, s, cus);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_per_head(const PerHeadArgs& a, hipStream_t s, int cus) {
  switch (a.dtype) {
    case kBF16: return launch_per_head_dt<kBF16>(a, s, cus);
    case kF16: return launch_per_head_dt<kF16>(a, s, cus);
    case kFP8: return launch_per_head_dt<kFP8>(a, s, cus);
    default: return launch_per_head_dt<kF32>(a, s, cus);
  }
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
  G.inv_wq = wq ? 1.0f / (float)wq : 0.f;
  G.inv_wk = wk ? 1.0f / (float)wk : 0.f;
  return G;
}

// Waves per block and register slots per lane (Q and K) for a layerwise geometry.
static void layerwise_shape(const RowGeom& G, uint32_t* nw, uint32_t* qv, uint32_t* kv) {
  const uint32_t w = G.nshards < 8 ? G.nshards : 8;
  const uint32_t per_wave = (G.nshards + w - 1) / w;
  *nw = w;
  *qv = G.q_vecs ? per_wave * ((G.q_svecs + 63) / 64) : 0;
  *kv = G.k_vecs ? per_wave * ((G.k_svecs + 63) / 64) : 0;
}

static uint32_t row_blocks(uint32_t T, uint32_t nw, int cus) {
  uint64_t cap = (uint64_t)cus * (QKNORM_LW_WAVES_PER_CU / nw);
  if (cap < (uint64_t)cus) cap = cus;
  uint64_t b = T < cap ? T : cap;
  return (uint32_t)(b < 1 ? 1 : b);
}

template <int DT, int QV, int KV>
static hipError_t launch_lw_regs(const RowGeom& G, uint32_t nw, const LayerwiseArgs& a,
                                 hipStream_t s, int cus) {
  hipLaunchKernelGGL((layerwise_regs_kernel<DT, QV, KV>), dim3(row_blocks(G.T, nw, cus)),
                     dim3(nw * 64), (size_t)4 * G.nshards * sizeof(float), s, (uint8_t*)a.qkv, G,
                     (const uint8_t*)a.gamma_q, (const uint8_t*)a.gamma_k, a.eps);
  return hipGetLastError();
}

static int slot_class(uint32_t n) { return n <= 1 ? 1 : n <= 2 ? 2 : n <= 4 ? 4 : 0; }

// Rows too wide for the register slots.
template <int DT>
static hipError_t launch_lw_stream(const RowGeom& G, uint32_t nw, const LayerwiseArgs& a,
                                   hipStream_t s, int cus) {
  hipLaunchKernelGGL((layerwise_stream_kernel<DT>), dim3(row_blocks(G.T, nw, cus)), dim3(nw * 64),
                     (size_t)4 * G.nshards * sizeof(float), s, (uint8_t*)a.qkv, G,
                     (const uint8_t*)a.gamma_q, (const uint8_t*)a.gamma_k, a.eps);
  return hipGetLastError();
}

template <int DT, int QV>
static hipError_t launch_lw_regs_k(const RowGeom& G, uint32_t nw, int kc, const LayerwiseArgs& a,
                                   hipStream_t s, int cus) {
  switch (kc) {
    case 1: return launch_lw_regs<DT, QV, 1>(G, nw, a, s, cus);
    case 2: return launch_lw_regs<DT, QV, 2>(G, nw, a, s, cus);
    default:
      // FP8 slots carry two gamma vectors each: four Q and four K slots would
      // not fit in registers
      if constexpr (DT == kFP8 && QV == 4) return launch_lw_stream<DT>(G, nw, a, s, cus);
      else return launch_lw_regs<DT, QV, 4>(G, nw, a, s, cus);
  }
}

// The one-wave-per-row kernel serves FP8 rows: on the [32768, 10240] prefill
// rows it takes 101 us against the block kernel's 112 us.  For bf16 rows it
// measured 213-226 us against 198 us (at 8 to 128 waves per CU, with or
// without the next row's loads overlapping the stores), so 16- and 32-bit rows
// keep the block kernel.  One row per wave measured best (128 waves per CU).
#ifndef QKNORM_LWW_WAVES_PER_CU
#define QKNORM_LWW_WAVES_PER_CU 128  // grid cap of the one-wave-per-row kernel
#endif
#ifndef QKNORM_LWW
#define QKNORM_LWW 1                 // 0: FP8 rows take the block-per-row kernels too
#endif
static constexpr bool kLwWave = QKNORM_LWW != 0;

// The shard layout of a region for the one-wave-per-row kernel, if it has one.
static bool wave_shards(uint32_t vecs, uint32_t svecs, WaveShards* w) {
  if (vecs == 0 || vecs % 64 != 0) return false;
  if (svecs % 64 == 0) {
    *w = WaveShards{svecs / 64, svecs, 1};
    return true;
  }
  if (64 % svecs == 0) {
    *w = WaveShards{1, svecs, 64 / svecs};
    return true;
  }
  return false;
}

template <int DT, int NQ, int NK>
static hipError_t launch_lw_wave(const RowGeom& G, WaveShards wq, WaveShards wk,
                                 const LayerwiseArgs& a, hipStream_t s, int cus) {
  constexpr uint32_t kWaves = QKNORM_LWW_BLOCK / 64;
  uint64_t waves = (uint64_t)cus * QKNORM_LWW_WAVES_PER_CU;
  if (waves > G.T) waves = G.T;
  const uint32_t blocks = (uint32_t)((waves + kWaves - 1) / kWaves);
  const size_t lds = (size_t)(NQ + NK) * 64 * Gam<DT>::kVecs * 16;
  hipLaunchKernelGGL((layerwise_wave_kernel<DT, NQ, NK, false>), dim3(blocks), dim3(QKNORM_LWW_BLOCK), lds,
                     s, (uint8_t*)a.qkv, G, wq, wk, (const uint8_t*)a.gamma_q,
                     (const uint8_t*)a.gamma_k, a.eps, (const float*)nullptr, (const float*)nullptr, 0u);
  return hipGetLastError();
}

// Phase C through the one-wave-per-row kernel (G.inv_wq / inv_wk: 1 / the full widths).
template <int DT, int NQ, int NK>
static hipError_t launch_lw_wave_apply(const RowGeom& G, const ApplyArgs& a, hipStream_t s, int cus) {
  constexpr uint32_t kWaves = QKNORM_LWW_BLOCK / 64;
  uint64_t waves = (uint64_t)cus * QKNORM_LWW_WAVES_PER_CU;
  if (waves > G.T) waves = G.T;
  const uint32_t blocks = (uint32_t)((waves + kWaves - 1) / kWaves);
  const size_t lds = (size_t)(NQ + NK) * 64 * Gam<DT>::kVecs * 16;
  const WaveShards none{1, 64, 1};
  hipLaunchKernelGGL((layerwise_wave_kernel<DT, NQ, NK, true>), dim3(blocks), dim3(QKNORM_LWW_BLOCK), lds,
                     s, (uint8_t*)a.qkv, G, none, none, (const uint8_t*)a.gamma_q,
                     (const uint8_t*)a.gamma_k, a.eps, a.part_q, a.part_k, (uint32_t)a.nparts);
  return hipGetLastError();
}

// The slot counts (Q, K) the one-wave-per-row kernel is built for.
#define QKNORM_LWW_SHAPES(X) X(4, 1) X(8, 1) X(8, 2) X(16, 2) X(16, 4)

// Whether the one-wave-per-row kernel takes this geometry.
static bool lw_wave_fits(const RowGeom& G, WaveShards* wq, WaveShards* wk) {
  if (!wave_shards(G.q_vecs, G.q_svecs, wq) || !wave_shards(G.k_vecs, G.k_svecs, wk)) return false;
  const uint32_t nq = G.q_vecs / 64, nk = G.k_vecs / 64;
#define QKNORM_LWW_FITS(Q, K) if (nq == Q && nk == K) return true;
  QKNORM_LWW_SHAPES(QKNORM_LWW_FITS)
#undef QKNORM_LWW_FITS
  return false;
}

template <int DT>
static hipError_t launch_lw_wave_dt(const RowGeom& G, WaveShards wq, WaveShards wk,
                                    const LayerwiseArgs& a, hipStream_t s, int cus) {
  const uint32_t nq = G.q_vecs / 64, nk = G.k_vecs / 64;
#define QKNORM_LWW_LAUNCH(Q, K) \
  if (nq == Q && nk == K) return launch_lw_wave<DT, Q, K>(G, wq, wk, a, s, cus);
  QKNORM_LWW_SHAPES(QKNORM_LWW_LAUNCH)
#undef QKNORM_LWW_LAUNCH
  return hipErrorInvalidValue;                 // not reached: lw_wave_fits() was checked
}

template <int DT>
static hipError_t launch_layerwise_dt(const LayerwiseArgs& a, hipStream_t s, int cus) {
  const RowGeom G = make_geom(a.T, a.ld, a.wq, a.wk, a.nshards, IoTraits<DT>::kBytes);
  if constexpr (DT == kFP8 && kLwWave) {
    WaveShards wq, wk;
    if (lw_wave_fits(G, &wq, &wk)) return launch_lw_wave_dt<DT>(G, wq, wk, a, s, cus);
  }
  uint32_t nw, qv, kv;
  layerwise_shape(G, &nw, &qv, &kv);
  const int qc = slot_class(qv), kc = slot_class(kv);
  if (qc && kc) {
    switch (qc) {
      case 1: return launch_lw_regs_k<DT, 1>(G, nw, kc, a, s, cus);
      case 2: return launch_lw_regs_k<DT, 2>(G, nw, kc, a, s, cus);
      default: return launch_lw_regs_k<DT, 4>(G, nw, kc, a, s, cus);
    }
  }
  return launch_lw_stream<DT>(G, nw, a, s, cus);
}

hipError_t launch_layerwise(const LayerwiseArgs& a, hipStream_t s, int cus) {
  switch (a.dtype) {
    case kBF16: return launch_layerwise_dt<kBF16>(a, s, cus);
    case kF16: return launch_layerwise_dt<kF16>(a, s, cus);
    case kFP8: return launch_layerwise_dt<kFP8>(a, s, cus);
    default: return launch_layerwise_dt<kF32>(a, s, cus);
  }
}

template <int DT>
static hipError_t launch_partial_dt(const PartialArgs& a, hipStream_t s, int cus) {
  const RowGeom G = make_geom(a.T, a.ld, a.wq, a.wk, a.nshards, IoTraits<DT>::kBytes);
  const uint64_t items = (uint64_t)((a.T + kRowBlock - 1) / kRowBlock) * a.nshards *
                         ((a.wq > 0) + (a.wk > 0));
  uint64_t blocks = (items + 3) / 4;
  const uint64_t cap = (uint64_t)cus * (QKNORM_LW_WAVES_PER_CU / 4);
  if (blocks > cap) blocks = cap;
  if (blocks < 1) blocks = 1;
  hipLaunchKernelGGL((partial_sumsq_kernel<DT>), dim3((uint32_t)blocks), dim3(256), 0, s,
                     (const uint8_t*)a.qkv, G, a.part_q, a.part_k);
  return hipGetLastError();
}

hipError_t launch_partial_sumsq(const PartialArgs& a, hipStream_t s, int cus) {
  switch (a.dtype) {
    case kBF16: return launch_partial_dt<kBF16>(a, s, cus);
    case kF16: return launch_partial_dt<kF16>(a, s, cus);
    case kFP8: return launch_partial_dt<kFP8>(a, s, cus);
    default: return launch_partial_dt<kF32>(a, s, cus);
  }
}

template <int DT, int VPT>
static hipError_t launch_apply_rows(const ApplyArgs& a, hipStream_t s, int cus, uint32_t qv,
                                    uint32_t kv, float iq, float ik, uint32_t threads) {
  uint64_t blocks = ((uint64_t)a.T + kApplyRows - 1) / kApplyRows;
  const uint64_t cap = (uint64_t)cus * (QKNORM_LW_WAVES_PER_CU / (threads / 64));
  if (blocks > cap) blocks = cap;
  if (blocks < 1) blocks = 1;
  hipLaunchKernelGGL((apply_scalar_kernel<DT, VPT>), dim3((uint32_t)blocks), dim3(threads), 0, s,
                     (uint8_t*)a.qkv, (uint64_t)(a.ld * IoTraits<DT>::kBytes), (uint32_t)a.T, qv, kv,
                     a.part_q, a.part_k, (uint32_t)a.nparts, iq, ik, (const uint8_t*)a.gamma_q,
                     (const uint8_t*)a.gamma_k, a.eps);
  return hipGetLastError();
}

template <int DT>
static hipError_t launch_apply_dt(const ApplyArgs& a, hipStream_t s, int cus) {
  const int esize = IoTraits<DT>::kBytes;
  const uint32_t qv = (uint32_t)(a.wq * esize / 16), kv = (uint32_t)(a.wk * esize / 16);
  const float iq = a.norm_wq ? 1.0f / (float)a.norm_wq : 0.f;
  const float ik = a.norm_wk ? 1.0f / (float)a.norm_wk : 0.f;
  if constexpr (DT == kFP8 && kLwWave) {
    // FP8 rows of whole slots take the one-wave-per-row kernel, as in the fused call
    if (qv % 64 == 0 && kv % 64 == 0) {
      RowGeom G = make_geom(a.T, a.ld, a.wq, a.wk, 1, esize);
      G.inv_wq = iq;
      G.inv_wk = ik;
      const uint32_t nq = qv / 64, nk = kv / 64;
#define QKNORM_LWW_APPLY(Q, K) \
  if (nq == Q && nk == K) return launch_lw_wave_apply<DT, Q, K>(G, a, s, cus);
      QKNORM_LWW_SHAPES(QKNORM_LWW_APPLY)
#undef QKNORM_LWW_APPLY
    }
  }
  // vectors per thread and block size: at most 512 threads, as few idle
  // (thread, vector) slots as possible, fewer vectors per thread on a tie
  const uint32_t nv = qv + kv;
  uint32_t vpt = 0, threads = 512;
  uint64_t best = ~0ull;
  for (uint32_t c = 1; c <= 4; ++c) {
    const uint32_t t = ((nv + c - 1) / c + 63) / 64 * 64;
    if (t > 512) continue;
    const uint64_t idle = (uint64_t)t * c - nv;
    if (idle < best) { best = idle; vpt = c; threads = t; }
  }
  switch (vpt) {
    case 1: return launch_apply_rows<DT, 1>(a, s, cus, qv, kv, iq, ik, threads);
    case 2: return launch_apply_rows<DT, 2>(a, s, cus, qv, kv, iq, ik, threads);
    case 3: return launch_apply_rows<DT, 3>(a, s, cus, qv, kv, iq, ik, threads);
    case 4: return launch_apply_rows<DT, 4>(a, s, cus, qv, kv, iq, ik, threads);
    default: break;
  }
  uint64_t blocks = a.T;
  const uint64_t cap = (uint64_t)cus * (QKNORM_LW_WAVES_PER_CU / 4);
  if (blocks > cap) blocks = cap;
  if (blocks < 1) blocks = 1;
  hipLaunchKernelGGL((apply_scalar_wide_kernel<DT>), dim3((uint32_t)blocks), dim3(256), 0, s,
                     (uint8_t*)a.qkv, (uint64_t)(a.ld * esize), (uint32_t)a.T, qv, kv, a.part_q,
                     a.part_k, (uint32_t)a.nparts, iq, ik, (const uint8_t*)a.gamma_q,
                     (const uint8_t*)a.gamma_k, a.eps);
  return hipGetLastError();
}

hipError_t launch_apply_scalar(const ApplyArgs& a, hipStream_t s, int cus) {
  switch (a.dtype) {
    case kBF16: return launch_apply_dt<kBF16>(a, s, cus);
    case kF16: return launch_apply_dt<kF16>(a, s, cus);
    case kFP8: return launch_apply_dt<kFP8>(a, s, cus);
    default: return launch_apply_dt<kF32>(a, s, cus);
  }
}

}  // namespace qknorm
