// Residual activation compensation on the rollout side (QUADS technical
// summary, section 2.2B; yfxerp digest): per selection unit, score every
// channel by the magnitude of the FP4 residual R = x - DQ(Q(x)), keep the
// top-k channels (a binary channel mask), and quantize the compact residual
// R_S a second time with its own global scale.
//
// Kernels (one stream, in order):
//   plan      tile_start[u]: first 128-row tile of unit u (exclusive scan), and
//             a record per score tile and per gather slot (its unit and rows),
//             so that the later kernels find their rows in one read
//   scores    per (128-row tile, 64 channels): fp32 sum of |R| over the tile's
//             rows in increasing row order          (skipped when nvfp4_quantize
//                                                    already produced them)
//   select    per unit: tile sums added in tile order; the k-th largest score
//             found two bits per pass (keys in registers for K <= 8192,
//             else in LDS one bit per pass); ties to the lower channel;
//             compaction in ascending channel order (block scans)
//   gather    per 32-row slot: R_S = x[:, sel] - DQ(codes, scales)[:, sel] ->
//             workspace, with the slot's max |R_S|
//   requant   per 32-row slot: unit amax -> g_R, NVFP4 of R_S rows (16-blocks
//             along the compact axis) -> r_codes, r_scales, r_global
#include "device_common.h"
#include "kernels.h"

namespace nvfp4 {

constexpr int kGatherRows = 32;               // rows per gather / requant slot

int64_t resq_max_slots(int64_t rows_total, int64_t U) {
  return (rows_total + kScoreTileRows - 1) / kScoreTileRows + U;
}
int64_t resq_max_gather_slots(int64_t rows_total, int64_t U) {
  return (rows_total + kGatherRows - 1) / kGatherRows + U;
}

struct Units {
  const int64_t* offsets;   // NULL: unit u = rows [128u, 128u+128)
  int64_t U;
  int64_t rows_total;
  __device__ __forceinline__ void range(int64_t u, int64_t& b, int64_t& e) const {
    if (offsets) {
      b = offsets[u];
      e = offsets[u + 1];
      b = b < 0 ? 0 : (b > rows_total ? rows_total : b);
      e = e < b ? b : (e > rows_total ? rows_total : e);
    } else {
      b = u * kScoreTileRows;
      e = b + kScoreTileRows < rows_total ? b + kScoreTileRows : rows_total;
    }
  }
};

// ---------------------------------------------------------------------------
// block-wide exclusive scan of one uint32 per thread (blockDim multiple of 64)
// ---------------------------------------------------------------------------
__device__ __forceinline__ uint32_t block_exclusive_scan(uint32_t v, uint32_t* sh_waves,
                                                         uint32_t* total) {
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6, nw = blockDim.x >> 6;
  uint32_t inc = v;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    uint32_t t = __shfl_up(inc, o, 64);
    if (lane >= o) inc += t;
  }
  if (lane == 63) sh_waves[wid] = inc;
  __syncthreads();
  uint32_t base = 0, tot = 0;
  for (int w = 0; w < nw; ++w) {
    uint32_t s = sh_waves[w];
    if (w < wid) base += s;
    tot += s;
  }
  __syncthreads();
  *total = tot;
  return base + inc - v;
}

// ---------------------------------------------------------------------------
// plan
// ---------------------------------------------------------------------------
// Records: score tile t -> {unit, first row, the unit's end row, 0}; gather
// slot q -> {unit, first row, end row (at most 32 rows), the unit's first
// slot} {the unit's end slot, 0, 0, 0}.  Records past the last tile or slot
// (the grids are sized by upper bounds) get unit -1.
// A unit's thread writes its records itself, except for units of more than
// kPlanBigSlots gather slots (a hot expert's thousands of rows): the first
// kPlanBig of those go to a list in LDS, and after the scan whole waves write
// their records, one record per lane.
constexpr int kPlanBigSlots = 32, kPlanBig = 64;
struct PlanBigUnit {
  int64_t b, e;
  int32_t u, ts, nt, ss, ns;
};
__global__ __launch_bounds__(1024) void resq_plan_kernel(Units units, int32_t* tile_start,
                                                         int32_t* slot_start, int4* tile_info,
                                                         int64_t max_tiles, int4* slot_info,
                                                         int64_t max_slots) {
  __shared__ uint32_t sh[16];
  __shared__ PlanBigUnit big[kPlanBig];
  __shared__ int nbig;
  if (threadIdx.x == 0) nbig = 0;             // the scans' barriers order this before any use
  uint32_t carry_t = 0, carry_s = 0;
  for (int64_t base = 0; base < units.U; base += blockDim.x) {
    int64_t u = base + threadIdx.x;
    uint32_t nt = 0, ns = 0;
    int64_t b = 0, e = 0;
    if (u < units.U) {
      units.range(u, b, e);
      nt = (uint32_t)((e - b + kScoreTileRows - 1) / kScoreTileRows);
      ns = (uint32_t)((e - b + kGatherRows - 1) / kGatherRows);
    }
    uint32_t tot_t, tot_s;
    const uint32_t ex_t = block_exclusive_scan(nt, sh, &tot_t);
    const uint32_t ex_s = block_exclusive_scan(ns, sh, &tot_s);
    bool deferred = false;
    if (u < units.U && ns > (uint32_t)kPlanBigSlots) {
      const int j = atomicAdd(&nbig, 1);
      if (j < kPlanBig) {
        big[j] = PlanBigUnit{b, e, (int32_t)u, (int32_t)(carry_t + ex_t), (int32_t)nt,
                             (int32_t)(carry_s + ex_s), (int32_t)ns};
        deferred = true;
      }
    }
    if (u < units.U) {
      const int32_t ts = (int32_t)(carry_t + ex_t), ss = (int32_t)(carry_s + ex_s);
      tile_start[u] = ts;
      slot_start[u] = ss;
    }
    if (u < units.U && !deferred) {
      const int32_t ts = (int32_t)(carry_t + ex_t), ss = (int32_t)(carry_s + ex_s);
      for (uint32_t t = 0; t < nt; ++t)
        tile_info[ts + t] = int4{(int32_t)u, (int32_t)(b + (int64_t)t * kScoreTileRows), (int32_t)e, 0};
      for (uint32_t q = 0; q < ns; ++q) {
        const int64_t r0 = b + (int64_t)q * kGatherRows;
        slot_info[2 * (ss + q)] = int4{(int32_t)u, (int32_t)r0, (int32_t)(r0 + kGatherRows < e ? r0 + kGatherRows : e), ss};
        slot_info[2 * (ss + q) + 1] = int4{ss + (int32_t)ns, 0, 0, 0};
      }
    }
    carry_t += tot_t;
    carry_s += tot_s;
  }
  if (threadIdx.x == 0) {
    tile_start[units.U] = (int32_t)carry_t;
    slot_start[units.U] = (int32_t)carry_s;
  }
  __syncthreads();
  const int lane = threadIdx.x & 63, nb = nbig < kPlanBig ? nbig : kPlanBig;
  for (int j = threadIdx.x >> 6; j < nb; j += blockDim.x >> 6) {
    const PlanBigUnit g = big[j];
    for (int32_t t = lane; t < g.nt; t += 64)
      tile_info[g.ts + t] = int4{g.u, (int32_t)(g.b + (int64_t)t * kScoreTileRows), (int32_t)g.e, 0};
    for (int32_t q = lane; q < g.ns; q += 64) {
      const int64_t r0 = g.b + (int64_t)q * kGatherRows;
      slot_info[2 * (g.ss + q)] = int4{g.u, (int32_t)r0, (int32_t)(r0 + kGatherRows < g.e ? r0 + kGatherRows : g.e), g.ss};
      slot_info[2 * (g.ss + q) + 1] = int4{g.ss + g.ns, 0, 0, 0};
    }
  }
  for (int64_t t = carry_t + threadIdx.x; t < max_tiles; t += blockDim.x) tile_info[t] = int4{-1, 0, 0, 0};
  for (int64_t q = carry_s + threadIdx.x; q < max_slots; q += blockDim.x) slot_info[2 * q] = int4{-1, 0, 0, 0};
}

// ---------------------------------------------------------------------------
// scores: per-tile partial sums of |R|
// ---------------------------------------------------------------------------
template <typename T>
__device__ __forceinline__ void load16(const T* p, float* v);
template <>
__device__ __forceinline__ void load16<__bf16>(const __bf16* p, float* v) {
  const u32x4* q = reinterpret_cast<const u32x4*>(p);
  u32x4 a = q[0], b = q[1];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    v[2 * i] = bf16_lo(a[i]);
    v[2 * i + 1] = bf16_hi(a[i]);
    v[8 + 2 * i] = bf16_lo(b[i]);
    v[8 + 2 * i + 1] = bf16_hi(b[i]);
  }
}
template <>
__device__ __forceinline__ void load16<float>(const float* p, float* v) {
  const f32x4* q = reinterpret_cast<const f32x4*>(p);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    f32x4 a = q[i];
    v[4 * i] = a[0]; v[4 * i + 1] = a[1]; v[4 * i + 2] = a[2]; v[4 * i + 3] = a[3];
  }
}

template <typename T>
__device__ __forceinline__ float load1(const T* p) {
  if constexpr (sizeof(T) == 2) {
    return __uint_as_float((uint32_t)(*reinterpret_cast<const uint16_t*>(p)) << 16);
  } else {
    return *p;
  }
}

// Contiguous rows (no row index): one workgroup per (128-row tile of a unit,
// 64 channels).  Thread t computes |R| of block column t % 4 for rows t / 4
// and t / 4 + 64 (loads first, then arithmetic) into LDS; then threads 0..63
// add one channel each over the tile's rows in increasing row order (missing
// rows add +0, which changes no fp32 sum).  The whole tile's loads go out at
// once, which suits rows streamed from HBM once.
constexpr int kScoreCols = 64;
constexpr int kScoreBlocks = kScoreCols / kBlock;
constexpr int kAbsStride = kScoreCols + 4;

// MX: the operand is MXFP4 (E8M0 scale per 32-block, no global scale; gp
// unused), else NVFP4 (E4M3 per 16-block times *gp).
template <typename T, bool MX>
__global__ __launch_bounds__(256) void resq_scores_tile_kernel(
    const T* __restrict__ x, int64_t x_rows, int64_t K, int64_t ldx,
    const int32_t* __restrict__ row_index, const uint8_t* __restrict__ codes,
    const uint8_t* __restrict__ scales, const float* __restrict__ gp,
    const int4* __restrict__ tile_info, float* __restrict__ partials) {
  __shared__ float absr[kScoreTileRows * kAbsStride];
  const int64_t slot = blockIdx.y;
  const int4 ti = tile_info[slot];
  if (ti.x < 0) return;
  const int tid = threadIdx.x;
  const int64_t nb = K / kBlock;
  const int bl = tid % kScoreBlocks, rsub = tid / kScoreBlocks;
  const int64_t bc = (int64_t)blockIdx.x * kScoreBlocks + bl;
  const int64_t r0 = ti.y, e = ti.z;
  const float g = MX ? 1.0f : *gp;
  const int64_t nsb = MX ? K / kMxBlock : nb;           // scale bytes per row
  float v[2][16];
  u32x2 w[2];
  uint32_t sb[2];
  bool live[2];
#pragma unroll
  for (int j = 0; j < 2; ++j) {                  // all loads first
    const int64_t r = r0 + rsub + 64 * j;
    const int64_t xr = r < e ? (row_index ? (int64_t)row_index[r] : r) : -1;
    live[j] = xr >= 0 && xr < x_rows && bc < nb;
    if (live[j]) {
      load16<T>(x + xr * ldx + bc * kBlock, v[j]);
      w[j] = *reinterpret_cast<const u32x2*>(codes + xr * (K / 2) + bc * 8);
      sb[j] = scales[xr * nsb + (MX ? bc >> 1 : bc)];
    }
  }
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int rl = rsub + 64 * j;
    float res[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) res[i] = 0.0f;
    if (live[j]) {
      const float S = MX ? e8m0_value(sb[j]) : e4m3_value(sb[j]) * g;
      float f[16];
      e2m1_unpack8(w[j][0], f);
      e2m1_unpack8(w[j][1], f + 8);
#pragma unroll
      for (int i = 0; i < 16; ++i) res[i] = fabsf(v[j][i] - f[i] * S);   // exact; no contraction
    }
    f32x4* dst = reinterpret_cast<f32x4*>(absr + rl * kAbsStride + bl * kBlock);
#pragma unroll
    for (int i = 0; i < 4; ++i) dst[i] = f32x4{res[4 * i], res[4 * i + 1], res[4 * i + 2], res[4 * i + 3]};
  }
  __syncthreads();
  const int64_t c = (int64_t)blockIdx.x * kScoreCols + tid;
  if (tid < kScoreCols && c < K) {
    float sum = 0.0f;
#pragma unroll 16
    for (int rl = 0; rl < kScoreTileRows; ++rl) sum = sum + absr[rl * kAbsStride + tid];
    partials[slot * K + c] = sum;
  }
}

// Gathered rows (a row index, each row read by every unit that it is routed
// to, mostly from cache): one wave per (128-row tile of a unit, 512
// channels), four tiles per workgroup.  Lane l owns channels c0 + 8l .. c0 + 8l + 7 and adds |R| of
// the tile's rows into its eight sums in increasing row order (rows past the
// unit's end, or whose index lies outside x, add nothing, which changes no
// fp32 sum); the rows go eight at a time, their loads (16 or 32 bytes of x,
// one code word and one scale byte per lane) issued before their additions.
// No LDS and no barrier: every lane of every wave works through the sum.  On
// the 8192-token layer's X (65536 gathered rows of 4096 channels) this took
// 0.09 ms where the tile kernel above took 0.16; on contiguous rows the tile
// kernel is the faster one.
constexpr int kScoreLaneCols = 8;
constexpr int kScoreWaveCols = 64 * kScoreLaneCols;
constexpr int kScoreBatch = 8;
// MX: as in the tile kernel above.
template <typename T, bool MX>
__global__ __launch_bounds__(256) void resq_scores_rows_kernel(
    const T* __restrict__ x, int64_t x_rows, int64_t K, int64_t ldx,
    const int32_t* __restrict__ row_index, const uint8_t* __restrict__ codes,
    const uint8_t* __restrict__ scales, const float* __restrict__ gp,
    const int4* __restrict__ tile_info, int64_t slots, float* __restrict__ partials) {
  constexpr int XW = sizeof(T) / 2;                      // 16-byte words of x per lane and row
  const int lane = threadIdx.x & 63;
  // The wave's tile, hence its rows and their row indexes, are the same for
  // all its lanes: kept uniform, they come through scalar loads and the row
  // addresses are scalar arithmetic.
  const int64_t slot = (int64_t)blockIdx.y * 4 + __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
  if (slot >= slots) return;
  const int4 ti = tile_info[slot];
  if (ti.x < 0) return;
  const int64_t c = (int64_t)blockIdx.x * kScoreWaveCols + lane * kScoreLaneCols;
  if (c >= K) return;                                    // K % 16 == 0: all eight channels exist
  const float g = MX ? 1.0f : *gp;
  const int64_t nsb = MX ? K / kMxBlock : K / kBlock;    // scale bytes per row
  const int64_t sc = MX ? c / kMxBlock : c / kBlock;
  const int64_t r0 = ti.y;
  const int nr = (int)(ti.z - r0 < kScoreTileRows ? ti.z - r0 : kScoreTileRows);
  float acc[kScoreLaneCols];
#pragma unroll
  for (int i = 0; i < kScoreLaneCols; ++i) acc[i] = 0.0f;
  for (int i0 = 0; i0 < nr; i0 += kScoreBatch) {
    u32x4 xv[kScoreBatch][XW];
    uint32_t cw[kScoreBatch], sb[kScoreBatch];
    bool live[kScoreBatch];
#pragma unroll
    for (int q = 0; q < kScoreBatch; ++q) {              // all loads first
      const int64_t r = r0 + i0 + q;
      const int64_t xr = i0 + q < nr ? (row_index ? (int64_t)row_index[r] : r) : -1;
      live[q] = xr >= 0 && xr < x_rows;
      if (live[q]) {
        const u32x4* src = reinterpret_cast<const u32x4*>(x + xr * ldx + c);
#pragma unroll
        for (int w = 0; w < XW; ++w) xv[q][w] = src[w];
        cw[q] = *reinterpret_cast<const uint32_t*>(codes + xr * (K / 2) + c / 2);
        sb[q] = scales[xr * nsb + sc];
      }
    }
#pragma unroll
    for (int q = 0; q < kScoreBatch; ++q) {              // then the sums, in row order
      if (!live[q]) continue;
      const float S = MX ? e8m0_value(sb[q]) : e4m3_value(sb[q]) * g;
      float f[8], v[8];
      e2m1_unpack8(cw[q], f);
      if constexpr (XW == 1) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          v[2 * i] = bf16_lo(xv[q][0][i]);
          v[2 * i + 1] = bf16_hi(xv[q][0][i]);
        }
      } else {
#pragma unroll
        for (int i = 0; i < 8; ++i) v[i] = __uint_as_float(xv[q][i >> 2][i & 3]);
      }
#pragma unroll
      for (int i = 0; i < 8; ++i) acc[i] = acc[i] + fabsf(v[i] - f[i] * S);   // exact; no contraction
    }
  }
  f32x4* dst = reinterpret_cast<f32x4*>(partials + slot * K + c);
  dst[0] = f32x4{acc[0], acc[1], acc[2], acc[3]};
  dst[1] = f32x4{acc[4], acc[5], acc[6], acc[7]};
}

// ---------------------------------------------------------------------------
// select: scores -> top-k (ties to the lower index) -> ascending channel list
// ---------------------------------------------------------------------------
// Block-wide sum of one uint32 per thread (256 threads); all threads get it.
__device__ __forceinline__ uint32_t block_sum256(uint32_t v, uint32_t* sh4) {
  v = wave_sum_u32(v);
  __syncthreads();
  if ((threadIdx.x & 63) == 0) sh4[threadIdx.x >> 6] = v;
  __syncthreads();
  return sh4[0] + sh4[1] + sh4[2] + sh4[3];
}

// Wave-level sum and exclusive prefix of small counts (0 <= v < 2^BITS) from
// bit-plane ballots: no lane shuffles, each bit plane is one ballot, its
// population count and mbcnt (the set bits below this lane).
template <int BITS>
__device__ __forceinline__ uint32_t wave_scan_small(uint32_t v, uint32_t* total) {
  uint32_t pre = 0, tot = 0;
#pragma unroll
  for (int b = 0; b < BITS; ++b) {
    const unsigned long long m = __ballot((v >> b) & 1u);
    pre += __builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0u)) << b;
    tot += (uint32_t)__popcll(m) << b;
  }
  *total = tot;
  return pre;
}

// Workgroup (4 waves) sums of three counts (each below 2^16 over a wave)
// with one barrier: two DPP wave sums (a and b packed in one word), the wave
// totals to sh[parity], and callers alternate the parity, so a slot is
// rewritten only after the next call's barrier, which every reader of it has
// passed.
__device__ __forceinline__ void block_sum3(uint32_t& a, uint32_t& b, uint32_t& c,
                                           uint32_t (*sh)[3][4], int parity) {
  const uint32_t ab = wave_sum_dpp(a | (b << 16)), cc = wave_sum_dpp(c);
  const int w = threadIdx.x >> 6;
  if ((threadIdx.x & 63) == 0) {
    sh[parity][0][w] = ab;
    sh[parity][1][w] = cc;
  }
  __syncthreads();
  uint32_t ta = 0, tb = 0, tc = 0;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const uint32_t t = sh[parity][0][i];
    ta += t & 0xFFFFu;
    tb += t >> 16;
    tc += sh[parity][1][i];
  }
  a = ta;
  b = tb;
  c = tc;
}

// Workgroup (4 waves) exclusive prefix and total of a small count, with the
// same alternating-parity slots (sh[parity][0..3]).
template <int BITS>
__device__ __forceinline__ uint32_t block_scan_small(uint32_t v, uint32_t* total, uint32_t (*sh)[3][4],
                                                     int parity) {
  uint32_t wt;
  const uint32_t pre = wave_scan_small<BITS>(v, &wt);
  const int w = threadIdx.x >> 6;
  if ((threadIdx.x & 63) == 0) sh[parity][0][w] = wt;
  __syncthreads();
  uint32_t base = 0, tot = 0;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const uint32_t t = sh[parity][0][i];
    base += i < w ? t : 0u;
    tot += t;
  }
  *total = tot;
  return base + pre;
}

// Top-k of the scores held in registers: thread t owns channels [c0, c0 +
// n_my) (c0 = t CH) as non-negative float bits key[].  The k-th largest key T
// is found two bits per pass: the three candidates T | d << lo (d = 1..3) are
// counted together and the largest with at least k keys >= it is kept (16
// passes for the 31 bits of a non-negative float).  Then keys > T, and keys
// == T in channel order up to k, are written in ascending channel order to
// out (and to out_lds when given).  All 256 threads call it.
template <int CH>
__device__ __forceinline__ void topk_reg(const uint32_t (&key)[CH], int n_my, int64_t c0, int32_t k,
                                         int32_t* __restrict__ out, int32_t* out_lds,
                                         uint32_t (*sh)[3][4]) {
  // per-thread counts are at most CH (<= 32): 6 bit planes
  constexpr int kBits = 6;
  uint32_t T = 0;
  int parity = 0;
  for (int hi = 30; hi >= 0; hi -= 2) {       // bits hi and hi - 1; the last pass bit 0 alone
    const int lo = hi > 0 ? hi - 1 : 0;
    const uint32_t c1 = T | (1u << lo), c2 = T | (2u << lo), c3 = T | (3u << lo);
    uint32_t n1 = 0, n2 = 0, n3 = 0;
#pragma unroll
    for (int j = 0; j < CH; ++j) {            // padding keys (0) are below every candidate
      n1 += (uint32_t)(key[j] >= c1);
      n2 += (uint32_t)(key[j] >= c2);
      n3 += (uint32_t)(key[j] >= c3);
    }
    block_sum3(n1, n2, n3, sh, parity);
    parity ^= 1;
    if (hi > 0 && n3 >= (uint32_t)k) T = c3;
    else if (hi > 0 && n2 >= (uint32_t)k) T = c2;
    else if (n1 >= (uint32_t)k) T = c1;
  }
  uint32_t n_gt = 0, n_eq = 0;
#pragma unroll
  for (int j = 0; j < CH; ++j) {              // branch-free: padding keys are not channels
    const uint32_t valid = (uint32_t)(j < n_my);
    n_gt += valid & (uint32_t)(key[j] > T);
    n_eq += valid & (uint32_t)(key[j] == T);
  }
  uint32_t tot_gt, tot_eq;
  block_scan_small<kBits>(n_gt, &tot_gt, sh, parity);
  parity ^= 1;
  const uint32_t remaining = (uint32_t)k - tot_gt;            // keys == T to take
  const uint32_t eq_before = block_scan_small<kBits>(n_eq, &tot_eq, sh, parity);
  parity ^= 1;
  uint32_t take = 0, n_sel = 0, eq_seen = eq_before;   // take: bit j = channel c0 + j selected
#pragma unroll
  for (int j = 0; j < CH; ++j) {
    const uint32_t valid = (uint32_t)(j < n_my);
    const uint32_t is_eq = valid & (uint32_t)(key[j] == T);
    const uint32_t t = valid & ((uint32_t)(key[j] > T) | (is_eq & (uint32_t)(eq_seen < remaining)));
    eq_seen += is_eq;
    take |= t << j;
    n_sel += t;
  }
  uint32_t tot;
  uint32_t pos = block_scan_small<kBits>(n_sel, &tot, sh, parity);
  while (take) {                              // ascending channel order
    const int j = __builtin_ctz(take);
    take &= take - 1;
    if (pos < (uint32_t)k) {
      if (out_lds) out_lds[pos] = (int32_t)(c0 + j);
      out[pos++] = (int32_t)(c0 + j);
    }
  }
}

// Selection with the keys in registers (K <= 256 CH): thread t adds the tile
// sums of channels [t CH, t CH + CH) in tile order, then topk_reg.
template <int CH>
__global__ __launch_bounds__(256) void resq_select_reg_kernel(
    const float* __restrict__ partials, int64_t K, Units units,
    const int32_t* __restrict__ tile_start, int32_t k, int32_t* __restrict__ sel_idx,
    float* __restrict__ r_global) {
  __shared__ uint32_t sh[2][3][4];
  const int64_t u = blockIdx.x;
  const int tid = threadIdx.x;
  int64_t b, e;
  units.range(u, b, e);
  int32_t* out = sel_idx + u * k;
  if (e == b) {                               // empty unit: channels 0..k-1, g_R = 1
    for (int j = tid; j < k; j += blockDim.x) out[j] = j;
    if (tid == 0 && r_global) r_global[u] = 1.0f;   // NULL for MXFP4 (no global scale)
    return;
  }
  const int64_t t0 = tile_start[u], t1 = tile_start[u + 1];
  const int64_t c0 = (int64_t)tid * CH;
  const int n_my = (int)(c0 >= K ? 0 : (c0 + CH <= K ? CH : K - c0));
  float acc[CH];
#pragma unroll
  for (int j = 0; j < CH; ++j) acc[j] = 0.0f;
  if (n_my == CH) {                           // K % 16 == 0: whole 16-byte groups
    // NB tiles' loads go out before their additions (a unit of many tiles,
    // e.g. a hot expert's 124, would otherwise wait out one round trip per
    // tile); the additions keep the tile order.
    constexpr int NB = 128 / CH;
    int64_t t = t0;
    for (; t + NB <= t1; t += NB) {
      f32x4 v[NB][CH / 4];
#pragma unroll
      for (int bt = 0; bt < NB; ++bt)
#pragma unroll
        for (int q = 0; q < CH / 4; ++q)
          v[bt][q] = reinterpret_cast<const f32x4*>(partials + (t + bt) * K + c0)[q];
#pragma unroll
      for (int bt = 0; bt < NB; ++bt)
#pragma unroll
        for (int q = 0; q < CH / 4; ++q)
#pragma unroll
          for (int i = 0; i < 4; ++i) acc[4 * q + i] = acc[4 * q + i] + v[bt][q][i];
    }
    for (; t < t1; ++t) {                     // the rest, in tile order
      const f32x4* src = reinterpret_cast<const f32x4*>(partials + t * K + c0);
#pragma unroll
      for (int q = 0; q < CH / 4; ++q) {
        const f32x4 v = src[q];
#pragma unroll
        for (int i = 0; i < 4; ++i) acc[4 * q + i] = acc[4 * q + i] + v[i];
      }
    }
  } else {
    for (int64_t t = t0; t < t1; ++t)
#pragma unroll
      for (int j = 0; j < CH; ++j)
        if (j < n_my) acc[j] = acc[j] + partials[t * K + c0 + j];
  }
  uint32_t key[CH];
#pragma unroll
  for (int j = 0; j < CH; ++j) key[j] = __float_as_uint(acc[j]);
  topk_reg<CH>(key, n_my, c0, k, out, nullptr, sh);
}

// Keys live in LDS chunk by chunk: thread t owns channels [t*chunk, (t+1)*chunk)
// stored at t*(chunk+1) + j, one pad word per chunk so that the 64 lanes of a
// wave reading "their" j-th key hit different banks.
__global__ __launch_bounds__(256) void resq_select_kernel(
    const float* __restrict__ partials, int64_t K, Units units,
    const int32_t* __restrict__ tile_start, int32_t k, int32_t* __restrict__ sel_idx,
    float* __restrict__ r_global) {
  extern __shared__ uint32_t keys[];          // [256 * (chunk + 1)] score bits (scores >= +0)
  __shared__ uint32_t sh_waves[4];
  const int64_t u = blockIdx.x;
  const int tid = threadIdx.x;
  int64_t b, e;
  units.range(u, b, e);
  int32_t* out = sel_idx + u * k;
  if (e == b) {                               // empty unit: channels 0..k-1, g_R = 1
    for (int j = tid; j < k; j += blockDim.x) out[j] = j;
    if (tid == 0 && r_global) r_global[u] = 1.0f;   // NULL for MXFP4 (no global scale)
    return;
  }
  const int chunk = (int)((K + blockDim.x - 1) / blockDim.x);
  const int64_t t0 = tile_start[u], t1 = tile_start[u + 1];
  for (int64_t c = tid; c < K; c += blockDim.x) {
    float s = 0.0f;
    for (int64_t t = t0; t < t1; ++t) s = s + partials[t * K + c];   // tile order
    keys[(c / chunk) * (chunk + 1) + c % chunk] = __float_as_uint(s);
  }
  __syncthreads();
  const uint32_t* my = keys + tid * (chunk + 1);
  const int64_t c0 = (int64_t)tid * chunk;
  const int n_my = (int)(c0 >= K ? 0 : (c0 + chunk <= K ? chunk : K - c0));

  // The k-th largest key T, one bit at a time from the top: T is the largest
  // value with at least k keys >= T.  Non-negative float bits order like the
  // floats, and bit 31 (sign) is 0.
  uint32_t T = 0;
  for (int bit = 30; bit >= 0; --bit) {
    const uint32_t cand = T | (1u << bit);
    uint32_t n = 0;
    for (int j = 0; j < n_my; ++j) n += my[j] >= cand;
    if (block_sum256(n, sh_waves) >= (uint32_t)k) T = cand;
  }
  uint32_t n_gt = 0, n_eq = 0;
  for (int j = 0; j < n_my; ++j) {
    n_gt += my[j] > T;
    n_eq += my[j] == T;
  }
  const uint32_t remaining = (uint32_t)k - block_sum256(n_gt, sh_waves);   // keys == T to take

  // selection in index order: thread owns the contiguous chunk [c0, c0 + n_my)
  uint32_t tot;
  const uint32_t eq_before = block_exclusive_scan(n_eq, sh_waves, &tot);
  uint32_t n_sel = 0;
  {
    uint32_t eq_seen = eq_before;
    for (int j = 0; j < n_my; ++j) {
      const uint32_t key = my[j];
      if (key > T) ++n_sel;
      else if (key == T && eq_seen++ < remaining) ++n_sel;
    }
  }
  uint32_t pos = block_exclusive_scan(n_sel, sh_waves, &tot);
  {
    uint32_t eq_seen = eq_before;
    for (int j = 0; j < n_my; ++j) {
      const uint32_t key = my[j];
      const bool take = key > T || (key == T && eq_seen++ < remaining);
      if (take && pos < (uint32_t)k) out[pos++] = (int32_t)(c0 + j);
    }
  }
}

// ---------------------------------------------------------------------------
// gather R_S and per-slot max |R_S|
// ---------------------------------------------------------------------------
// One workgroup per 32-row slot.  The slot's row indexes and the unit's
// selected channels go to LDS first; then every thread issues the loads of
// its (row, channel) elements in batches of 8 before any arithmetic, so a
// thread waits for one memory round trip per batch, not per element.  Rows
// with a bad index read nothing and give R_S = 0.
template <typename T, bool MX>
__global__ __launch_bounds__(256) void resq_gather_kernel(
    const T* __restrict__ x, int64_t x_rows, int64_t K, int64_t ldx,
    const int32_t* __restrict__ row_index, const uint8_t* __restrict__ codes,
    const uint8_t* __restrict__ scales, const float* __restrict__ gp,
    const int4* __restrict__ slot_info, const int32_t* __restrict__ sel_idx, int32_t k,
    float* __restrict__ r_s, float* __restrict__ amax_part) {
  extern __shared__ int32_t sel[];           // [k]
  __shared__ int32_t xrow[kGatherRows];
  __shared__ float red[4];
  const int64_t slot = blockIdx.x;
  const int4 si = slot_info[2 * slot];
  const int u = si.x;
  if (u < 0) return;
  const int64_t r0 = si.y;
  const int nrows = si.z - si.y;
  const float g = MX ? 1.0f : *gp;
  for (int j = threadIdx.x; j < k; j += blockDim.x) {
    int32_t c = sel_idx[(int64_t)u * k + j];
    sel[j] = c < 0 ? 0 : (c >= K ? (int32_t)(K - 1) : c);
  }
  if ((int)threadIdx.x < nrows) {
    const int64_t r = r0 + threadIdx.x;
    const int64_t xr = row_index ? (int64_t)row_index[r] : r;
    xrow[threadIdx.x] = xr >= 0 && xr < x_rows ? (int32_t)xr : -1;
  }
  __syncthreads();
  const int64_t nb = K / (MX ? kMxBlock : kBlock);
  constexpr int B = 8;
  float m = 0.0f;
  const int n = nrows * k;
  for (int i0 = 0; i0 < n; i0 += 256 * B) {
    float xv[B];
    uint32_t cb[B], sbyte[B];
    int rl[B], j[B], c[B], xr[B];
#pragma unroll
    for (int q = 0; q < B; ++q) {             // the batch's loads
      const int i = i0 + (int)threadIdx.x + 256 * q;
      const int ii = i < n ? i : n - 1;
      rl[q] = ii / k;
      j[q] = ii - rl[q] * k;
      xr[q] = xrow[rl[q]];
      c[q] = sel[j[q]];
      xv[q] = 0.0f;
      cb[q] = 0;
      sbyte[q] = 0;
      if (xr[q] >= 0) {
        const int64_t xe = xr[q];
        xv[q] = load1<T>(x + xe * ldx + c[q]);
        cb[q] = codes[xe * (K / 2) + (c[q] >> 1)];
        sbyte[q] = scales[xe * nb + (c[q] >> (MX ? 5 : 4))];
      }
    }
#pragma unroll
    for (int q = 0; q < B; ++q) {
      const int i = i0 + (int)threadIdx.x + 256 * q;
      if (i < n) {
        float res = 0.0f;
        if (xr[q] >= 0) {
          const uint32_t code = (cb[q] >> (4 * (c[q] & 1))) & 15u;
          const float S = MX ? e8m0_value(sbyte[q]) : e4m3_value(sbyte[q]) * g;
          res = xv[q] - dq(code, S);
        }
        r_s[(r0 + rl[q]) * k + j[q]] = res;
        m = fmaxf(m, fabsf(res));
      }
    }
  }
  m = wave_max(m);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = m;
  __syncthreads();
  if (threadIdx.x == 0) {
    float t = red[0];
    for (int w = 1; w < (int)(blockDim.x >> 6); ++w) t = fmaxf(t, red[w]);
    amax_part[slot] = t;
  }
}

// ---------------------------------------------------------------------------
// requantize R_S with the unit's own global scale
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void resq_requant_kernel(
    const float* __restrict__ r_s, const int4* __restrict__ slot_info,
    const float* __restrict__ amax_part, int32_t k, uint8_t* __restrict__ r_codes,
    uint8_t* __restrict__ r_scales, float* __restrict__ r_global) {
  __shared__ float sh_g;
  const int64_t slot = blockIdx.x;
  const int4 si = slot_info[2 * slot];
  const int u = si.x;
  if (u < 0) return;
  const int s_end = slot_info[2 * slot + 1].x;
  if (threadIdx.x < 64) {
    float m = 0.0f;
    for (int t = si.w + (int)threadIdx.x; t < s_end; t += 64)
      m = fmaxf(m, amax_part[t]);
    m = wave_max(m);
    if (threadIdx.x == 0) sh_g = global_scale_from_amax(m);
  }
  __syncthreads();
  const float g = sh_g;
  const BlockScaler bsc = make_block_scaler(g);
  if (slot == si.w && threadIdx.x == 0) r_global[u] = g;
  const int64_t r0 = si.y, r1 = si.z;
  const int kb = k / kBlock;
  const int64_t n = (r1 - r0) * kb;
  for (int64_t i = threadIdx.x; i < n; i += blockDim.x) {
    const int64_t r = r0 + i / kb;
    const int bl = (int)(i % kb);
    float v[16];
    load16<float>(r_s + r * k + bl * kBlock, v);
    uint32_t sb, w0, w1;
    quantize_block16(v, bsc, &sb, &w0, &w1);
    *reinterpret_cast<u32x2*>(r_codes + r * (k / 2) + bl * 8) = u32x2{w0, w1};
    r_scales[r * kb + bl] = (uint8_t)sb;
  }
}

// Dense-mask form: Q(R * M), the residual of the selected channels at their
// own positions and zeros elsewhere, quantized along K with the unit's own
// global scale.  R * M has the same nonzero entries as R_S, so the slots'
// amax of |R_S| give its global scale.  pos[c] is the compact index of
// channel c, or -1 outside the mask (K <= kMaskMaxK).
constexpr int kMaskMaxK = 16384;
__global__ __launch_bounds__(256) void resq_mask_requant_kernel(
    const float* __restrict__ r_s, const int4* __restrict__ slot_info,
    const float* __restrict__ amax_part, const int32_t* __restrict__ sel_idx, int32_t k, int64_t K,
    uint8_t* __restrict__ m_codes, uint8_t* __restrict__ m_scales, float* __restrict__ m_global) {
  __shared__ int16_t pos[kMaskMaxK];
  __shared__ float sh_g;
  const int64_t slot = blockIdx.x;
  const int4 si = slot_info[2 * slot];
  const int u = si.x;
  if (u < 0) return;
  const int s_end = slot_info[2 * slot + 1].x;
  for (int64_t c = threadIdx.x; c < K; c += blockDim.x) pos[c] = -1;
  __syncthreads();
  for (int j = threadIdx.x; j < k; j += blockDim.x) {
    int32_t c = sel_idx[(int64_t)u * k + j];
    c = c < 0 ? 0 : (c >= K ? (int32_t)(K - 1) : c);
    pos[c] = (int16_t)j;
  }
  if (threadIdx.x < 64) {
    float m = 0.0f;
    for (int t = si.w + (int)threadIdx.x; t < s_end; t += 64)
      m = fmaxf(m, amax_part[t]);
    m = wave_max(m);
    if (threadIdx.x == 0) sh_g = global_scale_from_amax(m);
  }
  __syncthreads();
  const float g = sh_g;
  const BlockScaler bsc = make_block_scaler(g);
  if (slot == si.w && threadIdx.x == 0) m_global[u] = g;
  const int64_t r0 = si.y, r1 = si.z;
  const int64_t kb = K / kBlock;
  const int64_t n = (r1 - r0) * kb;
  for (int64_t i = threadIdx.x; i < n; i += blockDim.x) {
    const int64_t r = r0 + i / kb;
    const int64_t bl = i % kb;
    float v[16];
#pragma unroll
    for (int q = 0; q < 16; ++q) {
      const int j = pos[bl * kBlock + q];
      v[q] = j >= 0 ? r_s[r * k + j] : 0.0f;
    }
    uint32_t sb, w0, w1;
    quantize_block16(v, bsc, &sb, &w0, &w1);
    *reinterpret_cast<u32x2*>(m_codes + r * (K / 2) + bl * 8) = u32x2{w0, w1};
    m_scales[r * kb + bl] = (uint8_t)sb;
  }
}

// MXFP4 of R_S: 32-blocks along the compact axis, each with its own E8M0
// scale; no global scale.
__global__ __launch_bounds__(256) void resq_requant_mx_kernel(
    const float* __restrict__ r_s, const int4* __restrict__ slot_info, int32_t k,
    uint8_t* __restrict__ r_codes, uint8_t* __restrict__ r_scales) {
  const int64_t slot = blockIdx.x;
  const int4 si = slot_info[2 * slot];
  if (si.x < 0) return;
  const int64_t r0 = si.y, r1 = si.z;
  const int kb = k / kMxBlock;
  const int64_t n = (r1 - r0) * kb;
  for (int64_t i = threadIdx.x; i < n; i += blockDim.x) {
    const int64_t r = r0 + i / kb;
    const int bl = (int)(i % kb);
    float v[32];
    load16<float>(r_s + r * k + bl * kMxBlock, v);
    load16<float>(r_s + r * k + bl * kMxBlock + 16, v + 16);
    float amax = 0.0f;
#pragma unroll
    for (int q = 0; q < 32; ++q) amax = fmaxf(amax, fabsf(v[q]));
    const uint32_t sb = mx_scale_byte(amax);
    uint32_t w[4];
    mx_pack32(v, sb, w);
    *reinterpret_cast<u32x4*>(r_codes + r * (k / 2) + bl * 16) = u32x4{w[0], w[1], w[2], w[3]};
    r_scales[r * kb + bl] = (uint8_t)sb;
  }
}

// ---------------------------------------------------------------------------
// small units: the whole step in one workgroup per unit
// ---------------------------------------------------------------------------
// Where the units hold a few rows each (decode batches), one workgroup per
// unit runs the scores, the selection, the gather and the requantization in
// one launch, with the unit's rows in L2.  The arithmetic and its order are
// those of the kernels above: a score is the fp32 sum of |R| over each
// 128-row tile in row order, the tile sums added in tile order; the selection
// is topk_reg; R_S = x - DQ at the selected channels; the unit's max |R_S|
// gives g_R and quantize_block16 the codes.  Thread t owns the score
// channels [t CH, t CH + CH) (CH = 8 for K <= 2048, 16 for K <= 4096).  R_S
// stays in LDS when the unit's rows x k fit in kSmallRs floats, else it is
// computed again (the same values) for the requantization.
constexpr int kSmallRs = 8192;
constexpr int kSmallMaxK = 4096;

template <typename T, int CH>
__device__ __forceinline__ void load_ch(const T* p, float* v) {
  static_assert(CH == 8 || CH == 16, "channels per thread");
  if constexpr (sizeof(T) == 2) {
#pragma unroll
    for (int h = 0; h < CH / 8; ++h) {
      const u32x4 a = reinterpret_cast<const u32x4*>(p)[h];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        v[8 * h + 2 * i] = bf16_lo(a[i]);
        v[8 * h + 2 * i + 1] = bf16_hi(a[i]);
      }
    }
  } else {
#pragma unroll
    for (int h = 0; h < CH / 4; ++h) {
      const f32x4 a = reinterpret_cast<const f32x4*>(p)[h];
#pragma unroll
      for (int i = 0; i < 4; ++i) v[4 * h + i] = a[i];
    }
  }
}

template <typename T, int CH>
__global__ __launch_bounds__(256) void resq_small_kernel(
    const T* __restrict__ x, int64_t x_rows, int64_t K, int64_t ldx,
    const int32_t* __restrict__ row_index, const uint8_t* __restrict__ codes,
    const uint8_t* __restrict__ scales, const float* __restrict__ gp, Units units, int32_t k,
    int32_t* __restrict__ sel_idx, uint8_t* __restrict__ r_codes, uint8_t* __restrict__ r_scales,
    float* __restrict__ r_global) {
  __shared__ int32_t xrow[kScoreTileRows];
  __shared__ int32_t sel[kSmallMaxK];
  __shared__ float rs[kSmallRs];
  __shared__ uint32_t sh[2][3][4];
  __shared__ float red[4];
  const int u = blockIdx.x;
  const int tid = threadIdx.x;
  int64_t b, e;
  units.range(u, b, e);
  int32_t* out = sel_idx + (int64_t)u * k;
  if (e == b) {                               // empty unit: channels 0..k-1, g_R = 1
    for (int j = tid; j < k; j += blockDim.x) out[j] = j;
    if (tid == 0) r_global[u] = 1.0f;
    return;
  }
  const float g = *gp;
  const int64_t nb = K / kBlock;
  const int64_t c0 = (int64_t)tid * CH;
  const bool mine = c0 < K;                   // K % 16 == 0: whole groups of CH
  // x row indexes of the unit rows [t0, t0 + nr) into xrow (-1: bad index)
  auto load_rows = [&](int64_t t0, int nr) {
    __syncthreads();                          // earlier readers of xrow are done
    if (tid < nr) {
      const int64_t r = t0 + tid;
      const int64_t xr = row_index ? (int64_t)row_index[r] : r;
      xrow[tid] = xr >= 0 && xr < x_rows ? (int32_t)xr : -1;
    }
    __syncthreads();
  };

  // ---- scores
  float total[CH];
#pragma unroll
  for (int i = 0; i < CH; ++i) total[i] = 0.0f;
  for (int64_t t0 = b; t0 < e; t0 += kScoreTileRows) {
    const int nr = (int)(e - t0 < kScoreTileRows ? e - t0 : kScoreTileRows);
    load_rows(t0, nr);
    float ts[CH];
#pragma unroll
    for (int i = 0; i < CH; ++i) ts[i] = 0.0f;
    if (mine) {
      for (int rb = 0; rb < nr; rb += 8) {    // 8 rows' loads, then their arithmetic
        float v[8][CH];
        uint32_t cw[8][CH / 8], sb[8];
#pragma unroll
        for (int q = 0; q < 8; ++q) {
          const int xr = rb + q < nr ? xrow[rb + q] : -1;
          if (xr >= 0) {
            load_ch<T, CH>(x + (int64_t)xr * ldx + c0, v[q]);
            const uint32_t* cp = reinterpret_cast<const uint32_t*>(codes + (int64_t)xr * (K / 2) + c0 / 2);
#pragma unroll
            for (int h = 0; h < CH / 8; ++h) cw[q][h] = cp[h];
            sb[q] = scales[(int64_t)xr * nb + c0 / kBlock];
          } else {                            // a bad index scores |0 - 0| = 0
#pragma unroll
            for (int i = 0; i < CH; ++i) v[q][i] = 0.0f;
#pragma unroll
            for (int h = 0; h < CH / 8; ++h) cw[q][h] = 0;
            sb[q] = 0;
          }
        }
#pragma unroll
        for (int q = 0; q < 8; ++q) {
          if (rb + q < nr) {
            const float S = e4m3_value(sb[q]) * g;
            float f[CH];
#pragma unroll
            for (int h = 0; h < CH / 8; ++h) e2m1_unpack8(cw[q][h], f + 8 * h);
#pragma unroll
            for (int i = 0; i < CH; ++i) ts[i] = ts[i] + fabsf(v[q][i] - f[i] * S);   // exact; no contraction
          }
        }
      }
    }
#pragma unroll
    for (int i = 0; i < CH; ++i) total[i] = total[i] + ts[i];
  }

  // ---- selection (ascending channel list in out and in sel)
  uint32_t key[CH];
#pragma unroll
  for (int i = 0; i < CH; ++i) key[i] = __float_as_uint(total[i]);
  topk_reg<CH>(key, mine ? CH : 0, c0, k, out, sel, sh);

  // ---- R_S of (row, 16-channel block) items and the unit's max |R_S|
  const int kb = k / kBlock;
  const int64_t n = e - b;
  const bool keep = n * k <= kSmallRs;
  auto r_item = [&](int xr, int bl, float* R) {
    float xv[kBlock];
    uint32_t cb[kBlock], sbb[kBlock];
    int c[kBlock];
#pragma unroll
    for (int q = 0; q < kBlock; ++q) {
      c[q] = sel[bl * kBlock + q];
      xv[q] = 0.0f;
      cb[q] = 0;
      sbb[q] = 0;
      if (xr >= 0) {
        xv[q] = load1<T>(x + (int64_t)xr * ldx + c[q]);
        cb[q] = codes[(int64_t)xr * (K / 2) + (c[q] >> 1)];
        sbb[q] = scales[(int64_t)xr * nb + (c[q] >> 4)];
      }
    }
#pragma unroll
    for (int q = 0; q < kBlock; ++q) {
      float res = 0.0f;
      if (xr >= 0) {
        const uint32_t code = (cb[q] >> (4 * (c[q] & 1))) & 15u;
        res = xv[q] - dq(code, e4m3_value(sbb[q]) * g);
      }
      R[q] = res;
    }
  };
  float m = 0.0f;
  for (int64_t t0 = b; t0 < e; t0 += kScoreTileRows) {
    const int nr = (int)(e - t0 < kScoreTileRows ? e - t0 : kScoreTileRows);
    load_rows(t0, nr);                        // its first barrier also orders the sel writes
    for (int i = tid; i < nr * kb; i += blockDim.x) {
      const int rl = i / kb, bl = i - rl * kb;
      float R[kBlock];
      r_item(xrow[rl], bl, R);
#pragma unroll
      for (int q = 0; q < kBlock; ++q) {
        m = fmaxf(m, fabsf(R[q]));
        if (keep) rs[(t0 - b + rl) * k + bl * kBlock + q] = R[q];
      }
    }
  }
  m = wave_max(m);
  if ((tid & 63) == 0) red[tid >> 6] = m;
  __syncthreads();
  const float gr = global_scale_from_amax(fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3])));
  const BlockScaler bsc = make_block_scaler(gr);
  if (tid == 0) r_global[u] = gr;

  // ---- requantization of R_S with the unit's own global scale
  auto requant = [&](int64_t r, int bl, const float* R) {
    uint32_t sb, w0, w1;
    quantize_block16(R, bsc, &sb, &w0, &w1);
    *reinterpret_cast<u32x2*>(r_codes + r * (k / 2) + bl * 8) = u32x2{w0, w1};
    r_scales[r * kb + bl] = (uint8_t)sb;
  };
  if (keep) {
    for (int64_t i = tid; i < n * kb; i += blockDim.x) {
      const int64_t rl = i / kb;
      const int bl = (int)(i - rl * kb);
      float R[kBlock];
#pragma unroll
      for (int q = 0; q < kBlock; ++q) R[q] = rs[rl * k + bl * kBlock + q];
      requant(b + rl, bl, R);
    }
  } else {
    for (int64_t t0 = b; t0 < e; t0 += kScoreTileRows) {
      const int nr = (int)(e - t0 < kScoreTileRows ? e - t0 : kScoreTileRows);
      load_rows(t0, nr);
      for (int i = tid; i < nr * kb; i += blockDim.x) {
        const int rl = i / kb, bl = i - rl * kb;
        float R[kBlock];
        r_item(xrow[rl], bl, R);
        requant(t0 + rl, bl, R);
      }
    }
  }
}

// ---------------------------------------------------------------------------
// launcher
// ---------------------------------------------------------------------------
template <typename T, bool MX>
static hipError_t launch_resq_t(const T* x, int64_t x_rows, int64_t K, int64_t ldx,
                                const int32_t* row_index, const uint8_t* codes,
                                const uint8_t* scales, const float* g,
                                const int64_t* unit_offsets, int64_t U, int64_t rows_total,
                                int32_t k, const float* tile_partials, int32_t* sel_idx,
                                uint8_t* r_codes, uint8_t* r_scales, float* r_global,
                                const ResqWorkspace& ws, hipStream_t stream, bool masked) {
  Units units{tile_partials ? nullptr : unit_offsets, U, rows_total};
  // Few rows per unit (at most 32 on average, at most 8192 in all): the whole
  // step per unit in one launch.
  if constexpr (!MX) {
    if (!masked && !tile_partials && K <= kSmallMaxK && rows_total <= 32 * U && rows_total <= 8192) {
      if (K <= 256 * 8)
        resq_small_kernel<T, 8><<<(unsigned)U, 256, 0, stream>>>(x, x_rows, K, ldx, row_index, codes, scales, g,
                                                                 units, k, sel_idx, r_codes, r_scales, r_global);
      else
        resq_small_kernel<T, 16><<<(unsigned)U, 256, 0, stream>>>(x, x_rows, K, ldx, row_index, codes, scales, g,
                                                                  units, k, sel_idx, r_codes, r_scales, r_global);
      return hipGetLastError();
    }
  }
  const int64_t slots = tile_partials ? U : resq_max_slots(rows_total, U);
  const int64_t gslots = resq_max_gather_slots(rows_total, U);
  int4* tile_info = reinterpret_cast<int4*>(ws.tile_info);
  int4* slot_info = reinterpret_cast<int4*>(ws.slot_info);
  resq_plan_kernel<<<1, 1024, 0, stream>>>(units, ws.tile_start, ws.slot_start, tile_info, slots,
                                           slot_info, gslots);
  const float* partials = tile_partials;
  if (!tile_partials) {
    if (row_index) {
      dim3 grid((unsigned)((K + kScoreWaveCols - 1) / kScoreWaveCols), (unsigned)((slots + 3) / 4));
      resq_scores_rows_kernel<T, MX><<<grid, 256, 0, stream>>>(x, x_rows, K, ldx, row_index, codes, scales,
                                                               g, tile_info, slots, ws.partials);
    } else {
      dim3 grid((unsigned)((K + kScoreCols - 1) / kScoreCols), (unsigned)slots);
      resq_scores_tile_kernel<T, MX><<<grid, 256, 0, stream>>>(x, x_rows, K, ldx, row_index, codes, scales,
                                                               g, tile_info, ws.partials);
    }
    partials = ws.partials;
  }
  if (K <= 256 * 4) {
    resq_select_reg_kernel<4><<<(unsigned)U, 256, 0, stream>>>(partials, K, units, ws.tile_start, k,
                                                               sel_idx, r_global);
  } else if (K <= 256 * 8) {
    resq_select_reg_kernel<8><<<(unsigned)U, 256, 0, stream>>>(partials, K, units, ws.tile_start, k,
                                                               sel_idx, r_global);
  } else if (K <= 256 * 16) {
    resq_select_reg_kernel<16><<<(unsigned)U, 256, 0, stream>>>(partials, K, units, ws.tile_start, k,
                                                                sel_idx, r_global);
  } else if (K <= 256 * 32) {
    resq_select_reg_kernel<32><<<(unsigned)U, 256, 0, stream>>>(partials, K, units, ws.tile_start, k,
                                                                sel_idx, r_global);
  } else {
    const size_t sel_lds = (size_t)256 * ((K + 255) / 256 + 1) * 4;
    if (sel_lds > 65536) {
      hipError_t err = hipFuncSetAttribute(reinterpret_cast<const void*>(&resq_select_kernel),
                                           hipFuncAttributeMaxDynamicSharedMemorySize, (int)sel_lds);
      if (err != hipSuccess) return err;
    }
    resq_select_kernel<<<(unsigned)U, 256, sel_lds, stream>>>(partials, K, units, ws.tile_start, k,
                                                              sel_idx, r_global);
  }
  if (gslots > 0) {
    resq_gather_kernel<T, MX><<<(unsigned)gslots, 256, (size_t)k * 4, stream>>>(
        x, x_rows, K, ldx, row_index, codes, scales, g, slot_info, sel_idx, k, ws.r_s,
        ws.amax_part);
    if constexpr (MX)
      resq_requant_mx_kernel<<<(unsigned)gslots, 256, 0, stream>>>(ws.r_s, slot_info, k, r_codes,
                                                                   r_scales);
    else if (masked)
      resq_mask_requant_kernel<<<(unsigned)gslots, 256, 0, stream>>>(
          ws.r_s, slot_info, ws.amax_part, sel_idx, k, K, r_codes, r_scales, r_global);
    else
      resq_requant_kernel<<<(unsigned)gslots, 256, 0, stream>>>(ws.r_s, slot_info, ws.amax_part, k,
                                                                r_codes, r_scales, r_global);
  }
  return hipGetLastError();
}

hipError_t launch_resq(const void* x, int dtype, int64_t x_rows, int64_t K, int64_t ldx,
                       const int32_t* row_index, const uint8_t* codes, const uint8_t* scales,
                       const float* g, const int64_t* unit_offsets, int64_t U, int64_t rows_total,
                       int32_t k, const float* tile_partials, int32_t* sel_idx, uint8_t* r_codes,
                       uint8_t* r_scales, float* r_global, const ResqWorkspace& ws,
                       hipStream_t stream, bool mx, bool masked) {
  if (masked && (mx || K > kMaskMaxK)) return hipErrorInvalidValue;
#define RESQ_ARGS x_rows, K, ldx, row_index, codes, scales, g, unit_offsets, U, rows_total, k, \
                  tile_partials, sel_idx, r_codes, r_scales, r_global, ws, stream, masked
  const __bf16* xb = static_cast<const __bf16*>(x);
  const float* xf = static_cast<const float*>(x);
  if (mx) return dtype == 0 ? launch_resq_t<__bf16, true>(xb, RESQ_ARGS) : launch_resq_t<float, true>(xf, RESQ_ARGS);
  return dtype == 0 ? launch_resq_t<__bf16, false>(xb, RESQ_ARGS) : launch_resq_t<float, false>(xf, RESQ_ARGS);
#undef RESQ_ARGS
}

}  // namespace nvfp4
