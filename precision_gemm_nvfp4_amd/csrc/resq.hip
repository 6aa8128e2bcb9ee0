// Residual activation compensation on the rollout side (QUADS technical
// summary, section 2.2B; yfxerp digest): per selection unit, score every
// channel by the magnitude of the FP4 residual R = x - DQ(Q(x)), keep the
// top-k channels (a binary channel mask), and quantize the compact residual
// R_S a second time with its own global scale.
//
// Kernels (one stream, in order):
//   plan      tile_start[u]: first 128-row tile of unit u (exclusive scan)
//   scores    per (tile, 1024-channel slice): fp32 sum of |R| over the tile's
//             rows in increasing row order          (skipped when nvfp4_quantize
//                                                    already produced them)
//   select    per unit: tile sums added in tile order -> LDS; radix select of
//             the k-th largest score; ties to the lower channel; compaction in
//             ascending channel order (block scans)
//   gather    per tile: R_S = x[:, sel] - DQ(codes, scales)[:, sel] -> workspace,
//             with the tile's max |R_S|
//   requant   per tile: unit amax -> g_R, NVFP4 of R_S rows (16-blocks along
//             the compact axis) -> r_codes, r_scales, r_global
#include "device_common.h"
#include "kernels.h"

namespace nvfp4 {

int64_t resq_max_slots(int64_t rows_total, int64_t U) {
  return (rows_total + kScoreTileRows - 1) / kScoreTileRows + U;
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

// Unit of a tile slot (largest u with tile_start[u] <= slot); -1 if none.
__device__ __forceinline__ int64_t unit_of_slot(const int32_t* tile_start, int64_t U, int64_t slot) {
  if (slot >= tile_start[U]) return -1;
  int64_t lo = 0, hi = U;            // tile_start[lo] <= slot < tile_start[hi]
  while (hi - lo > 1) {
    int64_t mid = (lo + hi) >> 1;
    if (tile_start[mid] <= slot) lo = mid; else hi = mid;
  }
  return lo;
}

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
__global__ __launch_bounds__(1024) void resq_plan_kernel(Units units, int32_t* tile_start) {
  __shared__ uint32_t sh[16];
  uint32_t carry = 0;
  for (int64_t base = 0; base < units.U; base += blockDim.x) {
    int64_t u = base + threadIdx.x;
    uint32_t n = 0;
    if (u < units.U) {
      int64_t b, e;
      units.range(u, b, e);
      n = (uint32_t)((e - b + kScoreTileRows - 1) / kScoreTileRows);
    }
    uint32_t tot;
    uint32_t ex = block_exclusive_scan(n, sh, &tot);
    if (u < units.U) tile_start[u] = (int32_t)(carry + ex);
    carry += tot;
  }
  if (threadIdx.x == 0) tile_start[units.U] = (int32_t)carry;
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

template <typename T>
__global__ __launch_bounds__(64) void resq_scores_kernel(
    const T* __restrict__ x, int64_t x_rows, int64_t K, int64_t ldx,
    const int32_t* __restrict__ row_index, const uint8_t* __restrict__ codes,
    const uint8_t* __restrict__ scales, const float* __restrict__ gp, Units units,
    const int32_t* __restrict__ tile_start, float* __restrict__ partials) {
  const int64_t slot = blockIdx.x;
  const int64_t u = unit_of_slot(tile_start, units.U, slot);
  if (u < 0) return;
  const int64_t nb = K / kBlock;
  const int64_t bc = (int64_t)blockIdx.y * 64 + threadIdx.x;
  if (bc >= nb) return;
  int64_t b, e;
  units.range(u, b, e);
  const int64_t r0 = b + (slot - tile_start[u]) * kScoreTileRows;
  const int64_t r1 = r0 + kScoreTileRows < e ? r0 + kScoreTileRows : e;
  const float g = *gp;
  float acc[16];
#pragma unroll
  for (int j = 0; j < 16; ++j) acc[j] = 0.0f;
  for (int64_t r = r0; r < r1; ++r) {
    const int64_t xr = row_index ? (int64_t)row_index[r] : r;
    if (xr < 0 || xr >= x_rows) continue;
    float v[16];
    load16<T>(x + xr * ldx + bc * kBlock, v);
    const u32x2 w = *reinterpret_cast<const u32x2*>(codes + xr * (K / 2) + bc * 8);
    const float S = e4m3_value(scales[xr * nb + bc]) * g;
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      const uint32_t c = (w[j >> 3] >> (4 * (j & 7))) & 15u;
      acc[j] = acc[j] + fabsf(v[j] - dq(c, S));
    }
  }
  f32x4* out = reinterpret_cast<f32x4*>(partials + slot * K + bc * kBlock);
#pragma unroll
  for (int i = 0; i < 4; ++i) out[i] = f32x4{acc[4 * i], acc[4 * i + 1], acc[4 * i + 2], acc[4 * i + 3]};
}

// ---------------------------------------------------------------------------
// select: scores -> top-k (ties to the lower index) -> ascending channel list
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void resq_select_kernel(
    const float* __restrict__ partials, int64_t K, Units units,
    const int32_t* __restrict__ tile_start, int32_t k, int32_t* __restrict__ sel_idx,
    float* __restrict__ r_global) {
  extern __shared__ uint32_t keys[];          // [K] score bits (scores are >= +0)
  __shared__ uint32_t hist[256];
  __shared__ uint32_t sh_waves[4];
  __shared__ uint32_t sh_digit, sh_rem;
  const int64_t u = blockIdx.x;
  const int tid = threadIdx.x;
  int64_t b, e;
  units.range(u, b, e);
  int32_t* out = sel_idx + u * k;
  if (e == b) {                               // empty unit: channels 0..k-1, g_R = 1
    for (int j = tid; j < k; j += blockDim.x) out[j] = j;
    if (tid == 0) r_global[u] = 1.0f;
    return;
  }
  const int64_t t0 = tile_start[u], t1 = tile_start[u + 1];
  for (int64_t c = tid; c < K; c += blockDim.x) {
    float s = 0.0f;
    for (int64_t t = t0; t < t1; ++t) s = s + partials[t * K + c];   // tile order
    keys[c] = __float_as_uint(s);
  }
  __syncthreads();

  // radix select (8-bit digits, most significant first) of the k-th largest key
  uint32_t prefix = 0, mask = 0;
  uint32_t remaining = (uint32_t)k;
  for (int shift = 24; shift >= 0; shift -= 8) {
    hist[tid] = 0;
    __syncthreads();
    for (int64_t c = tid; c < K; c += blockDim.x) {
      uint32_t key = keys[c];
      if ((key & mask) == prefix) atomicAdd(&hist[(key >> shift) & 255u], 1u);
    }
    __syncthreads();
    if (tid == 0) {
      uint32_t above = 0;
      int d = 255;
      for (; d > 0; --d) {
        if (above + hist[d] >= remaining) break;
        above += hist[d];
      }
      sh_digit = (uint32_t)d;
      sh_rem = remaining - above;
    }
    __syncthreads();
    prefix |= sh_digit << shift;
    mask |= 255u << shift;
    remaining = sh_rem;
    __syncthreads();
  }
  const uint32_t T = prefix;     // k-th largest key; `remaining` keys equal to T are taken

  // selection in index order: thread owns a contiguous chunk of channels
  const int64_t chunk = (K + blockDim.x - 1) / blockDim.x;
  const int64_t c0 = tid * chunk;
  const int64_t c1 = c0 + chunk < K ? c0 + chunk : K;
  uint32_t n_eq = 0;
  for (int64_t c = c0; c < c1; ++c) n_eq += keys[c] == T;
  uint32_t tot;
  uint32_t eq_before = block_exclusive_scan(n_eq, sh_waves, &tot);
  uint32_t n_sel = 0;
  {
    uint32_t eq_seen = eq_before;
    for (int64_t c = c0; c < c1; ++c) {
      uint32_t key = keys[c];
      if (key > T) ++n_sel;
      else if (key == T && eq_seen++ < remaining) ++n_sel;
    }
  }
  uint32_t pos = block_exclusive_scan(n_sel, sh_waves, &tot);
  {
    uint32_t eq_seen = eq_before;
    for (int64_t c = c0; c < c1; ++c) {
      uint32_t key = keys[c];
      bool take = key > T || (key == T && eq_seen++ < remaining);
      if (take && pos < (uint32_t)k) out[pos++] = (int32_t)c;
    }
  }
}

// ---------------------------------------------------------------------------
// gather R_S and per-tile max |R_S|
// ---------------------------------------------------------------------------
template <typename T>
__global__ __launch_bounds__(256) void resq_gather_kernel(
    const T* __restrict__ x, int64_t x_rows, int64_t K, int64_t ldx,
    const int32_t* __restrict__ row_index, const uint8_t* __restrict__ codes,
    const uint8_t* __restrict__ scales, const float* __restrict__ gp, Units units,
    const int32_t* __restrict__ tile_start, const int32_t* __restrict__ sel_idx, int32_t k,
    float* __restrict__ r_s, float* __restrict__ amax_part) {
  extern __shared__ int32_t sel[];           // [k]
  __shared__ float red[4];
  const int64_t slot = blockIdx.x;
  const int64_t u = unit_of_slot(tile_start, units.U, slot);
  if (u < 0) return;
  int64_t b, e;
  units.range(u, b, e);
  const int64_t r0 = b + (slot - tile_start[u]) * kScoreTileRows;
  const int64_t r1 = r0 + kScoreTileRows < e ? r0 + kScoreTileRows : e;
  for (int j = threadIdx.x; j < k; j += blockDim.x) {
    int32_t c = sel_idx[u * k + j];
    sel[j] = c < 0 ? 0 : (c >= K ? (int32_t)(K - 1) : c);
  }
  __syncthreads();
  const float g = *gp;
  const int64_t nb = K / kBlock;
  float m = 0.0f;
  const int64_t n = (r1 - r0) * k;
  for (int64_t i = threadIdx.x; i < n; i += blockDim.x) {
    const int64_t r = r0 + i / k;
    const int j = (int)(i % k);
    const int64_t xr = row_index ? (int64_t)row_index[r] : r;
    float res = 0.0f;
    if (xr >= 0 && xr < x_rows) {
      const int64_t c = sel[j];
      const float xv = load1<T>(x + xr * ldx + c);
      const uint32_t code = (codes[xr * (K / 2) + (c >> 1)] >> (4 * (c & 1))) & 15u;
      const float S = e4m3_value(scales[xr * nb + (c >> 4)]) * g;
      res = xv - dq(code, S);
    }
    r_s[r * k + j] = res;
    m = fmaxf(m, fabsf(res));
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
    const float* __restrict__ r_s, Units units, const int32_t* __restrict__ tile_start,
    const float* __restrict__ amax_part, int32_t k, uint8_t* __restrict__ r_codes,
    uint8_t* __restrict__ r_scales, float* __restrict__ r_global) {
  __shared__ float sh_g;
  const int64_t slot = blockIdx.x;
  const int64_t u = unit_of_slot(tile_start, units.U, slot);
  if (u < 0) return;
  int64_t b, e;
  units.range(u, b, e);
  if (threadIdx.x < 64) {
    float m = 0.0f;
    for (int64_t t = tile_start[u] + threadIdx.x; t < tile_start[u + 1]; t += 64)
      m = fmaxf(m, amax_part[t]);
    m = wave_max(m);
    if (threadIdx.x == 0) sh_g = global_scale_from_amax(m);
  }
  __syncthreads();
  const float g = sh_g;
  const double six_g = 6.0 * (double)g;
  if (slot == tile_start[u] && threadIdx.x == 0) r_global[u] = g;
  const int64_t r0 = b + (slot - tile_start[u]) * kScoreTileRows;
  const int64_t r1 = r0 + kScoreTileRows < e ? r0 + kScoreTileRows : e;
  const int kb = k / kBlock;
  const int64_t n = (r1 - r0) * kb;
  for (int64_t i = threadIdx.x; i < n; i += blockDim.x) {
    const int64_t r = r0 + i / kb;
    const int bl = (int)(i % kb);
    float v[16];
    load16<float>(r_s + r * k + bl * kBlock, v);
    uint32_t sb, w0, w1;
    quantize_block16(v, g, six_g, &sb, &w0, &w1);
    *reinterpret_cast<u32x2*>(r_codes + r * (k / 2) + bl * 8) = u32x2{w0, w1};
    r_scales[r * kb + bl] = (uint8_t)sb;
  }
}

// ---------------------------------------------------------------------------
// launcher
// ---------------------------------------------------------------------------
template <typename T>
static hipError_t launch_resq_t(const T* x, int64_t x_rows, int64_t K, int64_t ldx,
                                const int32_t* row_index, const uint8_t* codes,
                                const uint8_t* scales, const float* g,
                                const int64_t* unit_offsets, int64_t U, int64_t rows_total,
                                int32_t k, const float* tile_partials, int32_t* sel_idx,
                                uint8_t* r_codes, uint8_t* r_scales, float* r_global,
                                const ResqWorkspace& ws, hipStream_t stream) {
  Units units{tile_partials ? nullptr : unit_offsets, U, rows_total};
  const int64_t slots = tile_partials ? U : resq_max_slots(rows_total, U);
  resq_plan_kernel<<<1, 1024, 0, stream>>>(units, ws.tile_start);
  const float* partials = tile_partials;
  if (!tile_partials) {
    dim3 grid((unsigned)slots, (unsigned)((K / kBlock + 63) / 64));
    resq_scores_kernel<T><<<grid, 64, 0, stream>>>(x, x_rows, K, ldx, row_index, codes, scales, g,
                                                   units, ws.tile_start, ws.partials);
    partials = ws.partials;
  }
  resq_select_kernel<<<(unsigned)U, 256, (size_t)K * 4, stream>>>(partials, K, units, ws.tile_start,
                                                                   k, sel_idx, r_global);
  if (slots > 0) {
    resq_gather_kernel<T><<<(unsigned)slots, 256, (size_t)k * 4, stream>>>(
        x, x_rows, K, ldx, row_index, codes, scales, g, units, ws.tile_start, sel_idx, k, ws.r_s,
        ws.amax_part);
    resq_requant_kernel<<<(unsigned)slots, 256, 0, stream>>>(ws.r_s, units, ws.tile_start,
                                                             ws.amax_part, k, r_codes, r_scales,
                                                             r_global);
  }
  return hipGetLastError();
}

hipError_t launch_resq(const void* x, int dtype, int64_t x_rows, int64_t K, int64_t ldx,
                       const int32_t* row_index, const uint8_t* codes, const uint8_t* scales,
                       const float* g, const int64_t* unit_offsets, int64_t U, int64_t rows_total,
                       int32_t k, const float* tile_partials, int32_t* sel_idx, uint8_t* r_codes,
                       uint8_t* r_scales, float* r_global, const ResqWorkspace& ws,
                       hipStream_t stream) {
  if (dtype == 0)
    return launch_resq_t(static_cast<const __bf16*>(x), x_rows, K, ldx, row_index, codes, scales, g,
                         unit_offsets, U, rows_total, k, tile_partials, sel_idx, r_codes, r_scales,
                         r_global, ws, stream);
  return launch_resq_t(static_cast<const float*>(x), x_rows, K, ldx, row_index, codes, scales, g,
                       unit_offsets, U, rows_total, k, tile_partials, sel_idx, r_codes, r_scales,
                       r_global, ws, stream);
}

}  // namespace nvfp4
