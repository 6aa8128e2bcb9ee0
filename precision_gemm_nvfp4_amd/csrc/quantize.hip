// Online NVFP4 activation quantization (QUADS technical summary, section 2.1:
// activations are re-quantized online at every rollout forward; TRACE summary,
// "Prerequisites: NVFP4 and the E2M1 codebook": global scale, per-block scale,
// round-to-nearest onto the E2M1 codebook).
//
// Two passes over x, both coalesced HBM streams:
//   amax_partials_kernel  per-workgroup max |x|  -> workspace (no atomics, no
//                         initialisation, order-independent hence deterministic)
//   quantize_tile_kernel  every workgroup folds the partial maxima into the
//                         tensor's amax, derives g from it, then quantizes a
//                         128 x 64 tile;
//                         optionally it also sums |x - DQ| of each channel over
//                         the tile's 128 rows in fp32, in row order (the residual
//                         channel-score partials of the residual activation
//                         compensation, QUADS section 2.2B).
#include "device_common.h"
#include "kernels.h"

namespace nvfp4 {

template <typename T>
struct Row16;  // loads 16 consecutive elements as fp32

template <>
struct Row16<__bf16> {
  __device__ __forceinline__ static void load(const __bf16* p, float* v) {
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
};

template <>
struct Row16<float> {
  __device__ __forceinline__ static void load(const float* p, float* v) {
    const f32x4* q = reinterpret_cast<const f32x4*>(p);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      f32x4 a = q[i];
      v[4 * i] = a[0];
      v[4 * i + 1] = a[1];
      v[4 * i + 2] = a[2];
      v[4 * i + 3] = a[3];
    }
  }
};

// ---------------------------------------------------------------------------
// pass 1: per-workgroup amax
// ---------------------------------------------------------------------------
// The tensor is a flat sequence of 16-byte chunks (row r's chunks after row
// r - 1's, the row stride skipped); thread t of the grid takes chunks t,
// t + G, t + 2G, ... (G = grid threads), eight at a time, all eight loaded
// before their maxima are taken.
template <typename T>
__device__ __forceinline__ float absmax_chunk(const u32x4& w, float m) {
  if constexpr (sizeof(T) == 2) {
#pragma unroll
    for (int i = 0; i < 4; ++i) m = fmaxf(m, fmaxf(fabsf(bf16_lo(w[i])), fabsf(bf16_hi(w[i]))));
  } else {
#pragma unroll
    for (int i = 0; i < 4; ++i) m = fmaxf(m, fabsf(__uint_as_float(w[i])));
  }
  return m;
}
constexpr int kAmaxBatch = 8;
constexpr int kAmaxThreads = 1024;
template <typename T>
__global__ __launch_bounds__(kAmaxThreads) void amax_partials_kernel(const T* __restrict__ x, int64_t M,
                                                            int64_t K, int64_t ldx,
                                                            float* __restrict__ partials) {
  constexpr int kPer = 16 / sizeof(T);                       // elements per 16-byte chunk
  const int64_t cpr = K / kPer;                              // chunks per row
  const int64_t total = M * cpr;
  const int64_t G = (int64_t)gridDim.x * blockDim.x;
  const bool dense = ldx == K;
  auto chunk = [&](int64_t c) -> u32x4 {
    if (dense) return reinterpret_cast<const u32x4*>(x)[c];
    const int64_t r = c / cpr;
    return reinterpret_cast<const u32x4*>(x + r * ldx)[c - r * cpr];
  };
  float m = 0.0f;
  int64_t c = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  for (; c + (kAmaxBatch - 1) * G < total; c += kAmaxBatch * G) {
    u32x4 w[kAmaxBatch];
#pragma unroll
    for (int q = 0; q < kAmaxBatch; ++q) w[q] = chunk(c + q * G);
#pragma unroll
    for (int q = 0; q < kAmaxBatch; ++q) m = absmax_chunk<T>(w[q], m);
  }
  for (; c < total; c += G) m = absmax_chunk<T>(chunk(c), m);
  m = wave_max(m);
  __shared__ float red[kAmaxThreads / 64];
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = m;
  __syncthreads();
  if (threadIdx.x == 0) {
    float b = red[0];
    for (int i = 1; i < (int)(blockDim.x >> 6); ++i) b = fmaxf(b, red[i]);
    partials[blockIdx.x] = b;
  }
}

// ---------------------------------------------------------------------------
// pass 2: block quantization (+ optional residual-score partials)
// ---------------------------------------------------------------------------
// One workgroup (256 threads) owns a tile of 128 rows x 64 columns.  The
// tiles (row bands outer, column tiles inner) are dealt to the 8 XCDs in
// contiguous eighths -- hardware workgroup h runs on XCD h % 8 and takes tile
// (h % 8) * ceil(T / 8) + h / 8 -- because neighbouring column tiles share
// output lines (4 tiles per 128-byte line of codes, 32 per line of scales):
// written from one XCD, a line is completed in that XCD's L2 and leaves as one
// write; spread over XCDs, each L2 writes its pieces back separately (1.7x the
// output bytes in HBM writes, measured).  Thread t
// quantizes the 16-element block column t % 4 of rows t / 4 and t / 4 + 64:
// both rows are loaded before any arithmetic, so every thread has two loads in
// flight.  With SCORES, each thread also writes |x - DQ| of its blocks into LDS
// (34 KB: four workgroups fit a CU), and after a barrier threads 0..63 each add
// one column's 128 values in increasing row order (rows past the tensor
// contribute +0, which leaves an fp32 sum unchanged).
constexpr int kTileCols = 64;
constexpr int kTileBlocks = kTileCols / kBlock;     // 4
constexpr int kRowsPerThread = kScoreTileRows / (256 / kTileBlocks);   // 2
constexpr int kAbsStride = kTileCols + 4;          // floats per LDS row

template <typename T, bool SCORES>
__global__ __launch_bounds__(256) void quantize_tile_kernel(
    const T* __restrict__ x, int64_t M, int64_t K, int64_t ldx,
    const float* __restrict__ amax, int n_amax, uint8_t* __restrict__ codes,
    uint8_t* __restrict__ scales, float* __restrict__ g_out, float* __restrict__ tile_partials) {
  __shared__ float absr[SCORES ? kScoreTileRows * kAbsStride : 1];
  const int tid = threadIdx.x;

  const int64_t nb = K / kBlock;
  const int64_t tiles_x = (nb + kTileBlocks - 1) / kTileBlocks;
  const int64_t ntiles = tiles_x * ((M + kScoreTileRows - 1) / kScoreTileRows);
  const int64_t per_xcd = (ntiles + 7) / 8;
  const int64_t tile = (int64_t)(blockIdx.x % 8) * per_xcd + blockIdx.x / 8;
  if ((int64_t)(blockIdx.x / 8) >= per_xcd || tile >= ntiles) return;   // uniform
  const int64_t tx = tile % tiles_x, ty = tile / tiles_x;
  const int bl = tid % kTileBlocks, rsub = tid / kTileBlocks;
  const int64_t bc = tx * kTileBlocks + bl;
  const int64_t r0 = ty * kScoreTileRows;
  // The tensor's amax: one value, or the n_amax (<= 256) partial maxima of
  // the amax pass, which every wave folds by itself, four per lane (max is
  // exact in any order).  Loaded ahead of x, so that waiting for them does
  // not wait for x.
  float pm[4] = {0.0f, 0.0f, 0.0f, 0.0f};
  if (n_amax == 1) {
    pm[0] = *amax;                                   // as given (a caller's amax_in)
  } else {
    const int l4 = (tid & 63) * 4;
#pragma unroll
    for (int i = 0; i < 4; ++i) pm[i] = l4 + i < n_amax ? amax[l4 + i] : 0.0f;
  }
  float v[kRowsPerThread][16];
  bool live[kRowsPerThread];
#pragma unroll
  for (int j = 0; j < kRowsPerThread; ++j) {         // all loads first
    const int64_t r = r0 + rsub + (256 / kTileBlocks) * j;
    live[j] = r < M && bc < nb;
    if (live[j]) Row16<T>::load(x + r * ldx + bc * kBlock, v[j]);
  }
  const float am = n_amax == 1 ? pm[0] : wave_max(fmaxf(fmaxf(pm[0], pm[1]), fmaxf(pm[2], pm[3])));
  const float g = global_scale_from_amax(am);
  const BlockScaler bsc = make_block_scaler(g);
  if (g_out && tile == 0 && tid == 0) *g_out = g;
#pragma unroll
  for (int j = 0; j < kRowsPerThread; ++j) {
    const int rl = rsub + (256 / kTileBlocks) * j;
    const int64_t r = r0 + rl;
    float res[16];
    if (live[j]) {
      uint32_t sb, w0, w1;
      const float S = quantize_block16(v[j], bsc, &sb, &w0, &w1);
      *reinterpret_cast<u32x2*>(codes + r * (K / 2) + bc * 8) = u32x2{w0, w1};
      scales[r * nb + bc] = (uint8_t)sb;
      if constexpr (SCORES) {
        float f[16];
        e2m1_unpack8(w0, f);
        e2m1_unpack8(w1, f + 8);
#pragma unroll
        for (int i = 0; i < 16; ++i) res[i] = fabsf(v[j][i] - f[i] * S);   // exact; no contraction
      }
    } else if constexpr (SCORES) {
#pragma unroll
      for (int i = 0; i < 16; ++i) res[i] = 0.0f;
    }
    if constexpr (SCORES) {
      f32x4* dst = reinterpret_cast<f32x4*>(absr + rl * kAbsStride + bl * kBlock);
#pragma unroll
      for (int i = 0; i < 4; ++i) dst[i] = f32x4{res[4 * i], res[4 * i + 1], res[4 * i + 2], res[4 * i + 3]};
    }
  }
  if constexpr (SCORES) {
    __syncthreads();
    const int64_t c = tx * kTileCols + tid;
    if (tid < kTileCols && c < K) {
      float sum = 0.0f;
#pragma unroll 16
      for (int rl = 0; rl < kScoreTileRows; ++rl) sum = sum + absr[rl * kAbsStride + tid];
      tile_partials[ty * K + c] = sum;
    }
  }
}

// ---------------------------------------------------------------------------
// launcher
// ---------------------------------------------------------------------------
// One partial maximum per workgroup of the amax pass: enough workgroups of
// 1024 threads for one batch of eight 16-byte loads per thread on a bf16
// tensor (8192 elements per thread), at most 256, one per CU (each quantize
// wave folds them with one load per lane).
int amax_partials_count(int64_t M, int64_t K) {
  const int64_t per = (int64_t)kAmaxThreads * kAmaxBatch * 8;
  const int64_t n = (M * K + per - 1) / per;
  return n < 1 ? 1 : (n > 256 ? 256 : (int)n);
}

template <typename T>
static hipError_t launch_quantize_t(const T* x, int64_t M, int64_t K, int64_t ldx,
                                    const float* amax_in, uint8_t* codes, uint8_t* scales,
                                    float* g_out, float* tile_partials, float* ws_partials,
                                    hipStream_t stream) {
  const float* amax = amax_in;
  int n_amax = 1;
  if (!amax_in) {
    n_amax = amax_partials_count(M, K);
    amax_partials_kernel<T><<<n_amax, kAmaxThreads, 0, stream>>>(x, M, K, ldx, ws_partials);
    amax = ws_partials;
  }
  const int64_t ntiles = ((K / kBlock + kTileBlocks - 1) / kTileBlocks) *
                         ((M + kScoreTileRows - 1) / kScoreTileRows);
  const unsigned grid = (unsigned)(ntiles > 0 ? (ntiles + 7) / 8 * 8 : 8);   // whole eighths, one per XCD
  if (tile_partials)
    quantize_tile_kernel<T, true><<<grid, 256, 0, stream>>>(x, M, K, ldx, amax, n_amax, codes,
                                                            scales, g_out, tile_partials);
  else
    quantize_tile_kernel<T, false><<<grid, 256, 0, stream>>>(x, M, K, ldx, amax, n_amax, codes,
                                                             scales, g_out, nullptr);
  return hipGetLastError();
}

hipError_t launch_quantize(const void* x, int dtype, int64_t M, int64_t K, int64_t ldx,
                           const float* amax_in, uint8_t* codes, uint8_t* scales, float* g_out,
                           float* tile_partials, float* ws_partials, hipStream_t stream) {
  if (dtype == 0)
    return launch_quantize_t(static_cast<const __bf16*>(x), M, K, ldx, amax_in, codes, scales,
                             g_out, tile_partials, ws_partials, stream);
  return launch_quantize_t(static_cast<const float*>(x), M, K, ldx, amax_in, codes, scales, g_out,
                           tile_partials, ws_partials, stream);
}

// Writes v into *p from one thread (used for g_out = 1 on empty tensors and
// for zero-initialising counters without hipMemsetAsync).
__global__ void fill_f32_kernel(float* p, int64_t n, float v) {
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n;
       i += (int64_t)gridDim.x * blockDim.x)
    p[i] = v;
}

hipError_t launch_fill_f32(float* p, int64_t n, float v, hipStream_t stream) {
  if (n <= 0) return hipSuccess;
  int64_t blocks = (n + 255) / 256;
  fill_f32_kernel<<<(unsigned)(blocks > 1024 ? 1024 : blocks), 256, 0, stream>>>(p, n, v);
  return hipGetLastError();
}

}  // namespace nvfp4
