// Online NVFP4 activation quantization (QUADS technical summary, section 2.1:
// activations are re-quantized online at every rollout forward; TRACE summary,
// "Prerequisites: NVFP4 and the E2M1 codebook": global scale, per-block scale,
// round-to-nearest onto the E2M1 codebook).
//
// Two passes over x, both coalesced HBM streams:
//   amax_partials_kernel  per-workgroup max |x|  -> workspace (no atomics, no
//                         initialisation, order-independent hence deterministic)
//   amax_fold_kernel      one workgroup folds the partial maxima into one float
//   quantize_tile_kernel  every workgroup derives g from that amax, then
//                         quantizes a 128 x 64 tile;
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
// Workgroup b takes rows b, b + G, b + 2G, ... four at a time: the four rows'
// chunks at a thread's position are loaded before their maxima are taken, so
// each thread keeps four loads in flight.
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
template <typename T>
__global__ __launch_bounds__(256) void amax_partials_kernel(const T* __restrict__ x, int64_t M,
                                                            int64_t K, int64_t ldx,
                                                            float* __restrict__ partials) {
  constexpr int kPer = 16 / sizeof(T);                       // elements per 16-byte chunk
  const int64_t chunks = K / kPer;
  const int64_t G = gridDim.x;
  float m = 0.0f;
  int64_t r = blockIdx.x;
  for (; r + 3 * G < M; r += 4 * G) {
    const T* row = x + r * ldx;
    for (int64_t c = threadIdx.x; c < chunks; c += blockDim.x) {
      const u32x4 w0 = *reinterpret_cast<const u32x4*>(row + c * kPer);
      const u32x4 w1 = *reinterpret_cast<const u32x4*>(row + G * ldx + c * kPer);
      const u32x4 w2 = *reinterpret_cast<const u32x4*>(row + 2 * G * ldx + c * kPer);
      const u32x4 w3 = *reinterpret_cast<const u32x4*>(row + 3 * G * ldx + c * kPer);
      m = absmax_chunk<T>(w3, absmax_chunk<T>(w2, absmax_chunk<T>(w1, absmax_chunk<T>(w0, m))));
    }
  }
  for (; r < M; r += G) {
    const T* row = x + r * ldx;
    for (int64_t c = threadIdx.x; c < chunks; c += blockDim.x)
      m = absmax_chunk<T>(*reinterpret_cast<const u32x4*>(row + c * kPer), m);
  }
  m = wave_max(m);
  __shared__ float red[4];
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = m;
  __syncthreads();
  if (threadIdx.x == 0) {
    float b = red[0];
    for (int i = 1; i < (int)(blockDim.x >> 6); ++i) b = fmaxf(b, red[i]);
    partials[blockIdx.x] = b;
  }
}

// Folds the n partial maxima into partials[n] (one workgroup), so that every
// quantize workgroup reads a single float.
__global__ __launch_bounds__(256) void amax_fold_kernel(float* __restrict__ partials, int n) {
  float m = 0.0f;
  for (int i = threadIdx.x; i < n; i += blockDim.x) m = fmaxf(m, partials[i]);
  m = wave_max(m);
  __shared__ float red[4];
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = m;
  __syncthreads();
  if (threadIdx.x == 0) partials[n] = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
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
    const float* __restrict__ amax, uint8_t* __restrict__ codes, uint8_t* __restrict__ scales,
    float* __restrict__ g_out, float* __restrict__ tile_partials) {
  __shared__ float absr[SCORES ? kScoreTileRows * kAbsStride : 1];
  const int tid = threadIdx.x;
  const float g = global_scale_from_amax(*amax);
  const BlockScaler bsc = make_block_scaler(g);
  if (g_out && blockIdx.x == 0 && tid == 0) *g_out = g;

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
  float v[kRowsPerThread][16];
  bool live[kRowsPerThread];
#pragma unroll
  for (int j = 0; j < kRowsPerThread; ++j) {         // all loads first
    const int64_t r = r0 + rsub + (256 / kTileBlocks) * j;
    live[j] = r < M && bc < nb;
    if (live[j]) Row16<T>::load(x + r * ldx + bc * kBlock, v[j]);
  }
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
int amax_partials_count(int64_t M, int64_t K) {
  (void)K;
  int64_t n = M < 1024 ? M : 1024;
  return n < 1 ? 1 : (int)n;
}

template <typename T>
static hipError_t launch_quantize_t(const T* x, int64_t M, int64_t K, int64_t ldx,
                                    const float* amax_in, uint8_t* codes, uint8_t* scales,
                                    float* g_out, float* tile_partials, float* ws_partials,
                                    hipStream_t stream) {
  const int np = amax_partials_count(M, K);
  const float* amax = amax_in;
  if (!amax_in) {
    amax_partials_kernel<T><<<np, 256, 0, stream>>>(x, M, K, ldx, ws_partials);
    amax_fold_kernel<<<1, 256, 0, stream>>>(ws_partials, np);
    amax = ws_partials + np;
  }
  const int64_t ntiles = ((K / kBlock + kTileBlocks - 1) / kTileBlocks) *
                         ((M + kScoreTileRows - 1) / kScoreTileRows);
  const unsigned grid = (unsigned)(ntiles > 0 ? (ntiles + 7) / 8 * 8 : 8);   // whole eighths, one per XCD
  if (tile_partials)
    quantize_tile_kernel<T, true><<<grid, 256, 0, stream>>>(x, M, K, ldx, amax, codes, scales,
                                                            g_out, tile_partials);
  else
    quantize_tile_kernel<T, false><<<grid, 256, 0, stream>>>(x, M, K, ldx, amax, codes, scales,
                                                             g_out, nullptr);
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
