// Online NVFP4 activation quantization (QUADS technical summary, section 2.1:
// activations are re-quantized online at every rollout forward; TRACE summary,
// "Prerequisites: NVFP4 and the E2M1 codebook": global scale, per-block scale,
// round-to-nearest onto the E2M1 codebook).
//
// Two passes over x, both coalesced HBM streams:
//   amax_partials_kernel  per-workgroup max |x|  -> workspace (no atomics, no
//                         initialisation, order-independent hence deterministic)
//   quantize_kernel       every workgroup folds the partial maxima into the
//                         tensor amax and g, then quantizes its tile: one lane
//                         owns one 16-element block column and walks the tile's
//                         rows; optionally it accumulates |x - DQ| of its 16
//                         channels over the 128-row tile in fp32, in row order
//                         (the residual channel-score partials of the residual
//                         activation compensation, QUADS section 2.2B).
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
template <typename T>
__global__ __launch_bounds__(256) void amax_partials_kernel(const T* __restrict__ x, int64_t M,
                                                            int64_t K, int64_t ldx,
                                                            float* __restrict__ partials) {
  constexpr int kPer = 16 / sizeof(T);                       // elements per 16-byte chunk
  const int64_t chunks = K / kPer;
  float m = 0.0f;
  for (int64_t r = blockIdx.x; r < M; r += gridDim.x) {
    const T* row = x + r * ldx;
    for (int64_t c = threadIdx.x; c < chunks; c += blockDim.x) {
      u32x4 w = *reinterpret_cast<const u32x4*>(row + c * kPer);
      if constexpr (sizeof(T) == 2) {
#pragma unroll
        for (int i = 0; i < 4; ++i) m = fmaxf(m, fmaxf(fabsf(bf16_lo(w[i])), fabsf(bf16_hi(w[i]))));
      } else {
#pragma unroll
        for (int i = 0; i < 4; ++i) m = fmaxf(m, fabsf(__uint_as_float(w[i])));
      }
    }
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

// Max over n partial maxima, read by one wave (lanes stride the array).
__device__ __forceinline__ float fold_partials(const float* partials, int n) {
  float m = 0.0f;
  for (int i = threadIdx.x & 63; i < n; i += 64) m = fmaxf(m, partials[i]);
  return wave_max(m);
}

// ---------------------------------------------------------------------------
// pass 2: block quantization (+ optional residual-score partials)
// ---------------------------------------------------------------------------
// grid: x = ceil(K/16 / 64) block columns of 64 lanes, y = row tiles of ROWS.
template <typename T, bool SCORES, int ROWS>
__global__ __launch_bounds__(64) void quantize_kernel(
    const T* __restrict__ x, int64_t M, int64_t K, int64_t ldx,
    const float* __restrict__ amax_partials, int n_partials, const float* __restrict__ amax_in,
    uint8_t* __restrict__ codes, uint8_t* __restrict__ scales, float* __restrict__ g_out,
    float* __restrict__ tile_partials) {
  const float amax = amax_in ? *amax_in : fold_partials(amax_partials, n_partials);
  const float g = global_scale_from_amax(amax);
  const double six_g = 6.0 * (double)g;
  if (g_out && blockIdx.x == 0 && blockIdx.y == 0 && threadIdx.x == 0) *g_out = g;

  const int64_t nb = K / kBlock;
  const int64_t bc = (int64_t)blockIdx.x * 64 + threadIdx.x;
  if (bc >= nb) return;
  const int64_t r0 = (int64_t)blockIdx.y * ROWS;
  const int64_t r1 = r0 + ROWS < M ? r0 + ROWS : M;

  float acc[16];
#pragma unroll
  for (int j = 0; j < 16; ++j) acc[j] = 0.0f;

#pragma unroll 4
  for (int64_t r = r0; r < r1; ++r) {
    float v[16];
    Row16<T>::load(x + r * ldx + bc * kBlock, v);
    uint32_t sb, w0, w1;
    const float S = quantize_block16(v, g, six_g, &sb, &w0, &w1);
    *reinterpret_cast<u32x2*>(codes + r * (K / 2) + bc * 8) = u32x2{w0, w1};
    scales[r * nb + bc] = (uint8_t)sb;
    if constexpr (SCORES) {
#pragma unroll
      for (int j = 0; j < 16; ++j) {
        const uint32_t c = ((j < 8 ? w0 : w1) >> (4 * (j & 7))) & 15u;
        const float res = v[j] - dq(c, S);         // exact (Sterbenz); no contraction
        acc[j] = acc[j] + fabsf(res);
      }
    }
  }
  if constexpr (SCORES) {
    f32x4* out = reinterpret_cast<f32x4*>(tile_partials + (int64_t)blockIdx.y * K + bc * kBlock);
#pragma unroll
    for (int i = 0; i < 4; ++i) out[i] = f32x4{acc[4 * i], acc[4 * i + 1], acc[4 * i + 2], acc[4 * i + 3]};
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
  if (!amax_in) {
    amax_partials_kernel<T><<<np, 256, 0, stream>>>(x, M, K, ldx, ws_partials);
  }
  const int64_t nb = K / kBlock;
  const unsigned gx = (unsigned)((nb + 63) / 64);
  if (tile_partials) {
    dim3 grid(gx, (unsigned)((M + kScoreTileRows - 1) / kScoreTileRows));
    quantize_kernel<T, true, kScoreTileRows><<<grid, 64, 0, stream>>>(
        x, M, K, ldx, ws_partials, np, amax_in, codes, scales, g_out, tile_partials);
  } else {
    constexpr int R = 8;
    dim3 grid(gx, (unsigned)((M + R - 1) / R));
    quantize_kernel<T, false, R><<<grid, 64, 0, stream>>>(
        x, M, K, ldx, ws_partials, np, amax_in, codes, scales, g_out, nullptr);
  }
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
