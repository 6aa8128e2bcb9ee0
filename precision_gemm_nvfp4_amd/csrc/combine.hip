// Scatter-add combine of the routed expert outputs:
//   out[t, :] += sum over rows r with scatter_index[r] == t of y_rows[r, :]
// (or, overwriting, out[t, :] = that sum, every output row written)
// where y_rows already holds row_weight[r] * Y[r] (written by the grouped GEMM
// into the workspace).  The rows of each output row are added in increasing
// row order, so the result does not depend on scheduling (fp32 atomics would).
//
//   count    rows per output row (atomic increments: order-free)
//   scan     exclusive prefix of the counts (one workgroup)
//   place    each row appended to its output row's list (atomic cursor), then
//   combine  one workgroup per output row: the list is sorted ascending in LDS
//            and the rows are added in that order, 4 columns per thread.
// With few output rows (decode batches) count, scan and place run in one
// workgroup with the counters in LDS: two launches in all instead of six.
#include "device_common.h"
#include "kernels.h"

namespace nvfp4 {

constexpr int kMaxListLds = 1024;           // rows per output row sorted in LDS
constexpr int kPlanSmallOut = 4096;         // output rows of the one-workgroup plan

// zeroes p[0..n) and q[0..n)
__global__ void combine_zero_kernel(int32_t* p, int32_t* q, int64_t n) {
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n;
       i += (int64_t)gridDim.x * blockDim.x) {
    p[i] = 0;
    q[i] = 0;
  }
}

__global__ void combine_count_kernel(const int32_t* __restrict__ scatter_index, int64_t rows,
                                     int64_t out_rows, int32_t* __restrict__ count) {
  for (int64_t r = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; r < rows;
       r += (int64_t)gridDim.x * blockDim.x) {
    const int64_t t = scatter_index[r];
    if (t >= 0 && t < out_rows) atomicAdd(count + t, 1);
  }
}

__global__ __launch_bounds__(1024) void combine_scan_kernel(const int32_t* __restrict__ count,
                                                            int64_t out_rows,
                                                            int32_t* __restrict__ start) {
  __shared__ int32_t sh[16];
  int32_t carry = 0;
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
  for (int64_t base = 0; base < out_rows; base += blockDim.x) {
    const int64_t t = base + threadIdx.x;
    const int32_t v = t < out_rows ? count[t] : 0;
    int32_t inc = v;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      int32_t u = __shfl_up(inc, o, 64);
      if (lane >= o) inc += u;
    }
    if (lane == 63) sh[wid] = inc;
    __syncthreads();
    int32_t before = carry, tot = 0;
    for (int w = 0; w < (int)(blockDim.x >> 6); ++w) {
      if (w < wid) before += sh[w];
      tot += sh[w];
    }
    if (t < out_rows) start[t] = before + inc - v;
    carry += tot;
    __syncthreads();
  }
  if (threadIdx.x == 0) start[out_rows] = carry;
}

__global__ void combine_place_kernel(const int32_t* __restrict__ scatter_index, int64_t rows,
                                     int64_t out_rows, const int32_t* __restrict__ start,
                                     int32_t* __restrict__ cursor, int32_t* __restrict__ list) {
  for (int64_t r = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; r < rows;
       r += (int64_t)gridDim.x * blockDim.x) {
    const int64_t t = scatter_index[r];
    if (t >= 0 && t < out_rows) list[start[t] + atomicAdd(cursor + t, 1)] = (int32_t)r;
  }
}

// count, scan and place in one workgroup (out_rows <= kPlanSmallOut): the
// counts and the cursors live in LDS, start[] goes to memory.
__global__ __launch_bounds__(1024) void combine_plan_small_kernel(const int32_t* __restrict__ scatter_index,
                                                                 int64_t rows, int64_t out_rows,
                                                                 int32_t* __restrict__ start,
                                                                 int32_t* __restrict__ list) {
  __shared__ int32_t cnt[kPlanSmallOut + 1];
  __shared__ int32_t sh[16];
  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  for (int64_t t = tid; t <= out_rows; t += blockDim.x) cnt[t] = 0;
  __syncthreads();
  for (int64_t r = tid; r < rows; r += blockDim.x) {
    const int64_t t = scatter_index[r];
    if (t >= 0 && t < out_rows) atomicAdd(cnt + t, 1);
  }
  __syncthreads();
  // exclusive prefix of cnt in chunks of blockDim; cnt[t] becomes start[t]
  int32_t carry = 0;
  for (int64_t base = 0; base < out_rows; base += blockDim.x) {
    const int64_t t = base + tid;
    const int32_t v = t < out_rows ? cnt[t] : 0;
    int32_t inc = v;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const int32_t u = __shfl_up(inc, o, 64);
      if (lane >= o) inc += u;
    }
    if (lane == 63) sh[wid] = inc;
    __syncthreads();
    int32_t before = carry, tot = 0;
    for (int w = 0; w < (int)(blockDim.x >> 6); ++w) {
      if (w < wid) before += sh[w];
      tot += sh[w];
    }
    if (t < out_rows) {
      cnt[t] = before + inc - v;
      start[t] = before + inc - v;
    }
    carry += tot;
    __syncthreads();
  }
  if (tid == 0) start[out_rows] = carry;
  for (int64_t r = tid; r < rows; r += blockDim.x) {
    const int64_t t = scatter_index[r];
    if (t >= 0 && t < out_rows) list[atomicAdd(cnt + t, 1)] = (int32_t)r;
  }
}

__global__ __launch_bounds__(256) void combine_rows_kernel(const float* __restrict__ y_rows,
                                                           int64_t N, const int32_t* __restrict__ start,
                                                           int32_t* __restrict__ list,
                                                           float* __restrict__ out, int64_t ldo,
                                                           bool vec4, bool overwrite) {
  __shared__ int32_t srt[kMaxListLds], raw[kMaxListLds];
  const int64_t t = blockIdx.x;
  const int32_t b = start[t], n = start[t + 1] - b;
  if (n == 0) {
    if (overwrite)
      for (int64_t c = threadIdx.x; c < N; c += blockDim.x) out[t * ldo + c] = 0.0f;
    return;
  }
  // ascending row order.  Lists that fit in LDS: each entry's rank is the
  // number of smaller entries (the rows are distinct), computed by all
  // threads at once.  Longer lists: insertion sort in place by one thread.
  int32_t* lst = list + b;
  if (n <= kMaxListLds) {
    for (int32_t i = threadIdx.x; i < n; i += blockDim.x) raw[i] = lst[i];
    __syncthreads();
    for (int32_t i = threadIdx.x; i < n; i += blockDim.x) {
      const int32_t v = raw[i];
      int32_t rank = 0;
      for (int32_t j = 0; j < n; ++j) rank += raw[j] < v;
      srt[rank] = v;
    }
  } else if (threadIdx.x == 0) {
    for (int32_t i = 1; i < n; ++i) {
      const int32_t v = lst[i];
      int32_t j = i - 1;
      while (j >= 0 && lst[j] > v) {
        lst[j + 1] = lst[j];
        --j;
      }
      lst[j + 1] = v;
    }
    for (int32_t i = 0; i < kMaxListLds; ++i) srt[i] = lst[i];
  }
  __syncthreads();
  float* o = out + t * ldo;
  for (int64_t c = (int64_t)threadIdx.x * 4; c < N; c += (int64_t)blockDim.x * 4) {
    if (vec4 && c + 4 <= N) {
      f32x4 acc = overwrite ? f32x4{0.0f, 0.0f, 0.0f, 0.0f} : *reinterpret_cast<const f32x4*>(o + c);
      // rows in groups of 8: the group's loads go out before its additions
      // (non-temporal: each routed row is read once)
      for (int32_t i0 = 0; i0 < n; i0 += 8) {
        f32x4 v[8];
#pragma unroll
        for (int q = 0; q < 8; ++q) {
          const int32_t i = i0 + q < n ? i0 + q : n - 1;
          const int32_t r = i < kMaxListLds ? srt[i] : lst[i];
          v[q] = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(y_rows + (int64_t)r * N + c));
        }
#pragma unroll
        for (int q = 0; q < 8; ++q) {
          if (i0 + q < n) {
            acc[0] = acc[0] + v[q][0];
            acc[1] = acc[1] + v[q][1];
            acc[2] = acc[2] + v[q][2];
            acc[3] = acc[3] + v[q][3];
          }
        }
      }
      *reinterpret_cast<f32x4*>(o + c) = acc;
    } else {
      for (int64_t cc = c; cc < c + 4 && cc < N; ++cc) {
        float acc = overwrite ? 0.0f : o[cc];
        for (int32_t i = 0; i < n; ++i) {
          const int32_t r = i < kMaxListLds ? srt[i] : lst[i];
          acc = acc + y_rows[(int64_t)r * N + cc];
        }
        o[cc] = acc;
      }
    }
  }
}

size_t combine_workspace_bytes(int64_t rows, int64_t N, int64_t out_rows) {
  auto a256 = [](size_t n) { return (n + 255) & ~size_t(255); };
  return a256((size_t)rows * N * 4) + 3 * a256((size_t)(out_rows + 1) * 4) + a256((size_t)rows * 4);
}

// The workspace: the rows, then count, start and cursor ([out_rows + 1]
// each) and the row lists ([rows]).
struct CombineWs {
  int32_t *count, *start, *cursor, *list;
  CombineWs(void* ws, int64_t rows, int64_t N, int64_t out_rows) {
    auto a256 = [](size_t n) { return (n + 255) & ~size_t(255); };
    char* w = static_cast<char*>(ws) + a256((size_t)rows * N * 4);
    count = reinterpret_cast<int32_t*>(w);
    w += a256((size_t)(out_rows + 1) * 4);
    start = reinterpret_cast<int32_t*>(w);
    w += a256((size_t)(out_rows + 1) * 4);
    cursor = reinterpret_cast<int32_t*>(w);
    w += a256((size_t)(out_rows + 1) * 4);
    list = reinterpret_cast<int32_t*>(w);
  }
};

hipError_t launch_combine_plan(int64_t rows, int64_t N, const int32_t* scatter_index,
                               int64_t out_rows, void* ws, hipStream_t stream) {
  const CombineWs w(ws, rows, N, out_rows);
  if (out_rows <= kPlanSmallOut) {
    combine_plan_small_kernel<<<1, 1024, 0, stream>>>(scatter_index, rows, out_rows, w.start, w.list);
    return hipGetLastError();
  }
  const int64_t zb = (out_rows + 255) / 256;
  combine_zero_kernel<<<(unsigned)(zb > 1024 ? 1024 : (zb < 1 ? 1 : zb)), 256, 0, stream>>>(w.count, w.cursor,
                                                                                          out_rows + 1);
  const int64_t rb = (rows + 255) / 256;
  const unsigned rg = (unsigned)(rb > 2048 ? 2048 : (rb < 1 ? 1 : rb));
  combine_count_kernel<<<rg, 256, 0, stream>>>(scatter_index, rows, out_rows, w.count);
  combine_scan_kernel<<<1, 1024, 0, stream>>>(w.count, out_rows, w.start);
  combine_place_kernel<<<rg, 256, 0, stream>>>(scatter_index, rows, out_rows, w.start, w.cursor, w.list);
  return hipGetLastError();
}

hipError_t launch_combine_rows(const float* y_rows, int64_t rows, int64_t N, int64_t out_rows,
                               float* out, int64_t ldo, bool overwrite, void* ws,
                               hipStream_t stream) {
  const CombineWs w(ws, rows, N, out_rows);
  if (out_rows > 0)
    combine_rows_kernel<<<(unsigned)out_rows, 256, 0, stream>>>(
        y_rows, N, w.start, w.list, out, ldo,
        N % 4 == 0 && ldo % 4 == 0 && (reinterpret_cast<uintptr_t>(out) & 15u) == 0, overwrite);
  return hipGetLastError();
}

hipError_t launch_combine(const float* y_rows, int64_t rows, int64_t N,
                          const int32_t* scatter_index, int64_t out_rows, float* out, int64_t ldo,
                          bool overwrite, void* ws, hipStream_t stream) {
  const hipError_t err = launch_combine_plan(rows, N, scatter_index, out_rows, ws, stream);
  if (err != hipSuccess) return err;
  return launch_combine_rows(y_rows, rows, N, out_rows, out, ldo, overwrite, ws, stream);
}

}  // namespace nvfp4
