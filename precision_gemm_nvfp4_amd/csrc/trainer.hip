// Trainer-side elementwise kernels.
//
// qdq_weights: the asymmetric W4A16 QAT of the QUADS technical summary
// (section 2.2A) fake-quantizes weights to NVFP4 on the trainer so its
// forward pass sees the same discretized weights as the rollout; activations
// stay BF16.  Per matrix: amax pass (atomic max per workgroup), then one pass
// that quantizes every 16-block and writes bf16(DQ) (plus, optionally, the
// codes, scales and global scale).
//
// guided_round: the rollout-guided rounding of the TRACE summary ("Core
// method", method step four).  Under the rollout block's scale S, the trainer
// value v = x/S has two neighbouring E2M1 levels q- <= v <= q+; instead of
// round-to-nearest the kernel keeps whichever is closer to the recorded
// rollout level.  Round-to-nearest is one of the two neighbours, so the
// kernel computes it (exactly), finds on which side of v it lies with one
// exact fma, takes the neighbour on the other side, and compares distances
// to the rollout level.
#include "device_common.h"
#include "kernels.h"

namespace nvfp4 {

// ---------------------------------------------------------------------------
// weight QDQ
// ---------------------------------------------------------------------------
__device__ __forceinline__ float absmax8(const u32x4& a, float m) {
#pragma unroll
  for (int i = 0; i < 4; ++i) m = fmaxf(m, fmaxf(fabsf(bf16_lo(a[i])), fabsf(bf16_hi(a[i]))));
  return m;
}

// grid: x over the matrix's 16-byte chunks (grid-stride, four loads in flight
// per thread), y = matrix
__global__ __launch_bounds__(256) void qdq_amax_kernel(const __bf16* __restrict__ w, int64_t per_mat,
                                                       float* __restrict__ amax) {
  const int64_t mat = blockIdx.y;
  const u32x4* p = reinterpret_cast<const u32x4*>(w + mat * per_mat);
  const int64_t chunks = per_mat / 8;
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  int64_t c = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  float m = 0.0f;
  for (; c + 3 * stride < chunks; c += 4 * stride) {
    const u32x4 v0 = p[c], v1 = p[c + stride], v2 = p[c + 2 * stride], v3 = p[c + 3 * stride];
    m = absmax8(v3, absmax8(v2, absmax8(v1, absmax8(v0, m))));
  }
  for (; c < chunks; c += stride) m = absmax8(p[c], m);
  m = wave_max(m);
  __shared__ float red[4];
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = m;
  __syncthreads();
  if (threadIdx.x == 0) {
    float b = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
    atomic_max_nonneg(amax + mat, b);
  }
}

// One 16-block (elements a, c as bf16 pairs) quantized under g: writes
// bf16(DQ) at w_qdq + base and, when asked, the codes and the block scale.
__device__ __forceinline__ void qdq_block(const u32x4& a, const u32x4& c, const BlockScaler& bsc,
                                          int64_t base, __bf16* __restrict__ w_qdq,
                                          uint8_t* __restrict__ codes, uint8_t* __restrict__ scales) {
  float v[16];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    v[2 * i] = bf16_lo(a[i]);
    v[2 * i + 1] = bf16_hi(a[i]);
    v[8 + 2 * i] = bf16_lo(c[i]);
    v[8 + 2 * i + 1] = bf16_hi(c[i]);
  }
  uint32_t sb, w0, w1;
  const float S = quantize_block16(v, bsc, &sb, &w0, &w1);
  // bf16(DQ) two elements at a time: the hardware FP4 convert gives the codes'
  // exact values, one fp32 multiply each rounds value * S, one packed convert
  // rounds both to bf16.
  float d[16];
  e2m1_unpack8(w0, d);
  e2m1_unpack8(w1, d + 8);
  u32x4 o0, o1;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const uint32_t word = pack_bf16x2_rne(d[2 * i] * S, d[2 * i + 1] * S);
    if (i < 4) o0[i] = word; else o1[i - 4] = word;
  }
  u32x4* dst = reinterpret_cast<u32x4*>(w_qdq + base);
  dst[0] = o0;
  dst[1] = o1;
  if (codes) *reinterpret_cast<u32x2*>(codes + base / 2) = u32x2{w0, w1};
  if (scales) scales[base / kBlock] = (uint8_t)sb;
}

// grid: x over the matrix's 16-blocks (grid-stride), y = matrix in the group
__global__ __launch_bounds__(256) void qdq_kernel(const __bf16* __restrict__ w, int64_t N, int64_t K,
                                                  const float* __restrict__ amax,
                                                  __bf16* __restrict__ w_qdq, uint8_t* __restrict__ codes,
                                                  uint8_t* __restrict__ scales, float* __restrict__ g_out) {
  const int64_t mat = blockIdx.y;
  const float g = global_scale_from_amax(amax[mat]);
  const BlockScaler bsc = make_block_scaler(g);
  if (g_out && blockIdx.x == 0 && threadIdx.x == 0) g_out[mat] = g;
  const int64_t nb = N * (K / kBlock);                  // blocks in this matrix
  for (int64_t b = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; b < nb;
       b += (int64_t)gridDim.x * blockDim.x) {
    const int64_t base = mat * N * K + b * kBlock;      // blocks are contiguous in row-major order
    const u32x4* src = reinterpret_cast<const u32x4*>(w + base);
    qdq_block(src[0], src[1], bsc, base, w_qdq, codes, scales);
  }
}

// ---------------------------------------------------------------------------
// One-pass weight QDQ: every matrix read once
// ---------------------------------------------------------------------------
// A cooperative grid (every workgroup resident, one per CU) keeps each
// workgroup's slice of the matrices on chip from their amax to their
// quantization.  The matrices go P at a time ("step" j covers matrices
// j P .. j P + P - 1, each with its own amax), so that a step holds KB P
// blocks per data thread whatever the matrix size.  A workgroup is QDQ1_DW
// data waves plus one sync wave, which talk only through LDS flags (no
// workgroup barrier after the start), so a data wave never waits for the
// grid-wide gather unless it is not done by the time it is needed.
//
// Data wave, step s: wait for its own direct loads of step s + 1 into the
// LDS slice buffer (a wave loads and reads only its own 2 KB of each
// segment, so the buffer needs no barrier), copy its blocks into registers
// while reducing each matrix's amax, post the maxima and then its flag;
// issue the loads of step s + 2 into the slice buffer; wait until the sync
// wave has posted step s's global maxima and quantize step s from registers
// (buffer stores).  So one step lands in LDS while the previous one is
// reduced and the one before it is written.
//
// The maxima go through two LDS buffers by step parity: a data wave writes
// step j + 1's while the sync wave may still read step j's, and writes step
// j + 2's only after quantizing step j, which waited for the sync wave to
// finish step j.
//
// Sync wave, step j: wait until every data wave has posted step j, reduce
// the maxima, publish them (one 64-bit store of sequence number and value
// per matrix into this workgroup's own slot: nothing is read-modify-written)
// and poll every workgroup's slots until all carry step j's sequence number,
// then post the global maxima for the data waves.  Only the sync wave
// touches the slots, so no data wave waits for its own loads to publish
// anything (a wave's memory fence would wait for all of them).  A wait that
// runs past spin_limit gives up, sets a flag in the workspace and lets every
// wave finish (only possible when the workgroups were not all resident).
constexpr int QDQ1_DW = 12;                    // data waves per workgroup
constexpr int QDQ1_DT = 64 * QDQ1_DW;          // data threads
constexpr int QDQ1_SEG = QDQ1_DT * 32;         // bytes of one block per data thread
constexpr int QDQ1_MAX_BLK = 4;                // blocks per data thread and step
constexpr int QDQ1_MAX_WG = 1024;              // workgroups (CUs) the publication slots hold
constexpr int QDQ1_MAX_P = 4;                  // matrices per step

__device__ __forceinline__ __amdgpu_buffer_rsrc_t qdq1_rsrc(const void* base, int64_t bytes) {
  const uint64_t b = reinterpret_cast<uint64_t>(base);
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)b);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(b >> 32));
  const uint32_t n = __builtin_amdgcn_readfirstlane((uint32_t)(bytes < 0 ? 0 : (bytes < 0xFFFFFFFFll ? bytes : 0xFFFFFFFFll)));
  return __builtin_amdgcn_make_buffer_rsrc(reinterpret_cast<void*>(((uint64_t)hi << 32) | lo), (short)0, (int)n,
                                           0x00020000);
}

// LDS flag accesses: volatile, and fenced against the compiler moving other
// LDS accesses across them.  A wave's LDS operations complete in order, and
// a writer waits for its data writes before writing the flag.
__device__ __forceinline__ uint32_t lds_flag_read(const uint32_t* f) {
  asm volatile("" ::: "memory");
  const uint32_t v = *reinterpret_cast<const volatile uint32_t*>(f);
  asm volatile("" ::: "memory");
  return v;
}
__device__ __forceinline__ void lds_flag_write(uint32_t* f, uint32_t v) {
  __builtin_amdgcn_s_waitcnt(0xc07f);         // lgkmcnt(0): the data went first
  asm volatile("" ::: "memory");
  *reinterpret_cast<volatile uint32_t*>(f) = v;
  asm volatile("" ::: "memory");
}

// KB: blocks per data thread and matrix; P: matrices per step; STORES: store
// instructions per block (bf16 output, plus the codes and the scale byte
// when asked).  Every store instruction is issued (a block past its matrix,
// or of a matrix past the last, stores out of bounds and is dropped), so the
// wait for a step's loads can leave exactly KB P STORES stores outstanding.
template <int KB, int P, int STORES>
__global__ __launch_bounds__(64 * (QDQ1_DW + 1), 1) void qdq_onepass_kernel(
    const __bf16* __restrict__ w, int64_t nmat, int64_t nb, __bf16* __restrict__ w_qdq,
    uint8_t* __restrict__ codes, uint8_t* __restrict__ scales, float* __restrict__ g_out,
    uint32_t* __restrict__ sync, uint32_t spin_limit) {
  constexpr int NB = KB * P;                   // blocks per data thread and step
  static_assert(NB <= QDQ1_MAX_BLK && P <= QDQ1_MAX_P && NB * STORES <= 63, "step size");
  extern __shared__ __attribute__((aligned(16))) unsigned char slice[];   // NB * QDQ1_SEG bytes
  __shared__ float red[2][QDQ1_DW][P];         // data wave w's maxima of step j in [j & 1]
  __shared__ uint32_t posted[QDQ1_DW];         // j + 1: data wave w posted step j
  __shared__ float sh_amax[2][P];              // global maxima of step j in [j & 1]
  __shared__ uint32_t ready;                   // j + 1: sh_amax holds step j
  // publication slots [2][P][nwg] (parity of the step) and the give-up flag
  uint64_t* slots = reinterpret_cast<uint64_t*>(sync);
  uint32_t* gave_up = sync + 4 * QDQ1_MAX_P * QDQ1_MAX_WG;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const uint32_t nwg = gridDim.x;
  const int64_t wg = blockIdx.x;
  const int64_t nsteps = (nmat + P - 1) / P;
  constexpr uint32_t OOB = 0x80000000u;        // past every per-matrix array

  if (tid < QDQ1_DW) posted[tid] = 0u;
  if (tid == 0) ready = 0u;
  __syncthreads();

  if (wave == QDQ1_DW) {
    // ---- sync wave ----
    bool gave = false;
    for (int64_t j = 0; j < nsteps; ++j) {
      const uint32_t tag = (uint32_t)(j + 1);
      // every data wave's maxima of step j (lane w watches data wave w)
      uint32_t spins = 0;
      while (!__all(lane >= QDQ1_DW || lds_flag_read(&posted[lane < QDQ1_DW ? lane : 0]) >= tag)) {
        __builtin_amdgcn_s_sleep(1);
        if (++spins >= spin_limit) { gave = true; break; }
      }
      float m[P];
#pragma unroll
      for (int p = 0; p < P; ++p) {
        m[p] = 0.0f;
#pragma unroll
        for (int i = 0; i < QDQ1_DW; ++i) m[p] = fmaxf(m[p], red[j & 1][i][p]);
      }
      // publish this workgroup's maxima, gather everyone's
      uint64_t* sl = slots + (j & 1) * P * nwg;
      const uint64_t seq = (uint64_t)tag << 32;
      if (lane == 0) {
#pragma unroll
        for (int p = 0; p < P; ++p)
          __hip_atomic_store(&sl[p * nwg + wg], seq | __float_as_uint(m[p]), __ATOMIC_RELAXED,
                             __HIP_MEMORY_SCOPE_AGENT);
      }
      float a[P];
      spins = 0;
      for (;;) {
        bool all = true;
#pragma unroll
        for (int p = 0; p < P; ++p) {
          a[p] = 0.0f;
          for (uint32_t i = (uint32_t)lane; i < nwg; i += 64) {
            const uint64_t v = __hip_atomic_load(&sl[p * nwg + i], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            all = all && (v >> 32) == (uint64_t)tag;
            a[p] = fmaxf(a[p], __uint_as_float((uint32_t)v));
          }
        }
        if (__all(all) || gave) break;
        __builtin_amdgcn_s_sleep(2);
        if (++spins >= spin_limit) { gave = true; break; }
      }
#pragma unroll
      for (int p = 0; p < P; ++p) {
        const float v = wave_max(a[p]);
        if (lane == 0) sh_amax[j & 1][p] = v;
      }
      if (lane == 0) lds_flag_write(&ready, tag);
    }
    if (gave && lane == 0) __hip_atomic_store(gave_up, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    return;
  }

  // ---- data waves ----
  const int dt = tid;                          // 0 .. QDQ1_DT - 1
  // Block k of a step (matrix p = k / KB of the step, kk = k % KB) of data
  // thread dt is block (kk * nwg + wg) * QDQ1_DT + dt of that matrix, so
  // segment k of the slice is QDQ1_SEG contiguous bytes of the matrix, and
  // wave `wave` loads (and later reads) its own 2 KB of every segment.
  uint32_t voff[KB][2];
#pragma unroll
  for (int k = 0; k < KB; ++k)
#pragma unroll
    for (int i = 0; i < 2; ++i)
      voff[k][i] = (uint32_t)(((int64_t)k * nwg + wg) * QDQ1_SEG) + (uint32_t)(wave * 2048 + i * 1024 + lane * 16);
  // matrix mi's bytes, or none past the last matrix (reads give zeros,
  // stores are dropped)
  auto mat_bytes = [&](int64_t mi, int64_t per) { return mi < nmat ? per : (int64_t)0; };
  // The slice of step s into LDS (reads past a matrix return zeros).
  auto issue = [&](int64_t s) {
#pragma unroll
    for (int p = 0; p < P; ++p) {
      const int64_t mi = s * P + p;
      const __amdgpu_buffer_rsrc_t r = qdq1_rsrc(w + (mi < nmat ? mi : 0) * nb * kBlock, mat_bytes(mi, nb * kBlock * 2));
#pragma unroll
      for (int k = 0; k < KB; ++k)
#pragma unroll
        for (int i = 0; i < 2; ++i)
          __builtin_amdgcn_raw_ptr_buffer_load_lds(
              r, (__attribute__((address_space(3))) void*)(slice + (p * KB + k) * QDQ1_SEG + wave * 2048 + i * 1024),
              16, (int)voff[k][i], 0, 0, 0);
    }
  };
  // step s's blocks into registers, its maxima and then this wave's flag
  auto copy_amax = [&](int64_t s, u32x4 (&b)[NB][2]) {
#pragma unroll
    for (int p = 0; p < P; ++p) {
      float m = 0.0f;
#pragma unroll
      for (int k = 0; k < KB; ++k) {
        const int j = p * KB + k;
        const u32x4* src = reinterpret_cast<const u32x4*>(slice + j * QDQ1_SEG + dt * 32);
        b[j][0] = src[0];
        b[j][1] = src[1];
        m = absmax8(b[j][1], absmax8(b[j][0], m));
      }
      m = wave_max(m);
      if (lane == 0) red[s & 1][wave][p] = m;
    }
    if (lane == 0) lds_flag_write(&posted[wave], (uint32_t)(s + 1));
  };
  // Step s's blocks under their matrices' global amax: bf16(DQ) (two
  // elements per fp32 multiply and packed convert, as in qdq_block), codes
  // and scales.
  auto quant = [&](int64_t s, const u32x4 (&b)[NB][2]) {
    uint32_t spins = 0;
    while (lds_flag_read(&ready) < (uint32_t)(s + 1)) {   // uniform: one LDS word
      __builtin_amdgcn_s_sleep(1);
      if (++spins >= spin_limit) {
        if (lane == 0) __hip_atomic_store(gave_up, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        break;
      }
    }
#pragma unroll
    for (int p = 0; p < P; ++p) {
      const int64_t mi = s * P + p;
      const int64_t mb = mi < nmat ? mi : 0;
      const float g = global_scale_from_amax(sh_amax[s & 1][p]);
      const BlockScaler bsc = make_block_scaler(g);
      if (g_out && mi < nmat && wg == 0 && dt == 0) g_out[mi] = g;
      const __amdgpu_buffer_rsrc_t ro = qdq1_rsrc(w_qdq + mb * nb * kBlock, mat_bytes(mi, nb * kBlock * 2));
      const __amdgpu_buffer_rsrc_t rc = qdq1_rsrc(codes ? codes + mb * nb * 8 : nullptr, codes ? mat_bytes(mi, nb * 8) : 0);
      const __amdgpu_buffer_rsrc_t rs = qdq1_rsrc(scales ? scales + mb * nb : nullptr, scales ? mat_bytes(mi, nb) : 0);
#pragma unroll
      for (int k = 0; k < KB; ++k) {
        const int j = p * KB + k;
        const int64_t bi = ((int64_t)k * nwg + wg) * QDQ1_DT + dt;
        const bool in = bi < nb;
        float v[16];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          v[2 * i] = bf16_lo(b[j][0][i]);
          v[2 * i + 1] = bf16_hi(b[j][0][i]);
          v[8 + 2 * i] = bf16_lo(b[j][1][i]);
          v[8 + 2 * i + 1] = bf16_hi(b[j][1][i]);
        }
        uint32_t sb, w0, w1;
        const float S = quantize_block16(v, bsc, &sb, &w0, &w1);
        float d[16];
        e2m1_unpack8(w0, d);
        e2m1_unpack8(w1, d + 8);
        u32x4 o0, o1;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          const uint32_t word = pack_bf16x2_rne(d[2 * i] * S, d[2 * i + 1] * S);
          if (i < 4) o0[i] = word; else o1[i - 4] = word;
        }
        const uint32_t ob = in ? (uint32_t)(bi * 32) : OOB;
        __builtin_amdgcn_raw_buffer_store_b128(o0, ro, (int)ob, 0, 0);
        __builtin_amdgcn_raw_buffer_store_b128(o1, ro, (int)(in ? ob + 16 : OOB), 0, 0);
        if constexpr (STORES >= 3) {
          if (codes) __builtin_amdgcn_raw_buffer_store_b64(u32x2{w0, w1}, rc, (int)(in ? (uint32_t)(bi * 8) : OOB), 0, 0);
          else __builtin_amdgcn_raw_buffer_store_b8((uint8_t)sb, rs, (int)(in ? (uint32_t)bi : OOB), 0, 0);
        }
        if constexpr (STORES == 4)
          __builtin_amdgcn_raw_buffer_store_b8((uint8_t)sb, rs, (int)(in ? (uint32_t)bi : OOB), 0, 0);
      }
    }
  };
  u32x4 R0[NB][2], R1[NB][2];
  // Step s: R_nxt receives step s + 1 (its loads went out in step s - 1, and
  // `after` store instructions followed them), R_cur holds step s.
  auto step = [&](int64_t s, u32x4 (&cur)[NB][2], u32x4 (&nxt)[NB][2], auto after_c) {
    constexpr int after = decltype(after_c)::value;
    if (s >= nsteps) return;                   // uniform
    if (s + 1 < nsteps) {
      __builtin_amdgcn_s_waitcnt((after & 15) | 0x70 | 0xf00 | ((after >> 4) << 14));   // vmcnt(after)
      copy_amax(s + 1, nxt);
    }
    if (s + 2 < nsteps) issue(s + 2);
    if (s >= 0) quant(s, cur);
  };
  issue(0);
  step(-1, R1, R0, std::integral_constant<int, 0>{});     // step 0 into R0, step 1 out
  step(0, R0, R1, std::integral_constant<int, 0>{});      // step 0 quantized, 1 into R1, 2 out
  for (int64_t s = 1; s < nsteps; s += 2) {
    step(s, R1, R0, std::integral_constant<int, NB * STORES>{});
    step(s + 1, R0, R1, std::integral_constant<int, NB * STORES>{});
  }
}

// Two passes over all matrices (one amax launch, then one quantize launch):
// for shapes the one-pass kernel does not take.
static hipError_t launch_qdq_two_pass(const __bf16* w, int64_t nmat, int64_t N, int64_t K, __bf16* w_qdq,
                                      uint8_t* codes, uint8_t* scales, float* g, float* ws_amax,
                                      hipStream_t stream) {
  hipError_t err = launch_fill_f32(ws_amax, nmat, 0.0f, stream);
  if (err != hipSuccess) return err;
  const int64_t per_mat = N * K;
  const int64_t nb = N * (K / kBlock);
  int64_t ga = (per_mat / 8 + 255) / 256;                // about 4096 workgroups in all
  ga = ga > 4096 / nmat + 1 ? 4096 / nmat + 1 : (ga < 1 ? 1 : ga);
  qdq_amax_kernel<<<dim3((unsigned)ga, (unsigned)nmat), 256, 0, stream>>>(w, per_mat, ws_amax);
  int64_t gq = (nb + 255) / 256;                         // about 16384 workgroups in all
  gq = gq > 16384 / nmat + 1 ? 16384 / nmat + 1 : gq;
  qdq_kernel<<<dim3((unsigned)gq, (unsigned)nmat), 256, 0, stream>>>(w, N, K, ws_amax, w_qdq, codes,
                                                                     scales, g);
  return hipGetLastError();
}

// Workspace: the one-pass kernel's publication slots and give-up flag, or
// the two-pass launch's per-matrix amax.
size_t qdq_workspace_bytes(int64_t nmat) {
  const size_t one = (size_t)QDQ1_MAX_P * QDQ1_MAX_WG * 16 + 4, two = (size_t)(nmat > 0 ? nmat : 0) * 4;
  return ((one > two ? one : two) + 255) / 256 * 256;
}

template <int KB, int P, int STORES>
static hipError_t launch_qdq_onepass_kb(const __bf16* w, int64_t nmat, int64_t nb, __bf16* w_qdq, uint8_t* codes,
                                        uint8_t* scales, float* g, uint32_t* sync, int grid, hipStream_t stream) {
  auto kern = qdq_onepass_kernel<KB, P, STORES>;
  const size_t lds = (size_t)KB * P * QDQ1_SEG;
  hipError_t err = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
  if (err != hipSuccess) return err;
  int per_cu = 0;
  err = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kern, 64 * (QDQ1_DW + 1), lds);
  if (err != hipSuccess) return err;
  if (per_cu < 1) return hipErrorCooperativeLaunchTooLarge;
  uint32_t spin_limit = 1u << 21;              // polls of about 256 cycles: well over a second
  void* args[] = {(void*)&w, (void*)&nmat, (void*)&nb, (void*)&w_qdq, (void*)&codes, (void*)&scales,
                  (void*)&g, (void*)&sync, (void*)&spin_limit};
  return hipLaunchCooperativeKernel(reinterpret_cast<const void*>(kern), dim3((unsigned)grid),
                                    dim3(64 * (QDQ1_DW + 1)), args, (unsigned)lds, stream);
}

template <int STORES>
static hipError_t launch_qdq_onepass(const __bf16* w, int64_t nmat, int64_t nb, int kb, __bf16* w_qdq,
                                     uint8_t* codes, uint8_t* scales, float* g, uint32_t* sync, int grid,
                                     hipStream_t stream) {
  // P = 4 / KB matrices per step: four blocks per data thread and step
  switch (kb) {
    case 1: return launch_qdq_onepass_kb<1, 4, STORES>(w, nmat, nb, w_qdq, codes, scales, g, sync, grid, stream);
    case 2: return launch_qdq_onepass_kb<2, 2, STORES>(w, nmat, nb, w_qdq, codes, scales, g, sync, grid, stream);
    case 3: return launch_qdq_onepass_kb<3, 1, STORES>(w, nmat, nb, w_qdq, codes, scales, g, sync, grid, stream);
    default: return launch_qdq_onepass_kb<4, 1, STORES>(w, nmat, nb, w_qdq, codes, scales, g, sync, grid, stream);
  }
}

// The one-pass kernel when the device runs cooperative launches, there are
// at least two steps of matrices, and each matrix fills one to QDQ1_MAX_BLK
// blocks per data thread (3.1 M to 12.6 M elements on 256 CUs); else two
// passes.
hipError_t launch_qdq(const __bf16* w, int64_t nmat, int64_t N, int64_t K, __bf16* w_qdq,
                      uint8_t* codes, uint8_t* scales, float* g, void* ws, hipStream_t stream) {
  uint32_t* sync = static_cast<uint32_t*>(ws);
  const int64_t nb = N * (K / kBlock);
  int dev = 0, cus = 0, coop = 0;
  hipError_t err = hipGetDevice(&dev);
  if (err == hipSuccess) err = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
  if (err == hipSuccess) err = hipDeviceGetAttribute(&coop, hipDeviceAttributeCooperativeLaunch, dev);
  if (err != hipSuccess) return err;
  const int64_t per = (int64_t)cus * QDQ1_DT;                // blocks one pass of the grid takes
  const int64_t kb = per > 0 ? (nb + per - 1) / per : 0;
  const int64_t p = kb >= 1 && kb <= QDQ1_MAX_BLK ? QDQ1_MAX_BLK / kb : 1;
  if (!coop || cus > QDQ1_MAX_WG || nb < per || kb > QDQ1_MAX_BLK || nmat < 2 * p)
    return launch_qdq_two_pass(w, nmat, N, K, w_qdq, codes, scales, g, reinterpret_cast<float*>(sync), stream);
  err = launch_fill_f32(reinterpret_cast<float*>(sync), 4 * QDQ1_MAX_P * QDQ1_MAX_WG + 1, 0.0f, stream);
  if (err != hipSuccess) return err;
  const int stores = 2 + (codes ? 1 : 0) + (scales ? 1 : 0);
  switch (stores) {
    case 2: return launch_qdq_onepass<2>(w, nmat, nb, (int)kb, w_qdq, codes, scales, g, sync, cus, stream);
    case 3: return launch_qdq_onepass<3>(w, nmat, nb, (int)kb, w_qdq, codes, scales, g, sync, cus, stream);
    default: return launch_qdq_onepass<4>(w, nmat, nb, (int)kb, w_qdq, codes, scales, g, sync, cus, stream);
  }
}

// MXFP4 weight QDQ: blocks of 32 along K with their own E8M0 scale and no
// global scale, so one pass suffices.  bf16(DQ) is DQ itself: value * 2^X has
// at most two significant bits.  grid-stride over the 32-blocks of all rows.
__global__ __launch_bounds__(256) void mx_qdq_kernel(const __bf16* __restrict__ w, int64_t nblk,
                                                     __bf16* __restrict__ w_qdq,
                                                     uint8_t* __restrict__ codes,
                                                     uint8_t* __restrict__ scales) {
  for (int64_t b = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; b < nblk;
       b += (int64_t)gridDim.x * blockDim.x) {
    const u32x4* src = reinterpret_cast<const u32x4*>(w + b * kMxBlock);
    u32x4 q[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) q[i] = src[i];
    float v[32];
    float amax = 0.0f;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      v[2 * i] = bf16_lo(q[i >> 2][i & 3]);
      v[2 * i + 1] = bf16_hi(q[i >> 2][i & 3]);
      amax = fmaxf(amax, fmaxf(fabsf(v[2 * i]), fabsf(v[2 * i + 1])));
    }
    const uint32_t sb = mx_scale_byte(amax);
    uint32_t cw[4];
    mx_pack32(v, sb, cw);
    const float S = e8m0_value(sb);
    u32x4 o[4];
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      float d[8];
      e2m1_unpack8(cw[c], d);
#pragma unroll
      for (int i = 0; i < 4; ++i) o[c][i] = pack_bf16x2_rne(d[2 * i] * S, d[2 * i + 1] * S);
    }
    u32x4* dst = reinterpret_cast<u32x4*>(w_qdq + b * kMxBlock);
#pragma unroll
    for (int i = 0; i < 4; ++i) dst[i] = o[i];
    if (codes) *reinterpret_cast<u32x4*>(codes + b * 16) = u32x4{cw[0], cw[1], cw[2], cw[3]};
    if (scales) scales[b] = (uint8_t)sb;
  }
}

hipError_t launch_mx_qdq(const __bf16* w, int64_t rows, int64_t K, __bf16* w_qdq, uint8_t* codes,
                         uint8_t* scales, hipStream_t stream) {
  const int64_t nblk = rows * (K / kMxBlock);
  if (nblk == 0) return hipGetLastError();
  int64_t grid = (nblk + 255) / 256;
  if (grid > 8192) grid = 8192;
  mx_qdq_kernel<<<(unsigned)grid, 256, 0, stream>>>(w, nblk, w_qdq, codes, scales);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// guided rounding
// ---------------------------------------------------------------------------
// Nibble-parallel helpers: eight 4-bit fields of a word at once.
// Bit 3 of each nibble set where the nibble's low three bits are zero (bit 3
// of the nibble must be clear: t + 7 <= 14 carries into bit 3 only).
__device__ __forceinline__ uint32_t nibble_zero3(uint32_t t) { return ~(t + 0x77777777u) & 0x88888888u; }
// Bit 3 of each nibble set where the whole nibble is zero.
__device__ __forceinline__ uint32_t nibble_zero4(uint32_t t) {
  return ~(t | ((t & 0x77777777u) + 0x77777777u)) & 0x88888888u;
}
// Bit j of b (j < 8) to bit 0 of nibble j.
__device__ __forceinline__ uint32_t nibble_spread8(uint32_t b) {
  b = (b | (b << 12)) & 0x000F000Fu;
  b = (b | (b << 6)) & 0x03030303u;
  return (b | (b << 3)) & 0x11111111u;
}

// RECORD = false: roll holds the rollout codes [M, K/2], and hist counts the
// elements whose round-to-nearest index is 0, 1 and >= 2 from the rollout's.
// RECORD = true: roll holds the mantissa-only record [M, K/8] (the low code
// bit of each element, element 8i + j in bit j of byte i); the output is the
// neighbour whose magnitude index has that low bit (neighbouring levels differ
// in it), and hist counts the elements kept at round-to-nearest and moved.
// MX = true: MXFP4 rollout scales, one E8M0 byte per 32 elements, S = 2^X
// and no global scale (roll_global unused).
//
// Every element is rounded on its own once its block's rollout scale is
// known, so a lane takes 8 consecutive elements (item e: elements 8e .. 8e+7
// of the row-major [M, K] tensor, half a scale block): its 16-byte load of x,
// its code word or record byte, and its 16-byte store of x_fq sit next to the
// neighbouring lanes' and every access of a wave is one contiguous run.
constexpr int kGuidedThreads = 1024;

template <typename T, bool RECORD, bool MX = false>
__global__ __launch_bounds__(kGuidedThreads) void guided_kernel(
    const T* __restrict__ x, uint32_t M, uint32_t K, int64_t ldx, const uint8_t* __restrict__ roll,
    const uint8_t* __restrict__ roll_scales, const float* __restrict__ roll_global,
    uint8_t* __restrict__ guided, __bf16* __restrict__ x_fq, unsigned long long* __restrict__ hist) {
  const uint32_t per_row = K / 8;
  const uint64_t total = (uint64_t)M * per_row;   // >= 1: the launcher skips empty inputs
  const float g_roll = MX ? 1.0f : *roll_global;
  const bool dense = ldx == (int64_t)K;
  uint32_t h0 = 0, h1 = 0, h2 = 0;
  // A lane's next item is loaded before the current one is rounded (from a
  // clamped index, unconditionally), so each trip of the grid-stride loop has
  // its loads in flight during the previous trip's arithmetic.
  struct In {
    u32x4 q[sizeof(T) / 2];                       // 8 elements
    uint32_t sc;                                  // rollout scale byte
    uint32_t rw;                                  // code word or record byte
  };
  auto fetch = [&](uint64_t i, In& in) {
    int64_t xo = (int64_t)i * 8;
    if (!dense) xo += (int64_t)((uint32_t)i / per_row) * (ldx - (int64_t)K);
#pragma unroll
    for (int j = 0; j < (int)(sizeof(T) / 2); ++j)   // x_train is read once: non-temporal
      in.q[j] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(x + xo) + j);
    in.sc = roll_scales[MX ? i >> 2 : i >> 1];
    in.rw = RECORD ? (uint32_t)roll[i] : reinterpret_cast<const uint32_t*>(roll)[i];
  };
  const uint64_t stride = (uint64_t)gridDim.x * blockDim.x;
  uint64_t e = (uint64_t)blockIdx.x * blockDim.x + threadIdx.x;
  In cur, nxt;
  fetch(e < total ? e : total - 1, cur);
  for (; e < total; e += stride) {
    fetch(e + stride < total ? e + stride : e, nxt);
    const u32x4* q = cur.q;
    const uint32_t sc = cur.sc, rw = cur.rw;
    float v[8];
    if constexpr (sizeof(T) == 2) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        v[2 * i] = bf16_lo(q[0][i]);
        v[2 * i + 1] = bf16_hi(q[0][i]);
      }
    } else {
#pragma unroll
      for (int i = 0; i < 8; ++i) v[i] = __uint_as_float(q[i >> 2][i & 3]);
    }
    const float S = MX ? e8m0_value(sc) : e4m3_value(sc) * g_roll;
    // round-to-nearest codes under S (fast path, exact fallback)
    uint32_t w;
    if (S >= 0x1p-100f) {
      float iu, id;
      e2m1_brackets(S, iu, id);
      w = e2m1_pack8_fast(v, iu, id, S);
    } else {
      w = e2m1_pack8_exact(v, S);
    }
    // Candidates in magnitude space: the round-to-nearest index i and, by the
    // exact sign of i's level * S - |x|, its neighbour on x's side (i + 1 up
    // to 7, i - 1, or none when x sits on the level).  Both carry x's sign
    // bit (neighbours never straddle zero with opposite signs, and a zero
    // takes x's sign).  The full-code rule picks the candidate on the rollout
    // level's side in signed index order, which for two adjacent levels is
    // the one closer to it; the record rule picks the one whose index has the
    // recorded low bit.  Only the sign of each element's difference is taken
    // per element (bit 3 of its nibble in LT or GT); the choice itself runs
    // on the eight nibbles of the code word at once (nibble_*: no carry or
    // borrow crosses a nibble, as each comment shows).
    const bool live = S != 0.0f;                  // S == 0: every code stays at magnitude 0
    float Lm[8];
    e2m1_unpack8(w & 0x77777777u, Lm);
    uint32_t LT = 0, GT = 0;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const float d = __builtin_fmaf(Lm[j], S, -fabsf(v[j]));   // exact sign
      LT |= d < 0.0f ? 8u << (4 * j) : 0u;
      GT |= d > 0.0f ? 8u << (4 * j) : 0u;
    }
    const uint32_t I = w & 0x77777777u, SGN = w & 0x88888888u;
    // i < 7: bit 3 of i + 1 clear (i + 1 <= 8)
    const uint32_t INC = (LT & ~(I + 0x11111111u) & 0x88888888u) >> 3;   // neighbour i + 1
    const uint32_t DEC = GT >> 3;                 // neighbour i - 1 (d > 0 needs i >= 1)
    uint32_t pick;
    if constexpr (RECORD) {
      const uint32_t flip = live ? (I ^ nibble_spread8(rw)) & 0x11111111u : 0u;
      pick = I + (flip & INC) - (flip & DEC);
      const uint32_t moved = __builtin_popcount(flip & (INC | DEC));
      h0 += 8u - moved;
      h1 += moved;
    } else {
      // r = the rollout index, on x's side when its sign is x's or it is
      // zero ("same"); the larger candidate HI is picked when same and
      // r >= HI, else the smaller one.  (Checked against the signed-index
      // rule for every index, neighbour, sign and rollout code.)
      const uint32_t R = rw & 0x77777777u, RS = rw & 0x88888888u;
      const uint32_t same = (~(RS ^ SGN) | ~(R + 0x77777777u)) & 0x88888888u;   // r + 7 <= 14
      const uint32_t HI = I + INC;
      const uint32_t ge = ((R | 0x88888888u) - HI) & 0x88888888u;           // 8 + r - HI in 1..15
      const uint32_t sel = live ? (same & ge) >> 3 : 0u;
      pick = I - DEC + (sel & (INC | DEC));
      // index distance 0 and 1 (same side: |r - i|, else r + i)
      const uint32_t AD = (R | 0x88888888u) - I;                         // 8 + r - i in 1..15
      const uint32_t e0 = same & nibble_zero3(R ^ I);
      const uint32_t e1 = (same & (nibble_zero4(AD ^ 0x99999999u) | nibble_zero4(AD ^ 0x77777777u))) |
                          (~same & nibble_zero4((R + I) ^ 0x11111111u));  // r + i <= 14
      const uint32_t n0 = __builtin_popcount(e0), n1 = __builtin_popcount(e1);
      h0 += n0;
      h1 += n1;
      h2 += 8u - n0 - n1;
    }
    const uint32_t gw = SGN | pick;
    reinterpret_cast<uint32_t*>(guided)[e] = gw;
    if (x_fq) {
      // bf16(RNE32(value * S)) two elements at a time, as in the weight QDQ
      float d[8];
      e2m1_unpack8(gw, d);
      u32x4 fq;
#pragma unroll
      for (int i = 0; i < 4; ++i) fq[i] = pack_bf16x2_rne(d[2 * i] * S, d[2 * i + 1] * S);
      reinterpret_cast<u32x4*>(x_fq)[e] = fq;
    }
    cur = nxt;
  }
  if (hist) {                                // one atomic per bin per workgroup
    __shared__ uint32_t sh[3][kGuidedThreads / 64];
    h0 = wave_sum_u32(h0);
    h1 = wave_sum_u32(h1);
    h2 = wave_sum_u32(h2);
    if ((threadIdx.x & 63) == 0) {
      sh[0][threadIdx.x >> 6] = h0;
      sh[1][threadIdx.x >> 6] = h1;
      sh[2][threadIdx.x >> 6] = h2;
    }
    __syncthreads();
    if (threadIdx.x < 3) {
      unsigned long long t = 0;
      for (int w = 0; w < (int)(blockDim.x >> 6); ++w) t += sh[threadIdx.x][w];
      if (t) atomicAdd(hist + threadIdx.x, t);
    }
  }
}

__global__ void zero_i64_kernel(unsigned long long* p, int n) {
  if ((int)threadIdx.x < n) p[threadIdx.x] = 0ull;
}

constexpr int64_t kGuidedGrid = 512;   // also bounds the histogram's atomics (3 per workgroup)

template <bool RECORD, bool MX = false>
static hipError_t launch_guided_t(const void* x, int dtype, int64_t M, int64_t K, int64_t ldx,
                                  const uint8_t* roll, const uint8_t* roll_scales,
                                  const float* roll_global, uint8_t* guided, __bf16* x_fq,
                                  int64_t* hist, hipStream_t stream) {
  unsigned long long* h = reinterpret_cast<unsigned long long*>(hist);
  if (h) zero_i64_kernel<<<1, 64, 0, stream>>>(h, RECORD ? 2 : 3);
  const int64_t items = M * (K / 8);             // 8-element items, one per lane and trip
  if (items == 0) return hipGetLastError();
  int64_t grid = (items + kGuidedThreads - 1) / kGuidedThreads;
  if (grid > kGuidedGrid) grid = kGuidedGrid;
  if (dtype == 0)
    guided_kernel<__bf16, RECORD, MX><<<(unsigned)grid, kGuidedThreads, 0, stream>>>(
        static_cast<const __bf16*>(x), (uint32_t)M, (uint32_t)K, ldx, roll, roll_scales,
        roll_global, guided, x_fq, h);
  else
    guided_kernel<float, RECORD, MX><<<(unsigned)grid, kGuidedThreads, 0, stream>>>(
        static_cast<const float*>(x), (uint32_t)M, (uint32_t)K, ldx, roll, roll_scales,
        roll_global, guided, x_fq, h);
  return hipGetLastError();
}

hipError_t launch_guided(const void* x, int dtype, int64_t M, int64_t K, int64_t ldx,
                         const uint8_t* roll_codes, const uint8_t* roll_scales,
                         const float* roll_global, uint8_t* guided, __bf16* x_fq,
                         int64_t* hist, hipStream_t stream) {
  return launch_guided_t<false>(x, dtype, M, K, ldx, roll_codes, roll_scales, roll_global, guided,
                                x_fq, hist, stream);
}

hipError_t launch_mx_guided(const void* x, int dtype, int64_t M, int64_t K, int64_t ldx,
                            const uint8_t* roll_codes, const uint8_t* roll_scales, uint8_t* guided,
                            __bf16* x_fq, int64_t* hist, hipStream_t stream) {
  return launch_guided_t<false, true>(x, dtype, M, K, ldx, roll_codes, roll_scales, nullptr,
                                      guided, x_fq, hist, stream);
}

hipError_t launch_mx_guided_record(const void* x, int dtype, int64_t M, int64_t K, int64_t ldx,
                                   const uint8_t* record, const uint8_t* roll_scales,
                                   uint8_t* guided, __bf16* x_fq, int64_t* moved,
                                   hipStream_t stream) {
  return launch_guided_t<true, true>(x, dtype, M, K, ldx, record, roll_scales, nullptr, guided,
                                     x_fq, moved, stream);
}

hipError_t launch_guided_record(const void* x, int dtype, int64_t M, int64_t K, int64_t ldx,
                                const uint8_t* record, const uint8_t* roll_scales,
                                const float* roll_global, uint8_t* guided, __bf16* x_fq,
                                int64_t* moved, hipStream_t stream) {
  return launch_guided_t<true>(x, dtype, M, K, ldx, record, roll_scales, roll_global, guided,
                               x_fq, moved, stream);
}

// ---------------------------------------------------------------------------
// mantissa-only guidance record
// ---------------------------------------------------------------------------
// Thread i turns code bytes [8i, 8i + 8) (16 elements) into record bytes
// [2i, 2i + 2): the low bit of each nibble, gathered by shift-and-mask steps
// (nibble j's bit 4j goes to bit j).
__device__ __forceinline__ uint32_t low_bits8(uint32_t w) {
  uint32_t t = w & 0x11111111u;
  t = (t | (t >> 3)) & 0x03030303u;
  t = (t | (t >> 6)) & 0x000F000Fu;
  return (t | (t >> 12)) & 0xFFu;
}

__global__ __launch_bounds__(256) void guidance_pack_kernel(const uint8_t* __restrict__ codes,
                                                            int64_t n16, uint8_t* __restrict__ record) {
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n16;
       i += (int64_t)gridDim.x * blockDim.x) {
    const u32x2 w = *reinterpret_cast<const u32x2*>(codes + i * 8);
    *reinterpret_cast<uint16_t*>(record + i * 2) = (uint16_t)(low_bits8(w[0]) | (low_bits8(w[1]) << 8));
  }
}

hipError_t launch_guidance_pack(const uint8_t* codes, int64_t M, int64_t K, uint8_t* record,
                                hipStream_t stream) {
  const int64_t n16 = M * (K / kBlock);
  if (n16 == 0) return hipSuccess;
  int64_t grid = (n16 + 255) / 256;
  if (grid > 4096) grid = 4096;
  guidance_pack_kernel<<<(unsigned)grid, 256, 0, stream>>>(codes, n16, record);
  return hipGetLastError();
}

}  // namespace nvfp4
