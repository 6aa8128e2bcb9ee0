// Routed grouped expert GEMM over NVFP4 weights and activations with the
// residual compensation term fused in (QUADS technical summary, section 1:
// native W4A4 GEMM on the rollout; section 2.2B and the yfxerp digest: the
// second FP4 quantization of the high-residual channels is added back into
// the result).
//
//   Y[r, n] = gA gW sum_k (a s_a)[r, k] (w s_w)[n, k]
//           + gR gW sum_j (q s_q)[r, j] (w s_w)[n, sel[j]]
//
// How the NVFP4 scales are applied (gfx950): the per-16 E4M3 block scales are
// folded into the operands while a K-tile is staged: codes are widened to fp32
// by the hardware FP4 convert, multiplied by the block's E4M3 scale (exact:
// at most 2 + 4 significant bits) and stored to LDS as bf16, which holds the
// product exactly.  The MFMA is v_mfma_f32_32x32x16_bf16 with fp32
// accumulation; the two fp32 global scales are applied in the epilogue.  An
// FP8 operand cannot hold e2m1 * e4m3 exactly (6 significant bits), and the
// block-scaled FP4 MFMA takes power-of-two scales per 32 elements, not E4M3
// per 16, so exact NVFP4 runs at the bf16 MFMA rate.
//
// The compensation term is one extra K-chunk: while the main loop streams the
// expert's weight tile through LDS, the columns listed in sel are copied out
// of LDS into a small [BN, kc] buffer, so W is read from memory once.  After
// the main loop the accumulators are rescaled by gA/gR, the chunk
// Q(R_S) x W_S is accumulated, and the epilogue multiplies by gR gW.
//
// Work decomposition: grid.x enumerates (expert, 128-row tile) pairs of the
// ragged groups (upper bound ceil(rows/128) + E, surplus workgroups exit),
// grid.y the N tiles.  Each workgroup (4 waves, 2x2) computes a 128x128 tile;
// each wave a 64x64 tile as 2x2 MFMAs of 32x32.
#include "device_common.h"
#include "kernels.h"

namespace nvfp4 {

constexpr int BM = 128, BN = 128, BK = 64;
constexpr int LDS_STRIDE = BK + 8;          // bf16 elements per LDS row (144 B: conflict-free b128)
constexpr int MAX_KC = 256;                 // largest compensated channel count handled

struct TileLoad {                            // one thread's share of a 128 x 64 NVFP4 tile
  u32x4 codes;                               // 32 E2M1 codes
  uint32_t scales;                           // 2 E4M3 bytes (low 16 bits)
};

// 32 codes (16 bytes) with two block scales -> 32 bf16 written as 4 x 16 B to LDS.
__device__ __forceinline__ void dequant32_to_lds(const TileLoad& t, __bf16* dst) {
  const float s0 = e4m3_value(t.scales & 0xFFu);
  const float s1 = e4m3_value((t.scales >> 8) & 0xFFu);
#pragma unroll
  for (int q = 0; q < 4; ++q) {              // q-th 8 elements (4 bytes of codes)
    const uint32_t w = t.codes[q];
    const float s = q < 2 ? s0 : s1;
    float f[8];
    e2m1_unpack8(w, f);
    u32x4 out;
#pragma unroll
    for (int b = 0; b < 4; ++b) {            // elements 2b, 2b+1 -> one bf16 pair
      const float lo = f[2 * b] * s, hi = f[2 * b + 1] * s;   // exact (<= 6 significant bits)
      out[b] = __builtin_amdgcn_perm(__float_as_uint(hi), __float_as_uint(lo), 0x07060302u);
    }
    *reinterpret_cast<u32x4*>(dst + q * 8) = out;
  }
}

__device__ __forceinline__ float silu_f32(float z) { return z / (1.0f + __expf(-z)); }

__global__ __launch_bounds__(256, 2) void grouped_gemm_kernel(GemmArgs p) {
  __shared__ __attribute__((aligned(16))) __bf16 As[BM * LDS_STRIDE];
  __shared__ __attribute__((aligned(16))) __bf16 Bs[BN * LDS_STRIDE];
  extern __shared__ __attribute__((aligned(16))) unsigned char dyn[];
  __shared__ int32_t sh_e, sh_mt;
  __shared__ uint32_t sh_waves[4];

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;

  // ---- locate (expert, m-tile) of this workgroup --------------------------
  if (tid == 0) sh_e = -1;
  __syncthreads();
  {
    uint32_t carry = 0;
    for (int base = 0; base < p.E; base += blockDim.x) {
      const int e = base + tid;
      int64_t rb = 0, re = 0;
      if (e < p.E) {
        rb = p.group_offsets[e];
        re = p.group_offsets[e + 1];
        rb = rb < 0 ? 0 : (rb > p.rows_total ? p.rows_total : rb);
        re = re < rb ? rb : (re > p.rows_total ? p.rows_total : re);
      }
      const uint32_t n = (uint32_t)((re - rb + BM - 1) / BM);
      // block exclusive scan of n
      uint32_t inc = n;
#pragma unroll
      for (int o = 1; o < 64; o <<= 1) {
        uint32_t t = __shfl_up(inc, o, 64);
        if (lane >= o) inc += t;
      }
      if (lane == 63) sh_waves[wave] = inc;
      __syncthreads();
      uint32_t before = carry, tot = 0;
      for (int w = 0; w < 4; ++w) {
        if (w < wave) before += sh_waves[w];
        tot += sh_waves[w];
      }
      before += inc - n;
      if (e < p.E && blockIdx.x >= before && blockIdx.x < before + n) {
        sh_e = e;
        sh_mt = (int32_t)(blockIdx.x - before);
      }
      carry += tot;
      __syncthreads();
    }
  }
  const int e = sh_e;
  if (e < 0) return;
  int64_t g0 = p.group_offsets[e], g1 = p.group_offsets[e + 1];
  g0 = g0 < 0 ? 0 : (g0 > p.rows_total ? p.rows_total : g0);
  g1 = g1 < g0 ? g0 : (g1 > p.rows_total ? p.rows_total : g1);
  const int64_t row0 = g0 + (int64_t)sh_mt * BM;            // first unit row of the tile
  const int rows_valid = (int)((g1 - row0) < BM ? (g1 - row0) : BM);

  const int64_t K = p.K;
  const int64_t nsteps = K / BK;
  const bool comp = p.sel_idx != nullptr;
  const int kc = comp ? p.kc : 0;
  const int kcp = (kc + BK - 1) / BK * BK;                   // padded to whole K-steps
  const int ws_stride = kcp + 8;
  __bf16* WS = reinterpret_cast<__bf16*>(dyn);               // [BN][ws_stride]
  int32_t* sel = reinterpret_cast<int32_t*>(dyn + (comp ? BN * ws_stride * 2 : 0));   // [kc]
  int32_t* jr = sel + MAX_KC;                                // [nsteps + 1]

  const bool swiglu = p.epilogue == 1;
  const int64_t inter = p.N / 2;

  // W row of LDS row r of this N tile (-1: outside the matrix)
  auto w_row = [&](int r) -> int64_t {
    if (swiglu) {
      const int q = r >> 5;
      const int64_t i = (int64_t)blockIdx.y * 64 + (q >> 1) * 32 + (r & 31);
      if (i >= inter) return -1;
      return (q & 1) ? inter + i : i;
    }
    const int64_t n = (int64_t)blockIdx.y * BN + r;
    return n < p.N ? n : -1;
  };

  // ---- per-thread load assignment: row = tid/2, half = tid%2 (32 elements)
  const int lr = tid >> 1, lh = tid & 1;
  const int64_t a_unit_row = row0 + lr;
  int64_t a_row = -1;
  if (lr < rows_valid) {
    a_row = p.a_row_index ? (int64_t)p.a_row_index[a_unit_row] : a_unit_row;
    if (a_row < 0 || a_row >= p.a_rows) a_row = -1;
  }
  const int64_t b_row = w_row(lr);
  const uint8_t* a_cp = a_row >= 0 ? p.a_codes + a_row * (K / 2) + lh * 16 : nullptr;
  const uint8_t* a_sp = a_row >= 0 ? p.a_scales + a_row * (K / 16) + lh * 2 : nullptr;
  const uint8_t* w_base_c = p.w_codes + (int64_t)e * p.N * (K / 2);
  const uint8_t* w_base_s = p.w_scales + (int64_t)e * p.N * (K / 16);
  const uint8_t* b_cp = b_row >= 0 ? w_base_c + b_row * (K / 2) + lh * 16 : nullptr;
  const uint8_t* b_sp = b_row >= 0 ? w_base_s + b_row * (K / 16) + lh * 2 : nullptr;

  auto load_step = [&](int64_t s, TileLoad& ta, TileLoad& tb) {
    if (a_cp) {
      ta.codes = *reinterpret_cast<const u32x4*>(a_cp + s * (BK / 2));
      ta.scales = *reinterpret_cast<const uint16_t*>(a_sp + s * (BK / 16));
    } else {
      ta.codes = u32x4{0, 0, 0, 0};
      ta.scales = 0;
    }
    if (b_cp) {
      tb.codes = *reinterpret_cast<const u32x4*>(b_cp + s * (BK / 2));
      tb.scales = *reinterpret_cast<const uint16_t*>(b_sp + s * (BK / 16));
    } else {
      tb.codes = u32x4{0, 0, 0, 0};
      tb.scales = 0;
    }
  };

  // ---- compensation set-up: selected channels, their K-step ranges, zero W_S
  if (comp) {
    for (int j = tid; j < kc; j += blockDim.x) {
      int32_t c = p.sel_idx[(int64_t)e * kc + j];
      sel[j] = c < 0 ? 0 : (c >= K ? (int32_t)(K - 1) : c);
    }
    for (int i = tid; i < BN * ws_stride; i += blockDim.x) WS[i] = (__bf16)0.0f;
    __syncthreads();
    for (int64_t s = tid; s <= nsteps; s += blockDim.x) {
      // first j with sel[j] >= s*BK (sel ascending)
      int lo = 0, hi = kc;
      while (lo < hi) {
        int mid = (lo + hi) >> 1;
        if (sel[mid] < s * BK) lo = mid + 1; else hi = mid;
      }
      jr[s] = lo;
    }
  }

  f32x16 acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int q = 0; q < 16; ++q) acc[i][j][q] = 0.0f;

  auto mma_tile = [&](const __bf16* A, const __bf16* B) {
#pragma unroll
    for (int ks = 0; ks < BK / 16; ++ks) {
      bf16x8 af[2], bfr[2];
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        const int ar = wm * 64 + i * 32 + (lane & 31);
        af[i] = *reinterpret_cast<const bf16x8*>(A + ar * LDS_STRIDE + ks * 16 + (lane >> 5) * 8);
      }
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const int br = wn * 64 + j * 32 + (lane & 31);
        bfr[j] = *reinterpret_cast<const bf16x8*>(B + br * LDS_STRIDE + ks * 16 + (lane >> 5) * 8);
      }
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[i], bfr[j], acc[i][j], 0, 0, 0);
    }
  };

  // ---- main K loop ----------------------------------------------------------
  TileLoad ta, tb;
  load_step(0, ta, tb);
  for (int64_t s = 0; s < nsteps; ++s) {
    __syncthreads();                                        // LDS free
    dequant32_to_lds(ta, As + lr * LDS_STRIDE + lh * 32);
    dequant32_to_lds(tb, Bs + lr * LDS_STRIDE + lh * 32);
    __syncthreads();
    if (s + 1 < nsteps) load_step(s + 1, ta, tb);           // prefetch
    if (comp) {                                             // copy W columns of sel
      const int j0 = jr[s], nj = jr[s + 1] - j0;
      for (int i = tid; i < nj * BN; i += blockDim.x) {
        const int n = i & (BN - 1), jj = j0 + (i >> 7);
        WS[n * ws_stride + jj] = Bs[n * LDS_STRIDE + (sel[jj] - (int)(s * BK))];
      }
    }
    mma_tile(As, Bs);
  }

  // ---- compensation chunk ---------------------------------------------------
  float scale = *p.a_global * p.w_global[e];
  if (comp) {
    const float ga = *p.a_global, gr = p.r_global[e];
    const float ratio = ga / gr;
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int q = 0; q < 16; ++q) acc[i][j][q] = acc[i][j][q] * ratio;
    scale = gr * p.w_global[e];
    const int64_t r_unit = row0 + lr;
    for (int c = 0; c < kcp / BK; ++c) {
      __syncthreads();
      // A: Q(R_S) row lr, compact columns c*64 + lh*32 .. +32 (16-element groups)
      TileLoad tr;
      tr.codes = u32x4{0, 0, 0, 0};
      tr.scales = 0;
      if (lr < rows_valid) {
#pragma unroll
        for (int q = 0; q < 2; ++q) {
          const int j = c * BK + lh * 32 + q * 16;
          if (j < kc) {
            const u32x2 w = *reinterpret_cast<const u32x2*>(p.r_codes + r_unit * (kc / 2) + j / 2);
            tr.codes[2 * q] = w[0];
            tr.codes[2 * q + 1] = w[1];
            tr.scales |= (uint32_t)p.r_scales[r_unit * (kc / 16) + j / 16] << (8 * q);
          }
        }
      }
      dequant32_to_lds(tr, As + lr * LDS_STRIDE + lh * 32);
      // B: W_S columns c*64 .. c*64+63 copied into the main B tile layout
      for (int i = tid; i < BN * (BK / 8); i += blockDim.x) {
        const int n = i >> 3, q = i & 7;
        *reinterpret_cast<u32x4*>(Bs + n * LDS_STRIDE + q * 8) =
            *reinterpret_cast<const u32x4*>(WS + n * ws_stride + c * BK + q * 8);
      }
      __syncthreads();
      mma_tile(As, Bs);
    }
  }

  // ---- epilogue -------------------------------------------------------------
  if (p.epilogue == 0 || p.epilogue == 2) {
    float* out = static_cast<float*>(p.out);
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const int64_t n = (int64_t)blockIdx.y * BN + wn * 64 + j * 32 + (lane & 31);
        if (n >= p.N) continue;
#pragma unroll
        for (int q = 0; q < 16; ++q) {
          const int r = wm * 64 + i * 32 + (q >> 2) * 8 + (lane >> 5) * 4 + (q & 3);
          if (r >= rows_valid) continue;
          const int64_t s = row0 + r;
          const float y = acc[i][j][q] * scale;
          if (p.epilogue == 0) {
            out[s * p.ldo + n] = y;
          } else {
            const int64_t t = p.scatter_index[s];
            if (t >= 0 && t < p.out_rows) unsafeAtomicAdd(out + t * p.ldo + n, p.row_weight[s] * y);
          }
        }
      }
  } else {
    // SwiGLU: MFMA column block j=0 holds gate, j=1 up, for the same 32 channels
    __bf16* out = static_cast<__bf16*>(p.out);
    const int64_t i_col = (int64_t)blockIdx.y * 64 + wn * 32 + (lane & 31);
    float m = 0.0f;
    if (i_col < inter) {
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int q = 0; q < 16; ++q) {
          const int r = wm * 64 + i * 32 + (q >> 2) * 8 + (lane >> 5) * 4 + (q & 3);
          if (r >= rows_valid) continue;
          const float gte = acc[i][0][q] * scale, up = acc[i][1][q] * scale;
          const float h = silu_f32(gte) * up;
          const uint32_t hb = f32_to_bf16_rne(h);
          m = fmaxf(m, fabsf(__uint_as_float(hb << 16)));
          reinterpret_cast<uint16_t*>(out)[(row0 + r) * p.ldo + i_col] = (uint16_t)hb;
        }
    }
    if (p.out_amax) {
      m = wave_max(m);
      if (lane == 0) atomic_max_nonneg(p.out_amax, m);
    }
  }
}

hipError_t launch_grouped_gemm(const GemmArgs& a, hipStream_t stream) {
  if (a.epilogue == 1 && a.out_amax) {
    hipError_t err = launch_fill_f32(a.out_amax, 1, 0.0f, stream);
    if (err != hipSuccess) return err;
  }
  if (a.rows_total == 0) return hipSuccess;
  const int64_t mtiles = (a.rows_total + BM - 1) / BM + a.E;
  const int64_t ntiles = a.epilogue == 1 ? (a.N / 2 + 63) / 64 : (a.N + BN - 1) / BN;
  const int kcp = a.sel_idx ? (a.kc + BK - 1) / BK * BK : 0;
  const size_t dyn = (a.sel_idx ? (size_t)BN * (kcp + 8) * 2 : 0) +
                     (size_t)(MAX_KC + a.K / BK + 1) * 4;
  if (dyn > 65536) {
    hipError_t err = hipFuncSetAttribute(reinterpret_cast<const void*>(&grouped_gemm_kernel),
                                         hipFuncAttributeMaxDynamicSharedMemorySize, (int)dyn);
    if (err != hipSuccess) return err;
  }
  dim3 grid((unsigned)mtiles, (unsigned)ntiles);
  grouped_gemm_kernel<<<grid, 256, dyn, stream>>>(a);
  return hipGetLastError();
}

}  // namespace nvfp4
