// Routed grouped expert GEMM over NVFP4 weights and activations with the
// residual compensation term fused in (QUADS technical summary, section 1:
// native W4A4 GEMM on the rollout; section 2.2B and the yfxerp digest: the
// second FP4 quantization of the high-residual channels is added back into
// the result).
//
//   Y[r, n] = gA gW sum_k (a s_a)[r, k] (w s_w)[n, k]
//           + gR gW sum_j (q s_q)[r, j] (w s_w)[n, sel[j]]
//
// How the NVFP4 scales are applied (gfx950).  An element's value is
// e2m1 * e4m3 * g.  e2m1 * e4m3 has at most 6 significant bits: exact in bf16,
// not in FP8 (4 bits), and the block-scaled FP4 MFMA takes one power-of-two
// scale per 32 elements, not an E4M3 per 16.  So the operands stay NVFP4 in
// memory and in LDS, and each wave dequantizes its own MFMA fragments in
// registers right before use: the hardware FP4 -> fp32 convert, one multiply
// by the block's E4M3 scale (exact), one byte permute to bf16.  The MFMA is
// v_mfma_f32_32x32x16_bf16 with fp32 accumulation; the global scales gA gW
// (gR gW) are applied in the epilogue.
//
// K order inside a 32-wide K-step: in both MFMA substeps, lane half h (lanes
// 32h .. 32h+31) supplies the 16 consecutive k of NVFP4 block h of the step
// (first 8 in substep 0, last 8 in substep 1), so one 8-byte LDS read and one
// scale byte give a lane a whole block.  A and B use the same order, so the
// sum over the step's 32 k is unchanged.
//
// Pipeline: LDS holds three stages of raw codes + scales (9 KB per stage for a
// 256 x 256 tile); global loads run two steps ahead in a double register set;
// one barrier per step.
//
// The compensation term is an extra chunk of kc: while the main loop streams
// the expert's weight tile through LDS, the elements of the selected columns
// are dequantized into a bf16 [BN, kc] buffer, so W is read from memory once.
// After the main loop the accumulators are rescaled by gA/gR, Q(R_S) x W_S is
// accumulated, and the epilogue multiplies by gR gW.
//
// Scatter epilogue: row_weight * Y rows are stored (plain, coalesced) into the
// workspace and combine.hip adds them into the output rows in a fixed order.
//
// Work decomposition: the logical tiles are the (expert, n-tile, m-tile)
// triples of the ragged groups, expert-major, then n-tile, m-tile innermost
// (upper bound (ceil(rows/BM) + E) x n-tiles; surplus workgroups exit).
// Workgroup ids are dealt round-robin to the 8 XCDs, so hardware id h runs
// logical tile (h % 8) * ceil(total / 8) + h / 8: each XCD owns a contiguous
// range of experts; the m-tiles that share one weight tile run side by side
// on it (the weight tile is read once), and the expert's activation rows stay
// in its L2 across the n-tiles.  Four waves per workgroup; each wave owns
// MI x NJ MFMA blocks of 32 x 32.
#include "device_common.h"
#include "kernels.h"

namespace nvfp4 {

constexpr int BN = 256, BK = 32;
constexpr int NSTAGE = 3;                   // LDS stages of raw NVFP4 tiles
constexpr int MAX_KC = 128;                 // largest compensated channel count handled

struct RowLoad {                            // one row's K-step: 32 codes + 2 scale bytes
  u32x4 codes;
  uint32_t scales;
};

// Two bf16x8 fragments (substeps 0 and 1) from 16 codes (8 bytes) and a scale.
__device__ __forceinline__ void dequant16(u32x2 c, float s, bf16x8& f0, bf16x8& f1) {
  float f[16];
  e2m1_unpack8(c[0], f);
  e2m1_unpack8(c[1], f + 8);
  u32x4 o0, o1;
#pragma unroll
  for (int b = 0; b < 4; ++b) {
    o0[b] = __builtin_amdgcn_perm(__float_as_uint(f[2 * b + 1] * s), __float_as_uint(f[2 * b] * s),
                                  0x07060302u);
    o1[b] = __builtin_amdgcn_perm(__float_as_uint(f[8 + 2 * b + 1] * s),
                                  __float_as_uint(f[8 + 2 * b] * s), 0x07060302u);
  }
  f0 = __builtin_bit_cast(bf16x8, o0);
  f1 = __builtin_bit_cast(bf16x8, o1);
}

__device__ __forceinline__ float silu_f32(float z) { return z / (1.0f + __expf(-z)); }

__device__ __forceinline__ int64_t clamp64(int64_t v, int64_t lo, int64_t hi) {
  return v < lo ? lo : (v > hi ? hi : v);
}

template <int MI, int NJ, int WM, int WN>
__global__ __launch_bounds__(256, 1) void grouped_gemm_kernel(GemmArgs p, int ntiles, int total) {
  constexpr int BM = WM * MI * 32;
  static_assert(WN * NJ * 32 == BN, "N tile");
  static_assert(WM * WN == 4, "four waves");
  // LDS: NSTAGE x {A codes [BM][16 B], A scales [BM][2 B], B codes [BN][16 B],
  // B scales [BN][2 B]}, then the bf16 W_S buffer, the selected channels and
  // their K-step ranges.
  constexpr int A_CODES = 0, A_SC = BM * 16, B_CODES = A_SC + BM * 2, B_SC = B_CODES + BN * 16;
  constexpr int STAGE = B_SC + BN * 2;
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  __bf16* WS = reinterpret_cast<__bf16*>(smem + NSTAGE * STAGE);    // [BN][ws_stride]
  __shared__ int32_t sh_e, sh_mt, sh_nt;
  __shared__ uint32_t sh_waves[4];

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int wm = wave / WN, wn = wave % WN;
  const int half = lane >> 5, l32 = lane & 31;

  // ---- logical tile of this workgroup (XCD-contiguous ranges) --------------
  // Logical tiles are ordered expert by expert; inside an expert's block of
  // cnt_e * ntiles tiles, n-tile major and m-tile minor, so the m-tiles that
  // share a weight tile run together on one XCD.  Expert e's block starts at
  // tile_start_e * ntiles, where tile_start_e counts the m-tiles of experts < e.
  const int per_xcd = (total + 7) / 8;
  const int logical = (int)(blockIdx.x % 8) * per_xcd + (int)(blockIdx.x / 8);
  if (logical >= total) return;
  const int m_key = logical / ntiles;        // lies inside expert e's m-tile range

  if (tid == 0) sh_e = -1;
  __syncthreads();
  {
    uint32_t carry = 0;
    for (int base = 0; base < p.E; base += 256) {
      const int e = base + tid;
      int64_t rb = 0, re = 0;
      if (e < p.E) {
        rb = clamp64(p.group_offsets[e], 0, p.rows_total);
        re = clamp64(p.group_offsets[e + 1], rb, p.rows_total);
      }
      const uint32_t n = (uint32_t)((re - rb + BM - 1) / BM);
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
      if (e < p.E && (uint32_t)m_key >= before && (uint32_t)m_key < before + n) {
        const int off = logical - (int)before * ntiles;   // position inside the expert's block
        sh_e = e;
        sh_nt = off / (int)n;
        sh_mt = off % (int)n;
      }
      carry += tot;
      __syncthreads();
    }
  }
  const int e = sh_e;
  if (e < 0) return;
  const int n_tile = sh_nt;
  const int64_t g0 = clamp64(p.group_offsets[e], 0, p.rows_total);
  const int64_t g1 = clamp64(p.group_offsets[e + 1], g0, p.rows_total);
  const int64_t row0 = g0 + (int64_t)sh_mt * BM;            // first unit row of the tile
  const int rows_valid = (int)((g1 - row0) < BM ? (g1 - row0) : BM);

  const int64_t K = p.K;
  const int nsteps = (int)(K / BK);
  const bool comp = p.sel_idx != nullptr;
  const int kc = comp ? p.kc : 0;
  const int kcp = (kc + BK - 1) / BK * BK;                   // padded to whole K-steps
  const int ws_stride = kcp + 8;
  int32_t* sel = reinterpret_cast<int32_t*>(WS + (comp ? BN * ws_stride : 0));   // [MAX_KC]
  int32_t* jr = sel + MAX_KC;                                                   // [nsteps + 1]

  const bool swiglu = p.epilogue == 1;
  const int64_t inter = p.N / 2;

  // ---- this thread's rows: A row tid (if < BM), W row tid ------------------
  // Loads are branch-free: a row outside the tile reads row 0 of its operand
  // (always valid) and is zeroed by a select, so the compiler can count the
  // loads in flight and keep the prefetch of later K-steps outstanding.
  bool a_ok = false;
  int64_t ar = 0;
  if (tid < rows_valid) {
    const int64_t ur = row0 + tid;
    ar = p.a_row_index ? (int64_t)p.a_row_index[ur] : ur;
    a_ok = ar >= 0 && ar < p.a_rows;
    if (!a_ok) ar = 0;
  }
  const uint8_t* a_cp = p.a_codes + ar * (K / 2);
  const uint8_t* a_sp = p.a_scales + ar * (K / 16);
  int64_t b_row;
  if (swiglu) {                               // LDS row r: 32-row groups alternate gate / up
    const int q = tid >> 5;
    const int64_t i = (int64_t)n_tile * (BN / 2) + (q >> 1) * 32 + (tid & 31);
    b_row = i < inter ? ((q & 1) ? inter + i : i) : -1;
  } else {
    const int64_t n = (int64_t)n_tile * BN + tid;
    b_row = n < p.N ? n : -1;
  }
  const bool b_ok = b_row >= 0;
  const uint8_t* b_cp = p.w_codes + ((int64_t)e * p.N + (b_ok ? b_row : 0)) * (K / 2);
  const uint8_t* b_sp = p.w_scales + ((int64_t)e * p.N + (b_ok ? b_row : 0)) * (K / 16);
  const uint32_t a_mask = a_ok ? 0xFFFFFFFFu : 0u, b_mask = b_ok ? 0xFFFFFFFFu : 0u;

  auto load_step = [&](int s, RowLoad& ta, RowLoad& tb) {
    ta.codes = *reinterpret_cast<const u32x4*>(a_cp + s * (BK / 2));   // masked when staged
    ta.scales = *reinterpret_cast<const uint16_t*>(a_sp + s * (BK / 16));
    tb.codes = *reinterpret_cast<const u32x4*>(b_cp + s * (BK / 2));
    tb.scales = *reinterpret_cast<const uint16_t*>(b_sp + s * (BK / 16));
  };

  auto stage_write = [&](int st, const RowLoad& ta, const RowLoad& tb) {
    unsigned char* base = smem + st * STAGE;
    if (tid < BM) {
      *reinterpret_cast<u32x4*>(base + A_CODES + tid * 16) = ta.codes & a_mask;
      *reinterpret_cast<uint16_t*>(base + A_SC + tid * 2) = (uint16_t)ta.scales;
    }
    *reinterpret_cast<u32x4*>(base + B_CODES + tid * 16) = tb.codes & b_mask;
    *reinterpret_cast<uint16_t*>(base + B_SC + tid * 2) = (uint16_t)tb.scales;
  };

  // ---- compensation set-up: selected channels, their K-step ranges, zero W_S
  if (comp) {
    for (int j = tid; j < kc; j += 256) {
      int32_t c = p.sel_idx[(int64_t)e * kc + j];
      sel[j] = c < 0 ? 0 : (c >= K ? (int32_t)(K - 1) : c);
    }
    for (int i = tid; i < BN * ws_stride / 8; i += 256)
      reinterpret_cast<u32x4*>(WS)[i] = u32x4{0, 0, 0, 0};
    __syncthreads();
    for (int s = tid; s <= nsteps; s += 256) {
      int lo = 0, hi = kc;                    // first j with sel[j] >= s * BK
      while (lo < hi) {
        int mid = (lo + hi) >> 1;
        if (sel[mid] < s * BK) lo = mid + 1; else hi = mid;
      }
      jr[s] = lo;
    }
  }

  f32x16 acc[MI][NJ];
#pragma unroll
  for (int i = 0; i < MI; ++i)
#pragma unroll
    for (int j = 0; j < NJ; ++j)
#pragma unroll
      for (int q = 0; q < 16; ++q) acc[i][j][q] = 0.0f;

  // One K-step from LDS stage st: each lane dequantizes its 16-element block of
  // every fragment, then both substeps of MFMAs run.
  auto compute_step = [&](int st) {
    const unsigned char* base = smem + st * STAGE;
    bf16x8 a0[MI], a1[MI];
#pragma unroll
    for (int i = 0; i < MI; ++i) {
      const int r = wm * MI * 32 + i * 32 + l32;
      const u32x2 c = *reinterpret_cast<const u32x2*>(base + A_CODES + r * 16 + half * 8);
      const float s = e4m3_value(base[A_SC + r * 2 + half]);
      dequant16(c, s, a0[i], a1[i]);
    }
#pragma unroll
    for (int j = 0; j < NJ; ++j) {            // one B fragment pair live at a time
      const int r = wn * NJ * 32 + j * 32 + l32;
      const u32x2 c = *reinterpret_cast<const u32x2*>(base + B_CODES + r * 16 + half * 8);
      const float s = e4m3_value(base[B_SC + r * 2 + half]);
      bf16x8 b0, b1;
      dequant16(c, s, b0, b1);
#pragma unroll
      for (int i = 0; i < MI; ++i)
        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a0[i], b0, acc[i][j], 0, 0, 0);
#pragma unroll
      for (int i = 0; i < MI; ++i)
        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a1[i], b1, acc[i][j], 0, 0, 0);
    }
  };

  // W columns of sel inside K-step s, from LDS stage st, dequantized into W_S.
  auto gather_ws = [&](int s, int st) {
    const unsigned char* base = smem + st * STAGE;
    const int j0 = jr[s], nj = jr[s + 1] - j0;
    for (int i = tid; i < nj * BN; i += 256) {
      const int n = i & (BN - 1), jj = j0 + (i >> 8);
      const int kk = sel[jj] - s * BK;                       // 0..31 inside the step
      const uint32_t code = (base[B_CODES + n * 16 + (kk >> 1)] >> (4 * (kk & 1))) & 15u;
      const float v = e2m1_value(code) * e4m3_value(base[B_SC + n * 2 + (kk >> 4)]);
      reinterpret_cast<uint16_t*>(WS)[n * ws_stride + jj] = (uint16_t)(__float_as_uint(v) >> 16);
    }
  };

  // ---- main K loop: stage s%3 is read, stage (s+2)%3 written, loads 2 ahead --
  // Every load is issued unconditionally (a step past the end re-reads the last
  // step, and its stage is never read): with no path that skips a load, the
  // compiler waits only for the older step's loads (vmcnt = 4), not for all.
  // K is a multiple of 64, so nsteps is even and at least 2.
  RowLoad ra[2], rb[2];
  const int last = nsteps - 1;
  load_step(0, ra[0], rb[0]);
  load_step(1, ra[1], rb[1]);
  stage_write(0, ra[0], rb[0]);
  stage_write(1, ra[1], rb[1]);
  load_step(2 < last ? 2 : last, ra[0], rb[0]);
  __builtin_amdgcn_sched_barrier(0);          // keep the loop's load order in the prologue
  load_step(3 < last ? 3 : last, ra[1], rb[1]);
  lds_barrier();
  auto step = [&](int s, RowLoad& ta, RowLoad& tb) {
    const int st = s % NSTAGE;
    compute_step(st);
    stage_write((s + 2) % NSTAGE, ta, tb);                    // data of step s+2
    load_step(s + 4 < last ? s + 4 : last, ta, tb);
    if (comp) gather_ws(s, st);
    lds_barrier();
  };
  int s = 0;
  for (; s + 1 < nsteps; s += 2) {
    step(s, ra[0], rb[0]);
    step(s + 1, ra[1], rb[1]);
  }
  if (s < nsteps) step(s, ra[0], rb[0]);

  // ---- compensation chunk ---------------------------------------------------
  float scale = *p.a_global * p.w_global[e];
  if (comp) {
    const float ga = *p.a_global, gr = p.r_global[e];
    const float ratio = ga / gr;
#pragma unroll
    for (int i = 0; i < MI; ++i)
#pragma unroll
      for (int j = 0; j < NJ; ++j)
#pragma unroll
        for (int q = 0; q < 16; ++q) acc[i][j][q] = acc[i][j][q] * ratio;
    scale = gr * p.w_global[e];
    for (int c = 0; c < kcp / BK; ++c) {
      unsigned char* base = smem + (c & 1) * STAGE;
      if (tid < BM) {                            // Q(R_S) row tid, compact columns c*32 ..
        u32x4 codes = u32x4{0, 0, 0, 0};
        uint32_t sc = 0;
        if (tid < rows_valid) {
          const int64_t ur = row0 + tid;
#pragma unroll
          for (int q = 0; q < 2; ++q) {
            const int j = c * BK + q * 16;
            if (j < kc) {
              const u32x2 w = *reinterpret_cast<const u32x2*>(p.r_codes + ur * (kc / 2) + j / 2);
              codes[2 * q] = w[0];
              codes[2 * q + 1] = w[1];
              sc |= (uint32_t)p.r_scales[ur * (kc / 16) + j / 16] << (8 * q);
            }
          }
        }
        *reinterpret_cast<u32x4*>(base + A_CODES + tid * 16) = codes;
        *reinterpret_cast<uint16_t*>(base + A_SC + tid * 2) = (uint16_t)sc;
      }
      lds_barrier();
      bf16x8 a0[MI], a1[MI], b0[NJ], b1[NJ];
#pragma unroll
      for (int i = 0; i < MI; ++i) {
        const int r = wm * MI * 32 + i * 32 + l32;
        const u32x2 cc = *reinterpret_cast<const u32x2*>(base + A_CODES + r * 16 + half * 8);
        dequant16(cc, e4m3_value(base[A_SC + r * 2 + half]), a0[i], a1[i]);
      }
#pragma unroll
      for (int j = 0; j < NJ; ++j) {            // W_S in the same K order: block half of the chunk
        const int r = wn * NJ * 32 + j * 32 + l32;
        b0[j] = *reinterpret_cast<const bf16x8*>(WS + r * ws_stride + c * BK + half * 16);
        b1[j] = *reinterpret_cast<const bf16x8*>(WS + r * ws_stride + c * BK + half * 16 + 8);
      }
#pragma unroll
      for (int i = 0; i < MI; ++i)
#pragma unroll
        for (int j = 0; j < NJ; ++j) {
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a0[i], b0[j], acc[i][j], 0, 0, 0);
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a1[i], b1[j], acc[i][j], 0, 0, 0);
        }
    }
  }

  // ---- epilogue -------------------------------------------------------------
  if (p.epilogue == 0 || p.epilogue == 2) {
    float* out = static_cast<float*>(p.out);
#pragma unroll
    for (int i = 0; i < MI; ++i)
#pragma unroll
      for (int j = 0; j < NJ; ++j) {
        const int64_t n = (int64_t)n_tile * BN + wn * NJ * 32 + j * 32 + l32;
        if (n >= p.N) continue;
#pragma unroll
        for (int q = 0; q < 16; ++q) {
          const int r = wm * MI * 32 + i * 32 + (q >> 2) * 8 + half * 4 + (q & 3);
          if (r >= rows_valid) continue;
          const int64_t s2 = row0 + r;
          const float y = acc[i][j][q] * scale;
          if (p.epilogue == 0) out[s2 * p.ldo + n] = y;
          else p.y_rows[s2 * p.N + n] = p.row_weight[s2] * y;   // added into out by the combine
        }
      }
  } else {
    // SwiGLU: block j (even) is gate, j+1 is up, for the same 32 channels
    uint16_t* out = static_cast<uint16_t*>(p.out);
    float m = 0.0f;
#pragma unroll
    for (int j = 0; j < NJ; j += 2) {
      const int64_t ch = (int64_t)n_tile * (BN / 2) + wn * (NJ / 2) * 32 + (j / 2) * 32 + l32;
      if (ch >= inter) continue;
#pragma unroll
      for (int i = 0; i < MI; ++i)
#pragma unroll
        for (int q = 0; q < 16; ++q) {
          const int r = wm * MI * 32 + i * 32 + (q >> 2) * 8 + half * 4 + (q & 3);
          if (r >= rows_valid) continue;
          const float gte = acc[i][j][q] * scale, up = acc[i][j + 1][q] * scale;
          const uint32_t hb = f32_to_bf16_rne(silu_f32(gte) * up);
          m = fmaxf(m, fabsf(__uint_as_float(hb << 16)));
          out[(row0 + r) * p.ldo + ch] = (uint16_t)hb;
        }
    }
    if (p.out_amax) {
      m = wave_max(m);
      if (lane == 0) atomic_max_nonneg(p.out_amax, m);
    }
  }
}

template <int MI, int NJ, int WM, int WN>
static hipError_t launch_cfg(const GemmArgs& a, hipStream_t stream) {
  constexpr int BM = WM * MI * 32;
  const int64_t mtiles = (a.rows_total + BM - 1) / BM + a.E;
  const int64_t ntiles = a.epilogue == 1 ? (a.N / 2 + BN / 2 - 1) / (BN / 2) : (a.N + BN - 1) / BN;
  const int64_t total = mtiles * ntiles;
  const int kcp = a.sel_idx ? (a.kc + BK - 1) / BK * BK : 0;
  const size_t stage = (size_t)BM * 18 + (size_t)BN * 18;
  const size_t lds = NSTAGE * stage + (a.sel_idx ? (size_t)BN * (kcp + 8) * 2 : 0) +
                     (size_t)(MAX_KC + a.K / BK + 1) * 4;
  auto kern = grouped_gemm_kernel<MI, NJ, WM, WN>;
  hipError_t err = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
  if (err != hipSuccess) return err;
  const int64_t grid = (total + 7) / 8 * 8;
  kern<<<(unsigned)grid, 256, lds, stream>>>(a, (int)ntiles, (int)total);
  return hipGetLastError();
}

int grouped_gemm_block_m(int64_t rows_total, int32_t E) {
  const int64_t avg = E > 0 ? rows_total / E : rows_total;
  if (avg >= 512) return 256;
  if (avg >= 128) return 128;
  if (avg >= 48) return 64;
  return 32;
}

hipError_t launch_grouped_gemm(const GemmArgs& a, hipStream_t stream) {
  if (a.epilogue == 1 && a.out_amax) {
    hipError_t err = launch_fill_f32(a.out_amax, 1, 0.0f, stream);
    if (err != hipSuccess) return err;
  }
  if (a.rows_total == 0) return hipSuccess;
  hipError_t err;
  switch (a.block_m > 0 ? a.block_m : grouped_gemm_block_m(a.rows_total, a.E)) {
    case 256: err = launch_cfg<4, 4, 2, 2>(a, stream); break;
    case 128: err = launch_cfg<2, 4, 2, 2>(a, stream); break;
    case 64: err = launch_cfg<1, 4, 2, 2>(a, stream); break;
    default: err = launch_cfg<1, 2, 1, 4>(a, stream); break;
  }
  if (err != hipSuccess || a.epilogue != 2) return err;
  return launch_combine(a.y_rows, a.rows_total, a.N, a.scatter_index, a.out_rows,
                        static_cast<float*>(a.out), a.ldo, a.y_rows, stream);
}

}  // namespace nvfp4
