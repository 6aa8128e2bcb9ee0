// MXFP4 variant of the rollout path: the same online activation quantization
// and compensated grouped expert GEMM with 32-element blocks and E8M0
// power-of-two block scales instead of NVFP4's E4M3 per-16 scales under a
// global scale (the TRACE summary validates its method in both FP4 formats:
// the novelty and results paragraphs and Table 4).
//
// Format (OCP MX, the reading of the name "MXFP4"): X = floor(log2 amax_b) - 2
// clamped to [-127, 127] (-127 for an all-zero block), byte X + 127; element
// = nearest-even E2M1 index of |x| / 2^X, saturating at 6, sign of x.
//
// The GEMM is where the format pays off on gfx950: v_mfma_scale_f32_32x32x64_
// f8f6f4 consumes E2M1 codes and one E8M0 scale per lane and 32 K-values --
// exactly an MX block -- so the operands go from HBM through LDS into the
// matrix cores as raw codes, with no dequantization.  Lane l of a 32 x 32 x 64
// MFMA supplies row (A) or column (B) l % 32 and the 32 consecutive K-values
// 32 (l / 32) ..; a 32-bit scale operand and op_sel pick its scale byte; the
// 32 x 32 fp32 result sits in lane l, element q at row (q / 4) * 8 +
// (l / 32) * 4 + q % 4, column l % 32 (the layout of the fp16 MFMA the shared
// epilogues assume).
#include "gemm_common.h"

namespace nvfp4 {

// ---------------------------------------------------------------------------
// quantizer (+ optional residual-score tile partials)
// ---------------------------------------------------------------------------
// One workgroup (256 threads) owns 128 rows x 64 columns; thread t quantizes
// the 32-block t % 2 of row t / 2 (all its loads first).  Tiles are dealt to
// the XCDs in contiguous eighths as in the NVFP4 quantizer.  With SCORES the
// thread writes |x - DQ| of its block into LDS and threads 0..63 each add one
// column over the tile's 128 rows in increasing row order (rows past the
// tensor add +0).
constexpr int kMxTileCols = 64;
constexpr int kMxAbsStride = kMxTileCols + 4;

template <typename T>
__device__ __forceinline__ void mx_load32(const T* p, float* v) {
  if constexpr (sizeof(T) == 2) {
    const u32x4* q = reinterpret_cast<const u32x4*>(p);
    u32x4 w[4];
#pragma unroll
    for (int c = 0; c < 4; ++c) w[c] = q[c];
#pragma unroll
    for (int c = 0; c < 4; ++c)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        v[8 * c + 2 * i] = bf16_lo(w[c][i]);
        v[8 * c + 2 * i + 1] = bf16_hi(w[c][i]);
      }
  } else {
    const f32x4* q = reinterpret_cast<const f32x4*>(p);
    f32x4 w[8];
#pragma unroll
    for (int c = 0; c < 8; ++c) w[c] = q[c];
#pragma unroll
    for (int c = 0; c < 8; ++c)
#pragma unroll
      for (int i = 0; i < 4; ++i) v[4 * c + i] = w[c][i];
  }
}

template <typename T, bool SCORES>
__global__ __launch_bounds__(256) void mx_quantize_tile_kernel(
    const T* __restrict__ x, int64_t M, int64_t K, int64_t ldx, uint8_t* __restrict__ codes,
    uint8_t* __restrict__ scales, float* __restrict__ tile_partials) {
  __shared__ float absr[SCORES ? kScoreTileRows * kMxAbsStride : 1];
  const int tid = threadIdx.x;
  const int64_t nb = K / kMxBlock;
  const int64_t tiles_x = (K + kMxTileCols - 1) / kMxTileCols;
  const int64_t ntiles = tiles_x * ((M + kScoreTileRows - 1) / kScoreTileRows);
  const int64_t per_xcd = (ntiles + 7) / 8;
  const int64_t tile = (int64_t)(blockIdx.x % 8) * per_xcd + blockIdx.x / 8;
  if ((int64_t)(blockIdx.x / 8) >= per_xcd || tile >= ntiles) return;   // uniform
  const int64_t tx = tile % tiles_x, ty = tile / tiles_x;
  const int bl = tid & 1, rl = tid >> 1;
  const int64_t bc = tx * 2 + bl;
  const int64_t r = ty * kScoreTileRows + rl;
  const bool live = r < M && bc < nb;
  float v[32];
  if (live) mx_load32<T>(x + r * ldx + bc * kMxBlock, v);
  float res[32];
  if (live) {
    float amax = 0.0f;
#pragma unroll
    for (int i = 0; i < 32; ++i) amax = fmaxf(amax, fabsf(v[i]));
    const uint32_t sb = mx_scale_byte(amax);
    uint32_t w[4];
    mx_pack32(v, sb, w);
    *reinterpret_cast<u32x4*>(codes + r * (K / 2) + bc * 16) = u32x4{w[0], w[1], w[2], w[3]};
    scales[r * nb + bc] = (uint8_t)sb;
    if constexpr (SCORES) {
      const float S = e8m0_value(sb);
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        float f[8];
        e2m1_unpack8(w[q], f);
#pragma unroll
        for (int i = 0; i < 8; ++i) res[8 * q + i] = fabsf(v[8 * q + i] - f[i] * S);   // exact
      }
    }
  } else if constexpr (SCORES) {
#pragma unroll
    for (int i = 0; i < 32; ++i) res[i] = 0.0f;
  }
  if constexpr (SCORES) {
    f32x4* dst = reinterpret_cast<f32x4*>(absr + rl * kMxAbsStride + bl * kMxBlock);
#pragma unroll
    for (int i = 0; i < 8; ++i) dst[i] = f32x4{res[4 * i], res[4 * i + 1], res[4 * i + 2], res[4 * i + 3]};
    __syncthreads();
    const int64_t c = tx * kMxTileCols + tid;
    if (tid < kMxTileCols && c < K) {
      float sum = 0.0f;
#pragma unroll 16
      for (int q = 0; q < kScoreTileRows; ++q) sum = sum + absr[q * kMxAbsStride + tid];
      tile_partials[ty * K + c] = sum;
    }
  }
}

template <typename T>
static hipError_t launch_mx_quantize_t(const T* x, int64_t M, int64_t K, int64_t ldx,
                                       uint8_t* codes, uint8_t* scales, float* tile_partials,
                                       hipStream_t stream) {
  const int64_t ntiles = ((K + kMxTileCols - 1) / kMxTileCols) * ((M + kScoreTileRows - 1) / kScoreTileRows);
  const unsigned grid = (unsigned)(ntiles > 0 ? (ntiles + 7) / 8 * 8 : 8);
  if (tile_partials)
    mx_quantize_tile_kernel<T, true><<<grid, 256, 0, stream>>>(x, M, K, ldx, codes, scales, tile_partials);
  else
    mx_quantize_tile_kernel<T, false><<<grid, 256, 0, stream>>>(x, M, K, ldx, codes, scales, nullptr);
  return hipGetLastError();
}

hipError_t launch_mx_quantize(const void* x, int dtype, int64_t M, int64_t K, int64_t ldx,
                              uint8_t* codes, uint8_t* scales, float* tile_partials,
                              hipStream_t stream) {
  if (M == 0) return hipSuccess;
  if (dtype == 0)
    return launch_mx_quantize_t(static_cast<const __bf16*>(x), M, K, ldx, codes, scales,
                                tile_partials, stream);
  return launch_mx_quantize_t(static_cast<const float*>(x), M, K, ldx, codes, scales,
                              tile_partials, stream);
}

// ---------------------------------------------------------------------------
// grouped GEMM
// ---------------------------------------------------------------------------
//   Y[r, n] = sum_k (a 2^Xa)[r, k] (w 2^Xw)[n, k] + sum_j (q 2^Xq)[r, j] (w 2^Xw)[n, sel[j]]
//
// Tiles: BM (256/128/64/32) rows x 256 weight rows, four waves each owning
// MI x NJ blocks of 32 x 32; the (expert, m-tile, n-tile) decomposition, the
// XCD-aware tile order and the epilogues are the NVFP4 GEMM's
// (gemm_common.h).  K moves 128 per pipeline stage: an LDS row is 64 code
// bytes, the 4 scale bytes of the stage's blocks and 12 bytes of padding
// (an 80-byte stride keeps the 16-byte fragment reads of 8 consecutive rows
// on distinct banks).  Thread t loads 16-byte chunk t % 4 of rows t / 4 + 64 i
// of both operands and the scale word of row t.  Two LDS stages and two
// register sets: in stage m a wave reads its fragments of stage m, writes
// the data of stage m + 1 into the other LDS stage and issues the loads of
// stage m + 3, then runs its 2 MI NJ MFMAs; one barrier per stage.
//
// Compensation.  A lane of the MFMA applies one scale to its 32 K-values,
// but the selected channels W[n, sel[j]] keep the scales of the blocks they
// come from.  So W_S is re-expressed in FP8 E4M3 against one scale per
// weight row, the row's largest block scale 2^Xmax: element
// e2m1 * 2^(X - Xmax) is exact in E4M3 when X - Xmax >= -8 (its smallest
// part, 0.5 * 2^-8, is E4M3's smallest subnormal) and is rounded to nearest
// E4M3 otherwise (weights whose blocks span more than 8 binades in one row).
// The W_S bytes are picked from the LDS stages during the main loop (thread t
// handles weight row t), so W is read once.  Q(R_S) is read from memory after
// the loop and widened to E4M3 the same way against the larger scale of a
// row's two blocks in a 64-wide K-step (exact when the two differ by at most
// 8 binades), and the correction runs on the FP8 form of the same scaled
// MFMA.  Its scales are then uniform over each row of A and each column of B,
// so the result does not depend on how the FP8 form pairs lanes with scales.
namespace mxg {

constexpr int BN = 256;
constexpr int KS = 128;                    // K per pipeline stage
constexpr int ROW = 80;                    // LDS bytes per row
constexpr int MAX_KC = 128;

// Bytes per W_S row in LDS for kc compensated channels: one byte per channel
// of the padded width plus 16 of padding (0 without compensation).
__host__ __device__ constexpr int ws_stride(int kc) {
  return kc > 0 ? (kc + 63) / 64 * 64 + 16 : 0;
}

template <int BM>
struct Layout {
  static constexpr int AR = BM + 1;                  // row BM: spare for threads past the tile
  static constexpr int NA = BM < 64 ? 1 : BM / 64;   // A chunk loads per thread
  static constexpr int STAGE = (AR + BN) * ROW;
  static constexpr int B_OFF = AR * ROW;
};

typedef int v8i __attribute__((ext_vector_type(8)));

__device__ __forceinline__ v8i as_v8i(const u32x4& w) {
  return v8i{(int)w[0], (int)w[1], (int)w[2], (int)w[3], 0, 0, 0, 0};
}

// E4M3 bytes of the 8 E2M1 codes of w times the power of two f (exact when
// the products stay at or above 2^-9, E4M3's smallest subnormal).
__device__ __forceinline__ u32x2 e2m1x8_to_e4m3(uint32_t w, float f) {
  const f32x2 a = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, 0) * f;
  const f32x2 b = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, 1) * f;
  const f32x2 c = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, 2) * f;
  const f32x2 d = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, 3) * f;
  int lo = __builtin_amdgcn_cvt_pk_fp8_f32(a[0], a[1], 0, false);
  lo = __builtin_amdgcn_cvt_pk_fp8_f32(b[0], b[1], lo, true);
  int hi = __builtin_amdgcn_cvt_pk_fp8_f32(c[0], c[1], 0, false);
  hi = __builtin_amdgcn_cvt_pk_fp8_f32(d[0], d[1], hi, true);
  return u32x2{(uint32_t)lo, (uint32_t)hi};
}

// 2^d for d <= 0 (0 below 2^-126, where every E4M3 rounding gives 0 anyway).
__device__ __forceinline__ float pow2_nonpos(int d) {
  return d >= -126 ? __uint_as_float((uint32_t)(127 + d) << 23) : 0.0f;
}

template <int MI, int NJ, int WM, int WN, int EPI>
__global__ __launch_bounds__(256, 1) void mx_grouped_gemm_kernel(GemmArgs p, int ntiles) {
  constexpr int BM = WM * MI * 32;
  static_assert(WN * NJ * 32 == BN, "N tile");
  static_assert(WM * WN == 4, "four waves");
  using L = Layout<BM>;
  constexpr int STAGE = L::STAGE, B_OFF = L::B_OFF, NA = L::NA;
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  // LDS: 2 stages | W_S [BN][wss] bytes | Xmax bytes [BN] | sel [MAX_KC] |
  // gather table [nst] (u32x2 per stage).  W_S row t holds, for each selected
  // channel j, code | min(xmax - scale byte, 15) << 4 during the K loop, and
  // the E4M3 byte of W[t, sel[j]] / 2^(xmax - 127) after it (convert_ws).
  const int wss = ws_stride(p.sel_idx ? p.kc : 0);
  unsigned char* WS = smem + 2 * STAGE;
  unsigned char* WX = WS + BN * wss;
  int32_t* sel = reinterpret_cast<int32_t*>(WX + BN);
  u32x2* tab = reinterpret_cast<u32x2*>(sel + MAX_KC);

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int wm = wave / WN, wn = wave % WN;
  const int half = lane >> 5, l32 = lane & 31;

  const int real = (int)count_mtiles<BM>(p) * ntiles;
  const int per_xcd = (real + 7) / 8;
  const int jt = (int)blockIdx.x / 8;
  const int logical = ((int)blockIdx.x % 8) * per_xcd + jt;
  if (jt >= per_xcd || logical >= real) return;     // uniform over the workgroup
  const TileCoord tc = locate_tile<BM>(p, ntiles, logical);
  const int e = tc.e, n_tile = tc.n_tile, rows_valid = tc.rows_valid;
  const int64_t row0 = tc.row0;
  const int64_t K = p.K;
  const int nst = (int)(K / KS);
  const int64_t rbytes = K / 2, sbytes = K / kMxBlock;
  const bool comp = p.sel_idx != nullptr;
  const int kc = comp ? p.kc : 0;
  const int kcp = (kc + 63) / 64 * 64;
  float* RW = reinterpret_cast<float*>(smem + p.rw_lds_offset);

  // ---- row pointers (branch-free loads: rows outside the tile read row 0) --
  const int g4 = tid & 3;
  const uint8_t* a_cp[NA];
  uint32_t a_keep[NA];
#pragma unroll
  for (int i = 0; i < NA; ++i) {
    const int r = (tid >> 2) + 64 * i;
    int64_t ar = 0;
    bool ok = false;
    if (r < rows_valid) {
      const int64_t ur = row0 + r;
      ar = p.a_row_index ? (int64_t)p.a_row_index[ur] : ur;
      ok = ar >= 0 && ar < p.a_rows;
      if (!ok) ar = 0;
    }
    a_keep[i] = ok ? 0xFFFFFFFFu : 0u;       // a row index outside [0, a_rows) reads as zeros
    a_cp[i] = p.a_codes + ar * rbytes + g4 * 16;
  }
  int64_t as_row = 0;
  if (tid < rows_valid) {
    const int64_t ur = row0 + tid;
    as_row = p.a_row_index ? (int64_t)p.a_row_index[ur] : ur;
    if (as_row < 0 || as_row >= p.a_rows) as_row = 0;
  }
  const uint8_t* a_sp = p.a_scales + as_row * sbytes;
  const uint8_t* b_cp[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int64_t br = weight_row<BN>(p, n_tile, (tid >> 2) + 64 * i);
    b_cp[i] = p.w_codes + ((int64_t)e * p.N + (br >= 0 ? br : 0)) * rbytes + g4 * 16;
  }
  const int64_t b_own = weight_row<BN>(p, n_tile, tid);
  const uint8_t* b_sp = p.w_scales + ((int64_t)e * p.N + (b_own >= 0 ? b_own : 0)) * sbytes;

  struct Ld {
    u32x4 a[NA], b[4];
    uint32_t as, bs;
  };
  auto gload = [&](int m, Ld& r) {
    const int64_t co = (int64_t)m * 64;
#pragma unroll
    for (int i = 0; i < NA; ++i) r.a[i] = *reinterpret_cast<const u32x4*>(a_cp[i] + co);
#pragma unroll
    for (int i = 0; i < 4; ++i) r.b[i] = *reinterpret_cast<const u32x4*>(b_cp[i] + co);
    r.as = *reinterpret_cast<const uint32_t*>(a_sp + (int64_t)m * 4);
    r.bs = *reinterpret_cast<const uint32_t*>(b_sp + (int64_t)m * 4);
  };
  // xmax: the largest scale byte of weight row tid (read in the prologue).
  uint32_t xmax = 0;
  auto max_bytes = [&](uint32_t w) {
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const uint32_t b = (w >> (8 * q)) & 0xFFu;
      xmax = b > xmax ? b : xmax;
    }
  };
  auto swrite = [&](int st, const Ld& r) {
    unsigned char* base = smem + st * STAGE;
#pragma unroll
    for (int i = 0; i < NA; ++i) {
      const int row = (tid >> 2) + 64 * i;
      const u32x4 v = r.a[i] & a_keep[i];
      *reinterpret_cast<u32x4*>(base + (row < BM ? row : BM) * ROW + g4 * 16) = v;
    }
#pragma unroll
    for (int i = 0; i < 4; ++i)
      *reinterpret_cast<u32x4*>(base + B_OFF + ((tid >> 2) + 64 * i) * ROW + g4 * 16) = r.b[i];
    *reinterpret_cast<uint32_t*>(base + (tid < BM ? tid : BM) * ROW + 64) = r.as;
    *reinterpret_cast<uint32_t*>(base + B_OFF + tid * ROW + 64) = r.bs;
  };

  // ---- prologue: compensation set-up, row weights -----------------------------
  // Q(R_S) of this wave's rows for one 64-wide K-step: codes of lane half
  // `half` and the scale bytes of both halves.  Step 0 is loaded ahead of
  // the K loop, step 1 (kc > 64) after it.
  const int rb = kc / 2, sbr = kc / kMxBlock;
  u32x4 rq[MI];
  uint32_t rsc[MI];
  auto load_rs = [&](int ks) {
#pragma unroll
    for (int i = 0; i < MI; ++i) {
      const int r = wm * MI * 32 + i * 32 + l32;
      rq[i] = u32x4{0, 0, 0, 0};
      rsc[i] = 0;
      if (r < rows_valid) {
        const int64_t ur = row0 + r;
        if (ks * 64 + half * 32 < kc)
          rq[i] = *reinterpret_cast<const u32x4*>(p.r_codes + ur * rb + ks * 32 + half * 16);
        const uint32_t s0 = p.r_scales[ur * sbr + ks * 2];
        const uint32_t s1 = ks * 64 + 32 < kc ? p.r_scales[ur * sbr + ks * 2 + 1] : 0u;
        rsc[i] = s0 | (s1 << 8);
      }
    }
  };
  // First selected channel at or after channel c (binary search in LDS).
  auto lower = [&](int c) {
    int lo = 0, hi = kc;
    while (lo < hi) {
      const int mid = (lo + hi) >> 1;
      if (sel[mid] < c) lo = mid + 1; else hi = mid;
    }
    return lo;
  };
  if (comp) {
    for (int j = tid; j < kc; j += 256) {
      int32_t c = p.sel_idx[(int64_t)e * kc + j];
      sel[j] = c < 0 ? 0 : (c >= K ? (int32_t)(K - 1) : c);
    }
    load_rs(0);
    // the row's scale bytes, all loads in flight together (K <= 4096 takes one pass)
    const int n16 = (int)(sbytes / 16), n4 = (int)(sbytes / 4);
    for (int q = 0; q < n16; q += 8) {
      u32x4 w[8];
#pragma unroll
      for (int u = 0; u < 8; ++u)
        w[u] = q + u < n16 ? *reinterpret_cast<const u32x4*>(b_sp + 16 * (q + u)) : u32x4{0, 0, 0, 0};
#pragma unroll
      for (int u = 0; u < 8; ++u) { max_bytes(w[u][0]); max_bytes(w[u][1]); max_bytes(w[u][2]); max_bytes(w[u][3]); }
    }
    for (int q = 4 * n16; q < n4; ++q) max_bytes(*reinterpret_cast<const uint32_t*>(b_sp + 4 * q));
    // padding channels kc .. kcp-1 of W_S are zero (entry 0 converts to +0)
    for (int j = kc; j < kcp; ++j) WS[tid * wss + j] = 0;
    __syncthreads();
    // gather table of stage m: first selected channel j0 and count n, and the
    // in-stage offsets of its first four channels
    for (int m = tid; m < nst; m += 256) {
      const int j0 = lower(m * KS), n = lower((m + 1) * KS) - j0;
      uint32_t kk = 0;
      for (int q = 0; q < 4 && q < n; ++q) kk |= (uint32_t)((sel[j0 + q] - m * KS) & 0x7F) << (8 * q);
      tab[m] = u32x2{(uint32_t)j0 | ((uint32_t)n << 8), kk};
    }
  }
  if constexpr (EPI == 2) {
    if (tid < BM) RW[tid] = tid < rows_valid ? p.row_weight[row0 + tid] : 0.0f;
  }

  f32x16 acc[MI][NJ];
#pragma unroll
  for (int i = 0; i < MI; ++i)
#pragma unroll
    for (int j = 0; j < NJ; ++j)
#pragma unroll
      for (int q = 0; q < 16; ++q) acc[i][j][q] = 0.0f;

  // W_S entry of weight row tid for a selected channel at offset kk inside
  // the stage held in LDS row `row`: code | min(xmax - scale byte, 15) << 4
  // (E2M1 times 2^-15 or less is below half of E4M3's smallest subnormal,
  // so the clamp changes no E4M3 rounding).
  unsigned char* WSt = WS + tid * wss;
  auto ws_entry = [&](uint32_t code_byte, uint32_t scale, int kk) {
    const uint32_t code = (code_byte >> (4 * (kk & 1))) & 15u;
    const uint32_t d = xmax - scale;                          // >= 0
    return code | ((d < 15u ? d : 15u) << 4);
  };
  // Stage m's selected channels beyond the first four (rare): a plain loop.
  auto gather_rest = [&](const unsigned char* row, int m, int j0, int n) {
    for (int jj = j0 + 4; jj < j0 + n; ++jj) {
      const int kk = sel[jj] - m * KS;
      if ((unsigned)kk < (unsigned)KS)                        // false only if sel is not ascending
        WSt[jj] = (uint8_t)ws_entry(row[kk >> 1], row[64 + (kk >> 5)], kk);
    }
  };
  // After the K loop: W_S row tid in E4M3 against 2^xmax, in place.
  auto convert_ws = [&]() {
#pragma unroll 4
    for (int q = 0; q < kcp / 8; ++q) {
      const u32x2 v = *reinterpret_cast<const u32x2*>(WSt + 8 * q);
      float f[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const uint32_t b = (v[u >> 2] >> (8 * (u & 3))) & 0xFFu;
        f[u] = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(b & 15u, 1.0f, 0)[0] * pow2_nonpos(-(int)(b >> 4));
      }
      int lo = __builtin_amdgcn_cvt_pk_fp8_f32(f[0], f[1], 0, false);
      lo = __builtin_amdgcn_cvt_pk_fp8_f32(f[2], f[3], lo, true);
      int hi = __builtin_amdgcn_cvt_pk_fp8_f32(f[4], f[5], 0, false);
      hi = __builtin_amdgcn_cvt_pk_fp8_f32(f[6], f[7], hi, true);
      *reinterpret_cast<u32x2*>(WSt + 8 * q) = u32x2{(uint32_t)lo, (uint32_t)hi};
    }
    WX[tid] = (uint8_t)xmax;
  };

  // tm: gather table entry of the current stage (uniform; read one stage ahead)
  u32x2 tm = u32x2{0, 0};
  auto stage = [&](int m, int st, Ld& rset) {
    const unsigned char* base = smem + st * STAGE;
    u32x4 fa[2][MI], fb[2][NJ];
    uint32_t sa[MI], sb[NJ];
#pragma unroll
    for (int i = 0; i < MI; ++i) {
      const unsigned char* row = base + (wm * MI * 32 + i * 32 + l32) * ROW;
      fa[0][i] = *reinterpret_cast<const u32x4*>(row + half * 16);
      fa[1][i] = *reinterpret_cast<const u32x4*>(row + 32 + half * 16);
      sa[i] = *reinterpret_cast<const uint32_t*>(row + 64) >> (8 * half);
    }
#pragma unroll
    for (int j = 0; j < NJ; ++j) {
      const unsigned char* row = base + B_OFF + (wn * NJ * 32 + j * 32 + l32) * ROW;
      fb[0][j] = *reinterpret_cast<const u32x4*>(row + half * 16);
      fb[1][j] = *reinterpret_cast<const u32x4*>(row + 32 + half * 16);
      sb[j] = *reinterpret_cast<const uint32_t*>(row + 64) >> (8 * half);
    }
    // the gather's LDS reads go out now and are consumed after the MFMAs
    const unsigned char* grow = base + B_OFF + tid * ROW;
    int j0 = 0, n = 0;
    uint32_t gcb[4], gsb[4];
    u32x2 tnext = u32x2{0, 0};
    if (comp) {
      j0 = __builtin_amdgcn_readfirstlane((int)(tm[0] & 0xFFu));
      n = __builtin_amdgcn_readfirstlane((int)(tm[0] >> 8));
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int kk = (int)((tm[1] >> (8 * q)) & 0x7Fu);
        gcb[q] = q < n ? grow[kk >> 1] : 0u;
        gsb[q] = q < n ? grow[64 + (kk >> 5)] : 0u;
      }
      if (m + 1 < nst) tnext = tab[m + 1];
    }
#pragma unroll
    for (int j = 0; j < NJ; ++j)
#pragma unroll
      for (int i = 0; i < MI; ++i)
        acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
            as_v8i(fa[0][i]), as_v8i(fb[0][j]), acc[i][j], 4, 4, 0, (int)sa[i], 0, (int)sb[j]);
    swrite(st ^ 1, rset);                                    // data of stage m + 1
    if (m + 3 < nst) gload(m + 3, rset);
#pragma unroll
    for (int j = 0; j < NJ; ++j)
#pragma unroll
      for (int i = 0; i < MI; ++i)
        acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
            as_v8i(fa[1][i]), as_v8i(fb[1][j]), acc[i][j], 4, 4, 2, (int)sa[i], 2, (int)sb[j]);
    if (comp) {
#pragma unroll
      for (int q = 0; q < 4; ++q)
        if (q < n) WSt[j0 + q] = (uint8_t)ws_entry(gcb[q], gsb[q], (int)((tm[1] >> (8 * q)) & 0x7Fu));
      if (n > 4) gather_rest(grow, m, j0, n);
      tm = tnext;
    }
    lds_barrier();
  };

  {
    Ld R0, R1;
    gload(0, R0);
    if (nst > 1) gload(1, R1); else R1 = R0;
    swrite(0, R0);
    if (nst > 2) gload(2, R0);
    __syncthreads();
    if (comp) tm = tab[0];
    for (int m = 0; m < nst; m += 2) {
      stage(m, 0, R1);
      if (m + 1 < nst) stage(m + 1, 1, R0);
    }
  }

  // ---- compensation: Q(R_S) (widened to E4M3) x W_S (E4M3, row scale) -----
  if (comp) {
    convert_ws();
    __syncthreads();
    for (int ks = 0; ks < 2; ++ks) {
      if (ks * 64 >= kc) break;                               // uniform
      if (ks == 1) load_rs(1);
      v8i fa[MI], fb[NJ];
      uint32_t sa[MI], sb[NJ];
#pragma unroll
      for (int i = 0; i < MI; ++i) {
        // Both lane halves of a row take one scale, the larger of the row's
        // two blocks in this K-step (the FP8 form of the MFMA is only used
        // with a scale shared by all 64 K-values of a row or column, so the
        // order in which it pairs K-values and scales does not matter).
        const u32x4 w = rq[i];
        const uint32_t s0 = rsc[i] & 0xFFu, s1 = rsc[i] >> 8;
        const uint32_t s_max = s0 > s1 ? s0 : s1, s_own = half ? s1 : s0;
        const float f = pow2_nonpos((int)s_own - (int)s_max);
        u32x2 q[4];
#pragma unroll
        for (int c = 0; c < 4; ++c) q[c] = e2m1x8_to_e4m3(w[c], f);
        fa[i] = v8i{(int)q[0][0], (int)q[0][1], (int)q[1][0], (int)q[1][1],
                    (int)q[2][0], (int)q[2][1], (int)q[3][0], (int)q[3][1]};
        sa[i] = s_max;
      }
#pragma unroll
      for (int j = 0; j < NJ; ++j) {
        const int r = wn * NJ * 32 + j * 32 + l32;
        const u32x4 lo = *reinterpret_cast<const u32x4*>(WS + r * wss + ks * 64 + half * 32);
        const u32x4 hi = *reinterpret_cast<const u32x4*>(WS + r * wss + ks * 64 + half * 32 + 16);
        fb[j] = v8i{(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3],
                    (int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]};
        sb[j] = WX[r];
      }
#pragma unroll
      for (int j = 0; j < NJ; ++j)
#pragma unroll
        for (int i = 0; i < MI; ++i)
          acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
              fa[i], fb[j], acc[i][j], 0, 0, 0, (int)sa[i], 0, (int)sb[j]);
    }
  }

  __syncthreads();                             // LDS free for the epilogue staging
  gemm_epilogue<MI, NJ, BN, EPI>(p, acc, tc, wm * MI * 32, wn * NJ * 32, 1.0f,
                                 reinterpret_cast<float*>(smem) + wave * epilogue_wave_floats<NJ>(), RW);
}

template <int MI, int NJ, int WM, int WN>
__host__ constexpr size_t loop_lds_bytes(int64_t K, int kc) {
  return 2 * (size_t)Layout<WM * MI * 32>::STAGE + (size_t)BN * ws_stride(kc) + BN +
         (size_t)MAX_KC * 4 + (size_t)(K / KS) * 8;
}

template <int MI, int NJ, int WM, int WN, int EPI>
static hipError_t launch_cfg(GemmArgs a, hipStream_t stream) {
  constexpr int BM = WM * MI * 32;
  const int64_t mtiles = (a.rows_total + BM - 1) / BM + a.E;
  const int64_t ntiles = a.epilogue == 1 ? (a.N / 2 + BN / 2 - 1) / (BN / 2) : (a.N + BN - 1) / BN;
  const int64_t total = mtiles * ntiles;
  const size_t loop = (loop_lds_bytes<MI, NJ, WM, WN>(a.K, a.sel_idx ? a.kc : 0) + 15) / 16 * 16;
  const size_t epi = (size_t)4 * epilogue_wave_floats<NJ>() * 4;
  const size_t body = loop > epi ? loop : epi;
  a.rw_lds_offset = (int)body;
  const size_t lds = body + (EPI == 2 ? (size_t)BM * 4 : 0);
  auto kern = mx_grouped_gemm_kernel<MI, NJ, WM, WN, EPI>;
  hipError_t err = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
  if (err != hipSuccess) return err;
  const int64_t grid = (total + 7) / 8 * 8;       // upper bound on the tiles, one share per XCD
  kern<<<(unsigned)grid, 256, lds, stream>>>(a, (int)ntiles);
  return hipGetLastError();
}

template <int MI, int NJ, int WM, int WN>
static hipError_t launch_epi(const GemmArgs& a, hipStream_t stream) {
  switch (a.epilogue) {
    case 0: return launch_cfg<MI, NJ, WM, WN, 0>(a, stream);
    case 1: return launch_cfg<MI, NJ, WM, WN, 1>(a, stream);
    default: return launch_cfg<MI, NJ, WM, WN, 2>(a, stream);
  }
}

}  // namespace mxg

size_t mx_gemm_max_lds(int64_t K) {
  return mxg::loop_lds_bytes<4, 4, 2, 2>(K, mxg::MAX_KC) + 16 + 256 * 4;
}

hipError_t launch_mx_grouped_gemm(const GemmArgs& a, hipStream_t stream) {
  if (a.epilogue == 1 && a.out_amax) {
    hipError_t err = launch_fill_f32(a.out_amax, 1, 0.0f, stream);
    if (err != hipSuccess) return err;
  }
  if (a.rows_total == 0) return hipSuccess;
  hipError_t err;
  const int bm = a.block_m > 0 ? a.block_m : grouped_gemm_block_m(a.rows_total, a.E);
  switch (bm) {
    case 256: err = mxg::launch_epi<4, 4, 2, 2>(a, stream); break;
    case 128: err = mxg::launch_epi<2, 4, 2, 2>(a, stream); break;
    case 64: err = mxg::launch_epi<1, 4, 2, 2>(a, stream); break;
    default: err = mxg::launch_epi<1, 2, 1, 4>(a, stream); break;
  }
  if (err != hipSuccess || a.epilogue != 2) return err;
  return launch_combine(a.y_rows, a.rows_total, a.N, a.scatter_index, a.out_rows,
                        static_cast<float*>(a.out), a.ldo, a.y_rows, stream);
}

}  // namespace nvfp4
