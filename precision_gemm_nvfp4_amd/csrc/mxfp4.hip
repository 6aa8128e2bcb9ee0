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
#include <type_traits>

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
// (gemm_common.h).  K moves 128 per pipeline stage through a ring of LDS
// slots (four for tiles of 128 rows or more, else three), filled by direct
// global-to-LDS buffer loads (lane l of an instruction writes 16 bytes at
// base + 16 l, so no registers carry the tiles).  A slot holds the stage's 64 code bytes of every A and W
// row, 16-byte chunks swizzled within a row (chunk c of row r at position
// c ^ ((r >> 1) & 3), so that the fragment reads of 8 consecutive rows hit
// distinct banks), then the 4 scale bytes of every row.  Each wave issues the
// same number of load instructions per stage (padding ones go to a dummy
// area), so one vmcnt wait tells it its share of a stage has landed.
// Iteration m: run the first half of the stage-m MFMAs from registers, wait
// for stage m + 1 and meet at the one barrier, issue the loads of stage
// m + PD (PD = slots - 1) into the slot stage m - 1 used, and read the
// stage-(m + 1) fragments while the second half of the stage-m MFMAs runs.
// So LDS reads and loads overlap the matrix cores, and a slot is refilled
// only after every wave has passed the barrier that followed its last read.
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
constexpr int MAX_KC = 128;
constexpr int DUMMY_BYTES = 1024;          // target of the padding loads

// Bytes per W_S row in LDS for kc compensated channels: one byte per channel
// of the padded width plus 16 of padding (0 without compensation).
__host__ __device__ constexpr int ws_stride(int kc) {
  return kc > 0 ? (kc + 63) / 64 * 64 + 16 : 0;
}

// One LDS slot: A codes [BM][64], W codes [BN][64], A scale words
// [max(BM, 64)], W scale words [BN].  Load instructions per wave and stage:
// NAI A-code blocks of 16 rows, 4 W-code blocks, one A-scale and one W-scale
// block of 64 rows.
// A8: the activations are MXFP8 (one byte per element, 128 bytes a row per
// stage, 8 rows per 1 KB load instruction) instead of MXFP4.
template <int BM, bool A8 = false>
struct Layout {
  static constexpr int AROW = A8 ? 128 : 64;           // A bytes per row and stage
  static constexpr int A_OFF = 0;
  static constexpr int B_OFF = BM * AROW;
  static constexpr int AS_OFF = B_OFF + BN * 64;
  static constexpr int ASR = BM < 64 ? 64 : BM;
  static constexpr int BS_OFF = AS_OFF + ASR * 4;
  static constexpr int STAGE = BS_OFF + BN * 4;
  static constexpr int ABLK = BM * AROW / 1024;        // A-code load instructions per stage
  static constexpr int NAI = ABLK < 4 ? 1 : ABLK / 4;  // ... per wave (padding ones included)
  static constexpr int LPW = NAI + 6;                  // load instructions per wave and stage
  // LDS ring: four slots (three stages in flight) for the tall tiles, whose
  // time per stage is set by how many bytes a CU keeps in flight; three for
  // the short ones, so that two of them still share a CU, and for the
  // 256-row MXFP8 tile, whose slots are larger
  static constexpr int NSLOT = BM >= 128 && STAGE * 4 <= 144 * 1024 ? 4 : 3;
  static constexpr int PD = NSLOT - 1;                 // prefetch distance in stages
};

__device__ __forceinline__ int swz(int r) { return (r >> 1) & 3; }

template <int V>
struct KC {                                 // a compile-time count
  static constexpr int value = V;
};


// Direct global-to-LDS loads through buffer resources: base and size in
// scalar registers, the stage's advance as the scalar offset, each lane's
// position a vector offset fixed for the tile, so a load costs no vector
// arithmetic.  Lane l writes its 16 / 4 bytes at LDS l * 16 / l * 4 past the
// (uniform) destination.
typedef __attribute__((address_space(3))) void lds_void_t;
typedef __amdgpu_buffer_rsrc_t Rsrc;
__device__ __forceinline__ void load_lds16(Rsrc r, uint32_t voff, int soff, unsigned char* l) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void_t*)l, 16, voff, soff, 0, 0);
}
__device__ __forceinline__ void load_lds4(Rsrc r, uint32_t voff, int soff, unsigned char* l) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void_t*)l, 4, voff, soff, 0, 0);
}
// s_waitcnt vmcnt(N) lgkmcnt(0) (gfx9 encoding: vmcnt in bits 0-3 and 14-15)
template <int N>
__device__ __forceinline__ void wait_vm_lgkm0() {
  __builtin_amdgcn_s_waitcnt((N & 15) | 0x70 | ((N >> 4) << 14));
}

typedef int v8i __attribute__((ext_vector_type(8)));

__device__ __forceinline__ v8i as_v8i(const u32x4& w) {
  return v8i{(int)w[0], (int)w[1], (int)w[2], (int)w[3], 0, 0, 0, 0};
}
__device__ __forceinline__ v8i a_v8i(const u32x4& w) { return as_v8i(w); }
__device__ __forceinline__ v8i a_v8i(const v8i& w) { return w; }

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

template <int MI, int NJ, int WM, int WN, int EPI, bool COMP, bool A8>
__global__ __launch_bounds__(256, 1) void mx_grouped_gemm_kernel(GemmArgs p, int ntiles) {
  constexpr int BM = WM * MI * 32;
  static_assert(WN * NJ * 32 == BN, "N tile");
  static_assert(WM * WN == 4, "four waves");
  static_assert(!(A8 && COMP), "the MXFP8-activation GEMM has no compensation");
  using L = Layout<BM, A8>;
  constexpr int STAGE = L::STAGE, NAI = L::NAI, LPW = L::LPW, NSLOT = L::NSLOT, PD = L::PD;
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  // LDS: NSLOT slots | dummy | W_S [BN][wss] bytes | Xmax bytes [BN] |
  // sel [MAX_KC] | gather table [nst] (u32x2 per stage).  W_S row t holds, for
  // each selected channel j, code | min(xmax - scale byte, 15) << 4 during the
  // K loop, and the E4M3 byte of W[t, sel[j]] / 2^(xmax - 127) after it.
  const int wss = ws_stride(p.sel_idx ? p.kc : 0);
  unsigned char* DUMMY = smem + NSLOT * STAGE;
  unsigned char* WS = DUMMY + DUMMY_BYTES;
  unsigned char* WX = WS + BN * wss;
  int32_t* sel = reinterpret_cast<int32_t*>(WX + BN);
  u32x2* tab = reinterpret_cast<u32x2*>(sel + MAX_KC);

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // uniform: LDS targets in SGPRs
  const int wm = wave / WN, wn = wave % WN;
  const int half = lane >> 5, l32 = lane & 31;

  TileCoord tc;
  if (!map_tile<BM>(p, ntiles, tc)) return;       // uniform over the workgroup
  const int e = tc.e, n_tile = tc.n_tile, rows_valid = tc.rows_valid;
  const int64_t row0 = tc.row0;
  const int64_t K = p.K;
  const int nst = (int)(K / KS);
  const int64_t rbytes = K / 2, sbytes = K / kMxBlock;
  constexpr bool comp = COMP;
  const int kc = comp ? p.kc : 0;
  const int kcp = (kc + 63) / 64 * 64;
  float* RW = reinterpret_cast<float*>(smem + p.rw_lds_offset);

  // ---- load addressing ---------------------------------------------------------
  // Lane l of a 16-row block instruction loads row 16 b + l / 4, position
  // l % 4, i.e. logical chunk (l % 4) ^ swz(row).  Rows outside the tile, and
  // A rows whose index lies outside [0, a_rows), read row 0 (their results are
  // never stored, or unspecified for a bad index).
  auto a_row = [&](int r) -> int64_t {
    if (r >= rows_valid) return 0;
    const int64_t ur = row0 + r;
    const int64_t ar = p.a_row_index ? (int64_t)p.a_row_index[ur] : ur;
    return ar >= 0 && ar < p.a_rows ? ar : 0;
  };
  // weight row of tile row r inside expert e's matrix (row 0 past N)
  auto w_row = [&](int r) -> int64_t {
    const int64_t br = weight_row<BN>(p, n_tile, r);
    return br >= 0 ? br : 0;
  };
  // Buffer resources of A's and this expert's W codes and scales (the host
  // checks that each operand spans less than 4 GiB), built once.
  const uint8_t* wc_e = p.w_codes + (int64_t)e * p.N * rbytes;
  const uint8_t* ws_e = p.w_scales + (int64_t)e * p.N * sbytes;
  const int lr = lane >> 2, lp = lane & 3;
  // MXFP8 rows: 8 chunks of 16 bytes a stage, chunk c at position c ^ (r & 7)
  const int64_t arbytes = A8 ? K : rbytes;
  const Rsrc r_ac = make_rsrc(p.a_codes, p.a_rows * arbytes);
  const Rsrc r_as = make_rsrc(p.a_scales, p.a_rows * sbytes);
  const Rsrc r_wc = make_rsrc(wc_e, p.N * rbytes);
  const Rsrc r_ws = make_rsrc(ws_e, p.N * sbytes);
  uint32_t a_off[NAI];
#pragma unroll
  for (int i = 0; i < NAI; ++i) {
    const int b = wave * NAI + i;
    if constexpr (A8) {
      const int r = b * 8 + (lane >> 3), q = lane & 7;
      a_off[i] = (uint32_t)(a_row(b < L::ABLK ? r : BM) * arbytes) + ((q ^ (r & 7)) << 4);
    } else {
      const int r = b * 16 + lr;
      a_off[i] = (uint32_t)(a_row(b < L::ABLK ? r : BM) * arbytes) + ((lp ^ swz(r)) << 4);
    }
  }
  uint32_t b_off[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int r = (wave * 4 + i) * 16 + lr;
    b_off[i] = (uint32_t)(w_row(r) * rbytes) + ((lp ^ swz(r)) << 4);
  }
  // Scale words are stored in the order the fragment reads want them: the
  // word of A row wm MI 32 + 32 i + l32 at position (wm 32 + l32) MI + i, so
  // a lane reads its MI words (likewise NJ for W) with one LDS instruction.
  // Lane l of the scale instruction of wave w fills position 64 w + l.
  const int rs_pos = 64 * wave + lane;
  const int ra_s = (rs_pos / (32 * MI)) * (32 * MI) + (rs_pos % MI) * 32 + (rs_pos / MI) % 32;
  const int rb_s = (rs_pos / (32 * NJ)) * (32 * NJ) + (rs_pos % NJ) * 32 + (rs_pos / NJ) % 32;
  const uint32_t as_off = (uint32_t)(a_row(rs_pos < BM ? ra_s : BM) * sbytes);
  const uint32_t bs_off = (uint32_t)(w_row(rb_s) * sbytes);
  const uint8_t* b_sp = ws_e + w_row(tid) * sbytes;   // weight row tid (compensation)

  // the LPW load instructions of stage m into slot `slot`
  auto issue = [&](int m, int slot) {
    unsigned char* base = smem + slot * STAGE;
#pragma unroll
    for (int i = 0; i < NAI; ++i) {
      const int b = wave * NAI + i;
      load_lds16(r_ac, a_off[i], m * L::AROW, b < L::ABLK ? base + L::A_OFF + b * 1024 : DUMMY);
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) load_lds16(r_wc, b_off[i], m * 64, base + L::B_OFF + (wave * 4 + i) * 1024);
    load_lds4(r_as, as_off, m * 4, 64 * wave < BM ? base + L::AS_OFF + wave * 256 : DUMMY);
    load_lds4(r_ws, bs_off, m * 4, base + L::BS_OFF + wave * 256);
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

  // the first two stages go out first, so that their latency overlaps the
  // compensation set-up below
#pragma unroll
  for (int q = 0; q < PD; ++q) issue(q < nst ? q : nst - 1, q);

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

  // W_S entry of weight row tid for a selected channel at K-offset kk of a
  // stage, from its code byte and scale byte: code | min(xmax - scale, 15) << 4
  // (E2M1 times 2^-15 or less is below half of E4M3's smallest subnormal,
  // so the clamp changes no E4M3 rounding).
  unsigned char* WSt = WS + tid * wss;
  auto ws_entry = [&](uint32_t code_byte, uint32_t scale, int kk) {
    const uint32_t code = (code_byte >> (4 * (kk & 1))) & 15u;
    const uint32_t d = xmax - scale;                          // >= 0
    return code | ((d < 15u ? d : 15u) << 4);
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

  // A wave's fragments: A0/B0 feed the stage's first 64-wide K-step, A1/B1
  // its second (lane half h takes logical chunk 2 ks + h), SA/SB the scale
  // words shifted so that op_sel 0 / 2 picks the lane's block of step 0 / 1.
  // A0/B0 of stage m + 1 are read as soon as the step-0 MFMAs of stage m have
  // been issued, A1/B1 and the scale words after the step-1 ones.
  using AFrag = typename std::conditional<A8, v8i, u32x4>::type;
  AFrag A0[MI], A1[MI];
  u32x4 B0[NJ], B1[NJ];
  uint32_t SA[MI], SB[NJ];
  // Per-lane LDS offsets: the swizzle of rows r = 32 i + l32 (+ a multiple of
  // 32) depends on l32 only, so the row blocks are immediate offsets.
  const int sw = swz(l32);
  const uint32_t fa_off[2] = {(uint32_t)(L::A_OFF + (wm * MI * 32 + l32) * 64 + ((half ^ sw) << 4)),
                              (uint32_t)(L::A_OFF + (wm * MI * 32 + l32) * 64 + (((2 + half) ^ sw) << 4))};
  const uint32_t fb_off[2] = {(uint32_t)(L::B_OFF + (wn * NJ * 32 + l32) * 64 + ((half ^ sw) << 4)),
                              (uint32_t)(L::B_OFF + (wn * NJ * 32 + l32) * 64 + (((2 + half) ^ sw) << 4))};
  const uint32_t sa_off = (uint32_t)(L::AS_OFF + (wm * 32 + l32) * MI * 4);
  const uint32_t sb_off = (uint32_t)(L::BS_OFF + (wn * 32 + l32) * NJ * 4);
  // MXFP8 A: lane half h of K-step ks takes chunks 4 ks + h and 4 ks + 2 + h
  // (the FP8 form of the MFMA holds K 16 h .. and 32 + 16 h .. of the step in
  // a lane, checked on the GPU), each at position c ^ (r & 7); r & 7 = l32 & 7
  const uint32_t fa8_off[2][2] = {
      {(uint32_t)(L::A_OFF + (wm * MI * 32 + l32) * 128 + ((half ^ (l32 & 7)) << 4)),
       (uint32_t)(L::A_OFF + (wm * MI * 32 + l32) * 128 + (((2 + half) ^ (l32 & 7)) << 4))},
      {(uint32_t)(L::A_OFF + (wm * MI * 32 + l32) * 128 + (((4 + half) ^ (l32 & 7)) << 4)),
       (uint32_t)(L::A_OFF + (wm * MI * 32 + l32) * 128 + (((6 + half) ^ (l32 & 7)) << 4))}};
  auto read_half = [&](int slot, int ks, AFrag* A, u32x4* B) {
    const unsigned char* base = smem + slot * STAGE;
#pragma unroll
    for (int i = 0; i < MI; ++i) {
      if constexpr (A8) {
        const u32x4 lo = *reinterpret_cast<const u32x4*>(base + fa8_off[ks][0] + i * 4096);
        const u32x4 hi = *reinterpret_cast<const u32x4*>(base + fa8_off[ks][1] + i * 4096);
        A[i] = v8i{(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3], (int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]};
      } else {
        A[i] = *reinterpret_cast<const u32x4*>(base + fa_off[ks] + i * 2048);
      }
    }
#pragma unroll
    for (int j = 0; j < NJ; ++j) B[j] = *reinterpret_cast<const u32x4*>(base + fb_off[ks] + j * 2048);
  };
  auto read_words = [&](const unsigned char* p_, uint32_t* w, auto NW) {
    constexpr int n = decltype(NW)::value;
    if constexpr (n == 4) {
      const u32x4 v = *reinterpret_cast<const u32x4*>(p_);
      w[0] = v[0]; w[1] = v[1]; w[2] = v[2]; w[3] = v[3];
    } else if constexpr (n == 2) {
      const u32x2 v = *reinterpret_cast<const u32x2*>(p_);
      w[0] = v[0]; w[1] = v[1];
    } else {
      w[0] = *reinterpret_cast<const uint32_t*>(p_);
    }
  };
  auto read_scales = [&](int slot) {
    const unsigned char* base = smem + slot * STAGE;
    read_words(base + sa_off, SA, KC<MI>{});
    read_words(base + sb_off, SB, KC<NJ>{});
#pragma unroll
    for (int i = 0; i < MI; ++i) SA[i] >>= 8 * half;
#pragma unroll
    for (int j = 0; j < NJ; ++j) SB[j] >>= 8 * half;
  };

  // gather table entry of the current stage (uniform; read one stage ahead)
  u32x2 tm = u32x2{0, 0};
  // The byte holding K-offset kk of weight row tid in a slot, and its scale byte.
  // (the row is 64-byte aligned; the in-row byte (kk >> 5) << 4 | (kk & 31) >> 1
  // is uniform, the chunk swizzle of row tid is an XOR on bits 4-5)
  const uint32_t g_row = (uint32_t)(L::B_OFF + tid * 64), g_sw = (uint32_t)(swz(tid) << 4);
  const uint32_t g_srow = (uint32_t)(L::BS_OFF +
      (((tid / (32 * NJ)) * 32 + tid % 32) * NJ + (tid % (32 * NJ)) / 32) * 4);
  auto w_byte = [&](const unsigned char* base, int kk) {
    return base + (g_row | ((uint32_t)(((kk >> 5) << 4) | ((kk & 31) >> 1)) ^ g_sw));
  };
  auto w_scale = [&](const unsigned char* base, int kk) {
    return base + g_srow + (kk >> 5);
  };

  // Iteration m, the same straight-line code for every m (so the
  // accumulators keep their registers): the loads of stage m + PD -- for the
  // last PD iterations a repeat of the last stage into a slot nobody reads,
  // which keeps every wave's count of loads in flight the same -- then the
  // stage-m MFMAs with the stage-(m + 1) fragment reads between and after
  // them (in the last iteration those read a slot whose contents go unused).
  auto body = [&](int m, int slot) {
    const unsigned char* base = smem + slot * STAGE;
    const int nslot = slot == NSLOT - 1 ? 0 : slot + 1;
    int j0 = 0, n = 0;
    uint32_t gcb[4], gsb[4];
    u32x2 tnext = u32x2{0, 0};
    if constexpr (COMP) {             // the gather's LDS reads go out first
      j0 = __builtin_amdgcn_readfirstlane((int)(tm[0] & 0xFFu));
      n = __builtin_amdgcn_readfirstlane((int)(tm[0] >> 8));
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int kk = __builtin_amdgcn_readfirstlane((int)((tm[1] >> (8 * q)) & 0x7Fu));
        gcb[q] = *w_byte(base, kk);
        gsb[q] = *w_scale(base, kk);
      }
      tnext = tab[m + 1 < nst ? m + 1 : m];
    }
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int j = 0; j < NJ; ++j)
#pragma unroll
      for (int i = 0; i < MI; ++i)
        acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
            a_v8i(A0[i]), as_v8i(B0[j]), acc[i][j], A8 ? 0 : 4, 4, 0, (int)SA[i], 0, (int)SB[j]);
    __builtin_amdgcn_sched_barrier(0);
    // this wave's loads of stage m + 1 have landed (only those of stages
    // m + 2 .. m + PD - 1 may be outstanding); after the barrier every wave's
    // have.  The loads of stage m + PD go out here, where no LDS access is in
    // flight (setting M0 for them waits for those).
    wait_vm_lgkm0<(PD - 2) * LPW>();
    asm volatile("s_barrier" ::: "memory");
    issue(m + PD < nst ? m + PD : nst - 1, slot == 0 ? NSLOT - 1 : slot - 1);   // slot (m + PD) % NSLOT
    read_half(nslot, 0, A0, B0);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int j = 0; j < NJ; ++j)
#pragma unroll
      for (int i = 0; i < MI; ++i)
        acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
            a_v8i(A1[i]), as_v8i(B1[j]), acc[i][j], A8 ? 0 : 4, 4, 2, (int)SA[i], 2, (int)SB[j]);
    __builtin_amdgcn_sched_barrier(0);
    read_half(nslot, 1, A1, B1);
    read_scales(nslot);
    if constexpr (COMP) {
      // entries past the stage's count go to the row's padding bytes
#pragma unroll
      for (int q = 0; q < 4; ++q)
        WSt[q < n ? j0 + q : kcp + q] =
            (uint8_t)ws_entry(gcb[q], gsb[q], (int)((tm[1] >> (8 * q)) & 0x7Fu));
      for (int jj = j0 + 4; jj < j0 + n; ++jj) {               // more than four: rare
        const int kk = sel[jj] - m * KS;
        if ((unsigned)kk < (unsigned)KS)                        // false only if sel is not ascending
          WSt[jj] = (uint8_t)ws_entry(*w_byte(base, kk), *w_scale(base, kk), kk);
      }
      tm = tnext;
    }
  };

  {
    wait_vm_lgkm0<(PD - 1) * LPW>();  // stage 0 has landed (stages 1 .. PD - 1 may be in flight)
    asm volatile("s_barrier" ::: "memory");
    read_half(0, 0, A0, B0);
    read_half(0, 1, A1, B1);
    read_scales(0);
    if constexpr (COMP) tm = tab[0];
    int slot = 0;                     // uniform: the slot offsets are scalar adds
    for (int m = 0; m < nst; ++m) {
      body(m, slot);
      slot = slot == NSLOT - 1 ? 0 : slot + 1;
    }
    wait_vm_lgkm0<0>();               // the repeat loads of the last iterations
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

template <int MI, int NJ, int WM, int WN, bool A8 = false>
__host__ constexpr size_t loop_lds_bytes(int64_t K, int kc) {
  using L = Layout<WM * MI * 32, A8>;
  return L::NSLOT * (size_t)L::STAGE + DUMMY_BYTES + (size_t)BN * ws_stride(kc) + BN +
         (size_t)MAX_KC * 4 + (size_t)(K / KS) * 8;
}

// LDS bytes a tile configuration needs (0 if over the 160 KB of a CU).
template <int MI, int NJ, int WM, int WN, bool A8 = false>
static size_t cfg_lds(const GemmArgs& a) {
  const size_t loop = (loop_lds_bytes<MI, NJ, WM, WN, A8>(a.K, a.sel_idx ? a.kc : 0) + 15) / 16 * 16;
  const size_t epi = (size_t)4 * epilogue_wave_floats<NJ>() * 4;
  const size_t lds = (loop > epi ? loop : epi) + (size_t)WM * MI * 32 * 4 + 256;   // + row weights, static
  return lds <= 160 * 1024 ? lds : 0;
}

template <int MI, int NJ, int WM, int WN, int EPI, bool COMP, bool A8>
static hipError_t launch_cfg(GemmArgs a, hipStream_t stream) {
  constexpr int BM = WM * MI * 32;
  const int64_t mtiles = (a.rows_total + BM - 1) / BM + a.E;
  const int64_t ntiles = a.epilogue == 1 ? (a.N / 2 + BN / 2 - 1) / (BN / 2) : (a.N + BN - 1) / BN;
  const int64_t total = mtiles * ntiles;
  const size_t loop = (loop_lds_bytes<MI, NJ, WM, WN, A8>(a.K, a.sel_idx ? a.kc : 0) + 15) / 16 * 16;
  const size_t epi = (size_t)4 * epilogue_wave_floats<NJ>() * 4;
  const size_t body = loop > epi ? loop : epi;
  a.rw_lds_offset = (int)body;
  const size_t lds = body + (EPI == 2 ? (size_t)BM * 4 : 0);
  auto kern = mx_grouped_gemm_kernel<MI, NJ, WM, WN, EPI, COMP, A8>;
  hipError_t err = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
  if (err != hipSuccess) return err;
  const int64_t grid = (total + 7) / 8 * 8;       // upper bound on the tiles, one share per XCD
  kern<<<(unsigned)grid, 256, lds, stream>>>(a, (int)ntiles);
  return hipGetLastError();
}

template <int MI, int NJ, int WM, int WN, bool A8>
static hipError_t launch_epi(const GemmArgs& a, hipStream_t stream) {
  if constexpr (A8) {                          // no compensation with MXFP8 activations
    switch (a.epilogue) {
      case 0: return launch_cfg<MI, NJ, WM, WN, 0, false, true>(a, stream);
      case 1: return launch_cfg<MI, NJ, WM, WN, 1, false, true>(a, stream);
      default: return launch_cfg<MI, NJ, WM, WN, 2, false, true>(a, stream);
    }
  } else {
    const bool c = a.sel_idx != nullptr;
    switch (a.epilogue) {
      case 0: return c ? launch_cfg<MI, NJ, WM, WN, 0, true, false>(a, stream) : launch_cfg<MI, NJ, WM, WN, 0, false, false>(a, stream);
      case 1: return c ? launch_cfg<MI, NJ, WM, WN, 1, true, false>(a, stream) : launch_cfg<MI, NJ, WM, WN, 1, false, false>(a, stream);
      default: return c ? launch_cfg<MI, NJ, WM, WN, 2, true, false>(a, stream) : launch_cfg<MI, NJ, WM, WN, 2, false, false>(a, stream);
    }
  }
}

template <bool A8>
static hipError_t launch_any(const GemmArgs& a, hipStream_t stream) {
  if (a.epilogue == 1 && a.out_amax) {
    hipError_t err = launch_fill_f32(a.out_amax, 1, 0.0f, stream);
    if (err != hipSuccess) return err;
  }
  if (a.rows_total == 0)     // nothing to add; an overwriting scatter still writes zeros
    return a.epilogue == 2 && a.combine_overwrite
               ? launch_combine(a.y_rows, 0, a.N, a.scatter_index, a.out_rows, static_cast<float*>(a.out),
                                a.ldo, true, a.y_rows, stream)
               : hipSuccess;
  hipError_t err;
  int bm = a.block_m > 0 ? a.block_m : grouped_gemm_block_m(a.rows_total, a.E);
  // a long K (a long gather table) can push the tallest tile past the LDS
  if (bm == 256 && cfg_lds<4, 4, 2, 2, A8>(a) == 0) bm = 128;
  if (bm == 128 && cfg_lds<2, 4, 2, 2, A8>(a) == 0) bm = 64;
  auto gemm = [&]() -> hipError_t {
    switch (bm) {
      case 256: return launch_epi<4, 4, 2, 2, A8>(a, stream);
      case 128: return launch_epi<2, 4, 2, 2, A8>(a, stream);
      case 64: return launch_epi<1, 4, 2, 2, A8>(a, stream);
      default: return launch_epi<1, 2, 1, 4, A8>(a, stream);
    }
  };
  // The scatter's plan (the row lists of each output row) needs only the
  // scatter index: with 256-row tiles (a long launch) it runs beside the GEMM
  // on the side stream, and the ordered sum of the rows follows the join.
  // Beside a short launch of small tiles its one workgroup waits for a CU
  // and the fork and join cost more than they hide.
  if (a.epilogue == 2 && bm == 256) {
    if (SideStream* ss = side_stream(stream)) {
      std::lock_guard<std::mutex> lk(ss->mu);
      err = hipEventRecord(ss->fork, stream);
      if (err == hipSuccess) err = hipStreamWaitEvent(ss->s, ss->fork, 0);
      if (err == hipSuccess)
        err = launch_combine_plan(a.rows_total, a.N, a.scatter_index, a.out_rows, a.y_rows, ss->s);
      if (err == hipSuccess) err = hipEventRecord(ss->join, ss->s);
      if (err == hipSuccess) err = gemm();
      if (err == hipSuccess) err = hipStreamWaitEvent(stream, ss->join, 0);
      if (err != hipSuccess) return err;
      return launch_combine_rows(a.y_rows, a.rows_total, a.N, a.out_rows, static_cast<float*>(a.out),
                                 a.ldo, a.combine_overwrite, a.y_rows, stream);
    }
  }
  err = gemm();
  if (err != hipSuccess || a.epilogue != 2) return err;
  return launch_combine(a.y_rows, a.rows_total, a.N, a.scatter_index, a.out_rows,
                        static_cast<float*>(a.out), a.ldo, a.combine_overwrite, a.y_rows, stream);
}

}  // namespace mxg

size_t mx_gemm_max_lds(int64_t K) {
  return mxg::loop_lds_bytes<4, 4, 2, 2>(K, mxg::MAX_KC) + 16 + 256 * 4;
}

hipError_t launch_mx_grouped_gemm(const GemmArgs& a, hipStream_t stream) {
  return mxg::launch_any<false>(a, stream);
}

hipError_t launch_mx_w4a8_grouped_gemm(const GemmArgs& a, hipStream_t stream) {
  return mxg::launch_any<true>(a, stream);
}

// ---------------------------------------------------------------------------
// MXFP8 quantizer (activations of the W4A8 GEMM)
// ---------------------------------------------------------------------------
// Scale byte X + 127 with X = floor(log2 amax) - 8 (8 is the exponent of
// E4M3's largest value 448), clamped: from the fp32 exponent field E of amax
// it is max(E - 8, 0).  Elements: |x| 2^-X is exact (a power-of-two multiply;
// results small enough to underflow lie far below E4M3's smallest subnormal),
// clamped to 448 (MX saturates), then the hardware convert rounds to nearest
// even; the sign stays with the value.
__device__ __forceinline__ uint32_t mx8_scale_byte(float amax) {
  const int E = (int)((__float_as_uint(amax) >> 23) & 0xFFu);
  return (uint32_t)(E > 8 ? E - 8 : 0);
}

template <typename T>
__global__ __launch_bounds__(256) void mx8_quantize_kernel(const T* __restrict__ x, int64_t M,
                                                           int64_t K, int64_t ldx,
                                                           uint8_t* __restrict__ codes,
                                                           uint8_t* __restrict__ scales) {
  const int64_t nb = K / kMxBlock;
  const int64_t total = M * nb;
  for (int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; t < total;
       t += (int64_t)gridDim.x * blockDim.x) {
    const int64_t r = t / nb, bc = t % nb;
    float v[32];
    mx_load32<T>(x + r * ldx + bc * kMxBlock, v);
    float amax = 0.0f;
#pragma unroll
    for (int i = 0; i < 32; ++i) amax = fmaxf(amax, fabsf(v[i]));
    const uint32_t sb = mx8_scale_byte(amax);
    const float inv = __uint_as_float((254u - sb) << 23);   // 2^-X, a normal fp32
    uint32_t w[8];
#pragma unroll
    for (int q = 0; q < 8; ++q) {
      float f[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) f[u] = fminf(fmaxf(v[4 * q + u] * inv, -448.0f), 448.0f);
      int lo = __builtin_amdgcn_cvt_pk_fp8_f32(f[0], f[1], 0, false);
      lo = __builtin_amdgcn_cvt_pk_fp8_f32(f[2], f[3], lo, true);
      w[q] = (uint32_t)lo;
    }
    u32x4* dst = reinterpret_cast<u32x4*>(codes + r * K + bc * kMxBlock);
    dst[0] = u32x4{w[0], w[1], w[2], w[3]};
    dst[1] = u32x4{w[4], w[5], w[6], w[7]};
    scales[r * nb + bc] = (uint8_t)sb;
  }
}

hipError_t launch_mx8_quantize(const void* x, int dtype, int64_t M, int64_t K, int64_t ldx,
                               uint8_t* codes, uint8_t* scales, hipStream_t stream) {
  if (M == 0) return hipSuccess;
  const int64_t total = M * (K / kMxBlock);
  const int64_t blocks = (total + 255) / 256;
  const unsigned grid = (unsigned)(blocks < 8192 ? blocks : 8192);
  if (dtype == 0)
    mx8_quantize_kernel<__bf16><<<grid, 256, 0, stream>>>(static_cast<const __bf16*>(x), M, K, ldx, codes, scales);
  else
    mx8_quantize_kernel<float><<<grid, 256, 0, stream>>>(static_cast<const float*>(x), M, K, ldx, codes, scales);
  return hipGetLastError();
}

}  // namespace nvfp4
