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
// e2m1 * e4m3 * g.  e2m1 * e4m3 has at most 6 significant bits and lies in
// [2^-10, 2688]: exact in fp16 (and bf16), not in FP8 (4 bits), and the
// block-scaled FP4 MFMA takes one power-of-two scale per 32 elements, not an
// E4M3 per 16.  So the operands stay NVFP4 in memory and in LDS, and each wave
// dequantizes its own MFMA fragments in registers right before use: the
// hardware FP4 -> fp16 convert (two elements per instruction) and one packed
// fp16 multiply by the block's E4M3 scale (itself converted to fp16 by the
// hardware FP8 -> fp16 convert), both exact.  The MFMA is
// v_mfma_f32_32x32x16_f16 with fp32 accumulation (the same rate as bf16);
// the global scales gA gW (gR gW) are applied in the epilogue.
//
// K order inside a 32-wide K-step: in both MFMA substeps, lane half h (lanes
// 32h .. 32h+31) supplies the 16 consecutive k of NVFP4 block h of the step
// (first 8 in substep 0, last 8 in substep 1), so one 8-byte LDS read and one
// scale byte give a lane a whole block.  A and B use the same order, so the
// sum over the step's 32 k is unchanged.
//
// Pipeline: LDS holds two stages of raw codes + scales (9 KB per stage for a
// 256 x 256 tile); global loads run two K-steps ahead in a double register
// set.  In step s each wave issues its MFMAs of step s one at a time, and
// between them (fenced groups, so the order survives scheduling) the LDS
// reads of its step s+1 fragments, the stage write of step s+2, the global
// loads of step s+4 and the dequantization of the step s+1 fragments, half a
// fragment per MFMA.  One barrier per step.  On gfx950 a SIMD does not run
// VALU instructions while an MFMA executes, so the dequantization adds to the
// MFMA time (about 4.5 VALU instructions per MFMA for a 128 x 128 wave tile);
// the schedule keeps the MFMA pipe from also waiting on LDS or memory.  The
// 32-row tile, bound by memory rather than MFMA, uses 128-K stages with
// coalesced loads instead (MacroTile below).
//
// The compensation term is an extra chunk of kc: while the main loop streams
// the expert's weight tile through LDS, the elements of the selected columns
// are dequantized into an fp16 [BN, kc] buffer, so W is read from memory once.
// After the main loop the accumulators are rescaled by gA/gR, Q(R_S) x W_S is
// accumulated, and the epilogue multiplies by gR gW.
//
// Epilogues (gemm_common.h) stage each wave's 32-row blocks through LDS and
// write whole row segments with 16-byte stores.  Scatter epilogue:
// row_weight * Y rows go into the workspace and combine.hip adds them into
// the output rows in a fixed order.
//
// Work decomposition: the logical tiles are the (expert, m-tile, n-tile)
// triples of the ragged groups, expert-major, then m-tile, n-tile innermost;
// their number T comes from the group offsets on the device, and the grid is
// an upper bound ((ceil(rows / BM) + E) x n-tiles, rounded up to a multiple of
// 8).  Workgroup ids are dealt round-robin to the 8 XCDs, so hardware id h
// runs logical tile (h % 8) * ceil(T / 8) + h / 8 and the rest exit: each XCD
// owns a contiguous eighth of the real tiles (dividing the upper bound instead
// would leave whole XCDs with surplus workgroups only).  Inside an XCD the
// workgroups go to its shader engines in a fixed rotation and in order, so
// neighbouring tiles should cost the same: with n-tiles innermost a ragged
// last m-tile is a run of equally cheap tiles (with m-tiles innermost, full
// and nearly empty tiles alternate and half the engines get all the full
// ones).  The m-tiles that share one weight tile still run within one
// window of the XCD's CUs (the weight tile comes from L2 the second time),
// and an A tile is reused by consecutive n-tiles.  Four waves per workgroup;
// each wave owns MI x NJ MFMA blocks of 32 x 32.
#include "gemm_common.h"

namespace nvfp4 {

constexpr int BN = 256, BK = 32;

// 32-channel chunks of a padded compensation width
__host__ __device__ constexpr int nchunk_of(int kcp) { return kcp / 32; }

// LDS bytes of the epilogue staging (four waves), and the offset of the
// scatter epilogue's row weights: past the K-loop region (loop_end bytes) and
// the staging.
template <int NJ>
__host__ __device__ constexpr size_t epilogue_lds_bytes() { return (size_t)4 * epilogue_wave_floats<NJ>() * 4; }
__host__ __device__ constexpr size_t rw_offset(size_t loop_end, size_t epi_end) {
  return ((loop_end > epi_end ? loop_end : epi_end) + 15) / 16 * 16;
}

template <int V>
struct IntC {
  static constexpr int value = V;
};
constexpr int NSTAGE = 2;                   // LDS stages of raw NVFP4 tiles
constexpr int MAX_KC = 128;                 // largest compensated channel count handled

struct RowLoad {                            // one row's K-step: 32 codes + 2 scale bytes
  u32x4 codes;
  uint32_t scales;
};

// The E4M3 scale byte b (bits 0..7 of the argument) as fp16 in both halves.
__device__ __forceinline__ f16x2 e4m3_f16x2(uint32_t b) {
  const f16x2 v = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(b, 1.0f, false);
  return f16x2{v[0], v[0]};
}

// Two fp16x8 fragments (substeps 0 and 1) from 16 codes (8 bytes) and the
// block scale s: element i is the code of nibble i (low nibble first).
__device__ __forceinline__ void dequant16(u32x2 c, f16x2 s, f16x8& f0, f16x8& f1) {
#define NVFP4_CVT(w, sel) (__builtin_amdgcn_cvt_scalef32_pk_f16_fp4((w), 1.0f, (sel)) * s)
  const f16x2 v0 = NVFP4_CVT(c[0], 0), v1 = NVFP4_CVT(c[0], 1), v2 = NVFP4_CVT(c[0], 2),
              v3 = NVFP4_CVT(c[0], 3), v4 = NVFP4_CVT(c[1], 0), v5 = NVFP4_CVT(c[1], 1),
              v6 = NVFP4_CVT(c[1], 2), v7 = NVFP4_CVT(c[1], 3);
#undef NVFP4_CVT
  f0 = f16x8{v0[0], v0[1], v1[0], v1[1], v2[0], v2[1], v3[0], v3[1]};
  f1 = f16x8{v4[0], v4[1], v5[0], v5[1], v6[0], v6[1], v7[0], v7[1]};
}

// One fp16x8 fragment half from 8 codes (4 bytes) and the block scale.
__device__ __forceinline__ f16x8 dequant8(uint32_t w, f16x2 s) {
#define NVFP4_CVT(sel) (__builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, (sel)) * s)
  const f16x2 v0 = NVFP4_CVT(0), v1 = NVFP4_CVT(1), v2 = NVFP4_CVT(2), v3 = NVFP4_CVT(3);
#undef NVFP4_CVT
  return f16x8{v0[0], v0[1], v1[0], v1[1], v2[0], v2[1], v3[0], v3[1]};
}

// LDS layout of one pipeline stage for a BM-row A tile and the BN-row W tile.
template <int BM>
struct StageLayout {
  static constexpr int AR = BM < 256 ? BM + 1 : BM;
  static constexpr int A_CODES = 0;
  static constexpr int A_SC = AR * 16;
  static constexpr int B_CODES = (A_SC + AR * 2 + 15) / 16 * 16;
  static constexpr int B_SC = B_CODES + BN * 16;
  static constexpr int BYTES = (B_SC + BN * 2 + 15) / 16 * 16;
};

// The 32-row tile (MI = WM = 1) streams W with little reuse (a decode batch
// gives each expert a few rows), so it is bound by the memory system rather
// than the matrix cores, and it moves 128 K per pipeline stage instead of 32:
// four lanes load one row's 64 contiguous code bytes (one 64-byte request
// where the 32-wide stage needs four 16-byte ones, plus as many for the scale
// bytes), and there is one barrier per 128 K.  LDS row: 64 code bytes then
// the 8 scale bytes of its blocks; the 72-byte row stride makes the 8-byte
// fragment reads of 32 consecutive rows conflict-free.
template <int MI, int WM>
struct MacroTile {
  static constexpr bool on = MI == 1 && WM == 1;
};
template <int BM>
struct MacroLayout {
  static constexpr int KM = 128;              // K per stage
  static constexpr int ROW = 72;
  static constexpr int A_OFF = 0;             // A rows [BM + 1] (row BM: the spare)
  static constexpr int B_OFF = (BM + 1) * ROW;
  static constexpr int BYTES = (B_OFF + BN * ROW + 15) / 16 * 16;
};
template <int MI, int WM>
__host__ __device__ constexpr int stage_bytes() {
  return MacroTile<MI, WM>::on ? MacroLayout<WM * MI * 32>::BYTES : StageLayout<WM * MI * 32>::BYTES;
}

// EPI: the epilogue (0 F32, 1 SwiGLU bf16, 2 scatter rows), fixed per kernel.
template <int MI, int NJ, int WM, int WN, int EPI>
__global__ __launch_bounds__(256, 1) void grouped_gemm_kernel(GemmArgs p, int ntiles) {
  constexpr int BM = WM * MI * 32;
  static_assert(WN * NJ * 32 == BN, "N tile");
  static_assert(WM * WN == 4, "four waves");
  // LDS: NSTAGE x {A codes [AR][16 B], A scales [AR][2 B], B codes [BN][16 B],
  // B scales [BN][2 B]}, then the fp16 W_S buffer, the selected channels and
  // their K-step ranges.  AR = BM + 1 when BM < 256: threads past BM write
  // their A data into the spare row, so staging has no branch.
  using L = StageLayout<BM>;
  constexpr int A_CODES = L::A_CODES, A_SC = L::A_SC, B_CODES = L::B_CODES, B_SC = L::B_SC;
  constexpr bool kMacro = MacroTile<MI, WM>::on;
  constexpr int STAGE = stage_bytes<MI, WM>();
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  _Float16* WS = reinterpret_cast<_Float16*>(smem + NSTAGE * STAGE);   // [BN][ws_stride]

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int wm = wave / WN, wn = wave % WN;
  const int half = lane >> 5, l32 = lane & 31;

  // XCD x = blockIdx % 8 takes the logical tiles [x * per_xcd, (x + 1) * per_xcd)
  // of the T real ones (per_xcd = ceil(T / 8)); the grid, a multiple of 8 and
  // at least T, leaves surplus workgroups that exit here.
  const int real = (int)count_mtiles<BM>(p) * ntiles;
  const int per_xcd = (real + 7) / 8;
  const int jt = (int)blockIdx.x / 8;
  const int logical = ((int)blockIdx.x % 8) * per_xcd + jt;
  if (jt >= per_xcd || logical >= real) return;     // uniform over the workgroup
  const TileCoord tc = locate_tile<BM>(p, ntiles, logical);
  const int e = tc.e, n_tile = tc.n_tile, rows_valid = tc.rows_valid;
  const int64_t row0 = tc.row0;

  const int64_t K = p.K;
  const int nsteps = (int)(K / BK);
  const bool comp = p.sel_idx != nullptr;
  const int kc = comp ? p.kc : 0;
  const int kcp = (kc + BK - 1) / BK * BK;                   // padded to whole K-steps
  const int ws_stride = kcp + 8;
  int32_t* sel = reinterpret_cast<int32_t*>(WS + (comp ? BN * ws_stride : 0));   // [MAX_KC]
  int32_t* jr = sel + MAX_KC;                                                   // [nsteps + 1]
  // Q(R_S) rows of the tile: chunk c of 32 compact channels at c * BM * 18
  // bytes, codes [BM][16 B] then scales [BM][2 B]
  unsigned char* RS = reinterpret_cast<unsigned char*>(
      (reinterpret_cast<uintptr_t>(jr + nsteps + 1) + 15) & ~static_cast<uintptr_t>(15));
  // scatter epilogue: row_weight of the tile's rows [BM] (0 past the group),
  // past both the K-loop region and the epilogue's staging (which it outlives)
  float* RW = reinterpret_cast<float*>(
      smem + rw_offset((size_t)(RS - smem) + (comp ? (size_t)nchunk_of(kcp) * BM * 18 : 0),
                       epilogue_lds_bytes<NJ>()));


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
  const int64_t b_row = weight_row<BN>(p, n_tile, tid);
  const bool b_ok = b_row >= 0;
  const uint8_t* b_cp = p.w_codes + ((int64_t)e * p.N + (b_ok ? b_row : 0)) * (K / 2);
  const uint8_t* b_sp = p.w_scales + ((int64_t)e * p.N + (b_ok ? b_row : 0)) * (K / 16);
  // A row outside the tile or with an index outside [0, a_rows) gets zero
  // scales (so it reads as zeros); a W row past N keeps row 0's data: those
  // output columns are never stored.
  const uint32_t a_mask = a_ok ? 0xFFFFu : 0u;

  auto load_step = [&](int s, RowLoad& ta, RowLoad& tb) {
    ta.codes = *reinterpret_cast<const u32x4*>(a_cp + s * (BK / 2));
    ta.scales = *reinterpret_cast<const uint16_t*>(a_sp + s * (BK / 16));
    tb.codes = *reinterpret_cast<const u32x4*>(b_cp + s * (BK / 2));
    tb.scales = *reinterpret_cast<const uint16_t*>(b_sp + s * (BK / 16));
  };

  auto stage_write = [&](int st, const RowLoad& ta, const RowLoad& tb) {
    unsigned char* base = smem + st * STAGE;
    const int a_slot = tid < BM ? tid : BM;                   // BM: the spare row
    *reinterpret_cast<u32x4*>(base + A_CODES + a_slot * 16) = ta.codes;
    *reinterpret_cast<uint16_t*>(base + A_SC + a_slot * 2) = (uint16_t)(ta.scales & a_mask);
    *reinterpret_cast<u32x4*>(base + B_CODES + tid * 16) = tb.codes;
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
    // jr[s]: the first j with sel[j] in pipeline stage s or later
    constexpr int KSTEP = kMacro ? MacroLayout<BM>::KM : BK;
    const int nst = kMacro ? (int)((K + KSTEP - 1) / KSTEP) : nsteps;
    for (int s = tid; s <= nst; s += 256) {
      int lo = 0, hi = kc;
      while (lo < hi) {
        int mid = (lo + hi) >> 1;
        if (sel[mid] < s * KSTEP) lo = mid + 1; else hi = mid;
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

  // A wave's dequantized fragments of one K-step: a0/b0 feed MFMA substep 0,
  // a1/b1 substep 1.
  struct Frags {
    f16x8 a0[MI], a1[MI], b0[NJ], b1[NJ];
  };
  auto read_frags = [&](int st, Frags& f) {
    const unsigned char* base = smem + st * STAGE;
#pragma unroll
    for (int i = 0; i < MI; ++i) {
      const int r = wm * MI * 32 + i * 32 + l32;
      const u32x2 c = *reinterpret_cast<const u32x2*>(base + A_CODES + r * 16 + half * 8);
      dequant16(c, e4m3_f16x2(base[A_SC + r * 2 + half]), f.a0[i], f.a1[i]);
    }
#pragma unroll
    for (int j = 0; j < NJ; ++j) {
      const int r = wn * NJ * 32 + j * 32 + l32;
      const u32x2 c = *reinterpret_cast<const u32x2*>(base + B_CODES + r * 16 + half * 8);
      dequant16(c, e4m3_f16x2(base[B_SC + r * 2 + half]), f.b0[j], f.b1[j]);
    }
  };
  auto mfma_step = [&](const Frags& f) {
#pragma unroll
    for (int j = 0; j < NJ; ++j)
#pragma unroll
      for (int i = 0; i < MI; ++i)
        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(f.a0[i], f.b0[j], acc[i][j], 0, 0, 0);
#pragma unroll
    for (int j = 0; j < NJ; ++j)
#pragma unroll
      for (int i = 0; i < MI; ++i)
        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(f.a1[i], f.b1[j], acc[i][j], 0, 0, 0);
  };

  // W elements of the selected channels inside K-step s (LDS stage st) into
  // W_S: thread t handles weight row t of the tile, so the loop count is the
  // same for every thread.
  auto gather_ws = [&](int s, int st) {
    const unsigned char* base = smem + st * STAGE;
    const int j1 = jr[s + 1];
    for (int jj = jr[s]; jj < j1; ++jj) {
      const int kk = sel[jj] - s * BK;                       // 0..31 inside the step
      const uint32_t byte = base[B_CODES + tid * 16 + (kk >> 1)] >> (4 * (kk & 1));
      const f16x2 v = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(byte, 1.0f, 0);
      const f16x2 sc = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(base[B_SC + tid * 2 + (kk >> 4)], 1.0f, false);
      WS[tid * ws_stride + jj] = v[0] * sc[0];               // exact: see the header
    }
  };

  // ---- 128-K pipeline of the 32-row tile (MacroTile) -----------------------
  // Stage m covers K [128 m, 128 m + 128): code bytes [64 m, 64 m + 64) and
  // scale bytes [8 m, 8 m + 8) of every row.  Thread t loads the 16 code bytes
  // 16 (t % 4) .. of W rows t / 4 + 64 i (i = 0..3) and of A row t / 4, and
  // the 8 scale bytes of W row t and A row t; threads past the tile's A rows
  // load row 0 and write the spare LDS row.  When K is not a multiple of 128
  // the last stage is half full: its missing code bytes are read from the
  // row's start and its missing blocks get scale 0 in A and W, so they add
  // nothing.  Two LDS stages and two register sets: in stage m a wave reads
  // its raw fragments of stage m, writes the data of stage m + 1 into the
  // other LDS stage and issues the loads of stage m + 3 into the register set
  // just written, so loads have two stages (256 K) to arrive.
  //
  // K order of one stage: MFMA substep q (0..7) takes, in lane half h, the 8
  // codes 8 (q % 4) .. of 16-byte granule 2 (q / 4) + h (granule G holds
  // blocks 2G and 2G + 1), the same in A and W, so every k of the stage is
  // summed once.
  auto macro_loop = [&](auto&& park) {
    using ML = MacroLayout<BM>;
    constexpr int KM = ML::KM, ROW = ML::ROW, AO = ML::A_OFF, BO = ML::B_OFF;
    typedef uint32_t u32x2a __attribute__((ext_vector_type(2), aligned(4)));
    const int nmac = (int)((K + KM - 1) / KM);
    const int mlast = nmac - 1;
    const bool half_last = (K % KM) != 0;
    const int g4 = tid & 3;
    const int64_t rbytes = K / 2;
    int64_t ac = 0;                            // A row of the code loads: tile row tid / 4
    if ((tid >> 2) < rows_valid) {
      const int64_t ur = row0 + (tid >> 2);
      ac = p.a_row_index ? (int64_t)p.a_row_index[ur] : ur;
      if (ac < 0 || ac >= p.a_rows) ac = 0;    // its scales (row tid / 4's) are zero
    }
    const uint8_t* a_cm = p.a_codes + ac * rbytes + g4 * 16;
    const uint8_t* b_cm[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int64_t br = weight_row<BN>(p, n_tile, i * 64 + (tid >> 2));
      b_cm[i] = p.w_codes + ((int64_t)e * p.N + (br >= 0 ? br : 0)) * rbytes + g4 * 16;
    }
    const uint32_t am32 = a_mask ? 0xFFFFFFFFu : 0u;

    struct MacLoad {
      u32x4 wc[4], ac;
      u32x2 ws, as;
    };
    auto mload = [&](int m, MacLoad& r) {
      const int64_t cb = (int64_t)m * 64;
      const int64_t co = cb + g4 * 16 < rbytes ? cb : -(int64_t)g4 * 16;   // past K: row start
      const bool part = half_last && m == mlast;
      const int64_t so = part ? (int64_t)m * 8 - 4 : (int64_t)m * 8;      // 4 valid bytes: the high half
#pragma unroll
      for (int i = 0; i < 4; ++i) r.wc[i] = *reinterpret_cast<const u32x4*>(b_cm[i] + co);
      r.ac = *reinterpret_cast<const u32x4*>(a_cm + co);
      const u32x2a ws = *reinterpret_cast<const u32x2a*>(b_sp + so);
      const u32x2a as = *reinterpret_cast<const u32x2a*>(a_sp + so);
      r.ws = part ? u32x2{ws[1], 0u} : u32x2{ws[0], ws[1]};
      r.as = part ? u32x2{as[1] & am32, 0u} : u32x2{as[0] & am32, as[1] & am32};
    };
    auto mwrite = [&](int st, const MacLoad& r) {
      unsigned char* base = smem + st * STAGE;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        unsigned char* d = base + BO + (i * 64 + (tid >> 2)) * ROW + g4 * 16;
        *reinterpret_cast<u32x2*>(d) = u32x2{r.wc[i][0], r.wc[i][1]};
        *reinterpret_cast<u32x2*>(d + 8) = u32x2{r.wc[i][2], r.wc[i][3]};
      }
      *reinterpret_cast<u32x2*>(base + BO + tid * ROW + 64) = r.ws;
      unsigned char* da = base + AO + ((tid >> 2) < BM ? (tid >> 2) : BM) * ROW + g4 * 16;
      *reinterpret_cast<u32x2*>(da) = u32x2{r.ac[0], r.ac[1]};
      *reinterpret_cast<u32x2*>(da + 8) = u32x2{r.ac[2], r.ac[3]};
      *reinterpret_cast<u32x2*>(base + AO + (tid < BM ? tid : BM) * ROW + 64) = r.as;
    };
    // A fragment row's raw data of a stage: granules h and 2 + h, and the
    // scale pairs of their blocks as fp16 ({2h, 2h+1} and {4+2h, 5+2h})
    struct RawRow {
      u32x2 g0a, g0b, g1a, g1b;
      f16x2 s0, s1;
    };
    auto read_raw = [&](const unsigned char* row, RawRow& o) {
      o.g0a = *reinterpret_cast<const u32x2*>(row + half * 16);
      o.g0b = *reinterpret_cast<const u32x2*>(row + half * 16 + 8);
      o.g1a = *reinterpret_cast<const u32x2*>(row + 32 + half * 16);
      o.g1b = *reinterpret_cast<const u32x2*>(row + 32 + half * 16 + 8);
      const u32x2 sc = *reinterpret_cast<const u32x2*>(row + 64);
      o.s0 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(sc[0] >> (16 * half), 1.0f, false);
      o.s1 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(sc[1] >> (16 * half), 1.0f, false);
    };
    auto frag_q = [&](const RawRow& o, int q) {
      const u32x2 g = q < 4 ? ((q & 2) ? o.g0b : o.g0a) : ((q & 2) ? o.g1b : o.g1a);
      const f16x2 sp = q < 4 ? o.s0 : o.s1;
      const _Float16 sv = (q & 2) ? sp[1] : sp[0];
      return dequant8(g[q & 1], f16x2{sv, sv});
    };
    auto gather_ws_m = [&](int m, int st) {
      const unsigned char* row = smem + st * STAGE + BO + tid * ROW;
      const int j1 = jr[m + 1];
      for (int jj = jr[m]; jj < j1; ++jj) {
        const int kk = sel[jj] - m * KM;                      // 0..127 inside the stage
        const uint32_t byte = row[kk >> 1] >> (4 * (kk & 1));
        const f16x2 v = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(byte, 1.0f, 0);
        const f16x2 sc = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(row[64 + (kk >> 4)], 1.0f, false);
        WS[tid * ws_stride + jj] = v[0] * sc[0];
      }
    };
    auto mstep = [&](int m, int st, MacLoad& rset) {
      const unsigned char* base = smem + st * STAGE;
      RawRow ra_, rb_[NJ];
      read_raw(base + AO + l32 * ROW, ra_);
#pragma unroll
      for (int j = 0; j < NJ; ++j) read_raw(base + BO + (wn * NJ * 32 + j * 32 + l32) * ROW, rb_[j]);
      if (comp) gather_ws_m(m, st);
      mwrite(st ^ 1, rset);                     // data of stage m + 1
      mload(m + 3 < nmac ? m + 3 : mlast, rset);
#pragma unroll
      for (int q = 0; q < 8; ++q) {
        const f16x8 fa = frag_q(ra_, q);
#pragma unroll
        for (int j = 0; j < NJ; ++j)
          acc[0][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(fa, frag_q(rb_[j], q), acc[0][j], 0, 0, 0);
      }
    };

    MacLoad R0, R1;
    mload(0, R0);
    mload(1 < nmac ? 1 : mlast, R1);
    park();
    mwrite(0, R0);
    mload(2 < nmac ? 2 : mlast, R0);
    lds_barrier();
    int m = 0;
    for (; m + 2 <= nmac; m += 2) {
      mstep(m, 0, R1);
      lds_barrier();
      mstep(m + 1, 1, R0);
      lds_barrier();
    }
    if (m < nmac) {
      mstep(m, 0, R1);
      lds_barrier();
    }
  };

  // ---- main K loop ----------------------------------------------------------
  // Step s: MFMAs on the fragments of step s (registers), while the fragments
  // of step s+1 are read from LDS stage (s+1)%2 and dequantized (and the
  // selected W columns of step s+1 copied into W_S), the raw data of step s+2
  // goes from register set s%PD into stage s%2 and the loads of step s+2+PD
  // are issued into that set: PD K-steps between a load and its use.  Small
  // tiles (BM <= 64) have short K-steps, so they keep more loads in flight
  // (PD = 4) to cover the memory latency; large tiles use PD = 2.
  // One barrier per step: it orders this step's writes of stage s%2 before
  // the next step's reads of it, and this step's reads of stage (s+1)%2
  // before the next step's writes.  Every load is issued unconditionally (a step past
  // the end re-reads the last step; its stage is never read), so the compiler
  // waits only for the older step's loads.  K is a multiple of 64, so nsteps
  // is even and at least 2, and the loop, unrolled by PD (plus two steps when
  // nsteps % PD == 2), sees each stage and register set at a fixed place.
  constexpr int PD = BM <= 64 ? 4 : 2;
  RowLoad ra[PD], rb[PD];
  const int last = nsteps - 1;
  // The Q(R_S) rows are loaded with the first K-steps (loads complete in
  // order, so they are in once steps 0 and 1 are) and parked in LDS before
  // the K loop: the compensation chunk after it waits for no global memory.
  constexpr int kMaxChunks = MAX_KC / BK;
  const int nchunk = nchunk_of(kcp);
  u32x4 rq_codes[kMaxChunks];
  uint32_t rq_sc[kMaxChunks];
  if (comp) {
    const bool ok = tid < rows_valid;
    const int64_t ur = row0 + (ok ? tid : 0);
#pragma unroll
    for (int c = 0; c < kMaxChunks; ++c) {
      rq_codes[c] = u32x4{0, 0, 0, 0};
      rq_sc[c] = 0;
#pragma unroll
      for (int q = 0; q < 2; ++q) {
        const int j = c * BK + q * 16;
        if (ok && j < kc) {
          const u32x2 w = *reinterpret_cast<const u32x2*>(p.r_codes + ur * (kc / 2) + j / 2);
          rq_codes[c][2 * q] = w[0];
          rq_codes[c][2 * q + 1] = w[1];
          rq_sc[c] |= (uint32_t)p.r_scales[ur * (kc / 16) + j / 16] << (8 * q);
        }
      }
    }
  }
  float rw = 0.0f;
  if (EPI == 2 && tid < rows_valid) rw = p.row_weight[row0 + tid];
  auto park_rows = [&]() {                    // row weights and Q(R_S) rows into LDS
    if (EPI == 2 && tid < BM) RW[tid] = rw;
    if (comp && tid < BM) {
#pragma unroll
      for (int c = 0; c < kMaxChunks; ++c) {
        if (c < nchunk) {
          *reinterpret_cast<u32x4*>(RS + c * (BM * 18) + tid * 16) = rq_codes[c];
          *reinterpret_cast<uint16_t*>(RS + c * (BM * 18) + BM * 16 + tid * 2) = (uint16_t)rq_sc[c];
        }
      }
    }
  };
  if constexpr (kMacro) {
    macro_loop(park_rows);
  } else {
  load_step(0, ra[0], rb[0]);
  load_step(1, ra[1], rb[1]);
  stage_write(0, ra[0], rb[0]);
  stage_write(1, ra[1], rb[1]);
  park_rows();
  load_step(2 < last ? 2 : last, ra[0], rb[0]);
#pragma unroll
  for (int i = 1; i < PD; ++i) {
    __builtin_amdgcn_sched_barrier(0);        // keep the loop's load order in the prologue
    load_step(2 + i < last ? 2 + i : last, ra[i], rb[i]);
  }
  lds_barrier();
  if (comp) gather_ws(0, 0);

  auto main_loop = [&](auto ma_c) {
  constexpr int MA = decltype(ma_c)::value;
  // fragment f of the step is read and dequantized only if some MFMA uses it
  auto frag_live = [&](int f) { return f < MI ? f < MA : MA > 0; };
  Frags fr[2];
  {
    const unsigned char* base = smem;                          // stage 0: fragments of step 0
#pragma unroll
    for (int i = 0; i < MI; ++i) {
      if (i >= MA) continue;
      const int r = wm * MI * 32 + i * 32 + l32;
      const u32x2 c = *reinterpret_cast<const u32x2*>(base + A_CODES + r * 16 + half * 8);
      dequant16(c, e4m3_f16x2(base[A_SC + r * 2 + half]), fr[0].a0[i], fr[0].a1[i]);
    }
#pragma unroll
    for (int j = 0; j < NJ; ++j) {
      if (MA == 0) continue;
      const int r = wn * NJ * 32 + j * 32 + l32;
      const u32x2 c = *reinterpret_cast<const u32x2*>(base + B_CODES + r * 16 + half * 8);
      dequant16(c, e4m3_f16x2(base[B_SC + r * 2 + half]), fr[0].b0[j], fr[0].b1[j]);
    }
  }
  // Step 0 overwrites stage 0 (with the data of step 2) once every wave has
  // read its step-0 fragments from it; waves with fewer live fragments get
  // there sooner.
  lds_barrier();

  // One K-step in issue order: the MFMAs of this step one at a time, and
  // between them (each group fenced off from the scheduler) the rest of the
  // step's work: the LDS reads of the next step's fragments right after MFMA
  // 0, the stage writes after MFMA 1, the global loads after MFMA 2, and the
  // dequantization of the next step's fragments, half a fragment (8 VALU
  // instructions, about one MFMA's duration) per MFMA from MFMA kDeq0 on.
  constexpr int kFr = MI + NJ;                // fragments per wave and step
  constexpr int kMf = 2 * MI * NJ;            // MFMAs per wave and step
  constexpr int kDeq0 = kMf > 8 ? 4 : 3;
  auto step = [&](int s, int st, const Frags& cur, Frags& nxt, RowLoad& ta, RowLoad& tb) {
    const unsigned char* nb = smem + (st ^ 1) * STAGE;       // stage of step s+1
    u32x2 rc[kFr];
    uint32_t rs[kFr];
    f16x2 sc[kFr];
#pragma unroll
    for (int m = 0; m < kMf; ++m) {
      __builtin_amdgcn_sched_barrier(0);
      {
        const int sub = m / (MI * NJ), j = (m % (MI * NJ)) / MI, i = m % MI;
        if (i < MA)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(sub ? cur.a1[i] : cur.a0[i],
                                                             sub ? cur.b1[j] : cur.b0[j],
                                                             acc[i][j], 0, 0, 0);
      }
      if (m == 0) {
#pragma unroll
        for (int f = 0; f < kFr; ++f) {
          if (!frag_live(f)) continue;
          const int r = f < MI ? wm * MI * 32 + f * 32 + l32 : wn * NJ * 32 + (f - MI) * 32 + l32;
          const int co = f < MI ? A_CODES : B_CODES, so = f < MI ? A_SC : B_SC;
          rc[f] = *reinterpret_cast<const u32x2*>(nb + co + r * 16 + half * 8);
          rs[f] = nb[so + r * 2 + half];
        }
      }
      if (m == 1) stage_write(st, ta, tb);                    // data of step s+2
      if (m == 2) load_step(s + 2 + PD < last ? s + 2 + PD : last, ta, tb);
      if (m >= kDeq0 || kMf <= kDeq0) {
#pragma unroll
        for (int hf = 0; hf < 2 * kFr; ++hf) {
          const int at = kMf <= kDeq0 ? kMf - 1 : kDeq0 + hf * (kMf - kDeq0) / (2 * kFr);
          if (at != m) continue;
          const int f = hf >> 1, h = hf & 1;
          if (!frag_live(f)) continue;
          // The empty asm statements fix this work to this slot: inputs pass
          // through one before it (nothing is hoisted to its loads), outputs
          // after it (nothing is sunk to its use).
          uint32_t w = rc[f][h];
          asm volatile("" : "+v"(w));
          if (h == 0) {
            uint32_t b = rs[f];
            asm volatile("" : "+v"(b));
            sc[f] = e4m3_f16x2(b);
            asm volatile("" : "+v"(sc[f]));
          }
          f16x8 v = dequant8(w, sc[f]);
          asm volatile("" : "+v"(v));
          if (f < MI) {
            if (h == 0) nxt.a0[f] = v; else nxt.a1[f] = v;
          } else {
            if (h == 0) nxt.b0[f - MI] = v; else nxt.b1[f - MI] = v;
          }
        }
      }
    }
    __builtin_amdgcn_sched_barrier(0);
    if (comp && s + 1 < nsteps) gather_ws(s + 1, st ^ 1);
  };
  int s = 0;
  for (; s + PD <= nsteps; s += PD) {
    step(s, 0, fr[0], fr[1], ra[0], rb[0]);
    lds_barrier();
    step(s + 1, 1, fr[1], fr[0], ra[1], rb[1]);
    lds_barrier();
    if constexpr (PD == 4) {
      step(s + 2, 0, fr[0], fr[1], ra[2], rb[2]);
      lds_barrier();
      step(s + 3, 1, fr[1], fr[0], ra[3], rb[3]);
      lds_barrier();
    }
  }
  if constexpr (PD == 4) {
    if (s < nsteps) {                          // nsteps % 4 == 2
      step(s, 0, fr[0], fr[1], ra[0], rb[0]);
      lds_barrier();
      step(s + 1, 1, fr[1], fr[0], ra[1], rb[1]);
      lds_barrier();
    }
  }
  };
  // The number of this wave's 32-row A fragments that hold rows of the tile
  // (0 .. MI): a ragged last m-tile of an expert skips the MFMAs and the
  // dequantization of its empty fragments (a wave with none skips its W
  // fragments too), with the loop specialized for each count.
  // The count is the same for every lane of the wave; readfirstlane makes
  // that visible to the compiler, so the switch is a scalar branch (a
  // lane-divergent branch around loops holding barriers would be undefined).
  const int ma_rows = rows_valid - wm * MI * 32;
  const int ma = __builtin_amdgcn_readfirstlane(
      ma_rows <= 0 ? 0 : (ma_rows >= MI * 32 ? MI : (ma_rows + 31) / 32));
  switch (ma) {
    case 0: main_loop(IntC<0>{}); break;
    case 1: main_loop(IntC<1>{}); break;
    case 2: if constexpr (MI >= 2) main_loop(IntC<2>{}); break;
    case 3: if constexpr (MI >= 3) main_loop(IntC<3>{}); break;
    default: main_loop(IntC<MI>{}); break;
  }
  }

  // ---- compensation chunk ---------------------------------------------------
  const float ga = p.a_global[p.a_global_per_group ? e : 0];
  float scale = ga * p.w_global[e];
  if (comp) {
    const float gr = p.r_global[e];
    const float ratio = ga / gr;
#pragma unroll
    for (int i = 0; i < MI; ++i)
#pragma unroll
      for (int j = 0; j < NJ; ++j)
#pragma unroll
        for (int q = 0; q < 16; ++q) acc[i][j][q] = acc[i][j][q] * ratio;
    scale = gr * p.w_global[e];
    // Q(R_S) x W_S over the compact channels (Q(R_S) parked in RS before
    // the K loop, W_S gathered during it)
    for (int c = 0; c < nchunk; ++c) {
      const unsigned char* base = RS + c * (BM * 18);
      Frags f;
#pragma unroll
      for (int i = 0; i < MI; ++i) {
        const int r = wm * MI * 32 + i * 32 + l32;
        const u32x2 cc = *reinterpret_cast<const u32x2*>(base + r * 16 + half * 8);
        dequant16(cc, e4m3_f16x2(base[BM * 16 + r * 2 + half]), f.a0[i], f.a1[i]);
      }
#pragma unroll
      for (int j = 0; j < NJ; ++j) {            // W_S in the same K order: block half of the chunk
        const int r = wn * NJ * 32 + j * 32 + l32;
        f.b0[j] = *reinterpret_cast<const f16x8*>(WS + r * ws_stride + c * BK + half * 16);
        f.b1[j] = *reinterpret_cast<const f16x8*>(WS + r * ws_stride + c * BK + half * 16 + 8);
      }
      mfma_step(f);
    }
  }

  __syncthreads();                             // LDS free for the epilogue staging
  gemm_epilogue<MI, NJ, BN, EPI>(p, acc, tc, wm * MI * 32, wn * NJ * 32, scale,
                            reinterpret_cast<float*>(smem) + wave * epilogue_wave_floats<NJ>(), RW);
}

template <int MI, int NJ, int WM, int WN, int EPI>
static hipError_t launch_cfg(const GemmArgs& a, hipStream_t stream) {
  constexpr int BM = WM * MI * 32;
  const int64_t mtiles = (a.rows_total + BM - 1) / BM + a.E;
  const int64_t ntiles = a.epilogue == 1 ? (a.N / 2 + BN / 2 - 1) / (BN / 2) : (a.N + BN - 1) / BN;
  const int64_t total = mtiles * ntiles;
  const int kcp = a.sel_idx ? (a.kc + BK - 1) / BK * BK : 0;
  const size_t stage = stage_bytes<MI, WM>();
  const size_t loop_lds = NSTAGE * stage + (a.sel_idx ? (size_t)BN * (kcp + 8) * 2 : 0) +
                          ((size_t)(MAX_KC + a.K / BK + 1) * 4 + 15) / 16 * 16 +
                          (a.sel_idx ? (size_t)nchunk_of(kcp) * BM * 18 : 0);
  const size_t epi_lds = epilogue_lds_bytes<NJ>();
  const size_t lds = EPI == 2 ? rw_offset(loop_lds, epi_lds) + (size_t)BM * 4
                              : (loop_lds > epi_lds ? loop_lds : epi_lds);
  auto kern = grouped_gemm_kernel<MI, NJ, WM, WN, EPI>;
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

// Rows per m-tile from the average rows per expert.  The last m-tile of an
// expert is ragged; its empty 32-row fragments cost no MFMAs and no A
// dequantization, so large tiles (which dequantize fewer W elements per MFMA)
// pay off from about 160 rows per expert.
int grouped_gemm_block_m(int64_t rows_total, int32_t E) {
  const int64_t avg = E > 0 ? rows_total / E : rows_total;
  if (avg >= 160) return 256;
  if (avg >= 64) return 128;
  if (avg >= 24) return 64;
  return 32;
}

hipError_t launch_grouped_gemm(const GemmArgs& a, hipStream_t stream) {
  if (a.epilogue == 1 && a.out_amax) {
    hipError_t err = launch_fill_f32(a.out_amax, 1, 0.0f, stream);
    if (err != hipSuccess) return err;
  }
  if (a.rows_total == 0) return hipSuccess;
  hipError_t err;
  const int bm = a.block_m > 0 ? a.block_m : grouped_gemm_block_m(a.rows_total, a.E);
  switch (bm) {
    case 256: err = launch_epi<4, 4, 2, 2>(a, stream); break;
    case 128: err = launch_epi<2, 4, 2, 2>(a, stream); break;
    case 64: err = launch_epi<1, 4, 2, 2>(a, stream); break;
    // the 32-row tile moves 128 K per stage: K = 64 takes the 64-row tile
    default: err = a.K >= 128 ? launch_epi<1, 2, 1, 4>(a, stream) : launch_epi<1, 4, 2, 2>(a, stream); break;
  }
  if (err != hipSuccess || a.epilogue != 2) return err;
  return launch_combine(a.y_rows, a.rows_total, a.N, a.scatter_index, a.out_rows,
                        static_cast<float*>(a.out), a.ldo, a.y_rows, stream);
}

}  // namespace nvfp4
