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
// hardware FP8 -> fp16 convert), both exact: one VALU instruction per
// element.  The MFMA is v_mfma_f32_32x32x16_f16 with fp32 accumulation; the
// global scales are applied after the K loop.  A wave owns 128 x 128 outputs
// (MI = NJ = 4 blocks of 32 x 32) in the large tiles, so it dequantizes 8
// fragments for every 16 MFMAs: about 4 VALU instructions per MFMA, which
// gfx950 issues while the matrix core works (a SIMD overlaps independent
// VALU work with an f16 MFMA up to about that rate, measured).
//
// Data path (per 256-thread workgroup, one tile of BM rows x 256 weight rows):
// K moves 128 per pipeline stage through a ring of NSLOT LDS slots, filled by
// direct global-to-LDS loads (global_load_lds_dwordx4 / _dword: lane l of an
// instruction writes 16 / 4 bytes at base + 16 l / 4 l, so no registers carry
// the tiles).  A slot holds, for every A row and W row, the stage's 64 code
// bytes (16-byte chunks swizzled within a row: chunk c of row r at position
// c ^ ((r >> 1) & 3), so that the fragment reads of 8 consecutive rows hit
// distinct banks) and its 8 scale bytes as two words, stored in the order the
// fragment reads want them.  Every wave issues the same number of load
// instructions per stage (padding ones go to a dummy area), so one vmcnt wait
// tells it that its share of a stage has landed.
//
// K order inside a stage: lane half h takes chunks h*2 + t (t = 0, 1), i.e.
// the 64 K-values of scale word h, and MFMA substep q = 4 t + u (u = 0..3)
// takes the u-th 8 codes of chunk 2h + t from every lane: 16 K-values per
// substep, 128 per stage, the same order in A and W, so the sum over the
// stage is unchanged.  A lane's scale word then holds exactly its four
// blocks, and the FP8 convert's word select (t) picks the pair it needs
// without a shift.
//
// Per stage s a wave holds the stage's raw fragments in registers (read from
// LDS during stage s - 1) and runs its 8 substeps; during substep q it issues
// the 16 MFMAs of q and dequantizes the fragments of q + 1.  At substep 3
// (raw chunk-0 registers consumed) it waits for its loads of stage s + 1,
// meets the other waves at the stage's one barrier, issues the loads of stage
// s + NSLOT into the slot stage s used, and reads the chunk-0 fragments and
// scale words of stage s + 1; at substep 7 the chunk-1 fragments.  A slot is
// therefore refilled only after every wave passed the barrier that followed
// its last read, and loads have NSLOT - 1 stages to land.
//
// Compensation: while the K loop streams the expert's weight tile through
// the slots, each thread copies the elements of the selected columns of its
// weight row into an fp16 W_S [BN, kc] buffer (exact), so W is read once.
// The Q(R_S) codes of the tile's rows come into LDS by direct loads issued
// ahead of the stages, their scale bytes into registers.  After the loop each
// 32 x 32 block's correction is accumulated separately (kc / 16 MFMAs) and
// combined as acc * gA gW + corr * gR gW, so no ratio of global scales can
// overflow.
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
// owns a contiguous eighth of the real tiles.  Inside an XCD the workgroups go
// to its shader engines in a fixed rotation and in order, so neighbouring
// tiles should cost the same: with n-tiles innermost a ragged last m-tile is
// a run of equally cheap tiles.  The m-tiles that share one weight tile run
// within one window of the XCD's CUs (the weight tile comes from L2 the
// second time), and an A tile is reused by consecutive n-tiles.
#include "gemm_common.h"

#include <mutex>

namespace nvfp4 {
namespace nvg {

constexpr int BN = 256;                     // weight rows per tile
constexpr int KS = 128;                     // K per pipeline stage
constexpr int MAX_KC = 128;                 // largest compensated channel count
constexpr int DUMMY_BYTES = 1024;           // target of the padding loads

// One LDS slot: A codes [BM][64], W codes [BN][64], A scale words [2 BM],
// W scale words [2 BN].  Load instructions per stage: NA A-code blocks of 16
// rows (1 KB), NW W-code blocks, NAS / NWS scale blocks of 64 words; per wave
// the ceiling of a quarter of each.
template <int BM>
struct Layout {
  static constexpr int A_OFF = 0;
  static constexpr int B_OFF = BM * 64;
  static constexpr int AS_OFF = B_OFF + BN * 64;
  static constexpr int BS_OFF = AS_OFF + BM * 8;
  static constexpr int STAGE = BS_OFF + BN * 8;
  static constexpr int NA = BM / 16, NW = BN / 16, NAS = BM / 32, NWS = BN / 32;
  static constexpr int PA = (NA + 3) / 4, PW = (NW + 3) / 4, PAS = (NAS + 3) / 4, PWS = (NWS + 3) / 4;
  static constexpr int LPW = PA + PW + PAS + PWS;      // load instructions per wave and stage
};

__device__ __forceinline__ int swz(int r) { return (r >> 1) & 3; }

template <int V>
struct IntC {
  static constexpr int value = V;
};

// Direct global-to-LDS loads through buffer resources: the operand's base
// and byte size live in four scalar registers, the stage's advance is the
// scalar offset and each lane's position within the stage a 32-bit vector
// offset fixed for the whole tile, so a load costs no vector arithmetic.
// Lane l of an instruction writes its 16 / 4 bytes at LDS l * 16 / l * 4 past
// the (uniform) destination.  A read at or past the resource's size returns
// zeros, which is how rows with a bad index and the blocks past K of a
// half-full last stage get zero scales.
typedef __attribute__((address_space(3))) void lds_void_t;
typedef __amdgpu_buffer_rsrc_t Rsrc;
constexpr uint32_t OOB = 0x80000000u;       // vector offset past every scale array
__device__ __forceinline__ void load_lds16(Rsrc r, uint32_t voff, int soff, unsigned char* l) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void_t*)l, 16, voff, soff, 0, 0);
}
__device__ __forceinline__ void load_lds4(Rsrc r, uint32_t voff, int soff, unsigned char* l) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void_t*)l, 4, voff, soff, 0, 0);
}
// s_waitcnt vmcnt(N) lgkmcnt(0) (gfx9 encoding: vmcnt in bits 0-3 and 14-15)
template <int N>
__device__ __forceinline__ void wait_vm_lgkm0() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | 0x70 | ((N >> 4) << 14));
}

// The E4M3 bytes 2 t and 2 t + 1 of word w as fp16 (t = 0: bytes 0, 1).
template <int T>
__device__ __forceinline__ f16x2 scale_pair(uint32_t w) {
  return __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w, 1.0f, T != 0);
}

// One MFMA operand: the 8 E2M1 codes of w (low nibble first) times scale s.
__device__ __forceinline__ f16x8 dequant8(uint32_t w, _Float16 s) {
  const f16x2 ss = f16x2{s, s};
  const f16x2 v0 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 0) * ss;
  const f16x2 v1 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 1) * ss;
  const f16x2 v2 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 2) * ss;
  const f16x2 v3 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 3) * ss;
  return f16x8{v0[0], v0[1], v1[0], v1[1], v2[0], v2[1], v3[0], v3[1]};
}

// An empty asm that takes the first n registers of v: their values must
// exist at this point of the program.
template <int n, int N>
__device__ __forceinline__ void pin_regs(f16x8 (&v)[N]) {
#pragma unroll
  for (int i = 0; i < n; ++i) asm volatile("" : "+v"(v[i]));
}

// LDS bytes of the K-loop region: slots, dummy, W_S (fp16 [BN][kq*16 + 8]),
// sel [MAX_KC], the per-stage gather table [nst + 2] (16 bytes each), and the
// Q(R_S) codes [BM][kc / 2].
template <int BM, int NSLOT, int KQ>
__host__ __device__ constexpr size_t loop_lds_bytes(int64_t K) {
  return (size_t)NSLOT * Layout<BM>::STAGE + DUMMY_BYTES +
         (KQ > 0 ? (size_t)BN * (KQ * 16 + 8) * 2 + (size_t)MAX_KC * 4 : 0) +
         (((size_t)((K + KS - 1) / KS) + 2) * 16) +
         (KQ > 0 ? (size_t)BM * KQ * 8 : 0);
}

// One tile.  EPI: the epilogue (0 F32, 1 SwiGLU bf16, 2 scatter rows).  KQ:
// 0 without compensation, else the largest kc / 16 handled.  GW: selected
// channels per stage that the gather takes beside the MFMAs (4 or 8; more
// take a slower loop at the stage's end).  Inlined into the kernel: as a call
// it would take the kernel argument's address.
template <int MI, int NJ, int WM, int WN, int NSLOT, int EPI, int KQ, int GW>
__device__ __forceinline__ void gemm_tile(const GemmArgs& p, const TileCoord& tc) {
  constexpr int BM = WM * MI * 32;
  static_assert(WN * NJ * 32 == BN, "N tile");
  static_assert(WM * WN == 4, "four waves");
  using L = Layout<BM>;
  constexpr int STAGE = L::STAGE, LPW = L::LPW;
  constexpr bool COMP = KQ > 0;
  static_assert(GW == 4 || GW == 8, "gather width");
  constexpr int WSS = KQ * 16 + 8;                        // W_S row stride (halves)
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  unsigned char* DUMMY = smem + NSLOT * STAGE;
  _Float16* WS = reinterpret_cast<_Float16*>(DUMMY + DUMMY_BYTES);
  int32_t* sel = reinterpret_cast<int32_t*>(WS + (COMP ? BN * WSS : 0));
  // gather table: per stage the first selected channel j0 and their count
  // n (j0 | n << 8), then the in-stage offsets of the first eight (one byte
  // each, words 1 and 2)
  u32x4* tab = reinterpret_cast<u32x4*>(sel + (COMP ? MAX_KC : 0));
  // Q(R_S) codes of the tile's rows [BM][kc / 2], 16-byte aligned, after tab
  unsigned char* RSC = reinterpret_cast<unsigned char*>(tab + ((p.K + KS - 1) / KS) + 2);
  float* RW = reinterpret_cast<float*>(smem + p.rw_lds_offset);

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // uniform: LDS targets in SGPRs
  const int wm = wave / WN, wn = wave % WN;
  const int half = lane >> 5, l32 = lane & 31;

  const int e = tc.e, n_tile = tc.n_tile, rows_valid = tc.rows_valid;
  const int64_t row0 = tc.row0;
  const int64_t K = p.K;
  const int nst = (int)((K + KS - 1) / KS);
  const int mh = (K % KS) != 0 ? nst - 1 : -1;     // the half-full last stage, if any
  const uint32_t rbytes = (uint32_t)(K / 2), sbytes = (uint32_t)(K / 16);
  const int kc = COMP ? p.kc : 0;

  // ---- prologue ------------------------------------------------------------------
  // The global reads the set-up needs (row indexes of the tile's A rows, the
  // selected channels, the row weights) go out together, then the LDS set-up,
  // then the stage loads: few dependent memory round trips per tile.
  //
  // A unit row r of the tile reads activation row a_row(r); rows past the
  // group read row 0 (their outputs are never stored); a row index outside
  // [0, a_rows) reads row 0 and its scales are zeroed in registers, so that
  // row reads as zeros.  Weight rows past N read row 0 (never stored).
  auto a_index = [&](int r) -> int64_t {
    if (r >= rows_valid) return 0;
    const int64_t ur = row0 + r;
    return p.a_row_index ? (int64_t)p.a_row_index[ur] : ur;
  };
  auto a_row = [&](int r) -> int64_t {
    const int64_t ar = a_index(r);
    return ar >= 0 && ar < p.a_rows ? ar : 0;
  };
  auto w_row = [&](int r) -> int64_t {
    const int64_t br = weight_row<BN>(p, n_tile, r);
    return br >= 0 ? br : 0;
  };
  // Buffer resources of A's and this expert's W codes and scales (the host
  // checks that A and one expert's W span less than 4 GiB), built once: the
  // loop must not read the argument struct from memory.
  const Rsrc r_ac = make_rsrc(p.a_codes, p.a_rows * rbytes);
  const Rsrc r_as = make_rsrc(p.a_scales, p.a_rows * sbytes);
  const Rsrc r_wc = make_rsrc(p.w_codes + (int64_t)e * p.N * rbytes, p.N * rbytes);
  const Rsrc r_ws = make_rsrc(p.w_scales + (int64_t)e * p.N * sbytes, p.N * sbytes);
  const int lr = lane >> 2, lp = lane & 3;
  // code loads: lane l of block b loads tile row 16 b + l / 4, LDS position
  // l % 4, i.e. logical chunk (l % 4) ^ swz(row)
  uint32_t a_off[L::PA], b_off[L::PW];
  int a_chk[L::PA], b_chk[L::PW];
#pragma unroll
  for (int i = 0; i < L::PA; ++i) {
    const int b = wave * L::PA + i;
    const int r = (b < L::NA ? b : 0) * 16 + lr;
    a_chk[i] = lp ^ swz(r);
    a_off[i] = (uint32_t)(a_row(r) * rbytes) + (uint32_t)(a_chk[i] << 4);
  }
#pragma unroll
  for (int i = 0; i < L::PW; ++i) {
    const int b = wave * L::PW + i;
    const int r = (b < L::NW ? b : 0) * 16 + lr;
    b_chk[i] = lp ^ swz(r);
    b_off[i] = (uint32_t)(w_row(r) * rbytes) + (uint32_t)(b_chk[i] << 4);
  }
  // scale loads: word position P = 64 b + l holds, in the read order
  // ((wm 2 + h) 32 + l32) MI + i, word h of A row wm MI 32 + 32 i + l32
  // (likewise NJ / wn for W).  A row of the tile whose index lies outside
  // [0, a_rows) reads its scales past the end of the array: zeros, so the row
  // reads as zeros.
  uint32_t as_off[L::PAS], bs_off[L::PWS];
  int as_h[L::PAS], bs_h[L::PWS];
#pragma unroll
  for (int i = 0; i < L::PAS; ++i) {
    const int b = wave * L::PAS + i;
    const int P = (b < L::NAS ? b : 0) * 64 + lane;
    const int ii = P % MI, ll = (P / MI) % 32, hh = (P / (MI * 32)) % 2, ww = P / (MI * 64);
    const int r = ww * MI * 32 + ii * 32 + ll;
    const int64_t ar = a_index(r);
    as_h[i] = hh;
    as_off[i] = (r < rows_valid && (ar < 0 || ar >= p.a_rows))
                    ? OOB
                    : (uint32_t)(a_row(r) * sbytes) + (uint32_t)(hh * 4);
  }
#pragma unroll
  for (int i = 0; i < L::PWS; ++i) {
    const int b = wave * L::PWS + i;
    const int P = (b < L::NWS ? b : 0) * 64 + lane;
    const int jj = P % NJ, ll = (P / NJ) % 32, hh = (P / (NJ * 32)) % 2, ww = P / (NJ * 64);
    bs_h[i] = hh;
    bs_off[i] = (uint32_t)(w_row(ww * NJ * 32 + jj * 32 + ll) * sbytes) + (uint32_t)(hh * 4);
  }
  if constexpr (COMP) {
    for (int j = tid; j < kc; j += 256) {
      const int32_t c = p.sel_idx[(int64_t)e * kc + j];
      sel[j] = c < 0 ? 0 : (c >= K ? (int32_t)(K - 1) : c);
    }
    // the padding channels kc .. 16 KQ - 1 of W_S are zero (every selected
    // channel is written by the gather)
    for (int i = tid; i < BN * (KQ * 16 - kc); i += 256) {
      const int r = i / (KQ * 16 - kc), c = kc + i % (KQ * 16 - kc);
      WS[r * WSS + c] = (_Float16)0.0f;
    }
  }
  if constexpr (EPI == 2) {
    if (tid < BM) RW[tid] = tid < rows_valid ? p.row_weight[row0 + tid] : 0.0f;
  }
  if constexpr (COMP) {
    __syncthreads();
    // gather table of stage s (stages nst and nst + 1 are empty)
    auto lower = [&](int64_t c) {           // first j with sel[j] >= c
      int lo = 0, hi = kc;
      while (lo < hi) {
        const int mid = (lo + hi) >> 1;
        if (sel[mid] < c) lo = mid + 1; else hi = mid;
      }
      return lo;
    };
    for (int s = tid; s <= nst + 1; s += 256) {
      const int j0 = lower((int64_t)s * KS), n = lower((int64_t)(s + 1) * KS) - j0;
      uint32_t kk[2] = {0, 0};
      for (int q = 0; q < 8 && q < n; ++q) kk[q >> 2] |= (uint32_t)((sel[j0 + q] - s * KS) & 0x7F) << (8 * (q & 3));
      tab[s] = u32x4{(uint32_t)j0 | ((uint32_t)n << 8), kk[0], kk[1], 0u};
    }
  }

  // The LPW load instructions of stage m into slot `slot`.  In the half-full
  // last stage (K % 128 == 64) the code chunks past K are read from the row's
  // first half instead, so no load leaves its row, and the scale words past K
  // are read out of bounds: zeros, so those chunks add nothing.
  auto issue = [&](int m, int slot) {
    unsigned char* base = smem + slot * STAGE;
    const int sc = m * 64, ss = m * 8;                  // the stage's offset in a row
    if (m != mh) {
#pragma unroll
      for (int i = 0; i < L::PA; ++i) {
        const int b = wave * L::PA + i;
        load_lds16(r_ac, a_off[i], sc, b < L::NA ? base + L::A_OFF + b * 1024 : DUMMY);
      }
#pragma unroll
      for (int i = 0; i < L::PW; ++i) {
        const int b = wave * L::PW + i;
        load_lds16(r_wc, b_off[i], sc, b < L::NW ? base + L::B_OFF + b * 1024 : DUMMY);
      }
#pragma unroll
      for (int i = 0; i < L::PAS; ++i) {
        const int b = wave * L::PAS + i;
        load_lds4(r_as, as_off[i], ss, b < L::NAS ? base + L::AS_OFF + b * 256 : DUMMY);
      }
#pragma unroll
      for (int i = 0; i < L::PWS; ++i) {
        const int b = wave * L::PWS + i;
        load_lds4(r_ws, bs_off[i], ss, b < L::NWS ? base + L::BS_OFF + b * 256 : DUMMY);
      }
    } else {
#pragma unroll
      for (int i = 0; i < L::PA; ++i) {
        const int b = wave * L::PA + i;
        load_lds16(r_ac, a_off[i] - (uint32_t)((a_chk[i] & 2) << 4), sc,
                   b < L::NA ? base + L::A_OFF + b * 1024 : DUMMY);
      }
#pragma unroll
      for (int i = 0; i < L::PW; ++i) {
        const int b = wave * L::PW + i;
        load_lds16(r_wc, b_off[i] - (uint32_t)((b_chk[i] & 2) << 4), sc,
                   b < L::NW ? base + L::B_OFF + b * 1024 : DUMMY);
      }
#pragma unroll
      for (int i = 0; i < L::PAS; ++i) {
        const int b = wave * L::PAS + i;
        load_lds4(r_as, as_h[i] ? OOB : as_off[i], ss, b < L::NAS ? base + L::AS_OFF + b * 256 : DUMMY);
      }
#pragma unroll
      for (int i = 0; i < L::PWS; ++i) {
        const int b = wave * L::PWS + i;
        load_lds4(r_ws, bs_h[i] ? OOB : bs_off[i], ss, b < L::NWS ? base + L::BS_OFF + b * 256 : DUMMY);
      }
    }
  };

  // The first NSLOT stages go out (stages past the end repeat the last one
  // into slots nobody reads, so every wave issues the same count).  Between
  // stage 0 and the others, the Q(R_S) codes of the tile's rows (a contiguous
  // byte range of r_codes) go into LDS by direct loads (4 bytes a lane; words
  // past the end of r_codes read as zeros: those rows are never stored) and
  // their scale bytes into registers, all used after the K loop: the wait for
  // stage 0 covers them, the loop's waits for later stages are unchanged.  In
  // compensation substep q (16 compact channels) lane half h takes channels
  // 16 q + 8 h .. + 7, i.e. code word 2 q + h of the row and scale byte q.
  issue(0, 0);
  constexpr int KQW = COMP ? KQ : 1;
  uint32_t rqs[MI][(KQW + 3) / 4];
  if constexpr (COMP) {
    const int64_t rrow = kc / 2;                                // code bytes per row
    const Rsrc r_rc = make_rsrc(p.r_codes + row0 * rrow, (p.rows_total - row0) * rrow);
    const int nword = BM * (kc / 8);                            // words of the tile
    for (int w0 = wave * 64; w0 < nword; w0 += 256)             // uniform trip count per wave
      load_lds4(r_rc, 4u * (uint32_t)(w0 + lane), 0, RSC + 4 * w0);
    const int sb = kc / 16;                                     // scale bytes per row
    const Rsrc r_rs = make_rsrc(p.r_scales + row0 * sb, (p.rows_total - row0) * sb);
    const bool words = (sb & 3) == 0 && (reinterpret_cast<uintptr_t>(p.r_scales) & 3) == 0;
#pragma unroll
    for (int i = 0; i < MI; ++i) {
      const uint32_t rb = (uint32_t)((wm * MI * 32 + i * 32 + l32) * sb);
#pragma unroll
      for (int w = 0; w < (KQ + 3) / 4; ++w) {
        uint32_t v = 0;
        if (words) {                                            // uniform
          if (16 * 4 * w < kc) v = __builtin_amdgcn_raw_buffer_load_b32(r_rs, (int)(rb + 4 * w), 0, 0);
        } else {
#pragma unroll
          for (int b = 0; b < 4; ++b)
            if (16 * (4 * w + b) < kc)
              v |= (uint32_t)__builtin_amdgcn_raw_buffer_load_b8(r_rs, (int)(rb + 4 * w + b), 0, 0) << (8 * b);
        }
        rqs[i][w] = v;
      }
    }
  }
#pragma unroll
  for (int q = 1; q < NSLOT; ++q) issue(q < nst ? q : nst - 1, q);

  // W_S gather of a stage: thread t copies the selected channels of weight
  // row t that fall in the stage, as exact fp16 values.  Weight row t's
  // 16-byte chunk c of a stage sits at t * 64 + ((c ^ swz(t)) << 4), i.e. at
  // g_rowsw ^ (c << 4) with the swizzle bits folded into g_rowsw (the row base
  // is a multiple of 64, so the XOR only touches bits 4-5); its scale word h
  // at position ((wn 2 + h) 32 + l32) NJ + j for t = wn NJ 32 + 32 j + l32.
  // The first GW channels of a stage come from the gather table: the code
  // word and scale word of each are read right after the barrier that makes
  // the stage visible, and the nibble and the scale byte are picked out
  // (uniform positions) and written to W_S two substeps later, so nothing
  // waits on LDS latency.  More than GW channels in one stage take a slower
  // loop.
  const uint32_t g_rowsw = (uint32_t)(L::B_OFF + tid * 64 + (swz(tid) << 4));
  const uint32_t g_srow = (uint32_t)(L::BS_OFF + (((tid / (NJ * 32)) * 2 * 32 + tid % 32) * NJ + (tid % (NJ * 32)) / 32) * 4);
  // the code word and the scale word that hold K-offset kk of a stage in slot
  // byte offset sb (kk and sb uniform)
  auto g_cword = [&](uint32_t sb, int kk) {
    return *reinterpret_cast<const uint32_t*>(smem + sb + ((g_rowsw ^ (uint32_t)((kk >> 5) << 4)) + ((kk & 31) >> 3) * 4));
  };
  auto g_sword = [&](uint32_t sb, int kk) {
    return *reinterpret_cast<const uint32_t*>(smem + sb + g_srow + (kk >> 6) * 32 * NJ * 4);
  };
  // the element as an exact fp16 value from its code word and scale word
  auto ws_value = [&](uint32_t cw, uint32_t sw, int kk) {
    const uint32_t code = (cw >> (4 * (kk & 7))) & 15u;
    const uint32_t sbyte = (sw >> (8 * ((kk >> 4) & 3))) & 0xFFu;
    const f16x2 v = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(code, 1.0f, 0);
    const f16x2 sc = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(sbyte, 1.0f, false);
    return (_Float16)(v[0] * sc[0]);                          // exact: see the header
  };
  struct Gather {
    uint32_t cw[GW], sw[GW];
    int j0, n, kk[GW];
  };
  auto gather_read = [&](int slot, u32x4 t, Gather& g) {
    const uint32_t sb = (uint32_t)(slot * STAGE);
    g.j0 = __builtin_amdgcn_readfirstlane((int)(t[0] & 0xFFu));
    g.n = __builtin_amdgcn_readfirstlane((int)(t[0] >> 8));
#pragma unroll
    for (int q = 0; q < GW; ++q) {
      g.kk[q] = __builtin_amdgcn_readfirstlane((int)((t[1 + q / 4] >> (8 * (q % 4))) & 0x7Fu));
      g.cw[q] = g_cword(sb, g.kk[q]);
      g.sw[q] = g_sword(sb, g.kk[q]);
    }
  };
  // entries past the stage's count go to the row's padding halves (no
  // branch: this runs beside MFMAs)
  auto gather_write = [&](const Gather& g) {
#pragma unroll
    for (int q = 0; q < GW; ++q)
      WS[tid * WSS + (q < g.n ? g.j0 + q : KQ * 16 + q)] = ws_value(g.cw[q], g.sw[q], g.kk[q]);
  };
  // channels past the first GW of a stage (rare; at the end of the stage)
  auto gather_rest = [&](int m, int slot, const Gather& g) {
    if (g.n > GW) {                                           // uniform
      const uint32_t sb = (uint32_t)(slot * STAGE);
      for (int jj = g.j0 + GW; jj < g.j0 + g.n; ++jj) {
        const int kk = sel[jj] - m * KS;
        if ((unsigned)kk < (unsigned)KS)                      // false only if sel is not ascending
          WS[tid * WSS + jj] = ws_value(g_cword(sb, kk), g_sword(sb, kk), kk);
      }
    }
  };

  f32x16 acc[MI][NJ];
#pragma unroll
  for (int i = 0; i < MI; ++i)
#pragma unroll
    for (int j = 0; j < NJ; ++j)
#pragma unroll
      for (int q = 0; q < 16; ++q) acc[i][j][q] = 0.0f;

  // Per-lane LDS offsets of the fragment reads: row r = (wm MI or wn NJ) 32 +
  // 32 i + l32, whose swizzle depends on l32 only; chunk 2 half + t.
  const int sw = swz(l32);
  const uint32_t fa_off[2] = {(uint32_t)(L::A_OFF + (wm * MI * 32 + l32) * 64 + (((2 * half) ^ sw) << 4)),
                              (uint32_t)(L::A_OFF + (wm * MI * 32 + l32) * 64 + (((2 * half + 1) ^ sw) << 4))};
  const uint32_t fb_off[2] = {(uint32_t)(L::B_OFF + (wn * NJ * 32 + l32) * 64 + (((2 * half) ^ sw) << 4)),
                              (uint32_t)(L::B_OFF + (wn * NJ * 32 + l32) * 64 + (((2 * half + 1) ^ sw) << 4))};
  const uint32_t sa_off = (uint32_t)(L::AS_OFF + ((wm * 2 + half) * 32 + l32) * MI * 4);
  const uint32_t sb_off = (uint32_t)(L::BS_OFF + ((wn * 2 + half) * 32 + l32) * NJ * 4);

  auto main_loop = [&](auto ma_c) {
    constexpr int MA = decltype(ma_c)::value;       // live A fragments of this wave (0 .. MI)
    constexpr int NB = MA > 0 ? NJ : 0;             // live W fragments
    // raw fragments of the current stage: RA[i][t] = chunk 2 half + t of row i
    u32x4 RA[MI][2], RB[NJ][2];
    uint32_t SWA[MI], SWB[NJ];                      // scale words of the next stage
    f16x2 SCA[MI][2], SCB[NJ][2];                   // scale pairs of the current stage
    f16x8 DA[2][MI], DB[2][NJ];                     // dequantized operands, by substep parity

    auto read_raw = [&](int slot, auto t_c) {
      constexpr int T = decltype(t_c)::value;
      const unsigned char* base = smem + slot * STAGE;
#pragma unroll
      for (int i = 0; i < MA; ++i) RA[i][T] = *reinterpret_cast<const u32x4*>(base + fa_off[T] + i * 2048);
#pragma unroll
      for (int j = 0; j < NB; ++j) RB[j][T] = *reinterpret_cast<const u32x4*>(base + fb_off[T] + j * 2048);
    };
    auto read_words = [&](const unsigned char* ptr, uint32_t* w, auto n_c) {
      constexpr int n = decltype(n_c)::value;
      if constexpr (n == 4) {
        const u32x4 v = *reinterpret_cast<const u32x4*>(ptr);
        w[0] = v[0]; w[1] = v[1]; w[2] = v[2]; w[3] = v[3];
      } else if constexpr (n == 2) {
        const u32x2 v = *reinterpret_cast<const u32x2*>(ptr);
        w[0] = v[0]; w[1] = v[1];
      } else {
        w[0] = *reinterpret_cast<const uint32_t*>(ptr);
      }
    };
    // scale words of a stage from its slot (used a long while later)
    auto read_scales = [&](int slot) {
      if constexpr (MA > 0) {
        const unsigned char* base = smem + slot * STAGE;
        read_words(base + sa_off, SWA, IntC<MI>{});
        read_words(base + sb_off, SWB, IntC<NJ>{});
      }
    };
    // scale pairs of the stage whose words were read last (the loads left
    // zeros for the blocks past K and for rows with a bad index)
    auto convert_scales = [&]() {
#pragma unroll
      for (int i = 0; i < MA; ++i) {
        SCA[i][0] = scale_pair<0>(SWA[i]);
        SCA[i][1] = scale_pair<1>(SWA[i]);
      }
#pragma unroll
      for (int j = 0; j < NB; ++j) {
        SCB[j][0] = scale_pair<0>(SWB[j]);
        SCB[j][1] = scale_pair<1>(SWB[j]);
      }
    };
    // operands of substep q = 4 t + u into buffer D[q & 1]
    auto dequant = [&](auto q_c) {
      constexpr int Q = decltype(q_c)::value, T = Q / 4, U = Q % 4, B = Q & 1;
#pragma unroll
      for (int i = 0; i < MA; ++i) DA[B][i] = dequant8(RA[i][T][U], SCA[i][T][U >> 1]);
#pragma unroll
      for (int j = 0; j < NB; ++j) DB[B][j] = dequant8(RB[j][T][U], SCB[j][T][U >> 1]);
    };
    auto mfmas = [&](auto q_c) {
      constexpr int B = decltype(q_c)::value & 1;
#pragma unroll
      for (int j = 0; j < NB; ++j)
#pragma unroll
        for (int i = 0; i < MA; ++i)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(DA[B][i], DB[B][j], acc[i][j], 0, 0, 0);
    };
    // one substep: the MFMAs of q with the dequantization of q + 1 (in the
    // last substep, of the next stage's first) between them
    constexpr int NMF = MA * NB;
    constexpr int NVALU = 8 * (MA + NB);
    // The dequantized operands are pinned at the end of their substep (an
    // empty asm that takes them): without it the compiler may sink the
    // dequantization past a later branch of the stage, next to its MFMAs,
    // and the substep's MFMAs would run with no VALU work beside them.
    auto pin = [&](auto q_c) {
      constexpr int B = decltype(q_c)::value & 1;
      pin_regs<MA>(DA[B]);
      pin_regs<NB>(DB[B]);
    };
    auto substep = [&](auto q_c, auto next_c, auto&& extra, auto extra_valu) {
      mfmas(q_c);
      dequant(next_c);
      extra();
      if constexpr (NMF > 0) {
        constexpr int V = NVALU + decltype(extra_valu)::value;
#pragma unroll
        for (int k = 0; k < NMF; ++k) {
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
          __builtin_amdgcn_sched_group_barrier(0x002, (V + NMF - 1) / NMF, 0);
        }
      }
      __builtin_amdgcn_sched_barrier(0);
      pin(next_c);
    };
    auto nothing = [] {};

    // prologue: stage 0 has landed (stages 1 .. NSLOT - 1 may be in flight)
    wait_vm_lgkm0<(NSLOT - 1) * LPW>();
    asm volatile("s_barrier" ::: "memory");
    read_raw(0, IntC<0>{});
    read_raw(0, IntC<1>{});
    read_scales(0);
    [[maybe_unused]] Gather gth;
    [[maybe_unused]] u32x4 tnext = u32x4{0, 0, 0, 0};
    if constexpr (COMP) {
      gather_read(0, tab[0], gth);
      gather_write(gth);
      gather_rest(0, 0, gth);
      tnext = tab[1];
    }
    convert_scales();
    dequant(IntC<0>{});
    __builtin_amdgcn_sched_barrier(0);

    int slot = 0;                               // uniform: slot offsets are scalar adds
    // LDS reads that go out beside the MFMAs of substep 3 (the chunk-0
    // fragments and the scale words of the next stage, the gather's words)
    // and of substep 7 (the chunk-1 fragments)
    constexpr int NDS3 = MA + NB + (MA > 0 ? 2 : 0) + (COMP ? 2 * GW : 0);
    constexpr int NDS7 = MA + NB;
    for (int m = 0; m < nst; ++m) {
      const int nslot = slot == NSLOT - 1 ? 0 : slot + 1;
      substep(IntC<0>{}, IntC<1>{}, nothing, IntC<0>{});
      substep(IntC<1>{}, IntC<2>{}, nothing, IntC<0>{});
      substep(IntC<2>{}, IntC<3>{}, nothing, IntC<0>{});
      // chunk-0 registers are free: stage m + 1 in, stage m + NSLOT out.  The
      // loads and the LDS reads go out between the MFMAs of substep 3, so the
      // matrix core keeps working across the barrier's aftermath.
      wait_vm_lgkm0<(NSLOT - 2) * LPW>();
      asm volatile("s_barrier" ::: "memory");
      mfmas(IntC<3>{});
      dequant(IntC<4>{});
      issue(m + NSLOT < nst ? m + NSLOT : nst - 1, slot);
      read_raw(nslot, IntC<0>{});
      read_scales(nslot);
      if constexpr (COMP) gather_read(nslot, tnext, gth);
      if constexpr (NMF > 0) {
#pragma unroll
        for (int k = 0; k < NMF; ++k) {
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
          __builtin_amdgcn_sched_group_barrier(0x020, (LPW + NMF - 1) / NMF, 0);
          __builtin_amdgcn_sched_group_barrier(0x100, (NDS3 + NMF - 1) / NMF, 0);
          __builtin_amdgcn_sched_group_barrier(0x002, (NVALU + NMF - 1) / NMF, 0);
        }
      }
      __builtin_amdgcn_sched_barrier(0);
      pin(IntC<4>{});
      substep(IntC<4>{}, IntC<5>{}, nothing, IntC<0>{});
      // the gather reads issued at substep 3 are in by now
      if constexpr (COMP) {
        substep(IntC<5>{}, IntC<6>{}, [&] { gather_write(gth); tnext = tab[m + 2]; }, IntC<10 * GW>{});
      } else {
        substep(IntC<5>{}, IntC<6>{}, nothing, IntC<0>{});
      }
      substep(IntC<6>{}, IntC<7>{}, nothing, IntC<0>{});
      // the last substep dequantizes the next stage's first operands (its
      // scale pairs are converted first: the current ones are used up) and
      // reads the next stage's chunk-1 fragments (chunk 1 of this stage was
      // dequantized in substep 6)
      mfmas(IntC<7>{});
      read_raw(nslot, IntC<1>{});
      convert_scales();
      dequant(IntC<0>{});
      if constexpr (NMF > 0) {
#pragma unroll
        for (int k = 0; k < NMF; ++k) {
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
          __builtin_amdgcn_sched_group_barrier(0x100, (NDS7 + NMF - 1) / NMF, 0);
          __builtin_amdgcn_sched_group_barrier(0x002, (NVALU + 2 * (MA + NB) + NMF - 1) / NMF, 0);
        }
      }
      __builtin_amdgcn_sched_barrier(0);
      pin(IntC<0>{});
      if constexpr (COMP) gather_rest(m + 1, nslot, gth);
      slot = nslot;
    }
    wait_vm_lgkm0<0>();                         // the repeat loads of the last stages
  };

  // The number of this wave's 32-row A fragments that hold rows of the tile
  // (0 .. MI): a ragged last m-tile of an expert skips the MFMAs and the
  // dequantization of its empty fragments (a wave with none skips its W
  // fragments too; it still issues its share of the loads), with the loop
  // specialized for each count.  readfirstlane makes the count visibly
  // uniform, so the switch is a scalar branch.
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
  __syncthreads();                             // W_S complete; LDS free afterwards

  // ---- global scales, the compensation and the epilogue ------------------------
  const float ga = p.a_global[p.a_global_per_group ? e : 0];
  const float gw = p.w_global[e];
  const float scale = COMP ? 1.0f : ga * gw;
  // Row block i's compensation: corr = sum_q R_q W_S,q per 32 x 32 block (the
  // Q(R_S) operands of the block's rows dequantized once, the W_S operands
  // read per block); the output is acc * gA gW + corr * gR gW, so no ratio of
  // global scales can overflow.  Substeps past kc add zero: their scale bytes
  // are 0 and the padding channels of W_S are 0 (the code words read stay
  // inside the Q(R_S) region).  The epilogue's LDS staging reaches past the
  // slot ring into W_S in the narrow-ring variants (STAGING_OVERLAPS below):
  // there the sum goes back into acc, else it is formed as the output
  // element is read.
  constexpr size_t WAVE_STAGE = EPI == 1 ? (size_t)32 * (NJ * 16 + 8) * 2 : (size_t)epilogue_wave_floats<NJ>() * 4;
  constexpr bool STAGING_OVERLAPS = COMP && 4 * WAVE_STAGE > (size_t)NSLOT * STAGE + DUMMY_BYTES;
  const float sa = ga * gw, sr = COMP ? p.r_global[e] * gw : 0.0f;
  [[maybe_unused]] f32x16 corr[COMP && !STAGING_OVERLAPS ? NJ : 1];
  auto prep = [&](int i) {
    if constexpr (COMP) {
      const uint32_t* cw = reinterpret_cast<const uint32_t*>(RSC + (wm * MI * 32 + i * 32 + l32) * (kc / 2));
      f16x8 rf[KQ];
#pragma unroll
      for (int q = 0; q < KQ; ++q) {
        const uint32_t sbyte = (rqs[i][q >> 2] >> (8 * (q & 3))) & 0xFFu;
        rf[q] = dequant8(cw[2 * q + half], __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(sbyte, 1.0f, false)[0]);
      }
#pragma unroll
      for (int j = 0; j < NJ; ++j) {
        const _Float16* wsr = WS + (wn * NJ * 32 + j * 32 + l32) * WSS + 8 * half;
        f32x16 c;
#pragma unroll
        for (int v = 0; v < 16; ++v) c[v] = 0.0f;
#pragma unroll
        for (int q = 0; q < KQ; ++q)
          c = __builtin_amdgcn_mfma_f32_32x32x16_f16(rf[q], *reinterpret_cast<const f16x8*>(wsr + 16 * q), c, 0, 0, 0);
        if constexpr (STAGING_OVERLAPS) {
#pragma unroll
          for (int v = 0; v < 16; ++v) acc[i][j][v] = acc[i][j][v] * sa + c[v] * sr;
        } else {
          corr[j] = c;
        }
      }
    }
  };
  auto val = [&](int i, int j, int q) {
    if constexpr (COMP && !STAGING_OVERLAPS) return acc[i][j][q] * sa + corr[j][q] * sr;
    else return acc[i][j][q] * scale;
  };
  // Row blocks are compensated right before their output leaves, unless the
  // epilogue's LDS staging (per wave: 32 rows of bf16 h for SwiGLU, of fp32
  // otherwise) reaches past the slot ring into W_S and is used (SwiGLU, or
  // an F32 tile that does not store straight from the accumulators): then
  // all row blocks first.
  bool early = false;
  if constexpr (STAGING_OVERLAPS) early = EPI == 1 || !epilogue_direct<MI, BN, EPI>(p, tc);
  if (early) {                                   // uniform over the workgroup
#pragma unroll
    for (int i = 0; i < MI; ++i) prep(i);
    __syncthreads();                             // W_S reads done before the staging writes
  }
  gemm_epilogue_blocks<MI, NJ, BN, EPI>(
      p, tc, wm * MI * 32, wn * NJ * 32, reinterpret_cast<float*>(smem + wave * WAVE_STAGE), RW,
      [&](int i) {
        if (!early) prep(i);
      },
      val);
}

// One tile per workgroup; with 32-row tiles the workgroups may go round the
// tiles (a capped grid: one round when it has one workgroup per tile), with
// map_tile's barriers between one tile's last LDS reads and the next tile's
// first writes.  (A loop around the larger tiles costs them registers.)
template <int MI, int NJ, int WM, int WN, int NSLOT, int EPI, int KQ, int GW>
__global__ __launch_bounds__(256, 1) void grouped_gemm_kernel(GemmArgs p, int ntiles) {
  constexpr int BM = WM * MI * 32;
  if constexpr (BM == 32) {
    for (int round = 0;; ++round) {
      TileCoord tc;
      if (!map_tile<BM>(p, ntiles, tc, round)) return;   // uniform over the workgroup
      gemm_tile<MI, NJ, WM, WN, NSLOT, EPI, KQ, GW>(p, tc);
    }
  } else {
    TileCoord tc;
    if (!map_tile<BM>(p, ntiles, tc)) return;            // uniform over the workgroup
    gemm_tile<MI, NJ, WM, WN, NSLOT, EPI, KQ, GW>(p, tc);
  }
}

template <int MI, int NJ, int WM, int WN, int NSLOT, int EPI, int KQ, int GW>
static hipError_t launch_cfg(GemmArgs a, hipStream_t stream, size_t lds_cap) {
  constexpr int BM = WM * MI * 32;
  const int64_t mtiles = (a.rows_total + BM - 1) / BM + a.E;
  const int64_t ntiles = a.epilogue == 1 ? (a.N / 2 + BN / 2 - 1) / (BN / 2) : (a.N + BN - 1) / BN;
  const int64_t total = mtiles * ntiles;
  const size_t loop = (loop_lds_bytes<BM, NSLOT, KQ>(a.K) + 15) / 16 * 16;
  const size_t epi = (size_t)4 * epilogue_wave_floats<NJ>() * 4;
  const size_t body = loop > epi ? loop : epi;
  a.rw_lds_offset = (int)body;
  const size_t lds = body + (EPI == 2 ? (size_t)BM * 4 : 0);
  if (lds > lds_cap) return hipErrorInvalidConfiguration;
  auto kern = grouped_gemm_kernel<MI, NJ, WM, WN, NSLOT, EPI, KQ, GW>;
  hipError_t err = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
  if (err != hipSuccess) return err;
  int64_t grid = (total + 7) / 8 * 8;             // upper bound on the tiles, one share per XCD
  if (BM == 32 && a.grid_cap > 0 && grid > a.grid_cap) grid = (a.grid_cap + 7) / 8 * 8;
  kern<<<(unsigned)grid, 256, lds, stream>>>(a, (int)ntiles);
  return hipGetLastError();
}

template <int MI, int NJ, int WM, int WN, int NSLOT, int KQ, int GW>
static hipError_t launch_epi(const GemmArgs& a, hipStream_t stream, size_t lds_cap = 160 * 1024) {
  switch (a.epilogue) {
    case 0: return launch_cfg<MI, NJ, WM, WN, NSLOT, 0, KQ, GW>(a, stream, lds_cap);
    case 1: return launch_cfg<MI, NJ, WM, WN, NSLOT, 1, KQ, GW>(a, stream, lds_cap);
    default: return launch_cfg<MI, NJ, WM, WN, NSLOT, 2, KQ, GW>(a, stream, lds_cap);
  }
}

// The gather takes 8 channels per stage beside the MFMAs where the stages
// hold more than 3 selected channels on average (e.g. 64 of K = 1536), else 4.
template <int MI, int NJ, int WM, int WN, int NSLOT>
static hipError_t launch_comp(const GemmArgs& a, hipStream_t stream) {
  if (!a.sel_idx) return launch_epi<MI, NJ, WM, WN, NSLOT, 0, 4>(a, stream);
  const bool wide = (int64_t)a.kc * KS > 3 * a.K;
  if (a.kc <= 64)
    return wide ? launch_epi<MI, NJ, WM, WN, NSLOT, 4, 8>(a, stream) : launch_epi<MI, NJ, WM, WN, NSLOT, 4, 4>(a, stream);
  // a wider W_S: one slot fewer
  return wide ? launch_epi<MI, NJ, WM, WN, NSLOT - 1, 8, 8>(a, stream)
              : launch_epi<MI, NJ, WM, WN, NSLOT - 1, 8, 4>(a, stream);
}

// 32-row tiles stream weights with little reuse per byte, so the number of
// workgroups that a CU holds matters more than the ring depth: with up to 64
// compensated channels a ring of two slots fits two workgroups per CU.
static hipError_t launch_32(const GemmArgs& a, hipStream_t stream) {
  if (a.sel_idx && a.kc <= 64) {
    constexpr size_t HALF_CU = 80 * 1024 - 256;          // two workgroups' LDS, static arrays included
    const bool wide = (int64_t)a.kc * KS > 3 * a.K;
    const hipError_t err = wide ? launch_epi<1, 2, 1, 4, 2, 4, 8>(a, stream, HALF_CU)
                                : launch_epi<1, 2, 1, 4, 2, 4, 4>(a, stream, HALF_CU);
    if (err != hipErrorInvalidConfiguration) return err;
  }
  return launch_comp<1, 2, 1, 4, 3>(a, stream);
}

}  // namespace nvg

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

// The kernel reads A codes and one expert's W codes with 32-bit offsets.
bool grouped_gemm_offsets_fit(int64_t a_rows, int64_t N, int64_t K) {
  const int64_t lim = (int64_t)1 << 32;
  return a_rows * (K / 2) < lim && N * (K / 2) < lim;
}

// A second stream per device for the launch of ragged remainders (and, ahead
// of it, the scatter's plan), forked from and joined back into the caller's
// stream with two events: its 32-row tiles then run on the CUs that the
// 256-row launch's last round leaves idle (0.02-0.06 ms per projection on the
// 8192-token layer, 0.04-0.07 on the 16384-token prefill).  Created on first use and kept for the process; the
// mutex keeps the event record/wait pairs of concurrent host threads apart.
// Where the stream or its events cannot be had, the launch stays on the
// caller's stream.
SideStream* side_stream(hipStream_t caller) {
  static std::mutex mu;
  static SideStream per_dev[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return nullptr;
  // Not while the caller's stream is being captured into a graph: the fork
  // would pull the shared stream into that capture, and with it the work of
  // other threads.  Captured calls keep to the caller's stream.
  hipStreamCaptureStatus st = hipStreamCaptureStatusNone;
  if (hipStreamIsCapturing(caller, &st) != hipSuccess || st != hipStreamCaptureStatusNone) return nullptr;
  std::lock_guard<std::mutex> lk(mu);
  SideStream& ss = per_dev[dev];
  if (!ss.tried) {
    ss.tried = true;
    if (hipStreamCreateWithFlags(&ss.s, hipStreamNonBlocking) != hipSuccess ||
        hipEventCreateWithFlags(&ss.fork, hipEventDisableTiming) != hipSuccess ||
        hipEventCreateWithFlags(&ss.join, hipEventDisableTiming) != hipSuccess)
      ss.s = nullptr;
  }
  return ss.s ? &ss : nullptr;
}

hipError_t launch_grouped_gemm(const GemmArgs& a, hipStream_t stream) {
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
  // a compensation wider than 64 channels (a larger W_S) needs a shorter tile
  if (a.sel_idx && a.kc > 64 && bm > 128) bm = 128;
  if (bm == 256 && a.block_m == 0) {
    // 256-row tiles over each group's rows except a remainder of fewer than
    // 96 rows, and those remainders in 32-row tiles: 256 workgroups (one
    // per CU) go round them, as the host does not know how many there are.
    // The two launches write disjoint rows (and max into one amax).
    GemmArgs big = a, rest = a;
    big.tail_split = 1;
    rest.tail_split = 2;
    rest.grid_cap = 256;
    // The scatter's plan (the row lists of each output row) needs only the
    // scatter index, so it goes on the side stream ahead of the remainder
    // launch and is hidden behind the 256-row launch; the ordered sum of the
    // rows follows the join.
    if (SideStream* ss = side_stream(stream)) {
      std::lock_guard<std::mutex> lk(ss->mu);
      err = hipEventRecord(ss->fork, stream);
      if (err == hipSuccess) err = hipStreamWaitEvent(ss->s, ss->fork, 0);
      if (err == hipSuccess && a.epilogue == 2)
        err = launch_combine_plan(a.rows_total, a.N, a.scatter_index, a.out_rows, a.y_rows, ss->s);
      if (err == hipSuccess) err = nvg::launch_32(rest, ss->s);
      if (err == hipSuccess) err = hipEventRecord(ss->join, ss->s);
      if (err == hipSuccess) err = nvg::launch_comp<4, 4, 2, 2, 3>(big, stream);
      if (err == hipSuccess) err = hipStreamWaitEvent(stream, ss->join, 0);
      if (err != hipSuccess || a.epilogue != 2) return err;
      return launch_combine_rows(a.y_rows, a.rows_total, a.N, a.out_rows, static_cast<float*>(a.out),
                                 a.ldo, a.combine_overwrite, a.y_rows, stream);
    }
    err = nvg::launch_comp<4, 4, 2, 2, 3>(big, stream);
    if (err == hipSuccess) err = nvg::launch_32(rest, stream);
    if (err != hipSuccess || a.epilogue != 2) return err;
    return launch_combine(a.y_rows, a.rows_total, a.N, a.scatter_index, a.out_rows,
                          static_cast<float*>(a.out), a.ldo, a.combine_overwrite, a.y_rows, stream);
  }
  switch (bm) {
    case 256: err = nvg::launch_comp<4, 4, 2, 2, 3>(a, stream); break;
    case 128: err = nvg::launch_comp<2, 4, 2, 2, 3>(a, stream); break;
    case 64: err = nvg::launch_comp<1, 4, 2, 2, 3>(a, stream); break;
    default: err = nvg::launch_32(a, stream); break;
  }
  if (err != hipSuccess || a.epilogue != 2) return err;
  return launch_combine(a.y_rows, a.rows_total, a.N, a.scatter_index, a.out_rows,
                        static_cast<float*>(a.out), a.ldo, a.combine_overwrite, a.y_rows, stream);
}

}  // namespace nvfp4
