// Device-side NVFP4 helpers for gfx950: E4M3 scale encode/decode, exact
// E2M1 rounding, the fast convert-and-verify element quantizer, and wave
// reductions.
//
// Format and rounding rules (one definition for the whole library):
//   g   = RNE32(amax / 2688), 1 when that is 0;
//   s_b = E4M3FN value nearest to amax_b / (6 g) (ties to the even byte,
//         saturating at 448); S_b = RNE32(s_b * g);
//   element index = E2M1 index nearest to |x| / S_b, ties to the even index,
//         saturating at 6, 0 when S_b == 0; sign bit = sign bit of x;
//   DQ  = RNE32(value * S_b).
// The pages fix the codebook, the round-to-nearest rule under a global and
// a per-block scale, and the worked example (TRACE summary, "Prerequisites:
// NVFP4 and the E2M1 codebook" and "Research motivation"); the formulas for
// the scales and the tie rule are readings of what the pages leave open.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace nvfp4 {

constexpr int kBlock = 16;                  // elements per block scale
constexpr float kBlockMax = 2688.0f;        // 6 (E2M1 max) * 448 (E4M3 max)
constexpr int kScoreTileRows = 128;         // rows per tile of the residual-score sum order

typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

// ---------------------------------------------------------------------------
// bf16
// ---------------------------------------------------------------------------
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

// fp32 -> bf16 bits, round to nearest even (finite inputs).
__device__ __forceinline__ uint32_t f32_to_bf16_rne(float f) {
  uint32_t u = __float_as_uint(f);
  return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}

// Two fp32 values to packed bf16 bits (a in the low half), round to nearest
// even: one hardware convert (v_cvt_pk_bf16_f32; the kernels keep fp32
// denormals, so subnormal inputs round like normal ones).
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t pack_bf16x2_rne(float a, float b) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{a, b}, bf16x2_t));
}

// ---------------------------------------------------------------------------
// global scale
// ---------------------------------------------------------------------------
// g = RNE32(amax / 2688): '/' on floats is the correctly rounded division
// (hipcc's default); a zero quotient gives 1.
__device__ __forceinline__ float global_scale_from_amax(float amax) {
  float g = amax / kBlockMax;
  return g == 0.0f ? 1.0f : g;
}

// ---------------------------------------------------------------------------
// E4M3FN block scale
// ---------------------------------------------------------------------------
// Value of an E4M3FN byte 0x00..0x7E: subnormal m * 2^-9, normal
// (1 + m/8) * 2^(e-7) whose fp32 exponent field is e + 120.
__device__ __forceinline__ float e4m3_value(uint32_t b) {
  uint32_t e = (b >> 3) & 15u, m = b & 7u;
  return e == 0 ? (float)m * 0x1p-9f : __uint_as_float(((e + 120u) << 23) | (m << 20));
}

// E4M3FN byte nearest to q >= 0 (ties to even, saturating at 448).
// q is the correctly rounded float64 quotient amax_b / (6 g).  That is as good
// as the exact quotient: every E4M3 rounding boundary has at most 5
// significant bits, so "quotient == boundary" means amax_b == boundary * 6g
// with both sides exact in float64 (<= 31 bits), and a quotient that is not
// on a boundary lies at least 2^-31 (relative) away from it -- far beyond the
// 2^-53 of the float64 rounding, which therefore never crosses a boundary.
__device__ __forceinline__ uint32_t e4m3_nearest(double q) {
  if (q >= 448.0) return 0x7Eu;
  // below the smallest normal (2^-6) the spacing is 2^-9; n == 8 is byte 0x08 = 2^-6
  if (q < 0x1p-6) return (uint32_t)rint(q * 512.0);
  int e;
  (void)frexp(q, &e);                        // q = f * 2^e, f in [0.5, 1)
  int lead = e - 1;                          // q in [2^lead, 2^(lead+1)), lead >= -6
  uint32_t n = (uint32_t)rint(ldexp(q, 3 - lead));   // exact scaling, RNE: 8..16
  if (n == 16) { n = 8; ++lead; }
  uint32_t byte = ((uint32_t)(lead + 7) << 3) | (n - 8);
  return byte > 0x7Eu ? 0x7Eu : byte;
}

// Per-tensor constants of the block-scale choice for global scale g.
struct BlockScaler {
  float g;
  float inv_up, inv_dn;                      // 1/(6g) times (1 + 2^-20), (1 - 2^-20)
  double six_g;
  bool fast;                                 // g >= 2^-100: the fp32 path below is exact
};
__device__ __forceinline__ BlockScaler make_block_scaler(float g) {
  BlockScaler b;
  b.g = g;
  b.six_g = 6.0 * (double)g;
  b.fast = g >= 0x1p-100f;
  const float inv = __builtin_amdgcn_rcpf(6.0f * g);
  b.inv_up = inv * (1.0f + 0x1p-20f);
  b.inv_dn = inv * (1.0f - 0x1p-20f);
  return b;
}

// Block scale byte and effective fp32 scale S_b for a block amax.
// The byte is the E4M3 value nearest to the exact quotient q = amax_b / (6g)
// (ties to even, saturating at 448), as e4m3_nearest decides it.  Fast path:
// amax_b * inv_up and amax_b * inv_dn bracket q (1/(6g) is within 2^-22 of
// exact after the rounding of 6g, the reciprocal and the two products, well
// inside the 2^-20 margins), and the hardware FP8 convert (round to nearest
// even) of both, clamped to 448, gives the byte wherever they agree.  Where
// they differ, exactly one rounding boundary m (the midpoint of the two
// adjacent values, at most 5 significant bits) lies between them, and the sign
// of fma(6m, g, -amax_b) -- 6m is exact, so this is 6mg - amax_b rounded once,
// which keeps its sign and is zero only on a tie (no underflow to zero for
// g >= 2^-100) -- picks the side; a tie goes to the even byte.
__device__ __forceinline__ uint32_t block_scale(float amax_b, const BlockScaler& bs, float& S) {
  uint32_t sb;
  if (bs.fast) {
    const float qu = fminf(amax_b * bs.inv_up, 448.0f), qd = fminf(amax_b * bs.inv_dn, 448.0f);
    typedef short s16x2 __attribute__((ext_vector_type(2)));
    const s16x2 r = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(s16x2{0, 0}, qu, qd, 1.0f, false);
    const uint32_t w = (uint16_t)r[0];
    const uint32_t bu = w & 0xFFu, bd = w >> 8;
    sb = bu;
    if (bu != bd) {                            // rare: q near a rounding boundary
      const float m = 0.5f * (e4m3_value(bd) + e4m3_value(bu));   // exact
      const float d = __builtin_fmaf(6.0f * m, bs.g, -amax_b);
      sb = d < 0.0f ? bu : (d > 0.0f ? bd : ((bd & 1u) ? bu : bd));
    }
  } else {
    sb = e4m3_nearest((double)amax_b / bs.six_g);
  }
  S = e4m3_value(sb) * bs.g;                 // RNE32(s_b * g): one rounding
  return sb;
}

// ---------------------------------------------------------------------------
// E2M1
// ---------------------------------------------------------------------------
// Magnitude of E2M1 index i (0..7): 0, 0.5, then (1 + (i&1)/2) * 2^((i>>1)-1),
// whose fp32 bits are (i + 252) << 22.
__device__ __forceinline__ float e2m1_mag(uint32_t i) {
  return i < 2 ? (i ? 0.5f : 0.0f) : __uint_as_float((i + 252u) << 22);
}
__device__ __forceinline__ float e2m1_value(uint32_t code) {
  return __uint_as_float(__float_as_uint(e2m1_mag(code & 7u)) | ((code & 8u) << 28));
}

// Exact E2M1 code of x under S: the index counts midpoints m below |x|/S,
// deciding each by the sign of fma(m, S, -|x|) -- the exact m*S - |x|
// rounded once, which keeps its sign and is zero only on an exact tie.
// Midpoint j lies between index j and j+1; on a tie the even index wins,
// i.e. index j+1 exactly when j is odd.
__device__ __forceinline__ uint32_t e2m1_code_exact(float x, float S) {
  uint32_t sign = __float_as_uint(x) >> 31;
  if (S == 0.0f) return sign << 3;
  float ax = fabsf(x);
  const float mid[7] = {0.25f, 0.75f, 1.25f, 1.75f, 2.5f, 3.5f, 5.0f};
  uint32_t idx = 0;
#pragma unroll
  for (int j = 0; j < 7; ++j) {
    float d = __builtin_fmaf(mid[j], S, -ax);
    idx += (j & 1) ? (d <= 0.0f) : (d < 0.0f);
  }
  return (sign << 3) | idx;
}

// Fast path for 8 elements sharing a scale.  iu and id are 1/S (within 1 ulp)
// times (1 + 2^-20) and (1 - 2^-20), each rounded once (e2m1_brackets), so
// x * iu and x * id lie above and below the exact quotient x / S (the three
// roundings stay within 2^-22); the hardware FP4 convert (round to nearest
// even, saturating, sign kept) of both brackets the exact code.  Where the
// two agree, no rounding boundary lies in the band and the code is exact.  Where they differ, exactly one midpoint m
// lies in the band, between the two (adjacent) magnitudes the brackets gave;
// the sign of fma(m, S, -|x|) -- the exact m*S - |x| rounded once -- decides
// the side, and a zero (an exact tie, common when S has few significant bits)
// goes to the even index.  Returns the packed codes (element 2j in the low
// nibble of byte j).
__device__ __forceinline__ void e2m1_brackets(float S, float& iu, float& id) {
  const float inv = __builtin_amdgcn_rcpf(S);   // within 1 ulp
  iu = inv * (1.0f + 0x1p-20f);
  id = inv * (1.0f - 0x1p-20f);
}
__device__ __forceinline__ uint32_t e2m1_pack8_fast(const float* x, float iu, float id, float S) {
  uint32_t wu = 0, wd = 0;
#define NVFP4_CVT_PAIR(P)                                                                   \
  wu = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(wu, x[2 * P] * iu, x[2 * P + 1] * iu, 1.0f, P); \
  wd = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(wd, x[2 * P] * id, x[2 * P + 1] * id, 1.0f, P);
  NVFP4_CVT_PAIR(0)
  NVFP4_CVT_PAIR(1)
  NVFP4_CVT_PAIR(2)
  NVFP4_CVT_PAIR(3)
#undef NVFP4_CVT_PAIR
  uint32_t diff = wu ^ wd;
  while (diff) {                               // rare: elements near a rounding boundary
    const int sh = (__builtin_ctz(diff) >> 2) << 2;
    const uint32_t iu = (wu >> sh) & 7u, id = (wd >> sh) & 7u;
    const uint32_t lo = iu < id ? iu : id, hi = iu < id ? id : iu;   // hi == lo + 1
    const float m = 0.5f * (e2m1_mag(lo) + e2m1_mag(hi));            // exact
    float xi = x[0];
#pragma unroll
    for (int i = 1; i < 8; ++i) xi = (sh >> 2) == i ? x[i] : xi;
    const float d = __builtin_fmaf(m, S, -fabsf(xi));
    const uint32_t idx = d < 0.0f ? hi : (d > 0.0f ? lo : ((lo & 1u) ? hi : lo));
    wu = (wu & ~(7u << sh)) | (idx << sh);    // the sign bit (bit 3) already copies x's
    diff &= ~(15u << sh);
  }
  return wu;
}

__device__ __forceinline__ uint32_t e2m1_pack8_exact(const float* x, float S) {
  uint32_t w = 0;
#pragma unroll
  for (int j = 0; j < 8; ++j) w |= e2m1_code_exact(x[j], S) << (4 * j);
  return w;
}

// Quantize one 16-element block held in registers.  Writes the scale byte and
// two packed code words; returns S_b.
__device__ __forceinline__ float quantize_block16(const float* v, const BlockScaler& bs,
                                                  uint32_t* sbyte, uint32_t* w0, uint32_t* w1) {
  float amax = 0.0f;
#pragma unroll
  for (int i = 0; i < 16; ++i) amax = fmaxf(amax, fabsf(v[i]));
  float S;
  *sbyte = block_scale(amax, bs, S);
  // The fast path needs 1/S finite and accurate: S >= 2^-100 (a normal number).
  if (S >= 0x1p-100f) {
    float iu, id;
    e2m1_brackets(S, iu, id);
    *w0 = e2m1_pack8_fast(v, iu, id, S);
    *w1 = e2m1_pack8_fast(v + 8, iu, id, S);
  } else {
    *w0 = e2m1_pack8_exact(v, S);
    *w1 = e2m1_pack8_exact(v + 8, S);
  }
  return S;
}

// Values of the 8 codes packed in w (element 2j in the low nibble of byte j),
// by the hardware FP4 -> fp32 convert (exact).
__device__ __forceinline__ void e2m1_unpack8(uint32_t w, float* f) {
  f32x2 t;
  t = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, 0); f[0] = t[0]; f[1] = t[1];
  t = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, 1); f[2] = t[0]; f[3] = t[1];
  t = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, 2); f[4] = t[0]; f[5] = t[1];
  t = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, 3); f[6] = t[0]; f[7] = t[1];
}

// Dequantized value of 4-bit code c under S: RNE32(value * S).
__device__ __forceinline__ float dq(uint32_t c, float S) { return e2m1_value(c) * S; }

// ---------------------------------------------------------------------------
// MXFP4 (32-element blocks, E8M0 power-of-two scales)
// ---------------------------------------------------------------------------
// Shared scale 2^X of a block with largest magnitude amax: X = floor(log2
// amax) - 2 (2 is the exponent of the largest E2M1 level), clamped to
// [-127, 127], and -127 for amax == 0.  With E the fp32 exponent field of
// amax, floor(log2 amax) = E - 127 for normal amax; a subnormal or zero amax
// (E == 0) lies below 2^-126 and clamps to -127 as well, as does E == 1.
// The stored byte is X + 127 = max(E - 2, 0); finite fp32 inputs give at most
// 252 (X = 125).
constexpr int kMxBlock = 32;
__device__ __forceinline__ uint32_t mx_scale_byte(float amax) {
  const int E = (int)((__float_as_uint(amax) >> 23) & 0xFFu);
  return (uint32_t)(E > 2 ? E - 2 : 0);
}
// 2^X of a scale byte b = X + 127 (b <= 254): a normal fp32 for b >= 1,
// 2^-127 (an fp32 subnormal) for b == 0.
__device__ __forceinline__ float e8m0_value(uint32_t b) {
  return b ? __uint_as_float(b << 23) : __uint_as_float(0x00400000u);
}
// 2^-X, always a normal fp32 (X in [-127, 125]).
__device__ __forceinline__ float e8m0_inverse(uint32_t b) {
  return __uint_as_float((254u - b) << 23);
}

// MXFP4 codes of 32 elements sharing scale byte b, packed 8 to a word.
// |x| * 2^-X is exact (a power-of-two multiply; results small enough to
// underflow lie far below the first rounding midpoint), so the E2M1 rounding
// of the NVFP4 fast path applies with brackets 2^-X (1 +- 2^-20): the
// hardware convert of both brackets agrees except where an exact midpoint
// lies between them, and there the sign of fma(m, 2^X, -|x|) -- exact, also
// when 2^X is subnormal -- decides, a tie going to the even index.
__device__ __forceinline__ void mx_pack32(const float* v, uint32_t b, uint32_t* w) {
  const float inv = e8m0_inverse(b), S = e8m0_value(b);
  const float iu = inv * (1.0f + 0x1p-20f), id = inv * (1.0f - 0x1p-20f);
#pragma unroll
  for (int q = 0; q < 4; ++q) w[q] = e2m1_pack8_fast(v + 8 * q, iu, id, S);
}

// Workgroup barrier for LDS hand-offs only: waits for this wave's LDS
// operations, then meets the other waves.  Unlike __syncthreads() it does not
// wait for outstanding global loads, so loads issued ahead for later K-steps
// stay in flight across the barrier.  The memory clobber keeps the compiler
// from moving LDS accesses across it.
__device__ __forceinline__ void lds_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// ---------------------------------------------------------------------------
// wave reductions (64 lanes)
// ---------------------------------------------------------------------------
__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
  return v;
}
__device__ __forceinline__ uint32_t wave_sum_u32(uint32_t v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}
// The same sum by DPP row operations (no LDS traffic), returned as a uniform
// value: sums within quads, half rows and rows of 16 lanes, then row 0 into
// row 1 and row 2 into row 3 (row_bcast:15), then rows 0-1 into rows 2-3
// (row_bcast:31), leaving the total in lane 63.  Lanes outside a row mask
// take the old operand, 0.
__device__ __forceinline__ uint32_t wave_sum_dpp(uint32_t v) {
  v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0xB1, 0xF, 0xF, false);    // quad_perm [1,0,3,2]
  v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x4E, 0xF, 0xF, false);    // quad_perm [2,3,0,1]
  v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x141, 0xF, 0xF, false);   // row_half_mirror
  v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x140, 0xF, 0xF, false);   // row_mirror
  v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x142, 0xA, 0xF, false);   // row_bcast:15
  v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x143, 0xC, 0xF, false);   // row_bcast:31
  return (uint32_t)__builtin_amdgcn_readlane((int)v, 63);
}

// Atomic max of a non-negative float stored as fp32 bits (non-negative
// floats order like their bit patterns).
__device__ __forceinline__ void atomic_max_nonneg(float* p, float v) {
  atomicMax(reinterpret_cast<unsigned int*>(p), __float_as_uint(v));
}

}  // namespace nvfp4
