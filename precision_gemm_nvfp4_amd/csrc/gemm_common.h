// Pieces of the grouped GEMM kept apart from its main loop: the mapping of
// workgroups to (expert, m-tile, n-tile), the weight-row order of a SwiGLU
// tile, and the epilogues.
#pragma once
#include "device_common.h"
#include "kernels.h"

namespace nvfp4 {

__device__ __forceinline__ int64_t clamp64(int64_t v, int64_t lo, int64_t hi) {
  return v < lo ? lo : (v > hi ? hi : v);
}

// silu(z) = z / (1 + e^-z), with the hardware reciprocal (about 1 ulp) in
// place of a correctly rounded division; z -> -inf gives -0.
__device__ __forceinline__ float silu_f32(float z) {
  return z * __builtin_amdgcn_rcpf(1.0f + __expf(-z));
}

// A raw buffer resource (stride 0, 32-bit data format, what untyped loads
// and stores need on gfx9) over `bytes` bytes from `base`.  Every field goes
// through readfirstlane: a resource must sit in scalar registers, and a value
// the compiler happened to compute on the vector unit would otherwise cost a
// loop over its distinct values around every instruction that uses it.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, int64_t bytes) {
  const uint64_t b = reinterpret_cast<uint64_t>(base);
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)b);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(b >> 32));
  const uint32_t n = __builtin_amdgcn_readfirstlane(
      (uint32_t)(bytes < 0 ? 0 : (bytes < 0xFFFFFFFFll ? bytes : 0xFFFFFFFFll)));
  return __builtin_amdgcn_make_buffer_rsrc(reinterpret_cast<void*>(((uint64_t)hi << 32) | lo), (short)0, (int)n,
                                           0x00020000);
}

struct TileCoord {
  int e;            // expert
  int n_tile;
  int64_t row0;     // first unit row of the tile
  int rows_valid;   // rows of the tile inside the expert's group
};

// The coordinates as visibly uniform values (they come out of LDS, which the
// compiler cannot prove uniform): scalar registers for everything derived
// from them, e.g. buffer resources, which would otherwise need a loop per
// instruction over the distinct values.
__device__ __forceinline__ TileCoord uniform_tile(TileCoord t) {
  TileCoord u;
  u.e = __builtin_amdgcn_readfirstlane(t.e);
  u.n_tile = __builtin_amdgcn_readfirstlane(t.n_tile);
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)(uint64_t)t.row0);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)((uint64_t)t.row0 >> 32));
  u.row0 = (int64_t)(((uint64_t)hi << 32) | lo);
  u.rows_valid = __builtin_amdgcn_readfirstlane(t.rows_valid);
  return u;
}

// A group's rows in 256-row tiles leave a ragged remainder; one of fewer
// than TAIL_MIN rows costs a 256-row tile about two thirds of a full one, so
// the launcher gives those remainders to a second launch of 32-row tiles.
constexpr int64_t TAIL_BM = 256, TAIL_MIN = 96;

// The rows [g0, g1) of group e that this launch covers (tail_split: 0 all of
// them; 1 the rows up to the group's last multiple of TAIL_BM, and the
// remainder too when it has at least TAIL_MIN rows; 2 the remainder
// otherwise).
__device__ __forceinline__ void group_rows(const GemmArgs& p, int e, int64_t& g0, int64_t& g1) {
  const int64_t b = clamp64(p.group_offsets[e], 0, p.rows_total);
  const int64_t en = clamp64(p.group_offsets[e + 1], b, p.rows_total);
  if (p.tail_split == 0) {
    g0 = b;
    g1 = en;
    return;
  }
  const int64_t cnt = en - b, rem = cnt % TAIL_BM;
  const int64_t big = rem >= TAIL_MIN ? cnt : cnt - rem;
  g0 = p.tail_split == 1 ? b : b + big;
  g1 = p.tail_split == 1 ? b + big : en;
}

// m-tiles of BM rows of expert e's group, for the threads of a 256-thread
// workgroup in chunks of 256 experts.
template <int BM>
__device__ __forceinline__ uint32_t expert_mtiles(const GemmArgs& p, int e) {
  if (e >= p.E) return 0;
  int64_t rb, re;
  group_rows(p, e, rb, re);
  return (uint32_t)((re - rb + BM - 1) / BM);
}

// Inclusive prefix sum over the 256 threads of a workgroup; every thread also
// gets the workgroup total.  sh_waves: 4 words of LDS, free on entry.
__device__ __forceinline__ uint32_t block_scan_256(uint32_t v, uint32_t* sh_waves, uint32_t& total) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    uint32_t u = __shfl_up(v, o, 64);
    if (lane >= o) v += u;
  }
  if (lane == 63) sh_waves[wave] = v;
  __syncthreads();
  uint32_t before = 0;
  total = 0;
  for (int w = 0; w < 4; ++w) {
    if (w < wave) before += sh_waves[w];
    total += sh_waves[w];
  }
  __syncthreads();
  return before + v;
}

// Number of m-tiles over all experts (the same in every thread).  This and
// locate_tile are inlined: as calls they would take the kernel argument's
// address, which puts the whole argument block in scratch memory, and every
// later read of a field from there waits for all earlier memory operations.
template <int BM>
__device__ __forceinline__ uint32_t count_mtiles(const GemmArgs& p) {
  __shared__ uint32_t sh_waves[4];
  uint32_t carry = 0;
  for (int base = 0; base < p.E; base += 256) {
    uint32_t tot;
    block_scan_256(expert_mtiles<BM>(p, base + (int)threadIdx.x), sh_waves, tot);
    carry += tot;
  }
  return carry;
}

// Coordinates of logical tile `logical` (0 <= logical < m-tiles x ntiles).
// The logical tiles are the (expert, m-tile, n-tile) triples, expert by
// expert; inside an expert's block of cnt_e * ntiles tiles m-tile major and
// n-tile minor, so consecutive tiles cost the same (a ragged last m-tile
// comes as a run of ntiles cheap tiles).  Called by all threads of a
// 256-thread workgroup.
template <int BM>
__device__ __forceinline__ TileCoord locate_tile(const GemmArgs& p, int ntiles, int logical) {
  __shared__ int32_t sh_e, sh_mt, sh_nt;
  __shared__ uint32_t sh_waves[4];
  const int tid = threadIdx.x;
  const uint32_t m_key = (uint32_t)(logical / ntiles);   // lies inside expert e's m-tile range
  uint32_t carry = 0;
  for (int base = 0; base < p.E; base += 256) {
    const int e = base + tid;
    const uint32_t n = expert_mtiles<BM>(p, e);
    uint32_t tot;
    const uint32_t before = carry + block_scan_256(n, sh_waves, tot) - n;
    if (e < p.E && m_key >= before && m_key < before + n) {   // exactly one thread
      const int off = logical - (int)before * ntiles;          // position inside the expert's block
      sh_e = e;
      sh_mt = off / ntiles;
      sh_nt = off % ntiles;
    }
    carry += tot;
  }
  __syncthreads();
  TileCoord t;
  t.e = sh_e;
  t.n_tile = sh_nt;
  int64_t g0, g1;
  group_rows(p, t.e, g0, g1);
  t.row0 = g0 + (int64_t)sh_mt * BM;
  t.rows_valid = (int)((g1 - t.row0) < BM ? (g1 - t.row0) : BM);
  return t;
}

// This workgroup's tile in round `round`, from one pass over the group
// offsets: the m-tiles of every expert, their prefix sum and total T (T x
// ntiles real tiles), the XCD mapping of workgroup ids (hardware id h runs
// logical tiles (h % 8) * ceil(T' / 8) + h / 8 + r * G / 8 of the T' = T x
// ntiles real ones, r = 0, 1, .. for a grid of G workgroups), and the
// coordinates of that tile.  Returns false (the same in every thread) once
// the workgroup has none left.  With E <= 256 the offsets are read once (one
// memory round trip); more experts take a counting pass first.  Called by all
// threads of a 256-thread workgroup.
template <int BM>
__device__ __forceinline__ bool map_tile(const GemmArgs& p, int ntiles, TileCoord& t, int round = 0) {
  __shared__ int32_t sh_e, sh_mt, sh_nt;
  __shared__ int64_t sh_g0, sh_g1;
  __shared__ uint32_t sh_waves[4];
  const int tid = threadIdx.x;
  uint32_t total = 0;
  int64_t g0 = 0, g1 = 0;
  uint32_t n = 0, before = 0;
  if (p.E <= 256) {
    if (tid < p.E) {
      group_rows(p, tid, g0, g1);
      n = (uint32_t)((g1 - g0 + BM - 1) / BM);
    }
    before = block_scan_256(n, sh_waves, total) - n;
  } else {
    total = count_mtiles<BM>(p);
  }
  const int real = (int)total * ntiles;
  const int per_xcd = (real + 7) / 8;
  const int jt = (int)blockIdx.x / 8 + round * (int)(gridDim.x / 8);
  const int logical = ((int)blockIdx.x % 8) * per_xcd + jt;
  if (jt >= per_xcd || logical >= real) return false;
  if (p.E > 256) {
    t = uniform_tile(locate_tile<BM>(p, ntiles, logical));
    return true;
  }
  const uint32_t m_key = (uint32_t)(logical / ntiles);
  if (tid < p.E && m_key >= before && m_key < before + n) {    // exactly one thread
    const int off = logical - (int)before * ntiles;
    sh_e = tid;
    sh_mt = off / ntiles;
    sh_nt = off % ntiles;
    sh_g0 = g0;
    sh_g1 = g1;
  }
  __syncthreads();
  t.e = sh_e;
  t.n_tile = sh_nt;
  t.row0 = sh_g0 + (int64_t)sh_mt * BM;
  t.rows_valid = (int)((sh_g1 - t.row0) < BM ? (sh_g1 - t.row0) : BM);
  t = uniform_tile(t);
  return true;
}

// Weight row held at row r (0 .. BN-1) of an n-tile, or -1 past the end.
// With SwiGLU the 32-row groups alternate gate / up for the same 32
// channels, so a wave's column blocks j (gate) and j+1 (up) pair up.
template <int BN>
__device__ __forceinline__ int64_t weight_row(const GemmArgs& p, int n_tile, int r) {
  if (p.epilogue == 1) {
    const int64_t inter = p.N / 2;
    const int q = r >> 5;
    const int64_t i = (int64_t)n_tile * (BN / 2) + (q >> 1) * 32 + (r & 31);
    return i < inter ? ((q & 1) ? inter + i : i) : -1;
  }
  const int64_t n = (int64_t)n_tile * BN + r;
  return n < p.N ? n : -1;
}

// LDS floats a wave needs for the epilogue: one 32-row block of its
// 32 NJ columns, rows padded by 8 floats.
template <int NJ>
constexpr int epilogue_wave_floats() { return 32 * (NJ * 32 + 8); }

// Epilogue of a wave's MI x NJ blocks of 32 x 32 (tile rows wr0 + 32 i ..,
// tile columns wc0 + 32 j ..), block row by block row: prep(i) runs first
// (e.g. the compensation of row block i), then val(i, j, q) gives output
// element q of block (i, j) in fp32.  MFMA 32x32 output element q of lane l
// sits at row (q / 4) * 8 + (l / 32) * 4 + q % 4 and column l % 32 of its
// block.  rw_lds: the tile's row weights (scatter epilogue).  The caller has
// synchronized the workgroup, so `lds` (the wave's own region of
// epilogue_wave_floats<NJ>() floats) is free.
//
// F32 and scatter rows: when the tile's columns lie inside N and nothing is
// accumulated, every element goes straight out with one 4-byte buffer store
// per (block, q) (a 32-lane half writes one 128-byte row segment), through a
// buffer resource that ends at the last valid row, so rows past the group
// are dropped by the hardware and the stores need no branches.  Otherwise
// each 32-row block goes through LDS and leaves as whole row segments with
// 16-byte stores.
// Whether the F32 / scatter epilogue of this tile stores straight from the
// accumulators (the tile's columns inside N, nothing accumulated, row offsets
// within 31 bits); the same for every wave of the tile.
template <int MI, int BN, int EPI>
__device__ __forceinline__ bool epilogue_direct(const GemmArgs& p, const TileCoord& t) {
  if constexpr (EPI == 1) {
    return false;
  } else {
    const int64_t ld = EPI == 2 ? p.N : p.ldo;
    return (EPI == 2 || !p.accumulate) && (int64_t)(t.n_tile + 1) * BN <= p.N && ld * 4 * MI * 32 < (1ll << 31);
  }
}

template <int MI, int NJ, int BN, int EPI, typename Prep, typename Val>
__device__ __forceinline__ void gemm_epilogue_blocks(const GemmArgs& p, const TileCoord& t, int wr0, int wc0,
                                                     float* lds, const float* rw_lds, Prep&& prep, Val&& val) {
  constexpr int CS = NJ * 32 + 8;               // LDS row stride (floats)
  const int lane = threadIdx.x & 63, half = lane >> 5, l32 = lane & 31;
  if constexpr (EPI == 0 || EPI == 2) {
    constexpr bool scatter = EPI == 2;
    float* out = scatter ? p.y_rows : static_cast<float*>(p.out);
    const int64_t ld = scatter ? p.N : p.ldo;
    const int64_t n0 = (int64_t)t.n_tile * BN + wc0;     // first column of the wave
    if (epilogue_direct<MI, BN, EPI>(p, t)) {
      // rows wr0 .. rows_valid - 1 of the tile, as bytes from row wr0
      const int nrows = t.rows_valid - wr0 < 0 ? 0 : (t.rows_valid - wr0 > MI * 32 ? MI * 32 : t.rows_valid - wr0);
      const __amdgpu_buffer_rsrc_t r_out = make_rsrc(out + (t.row0 + wr0) * ld, (int64_t)nrows * ld * 4);
      const uint32_t voff = (uint32_t)(((int64_t)half * 4 * ld + n0 + l32) * 4);
#pragma unroll
      for (int i = 0; i < MI; ++i) {
        prep(i);
        float w[16];
#pragma unroll
        for (int q = 0; q < 16; ++q) w[q] = 1.0f;
        if constexpr (scatter) {
#pragma unroll
          for (int g = 0; g < 4; ++g) {
            const f32x4 v = *reinterpret_cast<const f32x4*>(rw_lds + wr0 + i * 32 + g * 8 + half * 4);
            w[4 * g] = v[0]; w[4 * g + 1] = v[1]; w[4 * g + 2] = v[2]; w[4 * g + 3] = v[3];
          }
        }
        // The scatter's rows are read once, by the combine: non-temporal
        // stores (cache policy bit 1, nt on gfx950).
#pragma unroll
        for (int q = 0; q < 16; ++q) {
          const uint32_t ro = (uint32_t)((i * 32 + (q >> 2) * 8 + (q & 3)) * ld * 4);
#pragma unroll
          for (int j = 0; j < NJ; ++j)
            __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(uint32_t, val(i, j, q) * w[q]), r_out,
                                                  (int)(voff + ro + j * 128), 0, scatter ? 2 : 0);
        }
      }
      return;
    }
    const bool vec = (ld & 3) == 0 && (reinterpret_cast<uintptr_t>(out) & 15) == 0;
    constexpr int LPR = NJ * 8;                         // lanes per row (4 floats each)
    constexpr int RPI = 64 / LPR;                       // rows per store instruction
#pragma unroll
    for (int i = 0; i < MI; ++i) {
      prep(i);
#pragma unroll
      for (int j = 0; j < NJ; ++j)
#pragma unroll
        for (int q = 0; q < 16; ++q)
          lds[((q >> 2) * 8 + half * 4 + (q & 3)) * CS + j * 32 + l32] = val(i, j, q);
      __builtin_amdgcn_s_waitcnt(0xc07f);               // lgkmcnt(0): the wave's writes landed
#pragma unroll
      for (int rr = 0; rr < 32; rr += RPI) {
        const int rl = rr + lane / LPR, c4 = (lane % LPR) * 4;
        const int r = wr0 + i * 32 + rl;
        const f32x4 v = *reinterpret_cast<const f32x4*>(lds + rl * CS + c4);
        if (r < t.rows_valid) {
          const int64_t s2 = t.row0 + r;
          const float w = scatter ? rw_lds[r] : 1.0f;      // row_weight[s2], staged in LDS
          float* dst = out + s2 * ld + n0 + c4;
          if (vec && n0 + c4 + 4 <= p.N) {
            f32x4 o = f32x4{v[0] * w, v[1] * w, v[2] * w, v[3] * w};
            if (!scatter && p.accumulate) {
              const f32x4 old = *reinterpret_cast<const f32x4*>(dst);
              o = f32x4{old[0] + o[0], old[1] + o[1], old[2] + o[2], old[3] + o[3]};
            }
            *reinterpret_cast<f32x4*>(dst) = o;
          } else {
#pragma unroll
            for (int u = 0; u < 4; ++u)
              if (n0 + c4 + u < p.N) dst[u] = !scatter && p.accumulate ? dst[u] + v[u] * w : v[u] * w;
          }
        }
      }
      __builtin_amdgcn_s_waitcnt(0xc07f);               // reads done before the next block's writes
    }
  } else {
    // SwiGLU: block j (even) is gate, j+1 is up, for the same 32 channels;
    // h = bf16(silu(gate) * up) staged as 16-bit values.  Rows q and q + 1 of
    // a lane are rounded by one packed convert.  The amax is taken over the
    // fp32 values and rounded once at the end: rounding to nearest is
    // monotonic, so that equals the largest |h| of the bf16 outputs.
    const int64_t inter = p.N / 2;
    uint16_t* out = static_cast<uint16_t*>(p.out);
    uint16_t* lh = reinterpret_cast<uint16_t*>(lds);
    constexpr int CH = NJ * 16;                         // channels of the wave
    constexpr int HS = CH + 8;                          // LDS row stride (halves)
    constexpr int LPR = CH / 8;                         // lanes per row (8 channels each)
    constexpr int RPI = 64 / LPR;
    const bool vec = (p.ldo & 7) == 0 && (reinterpret_cast<uintptr_t>(out) & 15) == 0;
    const int64_t c0 = (int64_t)t.n_tile * (BN / 2) + wc0 / 2;   // first channel of the wave
    float m = 0.0f;
#pragma unroll
    for (int i = 0; i < MI; ++i) {
      prep(i);
#pragma unroll
      for (int j = 0; j < NJ; j += 2) {
        const float col_ok = c0 + (j / 2) * 32 + l32 < inter ? 1.0f : 0.0f;
#pragma unroll
        for (int q = 0; q < 16; q += 2) {
          const int rl = (q >> 2) * 8 + half * 4 + (q & 3);        // rows rl and rl + 1
          const float v0 = silu_f32(val(i, j, q)) * val(i, j + 1, q);
          const float v1 = silu_f32(val(i, j, q + 1)) * val(i, j + 1, q + 1);
          const uint32_t hb = pack_bf16x2_rne(v0, v1);
          lh[rl * HS + (j / 2) * 32 + l32] = (uint16_t)hb;
          lh[(rl + 1) * HS + (j / 2) * 32 + l32] = (uint16_t)(hb >> 16);
          const float ok0 = wr0 + i * 32 + rl < t.rows_valid ? col_ok : 0.0f;
          const float ok1 = wr0 + i * 32 + rl + 1 < t.rows_valid ? col_ok : 0.0f;
          m = fmaxf(m, fmaxf(fabsf(v0 * ok0), fabsf(v1 * ok1)));
        }
      }
      __builtin_amdgcn_s_waitcnt(0xc07f);
#pragma unroll
      for (int rr = 0; rr < 32; rr += RPI) {
        const int rl = rr + lane / LPR, c8 = (lane % LPR) * 8;
        const int r = wr0 + i * 32 + rl;
        const u32x4 v = *reinterpret_cast<const u32x4*>(lh + rl * HS + c8);
        if (r < t.rows_valid) {
          uint16_t* dst = out + (t.row0 + r) * p.ldo + c0 + c8;
          if (vec && c0 + c8 + 8 <= inter) {
            *reinterpret_cast<u32x4*>(dst) = v;
          } else {
#pragma unroll
            for (int u = 0; u < 8; ++u)
              if (c0 + c8 + u < inter) dst[u] = (uint16_t)(v[u >> 1] >> (16 * (u & 1)));
          }
        }
      }
      __builtin_amdgcn_s_waitcnt(0xc07f);
    }
    m = __uint_as_float(f32_to_bf16_rne(m) << 16);
    if (p.out_amax) {
      m = wave_max(m);
      if (lane == 0) atomic_max_nonneg(p.out_amax, m);
    }
  }
}

// The plain form: output element = acc * scale.
template <int MI, int NJ, int BN, int EPI>
__device__ __forceinline__ void gemm_epilogue(const GemmArgs& p, const f32x16 (&acc)[MI][NJ],
                                              const TileCoord& t, int wr0, int wc0, float scale,
                                              float* lds, const float* rw_lds) {
  gemm_epilogue_blocks<MI, NJ, BN, EPI>(p, t, wr0, wc0, lds, rw_lds, [](int) {},
                                        [&](int i, int j, int q) { return acc[i][j][q] * scale; });
}

}  // namespace nvfp4
