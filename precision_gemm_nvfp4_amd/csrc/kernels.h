// Internal launchers of the HIP kernels (host side).  The C ABI in api.cpp
// validates arguments and carves the caller's workspace, then calls these.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <mutex>

namespace nvfp4 {

// quantize.hip
int amax_partials_count(int64_t M, int64_t K);
hipError_t launch_quantize(const void* x, int dtype, int64_t M, int64_t K, int64_t ldx,
                           const float* amax_in, uint8_t* codes, uint8_t* scales, float* g_out,
                           float* tile_partials, float* ws_partials, hipStream_t stream);
hipError_t launch_fill_f32(float* p, int64_t n, float v, hipStream_t stream);

// resq.hip
struct ResqWorkspace {
  int32_t* tile_start;   // [U+1] first 128-row score tile of each unit
  int32_t* slot_start;   // [U+1] first 32-row gather slot of each unit
  int32_t* tile_info;    // [max_slots][4] per score tile: unit (-1: none), first row, unit end
  int32_t* slot_info;    // [max_gather_slots][8] per gather slot: unit (-1: none), first row,
                         // end row, the unit's first and end slot
  float* partials;       // [max_slots, K] (unused when the caller gives tile partials)
  float* r_s;            // [rows_total, k]
  float* amax_part;      // [max_gather_slots]
};
int64_t resq_max_slots(int64_t rows_total, int64_t U);
int64_t resq_max_gather_slots(int64_t rows_total, int64_t U);
hipError_t launch_resq(const void* x, int dtype, int64_t x_rows, int64_t K, int64_t ldx,
                       const int32_t* row_index, const uint8_t* codes, const uint8_t* scales,
                       const float* g, const int64_t* unit_offsets, int64_t U, int64_t rows_total,
                       int32_t k, const float* tile_partials, int32_t* sel_idx, uint8_t* r_codes,
                       uint8_t* r_scales, float* r_global, const ResqWorkspace& ws,
                       hipStream_t stream, bool mx = false, bool masked = false);

// gemm.hip
struct GemmArgs {
  const uint8_t* a_codes;
  const uint8_t* a_scales;
  const float* a_global;
  const int32_t* a_row_index;
  int64_t a_rows;
  const int64_t* group_offsets;
  int32_t E;
  int64_t rows_total;
  int64_t K;
  const uint8_t* w_codes;
  const uint8_t* w_scales;
  const float* w_global;
  int64_t N;
  const int32_t* sel_idx;
  const uint8_t* r_codes;
  const uint8_t* r_scales;
  const float* r_global;
  int32_t kc;
  int epilogue;
  const float* row_weight;
  const int32_t* scatter_index;
  int64_t out_rows;
  void* out;
  int64_t ldo;
  float* out_amax;
  float* y_rows;         // scatter epilogue: row_weight * Y rows [rows_total, N] (workspace)
  bool combine_overwrite = false;   // scatter epilogue: out = the sums (else out += the sums)
  int block_m;           // rows per tile: 256, 128, 64, 32, or 0 to pick from the average group size
  int rw_lds_offset;     // set by the launcher: LDS byte offset of the scatter epilogue's row weights
  int a_global_per_group = 0;  // a_global holds one scale per group (else one for all)
  int accumulate = 0;          // F32 epilogue: out += Y instead of out = Y
  // set by the launcher: which rows of each group this launch covers (0 all;
  // 1 the 256-row tiles, plus a remainder of at least 96 rows; 2 the other
  // remainders) and at most how many workgroups it takes (0: one per tile,
  // else they go round the tiles)
  int tail_split = 0;
  int64_t grid_cap = 0;
};
int grouped_gemm_block_m(int64_t rows_total, int32_t E);
bool grouped_gemm_offsets_fit(int64_t a_rows, int64_t N, int64_t K);
hipError_t launch_grouped_gemm(const GemmArgs& a, hipStream_t stream);

// mxfp4.hip
hipError_t launch_mx_quantize(const void* x, int dtype, int64_t M, int64_t K, int64_t ldx,
                              uint8_t* codes, uint8_t* scales, float* tile_partials,
                              hipStream_t stream);
size_t mx_gemm_max_lds(int64_t K);
hipError_t launch_mx_grouped_gemm(const GemmArgs& a, hipStream_t stream);
hipError_t launch_mx_w4a8_grouped_gemm(const GemmArgs& a, hipStream_t stream);
hipError_t launch_mx8_quantize(const void* x, int dtype, int64_t M, int64_t K, int64_t ldx,
                               uint8_t* codes, uint8_t* scales, hipStream_t stream);

// combine.hip
size_t combine_workspace_bytes(int64_t rows, int64_t N, int64_t out_rows);
hipError_t launch_combine(const float* y_rows, int64_t rows, int64_t N,
                          const int32_t* scatter_index, int64_t out_rows, float* out, int64_t ldo,
                          bool overwrite, void* ws, hipStream_t stream);
// The two halves of launch_combine: the plan (row lists per output row, from
// scatter_index alone) and the ordered sum of the rows.
hipError_t launch_combine_plan(int64_t rows, int64_t N, const int32_t* scatter_index,
                               int64_t out_rows, void* ws, hipStream_t stream);
hipError_t launch_combine_rows(const float* y_rows, int64_t rows, int64_t N, int64_t out_rows,
                               float* out, int64_t ldo, bool overwrite, void* ws,
                               hipStream_t stream);

// trainer.hip
size_t qdq_workspace_bytes(int64_t nmat);
hipError_t launch_qdq(const __bf16* w, int64_t nmat, int64_t N, int64_t K, __bf16* w_qdq,
                      uint8_t* codes, uint8_t* scales, float* g, void* ws, hipStream_t stream);
hipError_t launch_guided(const void* x, int dtype, int64_t M, int64_t K, int64_t ldx,
                         const uint8_t* roll_codes, const uint8_t* roll_scales,
                         const float* roll_global, uint8_t* guided, __bf16* x_fq,
                         int64_t* hist, hipStream_t stream);
hipError_t launch_mx_qdq(const __bf16* w, int64_t rows, int64_t K, __bf16* w_qdq, uint8_t* codes,
                         uint8_t* scales, hipStream_t stream);
hipError_t launch_mx_guided(const void* x, int dtype, int64_t M, int64_t K, int64_t ldx,
                            const uint8_t* roll_codes, const uint8_t* roll_scales, uint8_t* guided,
                            __bf16* x_fq, int64_t* hist, hipStream_t stream);
hipError_t launch_mx_guided_record(const void* x, int dtype, int64_t M, int64_t K, int64_t ldx,
                                   const uint8_t* record, const uint8_t* roll_scales,
                                   uint8_t* guided, __bf16* x_fq, int64_t* moved,
                                   hipStream_t stream);
hipError_t launch_guided_record(const void* x, int dtype, int64_t M, int64_t K, int64_t ldx,
                                const uint8_t* record, const uint8_t* roll_scales,
                                const float* roll_global, uint8_t* guided, __bf16* x_fq,
                                int64_t* moved, hipStream_t stream);
hipError_t launch_guidance_pack(const uint8_t* codes, int64_t M, int64_t K, uint8_t* record,
                                hipStream_t stream);

// The library's second stream on the current device, with the two events
// that fork it from and join it into a caller's stream; the mutex keeps the
// record/wait pairs of concurrent host threads apart.  nullptr while the
// caller's stream is being captured into a graph, or where the stream or its
// events cannot be had: the work then stays on the caller's stream.
struct SideStream {
  std::mutex mu;
  bool tried = false;
  hipStream_t s = nullptr;
  hipEvent_t fork = nullptr, join = nullptr;
};
SideStream* side_stream(hipStream_t caller);

}  // namespace nvfp4
