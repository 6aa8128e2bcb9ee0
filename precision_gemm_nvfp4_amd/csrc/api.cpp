// C ABI of the library: argument validation, workspace carving, launches.
// Every check runs on the host before anything is enqueued, so a failing call
// writes nothing.  See include/nvfp4_resq.h for the contract of each entry.
#include <hip/hip_runtime.h>

#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <mutex>

#include "../../include/nvfp4_resq.h"
#include "kernels.h"

namespace {

thread_local char g_err[512] = "";

int fail(int code, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
  return code;
}

int ok() {
  g_err[0] = '\0';
  return NVFP4_OK;
}

int hip_status(hipError_t e, const char* what) {
  if (e != hipSuccess) return fail(NVFP4_EHIP, "%s: %s", what, hipGetErrorString(e));
  return ok();
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

size_t align256(size_t n) { return (n + 255) & ~size_t(255); }

int elem_size(int dtype) { return dtype == NVFP4_DTYPE_BF16 ? 2 : 4; }

// Common checks of an activation operand x [M, ldx] with K used columns.
int check_act(const void* x, int dtype, int64_t M, int64_t K, int64_t ldx, const char* fn) {
  if (dtype != NVFP4_DTYPE_BF16 && dtype != NVFP4_DTYPE_F32)
    return fail(NVFP4_EUNSUPPORTED, "%s: dtype %d is not BF16 (0) or F32 (1)", fn, dtype);
  if (M < 0 || K <= 0) return fail(NVFP4_EINVAL, "%s: M=%lld K=%lld", fn, (long long)M, (long long)K);
  if (K % 16 != 0) return fail(NVFP4_EINVAL, "%s: K=%lld is not a multiple of 16", fn, (long long)K);
  if (ldx < K) return fail(NVFP4_EINVAL, "%s: ldx=%lld < K=%lld", fn, (long long)ldx, (long long)K);
  if ((ldx * elem_size(dtype)) % 16 != 0)
    return fail(NVFP4_EINVAL, "%s: row stride ldx=%lld elements is not a multiple of 16 bytes", fn,
                (long long)ldx);
  if (M > 0 && !x) return fail(NVFP4_EINVAL, "%s: x is NULL", fn);
  if (x && !aligned16(x)) return fail(NVFP4_EINVAL, "%s: x is not 16-byte aligned", fn);
  return NVFP4_OK;
}

}  // namespace

extern "C" {

int nvfp4_version(void) { return 100; }

const char* nvfp4_last_error(void) { return g_err; }

// ---------------------------------------------------------------------------
size_t nvfp4_quantize_workspace_size(int64_t M, int64_t K) {
  return align256((size_t)(nvfp4::amax_partials_count(M, K) + 1) * sizeof(float));
}

}  // extern "C"

namespace {
// Validation shared by nvfp4_quantize and nvfp4_quantize_noalloc (everything
// but the workspace).  Returns NVFP4_OK, or the status of the first failure.
int check_quantize(const void* x, int dtype, int64_t M, int64_t K, int64_t ldx,
                   const uint8_t* codes, const uint8_t* scales, const float* tile_partials,
                   const char* fn) {
  if (int s = check_act(x, dtype, M, K, ldx, fn)) return s;
  if (M > 0 && (!codes || !scales)) return fail(NVFP4_EINVAL, "%s: codes/scales are NULL", fn);
  if (codes && !aligned16(codes)) return fail(NVFP4_EINVAL, "%s: codes not 16-byte aligned", fn);
  if (tile_partials && !aligned16(tile_partials))
    return fail(NVFP4_EINVAL, "%s: tile_partials not 16-byte aligned", fn);
  return NVFP4_OK;
}

// ---- scratch of nvfp4_quantize_noalloc --------------------------------------
// The amax partial maxima: amax_partials_count(M, K) floats, at most 256 for
// any shape (the count is capped), within this bound.
// Every GPU the library runs on holds its own copy of the array until the
// process ends.  In host code `scratch` names a host-side stand-in, never a
// device address: the device address comes from hipGetSymbolAddress, taken
// once per device with that device current and kept in g_scratch_ptr.
constexpr size_t kScratchBytes = 8192;
static __device__ __align__(256) unsigned char scratch[kScratchBytes];
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// The device address of the current device's scratch (nullptr and a status
// in *status on failure).
void* scratch_of_current_device(int* status, const char* fn) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) {
    *status = fail(NVFP4_EHIP, "%s: hipGetDevice: %s", fn, hipGetErrorString(e));
    return nullptr;
  }
  if (dev < 0 || dev >= kMaxDevices) {
    *status = fail(NVFP4_EUNSUPPORTED, "%s: device %d >= %d", fn, dev, kMaxDevices);
    return nullptr;
  }
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* ptr = nullptr;
    e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !ptr) {
      *status = fail(NVFP4_EHIP, "%s: hipGetSymbolAddress(scratch): %s", fn, hipGetErrorString(e));
      return nullptr;
    }
    g_scratch_ptr[dev] = ptr;
  }
  *status = NVFP4_OK;
  return g_scratch_ptr[dev];
}
}  // namespace

extern "C" {

int nvfp4_quantize_noalloc(const void* x, int dtype, int64_t M, int64_t K, int64_t ldx,
                           const float* amax_in, uint8_t* codes, uint8_t* scales, float* g_out,
                           float* tile_partials, void* stream) {
  const char* fn = "nvfp4_quantize_noalloc";
  if (int s = check_quantize(x, dtype, M, K, ldx, codes, scales, tile_partials, fn)) return s;
  const size_t need = nvfp4_quantize_workspace_size(M, K);
  if (need > kScratchBytes)
    return fail(NVFP4_EUNSUPPORTED, "%s: needs %zu bytes of scratch, more than its %zu", fn, need,
                kScratchBytes);
  int status = NVFP4_OK;
  void* ptr = scratch_of_current_device(&status, fn);
  if (!ptr) return status;
  hipStream_t st = static_cast<hipStream_t>(stream);
  if (M == 0) {
    if (g_out) return hip_status(nvfp4::launch_fill_f32(g_out, 1, 1.0f, st), fn);
    return ok();
  }
  return hip_status(nvfp4::launch_quantize(x, dtype, M, K, ldx, amax_in, codes, scales, g_out,
                                           tile_partials, static_cast<float*>(ptr), st),
                    fn);
}

int nvfp4_quantize(const void* x, int dtype, int64_t M, int64_t K, int64_t ldx,
                   const float* amax_in, uint8_t* codes, uint8_t* scales, float* g_out,
                   float* tile_partials, void* ws, size_t ws_bytes, void* stream) {
  const char* fn = "nvfp4_quantize";
  if (int s = check_quantize(x, dtype, M, K, ldx, codes, scales, tile_partials, fn)) return s;
  hipStream_t st = static_cast<hipStream_t>(stream);
  if (M == 0) {
    if (g_out) return hip_status(nvfp4::launch_fill_f32(g_out, 1, 1.0f, st), fn);
    return ok();
  }
  if (!amax_in) {
    if (!ws) return fail(NVFP4_EWORKSPACE, "%s: workspace is NULL", fn);
    if (ws_bytes < nvfp4_quantize_workspace_size(M, K))
      return fail(NVFP4_EWORKSPACE, "%s: workspace %zu < %zu bytes", fn, ws_bytes,
                  nvfp4_quantize_workspace_size(M, K));
  }
  return hip_status(nvfp4::launch_quantize(x, dtype, M, K, ldx, amax_in, codes, scales, g_out,
                                           tile_partials, static_cast<float*>(ws), st),
                    fn);
}

// ---------------------------------------------------------------------------
size_t resq_select_and_requant_workspace_size(int64_t K, int64_t rows_total, int64_t U, int32_t k) {
  const int64_t slots = nvfp4::resq_max_slots(rows_total, U);
  const int64_t gslots = nvfp4::resq_max_gather_slots(rows_total, U);
  return 2 * align256((size_t)(U + 1) * 4) + align256((size_t)slots * 16) +
         align256((size_t)gslots * 32) + align256((size_t)slots * K * 4) +
         align256((size_t)rows_total * k * 4) + align256((size_t)gslots * 4);
}

}  // extern "C"

namespace {
// The compact (masked = false) and dense-mask residual steps share validation,
// workspace and the selection; they differ in the requantized output.
int resq_entry(const void* x, int dtype, int64_t x_rows, int64_t K, int64_t ldx,
               const int32_t* row_index, const uint8_t* codes, const uint8_t* scales,
               const float* g, const int64_t* unit_offsets, int64_t U, int64_t rows_total,
               int32_t k, const float* tile_partials, int32_t* sel_idx, uint8_t* r_codes,
               uint8_t* r_scales, float* r_global, void* ws, size_t ws_bytes, void* stream,
               bool masked, const char* fn) {
  if (int s = check_act(x, dtype, x_rows, K, ldx, fn)) return s;
  if (K > 16384) return fail(NVFP4_EUNSUPPORTED, "%s: K=%lld > 16384", fn, (long long)K);
  if (k < 16 || k % 16 != 0 || k > K)
    return fail(NVFP4_EINVAL, "%s: k=%d must be a multiple of 16 in [16, K]", fn, k);
  if (U < 0 || rows_total < 0) return fail(NVFP4_EINVAL, "%s: U or rows_total negative", fn);
  if (U > 2147483647LL || rows_total > 2147483647LL)
    return fail(NVFP4_EUNSUPPORTED, "%s: U or rows_total above 2^31-1", fn);
  if (!codes || !scales || !g) return fail(NVFP4_EINVAL, "%s: codes/scales/g NULL", fn);
  if (U > 0 && (!sel_idx || !r_global)) return fail(NVFP4_EINVAL, "%s: sel_idx/r_global NULL", fn);
  if (rows_total > 0 && (!r_codes || !r_scales))
    return fail(NVFP4_EINVAL, "%s: r_codes/r_scales NULL", fn);
  if (r_codes && !aligned16(r_codes)) return fail(NVFP4_EINVAL, "%s: r_codes not aligned", fn);
  if (tile_partials) {
    if (row_index) return fail(NVFP4_EINVAL, "%s: tile_partials needs row_index == NULL", fn);
    if (rows_total != x_rows || U != (x_rows + 127) / 128)
      return fail(NVFP4_EINVAL, "%s: tile_partials needs rows_total == x_rows and U == ceil(x_rows/128)", fn);
  } else if (U > 0 && !unit_offsets) {
    return fail(NVFP4_EINVAL, "%s: unit_offsets NULL", fn);
  }
  if (!ws) return fail(NVFP4_EWORKSPACE, "%s: workspace is NULL", fn);
  const size_t need = resq_select_and_requant_workspace_size(K, rows_total, U, k);
  if (ws_bytes < need) return fail(NVFP4_EWORKSPACE, "%s: workspace %zu < %zu bytes", fn, ws_bytes, need);
  if (U == 0) return ok();
  char* w = static_cast<char*>(ws);
  const int64_t slots = nvfp4::resq_max_slots(rows_total, U);
  nvfp4::ResqWorkspace rw;
  rw.tile_start = reinterpret_cast<int32_t*>(w);
  w += align256((size_t)(U + 1) * 4);
  rw.slot_start = reinterpret_cast<int32_t*>(w);
  w += align256((size_t)(U + 1) * 4);
  rw.tile_info = reinterpret_cast<int32_t*>(w);
  w += align256((size_t)slots * 16);
  rw.slot_info = reinterpret_cast<int32_t*>(w);
  w += align256((size_t)nvfp4::resq_max_gather_slots(rows_total, U) * 32);
  rw.partials = reinterpret_cast<float*>(w);
  w += align256((size_t)slots * K * 4);
  rw.r_s = reinterpret_cast<float*>(w);
  w += align256((size_t)rows_total * k * 4);
  rw.amax_part = reinterpret_cast<float*>(w);
  return hip_status(nvfp4::launch_resq(x, dtype, x_rows, K, ldx, row_index, codes, scales, g,
                                       unit_offsets, U, rows_total, k, tile_partials, sel_idx,
                                       r_codes, r_scales, r_global, rw,
                                       static_cast<hipStream_t>(stream), false, masked),
                    fn);
}
}  // namespace

extern "C" {

int resq_select_and_requant(const void* x, int dtype, int64_t x_rows, int64_t K, int64_t ldx,
                            const int32_t* row_index, const uint8_t* codes, const uint8_t* scales,
                            const float* g, const int64_t* unit_offsets, int64_t U,
                            int64_t rows_total, int32_t k, const float* tile_partials,
                            int32_t* sel_idx, uint8_t* r_codes, uint8_t* r_scales,
                            float* r_global, void* ws, size_t ws_bytes, void* stream) {
  return resq_entry(x, dtype, x_rows, K, ldx, row_index, codes, scales, g, unit_offsets, U,
                    rows_total, k, tile_partials, sel_idx, r_codes, r_scales, r_global, ws,
                    ws_bytes, stream, false, "resq_select_and_requant");
}

int resq_mask_select_and_requant(const void* x, int dtype, int64_t x_rows, int64_t K, int64_t ldx,
                                 const int32_t* row_index, const uint8_t* codes,
                                 const uint8_t* scales, const float* g,
                                 const int64_t* unit_offsets, int64_t U, int64_t rows_total,
                                 int32_t k, const float* tile_partials, int32_t* sel_idx,
                                 uint8_t* m_codes, uint8_t* m_scales, float* m_global, void* ws,
                                 size_t ws_bytes, void* stream) {
  return resq_entry(x, dtype, x_rows, K, ldx, row_index, codes, scales, g, unit_offsets, U,
                    rows_total, k, tile_partials, sel_idx, m_codes, m_scales, m_global, ws,
                    ws_bytes, stream, true, "resq_mask_select_and_requant");
}

// ---------------------------------------------------------------------------
// NVFP4_EPI_SCATTER_F32 is the scatter-add epilogue into zeros: the same GEMM
// kernels, with the combine writing its sums instead of adding them to out.
static bool scatter_overwrite(int& epilogue) {
  if (epilogue != NVFP4_EPI_SCATTER_F32) return false;
  epilogue = NVFP4_EPI_SCATTER_ADD_F32;
  return true;
}

size_t moe_w4a4_grouped_gemm_workspace_size(int32_t E, int64_t rows_total, int64_t N, int64_t K,
                                            int epilogue, int64_t out_rows) {
  (void)E; (void)K;
  scatter_overwrite(epilogue);
  if (epilogue != NVFP4_EPI_SCATTER_ADD_F32 || rows_total < 0 || N < 0 || out_rows < 0) return 0;
  return nvfp4::combine_workspace_bytes(rows_total, N, out_rows);
}

int moe_w4a4_grouped_gemm(const uint8_t* a_codes, const uint8_t* a_scales, const float* a_global,
                          const int32_t* a_row_index, int64_t a_rows,
                          const int64_t* group_offsets, int32_t E, int64_t rows_total, int64_t K,
                          const uint8_t* w_codes, const uint8_t* w_scales, const float* w_global,
                          int64_t N, const int32_t* sel_idx, const uint8_t* r_codes,
                          const uint8_t* r_scales, const float* r_global, int32_t kc,
                          int epilogue, const float* row_weight, const int32_t* scatter_index,
                          int64_t out_rows, void* out, int64_t ldo, float* out_amax,
                          void* ws, size_t ws_bytes, void* stream) {
  const char* fn = "moe_w4a4_grouped_gemm";
  const bool overwrite = scatter_overwrite(epilogue);
  if (E <= 0 || K <= 0 || N <= 0 || rows_total < 0 || a_rows < 0)
    return fail(NVFP4_EINVAL, "%s: E=%d K=%lld N=%lld rows_total=%lld", fn, E, (long long)K,
                (long long)N, (long long)rows_total);
  if (K % 64 != 0) return fail(NVFP4_EINVAL, "%s: K=%lld is not a multiple of 64", fn, (long long)K);
  if (K > 65536) return fail(NVFP4_EUNSUPPORTED, "%s: K=%lld > 65536", fn, (long long)K);
  if (rows_total > 2147483647LL) return fail(NVFP4_EUNSUPPORTED, "%s: rows_total above 2^31-1", fn);
  if (!group_offsets || !w_codes || !w_scales || !w_global || !a_global || !out)
    return fail(NVFP4_EINVAL, "%s: required pointer is NULL", fn);
  if (rows_total > 0 && (!a_codes || !a_scales)) return fail(NVFP4_EINVAL, "%s: a_codes/a_scales NULL", fn);
  if (rows_total > 0 && a_rows < 1)      // the kernel reads row 0 in place of rows outside a tile
    return fail(NVFP4_EINVAL, "%s: a_rows must be at least 1 when rows_total > 0", fn);
  if (!nvfp4::grouped_gemm_offsets_fit(a_rows, N, K))
    return fail(NVFP4_EUNSUPPORTED, "%s: A codes or one expert's W codes span 4 GiB or more", fn);
  if (!aligned16(w_codes) || (a_codes && !aligned16(a_codes)))
    return fail(NVFP4_EINVAL, "%s: codes not 16-byte aligned", fn);
  if (sel_idx) {
    if (kc < 16 || kc % 16 != 0 || kc > K || kc > 128)
      return fail(NVFP4_EINVAL, "%s: kc=%d must be a multiple of 16 in [16, min(K, 128)]", fn, kc);
    if (rows_total > 0 && (!r_codes || !r_scales)) return fail(NVFP4_EINVAL, "%s: r_codes/r_scales NULL", fn);
    if (!r_global) return fail(NVFP4_EINVAL, "%s: r_global NULL", fn);
  }
  if (epilogue == NVFP4_EPI_F32) {
    if (ldo < N) return fail(NVFP4_EINVAL, "%s: ldo=%lld < N", fn, (long long)ldo);
  } else if (epilogue == NVFP4_EPI_SWIGLU_BF16) {
    if (N % 2 != 0) return fail(NVFP4_EINVAL, "%s: SwiGLU needs N even", fn);
    if (ldo < N / 2) return fail(NVFP4_EINVAL, "%s: ldo=%lld < N/2", fn, (long long)ldo);
  } else if (epilogue == NVFP4_EPI_SCATTER_ADD_F32) {
    if (ldo < N) return fail(NVFP4_EINVAL, "%s: ldo=%lld < N", fn, (long long)ldo);
    if (!row_weight || !scatter_index) return fail(NVFP4_EINVAL, "%s: scatter needs row_weight and scatter_index", fn);
    if (out_rows < 0 || out_rows > 2147483647LL)
      return fail(NVFP4_EINVAL, "%s: out_rows must be in [0, 2^31-1]", fn);
    const size_t need = moe_w4a4_grouped_gemm_workspace_size(E, rows_total, N, K, epilogue, out_rows);
    if (!ws || ws_bytes < need)
      return fail(NVFP4_EWORKSPACE, "%s: scatter epilogue needs a %zu-byte workspace", fn, need);
  } else {
    return fail(NVFP4_EINVAL, "%s: unknown epilogue %d", fn, epilogue);
  }
  nvfp4::GemmArgs a;
  a.a_codes = a_codes; a.a_scales = a_scales; a.a_global = a_global;
  a.a_row_index = a_row_index; a.a_rows = a_rows;
  a.group_offsets = group_offsets; a.E = E; a.rows_total = rows_total; a.K = K;
  a.w_codes = w_codes; a.w_scales = w_scales; a.w_global = w_global; a.N = N;
  a.sel_idx = sel_idx; a.r_codes = r_codes; a.r_scales = r_scales; a.r_global = r_global;
  a.kc = sel_idx ? kc : 0;
  a.epilogue = epilogue; a.row_weight = row_weight; a.scatter_index = scatter_index;
  a.out_rows = out_rows; a.out = out; a.ldo = ldo;
  a.out_amax = epilogue == NVFP4_EPI_SWIGLU_BF16 ? out_amax : nullptr;
  a.block_m = 0;
  a.y_rows = epilogue == NVFP4_EPI_SCATTER_ADD_F32 ? static_cast<float*>(ws) : nullptr;
  a.combine_overwrite = overwrite;
  return hip_status(nvfp4::launch_grouped_gemm(a, static_cast<hipStream_t>(stream)), fn);
}

int moe_w4a4_masked_comp_gemm(const uint8_t* m_codes, const uint8_t* m_scales,
                              const float* m_global, const int64_t* group_offsets, int32_t E,
                              int64_t rows_total, int64_t K, const uint8_t* w_codes,
                              const uint8_t* w_scales, const float* w_global, int64_t N,
                              float* out, int64_t ldo, void* stream) {
  const char* fn = "moe_w4a4_masked_comp_gemm";
  if (E <= 0 || K <= 0 || N <= 0 || rows_total < 0)
    return fail(NVFP4_EINVAL, "%s: E=%d K=%lld N=%lld rows_total=%lld", fn, E, (long long)K,
                (long long)N, (long long)rows_total);
  if (K % 64 != 0) return fail(NVFP4_EINVAL, "%s: K=%lld is not a multiple of 64", fn, (long long)K);
  if (K > 65536) return fail(NVFP4_EUNSUPPORTED, "%s: K=%lld > 65536", fn, (long long)K);
  if (rows_total > 2147483647LL) return fail(NVFP4_EUNSUPPORTED, "%s: rows_total above 2^31-1", fn);
  if (!group_offsets || !w_codes || !w_scales || !w_global || !m_global || !out)
    return fail(NVFP4_EINVAL, "%s: required pointer is NULL", fn);
  if (rows_total > 0 && (!m_codes || !m_scales)) return fail(NVFP4_EINVAL, "%s: m_codes/m_scales NULL", fn);
  if (!aligned16(w_codes) || (m_codes && !aligned16(m_codes)))
    return fail(NVFP4_EINVAL, "%s: codes not 16-byte aligned", fn);
  if (ldo < N) return fail(NVFP4_EINVAL, "%s: ldo=%lld < N", fn, (long long)ldo);
  if (!nvfp4::grouped_gemm_offsets_fit(rows_total, N, K))
    return fail(NVFP4_EUNSUPPORTED, "%s: m_codes or one expert's W codes span 4 GiB or more", fn);
  if (rows_total == 0) return ok();
  nvfp4::GemmArgs a;
  a.a_codes = m_codes; a.a_scales = m_scales; a.a_global = m_global;
  a.a_global_per_group = 1;
  a.a_row_index = nullptr; a.a_rows = rows_total;
  a.group_offsets = group_offsets; a.E = E; a.rows_total = rows_total; a.K = K;
  a.w_codes = w_codes; a.w_scales = w_scales; a.w_global = w_global; a.N = N;
  a.sel_idx = nullptr; a.r_codes = nullptr; a.r_scales = nullptr; a.r_global = nullptr;
  a.kc = 0;
  a.epilogue = NVFP4_EPI_F32; a.row_weight = nullptr; a.scatter_index = nullptr;
  a.out_rows = 0; a.out = out; a.ldo = ldo; a.out_amax = nullptr;
  a.block_m = 0; a.y_rows = nullptr;
  a.accumulate = 1;
  return hip_status(nvfp4::launch_grouped_gemm(a, static_cast<hipStream_t>(stream)), fn);
}

// ---------------------------------------------------------------------------
// MXFP4 variant
// ---------------------------------------------------------------------------
int mxfp4_quantize(const void* x, int dtype, int64_t M, int64_t K, int64_t ldx, uint8_t* codes,
                   uint8_t* scales, float* tile_partials, void* stream) {
  const char* fn = "mxfp4_quantize";
  if (int s = check_act(x, dtype, M, K, ldx, fn)) return s;
  if (K % 32 != 0) return fail(NVFP4_EINVAL, "%s: K=%lld is not a multiple of 32", fn, (long long)K);
  if (M > 0 && (!codes || !scales)) return fail(NVFP4_EINVAL, "%s: codes/scales are NULL", fn);
  if ((codes && !aligned16(codes)) || (tile_partials && !aligned16(tile_partials)))
    return fail(NVFP4_EINVAL, "%s: codes/tile_partials not 16-byte aligned", fn);
  return hip_status(nvfp4::launch_mx_quantize(x, dtype, M, K, ldx, codes, scales, tile_partials,
                                              static_cast<hipStream_t>(stream)),
                    fn);
}

size_t mxfp4_resq_select_and_requant_workspace_size(int64_t K, int64_t rows_total, int64_t U,
                                                    int32_t k) {
  return resq_select_and_requant_workspace_size(K, rows_total, U, k);
}

int mxfp4_resq_select_and_requant(const void* x, int dtype, int64_t x_rows, int64_t K, int64_t ldx,
                                  const int32_t* row_index, const uint8_t* codes,
                                  const uint8_t* scales, const int64_t* unit_offsets, int64_t U,
                                  int64_t rows_total, int32_t k, const float* tile_partials,
                                  int32_t* sel_idx, uint8_t* r_codes, uint8_t* r_scales, void* ws,
                                  size_t ws_bytes, void* stream) {
  const char* fn = "mxfp4_resq_select_and_requant";
  if (int s = check_act(x, dtype, x_rows, K, ldx, fn)) return s;
  if (K % 32 != 0) return fail(NVFP4_EINVAL, "%s: K=%lld is not a multiple of 32", fn, (long long)K);
  if (K > 16384) return fail(NVFP4_EUNSUPPORTED, "%s: K=%lld > 16384", fn, (long long)K);
  if (k < 32 || k % 32 != 0 || k > K)
    return fail(NVFP4_EINVAL, "%s: k=%d must be a multiple of 32 in [32, K]", fn, k);
  if (U < 0 || rows_total < 0) return fail(NVFP4_EINVAL, "%s: U or rows_total negative", fn);
  if (U > 2147483647LL || rows_total > 2147483647LL)
    return fail(NVFP4_EUNSUPPORTED, "%s: U or rows_total above 2^31-1", fn);
  if (!codes || !scales) return fail(NVFP4_EINVAL, "%s: codes/scales NULL", fn);
  if (U > 0 && !sel_idx) return fail(NVFP4_EINVAL, "%s: sel_idx NULL", fn);
  if (rows_total > 0 && (!r_codes || !r_scales))
    return fail(NVFP4_EINVAL, "%s: r_codes/r_scales NULL", fn);
  if (r_codes && !aligned16(r_codes)) return fail(NVFP4_EINVAL, "%s: r_codes not aligned", fn);
  if (tile_partials) {
    if (row_index) return fail(NVFP4_EINVAL, "%s: tile_partials needs row_index == NULL", fn);
    if (rows_total != x_rows || U != (x_rows + 127) / 128)
      return fail(NVFP4_EINVAL, "%s: tile_partials needs rows_total == x_rows and U == ceil(x_rows/128)", fn);
  } else if (U > 0 && !unit_offsets) {
    return fail(NVFP4_EINVAL, "%s: unit_offsets NULL", fn);
  }
  if (!ws) return fail(NVFP4_EWORKSPACE, "%s: workspace is NULL", fn);
  const size_t need = resq_select_and_requant_workspace_size(K, rows_total, U, k);
  if (ws_bytes < need) return fail(NVFP4_EWORKSPACE, "%s: workspace %zu < %zu bytes", fn, ws_bytes, need);
  if (U == 0) return ok();
  char* w = static_cast<char*>(ws);
  const int64_t slots = nvfp4::resq_max_slots(rows_total, U);
  nvfp4::ResqWorkspace rw;
  rw.tile_start = reinterpret_cast<int32_t*>(w);
  w += align256((size_t)(U + 1) * 4);
  rw.slot_start = reinterpret_cast<int32_t*>(w);
  w += align256((size_t)(U + 1) * 4);
  rw.tile_info = reinterpret_cast<int32_t*>(w);
  w += align256((size_t)slots * 16);
  rw.slot_info = reinterpret_cast<int32_t*>(w);
  w += align256((size_t)nvfp4::resq_max_gather_slots(rows_total, U) * 32);
  rw.partials = reinterpret_cast<float*>(w);
  w += align256((size_t)slots * K * 4);
  rw.r_s = reinterpret_cast<float*>(w);
  w += align256((size_t)rows_total * k * 4);
  rw.amax_part = reinterpret_cast<float*>(w);
  return hip_status(nvfp4::launch_resq(x, dtype, x_rows, K, ldx, row_index, codes, scales, nullptr,
                                       unit_offsets, U, rows_total, k, tile_partials, sel_idx,
                                       r_codes, r_scales, nullptr, rw,
                                       static_cast<hipStream_t>(stream), true),
                    fn);
}

size_t moe_mxfp4_grouped_gemm_workspace_size(int32_t E, int64_t rows_total, int64_t N, int64_t K,
                                             int epilogue, int64_t out_rows) {
  return moe_w4a4_grouped_gemm_workspace_size(E, rows_total, N, K, epilogue, out_rows);
}

int moe_mxfp4_grouped_gemm(const uint8_t* a_codes, const uint8_t* a_scales,
                           const int32_t* a_row_index, int64_t a_rows,
                           const int64_t* group_offsets, int32_t E, int64_t rows_total, int64_t K,
                           const uint8_t* w_codes, const uint8_t* w_scales, int64_t N,
                           const int32_t* sel_idx, const uint8_t* r_codes, const uint8_t* r_scales,
                           int32_t kc, int epilogue, const float* row_weight,
                           const int32_t* scatter_index, int64_t out_rows, void* out, int64_t ldo,
                           float* out_amax, void* ws, size_t ws_bytes, void* stream) {
  const char* fn = "moe_mxfp4_grouped_gemm";
  const bool overwrite = scatter_overwrite(epilogue);
  if (E <= 0 || K <= 0 || N <= 0 || rows_total < 0 || a_rows < 0)
    return fail(NVFP4_EINVAL, "%s: E=%d K=%lld N=%lld rows_total=%lld", fn, E, (long long)K,
                (long long)N, (long long)rows_total);
  if (K % 128 != 0) return fail(NVFP4_EINVAL, "%s: K=%lld is not a multiple of 128", fn, (long long)K);
  if (K > 65536) return fail(NVFP4_EUNSUPPORTED, "%s: K=%lld > 65536", fn, (long long)K);
  if (a_rows * (K / 2) >= (1LL << 32) || N * (K / 2) >= (1LL << 32))   // 32-bit lane offsets
    return fail(NVFP4_EUNSUPPORTED, "%s: A or one expert's W spans 4 GiB or more", fn);
  if (rows_total > 2147483647LL) return fail(NVFP4_EUNSUPPORTED, "%s: rows_total above 2^31-1", fn);
  if (!group_offsets || !w_codes || !w_scales || !out)
    return fail(NVFP4_EINVAL, "%s: required pointer is NULL", fn);
  if (rows_total > 0 && (!a_codes || !a_scales)) return fail(NVFP4_EINVAL, "%s: a_codes/a_scales NULL", fn);
  if (rows_total > 0 && a_rows < 1)      // the kernel reads row 0 in place of rows outside a tile
    return fail(NVFP4_EINVAL, "%s: a_rows must be at least 1 when rows_total > 0", fn);
  if (!nvfp4::grouped_gemm_offsets_fit(a_rows, N, K))
    return fail(NVFP4_EUNSUPPORTED, "%s: A codes or one expert's W codes span 4 GiB or more", fn);
  if (!aligned16(w_codes) || (a_codes && !aligned16(a_codes)))
    return fail(NVFP4_EINVAL, "%s: codes not 16-byte aligned", fn);
  if ((reinterpret_cast<uintptr_t>(w_scales) & 3u) || (reinterpret_cast<uintptr_t>(a_scales) & 3u))
    return fail(NVFP4_EINVAL, "%s: scales not 4-byte aligned", fn);
  if (sel_idx) {
    if (kc < 32 || kc % 32 != 0 || kc > K || kc > 128)
      return fail(NVFP4_EINVAL, "%s: kc=%d must be a multiple of 32 in [32, min(K, 128)]", fn, kc);
    if (rows_total > 0 && (!r_codes || !r_scales)) return fail(NVFP4_EINVAL, "%s: r_codes/r_scales NULL", fn);
    if (r_codes && !aligned16(r_codes)) return fail(NVFP4_EINVAL, "%s: r_codes not 16-byte aligned", fn);
  }
  if (epilogue == NVFP4_EPI_F32) {
    if (ldo < N) return fail(NVFP4_EINVAL, "%s: ldo=%lld < N", fn, (long long)ldo);
  } else if (epilogue == NVFP4_EPI_SWIGLU_BF16) {
    if (N % 2 != 0) return fail(NVFP4_EINVAL, "%s: SwiGLU needs N even", fn);
    if (ldo < N / 2) return fail(NVFP4_EINVAL, "%s: ldo=%lld < N/2", fn, (long long)ldo);
  } else if (epilogue == NVFP4_EPI_SCATTER_ADD_F32) {
    if (ldo < N) return fail(NVFP4_EINVAL, "%s: ldo=%lld < N", fn, (long long)ldo);
    if (!row_weight || !scatter_index) return fail(NVFP4_EINVAL, "%s: scatter needs row_weight and scatter_index", fn);
    if (out_rows < 0 || out_rows > 2147483647LL)
      return fail(NVFP4_EINVAL, "%s: out_rows must be in [0, 2^31-1]", fn);
    const size_t need = moe_mxfp4_grouped_gemm_workspace_size(E, rows_total, N, K, epilogue, out_rows);
    if (!ws || ws_bytes < need)
      return fail(NVFP4_EWORKSPACE, "%s: scatter epilogue needs a %zu-byte workspace", fn, need);
  } else {
    return fail(NVFP4_EINVAL, "%s: unknown epilogue %d", fn, epilogue);
  }
  nvfp4::GemmArgs a = {};
  a.a_codes = a_codes; a.a_scales = a_scales;
  a.a_row_index = a_row_index; a.a_rows = a_rows;
  a.group_offsets = group_offsets; a.E = E; a.rows_total = rows_total; a.K = K;
  a.w_codes = w_codes; a.w_scales = w_scales; a.N = N;
  a.sel_idx = sel_idx; a.r_codes = r_codes; a.r_scales = r_scales;
  a.kc = sel_idx ? kc : 0;
  a.epilogue = epilogue; a.row_weight = row_weight; a.scatter_index = scatter_index;
  a.out_rows = out_rows; a.out = out; a.ldo = ldo;
  a.out_amax = epilogue == NVFP4_EPI_SWIGLU_BF16 ? out_amax : nullptr;
  a.block_m = 0;
  a.y_rows = epilogue == NVFP4_EPI_SCATTER_ADD_F32 ? static_cast<float*>(ws) : nullptr;
  a.combine_overwrite = overwrite;
  return hip_status(nvfp4::launch_mx_grouped_gemm(a, static_cast<hipStream_t>(stream)), fn);
}

// ---------------------------------------------------------------------------
// MXFP4 W4A8: MXFP8 activations x MXFP4 weights
// ---------------------------------------------------------------------------
int mxfp8_quantize(const void* x, int dtype, int64_t M, int64_t K, int64_t ldx, uint8_t* codes,
                   uint8_t* scales, void* stream) {
  const char* fn = "mxfp8_quantize";
  if (int s = check_act(x, dtype, M, K, ldx, fn)) return s;
  if (K % 32 != 0) return fail(NVFP4_EINVAL, "%s: K=%lld is not a multiple of 32", fn, (long long)K);
  if (M > 0 && (!codes || !scales)) return fail(NVFP4_EINVAL, "%s: codes/scales are NULL", fn);
  if (codes && !aligned16(codes)) return fail(NVFP4_EINVAL, "%s: codes not 16-byte aligned", fn);
  return hip_status(nvfp4::launch_mx8_quantize(x, dtype, M, K, ldx, codes, scales,
                                               static_cast<hipStream_t>(stream)),
                    fn);
}

size_t moe_mxfp4_w4a8_grouped_gemm_workspace_size(int32_t E, int64_t rows_total, int64_t N,
                                                  int64_t K, int epilogue, int64_t out_rows) {
  return moe_w4a4_grouped_gemm_workspace_size(E, rows_total, N, K, epilogue, out_rows);
}

int moe_mxfp4_w4a8_grouped_gemm(const uint8_t* a_codes, const uint8_t* a_scales,
                                const int32_t* a_row_index, int64_t a_rows,
                                const int64_t* group_offsets, int32_t E, int64_t rows_total,
                                int64_t K, const uint8_t* w_codes, const uint8_t* w_scales,
                                int64_t N, int epilogue, const float* row_weight,
                                const int32_t* scatter_index, int64_t out_rows, void* out,
                                int64_t ldo, float* out_amax, void* ws, size_t ws_bytes,
                                void* stream) {
  const char* fn = "moe_mxfp4_w4a8_grouped_gemm";
  const bool overwrite = scatter_overwrite(epilogue);
  if (E <= 0 || K <= 0 || N <= 0 || rows_total < 0 || a_rows < 0)
    return fail(NVFP4_EINVAL, "%s: E=%d K=%lld N=%lld rows_total=%lld", fn, E, (long long)K,
                (long long)N, (long long)rows_total);
  if (K % 128 != 0) return fail(NVFP4_EINVAL, "%s: K=%lld is not a multiple of 128", fn, (long long)K);
  if (K > 65536) return fail(NVFP4_EUNSUPPORTED, "%s: K=%lld > 65536", fn, (long long)K);
  if (a_rows * K >= (1LL << 32) || N * (K / 2) >= (1LL << 32))   // 32-bit lane offsets
    return fail(NVFP4_EUNSUPPORTED, "%s: A or one expert's W spans 4 GiB or more", fn);
  if (rows_total > 2147483647LL) return fail(NVFP4_EUNSUPPORTED, "%s: rows_total above 2^31-1", fn);
  if (!group_offsets || !w_codes || !w_scales || !out)
    return fail(NVFP4_EINVAL, "%s: required pointer is NULL", fn);
  if (rows_total > 0 && (!a_codes || !a_scales)) return fail(NVFP4_EINVAL, "%s: a_codes/a_scales NULL", fn);
  if (rows_total > 0 && a_rows < 1)
    return fail(NVFP4_EINVAL, "%s: a_rows must be at least 1 when rows_total > 0", fn);
  if (!aligned16(w_codes) || (a_codes && !aligned16(a_codes)))
    return fail(NVFP4_EINVAL, "%s: codes not 16-byte aligned", fn);
  if ((reinterpret_cast<uintptr_t>(w_scales) & 3u) || (reinterpret_cast<uintptr_t>(a_scales) & 3u))
    return fail(NVFP4_EINVAL, "%s: scales not 4-byte aligned", fn);
  if (epilogue == NVFP4_EPI_F32) {
    if (ldo < N) return fail(NVFP4_EINVAL, "%s: ldo=%lld < N", fn, (long long)ldo);
  } else if (epilogue == NVFP4_EPI_SWIGLU_BF16) {
    if (N % 2 != 0) return fail(NVFP4_EINVAL, "%s: SwiGLU needs N even", fn);
    if (ldo < N / 2) return fail(NVFP4_EINVAL, "%s: ldo=%lld < N/2", fn, (long long)ldo);
  } else if (epilogue == NVFP4_EPI_SCATTER_ADD_F32) {
    if (ldo < N) return fail(NVFP4_EINVAL, "%s: ldo=%lld < N", fn, (long long)ldo);
    if (!row_weight || !scatter_index) return fail(NVFP4_EINVAL, "%s: scatter needs row_weight and scatter_index", fn);
    if (out_rows < 0 || out_rows > 2147483647LL)
      return fail(NVFP4_EINVAL, "%s: out_rows must be in [0, 2^31-1]", fn);
    const size_t need = moe_mxfp4_w4a8_grouped_gemm_workspace_size(E, rows_total, N, K, epilogue, out_rows);
    if (!ws || ws_bytes < need)
      return fail(NVFP4_EWORKSPACE, "%s: scatter epilogue needs a %zu-byte workspace", fn, need);
  } else {
    return fail(NVFP4_EINVAL, "%s: unknown epilogue %d", fn, epilogue);
  }
  nvfp4::GemmArgs a = {};
  a.a_codes = a_codes; a.a_scales = a_scales;
  a.a_row_index = a_row_index; a.a_rows = a_rows;
  a.group_offsets = group_offsets; a.E = E; a.rows_total = rows_total; a.K = K;
  a.w_codes = w_codes; a.w_scales = w_scales; a.N = N;
  a.epilogue = epilogue; a.row_weight = row_weight; a.scatter_index = scatter_index;
  a.out_rows = out_rows; a.out = out; a.ldo = ldo;
  a.out_amax = epilogue == NVFP4_EPI_SWIGLU_BF16 ? out_amax : nullptr;
  a.block_m = 0;
  a.y_rows = epilogue == NVFP4_EPI_SCATTER_ADD_F32 ? static_cast<float*>(ws) : nullptr;
  a.combine_overwrite = overwrite;
  return hip_status(nvfp4::launch_mx_w4a8_grouped_gemm(a, static_cast<hipStream_t>(stream)), fn);
}

// ---------------------------------------------------------------------------
size_t qdq_weights_workspace_size(int64_t nmat, int64_t N, int64_t K) {
  (void)N; (void)K;
  return nvfp4::qdq_workspace_bytes(nmat);
}

int qdq_weights(const void* w, int64_t nmat, int64_t N, int64_t K, void* w_qdq, uint8_t* codes,
                uint8_t* scales, float* g, void* ws, size_t ws_bytes, void* stream) {
  const char* fn = "qdq_weights";
  if (nmat < 0 || N < 0 || K <= 0) return fail(NVFP4_EINVAL, "%s: bad shape", fn);
  if (K % 16 != 0) return fail(NVFP4_EINVAL, "%s: K=%lld not a multiple of 16", fn, (long long)K);
  if (nmat > 65535) return fail(NVFP4_EUNSUPPORTED, "%s: nmat > 65535", fn);
  if (nmat == 0 || N == 0) return ok();
  if (!w || !w_qdq) return fail(NVFP4_EINVAL, "%s: w / w_qdq NULL", fn);
  if (w == w_qdq) return fail(NVFP4_EINVAL, "%s: in-place operation is not supported", fn);
  if (!aligned16(w) || !aligned16(w_qdq) || (codes && !aligned16(codes)))
    return fail(NVFP4_EINVAL, "%s: pointers must be 16-byte aligned", fn);
  if (!ws || ws_bytes < qdq_weights_workspace_size(nmat, N, K))
    return fail(NVFP4_EWORKSPACE, "%s: workspace too small", fn);
  return hip_status(nvfp4::launch_qdq(static_cast<const __bf16*>(w), nmat, N, K,
                                      static_cast<__bf16*>(w_qdq), codes, scales, g, ws,
                                      static_cast<hipStream_t>(stream)),
                    fn);
}

int mxfp4_qdq_weights(const void* w, int64_t nmat, int64_t N, int64_t K, void* w_qdq,
                      uint8_t* codes, uint8_t* scales, void* stream) {
  const char* fn = "mxfp4_qdq_weights";
  if (nmat < 0 || N < 0 || K <= 0) return fail(NVFP4_EINVAL, "%s: bad shape", fn);
  if (K % 32 != 0) return fail(NVFP4_EINVAL, "%s: K=%lld not a multiple of 32", fn, (long long)K);
  if (nmat == 0 || N == 0) return ok();
  if (!w || !w_qdq) return fail(NVFP4_EINVAL, "%s: w / w_qdq NULL", fn);
  if (w == w_qdq) return fail(NVFP4_EINVAL, "%s: in-place operation is not supported", fn);
  if (!aligned16(w) || !aligned16(w_qdq) || (codes && !aligned16(codes)))
    return fail(NVFP4_EINVAL, "%s: pointers must be 16-byte aligned", fn);
  return hip_status(nvfp4::launch_mx_qdq(static_cast<const __bf16*>(w), nmat * N, K,
                                         static_cast<__bf16*>(w_qdq), codes, scales,
                                         static_cast<hipStream_t>(stream)),
                    fn);
}

int mxfp4_guided_round(const void* x_train, int dtype, int64_t M, int64_t K, int64_t ldx,
                       const uint8_t* roll_codes, const uint8_t* roll_scales,
                       uint8_t* guided_codes, void* x_fq, int64_t* dist_hist, void* stream) {
  const char* fn = "mxfp4_guided_round";
  if (int s = check_act(x_train, dtype, M, K, ldx, fn)) return s;
  if (K % 32 != 0) return fail(NVFP4_EINVAL, "%s: K=%lld is not a multiple of 32", fn, (long long)K);
  if (M * (K / 16) > 2147483647LL)
    return fail(NVFP4_EUNSUPPORTED, "%s: more than 2^31-1 blocks", fn);
  if (M > 0 && (!roll_codes || !roll_scales || !guided_codes))
    return fail(NVFP4_EINVAL, "%s: required pointer is NULL", fn);
  if ((roll_codes && !aligned16(roll_codes)) || (guided_codes && !aligned16(guided_codes)) ||
      (x_fq && !aligned16(x_fq)))
    return fail(NVFP4_EINVAL, "%s: pointers must be 16-byte aligned", fn);
  return hip_status(nvfp4::launch_mx_guided(x_train, dtype, M, K, ldx, roll_codes, roll_scales,
                                            guided_codes, static_cast<__bf16*>(x_fq), dist_hist,
                                            static_cast<hipStream_t>(stream)),
                    fn);
}

// ---------------------------------------------------------------------------
int guided_round(const void* x_train, int dtype, int64_t M, int64_t K, int64_t ldx,
                 const uint8_t* roll_codes, const uint8_t* roll_scales, const float* roll_global,
                 uint8_t* guided_codes, void* x_fq, int64_t* dist_hist, void* stream) {
  const char* fn = "guided_round";
  if (int s = check_act(x_train, dtype, M, K, ldx, fn)) return s;
  if (M * (K / 16) > 2147483647LL)
    return fail(NVFP4_EUNSUPPORTED, "%s: more than 2^31-1 blocks", fn);
  if (M > 0 && (!roll_codes || !roll_scales || !roll_global || !guided_codes))
    return fail(NVFP4_EINVAL, "%s: required pointer is NULL", fn);
  if ((roll_codes && !aligned16(roll_codes)) || (guided_codes && !aligned16(guided_codes)) ||
      (x_fq && !aligned16(x_fq)))
    return fail(NVFP4_EINVAL, "%s: pointers must be 16-byte aligned", fn);
  return hip_status(nvfp4::launch_guided(x_train, dtype, M, K, ldx, roll_codes, roll_scales,
                                         roll_global, guided_codes, static_cast<__bf16*>(x_fq),
                                         dist_hist, static_cast<hipStream_t>(stream)),
                    fn);
}

int mxfp4_guided_round_record(const void* x_train, int dtype, int64_t M, int64_t K, int64_t ldx,
                              const uint8_t* record, const uint8_t* roll_scales,
                              uint8_t* guided_codes, void* x_fq, int64_t* moved, void* stream) {
  const char* fn = "mxfp4_guided_round_record";
  if (int s = check_act(x_train, dtype, M, K, ldx, fn)) return s;
  if (K % 32 != 0) return fail(NVFP4_EINVAL, "%s: K=%lld is not a multiple of 32", fn, (long long)K);
  if (M * (K / 16) > 2147483647LL)
    return fail(NVFP4_EUNSUPPORTED, "%s: more than 2^31-1 blocks", fn);
  if (M > 0 && (!record || !roll_scales || !guided_codes))
    return fail(NVFP4_EINVAL, "%s: required pointer is NULL", fn);
  if ((record && !aligned16(record)) || (guided_codes && !aligned16(guided_codes)) ||
      (x_fq && !aligned16(x_fq)))
    return fail(NVFP4_EINVAL, "%s: pointers must be 16-byte aligned", fn);
  return hip_status(nvfp4::launch_mx_guided_record(x_train, dtype, M, K, ldx, record, roll_scales,
                                                   guided_codes, static_cast<__bf16*>(x_fq), moved,
                                                   static_cast<hipStream_t>(stream)),
                    fn);
}

int guidance_record_pack(const uint8_t* roll_codes, int64_t M, int64_t K, uint8_t* record,
                         void* stream) {
  const char* fn = "guidance_record_pack";
  if (M < 0 || K <= 0) return fail(NVFP4_EINVAL, "%s: M=%lld K=%lld", fn, (long long)M, (long long)K);
  if (K % 16 != 0) return fail(NVFP4_EINVAL, "%s: K=%lld is not a multiple of 16", fn, (long long)K);
  if (M > 0 && (!roll_codes || !record)) return fail(NVFP4_EINVAL, "%s: required pointer is NULL", fn);
  if ((roll_codes && !aligned16(roll_codes)) || (record && !aligned16(record)))
    return fail(NVFP4_EINVAL, "%s: pointers must be 16-byte aligned", fn);
  return hip_status(nvfp4::launch_guidance_pack(roll_codes, M, K, record,
                                                static_cast<hipStream_t>(stream)),
                    fn);
}

int guided_round_record(const void* x_train, int dtype, int64_t M, int64_t K, int64_t ldx,
                        const uint8_t* record, const uint8_t* roll_scales, const float* roll_global,
                        uint8_t* guided_codes, void* x_fq, int64_t* moved, void* stream) {
  const char* fn = "guided_round_record";
  if (int s = check_act(x_train, dtype, M, K, ldx, fn)) return s;
  if (M * (K / 16) > 2147483647LL)
    return fail(NVFP4_EUNSUPPORTED, "%s: more than 2^31-1 blocks", fn);
  if (M > 0 && (!record || !roll_scales || !roll_global || !guided_codes))
    return fail(NVFP4_EINVAL, "%s: required pointer is NULL", fn);
  if ((record && !aligned16(record)) || (guided_codes && !aligned16(guided_codes)) ||
      (x_fq && !aligned16(x_fq)))
    return fail(NVFP4_EINVAL, "%s: pointers must be 16-byte aligned", fn);
  return hip_status(nvfp4::launch_guided_record(x_train, dtype, M, K, ldx, record, roll_scales,
                                                roll_global, guided_codes,
                                                static_cast<__bf16*>(x_fq), moved,
                                                static_cast<hipStream_t>(stream)),
                    fn);
}

}  // extern "C"
