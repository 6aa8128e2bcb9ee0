/*
 * nvfp4_resq.h -- C ABI of the MI355X (gfx950) NVFP4 W4A4 MoE expert GEMM with
 * residual activation compensation, plus the trainer-side weight QDQ and
 * rollout-guided rounding.
 *
 * Sources of the operations (web pages; cited by title and section):
 *   [QUADS]  "QUADS: Stabilizing NVFP4 Reinforcement Learning for MoE via
 *            QUantization-error Alignment across Dual Sides", technical
 *            summary (gist.science), sections 1, 2.1, 2.2A, 2.2B; digest
 *            (yfxerp.com).
 *   [TRACE]  "TRACE: Rollout-Guided Quantization-Aware Training for FP4
 *            Reinforcement Learning of MoE Language Models", summary
 *            (paper.rainbus.top): "Prerequisites: NVFP4 and the E2M1
 *            codebook", "Research motivation", "Core method", "Method steps".
 *
 * Number format (NVFP4), one definition for every entry point:
 *   - element: 4-bit E2M1 code = sign<<3 | index, magnitudes by index
 *     0, 0.5, 1, 1.5, 2, 3, 4, 6 ([QUADS] sec. 1 counts eight levels a sign;
 *     [TRACE] prerequisites: E2M1 codebook, round-to-nearest);
 *   - block: 16 consecutive elements of a row share one E4M3 (OCP E4M3FN,
 *     max 448) scale byte s_b;
 *   - tensor: one fp32 global scale g = RNE32(amax / 2688) (1 if that is 0);
 *   - s_b = E4M3 nearest to amax_b / (6 g), ties to even, saturating at 448;
 *   - S_b = RNE32(s_b * g); element index = E2M1 index nearest to |x| / S_b
 *     (exact real quotient; ties to the even index; above 6 gives 6; S_b = 0
 *     gives 0); the sign bit copies x's sign bit;
 *   - dequantized value DQ = RNE32(value * S_b).
 *   Storage: codes [rows, K/2] bytes, element 2j in the low nibble of byte j;
 *   scales [rows, K/16] bytes, row-major.  4.5 bit per element.
 *
 * Conventions of every entry point:
 *   - All tensor pointers are DEVICE pointers owned by the caller; scalars
 *     such as g, amax and r_global stay on the device.  Sizes and counts are
 *     host integers.
 *   - `stream` is a hipStream_t passed as void* (NULL = the null stream).
 *     Calls are asynchronous on it; nothing synchronizes the host.
 *   - Arguments are validated on the host before any launch; on error
 *     nothing is written and a negative status is returned; the message is
 *     available from nvfp4_last_error() (thread-local).
 *   - Index inputs that only the device can read (row indexes, offsets,
 *     selected channels) are clamped or skipped when out of range; they
 *     never cause out-of-bounds accesses, but out-of-range values give
 *     unspecified results.
 *   - Workspace: `ws` points to at least <name>_workspace_size(...) bytes of
 *     device memory, 256-byte aligned; its contents need no initialization
 *     and are garbage afterwards.  The library allocates nothing.
 *   - Base pointers must be 16-byte aligned; K % 16 == 0 and the compensated
 *     channel count k % 16 == 0, 16 <= k <= K.  The grouped GEMMs need more
 *     of K (stated in their blocks): K % 64 == 0 for NVFP4, K % 128 == 0 for
 *     MXFP4.
 *   - Non-finite inputs are outside the contract.
 *   - Calls that share a workspace or outputs on one stream are ordered by
 *     the stream; concurrent use of one workspace from two streams races.
 */
#ifndef NVFP4_RESQ_H
#define NVFP4_RESQ_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* status codes */
#define NVFP4_OK            0
#define NVFP4_EINVAL       -1   /* invalid argument */
#define NVFP4_EUNSUPPORTED -2   /* unsupported dtype, shape or device */
#define NVFP4_EWORKSPACE   -3   /* workspace missing or too small */
#define NVFP4_EHIP         -4   /* a HIP call failed (message has the HIP error) */

/* activation dtypes */
#define NVFP4_DTYPE_BF16 0
#define NVFP4_DTYPE_F32  1

/* grouped-GEMM epilogues */
#define NVFP4_EPI_F32              0  /* out fp32 [rows, N] = Y */
#define NVFP4_EPI_SWIGLU_BF16      1  /* out bf16 [rows, N/2] = silu(Y[:, :N/2]) * Y[:, N/2:] */
#define NVFP4_EPI_SCATTER_ADD_F32  2  /* out fp32 [out_rows, N]: out[scatter_index[r]] += row_weight[r] * Y[r] */
#define NVFP4_EPI_SCATTER_F32      3  /* out fp32 [out_rows, N]: out[t] = sum of row_weight[r] * Y[r] over the rows with scatter_index[r] == t */

/* Library version (major*10000 + minor*100 + patch). */
int nvfp4_version(void);

/* Message of the last failed call on this thread ("" if none). */
const char* nvfp4_last_error(void);

/* ------------------------------------------------------------------------ *
 * nvfp4_quantize -- online NVFP4 quantization of an activation tensor.
 *
 * Computes, for x [M, K] (row stride ldx elements): the global scale g (from
 * the tensor's amax, or from *amax_in when given), the E4M3 block scales and
 * the packed E2M1 codes, with the format rules above ([TRACE] prerequisites
 * and the research-motivation worked example; online per-forward activation
 * quantization: [QUADS] sec. 2.1).
 *
 * Optionally (tile_partials != NULL) also the residual channel-score
 * partials used by resq_select_and_requant: for every 128-row tile t of x,
 * tile_partials[t, c] = sum of |x - DQ| over the tile's rows of channel c,
 * summed in fp32 in increasing row order from 0 ([QUADS] sec. 2.2B ranks
 * channels by residual magnitude).
 *
 *   x              bf16 or fp32 [M, ldx]
 *   dtype          NVFP4_DTYPE_BF16 | NVFP4_DTYPE_F32
 *   amax_in        NULL, or device fp32: use this amax instead of computing it
 *   codes          out [M, K/2];  scales out [M, K/16];  g_out out fp32 [1] (may be NULL)
 *   tile_partials  NULL or out fp32 [ceil(M/128), K]
 * Errors: EINVAL for null required pointers, K % 16 != 0, ldx < K, M < 0;
 *         EWORKSPACE if ws_bytes < nvfp4_quantize_workspace_size(M, K).
 * M == 0 is valid: g_out = 1, nothing else written.
 * ------------------------------------------------------------------------ */
size_t nvfp4_quantize_workspace_size(int64_t M, int64_t K);
int nvfp4_quantize(const void* x, int dtype, int64_t M, int64_t K, int64_t ldx,
                   const float* amax_in, uint8_t* codes, uint8_t* scales, float* g_out,
                   float* tile_partials, void* ws, size_t ws_bytes, void* stream);

/* ------------------------------------------------------------------------ *
 * nvfp4_quantize_noalloc -- nvfp4_quantize for callers that cannot allocate
 * device memory or pass a workspace: code under HIP graph capture, tight
 * serving loops, harnesses that forbid allocation.
 *
 * Arguments, results and errors are those of nvfp4_quantize without ws and
 * ws_bytes.  Its scratch (the amax partial maxima, at most 256 floats) is a
 * fixed 8 KB array of device memory inside the library, one per GPU, held
 * until the process ends; the call uses the copy of the current device
 * (hipGetDevice), whose address it looks up on its first call there.  It
 * calls no allocating routine.  EUNSUPPORTED if a shape ever needed more
 * scratch than the array holds (none does: the partial count is capped).
 * Calls share that array: two calls that overlap on one GPU (different
 * streams, or threads) race and give unspecified results; calls ordered on
 * one stream are safe.  Nothing in the array needs clearing between calls.
 * ------------------------------------------------------------------------ */
int nvfp4_quantize_noalloc(const void* x, int dtype, int64_t M, int64_t K, int64_t ldx,
                           const float* amax_in, uint8_t* codes, uint8_t* scales, float* g_out,
                           float* tile_partials, void* stream);

/* ------------------------------------------------------------------------ *
 * resq_select_and_requant -- residual activation compensation: pick the
 * high-residual channels of each selection unit and quantize their residual
 * a second time ([QUADS] sec. 2.2B: binary channel mask over channels of
 * largest residual magnitude, second FP4 quantization; the yfxerp digest:
 * the result is added back by the GEMM).
 *
 * Unit u owns "unit rows" unit_offsets[u] .. unit_offsets[u+1]-1; unit row r
 * is row row_index[r] of x (row r when row_index is NULL).  For each unit:
 *   R = x - DQ(codes, scales, *g) on its rows;
 *   score[c] = sum |R[:, c]|: unit rows cut into consecutive 128-row tiles,
 *              each summed in fp32 in increasing row order from 0, then the
 *              tile sums added in tile order from 0;
 *   sel_idx[u] = the k channels of largest score (ties to the lower index),
 *              written in ascending channel order;
 *   R_S = R[:, sel_idx[u]] (compact fp32 [rows_u, k]) quantized to NVFP4
 *         with its own global scale r_global[u] (blocks of 16 along the
 *         compact axis) -> r_codes / r_scales rows of the unit.
 * A unit with no rows gets sel_idx = 0..k-1 and r_global = 1.
 *
 *   x, dtype, K, ldx   the activation (bf16/fp32 [x_rows, ldx])
 *   row_index          NULL or int32 [rows_total]
 *   codes, scales, g   its NVFP4 quantization (from nvfp4_quantize)
 *   unit_offsets       int64 [U+1], non-decreasing, unit_offsets[U] == rows_total;
 *                      may be NULL when tile_partials is given
 *   tile_partials      NULL, or the partials nvfp4_quantize wrote for x; then
 *                      the units must be x's 128-row tiles: row_index NULL,
 *                      rows_total == x_rows, U == ceil(x_rows/128)
 *   sel_idx out int32 [U, k]; r_codes out [rows_total, k/2];
 *   r_scales out [rows_total, k/16]; r_global out fp32 [U]
 * Errors: EINVAL (shapes, k, null pointers, tile-unit mismatch), EWORKSPACE.
 * ------------------------------------------------------------------------ */
size_t resq_select_and_requant_workspace_size(int64_t K, int64_t rows_total, int64_t U, int32_t k);
int resq_select_and_requant(const void* x, int dtype, int64_t x_rows, int64_t K, int64_t ldx,
                            const int32_t* row_index, const uint8_t* codes, const uint8_t* scales,
                            const float* g, const int64_t* unit_offsets, int64_t U,
                            int64_t rows_total, int32_t k, const float* tile_partials,
                            int32_t* sel_idx, uint8_t* r_codes, uint8_t* r_scales,
                            float* r_global, void* ws, size_t ws_bytes, void* stream);

/* ------------------------------------------------------------------------ *
 * resq_mask_select_and_requant -- the dense binary-mask form of the same
 * compensation ([QUADS] sec. 2.2B: a binary channel mask keeps the top k% of
 * channels by residual magnitude, 50% in the pages' example, and those
 * channels are quantized a second time).
 *
 * Arguments, selection (scores, top-k, ties, empty units) and workspace
 * (resq_select_and_requant_workspace_size with the same K, rows_total, U, k)
 * are those of resq_select_and_requant.  The output differs: per unit,
 *   R * M  = R on the channels of sel_idx[u], 0 on the others (full width K),
 *   quantized to NVFP4 with its own global scale m_global[u] (the largest
 *   |R * M| of the unit's rows), blocks of 16 along K
 *   -> m_codes [rows_total, K/2] (16-byte aligned), m_scales [rows_total, K/16].
 * Blocks with no selected channel get codes 0 and scale 0.  The GEMM term is
 * moe_w4a4_masked_comp_gemm below.  K <= 16384.
 * Errors: as resq_select_and_requant.
 * ------------------------------------------------------------------------ */
int resq_mask_select_and_requant(const void* x, int dtype, int64_t x_rows, int64_t K, int64_t ldx,
                                 const int32_t* row_index, const uint8_t* codes,
                                 const uint8_t* scales, const float* g,
                                 const int64_t* unit_offsets, int64_t U, int64_t rows_total,
                                 int32_t k, const float* tile_partials, int32_t* sel_idx,
                                 uint8_t* m_codes, uint8_t* m_scales, float* m_global, void* ws,
                                 size_t ws_bytes, void* stream);

/* ------------------------------------------------------------------------ *
 * moe_w4a4_grouped_gemm -- routed grouped expert GEMM over NVFP4 weights and
 * NVFP4 activations, with the compensation term fused in ([QUADS] sec. 1:
 * native W4A4 GEMM; sec. 2.2B: the residual correction of the selected
 * channels is added back into the result).
 *
 * Group (expert) e owns unit rows group_offsets[e] .. group_offsets[e+1]-1;
 * unit row r reads activation row a_row_index[r] (r when NULL).  For every
 * unit row r of group e and output n < N:
 *   Y[r, n] = sum_k DQA[r, k] * DQW[e, n, k]
 *           + sum_j DQR[r, j] * DQW[e, n, sel_idx[e, j]]      (if sel_idx)
 * where DQW keeps each weight element's own block scale and w_global[e]
 * (the stored NVFP4 weight restricted to the selected channels).  Products
 * of dequantized operands are exact; accumulation is fp32.
 *
 *   K                  multiple of 64, at most 65536: the kernel moves K through
 *                      LDS in 128-wide stages of 16-byte code chunks and
 *                      4-byte scale words, and a half stage (64) is the finest
 *                      granule it handles; K % 16 != 0 or K % 64 != 0 gives EINVAL
 *   a_codes/a_scales   [a_rows, K/2] / [a_rows, K/16];  a_global fp32 [1];
 *                      a_rows >= 1 whenever rows_total > 0 (row 0 must exist);
 *                      a row index outside [0, a_rows) reads as zeros;
 *                      a_rows * K/2 and N * K/2 below 2^32 (the kernel addresses
 *                      A and one expert's W with 32-bit offsets; EUNSUPPORTED)
 *   group_offsets      int64 [E+1] (device), group_offsets[E] == rows_total
 *   w_codes/w_scales   [E, N, K/2] / [E, N, K/16];  w_global fp32 [E]
 *   sel_idx            NULL (no compensation) or int32 [E, kc] ascending, kc <= 128
 *   r_codes/r_scales   [rows_total, kc/2] / [rows_total, kc/16]; r_global fp32 [E]
 *   epilogue           NVFP4_EPI_*: F32 writes fp32 [rows_total, ldo];
 *                      SWIGLU_BF16 needs N even, gate = outputs 0..N/2-1,
 *                      up = N/2..N-1, writes bf16 h [rows_total, ldo] =
 *                      bf16(silu(gate) * up) and, when out_amax != NULL,
 *                      stores max |h| (fp32) into *out_amax;
 *                      SCATTER_ADD_F32 adds row_weight[r] * Y[r] into out row
 *                      scatter_index[r] (< out_rows) of fp32 [out_rows, ldo],
 *                      the rows of each output row in increasing r (a fixed
 *                      order: the result is reproducible); the caller
 *                      initializes out.  SCATTER_F32 writes the same sums
 *                      started from zero instead (every out row is written,
 *                      rows that no r names with zeros; out need not be
 *                      initialized).  Both need the workspace
 *                      (rows_total * N * 4 bytes plus index lists); the
 *                      other epilogues need none.
 * Errors: EINVAL (shapes, K % 64, pointers, epilogue arguments, kc),
 *         EUNSUPPORTED (K > 65536, rows_total >= 2^31, operands of 4 GiB),
 *         EWORKSPACE.
 * rows_total == 0 is valid (out_amax set to 0, nothing else written; with
 * SCATTER_F32, out is zeroed).
 * Streams: with 256-row tiles the groups' ragged remainders (and, for the
 * scatter epilogues, the plan of the row lists) run on a stream that the
 * library keeps per device, forked from `stream` and joined back into it
 * with events, so the call is ordered on `stream` as one operation.
 * While `stream` is being captured into a graph, everything stays on it.
 * ------------------------------------------------------------------------ */
size_t moe_w4a4_grouped_gemm_workspace_size(int32_t E, int64_t rows_total, int64_t N, int64_t K,
                                            int epilogue, int64_t out_rows);
int moe_w4a4_grouped_gemm(const uint8_t* a_codes, const uint8_t* a_scales, const float* a_global,
                          const int32_t* a_row_index, int64_t a_rows,
                          const int64_t* group_offsets, int32_t E, int64_t rows_total, int64_t K,
                          const uint8_t* w_codes, const uint8_t* w_scales, const float* w_global,
                          int64_t N, const int32_t* sel_idx, const uint8_t* r_codes,
                          const uint8_t* r_scales, const float* r_global, int32_t kc,
                          int epilogue, const float* row_weight, const int32_t* scatter_index,
                          int64_t out_rows, void* out, int64_t ldo, float* out_amax,
                          void* ws, size_t ws_bytes, void* stream);

/* ------------------------------------------------------------------------ *
 * moe_w4a4_masked_comp_gemm -- the dense-mask compensation's GEMM term, a
 * second grouped GEMM of the main one's shape ([QUADS] sec. 2.2B: the
 * correction of the masked residual is added back into the result).
 *
 * For every unit row r of group e (group_offsets as in moe_w4a4_grouped_gemm;
 * no row index: row r of m_codes) and output n < N:
 *   out[r * ldo + n] += sum_k DQM[r, k] * DQW[e, n, k]
 * where DQM dequantizes m_codes / m_scales with m_global[e] (one global scale
 * per group, as resq_mask_select_and_requant writes them).  Run it after
 * moe_w4a4_grouped_gemm (EPI_F32) wrote the main product into out on the same
 * stream: out then holds Q(X) Q(W)^T + Q(R * M) Q(W)^T.
 *   m_codes/m_scales   [rows_total, K/2] / [rows_total, K/16]; m_global fp32 [E]
 *   w_*                as moe_w4a4_grouped_gemm; K multiple of 64
 *   out                fp32 [rows_total, ldo], read and written; ldo >= N
 * Errors: EINVAL (shapes, pointers, alignment), EUNSUPPORTED (K > 65536).
 * ------------------------------------------------------------------------ */
int moe_w4a4_masked_comp_gemm(const uint8_t* m_codes, const uint8_t* m_scales,
                              const float* m_global, const int64_t* group_offsets, int32_t E,
                              int64_t rows_total, int64_t K, const uint8_t* w_codes,
                              const uint8_t* w_scales, const float* w_global, int64_t N,
                              float* out, int64_t ldo, void* stream);

/* ------------------------------------------------------------------------ *
 * qdq_weights -- trainer-side weight quantize-dequantize of the asymmetric
 * W4A16 QAT ([QUADS] sec. 2.2A: weights are fake-quantized to NVFP4 on the
 * trainer so that its forward sees the rollout's weights; activations stay
 * BF16).  Every matrix i of w [nmat, N, K] gets its own global scale;
 * blocks run along K.  w_qdq = bf16(DQ) with DQ = RNE32(value * S_b).
 *   w        bf16 [nmat, N, K];  w_qdq out bf16 [nmat, N, K]
 *   codes    NULL or out [nmat, N, K/2];  scales NULL or out [nmat, N, K/16]
 *   g        NULL or out fp32 [nmat]
 * Matrices of 3.1 M to 12.6 M elements on 256 CUs (one to four 16-blocks per
 * thread of the grid) take one pass: a cooperative launch keeps each matrix
 * on chip between its amax and its quantization; others take an amax pass
 * and a quantize pass.  The workspace (at least 64 KiB) holds the one-pass
 * kernel's per-workgroup amax slots and, in the 32-bit word at byte offset
 * 65536, a flag that is nonzero if a gather gave up waiting (it cannot when
 * the launch succeeded, as every workgroup is then resident); it is
 * overwritten by every call.
 * Errors: EINVAL (K % 16, null w / w_qdq, in-place w == w_qdq), EWORKSPACE.
 * ------------------------------------------------------------------------ */
size_t qdq_weights_workspace_size(int64_t nmat, int64_t N, int64_t K);
int qdq_weights(const void* w, int64_t nmat, int64_t N, int64_t K, void* w_qdq,
                uint8_t* codes, uint8_t* scales, float* g, void* ws, size_t ws_bytes,
                void* stream);

/* ------------------------------------------------------------------------ *
 * guided_round -- rollout-guided neighbour-codeword rounding ([TRACE] core
 * method and method step four).  For each element, with the rollout
 * block's scale S = RNE32(s_roll * g_roll) and v = x_train / S (exact), the
 * candidates are the neighbouring signed E2M1 levels q- <= v <= q+ (clamped
 * to +-6); the output is the one closer to the recorded rollout level,
 * instead of round-to-nearest.  This never moves farther from the rollout
 * level than round-to-nearest ([TRACE] Eq. (3)).  A zero result takes
 * x_train's sign bit; S == 0 gives magnitude 0.
 *   x_train       bf16/fp32 [M, ldx]
 *   roll_codes    [M, K/2];  roll_scales [M, K/16];  roll_global fp32 [1]
 *   guided_codes  out [M, K/2]
 *   x_fq          NULL or out bf16 [M, K] = bf16(RNE32(value * S))
 *   dist_hist     NULL or out int64 [3]: numbers of elements whose signed
 *                 level index under round-to-nearest differs from the
 *                 rollout's by 0, by 1, and by 2 or more (overwritten)
 * Errors: EINVAL (shapes, null pointers).
 * ------------------------------------------------------------------------ */
int guided_round(const void* x_train, int dtype, int64_t M, int64_t K, int64_t ldx,
                 const uint8_t* roll_codes, const uint8_t* roll_scales,
                 const float* roll_global, uint8_t* guided_codes, void* x_fq,
                 int64_t* dist_hist, void* stream);

/* ------------------------------------------------------------------------ *
 * guidance_record_pack -- the rollout side of the mantissa-only guidance
 * record ([TRACE] core method, second innovation; method step two): one bit
 * per element, the low bit of its E2M1 code (the level's mantissa bit).  With
 * the rollout block scales, which travel beside it unchanged, the record
 * costs 1.5 bits per element instead of 4.5.
 *   roll_codes  [M, K/2] (rows contiguous)
 *   record      out [M, K/8]: bit j of byte i of a row = low code bit of
 *               element 8i + j
 * Asynchronous on stream; writes nothing but record.
 * Errors: EINVAL (K % 16 != 0, null or misaligned pointers).
 * ------------------------------------------------------------------------ */
int guidance_record_pack(const uint8_t* roll_codes, int64_t M, int64_t K, uint8_t* record,
                         void* stream);

/* ------------------------------------------------------------------------ *
 * guided_round_record -- rollout-guided rounding from the mantissa-only
 * record ([TRACE] method steps two and four).  S, v = x_train / S and the
 * neighbouring levels q- <= v <= q+ are those of guided_round; the output is
 * the one whose magnitude index has the recorded low bit (neighbouring
 * levels always differ in it), q- when q- == q+.  Wherever the rollout level
 * is q- or q+ this equals guided_round.  A zero result takes x_train's sign
 * bit; S == 0 gives magnitude 0.
 *   x_train       bf16/fp32 [M, ldx]
 *   record        [M, K/8] from guidance_record_pack
 *   roll_scales   [M, K/16];  roll_global fp32 [1]
 *   guided_codes  out [M, K/2]
 *   x_fq          NULL or out bf16 [M, K] = bf16(RNE32(value * S))
 *   moved         NULL or out int64 [2]: numbers of elements left at and
 *                 moved from round-to-nearest (overwritten)
 * Errors: EINVAL (shapes, null pointers), EUNSUPPORTED (over 2^31-1 blocks).
 * ------------------------------------------------------------------------ */
int guided_round_record(const void* x_train, int dtype, int64_t M, int64_t K, int64_t ldx,
                        const uint8_t* record, const uint8_t* roll_scales,
                        const float* roll_global, uint8_t* guided_codes, void* x_fq,
                        int64_t* moved, void* stream);

/* ======================================================================== *
 * MXFP4 variant.  [TRACE] validates its method in MXFP4 rollouts as well as
 * NVFP4 (results paragraph and Table 4, MXFP4 W4A8 and W4A4) without stating
 * the format; it is read as the OCP MX format:
 *   - block: 32 consecutive elements of a row share one E8M0 scale byte
 *     b = X + 127, value 2^X; X = floor(log2 amax_b) - 2 clamped to
 *     [-127, 127], -127 for an all-zero block; no global scale;
 *   - element: E2M1 index nearest to |x| / 2^X (ties to the even index,
 *     above 6 gives 6), sign bit of x; DQ = value * 2^X (exact in fp32).
 *   Storage: codes [rows, K/2] as for NVFP4; scales [rows, K/32] bytes,
 *   row-major.  4.25 bit per element.
 * ======================================================================== */

/* ------------------------------------------------------------------------ *
 * mxfp4_quantize -- online MXFP4 quantization of an activation tensor
 * ([QUADS] sec. 2.1: activations are quantized online every forward).
 *   x              bf16 or fp32 [M, ldx]
 *   codes          out [M, K/2];  scales out [M, K/32]
 *   tile_partials  NULL or out fp32 [ceil(M/128), K]: per 128-row tile, the
 *                  fp32 sum of |x - DQ| of each channel in increasing row
 *                  order (the residual channel scores, [QUADS] sec. 2.2B)
 * Errors: EINVAL for null required pointers, K % 32 != 0, ldx < K, M < 0.
 * Needs no workspace.  M == 0 writes nothing.
 * ------------------------------------------------------------------------ */
int mxfp4_quantize(const void* x, int dtype, int64_t M, int64_t K, int64_t ldx, uint8_t* codes,
                   uint8_t* scales, float* tile_partials, void* stream);

/* ------------------------------------------------------------------------ *
 * mxfp4_resq_select_and_requant -- residual activation compensation in MXFP4
 * ([QUADS] sec. 2.2B): as resq_select_and_requant (units, row_index, the
 * channel scores of |x - DQ| in the fixed 128-row tile order, top-k with
 * ties to the lower channel, sel_idx ascending), with x's codes and scales
 * in MXFP4 and the compact residual R_S quantized to MXFP4 with 32-blocks
 * along the compact axis.  No global scales.
 *   k              multiple of 32 in [32, K]
 *   sel_idx        out int32 [U, k];  r_codes out [rows_total, k/2];
 *   r_scales       out [rows_total, k/32]
 * Errors: as resq_select_and_requant; K % 32 != 0 or k % 32 != 0 give EINVAL.
 * ------------------------------------------------------------------------ */
size_t mxfp4_resq_select_and_requant_workspace_size(int64_t K, int64_t rows_total, int64_t U,
                                                    int32_t k);
int mxfp4_resq_select_and_requant(const void* x, int dtype, int64_t x_rows, int64_t K, int64_t ldx,
                                  const int32_t* row_index, const uint8_t* codes,
                                  const uint8_t* scales, const int64_t* unit_offsets, int64_t U,
                                  int64_t rows_total, int32_t k, const float* tile_partials,
                                  int32_t* sel_idx, uint8_t* r_codes, uint8_t* r_scales, void* ws,
                                  size_t ws_bytes, void* stream);

/* ------------------------------------------------------------------------ *
 * mxfp4_qdq_weights -- trainer-side weight quantize-dequantize in MXFP4 (the
 * asymmetric W4A16 QAT of [QUADS] sec. 2.2A with the rollout's MXFP4 weights;
 * [TRACE] Table 4 trains MXFP4 rollouts).  Blocks of 32 along K, one E8M0
 * scale each, no global scale; w_qdq = bf16(value * 2^X), which is exact.
 *   w        bf16 [nmat, N, K];  w_qdq out bf16 [nmat, N, K] (not w itself)
 *   codes    NULL or out [nmat, N, K/2];  scales NULL or out [nmat, N, K/32]
 *   K multiple of 32; w, w_qdq, codes 16-byte aligned
 * Errors: EINVAL (shape, null or aliased or misaligned pointers).
 * ------------------------------------------------------------------------ */
int mxfp4_qdq_weights(const void* w, int64_t nmat, int64_t N, int64_t K, void* w_qdq,
                      uint8_t* codes, uint8_t* scales, void* stream);

/* ------------------------------------------------------------------------ *
 * mxfp4_guided_round -- rollout-guided rounding against MXFP4 rollout codes
 * ([TRACE] core method and method step four, with the MXFP4 rollout of its
 * Table 4): as guided_round, with S = 2^X of the element's rollout 32-block
 * and no global scale.
 *   x_train       bf16/fp32 [M, ldx];  K multiple of 32
 *   roll_codes    [M, K/2];  roll_scales [M, K/32]
 *   guided_codes  out [M, K/2];  x_fq NULL or out bf16 [M, K] = bf16(value * S)
 *   dist_hist     NULL or out int64 [3], as guided_round
 * Errors: EINVAL (shapes, null pointers), EUNSUPPORTED (M*K/16 >= 2^31).
 * ------------------------------------------------------------------------ */
int mxfp4_guided_round(const void* x_train, int dtype, int64_t M, int64_t K, int64_t ldx,
                       const uint8_t* roll_codes, const uint8_t* roll_scales,
                       uint8_t* guided_codes, void* x_fq, int64_t* dist_hist, void* stream);

/* ------------------------------------------------------------------------ *
 * mxfp4_guided_round_record -- guided rounding from the mantissa-only record
 * of MXFP4 rollout codes ([TRACE] core method, second innovation; method
 * steps two and four).  The record is guidance_record_pack's output for the
 * MXFP4 codes (the low code bit, the same for both formats); with the E8M0
 * scales beside it the guidance costs 1 + 8/32 = 1.25 bits per element.  As
 * guided_round_record with S = 2^X of the element's rollout 32-block.
 *   x_train       bf16/fp32 [M, ldx];  K multiple of 32
 *   record        [M, K/8];  roll_scales [M, K/32]
 *   guided_codes  out [M, K/2];  x_fq NULL or out bf16 [M, K]
 *   moved         NULL or out int64 [2], as guided_round_record
 * Errors: EINVAL (shapes, null pointers), EUNSUPPORTED (M*K/16 >= 2^31).
 * ------------------------------------------------------------------------ */
int mxfp4_guided_round_record(const void* x_train, int dtype, int64_t M, int64_t K, int64_t ldx,
                              const uint8_t* record, const uint8_t* roll_scales,
                              uint8_t* guided_codes, void* x_fq, int64_t* moved, void* stream);

/* ------------------------------------------------------------------------ *
 * moe_mxfp4_grouped_gemm -- the routed grouped expert GEMM over MXFP4
 * activations and weights with the residual compensation term ([QUADS]
 * sec. 1: native W4A4 GEMM on the rollout; sec. 2.2B: the second FP4
 * quantization of the selected channels added back into the result):
 *   Y[r, n] = sum_k A[r, k] W_e[n, k] + sum_j R_S[r, j] W_e[n, sel_e[j]]
 * with every operand element its MXFP4 value (no global scales).  Arguments
 * as moe_w4a4_grouped_gemm without a_global, w_global and r_global:
 *   a_scales       [a_rows, K/32];  w_scales [E, N, K/32]; both 4-byte aligned
 *   r_scales       [rows_total, kc/32];  kc multiple of 32 in [32, min(K, 128)]
 *   K              multiple of 128
 * The compensation's weight side is computed on the matrix cores in FP8 E4M3
 * against the largest block scale of each weight row: exact when a row's block
 * scales span at most 8 binades, else the smaller elements of W at the selected
 * channels are rounded to E4M3.
 * Errors: EINVAL (shapes, pointers, alignment, epilogue arguments, kc),
 *         EWORKSPACE (scatter epilogue).
 * ------------------------------------------------------------------------ */
size_t moe_mxfp4_grouped_gemm_workspace_size(int32_t E, int64_t rows_total, int64_t N, int64_t K,
                                             int epilogue, int64_t out_rows);
int moe_mxfp4_grouped_gemm(const uint8_t* a_codes, const uint8_t* a_scales,
                           const int32_t* a_row_index, int64_t a_rows,
                           const int64_t* group_offsets, int32_t E, int64_t rows_total, int64_t K,
                           const uint8_t* w_codes, const uint8_t* w_scales, int64_t N,
                           const int32_t* sel_idx, const uint8_t* r_codes, const uint8_t* r_scales,
                           int32_t kc, int epilogue, const float* row_weight,
                           const int32_t* scatter_index, int64_t out_rows, void* out, int64_t ldo,
                           float* out_amax, void* ws, size_t ws_bytes, void* stream);

/* ------------------------------------------------------------------------ *
 * mxfp8_quantize -- MXFP8 quantization of activations for the W4A8 GEMM
 * ([TRACE] results and Table 4: MXFP4 W4A8 rollouts, FP8 activations with FP4
 * weights).  Read as OCP MXFP8: 32-element blocks, E8M0 scale byte X + 127
 * with X = floor(log2 amax_b) - 8 clamped to [-127, 127] (-127 for an
 * all-zero block); element = E4M3FN byte nearest to |x| / 2^X (ties to the
 * even byte, above 448 gives 448), sign of x.
 *   codes  out [M, K] E4M3 bytes;  scales out [M, K/32]
 * Errors: EINVAL for null required pointers, K % 32 != 0, ldx < K, M < 0.
 * ------------------------------------------------------------------------ */
int mxfp8_quantize(const void* x, int dtype, int64_t M, int64_t K, int64_t ldx, uint8_t* codes,
                   uint8_t* scales, void* stream);

/* ------------------------------------------------------------------------ *
 * moe_mxfp4_w4a8_grouped_gemm -- the routed grouped expert GEMM with MXFP8
 * activations and MXFP4 weights (W4A8), on the matrix cores' mixed FP8 x FP4
 * form:  Y[r, n] = sum_k A[r, k] W_e[n, k]  (no residual compensation: that
 * step corrects FP4 activations).  Arguments as moe_mxfp4_grouped_gemm
 * without the compensation ones; a_codes are [a_rows, K] E4M3 bytes.
 * Errors: EINVAL (shapes, pointers, alignment, epilogue arguments),
 *         EUNSUPPORTED (A or one expert's W of 4 GiB or more),
 *         EWORKSPACE (scatter epilogue).
 * ------------------------------------------------------------------------ */
size_t moe_mxfp4_w4a8_grouped_gemm_workspace_size(int32_t E, int64_t rows_total, int64_t N,
                                                  int64_t K, int epilogue, int64_t out_rows);
int moe_mxfp4_w4a8_grouped_gemm(const uint8_t* a_codes, const uint8_t* a_scales,
                                const int32_t* a_row_index, int64_t a_rows,
                                const int64_t* group_offsets, int32_t E, int64_t rows_total,
                                int64_t K, const uint8_t* w_codes, const uint8_t* w_scales,
                                int64_t N, int epilogue, const float* row_weight,
                                const int32_t* scatter_index, int64_t out_rows, void* out,
                                int64_t ldo, float* out_amax, void* ws, size_t ws_bytes,
                                void* stream);

#ifdef __cplusplus
}
#endif

#endif /* NVFP4_RESQ_H */
