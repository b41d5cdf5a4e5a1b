/*
 * bsq.h -- C ABI of libbsq, dynamic block-scaled quantization of BF16
 * activations to MXFP4, MXFP8 and NVFP4 on AMD Instinct MI355X (gfx950).
 *
 * The operation is the one listed on the Modular "block_scaled_quantization"
 * module page: block-scaled quantization kernels for NVFP4, MXFP4 and MXFP8,
 * reached through a dispatcher (function list: quantize_dynamic_block_scaled,
 * quantize_dynamic_scaled_fp4fp8, quantize_mx_amd for AMD CDNA4).  The dense
 * NVFP4 arguments (a scalar fp32 tensor scale) and the number of elements per
 * block scale come from the "quantize_dynamic_scaled_async_fp4_kernel" page
 * (signature; Parameters: SF_VECTOR_SIZE).  The grouped per-expert arguments
 * (row_offsets and scales_offsets uint32, expert_ids int32, per-expert fp32
 * tensor scale, optional int32 row_indices gather) come from the
 * "grouped_quantize_dynamic_scaled_fp4_async_kernel" page (signature,
 * summary and Parameters).
 *
 * Formats and rules (the pages name the formats but define none of them):
 *   MXFP4  E2M1 codes, 2 per byte, 32-element blocks, E8M0 scale byte.
 *   MXFP8  E4M3 (FN) codes, 1 per byte, 32-element blocks, E8M0 scale byte.
 *   NVFP4  E2M1 codes, 2 per byte, 16-element blocks, E4M3 scale byte under
 *          an fp32 tensor scale tsf (decode: value = code * s * tsf).
 *   MX scale: X = max(floor(log2 amax) - emax, -127), emax = 2 (E2M1) or
 *          8 (E4M3); scale byte X + 127; code = RNE with saturation of
 *          x * 2^-X (OCP MX v1.0).
 *   NVFP4 scale: s = RNE_sat_E4M3(fl32(fl32(amax / 6) / tsf));
 *          inv = 0 if fl32(s * tsf) == 0 else fl32(1 / fl32(s * tsf));
 *          code = RNE_sat_E2M1(fl32(x * inv)).
 *   A block holding a NaN or Inf gets the NaN scale (0xFF for E8M0, 0x7F
 *          for E4M3) and all-zero codes.  Codes keep the sign bit of x, so
 *          -0 encodes as 0x8 (FP4) or 0x80 (FP8).  No subnormal is flushed.
 *   FP4 packing: element 2j in the low nibble of byte j, 2j+1 in the high.
 *   Blocks run along K, the contiguous dimension.
 *
 * Conventions for every entry point:
 *   - All pointers are device memory owned by the caller.  The library
 *     allocates nothing and keeps no device state.
 *   - The call is asynchronous on `stream` (a hipStream_t; NULL = the null
 *     stream).  Outputs are valid once the stream has been synchronised.
 *     Calls are thread-safe.
 *   - Arguments are validated on the host before any HIP call.  On failure
 *     nothing is launched, the status is returned, and bsq_last_error()
 *     describes it.  A launch failure returns BSQ_ERR_HIP.
 *   - For the quantizers, M == 0, K == 0 and (grouped) num_groups == 0 or
 *     max_rows == 0 are no-ops that return BSQ_OK.
 *   - Bytes of `codes` and `scales` outside what the call defines to write
 *     are never touched.
 */
#ifndef BSQ_H
#define BSQ_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum bsq_format { BSQ_MXFP4 = 0, BSQ_MXFP8 = 1, BSQ_NVFP4 = 2 };

/*
 * Scale layouts (any other value: BSQ_ERR_UNSUPPORTED).
 *
 * BSQ_SCALES_ROW_MAJOR  uint8 [rows, lds]: the scale of row r, block kb at
 *     r * lds + kb.
 *
 * BSQ_SCALES_MFMA16     MX formats only (NVFP4: BSQ_ERR_UNSUPPORTED): the
 *     operand layout of gfx950's v_mfma_scale_f32_16x16x128_f8f6f4, the
 *     CDNA4 counterpart of the SM100 scale interleave the
 *     "block_scaled_quantization" module page lists (block_scales_interleave).
 *     For one 128-element K step that instruction takes the scale of A row r
 *     (0..15) and 32-element block q (0..3) from lane r + 16 q of a 32-bit
 *     register, byte selected by opsel.  Rows form groups of 16 and blocks
 *     groups of 16 (512 elements); each (row group, block group) is a
 *     256-byte record in which the scale of (r, kb) is byte
 *         4 * ((r % 16) + 16 * (kb % 4)) + (kb % 16) / 4,
 *     and record (r / 16, kb / 16) starts at (r / 16) * lds + (kb / 16) * 256.
 *     So dword L of a record is lane L's register for four consecutive K
 *     steps (byte t for step t).  lds is the byte stride between 16-row
 *     groups: a multiple of 4, at least 256 * ceil(K / 512).  The buffer
 *     holds ceil(rows / 16) groups; bytes of incomplete records (rows past the
 *     last row, blocks past K) are not written.  In the grouped form, scale
 *     row so = scales_offsets[g] + (r - row_offsets[g]) goes to row group
 *     so / 16 (keeping scales_offsets multiples of 16 keeps each group's rows
 *     in their own records).  Measured on the hardware with one-wave probes
 *     of known FP4 and FP8 operands.
 */
enum bsq_scale_layout { BSQ_SCALES_ROW_MAJOR = 0, BSQ_SCALES_MFMA16 = 1 };

enum bsq_status {
    BSQ_OK = 0,
    BSQ_ERR_INVALID_ARG = 1, /* bad size, stride, alignment, pointer or scale */
    BSQ_ERR_UNSUPPORTED = 2, /* (format, block_size) pair or layout not provided */
    BSQ_ERR_HIP = 3          /* the HIP runtime reported an error at launch */
};

/*
 * Dense form: quantize every row of a BF16 matrix.
 *
 *   format, block_size  (BSQ_MXFP4, 32), (BSQ_MXFP8, 32) or (BSQ_NVFP4, 16);
 *                       any other pair -> BSQ_ERR_UNSUPPORTED.
 *   scale_layout        BSQ_SCALES_ROW_MAJOR, or BSQ_SCALES_MFMA16 (MX).
 *   x                   BF16 [M, K], row-major, row stride ldx elements.
 *                       16-byte aligned; ldx >= K and ldx % 8 == 0.
 *   M, K                M >= 0, K >= 0, K % block_size == 0.
 *   codes               uint8 [M, ldq]: row r holds K/2 bytes (FP4) or K
 *                       bytes (FP8) of codes.  FP4: 4-byte aligned,
 *                       ldq % 4 == 0, ldq >= K/2.  FP8: 8-byte aligned,
 *                       ldq % 8 == 0, ldq >= K.
 *   scales              row-major: uint8 [M, lds], row r holds the
 *                       K/block_size block scales of row r; lds >=
 *                       K/block_size.  MFMA layout: see above.
 *   tensor_sf           NVFP4 only (ignored for MX): finite and within
 *                       [2^-117, 2^100], so that s * tsf is a normal fp32 or
 *                       zero and its reciprocal is finite; else
 *                       BSQ_ERR_INVALID_ARG.
 *   stream              hipStream_t or NULL.
 *   Returns a bsq_status.
 */
int quantize_block_scaled(int format, int block_size, int scale_layout,
                          const void* x, int64_t M, int64_t K, int64_t ldx,
                          void* codes, int64_t ldq,
                          void* scales, int64_t lds,
                          float tensor_sf, void* stream);

/*
 * Grouped per-expert form (MoE).  Group g in [0, num_groups) owns the
 * routed rows [row_offsets[g], row_offsets[g+1]).  Routed row r:
 *   - reads source row row_indices[r] of x, or row r when row_indices is NULL;
 *   - is quantized like a dense row, NVFP4 with tsf = tensor_sf[expert_ids[g]];
 *   - writes its codes to row r of `codes` (routed order, unpadded);
 *   - writes its scales to row scales_offsets[g] + (r - row_offsets[g]) of
 *     `scales`.
 * Rows no group owns, and scale rows between groups (padding), are not
 * touched.  The group of r is found on the device (no host synchronisation):
 * g is the last index with row_offsets[g] <= r, so empty groups (repeated
 * offsets) are skipped.
 *
 *   x, num_src_rows, K, ldx   source BF16 rows, as for the dense form.
 *   row_indices      int32 [max_rows] or NULL.  With NULL, max_rows must not
 *                    exceed num_src_rows.
 *   row_offsets      uint32 [num_groups + 1], nondecreasing,
 *                    row_offsets[num_groups] <= max_rows.
 *   scales_offsets   uint32 [num_groups + 1], nondecreasing, with
 *                    scales_offsets[g+1] - scales_offsets[g] >= the rows of g.
 *   expert_ids       int32 [num_groups], values in [0, num_experts).
 *   tensor_sf        fp32 [num_experts] for NVFP4 (each value obeying the
 *                    dense tensor_sf domain); ignored (may be NULL) for MX.
 *   num_groups       >= 0 and at most 2^28.  num_experts >= 1 for NVFP4.
 *   max_rows         host-side bound on routed rows; sizes the grid, so the
 *                    device offsets are never read on the host.  <= 2^32.
 *   num_scale_rows   rows in the scales buffer.  This argument is the one
 *                    deliberate addition to the grouped kernel page's
 *                    argument list (offsets, ids, per-expert scale and gather
 *                    carry no buffer sizes there): with it the kernel skips a
 *                    routed row whose scale row would fall outside the buffer,
 *                    so violated device-side preconditions cannot make it
 *                    write out of bounds.
 *   codes, ldq       uint8 [max_rows, ldq], as for the dense form.
 *   scales, lds      uint8 [num_scale_rows, lds] (row-major), or the MFMA
 *                    layout over num_scale_rows rows.
 * The device-array contents above are preconditions and are not checked on
 * the host.  The kernels still never access memory outside the buffers the
 * sizes describe: a routed row whose group, source row, expert id or scale
 * row falls outside them is skipped.
 */
int grouped_quantize_block_scaled(int format, int block_size, int scale_layout,
                                  const void* x, int64_t num_src_rows, int64_t K, int64_t ldx,
                                  const int32_t* row_indices,
                                  const uint32_t* row_offsets,
                                  const uint32_t* scales_offsets,
                                  const int32_t* expert_ids,
                                  const float* tensor_sf,
                                  int64_t num_groups, int64_t num_experts,
                                  int64_t max_rows, int64_t num_scale_rows,
                                  void* codes, int64_t ldq,
                                  void* scales, int64_t lds,
                                  void* stream);

/*
 * NVFP4 tensor scale, the step before the NVFP4 quantizer (the pages take it
 * as an input: the scalar tensor_sf of the "quantize_dynamic_scaled_async_fp4_kernel"
 * page's signature, the per-expert sf of the grouped kernel page's Parameters).
 *
 *   tsf = fl32(amax / 2688), 2688 = 6 * 448 (the largest E2M1 code under the
 *   largest E4M3 block scale), amax = the largest |x| over the finite
 *   elements (NaN and Inf are skipped); 1.0 when amax is 0 (no finite
 *   non-zero element, or no element); clamped to [2^-117, 2^100] so that the
 *   result is always a valid tensor_sf for the quantizer.
 *
 * Dense: one value over the [M, K] matrix x (layout as for
 * quantize_block_scaled; K % 16 == 0) into tensor_sf_out[0], a device float.
 *
 * Grouped: tensor_sf_out[e] (device float [num_experts]) for every expert e,
 * over the routed rows of the groups g with expert_ids[g] == e (each routed
 * row r reads source row row_indices[r], or r when row_indices is NULL);
 * experts without routed rows get 1.0.  Arguments as for
 * grouped_quantize_block_scaled; num_experts >= 1.
 *
 * Both run three kernels on `stream` and use tensor_sf_out itself as the
 * accumulator: it is fully overwritten, and valid after the stream is
 * synchronised.  Errors and validation as for the quantizer.  The result can
 * feed grouped_quantize_block_scaled's tensor_sf directly (with one group
 * covering all rows, the grouped form is the dense form reading its tensor
 * scale from device memory), so quantization needs no host round trip.
 */
int tensor_scale_nvfp4(const void* x, int64_t M, int64_t K, int64_t ldx,
                       float* tensor_sf_out, void* stream);

int grouped_tensor_scale_nvfp4(const void* x, int64_t num_src_rows, int64_t K, int64_t ldx,
                               const int32_t* row_indices,
                               const uint32_t* row_offsets,
                               const int32_t* expert_ids,
                               int64_t num_groups, int64_t num_experts, int64_t max_rows,
                               float* tensor_sf_out, void* stream);

/*
 * Dequantization, the decode direction of the formats above: the consumer-
 * side check that codes and scales are usable as GEMM operands (the
 * "block_scaled_quantization" module page lists a naive block-scaled matmul
 * as the reference GEMM over such operands).
 *
 *   out[r, k] = fl32(value of code (r, k) times its block scale), where the
 *   block scale is 2^(b - 127) for MX (b = 0xFF: NaN) and s * tensor_sf for
 *   NVFP4 (s the E4M3 scale byte with its sign; 0x7F / 0xFF: NaN).  MX values
 *   are exact (or overflow to infinity for scale bytes no quantizer above
 *   writes); NVFP4 values are the exact product rounded once.  E4M3 element
 *   codes 0x7F / 0xFF decode to NaN; FP4 codes keep their sign (0x8 is -0).
 *
 *   format, block_size, scale_layout   as for quantize_block_scaled.
 *   codes, ldq, scales, lds, M, K      a quantizer's output (same layout,
 *                                      alignment and stride rules).
 *   tensor_sf                          NVFP4 only, same domain as the quantizer.
 *   out, ldo                           fp32 [M, ldo], 16-byte aligned,
 *                                      ldo >= K and ldo % 4 == 0 (elements).
 *   M == 0 or K == 0 is a no-op.
 */
int dequantize_block_scaled(int format, int block_size, int scale_layout,
                            const void* codes, int64_t M, int64_t K, int64_t ldq,
                            const void* scales, int64_t lds, float tensor_sf,
                            float* out, int64_t ldo, void* stream);

/*
 * Naive block-scaled GEMM (no matrix cores): c[m, n] = sum over k of
 * A[m, k] * B[n, k], where A ([M, K]) and B ([N, K]) are two quantizer
 * outputs of one format, both blocked along K (B is K-major, i.e. the GEMM
 * computes A B^T), dequantized exactly as dequantize_block_scaled does.  Each
 * thread computes one c[m, n], summing fl32(a * b) into an fp32 accumulator
 * in ascending k.  A reference consumer, not a fast GEMM.
 *
 *   a_codes, lda_q, a_scales, lda_s, a_tsf   operand A (a_tsf: NVFP4 only)
 *   b_codes, ldb_q, b_scales, ldb_s, b_tsf   operand B
 *   M, N, K        M, N >= 0; K % block_size == 0; M * N <= 2^38
 *   c, ldc         fp32 [M, ldc], 4-byte aligned, ldc >= N
 *   M == 0 or N == 0 is a no-op; K == 0 writes zeros.
 */
int block_scaled_matmul_naive(int format, int block_size, int scale_layout,
                              const void* a_codes, int64_t lda_q, const void* a_scales,
                              int64_t lda_s, float a_tsf,
                              const void* b_codes, int64_t ldb_q, const void* b_scales,
                              int64_t ldb_s, float b_tsf,
                              int64_t M, int64_t N, int64_t K, float* c, int64_t ldc,
                              void* stream);

/*
 * Block-scaled GEMM on the matrix cores: c = A B^T with gfx950's
 * v_mfma_scale_f32_16x16x128_f8f6f4, reading two MX quantizer outputs as
 * they are -- codes row-major, scales in BSQ_SCALES_MFMA16 -- the CDNA4
 * counterpart of the block-scaled matmuls the "block_scaled_quantization"
 * module page lists.  Workgroups compute 256 x 256 tiles of c (128 x 128
 * when the larger ones would not fill the chip), staging 128-byte K slices
 * of both operands and their scale records in LDS through the direct
 * global-to-LDS loads.  With few rows (a dense layer at decode: M <= 32)
 * they compute 16- or 32-row tiles, 64 columns wide, that stream B once
 * through each wave's own LDS slice, the grouped GEMM's decode form.  The
 * instruction's own arithmetic sets the accuracy:
 * FP4 products and their sums come out as exact fp32 sums would; FP8
 * products are summed inside each 128-element K step at reduced precision
 * (measured error up to about 2^-12 of the largest product of the step);
 * steps are accumulated in fp32 in ascending K.
 *
 *   format, block_size   (BSQ_MXFP4, 32) or (BSQ_MXFP8, 32); NVFP4 ->
 *                        BSQ_ERR_UNSUPPORTED.
 *   scale_layout         BSQ_SCALES_MFMA16 (anything else ->
 *                        BSQ_ERR_UNSUPPORTED).
 *   a_codes, lda_q       operand A [M, K]: code rows 16-byte aligned (base
 *                        and lda_q multiples of 16); a_scales, lda_s its
 *                        scales in the MFMA layout, ceil(M / 16) row groups
 *                        of lda_s bytes, 16-byte aligned (base and lda_s
 *                        multiples of 16).
 *   b_codes, ...         operand B [N, K], likewise.
 *   M, N, K              K % 128 == 0; M * N <= 2^38.
 *   c, ldc               fp32 [M, ldc], 4-byte aligned, ldc >= N.
 *   M == 0 or N == 0 is a no-op; K == 0 writes zeros.
 */
int block_scaled_matmul_mfma(int format, int block_size, int scale_layout,
                             const void* a_codes, int64_t lda_q, const void* a_scales,
                             int64_t lda_s,
                             const void* b_codes, int64_t ldb_q, const void* b_scales,
                             int64_t ldb_s,
                             int64_t M, int64_t N, int64_t K, float* c, int64_t ldc,
                             void* stream);

/*
 * Grouped per-expert block-scaled GEMM on the matrix cores (the counterpart
 * of the grouped per-expert MXFP4 matmul the "block_scaled_quantization"
 * module page lists for CDNA4): for each group g with expert e =
 * expert_ids[g], the routed rows r in [row_offsets[g], row_offsets[g+1]) get
 *     c[r, n] = sum over k of A[r, k] * B_e[n, k],
 * A being the grouped quantizer's output (codes row r; scales in the MFMA
 * layout at scale row scales_offsets[g] + r - row_offsets[g]) and B_e
 * expert e's weights.  Rows of c no group owns are not written.  Accuracy
 * as for block_scaled_matmul_mfma.
 *
 * The tile follows the rows per group on average, max_rows / num_groups,
 * chosen on the host (the offsets stay on the device), after the decode /
 * prefill split in the "NVFP4 routing" section of the grouped block-scaled
 * SM100 matmul's "dispatch" page: at most 4 take 16-row tiles and at most 16
 * take 32-row tiles, both streaming each expert's weights through each wave's
 * own LDS slice; more take 128-row tiles staged through LDS.  All give the
 * same results within the stated bound.
 *
 *   format, block_size, scale_layout   as for block_scaled_matmul_mfma.
 *   a_codes, lda_q       [max_rows, K] codes (routed order), 16-byte aligned rows.
 *   a_scales, lda_s      MFMA-layout scales over num_scale_rows rows, 16-byte
 *                        aligned row groups.
 *   row_offsets, scales_offsets, expert_ids, num_groups   as for the grouped
 *                        quantizer; each scales_offsets[g] must be a multiple
 *                        of 16 (the layout's row groups) -- a group that is
 *                        not, or whose rows or scale rows fall outside
 *                        max_rows / num_scale_rows, or whose expert id is out
 *                        of range, is skipped.
 *   b_codes, ldb_q       [num_experts * N, K] codes: expert e's rows e*N .. e*N+N-1.
 *   b_scales, ldb_s      MFMA-layout scales of those rows, expert e's row
 *                        groups starting at e * ceil(N / 16).
 *   num_experts          >= 1.   N, K: K % 128 == 0.
 *   c, ldc               fp32 [max_rows, ldc], ldc >= N.
 *   num_groups == 0, max_rows == 0 or N == 0 is a no-op.
 */
int grouped_block_scaled_matmul_mfma(int format, int block_size, int scale_layout,
                                     const void* a_codes, int64_t lda_q, const void* a_scales,
                                     int64_t lda_s,
                                     const uint32_t* row_offsets, const uint32_t* scales_offsets,
                                     const int32_t* expert_ids, int64_t num_groups,
                                     int64_t max_rows, int64_t num_scale_rows,
                                     const void* b_codes, int64_t ldb_q, const void* b_scales,
                                     int64_t ldb_s, int64_t num_experts,
                                     int64_t N, int64_t K, float* c, int64_t ldc, void* stream);

/*
 * Kernel timing, a measurement aid (no counterpart on the pages).  Arms the
 * calling thread's next call into this library that takes a stream: that call
 * launches its main kernel -- the quantizer, the amax pass of the tensor
 * scale, the dequantizer or the GEMM -- through hipExtLaunchKernel with these
 * events bound to the kernel's own dispatch, so hipEventElapsedTime(start,
 * stop) is that kernel's execution time on the GPU, without the gaps between
 * launches that events recorded around the call would include.  Both are
 * hipEvent_t created with timing enabled, owned by the caller.  The next such
 * call consumes the pair whatever it returns; if it launches nothing (a no-op
 * or an error), the events are not recorded.  Both NULL disarms.
 *   Returns BSQ_OK, or BSQ_ERR_INVALID_ARG (and disarms) when exactly one is
 *   NULL.
 */
int bsq_time_next_launch(void* start_event, void* stop_event);

/* Message of the calling thread's most recent call into this library when
   that call returned a non-OK status ("" after a call that returned
   BSQ_OK, or before any call).  The pointer stays valid until the next
   call on that thread. */
const char* bsq_last_error(void);

/* Library version, e.g. "1.0.0". */
const char* bsq_version(void);

#ifdef __cplusplus
}
#endif

#endif /* BSQ_H */
