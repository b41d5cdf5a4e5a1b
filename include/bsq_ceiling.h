/*
 * bsq_ceiling.h -- C ABI of libbsq_ceiling, a measurement aid beside libbsq:
 * trivial streams with the memory traffic of a dense quantizer launch and of
 * a dequantizer launch, with the kernels' own tiles and load and store
 * instructions, whose times are the bandwidth those byte mixes reach with
 * that instruction shape on this chip.  They compute nothing of the method
 * (no block amax, scale, rounding or decoding).
 *
 * bsq_ceiling_stream reads x, BF16 [M, K] (contiguous rows, 16-byte aligned),
 * and writes codes ([M, K/2] bytes for format 0 or 2, [M, K] for format 1;
 * contiguous rows, 8-byte aligned) and scales ([M, K/32] bytes for formats 0
 * and 1, [M, K/16] for format 2; contiguous rows) with the quantizer's own
 * tiles of chunks_per_wave (1, 2 or 4) chunks of 512 elements per wave, its
 * load and store instructions and cache policies.  Lane l's codes for the
 * chunk of elements [512 c, 512 c + 512) of a row are an XOR fold of the four
 * words it loaded (FP4: one word w0^w1^w2^w3; FP8: w0^w1 then w2^w3); the
 * scale byte of block b of that chunk is the low byte of the first word of
 * lane L b + (c mod min(chunks_per_wave, L)), with L = 4 lanes per 32-element
 * block and 2 per 16-element block.
 *
 *   format        0, 1 or 2 (the code width and block size of MXFP4, MXFP8, NVFP4).
 *   K             a multiple of 512.
 *   start_event, stop_event   hipEvent_t pair bound to the kernel's dispatch
 *                 (hipExtLaunchKernel), or both NULL.
 *   stream        hipStream_t or NULL.
 * Returns 0, 1 for an invalid argument (nothing launched) or 3 for a launch
 * error.  M == 0 or K == 0 is a no-op.  All pointers are caller-owned device
 * memory; nothing is allocated.
 */
/*
 * bsq_ceiling_expand reads codes ([M, K/2] bytes for format 0 or 2, [M, K] for
 * format 1; contiguous rows, 8-byte aligned) and row-major scales ([M, K/32]
 * bytes for formats 0 and 1, [M, K/16] for format 2; contiguous rows), and
 * writes out, fp32 [M, K] (contiguous rows, 16-byte aligned), with the
 * dequantizer's tiles of chunks_per_wave (1, 2 or 4) chunks of 512 elements
 * per wave and its load and store instructions.  For lane l of the chunk of
 * elements [512 c, 512 c + 512) of a row, with q0 the first code word of its
 * elements (bytes 256 c + 4 l .. + 3 for FP4, 512 c + 8 l .. + 3 for FP8), q1
 * the second (FP8: bytes 512 c + 8 l + 4 .. + 7; FP4: 0) and s the scale byte
 * of its block, out words 512 c + 8 l .. + 3 hold the bits q0 ^ s and words
 * + 4 .. + 7 the bits q1 ^ s.  Arguments, return codes and ownership as for
 * bsq_ceiling_stream.
 */
#ifndef BSQ_CEILING_H
#define BSQ_CEILING_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

int bsq_ceiling_stream(int format, const void* x, int64_t M, int64_t K, void* codes,
                       void* scales, int chunks_per_wave, void* start_event, void* stop_event,
                       void* stream);
int bsq_ceiling_expand(int format, const void* codes, const void* scales, int64_t M, int64_t K,
                       void* out, int chunks_per_wave, void* start_event, void* stop_event,
                       void* stream);

#ifdef __cplusplus
}
#endif

#endif /* BSQ_CEILING_H */
