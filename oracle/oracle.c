/*
 * oracle.c -- plain, slow, scalar CPU oracle for dynamic block-scaled
 * quantization of BF16 activations to MXFP4, MXFP8 and NVFP4.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the
 * benchmark's CPU-baseline leg load this library.  It shares no code, header,
 * table or constant with the GPU library; the product never calls it.
 *
 * What is computed follows the Modular "block_scaled_quantization" module
 * page (module summary: block-scaled kernels for NVFP4, MXFP4 and MXFP8;
 * function list: quantize_dynamic_block_scaled, quantize_mx_amd,
 * quantize_dynamic_scaled_fp4fp8), the "quantize_dynamic_scaled_async_fp4_kernel"
 * page (signature: scalar tensor_sf; Parameters: SF_VECTOR_SIZE = elements
 * per block scale) and the "grouped_quantize_dynamic_scaled_fp4_async_kernel"
 * page (signature: row_offsets, scales_offsets, expert_ids, per-expert sf,
 * optional row_indices; summary: each block finds its expert by a search over
 * the offsets).  The pages never define the formats, the scale rule or the
 * rounding; the readings used here are the OCP MX v1.0 rule for MX
 * (X = floor(log2 amax) - emax of the element format, E8M0 byte X + 127,
 * round to nearest even with saturation) and, for NVFP4, an E4M3 block scale
 * s = RNE_sat(fl32(fl32(amax / 6) / tensor_sf)), one fp32 reciprocal of
 * s * tensor_sf per block and an fp32 multiply per element.  Zero, NaN and
 * Inf rules are spelled out at each function.
 *
 * Arithmetic: element values are decoded exactly into double.  The NVFP4
 * steps that the reading fixes in fp32 are done in float; the library is
 * built -O2 -fno-fast-math -ffp-contract=off and sets the SSE control word
 * to round-to-nearest-even with no flush-to-zero / denormals-are-zero on
 * entry to every exported call (restoring it on exit).
 *
 * Nothing here is blocked, fused or reordered: rows, then blocks, then
 * elements, each step in the order given above.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#include <xmmintrin.h>
#include <float.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#if FLT_EVAL_METHOD != 0
#error "float arithmetic must be evaluated in float (SSE)"
#endif

#define O_MXFP4 0
#define O_MXFP8 1
#define O_NVFP4 2

#define O_OK 0
#define O_BAD 1

/* ---------------------------------------------------------------------- */
/* IEEE control word handling                                              */

static unsigned int enter_ieee(void) {
    unsigned int old = _mm_getcsr();
    /* round to nearest (bits 13-14 = 0), FZ (bit 15) off, DAZ (bit 6) off,
       all exceptions masked (bits 7-12 set). */
    _mm_setcsr(0x1F80u);
    return old;
}
static void leave_ieee(unsigned int old) { _mm_setcsr(old); }

/* ---------------------------------------------------------------------- */
/* Formats, from their field definitions                                   */

/* BF16: sign bit 15, 8 exponent bits (bias 127), 7 mantissa bits.
   Exponent field 0 is subnormal (m * 2^-133); 255 is Inf/NaN. */
static int bf16_is_special(uint16_t h) { return ((h >> 7) & 0xFF) == 0xFF; }
static int bf16_sign(uint16_t h) { return h >> 15; }
static double bf16_magnitude(uint16_t h) {
    int e = (h >> 7) & 0xFF;
    int m = h & 0x7F;
    if (e == 0) return ldexp((double)m, -133);
    return ldexp((double)(128 + m), e - 134);
}
static double bf16_value(uint16_t h) {
    double a = bf16_magnitude(h);
    return bf16_sign(h) ? -a : a;
}

/* E2M1 magnitude code c in 0..7: 2 exponent bits (bias 1), 1 mantissa bit.
   Exponent field 0 is subnormal: m * 0.5.  Largest magnitude 6. */
static double e2m1_magnitude(int c) {
    int e = (c >> 1) & 3, m = c & 1;
    if (e == 0) return 0.5 * m;
    return ldexp(1.0 + 0.5 * m, e - 1);
}

/* E4M3 ("FN": no infinities) magnitude code c in 0..126: 4 exponent bits
   (bias 7), 3 mantissa bits; exponent field 0 is subnormal m * 2^-9;
   c = 127 is NaN.  Largest magnitude 448. */
static double e4m3_magnitude(int c) {
    int e = (c >> 3) & 15, m = c & 7;
    if (e == 0) return ldexp((double)m, -9);
    return ldexp(1.0 + m / 8.0, e - 7);
}

/* E8M0 scale byte b: 2^(b-127); 255 is NaN. */
static double e8m0_value(int b) {
    if (b == 255) return NAN;
    return ldexp(1.0, b - 127);
}

/* Round-to-nearest-even with saturation of a magnitude a >= 0 (a may be
   +Inf) onto the ascending table vals[0..n-1] of a format's magnitudes,
   indexed by magnitude code.  Codes are consecutive in magnitude, so the
   even code is the one whose mantissa LSB is 0.  Anything at or above the
   largest magnitude returns the largest code. */
static int rne_sat_code(const double* vals, int n, double a) {
    if (a >= vals[n - 1]) return n - 1;
    /* binary search for k with vals[k] <= a < vals[k+1] */
    int lo = 0, hi = n - 1;
    while (hi - lo > 1) {
        int mid = (lo + hi) / 2;
        if (vals[mid] <= a) lo = mid; else hi = mid;
    }
    int k = lo;
    /* compare 2a with vals[k] + vals[k+1]; both sides exact in double */
    double twice = 2.0 * a, mid = vals[k] + vals[k + 1];
    if (twice < mid) return k;
    if (twice > mid) return k + 1;
    return (k % 2 == 0) ? k : k + 1;
}

static double E2M1_TAB[8];
static double E4M3_TAB[127];
static int tables_ready = 0;

static void init_tables(void) {
    if (tables_ready) return;
    for (int c = 0; c < 8; ++c) E2M1_TAB[c] = e2m1_magnitude(c);
    for (int c = 0; c < 127; ++c) E4M3_TAB[c] = e4m3_magnitude(c);
    tables_ready = 1;
}

/* signed 4-bit E2M1 code of value v (sign bit 3 = sign of v, -0 included) */
static uint8_t e2m1_code(double v, int neg) {
    return (uint8_t)((neg ? 8 : 0) | rne_sat_code(E2M1_TAB, 8, fabs(v)));
}
/* signed 8-bit E4M3 code of value v (sign bit 7) */
static uint8_t e4m3_code(double v, int neg) {
    return (uint8_t)((neg ? 0x80 : 0) | rne_sat_code(E4M3_TAB, 127, fabs(v)));
}

/* floor(log2 a) for finite a > 0: frexp gives a = f * 2^ex, f in [0.5, 1) */
static int floor_log2(double a) {
    int ex;
    frexp(a, &ex);
    return ex - 1;
}

/* ---------------------------------------------------------------------- */
/* One block                                                               */

/* MX block (OCP MX v1.0 reading).  emax is the element format's largest
   exponent (2 for E2M1, 8 for E4M3).  Outputs one code per element (not yet
   packed) and the E8M0 scale byte.
   - Any NaN/Inf element: scale 0xFF (the E8M0 NaN), every code 0.
   - amax = 0: X = -127 (scale byte 0), codes are signed zeros.
   - Else X = max(floor(log2 amax) - emax, -127); v = x * 2^-X exactly;
     code = RNE_sat(v) with the sign of x. */
static void mx_block(const uint16_t* x, int bs, int fmt, uint8_t* codes, uint8_t* scale) {
    int emax = (fmt == O_MXFP4) ? 2 : 8;
    int special = 0;
    double amax = 0.0;
    for (int i = 0; i < bs; ++i) {
        if (bf16_is_special(x[i])) special = 1;
        else if (bf16_magnitude(x[i]) > amax) amax = bf16_magnitude(x[i]);
    }
    if (special) {
        *scale = 0xFF;
        for (int i = 0; i < bs; ++i) codes[i] = 0;
        return;
    }
    int X = (amax == 0.0) ? -127 : floor_log2(amax) - emax;
    if (X < -127) X = -127;
    *scale = (uint8_t)(X + 127);
    for (int i = 0; i < bs; ++i) {
        double v = ldexp(bf16_value(x[i]), -X);
        int neg = bf16_sign(x[i]);
        codes[i] = (fmt == O_MXFP4) ? e2m1_code(v, neg) : e4m3_code(v, neg);
    }
}

/* NVFP4 block with fp32 tensor scale tsf (decode direction: value =
   code * s * tsf).
   - Any NaN/Inf element: scale 0x7F (the E4M3 NaN), every code 0.
   - t1 = fl32(amax / 6), t2 = fl32(t1 / tsf), s = E4M3 RNE_sat(t2).
   - d = fl32(s * tsf); inv = 0 if d == 0 else fl32(1 / d).
   - v = fl32(x * inv); code = E2M1 RNE_sat(v) with the sign of x. */
static void nvfp4_block(const uint16_t* x, int bs, float tsf, uint8_t* codes, uint8_t* scale) {
    int special = 0;
    double amax = 0.0;
    for (int i = 0; i < bs; ++i) {
        if (bf16_is_special(x[i])) special = 1;
        else if (bf16_magnitude(x[i]) > amax) amax = bf16_magnitude(x[i]);
    }
    if (special) {
        *scale = 0x7F;
        for (int i = 0; i < bs; ++i) codes[i] = 0;
        return;
    }
    float amax_f = (float)amax; /* exact: a BF16 value */
    float t1 = amax_f / 6.0f;
    float t2 = t1 / tsf;
    int s = rne_sat_code(E4M3_TAB, 127, (double)t2);
    *scale = (uint8_t)s;
    float d = (float)E4M3_TAB[s] * tsf;
    float inv = (d == 0.0f) ? 0.0f : 1.0f / d;
    for (int i = 0; i < bs; ++i) {
        float xf = (float)bf16_value(x[i]); /* exact */
        float v = xf * inv;
        codes[i] = e2m1_code((double)v, bf16_sign(x[i]));
    }
}

/* Quantize one row of K elements: codes for element k go to byte k (FP8) or
   to nibble k%2 of byte k/2, lower-indexed element in the low nibble (FP4);
   the scale of block j goes to scale byte j. */
static void quantize_row(int fmt, int bs, const uint16_t* x, int64_t K,
                         uint8_t* qrow, uint8_t* srow, float tsf, uint8_t* tmp) {
    for (int64_t j = 0; j < K / bs; ++j) {
        const uint16_t* xb = x + j * bs;
        if (fmt == O_NVFP4) nvfp4_block(xb, bs, tsf, tmp, &srow[j]);
        else mx_block(xb, bs, fmt, tmp, &srow[j]);
        for (int i = 0; i < bs; ++i) {
            int64_t k = j * bs + i;
            if (fmt == O_MXFP8) {
                qrow[k] = tmp[i];
            } else if (k % 2 == 0) {
                qrow[k / 2] = (uint8_t)((qrow[k / 2] & 0xF0) | tmp[i]);
            } else {
                qrow[k / 2] = (uint8_t)((qrow[k / 2] & 0x0F) | (tmp[i] << 4));
            }
        }
    }
}

static int check_common(int fmt, int bs, int64_t M, int64_t K, int64_t ldx, int64_t ldq, int64_t lds) {
    if (fmt != O_MXFP4 && fmt != O_MXFP8 && fmt != O_NVFP4) return O_BAD;
    if (bs < 1 || bs > 4096) return O_BAD;
    if (M < 0 || K < 0 || K % bs != 0) return O_BAD;
    if (fmt != O_MXFP8 && bs % 2 != 0 && K > 0) return O_BAD; /* FP4 pairs share a byte */
    if (ldx < K) return O_BAD;
    if (ldq < ((fmt == O_MXFP8) ? K : K / 2)) return O_BAD;
    if (lds < K / bs) return O_BAD;
    return O_OK;
}

/* ---------------------------------------------------------------------- */
/* Exported entry points                                                   */

/* Dense form: x is [M, K] BF16 bits with row stride ldx (elements); codes
   [M, ldq] bytes; scales [M, lds] bytes.  tsf is used by NVFP4 only.
   nthreads > 1 splits rows statically over OpenMP threads (same result). */
int oracle_quantize(int fmt, int bs, const uint16_t* x, int64_t M, int64_t K, int64_t ldx,
                    uint8_t* codes, int64_t ldq, uint8_t* scales, int64_t lds, float tsf,
                    int nthreads) {
    if (check_common(fmt, bs, M, K, ldx, ldq, lds) != O_OK) return O_BAD;
    init_tables();
    if (nthreads < 1) nthreads = 1;
    int bad = 0;
#pragma omp parallel for schedule(static) num_threads(nthreads) reduction(| : bad)
    for (int64_t r = 0; r < M; ++r) {
        unsigned int old = enter_ieee();
        uint8_t tmp[4096];
        quantize_row(fmt, bs, x + r * ldx, K, codes + r * ldq, scales + r * lds, tsf, tmp);
        leave_ieee(old);
    }
    return bad ? O_BAD : O_OK;
}

/* Grouped per-expert form.  Groups g in [0, G) own the routed rows
   [row_offsets[g], row_offsets[g+1]).  Routed row r reads source row
   row_indices[r] (or r when row_indices is NULL), is quantized with tensor
   scale sf[expert_ids[g]] (NVFP4), writes its codes to row r of codes and
   its scales to row scales_offsets[g] + (r - row_offsets[g]) of scales.
   The group of r is found by a plain linear scan.  Every other byte of
   codes and scales is left as it was. */
int oracle_grouped_quantize(int fmt, int bs, const uint16_t* x, int64_t num_src_rows, int64_t K,
                            int64_t ldx, const int32_t* row_indices, const uint32_t* row_offsets,
                            const uint32_t* scales_offsets, const int32_t* expert_ids,
                            const float* sf, int64_t G, int64_t E, uint8_t* codes, int64_t ldq,
                            uint8_t* scales, int64_t lds, int nthreads) {
    if (check_common(fmt, bs, num_src_rows, K, ldx, ldq, lds) != O_OK) return O_BAD;
    if (G < 0) return O_BAD;
    if (G == 0) return O_OK;
    init_tables();
    if (nthreads < 1) nthreads = 1;
    int64_t r0 = row_offsets[0], r1 = row_offsets[G];
    int bad = 0;
#pragma omp parallel for schedule(static) num_threads(nthreads) reduction(| : bad)
    for (int64_t r = r0; r < r1; ++r) {
        int64_t g = -1;
        for (int64_t h = 0; h < G; ++h) {
            if ((int64_t)row_offsets[h] <= r && r < (int64_t)row_offsets[h + 1]) { g = h; break; }
        }
        if (g < 0) { bad = 1; continue; }
        int64_t src = row_indices ? (int64_t)row_indices[r] : r;
        if (src < 0 || src >= num_src_rows) { bad = 1; continue; }
        float tsf = 0.0f;
        if (fmt == O_NVFP4) {
            int32_t e = expert_ids[g];
            if (e < 0 || e >= E) { bad = 1; continue; }
            tsf = sf[e];
        }
        int64_t srow = (int64_t)scales_offsets[g] + (r - (int64_t)row_offsets[g]);
        unsigned int old = enter_ieee();
        uint8_t tmp[4096];
        quantize_row(fmt, bs, x + src * ldx, K, codes + r * ldq, scales + srow * lds, tsf, tmp);
        leave_ieee(old);
    }
    return bad ? O_BAD : O_OK;
}

/* Preconditions of the grouped form that live in device arrays: offsets
   nondecreasing, row_offsets[G] <= max_rows, every group's scale rows fit in
   its scale-offset gap and below num_scale_rows, ids in [0, E), gather
   indices in [0, num_src_rows).  Returns 0 when all hold. */
int oracle_validate_grouped(const uint32_t* row_offsets, const uint32_t* scales_offsets,
                            const int32_t* expert_ids, const int32_t* row_indices, int64_t G,
                            int64_t E, int64_t max_rows, int64_t num_scale_rows,
                            int64_t num_src_rows) {
    if (G < 0) return 1;
    for (int64_t g = 0; g < G; ++g) {
        if (row_offsets[g + 1] < row_offsets[g]) return 2;
        if (scales_offsets[g + 1] < scales_offsets[g]) return 3;
        if ((int64_t)scales_offsets[g + 1] - scales_offsets[g] <
            (int64_t)row_offsets[g + 1] - row_offsets[g])
            return 4;
        if (expert_ids[g] < 0 || expert_ids[g] >= E) return 5;
    }
    if ((int64_t)row_offsets[G] > max_rows) return 6;
    if ((int64_t)scales_offsets[G] > num_scale_rows) return 7;
    if (row_indices) {
        for (int64_t r = row_offsets[0]; r < (int64_t)row_offsets[G]; ++r)
            if (row_indices[r] < 0 || row_indices[r] >= num_src_rows) return 8;
    } else if ((int64_t)row_offsets[G] > num_src_rows) {
        return 9;
    }
    return 0;
}

/* Dequantize: out[r*K + k] = decoded code * block scale, in double.  MX:
   code * 2^(b-127) (NaN for b = 255).  NVFP4: code * s * tsf (NaN for
   s = 0x7F).  The product is exact in double. */
int oracle_dequantize(int fmt, int bs, const uint8_t* codes, int64_t M, int64_t K, int64_t ldq,
                      const uint8_t* scales, int64_t lds, float tsf, double* out) {
    if (check_common(fmt, bs, M, K, K, ldq, lds) != O_OK) return O_BAD;
    init_tables();
    for (int64_t r = 0; r < M; ++r) {
        for (int64_t k = 0; k < K; ++k) {
            int c;
            double mag;
            int neg;
            if (fmt == O_MXFP8) {
                c = codes[r * ldq + k];
                neg = c >> 7;
                mag = ((c & 0x7F) == 0x7F) ? NAN : E4M3_TAB[c & 0x7F];
            } else {
                uint8_t b = codes[r * ldq + k / 2];
                c = (k % 2 == 0) ? (b & 0xF) : (b >> 4);
                neg = c >> 3;
                mag = E2M1_TAB[c & 7];
            }
            int sb = scales[r * lds + k / bs];
            double sc;
            if (fmt == O_NVFP4) sc = (sb == 0x7F || sb == 0xFF) ? NAN : e4m3_magnitude(sb & 0x7F) * (double)tsf;
            else sc = e8m0_value(sb);
            if (fmt == O_NVFP4 && (sb & 0x80)) sc = -sc;
            double v = mag * sc;
            out[r * K + k] = neg ? -v : v;
        }
    }
    return O_OK;
}

/* Scale layout for the gfx950 scaled matrix instruction
   v_mfma_scale_f32_16x16x128_f8f6f4 (MX formats; 32-element blocks, E8M0).
   That instruction takes, in each of the 64 lanes, one 32-bit register of
   scale bytes and a byte selector: the scale of A row r (0..15) and K-block
   q (0..3) of its 128-element K step comes from lane r + 16 q.  (Measured on
   the hardware with one-wave probes of known operands, for FP4 and FP8, both
   16x16x128 and 32x32x64 shapes; the pages describe only the SM100
   interleave.)  The layout packs four K steps into each lane's register:
   rows in groups of 16 and blocks in groups of 16 (512 elements) form one
   256-byte record, record (r / 16, kb / 16) at byte offset
   (r / 16) * lds + (kb / 16) * 256, and inside it the byte of (r, kb) at
   4 * ((r % 16) + 16 * (kb % 4)) + (kb % 16) / 4.  A GEMM wave loads one dword
   per lane per record and feeds byte t to the t-th of four instructions.

   mfma16_scale_offset gives that byte offset; oracle_scales_to_mfma16 copies
   row-major scales [rows, nblk] (stride lds_rm) into the layout (row-group
   stride lds_out bytes); bytes of incomplete records are left untouched. */
static int64_t mfma16_scale_offset(int64_t r, int64_t kb, int64_t lds) {
    return (r / 16) * lds + (kb / 16) * 256 + 4 * ((r % 16) + 16 * (kb % 4)) + (kb % 16) / 4;
}

int64_t oracle_mfma16_scale_offset(int64_t r, int64_t kb, int64_t lds) {
    return mfma16_scale_offset(r, kb, lds);
}

int oracle_scales_to_mfma16(const uint8_t* scales_rm, int64_t rows, int64_t nblk, int64_t lds_rm,
                            uint8_t* out, int64_t lds_out) {
    if (rows < 0 || nblk < 0 || lds_rm < nblk || lds_out < ((nblk + 15) / 16) * 256) return O_BAD;
    for (int64_t r = 0; r < rows; ++r)
        for (int64_t kb = 0; kb < nblk; ++kb)
            out[mfma16_scale_offset(r, kb, lds_out)] = scales_rm[r * lds_rm + kb];
    return O_OK;
}

/* Naive block-scaled GEMM, the consumer-side check (the Modular
   "block_scaled_quantization" module page lists a naive block-scaled matmul
   as the reference GEMM over such operands).  A and B are both quantized
   along K ([M, K] and [N, K], the second operand K-major); each is
   dequantized as above and rounded once to fp32 -- the operands a GEMM
   consumes -- and c[m * N + n] = sum over k of A[m, k] * B[n, k], summed in
   double in ascending k.  Each product of two fp32 values is exact in double,
   so the only roundings are the K - 1 double additions.  A NaN anywhere in
   row m of A or row n of B makes c[m, n] NaN. */
int oracle_block_scaled_matmul(int fmt, int bs,
                               const uint8_t* a_codes, int64_t lda_q, const uint8_t* a_scales,
                               int64_t lda_s, float a_tsf,
                               const uint8_t* b_codes, int64_t ldb_q, const uint8_t* b_scales,
                               int64_t ldb_s, float b_tsf,
                               int64_t M, int64_t N, int64_t K, double* c) {
    if (M < 0 || N < 0 || K < 0) return O_BAD;
    double* A = (double*)malloc((size_t)(M * K + 1) * sizeof(double));
    double* B = (double*)malloc((size_t)(N * K + 1) * sizeof(double));
    int rc = O_OK;
    if (!A || !B) rc = O_BAD;
    if (rc == O_OK && M > 0 && K > 0)
        rc = oracle_dequantize(fmt, bs, a_codes, M, K, lda_q, a_scales, lda_s, a_tsf, A);
    if (rc == O_OK && N > 0 && K > 0)
        rc = oracle_dequantize(fmt, bs, b_codes, N, K, ldb_q, b_scales, ldb_s, b_tsf, B);
    if (rc == O_OK) {
        unsigned int old = enter_ieee();
        for (int64_t i = 0; i < M * K; ++i) A[i] = (double)(float)A[i];
        for (int64_t i = 0; i < N * K; ++i) B[i] = (double)(float)B[i];
        for (int64_t m = 0; m < M; ++m) {
            for (int64_t n = 0; n < N; ++n) {
                double sum = 0.0;
                for (int64_t k = 0; k < K; ++k) sum += A[m * K + k] * B[n * K + k];
                c[m * N + n] = sum;
            }
        }
        leave_ieee(old);
    }
    free(A);
    free(B);
    return rc;
}

/* Tensor scale for NVFP4, the step before the quantizer (the pages take it as
   an input: the scalar tensor_sf of the dense kernel, the per-expert sf of the
   grouped one).  tsf = fl32(amax / 2688), 2688 = 6 * 448 mapping the amax onto
   the largest E2M1 code under the largest E4M3 block scale; amax is the largest
   |x| over the finite elements (NaN and Inf are skipped); amax = 0 (nothing
   finite and non-zero) gives 1.0; the result is clamped to [2^-117, 2^100],
   the domain the quantizer accepts. */
static float tensor_scale_of(double amax) {
    if (amax == 0.0) return 1.0f;
    float t = (float)amax / 2688.0f; /* (float)amax is exact: a BF16 value */
    if (t < ldexpf(1.0f, -117)) t = ldexpf(1.0f, -117);
    if (t > ldexpf(1.0f, 100)) t = ldexpf(1.0f, 100);
    return t;
}

static double row_amax(const uint16_t* x, int64_t K) {
    double amax = 0.0;
    for (int64_t k = 0; k < K; ++k)
        if (!bf16_is_special(x[k]) && bf16_magnitude(x[k]) > amax) amax = bf16_magnitude(x[k]);
    return amax;
}

/* Dense: one tensor scale over the [M, K] matrix. */
float oracle_tensor_scale(const uint16_t* x, int64_t M, int64_t K, int64_t ldx) {
    unsigned int old = enter_ieee();
    double amax = 0.0;
    for (int64_t r = 0; r < M; ++r) {
        double a = row_amax(x + r * ldx, K);
        if (a > amax) amax = a;
    }
    float t = tensor_scale_of(amax);
    leave_ieee(old);
    return t;
}

/* Grouped: out[e] for every expert e in [0, E) over the routed rows of the
   groups whose expert_ids[g] == e (source row row_indices[r] or r); experts
   with no routed rows get 1.0. */
int oracle_grouped_tensor_scale(const uint16_t* x, int64_t num_src_rows, int64_t K, int64_t ldx,
                                const int32_t* row_indices, const uint32_t* row_offsets,
                                const int32_t* expert_ids, int64_t G, int64_t E, float* out) {
    if (G < 0 || E < 0 || K < 0) return O_BAD;
    unsigned int old = enter_ieee();
    for (int64_t e = 0; e < E; ++e) {
        double amax = 0.0;
        for (int64_t g = 0; g < G; ++g) {
            if (expert_ids[g] != e) continue;
            for (int64_t r = row_offsets[g]; r < (int64_t)row_offsets[g + 1]; ++r) {
                int64_t src = row_indices ? (int64_t)row_indices[r] : r;
                if (src < 0 || src >= num_src_rows) { leave_ieee(old); return O_BAD; }
                double a = row_amax(x + src * ldx, K);
                if (a > amax) amax = a;
            }
        }
        out[e] = tensor_scale_of(amax);
    }
    leave_ieee(old);
    return O_OK;
}

/* Element-level views used by the pin tests. */
int oracle_e2m1_code(double v) { init_tables(); return e2m1_code(v, signbit(v) != 0); }
int oracle_e4m3_code(double v) { init_tables(); return e4m3_code(v, signbit(v) != 0); }
double oracle_e2m1_decode(int c) { double a = e2m1_magnitude(c & 7); return (c & 8) ? -a : a; }
double oracle_e4m3_decode(int c) {
    if ((c & 0x7F) == 0x7F) return NAN;
    double a = e4m3_magnitude(c & 0x7F);
    return (c & 0x80) ? -a : a;
}
double oracle_e8m0_decode(int b) { return e8m0_value(b & 0xFF); }
double oracle_bf16_decode(int h) {
    uint16_t u = (uint16_t)h;
    if (bf16_is_special(u)) return (u & 0x7F) ? NAN : (bf16_sign(u) ? -INFINITY : INFINITY);
    return bf16_value(u);
}
