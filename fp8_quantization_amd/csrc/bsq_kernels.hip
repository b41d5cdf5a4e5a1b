// bsq_kernels.hip -- gfx950 kernels for dynamic block-scaled quantization of
// BF16 activations to MXFP4, MXFP8 and NVFP4, dense and grouped per-expert.
//
// The operation is the one the Modular "block_scaled_quantization" module
// page lists (NVFP4, MXFP4, MXFP8 block-scaled quantization; quantize_mx_amd
// for CDNA4), with the dense NVFP4 tensor scale and block width of the
// "quantize_dynamic_scaled_async_fp4_kernel" page and the grouped
// offsets / expert ids / per-expert scale / optional gather of the
// "grouped_quantize_dynamic_scaled_fp4_async_kernel" page.  The pages' SM100
// design (TMA, warp specialisation, PDL) is not used; this is a streaming
// design for 64-wide wavefronts:
//
//  * a wave owns a tile of one row: up to chunks_per_tile chunks of 512
//    elements; lane l holds elements [8l, 8l + 8) of a chunk, fetched with one
//    16-byte load, so every wave-wide load is 1 KiB contiguous;
//  * a wave issues all of its tile's loads back to back (no per-lane
//    condition: lanes past the row's end read an in-row address and their
//    stores are dropped), then converts each chunk as soon as its own load
//    has landed;
//  * a block spans 4 lanes (MX, 32 elements) or 2 lanes (NVFP4, 16); its
//    amax is an integer max over |BF16| bit patterns, reduced across those
//    lanes with DPP quad permutes (no LDS, no barrier);
//  * codes are stored as one dword (FP4) or two dwords (FP8) per lane, so
//    code stores are contiguous per wave; every lane of a block holds its
//    scale byte, and one byte-store instruction writes the scales of up to
//    4 (MX) or 2 (NVFP4) chunks;
//  * grouped form: each wave finds its group (last g with row_offsets[g] <=
//    r) from one 16-byte load of four offsets per lane and four ballots,
//    issued ahead of its data loads;
//  * the NVFP4 tensor-scale producer is a separate reduction: persistent
//    waves over contiguous tile ranges, a per-workgroup LDS table, and one
//    device atomic max per workgroup and expert.
//
// Numerics (identical, byte for byte, to the CPU oracle):
//  MX:    X = max(floor(log2 amax) - emax, -127) from the amax bit pattern;
//         v = x * 2^-X in fp32 (exact, or an underflow far below half the
//         smallest element subnormal, which encodes as a signed zero);
//         code = RNE with saturation, computed on the fp32 bits.
//  NVFP4: t1 = amax / 6, t2 = t1 / tsf (IEEE division), s = RNE_sat_E4M3(t2),
//         d = s * tsf, inv = 1 / d (0 when d == 0), v = x * inv, RNE to E2M1.
//  Build flags keep IEEE fp32 semantics: -ffp-contract=off, correctly
//  rounded division, fp32 denormals not flushed.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "bsq_internal.h"

namespace bsq {
namespace {

template <int FMT>
struct FormatTraits;
// MXFP4: E2M1 codes (2 per byte), 32-element blocks (4 lanes), E8M0 scale.
template <>
struct FormatTraits<0> {
    static constexpr int kBlock = 32, kLanesPerBlock = 4, kEmax = 2, kFp4 = 1;
};
// MXFP8: E4M3 codes (1 per byte), 32-element blocks (4 lanes), E8M0 scale.
template <>
struct FormatTraits<1> {
    static constexpr int kBlock = 32, kLanesPerBlock = 4, kEmax = 8, kFp4 = 0;
};
// NVFP4: E2M1 codes, 16-element blocks (2 lanes), E4M3 scale.
template <>
struct FormatTraits<2> {
    static constexpr int kBlock = 16, kLanesPerBlock = 2, kFp4 = 1;
};

// ---------------------------------------------------------------- conversions
//
// Element codes come from gfx950's scaled conversion instructions.  Their
// rounding was checked exhaustively against the software definition of
// round-to-nearest-even with saturation (every BF16 pattern under every E8M0
// scale; every fp32 pattern at scale 1):
//  * v_cvt_scalef32_pk_fp4_bf16 with a scale operand whose exponent field is
//    the E8M0 byte b computes RNE_sat_E2M1(x / 2^(b-127)) (b = 0 included);
//  * v_cvt_scalef32_pk_fp4_f32 at scale 1.0 is RNE_sat_E2M1 of any fp32,
//    +-Inf saturating to +-6;
//  * the FP8 forms are RNE to E4M3 except on overflow, where they return
//    the NaN code instead of saturating, so inputs are first clamped to
//    448 * scale (which RNE maps to 448 anyway).
// All of them take the sign from the input, so -0 keeps its sign bit, and
// the low nibble / low byte receives the lower-indexed element.

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef short i16x2_t __attribute__((ext_vector_type(2)));
typedef unsigned short u16x2_t __attribute__((ext_vector_type(2)));

__device__ __forceinline__ bf16x2_t as_bf16x2(uint32_t w) { return __builtin_bit_cast(bf16x2_t, w); }

// Byte k of the result <- E2M1 codes of the two fp32 values (lo in the low
// nibble), at scale 1.0.
template <int K>
__device__ __forceinline__ uint32_t fp4_pair_f32(uint32_t acc, float lo, float hi) {
    return __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(acc, lo, hi, 1.0f, K);
}
// Byte k of the result <- E2M1 codes of the two BF16 elements of w divided by
// the power of two whose exponent field is in `scale`.
template <int K>
__device__ __forceinline__ uint32_t fp4_pair_bf16(uint32_t acc, uint32_t w, float scale) {
    return __builtin_amdgcn_cvt_scalef32_pk_fp4_bf16(acc, as_bf16x2(w), scale, K);
}

// E4M3 magnitude code of t in [0, +Inf]: RNE, saturating at 448 (0x7E).
__device__ __forceinline__ uint32_t e4m3_code_of(float t) {
    i16x2_t r = {0, 0};
    r = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(r, fminf(t, 448.0f), 0.0f, 1.0f, false);
    return (uint32_t)__builtin_bit_cast(uint32_t, r) & 0xFFu;
}

// ---------------------------------------------------------------- block amax

// |x| of two packed BF16 elements (the patterns without their sign bits).
__device__ __forceinline__ uint32_t magnitudes(uint32_t w) { return w & 0x7FFF7FFFu; }

// max |x| over the lane's 8 BF16 elements, as a 15-bit magnitude pattern.
// Integer order of |BF16| patterns is value order, with Inf above every
// finite value and NaN above Inf.
__device__ __forceinline__ uint32_t lane_amax_bits(const uint32_t (&mag)[4]) {
    u16x2_t a = __builtin_bit_cast(u16x2_t, mag[0]);
    u16x2_t b = __builtin_bit_cast(u16x2_t, mag[1]);
    u16x2_t c = __builtin_bit_cast(u16x2_t, mag[2]);
    u16x2_t d = __builtin_bit_cast(u16x2_t, mag[3]);
    u16x2_t m = __builtin_elementwise_max(__builtin_elementwise_max(a, b),
                                          __builtin_elementwise_max(c, d));
    return (uint32_t)(m.x > m.y ? m.x : m.y);
}

// Reduce across the lanes of one block (2 or 4 adjacent lanes) with DPP quad
// permutes: xor-1 swaps neighbours, xor-2 swaps pairs.  Written as a DPP move
// with bound_ctrl and a zero old value feeding an unsigned max (0 is the
// identity), which the compiler folds into a single v_max_u32_dpp.
template <int LANES>
__device__ __forceinline__ uint32_t block_amax_bits(uint32_t m) {
    m = max(m, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)m, 0xB1, 0xF, 0xF, true));  // [1,0,3,2]
    if constexpr (LANES == 4)
        m = max(m, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)m, 0x4E, 0xF, 0xF, true));  // [2,3,0,1]
    return m;
}

// ---------------------------------------------------------------- NVFP4 scale
//
// The reading fixes s = RNE_sat_E4M3(t2), t2 = fl(fl(amax / 6) / tsf), and
// inv = fl(1 / fl(dec(s) * tsf)).  Both are computed exactly, but without a
// division per block:
//
//  * s: q = fl(amax * k), k = fl(1 / fl(6 * tsf)), is within 6 fp32 ulps of
//    t2 (each of the four roundings involved adds at most 2^-24 relative
//    error; no over/underflow in the normal range).  E4M3 decisions in the
//    normal range change only at midpoints, whose fp32 patterns end in the 20
//    bits 0x80000, and none lies near a binade edge; so unless q is within 16
//    ulps of such a pattern, or below 2^-6 (the E4M3 subnormal range, zero
//    included), t2 and q round to the same s.  Those rare lanes take the
//    exact two divisions.
//  * inv: with s = (8 + m) * 2^(e-10) (e >= 1) or m * 2^-9 (e = 0), and
//    s * tsf and its reciprocal normal (the tensor-scale domain), rounding
//    commutes with the power of two, so inv = T[m or 8 + m] * 2^(10-e or 9)
//    with T[j] = fl(1 / fl((8 + j) * tsf)) and T[8 + j] = fl(1 / fl(j * tsf))
//    (T[8] = 0: s = 0 gives inv = 0).  Lanes 0..15 of each wave hold the 16
//    entries; lane 16 computes k.

struct Nvfp4Wave {
    float k;      // fl(1 / fl(6 * tsf)), wave-uniform
    int table;    // this lane's entry T[lane] (lanes 0..15), as bits
    float tsf;
};

__device__ __forceinline__ Nvfp4Wave nvfp4_wave_setup(float tsf, int lane) {
    const float mult = lane < 8 ? (float)(8 + lane) : lane < 16 ? (float)(lane - 8) : 6.0f;
    const float d = mult * tsf;
    const float r = (d == 0.0f) ? 0.0f : 1.0f / d;
    Nvfp4Wave w;
    w.k = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(r), 16));
    w.table = __float_as_int(r);
    w.tsf = tsf;
    return w;
}

// Returns the E4M3 block scale s and sets inv.  amax_f is the block's amax.
__device__ __forceinline__ uint32_t nvfp4_scale(float amax_f, const Nvfp4Wave& nw, float& inv) {
    float q = amax_f * nw.k;
    const uint32_t qb = __float_as_uint(q);
    const bool near_midpoint = ((qb & 0xFFFFFu) - 0x7FFF0u) < 0x21u;  // within 16 ulps
    if (q < 0.015625f || near_midpoint) {
        const float t1 = amax_f / 6.0f;
        q = t1 / nw.tsf;
    }
    const uint32_t s = e4m3_code_of(q);
    const uint32_t e = s >> 3, m = s & 7u;
    const int idx = e ? (int)m : 8 + (int)m;
    const float t = __int_as_float(__builtin_amdgcn_ds_bpermute(idx << 2, nw.table));
    inv = ldexpf(t, e ? 10 - (int)e : 9);
    return s;
}

// ---------------------------------------------------------------- one chunk

struct LaneOut {
    uint32_t c0, c1;  // packed codes: FP4 uses c0 (8 nibbles), FP8 c0 and c1
    uint32_t scale;   // the block's scale byte
};

template <int FMT>
__device__ __forceinline__ LaneOut quantize_lane(const uint4& w, const Nvfp4Wave& nw) {
    using T = FormatTraits<FMT>;
    const uint32_t wv[4] = {w.x, w.y, w.z, w.w};
    const uint32_t mag[4] = {magnitudes(w.x), magnitudes(w.y), magnitudes(w.z), magnitudes(w.w)};
    const uint32_t amax = block_amax_bits<T::kLanesPerBlock>(lane_amax_bits(mag));
    const bool special = amax >= 0x7F80u;  // exponent field 255: Inf or NaN
    LaneOut o;
    if constexpr (FMT == 2) {
        float inv;
        const uint32_t s = nvfp4_scale(__uint_as_float(amax << 16), nw, inv);
        float v[8];
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            v[2 * k] = __uint_as_float(wv[k] << 16) * inv;
            v[2 * k + 1] = __uint_as_float(wv[k] & 0xFFFF0000u) * inv;
        }
        uint32_t p = fp4_pair_f32<0>(0u, v[0], v[1]);
        p = fp4_pair_f32<1>(p, v[2], v[3]);
        p = fp4_pair_f32<2>(p, v[4], v[5]);
        p = fp4_pair_f32<3>(p, v[6], v[7]);
        o.c0 = special ? 0u : p;
        o.c1 = 0;
        o.scale = special ? 0x7Fu : s;
    } else {
        // E8M0 byte = X + 127 with X = max(floor(log2 amax) - emax, -127).  For a
        // normal amax floor(log2 amax) is its exponent field e minus 127, so the
        // byte is max(e - emax, 0); a subnormal or zero amax (e = 0) has
        // floor(log2 amax) <= -127 and clamps to byte 0 as well.
        const uint32_t sbyte = (uint32_t)max((int)(amax >> 7) - T::kEmax, 0);
        const float scale = __uint_as_float(sbyte << 23);  // exponent field = E8M0 byte
        if constexpr (FMT == 0) {
            uint32_t p = fp4_pair_bf16<0>(0u, wv[0], scale);
            p = fp4_pair_bf16<1>(p, wv[1], scale);
            p = fp4_pair_bf16<2>(p, wv[2], scale);
            p = fp4_pair_bf16<3>(p, wv[3], scale);
            o.c0 = special ? 0u : p;
            o.c1 = 0;
        } else {
            // clamp |x| to 448 * 2^X: BF16 pattern 1.75 * 2^(X+8), exponent
            // field X + 135 = sbyte + 8, mantissa 0x60
            const uint32_t cap = (sbyte << 7) + 0x460u;
            const u16x2_t cap2 = __builtin_bit_cast(u16x2_t, cap | (cap << 16));
            uint32_t cw[4];
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                const u16x2_t m = __builtin_elementwise_min(__builtin_bit_cast(u16x2_t, mag[k]), cap2);
                cw[k] = __builtin_bit_cast(uint32_t, m) | (wv[k] & 0x80008000u);
            }
            i16x2_t r0 = {0, 0}, r1 = {0, 0};
            r0 = __builtin_amdgcn_cvt_scalef32_pk_fp8_bf16(r0, as_bf16x2(cw[0]), scale, false);
            r0 = __builtin_amdgcn_cvt_scalef32_pk_fp8_bf16(r0, as_bf16x2(cw[1]), scale, true);
            r1 = __builtin_amdgcn_cvt_scalef32_pk_fp8_bf16(r1, as_bf16x2(cw[2]), scale, false);
            r1 = __builtin_amdgcn_cvt_scalef32_pk_fp8_bf16(r1, as_bf16x2(cw[3]), scale, true);
            o.c0 = special ? 0u : __builtin_bit_cast(uint32_t, r0);
            o.c1 = special ? 0u : __builtin_bit_cast(uint32_t, r1);
        }
        o.scale = special ? 0xFFu : sbyte;
    }
    return o;
}

// ---------------------------------------------------------------- kernel

typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2_t __attribute__((ext_vector_type(2)));

// Word 3 of a raw buffer descriptor on gfx9-family chips (32-bit data
// format; no swizzle, stride 0), and the load's nontemporal cache policy.
constexpr int kBufferWord3 = 0x00020000;
constexpr int kBufferNontemporal = 2;
// Cache policy of the quantizers' code and scale stores (the aux operand of
// the buffer store: bit 1 nt, bit 4 sc1).  Measured in alternation on one box:
//  * FP4 codes (4 bytes per lane per store) of large problems go out with
//    device scope (sc1), which writes through the XCD's L2: grouped MXFP4 on
//    the 16384 x 7168 prefill routing took 45.4 us against 48.5 with nt,
//    dense NVFP4 16384 x 7168 48.1 against 49.0, grouped NVFP4 49.3 against
//    49.8;
//  * FP8 codes (8 bytes per lane) go out non-temporal: grouped MXFP8 on the
//    same routing took 62.0 us with sc1 against 56.6 with nt;
//  * small problems (one chunk per wave) go out non-temporal: the MXFP4
//    decode gather (512 routed rows x 2048) took 3.96 us with sc1 against
//    3.09 with nt, where the write-through's latency is on the critical path.
constexpr int kStoreStream = 2;         // nt
constexpr int kStoreWriteThrough = 16;  // sc1

// The owning group of routed row r and its metadata.  The last g with
// row_offsets[g] <= r owns r (empty groups repeat an offset and never win),
// so g + 1 is the number of offsets <= r.
struct GroupInfo {
    int g;             // -1: r is before the first or at/after the last group
    uint32_t ro, so;   // row_offsets[g], scales_offsets[g]
    int32_t id;        // expert_ids[g] (NVFP4 only)
    float sf;          // expert_sf[id] (NVFP4 only, when id is in range)
};

// How many of row_offsets[0..G] are <= r (wave-uniform), on the scalar unit:
// an upper-bound search that halves the range twice per round trip -- the
// probe of the second halving is loaded for both outcomes of the first, so
// the three loads of a round are independent.  For nondecreasing offsets
// this is one more than the last group starting at or before r.  Every probe
// index lies in [0, G], whatever the offsets hold.  (The tensor-scale
// reduction places its cursor with it once per wave.)
__device__ __forceinline__ int offsets_at_or_below(const KernelArgs& a, uint32_t r) {
    const uint32_t* __restrict__ ro = a.row_offsets;
    uint32_t base = 0, n = (uint32_t)a.num_groups + 1;
    const uint32_t first = ro[0];
    while (n > 1) {
        const uint32_t h1 = n >> 1, n1 = n - h1, h2 = n1 >> 1;
        const uint32_t v_mid = ro[base + h1], v_lo = ro[base + h2], v_hi = ro[base + h1 + h2];
        const bool up = v_mid <= r;
        const uint32_t b1 = up ? base + h1 : base;
        base = ((up ? v_hi : v_lo) <= r) ? b1 + h2 : b1;
        n = n1 - h2;
    }
    return (int)(base + ((base > 0 || first <= r) ? 1u : 0u));
}

// Lane-parallel group lookup, the quantizers' search: the wave loads
// row_offsets 256 entries at a time, four per lane (one 16-byte buffer load,
// issued ahead of the data loads so it lands first); entries past G read as
// zeros and are masked by index.  Offsets are nondecreasing, so the entries
// <= r form a prefix, whose length is the number of set bits of four ballots.
// Then scalar loads of the group's entries, under the data loads.  Against a
// binary search on the scalar unit (about 100 scalar instructions and 8
// dependent round trips per wave) this took grouped NVFP4 on the 16384 x 7168
// prefill routing from 47.2-47.9 us to 45.4-45.9 and grouped MXFP4 from
// 44.8-45.0 to 44.2-44.5 (grouped MXFP8 56.3 -> 56.4-56.6), timed in
// alternation on one box.
// With REGS the same 256 entries of scales_offsets (and, for NVFP4,
// expert_ids) are loaded beside them, so a group among the first 256 takes its
// entries from these registers (v_readlane) instead of scalar loads issued
// after the search.  Measured on the 16384 x 7168 prefill routing it saves
// 0.2-0.7 us per format (NVFP4 45.4-45.8 -> 45.0-45.1 in two alternated
// runs); on the decode gathers (one chunk per wave, latency-bound) the extra
// load cost 0.07 us per launch where the scalar loads overlap the arithmetic,
// so one-chunk tiles keep them.
template <bool NVFP4>
struct OffsetsLoad {
    __amdgpu_buffer_rsrc_t rsrc;
    u32x4_t v, so, ids;
};
template <bool NVFP4, bool REGS>
__device__ __forceinline__ OffsetsLoad<NVFP4> issue_offsets(const KernelArgs& a, int lane) {
    OffsetsLoad<NVFP4> o;
    const int G = a.num_groups;
    o.rsrc = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint32_t*>(a.row_offsets), (short)0,
                                               (G + 1) * 4, kBufferWord3);
    o.v = __builtin_amdgcn_raw_buffer_load_b128(o.rsrc, lane * 16, 0, 0);
    o.so = o.ids = (u32x4_t){0u, 0u, 0u, 0u};
    if constexpr (REGS)
        o.so = __builtin_amdgcn_raw_buffer_load_b128(
            __builtin_amdgcn_make_buffer_rsrc(const_cast<uint32_t*>(a.scales_offsets), (short)0,
                                              (G + 1) * 4, kBufferWord3), lane * 16, 0, 0);
    if constexpr (REGS && NVFP4)
        o.ids = __builtin_amdgcn_raw_buffer_load_b128(
            __builtin_amdgcn_make_buffer_rsrc(const_cast<int32_t*>(a.expert_ids), (short)0,
                                              G * 4, kBufferWord3), lane * 16, 0, 0);
    return o;
}
// Entry g (< 256) of the four-per-lane registers w: lane g / 4, component g % 4.
__device__ __forceinline__ uint32_t entry_of(const u32x4_t& w, int g) {
    const int c = g & 3;
    const uint32_t x = c == 0 ? w.x : c == 1 ? w.y : c == 2 ? w.z : w.w;
    return (uint32_t)__builtin_amdgcn_readlane((int)x, g >> 2);
}
// Offsets <= r among entries [base, base + 256) held four per lane in v.
__device__ __forceinline__ uint32_t count_round(const u32x4_t& v, int base, int G1, uint32_t r,
                                                int lane) {
    const int i0 = base + 4 * lane;
    return (uint32_t)__builtin_popcountll(__builtin_amdgcn_ballot_w64(i0 < G1 && v.x <= r)) +
           (uint32_t)__builtin_popcountll(__builtin_amdgcn_ballot_w64(i0 + 1 < G1 && v.y <= r)) +
           (uint32_t)__builtin_popcountll(__builtin_amdgcn_ballot_w64(i0 + 2 < G1 && v.z <= r)) +
           (uint32_t)__builtin_popcountll(__builtin_amdgcn_ballot_w64(i0 + 3 < G1 && v.w <= r));
}

// Number of offsets <= r.  A second and later round (more than 255 groups, r
// at or past entry 256) loads and counts the next 256 entries.  PEEL takes the
// first round out of the loop, so the wait before it covers the offsets load
// alone, not the data loads issued after it: grouped NVFP4 45.99 -> 45.47 us;
// for the MX formats, whose stores wait for every data load anyway, the loop
// form measured faster (MXFP4 44.39 against 44.73, MXFP8 56.41 against 56.63;
// best of four alternated runs each, one box).
template <bool PEEL>
__device__ __forceinline__ int count_at_or_below(const KernelArgs& a,
                                                 const OffsetsLoad<PEEL>& o, uint32_t r,
                                                 int lane) {
    const int G1 = a.num_groups + 1;
    if constexpr (PEEL) {
        uint32_t c = count_round(o.v, 0, G1, r, lane);
        int cnt = (int)c;
        for (int base = 256; c == 256u && base < G1; base += 256) {
            const u32x4_t v =
                __builtin_amdgcn_raw_buffer_load_b128(o.rsrc, base * 4 + lane * 16, 0, 0);
            c = count_round(v, base, G1, r, lane);
            cnt += (int)c;
        }
        return cnt;
    } else {
        u32x4_t v = o.v;
        int cnt = 0;
        for (int base = 0;; base += 256) {
            const uint32_t c = count_round(v, base, G1, r, lane);
            cnt += (int)c;
            if (c < 256u || base + 256 >= G1) break;
            v = __builtin_amdgcn_raw_buffer_load_b128(o.rsrc, (base + 256) * 4 + lane * 16, 0, 0);
        }
        return cnt;
    }
}

// NVFP4 needs the expert's tensor scale and takes the peeled count.
template <bool NVFP4, bool REGS>
__device__ __forceinline__ GroupInfo find_group_vec(const KernelArgs& a,
                                                    const OffsetsLoad<NVFP4>& o, uint32_t r,
                                                    int lane) {
    const int G = a.num_groups;
    const int cnt = __builtin_amdgcn_readfirstlane(count_at_or_below<NVFP4>(a, o, r, lane));
    GroupInfo gi{-1, 0u, 0u, 0, 1.0f};
    if (cnt == 0 || cnt > G) return gi;
    gi.g = cnt - 1;
    if (REGS && gi.g < 256) {            // in the registers loaded with the first round
        gi.ro = entry_of(o.v, gi.g);
        gi.so = entry_of(o.so, gi.g);
        if constexpr (NVFP4) gi.id = (int32_t)entry_of(o.ids, gi.g);
    } else {
        gi.ro = a.row_offsets[gi.g];
        gi.so = a.scales_offsets[gi.g];
        if constexpr (NVFP4) gi.id = a.expert_ids[gi.g];
    }
    if constexpr (NVFP4)
        if (gi.id >= 0 && gi.id < a.num_experts) gi.sf = a.expert_sf[gi.id];
    return gi;
}
// t / tiles_per_row by multiply-high with the host's magic constant
// M = ceil(2^64 / d): for t < 2^32, floor(t * M / 2^64) = floor(t / d)
// because t * (M - 2^64 / d) / 2^64 < 2^-32 <= 1/d.  d = 1 is sent as M = 0.
__device__ __forceinline__ uint32_t div_tiles(uint32_t t, const KernelArgs& a) {
    if ((a.tpr_magic_lo | a.tpr_magic_hi) == 0) return t;
    const uint64_t lo = (uint64_t)t * a.tpr_magic_lo;
    const uint64_t hi = (uint64_t)t * a.tpr_magic_hi + (lo >> 32);
    return (uint32_t)(hi >> 32);
}

// One tile of N chunks (N <= U; fewer only for the last tile of a row).  Its
// N 16-byte loads are issued back to back with no per-lane condition (lanes
// past the row's end load the row's last 8 elements instead), so the wave
// converts chunk u as soon as its own load has landed while the later ones
// are still in flight.  Code stores go through a descriptor over the row's
// codes, which drops lanes past K.
template <int FMT, bool GROUPED, int N, int POLICY, bool REGS>
__device__ __forceinline__ void quantize_tile(const KernelArgs& a, uint32_t row, int c0,
                                              int lane) {
    using T = FormatTraits<FMT>;
    int64_t src = row;
    if constexpr (GROUPED) {
        if (a.row_indices) {
            src = a.row_indices[row];
            if (src < 0 || src >= a.num_src_rows) return;
        }
    }
    const uint16_t* xrow = a.x + src * a.ldx;
    OffsetsLoad<FMT == 2> offs{};
    if constexpr (GROUPED) offs = issue_offsets<FMT == 2, REGS>(a, lane);
    u32x4_t w[N];
#pragma unroll
    for (int u = 0; u < N; ++u) {
        const int col = min((c0 + u) * kChunkElems + lane * kElemsPerLane, a.K - kElemsPerLane);
        w[u] = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(xrow + col));
    }

    int64_t scale_row = row;
    float tsf = a.tensor_sf;
    if constexpr (GROUPED) {
        const GroupInfo gi = find_group_vec<FMT == 2, REGS>(a, offs, row, lane);
        if (gi.g < 0) return;
        scale_row = (int64_t)gi.so + ((int64_t)row - (int64_t)gi.ro);
        if (scale_row < 0 || scale_row >= a.num_scale_rows) return;
        if constexpr (FMT == 2) {
            if (gi.id < 0 || gi.id >= a.num_experts) return;
            tsf = gi.sf;
        }
    }
    uint8_t* qrow = a.codes + (int64_t)row * a.ldq;
    // row-major: the scale row; MFMA layout (MX only): the row's place in its
    // 16-row group, to which each block adds its record and lane offset
    const bool mfma_layout = FMT != 2 && a.scale_layout == 1;
    uint8_t* srow = mfma_layout ? a.scales + (scale_row >> 4) * a.lds + 4 * (scale_row & 15)
                                : a.scales + scale_row * a.lds;
    Nvfp4Wave nw{};
    if constexpr (FMT == 2) nw = nvfp4_wave_setup(tsf, lane);

    // store descriptors over this row's codes and its scale bytes (the
    // offsets below stay inside them; a store outside would be dropped)
    const int code_bytes = T::kFp4 ? a.K / 2 : a.K;
    const int scale_bytes = mfma_layout ? a.chunks_per_row * 256 - 4 * (int)(scale_row & 15)
                                        : a.K / T::kBlock;
    const __amdgpu_buffer_rsrc_t qrsrc =
        __builtin_amdgcn_make_buffer_rsrc(qrow, (short)0, code_bytes, kBufferWord3);
    const __amdgpu_buffer_rsrc_t srsrc =
        __builtin_amdgcn_make_buffer_rsrc(srow, (short)0, scale_bytes, kBufferWord3);

    uint32_t sb[N];  // per chunk: the block's scale byte
#pragma unroll
    for (int u = 0; u < N; ++u) {
        const LaneOut o = quantize_lane<FMT>(make_uint4(w[u].x, w[u].y, w[u].z, w[u].w), nw);
        sb[u] = o.scale;
        const int col = (c0 + u) * kChunkElems + lane * kElemsPerLane;
        if constexpr (T::kFp4) {
            __builtin_amdgcn_raw_buffer_store_b32(o.c0, qrsrc, col / 2, 0, POLICY);
        } else {
            const u32x2_t v = {o.c0, o.c1};
            __builtin_amdgcn_raw_buffer_store_b64(v, qrsrc, col, 0, POLICY);
        }
    }
    // Scale bytes: every lane of a block holds its byte, so one store
    // instruction covers up to kLanesPerBlock chunks -- lane (block * L + j)
    // writes chunk (g + j)'s byte for that block.  Blocks past K are not
    // stored (in the MFMA layout they would land inside a record).
    constexpr int L = T::kLanesPerBlock;
#pragma unroll
    for (int g = 0; g < N; g += L) {
        const int j = lane & (L - 1);
        const int u = g + j;
        uint32_t v = sb[g];
#pragma unroll
        for (int k = 1; k < L && g + k < N; ++k) v = (j == k) ? sb[g + k] : v;
        const int col = (c0 + u) * kChunkElems + (lane - j) * kElemsPerLane;
        // block b = lane / L of chunk c0 + u; in the MFMA layout a chunk is one
        // record and block b goes to lane-dword 16 (b % 4), byte b / 4
        const int b = lane / L;
        const int off = mfma_layout ? (c0 + u) * 256 + 64 * (b & 3) + (b >> 2) : col / T::kBlock;
        if (u < N && col < a.K)
            __builtin_amdgcn_raw_buffer_store_b8((uint8_t)v, srsrc, off, 0, POLICY);
    }
}

// One wave converts one tile: U consecutive chunks (U * 512 elements) of one
// row.  Loads carry the non-temporal hint: the data streams through once, so
// it should not displace anything from the caches.  Stores take the cache
// policy measured best for the code width and problem size (kStoreStream,
// kStoreWriteThrough above).  The last tile of a row may hold fewer chunks; it
// takes the tile body built for its count, so every body is straight-line.
template <int FMT, bool GROUPED, int U>
__global__ void __launch_bounds__(kThreadsPerBlock) quantize_kernel(const KernelArgs a) {
    using T = FormatTraits<FMT>;
    constexpr int kPolicy = (T::kFp4 && U > 1) ? kStoreWriteThrough : kStoreStream;
    constexpr bool kRegs = U > 1;        // group entries from registers (large problems)
    const int lane = (int)(threadIdx.x & (kWaveSize - 1));
    // the tile index is wave-uniform: keep it (and all row arithmetic) scalar
    const uint32_t t = __builtin_amdgcn_readfirstlane(blockIdx.x * kWavesPerBlock +
                                                      (threadIdx.x / kWaveSize));
    if (t >= (uint32_t)a.total_tiles) return;
    const uint32_t row = div_tiles(t, a);
    const int c0 = (int)(t - row * (uint32_t)a.tiles_per_row) * U;
    const int nch = min(U, a.chunks_per_row - c0);  // chunks in this tile (>= 1)
    if (nch == U) {
        quantize_tile<FMT, GROUPED, U, kPolicy, kRegs>(a, row, c0, lane);
    } else if constexpr (U > 1) {
        if (nch == 1) quantize_tile<FMT, GROUPED, 1, kPolicy, kRegs>(a, row, c0, lane);
        if constexpr (U > 2) {
            if (nch == 2) quantize_tile<FMT, GROUPED, 2, kPolicy, kRegs>(a, row, c0, lane);
            if (nch == 3) quantize_tile<FMT, GROUPED, 3, kPolicy, kRegs>(a, row, c0, lane);
        }
    }
}

// ---------------------------------------------------------------- tensor scale
//
// NVFP4 tensor scale, the step before the quantizer: tsf = fl32(amax / 2688)
// over the finite elements, 1.0 when that amax is 0, clamped to [2^-117,
// 2^100].  Three kernels on the caller's stream, using the caller's output
// array (one float per expert; one for the dense form) as the accumulator:
//  1. zero it;
//  2. waves take the max |x| over the finite elements of their rows, and
//     workgroups fold it in with atomic maxima on the fp32 bit pattern
//     (non-negative floats order like their patterns);
//  3. turn each amax into its tensor scale in place.

__global__ void __launch_bounds__(kThreadsPerBlock) tsf_zero_kernel(uint32_t* acc, int n) {
    const int i = (int)(blockIdx.x * blockDim.x + threadIdx.x);
    if (i < n) acc[i] = 0u;
}

__global__ void __launch_bounds__(kThreadsPerBlock) tsf_finish_kernel(uint32_t* acc, int n) {
    const int i = (int)(blockIdx.x * blockDim.x + threadIdx.x);
    if (i >= n) return;
    const float amax = __uint_as_float(acc[i]);
    float t = 1.0f;
    if (amax != 0.0f) {
        t = amax / 2688.0f;  // 2688 = 6 * 448
        t = fminf(fmaxf(t, 0x1p-117f), 0x1p100f);
    }
    acc[i] = __float_as_uint(t);
}

// max over the finite |x| of 8 BF16 elements, as a 15-bit pattern (0 if none):
// adding 0x80 to every magnitude sends finite values to [0x80, 0x7FFF] and
// Inf/NaN to [0x8000, 0x807F], which a signed 16-bit max never picks over a
// finite one.
__device__ __forceinline__ uint32_t lane_finite_amax_bits(const uint4& w) {
    typedef short i16x2 __attribute__((ext_vector_type(2)));
    const u16x2_t bias = {0x80, 0x80};
    i16x2 m = {0, 0};  // below every biased finite value
    const uint32_t wv[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        const u16x2_t b = __builtin_bit_cast(u16x2_t, magnitudes(wv[k])) + bias;
        m = __builtin_elementwise_max(m, __builtin_bit_cast(i16x2, b));
    }
    const int best = max((int)m.x, (int)m.y);
    return best >= 0x80 ? (uint32_t)(best - 0x80) : 0u;
}

// Max over a wave of a per-lane value: DPP within rows of 16 lanes, then the
// four row results read out.
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t m) {
    m = max(m, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)m, 0xB1, 0xF, 0xF, true));
    m = max(m, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)m, 0x4E, 0xF, 0xF, true));
    m = max(m, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)m, 0x114, 0xF, 0xF, true));  // row_shr:4
    m = max(m, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)m, 0x118, 0xF, 0xF, true));  // row_shr:8
    const uint32_t r0 = (uint32_t)__builtin_amdgcn_readlane((int)m, 15);
    const uint32_t r1 = (uint32_t)__builtin_amdgcn_readlane((int)m, 31);
    const uint32_t r2 = (uint32_t)__builtin_amdgcn_readlane((int)m, 47);
    const uint32_t r3 = (uint32_t)__builtin_amdgcn_readlane((int)m, 63);
    return max(max(r0, r1), max(r2, r3));
}

// Fold amax pattern v into acc[slot] with a device-scope atomic max.  With
// `check`, a relaxed read first skips the atomic when acc already holds as
// much (worth it where many blocks share one address, the dense form).
__device__ __forceinline__ void global_fold(uint32_t* acc, int slot, uint32_t v, bool check) {
    uint32_t* p = acc + slot;
    if (check && __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) >= v) return;
    __hip_atomic_fetch_max(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

__device__ __forceinline__ int expert_slot(const KernelArgs& a, int g) {
    const int id = a.expert_ids[g];
    return (id >= 0 && id < a.num_experts) ? id : -1;
}

// Step 2.  Each wave walks a contiguous range of tiles_per_wave tiles (of
// kTsfChunks chunks) in row order, keeping a per-lane running max; the
// workgroup's waves take consecutive ranges.  In the grouped form a wave
// carries a cursor over the groups -- found once by counting offsets, then
// advanced as rows go by -- and flushes its max when the expert changes and
// at the end.  With at most kTsfLdsSlots outputs a flush is an LDS atomic max
// into a per-workgroup table; after a barrier the workgroup folds each
// non-zero entry into the output with one device atomic (the grouped form
// finds its entries by scanning the groups its waves flushed from: the
// experts of one workgroup's contiguous rows).  Device atomics on one address
// are slow when thousands of waves issue them, so this keeps them to about
// one per workgroup and expert.  With more outputs a flush is a device atomic.
template <bool GROUPED>
__global__ void __launch_bounds__(kTsfMaxThreads)
tsf_amax_kernel(const KernelArgs a, uint32_t* acc, uint32_t tiles_per_wave, int n_out) {
    constexpr int U = kTsfChunks;
    extern __shared__ uint32_t s_tab[];  // [n_out] amax table (LDS mode), then the group span
    const bool lds = n_out <= kTsfLdsSlots;
    int* s_span = reinterpret_cast<int*>(s_tab + (lds ? n_out : 0));
    if (lds)
        for (int i = (int)threadIdx.x; i < n_out; i += (int)blockDim.x) s_tab[i] = 0u;
    if (threadIdx.x == 0) {
        s_span[0] = 0x7FFFFFFF;
        s_span[1] = -1;
    }
    __syncthreads();

    const int lane = (int)(threadIdx.x & (kWaveSize - 1));
    const uint32_t w = __builtin_amdgcn_readfirstlane(blockIdx.x * (blockDim.x / kWaveSize) +
                                                      (threadIdx.x / kWaveSize));
    // a flush of per-lane maxima m under (slot, from group g)
    auto flush = [&](int slot, int g, uint32_t m) {
        const uint32_t best = wave_max_u32(m) << 16;  // fp32 pattern of the amax
        if (lane != 0 || best == 0u || slot < 0) return;
        if (lds) {
            __hip_atomic_fetch_max(s_tab + slot, best, __ATOMIC_RELAXED,
                                   __HIP_MEMORY_SCOPE_WORKGROUP);
            if constexpr (GROUPED) {
                __hip_atomic_fetch_min(s_span, g, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
                __hip_atomic_fetch_max(s_span + 1, g, __ATOMIC_RELAXED,
                                       __HIP_MEMORY_SCOPE_WORKGROUP);
            }
        } else {
            global_fold(acc, slot, best, false);
        }
    };

    const uint64_t first = (uint64_t)w * tiles_per_wave;
    bool active = first < (uint64_t)a.total_tiles;
    uint32_t left = active ? (uint32_t)min((uint64_t)tiles_per_wave,
                                           (uint64_t)a.total_tiles - first) : 0u;
    uint32_t row = active ? div_tiles((uint32_t)first, a) : 0u;
    int c0 = (int)((uint32_t)first - row * (uint32_t)a.tiles_per_row) * U;

    // grouped: g = the last group with row_offsets[g] <= row (-1: none),
    // hi = row_offsets[g + 1]; slot = its expert (-1: out of range); the
    // running max belongs to acc_slot, first seen at group acc_g
    int g = -1, slot = 0, acc_slot = 0, acc_g = 0;
    uint32_t hi = 0;
    if constexpr (GROUPED) {
        if (active) {
            const int cnt = offsets_at_or_below(a, row);
            active = cnt <= a.num_groups;  // else at or past the end of the last group
            g = cnt - 1;
            if (active) {
                hi = a.row_offsets[g + 1];
                slot = g >= 0 ? expert_slot(a, g) : -1;
            }
            acc_slot = slot;
            acc_g = g;
        }
    }
    const bool started = active;
    // The range's tiles in order.  On entering a row the cursor advances and
    // the row's source and expert are resolved; a tile is read only when
    // `use` (owned row, source in range, expert in range).  Past the range,
    // or past the last group, `done`.
    struct Tile {
        const uint16_t* xrow;
        int cb, slot, g;
        bool use, done;
    };
    const uint16_t* row_ptr = a.x;
    bool row_use = false;
    uint32_t row_ready = 0xFFFFFFFFu;
    auto next = [&]() -> Tile {
        Tile t{a.x, 0, -1, -1, false, true};
        if (!active || left == 0) return t;
        if (row != row_ready) {
            row_ready = row;
            int64_t src = row;
            row_use = true;
            if constexpr (GROUPED) {
                bool moved = false;
                while (row >= hi && g + 1 < a.num_groups) {
                    ++g;
                    hi = a.row_offsets[g + 1];
                    moved = true;
                }
                if (row >= hi) {  // rows only grow: nothing later is owned either
                    active = false;
                    return t;
                }
                if (moved) slot = expert_slot(a, g);
                row_use = g >= 0 && slot >= 0;
                if (row_use && a.row_indices) {
                    src = a.row_indices[row];
                    row_use = src >= 0 && src < a.num_src_rows;
                }
            }
            row_ptr = row_use ? a.x + src * a.ldx : a.x;
        }
        t = Tile{row_ptr, c0, slot, g, row_use, false};
        --left;
        c0 += U;
        if (c0 >= a.chunks_per_row) {
            c0 = 0;
            ++row;
        }
        return t;
    };
    // Eight 16-byte buffer loads per lane through a descriptor that spans
    // the row from the tile's first element (none for a tile not read):
    // lanes past the row's end read zeros, which never raise the max, with
    // no branch and no per-load address registers, so the wait for one
    // tile's data leaves the next tile's loads in flight.
    auto issue = [&](const Tile& t, u32x4_t (&v)[U]) {
        const int bytes = t.use ? (a.K - t.cb * kChunkElems) * 2 : 0;
        const __amdgpu_buffer_rsrc_t r = __builtin_amdgcn_make_buffer_rsrc(
            const_cast<uint16_t*>(t.xrow + t.cb * kChunkElems), (short)0, bytes, kBufferWord3);
#pragma unroll
        for (int u = 0; u < U; ++u)
            v[u] = __builtin_amdgcn_raw_buffer_load_b128(r, lane * 16 + u * kChunkElems * 2, 0,
                                                         kBufferNontemporal);
    };
    uint32_t m = 0;
    auto reduce = [&](const Tile& t, const u32x4_t (&v)[U]) {
        if (!t.use) return;
        if constexpr (GROUPED) {
            if (t.slot != acc_slot) {
                flush(acc_slot, acc_g, m);
                m = 0;
                acc_slot = t.slot;
                acc_g = t.g;
            }
        }
#pragma unroll
        for (int u = 0; u < U; ++u)
            m = max(m, lane_finite_amax_bits(make_uint4(v[u].x, v[u].y, v[u].z, v[u].w)));
    };
    // ping-pong over two register sets: load one tile ahead
    u32x4_t va[U], vb[U];
    Tile ta = next();
    if (!ta.done) {
        issue(ta, va);
        for (;;) {
            const Tile tb = next();
            if (tb.done) {
                reduce(ta, va);
                break;
            }
            issue(tb, vb);
            reduce(ta, va);
            ta = next();
            if (ta.done) {
                reduce(tb, vb);
                break;
            }
            issue(ta, va);
            reduce(tb, vb);
        }
    }
    if (started) flush(acc_slot, acc_g, m);
    if (!lds) return;  // no barrier follows in this mode

    __syncthreads();
    if constexpr (!GROUPED) {
        if (threadIdx.x == 0 && s_tab[0] != 0u) global_fold(acc, 0, s_tab[0], true);
    } else {
        // every table entry that is non-zero was flushed from a group in
        // [span0, span1]; each expert is taken (and cleared) once
        // (no flush leaves the span empty: span0 = INT_MAX > span1 = -1)
        const int64_t g0 = max(s_span[0], 0), g1 = min(s_span[1], a.num_groups - 1);
        for (int64_t gg = g0 + threadIdx.x; gg <= g1; gg += blockDim.x) {
            const int sl = expert_slot(a, (int)gg);
            if (sl < 0) continue;
            const uint32_t v = __hip_atomic_exchange(s_tab + sl, 0u, __ATOMIC_RELAXED,
                                                     __HIP_MEMORY_SCOPE_WORKGROUP);
            if (v != 0u) global_fold(acc, sl, v, false);
        }
    }
}

template <int FMT, bool GROUPED, int U>
hipError_t launch(const KernelArgs& a, int64_t blocks, hipStream_t stream, const LaunchEvents& ev) {
    return launch_kernel(quantize_kernel<FMT, GROUPED, U>, dim3((uint32_t)blocks),
                         dim3(kThreadsPerBlock), 0, stream, ev, a);
}

// The tile sizes the host picks: 1 chunk for small problems; for large ones
// 2 (dense MXFP8) or 4 (the FP4 formats, and every grouped form).  Only
// those are built.
template <int FMT, bool GROUPED>
hipError_t launch_u(const KernelArgs& a, int64_t blocks, hipStream_t stream,
                    const LaunchEvents& ev) {
    constexpr int kLarge = (FMT == 1 && !GROUPED) ? 2 : 4;
    switch (a.chunks_per_tile) {
        case 1: return launch<FMT, GROUPED, 1>(a, blocks, stream, ev);
        case kLarge: return launch<FMT, GROUPED, kLarge>(a, blocks, stream, ev);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace

hipError_t launch_tensor_scale(bool grouped, const KernelArgs& a, int64_t blocks,
                               int waves_per_block, uint32_t tiles_per_wave, float* out, int n_out,
                               hipStream_t stream, const LaunchEvents& ev) {
    uint32_t* acc = reinterpret_cast<uint32_t*>(out);
    const uint32_t small_blocks = (uint32_t)((n_out + kThreadsPerBlock - 1) / kThreadsPerBlock);
    hipError_t e = launch_kernel(tsf_zero_kernel, dim3(small_blocks), dim3(kThreadsPerBlock), 0,
                                 stream, LaunchEvents{}, acc, n_out);
    if (e != hipSuccess) return e;
    if (blocks > 0) {
        const uint32_t lds_bytes = ((n_out <= kTsfLdsSlots) ? (uint32_t)n_out : 0u) * 4u + 8u;
        const dim3 block((uint32_t)(waves_per_block * kWaveSize));
        e = grouped ? launch_kernel(tsf_amax_kernel<true>, dim3((uint32_t)blocks), block,
                                    lds_bytes, stream, ev, a, acc, tiles_per_wave, n_out)
                    : launch_kernel(tsf_amax_kernel<false>, dim3((uint32_t)blocks), block,
                                    lds_bytes, stream, ev, a, acc, tiles_per_wave, n_out);
        if (e != hipSuccess) return e;
    }
    return launch_kernel(tsf_finish_kernel, dim3(small_blocks), dim3(kThreadsPerBlock), 0, stream,
                         LaunchEvents{}, acc, n_out);
}

hipError_t launch_quantize(int fmt, bool grouped, const KernelArgs& a, int64_t blocks,
                           hipStream_t stream, const LaunchEvents& ev) {
    switch (fmt * 2 + (grouped ? 1 : 0)) {
        case 0: return launch_u<0, false>(a, blocks, stream, ev);
        case 1: return launch_u<0, true>(a, blocks, stream, ev);
        case 2: return launch_u<1, false>(a, blocks, stream, ev);
        case 3: return launch_u<1, true>(a, blocks, stream, ev);
        case 4: return launch_u<2, false>(a, blocks, stream, ev);
        case 5: return launch_u<2, true>(a, blocks, stream, ev);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace bsq
