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
//  * the loads of the next batch of chunks are issued before the current
//    batch is converted, so each lane keeps several 16-byte loads in flight;
//  * a block spans 4 lanes (MX, 32 elements) or 2 lanes (NVFP4, 16); its
//    amax is an integer max over |BF16| bit patterns, reduced across those
//    lanes with DPP quad permutes (no LDS, no barrier);
//  * codes are stored as one dword (FP4) or two dwords (FP8) per lane, so
//    code stores are contiguous per wave; the first lane of each block
//    stores its scale byte;
//  * grouped form: each wave finds its group with a wave-wide ballot over
//    row_offsets (last g with row_offsets[g] <= r), after its first loads
//    are already in flight.
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

constexpr int kBatch = 4;  // chunks loaded per batch (16-byte loads in flight per lane)

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

// ---------------------------------------------------------------- element codes

// E2M1 magnitude code (0..7 for 0, .5, 1, 1.5, 2, 3, 4, 6) of a >= 0 (may be
// +Inf): round to nearest even, saturating at 6.
//  - a >= 1: E2M1 keeps one mantissa bit, so round the fp32 pattern at bit
//    22 (adding 2^21 - 1 plus the kept LSB gives ties-to-even) and rebias the
//    exponent (fp32 1.0 -> code 2).
//  - a < 1: the E2M1 grid there is the multiples of 0.5; adding 2^22 (whose
//    fp32 ulp is 0.5) rounds the exact sum once, to nearest even, so the
//    pattern difference counts halves: code 0, 1 or 2.
__device__ __forceinline__ uint32_t e2m1_magnitude_code(float a) {
    a = fminf(a, 6.0f);
    const uint32_t u = __float_as_uint(a);
    const uint32_t normal = ((u + 0x1FFFFFu + ((u >> 22) & 1u)) >> 22) - 0xFCu;
    const uint32_t sub = __float_as_uint(a + 4194304.0f) - 0x4A800000u;
    return a < 1.0f ? sub : normal;
}

// E4M3 (FN) magnitude code (0..0x7E) of a >= 0 (may be +Inf): round to
// nearest even, saturating at 448 = 0x7E.
//  - a >= 2^-6: three mantissa bits, round at bit 20 and rebias
//    (fp32 exponent 127 -> E4M3 exponent 7: subtract 120 << 3).
//  - a < 2^-6: the subnormal grid is the multiples of 2^-9; adding 2^14
//    (fp32 ulp 2^-9) rounds once; the pattern difference is the code 0..8.
__device__ __forceinline__ uint32_t e4m3_magnitude_code(float a) {
    a = fminf(a, 448.0f);
    const uint32_t u = __float_as_uint(a);
    const uint32_t normal = ((u + 0x7FFFFu + ((u >> 20) & 1u)) >> 20) - 0x3C0u;
    const uint32_t sub = __float_as_uint(a + 16384.0f) - 0x46800000u;
    return a < 0.015625f ? sub : normal;
}

// fp32 value of a positive E4M3 magnitude code (exact).
__device__ __forceinline__ float e4m3_decode(uint32_t s) {
    const uint32_t e = s >> 3, m = s & 7u;
    return e ? __uint_as_float(((e + 120u) << 23) | (m << 20)) : (float)m * 0.001953125f;
}

// ---------------------------------------------------------------- block amax

// max |x| over the lane's 8 BF16 elements, as a 15-bit magnitude pattern.
// Integer order of |BF16| patterns is value order, with Inf above every
// finite value and NaN above Inf.
__device__ __forceinline__ uint32_t lane_amax_bits(const uint4& w) {
    typedef unsigned short u16x2 __attribute__((ext_vector_type(2)));
    const uint32_t k = 0x7FFF7FFFu;
    u16x2 a = __builtin_bit_cast(u16x2, w.x & k);
    u16x2 b = __builtin_bit_cast(u16x2, w.y & k);
    u16x2 c = __builtin_bit_cast(u16x2, w.z & k);
    u16x2 d = __builtin_bit_cast(u16x2, w.w & k);
    u16x2 m = __builtin_elementwise_max(__builtin_elementwise_max(a, b),
                                        __builtin_elementwise_max(c, d));
    return (uint32_t)(m.x > m.y ? m.x : m.y);
}

// Reduce across the lanes of one block (2 or 4 adjacent lanes) with DPP quad
// permutes: xor-1 swaps neighbours, xor-2 swaps pairs.
template <int LANES>
__device__ __forceinline__ uint32_t block_amax_bits(uint32_t m) {
    int v = (int)m;
    int o = __builtin_amdgcn_update_dpp(v, v, 0xB1, 0xF, 0xF, false);  // quad_perm [1,0,3,2]
    v = max(v, o);
    if constexpr (LANES == 4) {
        o = __builtin_amdgcn_update_dpp(v, v, 0x4E, 0xF, 0xF, false);  // quad_perm [2,3,0,1]
        v = max(v, o);
    }
    return (uint32_t)v;
}

// ---------------------------------------------------------------- one chunk

struct LaneOut {
    uint32_t c0, c1;  // packed codes: FP4 uses c0 (8 nibbles), FP8 c0 and c1
    uint32_t scale;   // the block's scale byte
};

__device__ __forceinline__ uint32_t bf16_at(const uint4& w, int i) {
    const uint32_t d = (i < 2) ? w.x : (i < 4) ? w.y : (i < 6) ? w.z : w.w;
    return (i & 1) ? (d >> 16) : (d & 0xFFFFu);
}

template <int FMT>
__device__ __forceinline__ LaneOut quantize_lane(const uint4& w, float tsf) {
    using T = FormatTraits<FMT>;
    const uint32_t amax = block_amax_bits<T::kLanesPerBlock>(lane_amax_bits(w));
    const bool special = amax >= 0x7F80u;  // exponent field 255: Inf or NaN
    LaneOut o;
    uint32_t codes[8];
    if constexpr (FMT == 2) {
        const float amax_f = __uint_as_float(amax << 16);
        const float t1 = amax_f / 6.0f;
        const float t2 = t1 / tsf;
        const uint32_t s = e4m3_magnitude_code(t2);
        const float d = e4m3_decode(s) * tsf;
        const float inv = (d == 0.0f) ? 0.0f : 1.0f / d;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const uint32_t h = bf16_at(w, i);
            const float v = __uint_as_float(h << 16) * inv;
            codes[i] = e2m1_magnitude_code(fabsf(v)) | ((h >> 15) << 3);
        }
        o.scale = special ? 0x7Fu : s;
    } else {
        // floor(log2 amax): exponent field minus bias, or for a subnormal
        // (field 0) the position of the top mantissa bit minus 133.  amax = 0
        // gives -134, which the clamp below turns into X = -127.
        const int e = (int)(amax >> 7);
        const int E = e ? e - 127 : (31 - __clz((int)(amax & 0x7Fu))) - 133;
        const int X = max(E - T::kEmax, -127);
        const float sf = __uint_as_float((uint32_t)(127 - X) << 23);  // 2^-X, X in [-127, 126]
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const uint32_t h = bf16_at(w, i);
            const float v = __uint_as_float(h << 16) * sf;
            if constexpr (FMT == 0)
                codes[i] = e2m1_magnitude_code(fabsf(v)) | ((h >> 15) << 3);
            else
                codes[i] = e4m3_magnitude_code(fabsf(v)) | ((h >> 15) << 7);
        }
        o.scale = special ? 0xFFu : (uint32_t)(X + 127);
    }
    if constexpr (FormatTraits<FMT>::kFp4) {
        uint32_t p = 0;
#pragma unroll
        for (int i = 0; i < 8; ++i) p |= codes[i] << (4 * i);
        o.c0 = special ? 0u : p;
        o.c1 = 0;
    } else {
        uint32_t p0 = 0, p1 = 0;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            p0 |= codes[i] << (8 * i);
            p1 |= codes[i + 4] << (8 * i);
        }
        o.c0 = special ? 0u : p0;
        o.c1 = special ? 0u : p1;
    }
    return o;
}

// ---------------------------------------------------------------- kernel

__device__ __forceinline__ void load_batch(uint4 (&w)[kBatch], const uint16_t* xrow, int c,
                                           int c_end, int lane, int K) {
#pragma unroll
    for (int u = 0; u < kBatch; ++u) {
        const int col = (c + u) * kChunkElems + lane * kElemsPerLane;
        w[u] = make_uint4(0u, 0u, 0u, 0u);
        if (c + u < c_end && col < K) w[u] = *reinterpret_cast<const uint4*>(xrow + col);
    }
}

template <int FMT>
__device__ __forceinline__ void convert_batch(const uint4 (&w)[kBatch], uint8_t* qrow,
                                              uint8_t* srow, int c, int c_end, int lane, int K,
                                              float tsf) {
    using T = FormatTraits<FMT>;
#pragma unroll
    for (int u = 0; u < kBatch; ++u) {
        if (c + u >= c_end) break;  // wave-uniform
        const LaneOut o = quantize_lane<FMT>(w[u], tsf);
        const int col = (c + u) * kChunkElems + lane * kElemsPerLane;
        if (col < K) {
            if constexpr (T::kFp4) {
                *reinterpret_cast<uint32_t*>(qrow + col / 2) = o.c0;
            } else {
                *reinterpret_cast<uint2*>(qrow + col) = make_uint2(o.c0, o.c1);
            }
            if ((lane & (T::kLanesPerBlock - 1)) == 0) srow[col / T::kBlock] = (uint8_t)o.scale;
        }
    }
}

template <int FMT, bool GROUPED>
__global__ void __launch_bounds__(kThreadsPerBlock) quantize_kernel(const KernelArgs a) {
    const int lane = (int)(threadIdx.x & (kWaveSize - 1));
    const int64_t wave = (int64_t)blockIdx.x * kWavesPerBlock + (threadIdx.x / kWaveSize);
    const int64_t row = wave / a.tiles_per_row;
    if (row >= a.rows) return;
    const int tile = (int)(wave - row * a.tiles_per_row);
    const int c_begin = tile * a.chunks_per_tile;
    const int c_end = min(c_begin + a.chunks_per_tile, a.chunks_per_row);

    int64_t src = row;
    if constexpr (GROUPED) {
        if (a.row_indices) {
            src = a.row_indices[row];
            if (src < 0 || src >= a.num_src_rows) return;
        }
    }
    const uint16_t* xrow = a.x + src * a.ldx;

    uint4 cur[kBatch];
    load_batch(cur, xrow, c_begin, c_end, lane, a.K);

    int64_t scale_row = row;
    float tsf = a.tensor_sf;
    if constexpr (GROUPED) {
        // Count the offsets <= r over row_offsets[0..G] with a wave ballot;
        // that count minus one is the owning group (upper bound - 1).
        const uint32_t r = (uint32_t)row;
        int cnt = 0;
        for (int base = 0; base <= a.num_groups; base += kWaveSize) {
            const int i = base + lane;
            const bool le = (i <= a.num_groups) && (a.row_offsets[i] <= r);
            cnt += __popcll(__ballot(le));
        }
        if (cnt == 0 || cnt > a.num_groups) return;  // before the first or past the last group
        const int g = __builtin_amdgcn_readfirstlane(cnt - 1);
        scale_row = (int64_t)a.scales_offsets[g] + ((int64_t)r - (int64_t)a.row_offsets[g]);
        if (scale_row < 0 || scale_row >= a.num_scale_rows) return;
        if constexpr (FMT == 2) {
            const int e = a.expert_ids[g];
            if (e < 0 || e >= a.num_experts) return;
            tsf = a.expert_sf[e];
        }
    }
    uint8_t* qrow = a.codes + row * a.ldq;
    uint8_t* srow = a.scales + scale_row * a.lds;

    for (int c = c_begin; c < c_end; c += kBatch) {
        uint4 nxt[kBatch];
        const bool more = c + kBatch < c_end;
        if (more) load_batch(nxt, xrow, c + kBatch, c_end, lane, a.K);
        convert_batch<FMT>(cur, qrow, srow, c, c_end, lane, a.K, tsf);
        if (more) {
#pragma unroll
            for (int u = 0; u < kBatch; ++u) cur[u] = nxt[u];
        }
    }
}

template <int FMT, bool GROUPED>
hipError_t launch(const KernelArgs& a, int64_t blocks, hipStream_t stream) {
    hipLaunchKernelGGL((quantize_kernel<FMT, GROUPED>), dim3((uint32_t)blocks),
                       dim3(kThreadsPerBlock), 0, stream, a);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_quantize(int fmt, bool grouped, const KernelArgs& a, int64_t blocks,
                           hipStream_t stream) {
    switch (fmt * 2 + (grouped ? 1 : 0)) {
        case 0: return launch<0, false>(a, blocks, stream);
        case 1: return launch<0, true>(a, blocks, stream);
        case 2: return launch<1, false>(a, blocks, stream);
        case 3: return launch<1, true>(a, blocks, stream);
        case 4: return launch<2, false>(a, blocks, stream);
        case 5: return launch<2, true>(a, blocks, stream);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace bsq
