// bsq_consume.hip -- gfx950 kernels that read block-scaled codes back: the
// dequantization to fp32, a naive block-scaled GEMM (no MFMA) as the
// consumer-side check of the quantizers' output, and the dense and grouped
// block-scaled GEMMs on the matrix cores.  The Modular
// "block_scaled_quantization" module page lists a naive block-scaled matmul
// as the reference GEMM over such operands; the decode direction of the
// scales follows the quantizer's readings: an MX value is code * 2^(b - 127),
// an NVFP4 value is code * s * tensor_sf.
//
// Decoding:
//  * element codes go through gfx950's v_cvt_scalef32_pk_f32_{fp4,fp8} at
//    scale 1.0 (two codes per instruction, exact; E4M3 NaN codes give NaN);
//  * MX: the value is that code times the fp32 2^(b - 127) -- exact (every
//    such product is an fp32 value or overflows to infinity); b = 0xFF is NaN;
//  * NVFP4: fl32(fl32(code * s) * tensor_sf), where code * s is exact in fp32
//    (a 2-bit by 4-bit significand product), so the value is the exact
//    product rounded once; s keeps its sign bit; 0x7F / 0xFF are NaN.
// Build flags keep IEEE fp32 semantics (no contraction, no denormal flush).
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "bsq_internal.h"

namespace bsq {
namespace {

// the conversion builtins return a GCC vector of two floats
typedef float f32x2_t __attribute__((vector_size(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef unsigned int c32x2_t __attribute__((ext_vector_type(2)));

// 2^(b - 127) as fp32; b = 0 is the subnormal 2^-127; b = 0xFF is NaN.
__device__ __forceinline__ float e8m0_f32(uint32_t b) {
    if (b == 0xFFu) return __uint_as_float(0x7FC00000u);
    return __uint_as_float(b == 0u ? 0x00400000u : (b << 23));
}

// The E4M3 value of byte b (sign kept; 0x7F / 0xFF NaN).
__device__ __forceinline__ float e4m3_f32(uint32_t b) {
    return __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(b, 1.0f, false)[0];
}

// Codes of byte / word `SEL` of v as two floats (low element first).
template <int SEL>
__device__ __forceinline__ f32x2_t fp4_pair(uint32_t v) {
    return __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(v, 1.0f, SEL);
}
template <bool HI>
__device__ __forceinline__ f32x2_t fp8_pair(uint32_t v) {
    return __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(v, 1.0f, HI);
}

// Eight codes (one lane's share of a chunk) as floats: FP4 in q0, FP8 in q0, q1.
template <int FMT>
__device__ __forceinline__ void decode8(uint32_t q0, uint32_t q1, float (&f)[8]) {
    f32x2_t p[4];
    if constexpr (FMT == 1) {
        p[0] = fp8_pair<false>(q0);
        p[1] = fp8_pair<true>(q0);
        p[2] = fp8_pair<false>(q1);
        p[3] = fp8_pair<true>(q1);
    } else {
        p[0] = fp4_pair<0>(q0);
        p[1] = fp4_pair<1>(q0);
        p[2] = fp4_pair<2>(q0);
        p[3] = fp4_pair<3>(q0);
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        f[2 * j] = p[j][0];
        f[2 * j + 1] = p[j][1];
    }
}

// Scale one decoded code by its block scale byte (and, NVFP4, the tensor scale).
template <int FMT>
__device__ __forceinline__ float apply_scale(float code, float scale, float tsf) {
    if constexpr (FMT == 2) return (code * scale) * tsf;
    return code * scale;
}

template <int FMT>
__device__ __forceinline__ float scale_value(uint32_t b) {
    if constexpr (FMT == 2) return e4m3_f32(b);
    return e8m0_f32(b);
}

__device__ __forceinline__ uint32_t div_rows(uint32_t t, const DequantArgs& a) {
    if ((a.tpr_magic_lo | a.tpr_magic_hi) == 0) return t;
    const uint64_t lo = (uint64_t)t * a.tpr_magic_lo;
    const uint64_t hi = (uint64_t)t * a.tpr_magic_hi + (lo >> 32);
    return (uint32_t)(hi >> 32);
}

// Dequantization: one wave per tile of U chunks of one row (512 elements per
// chunk, lane l holding elements [8l, 8l + 8)).  All of a tile's code and
// scale loads are issued first; each lane then writes its 8 floats with two
// 16-byte stores, so every store instruction covers 1 KiB of the output row.
// The stores are ordinary ones: for this write-heavy stream (4 of every ~4.6
// bytes) non-temporal 16-byte stores measured at under half the bandwidth.
template <int FMT, int U>
__global__ void __launch_bounds__(kThreadsPerBlock) dequant_kernel(const DequantArgs a) {
    constexpr int kBlock = FMT == 2 ? 16 : 32;
    const int lane = (int)(threadIdx.x & (kWaveSize - 1));
    const uint32_t t = __builtin_amdgcn_readfirstlane(blockIdx.x * kWavesPerBlock +
                                                      (threadIdx.x / kWaveSize));
    if (t >= (uint32_t)a.total_tiles) return;
    const uint32_t row = div_rows(t, a);
    const int c0 = (int)(t - row * (uint32_t)a.tiles_per_row) * U;
    const uint8_t* crow = a.codes + (int64_t)row * a.ldq;
    const bool mfma_layout = FMT != 2 && a.scale_layout == 1;
    // row-major: the scale row; MFMA layout: the row's place in its group
    const uint8_t* srow = mfma_layout ? a.scales + (int64_t)(row >> 4) * a.lds + 4 * (row & 15)
                                      : a.scales + (int64_t)row * a.lds;
    float* orow = a.out + (int64_t)row * a.ldo;

    uint32_t q0[U], q1[U], sb[U];
    bool in[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
        const uint32_t col = (uint32_t)((c0 + u) * kChunkElems + lane * kElemsPerLane);
        in[u] = c0 + u < a.chunks_per_row && col < (uint32_t)a.K;
        q0[u] = q1[u] = sb[u] = 0u;
        if (in[u]) {
            if constexpr (FMT == 1) {
                const c32x2_t v = __builtin_nontemporal_load(
                    reinterpret_cast<const c32x2_t*>(crow + col));
                q0[u] = v.x;
                q1[u] = v.y;
            } else {
                q0[u] = __builtin_nontemporal_load(reinterpret_cast<const uint32_t*>(crow + col / 2));
            }
            const int b = lane / (kBlock / kElemsPerLane);  // block within the chunk
            sb[u] = mfma_layout ? srow[(c0 + u) * 256 + 64 * (b & 3) + (b >> 2)]
                                : srow[col / kBlock];
        }
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
        if (!in[u]) continue;
        const uint32_t col = (uint32_t)((c0 + u) * kChunkElems + lane * kElemsPerLane);
        float f[8];
        decode8<FMT>(q0[u], q1[u], f);
        const float s = scale_value<FMT>(sb[u]);
#pragma unroll
        for (int j = 0; j < 8; ++j) f[j] = apply_scale<FMT>(f[j], s, a.tensor_sf);
        f32x4_t* o = reinterpret_cast<f32x4_t*>(orow + col);
        o[0] = (f32x4_t){f[0], f[1], f[2], f[3]};
        o[1] = (f32x4_t){f[4], f[5], f[6], f[7]};
    }
}

// Two consecutive decoded values (k even) of one operand row.
template <int FMT>
__device__ __forceinline__ f32x2_t operand_pair(const uint8_t* codes, int k) {
    if constexpr (FMT == 1) {
        const uint32_t w = *reinterpret_cast<const uint16_t*>(codes + k);
        return fp8_pair<false>(w);
    } else {
        return fp4_pair<0>((uint32_t)codes[k / 2]);
    }
}

// Naive GEMM: one thread per output c[m, n] = sum over k of A[m, k] * B[n, k]
// (both operands K-major, dequantized on the fly exactly as above), summed in
// fp32 in ascending k as acc = acc + a * b.
template <int FMT>
__global__ void __launch_bounds__(kThreadsPerBlock) naive_matmul_kernel(const GemmArgs a) {
    constexpr int kBlock = FMT == 2 ? 16 : 32;
    const int64_t idx = (int64_t)blockIdx.x * kThreadsPerBlock + threadIdx.x;
    if (idx >= a.M * a.N) return;
    const int64_t m = idx / a.N, n = idx - m * a.N;
    const uint8_t* ac = a.a_codes + m * a.lda_q;
    const bool mfma_layout = FMT != 2 && a.scale_layout == 1;
    const uint8_t* as = mfma_layout ? a.a_scales + (m >> 4) * a.lda_s : a.a_scales + m * a.lda_s;
    const uint8_t* bc = a.b_codes + n * a.ldb_q;
    const uint8_t* bs = mfma_layout ? a.b_scales + (n >> 4) * a.ldb_s : a.b_scales + n * a.ldb_s;
    float acc = 0.0f;
    for (int kb = 0; kb < a.K / kBlock; ++kb) {
        const float sa = scale_value<FMT>(mfma_layout ? as[mfma16_scale_offset(m, kb)] : as[kb]);
        const float sb = scale_value<FMT>(mfma_layout ? bs[mfma16_scale_offset(n, kb)] : bs[kb]);
        for (int k = kb * kBlock; k < (kb + 1) * kBlock; k += 2) {
            const f32x2_t ca = operand_pair<FMT>(ac, k);
            const f32x2_t cb = operand_pair<FMT>(bc, k);
            acc = acc + apply_scale<FMT>(ca[0], sa, a.a_tsf) * apply_scale<FMT>(cb[0], sb, a.b_tsf);
            acc = acc + apply_scale<FMT>(ca[1], sa, a.a_tsf) * apply_scale<FMT>(cb[1], sb, a.b_tsf);
        }
    }
    a.c[m * a.ldc + n] = acc;
}

// ------------------------------------------------------------ MFMA consumer
//
// c = A B^T with gfx950's scaled matrix instruction
// v_mfma_scale_f32_16x16x128_f8f6f4, reading the quantizers' MX output as
// is: codes row-major, scales in the MFMA layout.  Per 512 elements of K each
// lane takes one scale dword per operand, whose byte t feeds K step t
// (opsel = t).
//
// Operand fragments (measured with one-wave probes of known operands):
// lane l serves row l % 16 of its operand and group g = l / 16;
//  * FP4 (E2M1): the 32 consecutive elements [32 g, 32 g + 32) of the step,
//    16 bytes, in the first four registers;
//  * FP8 (E4M3): elements [16 g, 16 g + 16) and [64 + 16 g, 64 + 16 g + 16),
//    two 16-byte pieces.
// c tile: lane l holds rows 4 (l / 16) .. 4 (l / 16) + 3, column l % 16.
typedef int mfma_v8i __attribute__((ext_vector_type(8)));
typedef float mfma_v4f __attribute__((ext_vector_type(4)));

template <int FMT>
__device__ __forceinline__ mfma_v8i load_fragment(const uint8_t* row, int k0, int g, bool valid) {
    mfma_v8i v = {0, 0, 0, 0, 0, 0, 0, 0};
    if (!valid) return v;
    if constexpr (FMT == 1) {
        const int4 lo = *reinterpret_cast<const int4*>(row + k0 + 16 * g);
        const int4 hi = *reinterpret_cast<const int4*>(row + k0 + 64 + 16 * g);
        v = (mfma_v8i){lo.x, lo.y, lo.z, lo.w, hi.x, hi.y, hi.z, hi.w};
    } else {
        const int4 q = *reinterpret_cast<const int4*>(row + (k0 + 32 * g) / 2);
        v = (mfma_v8i){q.x, q.y, q.z, q.w, 0, 0, 0, 0};
    }
    return v;
}

// Tiled form: a workgroup computes a TM x TN tile of c with a WAVES_M x
// WAVES_N grid of waves, each wave a (16 IM) x (16 JN) block of instructions'
// 16 x 16 tiles, stepping through K in stages of 128 bytes per operand row
// (one 128-element K step of E4M3, two of E2M1) that are staged in LDS; its
// scale bytes come from the 512-element records of the MFMA layout, staged
// once per record in buffers of their own.
template <int TM_, int TN_, int WAVES_M_, int WAVES_N_>
struct TileCfg {
    static constexpr int TM = TM_, TN = TN_, WAVES_M = WAVES_M_, WAVES_N = WAVES_N_;
    static constexpr int NW = WAVES_M * WAVES_N;              // waves per workgroup
    static constexpr int IM = TM / WAVES_M / 16, JN = TN / WAVES_N / 16;
    static constexpr int kChunksA = TM / 8 / NW;               // 1 KiB row chunks per wave
    static constexpr int kChunksB = TN / 8 / NW;
    static constexpr int kRecords = (TM + TN) / 16;            // scale records per 512 elements
    static constexpr int kRecordLoads = kRecords / (4 * NW);   // 1 KiB runs of records per wave
    static constexpr int kStageBytes = (TM + TN) * 128;        // one stage of operand rows
    static constexpr int kRecordBytes = kRecords * 256;        // one record of every row group
    // every wave moves the same number of rows and of 1 KiB runs of records
    static_assert(TM % (8 * NW) == 0 && TN % (8 * NW) == 0 && kRecords % (4 * NW) == 0,
                  "tile shape");
};
using Tile128 = TileCfg<128, 128, 2, 2>;   // 4 waves of 64 x 64
using Tile256 = TileCfg<256, 256, 2, 4>;   // 8 waves of 128 x 64
constexpr int kTileM = Tile128::TM, kTileN = Tile128::TN;  // grouped form

// One workgroup tile of c: operand rows and scale groups relative to the
// tile's first row, valid-row counts, and the output window.
struct GemmTile {
    const uint8_t* a;          // A codes, first row of the tile
    int64_t lda_q, a_rows;     // row stride; rows that exist from here on
    const uint8_t* as;         // A scales (MFMA layout), first row group of the tile
    int64_t lda_s, a_groups;   // row-group stride; row groups that exist from here on
    const uint8_t* b;
    int64_t ldb_q, b_rows;
    const uint8_t* bs;
    int64_t ldb_s, b_groups;
    float* c;                  // c[0, 0] of the tile
    int64_t ldc, c_rows, c_cols;
    int K;
};

// Tile descriptors.  Dense: workgroup -> TM x TN tile, row-major.
template <int TM, int TN>
__device__ __forceinline__ void dense_desc(const GemmArgs& a, int64_t tiles_n, GemmTile& d) {
    const int64_t m0 = (int64_t)(blockIdx.x / tiles_n) * TM;
    const int64_t n0 = (int64_t)(blockIdx.x % tiles_n) * TN;
    d.a = a.a_codes + m0 * a.lda_q;
    d.lda_q = a.lda_q;
    d.a_rows = a.M - m0;
    d.as = a.a_scales + (m0 >> 4) * a.lda_s;
    d.lda_s = a.lda_s;
    d.a_groups = (a.M + 15) / 16 - (m0 >> 4);
    d.b = a.b_codes + n0 * a.ldb_q;
    d.ldb_q = a.ldb_q;
    d.b_rows = a.N - n0;
    d.bs = a.b_scales + (n0 >> 4) * a.ldb_s;
    d.ldb_s = a.ldb_s;
    d.b_groups = (a.N + 15) / 16 - (n0 >> 4);
    d.c = a.c + m0 * a.ldc + n0;
    d.ldc = a.ldc;
    d.c_rows = a.M - m0;
    d.c_cols = a.N - n0;
    d.K = a.K;
}

// Grouped per-expert form.  Row tiles of TM rows are counted across the
// groups in order (group g has ceil(m_g / TM) of them).  Group g multiplies
// its routed rows (codes row r, scale row scales_offsets[g] + r -
// row_offsets[g]) by the B of expert expert_ids[g] ([N, K] codes from row
// e N, scales from row group e ceil(N / 16)).

// Total row tiles over all groups (wave-uniform): each lane takes one
// group's tile count, 64 groups per step, summed across the lanes.
template <int TM>
__device__ __forceinline__ uint32_t total_row_tiles(const GroupedGemmArgs& g) {
    const int lane = (int)(threadIdx.x & 63);
    uint32_t total = 0;
    for (int h0 = 0; h0 < g.num_groups; h0 += 64) {
        const int h = h0 + lane;
        uint32_t tiles = 0;
        if (h < g.num_groups) {
            const uint32_t l = g.row_offsets[h], u = g.row_offsets[h + 1];
            tiles = u > l ? (uint32_t)(((uint64_t)u - l + TM - 1) / TM) : 0u;
        }
#pragma unroll
        for (int off = 32; off >= 1; off >>= 1) tiles += (uint32_t)__shfl_xor((int)tiles, off);
        total += tiles;
    }
    return total;
}

// The descriptor of row tile t of group grp (rows [lo, hi) of A, scale rows from
// so, expert e) and TN-column tile col.  A group whose metadata falls outside
// the buffers, or whose scale offset is not a multiple of 16 (the layout's row
// groups), is skipped: returns false.
template <int TM, int TN>
__device__ __forceinline__ bool fill_grouped_desc(const GemmArgs& a, const GroupedGemmArgs& g,
                                                  int64_t lo, int64_t hi, int64_t so, int e,
                                                  int64_t t, int64_t col, GemmTile& d) {
    if (hi > g.max_rows || e < 0 || e >= g.num_experts || so % 16 != 0 ||
        so + (hi - lo) > g.num_scale_rows)
        return false;
    const int64_t n0 = col * TN, r0 = lo + t * TM;
    const int64_t groups_n = (a.N + 15) / 16;
    d.a = a.a_codes + r0 * a.lda_q;
    d.lda_q = a.lda_q;
    d.a_rows = hi - r0;
    d.as = a.a_scales + ((so + t * TM) >> 4) * a.lda_s;
    d.lda_s = a.lda_s;
    d.a_groups = (hi - r0 + 15) / 16;
    d.b = a.b_codes + ((int64_t)e * a.N + n0) * a.ldb_q;
    d.ldb_q = a.ldb_q;
    d.b_rows = a.N - n0;
    d.bs = a.b_scales + ((int64_t)e * groups_n + (n0 >> 4)) * a.ldb_s;
    d.ldb_s = a.ldb_s;
    d.b_groups = groups_n - (n0 >> 4);
    d.c = a.c + r0 * a.ldc + n0;
    d.ldc = a.ldc;
    d.c_rows = hi - r0;
    d.c_cols = a.N - n0;
    d.K = a.K;
    return true;
}

// The tile descriptor of row tile t and TN-column tile col: the wave reads 64
// groups' offsets at a time and finds the group holding tile t from the
// prefix sum of their tile counts across the lanes (t and every sum are
// wave-uniform).  A group-by-group walk measured 29 us on its own for the
// 128-expert prefill routing.  Returns false for a skipped group and for a t
// past the last group's tiles.
template <int TM, int TN>
__device__ __forceinline__ bool grouped_tile_desc(const GemmArgs& a, const GroupedGemmArgs& g,
                                                  int64_t t, int64_t col, GemmTile& d) {
    int grp = -1;
    int64_t lo = 0, hi = 0;
    const int lane = (int)(threadIdx.x & 63);
    for (int h0 = 0; h0 < g.num_groups; h0 += 64) {
        const int h = h0 + lane;
        uint32_t l = 0, u = 0, tiles = 0;
        if (h < g.num_groups) {
            l = g.row_offsets[h];
            u = g.row_offsets[h + 1];
            tiles = u > l ? (uint32_t)(((uint64_t)u - l + TM - 1) / TM) : 0u;
        }
        uint32_t incl = tiles;                               // at most 2^25 + 64 in total
#pragma unroll
        for (int off = 1; off < 64; off <<= 1) {
            const uint32_t v = (uint32_t)__shfl_up((int)incl, off);
            if (lane >= off) incl += v;
        }
        const uint32_t total = (uint32_t)__shfl((int)incl, 63);
        if (t < (int64_t)total) {
            // the first lane past t has tiles > 0, so it is a real group
            const int L = __ffsll(__ballot((int64_t)incl > t)) - 1;
            grp = h0 + L;
            lo = (uint32_t)__shfl((int)l, L);
            hi = (uint32_t)__shfl((int)u, L);
            t -= (uint32_t)__shfl((int)(incl - tiles), L);
            break;
        }
        t -= total;
    }
    if (grp < 0) return false;                               // past the last group's tiles
    return fill_grouped_desc<TM, TN>(a, g, lo, hi, g.scales_offsets[grp], g.expert_ids[grp], t,
                                     col, d);
}

// Decode form: workgroup w takes row tile w / n_col and column tile w % n_col,
// so consecutive workgroups stream consecutive 128-row blocks of one expert's
// weights (one contiguous run across the chip) and share the tile's A rows.
// Row tile fastest, they read blocks of different experts: 309.7 against
// 293.7 us on the decode routing (512 routed rows over 256 experts, N = 7168,
// K = 2048, MXFP4; same outputs, A/B on one box).
template <int TM, int TN>
__device__ __forceinline__ bool grouped_desc(const GemmArgs& a, const GroupedGemmArgs& g,
                                             GemmTile& d) {
    const int64_t n_col = (a.N + TN - 1) / TN;
    return grouped_tile_desc<TM, TN>(a, g, blockIdx.x / n_col, blockIdx.x % n_col, d);
}

// 128-row form: the work items (row tile t, column tile c), numbered t major,
// are dealt to the XCDs in contiguous runs.  The hardware hands workgroup w
// to XCD w % 8, so workgroup w takes item (w % 8) * per_xcd + w / 8: an XCD
// runs the column tiles of a row tile, and the row tiles of an expert, one
// after another, and serves their shared A rows and B weights from its own
// L2.  The grid holds at least 8 * per_xcd workgroups; the rest return.
constexpr int kXcds = 8;

// The item of this workgroup, or false when it has none.
__device__ __forceinline__ bool xcd_item(int64_t total_tiles, int64_t n_col, int64_t& item) {
    const int64_t items = total_tiles * n_col;
    const int64_t per_xcd = (items + kXcds - 1) / kXcds;
    const int64_t w = blockIdx.x, slot = w / kXcds;
    item = (w % kXcds) * per_xcd + slot;
    return slot < per_xcd && item < items;
}

// Up to kRegGroups groups, each lane loads its groups' row offsets, scale
// offset and expert id in one round of loads; the tile count, the item, its
// group and the group's metadata then come from registers.  Measured on the
// prefill routing: 70.2 us against 72.1 for the search below, which reads the
// offsets twice (the tile count, then the search) and the group's metadata
// after it: three loads in a row before a tile's first stage can be issued.
constexpr int kRegChunks = 4, kRegGroups = 64 * kRegChunks;
template <int TM, int TN>
__device__ __forceinline__ bool grouped_desc_xcd_regs(const GemmArgs& a, const GroupedGemmArgs& g,
                                                      GemmTile& d) {
    const int lane = (int)(threadIdx.x & 63);
    uint32_t l[kRegChunks], u[kRegChunks], so[kRegChunks], incl[kRegChunks], tot[kRegChunks];
    int ids[kRegChunks];
#pragma unroll
    for (int c = 0; c < kRegChunks; ++c) {
        const int h = 64 * c + lane;
        const bool ok = h < g.num_groups;
        l[c] = ok ? g.row_offsets[h] : 0u;
        u[c] = ok ? g.row_offsets[h + 1] : 0u;
        so[c] = ok ? g.scales_offsets[h] : 0u;
        ids[c] = ok ? g.expert_ids[h] : -1;
    }
    uint32_t total = 0;
#pragma unroll
    for (int c = 0; c < kRegChunks; ++c) {
        const uint32_t tiles = u[c] > l[c] ? (uint32_t)(((uint64_t)u[c] - l[c] + TM - 1) / TM) : 0u;
        uint32_t x = tiles;
#pragma unroll
        for (int off = 1; off < 64; off <<= 1) {
            const uint32_t v = (uint32_t)__shfl_up((int)x, off);
            if (lane >= off) x += v;
        }
        incl[c] = x;
        tot[c] = (uint32_t)__builtin_amdgcn_readfirstlane(__shfl((int)x, 63));
        total += tot[c];
    }
    const int64_t n_col = (a.N + TN - 1) / TN;
    int64_t item;
    if (!xcd_item(total, n_col, item)) return false;
    int64_t t = item / n_col;
#pragma unroll
    for (int c = 0; c < kRegChunks; ++c) {
        if (t >= (int64_t)tot[c]) {
            t -= tot[c];
            continue;
        }
        // the first lane past t has tiles > 0, so it is a real group
        const int L = __ffsll(__ballot((int64_t)incl[c] > t)) - 1;
        const uint32_t lo = (uint32_t)__builtin_amdgcn_readlane((int)l[c], L);
        const uint32_t hi = (uint32_t)__builtin_amdgcn_readlane((int)u[c], L);
        const uint32_t tiles = hi > lo ? (uint32_t)(((uint64_t)hi - lo + TM - 1) / TM) : 0u;
        t -= (uint32_t)__builtin_amdgcn_readlane((int)incl[c], L) - tiles;
        return fill_grouped_desc<TM, TN>(a, g, lo, hi,
                                         (uint32_t)__builtin_amdgcn_readlane((int)so[c], L),
                                         __builtin_amdgcn_readlane(ids[c], L), t, item % n_col, d);
    }
    return false;                                            // unreachable: item < items
}

template <int TM, int TN>
__device__ __forceinline__ bool grouped_desc_xcd(const GemmArgs& a, const GroupedGemmArgs& g,
                                                 GemmTile& d) {
    if (g.num_groups <= kRegGroups) return grouped_desc_xcd_regs<TM, TN>(a, g, d);
    const int64_t n_col = (a.N + TN - 1) / TN;
    int64_t item;
    if (!xcd_item(total_row_tiles<TM>(g), n_col, item)) return false;
    return grouped_tile_desc<TM, TN>(a, g, item / n_col, item % n_col, d);
}

// Pipelined form of the tile: the stages of A and B go straight from global
// memory to LDS (global_load_lds_dwordx4, 1 KiB per wave instruction), NBUF
// stages deep, so NBUF - 1 stages of loads are in flight while one is being
// multiplied, with no registers holding them.  A stage buffer holds the TM A
// rows and TN B rows of 128 bytes each, unpadded; logical 16-byte piece c
// of row R sits at piece c ^ (R % 8) (each lane chooses which global piece it
// fetches for its LDS slot), so the 8 rows a fragment read serves at once
// fall in distinct banks.  The scale records of a 512-element span of K
// (TM / 16 A row groups, then TN / 16 B row groups, 256 bytes each) go to one
// of two record buffers, loaded with the span's first stage: an E2M1 record
// serves two stages, an E4M3 one four.

__device__ __forceinline__ void dma16(const void* g, uint8_t* lds) {
    __builtin_amdgcn_global_load_lds(const_cast<void*>(g), lds, 16, 0, 0);
}

template <int N>
__device__ __forceinline__ void wait_vm() {
    // s_waitcnt with vmcnt <= N and the other counters unconstrained
    __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | 0x0F70);
}

// SKIP_PAD (the grouped form, whose partial row tiles average a third padding):
// chunks of A wholly past the rows are not loaded and 16-row blocks past them
// not multiplied; the dense form keeps straight-line stages (the skip costs its
// 256 x 256 MXFP8 tile registers enough to spill).
//
// NT_STORE (the grouped form): c leaves with nontemporal stores of whole
// rows of the wave's block, staged through LDS.  The grouped form's tiles end
// throughout the launch, and written through ordinary stores they stayed
// dirty in the XCDs' L2: nontemporal stores took 3-5 us off the 73-78 us of
// the prefill routing.  Stored straight from the MFMA layout, each such store
// covered 64 bytes of 16 rows, half lines that were written to memory apart
// (48.9 MB of writes for 33.5 MB of c); staged, each covers 256 bytes of 4
// rows: 71.2 -> 66.7 us.  The dense form's tiles all end together, and there
// ordinary stores from registers measured faster (4096 x 4096 x 7168: 68
// against 74 us for MXFP4, 112 against 117 for MXFP8).  Same outputs, A/B
// runs on one box.
template <int FMT, int NBUF, class Cfg, bool SKIP_PAD, bool NT_STORE>
__device__ __forceinline__ void gemm_tile_dma(const GemmTile& d, uint8_t* const (&bufs)[NBUF],
                                              uint8_t* const (&recs)[2]) {
    constexpr int kFmt = FMT == 1 ? 0 : 4;
    constexpr int kStepBytes = FMT == 1 ? 128 : 64;
    constexpr int kSteps = 128 / kStepBytes;                 // K steps per stage
    constexpr int kStageElems = kSteps * 128;
    constexpr int TM = Cfg::TM, IM = Cfg::IM, JN = Cfg::JN;
    constexpr int kPerRecord = 4 / kSteps;                   // stages per 512-element scale record
    // with two buffers a wave waits for all its loads (vmcnt 0) at the top of a stage, so
    // waves may issue different numbers of them (SKIP_PAD)
    static_assert(NBUF == 2, "the stage wait assumes two buffers");
    // the stage loop is unrolled over two records, so each unrolled stage's stage buffer,
    // record buffer and opsel byte are constants
    constexpr int kUnroll = 2 * kPerRecord;
    static_assert(kUnroll % NBUF == 0, "stage buffers per unrolled pass");
    const int tid = (int)threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // uniform in the wave
    const int wm = wave / Cfg::WAVES_N, wn = wave % Cfg::WAVES_N;
    const int row_bytes = FMT == 1 ? d.K : d.K / 2;
    const int nstages = (d.K + kStageElems - 1) / kStageElems;

    // this lane's slot in a 1 KiB chunk: row 8 c + lane / 8, physical piece lane % 8
    const int crow = lane >> 3, cpiece = lane & 7;
    // stage s goes to buffer s % NBUF and the records of its 512 elements to record
    // buffer (s / kPerRecord) % 2; the caller passes both as constants, so every LDS
    // access names one buffer (distinct LDS objects keep the compiler's waits for the
    // in-flight loads to the buffer actually read).  rec is null for a stage that does
    // not start a record.
    auto issue = [&](int s, uint8_t* buf, uint8_t* rec) {
        // row chunk c (rows 8 c .. 8 c + 7) of an operand goes to 1 KiB at c;
        // rows past the operand load its last row, bytes past K any in-row
        // bytes: their products are never stored
        const int kb0 = s * 128;
        int kb = kb0 + 16 * (cpiece ^ crow);
        kb = kb < row_bytes ? kb : 0;
        // with SKIP_PAD a chunk wholly past the operand's rows is not loaded (its rows'
        // products are never stored, so the stale bytes there are harmless)
#pragma unroll
        for (int i = 0; i < Cfg::kChunksA; ++i) {
            const int chunk = wave + Cfg::NW * i, row = 8 * chunk + crow;
            if (SKIP_PAD && 8 * chunk >= d.a_rows) break;
            const int64_t ra = row < d.a_rows ? row : d.a_rows - 1;
            dma16(d.a + ra * d.lda_q + kb, buf + chunk * 1024);
        }
#pragma unroll
        for (int i = 0; i < Cfg::kChunksB; ++i) {
            const int chunk = wave + Cfg::NW * i, row = 8 * chunk + crow;
            const int64_t rb = row < d.b_rows ? row : d.b_rows - 1;
            dma16(d.b + rb * d.ldb_q + kb, buf + TM * 128 + chunk * 1024);
        }
        if (rec == nullptr) return;
        // scale records of the stage's 512 elements (A row groups, then B row
        // groups): run j = wave + NW i holds records 4 j .. 4 j + 3, lane L moving
        // bytes 16 (L % 16) of record 4 j + L / 16
        const int k512 = (s * kStageElems) / 512;
#pragma unroll
        for (int i = 0; i < Cfg::kRecordLoads; ++i) {
            const int run = wave + Cfg::NW * i;
            const int r = 4 * run + (lane >> 4);
            const bool is_a = r < TM / 16;
            const int g = is_a ? r : r - TM / 16;
            const int64_t groups = is_a ? d.a_groups : d.b_groups;
            const int64_t gg = g < groups ? g : groups - 1;
            const uint8_t* src = (is_a ? d.as + gg * d.lda_s : d.bs + gg * d.ldb_s) +
                                 (int64_t)k512 * 256 + 16 * (lane & 15);
            dma16(src, rec + run * 1024);
        }
    };

    mfma_v4f acc[IM][JN];
#pragma unroll
    for (int i = 0; i < IM; ++i)
#pragma unroll
        for (int j = 0; j < JN; ++j) acc[i][j] = (mfma_v4f){0.0f, 0.0f, 0.0f, 0.0f};

    if (nstages > 0) issue(0, bufs[0], recs[0]);
    const int fr = lane & 15, fg = lane >> 4;
    for (int s0 = 0; s0 < nstages; s0 += kUnroll) {
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
        const int s = s0 + u;
        if (s >= nstages) break;
        // this wave's loads of stage s are done after the wait; after the barrier every
        // wave's are, and every wave has finished reading stage s - 1 (its MFMAs
        // consumed those reads), so its buffer can be refilled.  No fence: the loads
        // write LDS directly and the explicit wait is the one they need.
        wait_vm<0>();
        asm volatile("s_barrier" ::: "memory");
        const uint8_t* buf = bufs[u % NBUF];
        const uint8_t* rec = recs[(u / kPerRecord) % 2];
        // the scale dwords are read before the next stage's loads are issued: read after
        // them, the compiler made the stage's fragment reads wait for those loads too.
        // Row groups past the operand's end hold the last group's record (their outputs
        // are never stored), so every read is unconditional.
        uint32_t sa[IM], sb[JN];
#pragma unroll
        for (int i = 0; i < IM; ++i)
            sa[i] = *reinterpret_cast<const uint32_t*>(rec + ((IM * wm + i) * 256 + 4 * lane));
#pragma unroll
        for (int i = 0; i < JN; ++i)
            sb[i] = *reinterpret_cast<const uint32_t*>(
                rec + ((TM / 16 + JN * wn + i) * 256 + 4 * lane));
        // the next stage's rows, and its record when it starts one (into the record buffer
        // whose last reader finished before this barrier)
        if (s + 1 < nstages) {
            if ((u + 1) % kPerRecord == 0)
                issue(s + 1, bufs[(u + 1) % NBUF], recs[((u + 1) / kPerRecord) % 2]);
            else
                issue(s + 1, bufs[(u + 1) % NBUF], nullptr);
        }
        // every LDS address is the buffer plus one integer offset: a single step from
        // the LDS object keeps the compiler's knowledge of which buffer is read
        auto fragment = [&](int region, int r0, int j) {
            const int r = r0 + fr;
            const int row = region + r * 128;
            mfma_v8i v;
            if constexpr (FMT == 1) {
                const int4 lo = *reinterpret_cast<const int4*>(buf + (row + 16 * (fg ^ (r & 7))));
                const int4 hi =
                    *reinterpret_cast<const int4*>(buf + (row + 16 * ((4 + fg) ^ (r & 7))));
                v = (mfma_v8i){lo.x, lo.y, lo.z, lo.w, hi.x, hi.y, hi.z, hi.w};
            } else {
                const int4 q =
                    *reinterpret_cast<const int4*>(buf + (row + 16 * ((4 * j + fg) ^ (r & 7))));
                v = (mfma_v8i){q.x, q.y, q.z, q.w, 0, 0, 0, 0};
            }
            return v;
        };
#pragma unroll
        for (int j = 0; j < kSteps; ++j) {
            const int k = s * kStageElems + j * 128;
            if (k >= d.K) break;
            const int t = (u * kSteps + j) & 3;              // opsel byte: (k / 128) mod 4
            mfma_v8i fb[JN];
#pragma unroll
            for (int jn = 0; jn < JN; ++jn) fb[jn] = fragment(TM * 128, 16 * (JN * wn + jn), j);
#pragma unroll
            for (int im = 0; im < IM; ++im) {
                if (SKIP_PAD && 16 * (IM * wm + im) >= d.a_rows) break;  // past the rows
                const mfma_v8i fa = fragment(0, 16 * (IM * wm + im), j);
#pragma unroll
                for (int jn = 0; jn < JN; ++jn) {
                    // B as the first operand: the result is the tile of c transposed, so
                    // lane l holds row l % 16 and columns 4 (l / 16) .. + 3 of c
                    switch (t) {
                        case 0: acc[im][jn] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
                                    fb[jn], fa, acc[im][jn], kFmt, kFmt, 0, (int)sb[jn], 0,
                                    (int)sa[im]); break;
                        case 1: acc[im][jn] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
                                    fb[jn], fa, acc[im][jn], kFmt, kFmt, 1, (int)sb[jn], 1,
                                    (int)sa[im]); break;
                        case 2: acc[im][jn] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
                                    fb[jn], fa, acc[im][jn], kFmt, kFmt, 2, (int)sb[jn], 2,
                                    (int)sa[im]); break;
                        default: acc[im][jn] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
                                    fb[jn], fa, acc[im][jn], kFmt, kFmt, 3, (int)sb[jn], 3,
                                    (int)sa[im]); break;
                    }
                }
            }
        }
    }
    }
    const bool vec = ((reinterpret_cast<uintptr_t>(d.c) | (uintptr_t)(d.ldc * 4)) & 15) == 0;
    // one 16-byte store when its four columns exist and c's rows are 16-byte aligned, else
    // one per element
    auto store4 = [&](const mfma_v4f& v, int64_t row, int64_t col) {
        float* p = d.c + row * d.ldc + col;
        if (vec && col + 4 <= d.c_cols) {
            if constexpr (NT_STORE) __builtin_nontemporal_store(v, reinterpret_cast<mfma_v4f*>(p));
            else *reinterpret_cast<mfma_v4f*>(p) = v;
        } else {
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                if (col + e >= d.c_cols) continue;
                if constexpr (NT_STORE) __builtin_nontemporal_store(v[e], p + e);
                else p[e] = v[e];
            }
        }
    };
    if constexpr (NT_STORE) {
        // the wave's (16 IM) x (16 JN) block goes to its own part of the stage buffers, free
        // once every wave is past its last stage (16-byte piece q of row r at q ^ (r % 16)),
        // and leaves as runs of 64 JN bytes: lane l stores piece l % (4 JN) of a row
        constexpr int kPieces = 4 * JN, kRowsPer = 64 / kPieces;
        constexpr int kWaveBytes = 16 * IM * 16 * kPieces;
        static_assert(Cfg::NW == 4 && 2 * kWaveBytes == Cfg::kStageBytes && kPieces == 16,
                      "two waves' blocks per stage buffer");
        __syncthreads();
        uint8_t* blk = (wave < 2 ? bufs[0] : bufs[1]) + (wave & 1) * kWaveBytes;
#pragma unroll
        for (int im = 0; im < IM; ++im)
#pragma unroll
            for (int jn = 0; jn < JN; ++jn) {
                const int r = 16 * im + fr, q = 4 * jn + fg;
                *reinterpret_cast<mfma_v4f*>(blk + r * (16 * kPieces) + 16 * (q ^ (r & 15))) =
                    acc[im][jn];
            }
        const int q = lane % kPieces;
#pragma unroll
        for (int k = 0; k < 16 * IM / kRowsPer; ++k) {
            const int r = kRowsPer * k + lane / kPieces;
            const int64_t row = 16 * IM * wm + r;
            if (row >= d.c_rows) continue;
            store4(*reinterpret_cast<const mfma_v4f*>(blk + r * (16 * kPieces) + 16 * (q ^ (r & 15))),
                   row, 16 * JN * wn + 4 * q);
        }
    } else {
        // lane l holds row l % 16 and columns 4 (l / 16) .. + 3 of each 16 x 16 tile
#pragma unroll
        for (int im = 0; im < IM; ++im) {
            const int64_t row = 16 * (IM * wm + im) + fr;
            if (row >= d.c_rows) continue;
#pragma unroll
            for (int jn = 0; jn < JN; ++jn) store4(acc[im][jn], row, 16 * (JN * wn + jn) + 4 * fg);
        }
    }
}

// The stage and record buffers are separate LDS objects: the compiler then knows
// which buffer each LDS read and each direct load touches, and waits only for
// the loads into the buffer being read.
// Two stage buffers (a third leaves one 128 x 128 workgroup per CU and
// measured slower).
#define BSQ_STAGE_BUFFERS(Cfg)                                                             \
    __shared__ __attribute__((aligned(16))) uint8_t stage0[Cfg::kStageBytes];              \
    __shared__ __attribute__((aligned(16))) uint8_t stage1[Cfg::kStageBytes];              \
    __shared__ __attribute__((aligned(16))) uint8_t record0[Cfg::kRecordBytes];            \
    __shared__ __attribute__((aligned(16))) uint8_t record1[Cfg::kRecordBytes];            \
    uint8_t* const bufs[2] = {stage0, stage1};                                             \
    uint8_t* const recs[2] = {record0, record1};

template <int FMT, class Cfg>
__global__ void __launch_bounds__(64 * Cfg::NW) mfma_gemm_tiled_kernel(const GemmArgs a,
                                                                        int64_t tiles_n) {
    BSQ_STAGE_BUFFERS(Cfg)
    GemmTile d;
    dense_desc<Cfg::TM, Cfg::TN>(a, tiles_n, d);
    gemm_tile_dma<FMT, 2, Cfg, false, false>(d, bufs, recs);
}

// The grouped form for groups of more than 16 rows on average.  Measured on
// the prefill routing (16384 rows over 128 experts, N = 512, K = 7168,
// MXFP4), these 128 x 128 tiles of 4 waves with both operands staged through
// two LDS buffers run 66-68.5 us.  The alternatives tried ran slower: 128 x 256
// tiles of 8 waves (88.6 us), 128 x 512 tiles of 8 waves that read each A row
// tile once (77 against 77), B straight to registers with three LDS stages for
// A (92), 64 x 128 tiles (91), four stage buffers and one workgroup per CU (94
// against 77), every workgroup of an XCD given an equal run of K stages over
// consecutive tiles (99 against 73.5: neighbouring workgroups then no longer
// share A and B in the XCD's L2 at the same time).  A copy that skips the LDS
// fragment reads and the MFMAs runs within 6% of it; one that loads only its
// first stage ran at half its time.  Its 804 tiles fill 1.57 rounds of the
// 512 slots (two per CU), and a tile's time is set by its 28 stages' latency,
// not by how many tiles share the chip: the second, partial round costs about
// as much as the first.
template <int FMT>
__global__ void __launch_bounds__(64 * Tile128::NW)
mfma_gemm_grouped_kernel(const GemmArgs a, const GroupedGemmArgs g) {
    BSQ_STAGE_BUFFERS(Tile128)
    GemmTile d;
    if (!grouped_desc_xcd<kTileM, kTileN>(a, g, d)) return;
    gemm_tile_dma<FMT, 2, Tile128, true, true>(d, bufs, recs);
}

// ------------------------------------------------------------ decode regime
//
// Grouped GEMM for groups of a few rows each (a decode step: a handful of
// tokens per expert).  A 128-row tile would spend nearly all of its matrix
// work and LDS traffic on padding rows, and the expert's weights dominate the
// bytes, so this form is built around streaming B once per 16 routed rows:
//  * a workgroup takes 16 MB rows of one group (MB = 1 or 2 blocks of the
//    instruction's smallest M) and 128 columns of c, split over its waves;
//    each wave owns MB x J 16 x 16 tiles of c over the whole of K;
//  * each wave streams its own B rows through its own LDS slice, 512
//    elements of K (four K steps, one scale dword per operand) per round,
//    with no barrier; A fragments go straight to registers; the waves
//    sharing a CU cover each other's latency;
//  * rows past the group load its last row and columns past N the last B
//    row (their outputs are never stored), so every load is in bounds.
// It follows the decode entry in the "NVFP4 routing" section of the grouped
// block-scaled SM100 matmul's "dispatch" page (few rows per expert: a narrow
// tile on the token side), with the smallest tile the CDNA4 instruction has.
// Waves of a workgroup and 16-column tiles per wave, for MB row blocks: the
// tile is always kDecodeTileCols = 128 columns wide.  Measured (MXFP4, 256
// experts, N = 512, K = 7168): 16-row tiles 101.5 us at 8 rows per expert
// with 4 waves of J = 2, 107.0 with 2 waves of J = 4; 32-row tiles 94.4 /
// 99.4 us at 8 / 16 rows per expert with 2 waves of J = 4, 95.6 / 107.8 with
// 4 waves of J = 2 and 93.2 / 98.9 with 1 wave of J = 8.  MXFP8 keeps J = 2:
// with J = 4 its 32-row tiles take 332 registers, one wave per SIMD.
template <int FMT, int MB>
struct SkinnyShape {
    static constexpr int J = (MB == 2 && FMT == 0) ? 4 : 2;
    static constexpr int kWaves = kDecodeTileCols / (16 * J);
    static constexpr int kRowBytes = FMT == 1 ? 512 : 256;   // a B row's bytes per round
    static constexpr int kStageBytes = kWaves * 16 * J * kRowBytes;
};
static_assert(SkinnyShape<0, 1>::kWaves * 16 * SkinnyShape<0, 1>::J == kDecodeTileCols &&
                  SkinnyShape<1, 2>::kWaves * 16 * SkinnyShape<1, 2>::J == kDecodeTileCols,
              "decode tile shape");

template <int FMT, int S>
__device__ __forceinline__ mfma_v4f mfma_opsel(const mfma_v8i& fa, const mfma_v8i& fb,
                                              const mfma_v4f& acc, uint32_t sa, uint32_t sb) {
    constexpr int kFmt = FMT == 1 ? 0 : 4;  // instruction format codes: 0 E4M3, 4 E2M1
    return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(fa, fb, acc, kFmt, kFmt, S, (int)sa, S,
                                                            (int)sb);
}

// One K step S (of the round's four) of the wave's J tiles, if it exists.
// The products of one K step of the wave's MB x J tiles; S is the step's
// place in its 512-element scale record (the instruction's scale byte select).
template <int FMT, int J, int MB, int S>
__device__ __forceinline__ void skinny_step(const mfma_v8i (&fa)[MB], const mfma_v8i (&fb)[J],
                                            mfma_v4f (&acc)[MB][J], const uint32_t (&sa)[MB],
                                            const uint32_t (&sb)[J]) {
#pragma unroll
    for (int m = 0; m < MB; ++m)
#pragma unroll
        for (int j = 0; j < J; ++j)
            acc[m][j] = mfma_opsel<FMT, S>(fa[m], fb[j], acc[m][j], sa[m], sb[j]);
}

// A wave's MB x J 16 x 16 tiles of c (16 MB rows of one group, 16 J
// columns) over all of K, in rounds of 4 K steps (one 512-element scale
// record).  Each round's B rows (16 J rows) go to the
// wave's own LDS slice with direct loads, 1 KiB per instruction as whole
// 16-byte pieces of kRowBytes-byte row segments (4 rows per instruction for
// E2M1, 2 for E4M3), so every request covers whole cache lines; piece p of
// row r is stored at slot p ^ (r % kPieces), so the fragment reads of 16 rows
// fall in distinct banks.  A fragments (16 rows, shared by every wave and
// read from L2) go straight to registers, MB row blocks of them, so each
// B byte staged feeds MB products.  Only the wave itself reads its
// slice, so there is no barrier: the compiler's wait for the direct loads
// precedes the reads, and the reads are complete before the next round's
// loads overwrite the slice.
template <int FMT, int J, int MB>
__device__ __forceinline__ void gemm_tile_skinny(const GemmTile& d, uint8_t* stage) {
    constexpr int kRowBytes = FMT == 1 ? 512 : 256;          // a row's bytes per round
    constexpr int kPieces = kRowBytes / 16;
    constexpr int kRows = 16 * J;
    constexpr int kRowsPerInst = 64 / kPieces;
    constexpr int kInsts = kRows / kRowsPerInst;
    constexpr int kWaveBytes = kRows * kRowBytes;
    const int lane = (int)(threadIdx.x & 63);
    const int wave = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
    const int cb = 16 * J * wave;
    if (cb >= d.c_cols) return;
    const int fr = lane & 15, fg = lane >> 4;
    // row block m: rows 16 m .. 16 m + 15 of the tile; rows past the group
    // load its last row, row groups past it its last scale record
    const uint8_t* arow[MB];
    const uint8_t* asr[MB];
#pragma unroll
    for (int m = 0; m < MB; ++m) {
        const int64_t r = 16 * m + fr, gm = m;
        arow[m] = d.a + (r < d.a_rows ? r : d.a_rows - 1) * d.lda_q;
        asr[m] = d.as + (gm < d.a_groups ? gm : d.a_groups - 1) * d.lda_s + 4 * lane;
    }
    const uint8_t* bsr[J];
#pragma unroll
    for (int j = 0; j < J; ++j) {
        const int64_t gb = (cb + 16 * j) >> 4;
        bsr[j] = d.bs + (gb < d.b_groups ? gb : d.b_groups - 1) * d.ldb_s + 4 * lane;
    }
    // this lane's row and piece in each direct load of a round
    const int lrow = lane / kPieces, lslot = lane % kPieces;
    const uint8_t* src[kInsts];
    int piece_off[kInsts];
#pragma unroll
    for (int i = 0; i < kInsts; ++i) {
        const int r = i * kRowsPerInst + lrow;                // row within the wave's rows
        const int64_t rb = cb + r < d.b_rows ? cb + r : d.b_rows - 1;
        src[i] = d.b + rb * d.ldb_q;
        piece_off[i] = 16 * (lslot ^ (r % kPieces));
    }
    uint8_t* slice = stage + wave * kWaveBytes;
    const int row_bytes = FMT == 1 ? d.K : d.K / 2;
    mfma_v4f acc[MB][J];
#pragma unroll
    for (int m = 0; m < MB; ++m)
#pragma unroll
        for (int j = 0; j < J; ++j) acc[m][j] = (mfma_v4f){0.0f, 0.0f, 0.0f, 0.0f};

    const int nk = d.K / 128;
    for (int k0 = 0; k0 < nk; k0 += 4) {
        // reads of the previous round are done before their slots are refilled
        asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
        const int rb0 = k0 * (kRowBytes / 4);                 // the round's first byte in a row
#pragma unroll
        for (int i = 0; i < kInsts; ++i) {
            int off = rb0 + piece_off[i];
            off = off < row_bytes ? off : 0;                  // past K (a partial round): any in-row bytes
            __builtin_amdgcn_global_load_lds(const_cast<uint8_t*>(src[i] + off), slice + i * 1024, 16,
                                             0, 0);
        }
        const int rec = (k0 >> 2) * 256;
        uint32_t sa[MB], sb[J];
#pragma unroll
        for (int m = 0; m < MB; ++m) sa[m] = *reinterpret_cast<const uint32_t*>(asr[m] + rec);
#pragma unroll
        for (int j = 0; j < J; ++j) sb[j] = *reinterpret_cast<const uint32_t*>(bsr[j] + rec);
        mfma_v8i fa[4][MB];
#pragma unroll
        for (int st = 0; st < 4; ++st)
#pragma unroll
            for (int m = 0; m < MB; ++m)
                fa[st][m] = load_fragment<FMT>(arow[m], (k0 + st) * 128, fg, k0 + st < nk);
        auto frag = [&](int st, int j) {
            const int r = 16 * j + fr;
            const uint8_t* row = slice + r * kRowBytes;
            mfma_v8i v;
            if constexpr (FMT == 1) {
                const int p0 = 8 * st + fg, p1 = 8 * st + 4 + fg;
                const int4 lo = *reinterpret_cast<const int4*>(row + 16 * (p0 ^ (r % kPieces)));
                const int4 hi = *reinterpret_cast<const int4*>(row + 16 * (p1 ^ (r % kPieces)));
                v = (mfma_v8i){lo.x, lo.y, lo.z, lo.w, hi.x, hi.y, hi.z, hi.w};
            } else {
                const int p = 4 * st + fg;
                const int4 q = *reinterpret_cast<const int4*>(row + 16 * (p ^ (r % kPieces)));
                v = (mfma_v8i){q.x, q.y, q.z, q.w, 0, 0, 0, 0};
            }
            return v;
        };
        mfma_v8i fb[4][J];
#pragma unroll
        for (int st = 0; st < 4; ++st)
#pragma unroll
            for (int j = 0; j < J; ++j) fb[st][j] = frag(st, j);
        skinny_step<FMT, J, MB, 0>(fa[0], fb[0], acc, sa, sb);
        if (k0 + 1 < nk) skinny_step<FMT, J, MB, 1>(fa[1], fb[1], acc, sa, sb);
        if (k0 + 2 < nk) skinny_step<FMT, J, MB, 2>(fa[2], fb[2], acc, sa, sb);
        if (k0 + 3 < nk) skinny_step<FMT, J, MB, 3>(fa[3], fb[3], acc, sa, sb);
    }
#pragma unroll
    for (int m = 0; m < MB; ++m)
#pragma unroll
        for (int j = 0; j < J; ++j) {
            const int64_t col = cb + 16 * j + fr;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int64_t row = 16 * m + 4 * fg + e;
                if (row < d.c_rows && col < d.c_cols) d.c[row * d.ldc + col] = acc[m][j][e];
            }
        }
}

// One workgroup per 16 MB-row tile and 128-column tile (4 waves of J = 2
// columns of tiles).  With MB = 1, measured on the decode routing (512
// routed rows over 256 experts, N = 7168, K = 2048), MXFP4: 294 us with the
// column tile fastest; in the row-tile-fastest order 309 us, against 341 us
// for the same tiles with
// every fragment loaded straight from global memory into registers (each
// load then covers 64 bytes of each of 16 rows, so every cache line is
// requested twice), and 385 us for the 128-row kernel.  With the register
// form, other shapes and schedules measured no better: J = 1 / 4 / 8, 8
// waves, rounds of 8 or 16 K steps, a workgroup looping over several column
// tiles, non-temporal loads, and the next round's loads issued before this
// round's products (two register sets: one wave per SIMD).  With the LDS
// form, J = 1 (4 or 8 waves) took 315 us and 2 waves of J = 2 309 us.
template <int FMT, int MB>
__global__ void __launch_bounds__((64 * SkinnyShape<FMT, MB>::kWaves))
mfma_gemm_grouped_skinny_kernel(const GemmArgs a, const GroupedGemmArgs g) {
    using Sh = SkinnyShape<FMT, MB>;
    __shared__ __attribute__((aligned(16))) uint8_t stage[Sh::kStageBytes];
    GemmTile d;
    if (!grouped_desc<16 * MB, kDecodeTileCols>(a, g, d)) return;
    gemm_tile_skinny<FMT, Sh::J, MB>(d, stage);
}

// The dense GEMM with few rows (a dense layer at decode) on the same
// tiles: a 128-row tile would be mostly padding, and B, read once, is the
// bytes that matter.  Workgroup -> (row tile, column tile), row-major.  The
// grid is only N / columns workgroups wide, so the tiles are 64 columns wide
// (4 waves of one 16-column tile).  At N = 16384, K = 7168: 16-row tiles,
// M = 1 / 16, MXFP4 14.8 / 15.0 us against 18.4 / 20.9 with 128 columns (4
// waves of two), MXFP8 20.5 / 21.4 against 25.6 / 25.0; 32-row tiles,
// M = 24 / 32, MXFP4 19.4 / 19.9 us against 20.2 / 21.3 with 128 columns,
// MXFP8 30.0 / 34.1 against 33.1 / 37.2.
template <int FMT, int MB>
struct DenseSkinnyShape {
    static constexpr int J = 1;
    static constexpr int kWaves = 4;
    static constexpr int kCols = kWaves * 16 * J;
    static constexpr int kStageBytes = kWaves * 16 * J * (FMT == 1 ? 512 : 256);
};

template <int FMT, int MB>
__global__ void __launch_bounds__((64 * DenseSkinnyShape<FMT, MB>::kWaves))
mfma_gemm_skinny_kernel(const GemmArgs a, int64_t tiles_n) {
    using Sh = DenseSkinnyShape<FMT, MB>;
    __shared__ __attribute__((aligned(16))) uint8_t stage[Sh::kStageBytes];
    GemmTile d;
    dense_desc<16 * MB, Sh::kCols>(a, tiles_n, d);
    gemm_tile_skinny<FMT, Sh::J, MB>(d, stage);
}

template <int FMT, class Cfg>
hipError_t launch_tiles(const GemmArgs& a, hipStream_t stream, const LaunchEvents& ev) {
    const int64_t tiles_n = (a.N + Cfg::TN - 1) / Cfg::TN;
    const int64_t tiles = ((a.M + Cfg::TM - 1) / Cfg::TM) * tiles_n;
    return launch_kernel(mfma_gemm_tiled_kernel<FMT, Cfg>, dim3((uint32_t)tiles),
                         dim3(64 * Cfg::NW), 0, stream, ev, a, tiles_n);
}

template <int FMT, int MB>
hipError_t launch_mfma_skinny_mb(const GemmArgs& a, hipStream_t stream, const LaunchEvents& ev) {
    using Sh = DenseSkinnyShape<FMT, MB>;
    const int64_t tiles_n = (a.N + Sh::kCols - 1) / Sh::kCols;
    const int64_t tiles = ((a.M + 16 * MB - 1) / (16 * MB)) * tiles_n;
    return launch_kernel(mfma_gemm_skinny_kernel<FMT, MB>, dim3((uint32_t)tiles),
                         dim3(64 * Sh::kWaves), 0, stream, ev, a, tiles_n);
}

// Few rows (M <= 32): 16- or 32-row tiles streaming B.  Measured on
// N = 16384, K = 7168 against 128 x 128 tiles: MXFP4 15.0 / 19.9 us at
// M = 16 / 32 against 23.4 / 23.8; MXFP8 21.4 / 34.1 against 39.6 / 40.3.
// Otherwise 256 x 256 tiles (8 waves, 144 KiB of LDS in two stages, one
// workgroup per CU) once they alone fill the chip; 128 x 128 ones otherwise.
template <int FMT>
hipError_t launch_mfma_tiled(const GemmArgs& a, hipStream_t stream, const LaunchEvents& ev) {
    if (a.M <= 32)
        return a.M <= 16 ? launch_mfma_skinny_mb<FMT, 1>(a, stream, ev)
                         : launch_mfma_skinny_mb<FMT, 2>(a, stream, ev);
    const int64_t big = ((a.M + 255) / 256) * ((a.N + 255) / 256);
    if (big >= 256) return launch_tiles<FMT, Tile256>(a, stream, ev);
    return launch_tiles<FMT, Tile128>(a, stream, ev);
}

template <int FMT>
hipError_t launch_dq(const DequantArgs& a, int64_t blocks, hipStream_t stream,
                     const LaunchEvents& ev) {
    if (a.chunks_per_tile != kDequantChunks) return hipErrorInvalidValue;
    return launch_kernel(dequant_kernel<FMT, kDequantChunks>, dim3((uint32_t)blocks),
                         dim3(kThreadsPerBlock), 0, stream, ev, a);
}

template <int FMT>
hipError_t launch_mm(const GemmArgs& a, hipStream_t stream, const LaunchEvents& ev) {
    const int64_t blocks = (a.M * a.N + kThreadsPerBlock - 1) / kThreadsPerBlock;
    return launch_kernel(naive_matmul_kernel<FMT>, dim3((uint32_t)blocks),
                         dim3(kThreadsPerBlock), 0, stream, ev, a);
}

}  // namespace

hipError_t launch_dequantize(int fmt, const DequantArgs& a, int64_t blocks, hipStream_t stream,
                             const LaunchEvents& ev) {
    switch (fmt) {
        case 0: return launch_dq<0>(a, blocks, stream, ev);
        case 1: return launch_dq<1>(a, blocks, stream, ev);
        case 2: return launch_dq<2>(a, blocks, stream, ev);
        default: return hipErrorInvalidValue;
    }
}

namespace {
template <int FMT>
hipError_t launch_mfma_grouped(const GemmArgs& a, const GroupedGemmArgs& g, hipStream_t stream,
                               const LaunchEvents& ev) {
    if (g.row_blocks > 0) {
        const dim3 grid((uint32_t)(g.m_tiles * ((a.N + kDecodeTileCols - 1) / kDecodeTileCols)));
        switch (g.row_blocks) {
            case 1:
                return launch_kernel(mfma_gemm_grouped_skinny_kernel<FMT, 1>, grid,
                                     dim3(64 * SkinnyShape<FMT, 1>::kWaves), 0, stream, ev, a, g);
            case 2:
                return launch_kernel(mfma_gemm_grouped_skinny_kernel<FMT, 2>, grid,
                                     dim3(64 * SkinnyShape<FMT, 2>::kWaves), 0, stream, ev, a, g);
            default: return hipErrorInvalidValue;
        }
    }
    // one workgroup per work item, rounded up to a whole number per XCD
    const int64_t items = g.m_tiles * ((a.N + kTileN - 1) / kTileN);
    const dim3 grid((uint32_t)((items + kXcds - 1) / kXcds * kXcds));
    return launch_kernel(mfma_gemm_grouped_kernel<FMT>, grid, dim3(64 * Tile128::NW), 0, stream,
                         ev, a, g);
}
}  // namespace

hipError_t launch_mfma_grouped_matmul(int fmt, const GemmArgs& a, const GroupedGemmArgs& g,
                                      hipStream_t stream, const LaunchEvents& ev) {
    switch (fmt) {
        case 0: return launch_mfma_grouped<0>(a, g, stream, ev);
        case 1: return launch_mfma_grouped<1>(a, g, stream, ev);
        default: return hipErrorInvalidValue;
    }
}

hipError_t launch_mfma_matmul(int fmt, const GemmArgs& a, hipStream_t stream,
                              const LaunchEvents& ev) {
    switch (fmt) {
        case 0: return launch_mfma_tiled<0>(a, stream, ev);
        case 1: return launch_mfma_tiled<1>(a, stream, ev);
        default: return hipErrorInvalidValue;
    }
}

hipError_t launch_naive_matmul(int fmt, const GemmArgs& a, hipStream_t stream,
                               const LaunchEvents& ev) {
    switch (fmt) {
        case 0: return launch_mm<0>(a, stream, ev);
        case 1: return launch_mm<1>(a, stream, ev);
        case 2: return launch_mm<2>(a, stream, ev);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace bsq
