// bsq_internal.h -- launch interface between the C-ABI host layer
// (bsq_api.cpp) and the gfx950 kernels (bsq_kernels.hip).  Not installed.
#pragma once

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace bsq {

// Events a caller armed for the main kernel of its next call (both null: none).
struct LaunchEvents {
    hipEvent_t start = nullptr, stop = nullptr;
};

// Launch `kernel`; with events, through hipExtLaunchKernel, which binds them to
// the kernel's own dispatch: their elapsed time is the kernel's execution,
// without the gaps that events recorded around the launch would add.
template <typename F, typename... Args>
inline hipError_t launch_kernel(F kernel, dim3 grid, dim3 block, uint32_t lds_bytes,
                                hipStream_t stream, const LaunchEvents& ev, Args... args) {
    if (ev.start)
        hipExtLaunchKernelGGL(kernel, grid, block, lds_bytes, stream, ev.start, ev.stop, 0u,
                              args...);
    else
        hipLaunchKernelGGL(kernel, grid, block, lds_bytes, stream, args...);
    return hipGetLastError();
}

// Work is cut into tiles: up to chunks_per_tile (1, 2 or 4) consecutive
// chunks of one row, a chunk being 512 BF16 elements (64 lanes x one 16-byte
// load).  One wave converts one tile.
constexpr int kWaveSize = 64;
constexpr int kWavesPerBlock = 4;
constexpr int kThreadsPerBlock = kWaveSize * kWavesPerBlock;
constexpr int kElemsPerLane = 8;
constexpr int kChunkElems = kWaveSize * kElemsPerLane;
// Chunks per tile of the tensor-scale reduction (eight 16-byte loads per lane).
constexpr int kTsfChunks = 8;
// Largest workgroup of the tensor-scale reduction, and the most outputs it
// aggregates in an LDS table per workgroup.
constexpr int kTsfMaxThreads = 1024;
constexpr int kTsfLdsSlots = 4096;

struct KernelArgs {
    const uint16_t* x;            // BF16 source rows
    int64_t ldx;                  // elements
    uint8_t* codes;
    int64_t ldq;                  // bytes
    uint8_t* scales;
    int64_t lds;                  // bytes
    int64_t rows;                 // dense: M; grouped: max_rows (routed rows)
    int32_t K;
    int32_t chunks_per_row;       // ceil(K / 512)
    int32_t chunks_per_tile;
    int32_t tiles_per_row;
    int64_t total_tiles;          // rows * tiles_per_row (< 2^31)
    uint32_t tpr_magic_lo;        // ceil(2^64 / tiles_per_row), low and high words:
    uint32_t tpr_magic_hi;        //   t / tiles_per_row = (t * magic) >> 64 for t < 2^32
    float tensor_sf;              // dense NVFP4
    int32_t scale_layout;         // 0 row-major, 1 MFMA 16x16x128 (MX only)

    // grouped form only
    const int32_t* row_indices;   // nullable
    const uint32_t* row_offsets;  // [G + 1]
    const uint32_t* scales_offsets;
    const int32_t* expert_ids;
    const float* expert_sf;       // [num_experts] (NVFP4)
    int64_t num_src_rows;
    int64_t num_scale_rows;
    int32_t num_groups;
    int32_t num_experts;
};

// Byte offset, inside a row group's scale records, of the scale of row r
// (r % 16 is used) and 32-element block kb in the MFMA 16x16x128 layout:
// 256-byte records of 16 rows x 16 blocks; the scale of (r, kb) sits in the
// dword of lane (r % 16) + 16 (kb % 4) -- the lane the scaled matrix
// instruction takes it from for its 128-element K step -- at byte
// (kb % 16) / 4, so one dword per lane feeds four consecutive K steps.  The
// row group of r starts at (r / 16) * lds.
__host__ __device__ inline int64_t mfma16_scale_offset(int64_t r, int64_t kb) {
    return (kb / 16) * 256 + 4 * ((r % 16) + 16 * (kb % 4)) + (kb % 16) / 4;
}

// Dequantization to fp32: one wave per chunk (56.4 us against 64.2 with 2
// chunks and 72.9 with 4 for [8192, 7168] MXFP8).
constexpr int kDequantChunks = 1;

struct DequantArgs {
    const uint8_t* codes;   // [rows, ldq] bytes
    int64_t ldq;
    const uint8_t* scales;  // [rows, lds] bytes
    int64_t lds;
    float* out;             // [rows, ldo] fp32
    int64_t ldo;
    int64_t rows;
    int32_t K;
    int32_t chunks_per_row;
    int32_t chunks_per_tile;
    int32_t tiles_per_row;
    int64_t total_tiles;    // < 2^31
    uint32_t tpr_magic_lo, tpr_magic_hi;
    float tensor_sf;        // NVFP4
    int32_t scale_layout;   // as in KernelArgs
};

// Naive GEMM c = A B^T over two K-major block-scaled operands.
struct GemmArgs {
    const uint8_t* a_codes;
    int64_t lda_q;
    const uint8_t* a_scales;
    int64_t lda_s;
    float a_tsf;
    const uint8_t* b_codes;
    int64_t ldb_q;
    const uint8_t* b_scales;
    int64_t ldb_s;
    float b_tsf;
    float* c;
    int64_t ldc;
    int64_t M, N;
    int32_t K;
    int32_t scale_layout;   // as in KernelArgs
};

hipError_t launch_dequantize(int fmt, const DequantArgs& a, int64_t blocks, hipStream_t stream,
                             const LaunchEvents& ev);
hipError_t launch_naive_matmul(int fmt, const GemmArgs& a, hipStream_t stream,
                               const LaunchEvents& ev);
// MX formats, scales in the MFMA layout, K % 128 == 0, 16-byte aligned code rows.
hipError_t launch_mfma_matmul(int fmt, const GemmArgs& a, hipStream_t stream,
                              const LaunchEvents& ev);

// Grouped per-expert GEMM: A rows grouped by row_offsets (scale rows by
// scales_offsets), B = num_experts stacked [N, K] operands; GemmArgs.M unused.
// Columns of c in a tile of the grouped GEMM's decode form (its rows: 16 per
// row block).
constexpr int kDecodeTileCols = 128;
struct GroupedGemmArgs {
    const uint32_t* row_offsets;     // [num_groups + 1]
    const uint32_t* scales_offsets;  // [num_groups + 1]
    const int32_t* expert_ids;       // [num_groups]
    int32_t num_groups;
    int32_t num_experts;
    int64_t max_rows;                // rows of A codes and of c
    int64_t num_scale_rows;          // scale rows of A
    int64_t m_tiles;                 // grid bound on row tiles over all groups
    int32_t row_blocks;              // 1 or 2: tiles of 16 row_blocks rows, B streamed
                                     // through each wave's LDS (few rows per group); 0:
                                     // 128-row tiles staged through LDS
};
hipError_t launch_mfma_grouped_matmul(int fmt, const GemmArgs& a, const GroupedGemmArgs& g,
                                      hipStream_t stream, const LaunchEvents& ev);

// Launch the dense (grouped = false) or grouped kernel for format fmt
// (0 MXFP4, 1 MXFP8, 2 NVFP4).  Returns the launch status.
hipError_t launch_quantize(int fmt, bool grouped, const KernelArgs& a, int64_t blocks,
                           hipStream_t stream, const LaunchEvents& ev);

// NVFP4 tensor scale(s) into out[0 .. n_out): zero it, fold in the amax of
// every tile of a (kTsfChunks chunks per tile; blocks workgroups of
// waves_per_block waves, each wave taking tiles_per_wave consecutive tiles;
// blocks = 0 skips this pass), and turn each amax into its tensor scale.
// Events, when armed, time the amax pass.
hipError_t launch_tensor_scale(bool grouped, const KernelArgs& a, int64_t blocks,
                               int waves_per_block, uint32_t tiles_per_wave, float* out, int n_out,
                               hipStream_t stream, const LaunchEvents& ev);

}  // namespace bsq
