// bsq_api.cpp -- the C ABI of libbsq (declared in include/bsq.h): argument
// validation, launch geometry and error reporting.  Every check runs on the
// host before any HIP call, so a rejected call touches neither the device nor
// the HIP runtime.
//
// The entry points are the MI355X counterparts of the dispatcher and the
// launchers on the Modular "block_scaled_quantization" module page
// (quantize_dynamic_block_scaled, quantize_mx_amd,
// grouped_quantize_dynamic_scaled_fp4_async); format and block width replace
// the pages' compile-time output dtype and SF_VECTOR_SIZE parameter
// ("quantize_dynamic_scaled_async_fp4_kernel", Parameters).
#include <hip/hip_runtime.h>

#include <atomic>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <string>

#include "bsq.h"
#include "bsq_internal.h"

namespace {

thread_local std::string g_last_error;

// Events armed by bsq_time_next_launch for this thread's next call.
thread_local bsq::LaunchEvents g_armed;

bsq::LaunchEvents take_events() {
    const bsq::LaunchEvents e = g_armed;
    g_armed = bsq::LaunchEvents{};
    return e;
}

int fail(int status, const char* fmt, ...) {
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof(buf), fmt, ap);
    va_end(ap);
    g_last_error = buf;
    return status;
}

int ok() {
    g_last_error.clear();
    return BSQ_OK;
}

bool log_enabled() {
    static const bool on = [] {
        const char* v = std::getenv("BSQ_LOG");
        return v && v[0] && std::strcmp(v, "0") != 0;
    }();
    return on;
}

// Launch shape of the tensor-scale reduction: about this many resident
// waves per CU, in workgroups of this many waves.
constexpr int kTsfWavesPerCu = 16;
constexpr int kTsfWavesPerBlock = 16;

// Compute units of the current device, read once per device (a launch-shape
// heuristic only: a wrong count changes speed, never results).
int device_cus() {
    static std::atomic<int> cache[64];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
    int n = cache[dev].load(std::memory_order_relaxed);
    if (n > 0) return n;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
        n = 256;
    cache[dev].store(n, std::memory_order_relaxed);
    return n;
}


bool aligned(const void* p, uintptr_t n) { return (reinterpret_cast<uintptr_t>(p) % n) == 0; }

const char* fmt_name(int f) {
    return f == BSQ_MXFP4 ? "MXFP4" : f == BSQ_MXFP8 ? "MXFP8" : f == BSQ_NVFP4 ? "NVFP4" : "?";
}

int expected_block(int format) {
    switch (format) {
        case BSQ_MXFP4: return 32;
        case BSQ_MXFP8: return 32;
        case BSQ_NVFP4: return 16;
        default: return -1;
    }
}

// Checks shared by both forms.  rows is M (dense) or the source row count.
// Format, block size, layout and sizes (every entry point).
int check_layout(int format, int block_size, int scale_layout, int64_t rows, int64_t K) {
    const int bs = expected_block(format);
    if (bs < 0) return fail(BSQ_ERR_UNSUPPORTED, "unknown format %d", format);
    if (block_size != bs)
        return fail(BSQ_ERR_UNSUPPORTED, "%s uses %d-element blocks, got block_size=%d",
                    fmt_name(format), bs, block_size);
    if (scale_layout != BSQ_SCALES_ROW_MAJOR && scale_layout != BSQ_SCALES_MFMA16)
        return fail(BSQ_ERR_UNSUPPORTED, "scale layout %d is not provided", scale_layout);
    if (scale_layout == BSQ_SCALES_MFMA16 && format == BSQ_NVFP4)
        return fail(BSQ_ERR_UNSUPPORTED,
                    "the MFMA scale layout holds E8M0 scales of 32-element blocks (MX only)");
    if (rows < 0 || K < 0) return fail(BSQ_ERR_INVALID_ARG, "negative size (rows=%lld K=%lld)",
                                       (long long)rows, (long long)K);
    if (K % bs != 0)
        return fail(BSQ_ERR_INVALID_ARG, "K=%lld is not a multiple of the block size %d",
                    (long long)K, bs);
    if (K > (int64_t(1) << 30)) return fail(BSQ_ERR_INVALID_ARG, "K=%lld too large", (long long)K);
    return BSQ_OK;
}

// A codes + scales operand of K elements per row (`what` names it in errors).
// Row-major scales: lds bytes per row.  MFMA layout: lds bytes per 16-row
// group, at least one 256-byte record per 512 elements of K.
int check_operand(int format, int64_t K, const void* codes, int64_t ldq, const void* scales,
                  int64_t lds, const char* what, int scale_layout) {
    const int bs = expected_block(format);
    const int64_t code_row = (format == BSQ_MXFP8) ? K : K / 2;
    const int code_align = (format == BSQ_MXFP8) ? 8 : 4;
    if (!codes || !scales)
        return fail(BSQ_ERR_INVALID_ARG, "null pointer (%scodes=%p %sscales=%p)", what, codes,
                    what, scales);
    if (!aligned(codes, code_align))
        return fail(BSQ_ERR_INVALID_ARG, "%scodes must be %d-byte aligned for %s", what,
                    code_align, fmt_name(format));
    if (ldq < code_row || ldq % code_align != 0)
        return fail(BSQ_ERR_INVALID_ARG, "%sldq=%lld must be >= %lld and a multiple of %d", what,
                    (long long)ldq, (long long)code_row, code_align);
    if (scale_layout == BSQ_SCALES_MFMA16) {
        const int64_t need = ((K / bs + 15) / 16) * 256;
        if (lds < need || lds % 4 != 0)
            return fail(BSQ_ERR_INVALID_ARG,
                        "%slds=%lld must be >= %lld (256 bytes per 512 elements of K per 16-row "
                        "group) and a multiple of 4", what, (long long)lds, (long long)need);
        return BSQ_OK;
    }
    if (lds < K / bs)
        return fail(BSQ_ERR_INVALID_ARG, "%slds=%lld must be >= K/block_size=%lld", what,
                    (long long)lds, (long long)(K / bs));
    return BSQ_OK;
}

int check_common(int format, int block_size, int scale_layout, const void* x, int64_t rows,
                 int64_t K, int64_t ldx, const void* codes, int64_t ldq, const void* scales,
                 int64_t lds, bool has_work) {
    const int st = check_layout(format, block_size, scale_layout, rows, K);
    if (st != BSQ_OK || !has_work) return st;
    if (!x) return fail(BSQ_ERR_INVALID_ARG, "null pointer (x)");
    if (!aligned(x, 16)) return fail(BSQ_ERR_INVALID_ARG, "x must be 16-byte aligned");
    if (ldx < K || ldx % 8 != 0)
        return fail(BSQ_ERR_INVALID_ARG, "ldx=%lld must be >= K=%lld and a multiple of 8",
                    (long long)ldx, (long long)K);
    return check_operand(format, K, codes, ldq, scales, lds, "", scale_layout);
}

bool tsf_in_domain(float t) {
    // s * tsf must be a normal fp32 (or zero) for every E4M3 s, and its
    // reciprocal finite: 2^-9 * tsf >= 2^-126 and 448 * tsf < 2^127 hold on
    // [2^-117, 2^100].
    return std::isfinite(t) && t >= std::ldexp(1.0f, -117) && t <= std::ldexp(1.0f, 100);
}

// Tile geometry for a launch with u chunks per tile: fills chunks_per_row,
// chunks_per_tile, tiles_per_row, total_tiles, the tile->row magic divisor,
// and the number of 4-wave workgroups.
// Tiles of u chunks over rows x K: chunks and tiles per row, total tiles
// (< 2^31), the tile->row magic divisor, and workgroups of kWavesPerBlock.
template <typename Args>
int tile_geometry(Args& a, int u, int64_t* blocks) {
    a.chunks_per_row = (int32_t)((a.K + bsq::kChunkElems - 1) / bsq::kChunkElems);
    a.tiles_per_row = (a.chunks_per_row + u - 1) / u;
    a.total_tiles = a.rows * a.tiles_per_row;
    if (a.total_tiles > 0x7FFFFFFFLL)
        return fail(BSQ_ERR_INVALID_ARG, "problem too large for one launch (%lld tiles)",
                    (long long)a.total_tiles);
    if (a.tiles_per_row == 1) {
        a.tpr_magic_lo = a.tpr_magic_hi = 0;
    } else {  // ceil(2^64 / d) = floor((2^64 - 1) / d) + 1 for every d >= 2
        const uint64_t m = UINT64_MAX / (uint64_t)a.tiles_per_row + 1;
        a.tpr_magic_lo = (uint32_t)m;
        a.tpr_magic_hi = (uint32_t)(m >> 32);
    }
    *blocks = (a.total_tiles + bsq::kWavesPerBlock - 1) / bsq::kWavesPerBlock;
    return BSQ_OK;
}

int st_geometry(bsq::KernelArgs& a, int u, int64_t* blocks) {
    a.chunks_per_tile = u;
    return tile_geometry(a, u, blocks);
}

// Tensor-scale reduction: tiles of kTsfChunks chunks, split into contiguous
// ranges over about waves-per-CU x CUs waves, all resident at once so the
// grid has no tail of late waves.
int tsf_geometry(bsq::KernelArgs& a, int64_t* blocks, int* waves_per_block,
                 uint32_t* tiles_per_wave) {
    if (st_geometry(a, bsq::kTsfChunks, blocks) != BSQ_OK) return BSQ_ERR_INVALID_ARG;
    const int wpc = kTsfWavesPerCu;
    const int wpb = kTsfWavesPerBlock;
    const int64_t target = (int64_t)device_cus() * wpc;
    const int64_t tpw = (a.total_tiles + target - 1) / target;
    const int64_t waves = (a.total_tiles + tpw - 1) / tpw;
    *tiles_per_wave = (uint32_t)tpw;
    *waves_per_block = wpb;
    *blocks = (waves + wpb - 1) / wpb;
    if (log_enabled())
        std::fprintf(stderr, "[bsq] tensor scale rows=%lld K=%d tiles=%lld tiles/wave=%lld "
                     "waves=%lld waves/block=%d blocks=%lld\n", (long long)a.rows, a.K,
                     (long long)a.total_tiles, (long long)tpw, (long long)waves, wpb,
                     (long long)*blocks);
    return BSQ_OK;
}

// Launch geometry: one wave per tile, four waves per workgroup.  Chunks per
// tile, as measured on one box (the store policies of bsq_kernels.hip in
// place; a persistent grid walking the tiles measured slower everywhere):
//  * Dense MXFP8, large: 2 chunks (1024 elements, two 16-byte loads per
//    lane).  [8192, 7168]: 29.2 us against 29.9 with 4; earlier, with the
//    same stores, 31.0 against 35.5 with 1.
//  * Dense MXFP4 / NVFP4, large (FP4 codes stored write-through): 4 chunks.
//    [16384, 7168]: MXFP4 45.3 us against 46.0-46.3 with 2 and 46.0 with 8;
//    NVFP4 46.2-46.6 against 47.7-48.2 with 2 and 47.7 with 8.
//  * Grouped, large (more than 2^22 routed elements): 4 chunks, which also
//    amortise each wave's group search and (NVFP4) the expert's reciprocal
//    table.  16384 x 7168 prefill: NVFP4 49.5-49.8 us against 53.3-53.6 with
//    2 and 49.7-50.0 with 8; MXFP4 45.4-45.6 against 48.5 with 2 and 46.6
//    with 8; MXFP8 equal within noise at 2, 4 and 8.
//  * Small (at most 2^22 elements, latency-bound), dense or grouped: tiles of
//    1 chunk, for the most parallel waves.  Timed from a replayed HIP graph:
//    the 512 routed rows x 2048 decode gather 3.07 us against 3.10 with 2
//    chunks and 3.40 with 4; dense 128 x 4096 MXFP4 2.32 us against 2.40 and
//    2.61.
int launch(int format, bool grouped, bsq::KernelArgs& a, hipStream_t stream,
           const bsq::LaunchEvents& ev) {
    const bool small = (double)a.rows * (double)a.K <= (double)(1 << 22);
    const int u = small ? 1 : (grouped || format != BSQ_MXFP8) ? 4 : 2;
    int64_t blocks = 0;
    if (st_geometry(a, u, &blocks) != BSQ_OK) return BSQ_ERR_INVALID_ARG;
    if (log_enabled())
        std::fprintf(stderr,
                     "[bsq] %s %s rows=%lld K=%d chunks/row=%d chunks/tile=%d tiles=%lld "
                     "blocks=%lld\n",
                     grouped ? "grouped" : "dense", fmt_name(format), (long long)a.rows, a.K,
                     a.chunks_per_row, a.chunks_per_tile, (long long)a.total_tiles,
                     (long long)blocks);
    const hipError_t e = bsq::launch_quantize(format, grouped, a, blocks, stream, ev);
    if (e != hipSuccess) return fail(BSQ_ERR_HIP, "kernel launch failed: %s", hipGetErrorString(e));
    return ok();
}

}  // namespace

extern "C" {

int quantize_block_scaled(int format, int block_size, int scale_layout, const void* x,
                          int64_t M, int64_t K, int64_t ldx, void* codes, int64_t ldq,
                          void* scales, int64_t lds, float tensor_sf, void* stream) {
    const bsq::LaunchEvents ev = take_events();
    const bool work = M > 0 && K > 0;
    int st = check_common(format, block_size, scale_layout, x, M, K, ldx, codes, ldq, scales, lds,
                          work);
    if (st != BSQ_OK) return st;
    if (format == BSQ_NVFP4 && !tsf_in_domain(tensor_sf))
        return fail(BSQ_ERR_INVALID_ARG,
                    "tensor_sf=%g must be finite and within [2^-117, 2^100]", (double)tensor_sf);
    if (!work) return ok();
    bsq::KernelArgs a{};
    a.x = static_cast<const uint16_t*>(x);
    a.ldx = ldx;
    a.codes = static_cast<uint8_t*>(codes);
    a.ldq = ldq;
    a.scales = static_cast<uint8_t*>(scales);
    a.lds = lds;
    a.scale_layout = scale_layout;
    a.rows = M;
    a.K = (int32_t)K;
    a.tensor_sf = tensor_sf;
    return launch(format, false, a, static_cast<hipStream_t>(stream), ev);
}

int grouped_quantize_block_scaled(int format, int block_size, int scale_layout, const void* x,
                                  int64_t num_src_rows, int64_t K, int64_t ldx,
                                  const int32_t* row_indices, const uint32_t* row_offsets,
                                  const uint32_t* scales_offsets, const int32_t* expert_ids,
                                  const float* tensor_sf, int64_t num_groups,
                                  int64_t num_experts, int64_t max_rows, int64_t num_scale_rows,
                                  void* codes, int64_t ldq, void* scales, int64_t lds,
                                  void* stream) {
    const bsq::LaunchEvents ev = take_events();
    if (num_groups < 0 || max_rows < 0 || num_scale_rows < 0 || num_experts < 0)
        return fail(BSQ_ERR_INVALID_ARG,
                    "negative size (num_groups=%lld max_rows=%lld num_scale_rows=%lld "
                    "num_experts=%lld)",
                    (long long)num_groups, (long long)max_rows, (long long)num_scale_rows,
                    (long long)num_experts);
    const bool work = num_groups > 0 && max_rows > 0 && K > 0;
    int st = check_common(format, block_size, scale_layout, x, num_src_rows, K, ldx, codes, ldq,
                          scales, lds, work);
    if (st != BSQ_OK) return st;
    if (!work) return ok();
    // the lane-parallel search addresses the offsets with 32-bit byte offsets
    if (num_groups > (int64_t(1) << 28))
        return fail(BSQ_ERR_INVALID_ARG, "num_groups=%lld too large (at most 2^28)",
                    (long long)num_groups);
    if (max_rows > (int64_t(1) << 32))
        return fail(BSQ_ERR_INVALID_ARG, "max_rows=%lld exceeds the uint32 offset range",
                    (long long)max_rows);
    if (!row_offsets || !scales_offsets)
        return fail(BSQ_ERR_INVALID_ARG, "row_offsets and scales_offsets are required");
    if (!row_indices && max_rows > num_src_rows)
        return fail(BSQ_ERR_INVALID_ARG,
                    "without row_indices, max_rows=%lld may not exceed num_src_rows=%lld",
                    (long long)max_rows, (long long)num_src_rows);
    if (row_indices && num_src_rows == 0)
        return fail(BSQ_ERR_INVALID_ARG, "row_indices given but x has no rows");
    if (format == BSQ_NVFP4) {
        if (!expert_ids || !tensor_sf || num_experts < 1 || num_experts > 0x7FFFFFFFLL)
            return fail(BSQ_ERR_INVALID_ARG,
                        "NVFP4 needs expert_ids, a per-expert tensor_sf and num_experts >= 1");
    }
    bsq::KernelArgs a{};
    a.x = static_cast<const uint16_t*>(x);
    a.ldx = ldx;
    a.codes = static_cast<uint8_t*>(codes);
    a.ldq = ldq;
    a.scales = static_cast<uint8_t*>(scales);
    a.lds = lds;
    a.scale_layout = scale_layout;
    a.rows = max_rows;
    a.K = (int32_t)K;
    a.tensor_sf = 1.0f;
    a.row_indices = row_indices;
    a.row_offsets = row_offsets;
    a.scales_offsets = scales_offsets;
    a.expert_ids = expert_ids;
    a.expert_sf = tensor_sf;
    a.num_src_rows = num_src_rows;
    a.num_scale_rows = num_scale_rows;
    a.num_groups = (int32_t)num_groups;
    a.num_experts = (int32_t)num_experts;
    return launch(format, true, a, static_cast<hipStream_t>(stream), ev);
}

int tensor_scale_nvfp4(const void* x, int64_t M, int64_t K, int64_t ldx, float* tensor_sf_out,
                       void* stream) {
    const bsq::LaunchEvents ev = take_events();
    if (M < 0 || K < 0) return fail(BSQ_ERR_INVALID_ARG, "negative size (M=%lld K=%lld)",
                                    (long long)M, (long long)K);
    if (K % 16 != 0) return fail(BSQ_ERR_INVALID_ARG, "K=%lld is not a multiple of 16", (long long)K);
    if (K > (int64_t(1) << 30)) return fail(BSQ_ERR_INVALID_ARG, "K=%lld too large", (long long)K);
    if (!tensor_sf_out) return fail(BSQ_ERR_INVALID_ARG, "tensor_sf_out is required");
    if (!aligned(tensor_sf_out, 4)) return fail(BSQ_ERR_INVALID_ARG, "tensor_sf_out must be 4-byte aligned");
    const bool work = M > 0 && K > 0;
    if (work) {
        if (!x) return fail(BSQ_ERR_INVALID_ARG, "null x");
        if (!aligned(x, 16)) return fail(BSQ_ERR_INVALID_ARG, "x must be 16-byte aligned");
        if (ldx < K || ldx % 8 != 0)
            return fail(BSQ_ERR_INVALID_ARG, "ldx=%lld must be >= K=%lld and a multiple of 8",
                        (long long)ldx, (long long)K);
    }
    bsq::KernelArgs a{};
    a.x = static_cast<const uint16_t*>(x);
    a.ldx = ldx;
    a.rows = work ? M : 0;
    a.K = (int32_t)K;
    int64_t blocks = 0;
    uint32_t tpw = 0;
    int wpb = 0;
    if (work && tsf_geometry(a, &blocks, &wpb, &tpw) != BSQ_OK) return BSQ_ERR_INVALID_ARG;
    const hipError_t e = bsq::launch_tensor_scale(false, a, blocks, wpb, tpw, tensor_sf_out, 1,
                                                  static_cast<hipStream_t>(stream), ev);
    if (e != hipSuccess) return fail(BSQ_ERR_HIP, "kernel launch failed: %s", hipGetErrorString(e));
    return ok();
}

int grouped_tensor_scale_nvfp4(const void* x, int64_t num_src_rows, int64_t K, int64_t ldx,
                               const int32_t* row_indices, const uint32_t* row_offsets,
                               const int32_t* expert_ids, int64_t num_groups, int64_t num_experts,
                               int64_t max_rows, float* tensor_sf_out, void* stream) {
    const bsq::LaunchEvents ev = take_events();
    if (num_src_rows < 0 || K < 0 || num_groups < 0 || max_rows < 0)
        return fail(BSQ_ERR_INVALID_ARG, "negative size");
    if (num_experts < 1 || num_experts > (1 << 24))
        return fail(BSQ_ERR_INVALID_ARG, "num_experts=%lld must be in [1, 2^24]",
                    (long long)num_experts);
    if (K % 16 != 0) return fail(BSQ_ERR_INVALID_ARG, "K=%lld is not a multiple of 16", (long long)K);
    if (K > (int64_t(1) << 30)) return fail(BSQ_ERR_INVALID_ARG, "K=%lld too large", (long long)K);
    if (!tensor_sf_out || !aligned(tensor_sf_out, 4))
        return fail(BSQ_ERR_INVALID_ARG, "tensor_sf_out must be a 4-byte aligned device array");
    if (num_groups > 0x7FFFFFFFLL - 64)
        return fail(BSQ_ERR_INVALID_ARG, "num_groups=%lld too large", (long long)num_groups);
    if (max_rows > (int64_t(1) << 32))
        return fail(BSQ_ERR_INVALID_ARG, "max_rows=%lld exceeds the uint32 offset range",
                    (long long)max_rows);
    const bool work = num_groups > 0 && max_rows > 0 && K > 0;
    if (work) {
        if (!x || !row_offsets || !expert_ids)
            return fail(BSQ_ERR_INVALID_ARG, "x, row_offsets and expert_ids are required");
        if (!aligned(x, 16)) return fail(BSQ_ERR_INVALID_ARG, "x must be 16-byte aligned");
        if (ldx < K || ldx % 8 != 0)
            return fail(BSQ_ERR_INVALID_ARG, "ldx=%lld must be >= K=%lld and a multiple of 8",
                        (long long)ldx, (long long)K);
        if (!row_indices && max_rows > num_src_rows)
            return fail(BSQ_ERR_INVALID_ARG,
                        "without row_indices, max_rows=%lld may not exceed num_src_rows=%lld",
                        (long long)max_rows, (long long)num_src_rows);
        if (row_indices && num_src_rows == 0)
            return fail(BSQ_ERR_INVALID_ARG, "row_indices given but x has no rows");
    }
    bsq::KernelArgs a{};
    a.x = static_cast<const uint16_t*>(x);
    a.ldx = ldx;
    a.rows = work ? max_rows : 0;
    a.K = (int32_t)K;
    a.row_indices = row_indices;
    a.row_offsets = row_offsets;
    a.expert_ids = expert_ids;
    a.num_src_rows = num_src_rows;
    a.num_groups = (int32_t)num_groups;
    a.num_experts = (int32_t)num_experts;
    int64_t blocks = 0;
    uint32_t tpw = 0;
    int wpb = 0;
    if (work && tsf_geometry(a, &blocks, &wpb, &tpw) != BSQ_OK) return BSQ_ERR_INVALID_ARG;
    const hipError_t e = bsq::launch_tensor_scale(true, a, blocks, wpb, tpw, tensor_sf_out,
                                                  (int)num_experts,
                                                  static_cast<hipStream_t>(stream), ev);
    if (e != hipSuccess) return fail(BSQ_ERR_HIP, "kernel launch failed: %s", hipGetErrorString(e));
    return ok();
}

int dequantize_block_scaled(int format, int block_size, int scale_layout, const void* codes,
                            int64_t M, int64_t K, int64_t ldq, const void* scales, int64_t lds,
                            float tensor_sf, float* out, int64_t ldo, void* stream) {
    const bsq::LaunchEvents ev = take_events();
    int st = check_layout(format, block_size, scale_layout, M, K);
    if (st != BSQ_OK) return st;
    if (format == BSQ_NVFP4 && !tsf_in_domain(tensor_sf))
        return fail(BSQ_ERR_INVALID_ARG,
                    "tensor_sf=%g must be finite and within [2^-117, 2^100]", (double)tensor_sf);
    if (M == 0 || K == 0) return ok();
    st = check_operand(format, K, codes, ldq, scales, lds, "", scale_layout);
    if (st != BSQ_OK) return st;
    if (!out || !aligned(out, 16))
        return fail(BSQ_ERR_INVALID_ARG, "out must be a 16-byte aligned device array");
    if (ldo < K || ldo % 4 != 0)
        return fail(BSQ_ERR_INVALID_ARG, "ldo=%lld must be >= K=%lld and a multiple of 4",
                    (long long)ldo, (long long)K);
    bsq::DequantArgs a{};
    a.codes = static_cast<const uint8_t*>(codes);
    a.ldq = ldq;
    a.scales = static_cast<const uint8_t*>(scales);
    a.lds = lds;
    a.out = out;
    a.ldo = ldo;
    a.rows = M;
    a.K = (int32_t)K;
    a.tensor_sf = tensor_sf;
    a.scale_layout = scale_layout;
    int64_t blocks = 0;
    a.chunks_per_tile = bsq::kDequantChunks;
    if (tile_geometry(a, a.chunks_per_tile, &blocks) != BSQ_OK) return BSQ_ERR_INVALID_ARG;
    const hipError_t e = bsq::launch_dequantize(format, a, blocks, static_cast<hipStream_t>(stream), ev);
    if (e != hipSuccess) return fail(BSQ_ERR_HIP, "kernel launch failed: %s", hipGetErrorString(e));
    return ok();
}

int block_scaled_matmul_naive(int format, int block_size, int scale_layout,
                              const void* a_codes, int64_t lda_q, const void* a_scales,
                              int64_t lda_s, float a_tsf,
                              const void* b_codes, int64_t ldb_q, const void* b_scales,
                              int64_t ldb_s, float b_tsf,
                              int64_t M, int64_t N, int64_t K, float* c, int64_t ldc,
                              void* stream) {
    const bsq::LaunchEvents ev = take_events();
    int st = check_layout(format, block_size, scale_layout, M, K);
    if (st != BSQ_OK) return st;
    if (N < 0) return fail(BSQ_ERR_INVALID_ARG, "negative size (N=%lld)", (long long)N);
    if (format == BSQ_NVFP4 && (!tsf_in_domain(a_tsf) || !tsf_in_domain(b_tsf)))
        return fail(BSQ_ERR_INVALID_ARG,
                    "a_tsf=%g and b_tsf=%g must be finite and within [2^-117, 2^100]",
                    (double)a_tsf, (double)b_tsf);
    if (M == 0 || N == 0) return ok();
    if (M * N > (int64_t(1) << 38))
        return fail(BSQ_ERR_INVALID_ARG, "M*N=%lld too large for one launch", (long long)(M * N));
    if (K > 0) {
        st = check_operand(format, K, a_codes, lda_q, a_scales, lda_s, "a_", scale_layout);
        if (st != BSQ_OK) return st;
        st = check_operand(format, K, b_codes, ldb_q, b_scales, ldb_s, "b_", scale_layout);
        if (st != BSQ_OK) return st;
    }
    if (!c || !aligned(c, 4)) return fail(BSQ_ERR_INVALID_ARG, "c must be a 4-byte aligned device array");
    if (ldc < N) return fail(BSQ_ERR_INVALID_ARG, "ldc=%lld must be >= N=%lld", (long long)ldc,
                             (long long)N);
    bsq::GemmArgs a{};
    a.a_codes = static_cast<const uint8_t*>(a_codes);
    a.lda_q = lda_q;
    a.a_scales = static_cast<const uint8_t*>(a_scales);
    a.lda_s = lda_s;
    a.a_tsf = a_tsf;
    a.b_codes = static_cast<const uint8_t*>(b_codes);
    a.ldb_q = ldb_q;
    a.b_scales = static_cast<const uint8_t*>(b_scales);
    a.ldb_s = ldb_s;
    a.b_tsf = b_tsf;
    a.c = c;
    a.ldc = ldc;
    a.M = M;
    a.N = N;
    a.K = (int32_t)K;
    a.scale_layout = scale_layout;
    const hipError_t e = bsq::launch_naive_matmul(format, a, static_cast<hipStream_t>(stream), ev);
    if (e != hipSuccess) return fail(BSQ_ERR_HIP, "kernel launch failed: %s", hipGetErrorString(e));
    return ok();
}

int block_scaled_matmul_mfma(int format, int block_size, int scale_layout,
                             const void* a_codes, int64_t lda_q, const void* a_scales,
                             int64_t lda_s,
                             const void* b_codes, int64_t ldb_q, const void* b_scales,
                             int64_t ldb_s,
                             int64_t M, int64_t N, int64_t K, float* c, int64_t ldc,
                             void* stream) {
    const bsq::LaunchEvents ev = take_events();
    int st = check_layout(format, block_size, scale_layout, M, K);
    if (st != BSQ_OK) return st;
    if (format == BSQ_NVFP4)
        return fail(BSQ_ERR_UNSUPPORTED, "the scaled matrix instruction takes MX formats only");
    if (scale_layout != BSQ_SCALES_MFMA16)
        return fail(BSQ_ERR_UNSUPPORTED, "the MFMA GEMM reads scales in the MFMA layout only");
    if (N < 0) return fail(BSQ_ERR_INVALID_ARG, "negative size (N=%lld)", (long long)N);
    if (K % 128 != 0)
        return fail(BSQ_ERR_INVALID_ARG, "K=%lld must be a multiple of 128 (one K step)",
                    (long long)K);
    if (M == 0 || N == 0) return ok();
    if (M * N > (int64_t(1) << 38))
        return fail(BSQ_ERR_INVALID_ARG, "M*N=%lld too large for one launch", (long long)(M * N));
    if (K > 0) {
        st = check_operand(format, K, a_codes, lda_q, a_scales, lda_s, "a_", scale_layout);
        if (st != BSQ_OK) return st;
        st = check_operand(format, K, b_codes, ldb_q, b_scales, ldb_s, "b_", scale_layout);
        if (st != BSQ_OK) return st;
        if (!aligned(a_codes, 16) || !aligned(b_codes, 16) || lda_q % 16 != 0 || ldb_q % 16 != 0)
            return fail(BSQ_ERR_INVALID_ARG,
                        "code rows must be 16-byte aligned (codes and ldq multiples of 16)");
        if (!aligned(a_scales, 16) || !aligned(b_scales, 16) || lda_s % 16 != 0 ||
            ldb_s % 16 != 0)
            return fail(BSQ_ERR_INVALID_ARG,
                        "scale row groups must be 16-byte aligned (scales and lds multiples of 16)");
    }
    if (!c || !aligned(c, 4)) return fail(BSQ_ERR_INVALID_ARG, "c must be a 4-byte aligned device array");
    if (ldc < N) return fail(BSQ_ERR_INVALID_ARG, "ldc=%lld must be >= N=%lld", (long long)ldc,
                             (long long)N);
    bsq::GemmArgs a{};
    a.a_codes = static_cast<const uint8_t*>(a_codes);
    a.lda_q = lda_q;
    a.a_scales = static_cast<const uint8_t*>(a_scales);
    a.lda_s = lda_s;
    a.b_codes = static_cast<const uint8_t*>(b_codes);
    a.ldb_q = ldb_q;
    a.b_scales = static_cast<const uint8_t*>(b_scales);
    a.ldb_s = ldb_s;
    a.c = c;
    a.ldc = ldc;
    a.M = M;
    a.N = N;
    a.K = (int32_t)K;
    a.scale_layout = scale_layout;
    const hipError_t e = bsq::launch_mfma_matmul(format, a, static_cast<hipStream_t>(stream), ev);
    if (e != hipSuccess) return fail(BSQ_ERR_HIP, "kernel launch failed: %s", hipGetErrorString(e));
    return ok();
}

int grouped_block_scaled_matmul_mfma(int format, int block_size, int scale_layout,
                                     const void* a_codes, int64_t lda_q, const void* a_scales,
                                     int64_t lda_s,
                                     const uint32_t* row_offsets, const uint32_t* scales_offsets,
                                     const int32_t* expert_ids, int64_t num_groups,
                                     int64_t max_rows, int64_t num_scale_rows,
                                     const void* b_codes, int64_t ldb_q, const void* b_scales,
                                     int64_t ldb_s, int64_t num_experts,
                                     int64_t N, int64_t K, float* c, int64_t ldc, void* stream) {
    const bsq::LaunchEvents ev = take_events();
    int st = check_layout(format, block_size, scale_layout, max_rows, K);
    if (st != BSQ_OK) return st;
    if (format == BSQ_NVFP4)
        return fail(BSQ_ERR_UNSUPPORTED, "the scaled matrix instruction takes MX formats only");
    if (scale_layout != BSQ_SCALES_MFMA16)
        return fail(BSQ_ERR_UNSUPPORTED, "the MFMA GEMM reads scales in the MFMA layout only");
    if (N < 0 || num_groups < 0 || num_scale_rows < 0)
        return fail(BSQ_ERR_INVALID_ARG, "negative size");
    if (num_experts < 1 || num_experts > (1 << 24))
        return fail(BSQ_ERR_INVALID_ARG, "num_experts=%lld must be in [1, 2^24]",
                    (long long)num_experts);
    if (num_groups > (1 << 24))
        return fail(BSQ_ERR_INVALID_ARG, "num_groups=%lld too large", (long long)num_groups);
    if (max_rows > (int64_t(1) << 32))
        return fail(BSQ_ERR_INVALID_ARG, "max_rows=%lld exceeds the uint32 offset range",
                    (long long)max_rows);
    if (K % 128 != 0)
        return fail(BSQ_ERR_INVALID_ARG, "K=%lld must be a multiple of 128 (one K step)",
                    (long long)K);
    if (num_groups == 0 || max_rows == 0 || N == 0) return ok();
    if (!row_offsets || !scales_offsets || !expert_ids)
        return fail(BSQ_ERR_INVALID_ARG, "row_offsets, scales_offsets and expert_ids are required");
    if (K > 0) {
        st = check_operand(format, K, a_codes, lda_q, a_scales, lda_s, "a_", scale_layout);
        if (st != BSQ_OK) return st;
        st = check_operand(format, K, b_codes, ldb_q, b_scales, ldb_s, "b_", scale_layout);
        if (st != BSQ_OK) return st;
        if (!aligned(a_codes, 16) || !aligned(b_codes, 16) || lda_q % 16 != 0 || ldb_q % 16 != 0)
            return fail(BSQ_ERR_INVALID_ARG,
                        "code rows must be 16-byte aligned (codes and ldq multiples of 16)");
        if (!aligned(a_scales, 16) || !aligned(b_scales, 16) || lda_s % 16 != 0 ||
            ldb_s % 16 != 0)
            return fail(BSQ_ERR_INVALID_ARG,
                        "scale row groups must be 16-byte aligned (scales and lds multiples of 16)");
    }
    if (!c || !aligned(c, 4)) return fail(BSQ_ERR_INVALID_ARG, "c must be a 4-byte aligned device array");
    if (ldc < N) return fail(BSQ_ERR_INVALID_ARG, "ldc=%lld must be >= N=%lld", (long long)ldc,
                             (long long)N);
    bsq::GroupedGemmArgs g{};
    g.row_offsets = row_offsets;
    g.scales_offsets = scales_offsets;
    g.expert_ids = expert_ids;
    g.num_groups = (int32_t)num_groups;
    g.num_experts = (int32_t)num_experts;
    g.max_rows = max_rows;
    g.num_scale_rows = num_scale_rows;
    // Rows per tile from the rows per group on average (max_rows / num_groups;
    // the offsets stay on the device).  Few rows per group, as in a decode
    // step, take 16- or 32-row tiles with the weights streamed through each
    // wave's LDS; more take 128-row tiles staged through LDS.  Measured on 256
    // experts, N = 512, K = 7168 (MXFP4), 16 / 32 / 64 / 128-row tiles: at 4
    // rows per expert 90 / 92 / 106 / 117 us; at 8, 103 / 97 / 114 / 108; at
    // 16, 125 / 108 / 117 / 119; at 32, 190 / 155 / 148 / 124; at 64, 339 /
    // 229 / 224 / 130.
    const int tile_m = max_rows <= 4 * num_groups ? 16 : max_rows <= 16 * num_groups ? 32 : 128;
    g.row_blocks = tile_m < 128 ? tile_m / 16 : 0;
    const int64_t tile_n = g.row_blocks ? bsq::kDecodeTileCols : 128;
    g.m_tiles = (max_rows + tile_m - 1) / tile_m + num_groups;  // each group adds at most one
                                                                // partial tile
    // both forms take one workgroup per (row tile, column tile), in one dimension
    if (g.m_tiles > 0x7FFFFFFFLL || g.m_tiles * ((N + tile_n - 1) / tile_n) > 0x7FFFFFF0LL)
        return fail(BSQ_ERR_INVALID_ARG, "problem too large for one launch");
    bsq::GemmArgs a{};
    a.a_codes = static_cast<const uint8_t*>(a_codes);
    a.lda_q = lda_q;
    a.a_scales = static_cast<const uint8_t*>(a_scales);
    a.lda_s = lda_s;
    a.b_codes = static_cast<const uint8_t*>(b_codes);
    a.ldb_q = ldb_q;
    a.b_scales = static_cast<const uint8_t*>(b_scales);
    a.ldb_s = ldb_s;
    a.c = c;
    a.ldc = ldc;
    a.M = max_rows;
    a.N = N;
    a.K = (int32_t)K;
    a.scale_layout = scale_layout;
    const hipError_t e = bsq::launch_mfma_grouped_matmul(format, a, g,
                                                         static_cast<hipStream_t>(stream), ev);
    if (e != hipSuccess) return fail(BSQ_ERR_HIP, "kernel launch failed: %s", hipGetErrorString(e));
    return ok();
}

int bsq_time_next_launch(void* start_event, void* stop_event) {
    if ((start_event == nullptr) != (stop_event == nullptr)) {
        g_armed = bsq::LaunchEvents{};
        return fail(BSQ_ERR_INVALID_ARG, "start_event and stop_event must both be given, or neither");
    }
    g_armed.start = static_cast<hipEvent_t>(start_event);
    g_armed.stop = static_cast<hipEvent_t>(stop_event);
    return ok();
}

const char* bsq_last_error(void) { return g_last_error.c_str(); }

const char* bsq_version(void) { return "1.0.0"; }

}  // extern "C"
