// bsq_ceiling.hip -- trivial streams with the memory traffic of a dense
// quantizer launch and of a dequantizer launch, built into their own library
// (libbsq_ceiling.so) for measurement only.
//
// The dequantizer's stream (expand_kernel) is described above it.
// It reads a BF16 [M, K] matrix and writes codes and block-scale bytes exactly
// as quantize_kernel does -- the same tiles of U chunks of 512 elements per
// wave, four waves per workgroup, the same non-temporal 16-byte loads, the
// same code and scale store instructions and cache policies -- but computes
// nothing: a lane's codes are an XOR fold of the words it loaded and its
// scale byte is the low byte of its first loaded word.  Its time on a given
// problem is the bandwidth that byte mix reaches with the quantizer's own
// instruction shape on this chip, which is below the 8 TB/s peak (a stream
// with wider stores can do better for the FP4 mixes).
//
// What it writes, for chunk c of row r and lane l (elements 512 c + 8 l ..
// 512 c + 8 l + 7, loaded as words w0..w3):
//   FP4 (2 codes per byte): bytes 256 c + 4 l .. + 3 of codes row r = w0^w1^w2^w3;
//   FP8: bytes 512 c + 8 l .. + 3 = w0 ^ w1, + 4 .. + 7 = w2 ^ w3;
//   scale byte of block b of the chunk (lanes L b .. L b + L - 1, L = 4 for
//   32-element blocks and 2 for 16) = low byte of w0 of lane L b + j, with
//   j = c mod min(U, L) (the lane of the block that stores it).
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "bsq_ceiling.h"
#include "bsq_internal.h"

namespace {

using bsq::kChunkElems;
using bsq::kElemsPerLane;
using bsq::kThreadsPerBlock;
using bsq::kWaveSize;
using bsq::kWavesPerBlock;

typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2_t __attribute__((ext_vector_type(2)));
constexpr int kBufferWord3 = 0x00020000;
constexpr int kStoreStream = 2;         // nt
constexpr int kStoreWriteThrough = 16;  // sc1

struct CeilingArgs {
    const uint16_t* x;
    uint8_t* codes;
    uint8_t* scales;
    int32_t K;
    int32_t chunks_per_row;
    int32_t tiles_per_row;
    int64_t total_tiles;
};

// FP4: 4 code bytes per lane; FP8: 8.  L lanes per block.
template <bool FP4, int L, int U>
__global__ void __launch_bounds__(kThreadsPerBlock) ceiling_kernel(const CeilingArgs a) {
    const int lane = (int)(threadIdx.x & (kWaveSize - 1));
    const uint32_t t = __builtin_amdgcn_readfirstlane(blockIdx.x * kWavesPerBlock +
                                                      (threadIdx.x / kWaveSize));
    if (t >= (uint32_t)a.total_tiles) return;
    const uint32_t row = t / (uint32_t)a.tiles_per_row;
    const int c0 = (int)(t - row * (uint32_t)a.tiles_per_row) * U;
    const int nch = min(U, a.chunks_per_row - c0);
    const uint16_t* xrow = a.x + (int64_t)row * a.K;
    u32x4_t w[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
        w[u] = (u32x4_t){0u, 0u, 0u, 0u};
        if (u < nch)
            w[u] = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(
                xrow + (c0 + u) * kChunkElems + lane * kElemsPerLane));
    }
    constexpr int kBlock = L * kElemsPerLane;
    const int code_bytes = FP4 ? a.K / 2 : a.K;
    const int scale_bytes = a.K / kBlock;
    const __amdgpu_buffer_rsrc_t qr = __builtin_amdgcn_make_buffer_rsrc(
        a.codes + (int64_t)row * code_bytes, (short)0, code_bytes, kBufferWord3);
    const __amdgpu_buffer_rsrc_t sr = __builtin_amdgcn_make_buffer_rsrc(
        a.scales + (int64_t)row * scale_bytes, (short)0, scale_bytes, kBufferWord3);
    constexpr int kPolicy = (FP4 && U > 1) ? kStoreWriteThrough : kStoreStream;
#pragma unroll
    for (int u = 0; u < U; ++u) {
        if (u >= nch) continue;
        const int col = (c0 + u) * kChunkElems + lane * kElemsPerLane;
        if constexpr (FP4) {
            __builtin_amdgcn_raw_buffer_store_b32(w[u].x ^ w[u].y ^ w[u].z ^ w[u].w, qr, col / 2, 0,
                                                  kPolicy);
        } else {
            const u32x2_t v = {w[u].x ^ w[u].y, w[u].z ^ w[u].w};
            __builtin_amdgcn_raw_buffer_store_b64(v, qr, col, 0, kPolicy);
        }
    }
    // one byte-store instruction per L chunks: lane L b + j stores chunk g + j's byte
#pragma unroll
    for (int g = 0; g < U; g += L) {
        const int j = lane & (L - 1);
        const int u = g + j;
        uint32_t v = w[g].x;
#pragma unroll
        for (int k = 1; k < L && g + k < U; ++k) v = (j == k) ? w[g + k].x : v;
        const int col = (c0 + u) * kChunkElems + (lane - j) * kElemsPerLane;
        if (u < nch && u < U)
            __builtin_amdgcn_raw_buffer_store_b8((uint8_t)v, sr, col / kBlock, 0, kPolicy);
    }
}

struct ExpandArgs {
    const uint8_t* codes;
    const uint8_t* scales;
    float* out;
    int32_t K;
    int32_t chunks_per_row;
    int32_t tiles_per_row;
    int64_t total_tiles;
};

// The dequantizer's traffic with its tiles (U chunks of 512 elements of one
// row per wave), loads and stores: per lane and chunk the code word(s) with a
// non-temporal load (4 bytes FP4, 8 bytes FP8) and the block's scale byte with
// an ordinary one, all issued first; then 8 words out with two ordinary
// 16-byte stores.  Word j of lane l's 8 is (j < 4 ? q0 : q1) ^ s, with q0, q1
// the code words (q1 = 0 for FP4) and s the scale byte: nothing is decoded.
template <bool FP4, int BLOCK, int U>
__global__ void __launch_bounds__(kThreadsPerBlock) expand_kernel(const ExpandArgs a) {
    typedef float f32x4_t __attribute__((ext_vector_type(4)));
    const int lane = (int)(threadIdx.x & (kWaveSize - 1));
    const uint32_t t = __builtin_amdgcn_readfirstlane(blockIdx.x * kWavesPerBlock +
                                                      (threadIdx.x / kWaveSize));
    if (t >= (uint32_t)a.total_tiles) return;
    const uint32_t row = t / (uint32_t)a.tiles_per_row;
    const int c0 = (int)(t - row * (uint32_t)a.tiles_per_row) * U;
    const int nch = min(U, a.chunks_per_row - c0);
    const uint8_t* crow = a.codes + (int64_t)row * (FP4 ? a.K / 2 : a.K);
    const uint8_t* srow = a.scales + (int64_t)row * (a.K / BLOCK);
    float* orow = a.out + (int64_t)row * a.K;
    uint32_t q0[U], q1[U], sb[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
        q0[u] = q1[u] = sb[u] = 0u;
        if (u < nch) {
            const int col = (c0 + u) * kChunkElems + lane * kElemsPerLane;
            if constexpr (FP4) {
                q0[u] = __builtin_nontemporal_load(reinterpret_cast<const uint32_t*>(crow + col / 2));
            } else {
                const u32x2_t v = __builtin_nontemporal_load(
                    reinterpret_cast<const u32x2_t*>(crow + col));
                q0[u] = v.x;
                q1[u] = v.y;
            }
            sb[u] = srow[col / BLOCK];
        }
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
        if (u >= nch) continue;
        const int col = (c0 + u) * kChunkElems + lane * kElemsPerLane;
        const float lo = __uint_as_float(q0[u] ^ sb[u]), hi = __uint_as_float(q1[u] ^ sb[u]);
        f32x4_t* o = reinterpret_cast<f32x4_t*>(orow + col);
        o[0] = (f32x4_t){lo, lo, lo, lo};
        o[1] = (f32x4_t){hi, hi, hi, hi};
    }
}

template <bool FP4, int BLOCK>
hipError_t launch_expand_u(const ExpandArgs& a, int u, int64_t blocks, hipStream_t stream,
                           const bsq::LaunchEvents& ev) {
    switch (u) {
        case 1: return bsq::launch_kernel(expand_kernel<FP4, BLOCK, 1>, dim3((uint32_t)blocks),
                                          dim3(kThreadsPerBlock), 0, stream, ev, a);
        case 2: return bsq::launch_kernel(expand_kernel<FP4, BLOCK, 2>, dim3((uint32_t)blocks),
                                          dim3(kThreadsPerBlock), 0, stream, ev, a);
        case 4: return bsq::launch_kernel(expand_kernel<FP4, BLOCK, 4>, dim3((uint32_t)blocks),
                                          dim3(kThreadsPerBlock), 0, stream, ev, a);
        default: return hipErrorInvalidValue;
    }
}

template <bool FP4, int L>
hipError_t launch_u(const CeilingArgs& a, int u, int64_t blocks, hipStream_t stream,
                    const bsq::LaunchEvents& ev) {
    switch (u) {
        case 1: return bsq::launch_kernel(ceiling_kernel<FP4, L, 1>, dim3((uint32_t)blocks),
                                          dim3(kThreadsPerBlock), 0, stream, ev, a);
        case 2: return bsq::launch_kernel(ceiling_kernel<FP4, L, 2>, dim3((uint32_t)blocks),
                                          dim3(kThreadsPerBlock), 0, stream, ev, a);
        case 4: return bsq::launch_kernel(ceiling_kernel<FP4, L, 4>, dim3((uint32_t)blocks),
                                          dim3(kThreadsPerBlock), 0, stream, ev, a);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace

extern "C" int bsq_ceiling_stream(int format, const void* x, int64_t M, int64_t K, void* codes,
                                  void* scales, int chunks_per_wave, void* start_event,
                                  void* stop_event, void* stream) {
    if (format < 0 || format > 2 || M < 0 || K < 0 || K % kChunkElems != 0 ||
        K > (int64_t(1) << 30) || (chunks_per_wave != 1 && chunks_per_wave != 2 &&
                                   chunks_per_wave != 4) ||
        ((start_event == nullptr) != (stop_event == nullptr)))
        return 1;
    if (M == 0 || K == 0) return 0;
    if (!x || !codes || !scales || (reinterpret_cast<uintptr_t>(x) & 15) ||
        (reinterpret_cast<uintptr_t>(codes) & 7))
        return 1;
    CeilingArgs a{};
    a.x = static_cast<const uint16_t*>(x);
    a.codes = static_cast<uint8_t*>(codes);
    a.scales = static_cast<uint8_t*>(scales);
    a.K = (int32_t)K;
    a.chunks_per_row = (int32_t)(K / kChunkElems);
    a.tiles_per_row = (a.chunks_per_row + chunks_per_wave - 1) / chunks_per_wave;
    a.total_tiles = M * a.tiles_per_row;
    if (a.total_tiles > 0x7FFFFFFFLL) return 1;
    const int64_t blocks = (a.total_tiles + kWavesPerBlock - 1) / kWavesPerBlock;
    const bsq::LaunchEvents ev{static_cast<hipEvent_t>(start_event),
                               static_cast<hipEvent_t>(stop_event)};
    const hipStream_t s = static_cast<hipStream_t>(stream);
    hipError_t e;
    switch (format) {
        case 0: e = launch_u<true, 4>(a, chunks_per_wave, blocks, s, ev); break;
        case 1: e = launch_u<false, 4>(a, chunks_per_wave, blocks, s, ev); break;
        default: e = launch_u<true, 2>(a, chunks_per_wave, blocks, s, ev); break;
    }
    return e == hipSuccess ? 0 : 3;
}

extern "C" int bsq_ceiling_expand(int format, const void* codes, const void* scales, int64_t M,
                                  int64_t K, void* out, int chunks_per_wave, void* start_event,
                                  void* stop_event, void* stream) {
    if (format < 0 || format > 2 || M < 0 || K < 0 || K % kChunkElems != 0 ||
        K > (int64_t(1) << 30) || (chunks_per_wave != 1 && chunks_per_wave != 2 &&
                                   chunks_per_wave != 4) ||
        ((start_event == nullptr) != (stop_event == nullptr)))
        return 1;
    if (M == 0 || K == 0) return 0;
    if (!codes || !scales || !out || (reinterpret_cast<uintptr_t>(codes) & 7) ||
        (reinterpret_cast<uintptr_t>(out) & 15))
        return 1;
    ExpandArgs a{};
    a.codes = static_cast<const uint8_t*>(codes);
    a.scales = static_cast<const uint8_t*>(scales);
    a.out = static_cast<float*>(out);
    a.K = (int32_t)K;
    a.chunks_per_row = (int32_t)(K / kChunkElems);
    a.tiles_per_row = (a.chunks_per_row + chunks_per_wave - 1) / chunks_per_wave;
    a.total_tiles = M * a.tiles_per_row;
    if (a.total_tiles > 0x7FFFFFFFLL) return 1;
    const int64_t blocks = (a.total_tiles + kWavesPerBlock - 1) / kWavesPerBlock;
    const bsq::LaunchEvents ev{static_cast<hipEvent_t>(start_event),
                               static_cast<hipEvent_t>(stop_event)};
    const hipStream_t s = static_cast<hipStream_t>(stream);
    hipError_t e;
    switch (format) {
        case 0: e = launch_expand_u<true, 32>(a, chunks_per_wave, blocks, s, ev); break;
        case 1: e = launch_expand_u<false, 32>(a, chunks_per_wave, blocks, s, ev); break;
        default: e = launch_expand_u<true, 16>(a, chunks_per_wave, blocks, s, ev); break;
    }
    return e == hipSuccess ? 0 : 3;
}
