// Internal interface between the host dispatcher (wq_api.cpp) and the kernels
// (wq_kernels.hip).  Not installed; the public interface is include/wq.h.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace wq {

constexpr int kWavesPerWG = 4;            // work-group = 4 wave64 = 256 lanes
constexpr int kThreadsPerWG = kWavesPerWG * 64;

enum Kind : int {
    KIND_MFMA_FP8 = 0,   // 16-row BF16 MFMA tile, FP8 block-scaled weights
    KIND_MFMA_LUT = 1,   // 16-row FP16 MFMA tile, 3-bit LUT weights
    KIND_GEMV_FP8 = 2,   // strict-K-order FP32 GEMV, M <= 4, FP8 weights
};

// Everything a GEMM launch needs.  A "unit" is one column group (NT tiles of
// 16 output columns) times one 128-wide K block; the U = n_cg * KB units are
// split into G contiguous, near-equal ranges, one per persistent work-group.
struct GemmArgs {
    const uint8_t* codes;     // packed code units
    const void* scales;       // FP8: float [N/128][KB]; LUT: half [n_tiles][KB][16]
    const uint16_t* qmap;     // LUT: 8 FP16 map entries (16-byte aligned)
    const uint16_t* x;        // activations [rows][ldx]
    int64_t ldx;
    uint16_t* y;              // outputs [rows][ldy]
    int64_t ldy;
    int rows;                 // 1..16 rows in this launch
    int N;                    // output columns
    int KB;                   // K / 128
    int n_tiles;              // N / 16
    int n_cg;                 // column groups = ceil(n_tiles / NT)
    int G;                    // work-groups in the grid
    int64_t U;                // units = n_cg * KB
    float* partials;          // workspace: [G][2][16 * 16 * NT] FP32 partial tiles
    uint32_t* counters;       // workspace: [n_cg] arrival counters (kept at zero)
};

hipError_t launch_gemm(int kind, int nt, int gemv_rows, const GemmArgs& a, size_t lds_bytes,
                       hipStream_t stream);

hipError_t launch_pack_fp8(const uint8_t* w, int64_t ldw, const float* scales, int64_t N,
                           int64_t K, uint8_t* packed, hipStream_t stream);
hipError_t launch_pack_lut3(const uint8_t* codes, int64_t ldc, const uint16_t* qmap,
                            const uint16_t* scales, int64_t N, int64_t K, uint8_t* packed,
                            uint32_t* status, hipStream_t stream);
hipError_t launch_unpack_fp8(const uint8_t* packed, int64_t N, int64_t K, void* out,
                             bool f32_out, hipStream_t stream);
hipError_t launch_unpack_lut3(const uint8_t* packed, int64_t N, int64_t K, uint16_t* out,
                              hipStream_t stream);

}  // namespace wq
