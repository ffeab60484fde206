// Internal interface between the host dispatcher (wq_api.cpp) and the kernels
// (wq_kernels.hip).  Not installed; the public interface is include/wq.h.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace wq {

// Prefetch depth (K blocks in flight per wave beyond the one being computed).
constexpr int kDepthMfmaFp8 = 2;
constexpr int kDepthMfmaLut = 2;
constexpr int kDepthGemv = 2;

enum Kind : int {
    KIND_MFMA_FP8 = 0,   // 16-row BF16 MFMA tile, FP8 block-scaled weights
    KIND_MFMA_LUT = 1,   // 16-row FP16 MFMA tile, 3-bit LUT weights
    KIND_GEMV_FP8 = 2,   // strict-K-order FP32 GEMV, M <= 4, FP8 weights
};

// Largest split (waves per work-group) a kernel may use.  A work-group runs
// on one CU, so its S waves must fit the register file: the launch bound
// 64*S caps a wave at 512/ceil(S/4) VGPRs.  The GEMV and the 4-tile MFMA
// kernels, and the 2-tile ones that stage their own activations, need more
// than 128 (S <= 8); the others fit in 128 (S <= 16).
constexpr int max_split(int kind, int nt, int sn)
{
    return (kind == KIND_GEMV_FP8 || nt >= 4 || (nt == 2 && sn == 1)) ? 8 : 16;
}

// Everything a GEMM launch needs.  The grid has one work-group per column
// group (NT tiles of 16 output columns); its S waves split the K blocks.
struct GemmArgs {
    const uint8_t* codes;     // packed code units
    const void* scales;       // FP8: float [N/128][KB]; LUT: half [n_tiles][KB][16]
    const uint16_t* qmap;     // LUT: 8 FP16 map entries (4-byte aligned)
    const uint16_t* x;        // activations [rows][ldx]
    int64_t ldx;
    uint16_t* y;              // outputs [rows][ldy]
    int64_t ldy;
    int rows;                 // 1..16 rows in this launch
    int N;                    // output columns
    int KB;                   // K / 128
    int n_tiles;              // N / 16
    int n_cg;                 // column groups = grid size
};

// nt: tiles per wave; sn: column-waves sharing activations (split % sn == 0);
// split: waves per work-group; the grid has a.n_cg = ceil(n_tiles/(nt*sn)) groups.
hipError_t launch_gemm(int kind, int nt, int sn, int gemv_rows, const GemmArgs& a, int split, hipStream_t stream);

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
