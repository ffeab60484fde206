// Internal interface between the host dispatcher (wq_api.cpp) and the kernels
// (wq_kernels.hip).  Not installed; the public interface is include/wq.h.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace wq {

// Prefetch depth: weight units in flight per wave beyond the one being
// computed (the register ring has depth + 1 slots).  FP8 16-row tile: 4 where
// each wave streams its K range alone (one K group per work-group: gate/up
// 17.45 -> 17.24 us, FFN down in 4 parts 19.61 -> 19.56; at 5 and 6 units
// gate/up 17.31 / 17.37 and down 19.54 / 19.86 against 17.15 / 19.38), 3 where K groups
// split it (attention output 9.84 us at 3, 10.01 at 4, 10.20 at 5).  GEMV
// and 32-row tiles: 3.  LUT tile with the quad schedule, 28672 x 8192, M = 16
// (medians of 15 interleaved windows of 200 graph-replayed calls): one-tile
// waves at 4 units, nibbles 24.0 us against 24.5 at 5, 25.0 at 6 and ~24.9
// at 3, dense codes 23.2 us against 23.5 at 3 and 24.5 at 2; two-tile waves
// keep 3 (at 4 their 16-piece kernel spills).
constexpr int kDepthMfmaFp8 = 3;
constexpr int kDepthMfmaFp8Solo = 4;   // one K group per work-group
constexpr int kDepthGemv = 3;
constexpr int lut_depth(int nt) { return nt == 1 ? 4 : 3; }

enum Kind : int {
    KIND_MFMA_FP8 = 0,   // 16-row BF16 MFMA tile, FP8 block-scaled weights
    KIND_MFMA_LUT = 1,   // 16-row FP16 MFMA tile, 3-bit LUT weights
    KIND_GEMV_FP8 = 2,   // strict-K-order FP32 GEMV, M <= 4, FP8 weights, one tile per wave
    KIND_MFMA_LUT3D = 3, // 16-row FP16 MFMA tile, 3-bit LUT weights stored densely (3 bits a code)
    KIND_W8A8_STREAM = 4, // W8A8 product on the weight-streaming tile (M <= 64): FP8 weights through
                          // the register ring, packed FP8 activations and their scales staged in LDS
};

constexpr bool is_lut_kind(int kind) { return kind == KIND_MFMA_LUT || kind == KIND_MFMA_LUT3D; }

// K ranges of K groups and K parts start at multiples of this many K blocks:
// a LUT wave loads a row's group scales for 8 K blocks at once.
constexpr int k_align(int kind) { return is_lut_kind(kind) ? 8 : 1; }

// Size of an activation chunk (the K group synchronises once per chunk) in
// 16-row K blocks, per kernel kind and row tiles MT.  Measured on MI355X: the
// FP8 MFMA tile runs best with two K blocks per chunk at any M -- 6-15%
// faster than four at M <= 16 for the low-N projections, while one 32-row
// block per chunk costs 8-19% at M = 32.  The LUT tile's chunk is one quad of
// four K blocks at any M (its lane groups read four blocks at once); the GEMV
// stages four 4-row blocks.
constexpr int chunk_blocks16(int kind, int mt)
{
    return kind == KIND_MFMA_FP8 || kind == KIND_W8A8_STREAM ? 2 * mt : is_lut_kind(kind) ? 4 * mt : 4;
}

// LDS bytes of one staged activation chunk (16-row blocks, rows padded to 272 bytes)
constexpr int chunk_lds_bytes(int kind, int mt) { return chunk_blocks16(kind, mt) * 16 * (128 * 2 + 16); }

// Each K group of an MFMA work-group double-buffers one activation chunk in
// LDS; at M <= 16 that is at most 2 x 4 K blocks x 16 rows x 272 bytes =
// 34816 bytes, so the 160 KiB of LDS of a compute unit bound the K groups of
// one work-group at 4.
constexpr int kMaxKGroups = 4;
constexpr int kLdsBytes = 160 * 1024;

// Most K parts a GEMM splits across work-groups (grid y).
constexpr int kMaxKParts = 32;

// 16-byte activation pieces each lane loads per chunk when SN column-waves
// share it: ceil(chunk pieces / (64 * SN)); a chunk is chunk_blocks16 blocks
// x 16 rows x 16 pieces for the BF16/FP16 MFMA tiles, x 4 rows x 16 pieces for
// the GEMV, and x one 2 KiB FP8 unit (128 pieces) for the W8A8 streaming tile
// (whose activation scales are loaded apart).
constexpr int x_pieces_per_lane(int kind, int sn, int mt = 1)
{
    const int per_block = kind == KIND_GEMV_FP8 ? 4 * 16 : kind == KIND_W8A8_STREAM ? 128 : 16 * 16;
    const int pieces = chunk_blocks16(kind, mt) * per_block;
    return (pieces + 64 * sn - 1) / (64 * sn);
}

// Largest split (waves per work-group).  A work-group runs on one CU, and a
// launch bound of 64*S waves caps a wave at 512/ceil(S/4) VGPRs.  Most
// kernels are built for work-groups of at most 8 waves, which lets a wave
// hold up to 256 VGPRs: the register ring, the activation pieces in flight
// and the unrolled MFMA steps of a chunk need more than 128.  One-tile LUT
// waves with at most 5 activation pieces per lane (5 only occurs for 32-row
// chunks shared by 7 column-waves) fit in 128 and are built for up to 16
// waves, so a work-group can split K across more waves than it has SIMDs.
constexpr int max_split_xpl(int kind, int nt, int xpl)
{
    return ((is_lut_kind(kind) && nt == 1 && xpl <= 5) || kind == KIND_GEMV_FP8) ? 16 : 8;
}
constexpr int max_split(int kind, int nt, int sn) { return max_split_xpl(kind, nt, x_pieces_per_lane(kind, sn)); }

// Whether a one-tile LUT tiling also runs M = 17..32 in one pass (both
// 16-row halves share each dequantised operand).  Its 32-row quad chunks take
// twice the LDS and activation pieces of the 16-row ones: the pieces per lane
// must be a built count (4, 5, 6 or 8) within the work-group's launch bound and
// the double-buffered chunks of its K groups must fit in LDS.  Otherwise the
// host runs rows 0..15 and 16..M-1 as two passes.
constexpr bool lut_single_pass(int kind, int sn, int split)
{
    if (!is_lut_kind(kind) || sn < 1 || split < sn) return false;
    const int xpl = x_pieces_per_lane(kind, sn, 2);
    return (xpl == 4 || xpl == 5 || xpl == 6 || xpl == 8) && split <= max_split_xpl(kind, 1, xpl) &&
           (split / sn) * 2 * chunk_lds_bytes(kind, 2) <= kLdsBytes;
}

// Whether (nt, sn, split) is a launchable tiling for this kernel kind.
constexpr bool split_ok(int kind, int nt, int sn, int split)
{
    if (sn < 1 || split < 1 || split % sn || split > max_split(kind, nt, sn)) return false;
    if (sn > 8 || split / sn > kMaxKGroups) return false;
    if (kind == KIND_GEMV_FP8 || kind == KIND_W8A8_STREAM) return nt == 1;
    return nt == 1 || nt == 2;
}

// Everything a GEMM launch needs.  The grid has one work-group per column
// group (NT tiles of 16 output columns); its S waves split the K blocks.
struct GemmArgs {
    const uint8_t* codes;     // packed code units
    const void* scales;       // FP8: float [N/128][KB]; LUT: half [n_tiles][KB/8][16][8]
    const uint16_t* qmap;     // LUT: 8 FP16 map entries (4-byte aligned)
    const uint16_t* x;        // activations [rows][ldx]; W8A8 streaming tile: the packed FP8 activations
    int64_t ldx;              //   (units, then scales) and ldx = their padded row count
    uint16_t* y;              // outputs [rows][ldy]
    int64_t ldy;
    int rows;                 // rows in this launch: 1..16, or 17..32 (one-tile MFMA waves)
    int N;                    // output columns
    int KB;                   // K / 128
    int n_tiles;              // N / 16
    int n_cg;                 // column groups (grid x)
    int sn;                   // column-waves per work-group sharing activations
    int kp;                   // K parts across work-groups (grid y); > 1: partials go to ws
    float* ws;                // kp > 1: FP32 partial outputs [kp][rows][N]
};

// nt: tiles per wave; a.sn: column-waves sharing activations (split % sn == 0);
// split: waves per work-group; the grid has a.n_cg = ceil(n_tiles/(nt*sn))
// column groups times a.kp K parts.  With a.kp > 1 the GEMM writes FP32
// partials to a.ws and a second kernel sums the parts in order into y.
hipError_t launch_gemm(int kind, int nt, int gemv_rows, const GemmArgs& a, int split, hipStream_t stream);

hipError_t launch_pack_fp8(const uint8_t* w, int64_t ldw, const float* scales, int64_t N,
                           int64_t K, uint8_t* packed, hipStream_t stream);
// dense: the 3-bit-per-code layout (N*K*3/8 code bytes) instead of nibbles
hipError_t launch_pack_lut3(const uint8_t* codes, int64_t ldc, const uint16_t* qmap,
                            const uint16_t* scales, int64_t N, int64_t K, uint8_t* packed,
                            uint32_t* status, bool dense, hipStream_t stream);
hipError_t launch_unpack_fp8(const uint8_t* packed, int64_t N, int64_t K, void* out,
                             bool f32_out, hipStream_t stream);
hipError_t launch_unpack_lut3(const uint8_t* packed, int64_t N, int64_t K, uint16_t* out,
                              bool dense, hipStream_t stream);

// W8A8 tier (wq_w8a8.hip): activation quantiser into the packed activation
// layout, its test-hook inverse, and the FP8 x FP8 GEMM on packed FP8 weights.
hipError_t launch_quantize_x(const uint16_t* x, int64_t ldx, int M, int K, uint8_t* xq, hipStream_t stream);
hipError_t launch_unpack_x(const uint8_t* xq, int M, int K, uint8_t* codes, float* scales, hipStream_t stream);
// W8A8 work-group tiles (rows x columns of output)
enum W8Tile : int {
    W8_T128 = 0,      // 128 x 128: 4 waves of 64 x 64
    W8_T256 = 1,      // 256 x 256: 8 waves of 64 x 128
    W8_T64x128 = 2,   // 64 x 128: 4 waves of 64 x 32
    W8_T64x64 = 3,    // 64 x 64: 4 waves of 32 x 32
    W8_STREAM = 4,    // Mpad <= 64: the weight-streaming tile (KIND_W8A8_STREAM, launched by launch_gemm)
};
constexpr int w8_tile_rows(int t) { return t == W8_T256 ? 256 : t == W8_T128 ? 128 : 64; }
constexpr int w8_tile_cols(int t) { return t == W8_T256 ? 256 : t == W8_T64x64 ? 64 : 128; }

// codes: the packed FP8 code units of the N columns served (16 x K bytes per
// 16-column tile), sw: their block scales [N/128][K/128]; a band of columns of
// a packed matrix passes its first tile's units and first scale row.
// tile: a W8Tile; kp > 1: K split into kp parts across work-groups, FP32
// partials in ws [kp][M][N] summed in order into y by launch_sum_parts; cu:
// the device's compute units; stages: the LDS pipeline depth (2 or 4), 0 = 4
// where the grid has at most one work-group per CU
hipError_t launch_w8a8(const uint8_t* codes, const float* sw, int N, int K, const uint8_t* xq, int M, uint16_t* y,
                       int64_t ldy, int tile, int kp, float* ws, int cu, int stages, hipStream_t stream);

// y[m][n] = the parts ws[p][m][n] (p = 0 .. kp-1, [kp][rows][N] FP32) added in
// order and rounded once (RNE) to BF16, or FP16 with f16_out; N % 16 == 0.
hipError_t launch_sum_parts(const float* ws, int kp, int rows, int N, uint16_t* y, int64_t ldy, bool f16_out,
                            hipStream_t stream);

// Static device scratch for callers that cannot allocate (the no-allocation
// FP8 GEMM entry point): the K-split plan's FP32 partials go there instead of
// a caller's workspace.  kScratchBytes bounds the plan it can serve (FFN down
// 5120 x 17408 in 4 K parts needs 4 x 32 x 5120 x 4 = 2.6 MB).
constexpr size_t kScratchBytes = (size_t)4 << 20;
// Device address of the current device's copy of that array (dev = the
// current device's index); looked up once per device, with it current.
hipError_t scratch_address(int dev, void** out);

// Above this many (padded) rows the W8A8 GEMM takes the 256 x 256 tile
constexpr int kW8BigM = 4096;

}  // namespace wq
