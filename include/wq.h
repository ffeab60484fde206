/*
 * libwq -- decode-phase weight-only-quantized GEMM for AMD Instinct MI355X (gfx950).
 *
 *     y[M, N] = x[M, K] . dequant(W)[N, K]^T ,   M = 1 .. 32
 *
 * Two weight formats:
 *
 *   FP8 block-scaled: E4M3 codes with one FP32 scale per 128x128 block of W.
 *     The GEMM takes each 128-wide K block's partial sum in FP32 and folds it
 *     once onto an FP32 outer accumulator times the block's scale (the
 *     "two-level fold" of the atlas "Module m16_tc" docs, section NUMERICS;
 *     block geometry [128, 128] from the arc PR "FP8 bank conflict + the
 *     dispatch threshold's provenance", section "The threshold").  Activations
 *     and outputs are BF16.  The E4M3 flavour is OCP E4M3FN (max 448, NaN =
 *     S.1111.111, no infinity).
 *
 *   3-bit LUT: codes 0..7 looked up in an 8-entry learned FP16 map, times an
 *     FP16 scale per (row, 128-wide K group); each dequantised weight is
 *     rounded to FP16 before it is accumulated (FLUTE PR "Add optimized_w3:
 *     3-bit LUT GEMM on a new mainloop", "Core contributions" item 1 and
 *     "Results").  Activations and outputs are FP16.  Stored either with one
 *     code per 4-bit nibble (the FLUTE PR's "Core contributions" item 2: the
 *     loaded word is already the byte-permute selector) or densely at 3 bits
 *     a code (25% fewer bytes to stream, for 5 more ALU operations per 32
 *     codes to gather the selectors; the FLUTE PR's "Why this exists" names
 *     this trade in FLUTE's own bit-sliced 3-bit storage).  Both layouts give
 *     bit-identical GEMM results.
 *
 * Work flow (FLUTE PR, "Core contributions" item 2: pack once, offline):
 *   1. wq_pack_* reorders canonical row-major [N, K] codes (plus scales and
 *      map) into the library's packed layout, once per matrix.
 *   2. wq_gemm_* runs the decode GEMM on the packed matrix for each batch.
 *
 * Conventions for every call:
 *   - Pointers named as device pointers must point to memory of the current
 *     HIP device; the caller owns all memory.  The library allocates nothing
 *     and keeps no per-call state (only cached device properties and the
 *     options read once from the environment, see below).
 *   - Arguments are validated synchronously before any work is queued; an
 *     invalid call returns an error code and queues nothing.  No C++
 *     exception crosses this interface.
 *   - Work is queued asynchronously on `hip_stream` (a hipStream_t; NULL is
 *     the default stream).  Results are valid once the stream reaches them.
 *   - Calls are thread-safe.  Calls that share a workspace must be ordered
 *     (same stream, or synchronised): concurrent calls on one workspace race.
 *   - Size limits (the kernels address with 32-bit buffer offsets): N and K at
 *     most 2^24 and N*K at most 2^35, else WQ_ERR_SHAPE (size queries return
 *     0); for the decode GEMMs a call's activation span, ((min(M, 32) - 1) *
 *     ldx + K) * 2 bytes, under 4 GiB, else WQ_ERR_LD.
 *
 * Environment options, read once at the first call that needs them (for
 * sweeps without a rebuild; the defaults are the per-shape plan):
 *   WQ_FORCE_PATH   = auto | gemv | mfma  path for wq_gemm_fp8_block (default auto)
 *   WQ_NT           = 1 | 2               16-column MFMA tiles per wave
 *   WQ_SN           = 1 .. 8              column-waves sharing staged activations
 *   WQ_SPLIT        = 1 .. 16             waves per work-group (SN x K-groups)
 *   WQ_WAVES_PER_CU = 1 .. 32             resident waves per CU the plan aims for (4)
 *   WQ_KPARTS       = 1 .. 32             K parts across work-groups for calls that pass a
 *                                         workspace (default: per shape)
 *   WQ_W8A8_TILE    = 128 | 256           W8A8 work-group tile for every M (default: 128 x 128
 *                                         up to M = 4096, 256 x 256 above)
 */
#ifndef WQ_H_
#define WQ_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    WQ_OK = 0,
    WQ_ERR_NULL = 1,       /* a required pointer is NULL                              */
    WQ_ERR_SHAPE = 2,      /* M, N or K outside what the format/path supports         */
    WQ_ERR_LD = 3,         /* a leading dimension is smaller than the row length      */
    WQ_ERR_WORKSPACE = 4,  /* workspace given but smaller than wq_gemm_workspace_bytes() */
    WQ_ERR_CODE = 5,       /* a LUT packer found a code > 7 (packed buffer not valid) */
    WQ_ERR_DEVICE = 6,     /* current device is not gfx950                            */
    WQ_ERR_HIP = 7,        /* a HIP runtime call failed (includes: no device)         */
    WQ_ERR_ALIGN = 8,      /* pointer or leading dimension breaks a 16-byte alignment */
    WQ_ERR_PATH = 9,       /* requested path cannot serve this format / M             */
    WQ_ERR_SCRATCH = 10    /* the no-allocation GEMM's plan needs more than its static scratch */
} wq_status;

typedef enum { WQ_FMT_FP8_BLOCK = 0, WQ_FMT_LUT3 = 1, WQ_FMT_LUT3_DENSE = 2 } wq_format;

/* Kernel path for the GEMM.  AUTO follows the batch ladder of the atlas
 * "Module m16_tc" docs (section ARM ORDER) with the crossover measured on
 * MI355X (arc PR, "The threshold": both arms swept on one binary): the 16-row
 * MFMA tile serves every M = 1..16 for FP8 (it ties or beats the strict-K-order
 * GEMV already at M = 1 on every decode shape, and the GEMV slows with each
 * row; the GEMV serves M <= 4 when asked for explicitly); the LUT format uses
 * the MFMA tile for every M = 1..16
 * (one mainloop across the decode band, as in the FLUTE PR's "Results").
 * M = 17..32 runs the MFMA tile on the two contiguous row halves 0..15 and
 * 16..M-1 ("ARM ORDER"): in one pass, each dequantised weight operand feeding
 * both halves, when the plan has one tile per wave (every built-in plan; for
 * the LUT formats also only where the plan's 32-row activation chunks fit in
 * LDS and its launch bound, which the built-in LUT plans do), and as two
 * passes otherwise.  Either way each row gets the arithmetic of a 16-row
 * call. */
typedef enum { WQ_PATH_AUTO = 0, WQ_PATH_GEMV = 1, WQ_PATH_MFMA = 2 } wq_path;

/* Human-readable name of a status code (static storage, never NULL).
 * Source: arc PR "fix(ArcKernels): FP8 bank conflict + the dispatch
 * threshold's provenance", section "The threshold" (the eligibility of a
 * weight matrix for the block-scaled arm, which these codes report when a
 * call is refused); the pages give no error convention, the codes are this
 * library's reading. */
const char* wq_status_str(wq_status s);

/* Version of the packed layouts written by wq_pack_*; a packed buffer is a
 * deterministic, byte-for-byte function of the pack inputs and this number.
 * Source: FLUTE PR "Add optimized_w3: 3-bit LUT GEMM on a new mainloop",
 * "Core contributions" item 2 (weights packed once, offline, in the order
 * the kernel loads them: the layout is a contract between packer and
 * kernel). */
int wq_packed_format_version(void);

/* Tuning and test hook: override the per-shape plan of later calls.  nt =
 * 16-column tiles per wave (1, 2), sn = column-waves sharing activations
 * (1..8), split = waves per work-group (1..16, rounded down to a multiple of
 * sn and clamped to the kernel's limits: at most 4 K groups, and at most 8
 * waves except for one-tile LUT work-groups with sn >= 4), waves_per_cu = the
 * resident-wave target of the automatic plan; 0 selects the automatic choice
 * for each.  Replaces the
 * WQ_NT / WQ_SN / WQ_SPLIT / WQ_WAVES_PER_CU environment values.  The FP8
 * GEMV path always runs one tile per wave (it ignores nt).  Results stay within the documented tolerance
 * for every setting, but bit patterns may differ between settings.  Not meant
 * to be called while GEMMs are being queued from other threads.
 * Source: arc PR "fix(ArcKernels): FP8 bank conflict + the dispatch
 * threshold's provenance", "The threshold" (every arm selectable on one
 * binary without a rebuild); atlas docs "Module m16_tc", struct M16TcLevers
 * (levers resolved once). */
wq_status wq_set_tuning(int nt, int sn, int split, int waves_per_cu);

/* Tuning and test hook: the number of K parts (1..32) that later calls which
 * pass a workspace split K into across work-groups (the decode GEMMs and
 * wq_gemm_fp8_w8a8); 0 selects the per-shape choice.  Replaces WQ_KPARTS.
 * Parts are clamped so that each keeps at least one K block (8 for the LUT
 * formats).  wq_gemm_workspace_bytes and wq_w8a8_workspace_bytes follow the
 * setting.  Same thread rule as wq_set_tuning.
 * Source: FLUTE PR "Add optimized_w3: 3-bit LUT GEMM on a new mainloop",
 * "Core contributions" (striped stream-K adopted from Marlin); atlas docs
 * "Module m16_tc", "WHY THE FFN ARM LOSES" (low-N grids against the
 * machine's slots). */
wq_status wq_set_kparts(int kp);

/* Tuning and test hook: the LDS pipeline depth of later wq_gemm_fp8_w8a8
 * calls -- 2 (one K block in flight per work-group, two work-groups per CU)
 * or 4 (three in flight, one work-group per CU; the 128 x 128 tile only, the
 * 256 x 256 tile of M > 4096 keeps 2) -- or 0 for the automatic choice (4
 * where the grid has at most one work-group per CU).  The depth changes no
 * arithmetic: outputs are bitwise the same at either.  Returns WQ_ERR_SHAPE
 * for any other value.  Same thread rule as wq_set_tuning.
 * Source: atlas docs "Module m16_tc", ARM ORDER rung 6 (the W8A8 prefill
 * rung) and struct M16TcLevers (levers resolved once); arc PR "fix(ArcKernels):
 * FP8 bank conflict + the dispatch threshold's provenance", "The threshold"
 * (every arm selectable on one binary). */
wq_status wq_set_w8a8_stages(int stages);

/* ------------------------------------------------------------ FP8 block */

/* Bytes of the packed FP8 matrix: N*K code bytes + 4*(N/128)*(K/128) scale
 * bytes.  Returns 0 for an unsupported shape (N or K not a positive multiple
 * of 128).
 * Source: atlas docs "Module m16_tc", WHY (an 89 MB FP8 matrix: one byte a
 * weight); arc PR "fix(ArcKernels): FP8 bank conflict + the dispatch
 * threshold's provenance", "The threshold" (block geometry [128, 128]). */
size_t wq_fp8_block_packed_bytes(int64_t N, int64_t K);

/* Pack an FP8 weight matrix.
 *   w_e4m3  device, [N][ldw] bytes, row-major E4M3FN codes, ldw >= K
 *   scales  device, [N/128][K/128] FP32, row-major, contiguous
 *   packed  device, wq_fp8_block_packed_bytes(N, K) bytes, 16-byte aligned
 * N and K must be positive multiples of 128.  Every byte value is accepted
 * (NaN codes decode to NaN).  Asynchronous on hip_stream.
 * Source: FLUTE PR "Add optimized_w3: 3-bit LUT GEMM on a new mainloop",
 * "Core contributions" item 2 (offline pack in matrix-fragment order, one
 * coalesced 16-byte load per lane); arc PR "fix(ArcKernels): FP8 bank
 * conflict + the dispatch threshold's provenance", "The threshold" (128 x
 * 128 scale blocks). */
wq_status wq_pack_fp8_block(const uint8_t* w_e4m3, int64_t ldw, const float* scales,
                            int64_t N, int64_t K, void* packed, void* hip_stream);

/* y = x . dequant(W)^T for a packed FP8 matrix.
 *   packed     device, from wq_pack_fp8_block with the same N, K
 *   x          device, [M][ldx] BF16 bits; ldx >= K, ldx % 8 == 0, x 16-byte aligned
 *   y          device, [M][ldy] BF16 bits (RNE); ldy >= N; only columns < N are written
 *   M          0 .. 32; M == 0 queues nothing and returns WQ_OK
 *   workspace  NULL, or device scratch of at least wq_gemm_workspace_bytes(...)
 *              bytes, 16-byte aligned, owned by the caller (contents on entry do not
 *              matter; they are overwritten).  With NULL every output is reduced
 *              inside one work-group.  With a workspace, a shape whose column
 *              groups leave CUs idle (the low-N projections) also splits K across
 *              work-groups: each K part's work-group writes FP32 partial sums to
 *              the workspace and a second kernel on the same stream adds the parts
 *              in a fixed order and rounds once (the pages' split-K for low-N
 *              grids).  A workspace smaller than required returns
 *              WQ_ERR_WORKSPACE; a misaligned one WQ_ERR_ALIGN.
 * Numerics: every output is within 2 BF16 ULP of the exact result rounded to
 * BF16, or within 1e-3*sqrt(K)*max|x|*max|w| of the exact result.  Results are
 * deterministic, and row r of an M-row call equals row r of any other call on
 * the same path with the same row r of x, bit for bit, when both calls pass a
 * workspace or both pass NULL (the two schedules may round differently).
 * Source: atlas docs "Module m16_tc", WHY, NUMERICS (two-level fold, 2 BF16
 * ULP) and ARM ORDER (the batch ladder, row halves for M = 17..32). */
wq_status wq_gemm_fp8_block(const void* packed, int64_t N, int64_t K,
                            const uint16_t* x, int64_t ldx,
                            uint16_t* y, int64_t ldy, int64_t M,
                            void* workspace, size_t workspace_bytes, void* hip_stream);

/* Same as wq_gemm_fp8_block with an explicit path (WQ_PATH_GEMV serves
 * M <= 4 only; WQ_PATH_MFMA serves M <= 32; AUTO as above).  Used to sweep
 * the GEMV/MFMA crossover (arc PR, section "The threshold": one binary, arms
 * toggled without a rebuild).
 * Source: arc PR "fix(ArcKernels): FP8 bank conflict + the dispatch
 * threshold's provenance", "The threshold" (three arms on one binary,
 * toggled without a rebuild); atlas docs "Module m16_tc", ARM ORDER. */
wq_status wq_gemm_fp8_block_path(const void* packed, int64_t N, int64_t K,
                                 const uint16_t* x, int64_t ldx,
                                 uint16_t* y, int64_t ldy, int64_t M,
                                 void* workspace, size_t workspace_bytes,
                                 int path, void* hip_stream);

/* The FP8 GEMM without allocation and without a workspace argument: the
 * same computation, plan and result bits as wq_gemm_fp8_block called with a
 * workspace of wq_gemm_workspace_bytes(...) bytes, but the K-split partials
 * go to a static device array of the library (wq_noalloc_scratch_bytes()
 * bytes, 4 MiB; each device holds its own copy until the process ends).  The
 * call makes no allocation of any kind; the caller passes inputs and outputs
 * only.  A shape whose K-split plan needs more scratch than that returns
 * WQ_ERR_SCRATCH and queues nothing.  Every call on one device shares that
 * device's array: calls that overlap on one device (other streams, other
 * threads) race and must be ordered by the caller.  Arguments, validation,
 * numerics and determinism otherwise as wq_gemm_fp8_block.
 * Callers: code that cannot call hipMalloc -- work under HIP graph capture,
 * tight serving loops, harnesses that forbid allocation. */
wq_status wq_gemm_fp8_block_noalloc(const void* packed, int64_t N, int64_t K,
                                    const uint16_t* x, int64_t ldx,
                                    uint16_t* y, int64_t ldy, int64_t M, void* hip_stream);

/* Bytes of the static device scratch that wq_gemm_fp8_block_noalloc uses
 * (the largest K-split workspace it can serve).
 * Callers: those of wq_gemm_fp8_block_noalloc, to check a shape ahead
 * against wq_gemm_workspace_bytes. */
size_t wq_noalloc_scratch_bytes(void);

/* ----------------------------------------------------------------- LUT3 */

/* Bytes of the packed LUT matrix: N*K/2 nibble bytes + 16*N*ceil(K/1024)
 * scale bytes (K blocks padded to a multiple of 8) + 32 bytes (map and pack
 * status).  Returns 0 for an unsupported shape (N not a positive multiple of
 * 16 or K not of 128).
 * Source: FLUTE PR "Add optimized_w3: 3-bit LUT GEMM on a new mainloop",
 * "Core contributions" item 2 (one 3-bit code per nibble). */
size_t wq_lut3_packed_bytes(int64_t N, int64_t K);

/* Pack a 3-bit LUT weight matrix.
 *   codes   device, [N][ldc] bytes, one code 0..7 per byte, ldc >= K
 *   qmap    device, FP16 bits [8] (the learned map; entry c serves code c)
 *   scales  device, FP16 bits [N][K/128], row-major, contiguous
 *   packed  device, wq_lut3_packed_bytes(N, K) bytes, 16-byte aligned
 * This call synchronises hip_stream: it reads back whether any code exceeded
 * 7 and then returns WQ_ERR_CODE (the packed buffer is then not valid).
 * Source: FLUTE PR "Add optimized_w3: 3-bit LUT GEMM on a new mainloop",
 * "Core contributions" items 1 and 2 (learned 8-entry map, group scales,
 * nibble + fragment-order offline pack). */
wq_status wq_pack_lut3(const uint8_t* codes, int64_t ldc, const uint16_t* qmap,
                       const uint16_t* scales, int64_t N, int64_t K,
                       void* packed, void* hip_stream);

/* y = x . dequant(W)^T for a packed LUT matrix.
 *   x  device, [M][ldx] FP16 bits; ldx >= K, ldx % 8 == 0, x 16-byte aligned
 *   y  device, [M][ldy] FP16 bits (RNE); ldy >= N
 * Other arguments, limits and guarantees as wq_gemm_fp8_block (the ULP
 * criterion is applied after rounding the FP16 result to BF16).
 * Source: FLUTE PR "Add optimized_w3: 3-bit LUT GEMM on a new mainloop",
 * "Core contributions" item 1 (byte-permute lookup of the learned map) and
 * "Results" (the dequant rounds to FP16 before the accumulate; one mainloop
 * for M = 1..16). */
wq_status wq_gemm_lut3(const void* packed, int64_t N, int64_t K,
                       const uint16_t* x, int64_t ldx,
                       uint16_t* y, int64_t ldy, int64_t M,
                       void* workspace, size_t workspace_bytes, void* hip_stream);

/* Dense form of the LUT format: the same codes, map and scales, with the
 * codes stored at 3 bits each.  Packed bytes: N*K*3/8 code bytes + 16*N*
 * ceil(K/1024) scale bytes + 32; 0 for an unsupported shape (as
 * wq_lut3_packed_bytes).  Arguments, limits, errors and synchronisation of
 * the three calls are those of wq_pack_lut3 / wq_gemm_lut3 / wq_unpack_lut3;
 * a GEMM on a dense matrix returns the same bits as on the nibble-packed
 * matrix of the same inputs (the layouts differ only in how the codes are
 * stored, the arithmetic is the same).
 * Source: FLUTE PR "Add optimized_w3: 3-bit LUT GEMM on a new mainloop",
 * "Why this exists" (FLUTE's own bit-sliced 3-bit storage, which the nibble
 * pack trades away). */
size_t wq_lut3_dense_packed_bytes(int64_t N, int64_t K);

/* Source: FLUTE PR "Add optimized_w3: 3-bit LUT GEMM on a new mainloop",
 * "Why this exists" (3-bit storage) and "Core contributions" item 2 (offline
 * pack). */
wq_status wq_pack_lut3_dense(const uint8_t* codes, int64_t ldc, const uint16_t* qmap,
                             const uint16_t* scales, int64_t N, int64_t K,
                             void* packed, void* hip_stream);

/* Source: FLUTE PR "Add optimized_w3: 3-bit LUT GEMM on a new mainloop",
 * "Why this exists" and "Core contributions" item 1 (same lookup as the
 * nibble layout). */
wq_status wq_gemm_lut3_dense(const void* packed, int64_t N, int64_t K,
                             const uint16_t* x, int64_t ldx,
                             uint16_t* y, int64_t ldy, int64_t M,
                             void* workspace, size_t workspace_bytes, void* hip_stream);

/* ------------------------------------------------------------------ W8A8 */
/* The W8A8 block-scaled tier above the decode band (atlas "Module m16_tc",
 * "ARM ORDER" rung 6): activations are quantised to FP8 (the arc PR, "Worth a
 * separate change": block-scaled FP8 needs an activation quantiser) and
 * multiplied with the packed FP8 weights on the FP8 matrix cores.
 *
 * Quantiser reading (the pages give none): one FP32 scale per (row, 128-wide
 * K group), s = amax/448 in binary32 (1 for an all-zero group), code = E4M3
 * nearest-even of clamp(x/s, -448, 448) with x/s in binary32 -- the rule of
 * the weights' block quantiser.  A group holding an infinity or a NaN gets
 * a NaN scale and the E4M3 NaN code 0x7F for all its values, so every output
 * of that row is NaN (the weight-only paths give NaN or an infinity there).
 *
 * Measured on MI355X at the FFN sizes, quantiser + GEMM with the workspace
 * overtake the decode GEMM run as 32-row calls from M = 33 on. */

/* Workspace bytes of a W8A8 GEMM of this M, N, K that splits K across
 * work-groups (kp * M * n * 4 for kp parts over the n columns split, following
 * wq_set_kparts); 0 when it keeps K inside one work-group, for an invalid
 * shape, or with no gfx950 device current.
 * Source: atlas docs "Module m16_tc", ARM ORDER rung 6 (W8A8 block-scaled
 * prefill); FLUTE PR "Add optimized_w3: 3-bit LUT GEMM on a new mainloop",
 * "Core contributions" (stream-K for thin grids). */
size_t wq_w8a8_workspace_bytes(int64_t M, int64_t N, int64_t K);

/* Bytes of a packed FP8 activation buffer: Mpad*K codes + 4*Mpad*(K/128)
 * scale bytes, Mpad = 16*ceil(M/16).  0 for an unsupported shape (K not a
 * positive multiple of 128, M < 1, or 2 GiB or more).
 * Source: arc PR "fix(ArcKernels): FP8 bank conflict + the dispatch
 * threshold's provenance", "Worth a separate change" (block-scaled FP8 needs
 * the activations in FP8: an activation quantiser). */
size_t wq_x_fp8_packed_bytes(int64_t M, int64_t K);

/* Quantise BF16 activations into the packed FP8 activation layout.
 *   x_bf16  device, [M][ldx] BF16 bits; ldx >= K, ldx % 8 == 0, 16-byte aligned
 *   xq      device, wq_x_fp8_packed_bytes(M, K) bytes, 16-byte aligned
 * M == 0 queues nothing.  Asynchronous on hip_stream.
 * Source: arc PR "fix(ArcKernels): FP8 bank conflict + the dispatch
 * threshold's provenance", "Worth a separate change" (an activation
 * quantiser for the block-scaled FP8 product). */
wq_status wq_quantize_x_fp8(const uint16_t* x_bf16, int64_t ldx, int64_t M, int64_t K,
                            void* xq, void* hip_stream);

/* y = dequant(xq) . dequant(W)^T with both operands FP8.  Up to 64 rows it
 * runs on the weight-streaming tile of the decode GEMM (FP8 weight units
 * through a register ring, the packed activations staged in LDS) where that
 * stages at most twice a work-group's weight bytes; otherwise, and above, on
 * an LDS-staged tile kernel (64-row, 128 x 128 or 256 x 256 tiles).
 *   packed  device, from wq_pack_fp8_block with the same N, K (the same packed
 *           matrix serves wq_gemm_fp8_block); N*K < 2^32
 *   xq      device, from wq_quantize_x_fp8 with the same M, K
 *   y       device, [M][ldy] BF16 bits (RNE); ldy >= N
 *   M       any M >= 1 with wq_x_fp8_packed_bytes(M, K) > 0; M == 0 queues nothing
 * Per 128-K block the FP32 matrix-core sum of e4m3(x)*e4m3(w) is folded onto an
 * FP32 accumulator times sx[m][kb]*s[n/128][kb].  Every output is within 2 BF16
 * ULP of the exact result (of the quantised operands) rounded to BF16, or within
 * 1e-3*sqrt(K)*max|xq*sx|*max|w| of it.  Deterministic.
 *   workspace  NULL, or device scratch of at least wq_w8a8_workspace_bytes(M, N, K)
 *           bytes, 16-byte aligned, contents on entry irrelevant.  With NULL
 *           every output is reduced inside one work-group and row r of the result
 *           depends only on row r of xq (its summation order may still differ
 *           between Ms that take different kernels, e.g. the streaming tile's K
 *           groups up to 64 rows).  With a workspace, an M whose output
 *           tiles leave CUs idle also splits K across work-groups: FP32 partial
 *           sums go to the workspace and a second kernel on the same stream adds
 *           them in a fixed order (results stay deterministic for a given M, N, K;
 *           the split, and so the rounding of a row, may differ between Ms).
 *           With or without a workspace, an M whose grid would end in a mostly
 *           idle round of work-group slots may be served in two column bands: a
 *           leading band of whole rounds in one K part, and the remaining
 *           columns as a second launch (K split there only with a workspace).
 *           A workspace smaller than required returns WQ_ERR_WORKSPACE, a
 *           misaligned one WQ_ERR_ALIGN.
 * Source: atlas docs "Module m16_tc", ARM ORDER rung 6 (W8A8 block-scaled
 * prefill) and NUMERICS (the two-level fold); arc PR "fix(ArcKernels): FP8
 * bank conflict + the dispatch threshold's provenance", "Worth a separate
 * change". */
wq_status wq_gemm_fp8_w8a8(const void* packed, int64_t N, int64_t K, const void* xq, int64_t M,
                           uint16_t* y, int64_t ldy, void* workspace, size_t workspace_bytes,
                           void* hip_stream);

/* ------------------------------------------------------------ workspace */

/* Workspace bytes a GEMM of this format and shape needs to run its
 * K-split schedule (the same for every M and path; the FP8 GEMV path never
 * uses it).  0 when the shape's plan keeps K inside one work-group, and for an
 * unsupported shape or when no gfx950 device is current; NULL may then be
 * passed.  Queries the current device (cached).
 * Source: FLUTE PR "Add optimized_w3: 3-bit LUT GEMM on a new mainloop",
 * "Core contributions" (striped stream-K with a serial reduction of the
 * partial sums); atlas docs "Module m16_tc", "WHY THE FFN ARM LOSES". */
size_t wq_gemm_workspace_bytes(int fmt, int64_t M, int64_t N, int64_t K);

/* ----------------------------------------------------------- test hooks */
/* Decode a packed matrix back to canonical row-major [N][K] with the same
 * device dequant code the GEMM runs.  Asynchronous on hip_stream. */

/* out[n][k] = BF16(e4m3(code)) -- unscaled; the MFMA path's converter.
 * Source: atlas docs "Module m16_tc", module oracle (one numerics contract
 * evaluated against the device and a host model: the device dequant checked
 * bit for bit). */
wq_status wq_unpack_fp8_block(const void* packed, int64_t N, int64_t K,
                              uint16_t* w_bf16, void* hip_stream);

/* out[n][k] = FP32(e4m3(code)) -- unscaled; the GEMV path's converter.
 * Source: atlas docs "Module m16_tc", module oracle (as wq_unpack_fp8_block;
 * the GEMV arm's converter). */
wq_status wq_unpack_fp8_block_f32(const void* packed, int64_t N, int64_t K,
                                  float* w_f32, void* hip_stream);

/* out[n][k] = fp16_rne(qmap[code] * scale[n][k/128])
 * Source: FLUTE PR "Add optimized_w3: 3-bit LUT GEMM on a new mainloop",
 * "Results" (the dequant rounds to FP16 before the accumulate; exactness-
 * gated kernels) and atlas docs "Module m16_tc", module oracle. */
wq_status wq_unpack_lut3(const void* packed, int64_t N, int64_t K,
                         uint16_t* w_f16, void* hip_stream);

/* Packed FP8 activations back to canonical codes [M][K] (E4M3) and scales
 * [M][K/128] (FP32, 4-byte aligned).
 * Source: arc PR "fix(ArcKernels): FP8 bank conflict + the dispatch
 * threshold's provenance", "Worth a separate change" (the activation
 * quantiser, checked bit for bit against the host rule). */
wq_status wq_unpack_x_fp8(const void* xq, int64_t M, int64_t K, uint8_t* codes, float* scales,
                          void* hip_stream);

/* The same for a matrix packed by wq_pack_lut3_dense.
 * Source: FLUTE PR "Add optimized_w3: 3-bit LUT GEMM on a new mainloop",
 * "Why this exists" (3-bit storage) and "Results" (FP16 dequant). */
wq_status wq_unpack_lut3_dense(const void* packed, int64_t N, int64_t K,
                               uint16_t* w_f16, void* hip_stream);

/* Host-only plan queries: the plan a call would take on a gfx950 device with
 * `cu` compute units (1..1024), computed on the host without touching any
 * device, so that the dispatch rules can be checked where no GPU is present.
 * Both follow wq_set_tuning, wq_set_kparts and the environment levers as the
 * calls do.  with_workspace != 0 plans a call that passes a workspace (K may
 * be split across work-groups).  Return WQ_ERR_NULL for a NULL plan,
 * WQ_ERR_SHAPE where the call would reject the shape or M, or cu is out of
 * range, and WQ_ERR_PATH where the call would reject the path.  Thread-safe.
 *
 * Decode GEMM (wq_gemm_fp8_block[_path], wq_gemm_lut3[_dense]; M = 1..32):
 * plan[6] = { path run (WQ_PATH_GEMV or WQ_PATH_MFMA), 16-column tiles per
 * wave, column-waves per work-group, waves per work-group, K parts across
 * work-groups, launches (rows of x are served 32 or 16 per launch) }.
 * Source: FLUTE PR "Add optimized_w3: 3-bit LUT GEMM on a new mainloop",
 * opening summary (a dispatch table chosen per shape from measurements);
 * atlas docs "Module m16_tc", "WHY THE FFN ARM LOSES" (grids against the
 * machine's slots). */
wq_status wq_query_gemm_plan(int fmt, int path, int64_t M, int64_t N, int64_t K, int cu,
                             int with_workspace, int* plan);

/* W8A8 (wq_gemm_fp8_w8a8; any M the activation packer accepts):
 * plan[4] = { output tile rows, tile columns, K parts across work-groups,
 * kernel: 0 = the LDS-staged tile kernel, 1 = the weight-streaming tile of up
 * to 64 rows (then the columns are those of one work-group) }.
 * Source: atlas docs "Module m16_tc", ARM ORDER rung 6 (the W8A8 prefill
 * rung) and "WHY THE FFN ARM LOSES" (grids against the machine's slots). */
wq_status wq_query_w8a8_plan(int64_t M, int64_t N, int64_t K, int cu, int with_workspace, int* plan);

#ifdef __cplusplus
}
#endif

#endif /* WQ_H_ */
