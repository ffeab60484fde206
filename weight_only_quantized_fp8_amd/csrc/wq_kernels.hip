// gfx950 kernels of libwq: the decode GEMM (MFMA tile and strict-order GEMV)
// for FP8 block-scaled and 3-bit LUT weights, and the pack / unpack kernels.
//
// Packed layouts (version 3).  A "unit" is 16 rows of W (one MFMA tile along
// N) by one 128-wide K block, stored contiguously, units ordered (tile, kb)
// with kb fastest.  Inside a unit every 16-byte piece is what one lane loads
// (the FLUTE PR "Add optimized_w3", "Core contributions" item 2: one
// coalesced 16-byte load lands directly in the lane's matrix-core operand).
// Both formats order K the same way: MFMA step s of a K block covers
// k = 32s .. 32s+31, and lane group g = l/16 holds k = 32s + 8g .. +7, so the
// four groups' activations of one batch row are one contiguous 64-byte run.
//
//   FP8   unit = 2048 B = two 1 KiB chunks j = 0, 1.  Lane l of chunk j holds
//         16 codes of row 16t + l%16: byte i is k = 128kb + 32(2j + i/8) +
//         8(l/16) + i%8 (steps 2j and 2j+1).  Block scales follow the codes as
//         FP32 [N/128][K/128].
//   LUT3  unit = 1024 B.  Lane l holds 32 codes of row 16t + l%16 in 4 dwords
//         s: byte b carries k = 128kb + 32s + 8(l/16) + e with e = b in its low
//         nibble and e = b + 4 in its high nibble.  Group scales follow as FP16
//         [tile][kb / 8][16 rows][kb % 8] (K blocks padded to a multiple of 8
//         with zeros), so one 16-byte load brings a row's scales for 8 K
//         blocks; then the 8 map entries (FP16), then a 16-byte pack-status
//         word.
//   LUT3D the dense 3-bit form of LUT3: unit = 768 B, lane l holds the same 32
//         codes in 3 dwords (12 bytes at 12l).  Dwords s = 0..2 carry step s
//         exactly as LUT3 does; the 8 codes of step 3 fill the spare bits 3
//         and 7 of every byte: bit i of code e = b at bit 3 of byte b of dword
//         i, and of code e = b + 4 at bit 7 (the byte-plane idea of FLUTE's own
//         3-bit storage, named in the FLUTE PR's "Why this exists", traded for
//         5 more ALU operations per 32 codes).  Scales, map and status word
//         follow as in LUT3.
//
// GEMM schedule.  One work-group owns one column group (SN column-waves of
// NT tiles of 16 output columns) over the whole of K, or over one of KP K
// parts.  Its waves form SK K groups that split its K blocks into contiguous
// ranges (split-K), so a low-N projection still puts enough waves on the
// chip; SN, SK and KP are chosen per shape by the host.  Each wave walks its
// range with the next D units' loads in flight (a register ring) while the
// column-waves of a K group share activation chunks staged in LDS.  Every
// 128-K block is folded onto FP32 accumulators.  With one K group each wave
// stores its own outputs; otherwise the other K groups' partial tiles pass
// through LDS and K group 0 adds them in a fixed order and stores (the GEMV:
// the work-group sums them in LDS in the same fixed order).  With KP = 1 no two work-groups share an
// output: no cross-work-group traffic, no workspace, no fence.  With KP > 1
// (the caller passed a workspace) each K part's work-group stores FP32 sums
// to the workspace and a second kernel adds the parts in order.  Every sum
// has a fixed order: results are deterministic and do not depend on M.
#include <atomic>
#include <mutex>

#include "wq_device.hpp"
#include "wq_internal.h"

namespace wq {

// 4 KiB of zeros: the source of the block-scale load of a unit with nothing
// to fetch (vector loads use a zero-byte buffer resource instead).
__device__ __attribute__((aligned(256))) uint8_t g_zero_page[4096];

// Scratch of the no-allocation GEMM entry point: each device that runs the
// library holds its own copy until the process ends.  In host code the name
// `scratch` is only a host-side handle of the symbol, not a device address;
// scratch_address() returns the device address (hipGetSymbolAddress with the
// device current), and only that address is ever passed to a kernel.  Every
// call on one device shares that device's copy: calls that overlap on one
// device race, and the array keeps whatever the last call left in it (every
// slot a call reads, it has written first).
static __device__ __align__(256) uint8_t scratch[kScratchBytes];

static constexpr int kScratchDevices = 64;
static std::atomic<void*> g_scratch_ptr[kScratchDevices];
static std::mutex g_scratch_mu;

hipError_t scratch_address(int dev, void** out)
{
    if (dev < 0 || dev >= kScratchDevices) return hipErrorInvalidDevice;
    void* p = g_scratch_ptr[dev].load(std::memory_order_acquire);
    if (!p) {
        std::lock_guard<std::mutex> lk(g_scratch_mu);
        p = g_scratch_ptr[dev].load(std::memory_order_relaxed);
        if (!p) {
            const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
            if (e != hipSuccess) return e;
            if (!p) return hipErrorInvalidSymbol;
            g_scratch_ptr[dev].store(p, std::memory_order_release);
        }
    }
    *out = p;
    return hipSuccess;
}

// ======================================================================
// Policies: per-unit loads and compute for each kernel kind.  A policy is
// bound to one wave's tiles; load(r, kb, valid, pos) issues the loads of K
// block kb into the register set r (zeros when !valid), compute(r, xblk, pos)
// consumes it with the staged activations of that block; pos is the unit's
// compile-time position in the unrolled loop.
// ======================================================================

// ---- activation staging for the MFMA tiles ---------------------------------
// x is staged through LDS in chunks of chunk_blocks16(kind, MT) 16-row K
// blocks.  The SN
// column-waves of a K group share every chunk: its 16-byte pieces are dealt
// round-robin over the group's SN*64 lanes, consecutive lanes taking
// consecutive pieces of one row, so each load instruction reads whole
// 256-byte row runs.  A chunk is loaded one chunk ahead of its use -- before
// the weight loads issued in between -- so the wait that precedes staging it
// never waits for weights still in flight, and the K group synchronises once
// per chunk (double buffer, one barrier) rather than once per K block.
// LDS rows are padded by 16 bytes: the 16 rows a 16-lane group reads for one
// MFMA operand then start 4 banks apart and cover all 64 banks once (the
// stride arithmetic of the shared-memory pad in the arc PR "FP8 bank conflict
// + the dispatch threshold's provenance", "What landed").
// With MT = 2 (single-pass M = 17..32) a staged block holds 32 rows and a
// chunk holds half as many K blocks, so the chunk's bytes and pieces stay the
// same.
constexpr int kXRowBytes = 128 * 2 + 16;                    // padded LDS row of one K block

// XPL: pieces per lane, >= kXChunkPieces / (64 * SN); MT: row tiles; CB: the
// chunk size in 16-row K blocks
template <int XPL, int MT, int CB>
struct XChunk {
    static constexpr int kXChunkPieces = CB * 16 * 16;      // 16-byte pieces per chunk
    static constexpr int kRows = 16 * MT;
    static constexpr int kBlocks = CB / MT;                 // K blocks per chunk
    static constexpr int kBlockBytes = kRows * kXRowBytes;
    static constexpr int kChunkBytes = kBlocks * kBlockBytes;
    static_assert(kBlocks * kRows * 16 == kXChunkPieces, "a chunk has the same pieces for every MT");
    buf_t rx;                 // x rows 0 .. M-1
    uint32_t vo[XPL];         // byte offset of piece i in the chunk at K block 0, or out of range
    int blk[XPL];             // K block of piece i inside the chunk (large: no piece)
    int dst[XPL];             // LDS offset of piece i inside a chunk buffer (-1: no piece)
    uint4 r[XPL];

    __device__ void init(const GemmArgs& a, int lane, int cw, int sn)
    {
        rx = make_buf(a.x, (uint32_t)(((int64_t)(a.rows - 1) * a.ldx + (int64_t)a.KB * 128) * 2));
#pragma unroll
        for (int i = 0; i < XPL; ++i) {
            const int q = cw * 64 + lane + i * sn * 64;
            const int b = q / (kRows * 16), row = (q >> 4) % kRows, seg = q & 15;
            const bool ok = q < kXChunkPieces && row < a.rows;
            blk[i] = ok ? b : (1 << 29);
            vo[i] = ok ? (uint32_t)(row * a.ldx * 2 + b * 256 + seg * 16) : kBufOutOfRange;
            dst[i] = q < kXChunkPieces ? b * kBlockBytes + row * kXRowBytes + seg * 16 : -1;
        }
    }

    // Issue the loads of the chunk that starts at K block kb; blocks >= kb_end,
    // rows >= M and pieces past the chunk read zeros.
    __device__ __forceinline__ void load(int kb, int kb_end)
    {
        const int lim = kb_end - kb;    // blocks of this chunk inside the range (wave-uniform)
#pragma unroll
        for (int i = 0; i < XPL; ++i)
            r[i] = buf_load16(rx, blk[i] < lim ? vo[i] : kBufOutOfRange, (uint32_t)kb * 256u);
    }

    __device__ __forceinline__ void stage(uint8_t* buf) const
    {
#pragma unroll
        for (int i = 0; i < XPL; ++i)
            if (dst[i] >= 0) *reinterpret_cast<uint4*>(buf + dst[i]) = r[i];
    }
};

// 8 consecutive activations of batch row 16*mt + lane % 16, from k on, of one staged K block
__device__ __forceinline__ uint4 x_frag(const uint8_t* blk, int lane, int k, int mt = 0)
{
    return *reinterpret_cast<const uint4*>(blk + (mt * 16 + (lane & 15)) * kXRowBytes + k * 2);
}

// ---- activation staging for the GEMV ----------------------------------------
// The GEMV needs rows 0..3 only, as FP32: a chunk is staged as FP32
// [block][4 rows][128] (each activation converted once per work-group, not
// once per use), loaded as 4 rows x 256-byte runs per instruction.
constexpr int kGemvRows = 4;
constexpr int kGemvBlockBytes = kGemvRows * 128 * 4;
constexpr int kGemvChunkBlocks = chunk_blocks16(KIND_GEMV_FP8, 1);
constexpr int kGemvChunkPieces = kGemvChunkBlocks * kGemvRows * 16;   // 16-byte BF16 pieces per chunk

template <int XPL>   // pieces per lane: >= kGemvChunkPieces / (64 * SN)
struct XChunkF32 {
    static constexpr int kBlocks = kGemvChunkBlocks;
    static constexpr int kChunkBytes = kGemvChunkBlocks * kGemvBlockBytes;
    static constexpr int kBlockBytes = kGemvBlockBytes;
    buf_t rx;
    uint32_t vo[XPL];
    int blk[XPL];
    int dst[XPL];
    uint4 r[XPL];

    __device__ void init(const GemmArgs& a, int lane, int cw, int sn)
    {
        rx = make_buf(a.x, (uint32_t)(((int64_t)(a.rows - 1) * a.ldx + (int64_t)a.KB * 128) * 2));
#pragma unroll
        for (int i = 0; i < XPL; ++i) {
            const int q = cw * 64 + lane + i * sn * 64;
            const int b = q >> 6, row = (q >> 4) & 3, seg = q & 15;
            const bool ok = q < kGemvChunkPieces && row < a.rows;
            blk[i] = ok ? b : (1 << 29);
            vo[i] = ok ? (uint32_t)(row * a.ldx * 2 + b * 256 + seg * 16) : kBufOutOfRange;
            dst[i] = q < kGemvChunkPieces ? b * kGemvBlockBytes + row * 512 + seg * 32 : -1;
        }
    }

    __device__ __forceinline__ void load(int kb, int kb_end)
    {
        const int lim = kb_end - kb;    // blocks of this chunk inside the range (wave-uniform)
#pragma unroll
        for (int i = 0; i < XPL; ++i)
            r[i] = buf_load16(rx, blk[i] < lim ? vo[i] : kBufOutOfRange, (uint32_t)kb * 256u);
    }

    // BF16 -> FP32 is exact: the BF16 bits become the top half of the FP32 word
    __device__ __forceinline__ void stage(uint8_t* buf) const
    {
#pragma unroll
        for (int i = 0; i < XPL; ++i)
            if (dst[i] >= 0) {
                const uint32_t d[4] = {r[i].x, r[i].y, r[i].z, r[i].w};
                uint32_t f[8];
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    f[2 * e] = d[e] << 16;
                    f[2 * e + 1] = d[e] & 0xFFFF0000u;
                }
                uint4* o = reinterpret_cast<uint4*>(buf + dst[i]);
                o[0] = make_uint4(f[0], f[1], f[2], f[3]);
                o[1] = make_uint4(f[4], f[5], f[6], f[7]);
            }
    }
};

// ---- FP8 weight stream (shared by the MFMA tile and the GEMV) ---------------
// A unit is one tile's 2 KiB of codes for one K block: lane l loads 16 codes
// of row l%16 from each 1 KiB chunk, plus the block scale (scalar load).
template <int NT>
struct Fp8Stream {
    struct Unit {
        uint4 w[NT][2];
        float s;
    };
    int lane;
    int KB;
    int ntiles;               // valid tiles of this wave
    buf_t rw;                 // code units of the wave's tiles (zero bytes past N)
    buf_t rnull;              // zero bytes: loads return zeros
    const float* srow;        // block-scale row of this wave's tiles

    __device__ Fp8Stream(const GemmArgs& a, int l, int tile0) : lane(l), KB(a.KB)
    {
        ntiles = max(0, min(NT, a.n_tiles - tile0));
        const uint8_t* base = a.codes + (((int64_t)min(tile0, a.n_tiles) * a.KB) << 11);
        rw = make_buf(base, (uint32_t)(ntiles * a.KB) << 11);
        rnull = make_buf(base, 0);
        srow = reinterpret_cast<const float*>(a.scales) + (int64_t)(min(tile0, a.n_tiles - 1) * 16 / 128) * a.KB;
    }

    __device__ __forceinline__ void set_range(int) {}

    __device__ __forceinline__ void load(Unit& r, int kb, bool valid, int) const
    {
#pragma unroll
        for (int t = 0; t < NT; ++t) {
            const buf_t rs = (valid && t < ntiles) ? rw : rnull;
            const uint32_t so = (uint32_t)(t * KB + kb) << 11;
            r.w[t][0] = buf_load_stream16(rs, lane * 16, so);
            r.w[t][1] = buf_load_stream16(rs, lane * 16 + 1024, so);
        }
        // a unit with nothing to fetch (and a wave past N) reads a zero scale
        r.s = load_uniform_f32((valid && ntiles > 0) ? (const void*)(srow + kb) : (const void*)g_zero_page);
    }
};

// ---- FP8 weights, 16-row BF16 MFMA tile ------------------------------------
// A operand = dequantised weights (lane: row n = l%16), B operand = x
// (lane: batch row m = l%16).  Output D[n][m] -> lane holds n = 4(l/16)+v.
// MT = 2 serves M = 17..32 in one pass: each dequantised A operand feeds two
// MFMAs, one per 16-row half of the batch, with the same per-row arithmetic
// as the 16-row tile.
template <int NT, int MT>
struct MfmaFp8 : Fp8Stream<NT> {
    static constexpr int KIND = KIND_MFMA_FP8;
    static constexpr bool kSumInRegisters = true;   // K groups combine through add_partial
    static constexpr int NTILES = NT;
    static constexpr int ROWS = 16 * MT;
    static constexpr int KALIGN = k_align(KIND);   // K-group ranges start at any K block
    template <int XPL> using Stage = XChunk<XPL, MT, chunk_blocks16(KIND_MFMA_FP8, MT)>;
    using typename Fp8Stream<NT>::Unit;
    using Fp8Stream<NT>::lane;
    using Fp8Stream<NT>::ntiles;
    f32x4_t outer[NT][MT];

    __device__ MfmaFp8(const GemmArgs& a, int l, int tile0) : Fp8Stream<NT>(a, l, tile0)
    {
#pragma unroll
        for (int t = 0; t < NT; ++t)
#pragma unroll
            for (int h = 0; h < MT; ++h) outer[t][h] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    }

    __device__ __forceinline__ void compute(const Unit& r, const uint8_t* xblk, int)
    {
        bf16x8_t b[MT][4];
#pragma unroll
        for (int h = 0; h < MT; ++h)
#pragma unroll
            for (int f = 0; f < 4; ++f)    // MFMA step f = 2j + h: lane group g holds k = 32f + 8g .. +7
                b[h][f] = __builtin_bit_cast(bf16x8_t, x_frag(xblk, lane, f * 32 + (lane >> 4) * 8, h));
        f32x4_t blk[NT][MT];
#pragma unroll
        for (int t = 0; t < NT; ++t)
#pragma unroll
            for (int h = 0; h < MT; ++h) blk[t][h] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int f = 0; f < 4; ++f) {
            const int j = f >> 1, hi = f & 1;
#pragma unroll
            for (int t = 0; t < NT; ++t) {
                const uint4 w = r.w[t][j];
                const bf16x8_t av = hi ? e4m3x8_to_bf16x8(w.z, w.w) : e4m3x8_to_bf16x8(w.x, w.y);
#pragma unroll
                for (int h = 0; h < MT; ++h) blk[t][h] = mfma_bf16(av, b[h][f], blk[t][h]);
            }
        }
        // two-level fold: one FP32 FMA per 128-K block and output
#pragma unroll
        for (int t = 0; t < NT; ++t)
#pragma unroll
            for (int h = 0; h < MT; ++h)
#pragma unroll
                for (int v = 0; v < 4; ++v) outer[t][h][v] = __builtin_fmaf(r.s, blk[t][h][v], outer[t][h][v]);
    }

    // no K split: round and store this wave's tiles (lane l holds rows
    // n = 4(l/16) .. +3 of batch row m = 16h + l % 16)
    template <bool F16_OUT>
    __device__ __forceinline__ void store_direct(const GemmArgs& a, int tile0) const
    {
#pragma unroll
        for (int h = 0; h < MT; ++h) {
            const int m = 16 * h + (lane & 15);
            if (m >= a.rows) continue;
#pragma unroll
            for (int t = 0; t < NT; ++t) {
                if (t < ntiles) {
                    uint16_t* yp = a.y + (int64_t)m * a.ldy + (tile0 + t) * 16 + (lane >> 4) * 4;
#pragma unroll
                    for (int i = 0; i < 4; ++i)
                        yp[i] = F16_OUT ? f32_to_f16_rne(outer[t][h][i]) : f32_to_bf16_rne(outer[t][h][i]);
                }
            }
        }
    }

    // slot: [ROWS][NT*16] FP32 partial tile of this wave
    __device__ __forceinline__ void store_partial(float* slot) const
    {
        const int n4 = (lane >> 4) * 4;
#pragma unroll
        for (int h = 0; h < MT; ++h) {
            const int m = 16 * h + (lane & 15);
#pragma unroll
            for (int t = 0; t < NT; ++t)
                *reinterpret_cast<f32x4_t*>(slot + m * NT * 16 + t * 16 + n4) = outer[t][h];
        }
    }

    // add another K group's partial tile (slot as written by store_partial)
    __device__ __forceinline__ void add_partial(const float* slot)
    {
        const int n4 = (lane >> 4) * 4;
#pragma unroll
        for (int h = 0; h < MT; ++h) {
            const int m = 16 * h + (lane & 15);
#pragma unroll
            for (int t = 0; t < NT; ++t)
                outer[t][h] += *reinterpret_cast<const f32x4_t*>(slot + m * NT * 16 + t * 16 + n4);
        }
    }

    // one K part's FP32 sums of this wave's tiles into dst[m][n] (row stride N)
    __device__ __forceinline__ void store_part(float* dst, const GemmArgs& a, int tile0) const
    {
#pragma unroll
        for (int h = 0; h < MT; ++h) {
            const int m = 16 * h + (lane & 15);
            if (m >= a.rows) continue;
#pragma unroll
            for (int t = 0; t < NT; ++t)
                if (t < ntiles)
                    *reinterpret_cast<f32x4_t*>(dst + (int64_t)m * a.N + (tile0 + t) * 16 + (lane >> 4) * 4) =
                        outer[t][h];
        }
    }
};

// ---- 3-bit LUT weights, 16-row FP16 MFMA tile -------------------------------
// Quad schedule.  A wave takes the K blocks of its range four at a time (a
// quad; ranges start at multiples of 8 blocks).  Lane group g = lane/16 works
// on block qb+g of quad qb at all four of the quad's loop positions
// p = 0..3: at position p it loads piece p of that block's unit -- the 32
// codes the packed layout gives lane 16p + lane%16, i.e. k = 32s + 8p .. +7
// for MFMA steps s = 0..3 -- and takes the matching activations from block
// qb+g of the staged chunk (a chunk is exactly one quad).  An MFMA sums over
// all 32 of its k slots, so the four lane groups may feed k values of four
// different blocks.  What this buys: a lane meets one (row, group scale) pair
// per quad instead of one per unit, so it scales the map and splits it into
// byte planes once per 4 units (the decode itself is unchanged).
// Group scales come as one 16-byte load per row and run of 8 K blocks, issued
// with the weights of the run's first unit; a unit's place in its run is its
// compile-time position in the unrolled loop, and a lane picks its block's
// scale from the run with one byte permute.  DENSE selects the
// 3-bit-per-code unit layout.
template <int NT, int MT, bool DENSE>
struct MfmaLut {
    static constexpr int KIND = DENSE ? KIND_MFMA_LUT3D : KIND_MFMA_LUT;
    static constexpr bool kSumInRegisters = true;   // K groups combine through add_partial
    static constexpr uint32_t kUnitBytes = DENSE ? 768u : 1024u;
    static constexpr uint32_t kPiece = DENSE ? 12u : 16u;     // one lane's bytes of a unit
    static constexpr int NTILES = NT;
    static constexpr int ROWS = 16 * MT;
    static constexpr int KALIGN = k_align(KIND);   // K blocks per group-scale load
    static constexpr int kXBlock = 16 * MT * kXRowBytes;     // LDS bytes of one staged K block
    template <int XPL> using Stage = XChunk<XPL, MT, chunk_blocks16(KIND, MT)>;
    static_assert(chunk_blocks16(KIND, MT) == 4 * MT, "an activation chunk holds one quad of K blocks");
    struct Unit {
        uint4 w[NT];
        uint4 gv[NT];        // FP16 group scales of 8 K blocks (loaded by a run's first unit only)
    };
    int lane;
    int KB;
    int KB8;
    int ntiles;
    int kb_end;              // end of the wave's K range
    buf_t rw;                // code units of the wave's tiles
    buf_t rg;                // group scales of the wave's tiles
    buf_t rnull;             // zero bytes: loads return zeros
    uint32_t q[4];           // map entries as FP16 pairs
    uint32_t vq;             // this lane's piece 0 in its block of a quad: row lane%16, block g
    uint32_t vqc[NT];        // vq for the current quad, or out of range (block past the K range or tile past N)
    uint32_t gsel;           // byte-permute selector: FP16 element g of four, as a pair
    uint4 gcur[NT];          // group scales of the current run
    LutPlanes pl[NT];        // scaled map of the current quad's block, as byte planes
    f32x4_t acc[NT][MT];

    __device__ MfmaLut(const GemmArgs& a, int l, int tile0) : lane(l), KB(a.KB), KB8((a.KB + 7) / 8), kb_end(0)
    {
        ntiles = max(0, min(NT, a.n_tiles - tile0));
        const int t0 = min(tile0, a.n_tiles);
        rw = make_buf(a.codes + (int64_t)t0 * a.KB * kUnitBytes, (uint32_t)(ntiles * a.KB) * kUnitBytes);
        rg = make_buf(reinterpret_cast<const uint8_t*>(a.scales) + (int64_t)t0 * KB8 * 256,
                      (uint32_t)(ntiles * KB8) * 256u);
        rnull = make_buf(a.codes, 0);
        const uint32_t g = (uint32_t)(l >> 4);
        vq = (uint32_t)(l & 15) * kPiece + g * kUnitBytes;
        gsel = (2 * g) | ((2 * g + 1) << 8) | ((2 * g) << 16) | ((2 * g + 1) << 24);
        const uint32_t* qm = reinterpret_cast<const uint32_t*>(a.qmap);
#pragma unroll
        for (int i = 0; i < 4; ++i) q[i] = qm[i];
#pragma unroll
        for (int t = 0; t < NT; ++t) {
#pragma unroll
            for (int h = 0; h < MT; ++h) acc[t][h] = f32x4_t{0.f, 0.f, 0.f, 0.f};
            gcur[t] = make_uint4(0, 0, 0, 0);
            vqc[t] = kBufOutOfRange;
        }
    }

    __device__ __forceinline__ void set_range(int kb1) { kb_end = kb1; }

    // pos: the unit's position in the unrolled loop, == kb (mod 8).  The
    // lane's block is past the K range only in the last, partial quad of K;
    // its loads then return zeros (valid is not used for the codes: a lane
    // whose block lies inside the range loads at all four positions of its
    // quad, whether or not the position's own block does).
    __device__ __forceinline__ void load(Unit& r, int kb, bool valid, int pos)
    {
        const int p = pos & 3;
        const int qb = kb - p;                           // first K block of the quad
#pragma unroll
        for (int t = 0; t < NT; ++t) {
            if (p == 0) vqc[t] = (t < ntiles && (lane >> 4) < kb_end - qb) ? vq : kBufOutOfRange;
            const uint32_t soff = (uint32_t)(t * KB + (qb < KB ? qb : 0)) * kUnitBytes;
            const uint32_t vo = vqc[t] + (uint32_t)p * 16u * kPiece;
            r.w[t] = DENSE ? buf_load_stream12(rw, vo, soff) : buf_load_stream16(rw, vo, soff);
            if ((pos & 7) == 0)
                r.gv[t] = buf_load16((valid && t < ntiles) ? rg : rnull, (lane & 15) * 16,
                                     (uint32_t)(t * KB8 + (kb >> 3)) * 256u);
        }
    }

    // xblk: the staged block of position pos; its quad's chunk starts p blocks earlier
    __device__ __forceinline__ void compute(const Unit& r, const uint8_t* xblk, int pos)
    {
        const int e = pos & 7;
        const int p = pos & 3;
        if (e == 0) {
#pragma unroll
            for (int t = 0; t < NT; ++t) gcur[t] = r.gv[t];
        }
        // MFMA step s: lane group g holds k = 32s + 8p .. +7 of block qb+g
        const uint8_t* xq = xblk + ((lane >> 4) - p) * kXBlock + (lane & 15) * kXRowBytes + p * 16;
        f16x8_t b[MT][4];
#pragma unroll
        for (int h = 0; h < MT; ++h)
#pragma unroll
            for (int s = 0; s < 4; ++s)
                b[h][s] = __builtin_bit_cast(f16x8_t, *reinterpret_cast<const uint4*>(xq + h * 16 * kXRowBytes + s * 64));
#pragma unroll
        for (int t = 0; t < NT; ++t) {
            if (p == 0) {
                // this lane's group scale (block qb+g: element (e + g) of the run) as an FP16 pair
                const uint32_t gp = e == 0 ? __builtin_amdgcn_perm(gcur[t].y, gcur[t].x, gsel)
                                           : __builtin_amdgcn_perm(gcur[t].w, gcur[t].z, gsel);
                pl[t] = lut_scaled_planes2(q, __builtin_bit_cast(f16x2_t, gp));
            }
            const uint32_t w3 = DENSE ? lut3d_step3_word(r.w[t].x, r.w[t].y, r.w[t].z) : r.w[t].w;
            const uint32_t wd[4] = {r.w[t].x, r.w[t].y, r.w[t].z, w3};
#pragma unroll
            for (int s = 0; s < 4; ++s) {
                const f16x8_t av = lut_decode8(wd[s], pl[t]);
#pragma unroll
                for (int h = 0; h < MT; ++h) acc[t][h] = mfma_f16(av, b[h][s], acc[t][h]);
            }
        }
    }

    template <bool F16_OUT>
    __device__ __forceinline__ void store_direct(const GemmArgs& a, int tile0) const
    {
#pragma unroll
        for (int h = 0; h < MT; ++h) {
            const int m = 16 * h + (lane & 15);
            if (m >= a.rows) continue;
#pragma unroll
            for (int t = 0; t < NT; ++t) {
                if (t < ntiles) {
                    uint16_t* yp = a.y + (int64_t)m * a.ldy + (tile0 + t) * 16 + (lane >> 4) * 4;
#pragma unroll
                    for (int i = 0; i < 4; ++i)
                        yp[i] = F16_OUT ? f32_to_f16_rne(acc[t][h][i]) : f32_to_bf16_rne(acc[t][h][i]);
                }
            }
        }
    }

    __device__ __forceinline__ void store_partial(float* slot) const
    {
        const int n4 = (lane >> 4) * 4;
#pragma unroll
        for (int h = 0; h < MT; ++h) {
            const int m = 16 * h + (lane & 15);
#pragma unroll
            for (int t = 0; t < NT; ++t)
                *reinterpret_cast<f32x4_t*>(slot + m * NT * 16 + t * 16 + n4) = acc[t][h];
        }
    }

    // add another K group's partial tile (slot as written by store_partial)
    __device__ __forceinline__ void add_partial(const float* slot)
    {
        const int n4 = (lane >> 4) * 4;
#pragma unroll
        for (int h = 0; h < MT; ++h) {
            const int m = 16 * h + (lane & 15);
#pragma unroll
            for (int t = 0; t < NT; ++t)
                acc[t][h] += *reinterpret_cast<const f32x4_t*>(slot + m * NT * 16 + t * 16 + n4);
        }
    }

    // one K part's FP32 sums of this wave's tiles into dst[m][n] (row stride N)
    __device__ __forceinline__ void store_part(float* dst, const GemmArgs& a, int tile0) const
    {
#pragma unroll
        for (int h = 0; h < MT; ++h) {
            const int m = 16 * h + (lane & 15);
            if (m >= a.rows) continue;
#pragma unroll
            for (int t = 0; t < NT; ++t)
                if (t < ntiles)
                    *reinterpret_cast<f32x4_t*>(dst + (int64_t)m * a.N + (tile0 + t) * 16 + (lane >> 4) * 4) =
                        acc[t][h];
        }
    }
};

// ---- W8A8 product on the weight-streaming tile (M <= 64) --------------------
// Activation staging for it: a chunk holds two K blocks, each the packed FP8
// activation units of MT row tiles (2 KiB each, in the operand order the
// MFMA reads: lane l's 16 bytes of each 1 KiB half) followed by the 16 MT
// rows' FP32 scales of that block.  The unit pieces are dealt over the K
// group's SN*64 lanes as in XChunk; the scale pieces (16 bytes = 4 rows)
// over the lanes of column-wave 0.  Blocks past the K range, row tiles past
// the padded rows and rows past them read zeros.
template <int XPL, int MT>
struct XqChunk {
    static constexpr int kBlocks = 2;                         // K blocks per chunk
    static constexpr int kUnitPieces = MT * 128;              // 16-byte pieces of one block's units
    static constexpr int kScalePieces = MT * 4;               // ... of one block's row scales
    static constexpr int kBlockBytes = MT * 2048 + MT * 64;
    static constexpr int kChunkBytes = kBlocks * kBlockBytes;
    static constexpr int kXChunkPieces = kBlocks * kUnitPieces;
    static_assert(kBlocks * kScalePieces <= 64, "the scale pieces fit one wave");
    buf_t rx;                 // activation units [Mpad/16][KB] x 2 KiB
    buf_t rs;                 // activation scales [KB][Mpad] FP32
    uint32_t sstride;         // bytes of one K block's scales (Mpad * 4)
    uint32_t vo[XPL];         // byte offset of unit piece i at K block 0, or out of range
    int blk[XPL];             // K block of piece i inside the chunk (large: no piece)
    int dst[XPL];             // LDS offset of piece i inside a chunk buffer (-1: no piece)
    uint4 r[XPL];
    uint32_t svo;             // the lane's scale piece, as vo
    int sblk, sdst;
    uint4 sr;

    __device__ void init(const GemmArgs& a, int lane, int cw, int sn)
    {
        const int mpad = (int)a.ldx;
        const uint8_t* base = reinterpret_cast<const uint8_t*>(a.x);
        rx = make_buf(base, (uint32_t)((int64_t)mpad * a.KB * 128));
        rs = make_buf(base + (int64_t)mpad * a.KB * 128, (uint32_t)((int64_t)a.KB * mpad * 4));
        sstride = (uint32_t)mpad * 4u;
#pragma unroll
        for (int i = 0; i < XPL; ++i) {
            const int q = cw * 64 + lane + i * sn * 64;
            const int b = q / kUnitPieces, rem = q % kUnitPieces, h = rem >> 7, off = rem & 127;
            const bool ok = q < kXChunkPieces && 16 * h < mpad;
            blk[i] = ok ? b : (1 << 29);
            vo[i] = ok ? (uint32_t)((h * a.KB + b) * 2048 + off * 16) : kBufOutOfRange;
            dst[i] = q < kXChunkPieces ? b * kBlockBytes + h * 2048 + off * 16 : -1;
        }
        const int q = cw * 64 + lane;
        const int b = q / kScalePieces, sp = q % kScalePieces;
        const bool ok = q < kBlocks * kScalePieces && 4 * sp < mpad;
        sblk = ok ? b : (1 << 29);
        svo = ok ? (uint32_t)b * sstride + (uint32_t)sp * 16u : kBufOutOfRange;
        sdst = q < kBlocks * kScalePieces ? b * kBlockBytes + MT * 2048 + sp * 16 : -1;
    }

    __device__ __forceinline__ void load(int kb, int kb_end)
    {
        const int lim = kb_end - kb;
#pragma unroll
        for (int i = 0; i < XPL; ++i) r[i] = buf_load16(rx, blk[i] < lim ? vo[i] : kBufOutOfRange, (uint32_t)kb * 2048u);
        sr = buf_load16(rs, sblk < lim ? svo : kBufOutOfRange, (uint32_t)kb * sstride);
    }

    __device__ __forceinline__ void stage(uint8_t* buf) const
    {
#pragma unroll
        for (int i = 0; i < XPL; ++i)
            if (dst[i] >= 0) *reinterpret_cast<uint4*>(buf + dst[i]) = r[i];
        if (sdst >= 0) *reinterpret_cast<uint4*>(buf + sdst) = sr;
    }
};

// One 16-column weight tile per wave, streamed as in the FP8 decode tile; per
// K block one v_mfma_f32_16x16x128_f8f6f4 per row tile (A = the activation
// unit, B = the weight unit: D[m][n] over the block's 128 codes) folded onto
// FP32 outer accumulators times sx[m][kb] * sw[n/128][kb].  Operands,
// products and fold are those of the W8A8 tile kernel, in the same order, so
// a plan with one K group gives its bits for the same K parts.  Lane l holds
// rows 16h + 4(l/16) .. +3 of column l % 16 of row tile h.
template <int MT>
struct MfmaW8A8 : Fp8Stream<1> {
    static constexpr int KIND = KIND_W8A8_STREAM;
    static constexpr bool kSumInRegisters = true;   // K groups combine through add_partial
    static constexpr int NTILES = 1;
    static constexpr int ROWS = 16 * MT;
    static constexpr int KALIGN = k_align(KIND);
    template <int XPL> using Stage = XqChunk<XPL, MT>;
    using typename Fp8Stream<1>::Unit;
    using Fp8Stream<1>::lane;
    using Fp8Stream<1>::ntiles;
    f32x4_t outer[MT];

    __device__ MfmaW8A8(const GemmArgs& a, int l, int tile0) : Fp8Stream<1>(a, l, tile0)
    {
#pragma unroll
        for (int h = 0; h < MT; ++h) outer[h] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    }

    __device__ __forceinline__ void compute(const Unit& r, const uint8_t* xblk, int)
    {
        const i32x8_t bw = i32x8_t{(int)r.w[0][0].x, (int)r.w[0][0].y, (int)r.w[0][0].z, (int)r.w[0][0].w,
                                   (int)r.w[0][1].x, (int)r.w[0][1].y, (int)r.w[0][1].z, (int)r.w[0][1].w};
        f32x4_t blk[MT];
#pragma unroll
        for (int h = 0; h < MT; ++h) blk[h] = mfma_fp8(lds_frag(xblk + h * 2048, lane), bw, f32x4_t{0.f, 0.f, 0.f, 0.f});
#pragma unroll
        for (int h = 0; h < MT; ++h) {
            const f32x4_t sx =
                *reinterpret_cast<const f32x4_t*>(xblk + MT * 2048 + (16 * h + 4 * (lane >> 4)) * 4);
#pragma unroll
            for (int q = 0; q < 4; ++q) outer[h][q] = __builtin_fmaf(blk[h][q], sx[q] * r.s, outer[h][q]);
        }
    }

    template <bool F16_OUT>
    __device__ __forceinline__ void store_direct(const GemmArgs& a, int tile0) const
    {
        if (ntiles < 1) return;
        const int n = tile0 * 16 + (lane & 15);
#pragma unroll
        for (int h = 0; h < MT; ++h)
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const int m = 16 * h + 4 * (lane >> 4) + q;
                if (m < a.rows)
                    a.y[(int64_t)m * a.ldy + n] = F16_OUT ? f32_to_f16_rne(outer[h][q]) : f32_to_bf16_rne(outer[h][q]);
            }
    }

    // slot: [ROWS][16] FP32 partial tile of this wave, lane-major
    __device__ __forceinline__ void store_partial(float* slot) const
    {
#pragma unroll
        for (int h = 0; h < MT; ++h) *reinterpret_cast<f32x4_t*>(slot + h * 256 + lane * 4) = outer[h];
    }

    __device__ __forceinline__ void add_partial(const float* slot)
    {
#pragma unroll
        for (int h = 0; h < MT; ++h) outer[h] += *reinterpret_cast<const f32x4_t*>(slot + h * 256 + lane * 4);
    }

    __device__ __forceinline__ void store_part(float* dst, const GemmArgs& a, int tile0) const
    {
        if (ntiles < 1) return;
        const int n = tile0 * 16 + (lane & 15);
#pragma unroll
        for (int h = 0; h < MT; ++h)
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const int m = 16 * h + 4 * (lane >> 4) + q;
                if (m < a.rows) dst[(int64_t)m * a.N + n] = outer[h][q];
            }
    }
};

// ---- FP8 weights, strict-K-order GEMV (MR <= 4 rows) ------------------------
// One tile per wave, loaded exactly as the MFMA tile loads it: lane l holds
// column c = l%16 and, within each 32-wide MFMA step s of a K block, the
// 8-wide run k = 32s + 8g .. +7 of lane group g = l/16.  Each (lane, row)
// keeps one FP32 accumulator that takes its products x*w in strictly
// increasing k over the lane's runs; each 128-K block is folded onto the
// outer accumulator times the block scale.  The four lane groups of a column
// are then summed by a fixed butterfly ((g0+g1) + (g2+g3)), and a K split
// across waves in K-group order.  The arithmetic of a row never depends on
// M, so row r of an M-row call equals the same row of a 1-row call bit for
// bit.
template <int MR>
struct GemvFp8 : Fp8Stream<1> {
    static constexpr int KIND = KIND_GEMV_FP8;
    static constexpr bool kSumInRegisters = false;  // K groups combine in LDS by all threads
    static constexpr int NTILES = 1;
    static constexpr int ROWS = 16;       // rows of the partial-tile slot (MR used)
    static constexpr int KALIGN = 1;
    template <int XPL> using Stage = XChunkF32<XPL>;
    float outer[MR];

    __device__ GemvFp8(const GemmArgs& a, int l, int tile0) : Fp8Stream<1>(a, l, tile0)
    {
#pragma unroll
        for (int m = 0; m < MR; ++m) outer[m] = 0.f;
    }

    __device__ __forceinline__ void compute(const Unit& r, const uint8_t* xblk, int)
    {
        const int g = lane >> 4;
        float blk[MR];
#pragma unroll
        for (int m = 0; m < MR; ++m) blk[m] = 0.f;
#pragma unroll
        for (int s = 0; s < 4; ++s) {   // increasing k: step s covers k = 32s + 8g .. +7
            const uint4 w = r.w[0][s >> 1];
            const uint32_t d0 = (s & 1) ? w.z : w.x, d1 = (s & 1) ? w.w : w.y;
            const f32x2_t w0 = e4m3x2_to_f32x2<false>(d0), w1 = e4m3x2_to_f32x2<true>(d0);
            const f32x2_t w2 = e4m3x2_to_f32x2<false>(d1), w3 = e4m3x2_to_f32x2<true>(d1);
            const float wf[8] = {w0[0], w0[1], w1[0], w1[1], w2[0], w2[1], w3[0], w3[1]};
#pragma unroll
            for (int m = 0; m < MR; ++m) {
                const float* xp = reinterpret_cast<const float*>(xblk + m * 512 + (32 * s + 8 * g) * 4);
                const f32x4_t xa = *reinterpret_cast<const f32x4_t*>(xp);
                const f32x4_t xc = *reinterpret_cast<const f32x4_t*>(xp + 4);
#pragma unroll
                for (int i = 0; i < 4; ++i) blk[m] = __builtin_fmaf(xa[i], wf[i], blk[m]);
#pragma unroll
                for (int i = 0; i < 4; ++i) blk[m] = __builtin_fmaf(xc[i], wf[4 + i], blk[m]);
            }
            // keep each step's activation reads next to their use: hoisting
            // them across steps and units would hold MR*32 floats per unit
#pragma unroll
            for (int m = 0; m < MR; ++m) asm volatile("" : "+v"(blk[m])::"memory");
        }
#pragma unroll
        for (int m = 0; m < MR; ++m) outer[m] = __builtin_fmaf(r.s, blk[m], outer[m]);
    }

    // the column's total over the four lane groups (identical in all four)
    __device__ __forceinline__ float column_sum(int m) const
    {
        float v = outer[m];
        v += __shfl_xor(v, 16);
        v += __shfl_xor(v, 32);
        return v;
    }

    template <bool F16_OUT>
    __device__ __forceinline__ void store_direct(const GemmArgs& a, int tile0) const
    {
        float v[MR];
#pragma unroll
        for (int m = 0; m < MR; ++m) v[m] = column_sum(m);
        if (lane >= 16 || ntiles < 1) return;
#pragma unroll
        for (int m = 0; m < MR; ++m)
            if (m < a.rows) a.y[(int64_t)m * a.ldy + tile0 * 16 + lane] = f32_to_bf16_rne(v[m]);
    }

    // slot: [16 rows][16] FP32 partial tile of this wave (rows < MR written)
    __device__ __forceinline__ void store_partial(float* slot) const
    {
        float v[MR];
#pragma unroll
        for (int m = 0; m < MR; ++m) v[m] = column_sum(m);
        if (lane < 16) {
#pragma unroll
            for (int m = 0; m < MR; ++m) slot[m * 16 + lane] = v[m];
        }
    }

    // one K part's FP32 sums of this wave's columns into dst[m][n] (row stride N)
    __device__ __forceinline__ void store_part(float* dst, const GemmArgs& a, int tile0) const
    {
        float v[MR];
#pragma unroll
        for (int m = 0; m < MR; ++m) v[m] = column_sum(m);
        if (lane >= 16 || ntiles < 1) return;
#pragma unroll
        for (int m = 0; m < MR; ++m)
            if (m < a.rows) dst[(int64_t)m * a.N + tile0 * 16 + lane] = v[m];
    }
};

// ======================================================================
// The GEMM kernel.  Grid: one work-group per column group of SN*NT tiles
// (x) and K part (y).  Block: S = SN*SK waves; wave w is column-wave
// cw = w % SN (tiles cw*NT .. +NT of the group) in K group kg = w / SN (the
// kg-th of SK contiguous runs of the part's K blocks).  Each wave streams its
// units through a ring of D+1 register slots with D units in flight.  The SN
// waves of a K group share staged activation chunks (see XChunk).  After the
// K loop every wave stores its tiles (SK = 1) or parks its partial tile in
// LDS and the work-group sums the SK partials of each column in K-group
// order; the result is rounded into y (KP = 1) or stored as FP32 to the
// part's slab of the workspace.
// ======================================================================
constexpr int gcd_c(int a, int b) { return b == 0 ? a : gcd_c(b, a % b); }
constexpr int lcm_c(int a, int b) { return a / gcd_c(a, b) * b; }

template <class Pol, int D, int XPL, bool F16_OUT>
__global__ void __launch_bounds__(64 * max_split_xpl(Pol::KIND, Pol::NTILES, XPL))
gemm_kernel(GemmArgs a)
{
    using XS = typename Pol::template Stage<XPL>;
    constexpr int NT = Pol::NTILES;
    constexpr int TW = NT * 16;                       // columns of one wave
    constexpr int R = D + 1;                          // ring slots
    constexpr int CH = XS::kBlocks;                   // K blocks per activation chunk
    constexpr int PR = Pol::ROWS;                     // rows of a partial tile
    // steps per unrolled body: whole ring turns, an even number of chunks and
    // whole scale runs, so ring slots, chunk buffers and a unit's place in its
    // scale run are compile-time in the body
    constexpr int L = lcm_c(lcm_c(R, 2 * CH), Pol::KALIGN);
    extern __shared__ __attribute__((aligned(16))) uint8_t lds[];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int S = blockDim.x >> 6;
    const int SN = a.sn;
    const int SK = S / SN;
    const int cw = wave % SN, kg = wave / SN;
    // The work-group's K part (grid y) covers aligned K blocks [pa0, pa1) and
    // its K group kg covers K blocks [kb0, kb1) of that; ranges start at
    // multiples of KALIGN
    constexpr int KA = Pol::KALIGN;
    const int KBA = (a.KB + KA - 1) / KA;
    const int kpart = blockIdx.y;
    const int pa0 = (KBA * kpart) / a.kp, pa1 = (KBA * (kpart + 1)) / a.kp;
    const int PBA = pa1 - pa0;
    const int kb0 = min(a.KB, KA * (pa0 + (PBA * kg) / SK));
    const int kb1 = min(a.KB, KA * (pa0 + (PBA * (kg + 1)) / SK));
    const int len = kb1 - kb0;
    const int steps = KA * ((PBA + SK - 1) / SK);      // the longest K range; every wave runs it
    const int tile0 = (blockIdx.x * SN + cw) * NT;

    Pol pol(a, lane, tile0);
    pol.set_range(kb1);
    {
        typename Pol::Unit r[R];
        uint8_t* xb = lds + kg * 2 * XS::kChunkBytes;   // this K group's two chunk buffers
        XS xc;
        xc.init(a, lane, cw, SN);
        xc.load(kb0, kb1);
        // FP8 tile: let the first activation chunk's requests reach memory
        // ahead of the weight ring's first burst, which they would otherwise
        // queue behind (~256 cycles; attention K/V 7.7 -> 7.2 us, the large
        // shapes within 1%; the LUT tile measured no gain from it)
        if constexpr (Pol::KIND == KIND_MFMA_FP8 || Pol::KIND == KIND_W8A8_STREAM) __builtin_amdgcn_s_sleep(4);
#pragma unroll
        for (int i = 0; i < D; ++i) pol.load(r[i], kb0 + i, i < len, i);
        xc.stage(xb);
        xc.load(kb0 + CH, kb1);
        if (SN > 1) __syncthreads();
        for (int i = 0; i < steps; i += L) {
#pragma unroll
            for (int j = 0; j < L; ++j) {
                const int step = i + j;
                const int par = (j / CH) & 1;         // buffer of the current chunk
                pol.load(r[(j + D) % R], kb0 + step + D, step + D < len, j + D);
                // past the K range the slot holds zero weights and a zero
                // scale and the chunk zero activations: the update adds +0
                pol.compute(r[j % R], xb + par * XS::kChunkBytes + (j % CH) * XS::kBlockBytes, j);
                if ((j + 1) % CH == 0) {
                    xc.stage(xb + (par ^ 1) * XS::kChunkBytes);
                    xc.load(kb0 + step + 1 + CH, kb1);
                    if (SN > 1) __syncthreads();
                    if (step + 1 >= steps) break;     // uniform: every wave leaves here
                }
            }
        }
    }
    float* const wsp = a.ws + (int64_t)kpart * a.rows * a.N;  // this K part's partials (a.kp > 1)
    if constexpr (Pol::kSumInRegisters) if (SK > 1) {
        // K groups 1..SK-1 park their partial tiles in LDS; each K-group-0
        // wave adds those of its columns in K-group order and stores its
        // tiles itself: ((kg0 + kg1) + kg2) + ..., the same sums, in the same
        // order, as an all-thread reduction, without its second pass over LDS
        __syncthreads();   // every wave is done with the staging buffers
        float* part = reinterpret_cast<float*>(lds);           // [S][PR][TW]
        if (kg > 0) pol.store_partial(part + wave * PR * TW);
        __syncthreads();
        if (kg > 0) return;
        for (int k = 1; k < SK; ++k) pol.add_partial(part + (k * SN + cw) * PR * TW);
    }
    if (Pol::kSumInRegisters || SK == 1) {
        if (a.kp == 1) pol.template store_direct<F16_OUT>(a, tile0);
        else pol.store_part(wsp, a, tile0);
        return;
    }
    __syncthreads();   // every wave is done with the staging buffers
    float* part = reinterpret_cast<float*>(lds);           // [S][PR][TW]
    pol.store_partial(part + wave * PR * TW);
    __syncthreads();

    const int cols = SN * TW;
    const int nout = a.rows * cols;
    for (int e = tid; e < nout; e += blockDim.x) {
        const int m = e / cols, c = e - m * cols;
        const int w0 = c / TW, cc = c - w0 * TW;
        const float* p = part + (w0 * PR + m) * TW + cc;    // wave w0 (K group 0)
        float v = p[0];
        for (int k = 1; k < SK; ++k) v += p[(int64_t)k * SN * PR * TW];
        const int64_t n = (int64_t)blockIdx.x * cols + c;
        if (n < a.N) {
            if (a.kp == 1) a.y[m * a.ldy + n] = F16_OUT ? f32_to_f16_rne(v) : f32_to_bf16_rne(v);
            else wsp[m * a.N + n] = v;
        }
    }
}

template <class Pol, int XPL>
int gemm_lds_bytes(int split, int sn)
{
    const int stage = (split / sn) * 2 * Pol::template Stage<XPL>::kChunkBytes;
    const int parts = split * Pol::ROWS * Pol::NTILES * 16 * 4;
    return stage > parts ? stage : parts;
}

// ======================================================================
// Pack / unpack kernels (offline; not on the timed path).
// ======================================================================

__device__ __forceinline__ uint4 gather16(const uint8_t* src)
{
    if ((reinterpret_cast<uintptr_t>(src) & 15) == 0) return *reinterpret_cast<const uint4*>(src);
    uint32_t d[4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
        d[i] = (uint32_t)src[4 * i] | ((uint32_t)src[4 * i + 1] << 8) | ((uint32_t)src[4 * i + 2] << 16) |
               ((uint32_t)src[4 * i + 3] << 24);
    return make_uint4(d[0], d[1], d[2], d[3]);
}

// the 8 codes of (row n, MFMA step s, lane group g) start at k = 128kb + 32s + 8g
__device__ __forceinline__ uint2 gather8(const uint8_t* src)
{
    if ((reinterpret_cast<uintptr_t>(src) & 7) == 0) return *reinterpret_cast<const uint2*>(src);
    uint32_t d[2];
#pragma unroll
    for (int i = 0; i < 2; ++i)
        d[i] = (uint32_t)src[4 * i] | ((uint32_t)src[4 * i + 1] << 8) | ((uint32_t)src[4 * i + 2] << 16) |
               ((uint32_t)src[4 * i + 3] << 24);
    return make_uint2(d[0], d[1]);
}

__global__ void pack_fp8_kernel(const uint8_t* __restrict__ w, int64_t ldw, const float* __restrict__ scales,
                                int64_t N, int64_t K, uint8_t* __restrict__ packed)
{
    const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    const int64_t KB = K / 128;
    if (idx < N * K / 16) {
        const int l = (int)(idx & 63), j = (int)((idx >> 6) & 1);
        const int64_t unit = idx >> 7;
        const int64_t t = unit / KB, kb = unit - t * KB;
        const int64_t n = t * 16 + (l & 15);
        const uint8_t* row = w + n * ldw + kb * 128 + (l >> 4) * 8;
        const uint2 a = gather8(row + 64 * j), b = gather8(row + 64 * j + 32);
        reinterpret_cast<uint4*>(packed)[idx] = make_uint4(a.x, a.y, b.x, b.y);
    }
    if (idx < (N / 128) * KB) reinterpret_cast<float*>(packed + N * K)[idx] = scales[idx];
}

__global__ void clear_status_kernel(uint32_t* status) { status[threadIdx.x] = 0u; }

__global__ void pack_lut3_kernel(const uint8_t* __restrict__ codes, int64_t ldc, const uint16_t* __restrict__ qmap,
                                 const uint16_t* __restrict__ scales, int64_t N, int64_t K,
                                 uint8_t* __restrict__ packed, uint32_t* status, int dense)
{
    const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    const int64_t KB = K / 128;
    const int64_t n_tiles = N / 16;
    if (idx < N * K / 32) {
        const int l = (int)(idx & 63);
        const int64_t unit = idx >> 6;
        const int64_t t = unit / KB, kb = unit - t * KB;
        const int64_t n = t * 16 + (l & 15);
        const uint8_t* src = codes + n * ldc + kb * 128 + (l >> 4) * 8;
        uint32_t d[4];
        uint32_t bad = 0;
#pragma unroll
        for (int s = 0; s < 4; ++s) {
            uint32_t word = 0;
#pragma unroll
            for (int b = 0; b < 4; ++b) {
                const uint32_t lo = src[32 * s + b], hi = src[32 * s + b + 4];
                bad |= (lo | hi) & ~7u;
                word |= ((lo & 15u) | ((hi & 15u) << 4)) << (8 * b);
            }
            d[s] = word;
        }
        if (dense) {
            // step 3's code bit i goes to bits 3 and 7 of dword i
            uint32_t o[3];
#pragma unroll
            for (int i = 0; i < 3; ++i) o[i] = (d[i] & 0x77777777u) | (((d[3] >> i) & 0x11111111u) << 3);
            uint32_t* dst = reinterpret_cast<uint32_t*>(packed) + idx * 3;
            dst[0] = o[0];
            dst[1] = o[1];
            dst[2] = o[2];
        } else {
            reinterpret_cast<uint4*>(packed)[idx] = make_uint4(d[0], d[1], d[2], d[3]);
        }
        if (bad) atomicOr(status, 1u);
    }
    uint16_t* sc_out = reinterpret_cast<uint16_t*>(packed + (dense ? N * K / 8 * 3 : N * K / 2));
    const int64_t KB8 = (KB + 7) / 8;
    if (idx < n_tiles * KB8 * 128) {
        const int64_t e = idx & 7, r = (idx >> 3) & 15, grp = idx >> 7;
        const int64_t t = grp / KB8, kb = (grp - t * KB8) * 8 + e;
        sc_out[idx] = kb < KB ? scales[(t * 16 + r) * KB + kb] : (uint16_t)0;
    }
    if (idx < 8) sc_out[n_tiles * KB8 * 128 + idx] = qmap[idx];
}

__global__ void unpack_fp8_kernel(const uint8_t* __restrict__ packed, int64_t N, int64_t K, void* out, int f32_out)
{
    const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (idx >= N * K / 16) return;
    const int64_t KB = K / 128;
    const int l = (int)(idx & 63), j = (int)((idx >> 6) & 1);
    const int64_t unit = idx >> 7;
    const int64_t t = unit / KB, kb = unit - t * KB;
    const int64_t n = t * 16 + (l & 15);
    const int64_t k0 = kb * 128 + 64 * j + (l >> 4) * 8;   // bytes 0..7 at k0, bytes 8..15 at k0 + 32
    const uint4 w = reinterpret_cast<const uint4*>(packed)[idx];
    if (f32_out) {
        const uint32_t d[4] = {w.x, w.y, w.z, w.w};
        float* o = reinterpret_cast<float*>(out) + n * K + k0;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const f32x2_t lo = e4m3x2_to_f32x2<false>(d[i]);
            const f32x2_t hi = e4m3x2_to_f32x2<true>(d[i]);
            float* q = o + (i >> 1) * 32 + (i & 1) * 4;
            q[0] = lo[0];
            q[1] = lo[1];
            q[2] = hi[0];
            q[3] = hi[1];
        }
    } else {
        uint16_t* o = reinterpret_cast<uint16_t*>(out) + n * K + k0;
        const bf16x8_t a = e4m3x8_to_bf16x8(w.x, w.y), b = e4m3x8_to_bf16x8(w.z, w.w);
        *reinterpret_cast<uint4*>(o) = __builtin_bit_cast(uint4, a);
        *reinterpret_cast<uint4*>(o + 32) = __builtin_bit_cast(uint4, b);
    }
}

__global__ void unpack_lut3_kernel(const uint8_t* __restrict__ packed, int64_t N, int64_t K, uint16_t* out, int dense)
{
    const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (idx >= N * K / 32) return;
    const int64_t KB = K / 128;
    const int64_t n_tiles = N / 16;
    const int l = (int)(idx & 63);
    const int64_t unit = idx >> 6;
    const int64_t t = unit / KB, kb = unit - t * KB;
    const int64_t n = t * 16 + (l & 15);
    const int64_t KB8 = (KB + 7) / 8;
    const uint16_t* sc = reinterpret_cast<const uint16_t*>(packed + (dense ? N * K / 8 * 3 : N * K / 2));
    const uint32_t* qm = reinterpret_cast<const uint32_t*>(sc + n_tiles * KB8 * 128);
    const uint32_t q[4] = {qm[0], qm[1], qm[2], qm[3]};
    const uint16_t g = sc[((t * KB8 + kb / 8) * 16 + (l & 15)) * 8 + kb % 8];
    const LutPlanes pl = lut_scaled_planes(q, __builtin_bit_cast(_Float16, g));
    uint32_t d[4];
    if (dense) {
        const uint32_t* src = reinterpret_cast<const uint32_t*>(packed) + idx * 3;
        d[0] = src[0];
        d[1] = src[1];
        d[2] = src[2];
        d[3] = lut3d_step3_word(d[0], d[1], d[2]);
    } else {
        const uint4 w = reinterpret_cast<const uint4*>(packed)[idx];
        d[0] = w.x;
        d[1] = w.y;
        d[2] = w.z;
        d[3] = w.w;
    }
    uint16_t* o = out + n * K + kb * 128 + (l >> 4) * 8;
#pragma unroll
    for (int s = 0; s < 4; ++s)
        *reinterpret_cast<uint4*>(o + 32 * s) = __builtin_bit_cast(uint4, lut_decode8(d[s], pl));
}

// ----------------------------------------------------------- K-part sum
// y[m][n] = the sum of the K parts' FP32 partials ws[p][m][n] taken in order
// p = 0, 1, .., kp-1, rounded once (RNE) to BF16 or FP16.  A thread takes 4
// consecutive columns (N is a multiple of 16).  The parts are loaded
// kSumBatch at a time, all of a batch's loads in flight together, and then
// added in order: one memory round trip per batch rather than per part.
constexpr int kSumBatch = 8;

__global__ void __launch_bounds__(256) reduce_parts_kernel(const float* __restrict__ ws, int kp, int rows, int N,
                                                           uint16_t* __restrict__ y, int64_t ldy, int f16_out)
{
    const int64_t q = (int64_t)blockIdx.x * 256 + threadIdx.x;   // 4-column group
    const int64_t groups = (int64_t)N / 4;
    if (q >= (int64_t)rows * groups) return;
    const int64_t m = q / groups, n = (q - m * groups) * 4;
    const float* p = ws + m * N + n;
    const int64_t part = (int64_t)rows * N;
    f32x4_t v = *reinterpret_cast<const f32x4_t*>(p);
    for (int k0 = 1; k0 < kp; k0 += kSumBatch) {
        f32x4_t w[kSumBatch];
#pragma unroll
        for (int j = 0; j < kSumBatch; ++j)
            if (k0 + j < kp) w[j] = *reinterpret_cast<const f32x4_t*>(p + (k0 + j) * part);
#pragma unroll
        for (int j = 0; j < kSumBatch; ++j)
            if (k0 + j < kp) {
#pragma unroll
                for (int i = 0; i < 4; ++i) v[i] += w[j][i];
            }
    }
    uint16_t* yp = y + m * ldy + n;
#pragma unroll
    for (int i = 0; i < 4; ++i) yp[i] = f16_out ? f32_to_f16_rne(v[i]) : f32_to_bf16_rne(v[i]);
}

// ======================================================================
// Launchers
// ======================================================================

// A launch with more than 64 KiB of dynamic LDS needs the kernel's limit
// raised first.  It is raised once per kernel instantiation and device, to the
// whole 160 KiB of a compute unit (a limit, not a reservation), and later
// launches only test a bit: no runtime call on the hot path.  `done` is the
// instantiation's own mask of devices already set.
static hipError_t allow_big_lds(const void* fn, size_t lds, std::atomic<uint64_t>& done)
{
    if (lds <= 64 * 1024) return hipSuccess;
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    const uint64_t bit = dev < 64 ? (uint64_t)1 << dev : 0;
    if (bit && (done.load(std::memory_order_acquire) & bit)) return hipSuccess;
    e = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, kLdsBytes);
    if (e == hipSuccess) done.fetch_or(bit, std::memory_order_release);
    return e;
}

template <class Pol, int D, int XPL, bool F16>
static hipError_t launch_one(const GemmArgs& a, int split, hipStream_t s)
{
    auto fn = gemm_kernel<Pol, D, XPL, F16>;
    static std::atomic<uint64_t> big_lds_set{0};
    const size_t lds = (size_t)gemm_lds_bytes<Pol, XPL>(split, a.sn);
    hipError_t e = allow_big_lds(reinterpret_cast<const void*>(fn), lds, big_lds_set);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(fn, dim3(a.n_cg, a.kp), dim3(split * 64), lds, s, a);
    return hipGetLastError();
}

// whether some SN in 1..8 stages XPL activation pieces per lane for this kind
// and row-tile count (only those kernels are built)
constexpr bool xpl_used(int kind, int mt, int xpl)
{
    for (int sn = 1; sn <= 8; ++sn)
        if (x_pieces_per_lane(kind, sn, mt) == xpl) return true;
    return false;
}

template <int NT, int MT, int XPL>
static hipError_t launch_mfma(int kind, const GemmArgs& a, int split, hipStream_t s)
{
    if (kind == KIND_MFMA_FP8) {
        if constexpr (xpl_used(KIND_MFMA_FP8, MT, XPL)) {
            if constexpr (MT == 1)
                if (split == a.sn)   // one K group: each wave streams its whole K part alone
                    return launch_one<MfmaFp8<NT, MT>, kDepthMfmaFp8Solo, XPL, false>(a, split, s);
            return launch_one<MfmaFp8<NT, MT>, kDepthMfmaFp8, XPL, false>(a, split, s);
        }
        return hipErrorInvalidValue;
    }
    // 32-row LUT tiles run only where lut_single_pass allows (4, 5, 6 or 8 pieces)
    if constexpr (xpl_used(KIND_MFMA_LUT, MT, XPL) && (MT == 1 || (XPL >= 4 && XPL <= 6) || XPL == 8)) {
        if (kind == KIND_MFMA_LUT3D) return launch_one<MfmaLut<NT, MT, true>, lut_depth(NT), XPL, true>(a, split, s);
        return launch_one<MfmaLut<NT, MT, false>, lut_depth(NT), XPL, true>(a, split, s);
    }
    return hipErrorInvalidValue;
}

template <int NT, int MT>
static hipError_t launch_nt(int kind, const GemmArgs& a, int split, hipStream_t s)
{
    switch (x_pieces_per_lane(kind, a.sn, MT)) {
    case 16: return launch_mfma<NT, MT, 16>(kind, a, split, s);
    case 8: return launch_mfma<NT, MT, 8>(kind, a, split, s);
    case 6: return launch_mfma<NT, MT, 6>(kind, a, split, s);
    case 5: return launch_mfma<NT, MT, 5>(kind, a, split, s);
    case 4: return launch_mfma<NT, MT, 4>(kind, a, split, s);
    case 3: return launch_mfma<NT, MT, 3>(kind, a, split, s);
    case 2: return launch_mfma<NT, MT, 2>(kind, a, split, s);
    case 1: return launch_mfma<NT, MT, 1>(kind, a, split, s);
    default: return hipErrorInvalidValue;
    }
}

template <int MR>
static hipError_t launch_gemv(const GemmArgs& a, int split, hipStream_t s)
{
    switch (x_pieces_per_lane(KIND_GEMV_FP8, a.sn)) {
    case 4: return launch_one<GemvFp8<MR>, kDepthGemv, 4, false>(a, split, s);
    case 2: return launch_one<GemvFp8<MR>, kDepthGemv, 2, false>(a, split, s);
    case 1: return launch_one<GemvFp8<MR>, kDepthGemv, 1, false>(a, split, s);
    default: return hipErrorInvalidValue;
    }
}

static hipError_t launch_gemm_parts(int kind, int nt, int gemv_rows, const GemmArgs& a, int split,
                                    hipStream_t stream);

hipError_t launch_gemm(int kind, int nt, int gemv_rows, const GemmArgs& a, int split, hipStream_t stream)
{
    if (a.kp < 1 || a.kp > kMaxKParts || (a.kp > 1 && !a.ws)) return hipErrorInvalidValue;
    hipError_t e = launch_gemm_parts(kind, nt, gemv_rows, a, split, stream);
    if (e != hipSuccess || a.kp == 1) return e;
    return launch_sum_parts(a.ws, a.kp, a.rows, a.N, a.y, a.ldy, is_lut_kind(kind), stream);
}

hipError_t launch_sum_parts(const float* ws, int kp, int rows, int N, uint16_t* y, int64_t ldy, bool f16_out,
                            hipStream_t stream)
{
    const int64_t groups = (int64_t)rows * (N / 4);
    hipLaunchKernelGGL(reduce_parts_kernel, dim3((unsigned)((groups + 255) / 256)), dim3(256), 0, stream, ws, kp,
                       rows, N, y, ldy, (int)f16_out);
    return hipGetLastError();
}

// W8A8 streaming tile: MT row tiles cover the padded rows (1, 2 or 4)
template <int MT>
static hipError_t launch_w8s(const GemmArgs& a, int split, hipStream_t s)
{
    const int d = split == a.sn ? kDepthMfmaFp8Solo : kDepthMfmaFp8;
    switch (x_pieces_per_lane(KIND_W8A8_STREAM, a.sn, MT)) {
#define WQ_W8S_CASE(X)                                                                              \
    case X:                                                                                         \
        if constexpr (xpl_used(KIND_W8A8_STREAM, MT, X))                                            \
            return d == kDepthMfmaFp8Solo ? launch_one<MfmaW8A8<MT>, kDepthMfmaFp8Solo, X, false>(a, split, s) \
                                          : launch_one<MfmaW8A8<MT>, kDepthMfmaFp8, X, false>(a, split, s);   \
        return hipErrorInvalidValue;
        WQ_W8S_CASE(16) WQ_W8S_CASE(8) WQ_W8S_CASE(6) WQ_W8S_CASE(5) WQ_W8S_CASE(4) WQ_W8S_CASE(3)
        WQ_W8S_CASE(2) WQ_W8S_CASE(1)
#undef WQ_W8S_CASE
    default: return hipErrorInvalidValue;
    }
}

static hipError_t launch_gemm_parts(int kind, int nt, int gemv_rows, const GemmArgs& a, int split,
                                    hipStream_t stream)
{
    if (!split_ok(kind, nt, a.sn, split)) return hipErrorInvalidValue;
    if (kind == KIND_W8A8_STREAM) {
        if (a.rows <= 16) return launch_w8s<1>(a, split, stream);
        if (a.rows <= 32) return launch_w8s<2>(a, split, stream);
        if (a.rows <= 64) return launch_w8s<4>(a, split, stream);
        return hipErrorInvalidValue;
    }
    if (kind == KIND_GEMV_FP8) {
        switch (gemv_rows) {
        case 1: return launch_gemv<1>(a, split, stream);
        case 2: return launch_gemv<2>(a, split, stream);
        case 3: return launch_gemv<3>(a, split, stream);
        case 4: return launch_gemv<4>(a, split, stream);
        default: return hipErrorInvalidValue;
        }
    }
    if (kind != KIND_MFMA_FP8 && !is_lut_kind(kind)) return hipErrorInvalidValue;
    if (a.rows > 16) {
        if (nt != 1 || a.rows > 32) return hipErrorInvalidValue;
        return launch_nt<1, 2>(kind, a, split, stream);
    }
    switch (nt) {
    case 1: return launch_nt<1, 1>(kind, a, split, stream);
    case 2: return launch_nt<2, 1>(kind, a, split, stream);
    default: return hipErrorInvalidValue;
    }
}

static unsigned blocks_for(int64_t n) { return (unsigned)((n + 255) / 256); }

hipError_t launch_pack_fp8(const uint8_t* w, int64_t ldw, const float* scales, int64_t N, int64_t K,
                           uint8_t* packed, hipStream_t stream)
{
    hipLaunchKernelGGL(pack_fp8_kernel, dim3(blocks_for(N * K / 16)), dim3(256), 0, stream, w, ldw, scales, N, K,
                       packed);
    return hipGetLastError();
}

hipError_t launch_pack_lut3(const uint8_t* codes, int64_t ldc, const uint16_t* qmap, const uint16_t* scales,
                            int64_t N, int64_t K, uint8_t* packed, uint32_t* status, bool dense, hipStream_t stream)
{
    hipLaunchKernelGGL(clear_status_kernel, dim3(1), dim3(4), 0, stream, status);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    const int64_t n_scales = (N / 16) * ((K / 128 + 7) / 8) * 128;
    const int64_t n = N * K / 32 > n_scales ? N * K / 32 : n_scales;
    hipLaunchKernelGGL(pack_lut3_kernel, dim3(blocks_for(n)), dim3(256), 0, stream, codes, ldc, qmap, scales, N, K,
                       packed, status, (int)dense);
    return hipGetLastError();
}

hipError_t launch_unpack_fp8(const uint8_t* packed, int64_t N, int64_t K, void* out, bool f32_out, hipStream_t stream)
{
    hipLaunchKernelGGL(unpack_fp8_kernel, dim3(blocks_for(N * K / 16)), dim3(256), 0, stream, packed, N, K, out,
                       (int)f32_out);
    return hipGetLastError();
}

hipError_t launch_unpack_lut3(const uint8_t* packed, int64_t N, int64_t K, uint16_t* out, bool dense,
                              hipStream_t stream)
{
    hipLaunchKernelGGL(unpack_lut3_kernel, dim3(blocks_for(N * K / 32)), dim3(256), 0, stream, packed, N, K, out,
                       (int)dense);
    return hipGetLastError();
}

}  // namespace wq
