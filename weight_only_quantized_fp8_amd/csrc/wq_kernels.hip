// gfx950 kernels of libwq: the decode GEMM (MFMA tile and strict-order GEMV)
// for FP8 block-scaled and 3-bit LUT weights, and the pack / unpack kernels.
//
// Packed layouts (version 1).  A "unit" is 16 rows of W (one MFMA tile along
// N) by one 128-wide K block, stored contiguously, units ordered (tile, kb)
// with kb fastest.  Inside a unit every 16-byte piece is what one lane loads
// (the FLUTE PR "Add optimized_w3", "Core contributions" item 2: one
// coalesced 16-byte load lands directly in the lane's matrix-core operand):
//
//   FP8   unit = 2048 B = two 1 KiB chunks j = 0, 1.  Lane l of chunk j holds
//         the 16 codes W[16t + l%16][128kb + 64j + 16(l/16) + i], i = 0..15.
//         Block scales follow the codes as FP32 [N/128][K/128].
//   LUT3  unit = 1024 B.  Lane l holds 32 codes of row n = 16t + l%16 at
//         k = 128kb + 32(l/16) + 8s + e (s, e = 0..7 blocks of the 4 dwords):
//         dword s, byte b carries e = b in its low nibble, e = b + 4 in its
//         high nibble.  Group scales follow as FP16 [tile][kb][16 rows], then
//         the 8 map entries (FP16), then a 16-byte pack-status word.
//
// GEMM schedule.  One work-group owns one column group (NT tiles of 16 output
// columns) over the whole of K.  Its S waves split the K blocks into S
// contiguous, near-equal ranges (split-K), so a low-N projection still puts
// enough waves on the chip; S is chosen per shape by the host.  Each wave walks
// its range with the next D units' loads in flight (a register ring), folds
// every 128-K block onto FP32 accumulators, and parks its partial tile in LDS;
// the work-group then sums the S partials in wave order and writes y.  No two
// work-groups share an output, so there is no cross-work-group traffic, no
// workspace and no fence, and every sum has a fixed order: results are
// deterministic and do not depend on M.
#include "wq_device.hpp"
#include "wq_internal.h"

namespace wq {

// 4 KiB of zeros: the source of loads that have nothing to fetch (prefetch
// past the end of a wave's range, tiles past N, batch rows >= M).  Loading
// from here keeps every load unconditional, so the compiler can count loads
// in flight statically.
__device__ __attribute__((aligned(256))) uint8_t g_zero_page[4096];

// ======================================================================
// Policies: per-unit loads and compute for each kernel kind.  A policy is
// bound to one column group; load(r, kb, valid) fetches K block kb into the
// register set r (from the zero page when !valid), compute(r) consumes it.
// ======================================================================

// ---- activation staging for the MFMA tiles ---------------------------------
// The MFMA operand layout gives consecutive lanes consecutive batch rows, so
// loading fragments straight from x would make every 16-byte lane piece its
// own L1 access.  Instead x for one K block (16 rows x 128 k, 4 KiB) is loaded
// coalesced, as four 1 KiB pieces f: 8 consecutive lanes read one row's
// 128-byte segment (rows (l>>3) + 8(f&1), k = 64(f>>1) + 8(l&7) .. +7).  The
// pieces go to an LDS buffer whose rows are padded by 16 bytes, and the
// fragments are read back with 16-byte LDS reads: with the pad, the 16 rows
// read by a 16-lane group start 4 banks apart and cover all 64 banks once
// (the same stride arithmetic as the shared-memory pad in the arc PR "FP8
// bank conflict + the dispatch threshold's provenance", "What landed").
// When SN column-waves share a K range, each loads 4/SN of the pieces and
// all of them read the shared buffer.
constexpr int kXRowBytes = 128 * 2 + 16;          // padded LDS row
constexpr int kXStageBytes = 16 * kXRowBytes;     // one K block of x

template <int XP>   // pieces this wave loads
struct XStage {
    const uint16_t* xl;       // x at this lane's k offset (8 * (l & 7))
    int64_t ldx;
    int rows;
    int lane;
    int f0;                   // first piece of this wave

    __device__ void init(const GemmArgs& a, int l, int first_piece)
    {
        lane = l;
        f0 = first_piece;
        xl = a.x + (l & 7) * 8;
        ldx = a.ldx;
        rows = a.rows;
    }

    __device__ __forceinline__ void load(uint4 (&xr)[XP], int kb, bool valid) const
    {
#pragma unroll
        for (int i = 0; i < XP; ++i) {
            const int f = f0 + i;
            const int r = (lane >> 3) + 8 * (f & 1);
            const void* p = (valid && r < rows) ? (const void*)(xl + r * ldx + kb * 128 + (f >> 1) * 64)
                                                : (const void*)(g_zero_page + 1024 + (lane & 7) * 16);
            xr[i] = load16(p);
        }
    }

    __device__ __forceinline__ void stage(uint8_t* buf, const uint4 (&xr)[XP]) const
    {
#pragma unroll
        for (int i = 0; i < XP; ++i) {
            const int f = f0 + i;
            const int r = (lane >> 3) + 8 * (f & 1);
            const int k = (f >> 1) * 64 + (lane & 7) * 8;
            *reinterpret_cast<uint4*>(buf + r * kXRowBytes + k * 2) = xr[i];
        }
    }

    // 8 consecutive activations of batch row (l % 16) starting at k
    __device__ __forceinline__ uint4 frag(const uint8_t* buf, int k) const
    {
        return *reinterpret_cast<const uint4*>(buf + (lane & 15) * kXRowBytes + k * 2);
    }
};

// ---- FP8 weights, 16-row BF16 MFMA tile ------------------------------------
// A operand = dequantised weights (lane: row n = l%16), B operand = x
// (lane: batch row m = l%16).  Output D[n][m] -> lane holds n = 4(l/16)+v.
template <int NT, int SN>
struct MfmaFp8 {
    static constexpr int KIND = KIND_MFMA_FP8;
    static constexpr int NTILES = NT;
    static constexpr int XP = 4 / SN;
    struct Unit {
        uint4 w[NT][2];
        uint4 x[XP];
        float s;
    };
    const GemmArgs& a;
    int lane;
    int ntiles;               // valid tiles of this wave
    const uint8_t* wbase;     // this lane's bytes of the wave's tile 0, K block 0
    const float* srow;        // block-scale row of this wave's tiles
    XStage<XP> xs;
    f32x4_t outer[NT];

    __device__ MfmaFp8(const GemmArgs& args, int l, int tile0, int piece0) : a(args), lane(l)
    {
        ntiles = min(NT, a.n_tiles - tile0);
        wbase = a.codes + (((int64_t)tile0 * a.KB) << 11) + l * 16;
        srow = reinterpret_cast<const float*>(a.scales) + (int64_t)(tile0 * 16 / 128) * a.KB;
        xs.init(a, l, piece0);
#pragma unroll
        for (int t = 0; t < NT; ++t) outer[t] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    }

    __device__ __forceinline__ void load(Unit& r, int kb, bool valid) const
    {
#pragma unroll
        for (int t = 0; t < NT; ++t) {
            const bool ok = valid && t < ntiles;
            const uint8_t* p = ok ? wbase + (((int64_t)t * a.KB + kb) << 11) : g_zero_page + lane * 16;
            r.w[t][0] = load_stream16(p);
            r.w[t][1] = load_stream16(p + (ok ? 1024 : 0));
        }
        xs.load(r.x, kb, valid);
        r.s = (valid && ntiles > 0) ? srow[kb] : 0.f;   // a wave past N reads no scale
    }

    __device__ __forceinline__ void stage(uint8_t* buf, const Unit& r) const { xs.stage(buf, r.x); }

    __device__ __forceinline__ void compute(const Unit& r, const uint8_t* buf)
    {
        f32x4_t blk[NT];
#pragma unroll
        for (int t = 0; t < NT; ++t) blk[t] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int f = 0; f < 4; ++f) {  // f = 2j + h -> k offset 64j + 16(l/16) + 8h
            const int j = f >> 1, h = f & 1;
            const bf16x8_t b = __builtin_bit_cast(bf16x8_t, xs.frag(buf, j * 64 + (lane >> 4) * 16 + h * 8));
#pragma unroll
            for (int t = 0; t < NT; ++t) {
                const uint4 w = r.w[t][j];
                const bf16x8_t av = h ? e4m3x8_to_bf16x8(w.z, w.w) : e4m3x8_to_bf16x8(w.x, w.y);
                blk[t] = mfma_bf16(av, b, blk[t]);
            }
        }
        // two-level fold: one FP32 FMA per 128-K block and output
#pragma unroll
        for (int t = 0; t < NT; ++t)
#pragma unroll
            for (int v = 0; v < 4; ++v) outer[t][v] = __builtin_fmaf(r.s, blk[t][v], outer[t][v]);
    }

    // slot: [16 rows][NT*16] FP32 partial tile of this wave
    __device__ __forceinline__ void store_partial(float* slot) const
    {
        const int m = lane & 15, n4 = (lane >> 4) * 4;
#pragma unroll
        for (int t = 0; t < NT; ++t) *reinterpret_cast<f32x4_t*>(slot + m * NT * 16 + t * 16 + n4) = outer[t];
    }
};

// ---- 3-bit LUT weights, 16-row FP16 MFMA tile -------------------------------
template <int NT, int SN>
struct MfmaLut {
    static constexpr int KIND = KIND_MFMA_LUT;
    static constexpr int NTILES = NT;
    static constexpr int XP = 4 / SN;
    struct Unit {
        uint4 w[NT];
        uint4 x[XP];
        uint32_t g[NT];      // FP16 group-scale bits, zero-extended
    };
    const GemmArgs& a;
    int lane;
    int ntiles;
    const uint8_t* wbase;
    const uint16_t* gbase;   // this lane's group scale of the wave's tile 0, K block 0
    XStage<XP> xs;
    uint32_t q[4];           // map entries as FP16 pairs
    f32x4_t acc[NT];

    __device__ MfmaLut(const GemmArgs& args, int l, int tile0, int piece0) : a(args), lane(l)
    {
        ntiles = min(NT, a.n_tiles - tile0);
        const int64_t unit0 = (int64_t)tile0 * a.KB;
        wbase = a.codes + (unit0 << 10) + l * 16;
        gbase = reinterpret_cast<const uint16_t*>(a.scales) + unit0 * 16 + (l & 15);
        xs.init(a, l, piece0);
        const uint32_t* qm = reinterpret_cast<const uint32_t*>(a.qmap);
#pragma unroll
        for (int i = 0; i < 4; ++i) q[i] = qm[i];
#pragma unroll
        for (int t = 0; t < NT; ++t) acc[t] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    }

    __device__ __forceinline__ void load(Unit& r, int kb, bool valid) const
    {
#pragma unroll
        for (int t = 0; t < NT; ++t) {
            const bool ok = valid && t < ntiles;
            const int64_t u = (int64_t)t * a.KB + kb;
            r.w[t] = load_stream16(ok ? wbase + (u << 10) : g_zero_page + lane * 16);
            r.g[t] = ok ? (uint32_t)gbase[u * 16] : 0u;
        }
        xs.load(r.x, kb, valid);
    }

    __device__ __forceinline__ void stage(uint8_t* buf, const Unit& r) const { xs.stage(buf, r.x); }

    __device__ __forceinline__ void compute(const Unit& r, const uint8_t* buf)
    {
        f16x8_t b[4];
#pragma unroll
        for (int s = 0; s < 4; ++s)   // K group (l/16) holds k = 32(l/16) + 8s + e
            b[s] = __builtin_bit_cast(f16x8_t, xs.frag(buf, (lane >> 4) * 32 + s * 8));
#pragma unroll
        for (int t = 0; t < NT; ++t) {
            const LutPlanes pl = lut_scaled_planes(q, __builtin_bit_cast(_Float16, (uint16_t)r.g[t]));
            const uint32_t wd[4] = {r.w[t].x, r.w[t].y, r.w[t].z, r.w[t].w};
#pragma unroll
            for (int s = 0; s < 4; ++s) acc[t] = mfma_f16(lut_decode8(wd[s], pl), b[s], acc[t]);
        }
    }

    __device__ __forceinline__ void store_partial(float* slot) const
    {
        const int m = lane & 15, n4 = (lane >> 4) * 4;
#pragma unroll
        for (int t = 0; t < NT; ++t) *reinterpret_cast<f32x4_t*>(slot + m * NT * 16 + t * 16 + n4) = acc[t];
    }
};

// ---- FP8 weights, strict-K-order GEMV (MR <= 4 rows) ------------------------
// The wave covers 4 tiles (64 columns): lane l owns column l%16 of tile l/16.
// For each 64-wide chunk it loads the chunk's four K groups g = 0..3 of its
// column (the same 16-byte pieces the MFMA path loads, just gathered per K
// group across four tiles), so every lane needs the same 16 activations at a
// time: x is wave-uniform and read with scalar loads.  Each (row, column)
// keeps one FP32 accumulator that takes its products in strictly increasing
// k over the wave's K range; each 128-K block is folded onto the outer
// accumulator times the block scale.  The K split across waves is summed in
// wave order afterwards.
template <int MR>
struct GemvFp8 {
    static constexpr int KIND = KIND_GEMV_FP8;
    static constexpr int NTILES = 4;
    static constexpr int CGW = 64;
    struct Unit {
        uint4 w[2][4];       // [chunk j][K group g]
        float s;
    };
    const GemmArgs& a;
    int lane;
    bool tile_ok;
    const uint8_t* wbase;    // this lane's column in tile l/16, K group 0, K block 0
    const uint16_t* xg;      // x (wave-uniform)
    const float* srow;
    float outer[MR];

    __device__ GemvFp8(const GemmArgs& args, int l, int tile0, int) : a(args), lane(l)
    {
        const int64_t tile = (int64_t)tile0 + (l >> 4);
        tile_ok = tile < a.n_tiles;
        wbase = a.codes + ((tile * a.KB) << 11) + (l & 15) * 16;
        xg = a.x;
        srow = reinterpret_cast<const float*>(a.scales) + (int64_t)(tile0 * 16 / 128) * a.KB;
#pragma unroll
        for (int m = 0; m < MR; ++m) outer[m] = 0.f;
    }

    __device__ __forceinline__ void load(Unit& r, int kb, bool valid) const
    {
        const bool ok = valid && tile_ok;
        const uint8_t* p = ok ? wbase + ((int64_t)kb << 11) : g_zero_page + (lane & 15) * 16;
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
            for (int g = 0; g < 4; ++g) r.w[j][g] = load_stream16(p + (ok ? j * 1024 + g * 256 : 0));
        r.s = valid ? srow[kb] : 0.f;
    }

    __device__ __forceinline__ void stage(uint8_t*, const Unit&) const {}

    __device__ __forceinline__ void compute(const Unit& r, int kb)
    {
        float blk[MR];
#pragma unroll
        for (int m = 0; m < MR; ++m) blk[m] = 0.f;
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                const uint4 w = r.w[j][g];
                const uint32_t d[4] = {w.x, w.y, w.z, w.w};
                float wf[16];
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const f32x2_t lo = e4m3x2_to_f32x2<false>(d[i]);
                    const f32x2_t hi = e4m3x2_to_f32x2<true>(d[i]);
                    wf[4 * i + 0] = lo[0];
                    wf[4 * i + 1] = lo[1];
                    wf[4 * i + 2] = hi[0];
                    wf[4 * i + 3] = hi[1];
                }
                const int k0 = kb * 128 + j * 64 + g * 16;
#pragma unroll
                for (int m = 0; m < MR; ++m) {
                    const uint16_t* xp = xg + (int64_t)m * a.ldx + k0;
                    const uint4 xa = load_uniform16(xp), xb = load_uniform16(xp + 8);
                    const uint32_t xd[8] = {xa.x, xa.y, xa.z, xa.w, xb.x, xb.y, xb.z, xb.w};
#pragma unroll
                    for (int i = 0; i < 8; ++i) {
                        blk[m] = __builtin_fmaf(bf16_bits_to_f32(xd[i] & 0xFFFFu), wf[2 * i], blk[m]);
                        blk[m] = __builtin_fmaf(bf16_bits_to_f32(xd[i] >> 16), wf[2 * i + 1], blk[m]);
                    }
                }
            }
#pragma unroll
        for (int m = 0; m < MR; ++m) outer[m] = __builtin_fmaf(r.s, blk[m], outer[m]);
    }

    __device__ __forceinline__ void store_partial(float* slot) const
    {
#pragma unroll
        for (int m = 0; m < MR; ++m) slot[m * CGW + lane] = outer[m];
    }
};

// ======================================================================
// The split-K GEMM kernel: grid = column groups, block = S waves.
// ======================================================================
// ======================================================================
// The GEMM kernel.  Grid: one work-group per column group of SN*NT tiles.
// Block: S = SN*SK waves; wave w is column-wave cw = w % SN (tiles
// cw*NT .. +NT of the group) in K group kg = w / SN (K blocks
// KB*kg/SK .. KB*(kg+1)/SK).  The SN waves of a K group share each K block's
// activations through an LDS buffer (double-buffered, one barrier per K
// block); with SN = 1 each wave stages its own activations and no barrier is
// needed.  After the K loop every wave parks its partial tile in LDS and the
// work-group sums the SK partials of each column in K-group order.
// ======================================================================
template <int SN>
constexpr int x_buffers() { return SN > 1 ? 2 : 1; }

template <class Pol, int D, int SN, bool F16_OUT>
__global__ void __launch_bounds__(64 * max_split(Pol::KIND, Pol::NTILES, SN))
gemm_kernel(GemmArgs a)
{
    constexpr int NT = Pol::NTILES;
    constexpr int TW = NT * 16;                       // columns of one wave
    constexpr int XB = x_buffers<SN>();
    extern __shared__ __attribute__((aligned(16))) uint8_t lds[];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int S = blockDim.x >> 6;
    const int SK = S / SN;
    const int cw = wave % SN, kg = wave / SN;
    const int kb0 = (a.KB * kg) / SK, kb1 = (a.KB * (kg + 1)) / SK;
    const int len = kb1 - kb0;
    const int steps = (a.KB + SK - 1) / SK;           // the longest K range; every wave runs it
    uint8_t* xbuf = lds + (SN > 1 ? kg : wave) * XB * kXStageBytes;
    const int tile0 = (blockIdx.x * SN + cw) * NT;

    Pol pol(a, lane, tile0, cw * (4 / SN));
    {
        typename Pol::Unit r[D + 1];
#pragma unroll
        for (int i = 0; i < D; ++i) pol.load(r[i], kb0 + i, i < len);
        pol.stage(xbuf, r[0]);
        for (int i = 0; i < steps; i += D + 1) {
#pragma unroll
            for (int j = 0; j <= D; ++j) {
                const int step = i + j;
                pol.load(r[(j + D) % (D + 1)], kb0 + step + D, step + D < len);
                if (SN > 1) __syncthreads();
                uint8_t* cur = xbuf + (step & (XB - 1)) * kXStageBytes;
                if (step < len) {
                    if constexpr (Pol::KIND == KIND_GEMV_FP8) pol.compute(r[j], kb0 + step);
                    else pol.compute(r[j], cur);
                }
                pol.stage(xbuf + ((step + 1) & (XB - 1)) * kXStageBytes, r[(j + 1) % (D + 1)]);
            }
        }
    }
    __syncthreads();   // every wave is done with the staging buffers
    float* part = reinterpret_cast<float*>(lds);           // [S][16][TW]
    pol.store_partial(part + wave * 16 * TW);
    __syncthreads();

    const int cols = SN * TW;
    const int nout = a.rows * cols;
    for (int e = tid; e < nout; e += blockDim.x) {
        const int m = e / cols, c = e - m * cols;
        const int w0 = c / TW, cc = c - w0 * TW;
        const float* p = part + (w0 * 16 + m) * TW + cc;    // wave w0 (K group 0)
        float v = p[0];
        for (int k = 1; k < SK; ++k) v += p[(int64_t)k * SN * 16 * TW];
        const int64_t n = (int64_t)blockIdx.x * cols + c;
        if (n < a.N) a.y[m * a.ldy + n] = F16_OUT ? f32_to_f16_rne(v) : f32_to_bf16_rne(v);
    }
}

template <class Pol, int SN>
constexpr int gemm_lds_bytes(int split)
{
    const int stage = (SN > 1 ? split / SN : split) * x_buffers<SN>() * kXStageBytes;
    const int parts = split * 16 * Pol::NTILES * 16 * 4;
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
        const int64_t k0 = kb * 128 + j * 64 + (l >> 4) * 16;
        reinterpret_cast<uint4*>(packed)[idx] = gather16(w + n * ldw + k0);
    }
    if (idx < (N / 128) * KB) reinterpret_cast<float*>(packed + N * K)[idx] = scales[idx];
}

__global__ void clear_status_kernel(uint32_t* status) { status[threadIdx.x] = 0u; }

__global__ void pack_lut3_kernel(const uint8_t* __restrict__ codes, int64_t ldc, const uint16_t* __restrict__ qmap,
                                 const uint16_t* __restrict__ scales, int64_t N, int64_t K,
                                 uint8_t* __restrict__ packed, uint32_t* status)
{
    const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    const int64_t KB = K / 128;
    const int64_t n_tiles = N / 16;
    if (idx < N * K / 32) {
        const int l = (int)(idx & 63);
        const int64_t unit = idx >> 6;
        const int64_t t = unit / KB, kb = unit - t * KB;
        const int64_t n = t * 16 + (l & 15);
        const uint8_t* src = codes + n * ldc + kb * 128 + (l >> 4) * 32;
        uint32_t d[4];
        uint32_t bad = 0;
#pragma unroll
        for (int s = 0; s < 4; ++s) {
            uint32_t word = 0;
#pragma unroll
            for (int b = 0; b < 4; ++b) {
                const uint32_t lo = src[8 * s + b], hi = src[8 * s + b + 4];
                bad |= (lo | hi) & ~7u;
                word |= ((lo & 15u) | ((hi & 15u) << 4)) << (8 * b);
            }
            d[s] = word;
        }
        reinterpret_cast<uint4*>(packed)[idx] = make_uint4(d[0], d[1], d[2], d[3]);
        if (bad) atomicOr(status, 1u);
    }
    uint16_t* sc_out = reinterpret_cast<uint16_t*>(packed + N * K / 2);
    if (idx < n_tiles * KB * 16) {
        const int64_t r = idx & 15, unit = idx >> 4;
        const int64_t t = unit / KB, kb = unit - t * KB;
        sc_out[idx] = scales[(t * 16 + r) * KB + kb];
    }
    if (idx < 8) sc_out[n_tiles * KB * 16 + idx] = qmap[idx];
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
    const int64_t k0 = kb * 128 + j * 64 + (l >> 4) * 16;
    const uint4 w = reinterpret_cast<const uint4*>(packed)[idx];
    if (f32_out) {
        const uint32_t d[4] = {w.x, w.y, w.z, w.w};
        float* o = reinterpret_cast<float*>(out) + n * K + k0;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const f32x2_t lo = e4m3x2_to_f32x2<false>(d[i]);
            const f32x2_t hi = e4m3x2_to_f32x2<true>(d[i]);
            o[4 * i + 0] = lo[0];
            o[4 * i + 1] = lo[1];
            o[4 * i + 2] = hi[0];
            o[4 * i + 3] = hi[1];
        }
    } else {
        uint16_t* o = reinterpret_cast<uint16_t*>(out) + n * K + k0;
        const bf16x8_t a = e4m3x8_to_bf16x8(w.x, w.y), b = e4m3x8_to_bf16x8(w.z, w.w);
        *reinterpret_cast<uint4*>(o) = __builtin_bit_cast(uint4, a);
        *reinterpret_cast<uint4*>(o + 8) = __builtin_bit_cast(uint4, b);
    }
}

__global__ void unpack_lut3_kernel(const uint8_t* __restrict__ packed, int64_t N, int64_t K, uint16_t* out)
{
    const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (idx >= N * K / 32) return;
    const int64_t KB = K / 128;
    const int64_t n_tiles = N / 16;
    const int l = (int)(idx & 63);
    const int64_t unit = idx >> 6;
    const int64_t t = unit / KB, kb = unit - t * KB;
    const int64_t n = t * 16 + (l & 15);
    const uint16_t* sc = reinterpret_cast<const uint16_t*>(packed + N * K / 2);
    const uint32_t* qm = reinterpret_cast<const uint32_t*>(sc + n_tiles * KB * 16);
    const uint32_t q[4] = {qm[0], qm[1], qm[2], qm[3]};
    const LutPlanes pl = lut_scaled_planes(q, __builtin_bit_cast(_Float16, sc[unit * 16 + (l & 15)]));
    const uint4 w = reinterpret_cast<const uint4*>(packed)[idx];
    const uint32_t d[4] = {w.x, w.y, w.z, w.w};
    uint16_t* o = out + n * K + kb * 128 + (l >> 4) * 32;
#pragma unroll
    for (int s = 0; s < 4; ++s)
        *reinterpret_cast<uint4*>(o + 8 * s) = __builtin_bit_cast(uint4, lut_decode8(d[s], pl));
}

// ======================================================================
// Launchers
// ======================================================================

template <class Pol, int D, int SN, bool F16>
static hipError_t launch_one(const GemmArgs& a, int split, hipStream_t s)
{
    auto fn = gemm_kernel<Pol, D, SN, F16>;
    const size_t lds = (size_t)gemm_lds_bytes<Pol, SN>(split);
    if (lds > 64 * 1024) {
        hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(fn),
                                           hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
        if (e != hipSuccess) return e;
    }
    hipLaunchKernelGGL(fn, dim3(a.n_cg), dim3(split * 64), lds, s, a);
    return hipGetLastError();
}

template <int NT, int SN>
static hipError_t launch_mfma(int kind, const GemmArgs& a, int split, hipStream_t s)
{
    if (kind == KIND_MFMA_FP8) return launch_one<MfmaFp8<NT, SN>, kDepthMfmaFp8, SN, false>(a, split, s);
    return launch_one<MfmaLut<NT, SN>, kDepthMfmaLut, SN, true>(a, split, s);
}

template <int NT>
static hipError_t launch_nt(int kind, int sn, const GemmArgs& a, int split, hipStream_t s)
{
    switch (sn) {
    case 1: return launch_mfma<NT, 1>(kind, a, split, s);
    case 2: return launch_mfma<NT, 2>(kind, a, split, s);
    case 4: return launch_mfma<NT, 4>(kind, a, split, s);
    default: return hipErrorInvalidValue;
    }
}

hipError_t launch_gemm(int kind, int nt, int sn, int gemv_rows, const GemmArgs& a, int split, hipStream_t stream)
{
    if (split < 1 || split > max_split(kind, nt, sn) || split % sn) return hipErrorInvalidValue;
    if (kind == KIND_GEMV_FP8) {
        if (nt != 4 || sn != 1) return hipErrorInvalidValue;
        switch (gemv_rows) {
        case 1: return launch_one<GemvFp8<1>, kDepthGemv, 1, false>(a, split, stream);
        case 2: return launch_one<GemvFp8<2>, kDepthGemv, 1, false>(a, split, stream);
        case 3: return launch_one<GemvFp8<3>, kDepthGemv, 1, false>(a, split, stream);
        case 4: return launch_one<GemvFp8<4>, kDepthGemv, 1, false>(a, split, stream);
        default: return hipErrorInvalidValue;
        }
    }
    if (kind != KIND_MFMA_FP8 && kind != KIND_MFMA_LUT) return hipErrorInvalidValue;
    switch (nt) {
    case 1: return launch_nt<1>(kind, sn, a, split, stream);
    case 2: return launch_nt<2>(kind, sn, a, split, stream);
    case 4: return launch_nt<4>(kind, sn, a, split, stream);
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
                            int64_t N, int64_t K, uint8_t* packed, uint32_t* status, hipStream_t stream)
{
    hipLaunchKernelGGL(clear_status_kernel, dim3(1), dim3(4), 0, stream, status);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    const int64_t n = N * K / 32 > N * (K / 128) ? N * K / 32 : N * (K / 128);
    hipLaunchKernelGGL(pack_lut3_kernel, dim3(blocks_for(n)), dim3(256), 0, stream, codes, ldc, qmap, scales, N, K,
                       packed, status);
    return hipGetLastError();
}

hipError_t launch_unpack_fp8(const uint8_t* packed, int64_t N, int64_t K, void* out, bool f32_out, hipStream_t stream)
{
    hipLaunchKernelGGL(unpack_fp8_kernel, dim3(blocks_for(N * K / 16)), dim3(256), 0, stream, packed, N, K, out,
                       (int)f32_out);
    return hipGetLastError();
}

hipError_t launch_unpack_lut3(const uint8_t* packed, int64_t N, int64_t K, uint16_t* out, hipStream_t stream)
{
    hipLaunchKernelGGL(unpack_lut3_kernel, dim3(blocks_for(N * K / 32)), dim3(256), 0, stream, packed, N, K, out);
    return hipGetLastError();
}

}  // namespace wq
