// gfx950 kernels of libwq's W8A8 tier: FP8 activations x FP8 block-scaled
// weights on the FP8 matrix cores.
//
// The atlas ladder ("ARM ORDER", rung 6) serves batches above the decode band
// with a W8A8 block-scaled GEMM, and the arc PR ("Worth a separate change")
// notes that block-scaled FP8 needs the activations in FP8 too, i.e. an
// activation quantiser.  Here:
//
//   quantiser  x (BF16) -> codes + one FP32 scale per (row, 128-wide K group):
//              s = amax / 448 (IEEE binary32 division; 1 for an all-zero
//              group), code = E4M3 nearest-even of clamp(x / s, -448, 448),
//              the rule of the weights' own 128x128 block quantiser; a group
//              holding an infinity or a NaN gets a NaN scale and NaN codes.
//   GEMM       y[m,n] = sum over K blocks kb of sx[m][kb] * sw[n/128][kb] *
//              (sum over the block of e4m3(xq) * e4m3(w)); one
//              v_mfma_f32_16x16x128_f8f6f4 covers a whole 128-K block of a
//              16x16 tile, and its FP32 result is folded once per block onto
//              an FP32 outer accumulator times the two scales (the two-level
//              fold of the atlas docs' NUMERICS section, with the activation
//              scale added).
//
// Quantised activation layout ("XQ"): rows padded to Mpad = 16 * ceil(M/16);
// units of 16 rows x one K block (2048 B) in (row tile, kb) order, kb fastest,
// each laid out exactly like an FP8 weight unit (lane l of chunk j holds 16
// codes of row 16t + l%16: byte i is k = 128kb + 32(2j + i/8) + 8(l/16) +
// i%8); then the scales as FP32 [K/128][Mpad].  Padding rows hold zero codes
// and zero scales.  A weight unit and an activation unit of the same K block
// therefore put the same k in the same (lane group, byte) slot, which is all
// the matrix core needs: it sums over the slots.
#include "wq_device.hpp"
#include "wq_internal.h"

namespace wq {

// ----------------------------------------------------------------- quantiser

// Nearest E4M3FN code (ties to even) of a finite binary32 value with
// |v| <= 448.  Normal range: round the binary32 pattern to 3 mantissa bits
// (half-even on the discarded 20 bits, the carry walks into the exponent) and
// rebias 127 -> 7; below 2^-6 the E4M3 grid is m * 2^-9, so the code is
// round-half-even(|v| * 512) (0 .. 8, 8 being the smallest normal).
__device__ __forceinline__ uint32_t e4m3_rne(float v)
{
    const uint32_t b = __float_as_uint(v);
    const uint32_t sign = (b >> 24) & 0x80u;
    const uint32_t mag = b & 0x7FFFFFFFu;
    const float a = __uint_as_float(mag);
    uint32_t code;
    if (a < 0.015625f) {
        code = (uint32_t)__builtin_rintf(a * 512.0f);
    } else {
        const uint32_t r = (mag + 0x7FFFFu + ((mag >> 20) & 1u)) >> 20;
        code = r - (120u << 3);
    }
    return sign | code;
}

// One wave per activation unit (16 rows x one 128-K block), laid out by its
// output: lane l writes the two 16-byte pieces it owns in the unit -- piece l
// of each 1 KiB chunk j, i.e. the codes of row r = l%16 at k = 32(2j + h) +
// 8g + e (g = l/16, h = 0, 1, e = 0..7) -- so each store instruction writes a
// whole 1 KiB chunk.  The lane reads those 32 activations with four 16-byte
// loads (the four 8-wide runs k = 8g + 32q, q = 0..3, of its row); the four
// lanes of a row (l = r, r+16, r+32, r+48) hold its whole K group and find
// the group's amax with two exchanges.  Per value the arithmetic is that of
// the quantiser rule above: s = amax / 448, code = e4m3_rne(clamp(x / s)),
// with x / s the correctly rounded binary32 quotient.
__global__ void __launch_bounds__(256) quantize_x_kernel(const uint16_t* __restrict__ x, int64_t ldx, int M,
                                                         int Mpad, int KB, uint8_t* __restrict__ xq)
{
    const int64_t unit = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);   // (row tile, kb), kb fastest
    if (unit >= (int64_t)(Mpad >> 4) * KB) return;                       // whole waves exit together
    const int lane = threadIdx.x & 63;
    const int mt = (int)(unit / KB), kb = (int)(unit - (int64_t)mt * KB);
    const int r = lane & 15, g = lane >> 4;
    const int m = 16 * mt + r;
    float v[4][8];                      // run q: k = 128kb + 32q + 8g + e
    float amax = 0.f;
    uint32_t expmax = 0u;               // largest BF16 exponent field seen (0xFF: Inf or NaN)
    if (m < M) {
        const uint16_t* row = x + (int64_t)m * ldx + kb * 128 + 8 * g;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const uint4 raw = *reinterpret_cast<const uint4*>(row + 32 * q);
            const uint32_t d[4] = {raw.x, raw.y, raw.z, raw.w};
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                v[q][2 * i] = __uint_as_float(d[i] << 16);
                v[q][2 * i + 1] = __uint_as_float(d[i] & 0xFFFF0000u);
                expmax = max(expmax, max((d[i] >> 7) & 0xFFu, (d[i] >> 23) & 0xFFu));
            }
#pragma unroll
            for (int e = 0; e < 8; ++e) amax = fmaxf(amax, fabsf(v[q][e]));
        }
    } else {
#pragma unroll
        for (int q = 0; q < 4; ++q)
#pragma unroll
            for (int e = 0; e < 8; ++e) v[q][e] = 0.f;
    }
    amax = fmaxf(amax, __shfl_xor(amax, 16));
    amax = fmaxf(amax, __shfl_xor(amax, 32));
    expmax = max(expmax, (uint32_t)__shfl_xor((int)expmax, 16));
    expmax = max(expmax, (uint32_t)__shfl_xor((int)expmax, 32));
    // a group holding an infinity or a NaN: NaN scale and the E4M3 NaN code
    // everywhere, so every product that uses the group is NaN
    const bool nonfinite = expmax == 0xFFu;
    const float s = nonfinite ? __uint_as_float(0x7FC00000u) : amax > 0.f ? amax / 448.0f : 1.0f;
    // x / s correctly rounded without a division per value: y = RN(1/s) once,
    // then q = RN(x y), the remainder x - q s exactly (one FMA) and RN(q + r y)
    // (Markstein's correction step), with x's sign put back so that -0 stays
    // -0.  Compared on gfx950 against the division for every pair of BF16
    // values with |x| <= amax: the same E4M3 code wherever amax >= 2^-104;
    // groups with 0 < amax < 2^-80 keep the division (below 2^-104 1/s nears
    // the top of the binary32 range and the two differ).
    if (!(amax > 0.f && amax < 0x1p-80f)) {
        const float y = 1.0f / s;
#pragma unroll
        for (int q = 0; q < 4; ++q)
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const float xv = v[q][e], q0 = xv * y;
                v[q][e] = __builtin_copysignf(__builtin_fmaf(__builtin_fmaf(-q0, s, xv), y, q0), xv);
            }
    } else {
#pragma unroll
        for (int q = 0; q < 4; ++q)
#pragma unroll
            for (int e = 0; e < 8; ++e) v[q][e] = v[q][e] / s;
    }
    uint32_t c[4][2];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        c[q][0] = c[q][1] = 0u;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const float qv = fminf(fmaxf(v[q][e], -448.0f), 448.0f);
            const uint32_t code = m < M ? (nonfinite ? 0x7Fu : e4m3_rne(qv)) : 0u;
            c[q][e >> 2] |= code << (8 * (e & 3));
        }
    }
    // chunk j holds runs q = 2j (bytes 0..7) and q = 2j + 1 (bytes 8..15)
    uint8_t* u = xq + unit * 2048 + lane * 16;
    *reinterpret_cast<uint4*>(u) = make_uint4(c[0][0], c[0][1], c[1][0], c[1][1]);
    *reinterpret_cast<uint4*>(u + 1024) = make_uint4(c[2][0], c[2][1], c[3][0], c[3][1]);
    if (g == 0) {
        float* sx = reinterpret_cast<float*>(xq + (int64_t)Mpad * KB * 128);
        sx[(int64_t)kb * Mpad + m] = m < M ? s : 0.f;
    }
}

// test hook: packed activations back to canonical codes [M][K] and scales [M][KB]
__global__ void unpack_x_kernel(const uint8_t* __restrict__ xq, int M, int Mpad, int KB, uint8_t* __restrict__ codes,
                                float* __restrict__ scales)
{
    const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    const int64_t K = (int64_t)KB * 128;
    if (idx >= (int64_t)M * K) return;
    const int m = (int)(idx / K);
    const int k = (int)(idx - (int64_t)m * K);
    const int kb = k >> 7, J = (k & 127) >> 3, e = k & 7;
    const int js = J >> 2, g = J & 3;
    const uint8_t* unit = xq + ((int64_t)(m >> 4) * KB + kb) * 2048;
    codes[idx] = unit[(js >> 1) * 1024 + (16 * g + (m & 15)) * 16 + 8 * (js & 1) + e];
    if ((k & 127) == 0) {
        const float* sx = reinterpret_cast<const float*>(xq + (int64_t)Mpad * KB * 128);
        scales[(int64_t)m * KB + kb] = sx[(int64_t)kb * Mpad + m];
    }
}

// ---------------------------------------------------------------------- GEMM

struct W8Args {
    const uint8_t* w;       // packed FP8 weight units (N/16 tiles x KB)
    const float* sw;        // weight block scales [N/128][KB]
    const uint8_t* xq;      // packed activation units (Mpad/16 tiles x KB), then sx
    const float* sx;        // activation scales [KB][Mpad]
    uint16_t* y;            // [M][ldy] BF16
    int64_t ldy;
    int M, Mpad, N, KB;
    int n_mt, n_tw, n_wg;   // row tiles, output tiles, work-groups with work (n_tw * kp)
    int kp;                 // K parts across work-groups (> 1: FP32 partials to ws)
    float* ws;              // kp > 1: partial outputs [kp][M][N]
};

// Wait until at most n vector-memory operations of this wave are outstanding
// (gfx9 s_waitcnt encoding: vmcnt in bits 3:0 and 15:14; expcnt and lgkmcnt
// left at their maxima, i.e. not waited for).
template <int N>
__device__ __forceinline__ void wait_vmcnt()
{
    static_assert(N >= 0 && N < 64, "vmcnt is 6 bits");
    __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | (15 << 8) | ((N >> 4) << 14));
}

// Wait until at most N vector-memory operations and no LDS access of this
// wave are outstanding (lgkmcnt = 0; expcnt left at its maximum).
template <int N>
__device__ __forceinline__ void wait_vmcnt_lgkmcnt0()
{
    static_assert(N >= 0 && N < 64, "vmcnt is 6 bits");
    __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | ((N >> 4) << 14));
}

// 16 bytes per lane from a buffer straight into LDS: lane l's bytes land at
// LDS address dst + 16 l (dst is wave-uniform; it goes to M0).  The data never
// passes through VGPRs.  Written as inline assembly on purpose: the compiler
// then does not treat the instruction as an LDS write and inserts no wait of
// its own before later LDS reads (it cannot tell the stages apart and would
// wait for the newest loads); the kernel orders every stage itself with an
// explicit vmcnt wait and a barrier, and no other vector-memory load is in
// flight in its loop.
typedef int i32x4_t __attribute__((ext_vector_type(4)));

struct RawBuf {
    i32x4_t d;                  // buffer descriptor: base, num_records, raw dword3 flags
};

__device__ __forceinline__ RawBuf raw_buf(const void* base, uint32_t bytes)
{
    const uint64_t p = reinterpret_cast<uint64_t>(base);
    return RawBuf{i32x4_t{(int)(uint32_t)p, (int)((uint32_t)(p >> 32) & 0xFFFFu), (int)bytes, 0x00020000}};
}

__device__ __forceinline__ uint32_t lds_addr(const void* p)
{
    return (uint32_t)(uintptr_t)(__attribute__((address_space(3))) const void*)p;
}

__device__ __forceinline__ void dma16(const RawBuf& r, uint32_t dst, uint32_t voff, uint32_t soff)
{
    asm volatile("buffer_load_dwordx4 %0, %1, %2 offen lds"
                 :
                 : "v"(voff), "s"(r.d), "s"(__builtin_amdgcn_readfirstlane(soff)),
                   "{m0}"(__builtin_amdgcn_readfirstlane(dst))
                 : "memory");
}

// Work-group tile BM x BN = (16 WMT WVM) x (16 WNT WVN): WVM x WVN waves, each
// owning WMT x WNT MFMA tiles of 16 x 16.  A K block's operands (BM/16
// activation units and BN/16 weight units of 2 KB) and the BM rows'
// activation scales go from memory straight into one of NS LDS stages
// (buffer loads to LDS, no VGPR staging), NS - 1 blocks ahead of the block
// being multiplied.  Per block every wave waits for its own loads of that
// stage (the later blocks' loads stay in flight), the work-group meets at one
// barrier (after which every wave's loads of the stage have landed and every
// wave is done with the stage it multiplied last), issues the loads of block
// kb + NS - 1 into that stage, and runs its WMT x WNT MFMAs, each folded onto
// the FP32 outer accumulators times sx[m][kb] * sw[nb][kb].  The stages are
// separate LDS arrays and the loop is unrolled by NS, so each read names a
// fixed stage.  NS = 2 lets two work-groups share a CU; NS = 4 (132 KB of LDS
// at 128 x 128) serves grids of at most one work-group per CU, where a
// work-group with one block in flight would wait out the memory latency on
// every block.
//
// Work order: XCD x (work-groups b = x mod 8) takes the contiguous run
// [x * per_xcd, (x+1) * per_xcd) of linear indices; these walk groups of GN
// column tiles row tile by row tile, so the work-groups an XCD runs at once
// cover a rectangle of tiles and share each K slice of both operands through
// that XCD's L2.  With kp K parts the part is the outermost index: work-group
// (part, tile) multiplies the part-th of kp contiguous runs of K blocks and
// stores its FP32 sums to the part's slab of the workspace.
template <int WMT, int WNT, int WVM, int WVN, int GN, int NS>
__global__ void __launch_bounds__(64 * WVM * WVN) __attribute__((amdgpu_waves_per_eu(NS == 2 ? 2 : 1, 2)))
w8a8_gemm_kernel(W8Args a)
{
    constexpr int WAVES = WVM * WVN;
    constexpr int TM = WMT * WVM, TN = WNT * WVN;       // 16-row / 16-column tiles of the work-group
    constexpr int BM = 16 * TM, BN = 16 * TN;
    constexpr int OPS = (TM + TN) * 2048;               // operand bytes of one stage
    constexpr int STAGE = OPS + BM * 4;                 // + the activation scales of BM rows
    constexpr int CPW = 2 * (TM + TN) / WAVES;          // 1 KB copy chunks per wave and stage
    constexpr int SROWS = BM / WAVES;                   // scale rows each wave copies
    static_assert(2 * (TM + TN) % WAVES == 0 && SROWS % 4 == 0 && SROWS <= 256, "copy split");
    static_assert(WNT * 16 <= 128 && 128 % (WNT * 16) == 0, "a wave's columns share one weight scale block");
    static_assert(NS >= 2 && NS * STAGE <= kLdsBytes, "stages fit in LDS");
    constexpr int LPS = CPW + 1;                        // loads a wave issues per stage (copies + scale row)
    static_assert((NS - 2) * LPS < 64, "the loads of NS - 2 stages fit the vmcnt field");
    __shared__ __attribute__((aligned(16))) uint8_t st[NS][STAGE];

    const int b = blockIdx.x;
    const int per_xcd = gridDim.x >> 3;                   // the grid is a multiple of 8
    const int wl = (b & 7) * per_xcd + (b >> 3);
    if (wl >= a.n_wg) return;                             // whole work-group, before any barrier
    const int kpart = wl / a.n_tw, wt0 = wl - kpart * a.n_tw;
    const int kbb = (a.KB * kpart) / a.kp, kbe = (a.KB * (kpart + 1)) / a.kp;   // this part's K blocks
    const int n_nt = (a.N + BN - 1) / BN;
    const int g = wt0 / (GN * a.n_mt), r = wt0 - g * (GN * a.n_mt);
    const int gn = min(GN, n_nt - g * GN);                // column tiles in this group
    const int nt = g * GN + r % gn, mt = r / gn;

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wave / WVN, wn = wave - wm * WVN;
    const int KB = a.KB;
    const int m_tiles = a.Mpad >> 4, n_tiles = a.N >> 4;

    // Buffer resources are work-group uniform; tile offsets sit in the VGPR
    // offset, which the bounds check covers: activation tiles and scale rows
    // past Mpad, and weight tiles past N, read zeros.
    const RawBuf rx = raw_buf(a.xq, (uint32_t)((int64_t)m_tiles * KB * 2048));
    const RawBuf rw = raw_buf(a.w, (uint32_t)((int64_t)n_tiles * KB * 2048));
    const RawBuf rsx = raw_buf(a.sx, (uint32_t)((int64_t)KB * a.Mpad * 4));

    // copy chunk c = wave + WAVES i (1 KB each): c < 2 TM is half c%2 of
    // activation unit c/2, the rest half c%2 of weight unit (c - 2 TM)/2
    uint32_t voff[CPW];
#pragma unroll
    for (int i = 0; i < CPW; ++i) {
        const int c = wave + WAVES * i;
        const int h = c & 1;
        if (c < 2 * TM) {
            const int xt = TM * mt + (c >> 1);
            voff[i] = xt < m_tiles ? (uint32_t)xt * KB * 2048u + h * 1024 + lane * 16 : kBufOutOfRange;
        } else {
            const int wt = TN * nt + ((c - 2 * TM) >> 1);
            voff[i] = wt < n_tiles ? (uint32_t)wt * KB * 2048u + h * 1024 + lane * 16 : kBufOutOfRange;
        }
    }
    // activation scales: wave w brings rows SROWS w .. SROWS (w+1) - 1 of the tile, 4 a lane
    const int srow = BM * mt + SROWS * wave + 4 * lane;
    const uint32_t svoff = srow < a.Mpad ? (uint32_t)srow * 4u : kBufOutOfRange;

    // LDS addresses of the stages (M0 operands), computed once
    uint32_t lds_st[NS];
#pragma unroll
    for (int s = 0; s < NS; ++s) lds_st[s] = __builtin_amdgcn_readfirstlane(lds_addr(st[s]));
    // the LPS loads of block kb into the stage at LDS address sa (every lane
    // range is non-empty, so each wave issues every one of them)
    auto issue = [&](int kb, uint32_t sa) {
#pragma unroll
        for (int i = 0; i < CPW; ++i) {
            const int c = wave + WAVES * i;
            dma16(c < 2 * TM ? rx : rw, sa + c * 1024, voff[i], (uint32_t)kb * 2048u);
        }
        if (lane < SROWS / 4)
            dma16(rsx, sa + OPS + SROWS * 4 * wave, svoff, (uint32_t)kb * (uint32_t)a.Mpad * 4u);
    };

    f32x4_t outer[WMT][WNT];
#pragma unroll
    for (int i = 0; i < WMT; ++i)
#pragma unroll
        for (int j = 0; j < WNT; ++j) outer[i][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};

    const int lrow = 16 * WMT * wm + 4 * (lane >> 4);     // this lane's first output row in the tile
    const int wcol = TN * nt + WNT * wn;                  // the wave's first 16-column tile
    const int nb = min(wcol >> 3, (a.N >> 7) - 1);        // its weight scale block (clamped past N)

    auto compute = [&](int kb, const uint8_t* st) {
        const float swv = load_uniform_f32(a.sw + (int64_t)nb * KB + kb);
        f32x4_t sc[WMT];
#pragma unroll
        for (int i = 0; i < WMT; ++i) {
            const f32x4_t v = *reinterpret_cast<const f32x4_t*>(st + OPS + (lrow + 16 * i) * 4);
            sc[i] = f32x4_t{v[0] * swv, v[1] * swv, v[2] * swv, v[3] * swv};
        }
        i32x8_t af[WMT];
#pragma unroll
        for (int i = 0; i < WMT; ++i) af[i] = lds_frag(st + (WMT * wm + i) * 2048, lane);
        // software-pipelined over column tiles: the products of column tile j + 1
        // are issued before those of tile j are folded, so a fold never waits
        // for an MFMA issued just before it
        f32x4_t blk[2][WMT];
        {
            const i32x8_t bf = lds_frag(st + (TM + WNT * wn) * 2048, lane);
#pragma unroll
            for (int i = 0; i < WMT; ++i) blk[0][i] = mfma_fp8(af[i], bf, f32x4_t{0.f, 0.f, 0.f, 0.f});
        }
#pragma unroll
        for (int j = 0; j < WNT; ++j) {
            if (j + 1 < WNT) {
                const i32x8_t bf = lds_frag(st + (TM + WNT * wn + j + 1) * 2048, lane);
#pragma unroll
                for (int i = 0; i < WMT; ++i) blk[(j + 1) & 1][i] = mfma_fp8(af[i], bf, f32x4_t{0.f, 0.f, 0.f, 0.f});
            }
#pragma unroll
            for (int i = 0; i < WMT; ++i)
#pragma unroll
                for (int q = 0; q < 4; ++q)
                    outer[i][j][q] = __builtin_fmaf(blk[j & 1][i][q], sc[i][q], outer[i][j][q]);
        }
    };

    // one block: own loads of `cur` done (those of the NS - 2 later blocks may
    // still be in flight: a wave's loads complete in order), barrier, refill
    // the stage multiplied last with block kb + NS - 1 (the part's last block
    // again near the end, so every wave always has the same loads in flight),
    // multiply.
    // Ordering of the stage reuse: the loads that fill `nxt` overwrite what
    // every wave read from it in the previous block.  Before the barrier each
    // wave waits for its own loads into `cur` (vmcnt) and for its own LDS
    // reads (lgkmcnt), and the workgroup-scope release/acquire fences keep
    // the compiler from moving any LDS access across the barrier; so when a
    // wave issues the refill after the barrier, every wave's reads of that
    // stage have returned.
    auto step = [&](int kb, const uint8_t* cur, uint32_t nxt) {
        wait_vmcnt_lgkmcnt0<(NS - 2) * LPS>();
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
        __builtin_amdgcn_s_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
        issue(min(kb + NS - 1, kbe - 1), nxt);
        compute(kb, cur);
    };

#pragma unroll
    for (int s = 0; s < NS - 1; ++s) issue(min(kbb + s, kbe - 1), lds_st[s]);
    for (int kb = kbb;; kb += NS) {
#pragma unroll
        for (int s = 0; s < NS; ++s) {
            step(kb + s, st[s], lds_st[(s + NS - 1) % NS]);
            if (kb + s + 1 >= kbe) goto k_done;      // uniform: every wave leaves here
        }
    }
k_done:
    wait_vmcnt<0>();                                      // no load left writing LDS

    // D of a 16x16 tile: lane l holds rows 4(l/16)..+3 of column l%16
    const int row0 = BM * mt + lrow;
    const int col0 = 16 * wcol + (lane & 15);
    float* const wsp = a.ws + (int64_t)kpart * a.M * a.N;   // this part's partials (kp > 1)
#pragma unroll
    for (int i = 0; i < WMT; ++i)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const int m = row0 + 16 * i + q;
            if (m < a.M) {
#pragma unroll
                for (int j = 0; j < WNT; ++j)
                    if (col0 + 16 * j < a.N) {
                        if (a.kp == 1) a.y[(int64_t)m * a.ldy + col0 + 16 * j] = f32_to_bf16_rne(outer[i][j][q]);
                        else wsp[(int64_t)m * a.N + col0 + 16 * j] = outer[i][j][q];
                    }
            }
        }
}

// --------------------------------------------------------------- launchers

static unsigned blocks_of(int64_t n) { return (unsigned)((n + 255) / 256); }

hipError_t launch_quantize_x(const uint16_t* x, int64_t ldx, int M, int K, uint8_t* xq, hipStream_t stream)
{
    const int Mpad = (M + 15) & ~15, KB = K / 128;
    const int64_t units = (int64_t)(Mpad / 16) * KB;
    hipLaunchKernelGGL(quantize_x_kernel, dim3((unsigned)((units + 3) / 4)), dim3(256), 0, stream, x, ldx, M, Mpad,
                       KB, xq);
    return hipGetLastError();
}

hipError_t launch_unpack_x(const uint8_t* xq, int M, int K, uint8_t* codes, float* scales, hipStream_t stream)
{
    const int Mpad = (M + 15) & ~15, KB = K / 128;
    hipLaunchKernelGGL(unpack_x_kernel, dim3(blocks_of((int64_t)M * K)), dim3(256), 0, stream, xq, M, Mpad, KB, codes,
                       scales);
    return hipGetLastError();
}

// Tiles (the host picks one per call, with the K-part count): 128 x 128 (4
// waves of 64 x 64, two work-groups per CU) for 64 < Mpad <= kW8BigM,
// 256 x 256 above (8 waves of 64 x 128: twice the MFMAs per byte read from
// LDS, one work-group per CU), and for Mpad <= 64 a 64-row tile: 64 x 128
// (4 waves of 64 x 32) or 64 x 64 (4 waves of 32 x 32), whichever fills
// the work-group slots better.  Measured on the FFN shapes: the 128 x 128
// tile is as fast or faster than 128 x 64, 64 x 128 and 64 x 64 from M = 96
// to 4096, the 256 x 256 one slightly faster at M = 8192; at M <= 64 the
// 64-row tiles are 1-5 us faster (the 128-row tile fetches, stages and
// multiplies padding rows).

// Pipeline depth: 4 stages where the grid has at most one work-group per CU
// (measured on the FFN shapes at M = 32 .. 256: with 2 stages every K block
// waits out the memory latency, ~0.85 us a block), else 2 (two work-groups
// share a CU); stages = 2 or 4 forces one.
template <int WMT, int WNT, int WVM, int WVN, int GN>
static hipError_t launch_w8a8_tile(W8Args a, int cu, int stages, hipStream_t stream)
{
    constexpr int BM = 16 * WMT * WVM, BN = 16 * WNT * WVN;
    a.n_mt = (a.Mpad + BM - 1) / BM;
    a.n_tw = a.n_mt * ((a.N + BN - 1) / BN);
    a.n_wg = a.n_tw * a.kp;
    const int grid = (a.n_wg + 7) & ~7;
    constexpr int kStage = (WMT * WVM + WNT * WVN) * 2048 + BM * 4;   // LDS bytes of one stage
    if constexpr (4 * kStage <= kLdsBytes) {                          // the 128 x 128 tile
        if (stages ? stages == 4 : a.n_wg <= cu) {
            hipLaunchKernelGGL((w8a8_gemm_kernel<WMT, WNT, WVM, WVN, GN, 4>), dim3(grid), dim3(64 * WVM * WVN), 0,
                               stream, a);
            return hipGetLastError();
        }
    }
    hipLaunchKernelGGL((w8a8_gemm_kernel<WMT, WNT, WVM, WVN, GN, 2>), dim3(grid), dim3(64 * WVM * WVN), 0, stream, a);
    return hipGetLastError();
}

hipError_t launch_w8a8(const uint8_t* codes, const float* sw, int N, int K, const uint8_t* xq, int M, uint16_t* y,
                       int64_t ldy, int tile, int kp, float* ws, int cu, int stages, hipStream_t stream)
{
    if (kp < 1 || kp > K / 128 || kp > kMaxKParts || (kp > 1 && !ws)) return hipErrorInvalidValue;
    W8Args a{};
    a.kp = kp;
    a.ws = ws;
    a.KB = K / 128;
    a.N = N;
    a.M = M;
    a.Mpad = (M + 15) & ~15;
    a.w = codes;
    a.sw = sw;
    a.xq = xq;
    a.sx = reinterpret_cast<const float*>(xq + (int64_t)a.Mpad * K);
    a.y = y;
    a.ldy = ldy;
    hipError_t e;
    switch (tile) {
    case W8_T128: e = launch_w8a8_tile<4, 4, 2, 2, 8>(a, cu, stages, stream); break;
    case W8_T256: e = launch_w8a8_tile<4, 8, 4, 2, 4>(a, cu, stages, stream); break;
    case W8_T64x128: e = launch_w8a8_tile<4, 2, 1, 4, 8>(a, cu, stages, stream); break;
    case W8_T64x64: e = launch_w8a8_tile<2, 2, 2, 2, 8>(a, cu, stages, stream); break;
    default: return hipErrorInvalidValue;
    }
    if (e != hipSuccess || kp == 1) return e;
    return launch_sum_parts(ws, kp, M, N, y, ldy, false, stream);
}

}  // namespace wq
