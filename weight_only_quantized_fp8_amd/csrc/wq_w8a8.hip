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
//              the rule of the weights' own 128x128 block quantiser.
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

// One lane per 8 consecutive k of one (row, K group); the 16 lanes of a group
// are adjacent in the wave and find the group's amax with a butterfly.
__global__ void __launch_bounds__(256) quantize_x_kernel(const uint16_t* __restrict__ x, int64_t ldx, int M,
                                                         int Mpad, int KB, uint8_t* __restrict__ xq)
{
    const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    const int64_t grp = idx >> 4;
    const int j = (int)(idx & 15);
    if (grp >= (int64_t)Mpad * KB) return;       // whole groups of 16 exit together
    const int m = (int)(grp / KB), kb = (int)(grp - (int64_t)m * KB);
    float v[8];
    float amax = 0.f;
    if (m < M) {
        const uint4 raw = *reinterpret_cast<const uint4*>(x + (int64_t)m * ldx + kb * 128 + 8 * j);
        const uint32_t d[4] = {raw.x, raw.y, raw.z, raw.w};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            v[2 * i] = __uint_as_float(d[i] << 16);
            v[2 * i + 1] = __uint_as_float(d[i] & 0xFFFF0000u);
        }
#pragma unroll
        for (int i = 0; i < 8; ++i) amax = fmaxf(amax, fabsf(v[i]));
    } else {
#pragma unroll
        for (int i = 0; i < 8; ++i) v[i] = 0.f;
    }
#pragma unroll
    for (int o = 1; o < 16; o <<= 1) amax = fmaxf(amax, __shfl_xor(amax, o, 16));
    const float s = amax > 0.f ? amax / 448.0f : 1.0f;
    uint32_t lo = 0, hi = 0;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const float q = fminf(fmaxf(v[i] / s, -448.0f), 448.0f);
        const uint32_t c = m < M ? e4m3_rne(q) : 0u;
        if (i < 4) lo |= c << (8 * i);
        else hi |= c << (8 * (i - 4));
    }
    // k = 128kb + 8j + e sits in MFMA step js = j/4, lane group g = j%4: chunk
    // js/2, lane 16g + m%16, byte 8(js%2) + e
    const int js = j >> 2, g = j & 3;
    uint8_t* unit = xq + ((int64_t)(m >> 4) * KB + kb) * 2048;
    *reinterpret_cast<uint2*>(unit + (js >> 1) * 1024 + (16 * g + (m & 15)) * 16 + 8 * (js & 1)) = make_uint2(lo, hi);
    if (j == 0) {
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
    int n_mt, n_wg;         // 128-row tiles, work-groups with work
};

typedef int i32x8_t __attribute__((ext_vector_type(8)));

__device__ __forceinline__ f32x4_t mfma_fp8(i32x8_t a, i32x8_t b, f32x4_t c)
{
    // scale operands 0: the unscaled v_mfma_f32_16x16x128_f8f6f4, both sides E4M3
    return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c, 0, 0, 0, 0, 0, 0);
}

// A 16-row x 128-K operand from a 2 KB unit staged in LDS: lane l takes its
// 16 bytes of chunk 0 and of chunk 1.
__device__ __forceinline__ i32x8_t lds_frag(const uint8_t* unit, int lane)
{
    const uint4 p = *reinterpret_cast<const uint4*>(unit + lane * 16);
    const uint4 q = *reinterpret_cast<const uint4*>(unit + 1024 + lane * 16);
    return i32x8_t{(int)p.x, (int)p.y, (int)p.z, (int)p.w, (int)q.x, (int)q.y, (int)q.z, (int)q.w};
}

// Work-group tile 128 rows x 128 columns (8 x 8 MFMA tiles, one weight scale
// block), 4 waves as 2 x 2, each owning 4 x 4 tiles.  Per K block the
// work-group stages its 8 activation units and 8 weight units (32 KB) in LDS
// (double-buffered: the next block's units are fetched into registers while
// the current block is multiplied), then every wave runs 16 MFMAs and folds
// them onto its FP32 outer accumulators.
//
// Work-groups are numbered so that those sharing a weight slab (same column
// tile, consecutive row tiles) land on the same XCD (the dispatcher deals
// work-groups to the 8 XCDs round-robin), where the slab stays in that XCD's
// L2 across the row tiles.
__global__ void __launch_bounds__(256) w8a8_gemm_kernel(W8Args a)
{
    constexpr int kStage = 16 * 2048;
    extern __shared__ __attribute__((aligned(16))) uint8_t lds[];
    const int b = blockIdx.x;
    const int per_xcd = gridDim.x >> 3;                   // the grid is a multiple of 8
    const int wl = (b & 7) * per_xcd + (b >> 3);
    if (wl >= a.n_wg) return;                             // whole work-group, before any barrier
    const int nt = wl / a.n_mt, mt = wl - nt * a.n_mt;

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wave >> 1, wn = wave & 1;
    const int KB = a.KB;

    // global -> LDS copy: thread t moves 64 bytes of activation unit t/32 and
    // 64 bytes of weight unit t/32
    const int cu = tid >> 5, cofs = (tid & 31) * 64;
    const int m_tiles = a.Mpad >> 4;
    const buf_t rx = make_buf(a.xq, (uint32_t)((int64_t)m_tiles * KB * 2048));
    const buf_t rw = make_buf(a.w + (int64_t)(8 * nt + cu) * KB * 2048, (uint32_t)KB * 2048u);
    const int xt = 8 * mt + cu;                           // activation tile of this thread's copy
    const uint32_t xoff = xt < m_tiles ? (uint32_t)xt * KB * 2048u + cofs : kBufOutOfRange;
    const buf_t rsx = make_buf(a.sx, (uint32_t)((int64_t)KB * a.Mpad * 4));

    uint4 px[4], pw[4];
    auto fetch = [&](int kb) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            px[i] = buf_load16(rx, xoff == kBufOutOfRange ? kBufOutOfRange : xoff + 16 * i, (uint32_t)kb * 2048u);
            pw[i] = buf_load_stream16(rw, cofs + 16 * i, (uint32_t)kb * 2048u);
        }
    };
    auto stage = [&](int buf) {
        uint8_t* s = lds + buf * kStage;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            *reinterpret_cast<uint4*>(s + cu * 2048 + cofs + 16 * i) = px[i];
            *reinterpret_cast<uint4*>(s + 8 * 2048 + cu * 2048 + cofs + 16 * i) = pw[i];
        }
    };

    f32x4_t outer[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) outer[i][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};

    // rows of this lane's outputs: 16 * (8mt + 4wm + i) + 4(l/16) + r
    const int row0 = 16 * (8 * mt + 4 * wm) + 4 * (lane >> 4);

    fetch(0);
    stage(0);
    __syncthreads();
    for (int kb = 0; kb < KB; ++kb) {
        if (kb + 1 < KB) fetch(kb + 1);
        const float swv = load_uniform_f32(a.sw + (int64_t)nt * KB + kb);
        f32x4_t sc[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            // the bounds check of a buffer load covers the VGPR offset only, so the
            // whole offset goes there; rows past Mpad (whole groups of 4) read zeros
            const int row = row0 + 16 * i;
            const uint32_t so = row < a.Mpad ? ((uint32_t)kb * (uint32_t)a.Mpad + (uint32_t)row) * 4u : kBufOutOfRange;
            const uint4 s4 = buf_load16(rsx, so, 0u);
            sc[i] = f32x4_t{__uint_as_float(s4.x) * swv, __uint_as_float(s4.y) * swv, __uint_as_float(s4.z) * swv,
                            __uint_as_float(s4.w) * swv};
        }
        const uint8_t* s = lds + (kb & 1) * kStage;
        i32x8_t af[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) af[i] = lds_frag(s + (4 * wm + i) * 2048, lane);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const i32x8_t bf = lds_frag(s + (8 + 4 * wn + j) * 2048, lane);
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const f32x4_t blk = mfma_fp8(af[i], bf, f32x4_t{0.f, 0.f, 0.f, 0.f});
#pragma unroll
                for (int r = 0; r < 4; ++r) outer[i][j][r] = __builtin_fmaf(blk[r], sc[i][r], outer[i][j][r]);
            }
        }
        if (kb + 1 < KB) stage((kb + 1) & 1);
        __syncthreads();
    }

    // D of a 16x16 tile: lane l holds rows 4(l/16)..+3 of column l%16
    const int col0 = 16 * (8 * nt + 4 * wn) + (lane & 15);
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int m = row0 + 16 * i + r;
            if (m < a.M) {
#pragma unroll
                for (int j = 0; j < 4; ++j) a.y[(int64_t)m * a.ldy + col0 + 16 * j] = f32_to_bf16_rne(outer[i][j][r]);
            }
        }
}

// --------------------------------------------------------------- launchers

static unsigned blocks_of(int64_t n) { return (unsigned)((n + 255) / 256); }

hipError_t launch_quantize_x(const uint16_t* x, int64_t ldx, int M, int K, uint8_t* xq, hipStream_t stream)
{
    const int Mpad = (M + 15) & ~15, KB = K / 128;
    hipLaunchKernelGGL(quantize_x_kernel, dim3(blocks_of((int64_t)Mpad * KB * 16)), dim3(256), 0, stream, x, ldx, M,
                       Mpad, KB, xq);
    return hipGetLastError();
}

hipError_t launch_unpack_x(const uint8_t* xq, int M, int K, uint8_t* codes, float* scales, hipStream_t stream)
{
    const int Mpad = (M + 15) & ~15, KB = K / 128;
    hipLaunchKernelGGL(unpack_x_kernel, dim3(blocks_of((int64_t)M * K)), dim3(256), 0, stream, xq, M, Mpad, KB, codes,
                       scales);
    return hipGetLastError();
}

hipError_t launch_w8a8(const uint8_t* packed_w, int N, int K, const uint8_t* xq, int M, uint16_t* y, int64_t ldy,
                       hipStream_t stream)
{
    W8Args a{};
    a.KB = K / 128;
    a.N = N;
    a.M = M;
    a.Mpad = (M + 15) & ~15;
    a.w = packed_w;
    a.sw = reinterpret_cast<const float*>(packed_w + (int64_t)N * K);
    a.xq = xq;
    a.sx = reinterpret_cast<const float*>(xq + (int64_t)a.Mpad * K);
    a.y = y;
    a.ldy = ldy;
    a.n_mt = (a.Mpad + 127) / 128;
    a.n_wg = a.n_mt * (N / 128);
    const int grid = (a.n_wg + 7) & ~7;
    const size_t lds = 2 * 16 * 2048;
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(w8a8_gemm_kernel),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(w8a8_gemm_kernel, dim3(grid), dim3(256), lds, stream, a);
    return hipGetLastError();
}

}  // namespace wq
