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
// GEMM schedule.  U = n_cg * KB units (a column group = NT tiles) are split
// into G contiguous ranges, one per persistent work-group, and each range into
// 4 contiguous per-wave ranges (stream-K; the FLUTE PR credits "striped
// Stream-K" for a tail-free grid, and the atlas "Module m16_tc" docs, section
// "WHY THE FFN ARM LOSES", show what a partial last wave costs).  A wave walks
// its units with the next unit's loads in flight, folds each 128-K block onto
// FP32 accumulators, and on leaving a column group parks its partial tile in
// LDS.  The work-group then sums its waves' partials in wave order; a column
// group shared with neighbouring work-groups goes through the workspace and
// the last work-group to arrive sums all contributions in work-group order.
// Every sum therefore has a fixed order: results are deterministic.
#include "wq_device.hpp"
#include "wq_internal.h"

namespace wq {

// 4 KiB of zeros: the source of loads that have nothing to fetch (the
// prefetch past the end of a wave's range, tiles past N, batch rows >= M).
// Loading from here keeps every load unconditional.
__device__ __attribute__((aligned(256))) uint8_t g_zero_page[4096];

__device__ __forceinline__ int64_t range_begin(int64_t U, int G, int g)
{
    return (U * g) / G;
}

// The work-group whose range holds unit u.
__device__ __forceinline__ int wg_of(int64_t U, int G, int64_t u)
{
    return (int)(((u + 1) * G - 1) / U);
}

// ======================================================================
// Policies: per-unit loads and compute for each kernel kind.
// ======================================================================

// ---- FP8 weights, 16-row BF16 MFMA tile ------------------------------------
// A operand = dequantised weights (lane: row n = l%16), B operand = x
// (lane: batch row m = l%16).  Output D[n][m] -> lane holds n = 4(l/16)+v.
template <int NT>
struct MfmaFp8 {
    static constexpr int CGW = NT * 16;
    struct Unit {
        uint4 w[NT][2];
        uint4 x[4];
        float s;
        int valid;
    };
    const GemmArgs& a;
    int lane;
    const uint16_t* xrow;   // this lane's batch row, or nullptr if >= rows
    f32x4_t outer[NT];

    __device__ MfmaFp8(const GemmArgs& args, int l) : a(args), lane(l)
    {
        int m = l & 15;
        xrow = (m < a.rows) ? a.x + (int64_t)m * a.ldx : nullptr;
#pragma unroll
        for (int t = 0; t < NT; ++t) outer[t] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    }

    __device__ __forceinline__ void load(Unit& r, int64_t u, bool valid) const
    {
        const int64_t cg = valid ? u / a.KB : 0;
        const int kb = valid ? (int)(u - cg * a.KB) : 0;
        const int g4 = lane >> 4;
#pragma unroll
        for (int t = 0; t < NT; ++t) {
            const int64_t tile = cg * NT + t;
            const uint8_t* p = (valid && tile < a.n_tiles)
                                   ? a.codes + ((tile * a.KB + kb) << 11) + lane * 16
                                   : g_zero_page + lane * 16;
            r.w[t][0] = load_stream16(p);
            r.w[t][1] = load_stream16(p + ((valid && tile < a.n_tiles) ? 1024 : 0));
        }
        const uint16_t* xb = (valid && xrow) ? xrow + kb * 128 + g4 * 16 : nullptr;
#pragma unroll
        for (int f = 0; f < 4; ++f) {  // f = 2j + h -> k offset 64j + 8h
            const void* p = xb ? (const void*)(xb + (f >> 1) * 64 + (f & 1) * 8)
                               : (const void*)(g_zero_page + 1024 + f * 16);
            r.x[f] = load16(p);
        }
        const float* sc = reinterpret_cast<const float*>(a.scales);
        r.s = valid ? sc[(cg * CGW / 128) * a.KB + kb] : 0.f;
        r.valid = valid;
    }

    __device__ __forceinline__ void compute(const Unit& r)
    {
        f32x4_t blk[NT];
#pragma unroll
        for (int t = 0; t < NT; ++t) blk[t] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int f = 0; f < 4; ++f) {
            const bf16x8_t b = __builtin_bit_cast(bf16x8_t, r.x[f]);
            const int j = f >> 1, h = f & 1;
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

    // slot: [16 rows][CGW] FP32 partial tile of this wave
    __device__ __forceinline__ void flush(float* slot)
    {
        const int m = lane & 15, n4 = (lane >> 4) * 4;
#pragma unroll
        for (int t = 0; t < NT; ++t) {
            *reinterpret_cast<f32x4_t*>(slot + m * CGW + t * 16 + n4) = outer[t];
            outer[t] = f32x4_t{0.f, 0.f, 0.f, 0.f};
        }
    }
};

// ---- 3-bit LUT weights, 16-row FP16 MFMA tile -------------------------------
template <int NT>
struct MfmaLut {
    static constexpr int CGW = NT * 16;
    struct Unit {
        uint4 w[NT];
        uint4 x[4];
        uint32_t g[NT];      // FP16 group-scale bits, zero-extended
        int valid;
    };
    const GemmArgs& a;
    int lane;
    const uint16_t* xrow;
    uint32_t q[4];          // map entries as FP16 pairs
    f32x4_t acc[NT];

    __device__ MfmaLut(const GemmArgs& args, int l) : a(args), lane(l)
    {
        int m = l & 15;
        xrow = (m < a.rows) ? a.x + (int64_t)m * a.ldx : nullptr;
        const uint32_t* qm = reinterpret_cast<const uint32_t*>(a.qmap);
#pragma unroll
        for (int i = 0; i < 4; ++i) q[i] = qm[i];
#pragma unroll
        for (int t = 0; t < NT; ++t) acc[t] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    }

    __device__ __forceinline__ void load(Unit& r, int64_t u, bool valid) const
    {
        const int64_t cg = valid ? u / a.KB : 0;
        const int kb = valid ? (int)(u - cg * a.KB) : 0;
        const int g4 = lane >> 4;
        const uint16_t* sc = reinterpret_cast<const uint16_t*>(a.scales);
#pragma unroll
        for (int t = 0; t < NT; ++t) {
            const int64_t tile = cg * NT + t;
            const bool ok = valid && tile < a.n_tiles;
            const int64_t unit = tile * a.KB + kb;
            const uint8_t* p = ok ? a.codes + (unit << 10) + lane * 16 : g_zero_page + lane * 16;
            r.w[t] = load_stream16(p);
            r.g[t] = ok ? (uint32_t)sc[unit * 16 + (lane & 15)] : 0u;
        }
        const uint16_t* xb = (valid && xrow) ? xrow + kb * 128 + g4 * 32 : nullptr;
#pragma unroll
        for (int s = 0; s < 4; ++s) {
            const void* p = xb ? (const void*)(xb + s * 8) : (const void*)(g_zero_page + 1024 + s * 16);
            r.x[s] = load16(p);
        }
        r.valid = valid;
    }

    __device__ __forceinline__ void compute(const Unit& r)
    {
#pragma unroll
        for (int t = 0; t < NT; ++t) {
            const LutPlanes pl = lut_scaled_planes(q, __builtin_bit_cast(_Float16, (uint16_t)r.g[t]));
            const uint32_t wd[4] = {r.w[t].x, r.w[t].y, r.w[t].z, r.w[t].w};
#pragma unroll
            for (int s = 0; s < 4; ++s)
                acc[t] = mfma_f16(lut_decode8(wd[s], pl), __builtin_bit_cast(f16x8_t, r.x[s]), acc[t]);
        }
    }

    __device__ __forceinline__ void flush(float* slot)
    {
        const int m = lane & 15, n4 = (lane >> 4) * 4;
#pragma unroll
        for (int t = 0; t < NT; ++t) {
            *reinterpret_cast<f32x4_t*>(slot + m * CGW + t * 16 + n4) = acc[t];
            acc[t] = f32x4_t{0.f, 0.f, 0.f, 0.f};
        }
    }
};

// ---- FP8 weights, strict-K-order GEMV (MR <= 4 rows) ------------------------
// Lane l owns output column n = l%16 of each tile and the K slice
// 16(l/16) .. +15 of each 64-wide chunk.  One FP32 accumulator per (tile, row)
// and lane takes its products in increasing k; each 128-K block is then folded
// onto the outer accumulator times the block scale.  At a column-group end
// the four K-slice lanes of a column are summed in a fixed butterfly.
template <int NT, int MR>
struct GemvFp8 {
    static constexpr int CGW = NT * 16;
    struct Unit {
        uint4 w[NT][2];
        uint4 x[MR][2][2];   // [row][chunk j][half]
        float s;
        int valid;
    };
    const GemmArgs& a;
    int lane;
    float outer[NT][MR];

    __device__ GemvFp8(const GemmArgs& args, int l) : a(args), lane(l)
    {
#pragma unroll
        for (int t = 0; t < NT; ++t)
#pragma unroll
            for (int m = 0; m < MR; ++m) outer[t][m] = 0.f;
    }

    __device__ __forceinline__ void load(Unit& r, int64_t u, bool valid) const
    {
        const int64_t cg = valid ? u / a.KB : 0;
        const int kb = valid ? (int)(u - cg * a.KB) : 0;
        const int g4 = lane >> 4;
#pragma unroll
        for (int t = 0; t < NT; ++t) {
            const int64_t tile = cg * NT + t;
            const bool ok = valid && tile < a.n_tiles;
            const uint8_t* p = ok ? a.codes + ((tile * a.KB + kb) << 11) + lane * 16
                                  : g_zero_page + lane * 16;
            r.w[t][0] = load_stream16(p);
            r.w[t][1] = load_stream16(p + (ok ? 1024 : 0));
        }
#pragma unroll
        for (int m = 0; m < MR; ++m)
#pragma unroll
            for (int j = 0; j < 2; ++j)
#pragma unroll
                for (int hh = 0; hh < 2; ++hh) {
                    const void* p = valid ? (const void*)(a.x + (int64_t)m * a.ldx + kb * 128 + j * 64 + g4 * 16 + hh * 8)
                                          : (const void*)(g_zero_page + 1024 + (m * 4 + j * 2 + hh) * 16);
                    r.x[m][j][hh] = load16(p);
                }
        const float* sc = reinterpret_cast<const float*>(a.scales);
        r.s = valid ? sc[(cg * CGW / 128) * a.KB + kb] : 0.f;
        r.valid = valid;
    }

    __device__ __forceinline__ void compute(const Unit& r)
    {
        float blk[NT][MR];
#pragma unroll
        for (int t = 0; t < NT; ++t)
#pragma unroll
            for (int m = 0; m < MR; ++m) blk[t][m] = 0.f;
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            float xf[MR][16];
#pragma unroll
            for (int m = 0; m < MR; ++m)
#pragma unroll
                for (int hh = 0; hh < 2; ++hh) {
                    const uint4 v = r.x[m][j][hh];
                    const uint32_t d[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        xf[m][hh * 8 + 2 * i] = bf16_bits_to_f32(d[i] & 0xFFFFu);
                        xf[m][hh * 8 + 2 * i + 1] = bf16_bits_to_f32(d[i] >> 16);
                    }
                }
#pragma unroll
            for (int t = 0; t < NT; ++t) {
                const uint4 w = r.w[t][j];
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
#pragma unroll
                for (int i = 0; i < 16; ++i)
#pragma unroll
                    for (int m = 0; m < MR; ++m) blk[t][m] = __builtin_fmaf(xf[m][i], wf[i], blk[t][m]);
            }
        }
#pragma unroll
        for (int t = 0; t < NT; ++t)
#pragma unroll
            for (int m = 0; m < MR; ++m) outer[t][m] = __builtin_fmaf(r.s, blk[t][m], outer[t][m]);
    }

    __device__ __forceinline__ void flush(float* slot)
    {
#pragma unroll
        for (int t = 0; t < NT; ++t)
#pragma unroll
            for (int m = 0; m < MR; ++m) {
                float v = outer[t][m];
                v += __shfl_xor(v, 16);
                v += __shfl_xor(v, 32);
                if (lane < 16) slot[m * CGW + t * 16 + lane] = v;
                outer[t][m] = 0.f;
            }
    }
};

// ======================================================================
// The persistent stream-K GEMM kernel.
// ======================================================================
template <class Pol, bool F16_OUT>
__global__ void __launch_bounds__(kThreadsPerWG)
gemm_kernel(GemmArgs a)
{
    constexpr int CGW = Pol::CGW;
    constexpr int SLOT = 16 * CGW;            // floats in one partial tile
    extern __shared__ float lds[];            // [slots][kWavesPerWG][SLOT]
    __shared__ uint32_t s_arrival;

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int g = blockIdx.x;
    const int64_t ub = range_begin(a.U, a.G, g), ue = range_begin(a.U, a.G, g + 1);
    const int64_t len = ue - ub;
    const int64_t cg_first = ub / a.KB;
    const int64_t cg_last = (ue - 1) / a.KB;

    // ---------------- per-wave stream over its unit range ----------------
    {
        const int64_t wb = ub + (len * wave) / kWavesPerWG;
        const int64_t we = ub + (len * (wave + 1)) / kWavesPerWG;
        Pol pol(a, lane);
        if (wb < we) {
            typename Pol::Unit r0, r1;
            pol.load(r0, wb, true);
            int64_t u = wb;
            while (true) {
                pol.load(r1, u + 1, u + 1 < we);
                pol.compute(r0);
                if (u + 1 == we || (u + 1) % a.KB == 0)
                    pol.flush(lds + ((u / a.KB - cg_first) * kWavesPerWG + wave) * SLOT);
                if (++u >= we) break;
                pol.load(r0, u + 1, u + 1 < we);
                pol.compute(r1);
                if (u + 1 == we || (u + 1) % a.KB == 0)
                    pol.flush(lds + ((u / a.KB - cg_first) * kWavesPerWG + wave) * SLOT);
                if (++u >= we) break;
            }
        }
    }
    __syncthreads();

    // ---------------- work-group reduction and epilogue ------------------
    for (int64_t c = cg_first; c <= cg_last; ++c) {
        const int64_t c0 = c * a.KB, c1 = c0 + a.KB;
        const bool covered = (c0 >= ub) && (c1 <= ue);
        uint32_t wmask = 0;
#pragma unroll
        for (int w = 0; w < kWavesPerWG; ++w) {
            const int64_t b = ub + (len * w) / kWavesPerWG, e = ub + (len * (w + 1)) / kWavesPerWG;
            if (b < e && b < c1 && e > c0) wmask |= 1u << w;
        }
        const float* slots = lds + (c - cg_first) * kWavesPerWG * SLOT;
        const int nout = a.rows * CGW;
        float* part = a.partials + ((int64_t)g * 2 + (c == cg_first ? 0 : 1)) * SLOT;
        for (int e = tid; e < nout; e += kThreadsPerWG) {
            float v = 0.f;
            bool first = true;
#pragma unroll
            for (int w = 0; w < kWavesPerWG; ++w)
                if (wmask & (1u << w)) {
                    const float p = slots[w * SLOT + e];
                    v = first ? p : v + p;
                    first = false;
                }
            if (covered) {
                const int m = e / CGW;
                const int64_t n = c * CGW + (e - m * CGW);
                if (n < a.N)
                    a.y[m * a.ldy + n] = F16_OUT ? f32_to_f16_rne(v) : f32_to_bf16_rne(v);
            } else {
                part[e] = v;
            }
        }
        if (covered) continue;

        // publish this work-group's partial; the last of the column group's
        // work-groups to arrive sums every contribution in work-group order
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");
        __syncthreads();
        if (tid == 0) {
            __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");
            s_arrival = __hip_atomic_fetch_add(a.counters + c, 1u, __ATOMIC_ACQ_REL,
                                               __HIP_MEMORY_SCOPE_AGENT);
        }
        __syncthreads();
        const int gf = wg_of(a.U, a.G, c0), gl = wg_of(a.U, a.G, c1 - 1);
        if (s_arrival == (uint32_t)(gl - gf)) {
            __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
            for (int e = tid; e < nout; e += kThreadsPerWG) {
                float v = 0.f;
                for (int gg = gf; gg <= gl; ++gg) {
                    const int64_t first_cg = range_begin(a.U, a.G, gg) / a.KB;
                    const float p = __builtin_nontemporal_load(
                        a.partials + ((int64_t)gg * 2 + (c == first_cg ? 0 : 1)) * SLOT + e);
                    v = (gg == gf) ? p : v + p;
                }
                const int m = e / CGW;
                const int64_t n = c * CGW + (e - m * CGW);
                if (n < a.N)
                    a.y[m * a.ldy + n] = F16_OUT ? f32_to_f16_rne(v) : f32_to_bf16_rne(v);
            }
            if (tid == 0)
                __hip_atomic_store(a.counters + c, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
        __syncthreads();   // s_arrival is reused by the next column group
    }
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

template <class Pol, bool F16>
static hipError_t launch_one(const GemmArgs& a, size_t lds, hipStream_t s)
{
    auto fn = gemm_kernel<Pol, F16>;
    if (lds > 64 * 1024) {
        hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(fn),
                                           hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
        if (e != hipSuccess) return e;
    }
    hipLaunchKernelGGL(fn, dim3(a.G), dim3(kThreadsPerWG), lds, s, a);
    return hipGetLastError();
}

template <int NT>
static hipError_t launch_nt(int kind, int rows, const GemmArgs& a, size_t lds, hipStream_t s)
{
    switch (kind) {
    case KIND_MFMA_FP8: return launch_one<MfmaFp8<NT>, false>(a, lds, s);
    case KIND_MFMA_LUT: return launch_one<MfmaLut<NT>, true>(a, lds, s);
    case KIND_GEMV_FP8:
        switch (rows) {
        case 1: return launch_one<GemvFp8<NT, 1>, false>(a, lds, s);
        case 2: return launch_one<GemvFp8<NT, 2>, false>(a, lds, s);
        case 3: return launch_one<GemvFp8<NT, 3>, false>(a, lds, s);
        case 4: return launch_one<GemvFp8<NT, 4>, false>(a, lds, s);
        default: return hipErrorInvalidValue;
        }
    default: return hipErrorInvalidValue;
    }
}

hipError_t launch_gemm(int kind, int nt, int gemv_rows, const GemmArgs& a, size_t lds_bytes, hipStream_t stream)
{
    switch (nt) {
    case 2: return launch_nt<2>(kind, gemv_rows, a, lds_bytes, stream);
    case 4: return launch_nt<4>(kind, gemv_rows, a, lds_bytes, stream);
    case 8: return launch_nt<8>(kind, gemv_rows, a, lds_bytes, stream);
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
