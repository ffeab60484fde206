// Device primitives for the gfx950 weight-only-quantized decode GEMM.
//
// Everything here runs inside the GEMM, pack and unpack kernels; the unpack
// test hooks call the very same dequant functions as the GEMM so that a
// bit-exact unpack proves the GEMM's dequant.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace wq {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef _Float16 f16x8_t __attribute__((ext_vector_type(8)));
typedef _Float16 f16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

constexpr int kBlock = 128;      // K extent of one scale block / group
constexpr int kTileN = 16;       // MFMA tile width along N (and along the batch M)
constexpr int kWave = 64;

// ------------------------------------------------------------- FP8 -> BF16
// E4M3FN -> BF16 is exact: every E4M3 value (including subnormals down to
// 2^-9) is a normal BF16 value, and NaN stays NaN.  gfx950's scaled converter
// with a unit scale performs exactly that conversion for two bytes at a time.
// HI selects bytes 2..3 of the word instead of bytes 0..1.
template <bool HI>
__device__ __forceinline__ uint32_t e4m3x2_to_bf16x2(uint32_t word)
{
    bf16x2_t r = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(word, 1.0f, HI);
    return __builtin_bit_cast(uint32_t, r);
}

// Eight consecutive codes (two dwords, bytes in memory order) -> eight BF16.
__device__ __forceinline__ bf16x8_t e4m3x8_to_bf16x8(uint32_t w0, uint32_t w1)
{
    u32x4_t r;
    r[0] = e4m3x2_to_bf16x2<false>(w0);
    r[1] = e4m3x2_to_bf16x2<true>(w0);
    r[2] = e4m3x2_to_bf16x2<false>(w1);
    r[3] = e4m3x2_to_bf16x2<true>(w1);
    return __builtin_bit_cast(bf16x8_t, r);
}

// E4M3FN pair -> FP32 pair (exact), used by the strict-order GEMV.
template <bool HI>
__device__ __forceinline__ f32x2_t e4m3x2_to_f32x2(uint32_t word)
{
    return __builtin_amdgcn_cvt_pk_f32_fp8(word, HI);
}

__device__ __forceinline__ float bf16_bits_to_f32(uint32_t bits16)
{
    return __builtin_bit_cast(float, bits16 << 16);
}

// ------------------------------------------------------- 3-bit LUT decode
// The learned 8-entry FP16 map is scaled by the row's group scale (one RNE
// FP16 multiply per entry, identical to rounding each dequantised weight) and
// split into two byte planes: LO holds the low bytes of entries 0..7, HI the
// high bytes.  A code word whose bytes are 0..7 is then a byte-permute
// selector into each plane.
struct LutPlanes {
    uint32_t lo0, lo1;   // low bytes of entries 0..3 / 4..7
    uint32_t hi0, hi1;   // high bytes of entries 0..3 / 4..7
};

// q[i] holds map entries (2i, 2i+1) as an FP16 pair; gg is the group scale
// in both halves.
__device__ __forceinline__ LutPlanes lut_scaled_planes2(const uint32_t q[4], f16x2_t gg)
{
    uint32_t e[4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
        e[i] = __builtin_bit_cast(uint32_t, __builtin_bit_cast(f16x2_t, q[i]) * gg);
    LutPlanes p;
    // v_perm pool = {S0 (bytes 4..7), S1 (bytes 0..3)}
    p.lo0 = __builtin_amdgcn_perm(e[1], e[0], 0x06040200u);
    p.hi0 = __builtin_amdgcn_perm(e[1], e[0], 0x07050301u);
    p.lo1 = __builtin_amdgcn_perm(e[3], e[2], 0x06040200u);
    p.hi1 = __builtin_amdgcn_perm(e[3], e[2], 0x07050301u);
    return p;
}

__device__ __forceinline__ LutPlanes lut_scaled_planes(const uint32_t q[4], _Float16 g)
{
    return lut_scaled_planes2(q, f16x2_t{g, g});
}

// One packed dword = eight 3-bit codes: byte b carries code e=b in its low
// nibble and code e=b+4 in its high nibble.  Returns the eight FP16 weights in
// order e = 0..7.
__device__ __forceinline__ f16x8_t lut_decode8(uint32_t word, const LutPlanes& p)
{
    uint32_t sl = word & 0x07070707u;
    uint32_t sh = (word >> 4) & 0x07070707u;
    uint32_t l0 = __builtin_amdgcn_perm(p.lo1, p.lo0, sl);
    uint32_t h0 = __builtin_amdgcn_perm(p.hi1, p.hi0, sl);
    uint32_t l1 = __builtin_amdgcn_perm(p.lo1, p.lo0, sh);
    uint32_t h1 = __builtin_amdgcn_perm(p.hi1, p.hi0, sh);
    u32x4_t r;
    r[0] = __builtin_amdgcn_perm(h0, l0, 0x05010400u);
    r[1] = __builtin_amdgcn_perm(h0, l0, 0x07030602u);
    r[2] = __builtin_amdgcn_perm(h1, l1, 0x05010400u);
    r[3] = __builtin_amdgcn_perm(h1, l1, 0x07030602u);
    return __builtin_bit_cast(f16x8_t, r);
}

// Dense 3-bit layout: a lane's 32 codes of one K block sit in three dwords.
// Dwords 0..2 carry MFMA steps 0..2 in the nibble positions above (bits 0-2
// and 4-6 of each byte); the codes of step 3 are spread over the spare bits:
// bit i of code e=b sits at bit 3 of byte b of dword i, and bit i of code
// e=b+4 at bit 7.  This gathers them into one word in the nibble layout (bits
// 3 and 7 of the result are junk; lut_decode8 ignores them): 3 shifts and 2
// bit-field inserts.
__device__ __forceinline__ uint32_t lut3d_step3_word(uint32_t d0, uint32_t d1, uint32_t d2)
{
    const uint32_t a = d0 >> 3, b = d1 >> 2, c = d2 >> 1;
    const uint32_t ab = (a & 0x11111111u) | (b & ~0x11111111u);     // bits 0, 4 from d0; 1, 5 from d1
    return (ab & 0x33333333u) | (c & ~0x33333333u);                 // bits 2, 6 from d2
}

// ------------------------------------------------------------------ MFMA
// D(16x16) += A(16x32) * B(32x16).  Lane l supplies A row (l % 16) and B
// column (l % 16), eight K values each at K group (l / 16); lane l receives
// D rows 4*(l/16) .. 4*(l/16)+3 of column (l % 16).
__device__ __forceinline__ f32x4_t mfma_bf16(bf16x8_t a, bf16x8_t b, f32x4_t c)
{
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ f32x4_t mfma_f16(f16x8_t a, f16x8_t b, f32x4_t c)
{
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}

// D(16x16) += A(16x128) * B(128x16) on E4M3 codes (the W8A8 product): lane l
// supplies its 32 codes of A row (l % 16) and of B column (l % 16), as the
// packed 2 KiB units lay them out (16 bytes of each 1 KiB chunk); lane l
// receives D rows 4*(l/16) .. 4*(l/16)+3 of column (l % 16).
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

// --------------------------------------------------------------- epilogue
__device__ __forceinline__ uint16_t f32_to_bf16_rne(float v)
{
    return __builtin_bit_cast(uint16_t, (__bf16)v);
}

__device__ __forceinline__ uint16_t f32_to_f16_rne(float v)
{
    return __builtin_bit_cast(uint16_t, (_Float16)v);
}

// Streaming 16-byte load for single-use weight bytes.
__device__ __forceinline__ uint4 load_stream16(const void* p)
{
    const u32x4_t v = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(p));
    return make_uint4(v[0], v[1], v[2], v[3]);
}

__device__ __forceinline__ uint4 load16(const void* p)
{
    return *reinterpret_cast<const uint4*>(p);
}

// 16-byte load of data that is read-only for the kernel's lifetime, through
// the constant address space: a wave-uniform address becomes a scalar load
// into SGPRs.
// ------------------------------------------------------------ buffer loads
// A buffer resource covers [base, base + bytes); a load whose per-lane offset
// (VGPR offset + instruction offset) lies at or past `bytes` returns zeros
// instead of touching memory.  The per-unit offset of a wave-uniform stream
// goes in the SGPR offset, so advancing a stream costs no VALU; selecting a
// resource with zero bytes turns a whole load into zeros.
typedef __amdgpu_buffer_rsrc_t buf_t;
constexpr uint32_t kBufOutOfRange = 0x80000000u;   // a VGPR offset past every resource used here

__device__ __forceinline__ buf_t make_buf(const void* base, uint32_t bytes)
{
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}

// streaming (non-temporal) 16-byte load
__device__ __forceinline__ uint4 buf_load_stream16(buf_t r, uint32_t voff, uint32_t soff)
{
    const u32x4_t v = __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(r, voff, soff, 2));
    return make_uint4(v[0], v[1], v[2], v[3]);
}

// 12 bytes (three dwords), non-temporal like buf_load_stream16; the fourth
// component of the result is zero.
__device__ __forceinline__ uint4 buf_load_stream12(buf_t r, uint32_t voff, uint32_t soff)
{
    typedef uint32_t u32x3_t __attribute__((ext_vector_type(3)));
    const u32x3_t v = __builtin_bit_cast(u32x3_t, __builtin_amdgcn_raw_buffer_load_b96(r, voff, soff, 2));
    return make_uint4(v[0], v[1], v[2], 0u);
}

__device__ __forceinline__ uint4 buf_load16(buf_t r, uint32_t voff, uint32_t soff)
{
    const u32x4_t v = __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(r, voff, soff, 0));
    return make_uint4(v[0], v[1], v[2], v[3]);
}

__device__ __forceinline__ uint32_t buf_load_u16(buf_t r, uint32_t voff, uint32_t soff)
{
    return (uint32_t)__builtin_amdgcn_raw_buffer_load_b16(r, voff, soff, 0);
}

// wave-uniform 4-byte load through the scalar (constant) cache
__device__ __forceinline__ float load_uniform_f32(const void* p)
{
    typedef const __attribute__((address_space(4))) float* cptr;
    return *(cptr)(p);
}

__device__ __forceinline__ uint4 load_uniform16(const void* p)
{
    typedef const __attribute__((address_space(4))) u32x4_t* cptr;
    const u32x4_t v = *(cptr)(p);
    return make_uint4(v[0], v[1], v[2], v[3]);
}

}  // namespace wq
