// Device-side helpers shared by the gfx950 kernels: vector types, bit casts,
// the 4-bit unpack/dequantize primitives and activation conversions.
//
// Nibble layout (zero-point page "Keep W4A16 zero-points packed at 4 bits
// instead of expanding to 2 bytes", section Change; the weight words use the
// same rule along K): value i of a packed word sits in bits 4*i.
//
// Element order inside a word (skinny GEMV form).  Masking a word with
// 0x0F0F0F0F leaves values 0, 2, 4, 6 in its four bytes, and shifting it right
// by 4 first leaves values 1, 3, 5, 7.  Pairing byte b with byte b + 2 of
// either gives 16-bit pairs holding values
//     (0,4) (1,5) (2,6) (3,7)
// so every consumer of that form stores the matching activations in that same
// order ("word order" below).  A dot product is invariant under a common
// permutation of both operands, so the order never changes a result.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace wob {

typedef _Float16 half2_t __attribute__((ext_vector_type(2)));
typedef _Float16 half8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf162_t __attribute__((ext_vector_type(2)));
typedef __bf16 bf168_t __attribute__((ext_vector_type(8)));
typedef float float4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

enum { DT_F16 = 0, DT_BF16 = 1 };

template <typename To, typename From>
__device__ __forceinline__ To bitcast(const From &f)
{
    static_assert(sizeof(To) == sizeof(From), "bitcast size");
    return __builtin_bit_cast(To, f);
}

// Word-order position p (0..7) holds value perm(p) of a packed word.
__host__ __device__ constexpr int word_order_value(int p) { return (p >> 1) + 4 * (p & 1); }

// Re-order eight consecutive 16-bit activations (natural order, four dwords)
// into word order: out dword j = (value j, value j+4).
__device__ __forceinline__ u32x4 to_word_order(u32x4 v)
{
    u32x4 o;
    // v_perm_b32 selector: bytes 0-3 come from src1, 4-7 from src0.
    o.x = __builtin_amdgcn_perm(v.z, v.x, 0x05040100u); // lo(v.x) | lo(v.z) << 16
    o.y = __builtin_amdgcn_perm(v.z, v.x, 0x07060302u); // hi(v.x) | hi(v.z) << 16
    o.z = __builtin_amdgcn_perm(v.w, v.y, 0x05040100u);
    o.w = __builtin_amdgcn_perm(v.w, v.y, 0x07060302u);
    return o;
}

// ---------------------------------------------------------------------------
// 4-bit unpack into exact (q - z) pairs (the skinny GEMV's weight operand),
// word order
// ---------------------------------------------------------------------------

// binary16 exponent byte of 1024: 0x64 in the high byte and a code q < 16 in
// the low byte read as the exact binary16 number 1024 + q.
constexpr uint32_t MAGIC4_F16 = 0x64646464u;

// binary16 pair -(1024 + z), -(1024 + z): adding it to a biased pair (1024 +
// q_a, 1024 + q_b) leaves (q_a - z, q_b - z) exactly.
__device__ __forceinline__ uint32_t f16_neg_bias2(uint32_t z)
{
    const uint32_t h = 0xE400u | z;
    return h | (h << 16);
}

// The same for the odd codes, which w4_diff_pairs_f16 reads in place in the
// high nibble under the exponent of 64: -(64 + z) twice.
__device__ __forceinline__ uint32_t f16_neg_bias2_hi(uint32_t z)
{
    const uint32_t h = 0xD400u | (z << 4);
    return h | (h << 16);
}

// Two binary16 exponent patterns in registers, opaque to the optimizer: with
// both constants of (a & m) | c known, the compiler emits a separate and and
// or (gfx950's three-operand encoding takes no literal); with c in a register
// it forms one v_and_or_b32.  Not volatile: the compiler may share and hoist
// them.
__device__ __forceinline__ uint32_t opaque_u32(uint32_t v)
{
    uint32_t r;
    asm("v_mov_b32 %0, %1" : "=v"(r) : "i"(v));
    return r;
}

// The four (q - z) pairs of a word in word order, as binary16.  Codes 0 and 4
// sit in the low nibbles of the word's two halves, codes 1 and 5 in the
// nibbles above them, and a shift by 8 brings codes 2, 6 and 3, 7 to the same
// places.  One and-or per pair keeps a pair's two nibbles and sets an
// exponent above them: 0x6400 over a low nibble reads as the exact binary16
// 1024 + q, 0x5400 over a high nibble (16 q in the mantissa, whose unit there
// is 1/16) as the exact 64 + q.  One packed add of -(1024 + z) or -(64 + z)
// per pair removes the bias exactly.  Nine vector operations per word (one
// shift, four and-or, four packed adds); byte permutes of the masked word
// took ten.
__device__ __forceinline__ u32x4 w4_diff_pairs_f16(uint32_t w, uint32_t negb2, uint32_t negb2_hi)
{
    const half2_t nb = bitcast<half2_t>(negb2);
    const half2_t nbh = bitcast<half2_t>(negb2_hi);
    const uint32_t w8 = w >> 8;
    const uint32_t e1024 = opaque_u32(0x64006400u), e64 = opaque_u32(0x54005400u);
    u32x4 o;
    o[0] = bitcast<uint32_t>(bitcast<half2_t>((w & 0x000F000Fu) | e1024) + nb);  // (v0, v4)
    o[1] = bitcast<uint32_t>(bitcast<half2_t>((w & 0x00F000F0u) | e64) + nbh);   // (v1, v5)
    o[2] = bitcast<uint32_t>(bitcast<half2_t>((w8 & 0x000F000Fu) | e1024) + nb); // (v2, v6)
    o[3] = bitcast<uint32_t>(bitcast<half2_t>((w8 & 0x00F000F0u) | e64) + nbh);  // (v3, v7)
    return o;
}

// Two fp32 values -> one dword of two bfloat16 (nearest even; exact for the
// small integers used here).
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b)
{
    typedef float f2_t __attribute__((ext_vector_type(2)));
    return bitcast<uint32_t>(__builtin_convertvector(f2_t{a, b}, bf162_t));
}

// The four (q - z) pairs of a word in word order, as bfloat16, with the same
// layout as w4_diff_pairs_f16: each code byte becomes an fp32 integer (the odd
// codes in place as 16 q, brought back to q by an fma with 1/16), z is
// subtracted exactly, and each pair is packed to bfloat16 (|q - z| <= 15 is
// exact there).  gfx950 has no packed bfloat16 add, so this goes through fp32.
__device__ __forceinline__ u32x4 w4_diff_pairs_bf16(uint32_t w, float zf)
{
    const uint32_t t0 = w & 0x0F0F0F0Fu; // codes 0, 2, 4, 6 in bytes 0..3
    const uint32_t t1 = w & 0xF0F0F0F0u; // 16 x codes 1, 3, 5, 7
    const float nz = -zf;
    auto hi = [&](uint32_t b) { return __builtin_fmaf((float)b, 0.0625f, nz); };
    u32x4 o;
    o[0] = pack_bf16x2((float)(t0 & 0xFFu) - zf, (float)((t0 >> 16) & 0xFFu) - zf); // (v0, v4)
    o[1] = pack_bf16x2(hi(t1 & 0xFFu), hi((t1 >> 16) & 0xFFu));                    // (v1, v5)
    o[2] = pack_bf16x2((float)((t0 >> 8) & 0xFFu) - zf, (float)(t0 >> 24) - zf);    // (v2, v6)
    o[3] = pack_bf16x2(hi((t1 >> 8) & 0xFFu), hi(t1 >> 24));                        // (v3, v7)
    return o;
}

// Zero-point of row r (0..7) in a packed zero-point word.
__device__ __forceinline__ uint32_t nib(uint32_t w, int r) { return (w >> (4 * r)) & 0xFu; }


// ---------------------------------------------------------------------------
// Activation conversions
// ---------------------------------------------------------------------------

__device__ __forceinline__ float act_to_f32(uint16_t v, int dt)
{
    if (dt == DT_F16)
        return (float)bitcast<_Float16>(v);
    return bitcast<float>((uint32_t)v << 16);
}

template <int DT>
__device__ __forceinline__ float act_to_f32(uint16_t v)
{
    if constexpr (DT == DT_F16)
        return (float)bitcast<_Float16>(v);
    else
        return bitcast<float>((uint32_t)v << 16);
}

// fp32 -> activation dtype, round to nearest even.
template <int DT>
__device__ __forceinline__ uint16_t f32_to_act(float f)
{
    if constexpr (DT == DT_F16)
        return bitcast<uint16_t>((_Float16)f);
    else
        return bitcast<uint16_t>((__bf16)f);
}

template <int DT>
__device__ __forceinline__ uint32_t f32x2_to_act2(float a, float b)
{
    // one packed conversion (v_cvt_pk_f16_f32 / v_cvt_pk_bf16_f32, nearest
    // even, as f32_to_act) instead of two conversions, a shift and an or
    typedef float f2_t __attribute__((ext_vector_type(2)));
    if constexpr (DT == DT_F16)
        return bitcast<uint32_t>(__builtin_convertvector(f2_t{a, b}, half2_t));
    else
        return bitcast<uint32_t>(__builtin_convertvector(f2_t{a, b}, bf162_t));
}


// ---------------------------------------------------------------------------
// MFMA operand forms: one packed word -> eight activation-dtype values in
// natural k order (value 2p and 2p+1 in 32-bit lane p), each the nearest-even
// rounding of the exact (q - z) * s.
// ---------------------------------------------------------------------------

// binary16: byte p of the word holds values 2p (low nibble) and 2p+1 (high
// nibble); one permute places it twice next to the binary16 exponent byte
// 0x64 and one mask keeps the low nibble in the first half and the high
// nibble (times 16) in the second: the exact halves (1024 + q_even,
// 1024 + 16 q_odd).  A packed fma with (1, 1/16) and -(1024 + z, 64 + z)
// gives the exact (q - z) pair, and a packed multiply by the scale rounds once.
__device__ __forceinline__ u32x4 w4_word_f16x8(uint32_t w, half2_t negb, half2_t s2)
{
    const half2_t mul = half2_t{(_Float16)1.0f, (_Float16)0.0625f};
    u32x4 o;
#pragma unroll
    for (int p = 0; p < 4; ++p) {
        const uint32_t sel = 0x04000400u | (uint32_t)p | ((uint32_t)p << 16);
        const uint32_t t = __builtin_amdgcn_perm(MAGIC4_F16, w, sel) & 0xFFF0FF0Fu;
        const half2_t d = __builtin_elementwise_fma(bitcast<half2_t>(t), mul, negb);
        o[p] = bitcast<uint32_t>(d * s2);
    }
    return o;
}

// The binary16 pair -(1024 + z, 64 + z) used by w4_word_f16x8.
__device__ __forceinline__ half2_t f16_neg_bias_pair(uint32_t z)
{
    return bitcast<half2_t>((0xE400u | z) | ((0xD400u | (z << 4)) << 16));
}

// bfloat16: the exact (q - z) pairs as binary16 (as w4_word_f16x8), each
// value scaled in fp32 by one v_fma_mix_f32 (binary16 operand, fp32 scale,
// addend -0): exactly (q - z) * s, since the product fits in 24 bits and the
// -0 addend keeps the IEEE sign of a zero product (0 * s, and s's Inf or
// NaN, pass through as in a multiply); one packed rounding to bfloat16 per
// pair.  `mz` must hold -0.0f in a way the compiler cannot see (a constant
// -0 addend is folded into a plain multiply, which costs a separate
// binary16-to-fp32 conversion per value).
__device__ __forceinline__ u32x4 w4_word_bf16x8(uint32_t w, float s, half2_t negb, float mz)
{
    const half2_t mul = half2_t{(_Float16)1.0f, (_Float16)0.0625f};
    u32x4 o;
#pragma unroll
    for (int p = 0; p < 4; ++p) {
        const uint32_t sel = 0x04000400u | (uint32_t)p | ((uint32_t)p << 16);
        const uint32_t t = __builtin_amdgcn_perm(MAGIC4_F16, w, sel) & 0xFFF0FF0Fu;
        const half2_t d = __builtin_elementwise_fma(bitcast<half2_t>(t), mul, negb);
        o[p] = f32x2_to_act2<DT_BF16>(__builtin_fmaf((float)d[0], s, mz),
                                      __builtin_fmaf((float)d[1], s, mz));
    }
    return o;
}

// -0.0f in a register, opaque to the optimizer (for w4_word_bf16x8).  Not
// volatile: the compiler may share and hoist it.
__device__ __forceinline__ float opaque_neg_zero()
{
    float mz;
    asm("v_mov_b32 %0, 0x80000000" : "=v"(mz));
    return mz;
}

// One weight word of the MFMA operand form from the scale bits and zero-point.
template <int DT>
__device__ __forceinline__ u32x4 w4_word_act8(uint32_t w, uint32_t sbits, uint32_t z)
{
    if constexpr (DT == DT_F16) {
        const _Float16 sh = bitcast<_Float16>((uint16_t)sbits);
        return w4_word_f16x8(w, f16_neg_bias_pair(z), half2_t{sh, sh});
    } else {
        return w4_word_bf16x8(w, act_to_f32<DT_BF16>((uint16_t)sbits), f16_neg_bias_pair(z),
                              opaque_neg_zero());
    }
}

// MXFP4: one word holds eight E2M1 elements in natural order (even element in
// the low nibble of each byte).  v_cvt_scalef32_pk_bf16_fp4 converts the two
// elements of one byte and multiplies them by the fp32 scale; the E8M0 byte
// becomes that scale by being placed in the binary32 exponent field ("Add
// BF16xFP4 MoE GEMM stage1 kernel", Technical Details).  Output pairs are in
// natural order: (0,1) (2,3) (4,5) (6,7).
//
// The byte-in-exponent placement is exact for b = 1..254.  The two ends of the
// E8M0 range follow the OCP MX definition instead: b = 0 is 2^-127, which
// binary32 holds as a subnormal (the shifted byte would read +0), and b = 255
// is NaN (the shifted byte would read +Inf).
__device__ __forceinline__ float e8m0_to_f32(uint32_t b)
{
    uint32_t bits = b << 23;
    bits = b == 0u ? 0x00400000u : bits;   // 2^-127
    bits = b == 255u ? 0x7FC00000u : bits; // NaN
    return bitcast<float>(bits);
}

__device__ __forceinline__ u32x4 fp4_word_bf16x8(uint32_t w, float scale)
{
    u32x4 o;
    o[0] = bitcast<uint32_t>(__builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, scale, 0));
    o[1] = bitcast<uint32_t>(__builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, scale, 1));
    o[2] = bitcast<uint32_t>(__builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, scale, 2));
    o[3] = bitcast<uint32_t>(__builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, scale, 3));
    return o;
}

// Wave-wide helpers.
__device__ __forceinline__ int lane_id() { return __lane_id(); }

} // namespace wob
