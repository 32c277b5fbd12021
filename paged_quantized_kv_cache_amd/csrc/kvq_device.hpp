// kvq_device.hpp -- device-side helpers shared by the libkvq kernels (gfx950).
//
// Element conversions used inside the attention loops.  They turn stored
// codes into exact fp16 values for the MFMA operands:
//   INT8 code c (|c| <= 127), stored as the excess-128 byte u = c + 128 ->
//     fp16 c: the 1024 + byte trick (an fp16 with exponent field 25 has a
//     unit step, so the bit pattern 0x6400 | u is the number 1024 + u) gives
//     c + 1152, and one packed fp16 subtraction per two codes removes 1152
//     exactly (all integers below 2048 are fp16 values).  The codes enter
//     the contractions unbiased: a bias removed after the dot products would
//     leave fp32 sums ~1152 / |c| times larger than the result, whose
//     rounding then shows in scores of large-scale keys and in outputs near
//     zero of large-scale values.
//   E4M3 code -> fp16 of the same value: gfx950's packed conversion
//     (v_cvt_scalef32_pk_f16_fp8, scale 1) turns two codes into two fp16 in
//     one instruction, exactly (every E4M3 value, subnormals included, is an
//     fp16 normal number); the NaN codes become NaN.
//   E5M2 code -> fp16 of the same value: E5M2 has fp16's sign and exponent
//     fields and its two top fraction bits, so the code is the fp16's high
//     byte.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

namespace kvq {

// FMT_FP8 is E4M3; FMT_E5M2 is the other OCP FP8 format; FMT_INT4 packs two
// codes per byte (head_dim 128 only).
enum { FMT_FP16 = 0, FMT_INT8 = 1, FMT_FP8 = 2, FMT_E5M2 = 3, FMT_INT4 = 4 };

// Largest finite value of each FP8 format.
template <int FMT>
constexpr float fp8_max()
{
    return FMT == FMT_E5M2 ? 57344.0f : 448.0f;
}

typedef _Float16 f16;
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// Compile-time loop: f(std::integral_constant<int, i>) for i in [B, E).
template <int B, int E, typename F>
__device__ __forceinline__ void static_for(F &&f)
{
    if constexpr (B < E) {
        f(std::integral_constant<int, B>{});
        static_for<B + 1, E>(f);
    }
}

template <typename To, typename From>
__device__ __forceinline__ To bit_cast(const From &x)
{
    static_assert(sizeof(To) == sizeof(From), "size mismatch");
    return __builtin_bit_cast(To, x);
}

// v_perm_b32: bytes 0..3 select from `lo`, 4..7 from `hi`, 0x0c -> 0x00.
__device__ __forceinline__ uint32_t byte_perm(uint32_t hi, uint32_t lo,
                                              uint32_t sel)
{
    return __builtin_amdgcn_perm(hi, lo, sel);
}

// Four excess-128 INT8 bytes (one dword) -> 4 exact fp16 holding c.
__device__ __forceinline__ f16x4 int8x4_to_f16x4(uint32_t w)
{
    const uint32_t lo = byte_perm(0x64646464u, w, 0x04010400u);  // 0x64 | byte 0, 0x64 | byte 1
    const uint32_t hi = byte_perm(0x64646464u, w, 0x04030402u);
    const f16x2 bias = {(f16)1152.0f, (f16)1152.0f};
    const f16x2 a = bit_cast<f16x2>(lo) - bias;
    const f16x2 b = bit_cast<f16x2>(hi) - bias;
    return f16x4{a.x, a.y, b.x, b.y};
}

// Four E4M3 bytes -> 4 fp16 of the same values (bytes 0, 1 from the low
// word, 2, 3 from the high word).
__device__ __forceinline__ f16x4 fp8x4_to_f16x4(uint32_t w)
{
    const f16x2 a = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w, 1.0f, false);
    const f16x2 b = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w, 1.0f, true);
    return f16x4{a.x, a.y, b.x, b.y};
}

// Eight excess-8 INT4 nibbles (one dword) -> two f16x4 holding c (1024 +
// nibble, less 1032): `lo` from the low nibbles of bytes 0..3, `hi` from the
// high nibbles.
__device__ __forceinline__ void int4x8_to_f16x4(uint32_t w, f16x4 &lo, f16x4 &hi)
{
    const uint32_t l = w & 0x0f0f0f0fu;
    const uint32_t h = (w >> 4) & 0x0f0f0f0fu;
    const f16x2 bias = {(f16)1032.0f, (f16)1032.0f};
    const f16x2 a = bit_cast<f16x2>(byte_perm(0x64646464u, l, 0x04010400u)) - bias;
    const f16x2 b = bit_cast<f16x2>(byte_perm(0x64646464u, l, 0x04030402u)) - bias;
    const f16x2 c = bit_cast<f16x2>(byte_perm(0x64646464u, h, 0x04010400u)) - bias;
    const f16x2 d = bit_cast<f16x2>(byte_perm(0x64646464u, h, 0x04030402u)) - bias;
    lo = f16x4{a.x, a.y, b.x, b.y};
    hi = f16x4{c.x, c.y, d.x, d.y};
}

// Four E5M2 bytes -> 4 fp16 of the same values (each byte becomes the high
// byte of an fp16 whose low byte is zero).
__device__ __forceinline__ f16x4 e5m2x4_to_f16x4(uint32_t w)
{
    const uint32_t h0 = byte_perm(0u, w, 0x010c000cu);  // b0 << 8, b1 << 24
    const uint32_t h1 = byte_perm(0u, w, 0x030c020cu);
    const f16x2 a = bit_cast<f16x2>(h0);
    const f16x2 b = bit_cast<f16x2>(h1);
    return f16x4{a.x, a.y, b.x, b.y};
}

__device__ __forceinline__ f16x4 f16x4_from_u2(uint32_t lo, uint32_t hi)
{
    const f16x2 a = bit_cast<f16x2>(lo);
    const f16x2 b = bit_cast<f16x2>(hi);
    return f16x4{a.x, a.y, b.x, b.y};
}

// Two fp32 values as fp16 pairs hi + lo with hi + lo within about 2^-21 of
// each value (relative, for values in fp16's normal range): hi keeps the top
// 11 significant bits (so converting it is exact), lo the remainder, which
// fp32 holds exactly, converted toward zero.
__device__ __forceinline__ void split_f16x2(float a, float b, f16x2 &hi, f16x2 &lo)
{
    const float ah = __uint_as_float(__float_as_uint(a) & 0xffffe000u);
    const float bh = __uint_as_float(__float_as_uint(b) & 0xffffe000u);
    hi = bit_cast<f16x2>(__builtin_amdgcn_cvt_pkrtz(ah, bh));
    lo = bit_cast<f16x2>(__builtin_amdgcn_cvt_pkrtz(a - ah, b - bh));
}

// The maxima of a and of b over the four 16-lane rows (lanes l, l ^ 16,
// l ^ 32, l ^ 48), each in every lane.  gfx950's lane-swap moves
// (v_permlane32_swap, v_permlane16_swap) keep it off the LDS path, and the
// first swap packs a's and b's half-reduced values into the two halves of
// one register, so the pair costs three swaps.
__device__ __forceinline__ void max_over_groups2(float &a, float &b)
{
    // lanes 0-31: max(a[l], a[l + 32]); lanes 32-63: max(b[l - 32], b[l])
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(a), __float_as_uint(b), false, false);
    float x = fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
    // rows 0, 1: a's maximum; rows 2, 3: b's
    const auto s = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    x = fmaxf(__uint_as_float(s[0]), __uint_as_float(s[1]));
    const auto t = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    a = __uint_as_float(t[0]);
    b = __uint_as_float(t[1]);
}

// The 8-element operand of a 16x16x32 MFMA from two 4-element halves.  A
// lane's 8 elements are 8 distinct positions of the summed (k) axis; which
// positions does not matter as long as both operands use the same order, so
// two 16x16x16 steps fold into one 16x16x32 step by concatenation.
__device__ __forceinline__ f16x8 cat8(f16x4 a, f16x4 b)
{
    return __builtin_shufflevector(a, b, 0, 1, 2, 3, 4, 5, 6, 7);
}

// D += A B over k = 16: lane (col, grp) holds k positions 4 grp .. 4 grp + 3
// of both operands and rows 4 grp .. 4 grp + 3 of column col of D.
__device__ __forceinline__ f32x4 mfma16(f16x4 a, f16x4 b, f32x4 c)
{
    return __builtin_amdgcn_mfma_f32_16x16x16f16(a, b, c, 0, 0, 0);
}

// D += A B over k = 32 (gfx950): the same output layout as 16x16x16 (lane
// (col, grp) holds rows 4 grp .. 4 grp + 3 of column col).
__device__ __forceinline__ f32x4 mfma32(f16x8 a, f16x8 b, f32x4 c)
{
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}

// Round to the nearest E4M3 value (ties to even), saturating to +-448; the
// sign of a zero result is kept.  Bit-level, from the format definition.
__device__ __forceinline__ uint32_t e4m3_rne_sat(float y)
{
    const uint32_t bits = __float_as_uint(y);
    const uint32_t sign = (bits >> 24) & 0x80u;
    const float a = __builtin_fabsf(y);
    if (a != a)
        return sign | 0x7fu;
    if (!(a < 448.0f))
        return sign | 0x7eu;
    if (a < 0.015625f) {  // below 2^-6: fixed spacing 2^-9
        const float q = __builtin_rintf(a * 512.0f);
        return sign | (uint32_t)q;  // 0..8, 8 is the smallest normal
    }
    const uint32_t ab = __float_as_uint(a);
    const uint32_t r = (ab + 0x7ffffu + ((ab >> 20) & 1u)) >> 20;  // 3 fraction bits, RNE
    return sign | (r - (120u << 3));  // exponent bias 127 -> 7
}

// Round to the nearest E5M2 value (ties to even), saturating to +-57344;
// the sign of a zero result is kept.  Bit-level, from the format definition.
__device__ __forceinline__ uint32_t e5m2_rne_sat(float y)
{
    const uint32_t bits = __float_as_uint(y);
    const uint32_t sign = (bits >> 24) & 0x80u;
    const float a = __builtin_fabsf(y);
    if (a != a)
        return sign | 0x7fu;
    if (!(a < 57344.0f))
        return sign | 0x7bu;
    if (a < 6.103515625e-05f) {  // below 2^-14: fixed spacing 2^-16
        const float q = __builtin_rintf(a * 65536.0f);
        return sign | (uint32_t)q;  // 0..4, 4 is the smallest normal
    }
    const uint32_t ab = __float_as_uint(a);
    const uint32_t r = (ab + 0xfffffu + ((ab >> 21) & 1u)) >> 21;  // 2 fraction bits, RNE
    return sign | (r - (112u << 2));  // exponent bias 127 -> 15
}

template <int FMT>
__device__ __forceinline__ uint32_t fp8_rne_sat(float y)
{
    if constexpr (FMT == FMT_E5M2)
        return e5m2_rne_sat(y);
    else
        return e4m3_rne_sat(y);
}

// ---------------------------------------------------------------- layouts
// Byte offset of element (token t, dim d) inside one (block, KV head) tile,
// EB bytes per element.  Both layouts are arranged so that every 16-byte
// load the decode kernel issues for a 16-token tile lands, across the 64
// lanes, on one contiguous 1 KiB run (whole 128-byte lines).
//
// K: rows of 64 bytes -- [D*EB/64 chunks][BS tokens][64 bytes]; a chunk is
//    64 int8/E4M3 dims or 32 fp16 dims of one token.
template <int D, int EB>
__host__ __device__ constexpr int k_offset(int BS, int t, int d)
{
    return ((d * EB / 64) * BS + t) * 64 + (d * EB) % 64;
}
// V: 16-byte micro-tiles of 4 tokens x (4 / EB) dims, grouped per 16-token
//    half of the block -- [BS/16][EB][D/4][4][4/EB dims][4 tokens][EB bytes]
//    with e = (d % 4) / (4 / EB).
template <int D, int EB>
__host__ __device__ constexpr int v_offset(int BS, int t, int d)
{
    return (((((t / 16) * EB + (d % 4) / (4 / EB)) * (D / 4) + d / 4) * 4 + (t % 16) / 4) * 16 +
            ((d % 4) % (4 / EB)) * 4 * EB + (t % 4) * EB);
}

// INT4 tiles (head_dim 128): 64 bytes per token of K, and per 16 tokens 1 KiB
// of V.  Byte of element (token t, dim d) and whether it is the high nibble:
// K: row t of 64 bytes; a 16-byte lane slice g = (d % 64) / 16 holds dwords
//    q = 2 (d / 64) + (d % 16) / 8 of 8 dims each, byte j of a dword holding
//    dims base + j (low nibble) and base + 4 + j (high).
// V: per 16-token half, [16 dim quads][4 token quads][4 dwords q][4 tokens]:
//    dword q = 2 (d / 64) + (d % 4) / 2 holds dims (even, odd) of a pair, byte
//    t % 4 the token's two codes (even dim low, odd dim high).
__host__ __device__ constexpr int int4_k_byte(int t, int d)
{
    return t * 64 + 16 * ((d % 64) / 16) + 4 * (2 * (d / 64) + (d % 16) / 8) + d % 4;
}
__host__ __device__ constexpr bool int4_k_high(int d) { return (d % 8) >= 4; }
__host__ __device__ constexpr int int4_v_byte(int t, int d)
{
    return (t / 16) * 1024 + ((((d % 64) / 4) * 4 + (t % 16) / 4) * 4 + 2 * (d / 64) + (d % 4) / 2) * 4 +
           t % 4;
}
__host__ __device__ constexpr bool int4_v_high(int d) { return (d % 2) == 1; }

__device__ __forceinline__ float wave_max(float x)
{
#pragma unroll
    for (int o = 1; o < 64; o <<= 1)
        x = fmaxf(x, __shfl_xor(x, o));
    return x;
}

__device__ __forceinline__ float wave_sum(float x)
{
#pragma unroll
    for (int o = 1; o < 64; o <<= 1)
        x += __shfl_xor(x, o);
    return x;
}

}  // namespace kvq
