// nvfp4.hpp -- device functions of the NVFP4 encoding of SpliceGEMM
// (FourSight, arXiv 2611.04887v1: Sec. 2 NVFP4 blocks, Sec. 5.1 data
// preparation, App. 9.3.1 Eq. 9): the protected-channel mask, the block amax,
// the E4M3 block scale and the E2M1 codes.  Shared by the quantize kernel and
// the decode kernel that prepares its activations in its prologue, so both
// take the same decisions.
#pragma once
#include "common.hpp"

// Every floating-point step below is one IEEE operation: the functions that
// do arithmetic open with a contract(off) pragma, scoped to their body so
// that including this header changes nothing in the including file.

namespace splice {

__device__ __forceinline__ float bf16_bits_to_f32(unsigned b) { return __uint_as_float(b << 16); }

// ===========================================================================
// Protected-channel bitmask in LDS (bit j of the mask = channel j is in S).
// ===========================================================================
constexpr int MAX_K = 65536;

__device__ __forceinline__ void build_mask(uint32_t *smask, int64_t K, const int32_t *idx,
                                           int32_t k)
{
    const int words = (int)((K + 31) / 32);
    for (int i = threadIdx.x; i < words; i += blockDim.x) smask[i] = 0;
    __syncthreads();
    for (int i = threadIdx.x; i < k; i += blockDim.x) {
        const int c = idx[i];
        if (c >= 0 && c < K) atomicOr(&smask[c >> 5], 1u << (c & 31));
    }
    __syncthreads();
}

__device__ __forceinline__ unsigned block_mask16(const uint32_t *smask, int64_t b)
{
    return (smask[b >> 1] >> ((b & 1) * 16)) & 0xFFFFu;
}

// The 16 elements of one NVFP4 block as 8 words of two bf16 each (element 2t
// in the low half of word t).
struct Block16 { unsigned w[8]; };

__device__ __forceinline__ Block16 load_block(const uint16_t *p)
{
    const u32x4 v0 = reinterpret_cast<const u32x4 *>(p)[0];
    const u32x4 v1 = reinterpret_cast<const u32x4 *>(p)[1];
    return Block16{{v0.x, v0.y, v0.z, v0.w, v1.x, v1.y, v1.z, v1.w}};
}

// Sets the protected elements (bit e of m) to +0.
__device__ __forceinline__ void clear_protected(Block16 &x, unsigned m)
{
    // bit 2t of m stays at 2t, bit 2t+1 moves to 2t+16
    const unsigned spread = (m & 0x5555u) | ((m & 0xAAAAu) << 15);
#pragma unroll
    for (int t = 0; t < 8; t++) {
        const unsigned b = (spread >> (2 * t)) & 0x00010001u;
        x.w[t] &= ~((b << 16) - b);                  // 0xFFFF in each flagged half
    }
}

typedef __attribute__((ext_vector_type(2))) unsigned short u16x2;
typedef __attribute__((ext_vector_type(2))) short s16x2;

// Largest bf16 magnitude bit pattern of the block.
__device__ __forceinline__ unsigned block_amax_bits(const Block16 &x)
{
    u16x2 m = {0, 0};
#pragma unroll
    for (int t = 0; t < 8; t++)
        m = __builtin_elementwise_max(m, __builtin_bit_cast(u16x2, x.w[t] & 0x7FFF7FFFu));
    return max((unsigned)m.x, (unsigned)m.y);
}

// ===========================================================================
// NVFP4 quantization of one 16-element block (the masked residual): the block
// amax with the protected lanes read as +0, the E4M3 scale, sixteen E2M1
// codes.
//
// Exact decisions:
//  - scale: v = a_b / (6 alpha) in fp64 (6 alpha exact; the quotient of an
//    8-bit by a 26-bit operand is never within 2^-53 of an E4M3 rounding
//    midpoint unless it equals it), then round-to-nearest-even onto E4M3FN
//    with saturation at 448;
//  - codes: the seven midpoints m_i of the E2M1 grid times s_b*alpha are exact
//    in fp64 (3 x 4 x 24 bits).  Each becomes a 16-bit key: the largest bf16
//    magnitude pattern whose value lies below the midpoint (at or below it
//    for the midpoints whose ties go to the lower, even code).  The code of
//    an element is then the number of keys below its magnitude pattern,
//    found for two elements at once by a three-step binary search on packed
//    16-bit lanes (keys are non-decreasing, patterns and keys < 2^15, so the
//    sign bit of key - pattern says pattern > key).  The keys come from the
//    exact fp64 products, or, when alpha >= 2^-80, from fp32 products with
//    their fma residual, which yields the same keys with fewer instructions.
// ===========================================================================

// Round v >= 0 to E4M3FN, nearest, ties to even mantissa, saturating at 448.
__device__ __forceinline__ unsigned e4m3_rne_sat(double v)
{
#pragma clang fp contract(off)
    if (v >= 448.0) return 0x7Eu;
    if (v < 0.015625) return (unsigned)rint(v * 512.0);          // subnormals: m * 2^-9, m <= 8
    const int e = ilogb(v);                                       // -6 .. 8
    const int n = (int)rint(ldexp(v, 3 - e));                     // 8 .. 16
    return (unsigned)(((e + 7) << 3) + n - 8);
}

__device__ __forceinline__ double e4m3_value(unsigned b)
{
#pragma clang fp contract(off)
    const int e = (b >> 3) & 15, m = b & 7;
    return e ? ldexp(1.0 + (double)m * 0.125, e - 7) : ldexp((double)m, -9);
}

// Key of threshold t > 0 (exact in fp64), duplicated into both 16-bit halves.
// A bf16 magnitude pattern p is above the key iff its value is > t, or >= t
// when tie_up.  fp32 bits of the largest float below t (or <= t) are formed
// first; a bf16 pattern p exceeds them iff p exceeds their upper 16 bits.
__device__ __forceinline__ unsigned key_pair(double t, bool tie_up)
{
#pragma clang fp contract(off)
    unsigned kb;
    if (t >= 0x1p-126) {
        const float f = (float)t;                                 // nearest, t < FLT_MAX
        const double fd = (double)f;
        kb = __float_as_uint(f) - ((tie_up ? fd >= t : fd > t) ? 1u : 0u);
    } else {                                                      // fp32 subnormal range
        const double q = ldexp(t, 149);
        const double f = floor(q);
        kb = (unsigned)f - ((tie_up && f == q) ? 1u : 0u);        // t >= 2^-160: q > 0
    }
    return (kb >> 16) | (kb & 0xFFFF0000u);
}

// The same key for t = ms * alpha in fp32 arithmetic: ms = m_i * s is exact
// (at most 3 + 4 significant bits), hi = fl(ms * alpha) is the nearest float
// to t, i.e. the fp32 value key_pair starts from, and lo = fma(ms, alpha, -hi)
// is exactly t - hi as long as nothing underflows, so its sign says whether
// hi lies above, on or below t.  Valid when alpha >= 2^-80 (t >= 2^-91).
__device__ __forceinline__ unsigned key_pair_f32(float ms, float alpha, bool tie_up)
{
#pragma clang fp contract(off)
    const float hi = ms * alpha;
    const float lo = __builtin_fmaf(ms, alpha, -hi);
    const unsigned kb = __float_as_uint(hi) - ((tie_up ? lo <= 0.0f : lo < 0.0f) ? 1u : 0u);
    return (kb >> 16) | (kb & 0xFFFF0000u);
}

// 0xFFFF in each half where the pattern half of p2 is above the key half of
// k2: packed 16-bit subtract, then an arithmetic shift of each half by 15.
// (Written as two instructions: left to the compiler, the shift is turned
// into per-half compares and selects.)
__device__ __forceinline__ unsigned pk_above(unsigned p2, unsigned k2)
{
    unsigned d;
    asm("v_pk_sub_u16 %0, %1, %2\n\tv_pk_ashrrev_i16 %0, %3, %0"
        : "=&v"(d) : "v"(k2), "v"(p2), "v"(0x000F000Fu));
    return d;
}

__device__ __forceinline__ unsigned pick(unsigned m, unsigned a, unsigned b) { return (m & a) | (~m & b); }

// Four words of two nibbles each (bits 3:0 and 19:16) -> one word of eight
// nibbles in element order.
__device__ __forceinline__ unsigned pack_nibbles(unsigned a, unsigned b, unsigned c, unsigned d)
{
    const unsigned x = a | (b << 8), y = c | (d << 8);
    return ((x | (x >> 12)) & 0xFFFFu) | (((y | (y >> 12)) & 0xFFFFu) << 16);
}

// The tensor scale in the forms the block functions use.  fast: alpha is
// large enough for the fp32 keys (a property of the whole tensor, so every
// lane takes the same branch).
struct TensorScale {
    double alpha, six_alpha;
    float alpha_f;
    bool fast;
};

__device__ __forceinline__ TensorScale tensor_scale(float alpha)
{
#pragma clang fp contract(off)
    return TensorScale{(double)alpha, 6.0 * (double)alpha, alpha, alpha >= 0x1p-80f};
}

// E4M3 scale byte of a block from its amax pattern (protected lanes at +0).
__device__ __forceinline__ unsigned block_scale(unsigned amax_bits, const TensorScale &ts)
{
#pragma clang fp contract(off)
    return e4m3_rne_sat((double)bf16_bits_to_f32(amax_bits) / ts.six_alpha);
}

// Keys of the seven E2M1 midpoints times s*alpha (key_pair above).  When the
// scale byte is 0 every element codes to 0: all keys at the top.
struct Keys { unsigned k[7]; };

__device__ __forceinline__ Keys block_keys(unsigned sc, const TensorScale &ts)
{
#pragma clang fp contract(off)
    Keys r;
#pragma unroll
    for (int i = 0; i < 7; i++) r.k[i] = 0x7FFF7FFFu;
    if (sc != 0) {
        if (ts.fast) {
            const float s = (float)e4m3_value(sc);                   // exact
            r.k[0] = key_pair_f32(0.25f * s, ts.alpha_f, false);
            r.k[1] = key_pair_f32(0.75f * s, ts.alpha_f, true);
            r.k[2] = key_pair_f32(1.25f * s, ts.alpha_f, false);
            r.k[3] = key_pair_f32(1.75f * s, ts.alpha_f, true);
            r.k[4] = key_pair_f32(2.5f * s, ts.alpha_f, false);
            r.k[5] = key_pair_f32(3.5f * s, ts.alpha_f, true);
            r.k[6] = key_pair_f32(5.0f * s, ts.alpha_f, false);
        } else {
            const double phys = e4m3_value(sc) * ts.alpha;           // exact
            r.k[0] = key_pair(0.25 * phys, false);
            r.k[1] = key_pair(0.75 * phys, true);
            r.k[2] = key_pair(1.25 * phys, false);
            r.k[3] = key_pair(1.75 * phys, true);
            r.k[4] = key_pair(2.5 * phys, false);
            r.k[5] = key_pair(3.5 * phys, true);
            r.k[6] = key_pair(5.0 * phys, false);
        }
    }
    return r;
}

// Codes of the two elements of one word (bits 3:0 and 19:16): the number of
// keys below each magnitude pattern, found by a three-step binary search over
// the sorted keys, and the sign bit.
__device__ __forceinline__ unsigned code_word(unsigned w, const Keys &ks)
{
    const unsigned p2 = w & 0x7FFF7FFFu;
    const unsigned a4 = pk_above(p2, ks.k[3]);
    const unsigned a2 = pk_above(p2, pick(a4, ks.k[5], ks.k[1]));
    const unsigned a1 = pk_above(p2, pick(a4, pick(a2, ks.k[6], ks.k[4]), pick(a2, ks.k[2], ks.k[0])));
    return (a4 & 0x00040004u) | (a2 & 0x00020002u) | (a1 & 0x00010001u) | ((w >> 12) & 0x00080008u);
}

// Codes (16 nibbles, element 2i in the low nibble of byte i) and E4M3 scale
// byte of one block whose protected lanes are already +0.
__device__ __forceinline__ unsigned quantize_block(const Block16 &x, const TensorScale &ts, u32x2 &codes)
{
    const unsigned sc = block_scale(block_amax_bits(x), ts);
    const Keys ks = block_keys(sc, ts);
    unsigned nib[8];
#pragma unroll
    for (int t = 0; t < 8; t++) nib[t] = code_word(x.w[t], ks);
    codes = u32x2{pack_nibbles(nib[0], nib[1], nib[2], nib[3]), pack_nibbles(nib[4], nib[5], nib[6], nib[7])};
    return sc;
}

}  // namespace splice
