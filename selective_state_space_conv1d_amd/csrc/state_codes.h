// 16-bit state storage shared by the decode update and the scans: the Philox4x32 generator, the
// fp16 / bf16 code formats (decode, round to nearest even, stochastic rounding) and the element-wise
// loads and stores of a state array or pool held as codes.
// Stochastic rounding (the modeling_nemotron_h.py walk-through, 部署时如何调这些缓存: the Mamba
// state cache in fp16 with Philox-driven stochastic rounding): element e (its flat index in the
// state array or pool) draws r16 = 16-bit half (e mod 2), low first, of word (e mod 8) div 2 of
// Philox4x32-R(counter (e/8 low, e/8 high, offset low, offset high), key (seed low, seed high)),
// and moves to the next code away from zero iff r16 < 65536 * (distance past the code toward
// zero) / spacing.  Philox4x32 is written from its publication (Salmon, Moraes, Dror, Shaw, SC 2011).
#pragma once
#include "ssd_device.h"
#include "ssd_kernels.h"

namespace ssd {

// Philox4x32-R: per round, words 0 and 2 are multiplied by the two multipliers; the high halves
// of the products are mixed with words 1 and 3 and the key, the low halves become words 1 and 3.
// The key advances by the Weyl increments before each round after the first.
template <int R>   // R > 0: that many rounds, unrolled; R = 0: `rounds` rounds
__device__ __forceinline__ void philox4x32_r(uint32_t (&c)[4], uint32_t k0, uint32_t k1, int rounds) {
#pragma unroll
    for (int r = 0; r < (R > 0 ? R : rounds); ++r) {
        if (r) {
            k0 += 0x9E3779B9u;
            k1 += 0xBB67AE85u;
        }
        const uint64_t p0 = static_cast<uint64_t>(0xD2511F53u) * c[0];
        const uint64_t p1 = static_cast<uint64_t>(0xCD9E8D57u) * c[2];
        const uint32_t n0 = static_cast<uint32_t>(p1 >> 32) ^ c[1] ^ k0;
        const uint32_t n2 = static_cast<uint32_t>(p0 >> 32) ^ c[3] ^ k1;
        c[0] = n0;
        c[1] = static_cast<uint32_t>(p1);
        c[2] = n2;
        c[3] = static_cast<uint32_t>(p0);
    }
}

// 5 rounds (the engine setting on the modeling_nemotron_h.py walk-through page, 部署时如何调这些缓存)
// run unrolled; other round counts loop.
__device__ __forceinline__ void philox4x32(uint32_t (&c)[4], uint32_t k0, uint32_t k1, int rounds) {
    if (rounds == 5) philox4x32_r<5>(c, k0, k1, rounds);
    else philox4x32_r<0>(c, k0, k1, rounds);
}

// 16-bit storage formats: decode to fp32, round-to-nearest-even, stochastic rounding.
// Stochastic rounding "up (away from zero) iff r16 < 65536 * dropped fraction" equals "add the noise
// 2^d - 1 - floor(r16 / 2^(16-d)) to the d dropped bits and truncate" (d = 16 for bf16, 13 for fp16's
// normal range): both carry exactly when floor(r16 / 2^(16-d)) < the dropped bits.  The noise is the
// complement's top d bits, (~r16) >> (16 - d).  sr_pair rounds the two values of one Philox word that
// way (finite values for bf16, 2^-14 <= |v| < 65504 for fp16); special() flags the others, which take
// sr().
struct Bf16Fmt {
    static __device__ __forceinline__ bool special(float v) { return !(fabsf(v) < __builtin_inff()); }
    // v0 into the low code, v1 into the high one, r16 the low and high halves of word
    static __device__ __forceinline__ uint32_t sr_pair(float v0, float v1, uint32_t word) {
        const uint32_t nw = ~word;
        const uint32_t x0 = __float_as_uint(v0) + (nw & 0xFFFFu);
        const uint32_t x1 = __float_as_uint(v1) + (nw >> 16);
        uint32_t r = (x0 >> 16) | (x1 & 0xFFFF0000u);
        const bool s0 = special(v0), s1 = special(v1);
        if (__builtin_expect(s0 || s1, 0)) {   // one branch per pair, taken by the lanes that need it
            const uint32_t c0 = s0 ? sr<true>(v0, word & 0xFFFFu) : (r & 0xFFFFu);
            const uint32_t c1 = s1 ? sr<true>(v1, word >> 16) : (r >> 16);
            r = c0 | (c1 << 16);
        }
        return r;
    }
    static __device__ __forceinline__ float dec(uint32_t code) { return __uint_as_float(code << 16); }
    static __device__ __forceinline__ uint32_t rne(float v) {
        return __builtin_bit_cast(uint16_t, static_cast<__bf16>(v));
    }
    // bf16 keeps fp32's exponent: the 16 dropped bits are the distance past the truncated code
    // in units of 2^-16 spacing, and the truncated code + 1 is the next code away from zero.
    // Written with selects only: a branch per element would split the wave.
    template <bool SUB = true>
    static __device__ __forceinline__ uint32_t sr(float v, uint32_t r16) {
        const uint32_t u = __float_as_uint(v);
        const uint32_t t = (u >> 16) + (r16 < (u & 0xFFFFu) ? 1u : 0u);
        return (u & 0x7F800000u) == 0x7F800000u ? rne(v) : t;
    }
};

struct F16Fmt {
    static __device__ __forceinline__ bool special(float v) {   // true for NaN too
        const float m = fabsf(v);
        return !(m >= 0x1p-14f && m < 65504.0f);
    }
    // The noise goes into the 13 dropped bits of the fp32 pattern (a carry reaches the next code away
    // from zero, past the top of a binade into the next exponent), and the hardware's pair conversion
    // with round-toward-zero drops them: one conversion for both values.  Below 65504 the sum stays
    // under 65536, where that conversion would give the largest finite code instead of infinity.
    static __device__ __forceinline__ uint32_t sr_pair(float v0, float v1, uint32_t word) {
        const uint32_t nw = ~word;
        const float f0 = __uint_as_float(__float_as_uint(v0) + ((nw & 0xFFFFu) >> 3));
        const float f1 = __uint_as_float(__float_as_uint(v1) + (nw >> 19));
        uint32_t r = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_pkrtz(f0, f1));
        const bool s0 = special(v0), s1 = special(v1);
        if (__builtin_expect(s0 || s1, 0)) {   // one branch per pair, taken by the lanes that need it
            const uint32_t c0 = s0 ? sr<true>(v0, word & 0xFFFFu) : (r & 0xFFFFu);
            const uint32_t c1 = s1 ? sr<true>(v1, word >> 16) : (r >> 16);
            r = c0 | (c1 << 16);
        }
        return r;
    }
    static __device__ __forceinline__ float dec(uint32_t code) {
        return static_cast<float>(__builtin_bit_cast(_Float16, static_cast<uint16_t>(code)));
    }
    static __device__ __forceinline__ uint32_t rne(float v) {
        return __builtin_bit_cast(uint16_t, static_cast<_Float16>(v));
    }
    // Selects only, as for bf16.  SUB: some value of the wave is in fp16's subnormal range (the
    // caller tests that once per octet for the whole wave; the normal-range path alone is cheaper).
    template <bool SUB = true>
    static __device__ __forceinline__ uint32_t sr(float v, uint32_t r16) {
        const uint32_t u = __float_as_uint(v);
        const uint32_t a = u & 0x7FFFFFFFu;
        // fp16 normal range (|v| >= 2^-14): the code is fp32's top 10 mantissa bits under the
        // exponent rebiased from 127 to 15; 13 bits are dropped, so frac * 65536 = dropped << 3
        const uint32_t cn = (a >> 13) - (112u << 10) + (r16 < ((a & 0x1FFFu) << 3) ? 1u : 0u);
        // fp16 subnormals: q = |v| * 2^24 counts units of 2^-24 and is exact in fp32, as are its
        // integer part (the code), its fraction and the fraction * 65536
        uint32_t c = cn;   // +1 carries into the exponent, past 65504 into infinity
        if constexpr (SUB) {
            const float q = __uint_as_float(a < 0x38800000u ? a : 0u) * 16777216.0f;   // < 1024 (0 outside)
            const uint32_t ci = static_cast<uint32_t>(q);
            const uint32_t cs = ci + (static_cast<float>(r16) < (q - static_cast<float>(ci)) * 65536.0f ? 1u : 0u);
            c = a < 0x38800000u ? cs : cn;
        }
        c = a >= 0x47800000u ? 0x7C00u : c;       // |v| >= 65536: infinity
        const uint32_t r = ((u >> 16) & 0x8000u) | c;
        return a >= 0x7F800000u ? rne(v) : r;     // inf, NaN
    }
};

__device__ __forceinline__ float code_dec(uint32_t code, bool f16) {
    return f16 ? F16Fmt::dec(code) : Bf16Fmt::dec(code);
}

// Elements e .. e + 3 (e a multiple of 4) of a code array as fp32.
__device__ __forceinline__ f32x4 codes_load4(const uint16_t* p, bool f16, int64_t e) {
    const uint2 w = *reinterpret_cast<const uint2*>(p + e);
    return f32x4{code_dec(w.x & 0xFFFFu, f16), code_dec(w.x >> 16, f16), code_dec(w.y & 0xFFFFu, f16),
                 code_dec(w.y >> 16, f16)};
}

// The code of v for element e, given the Philox words of e's octet (unused when rounding to nearest).
__device__ __forceinline__ uint32_t code_round(float v, const Codes& c, const uint32_t (&w)[4], int64_t e) {
    if (c.rounds == 0) return c.f16 ? F16Fmt::rne(v) : Bf16Fmt::rne(v);
    const int i = static_cast<int>(e & 7);
    const uint32_t r16 = (w[i >> 1] >> (16 * (i & 1))) & 0xFFFFu;
    return c.f16 ? F16Fmt::sr<true>(v, r16) : Bf16Fmt::sr<true>(v, r16);
}

// The Philox words of the octet holding element e (not computed when rounding to nearest).
__device__ __forceinline__ void octet_words(const Codes& c, int64_t e, uint32_t (&w)[4]) {
    if (c.rounds == 0) return;
    const uint64_t o = static_cast<uint64_t>(e) >> 3;
    w[0] = static_cast<uint32_t>(o);
    w[1] = static_cast<uint32_t>(o >> 32);
    w[2] = static_cast<uint32_t>(c.offset);
    w[3] = static_cast<uint32_t>(c.offset >> 32);
    philox4x32(w, static_cast<uint32_t>(c.seed), static_cast<uint32_t>(c.seed >> 32), c.rounds);
}

// v rounded into elements e .. e + 3 (e a multiple of 4) of a code array.
__device__ __forceinline__ void codes_store4(uint16_t* p, const Codes& c, int64_t e, const f32x4& v) {
    uint32_t w[4] = {0u, 0u, 0u, 0u};
    octet_words(c, e, w);
    uint32_t k[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) k[i] = code_round(v[i], c, w, e + i);
    *reinterpret_cast<uint2*>(p + e) = uint2{k[0] | (k[1] << 16), k[2] | (k[3] << 16)};
}

// v rounded into element e of a code array.
__device__ __forceinline__ void codes_store1(uint16_t* p, const Codes& c, int64_t e, float v) {
    uint32_t w[4] = {0u, 0u, 0u, 0u};
    octet_words(c, e, w);
    p[e] = static_cast<uint16_t>(code_round(v, c, w, e));
}

}  // namespace ssd
