// Single-token state update with the state stored in 16 bits (fp16 or bf16) and computed in
// fp32 (the modeling_nemotron_h.py walk-through, 部署时如何调这些缓存: inference engines keep the
// Mamba state cache in fp16 with stochastic rounding from a Philox generator of 5 rounds;
// "MAX 平台 Nemotron-H 混合架构解析", 5.4: a narrower stored state, fp32 accumulation).
//
// The state moves 2 + 2 bytes per element instead of 4 + 4.  Each thread owns octets of 8
// consecutive state elements (16 bytes, one wave-wide access of 1 KB); one Philox4x32 call per
// octet gives the 8 16-bit random numbers its stochastic rounding uses.  Stochastic rounding
// (Philox stream and rule as in include/ssd.h):
//   element e (flat index in the state array or pool) draws r16 = 16-bit half (e mod 2), low
//   first, of word (e mod 8) div 2 of Philox4x32-R(counter (e/8 low, e/8 high, offset low,
//   offset high), key (seed low, seed high)), and moves to the next code away from zero iff
//   r16 < 65536 * (distance past the code toward zero) / spacing.
// Philox4x32 is written from its publication (Salmon, Moraes, Dror, Shaw, SC 2011).
#include "ssd_device.h"
#include "ssd_kernels.h"

#include <type_traits>

namespace ssd {

constexpr int kLpThreads = 128;
constexpr int kLpPerThread = 2;   // octets per thread

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
struct Bf16Fmt {
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

// Eight consecutive activation values as fp32.
template <typename T>
__device__ __forceinline__ void load8_f32(const T* p, float (&out)[8]) {
    load16_f32(p, out);
    if constexpr (Vec16<T>::n == 4) load16_f32(p + 4, out + 4);
}

// Grid: one thread per kLpPerThread octets of the [B, H, P, N] walk, 128-thread strides.
template <typename T, typename TY, class F, int N, bool SR, bool DTP>
__global__ __launch_bounds__(kLpThreads) void state_update_lp_kernel(
    uint16_t* __restrict__ state, const T* __restrict__ x, int64_t xs, const T* __restrict__ Bm,
    const T* __restrict__ Cm, int64_t bcs, const T* __restrict__ dt, const float* __restrict__ A,
    const float* __restrict__ D, TY* __restrict__ y, int64_t total8, int H, int P, int hpg,
    const int32_t* __restrict__ slot_idx, int64_t nslots, DtParams dtp, uint64_t seed, uint64_t offset,
    int rounds) {
    constexpr int OPR = N / 8;  // octets per state row
    constexpr int kSpan = kLpThreads * kLpPerThread;
    const int64_t per_b = static_cast<int64_t>(H) * P * OPR;
    const int lp = __builtin_ctz(static_cast<unsigned>(P));   // head_dim is a power of two
    u32x4* st = reinterpret_cast<u32x4*>(state);
    const int64_t f0 = static_cast<int64_t>(blockIdx.x) * kSpan;
    const int64_t base = f0 + threadIdx.x;
    // The block's octets almost always lie in one batch entry (UNI): its index and slot are then
    // block constants (one slot lookup for the block) and each octet's offset in the entry is the
    // block's plus the thread's; otherwise each octet divides its flat index.
    const int64_t ub = f0 / per_b;
    const int64_t r0 = f0 - ub * per_b;
    const int64_t span = total8 - f0 < kSpan ? total8 - f0 : kSpan;
    auto body = [&](auto uni_tag) {
        constexpr bool UNI = decltype(uni_tag)::value;
        const int64_t uslot = UNI ? (slot_idx ? seq_slot(slot_idx, ub, nslots) : ub) : 0;

        // per octet: batch entry, offset inside its state (< 2^31: the ABI bounds H*P*N), octet index
        // in the state array (-1: padding)
        u32x4 raw[kLpPerThread];
        int64_t bb[kLpPerThread], so[kLpPerThread];
        uint32_t rem[kLpPerThread];
#pragma unroll
        for (int i = 0; i < kLpPerThread; ++i) {
            const int64_t f = base + i * kLpThreads;
            const int64_t ff = f < total8 ? f : 0;
            int64_t slot;
            if constexpr (UNI) {
                bb[i] = ub;
                rem[i] = f < total8 ? static_cast<uint32_t>(r0) + threadIdx.x + i * kLpThreads : 0u;
                slot = uslot;
            } else {
                bb[i] = ff / per_b;
                rem[i] = static_cast<uint32_t>(ff - bb[i] * per_b);
                slot = slot_idx ? seq_slot(slot_idx, bb[i], nslots) : bb[i];
            }
            so[i] = (f < total8 && slot >= 0) ? slot * per_b + rem[i] : -1;
            raw[i] = so[i] >= 0 ? __builtin_nontemporal_load(st + so[i]) : u32x4{0u, 0u, 0u, 0u};
        }
#pragma unroll
        for (int i = 0; i < kLpPerThread; ++i) {
            const bool ok = base + i * kLpThreads < total8;
            const int64_t b = bb[i];
            const uint32_t rin = rem[i] / OPR;  // h*P + p inside the batch entry
            const int q = static_cast<int>(rem[i] % OPR);
            const int h = static_cast<int>(rin >> lp);
            const int p = static_cast<int>(rin & static_cast<uint32_t>(P - 1));
            const int g = h / hpg;
            const int64_t bh = b * H + h;
            const int64_t row = bh * P + p;
            const float dtv = DTP ? dt_prologue(static_cast<float>(dt[bh]), dtp, h) : static_cast<float>(dt[bh]);
            const float a = __expf(dtv * A[h]);
            const float xv = static_cast<float>(x[b * xs + static_cast<int64_t>(h) * P + p]);
            const int64_t bo = b * bcs + static_cast<int64_t>(g) * N + 8 * q;
            float bv[8], cv[8], v[8];
            load8_f32(Bm + bo, bv);
            load8_f32(Cm + bo, cv);
            const float dx = dtv * xv;
            float part = 0.f;
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const uint32_t word = raw[i][e >> 1];
                v[e] = fmaf(a, F::dec((e & 1) ? word >> 16 : word & 0xFFFFu), dx * bv[e]);
                part = fmaf(v[e], cv[e], part);
            }
            if (!ok) part = 0.f;
            part = group_sum_last<OPR>(part);
            if (ok && q == OPR - 1) y[row] = static_cast<TY>(part + (D ? D[h] * xv : 0.f));
            if (so[i] >= 0) {
                uint32_t rw[4];
                if constexpr (SR) {
                    const uint64_t o = static_cast<uint64_t>(so[i]);
                    uint32_t c[4] = {static_cast<uint32_t>(o), static_cast<uint32_t>(o >> 32),
                                     static_cast<uint32_t>(offset), static_cast<uint32_t>(offset >> 32)};
                    philox4x32(c, static_cast<uint32_t>(seed), static_cast<uint32_t>(seed >> 32), rounds);
                    // values below 2^-14 (fp16's subnormal range) anywhere in the wave?
                    bool sub = false;
#pragma unroll
                    for (int e = 0; e < 8; ++e) sub |= (__float_as_uint(v[e]) & 0x7FFFFFFFu) < 0x38800000u;
                    if (__builtin_amdgcn_ballot_w64(sub)) {
#pragma unroll
                        for (int w = 0; w < 4; ++w)
                            rw[w] = F::template sr<true>(v[2 * w], c[w] & 0xFFFFu) |
                                    (F::template sr<true>(v[2 * w + 1], c[w] >> 16) << 16);
                    } else {
#pragma unroll
                        for (int w = 0; w < 4; ++w)
                            rw[w] = F::template sr<false>(v[2 * w], c[w] & 0xFFFFu) |
                                    (F::template sr<false>(v[2 * w + 1], c[w] >> 16) << 16);
                    }
                } else {
#pragma unroll
                    for (int w = 0; w < 4; ++w) rw[w] = F::rne(v[2 * w]) | (F::rne(v[2 * w + 1]) << 16);
                }
                __builtin_nontemporal_store(u32x4{rw[0], rw[1], rw[2], rw[3]}, st + so[i]);
            }
        }
    };
    if (r0 + span <= per_b) body(std::true_type{});
    else body(std::false_type{});
}

template <typename T, typename TY, class F, int N>
static hipError_t lp_launch(const LpUpdateArgs& a, hipStream_t s) {
    const UpdateArgs& u = a.u;
    const int64_t total8 = u.batch * u.nheads * static_cast<int64_t>(u.head_dim) * (N / 8);
    if (total8 == 0) return hipSuccess;
    const int64_t per_block = kLpThreads * kLpPerThread;
    const dim3 grid(static_cast<uint32_t>((total8 + per_block - 1) / per_block));
    const bool dtp = u.dtp.bias || u.dtp.softplus || u.dtp.lo < u.dtp.hi;
    auto go = [&](auto kern) {
        hipLaunchKernelGGL(kern, grid, dim3(kLpThreads), 0, s, static_cast<uint16_t*>(a.state),
                           static_cast<const T*>(u.x), u.x_row_stride, static_cast<const T*>(u.B),
                           static_cast<const T*>(u.C), u.bc_row_stride, static_cast<const T*>(u.dt), u.A, u.D,
                           static_cast<TY*>(u.y), total8, u.nheads, u.head_dim, u.nheads / u.ngroups, u.slot_idx,
                           u.nslots, u.dtp, a.seed, a.offset, a.rounds);
        return hipGetLastError();
    };
    if (a.rounds > 0)
        return dtp ? go(state_update_lp_kernel<T, TY, F, N, true, true>)
                   : go(state_update_lp_kernel<T, TY, F, N, true, false>);
    return dtp ? go(state_update_lp_kernel<T, TY, F, N, false, true>)
               : go(state_update_lp_kernel<T, TY, F, N, false, false>);
}

template <typename T, typename TY, class F>
static hipError_t lp_n(const LpUpdateArgs& a, hipStream_t s) {
    switch (a.u.d_state) {
        case 16: return lp_launch<T, TY, F, 16>(a, s);
        case 32: return lp_launch<T, TY, F, 32>(a, s);
        case 64: return lp_launch<T, TY, F, 64>(a, s);
        case 128: return lp_launch<T, TY, F, 128>(a, s);
        default: return hipErrorInvalidValue;
    }
}

template <typename T, typename TY>
static hipError_t lp_f(const LpUpdateArgs& a, hipStream_t s) {
    return a.f16 ? lp_n<T, TY, F16Fmt>(a, s) : lp_n<T, TY, Bf16Fmt>(a, s);
}

hipError_t launch_state_update_lp(const LpUpdateArgs& a, Dt act, Dt ydt, hipStream_t s) {
    if (act == Dt::BF16) return ydt == Dt::BF16 ? lp_f<bf16, bf16>(a, s) : lp_f<bf16, float>(a, s);
    return ydt == Dt::BF16 ? lp_f<float, bf16>(a, s) : lp_f<float, float>(a, s);
}

}  // namespace ssd
