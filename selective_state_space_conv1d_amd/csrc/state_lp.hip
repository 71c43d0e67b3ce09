// Single-token state update with the state stored in 16 bits (fp16 or bf16) and computed in
// fp32 (the modeling_nemotron_h.py walk-through, 部署时如何调这些缓存: inference engines keep the
// Mamba state cache in fp16 with stochastic rounding from a Philox generator of 5 rounds;
// "MAX 平台 Nemotron-H 混合架构解析", 5.4: a narrower stored state, fp32 accumulation).
//
// The state moves 2 + 2 bytes per element instead of 4 + 4.  Each thread owns octets of 8
// consecutive state elements (16 bytes) of one n position in several rows of a head, so the B and C
// octet it needs is loaded once; one Philox4x32 call per octet gives the 8 16-bit random numbers its
// stochastic rounding uses.  Stochastic rounding
// (Philox stream and rule as in include/ssd.h):
//   element e (flat index in the state array or pool) draws r16 = 16-bit half (e mod 2), low
//   first, of word (e mod 8) div 2 of Philox4x32-R(counter (e/8 low, e/8 high, offset low,
//   offset high), key (seed low, seed high)), and moves to the next code away from zero iff
//   r16 < 65536 * (distance past the code toward zero) / spacing.
#include "ssd_device.h"
#include "ssd_kernels.h"
#include "state_codes.h"

#include <type_traits>

namespace ssd {

constexpr int kLpThreads = 128;
constexpr int kLpRows = 32;   // state rows per block

// Eight consecutive activation values as fp32.
template <typename T>
__device__ __forceinline__ void load8_f32(const T* p, float (&out)[8]) {
    load16_f32(p, out);
    if constexpr (Vec16<T>::n == 4) load16_f32(p + 4, out + 4);
}

// Grid: each block takes RPB = max(RB, R) consecutive rows of one (batch entry, head) (R = 128 / (N/8)
// rows per pass).  Thread t owns octet q = t % (N/8) of rows p0 + t / (N/8) + R k: the group's B and C
// octet and the head's dt, A, D are loaded once and reused for every row, so the loads per state byte
// stay close to the state's own (the state is read and written once; the x value of a row is a
// broadcast load).  All of the thread's state octets are loaded before any is used.
template <typename T, typename TY, class F, int N, int RB, bool SR, bool DTP, bool HAS_STATE>
__global__ __launch_bounds__(kLpThreads) void state_update_lp_kernel(
    uint16_t* __restrict__ state, const T* __restrict__ x, int64_t xs, const T* __restrict__ Bm,
    const T* __restrict__ Cm, int64_t bcs, const T* __restrict__ dt, const float* __restrict__ A,
    const float* __restrict__ D, TY* __restrict__ y, int H, int P, int hpg,
    const int32_t* __restrict__ slot_idx, int64_t nslots, DtParams dtp, uint64_t seed, uint64_t offset,
    int rounds) {
    constexpr int OPR = N / 8;                 // octets per state row
    constexpr int R = kLpThreads / OPR;        // rows per pass
    constexpr int RPB = RB > R ? RB : R;       // rows per block
    constexpr int K = RPB / R;                 // passes
    const int nsplit = (P + RPB - 1) / RPB;    // blocks per head
    const int64_t per_b = static_cast<int64_t>(H) * P * OPR;
    u32x4* st = reinterpret_cast<u32x4*>(state);
    const int64_t bh = blockIdx.x / nsplit;
    const int p0 = static_cast<int>(blockIdx.x - bh * nsplit) * RPB;   // the block's first row
    const int64_t b = bh / H;
    const int h = static_cast<int>(bh - b * H);
    const int g = h / hpg;
    const int q = static_cast<int>(threadIdx.x) % OPR, rr = p0 + static_cast<int>(threadIdx.x) / OPR;
    const int64_t slot = slot_idx ? seq_slot(slot_idx, b, nslots) : b;
    const bool pad = slot < 0;
    // this thread's octets: rows rr + R k (< P); octet index in the state array or pool (-1: padding)
    const int64_t so0 = slot >= 0 ? slot * per_b + (static_cast<int64_t>(h) * P + rr) * OPR + q : -1;
    auto so_of = [&](int k) { return (so0 >= 0 && rr + R * k < P) ? so0 + static_cast<int64_t>(k) * R * OPR : -1; };
    // x, B and C first, then the state octets in order, all unconditional (rows past P and padding
    // requests read a valid row and drop it), so that the compiler's wait counts stay exact and the
    // first octet is computed while the later ones are still in flight
    float xv[K];
#pragma unroll
    for (int k = 0; k < K; ++k) {
        const int p = rr + R * k;
        const float v = static_cast<float>(x[b * xs + static_cast<int64_t>(h) * P + (p < P ? p : P - 1)]);
        xv[k] = p < P ? v : 0.f;
    }
    const float dtv = DTP ? dt_prologue(static_cast<float>(dt[bh]), dtp, h) : static_cast<float>(dt[bh]);
    const float a = __expf(dtv * A[h]);
    const float Dh = D ? D[h] : 0.f;
    const int64_t bo = b * bcs + static_cast<int64_t>(g) * N + 8 * q;
    float bv[8], cv[8];
    load8_f32(Bm + bo, bv);
    load8_f32(Cm + bo, cv);
    const int64_t sl0 = (pad ? 0 : slot) * per_b + static_cast<int64_t>(h) * P * OPR + q;   // row 0, octet q
    u32x4 raw[K];
#pragma unroll
    for (int k = 0; k < K; ++k) {
        const int p = rr + R * k;
        if constexpr (HAS_STATE) {
            raw[k] = __builtin_nontemporal_load(st + sl0 + static_cast<int64_t>(p < P ? p : P - 1) * OPR);
            if (pad) raw[k] = u32x4{0u, 0u, 0u, 0u};
        } else {
            raw[k] = u32x4{0u, 0u, 0u, 0u};
        }
    }
#pragma unroll
    for (int k = 0; k < K; ++k) {
        const int p = rr + R * k;
        if (p0 + R * k >= P) break;            // no row of this pass exists (uniform)
        const bool ok = p < P;
        const float dx = dtv * xv[k];
        float part = 0.f, v[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const uint32_t word = raw[k][e >> 1];
            v[e] = fmaf(a, F::dec((e & 1) ? word >> 16 : word & 0xFFFFu), dx * bv[e]);
            part = fmaf(v[e], cv[e], part);
        }
        if (!ok) part = 0.f;
        part = group_sum_last<OPR>(part);
        if (ok && q == OPR - 1) y[bh * P + p] = static_cast<TY>(part + (D ? Dh * xv[k] : 0.f));
        const int64_t so = so_of(k);
        if (so >= 0) {
            uint32_t rw[4];
            if constexpr (SR) {
                const uint64_t o = static_cast<uint64_t>(so);
                uint32_t c[4] = {static_cast<uint32_t>(o), static_cast<uint32_t>(o >> 32),
                                 static_cast<uint32_t>(offset), static_cast<uint32_t>(offset >> 32)};
                philox4x32(c, static_cast<uint32_t>(seed), static_cast<uint32_t>(seed >> 32), rounds);
                // the pair form for every value; the few outside its range (fp16 subnormals and values
                // near overflow, inf and NaN) are redone by the full form, in a branch only their lanes take
#pragma unroll
                for (int w = 0; w < 4; ++w) rw[w] = F::sr_pair(v[2 * w], v[2 * w + 1], c[w]);
            } else {
#pragma unroll
                for (int w = 0; w < 4; ++w) rw[w] = F::rne(v[2 * w]) | (F::rne(v[2 * w + 1]) << 16);
            }
            __builtin_nontemporal_store(u32x4{rw[0], rw[1], rw[2], rw[3]}, st + so);
        }
    }
}

template <typename T, typename TY, class F, int N>
static hipError_t lp_launch(const LpUpdateArgs& a, hipStream_t s) {
    const UpdateArgs& u = a.u;
    // a block takes kLpRows rows of a head (at least one pass); 32 rows at P = 64, N = 128 measured
    // faster than a whole head per block
    constexpr int R = kLpThreads / (N / 8);
    constexpr int RPB = kLpRows > R ? kLpRows : R;
    const int64_t blocks = u.batch * u.nheads * ((u.head_dim + RPB - 1) / RPB);
    if (blocks == 0) return hipSuccess;
    const bool dtp = u.dtp.bias || u.dtp.softplus || u.dtp.lo < u.dtp.hi;
    auto go = [&](auto kern) {
        hipLaunchKernelGGL(kern, dim3(static_cast<uint32_t>(blocks)), dim3(kLpThreads), 0, s,
                           static_cast<uint16_t*>(a.state), static_cast<const T*>(u.x), u.x_row_stride,
                           static_cast<const T*>(u.B), static_cast<const T*>(u.C), u.bc_row_stride,
                           static_cast<const T*>(u.dt), u.A, u.D, static_cast<TY*>(u.y), u.nheads, u.head_dim,
                           u.nheads / u.ngroups, u.slot_idx, u.nslots, u.dtp, a.seed, a.offset, a.rounds);
        return hipGetLastError();
    };
    if (!a.state)   // no pool (every request is padding): y from zero states, nothing stored
        return go(state_update_lp_kernel<T, TY, F, N, kLpRows, false, true, false>);
    if (a.rounds > 0)
        return dtp ? go(state_update_lp_kernel<T, TY, F, N, kLpRows, true, true, true>)
                   : go(state_update_lp_kernel<T, TY, F, N, kLpRows, true, false, true>);
    return dtp ? go(state_update_lp_kernel<T, TY, F, N, kLpRows, false, true, true>)
               : go(state_update_lp_kernel<T, TY, F, N, kLpRows, false, false, true>);
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
