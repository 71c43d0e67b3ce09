// Single-token selective state update for decode, in place on the fp32 state
// (modeling_nemotron_h.py walk-through, "Decode 阶段": the state decays by
// exp(dt*A), gains dt*B*x, and y contracts the updated state with C and adds
// D*x; "Mamba 与 Nemotron 系列模型深度调研", 状态契约: state [B, H, P, N]).
//
// The state is read once and written once per token, so the kernel is a pure
// HBM stream.  The whole [B, H, P, N] state is walked as one flat array of
// float4: each thread keeps 4 float4 in flight (one per 128-thread stride, so
// every wave-wide access is 1 KB contiguous), with non-temporal loads and
// stores because the state is far larger than the caches and is not re-read
// this step.  (Measured on MI355X at batch 64: 4 x 128 threads reaches ~98% of
// an in-place read+write of the same buffer; 8 or 16 in flight per thread, or
// cached accesses, are slower.)  One state row p (N floats) spans N/4 consecutive lanes; the
// output y[p] is a DPP reduction over those lanes.  No MFMA: the
// arithmetic is 2 FMAs per 4-byte element.
#include "ssd_device.h"
#include "ssd_kernels.h"

#include <type_traits>

namespace ssd {

constexpr int kUpdThreads = 128;
constexpr int kUpdPerThread = 4;

// SLOTS: batch entry b's state is slot slot_idx[b] of a pool (none for padding: it starts from
// zeros and is not stored); the walk is still over [B, H, P, N], so each wave-wide access stays
// 1 KB contiguous inside one slot.
// DTP: apply the dt prologue.  Without it the kernel has no uniform branches inside the unrolled
// element loop (with them the loads of the 4 elements were no longer issued together: 7 % slower).
template <typename T, typename TY, int N, bool SLOTS, bool DTP>
__global__ __launch_bounds__(kUpdThreads) void state_update_kernel(
    float* __restrict__ state, const T* __restrict__ x, int64_t xs, const T* __restrict__ Bm,
    const T* __restrict__ Cm, int64_t bcs, const T* __restrict__ dt, const float* __restrict__ A,
    const float* __restrict__ D, TY* __restrict__ y, int64_t total4, int H, int P, int hpg,
    const int32_t* __restrict__ slot_idx, int64_t nslots, DtParams dtp) {
    constexpr int QPR = N / 4;  // float4 per state row
    constexpr int kSpan = kUpdThreads * kUpdPerThread;
    f32x4* st4 = reinterpret_cast<f32x4*>(state);
    const int64_t per_b = static_cast<int64_t>(H) * P * QPR;
    const int lp = __builtin_ctz(static_cast<unsigned>(P));   // head_dim is a power of two
    const int64_t f0 = static_cast<int64_t>(blockIdx.x) * kSpan;
    const int64_t base = f0 + threadIdx.x;
    // The block's elements almost always lie in one batch entry (UNI): its index (and slot) are
    // then block constants, and each element's row, head and q come from shifts of its offset in
    // the entry; otherwise each element divides its flat index.
    const int64_t ub = f0 / per_b;
    const int64_t r0 = f0 - ub * per_b;
    const int64_t span = total4 - f0 < kSpan ? total4 - f0 : kSpan;
    auto body = [&](auto uni_tag) {
        constexpr bool UNI = decltype(uni_tag)::value;
        int64_t ushift = 0;   // with SLOTS and UNI: the entry's offset from its slot in the pool
        bool upad = false;    // that entry is padding
        if constexpr (SLOTS && UNI) {
            const int64_t slot = seq_slot(slot_idx, ub, nslots);
            upad = slot < 0;
            ushift = (slot - ub) * per_b;
        }
        f32x4 s[kUpdPerThread];
        int64_t sf[kUpdPerThread];   // float4 index of the state (in the pool with SLOTS), -1: padding
#pragma unroll
        for (int i = 0; i < kUpdPerThread; ++i) {
            const int64_t f = base + i * kUpdThreads;
            sf[i] = f;
            if constexpr (SLOTS) {
                if (UNI) {
                    sf[i] = upad ? -1 : f + ushift;
                } else if (f < total4) {
                    const int64_t b = f / per_b;
                    const int64_t slot = seq_slot(slot_idx, b, nslots);
                    sf[i] = slot < 0 ? -1 : f + (slot - b) * per_b;
                }
            }
            if constexpr (SLOTS) {
                if (f < total4) s[i] = sf[i] >= 0 ? __builtin_nontemporal_load(st4 + sf[i]) : f32x4{0.f, 0.f, 0.f, 0.f};
            } else {
                if (f < total4) s[i] = __builtin_nontemporal_load(st4 + f);
            }
        }
#pragma unroll
        for (int i = 0; i < kUpdPerThread; ++i) {
            const int64_t f = base + i * kUpdThreads;
            const bool ok = f < total4;
            int64_t b, row, bh;   // batch entry, state row (b, h, p), (b, h)
            int q, h, p;
            if constexpr (UNI) {
                const int rem = ok ? static_cast<int>(r0) + static_cast<int>(threadIdx.x) + i * kUpdThreads : 0;
                const int rw = rem / QPR;   // h * P + p
                q = rem % QPR;
                h = rw >> lp;
                p = rw & (P - 1);
                b = ub;
                row = ub * H * P + rw;
                bh = ub * H + h;
            } else {
                const int64_t ff = ok ? f : 0;
                row = ff / QPR;
                q = static_cast<int>(ff - row * QPR);
                bh = row >> lp;
                p = static_cast<int>(row & (P - 1));
                b = bh / H;
                h = static_cast<int>(bh - b * H);
            }
            const int g = h / hpg;
            const float dtv = DTP ? dt_prologue(static_cast<float>(dt[bh]), dtp, h) : static_cast<float>(dt[bh]);
            const float a = __expf(dtv * A[h]);
            const float xv = static_cast<float>(x[b * xs + static_cast<int64_t>(h) * P + p]);
            const int64_t bo = b * bcs + static_cast<int64_t>(g) * N + 4 * q;
            float bv[4], cv[4];
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                bv[k] = static_cast<float>(Bm[bo + k]);
                cv[k] = static_cast<float>(Cm[bo + k]);
            }
            const float dx = dtv * xv;
            f32x4 v = s[i];
            float part = 0.f;
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                v[k] = fmaf(a, v[k], dx * bv[k]);
                part = fmaf(v[k], cv[k], part);
            }
            if (!ok) part = 0.f;
            part = group_sum_last<QPR>(part);   // the row's QPR lanes are consecutive and aligned
            if (ok) {
                if (q == QPR - 1) y[row] = static_cast<TY>(part + (D ? D[h] * xv : 0.f));
                if (!SLOTS || sf[i] >= 0) __builtin_nontemporal_store(v, st4 + sf[i]);
            }
        }
    };
    if (r0 + span <= per_b && per_b < (1LL << 30)) body(std::true_type{});   // offsets fit 32 bits
    else body(std::false_type{});
}

template <typename T, typename TY, int N, bool SLOTS, bool DTP>
static hipError_t upd_launch(const UpdateArgs& a, hipStream_t s) {
    const int64_t total4 = a.batch * a.nheads * static_cast<int64_t>(a.head_dim) * (N / 4);
    if (total4 == 0) return hipSuccess;
    const int64_t per_block = kUpdThreads * kUpdPerThread;
    const int64_t blocks = (total4 + per_block - 1) / per_block;
    hipLaunchKernelGGL((state_update_kernel<T, TY, N, SLOTS, DTP>), dim3(static_cast<uint32_t>(blocks)),
                       dim3(kUpdThreads), 0, s, a.state, static_cast<const T*>(a.x), a.x_row_stride,
                       static_cast<const T*>(a.B), static_cast<const T*>(a.C), a.bc_row_stride,
                       static_cast<const T*>(a.dt), a.A, a.D, static_cast<TY*>(a.y), total4, a.nheads,
                       a.head_dim, a.nheads / a.ngroups, a.slot_idx, a.nslots, a.dtp);
    return hipGetLastError();
}

template <typename T, typename TY, int N>
static hipError_t upd_n(const UpdateArgs& a, hipStream_t s) {
    const bool dtp = a.dtp.bias || a.dtp.softplus || a.dtp.lo < a.dtp.hi;
    if (a.slot_idx) return dtp ? upd_launch<T, TY, N, true, true>(a, s) : upd_launch<T, TY, N, true, false>(a, s);
    return dtp ? upd_launch<T, TY, N, false, true>(a, s) : upd_launch<T, TY, N, false, false>(a, s);
}

template <typename T, typename TY>
static hipError_t upd_t(const UpdateArgs& a, hipStream_t s) {
    switch (a.d_state) {
        case 16: return upd_n<T, TY, 16>(a, s);
        case 32: return upd_n<T, TY, 32>(a, s);
        case 64: return upd_n<T, TY, 64>(a, s);
        case 128: return upd_n<T, TY, 128>(a, s);
        default: return hipErrorInvalidValue;
    }
}

hipError_t launch_state_update(const UpdateArgs& a, Dt act, Dt ydt, hipStream_t s) {
    if (act == Dt::BF16)
        return ydt == Dt::BF16 ? upd_t<bf16, bf16>(a, s) : upd_t<bf16, float>(a, s);
    return ydt == Dt::BF16 ? upd_t<float, bf16>(a, s) : upd_t<float, float>(a, s);
}

}  // namespace ssd
