// Small device helpers shared by the HIP kernels of this library.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "ssd_kernels.h"

namespace ssd {

typedef __bf16 bf16;
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

// 16-byte vector of T: 8 bf16 or 4 fp32.
template <typename T> struct Vec16;
template <> struct Vec16<bf16> {
    static constexpr int n = 8;
    typedef bf16x8 type;
};
template <> struct Vec16<float> {
    static constexpr int n = 4;
    typedef f32x4 type;
};

template <typename T>
__device__ __forceinline__ void load16_f32(const T* p, float* out) {
    typedef typename Vec16<T>::type V;
    V v = *reinterpret_cast<const V*>(p);
#pragma unroll
    for (int i = 0; i < Vec16<T>::n; ++i) out[i] = static_cast<float>(v[i]);
}

template <typename T>
__device__ __forceinline__ void store16_f32(T* p, const float* in) {
    typedef typename Vec16<T>::type V;
    V v;
#pragma unroll
    for (int i = 0; i < Vec16<T>::n; ++i) v[i] = static_cast<T>(in[i]);  // RNE for bf16
    *reinterpret_cast<V*>(p) = v;
}

// Non-temporal forms, for data a kernel reads or writes once and no kernel re-reads while it is
// cached.  Streamed this way, such data does not fill the caches with lines -- dirty ones above all --
// whose later eviction the next kernel pays for.  Measured on the prefill chain conv -> scan -> gated
// norm (1 x 8192 tokens, 256 heads): about 490 -> 450 us with the conv's input rows, the scan's y
// stores and the norm's loads and stores streamed.
template <typename T>
__device__ __forceinline__ void load16_f32_nt(const T* p, float* out) {
    typedef typename Vec16<T>::type V;
    V v = __builtin_nontemporal_load(reinterpret_cast<const V*>(p));
#pragma unroll
    for (int i = 0; i < Vec16<T>::n; ++i) out[i] = static_cast<float>(v[i]);
}

template <typename T>
__device__ __forceinline__ void store16_f32_nt(T* p, const float* in) {
    typedef typename Vec16<T>::type V;
    V v;
#pragma unroll
    for (int i = 0; i < Vec16<T>::n; ++i) v[i] = static_cast<T>(in[i]);  // RNE for bf16
    __builtin_nontemporal_store(v, reinterpret_cast<V*>(p));
}

// SiLU z * sigmoid(z) with the hardware reciprocal (about 1 ulp): outputs are stored in the
// activation dtype, and the division's exact rounding costs a dozen instructions per element.
__device__ __forceinline__ float silu_f(float z) { return z * __builtin_amdgcn_rcpf(1.0f + __expf(-z)); }

// Sum of v over each aligned group of G consecutive lanes (G = 2, 4, 8, 16 or 32), valid in the
// group's last lane.  DPP lane moves (VALU, a few cycles each) instead of LDS shuffles: quad
// permutes for 2 and 4 lanes, the half-row and row mirrors for 8 and 16, and the row-15 broadcast
// into rows 1 and 3 for 32 (the last lane of each 32-group is in those rows).  Lane semantics were
// checked on the device for every G.
template <int CTRL, int RMASK>
__device__ __forceinline__ float dpp_f(float x) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, RMASK, 0xF, false));
}
template <int G>
__device__ __forceinline__ float group_sum_last(float v) {
    static_assert(G == 2 || G == 4 || G == 8 || G == 16 || G == 32, "group of 2..32 lanes");
    if constexpr (G >= 2) v += dpp_f<0xB1, 0xF>(v);    // quad_perm [1,0,3,2]
    if constexpr (G >= 4) v += dpp_f<0x4E, 0xF>(v);    // quad_perm [2,3,0,1]
    if constexpr (G >= 8) v += dpp_f<0x141, 0xF>(v);   // row_half_mirror
    if constexpr (G >= 16) v += dpp_f<0x140, 0xF>(v);  // row_mirror
    if constexpr (G >= 32) v += dpp_f<0x142, 0xA>(v);  // row_bcast:15 into rows 1 and 3
    return v;
}

// dt prologue of head h (fp32): + bias, softplus (the identity above 20, where log(1 + e^v)
// rounds to v), clamp.  With every step off it returns v unchanged.
template <class DP>
__device__ __forceinline__ float dt_prologue(float v, const DP& p, int h) {
    if (p.bias) v += p.bias[h];
    if (p.softplus) v = v > 20.f ? v : log1pf(expf(v));
    if (p.lo < p.hi) v = fminf(fmaxf(v, p.lo), p.hi);
    return v;
}

// Token rows [start, start + len) of packed sequence s, with the table's values clamped into
// [0, total] so that a malformed table cannot address outside the packed tensors.
__device__ __forceinline__ void seq_span(const int32_t* cu, int64_t s, int64_t total, int64_t& start,
                                         int64_t& len) {
    int64_t a = cu[s], b = cu[s + 1];
    a = a < 0 ? 0 : (a > total ? total : a);
    b = b < a ? a : (b > total ? total : b);
    start = a;
    len = b - a;
}

// State slot of batch entry / sequence s, or -1 (padding: no state read or written) when the
// table says so (negative) or names a slot outside the pool.
__device__ __forceinline__ int64_t seq_slot(const int32_t* slot_idx, int64_t s, int64_t nslots) {
    const int64_t v = slot_idx ? static_cast<int64_t>(slot_idx[s]) : s;
    return (v >= 0 && v < nslots) ? v : -1;
}

// Where the scan stores the snapshot of head h's state after token t_end of sequence (or batch
// entry) s of length L, or NULL: t_end must close an interval.  Batched calls fill
// [B, L / interval, H, P, N]; packed ones the pool slot their table names for (s, interval k).
__device__ __forceinline__ float* snapshot_dst(const ScanArgs& a, int64_t s, int64_t L, int64_t t_end, int h) {
    if (!a.snapshots || t_end % a.snap_interval != 0 || t_end > L) return nullptr;
    const int64_t k = t_end / a.snap_interval - 1;
    const int64_t pn = static_cast<int64_t>(a.head_dim) * a.d_state;
    if (a.snap_table) {
        if (k >= a.snap_max) return nullptr;
        const int64_t sl = a.snap_table[s * a.snap_max + k];
        return (sl >= 0 && sl < a.snap_slots) ? a.snapshots + (sl * a.nheads + h) * pn : nullptr;
    }
    return a.snapshots + ((s * (L / a.snap_interval) + k) * a.nheads + h) * pn;
}

}  // namespace ssd
