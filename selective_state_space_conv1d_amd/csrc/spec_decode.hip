// Multi-token decode for speculative decoding ("Mamba 与 Nemotron 系列模型深度调研", 状态契约,
// MTP / speculative decoding): the k candidate tokens of a request advance its conv and SSM
// states one token at a time, every intermediate state is kept, and once the verifier has fixed
// how many tokens a request accepts, the state after the last accepted token is copied back into
// the request's state.  The request's own state is only read here until that copy.
//
// All three kernels are HBM streams with no reuse across threads:
//  * the SSM update reads each fp32 state element once and writes it k times (one intermediate
//    state per candidate), with the single-token update's arithmetic and y summation order, so
//    k = 1 reproduces it bitwise (a replay mode re-applies accepted tokens in place instead);
//  * the conv update keeps one 16-byte channel vector's 4-column window in registers across
//    the k tokens and writes the window after each;
//  * accept copies one intermediate state per request in 16-byte units.
#include "ssd_device.h"
#include "ssd_kernels.h"

#include <type_traits>

namespace ssd {

constexpr int kMultiThreads = 128;
// float4 of one state row per thread: 2 (with rows split one float4 per thread, 2 measured best at
// batch 64, k = 4, and 4 ran 30 % slower; 4 of one row would also leave rows of N = 16 one lane)
constexpr int kMultiPerThread = 2;
constexpr int kCopyThreads = 256;
constexpr int kCopyPerThread = 4;

// Four consecutive elements of T (8 bytes of bf16, 16 of fp32) in one load.
template <typename T> struct Quad;
template <> struct Quad<bf16> { typedef bf16x4 type; };
template <> struct Quad<float> { typedef f32x4 type; };

// Per thread and token: the raw inputs of its row (dt, x) and of its kMultiPerThread float4
// (B and C quads), kept in their storage type until used.
template <typename T>
struct TokIn {
    T dt, x;
    typename Quad<T>::type b[kMultiPerThread], c[kMultiPerThread];
};

// Grid: each thread takes kMultiPerThread (V) float4 of one state row: float4 q = l + LPR*v of the
// row, for lane l of the row's LPR = N/(4V) consecutive lanes, so the row's dt, x and decay are
// computed once per thread.  A block covers 128 V consecutive float4 (whole rows).
// Token j of request b is row b*k + j of x, B, C, dt and y, and entry b*k + j of inter.  The
// per-head constants are read once; each token's inputs are loaded one token ahead of their use.
// Each row's y dot product is a DPP reduction over its lanes, one token at a time (reducing 2 or
// 4 tokens together raised VGPRs to 100+ and ran 15-30 % slower): the V partial sums go through
// the same LPR-lane tree and are then added, which is the order of the single-token update's
// 2 LPR-lane tree, so k = 1 reproduces it bitwise.
// REPLAY (the accept step by recomputation): request b applies its first
// n = clamp(accept_len[b], 0, k) tokens and writes the state back in place; no y, no inter.
template <typename T, typename TY, int N, bool REPLAY>
__global__ __launch_bounds__(kMultiThreads) void state_update_multi_kernel(
    float* __restrict__ state, const T* __restrict__ x, int64_t xs, const T* __restrict__ Bm,
    const T* __restrict__ Cm, int64_t bcs, const T* __restrict__ dt, const float* __restrict__ A,
    const float* __restrict__ D, TY* __restrict__ y, float* __restrict__ inter, int64_t total4, int k, int H,
    int P, int hpg, const int32_t* __restrict__ slot_idx, int64_t nslots, DtParams dtp,
    const int32_t* __restrict__ accept_len) {
    constexpr int QPR = N / 4;                   // float4 per state row
    constexpr int V = kMultiPerThread;
    constexpr int LPR = QPR / V;                 // lanes per row
    constexpr int kSpan = kMultiThreads * V;     // float4 per block
    static_assert(QPR % V == 0 && LPR >= 2, "rows split over whole lanes");
    typedef typename Quad<T>::type Q;
    const int64_t per_b = static_cast<int64_t>(H) * P * QPR;
    const int lp = __builtin_ctz(static_cast<unsigned>(P));   // head_dim is a power of two
    f32x4* st4 = reinterpret_cast<f32x4*>(state);
    f32x4* in4 = reinterpret_cast<f32x4*>(inter);
    const int64_t f0 = static_cast<int64_t>(blockIdx.x) * kSpan;
    const int l = static_cast<int>(threadIdx.x) % LPR;
    const int64_t fr = f0 + (static_cast<int>(threadIdx.x) / LPR) * QPR;   // the thread's row, float4 0
    const bool live = fr < total4;                                          // total4 is whole rows
    auto tokens_of = [&](int64_t b) {   // tokens to apply: k, or the accepted count when replaying
        if constexpr (!REPLAY) return k;
        const int n = accept_len[b];
        return n < 0 ? 0 : (n > k ? k : n);
    };
    // The block's rows almost always lie in one request (UNI): its index, slot and token count are
    // then block constants, held in scalar registers, and every token's row addresses are scalar
    // too.  Otherwise each thread finds its request with a 64-bit division.
    const int64_t ub = f0 / per_b;
    const int64_t r0 = f0 - ub * per_b;
    const int64_t span = total4 - f0 < kSpan ? total4 - f0 : kSpan;
    auto body = [&](auto uni_tag) {
        constexpr bool UNI = decltype(uni_tag)::value;
        int64_t bb, rem, sl;   // request, offset of the thread's float4 0 in its state, slot
        int nk;                // tokens the thread applies
        if constexpr (UNI) {
            bb = ub;
            rem = live ? r0 + (fr - f0) + l : 0;
            sl = slot_idx ? seq_slot(slot_idx, ub, nslots) : ub;
            nk = tokens_of(ub);
            if (REPLAY && (nk == 0 || sl < 0)) return;   // nothing accepted, or padding
            if (!live) nk = 0;
        } else {
            const int64_t ff = live ? fr + l : 0;
            bb = ff / per_b;
            rem = ff - bb * per_b;
            sl = slot_idx ? seq_slot(slot_idx, bb, nslots) : bb;
            nk = live ? tokens_of(bb) : 0;
        }
        const int kmax = UNI ? tokens_of(ub) : k;
        const int rw = static_cast<int>(static_cast<uint64_t>(rem) / QPR);   // h * P + p
        const int h = rw >> lp;
        const int g = static_cast<int>(static_cast<unsigned>(h) / static_cast<unsigned>(hpg));
        const float Ah = A[h];
        const float Dh = D ? D[h] : 0.f;
        const float biash = dtp.bias ? dtp.bias[h] : 0.f;
        f32x4 s[V];
#pragma unroll
        for (int v = 0; v < V; ++v)
            s[v] = (live && sl >= 0 && nk > 0) ? __builtin_nontemporal_load(st4 + sl * per_b + rem + LPR * v)
                                               : f32x4{0.f, 0.f, 0.f, 0.f};
        // token row of the thread's request: a block constant when UNI (j < kmax there); rows past
        // a request's own count read its first
        auto tok_of = [&](int j) -> int64_t { return UNI ? ub * k + j : bb * k + (j < nk ? j : 0); };
        auto load_tok = [&](int j, TokIn<T>& in) {
            const int64_t tok = tok_of(j);
            in.dt = dt[tok * H + h];
            in.x = x[tok * xs + rw];
            const int64_t bo = tok * bcs + static_cast<int64_t>(g) * N + 4 * l;
#pragma unroll
            for (int v = 0; v < V; ++v) {
                in.b[v] = *reinterpret_cast<const Q*>(Bm + bo + 4 * LPR * v);
                in.c[v] = *reinterpret_cast<const Q*>(Cm + bo + 4 * LPR * v);
            }
        };
        // token j with its inputs: advance the state, store the intermediate state, reduce and store y
        auto step = [&](int j, const TokIn<T>& in) {
            // the dt prologue with the head's bias already loaded (same steps as dt_prologue)
            float dtv = static_cast<float>(in.dt);
            if (dtp.bias) dtv += biash;
            if (dtp.softplus) dtv = dtv > 20.f ? dtv : log1pf(expf(dtv));
            if (dtp.lo < dtp.hi) dtv = fminf(fmaxf(dtv, dtp.lo), dtp.hi);
            const float a = __expf(dtv * Ah);
            const float xv = static_cast<float>(in.x);
            const float dx = dtv * xv;
            const int64_t row = (UNI ? ub : bb) * k + j;
            float part[V];
#pragma unroll
            for (int v = 0; v < V; ++v) {
                f32x4 u = s[v];
                float pt = 0.f;
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    u[e] = fmaf(a, u[e], dx * static_cast<float>(in.b[v][e]));
                    pt = fmaf(u[e], static_cast<float>(in.c[v][e]), pt);
                }
                if (j < nk) s[v] = u;
                if constexpr (!REPLAY) {
                    if (inter && live) in4[row * per_b + rem + LPR * v] = u;   // plain stores measured faster here
                }
                part[v] = live ? pt : 0.f;
            }
            if constexpr (!REPLAY) {
                float sum = group_sum_last<LPR>(part[0]);
#pragma unroll
                for (int v = 1; v < V; ++v) sum = group_sum_last<LPR>(part[v]) + sum;
                if (live && l == LPR - 1)
                    y[row * H * static_cast<int64_t>(P) + rw] = static_cast<TY>(sum + (D ? Dh * xv : 0.f));
            }
        };
        // the inputs of token j + 1 are loaded while token j is computed, into the other of two
        // register sets (a copy between them would wait for the loads)
        TokIn<T> ta, tb;
        load_tok(0, ta);
        for (int j = 0; j < kmax; j += 2) {
            load_tok(j + 1 < kmax ? j + 1 : j, tb);   // past the last token: re-reads its rows
            step(j, ta);
            if (j + 1 >= kmax) break;
            load_tok(j + 2 < kmax ? j + 2 : j + 1, ta);
            step(j + 1, tb);
        }
        if constexpr (REPLAY) {
            if (live && sl >= 0 && nk > 0) {
#pragma unroll
                for (int v = 0; v < V; ++v) __builtin_nontemporal_store(s[v], st4 + sl * per_b + rem + LPR * v);
            }
        }
    };
    if (r0 + span <= per_b) body(std::true_type{});
    else body(std::false_type{});
}

template <typename T, typename TY, int N>
static hipError_t multi_launch(const UpdateArgs& a, hipStream_t s) {
    const int64_t total4 = a.batch * a.nheads * static_cast<int64_t>(a.head_dim) * (N / 4);
    if (total4 == 0 || a.k == 0) return hipSuccess;
    const int64_t per_block = kMultiThreads * kMultiPerThread;
    const int64_t blocks = (total4 + per_block - 1) / per_block;
    if (a.accept_len)
        hipLaunchKernelGGL((state_update_multi_kernel<T, TY, N, true>), dim3(static_cast<uint32_t>(blocks)),
                           dim3(kMultiThreads), 0, s, a.state, static_cast<const T*>(a.x), a.x_row_stride,
                           static_cast<const T*>(a.B), static_cast<const T*>(a.C), a.bc_row_stride,
                           static_cast<const T*>(a.dt), a.A, a.D, static_cast<TY*>(a.y), nullptr, total4, a.k,
                           a.nheads, a.head_dim, a.nheads / a.ngroups, a.slot_idx, a.nslots, a.dtp, a.accept_len);
    else
        hipLaunchKernelGGL((state_update_multi_kernel<T, TY, N, false>), dim3(static_cast<uint32_t>(blocks)),
                           dim3(kMultiThreads), 0, s, a.state, static_cast<const T*>(a.x), a.x_row_stride,
                           static_cast<const T*>(a.B), static_cast<const T*>(a.C), a.bc_row_stride,
                           static_cast<const T*>(a.dt), a.A, a.D, static_cast<TY*>(a.y), a.inter, total4, a.k,
                           a.nheads, a.head_dim, a.nheads / a.ngroups, a.slot_idx, a.nslots, a.dtp, nullptr);
    return hipGetLastError();
}

template <typename T, typename TY>
static hipError_t multi_t(const UpdateArgs& a, hipStream_t s) {
    switch (a.d_state) {
        case 16: return multi_launch<T, TY, 16>(a, s);
        case 32: return multi_launch<T, TY, 32>(a, s);
        case 64: return multi_launch<T, TY, 64>(a, s);
        case 128: return multi_launch<T, TY, 128>(a, s);
        default: return hipErrorInvalidValue;
    }
}

hipError_t launch_state_update_multi(const UpdateArgs& a, Dt act, Dt ydt, hipStream_t s) {
    if (act == Dt::BF16)
        return ydt == Dt::BF16 ? multi_t<bf16, bf16>(a, s) : multi_t<bf16, float>(a, s);
    return ydt == Dt::BF16 ? multi_t<float, bf16>(a, s) : multi_t<float, float>(a, s);
}

// One thread per (request, 16-byte channel vector).  The window of request b starts from its
// conv state (its pool slot with a slot table; zeros for padding) and rolls by one per token,
// with the single-token conv update's arithmetic.
template <typename T>
__global__ __launch_bounds__(kCopyThreads) void conv1d_update_multi_kernel(
    const T* __restrict__ xbc, int64_t xs, const T* __restrict__ w, const T* __restrict__ bias,
    const T* __restrict__ state, const int32_t* __restrict__ slot_idx, int64_t nslots, T* __restrict__ inter,
    T* __restrict__ out, int64_t CD, int64_t total, int k) {
    constexpr int V = Vec16<T>::n;
    const int64_t idx = static_cast<int64_t>(blockIdx.x) * kCopyThreads + threadIdx.x;
    if (idx >= total) return;
    const int64_t per_b = CD / V;
    const int64_t b = idx / per_b;
    const int64_t c0 = (idx - b * per_b) * V;

    float s[4 * V], wt[4 * V], bs[V];
    const int64_t slot = slot_idx ? seq_slot(slot_idx, b, nslots) : b;
    if (slot >= 0) {
#pragma unroll
        for (int q = 0; q < 4; ++q) load16_f32(state + (slot * CD + c0) * 4 + q * V, s + q * V);
    } else {
#pragma unroll
        for (int e = 0; e < 4 * V; ++e) s[e] = 0.f;
    }
#pragma unroll
    for (int q = 0; q < 4; ++q) load16_f32(w + c0 * 4 + q * V, wt + q * V);
    if (bias) load16_f32(bias + c0, bs);
    else
#pragma unroll
        for (int v = 0; v < V; ++v) bs[v] = 0.f;
    for (int j = 0; j < k; ++j) {
        const int64_t tok = b * k + j;
        float u[V], o[V];
        load16_f32(xbc + tok * xs + c0, u);
#pragma unroll
        for (int v = 0; v < V; ++v) {
            float* sv = s + v * 4;
            sv[0] = sv[1];
            sv[1] = sv[2];
            sv[2] = sv[3];
            sv[3] = u[v];
            float acc = bs[v];
#pragma unroll
            for (int e = 0; e < 4; ++e) acc = fmaf(wt[v * 4 + e], sv[e], acc);
            o[v] = silu_f(acc);
        }
        store16_f32(out + tok * CD + c0, o);
        if (inter) {
#pragma unroll
            for (int q = 0; q < 4; ++q) store16_f32(inter + (tok * CD + c0) * 4 + q * V, s + q * V);
        }
    }
}

template <typename T>
static hipError_t conv_multi_t(const ConvUpdateArgs& a, hipStream_t s) {
    constexpr int V = Vec16<T>::n;
    const int64_t total = a.batch * (a.channels / V);
    if (total == 0 || a.k == 0) return hipSuccess;
    const int64_t blocks = (total + kCopyThreads - 1) / kCopyThreads;
    hipLaunchKernelGGL(conv1d_update_multi_kernel<T>, dim3(static_cast<uint32_t>(blocks)), dim3(kCopyThreads), 0,
                       s, static_cast<const T*>(a.xbc), a.xbc_row_stride, static_cast<const T*>(a.w),
                       static_cast<const T*>(a.bias), static_cast<const T*>(a.state), a.slot_idx, a.nslots,
                       static_cast<T*>(a.inter), static_cast<T*>(a.out), a.channels, total, a.k);
    return hipGetLastError();
}

hipError_t launch_conv1d_update_multi(const ConvUpdateArgs& a, Dt act, hipStream_t s) {
    return act == Dt::BF16 ? conv_multi_t<bf16>(a, s) : conv_multi_t<float>(a, s);
}

// Accept by recomputation for the conv: request b's window after its first n candidate rows
// (n = accept_len clamped to [0, k]) is the last 4 of (old window, rows 0 .. n-1).  One thread
// per (request, 16-byte channel vector); nothing to do for n = 0 or padding.
template <typename T>
__global__ __launch_bounds__(kCopyThreads) void conv_accept_kernel(const T* __restrict__ xbc, int64_t xs,
                                                                   T* __restrict__ state,
                                                                   const int32_t* __restrict__ slot_idx, int64_t nslots,
                                                                   const int32_t* __restrict__ accept_len, int64_t CD,
                                                                   int64_t total, int k) {
    constexpr int V = Vec16<T>::n;
    const int64_t idx = static_cast<int64_t>(blockIdx.x) * kCopyThreads + threadIdx.x;
    if (idx >= total) return;
    const int64_t per_b = CD / V;
    const int64_t b = idx / per_b;
    const int64_t c0 = (idx - b * per_b) * V;
    int n = accept_len[b];
    n = n < 0 ? 0 : (n > k ? k : n);
    const int64_t slot = slot_idx ? seq_slot(slot_idx, b, nslots) : b;
    if (n == 0 || slot < 0) return;
    T* sp = state + (slot * CD + c0) * 4;
    float s[4 * V], o[4 * V];
#pragma unroll
    for (int q = 0; q < 4; ++q) load16_f32(sp + q * V, s + q * V);
#pragma unroll
    for (int col = 0; col < 4; ++col) {
        const int t = n - 4 + col;   // candidate row of window column col, or the old column 4 + t
        float u[V];
        if (t >= 0) load16_f32(xbc + (b * k + t) * xs + c0, u);
#pragma unroll
        for (int v = 0; v < V; ++v) o[v * 4 + col] = t >= 0 ? u[v] : s[v * 4 + 4 + t];
    }
#pragma unroll
    for (int q = 0; q < 4; ++q) store16_f32(sp + q * V, o + q * V);
}

template <typename T>
static hipError_t conv_accept_t(const ConvUpdateArgs& a, const int32_t* accept_len, hipStream_t s) {
    constexpr int V = Vec16<T>::n;
    const int64_t total = a.batch * (a.channels / V);
    if (total == 0 || a.k == 0) return hipSuccess;
    const int64_t blocks = (total + kCopyThreads - 1) / kCopyThreads;
    hipLaunchKernelGGL(conv_accept_kernel<T>, dim3(static_cast<uint32_t>(blocks)), dim3(kCopyThreads), 0, s,
                       static_cast<const T*>(a.xbc), a.xbc_row_stride, static_cast<T*>(a.state), a.slot_idx,
                       a.nslots, accept_len, a.channels, total, a.k);
    return hipGetLastError();
}

hipError_t launch_conv1d_update_accept(const ConvUpdateArgs& a, const int32_t* accept_len, Dt act, hipStream_t s) {
    return act == Dt::BF16 ? conv_accept_t<bf16>(a, accept_len, s) : conv_accept_t<float>(a, accept_len, s);
}

// Request blockIdx.y: with n = accept_len clamped to [0, k] and n >= 1, copy its intermediate
// state n-1 (units 16-byte vectors) into its slot.  Each thread moves kCopyPerThread vectors,
// all loads before the stores.
__global__ __launch_bounds__(kCopyThreads) void accept_copy_kernel(const int32_t* __restrict__ accept_len,
                                                                   const int32_t* __restrict__ slot_idx,
                                                                   int64_t nslots, int k, u32x4* __restrict__ dst,
                                                                   const u32x4* __restrict__ src, int64_t units) {
    const int64_t b = blockIdx.y;
    int n = accept_len[b];
    n = n < 0 ? 0 : (n > k ? k : n);
    const int64_t slot = slot_idx ? seq_slot(slot_idx, b, nslots) : b;
    if (n == 0 || slot < 0) return;
    const u32x4* from = src + (b * k + n - 1) * units;
    u32x4* to = dst + slot * units;
    const int64_t u0 = static_cast<int64_t>(blockIdx.x) * (kCopyThreads * kCopyPerThread) + threadIdx.x;
    u32x4 v[kCopyPerThread];
#pragma unroll
    for (int r = 0; r < kCopyPerThread; ++r) {
        const int64_t u = u0 + r * kCopyThreads;
        if (u < units) v[r] = __builtin_nontemporal_load(from + u);
    }
#pragma unroll
    for (int r = 0; r < kCopyPerThread; ++r) {
        const int64_t u = u0 + r * kCopyThreads;
        if (u < units) __builtin_nontemporal_store(v[r], to + u);
    }
}

static hipError_t accept_copy(const AcceptArgs& a, void* dst, const void* src, int64_t bytes, hipStream_t s) {
    const int64_t units = bytes / 16;
    if (!dst || units == 0 || a.batch == 0 || a.k == 0) return hipSuccess;
    const int64_t per_block = kCopyThreads * kCopyPerThread;
    dim3 grid(static_cast<uint32_t>((units + per_block - 1) / per_block), static_cast<uint32_t>(a.batch));
    hipLaunchKernelGGL(accept_copy_kernel, grid, dim3(kCopyThreads), 0, s, a.accept_len, a.slot_idx, a.nslots, a.k,
                       static_cast<u32x4*>(dst), static_cast<const u32x4*>(src), units);
    return hipGetLastError();
}

hipError_t launch_accept_states(const AcceptArgs& a, hipStream_t s) {
    hipError_t e = accept_copy(a, a.state, a.inter, a.state_bytes, s);
    if (e != hipSuccess) return e;
    return accept_copy(a, a.conv_state, a.inter_conv, a.conv_bytes, s);
}

}  // namespace ssd
