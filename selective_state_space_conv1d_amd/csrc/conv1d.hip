// Causal depthwise conv1d (width 4) + SiLU over the packed x|B|C channels.
//
// Prefill: the conv over a whole sequence, channels last ([B, L, CD]), taking
// its first three taps' inputs from the conv state ("MAX 平台 Nemotron-H 混合
// 架构解析", 5.4: channels-last conv, no transposes around it; the
// modeling_nemotron_h.py walk-through, "Prefill 阶段": the last 4 conv inputs
// become the new conv state).
// Decode: one token per sequence; the window rolls by one and the new input
// takes the last slot ("Decode 阶段" of the same walk-through).
//
// Both are HBM-streaming kernels with no reuse beyond the 3-token halo: each
// thread owns one 16-byte vector of channels (8 bf16 / 4 fp32) and walks a run
// of tokens keeping the sliding window in registers, so every row is read once
// with fully coalesced 16-byte accesses and written once.
#include "ssd_device.h"
#include "ssd_kernels.h"

namespace ssd {

constexpr int kConvThreads = 256;
constexpr int kConvTokens = 32;  // tokens per thread in the prefill conv

// Grid: x = channel blocks * token tiles (channel block fastest), y = batch.
// The thread of token tile 0 reads the incoming state before it writes the
// outgoing one, so conv_state_out may alias conv_state_in.
template <typename T>
__global__ __launch_bounds__(kConvThreads) void conv1d_fwd_kernel(
    const T* __restrict__ xbc, int64_t xs, const T* __restrict__ w, const T* __restrict__ bias,
    const T* s_in, T* s_out, T* __restrict__ out, int64_t L, int64_t CD, int64_t cblocks) {
    constexpr int V = Vec16<T>::n;
    const int64_t cb = blockIdx.x % cblocks;
    const int64_t tile = blockIdx.x / cblocks;
    const int64_t c0 = (cb * kConvThreads + threadIdx.x) * V;
    if (c0 >= CD) return;
    const int64_t b = blockIdx.y;
    const int64_t t0 = tile * kConvTokens;
    const int64_t t1 = (t0 + kConvTokens < L) ? t0 + kConvTokens : L;

    float wt[4][V];  // wt[k][v] = w[c0+v, k]
    if (t0 < t1) {   // L == 0 only carries the state through and never reads the taps
        float tmp[4 * V];
#pragma unroll
        for (int q = 0; q < 4; ++q) load16_f32(w + c0 * 4 + q * V, tmp + q * V);
#pragma unroll
        for (int v = 0; v < V; ++v)
#pragma unroll
            for (int k = 0; k < 4; ++k) wt[k][v] = tmp[v * 4 + k];
    }
    float bs[V];
    if (bias && t0 < t1) load16_f32(bias + c0, bs);
    else
#pragma unroll
        for (int v = 0; v < V; ++v) bs[v] = 0.f;

    const T* xb = xbc + b * L * xs;
    float win[3][V];   // inputs at t-3, t-2, t-1
    float st[4][V];    // incoming state (token tile 0 only)
    if (tile == 0) {
        if (s_in) {
            float tmp[4 * V];
#pragma unroll
            for (int q = 0; q < 4; ++q) load16_f32(s_in + (b * CD + c0) * 4 + q * V, tmp + q * V);
#pragma unroll
            for (int v = 0; v < V; ++v)
#pragma unroll
                for (int k = 0; k < 4; ++k) st[k][v] = tmp[v * 4 + k];
        } else {
#pragma unroll
            for (int k = 0; k < 4; ++k)
#pragma unroll
                for (int v = 0; v < V; ++v) st[k][v] = 0.f;
        }
#pragma unroll
        for (int k = 0; k < 3; ++k)
#pragma unroll
            for (int v = 0; v < V; ++v) win[k][v] = st[k + 1][v];
    } else {
#pragma unroll
        for (int k = 0; k < 3; ++k) load16_f32(xb + (t0 - 3 + k) * xs + c0, win[k]);
    }

    T* ob = out + b * L * CD;
    for (int64_t t = t0; t < t1; ++t) {
        float u[V], o[V];
        load16_f32(xb + t * xs + c0, u);
#pragma unroll
        for (int v = 0; v < V; ++v) {
            float acc = bs[v];
            acc = fmaf(wt[0][v], win[0][v], acc);
            acc = fmaf(wt[1][v], win[1][v], acc);
            acc = fmaf(wt[2][v], win[2][v], acc);
            acc = fmaf(wt[3][v], u[v], acc);
            o[v] = silu_f(acc);
            win[0][v] = win[1][v];
            win[1][v] = win[2][v];
            win[2][v] = u[v];
        }
        store16_f32(ob + t * CD + c0, o);
    }

    if (tile == 0 && s_out) {
        // new state column k = input at token L-4+k (from the old state when negative)
        float ns[4][V];
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            const int64_t tau = L - 4 + k;
            if (tau >= 0) {
                load16_f32(xb + tau * xs + c0, ns[k]);
            } else {
                const int j = 4 + static_cast<int>(tau);  // 0..3
#pragma unroll
                for (int v = 0; v < V; ++v) {
                    float s = st[0][v];
                    if (j == 1) s = st[1][v];
                    if (j == 2) s = st[2][v];
                    if (j == 3) s = st[3][v];
                    ns[k][v] = s;
                }
            }
        }
        float tmp[4 * V];
#pragma unroll
        for (int v = 0; v < V; ++v)
#pragma unroll
            for (int k = 0; k < 4; ++k) tmp[v * 4 + k] = ns[k][v];
#pragma unroll
        for (int q = 0; q < 4; ++q) store16_f32(s_out + (b * CD + c0) * 4 + q * V, tmp + q * V);
    }
}

// One thread per (batch, 16-byte channel vector).
template <typename T>
__global__ __launch_bounds__(kConvThreads) void conv1d_update_kernel(
    const T* __restrict__ xbc, int64_t xs, const T* __restrict__ w, const T* __restrict__ bias,
    T* __restrict__ state, T* __restrict__ out, int64_t CD, int64_t total) {
    constexpr int V = Vec16<T>::n;
    const int64_t idx = static_cast<int64_t>(blockIdx.x) * kConvThreads + threadIdx.x;
    if (idx >= total) return;
    const int64_t per_b = CD / V;
    const int64_t b = idx / per_b;
    const int64_t c0 = (idx - b * per_b) * V;

    float s[4 * V], wt[4 * V], u[V], bs[V], o[V];
    T* sp = state + (b * CD + c0) * 4;
#pragma unroll
    for (int q = 0; q < 4; ++q) load16_f32(sp + q * V, s + q * V);
#pragma unroll
    for (int q = 0; q < 4; ++q) load16_f32(w + c0 * 4 + q * V, wt + q * V);
    load16_f32(xbc + b * xs + c0, u);
    if (bias) load16_f32(bias + c0, bs);
    else
#pragma unroll
        for (int v = 0; v < V; ++v) bs[v] = 0.f;
#pragma unroll
    for (int v = 0; v < V; ++v) {
        float* sv = s + v * 4;
        sv[0] = sv[1];
        sv[1] = sv[2];
        sv[2] = sv[3];
        sv[3] = u[v];
        float acc = bs[v];
#pragma unroll
        for (int k = 0; k < 4; ++k) acc = fmaf(wt[v * 4 + k], sv[k], acc);
        o[v] = silu_f(acc);
    }
#pragma unroll
    for (int q = 0; q < 4; ++q) store16_f32(sp + q * V, s + q * V);
    store16_f32(out + b * CD + c0, o);
}

template <typename T>
static hipError_t conv_fwd_t(const ConvFwdArgs& a, hipStream_t s) {
    constexpr int V = Vec16<T>::n;
    const int64_t cblocks = (a.channels / V + kConvThreads - 1) / kConvThreads;
    const int64_t tiles = a.seqlen > 0 ? (a.seqlen + kConvTokens - 1) / kConvTokens : 1;
    if (a.batch == 0 || a.channels == 0) return hipSuccess;
    if (a.seqlen == 0 && a.state_out == nullptr) return hipSuccess;
    dim3 grid(static_cast<uint32_t>(cblocks * tiles), static_cast<uint32_t>(a.batch));
    hipLaunchKernelGGL(conv1d_fwd_kernel<T>, grid, dim3(kConvThreads), 0, s,
                       static_cast<const T*>(a.xbc), a.xbc_row_stride, static_cast<const T*>(a.w),
                       static_cast<const T*>(a.bias), static_cast<const T*>(a.state_in),
                       static_cast<T*>(a.state_out), static_cast<T*>(a.out), a.seqlen, a.channels,
                       cblocks);
    return hipGetLastError();
}

template <typename T>
static hipError_t conv_update_t(const ConvUpdateArgs& a, hipStream_t s) {
    constexpr int V = Vec16<T>::n;
    const int64_t total = a.batch * (a.channels / V);
    if (total == 0) return hipSuccess;
    const int64_t blocks = (total + kConvThreads - 1) / kConvThreads;
    hipLaunchKernelGGL(conv1d_update_kernel<T>, dim3(static_cast<uint32_t>(blocks)), dim3(kConvThreads),
                       0, s, static_cast<const T*>(a.xbc), a.xbc_row_stride, static_cast<const T*>(a.w),
                       static_cast<const T*>(a.bias), static_cast<T*>(a.state), static_cast<T*>(a.out),
                       a.channels, total);
    return hipGetLastError();
}

hipError_t launch_conv1d_fwd(const ConvFwdArgs& a, Dt act, hipStream_t s) {
    return act == Dt::BF16 ? conv_fwd_t<bf16>(a, s) : conv_fwd_t<float>(a, s);
}

hipError_t launch_conv1d_update(const ConvUpdateArgs& a, Dt act, hipStream_t s) {
    return act == Dt::BF16 ? conv_update_t<bf16>(a, s) : conv_update_t<float>(a, s);
}

}  // namespace ssd
