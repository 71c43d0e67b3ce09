// Gated group RMSNorm of the mixer output ("MAX 平台 Nemotron-H 混合架构解析", 5.4, item 4: one
// fused kernel, gate applied before the norm, fp32 arithmetic and an fp32 weight):
//   v = y * silu(z);  out = v / sqrt(mean over the group of v^2 + eps) * weight.
// One workgroup per (row, group).  Each thread takes 8-channel vectors of the group (16-byte loads
// of bf16); the first pass forms v and sums v^2 (wave reduction, then across the waves in LDS),
// the second scales v, held in registers (or, for groups of more than 4096 channels, recomputed
// from y and z, which the first pass left in the cache), and writes the result.  The kernel reads
// y and z and writes the output once: an HBM stream.
#include "ssd_device.h"
#include "ssd_kernels.h"

namespace ssd {

constexpr int kNormThreads = 256;
constexpr int kNormHold = 2;   // 8-channel vectors per thread held in registers between the two passes

template <typename T>
__device__ __forceinline__ void load8(const T* p, float (&o)[8]) {
    load16_f32(p, o);
    if constexpr (Vec16<T>::n == 4) load16_f32(p + 4, o + 4);
}
// y and z rows held in registers between the passes are read once, and the output is written once:
// non-temporal (143 -> 139 us on 8192 x 16384, and the launch before it runs faster too)
template <typename T>
__device__ __forceinline__ void load8_nt(const T* p, float (&o)[8]) {
    load16_f32_nt(p, o);
    if constexpr (Vec16<T>::n == 4) load16_f32_nt(p + 4, o + 4);
}
template <typename T>
__device__ __forceinline__ void store8(T* p, const float (&o)[8]) {
    store16_f32_nt(p, o);
    if constexpr (Vec16<T>::n == 4) store16_f32_nt(p + 4, o + 4);
}

template <typename TY, typename T>
__global__ __launch_bounds__(kNormThreads) void gated_rmsnorm_kernel(const TY* __restrict__ y, int64_t ys,
                                                                     const T* __restrict__ z, int64_t zs,
                                                                     const float* __restrict__ w, float eps,
                                                                     T* __restrict__ out, int64_t I, int gs,
                                                                     int ngroups) {
    __shared__ float part[kNormThreads / 64];
    const int64_t row = blockIdx.x / ngroups;
    const int g = static_cast<int>(blockIdx.x % ngroups);
    const int64_t c0 = static_cast<int64_t>(g) * gs;
    const TY* yr = y + row * ys + c0;
    const T* zr = z + row * zs + c0;
    constexpr int kSpan = 8 * kNormThreads;   // channels per pass of the workgroup
    // the first kNormHold vectors of each thread keep v = y * silu(z) in registers for the second
    // pass (groups up to 8 * 256 * kNormHold channels); later ones are re-read there
    float vh[kNormHold][8];
    float ss = 0.f;
#pragma unroll
    for (int k = 0; k < kNormHold; ++k) {
        const int c = 8 * threadIdx.x + k * kSpan;
        if (c < gs) {
            float yv[8], zv[8];
            load8_nt(yr + c, yv);
            load8_nt(zr + c, zv);
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                vh[k][e] = yv[e] * silu_f(zv[e]);
                ss = fmaf(vh[k][e], vh[k][e], ss);
            }
        }
    }
    for (int c = 8 * threadIdx.x + kNormHold * kSpan; c < gs; c += kSpan) {
        float yv[8], zv[8];
        load8(yr + c, yv);
        load8(zr + c, zv);
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const float v = yv[e] * silu_f(zv[e]);
            ss = fmaf(v, v, ss);
        }
    }
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) ss += __shfl_xor(ss, off, 64);
    if ((threadIdx.x & 63) == 0) part[threadIdx.x >> 6] = ss;
    __syncthreads();
    float tot = 0.f;
#pragma unroll
    for (int k = 0; k < kNormThreads / 64; ++k) tot += part[k];
    const float r = rsqrtf(tot / static_cast<float>(gs) + eps);
    T* orow = out + row * I + c0;
#pragma unroll
    for (int k = 0; k < kNormHold; ++k) {
        const int c = 8 * threadIdx.x + k * kSpan;
        if (c < gs) {
            float wv[8], o[8];
            load8(w + c0 + c, wv);
#pragma unroll
            for (int e = 0; e < 8; ++e) o[e] = vh[k][e] * r * wv[e];
            store8(orow + c, o);
        }
    }
    for (int c = 8 * threadIdx.x + kNormHold * kSpan; c < gs; c += kSpan) {
        float yv[8], zv[8], wv[8], o[8];
        load8(yr + c, yv);
        load8(zr + c, zv);
        load8(w + c0 + c, wv);
#pragma unroll
        for (int e = 0; e < 8; ++e) o[e] = yv[e] * silu_f(zv[e]) * r * wv[e];
        store8(orow + c, o);
    }
}

template <typename TY, typename T>
static hipError_t norm_t(const NormArgs& a, hipStream_t s) {
    const int64_t blocks = a.rows * a.ngroups;
    if (blocks == 0) return hipSuccess;
    hipLaunchKernelGGL((gated_rmsnorm_kernel<TY, T>), dim3(static_cast<uint32_t>(blocks)), dim3(kNormThreads), 0, s,
                       static_cast<const TY*>(a.y), a.y_row_stride, static_cast<const T*>(a.z), a.z_row_stride,
                       a.weight, a.eps, static_cast<T*>(a.out), a.channels, static_cast<int>(a.channels / a.ngroups),
                       a.ngroups);
    return hipGetLastError();
}

hipError_t launch_gated_rmsnorm(const NormArgs& a, Dt act, Dt ydt, hipStream_t s) {
    if (act == Dt::BF16) return ydt == Dt::BF16 ? norm_t<bf16, bf16>(a, s) : norm_t<float, bf16>(a, s);
    return ydt == Dt::BF16 ? norm_t<bf16, float>(a, s) : norm_t<float, float>(a, s);
}

}  // namespace ssd
