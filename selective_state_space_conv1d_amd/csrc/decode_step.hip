// One decode step of the mixer in one launch: the one-token conv over x|B|C and the selective
// state update ("modeling_nemotron_h.py" walk-through, "Decode 阶段": roll the conv window by one,
// convolve, then update the state in place and read y; fusing the step is one of the next steps
// the kernels are planned for).
//
// Each block updates rows [p0, p0 + RP) of one (batch entry b, head h) of the fp32 state -- the
// whole head when it fits -- as the single-token update does (flat float4 walk).  It first convolves the
// channels it needs -- its RP x channels and the N + N B/C channels of its group -- into LDS,
// rounded to the activation dtype as the two-launch path stores them, so the step is bitwise the
// two-launch one.  The group's B/C channels are convolved by all its blocks from the same old
// window, so the new conv state goes to a second buffer: each block writes its x channels, and
// the first block of each (b, group) writes the group's B/C channels.
#include "ssd_device.h"
#include "ssd_kernels.h"

namespace ssd {

constexpr int kStepThreads = 256;
constexpr int kStepF4 = 4;                                // float4 of state per thread (8: +2 %, 16: +8 %)
constexpr int kStepRowsF4 = kStepThreads * kStepF4;       // float4 per block (half a head at P = 64, N = 128)

// One conv channel: the loads (old window columns 1..3, the new input, taps, bias) are issued
// first, for all of a thread's channels, and used after one wait.
template <typename T>
struct ConvIn {
    T win[4], w[4], bias;
};
template <typename T>
__device__ __forceinline__ void conv_load(ConvIn<T>& in, const T* __restrict__ xbc, int64_t xs,
                                          const T* __restrict__ w, const T* __restrict__ bias,
                                          const T* __restrict__ s_in, int64_t CD, int64_t b, int64_t c) {
    const T* si = s_in + (b * CD + c) * 4;
    in.win[0] = si[1];
    in.win[1] = si[2];
    in.win[2] = si[3];
    in.win[3] = xbc[b * xs + c];
#pragma unroll
    for (int k = 0; k < 4; ++k) in.w[k] = w[c * 4 + k];
    in.bias = bias ? bias[c] : static_cast<T>(0.f);
}
// silu(bias + sum_k w[k] * window[k]) rounded to the activation dtype (as the conv call stores it);
// writes the rolled window when asked
template <typename T>
__device__ __forceinline__ float conv_out(const ConvIn<T>& in, T* __restrict__ s_out, int64_t CD, int64_t b,
                                          int64_t c, bool store) {
    float acc = static_cast<float>(in.bias);
#pragma unroll
    for (int k = 0; k < 4; ++k) acc = fmaf(static_cast<float>(in.w[k]), static_cast<float>(in.win[k]), acc);
    if (store) {
        T* so = s_out + (b * CD + c) * 4;
#pragma unroll
        for (int k = 0; k < 4; ++k) so[k] = in.win[k];
    }
    return static_cast<float>(static_cast<T>(silu_f(acc)));
}

// Grid: B * H * (P / RP) blocks; block (b, h, p-range).  RP * N / 4 <= kStepRowsF4.
template <typename T, typename TY, int N, bool DTP>
__global__ __launch_bounds__(kStepThreads) void decode_step_kernel(
    float* __restrict__ state, const T* __restrict__ xbc, int64_t xs, const T* __restrict__ w,
    const T* __restrict__ bias, const T* __restrict__ s_in, T* __restrict__ s_out, const T* __restrict__ dt,
    const float* __restrict__ A, const float* __restrict__ D, TY* __restrict__ y, int H, int P, int G, int RP,
    DtParams dtp) {
    constexpr int QPR = N / 4;
    __shared__ float cx[128];                            // x conv outputs of the block's rows (RP <= P <= 128)
    __shared__ float cb[N], cc[N];                       // the group's B and C conv outputs
    const int nrb = P / RP;                              // row blocks per head
    const int64_t bh = blockIdx.x / nrb;
    const int p0 = static_cast<int>(blockIdx.x % nrb) * RP;
    const int64_t b = bh / H;
    const int h = static_cast<int>(bh - b * H);
    const int g = h / (H / G);
    const int64_t I = static_cast<int64_t>(H) * P;
    const int64_t CD = I + 2LL * G * N;
    // the block's state rows, as the single-token update walks them: their loads are issued first,
    // so they are in flight while the block convolves
    f32x4* st4 = reinterpret_cast<f32x4*>(state) + (bh * P + p0) * QPR;
    const int nf4 = RP * QPR;
    const float dtv = DTP ? dt_prologue(static_cast<float>(dt[bh]), dtp, h) : static_cast<float>(dt[bh]);
    const float a = __expf(dtv * A[h]);
    f32x4 s[kStepF4];
#pragma unroll
    for (int i = 0; i < kStepF4; ++i) {
        const int f = threadIdx.x + i * kStepThreads;
        s[i] = f < nf4 ? __builtin_nontemporal_load(st4 + f) : f32x4{0.f, 0.f, 0.f, 0.f};
    }
    const bool bc_owner = (h % (H / G)) == 0 && p0 == 0;  // writes the group's new B/C windows
    // conv channels of the block: RP x channels, then the group's N B and N C channels
    const int nconv = RP + 2 * N;
    auto chan = [&](int c) -> int64_t {
        return c < RP ? static_cast<int64_t>(h) * P + p0 + c
                      : (c < RP + N ? I + static_cast<int64_t>(g) * N + (c - RP)
                                    : I + static_cast<int64_t>(G) * N + static_cast<int64_t>(g) * N + (c - RP - N));
    };
    constexpr int kCPT = 2;   // conv channels per thread: RP + 2N <= 128 + 256 <= 2 * 256 (one pass)
    ConvIn<T> cin[kCPT];
#pragma unroll
    for (int k = 0; k < kCPT; ++k) {
        const int c = threadIdx.x + k * kStepThreads;
        if (c < nconv) conv_load(cin[k], xbc, xs, w, bias, s_in, CD, b, chan(c));
    }
#pragma unroll
    for (int k = 0; k < kCPT; ++k) {
        const int c = threadIdx.x + k * kStepThreads;
        if (c < nconv) {
            const float v = conv_out(cin[k], s_out, CD, b, chan(c), c < RP || bc_owner);
            if (c < RP) cx[c] = v;
            else if (c < RP + N) cb[c - RP] = v;
            else cc[c - RP - N] = v;
        }
    }
    __syncthreads();

#pragma unroll
    for (int i = 0; i < kStepF4; ++i) {
        const int f = threadIdx.x + i * kStepThreads;
        const bool ok = f < nf4;
        const int ff = ok ? f : 0;
        const int r = ff / QPR, q = ff - r * QPR;
        const float xv = cx[r];
        const float dx = dtv * xv;
        f32x4 v = s[i];
        float part = 0.f;
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            v[k] = fmaf(a, v[k], dx * cb[4 * q + k]);
            part = fmaf(v[k], cc[4 * q + k], part);
        }
        if (!ok) part = 0.f;
        part = group_sum_last<QPR>(part);
        if (ok) {
            if (q == QPR - 1) y[bh * P + p0 + r] = static_cast<TY>(part + (D ? D[h] * xv : 0.f));
            __builtin_nontemporal_store(v, st4 + f);
        }
    }
}

template <typename T, typename TY, int N>
static hipError_t step_n(const DecodeStepArgs& a, hipStream_t s) {
    const UpdateArgs& u = a.u;
    const int P = u.head_dim;
    const int RP = P * (N / 4) <= kStepRowsF4 ? P : kStepRowsF4 / (N / 4);
    if (u.batch == 0) return hipSuccess;
    const int64_t blocks = u.batch * u.nheads * (P / RP);
    const bool dtp = u.dtp.bias || u.dtp.softplus || u.dtp.lo < u.dtp.hi;
    auto go = [&](auto kern) {
        hipLaunchKernelGGL(kern, dim3(static_cast<uint32_t>(blocks)), dim3(kStepThreads), 0, s, u.state,
                           static_cast<const T*>(a.xbc), a.xbc_row_stride, static_cast<const T*>(a.w),
                           static_cast<const T*>(a.bias), static_cast<const T*>(a.conv_in), static_cast<T*>(a.conv_out),
                           static_cast<const T*>(u.dt), u.A, u.D, static_cast<TY*>(u.y), u.nheads, P, u.ngroups, RP,
                           u.dtp);
        return hipGetLastError();
    };
    return dtp ? go(decode_step_kernel<T, TY, N, true>) : go(decode_step_kernel<T, TY, N, false>);
}

template <typename T, typename TY>
static hipError_t step_t(const DecodeStepArgs& a, hipStream_t s) {
    switch (a.u.d_state) {
        case 16: return step_n<T, TY, 16>(a, s);
        case 32: return step_n<T, TY, 32>(a, s);
        case 64: return step_n<T, TY, 64>(a, s);
        case 128: return step_n<T, TY, 128>(a, s);
        default: return hipErrorInvalidValue;
    }
}

hipError_t launch_decode_step(const DecodeStepArgs& a, Dt act, Dt ydt, hipStream_t s) {
    if (act == Dt::BF16) return ydt == Dt::BF16 ? step_t<bf16, bf16>(a, s) : step_t<bf16, float>(a, s);
    return ydt == Dt::BF16 ? step_t<float, bf16>(a, s) : step_t<float, float>(a, s);
}

}  // namespace ssd
