// Chunked SSD scan on fp32 FMA: the fp32-precision path (and any head_dim /
// d_state up to 128 outside the MFMA instantiation).
//
// The scan is the exact re-association of the recurrence in blocks of
// kT = 32 tokens (the structured semiseparable form of Mamba-2, "Mamba 与
// Nemotron 系列模型深度调研", Mamba 架构): inside a block, with cs the
// inclusive prefix sum of dt*A,
//   y_i = sum_{j<=i} (C_i.B_j) exp(cs_i - cs_j) dt_j x_j + D x_i      (intra)
//       + exp(cs_i) C_i . H                                           (carried state)
//   H  <- exp(cs_last) H + sum_j exp(cs_last - cs_j) dt_j x_j (x) B_j
// One workgroup per (batch, head) walks the blocks in order with H in LDS.
// The block length is internal (the result does not depend on it beyond
// rounding); the caller's chunk size only selects the MFMA kernel's tiling.
#include "ssd_device.h"
#include "ssd_kernels.h"
#include "state_codes.h"

namespace ssd {

constexpr int kT = 32;
constexpr int kFmaThreads = 256;
constexpr int kMaxPN = 128;

struct FmaSmem {
    float X[kT][kMaxPN];
    float B[kT][kMaxPN];
    float C[kT][kMaxPN];
    float M[kT][kT + 1];
    float H[kMaxPN][kMaxPN + 1];
    float cs[kT];
    float dt[kT];
    float wl[kT];
};

// LP: the initial and final states are 16-bit codes (a separate instantiation)
template <typename T, typename TY, bool LP>
__global__ __launch_bounds__(kFmaThreads) void chunk_scan_fma_kernel(ScanArgs a) {
    extern __shared__ __align__(16) unsigned char smem_raw[];
    FmaSmem& sm = *reinterpret_cast<FmaSmem*>(smem_raw);
    const int tid = threadIdx.x;
    const int H = a.nheads, P = a.head_dim, N = a.d_state;
    const int64_t b = blockIdx.x / H;   // batch entry, or sequence of a packed batch
    int64_t L = a.seqlen, row0 = b * a.seqlen, sidx = b;
    bool use_init = true, write_final = true;
    if (a.seq.cu_seqlens) {
        seq_span(a.seq.cu_seqlens, b, a.seqlen, row0, L);
        const int64_t slot = seq_slot(a.seq.slot_idx, b, a.seq.nslots);
        sidx = slot < 0 ? 0 : slot;
        use_init = slot >= 0 && a.seq.has_init && a.seq.has_init[b] != 0;
        write_final = slot >= 0;
    }
    const int h = static_cast<int>(blockIdx.x % H);
    const int g = h / (H / a.ngroups);
    const float Ah = a.A[h];
    const float Dh = a.D ? a.D[h] : 0.f;
    const T* xg = static_cast<const T*>(a.x);
    const T* Bg = static_cast<const T*>(a.B);
    const T* Cg = static_cast<const T*>(a.C);
    const T* dtg = static_cast<const T*>(a.dt);
    TY* yg = static_cast<TY*>(a.y);
    const int64_t sbase = (sidx * H + h) * static_cast<int64_t>(P) * N;

    for (int e = tid; e < P * N; e += kFmaThreads) {
        const int p = e / N, n = e - p * N;
        float v = 0.f;
        if constexpr (LP) {
            if (use_init && a.init16) v = code_dec(a.init16[sbase + e], a.codes.f16);
        } else {
            if (use_init && a.init_state) v = a.init_state[sbase + e];
        }
        sm.H[p][n] = v;
    }

    for (int64_t t0 = 0; t0 < L; t0 += kT) {
        const int valid = static_cast<int>((L - t0) < kT ? (L - t0) : kT);
        __syncthreads();
        for (int e = tid; e < kT * P; e += kFmaThreads) {
            const int j = e / P, p = e - j * P;
            sm.X[j][p] = j < valid ? static_cast<float>(xg[(row0 + t0 + j) * a.x_row_stride +
                                                         static_cast<int64_t>(h) * P + p])
                                   : 0.f;
        }
        for (int e = tid; e < kT * N; e += kFmaThreads) {
            const int j = e / N, n = e - j * N;
            const int64_t o = (row0 + t0 + j) * a.bc_row_stride + static_cast<int64_t>(g) * N + n;
            sm.B[j][n] = j < valid ? static_cast<float>(Bg[o]) : 0.f;
            sm.C[j][n] = j < valid ? static_cast<float>(Cg[o]) : 0.f;
        }
        if (tid < kT) {
            const float d = tid < valid ? dt_prologue(static_cast<float>(dtg[(row0 + t0 + tid) * H + h]), a.dtp, h)
                                        : 0.f;
            sm.dt[tid] = d;
            // inclusive prefix sum of dt*A over the block (lanes 0..31 of wave 0)
            float v = d * Ah;
#pragma unroll
            for (int off = 1; off < kT; off <<= 1) {
                const float u = __shfl_up(v, off, 64);
                if (tid >= off) v += u;
            }
            sm.cs[tid] = v;
        }
        __syncthreads();
        // weights to the block's last real token (its own weight is exp(0) = 1 exactly)
        if (tid < kT) sm.wl[tid] = tid < valid ? expf(sm.cs[valid - 1] - sm.cs[tid]) * sm.dt[tid] : 0.f;
        // M[i][j] = (C_i . B_j) exp(cs_i - cs_j) dt_j for j <= i, + D on the diagonal
        for (int e = tid; e < kT * kT; e += kFmaThreads) {
            const int i = e / kT, j = e - i * kT;
            float m = 0.f;
            if (j <= i) {
                float cb = 0.f;
                for (int n = 0; n < N; ++n) cb = fmaf(sm.C[i][n], sm.B[j][n], cb);
                m = cb * expf(sm.cs[i] - sm.cs[j]) * sm.dt[j];
                if (i == j) m += Dh;
            }
            sm.M[i][j] = m;
        }
        __syncthreads();
        for (int e = tid; e < kT * P; e += kFmaThreads) {
            const int i = e / P, p = e - i * P;
            if (i >= valid) continue;
            float yd = 0.f;
            for (int j = 0; j <= i; ++j) yd = fmaf(sm.M[i][j], sm.X[j][p], yd);
            float yo = 0.f;
            for (int n = 0; n < N; ++n) yo = fmaf(sm.C[i][n], sm.H[p][n], yo);
            yg[((row0 + t0 + i) * H + h) * static_cast<int64_t>(P) + p] =
                static_cast<TY>(yd + expf(sm.cs[i]) * yo);
        }
        __syncthreads();
        const float alpha = expf(sm.cs[valid - 1]);
        for (int e = tid; e < P * N; e += kFmaThreads) {
            const int p = e / N, n = e - p * N;
            float s = 0.f;
            for (int j = 0; j < kT; ++j) s = fmaf(sm.wl[j] * sm.X[j][p], sm.B[j][n], s);
            sm.H[p][n] = fmaf(alpha, sm.H[p][n], s);
        }
        // state snapshot after token t0 + kT - 1 when that closes an interval (a multiple of kT)
        float* snap = a.snapshots ? snapshot_dst(a, b, L, t0 + kT, h) : nullptr;
        if (snap) {
            __syncthreads();
            for (int e = tid; e < P * N; e += kFmaThreads) {
                const int p = e / N, n = e - p * N;
                snap[e] = sm.H[p][n];
            }
        }
    }
    __syncthreads();
    if ((LP ? a.final16 != nullptr : a.final_state != nullptr) && write_final)
        for (int e = tid; e < P * N; e += kFmaThreads) {
            const int p = e / N, n = e - p * N;
            if constexpr (LP) codes_store1(a.final16, a.codes, sbase + e, sm.H[p][n]);
            else a.final_state[sbase + e] = sm.H[p][n];
        }
}

template <typename T, typename TY>
static hipError_t fma_t(const ScanArgs& a, hipStream_t s) {
    const int64_t blocks = a.batch * a.nheads;
    if (blocks == 0) return hipSuccess;
    auto kern = (a.init16 || a.final16) ? chunk_scan_fma_kernel<T, TY, true> : chunk_scan_fma_kernel<T, TY, false>;
    const size_t smem = sizeof(FmaSmem);
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, static_cast<int>(smem));
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(kern, dim3(static_cast<uint32_t>(blocks)), dim3(kFmaThreads), smem, s, a);
    return hipGetLastError();
}

hipError_t launch_chunk_scan_fma(const ScanArgs& a, Dt act, Dt ydt, hipStream_t s) {
    if (act == Dt::BF16) return ydt == Dt::BF16 ? fma_t<bf16, bf16>(a, s) : fma_t<bf16, float>(a, s);
    return ydt == Dt::BF16 ? fma_t<float, bf16>(a, s) : fma_t<float, float>(a, s);
}

}  // namespace ssd
