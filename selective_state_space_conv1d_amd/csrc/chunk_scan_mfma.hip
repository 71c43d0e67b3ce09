// SSD chunked scan for prefill on bf16 MFMA (gfx950), head_dim 64, d_state 128,
// chunk 128 -- the Ultra-family Mamba layer.
//
// Method (the structured-semiseparable / chunked form of the Mamba-2 scan:
// "Mamba 与 Nemotron 系列模型深度调研", Mamba 架构, and the 128-token chunked
// scan that returns the final state in the modeling_nemotron_h.py walk-through,
// "Prefill 阶段").  Per chunk of Q tokens, with cs the inclusive prefix sum of
// dt*A (base-2 units so that decays are exp2 of differences):
//   M[i][j] = (C_i . B_j) * exp(cs_i - cs_j) * dt_j   (j <= i), + D on the diagonal
//   y_i     = sum_j M[i][j] x_j  +  exp(cs_i) * (C_i . H)
//   H       = exp(cs_last) * H + sum_j exp(cs_last - cs_j) dt_j  x_j (x) B_j
// which is the token recurrence re-associated exactly.
//
// Mapping: one persistent workgroup (4 waves) per (batch, head) walks the
// chunks in order; the fp32 state H never leaves registers between chunks
// (no per-chunk states in HBM).  Wave w owns head_dim rows p in [16w, 16w+16):
// it keeps H^T[n][p] for those p as eight 16x16 MFMA accumulator tiles, and
// produces y^T[p][i] for its p and every token i of the chunk.
//
// All products are v_mfma_f32_16x16x32_bf16.  x, B and C arrive in bf16 and
// are exact operands; operands derived in fp32 (the score matrix M, the state
// H and the decay-weighted x) are split into bf16 hi + lo and issued as two
// MFMAs, which keeps the products at about 16 mantissa bits.  Accumulator
// tiles are reused directly as MFMA operands (accumulator column = lane, rows
// = k), permuting k consistently on both operands; that is how H feeds the
// C.H product and how nothing else round-trips through LDS except M.
//
// LDS per chunk (bf16, rows padded by 16 B): B[j][n], B^T[n][j], C[i][n],
// X^T[p][j] and one half (64 rows) of M hi/lo at a time: ~154 KB.
#include "ssd_device.h"
#include "ssd_kernels.h"

namespace ssd {

namespace mfma64 {

constexpr int Q = 128;   // tokens per chunk
constexpr int P = 64;    // head_dim
constexpr int NS = 128;  // d_state
constexpr int LD = 136;  // padded row length (bf16 elements) of the [.][128] tiles
constexpr int kThreads = 256;
constexpr float kLog2e = 1.4426950408889634f;

struct Smem {
    bf16 B[Q][LD];
    bf16 BT[NS][LD];
    bf16 C[Q][LD];
    bf16 XT[P][LD];
    bf16 Mhi[Q / 2][LD];
    bf16 Mlo[Q / 2][LD];
    float cs[Q];
    float dt[Q];
};

__device__ __forceinline__ f32x4 mfma(bf16x8 a, bf16x8 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ float fexp2(float v) { return __builtin_amdgcn_exp2f(v); }

// 8x8 transpose of bf16 held as 8 rows of 4 dwords (dword d = columns 2d, 2d+1).
__device__ __forceinline__ void transpose8x8(const u32x4 (&r)[8], u32x4 (&c)[8]) {
#pragma unroll
    for (int col = 0; col < 8; ++col) {
        const int d = col >> 1;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const uint32_t lo = r[2 * e][d], hi = r[2 * e + 1][d];
            c[col][e] = (col & 1) ? ((lo >> 16) | (hi & 0xffff0000u)) : ((lo & 0xffffu) | (hi << 16));
        }
    }
}

// v ~= hi + lo with both in bf16 (about 16 significant bits in total).
__device__ __forceinline__ bf16 bf_hi(float v) { return static_cast<bf16>(v); }
__device__ __forceinline__ bf16 bf_lo(float v, bf16 hi) { return static_cast<bf16>(v - static_cast<float>(hi)); }

template <typename TY>
__global__ __launch_bounds__(kThreads, 1) void chunk_scan_kernel(ScanArgs a) {
    extern __shared__ __align__(16) unsigned char smem_raw[];
    Smem& sm = *reinterpret_cast<Smem*>(smem_raw);
    const int tid = threadIdx.x;
    const int w = tid >> 6;          // wave: head_dim rows [16w, 16w+16)
    const int lane = tid & 63;
    const int li = lane & 15;        // MFMA row/col index
    const int lg = lane >> 4;        // MFMA k-group
    const int H = a.nheads;
    const int64_t L = a.seqlen;
    const int64_t b = blockIdx.x / H;
    const int h = static_cast<int>(blockIdx.x % H);
    const int grp = h / (H / a.ngroups);
    const float A2 = a.A[h] * kLog2e;
    const float Dh = a.D ? a.D[h] : 0.f;
    const bf16* xg = static_cast<const bf16*>(a.x);
    const bf16* Bg = static_cast<const bf16*>(a.B);
    const bf16* Cg = static_cast<const bf16*>(a.C);
    const bf16* dtg = static_cast<const bf16*>(a.dt);
    TY* yg = static_cast<TY*>(a.y);

    // H^T accumulators: accH[nt][r] = H[p = 16w + li][n = 16nt + 4lg + r]
    const int64_t srow = ((b * H + h) * P + 16 * w + li) * static_cast<int64_t>(NS);
    f32x4 accH[8];
#pragma unroll
    for (int nt = 0; nt < 8; ++nt) {
        if (a.init_state) accH[nt] = *reinterpret_cast<const f32x4*>(a.init_state + srow + 16 * nt + 4 * lg);
        else accH[nt] = f32x4{0.f, 0.f, 0.f, 0.f};
    }

    const int64_t nchunks = (L + Q - 1) / Q;
    for (int64_t c = 0; c < nchunks; ++c) {
        const int64_t t0 = c * Q;
        const int valid = static_cast<int>((L - t0) < Q ? (L - t0) : Q);
        __syncthreads();  // previous chunk is done with LDS

        // ---- stage B (natural + transposed), C, X^T, dt
        {
            const int ta = tid >> 4;        // token block: tokens 8ta .. 8ta+7
            const int nb = tid & 15;        // state block: n 8nb .. 8nb+7
            u32x4 rb[8], rc[8];
#pragma unroll
            for (int r = 0; r < 8; ++r) {
                const int j = 8 * ta + r;
                if (j < valid) {
                    const int64_t o = (b * L + t0 + j) * a.bc_row_stride + static_cast<int64_t>(grp) * NS + 8 * nb;
                    rb[r] = *reinterpret_cast<const u32x4*>(Bg + o);
                    rc[r] = *reinterpret_cast<const u32x4*>(Cg + o);
                } else {
                    rb[r] = u32x4{0u, 0u, 0u, 0u};
                    rc[r] = u32x4{0u, 0u, 0u, 0u};
                }
            }
            u32x4 xr[8];
            const bool xthread = tid < 128;
            const int xa = tid >> 3;        // token block for X (tid < 128)
            const int pb = tid & 7;         // p block: p 8pb .. 8pb+7
            if (xthread) {
#pragma unroll
                for (int r = 0; r < 8; ++r) {
                    const int j = 8 * xa + r;
                    if (j < valid)
                        xr[r] = *reinterpret_cast<const u32x4*>(
                            xg + (b * L + t0 + j) * a.x_row_stride + static_cast<int64_t>(h) * P + 8 * pb);
                    else
                        xr[r] = u32x4{0u, 0u, 0u, 0u};
                }
            }
            float dv = 0.f;
            if (tid >= 128) {
                const int j = tid - 128;
                if (j < valid) dv = static_cast<float>(dtg[(b * L + t0 + j) * H + h]);
            }
#pragma unroll
            for (int r = 0; r < 8; ++r) {
                *reinterpret_cast<u32x4*>(&sm.B[8 * ta + r][8 * nb]) = rb[r];
                *reinterpret_cast<u32x4*>(&sm.C[8 * ta + r][8 * nb]) = rc[r];
            }
            u32x4 tb[8];
            transpose8x8(rb, tb);
#pragma unroll
            for (int k = 0; k < 8; ++k) *reinterpret_cast<u32x4*>(&sm.BT[8 * nb + k][8 * ta]) = tb[k];
            if (xthread) {
                u32x4 tx[8];
                transpose8x8(xr, tx);
#pragma unroll
                for (int k = 0; k < 8; ++k) *reinterpret_cast<u32x4*>(&sm.XT[8 * pb + k][8 * xa]) = tx[k];
            } else {
                const int j = tid - 128;
                sm.dt[j] = dv;
                sm.cs[j] = dv * A2;
            }
        }
        __syncthreads();
        if (w == 0) {  // inclusive prefix sum of dt*A*log2(e), two tokens per lane
            const float v0 = sm.cs[2 * lane], v1 = sm.cs[2 * lane + 1];
            float s = v0 + v1;
#pragma unroll
            for (int off = 1; off < 64; off <<= 1) {
                const float u = __shfl_up(s, off, 64);
                if (lane >= off) s += u;
            }
            const float ex = s - (v0 + v1);
            sm.cs[2 * lane] = ex + v0;
            sm.cs[2 * lane + 1] = ex + v0 + v1;
        }
        __syncthreads();

        // X^T fragments of this wave (A operand of y^T, and, decay-weighted, B operand of S)
        bf16x8 xf[4];
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) xf[ks] = *reinterpret_cast<const bf16x8*>(&sm.XT[16 * w + li][32 * ks + 8 * lg]);

        f32x4 accY[8];
#pragma unroll
        for (int it = 0; it < 8; ++it) accY[it] = f32x4{0.f, 0.f, 0.f, 0.f};

#pragma unroll
        for (int half = 0; half < 2; ++half) {
            // ---- M for token rows of this half: wave w builds i-tile it = 4*half + w
            {
                const int it = 4 * half + w;
                const int i = 16 * it + li;
                const float csi = sm.cs[i];
                bf16x8 cf[4];
#pragma unroll
                for (int ks = 0; ks < 4; ++ks) cf[ks] = *reinterpret_cast<const bf16x8*>(&sm.C[i][32 * ks + 8 * lg]);
                for (int jt = 0; jt <= it; ++jt) {
                    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                    for (int ks = 0; ks < 4; ++ks)
                        acc = mfma(*reinterpret_cast<const bf16x8*>(&sm.B[16 * jt + li][32 * ks + 8 * lg]), cf[ks], acc);
                    // acc[r] = (C_i . B_j), j = 16jt + 4lg + r
                    bf16x4 mh, ml;
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        const int j = 16 * jt + 4 * lg + r;
                        float m = 0.f;
                        if (j <= i) m = acc[r] * fexp2(csi - sm.cs[j]) * sm.dt[j] + (j == i ? Dh : 0.f);
                        mh[r] = bf_hi(m);
                        ml[r] = bf_lo(m, mh[r]);
                    }
                    *reinterpret_cast<bf16x4*>(&sm.Mhi[i - 64 * half][16 * jt + 4 * lg]) = mh;
                    *reinterpret_cast<bf16x4*>(&sm.Mlo[i - 64 * half][16 * jt + 4 * lg]) = ml;
                }
                if ((it & 1) == 0) {  // the upper half of the last 32-wide k step is read: zero it
                    const bf16x4 z = {bf16(0.f), bf16(0.f), bf16(0.f), bf16(0.f)};
                    *reinterpret_cast<bf16x4*>(&sm.Mhi[i - 64 * half][16 * (it + 1) + 4 * lg]) = z;
                    *reinterpret_cast<bf16x4*>(&sm.Mlo[i - 64 * half][16 * (it + 1) + 4 * lg]) = z;
                }
            }
            __syncthreads();
            // ---- y^T[p][i] += sum_j X^T[p][j] M^T[j][i]  (causal: k steps up to the diagonal)
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const int it = 4 * half + q;
                const int row = 16 * q + li;
#pragma unroll
                for (int ks = 0; ks <= it / 2; ++ks) {
                    const bf16x8 mh = *reinterpret_cast<const bf16x8*>(&sm.Mhi[row][32 * ks + 8 * lg]);
                    const bf16x8 ml = *reinterpret_cast<const bf16x8*>(&sm.Mlo[row][32 * ks + 8 * lg]);
                    accY[it] = mfma(xf[ks], mh, accY[it]);
                    accY[it] = mfma(xf[ks], ml, accY[it]);
                }
            }
            __syncthreads();
        }

        // ---- carried state: y^T[p][i] += exp(cs_i) * sum_n H[p][n] C[i][n]
        {
            bf16x8 hh[4], hl[4];
#pragma unroll
            for (int ks = 0; ks < 4; ++ks) {
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    hh[ks][r] = bf_hi(accH[2 * ks][r]);
                    hl[ks][r] = bf_lo(accH[2 * ks][r], hh[ks][r]);
                    hh[ks][4 + r] = bf_hi(accH[2 * ks + 1][r]);
                    hl[ks][4 + r] = bf_lo(accH[2 * ks + 1][r], hh[ks][4 + r]);
                }
            }
#pragma unroll
            for (int it = 0; it < 8; ++it) {
                const int i = 16 * it + li;
                f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int ks = 0; ks < 4; ++ks) {
                    const bf16x4 c0 = *reinterpret_cast<const bf16x4*>(&sm.C[i][32 * ks + 4 * lg]);
                    const bf16x4 c1 = *reinterpret_cast<const bf16x4*>(&sm.C[i][32 * ks + 16 + 4 * lg]);
                    const bf16x8 cfr = {c0[0], c0[1], c0[2], c0[3], c1[0], c1[1], c1[2], c1[3]};
                    acc = mfma(hh[ks], cfr, acc);
                    acc = mfma(hl[ks], cfr, acc);
                }
                const float e = fexp2(sm.cs[i]);
#pragma unroll
                for (int r = 0; r < 4; ++r) accY[it][r] = fmaf(e, acc[r], accY[it][r]);
            }
        }

        // ---- write y: lane holds y[token 16it+li][p = 16w + 4lg .. +3]
#pragma unroll
        for (int it = 0; it < 8; ++it) {
            const int i = 16 * it + li;
            if (i < valid) {
                TY* dst = yg + ((b * L + t0 + i) * H + h) * static_cast<int64_t>(P) + 16 * w + 4 * lg;
                if constexpr (sizeof(TY) == 4) {
                    *reinterpret_cast<f32x4*>(dst) = accY[it];
                } else {
                    const bf16x4 v = {bf16(accY[it][0]), bf16(accY[it][1]), bf16(accY[it][2]), bf16(accY[it][3])};
                    *reinterpret_cast<bf16x4*>(dst) = v;
                }
            }
        }

        // ---- state: H = exp(cs_last) H + sum_j B^T[n][j] (w_j x_j)[p]
        {
            // decay to the chunk's last real token; the cumulative sum is read at that
            // token itself so that its own weight is exp2(0) = 1 exactly
            const float cl = sm.cs[valid - 1];
            const float alpha = fexp2(cl);
            bf16x8 xh[4], xl[4];
#pragma unroll
            for (int ks = 0; ks < 4; ++ks) {
#pragma unroll
                for (int s = 0; s < 8; ++s) {
                    const int j = 32 * ks + 8 * lg + s;
                    const float v = j < valid ? static_cast<float>(xf[ks][s]) * (fexp2(cl - sm.cs[j]) * sm.dt[j]) : 0.f;
                    xh[ks][s] = bf_hi(v);
                    xl[ks][s] = bf_lo(v, xh[ks][s]);
                }
            }
#pragma unroll
            for (int nt = 0; nt < 8; ++nt) {
                f32x4 acc = accH[nt] * alpha;
#pragma unroll
                for (int ks = 0; ks < 4; ++ks) {
                    const bf16x8 bt = *reinterpret_cast<const bf16x8*>(&sm.BT[16 * nt + li][32 * ks + 8 * lg]);
                    acc = mfma(bt, xh[ks], acc);
                    acc = mfma(bt, xl[ks], acc);
                }
                accH[nt] = acc;
            }
        }
    }

    if (a.final_state) {
#pragma unroll
        for (int nt = 0; nt < 8; ++nt)
            *reinterpret_cast<f32x4*>(a.final_state + srow + 16 * nt + 4 * lg) = accH[nt];
    }
}

}  // namespace mfma64

bool mfma_scan_supports(int head_dim, int d_state, int chunk) {
    return head_dim == mfma64::P && d_state == mfma64::NS && chunk == mfma64::Q;
}

template <typename TY>
static hipError_t mfma_t(const ScanArgs& a, hipStream_t s) {
    const int64_t blocks = a.batch * a.nheads;
    if (blocks == 0) return hipSuccess;
    auto kern = mfma64::chunk_scan_kernel<TY>;
    const size_t smem = sizeof(mfma64::Smem);
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, static_cast<int>(smem));
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(kern, dim3(static_cast<uint32_t>(blocks)), dim3(mfma64::kThreads), smem, s, a);
    return hipGetLastError();
}

hipError_t launch_chunk_scan_mfma(const ScanArgs& a, Dt ydt, hipStream_t s) {
    return ydt == Dt::BF16 ? mfma_t<bf16>(a, s) : mfma_t<float>(a, s);
}

}  // namespace ssd
