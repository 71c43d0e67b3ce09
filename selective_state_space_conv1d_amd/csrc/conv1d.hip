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
// tokens per thread in the prefill conv: 24 measured fastest (prefill 1 x 8192 x 18432: 16 or 12 within
// 2 %, 32 and 20 7-10 % slower: fewer workgroups per CU round)
constexpr int kConvTokens = 24;

// Rows [ta, tb) of one thread's channel vector: out[t] = silu(bias + sum_k w[k] * in[t-3+k]), with
// win holding the inputs at ta-3..ta-1 on entry.  Four rows are loaded before any is used, so each
// thread keeps four 16-byte loads in flight.  STREAM reads the input rows non-temporally (125 -> 113 us
// on the 1 x 8192 x 18432 prefill); the output, which the scan reads next, stays cacheable.
template <typename T, int V, bool STREAM>
__device__ __forceinline__ void conv_rows(const T* __restrict__ xr, int64_t xs, T* __restrict__ orow, int64_t os,
                                          int64_t ta, int64_t tb, const float (&wt)[4][V], const float (&bs)[V],
                                          float (&win)[3][V]) {
    auto step = [&](const float (&u)[V], int64_t t) {
        float o[V];
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
        store16_f32(orow + t * os, o);
    };
    int64_t t = ta;
    for (; t + 4 <= tb; t += 4) {
        float u[4][V];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            if constexpr (STREAM) load16_f32_nt(xr + (t + r) * xs, u[r]);
            else load16_f32(xr + (t + r) * xs, u[r]);
        }
        // keeps the four loads ahead of the rows' arithmetic and stores (left to itself the scheduler
        // interleaves them, and each row's wait then also waits for the previous row's store)
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int r = 0; r < 4; ++r) step(u[r], t + r);
    }
    for (; t < tb; ++t) {
        float u[V];
        if constexpr (STREAM) load16_f32_nt(xr + t * xs, u);
        else load16_f32(xr + t * xs, u);
        step(u, t);
    }
}

// Launches of more than kWideGrid workgroups run many rounds on the chip.  There the workgroups are
// numbered XCD-contiguously (the hardware deals them to the 8 XCDs round-robin; XCD k takes the k-th
// eighth of the tiles) and the input is read through the caches: a tile's three halo rows are the
// previous tile's last rows, read on the same XCD shortly before (262144-token prefill: 3905 -> 3541
// us).  Smaller launches keep the plain numbering and stream the input, which measured faster for them
// and for the scan that reads their output (1 x 8192: conv 111 -> 110 us, scan after it 221 -> 214 us).
constexpr int64_t kWideGrid = 16384;

// Workgroup index in [0, n) for the linear dispatch index id: XCD-contiguous when WIDE.
template <bool WIDE>
__device__ __forceinline__ int64_t conv_wg_index(int64_t id, int64_t n) {
    if constexpr (!WIDE) return id;
    const int64_t per = n / 8, rem = n % 8, xcd = id % 8;
    return xcd * per + (xcd < rem ? xcd : rem) + id / 8;
}

// Grid: x = channel blocks * token tiles (channel block fastest), y = batch.
// The thread of token tile 0 reads the incoming state before it writes the
// outgoing one, so conv_state_out may alias conv_state_in.
template <typename T, bool WIDE>
__global__ __launch_bounds__(kConvThreads) void conv1d_fwd_kernel(
    const T* __restrict__ xbc, int64_t xs, const T* __restrict__ w, const T* __restrict__ bias,
    const T* s_in, T* s_out, T* __restrict__ out, int64_t L, int64_t CD, int64_t cblocks) {
    constexpr int V = Vec16<T>::n;
    const int64_t nx = gridDim.x;
    const int64_t wg = conv_wg_index<WIDE>(static_cast<int64_t>(blockIdx.y) * nx + blockIdx.x, nx * gridDim.y);
    const int64_t cb = wg % nx % cblocks;
    const int64_t tile = wg % nx / cblocks;
    const int64_t c0 = (cb * kConvThreads + threadIdx.x) * V;
    if (c0 >= CD) return;
    const int64_t b = wg / nx;
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
    if (tile == 0) {
        float st[4][V];    // incoming state
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

    conv_rows<T, V, !WIDE>(xb + c0, xs, out + b * L * CD + c0, CD, t0, t1, wt, bs, win);

    if (tile == 0 && s_out) {
        // new state column k = input at token L-4+k (from the old state when negative)
        float ns[4][V];
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            const int64_t tau = L - 4 + k;
            if (tau >= 0) {
                load16_f32(xb + tau * xs + c0, ns[k]);
            } else if (s_in) {
                // old column 4 + tau, read by address (a private array indexed by the run-time column
                // would live in scratch memory); every read precedes the stores below
                const T* col = s_in + (b * CD + c0) * 4 + (4 + tau);
#pragma unroll
                for (int v = 0; v < V; ++v) ns[k][v] = static_cast<float>(col[4 * v]);
            } else {
#pragma unroll
                for (int v = 0; v < V; ++v) ns[k][v] = 0.f;
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
    T* __restrict__ state, T* __restrict__ out, int64_t CD, int64_t total, const int32_t* __restrict__ slot_idx,
    int64_t nslots) {
    constexpr int V = Vec16<T>::n;
    const int64_t idx = static_cast<int64_t>(blockIdx.x) * kConvThreads + threadIdx.x;
    if (idx >= total) return;
    const int64_t per_b = CD / V;
    const int64_t b = idx / per_b;
    const int64_t c0 = (idx - b * per_b) * V;

    float s[4 * V], wt[4 * V], u[V], bs[V], o[V];
    // the window of batch entry b (its pool slot with a slot table; none for padding)
    const int64_t slot = slot_idx ? seq_slot(slot_idx, b, nslots) : b;
    T* sp = state + (slot < 0 ? 0 : slot * CD + c0) * 4;
    if (slot >= 0) {
#pragma unroll
        for (int q = 0; q < 4; ++q) load16_f32(sp + q * V, s + q * V);
    } else {
#pragma unroll
        for (int k = 0; k < 4 * V; ++k) s[k] = 0.f;
    }
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
    if (slot >= 0) {
#pragma unroll
        for (int q = 0; q < 4; ++q) store16_f32(sp + q * V, s + q * V);
    }
    store16_f32(out + b * CD + c0, o);
}

// ---------------------------------------------------------------------------
// Packed variable-length prefill: token rows [cu[s], cu[s+1]) belong to sequence s, whose halo
// comes from its conv-state slot (zeros without an initial state).  Token tiles run over the
// packed rows and may straddle sequences; the window restarts at each sequence's first token.
// Rows outside every sequence (only with a malformed table) are not written.
struct SeqView {
    const int32_t* cu; const int32_t* slot; const int32_t* init; int64_t nseq, nslots, total;
    __device__ __forceinline__ void span(int64_t s, int64_t& start, int64_t& end) const {
        int64_t len;
        seq_span(cu, s, total, start, len);
        end = start + len;
    }
};

template <typename T, bool WIDE>
__global__ __launch_bounds__(kConvThreads) void conv1d_fwd_varlen_kernel(
    const T* __restrict__ xbc, int64_t xs, const T* __restrict__ w, const T* __restrict__ bias,
    const T* pool, T* __restrict__ out, int64_t CD, int64_t cblocks, SeqView sv) {
    constexpr int V = Vec16<T>::n;
    const int64_t wg = conv_wg_index<WIDE>(blockIdx.x, gridDim.x);
    const int64_t cb = wg % cblocks;
    const int64_t tile = wg / cblocks;
    const int64_t c0 = (cb * kConvThreads + threadIdx.x) * V;
    if (c0 >= CD) return;
    const int64_t t0 = tile * kConvTokens;
    const int64_t t1 = (t0 + kConvTokens < sv.total) ? t0 + kConvTokens : sv.total;

    float wt[4][V], bs[V];
    {
        float tmp[4 * V];
#pragma unroll
        for (int q = 0; q < 4; ++q) load16_f32(w + c0 * 4 + q * V, tmp + q * V);
#pragma unroll
        for (int v = 0; v < V; ++v)
#pragma unroll
            for (int k = 0; k < 4; ++k) wt[k][v] = tmp[v * 4 + k];
    }
    if (bias) load16_f32(bias + c0, bs);
    else
#pragma unroll
        for (int v = 0; v < V; ++v) bs[v] = 0.f;

    // the last sequence whose first row is <= t0 (binary search; the table is nondecreasing)
    int64_t lo = 0, hi = sv.nseq - 1;
    while (lo < hi) {
        const int64_t mid = (lo + hi + 1) >> 1;
        int64_t st, en;
        sv.span(mid, st, en);
        if (st <= t0) lo = mid;
        else hi = mid - 1;
    }
    // One segment per sequence that overlaps the tile; inside a segment the row loop is the plain
    // sliding window of the batched kernel, with no per-row sequence test.
    for (int64_t s = lo; s < sv.nseq; ++s) {
        int64_t start, end;
        sv.span(s, start, end);
        if (start >= t1) break;
        const int64_t ta = start > t0 ? start : t0;
        const int64_t tb = end < t1 ? end : t1;
        if (ta >= tb) continue;
        // window at row ta: inputs ta-3..ta-1, from the slot's state (or zeros) before the sequence.
        // Input row ta-3+k precedes the sequence when k < 3 - d; it is then state column d+1+k.  The
        // column is read from the pool by address: a private array indexed by the (run-time) column
        // would live in scratch memory, whose writes cost every thread 96 bytes of HBM traffic.
        float win[3][V];
        {
            const int64_t d = ta - start;   // rows of the sequence before ta
            const int64_t slot = seq_slot(sv.slot, s, sv.nslots);
            const bool from_state = slot >= 0 && sv.init && sv.init[s] != 0;
#pragma unroll
            for (int k = 0; k < 3; ++k) {
                if (d >= 3 - k) {
                    load16_f32(xbc + (ta - 3 + k) * xs + c0, win[k]);
                } else if (from_state) {
                    const T* col = pool + (slot * CD + c0) * 4 + (d + 1 + k);
#pragma unroll
                    for (int v = 0; v < V; ++v) win[k][v] = static_cast<float>(col[4 * v]);
                } else {
#pragma unroll
                    for (int v = 0; v < V; ++v) win[k][v] = 0.f;
                }
            }
        }
        conv_rows<T, V, !WIDE>(xbc + c0, xs, out + c0, CD, ta, tb, wt, bs, win);
        if (tb == t1) break;   // tile done: no table read for a next sequence
    }
}

// New conv state of every sequence with a slot: column k = input row end - 4 + k, from the old
// state (or zeros) where that is before the sequence's first row.  Runs after the per-token pass,
// which reads the old states; each thread reads its own old columns before writing them.
template <typename T>
__global__ __launch_bounds__(kConvThreads) void conv_state_varlen_kernel(const T* __restrict__ xbc, int64_t xs,
                                                                         T* pool, int64_t CD, SeqView sv) {
    constexpr int V = Vec16<T>::n;
    const int64_t c0 = (static_cast<int64_t>(blockIdx.x) * kConvThreads + threadIdx.x) * V;
    if (c0 >= CD) return;
    const int64_t s = blockIdx.y;
    const int64_t slot = seq_slot(sv.slot, s, sv.nslots);
    if (slot < 0) return;
    int64_t start, end;
    sv.span(s, start, end);
    T* sp = pool + (slot * CD + c0) * 4;
    const bool from_state = sv.init && sv.init[s] != 0;
    // old columns are read by address (a private array indexed by the run-time column would live in
    // scratch memory), all of them before the new state is stored over them
    float ns[4][V];
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        const int64_t tau = end - 4 + k;
        if (tau >= start) {
            load16_f32(xbc + tau * xs + c0, ns[k]);
        } else if (from_state) {
            const T* col = sp + (4 + (tau - start));   // old column 4 + tau - start (at least k)
#pragma unroll
            for (int v = 0; v < V; ++v) ns[k][v] = static_cast<float>(col[4 * v]);
        } else {
#pragma unroll
            for (int v = 0; v < V; ++v) ns[k][v] = 0.f;
        }
    }
    float tmp[4 * V];
#pragma unroll
    for (int v = 0; v < V; ++v)
#pragma unroll
        for (int k = 0; k < 4; ++k) tmp[v * 4 + k] = ns[k][v];
#pragma unroll
    for (int q = 0; q < 4; ++q) store16_f32(sp + q * V, tmp + q * V);
}

template <typename T>
static hipError_t conv_fwd_varlen_t(const ConvFwdArgs& a, hipStream_t s) {
    constexpr int V = Vec16<T>::n;
    if (a.batch == 0 || a.channels == 0) return hipSuccess;
    const int64_t cblocks = (a.channels / V + kConvThreads - 1) / kConvThreads;
    SeqView sv{a.seq.cu_seqlens, a.seq.slot_idx, a.seq.has_init, a.batch, a.seq.nslots, a.seqlen};
    T* pool = static_cast<T*>(a.state_out);
    if (a.seqlen > 0) {
        const int64_t tiles = (a.seqlen + kConvTokens - 1) / kConvTokens;
        auto kern = cblocks * tiles > kWideGrid ? conv1d_fwd_varlen_kernel<T, true> : conv1d_fwd_varlen_kernel<T, false>;
        hipLaunchKernelGGL(kern, dim3(static_cast<uint32_t>(cblocks * tiles)),
                           dim3(kConvThreads), 0, s, static_cast<const T*>(a.xbc), a.xbc_row_stride,
                           static_cast<const T*>(a.w), static_cast<const T*>(a.bias), pool,
                           static_cast<T*>(a.out), a.channels, cblocks, sv);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    if (pool == nullptr || a.seq.nslots == 0) return hipSuccess;
    hipLaunchKernelGGL(conv_state_varlen_kernel<T>, dim3(static_cast<uint32_t>(cblocks), static_cast<uint32_t>(a.batch)),
                       dim3(kConvThreads), 0, s, static_cast<const T*>(a.xbc), a.xbc_row_stride, pool,
                       a.channels, sv);
    return hipGetLastError();
}

template <typename T>
static hipError_t conv_fwd_t(const ConvFwdArgs& a, hipStream_t s) {
    constexpr int V = Vec16<T>::n;
    const int64_t cblocks = (a.channels / V + kConvThreads - 1) / kConvThreads;
    const int64_t tiles = a.seqlen > 0 ? (a.seqlen + kConvTokens - 1) / kConvTokens : 1;
    if (a.batch == 0 || a.channels == 0) return hipSuccess;
    if (a.seqlen == 0 && a.state_out == nullptr) return hipSuccess;
    dim3 grid(static_cast<uint32_t>(cblocks * tiles), static_cast<uint32_t>(a.batch));
    auto kern = cblocks * tiles * a.batch > kWideGrid ? conv1d_fwd_kernel<T, true> : conv1d_fwd_kernel<T, false>;
    hipLaunchKernelGGL(kern, grid, dim3(kConvThreads), 0, s,
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
                       a.channels, total, a.slot_idx, a.nslots);
    return hipGetLastError();
}

hipError_t launch_conv1d_fwd(const ConvFwdArgs& a, Dt act, hipStream_t s) {
    return act == Dt::BF16 ? conv_fwd_t<bf16>(a, s) : conv_fwd_t<float>(a, s);
}

hipError_t launch_conv1d_fwd_varlen(const ConvFwdArgs& a, Dt act, hipStream_t s) {
    return act == Dt::BF16 ? conv_fwd_varlen_t<bf16>(a, s) : conv_fwd_varlen_t<float>(a, s);
}

hipError_t launch_conv1d_update(const ConvUpdateArgs& a, Dt act, hipStream_t s) {
    return act == Dt::BF16 ? conv_update_t<bf16>(a, s) : conv_update_t<float>(a, s);
}

}  // namespace ssd
