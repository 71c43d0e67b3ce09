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

constexpr int kCopyThreads = 256;
constexpr int kCopyPerThread = 4;

// Four consecutive elements of T (8 bytes of bf16, 16 of fp32) in one load.
template <typename T> struct Quad;
template <> struct Quad<bf16> { typedef bf16x4 type; };
template <> struct Quad<float> { typedef f32x4 type; };

// The k-token SSM update.  Token j of request b is row b*k + j of x, B, C, dt and y, and entry
// b*k + j of the intermediate states.  A thread holds kGroupRows consecutive state rows of one head,
// each as two float4 (quads o and o + L of the row, for lane o of the row group's L = N/8 lanes),
// read once and kept in registers across the k tokens, so each token's loads of B, C, x and dt serve
// four rows.  The rows' y dot products are reduced together: a DPP reduce-scatter halves the rows a
// lane carries at each of the first two lane levels (the lane keeps two rows, then one, and adds its
// partner's partial sums of them), then plain DPP adds finish the L-lane tree.  The partner lanes at
// each level are those of group_sum_last (lane ^ 1, lane ^ 2, the mirror within 8 and within 16), so
// every row's sum is the same binary tree over the row's N/4 quads as in the single-token update
// (the two quads' trees are added last), and k = 1 reproduces its y bitwise.  Which rows a lane
// keeps is chosen so that the mirror partners of the last two levels hold the same row: f1 = bit 0 ^
// bit 2 of the lane (kept at lane ^ 2 and under both mirrors, flipped at lane ^ 1) picks the pair of
// rows, f2 = bit 1 ^ bit 2 (flipped at lane ^ 2 only) the row within it.
// XV: the row group's four x values are one vector load (x_row_stride a multiple of 4).
// REPLAY (the accept step by recomputation): request b applies its first n = clamp(accept_len[b],
// 0, k) tokens and writes the state back in place; no y, no intermediate states.
constexpr int kGroupRows = 4;
constexpr int kGroupThreads = 256;

template <typename T, typename TY, int N, bool REPLAY, bool XV>
__global__ __launch_bounds__(kGroupThreads) void state_update_rows_kernel(
    float* __restrict__ state, const T* __restrict__ x, int64_t xs, const T* __restrict__ Bm,
    const T* __restrict__ Cm, int64_t bcs, const T* __restrict__ dt, const float* __restrict__ A,
    const float* __restrict__ D, TY* __restrict__ y, float* __restrict__ inter, int64_t ngroups_rows, int k,
    int H, int P, int hpg, const int32_t* __restrict__ slot_idx, int64_t nslots, DtParams dtp,
    const int32_t* __restrict__ accept_len) {
    constexpr int QPR = N / 4;     // float4 per state row
    constexpr int L = QPR / 2;     // lanes per row group
    constexpr int R = kGroupRows;
    static_assert(L >= 2 && L <= 16 && R == 4, "2..16 lanes of four rows");
    typedef typename Quad<T>::type Q;
    constexpr int GPB = kGroupThreads / L;   // row groups per block
    const int o = static_cast<int>(threadIdx.x) % L;
    const int64_t rg0 = static_cast<int64_t>(blockIdx.x) * GPB;
    const int64_t rg = rg0 + static_cast<int>(threadIdx.x) / L;
    if (rg >= ngroups_rows) return;   // whole row groups only: no live lane reads a returned one
    const int64_t HP = static_cast<int64_t>(H) * P;
    // The block's rows almost always lie in one request (UNI): the request, its slot and every
    // token's row offsets are then block constants in scalar registers, and the lanes add 32-bit
    // offsets of their own.  Otherwise each thread divides its own row index.
    const int64_t ub = rg0 * R / HP;
    const int64_t last = (rg0 + GPB < ngroups_rows ? rg0 + GPB : ngroups_rows) * R - 1;
    auto body = [&](auto uni_tag) {
        constexpr bool UNI = decltype(uni_tag)::value;
        const int64_t b = UNI ? ub : rg * R / HP;
        const int rw = static_cast<int>(rg * R - b * HP);   // h * P + p0
        const int h = rw >> __builtin_ctz(static_cast<unsigned>(P));
        const int go = (h / hpg) * N + 4 * o;                // B/C column offset of the lane's first quad
        const int64_t sl = slot_idx ? seq_slot(slot_idx, b, nslots) : b;
        int nk = k;
        if constexpr (REPLAY) {
            const int n = accept_len[b];
            nk = n < 0 ? 0 : (n > k ? k : n);
            if (nk == 0 || sl < 0) return;   // nothing accepted, or padding
        }
        f32x4* sp = reinterpret_cast<f32x4*>(state) + sl * HP * QPR;
        const int so = rw * QPR + o;                      // float4 of row 0, quad o
        f32x4 s[R][2];
#pragma unroll
        for (int r = 0; r < R; ++r)
#pragma unroll
            for (int v = 0; v < 2; ++v)
                s[r][v] = sl >= 0 ? __builtin_nontemporal_load(sp + so + r * QPR + v * L) : f32x4{0.f, 0.f, 0.f, 0.f};
        const float Ah = A[h];
        const float Dh = D ? D[h] : 0.f;
        const float biash = dtp.bias ? dtp.bias[h] : 0.f;
        struct In {
            T dt;
            T x[R];
            Q b[2], c[2];
        };
        auto load_tok = [&](int j, In& in) {
            const int64_t tok = b * k + j;
            in.dt = (dt + tok * H)[h];
            const T* xt = x + tok * xs;
            if constexpr (XV) {
                const Q xq = *reinterpret_cast<const Q*>(xt + rw);
#pragma unroll
                for (int r = 0; r < R; ++r) in.x[r] = xq[r];
            } else {
#pragma unroll
                for (int r = 0; r < R; ++r) in.x[r] = xt[rw + r];
            }
            const T* bt = Bm + tok * bcs;
            const T* ct = Cm + tok * bcs;
#pragma unroll
            for (int v = 0; v < 2; ++v) {
                in.b[v] = *reinterpret_cast<const Q*>(bt + go + 4 * L * v);
                if constexpr (!REPLAY) in.c[v] = *reinterpret_cast<const Q*>(ct + go + 4 * L * v);
            }
        };
        const bool f1 = ((o ^ (o >> 2)) & 1) != 0;          // the pair of rows kept at the first level
        const bool f2 = (((o >> 1) ^ (o >> 2)) & 1) != 0;   // the row of that pair kept at the second
        auto step = [&](int j, const In& in) {
            // the dt prologue with the head's bias already loaded (same steps as dt_prologue)
            float dtv = static_cast<float>(in.dt);
            if (dtp.bias) dtv += biash;
            if (dtp.softplus) dtv = dtv > 20.f ? dtv : log1pf(expf(dtv));
            if (dtp.lo < dtp.hi) dtv = fminf(fmaxf(dtv, dtp.lo), dtp.hi);
            const float a = __expf(dtv * Ah);
            const int64_t trow = b * k + j;
            f32x4* it = reinterpret_cast<f32x4*>(inter) + trow * HP * QPR;
            float bq[2][4], cq[2][4];
#pragma unroll
            for (int v = 0; v < 2; ++v)
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    bq[v][e] = static_cast<float>(in.b[v][e]);
                    cq[v][e] = REPLAY ? 0.f : static_cast<float>(in.c[v][e]);
                }
            float part[R][2];
            float xv[R];
#pragma unroll
            for (int r = 0; r < R; ++r) {
                xv[r] = static_cast<float>(in.x[r]);
                const float dx = dtv * xv[r];
#pragma unroll
                for (int v = 0; v < 2; ++v) {
                    f32x4 u = s[r][v];
                    float pt = 0.f;
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        u[e] = fmaf(a, u[e], dx * bq[v][e]);
                        pt = fmaf(u[e], cq[v][e], pt);
                    }
                    s[r][v] = u;
                    if constexpr (!REPLAY) {
                        if (inter) it[so + r * QPR + v * L] = u;
                    }
                    part[r][v] = pt;
                }
            }
            if constexpr (!REPLAY) {
                TY* yr = y + trow * HP + rw;   // the request's token row: a block constant when UNI
                // level lane ^ 1: keep rows 2 f1 + i, add the partner's partial sums of them
                float t[2][2];
#pragma unroll
                for (int i = 0; i < 2; ++i)
#pragma unroll
                    for (int v = 0; v < 2; ++v) {
                        const float keep = f1 ? part[2 + i][v] : part[i][v];
                        const float send = f1 ? part[i][v] : part[2 + i][v];
                        t[i][v] = keep + dpp_f<0xB1, 0xF>(send);   // quad_perm [1,0,3,2]
                    }
                if constexpr (L == 2) {
                    // two lanes: each ends with two rows
                    if (o == 0 || o == 1) {
#pragma unroll
                        for (int i = 0; i < 2; ++i) {
                            const int r = 2 * (f1 ? 1 : 0) + i;
                            const float xr = f1 ? xv[2 + i] : xv[i];
                            yr[r] = static_cast<TY>((t[i][1] + t[i][0]) + (D ? Dh * xr : 0.f));
                        }
                    }
                } else {
                    // level lane ^ 2: keep row 2 f1 + f2
                    float w[2];
#pragma unroll
                    for (int v = 0; v < 2; ++v) {
                        const float keep = f2 ? t[1][v] : t[0][v];
                        const float send = f2 ? t[0][v] : t[1][v];
                        w[v] = keep + dpp_f<0x4E, 0xF>(send);   // quad_perm [2,3,0,1]
                    }
#pragma unroll
                    for (int v = 0; v < 2; ++v) {
                        if constexpr (L >= 8) w[v] += dpp_f<0x141, 0xF>(w[v]);    // row_half_mirror
                        if constexpr (L >= 16) w[v] += dpp_f<0x140, 0xF>(w[v]);   // row_mirror
                    }
                    if (o < 4) {   // lanes 0..3 hold rows 0, 2, 1, 3
                        const int r = 2 * (f1 ? 1 : 0) + (f2 ? 1 : 0);
                        const float xr = f1 ? (f2 ? xv[3] : xv[2]) : (f2 ? xv[1] : xv[0]);
                        yr[r] = static_cast<TY>((w[1] + w[0]) + (D ? Dh * xr : 0.f));
                    }
                }
            }
        };
        // the inputs of token j + 1 are loaded while token j is computed, into the other of two register
        // sets (loading all k tokens' inputs with the state measured the same)
        In ta, tb;
        load_tok(0, ta);
        for (int j = 0; j < nk; j += 2) {
            load_tok(j + 1 < nk ? j + 1 : j, tb);   // past the last token: re-reads its rows
            step(j, ta);
            if (j + 1 >= nk) break;
            load_tok(j + 2 < nk ? j + 2 : j + 1, ta);
            step(j + 1, tb);
        }
        if constexpr (REPLAY) {
#pragma unroll
            for (int r = 0; r < R; ++r)
#pragma unroll
                for (int v = 0; v < 2; ++v) __builtin_nontemporal_store(s[r][v], sp + so + r * QPR + v * L);
        }
    };
    if (last / HP == ub) body(std::true_type{});
    else body(std::false_type{});
}

template <typename T, typename TY, int N, bool REPLAY, bool XV>
static void rows_launch(const UpdateArgs& a, float* inter, hipStream_t s) {
    const int64_t nrg = a.batch * a.nheads * static_cast<int64_t>(a.head_dim) / kGroupRows;
    constexpr int per_block = kGroupThreads / (N / 8);
    const int64_t blocks = (nrg + per_block - 1) / per_block;
    hipLaunchKernelGGL((state_update_rows_kernel<T, TY, N, REPLAY, XV>), dim3(static_cast<uint32_t>(blocks)),
                       dim3(kGroupThreads), 0, s, a.state, static_cast<const T*>(a.x), a.x_row_stride,
                       static_cast<const T*>(a.B), static_cast<const T*>(a.C), a.bc_row_stride,
                       static_cast<const T*>(a.dt), a.A, a.D, static_cast<TY*>(a.y), inter, nrg, a.k, a.nheads,
                       a.head_dim, a.nheads / a.ngroups, a.slot_idx, a.nslots, a.dtp, a.accept_len);
}

// y alone for 2 <= k <= kDualTokens tokens, in the chunk (dual) form of the recurrence over the k
// tokens ("Mamba 与 Nemotron 系列模型深度调研", Mamba 架构: the structured semiseparable form the
// chunked scan also uses): with a_t = exp(dt_t A), dx_t = dt_t x_t, alpha_t = a_1 ... a_t and
// beta_{t,u} = a_{u+1} ... a_t,
//     y_t = alpha_t (C_t . s_0) + sum_{u <= t} beta_{t,u} dx_u (C_t . B_u) + D x_t,
// the same value as C_t . s_t after t sequential updates, summed in another order.  The state is
// read and never updated, so each token costs one FMA per state element (C_t . s_0) instead of
// three; the C_t . B_u are per group and shared by the head's rows.  Rows, lanes and the
// reduce-scatter of the C_t . s_0 partial sums are those of state_update_rows_kernel.
constexpr int kDualTokens = 4;
constexpr int kDualRows = 8;   // state rows per thread

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

// partial dot product of a thread's 8 B and C values (its two quads); bf16 pairs in one instruction
template <typename T>
__device__ __forceinline__ float quad_pair_dot(const typename Quad<T>::type (&c)[2],
                                               const typename Quad<T>::type (&b)[2]) {
    if constexpr (sizeof(T) == 2) {
        float acc = 0.f;
#pragma unroll
        for (int v = 0; v < 2; ++v) {
            const bf16x4 cv = c[v], bv = b[v];
            acc = __builtin_amdgcn_fdot2_f32_bf16(bf16x2{cv[0], cv[1]}, bf16x2{bv[0], bv[1]}, acc, false);
            acc = __builtin_amdgcn_fdot2_f32_bf16(bf16x2{cv[2], cv[3]}, bf16x2{bv[2], bv[3]}, acc, false);
        }
        return acc;
    } else {
        float acc = 0.f;
#pragma unroll
        for (int v = 0; v < 2; ++v)
#pragma unroll
            for (int e = 0; e < 4; ++e) acc = fmaf(c[v][e], b[v][e], acc);
        return acc;
    }
}

// Reduce-scatter of R partial sums (rows) over a row group's L lanes: at lane levels 1, 2, 3 (partners
// lane ^ 1, lane ^ 2 and the mirror within 8) a lane that still carries more than one row keeps half of
// them, chosen by f1 = bit 0 ^ bit 2, f2 = bit 1 ^ bit 2, f3 = bit 2 ^ bit 3 of the lane, and adds its
// partner's partial sums of those; each f is unchanged under the later levels' partners (lane ^ 2, the
// two mirrors) and flips under its own level's, so partners always hold the same rows.  The remaining
// levels add plain.  Returns the lane's NR = max(1, R / L) rows' sums in v[0 .. NR); they are rows
// row_base(o) + i.
template <int R, int L>
struct RowScatter {
    static constexpr int NR = R / L > 1 ? R / L : 1;
    static __device__ __forceinline__ int row_base(int o) {
        int base = 0, cnt = R;
#pragma unroll
        for (int lvl = 1; lvl <= 3; ++lvl) {
            if ((1 << lvl) > L || cnt == 1) break;
            cnt >>= 1;
            if (bit(o, lvl)) base += cnt;
        }
        return base;
    }
    static __device__ __forceinline__ bool bit(int o, int lvl) {   // f1, f2, f3
        const int b0 = o & 1, b1 = (o >> 1) & 1, b2 = (o >> 2) & 1, b3 = (o >> 3) & 1;
        return (lvl == 1 ? b0 ^ b2 : lvl == 2 ? b1 ^ b2 : b2 ^ b3) != 0;
    }
    template <int CTRL>
    static __device__ __forceinline__ void level(float (&v)[R], int& cnt, bool keep_hi) {
        if (cnt > 1) {
            const int h = cnt >> 1;
#pragma unroll
            for (int i = 0; i < R / 2; ++i) {
                if (i < h) {
                    const float keep = keep_hi ? v[h + i] : v[i];
                    const float send = keep_hi ? v[i] : v[h + i];
                    v[i] = keep + dpp_f<CTRL, 0xF>(send);
                }
            }
            cnt = h;
        } else {
            v[0] += dpp_f<CTRL, 0xF>(v[0]);
        }
    }
    static __device__ __forceinline__ void run(float (&v)[R], int o) {
        int cnt = R;
        if constexpr (L >= 2) level<0xB1>(v, cnt, bit(o, 1));     // quad_perm [1,0,3,2]
        if constexpr (L >= 4) level<0x4E>(v, cnt, bit(o, 2));     // quad_perm [2,3,0,1]
        if constexpr (L >= 8) level<0x141>(v, cnt, bit(o, 3));    // row_half_mirror
        if constexpr (L >= 16) level<0x140>(v, cnt, false);       // row_mirror
    }
};

template <typename T, typename TY, int N, int R, bool XV>
__global__ __launch_bounds__(kGroupThreads) void state_multi_y_kernel(
    const float* __restrict__ state, const T* __restrict__ x, int64_t xs, const T* __restrict__ Bm,
    const T* __restrict__ Cm, int64_t bcs, const T* __restrict__ dt, const float* __restrict__ A,
    const float* __restrict__ D, TY* __restrict__ y, int64_t ngroups_rows, int k, int H, int P, int hpg,
    const int32_t* __restrict__ slot_idx, int64_t nslots, DtParams dtp) {
    constexpr int QPR = N / 4;     // float4 per state row
    constexpr int L = QPR / 2;     // lanes per row group
    constexpr int KM = kDualTokens;
    typedef RowScatter<4, L> RS;   // the rows are reduced four at a time
    constexpr int NR = RS::NR;     // rows of a four a lane ends with
    constexpr int GPB = kGroupThreads / L;   // row groups per block
    static_assert(L >= 2 && L <= 16 && (R == 4 || R == 8), "2..16 lanes of four or eight rows");
    typedef typename Quad<T>::type Q;
    const int o = static_cast<int>(threadIdx.x) % L;
    const int64_t rg0 = static_cast<int64_t>(blockIdx.x) * GPB;
    const int64_t rg = rg0 + static_cast<int>(threadIdx.x) / L;
    if (rg >= ngroups_rows) return;   // whole row groups only: no live lane reads a returned one
    const int64_t HP = static_cast<int64_t>(H) * P;
    const f32x4* st4 = reinterpret_cast<const f32x4*>(state);
    const float* Af = A;
    // The block's rows almost always lie in one request (UNI): the request, its slot and every
    // token's row offsets are then block constants in scalar registers, and the lanes add 32-bit
    // offsets of their own.  Otherwise each thread divides its own row index.
    const int64_t ub = rg0 * R / HP;
    const int64_t last = (rg0 + GPB < ngroups_rows ? rg0 + GPB : ngroups_rows) * R - 1;
    auto body = [&](auto uni_tag) {
        constexpr bool UNI = decltype(uni_tag)::value;
        const int64_t b = UNI ? ub : rg * R / HP;
        const int rw = static_cast<int>(rg * R - b * HP);   // h * P + p0
        const int h = rw >> __builtin_ctz(static_cast<unsigned>(P));
        const int go = (h / hpg) * N + 4 * o;                // B/C column offset of the lane's first quad
        const int64_t sl = slot_idx ? seq_slot(slot_idx, b, nslots) : b;
        const float Ah = Af[h];
        const float Dh = D ? D[h] : 0.f;
        const float biash = dtp.bias ? dtp.bias[h] : 0.f;
        // every token's inputs, loaded with the state (tokens past k re-read the last one's rows)
        T dtr[KM];
        T xr[KM][R];
        Q bq[KM][2], cq[KM][2];
#pragma unroll
        for (int t = 0; t < KM; ++t) {
            const int64_t tok = b * k + (t < k ? t : k - 1);
            dtr[t] = (dt + tok * H)[h];
            const T* xt = x + tok * xs;
#pragma unroll
            for (int r4 = 0; r4 < R; r4 += 4) {
                if constexpr (XV) {
                    const Q xq = *reinterpret_cast<const Q*>(xt + rw + r4);
#pragma unroll
                    for (int r = 0; r < 4; ++r) xr[t][r4 + r] = xq[r];
                } else {
#pragma unroll
                    for (int r = 0; r < 4; ++r) xr[t][r4 + r] = xt[rw + r4 + r];
                }
            }
            const T* bt = Bm + tok * bcs;
            const T* ct = Cm + tok * bcs;
#pragma unroll
            for (int v = 0; v < 2; ++v) {
                bq[t][v] = *reinterpret_cast<const Q*>(bt + go + 4 * L * v);
                cq[t][v] = *reinterpret_cast<const Q*>(ct + go + 4 * L * v);
            }
        }
        // then the state, four rows at a time: the first four rows' tokens are computed while the
        // next four rows are still in flight (the loads complete in issue order).  The loads are
        // unconditional, so that the compiler's wait counts stay exact: a padding request (no slot)
        // reads slot 0 and drops it from y below.
        __builtin_amdgcn_sched_barrier(0);
        const bool pad = sl < 0;
        const f32x4* sp = st4 + (pad ? 0 : sl) * HP * QPR;
        const int so = rw * QPR + o;
        f32x4 s[R][2];
#pragma unroll
        for (int r = 0; r < R; ++r) {
#pragma unroll
            for (int v = 0; v < 2; ++v) s[r][v] = __builtin_nontemporal_load(sp + so + r * QPR + v * L);
            if (r % 4 == 3) __builtin_amdgcn_sched_barrier(0);
        }
        float a[KM], dtv[KM];
#pragma unroll
        for (int t = 0; t < KM; ++t) {
            // the dt prologue with the head's bias already loaded (same steps as dt_prologue)
            float d = static_cast<float>(dtr[t]);
            if (dtp.bias) d += biash;
            if (dtp.softplus) d = d > 20.f ? d : log1pf(expf(d));
            if (dtp.lo < dtp.hi) d = fminf(fmaxf(d, dtp.lo), dtp.hi);
            dtv[t] = d;
            a[t] = __expf(d * Ah);
        }
        const int wr = RS::row_base(o);   // the lane's first row within a group of four
        float cb[KM][KM];                 // C_t . B_u over the group's N columns, u <= t
#pragma unroll
        for (int hh = 0; hh < R / 4; ++hh) {
            __builtin_amdgcn_sched_barrier(0);   // keep each half's work after the previous half's
            float dxl[KM][NR], xl[KM][NR];
#pragma unroll
            for (int t = 0; t < KM; ++t)
#pragma unroll
                for (int i = 0; i < NR; ++i) {
                    // x of the lane's row 4 hh + wr + i, selected from the four loaded values
                    float xv = 0.f;
#pragma unroll
                    for (int r = 0; r < 4; ++r) xv = (r == wr + i) ? static_cast<float>(xr[t][4 * hh + r]) : xv;
                    xl[t][i] = xv;
                    dxl[t][i] = dtv[t] * xv;
                }
            float alpha = 1.f;
            float beta[KM];
#pragma unroll
            for (int t = 0; t < KM; ++t) {
                if (t >= k) break;
                alpha *= a[t];
#pragma unroll
                for (int u = 0; u < t; ++u) beta[u] *= a[t];
                beta[t] = 1.f;
                // C_t . s_0, partial over the lane's 8 columns, for the four rows
                float cf[2][4];
#pragma unroll
                for (int v = 0; v < 2; ++v)
#pragma unroll
                    for (int e = 0; e < 4; ++e) cf[v][e] = static_cast<float>(cq[t][v][e]);
                float part[4];
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    float acc = 0.f;
#pragma unroll
                    for (int v = 0; v < 2; ++v)
#pragma unroll
                        for (int e = 0; e < 4; ++e) acc = fmaf(s[4 * hh + r][v][e], cf[v][e], acc);
                    part[r] = acc;
                }
                RS::run(part, o);
                if (hh == 0) {
#pragma unroll
                    for (int u = 0; u <= t; ++u) cb[t][u] = group_sum_last<L>(quad_pair_dot<T>(cq[t], bq[u]));
                }
                if (o < (L < 4 ? L : 4)) {   // these lanes hold distinct rows
                    TY* yt = y + (b * k + t) * HP + rw + 4 * hh;
#pragma unroll
                    for (int i = 0; i < NR; ++i) {
                        float acc = pad ? 0.f : alpha * part[i];
#pragma unroll
                        for (int u = 0; u <= t; ++u) acc = fmaf(beta[u] * dxl[u][i], cb[t][u], acc);
                        yt[wr + i] = static_cast<TY>(acc + (D ? Dh * xl[t][i] : 0.f));
                    }
                }
            }
        }
    };
    if (last / HP == ub) body(std::true_type{});
    else body(std::false_type{});
}

template <typename T, typename TY, int N, int R, bool XV>
static void multi_y_launch(const UpdateArgs& a, hipStream_t s) {
    const int64_t nrg = a.batch * a.nheads * static_cast<int64_t>(a.head_dim) / R;
    constexpr int per_block = kGroupThreads / (N / 8);
    const int64_t blocks = (nrg + per_block - 1) / per_block;
    hipLaunchKernelGGL((state_multi_y_kernel<T, TY, N, R, XV>), dim3(static_cast<uint32_t>(blocks)),
                       dim3(kGroupThreads), 0, s, a.state, static_cast<const T*>(a.x), a.x_row_stride,
                       static_cast<const T*>(a.B), static_cast<const T*>(a.C), a.bc_row_stride,
                       static_cast<const T*>(a.dt), a.A, a.D, static_cast<TY*>(a.y), nrg, a.k, a.nheads,
                       a.head_dim, a.nheads / a.ngroups, a.slot_idx, a.nslots, a.dtp);
}

template <typename T, typename TY, int N>
static hipError_t multi_launch(const UpdateArgs& a, hipStream_t s) {
    if (a.batch == 0 || a.k == 0) return hipSuccess;
    const bool xv = a.x_row_stride % kGroupRows == 0;
    if (!a.accept_len && !a.inter && a.state && a.k >= 2 && a.k <= kDualTokens) {   // y alone, in the dual form
        if (xv) multi_y_launch<T, TY, N, kDualRows, true>(a, s);
        else multi_y_launch<T, TY, N, kDualRows, false>(a, s);
        return hipGetLastError();
    }
    if (a.accept_len) {
        if (xv) rows_launch<T, TY, N, true, true>(a, nullptr, s);
        else rows_launch<T, TY, N, true, false>(a, nullptr, s);
    } else {
        if (xv) rows_launch<T, TY, N, false, true>(a, a.inter, s);
        else rows_launch<T, TY, N, false, false>(a, a.inter, s);
    }
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
