// SSD chunked scan for prefill on bf16 MFMA (gfx950): head_dim 64, d_state 128,
// chunk 128 -- the Ultra-family Mamba layer.
//
// Method (the structured-semiseparable / chunked form of the Mamba-2 scan:
// "Mamba 与 Nemotron 系列模型深度调研", Mamba 架构; the 128-token chunked scan
// that returns the final state in the modeling_nemotron_h.py walk-through,
// "Prefill 阶段").  Per chunk of Q tokens, with cs the inclusive prefix sum of
// dt*A in base-2 units (decays are exp2 of differences):
//   M[i][j] = (C_i . B_j) * exp2(cs_i - cs_j) * dt_j   (j <= i), + D on the diagonal
//   y_i     = sum_j M[i][j] x_j  +  exp2(cs_i) * (C_i . H)
//   H       = exp2(cs_last) * H + sum_j exp2(cs_last - cs_j) dt_j  x_j (x) B_j
// which is the token recurrence re-associated exactly.
//
// Mapping.  One persistent workgroup of 4 waves per (batch, head) walks the
// chunks in order; the fp32 state H lives in registers of the waves that own
// its tiles and never goes to HBM between chunks.  All products are
// v_mfma_f32_32x32x16_bf16 (a single wave issues these at full rate when it
// keeps >= 4 independent accumulators in flight).  Wave w owns token tile w
// (32 tokens): it computes C.B^T for the tiles j <= i of its rows, turns them
// into M in registers, and uses the accumulators directly as the B operand of
// y^T = X^T M^T (accumulator rows are the MFMA's k, so k is permuted the same
// way on both operands).  It then adds exp2(cs_i) C.H (H read from LDS) and
// writes y for its 32 tokens.  The chunk-state tiles H[p-tile][n-tile] are
// spread over the waves with the least causal work (wave 0: p-tile 0 x all four
// n-tiles, waves 1 and 2: p-tile 1 x two n-tiles, wave 3: none), which balances
// the MFMA count at <= 112 per wave and chunk; the decay weight of the chunk
// state is applied to the x operand, once per wave and p-tile.
//
// Precision.  x, B and C arrive in bf16 and are exact operands.  Operands
// computed in fp32 (M, H and the decay-weighted B) are split into bf16 hi + lo
// and issued as two MFMAs, keeping ~16 significant bits.  Decays inside a
// chunk are exp2 of differences of the prefix sums (exact exp2(0) = 1 on the
// diagonal); off-diagonal 32x32 blocks use the factorisation
// exp2(cs_i - cs_e) * exp2(cs_e - cs_j) about the block's last token e, both
// factors <= 1, so nothing overflows.
//
// Data movement.  B and x tiles are staged row-major in LDS, double-buffered:
// the next chunk's tiles stream in with direct global->LDS loads
// (global_load_lds_dwordx4, no registers) while the current chunk computes.
// Only the wave that owns a token tile reads its rows of C, so C goes straight
// from global memory into that wave's MFMA operand registers (prefetched one
// chunk ahead).  Operands that contract over tokens are read with
// ds_read_b64_tr_b16 (LDS transpose read), so no transposed copies are kept.
// Per-token decay vectors are built once per chunk by the wave with the fewest
// MFMAs.  Workgroups are numbered so that the heads sharing a B/C group sit on
// one XCD (its L2 then serves their common B and C).
#include "ssd_device.h"
#include "ssd_kernels.h"

namespace ssd {
namespace scan32 {

constexpr int Q = 128;    // tokens per chunk
constexpr int P = 64;     // head_dim
constexpr int NS = 128;   // d_state
constexpr int BS = 144;   // LDS row stride (bf16) of the [.][128] tiles: 72 dwords, 8-bank shift per row
constexpr int XS = 80;    // LDS row stride (bf16) of the x tile: 40 dwords
constexpr int kThreads = 256;
constexpr float kLog2e = 1.4426950408889634f;
constexpr int kBInstr = Q * BS * 2 / 1024;   // 1-KB direct-load instructions per B tile (36)
constexpr int kXInstr = Q * XS * 2 / 1024;   // per x tile (20)

typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef __attribute__((address_space(3))) bf16 lds_bf16;
typedef __attribute__((address_space(3))) bf16x4 lds_bf16x4;

struct Vec {            // per-token quantities of one chunk
    float cs[Q];        // inclusive prefix sum of dt*A*log2(e)
    float dt[Q];
    float fM[Q];        // exp2(cs_e - cs_j) * dt_j, e = last token of j's 32-token tile
    float wS[Q];        // exp2(cs_last - cs_j) * dt_j for real tokens, 0 for padding
    float eY[Q];        // exp2(cs_i)
    float csE[4];       // cs at the end of each 32-token tile
    float pad[4];
};

struct Smem {
    bf16 B[2][Q][BS];   // B[j][n], double-buffered over chunks
    bf16 X[2][Q][XS];   // x[j][p], double-buffered over chunks
    bf16 Hhi[P][BS];    // H[p][n], high and low bf16 parts
    bf16 Hlo[P][BS];
    Vec vec[2];         // the current chunk's and the next one's
};
static_assert(sizeof(Smem) <= 160 * 1024, "LDS budget");
static_assert(Q * BS * 2 % 1024 == 0 && Q * XS * 2 % 1024 == 0, "tiles are whole 1-KB load blocks");

__device__ __forceinline__ f32x16 mfma32(bf16x8 a, bf16x8 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ float fexp2(float v) { return __builtin_amdgcn_exp2f(v); }
__device__ __forceinline__ f32x16 zero16() {
    f32x16 z;
#pragma unroll
    for (int i = 0; i < 16; ++i) z[i] = 0.f;
    return z;
}
__device__ __forceinline__ bf16 bhi(float v) { return static_cast<bf16>(v); }
__device__ __forceinline__ bf16 blo(float v, bf16 hi) { return static_cast<bf16>(v - static_cast<float>(hi)); }

// MFMA operand whose k runs over tokens, read from a row-major [token][col] LDS
// tile with two transpose reads.  Lane (c32 = lane%32, hf = lane/32) receives
// column col_base + c32 at tokens j0 + 4hf + {0..3} (slots 0..3) and
// j0 + 8 + 4hf + {0..3} (slots 4..7) -- the row order of a 32x32 accumulator
// used as an operand.  Within each 16-lane group, lane m supplies the address
// of row (first + m/4), columns col0 + 4(m%4) .. +3.
__device__ __forceinline__ bf16x8 tr_frag(const bf16* mat, int rs, int j0, int col_base, int lane) {
    const int m = lane & 15;
    const int col = col_base + 16 * ((lane >> 4) & 1) + 4 * (m & 3);
    const int row = j0 + 4 * (lane >> 5) + (m >> 2);
    const bf16* p0 = mat + row * rs + col;
    const bf16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)(lds_bf16*)p0);
    const bf16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)(lds_bf16*)(p0 + 8 * rs));
    return bf16x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
}

struct Ctx {
    const bf16* xg; const bf16* Bg; const bf16* Cg; const bf16* dtg;
    int64_t xs, bcs, b, L;
    int H, h, grp;
};

// Direct global->LDS copy of one chunk's row-major tile into a padded LDS tile.
// The tile is a sequence of 1-KB blocks; block k is written by wave k % 4 with
// lane l storing LDS bytes [1024k + 16l, +16).  A lane whose bytes fall in a row's
// padding, or in a row past the sequence end, re-reads a real row instead (the
// padding is never read and rows past the end only meet zero weights).
template <int RS, int DC, int NBLK>
__device__ __forceinline__ void copy_tile(bf16* lds_tile, const bf16* g, int64_t row_stride, int64_t first_row,
                                          int valid, int col_off, int W, int lane) {
    constexpr int RB = RS * 2;            // LDS row bytes
#pragma unroll
    for (int m = 0; m < (NBLK + 3) / 4; ++m) {
        const int k = W + 4 * m;
        if (k < NBLK) {
            const int o = 1024 * k + 16 * lane;
            const int row = o / RB;
            const int cb = o - row * RB;
            const int r = row < valid ? row : valid - 1;
            const int col = cb < 2 * DC ? cb / 2 : 0;    // DC real columns, the rest is padding
            const bf16* src = g + (first_row + r) * row_stride + col_off + col;
            __builtin_amdgcn_global_load_lds((__attribute__((address_space(1))) void*)src,
                                             (__attribute__((address_space(3))) void*)((unsigned char*)lds_tile + 1024 * k),
                                             16, 0, 0);
        }
    }
}

// Per-token vectors of a chunk from its dt (two tokens per lane of one wave).
__device__ __forceinline__ void build_vec(Vec& v, bf16 r0, bf16 r1, float A2, int valid, int lane) {
    const float d0 = 2 * lane < valid ? static_cast<float>(r0) : 0.f;
    const float d1 = 2 * lane + 1 < valid ? static_cast<float>(r1) : 0.f;
    const float a0 = d0 * A2, a1 = d1 * A2;
    float s = a0 + a1;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
        const float u = __shfl_up(s, off, 64);
        if (lane >= off) s += u;
    }
    const float c1 = s, c0 = s - a1;  // inclusive sums at tokens 2*lane+1 and 2*lane
    const int last = valid - 1;
    const float cl0 = __shfl(c0, last >> 1, 64), cl1 = __shfl(c1, last >> 1, 64);
    const float csl = (last & 1) ? cl1 : cl0;
    const float ce = __shfl(c1, (lane & ~15) | 15, 64);   // end of this lane's 32-token tile
    const int j0 = 2 * lane, j1 = 2 * lane + 1;
    v.cs[j0] = c0;
    v.cs[j1] = c1;
    v.dt[j0] = d0;
    v.dt[j1] = d1;
    v.fM[j0] = fexp2(ce - c0) * d0;
    v.fM[j1] = fexp2(ce - c1) * d1;
    v.wS[j0] = j0 < valid ? fexp2(csl - c0) * d0 : 0.f;
    v.wS[j1] = j1 < valid ? fexp2(csl - c1) * d1 : 0.f;
    v.eY[j0] = fexp2(c0);
    v.eY[j1] = fexp2(c1);
    if ((lane & 15) == 15) v.csE[lane >> 4] = c1;
}

// Owned chunk-state tiles of wave W: tile k is H[p-tile pt][n-tile nt(k)].
template <int W> struct Own {
    static constexpr int n = W == 0 ? 4 : (W == 3 ? 0 : 2);
    static constexpr int pt = W == 0 ? 0 : 1;
    static constexpr int nt(int k) { return W == 2 ? 2 + k : k; }
};

template <int W, typename TY>
__device__ void run_wave(Smem& sm, const ScanArgs& a, const Ctx& cx, int lane) {
    constexpr int IT = W;                       // this wave's token tile
    constexpr int NO = Own<W>::n;
    constexpr int NOA = NO > 0 ? NO : 1;
    constexpr int PT = Own<W>::pt;
    const int c32 = lane & 31, hf = lane >> 5;
    const int64_t L = cx.L;
    const float A2 = a.A[cx.h] * kLog2e;
    const float Dh = a.D ? a.D[cx.h] : 0.f;
    TY* yg = static_cast<TY*>(a.y);
    const int64_t sbase = (cx.b * cx.H + cx.h) * static_cast<int64_t>(P) * NS;
    const int64_t nchunks = (L + Q - 1) / Q;
    const int64_t row0 = cx.b * L;                                  // first token row of the sequence
    const int bc_col = cx.grp * NS, x_col = cx.h * P;
    const bf16* crow = cx.Cg + bc_col + 8 * hf;                     // + row * bcs + 16 ks
    const int i = 32 * IT + c32;                                    // this lane's token in the chunk

    auto load_c = [&](bf16x8 (&cf)[8], int64_t t0, int valid) {
        const int r = i < valid ? i : valid - 1;
        const bf16* src = crow + (row0 + t0 + r) * cx.bcs;
#pragma unroll
        for (int ks = 0; ks < 8; ++ks) cf[ks] = *reinterpret_cast<const bf16x8*>(src + 16 * ks);
    };
    // dt of tokens 2*lane and 2*lane+1, read unconditionally from in-range rows; tokens past
    // the sequence end are zeroed later, in build_vec, so nothing waits on these loads early
    auto load_dt = [&](bf16& d0, bf16& d1, int64_t t0, int valid) {
        const int r0 = 2 * lane < valid ? 2 * lane : valid - 1;
        const int r1 = 2 * lane + 1 < valid ? 2 * lane + 1 : valid - 1;
        d0 = cx.dtg[(row0 + t0 + r0) * cx.H + cx.h];
        d1 = cx.dtg[(row0 + t0 + r1) * cx.H + cx.h];
    };

    // ---- owned state tiles: Hs[k][4j + r] = H[p = 32PT + c32][n = 32nt + 8j + 4hf + r]
    f32x16 Hs[NOA];
#pragma unroll
    for (int k = 0; k < NO; ++k) {
        const int p = 32 * PT + c32;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int n = 32 * Own<W>::nt(k) + 8 * j + 4 * hf;
            f32x4 v = {0.f, 0.f, 0.f, 0.f};
            if (a.init_state) v = *reinterpret_cast<const f32x4*>(a.init_state + sbase + p * NS + n);
#pragma unroll
            for (int r = 0; r < 4; ++r) Hs[k][4 * j + r] = v[r];
        }
    }
    auto write_h = [&]() {
#pragma unroll
        for (int k = 0; k < NO; ++k) {
            const int p = 32 * PT + c32;
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int n = 32 * Own<W>::nt(k) + 8 * j + 4 * hf;
                bf16x4 hh, hl;
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    hh[r] = bhi(Hs[k][4 * j + r]);
                    hl[r] = blo(Hs[k][4 * j + r], hh[r]);
                }
                *reinterpret_cast<bf16x4*>(&sm.Hhi[p][n]) = hh;
                *reinterpret_cast<bf16x4*>(&sm.Hlo[p][n]) = hl;
            }
        }
    };

    bf16x8 cf[8];
    if (nchunks > 0) {
        const int valid0 = static_cast<int>(L < Q ? L : Q);
        copy_tile<BS, NS, kBInstr>(&sm.B[0][0][0], cx.Bg, cx.bcs, row0, valid0, bc_col, W, lane);
        copy_tile<XS, P, kXInstr>(&sm.X[0][0][0], cx.xg, cx.xs, row0, valid0, x_col, W, lane);
        load_c(cf, 0, valid0);
        if (W == 3) {
            bf16 d0, d1;
            load_dt(d0, d1, 0, valid0);
            build_vec(sm.vec[0], d0, d1, A2, valid0, lane);
        }
        write_h();
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    }
    __syncthreads();

    for (int64_t c = 0; c < nchunks; ++c) {
        const int64_t t0 = c * Q;
        const int valid = static_cast<int>((L - t0) < Q ? (L - t0) : Q);
        const bool has_next = c + 1 < nchunks;
        const int valid1 = has_next ? static_cast<int>((L - t0 - Q) < Q ? (L - t0 - Q) : Q) : 0;
        const int cur = static_cast<int>(c & 1), nxt = cur ^ 1;
        const Vec& v = sm.vec[cur];
        const bf16* sB = &sm.B[cur][0][0];
        const bf16* sX = &sm.X[cur][0][0];

        // ---- stream the next chunk in: B and x straight to LDS, C rows and dt to registers
        bf16x8 cfn[8];
        bf16 nd0 = bf16(0.f), nd1 = bf16(0.f);
        if (has_next) {
            if (W == 3) load_dt(nd0, nd1, t0 + Q, valid1);
            copy_tile<BS, NS, kBInstr>(&sm.B[nxt][0][0], cx.Bg, cx.bcs, row0 + t0 + Q, valid1, bc_col, W, lane);
            copy_tile<XS, P, kXInstr>(&sm.X[nxt][0][0], cx.xg, cx.xs, row0 + t0 + Q, valid1, x_col, W, lane);
            load_c(cfn, t0 + Q, valid1);
        }

        // ---- carried state: yo^T[p][i] = sum_n H[p][n] C[i][n]  (hi and lo of H, one chain per p tile)
        f32x16 yo[2] = {zero16(), zero16()};
#pragma unroll
        for (int ks = 0; ks < 8; ++ks)
#pragma unroll
            for (int pt = 0; pt < 2; ++pt) {
                const bf16x8 hh = *reinterpret_cast<const bf16x8*>(&sm.Hhi[32 * pt + c32][16 * ks + 8 * hf]);
                const bf16x8 hl = *reinterpret_cast<const bf16x8*>(&sm.Hlo[32 * pt + c32][16 * ks + 8 * hf]);
                yo[pt] = mfma32(hh, cf[ks], yo[pt]);
                yo[pt] = mfma32(hl, cf[ks], yo[pt]);
            }

        // ---- C.B^T tiles (jt, IT), jt <= IT: acc rows = tokens j, cols = tokens i
        constexpr int KP = IT == 0 ? 2 : 1;  // independent partial sums per tile
        f32x16 cb[IT + 1][KP];
#pragma unroll
        for (int jt = 0; jt <= IT; ++jt)
#pragma unroll
            for (int kp = 0; kp < KP; ++kp) cb[jt][kp] = zero16();
#pragma unroll
        for (int ks = 0; ks < 8; ++ks) {
#pragma unroll
            for (int jt = 0; jt <= IT; ++jt) {
                const bf16x8 bf = *reinterpret_cast<const bf16x8*>(sB + (32 * jt + c32) * BS + 16 * ks + 8 * hf);
                cb[jt][ks % KP] = mfma32(bf, cf[ks], cb[jt][ks % KP]);
            }
        }

        // ---- per j tile: M = C.B^T * decay * dt (+ D on the diagonal) as bf16 hi/lo,
        //      then y^T[p][i] += sum_j X^T[p][j] M^T[j][i]
        const float csi = v.cs[i];
        f32x16 yd[2] = {zero16(), zero16()};
#pragma unroll
        for (int jt = 0; jt <= IT; ++jt) {
            f32x16 m = cb[jt][0];
#pragma unroll
            for (int kp = 1; kp < KP; ++kp) m += cb[jt][kp];
            if (jt < IT) {
                const float ai = fexp2(csi - v.csE[jt]);
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const f32x4 f = *reinterpret_cast<const f32x4*>(&v.fM[32 * jt + 8 * j + 4 * hf]);
#pragma unroll
                    for (int r = 0; r < 4; ++r) m[4 * j + r] *= f[r] * ai;
                }
            } else {
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const f32x4 cj = *reinterpret_cast<const f32x4*>(&v.cs[32 * jt + 8 * j + 4 * hf]);
                    const f32x4 dj = *reinterpret_cast<const f32x4*>(&v.dt[32 * jt + 8 * j + 4 * hf]);
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        const int jj = 32 * jt + 8 * j + 4 * hf + r;
                        float e = m[4 * j + r] * fexp2(csi - cj[r]) * dj[r];
                        if (jj == i) e += Dh;
                        m[4 * j + r] = jj <= i ? e : 0.f;
                    }
                }
            }
#pragma unroll
            for (int q = 0; q < 2; ++q) {
                bf16x8 mh, ml;
#pragma unroll
                for (int s = 0; s < 8; ++s) {
                    mh[s] = bhi(m[8 * q + s]);
                    ml[s] = blo(m[8 * q + s], mh[s]);
                }
#pragma unroll
                for (int pt = 0; pt < 2; ++pt) {
                    const bf16x8 xf = tr_frag(sX, XS, 32 * jt + 16 * q, 32 * pt, lane);
                    yd[pt] = mfma32(xf, mh, yd[pt]);
                    yd[pt] = mfma32(xf, ml, yd[pt]);
                }
            }
        }

        // ---- owned state tiles: H^T[n][p] = exp2(cs_last) H^T + sum_j B^T[n][j] (w_j x_j)[p]
        if constexpr (NO > 0) {
            const float alpha = fexp2(v.cs[valid - 1]);
#pragma unroll
            for (int k = 0; k < NO; ++k) Hs[k] *= alpha;
#pragma unroll
            for (int jt = 0; jt < 4; ++jt)
#pragma unroll
                for (int q = 0; q < 2; ++q) {
                    const int j0 = 32 * jt + 16 * q;
                    const f32x4 w0 = *reinterpret_cast<const f32x4*>(&v.wS[j0 + 4 * hf]);
                    const f32x4 w1 = *reinterpret_cast<const f32x4*>(&v.wS[j0 + 8 + 4 * hf]);
                    const bf16x8 xf = tr_frag(sX, XS, j0, 32 * PT, lane);
                    bf16x8 xh, xl;
#pragma unroll
                    for (int s = 0; s < 8; ++s) {
                        const float e = static_cast<float>(xf[s]) * (s < 4 ? w0[s] : w1[s - 4]);
                        xh[s] = bhi(e);
                        xl[s] = blo(e, xh[s]);
                    }
#pragma unroll
                    for (int k = 0; k < NO; ++k) {
                        const bf16x8 bt = tr_frag(sB, BS, j0, 32 * Own<W>::nt(k), lane);
                        Hs[k] = mfma32(bt, xh, Hs[k]);
                        Hs[k] = mfma32(bt, xl, Hs[k]);
                    }
                }
        }

        // ---- y = y_diag + exp2(cs_i) * y_off for this wave's 32 tokens (lane = token i)
        const float ey = v.eY[i];
        if (i < valid) {
            TY* dst = yg + ((row0 + t0 + i) * cx.H + cx.h) * static_cast<int64_t>(P);
#pragma unroll
            for (int pt = 0; pt < 2; ++pt) {
                const f32x16 yv = yd[pt] + ey * yo[pt];
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const int p = 32 * pt + 8 * j + 4 * hf;
                    if constexpr (sizeof(TY) == 4) {
                        *reinterpret_cast<f32x4*>(dst + p) = f32x4{yv[4 * j], yv[4 * j + 1], yv[4 * j + 2], yv[4 * j + 3]};
                    } else {
                        *reinterpret_cast<bf16x4*>(dst + p) =
                            bf16x4{bf16(yv[4 * j]), bf16(yv[4 * j + 1]), bf16(yv[4 * j + 2]), bf16(yv[4 * j + 3])};
                    }
                }
            }
        }

        if (W == 3 && has_next) build_vec(sm.vec[nxt], nd0, nd1, A2, valid1, lane);
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");   // the next chunk's tiles have landed
        __syncthreads();   // ... and every wave is done with this chunk's LDS and H
        write_h();
        __syncthreads();
        if (has_next) {
#pragma unroll
            for (int ks = 0; ks < 8; ++ks) cf[ks] = cfn[ks];
        }
    }

    if (a.final_state) {
#pragma unroll
        for (int k = 0; k < NO; ++k) {
            const int p = 32 * PT + c32;
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int n = 32 * Own<W>::nt(k) + 8 * j + 4 * hf;
                *reinterpret_cast<f32x4*>(a.final_state + sbase + p * NS + n) =
                    f32x4{Hs[k][4 * j], Hs[k][4 * j + 1], Hs[k][4 * j + 2], Hs[k][4 * j + 3]};
            }
        }
    }
}

template <typename TY>
__global__ __launch_bounds__(kThreads, 1) void chunk_scan_kernel(ScanArgs a) {
    extern __shared__ __align__(16) unsigned char smem_raw[];
    Smem& sm = *reinterpret_cast<Smem*>(smem_raw);
    // XCD-aware numbering: workgroup id % 8 picks the XCD, so give each XCD a
    // contiguous run of (batch, head) -- heads of one group share B and C in its L2.
    const int64_t nb = a.batch * a.nheads;
    int64_t id = blockIdx.x;
    if (nb % 8 == 0) id = (id % 8) * (nb / 8) + id / 8;
    Ctx cx;
    cx.xg = static_cast<const bf16*>(a.x);
    cx.Bg = static_cast<const bf16*>(a.B);
    cx.Cg = static_cast<const bf16*>(a.C);
    cx.dtg = static_cast<const bf16*>(a.dt);
    cx.xs = a.x_row_stride;
    cx.bcs = a.bc_row_stride;
    cx.b = id / a.nheads;
    cx.h = static_cast<int>(id % a.nheads);
    cx.L = a.seqlen;
    cx.H = a.nheads;
    cx.grp = cx.h / (a.nheads / a.ngroups);
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int lane = threadIdx.x & 63;
    switch (wave) {
        case 0: run_wave<0, TY>(sm, a, cx, lane); break;
        case 1: run_wave<1, TY>(sm, a, cx, lane); break;
        case 2: run_wave<2, TY>(sm, a, cx, lane); break;
        default: run_wave<3, TY>(sm, a, cx, lane); break;
    }
}

}  // namespace scan32

bool mfma_scan_supports(int head_dim, int d_state, int chunk) {
    return head_dim == scan32::P && d_state == scan32::NS && chunk == scan32::Q;
}

template <typename TY>
static hipError_t mfma_t(const ScanArgs& a, hipStream_t s) {
    const int64_t blocks = a.batch * a.nheads;
    if (blocks == 0) return hipSuccess;
    auto kern = scan32::chunk_scan_kernel<TY>;
    const size_t smem = sizeof(scan32::Smem);
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, static_cast<int>(smem));
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(kern, dim3(static_cast<uint32_t>(blocks)), dim3(scan32::kThreads), smem, s, a);
    return hipGetLastError();
}

hipError_t launch_chunk_scan_mfma(const ScanArgs& a, Dt ydt, hipStream_t s) {
    return ydt == Dt::BF16 ? mfma_t<bf16>(a, s) : mfma_t<float>(a, s);
}

}  // namespace ssd
