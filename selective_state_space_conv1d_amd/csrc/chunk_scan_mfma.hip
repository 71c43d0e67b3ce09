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
//   H       = exp2(cs_last) * H + sum_j (exp2(cs_last - cs_j) dt_j x_j) (x) B_j
// which is the token recurrence re-associated exactly.
//
// Mapping.  One persistent workgroup of 8 waves (two per SIMD) per (batch,
// head) walks the chunks in order; the fp32 state stays in registers and never
// goes to HBM between chunks.  When sequences x heads overfill the chip and the
// sequences are short, a workgroup instead walks the chunks of a token-balanced
// range of sequences as one flat (sequence, chunk) stream, handing the state over
// at each sequence end (the WALK kernel).  Token rows past a chunk's end are
// skipped.  The waves have fixed roles:
//   * y waves 0..3: wave t owns the 32 tokens of token tile t and both 32-wide
//     p tiles.  It keeps its tokens' C rows in registers (the B operand of both
//     C.H and C.B^T) and loads the next chunk's rows itself, straight into
//     registers.  Per chunk it computes y^T = H C^T, scales by exp2(cs_i), then
//     for each causal key tile the C.B^T tile, turns it into score-matrix operands
//     M (bf16 hi + lo) in registers and accumulates y^T += X^T M^T; y goes out
//     through a private LDS staging area as whole 128-byte rows.
//   * state waves 4..6 own the 8 [n-tile][p-tile] tiles of H^T (4, 3 and 1 of
//     them) and add B^T (w x) per chunk; the decay-weighted x is formed in
//     registers from x^T fragments.
//   * wave 7 copies the next chunk's x tile and the lower half of its B tile into
//     the other half of double-buffered LDS early in the chunk (x comes from HBM)
//     and builds its per-token decay vectors.  y wave 0, the lightest, copies the
//     upper half of B (L2-resident) once its single causal tile is done.  The
//     compiler makes every LDS transpose read or LDS atomic wait for all copies in
//     flight, so a wave copies only after its last transpose read and atomic of
//     the chunk.
// MFMAs per SIMD and chunk (wave w and wave w + 4 share SIMD w): 48 + 64,
// 64 + 48, 80 + 16, 96 + 0.  The C.B^T accumulator is used directly as the
// B operand of X^T M^T: accumulator rows are that MFMA's k, and k is permuted
// the same way on both operands.  All products are v_mfma_f32_32x32x16_bf16.
// One workgroup barrier per chunk (the chunk's tiles, vectors and the previous
// state are in LDS).  The state is single-buffered in LDS: each y wave bumps an
// LDS counter once it has read it, and the state waves wait for all four before
// writing the new one (a bounded wait; the y waves never wait on the state waves
// inside a chunk, so the counter always fills).  Should the wait ever run out, the
// state waves poison their state with NaN before writing it, so that y from then on
// and the final state are NaN instead of silently wrong.
//
// Precision.  x, B and C arrive in bf16 and are exact operands.  Operands
// computed in fp32 (M, H and the decay-weighted x) are split into bf16 hi + lo
// and issued as two MFMAs (~16 significant bits).  Decays are exp2 of
// differences of prefix sums (exactly 1 on the diagonal); off-diagonal 32x32
// blocks use exp2(cs_i - cs_e) * exp2(cs_e - cs_j) about the block's last token
// e -- both factors <= 1, so nothing overflows.
//
// Data movement.  Tiles are row-major and unpadded in LDS with the 16-byte
// chunks of each row XOR-permuted by a key of the row, so that 16-byte row reads
// and LDS transpose reads (ds_read_b64_tr_b16) are free of bank conflicts.
// Operands that contract over tokens use the transpose reads, so no transposed
// copies exist.  Workgroups are numbered so that the heads sharing a B/C group
// sit on one XCD.
#include "ssd_device.h"
#include "ssd_kernels.h"
#include "state_codes.h"

#include <atomic>
#include <cstdlib>

namespace ssd {
namespace scan32 {

constexpr int Q = 128;    // tokens per chunk
constexpr int P = 64;     // head_dim
constexpr int NS = 128;   // d_state
constexpr int kThreads = 512;
constexpr int kRowB = NS * 2;   // bytes per row of the B and H tiles
constexpr int kRowX = P * 2;    // bytes per row of the x tiles
constexpr float kLog2e = 1.4426950408889634f;

typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) bf16 lds_bf16;
typedef __attribute__((address_space(3))) bf16x4 lds_bf16x4;

struct Vec {            // per-token quantities of one chunk
    float cs[Q];        // inclusive prefix sum of dt*A*log2(e)
    float dt[Q];
    float fM[Q];        // exp2(cs_e - cs_j) * dt_j, e = last token of j's 32-token tile
    float wS[Q];        // exp2(cs_last - cs_j) * dt_j for real tokens, 0 for padding
    float eY[Q];        // exp2(cs_i)
    float csE[4];       // cs at the end of each 32-token tile
    float dec;          // exp2(cs at the last real token): the chunk's decay of H
    float pad[3];
};

constexpr int kStage = 32 * kRowX;      // per y wave: its 32 bf16 y rows
constexpr int kYB = 16;                 // B copy units [kYB, 32) are moved by y wave 0, the rest by the loader

struct Smem {
    unsigned char B[2][Q * kRowB];       // B[j][n], double-buffered
    unsigned char X[2][Q * kRowX];       // x[j][p], double-buffered
    unsigned char Hh[P * kRowB];         // H[p][n], high bf16 part
    unsigned char Hl[P * kRowB];         //          low bf16 part
    unsigned char stage[4][kStage];      // private to y wave t
    Vec vec[2];
    int hread;                           // y waves that have read the state (cumulative)
};
static_assert(sizeof(Smem) <= 160 * 1024, "LDS budget");

// LDS swizzle.  The LDS has 64 four-byte banks (256 bytes per bank row).  A 256-byte
// row (B, C, H) fills one bank row and has 16 chunks of 16 bytes; its chunks are
// XOR-permuted by a 4-bit key of the row that is a bijection on any 16 consecutive
// rows and gives 4 consecutive rows 4 different 4-chunk blocks.  A 128-byte row (x)
// is half a bank row; a 3-bit key gives rows r and r + 2 different 4-chunk blocks.
// Row reads (16 lanes per pass, 16 rows, one chunk each) and transpose reads (32
// lanes per pass, 4 rows x 4 chunks) are then free of bank conflicts.
__device__ __forceinline__ int key16(int r) { return ((r & 3) << 2) | ((r >> 2) & 3); }
__device__ __forceinline__ int key8(int r) { return ((r & 3) << 1) | ((r >> 2) & 1); }
template <int RB> __device__ __forceinline__ int rkey(int r) { return RB == 256 ? key16(r) : key8(r); }
// byte offset of logical 16-byte chunk c of row r in a tile of RB-byte rows
template <int RB> __device__ __forceinline__ int soff(int r, int c) { return r * RB + ((c ^ rkey<RB>(r)) << 4); }

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

// Two-term bf16 split of 8 fp32 values: hi = v with the low 16 bits cleared (exact),
// lo = RNE_bf16(v - hi); hi + lo carries ~16 significant bits.  Three VALU ops per
// value: and, sub and half each of a byte permute and a packed convert.
__device__ __forceinline__ void split8(const float* v, bf16x8& hi, bf16x8& lo) {
    u32x4 h, l;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        const unsigned u0 = __float_as_uint(v[2 * k]), u1 = __float_as_uint(v[2 * k + 1]);
        const float r0 = v[2 * k] - __uint_as_float(u0 & 0xFFFF0000u);
        const float r1 = v[2 * k + 1] - __uint_as_float(u1 & 0xFFFF0000u);
        h[k] = __builtin_amdgcn_perm(u1, u0, 0x07060302u);    // upper halves of u0 (low) and u1 (high)
        l[k] = __builtin_bit_cast(unsigned, __builtin_convertvector(f32x2{r0, r1}, bf16x2));
    }
    hi = __builtin_bit_cast(bf16x8, h);
    lo = __builtin_bit_cast(bf16x8, l);
}

// RNE bf16 pair packed in one dword (low half = a)
__device__ __forceinline__ unsigned pack_bf16(float a, float b) {
    return __builtin_bit_cast(unsigned, __builtin_convertvector(f32x2{a, b}, bf16x2));
}
// s_waitcnt vmcnt(0) (gfx9 encoding: expcnt and lgkmcnt fields at their maximum), as
// the builtin so that the compiler's own wait insertion knows the loads are complete.
__device__ __forceinline__ void wait_vmem() { __builtin_amdgcn_s_waitcnt(0x0F70); }

// Lane-dependent byte offsets, computed once; every LDS access below is one of
// these plus a compile-time constant (row block), so the compiler keeps only a
// handful of address registers.
//  * row reads: lane (c32, hf) reads row base + c32, 16-byte chunk 2ks + hf;
//    the row key depends on c32 only (bases are multiples of 16 rows).
//  * transpose reads (MFMA operands whose k runs over tokens): within each
//    16-lane group, lane m supplies the address of row first + 4hf + m/4,
//    columns col0 + 16g + 4(m%4) .. +3 (g = (lane/16)%2).  The receiving lane
//    (c32, hf) then holds column col0 + c32 at tokens first + 4hf + {0..3};
//    two reads (first and first + 8) give the 8 slots of an operand in the row
//    order of a 32x32 accumulator.  first is a multiple of 16, so the key of a
//    row read depends on rl (first read) or rl + 8 (second read) only.
struct LaneOff {
    int row[8];     // row reads of a 256-byte-row tile: c32 * 256 + swizzled chunk (2ks + hf)
    int rl, cl, hb;
    __device__ __forceinline__ LaneOff(int lane) {
        const int c32 = lane & 31, hf = lane >> 5, rk = key16(c32);
#pragma unroll
        for (int ks = 0; ks < 8; ++ks) row[ks] = c32 * 256 + (((2 * ks + hf) ^ rk) << 4);
        const int m = lane & 15;
        rl = 4 * hf + (m >> 2);
        cl = 2 * ((lane >> 4) & 1) + ((m & 3) >> 1);
        hb = (m & 1) << 3;
    }
    // transpose-read base for a tile with RB-byte rows, columns from col0 (a multiple of 32),
    // rows rl + 8h (h = 0 for the first read of an operand, 1 for the second)
    template <int RB> __device__ __forceinline__ int tr(int col0, int h) const {
        return rl * RB + ((((col0 >> 3) + cl) ^ rkey<RB>(rl + 8 * h)) << 4) + hb;
    }
};

__device__ __forceinline__ bf16x8 ld16(const unsigned char* p) { return *reinterpret_cast<const bf16x8*>(p); }

// operand from two transpose reads at rows j0 (base b0) and j0 + 8 (base b8), j0 % 16 == 0
template <int RB>
__device__ __forceinline__ bf16x8 tr_frag(const unsigned char* t, int b0, int b8, int j0) {
    const bf16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)(lds_bf16*)(t + b0 + j0 * RB));
    const bf16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)(lds_bf16*)(t + b8 + (j0 + 8) * RB));
    return bf16x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
}

// Per-token vectors of a chunk from its dt (two tokens per lane of one wave).
// r0, r1 are the raw dt of tokens 2*lane and 2*lane+1 (read from in-range rows), put
// through the dt prologue of head h; tokens at or past `valid` count as dt = 0.
__device__ __forceinline__ void build_vec(Vec& v, bf16 r0, bf16 r1, float A2, int valid, int lane,
                                          const DtParams& dtp, int h) {
    const float d0 = 2 * lane < valid ? dt_prologue(static_cast<float>(r0), dtp, h) : 0.f;
    const float d1 = 2 * lane + 1 < valid ? dt_prologue(static_cast<float>(r1), dtp, h) : 0.f;
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
    if (lane == 0) v.dec = fexp2(csl);
}

// A position in the chunk sequence a workgroup walks: chunk c of sequence s, whose rows are
// [row0, row0 + L); ok is false past the last chunk.
struct Cursor {
    int64_t row0;
    int s, c, L;
    bool ok;
    __device__ __forceinline__ int valid() const {
        const int r = L - c * Q;
        return r < Q ? r : Q;
    }
    __device__ __forceinline__ int64_t first_row() const { return row0 + static_cast<int64_t>(c) * Q; }
};

// A workgroup scans head h of sequences [s_begin, s_end) one after another (WALK), so that a
// sequence's first chunk is loaded while the previous one's last chunk is computed, or of
// sequence s_begin alone.
template <bool WALK>
struct Ctx {
    const bf16* xg; const bf16* Bg; const bf16* Cg; const bf16* dtg;
    int64_t xs, bcs, seqlen;
    int s_begin, s_end;
    const SeqMap* seq;            // packed sequences (cu_seqlens set), else batch entries of seqlen rows
    int H, h, grp;
    __device__ __forceinline__ void span(int64_t s, int64_t& row0, int64_t& L) const {
        if (seq->cu_seqlens) seq_span(seq->cu_seqlens, s, seqlen, row0, L);
        else { row0 = s * seqlen; L = seqlen; }
    }
    // state index of sequence s (-1: padding, nothing stored) and whether it starts from it
    __device__ __forceinline__ int64_t slot(int64_t s) const {
        return seq->cu_seqlens ? seq_slot(seq->slot_idx, s, seq->nslots) : s;
    }
    __device__ __forceinline__ bool use_init(int64_t s) const {
        return seq->cu_seqlens ? (slot(s) >= 0 && seq->has_init && seq->has_init[s] != 0) : true;
    }
    // the first chunk of sequence s or of the next non-empty one
    __device__ __forceinline__ Cursor at(int s) const {
        Cursor u{0, s, 0, 0, false};
        if (!WALK) {
            if (s < s_end) {
                int64_t L;
                span(s, u.row0, L);
                u.L = static_cast<int>(L);
                u.ok = u.L > 0;
            }
            return u;
        }
        for (; u.s < s_end; ++u.s) {
            int64_t L;
            span(u.s, u.row0, L);
            u.L = static_cast<int>(L);
            if (u.L > 0) { u.ok = true; break; }
        }
        return u;
    }
    __device__ __forceinline__ Cursor first() const { return at(s_begin); }
    __device__ __forceinline__ Cursor next(const Cursor& u) const {
        Cursor n = u;
        ++n.c;
        if (!WALK || n.c * Q < u.L) {
            n.ok = n.c * Q < u.L;
            return n;
        }
        return at(u.s + 1);
    }
};

// ---------------------------------------------------------------------------
// Direct global->LDS copies of RB-byte rows: copy instruction k writes LDS bytes
// [1024k, +1024) of dst, lane l the 16 bytes at 1024k + 16l.  The lane picks its
// source so that the tile comes out swizzled: LDS chunk position cp of tile row r
// receives logical chunk cp ^ rkey(r).  Copy k covers tile rows r_lo + RPK k + ...;
// rows at or past `valid` re-read row valid - 1 (in range; such rows only meet zero
// weights or are never stored).
//
// When every row is real the lane's part of the address is one of a few offsets
// precomputed per lane (the key of row 4k + lane/16 depends on lane and k % 4 only;
// that of row 8k + lane/8 on the lane only), added to a wave-uniform row base.
// AUX is the copies' cache policy: 2 (non-temporal) for rows that only this workgroup reads.
template <int RB, int K0, int K1, int AUX = 0>
__device__ __forceinline__ void dma_rows(unsigned char* dst, const bf16* src0, int64_t row_stride, int64_t row0,
                                         int r_lo, int valid, int lane) {
    constexpr int RPK = 1024 / RB;                 // rows per copy instruction
    constexpr int LPR = RB / 16;                   // lanes per row
    const unsigned char* g0 = reinterpret_cast<const unsigned char*>(src0 + (row0 + r_lo) * row_stride);
    const int64_t sb = row_stride * 2;             // row stride in bytes
    if (r_lo + RPK * K1 <= valid) {
        const int lr = lane / LPR, cp = lane % LPR;
        unsigned off[4];
#pragma unroll
        for (int v = 0; v < 4; ++v)
            off[v] = static_cast<unsigned>(lr * sb) + 16u * static_cast<unsigned>(cp ^ rkey<RB>(r_lo + lr + RPK * v));
#pragma unroll
        for (int k = K0; k < K1; ++k) {
            const unsigned char* src = g0 + k * RPK * sb + off[k & 3];
            __builtin_amdgcn_global_load_lds((__attribute__((address_space(1))) void*)src,
                                             (__attribute__((address_space(3))) void*)(dst + 1024 * k), 16, 0, AUX);
        }
    } else {
#pragma unroll
        for (int k = K0; k < K1; ++k) {
            const int o = 1024 * k + 16 * lane;
            const int row = o / RB, cp = (o % RB) >> 4;       // tile row r_lo + row
            const int r = r_lo + row < valid ? row : valid - 1 - r_lo;
            const unsigned char* src = g0 + r * sb + 16 * (cp ^ rkey<RB>(r_lo + row));
            __builtin_amdgcn_global_load_lds((__attribute__((address_space(1))) void*)src,
                                             (__attribute__((address_space(3))) void*)(dst + 1024 * k), 16, 0, AUX);
        }
    }
}

// s_waitcnt lgkmcnt(0) (gfx9 encoding), before a copy overwrites LDS this wave just read
__device__ __forceinline__ void wait_lds() { __builtin_amdgcn_s_waitcnt(0xC07F); }

// ---------------------------------------------------------------------------
// y wave: token tile IT (tokens 32IT .. 32IT+31 of each chunk), both p tiles.
template <typename TY, int IT, class CX>
__device__ void run_y(Smem& sm, const ScanArgs& a, const CX& cx, const int lane) {
    const int c32 = lane & 31, hf = lane >> 5;
    const int i = 32 * IT + c32;                     // this lane's token within the chunk
    const float Dh = a.D ? a.D[cx.h] : 0.f;
    TY* yg = static_cast<TY*>(a.y);
    const LaneOff lo(lane);
    const int trX0 = lo.tr<kRowX>(0, 0), trX1 = lo.tr<kRowX>(32, 0);   // 128-byte rows: key period 8
    unsigned char* st = sm.stage[IT];
    const bf16* csrc = cx.Cg + static_cast<int64_t>(cx.grp) * NS;

    // C row of token i of chunk c, 16-byte chunks 2ks + hf: k = n = 16ks + 8hf + s, the
    // B operand (column i) of both H C^T and B C^T; loaded straight into registers (an
    // LDS copy would make the compiler wait for it before every later transpose read).
    // Rows past the end re-read the last real row.
    auto c_load = [&](bf16x8 (&cr)[8], const Cursor& u, int k0, int k1) {
        const int valid = u.valid();
        const int r = i < valid ? i : valid - 1;
        const bf16* p = csrc + (u.first_row() + r) * cx.bcs + 8 * hf;
#pragma unroll
        for (int ks = k0; ks < k1; ++ks) cr[ks] = *reinterpret_cast<const bf16x8*>(p + 16 * ks);
    };

    bf16x8 cn[8];
    Cursor cur = cx.first();
    if (cur.ok) c_load(cn, cur, 0, 8);
    __syncthreads();                                            // chunk 0

    for (int64_t gc = 0; cur.ok; ++gc) {
        const Cursor nx = cx.next(cur);
        const int valid = cur.valid();
        const bool has_next = nx.ok;
        const int buf = static_cast<int>(gc & 1);
        if constexpr (IT > 0) {
            if (32 * IT >= valid) {     // none of this wave's tokens is in the chunk: nothing to compute
                if (lane == 0) __hip_atomic_fetch_add(&sm.hread, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
                if (has_next) c_load(cn, nx, 0, 8);
                __syncthreads();                                // chunk c + 1
                cur = nx;
                continue;
            }
        }
        const Vec& v = sm.vec[buf];
        const unsigned char* Bt = sm.B[buf];
        const unsigned char* Xt = sm.X[buf];
        bf16x8 cf[8];
#pragma unroll
        for (int ks = 0; ks < 8; ++ks) cf[ks] = cn[ks];

        // carried state: y^T[p][i] = sum_n H[p][n] C[i][n], p tiles 0 and 1.  The 32 state
        // fragments are read in batches of 8, one batch ahead of the MFMAs that use them
        // (scheduling barriers keep the compiler from sinking each read to its use).
        f32x16 y0 = zero16(), y1 = zero16();
        {
            auto hfrag = [&](int k) {   // k = 4ks + 2hl + pt
                const unsigned char* hb = (k & 2) ? sm.Hl : sm.Hh;
                return ld16(hb + (k & 1) * 32 * kRowB + lo.row[k >> 2]);
            };
            bf16x8 hf[32];
#pragma unroll
            for (int k = 0; k < 8; ++k) hf[k] = hfrag(k);
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                if (g < 3) {
#pragma unroll
                    for (int k = 8 * (g + 1); k < 8 * (g + 2); ++k) hf[k] = hfrag(k);
                }
                __builtin_amdgcn_sched_barrier(0);
#pragma unroll
                for (int k = 8 * g; k < 8 * (g + 1); ++k) {
                    if (k & 1) y1 = mfma32(hf[k], cf[k >> 2], y1);
                    else y0 = mfma32(hf[k], cf[k >> 2], y0);
                }
                __builtin_amdgcn_sched_barrier(0);
            }
        }
        // the state has been read: LDS executes a wave's operations in issue order, so the
        // counter update lands after this wave's state reads (no fence, which would also
        // wait for the C copy in flight)
        if (lane == 0) __hip_atomic_fetch_add(&sm.hread, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
        if (has_next) c_load(cn, nx, 0, 4);
        const float ey = v.eY[i];
        y0 *= ey;
        y1 *= ey;

        // per causal key tile jt <= IT: the C.B^T tile (acc rows = tokens j, cols = tokens i),
        // M = C.B^T * decay * dt (+ D on the diagonal) as bf16 hi/lo operands, and
        // y^T[p][i] += sum_j X^T[p][j] M^T[j][i]
        auto cbt = [&](int jt) {
            f32x16 acc = zero16();
#pragma unroll
            for (int ks = 0; ks < 8; ++ks) acc = mfma32(ld16(Bt + 32 * jt * kRowB + lo.row[ks]), cf[ks], acc);
            return acc;
        };
        const float csi = v.cs[i];
        f32x16 cbn = cbt(0);
#pragma unroll
        for (int jt = 0; jt <= IT; ++jt) {
            f32x16 m = cbn;          // m[4j + r] = C_i . B_jj,  jj = 32jt + 8j + 4hf + r
            if (jt < IT) cbn = cbt(jt + 1);   // the next tile's MFMAs overlap this tile's VALU work
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
                float mv[8];
#pragma unroll
                for (int s = 0; s < 8; ++s) mv[s] = m[8 * q + s];
                bf16x8 mh, ml;
                split8(mv, mh, ml);
                const bf16x8 x0 = tr_frag<kRowX>(Xt, trX0, trX0, 32 * jt + 16 * q);
                const bf16x8 x1 = tr_frag<kRowX>(Xt, trX1, trX1, 32 * jt + 16 * q);
                y0 = mfma32(x0, mh, y0);
                y1 = mfma32(x1, mh, y1);
                y0 = mfma32(x0, ml, y0);
                y1 = mfma32(x1, ml, y1);
            }
            if (jt == 0 && has_next) c_load(cn, nx, 4, 8);
        }
        if constexpr (IT == 0) {
            // the lightest y wave copies the upper half of the next chunk's B tile (L2-resident:
            // the group's heads share it), after its last transpose read of the chunk
            if (has_next)
                dma_rows<kRowB, kYB, 32>(sm.B[buf ^ 1], cx.Bg + static_cast<int64_t>(cx.grp) * NS, cx.bcs,
                                         nx.first_row(), 0, nx.valid(), lane);
        }

        // y[token i][p]: lane (c32, hf) holds p = 32pt + 8j + 4hf + r in y_pt[4j + r].  Swapping
        // j = 1 of the low half-wave with j = 0 of the high half-wave (and j = 3 with j = 2) leaves
        // each lane with p = 32pt + 16g + 8hf + {0..7} (g = 0, 1): two 16-byte pieces per p tile.
        TY* yrow = yg + (cur.first_row() * cx.H + cx.h) * static_cast<int64_t>(P);   // token 0, p 0
        const int64_t ystr = static_cast<int64_t>(cx.H) * P;                         // token stride
        if constexpr (sizeof(TY) == 4) {
            if (i < valid) {
                TY* dst = yrow + i * ystr + 8 * hf;
#pragma unroll
                for (int pt = 0; pt < 2; ++pt) {
                    const f32x16& yv = pt ? y1 : y0;
#pragma unroll
                    for (int g = 0; g < 2; ++g) {
                        u32x4 lo4, hi4;
#pragma unroll
                        for (int r = 0; r < 4; ++r) {
                            const float a0 = yv[8 * g + r], b0 = yv[8 * g + 4 + r];
                            const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(a0), __float_as_uint(b0),
                                                                             false, false);
                            lo4[r] = sw[0];
                            hi4[r] = sw[1];
                        }
                        __builtin_nontemporal_store(lo4, reinterpret_cast<u32x4*>(dst + 32 * pt + 16 * g));
                        __builtin_nontemporal_store(hi4, reinterpret_cast<u32x4*>(dst + 32 * pt + 16 * g + 4));
                    }
                }
            }
        } else {
            // bf16: the 32 x 128-byte tile goes through the staging area (row c32, 16-byte
            // chunk 4pt + 2g + hf, key of 128-byte rows by row pair), then out as whole rows:
            // read k gives lane l row 8k + l/8, chunk l%8.
#pragma unroll
            for (int pt = 0; pt < 2; ++pt) {
                const f32x16& yv = pt ? y1 : y0;
#pragma unroll
                for (int g = 0; g < 2; ++g) {
                    u32x4 o;
#pragma unroll
                    for (int h2 = 0; h2 < 2; ++h2) {
                        const unsigned pa = pack_bf16(yv[8 * g + 2 * h2], yv[8 * g + 2 * h2 + 1]);
                        const unsigned pb = pack_bf16(yv[8 * g + 4 + 2 * h2], yv[8 * g + 4 + 2 * h2 + 1]);
                        const auto sw = __builtin_amdgcn_permlane32_swap(pa, pb, false, false);
                        o[h2] = sw[0];
                        o[2 + h2] = sw[1];
                    }
                    const int ch = 4 * pt + 2 * g + hf;
                    *reinterpret_cast<u32x4*>(st + c32 * kRowX + ((ch ^ ((c32 >> 1) & 7)) << 4)) = o;
                }
            }
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                const int r = 8 * k + (lane >> 3), ch = lane & 7;
                const u32x4 o = *reinterpret_cast<const u32x4*>(st + r * kRowX + ((ch ^ ((r >> 1) & 7)) << 4));
                if (32 * IT + r < valid)
                    __builtin_nontemporal_store(o, reinterpret_cast<u32x4*>(yrow + (32 * IT + r) * ystr + 8 * ch));
            }
        }
        if constexpr (IT == 0) wait_vmem();
        __syncthreads();                                        // chunk c + 1
        cur = nx;
    }
}

// ---------------------------------------------------------------------------
// state wave: NT tiles of H^T, n tiles SN0 .. SN0+NT-1 of p tile SP.  Tile t holds
// Hs[t][4j + r] = H[p = 32SP + c32][n = 32(SN0 + t) + 8j + 4hf + r].
constexpr int kSpinMax = 1 << 20;   // iterations of the bounded wait (each ~64 cycles of sleep)

// LP: the initial and final states are 16-bit codes (a separate instantiation, so that the fp32
// kernel carries none of the rounding code)
template <int NT, int SP, int SN0, bool LP, class CX>
__device__ void run_s(Smem& sm, const ScanArgs& a, const CX& cx, const int lane) {
    const int c32 = lane & 31, hf = lane >> 5;
    const int hp = 32 * SP + c32;
    // the state of sequence s lives at slot(s) (nothing read or stored for padding)
    auto sbase = [&](int64_t sl) { return (sl * cx.H + cx.h) * static_cast<int64_t>(P) * NS; };
    const LaneOff lo(lane);
    const int trW = lo.tr<kRowX>(32 * SP, 0);            // x^T fragments of the p tile
    int trB0[NT], trB8[NT];                              // B^T fragments of the n tiles
#pragma unroll
    for (int t = 0; t < NT; ++t) {
        trB0[t] = lo.tr<kRowB>(32 * (SN0 + t), 0);
        trB8[t] = lo.tr<kRowB>(32 * (SN0 + t), 1);
    }

    f32x16 Hs[NT];
    // dst = the initial state of sequence s (zeros without one)
    auto load_init = [&](int64_t s, f32x16 (&dst)[NT]) {
        const int64_t sl = cx.slot(s);
        const bool from = (LP ? a.init16 != nullptr : a.init_state != nullptr) && sl >= 0 && cx.use_init(s);
#pragma unroll
        for (int t = 0; t < NT; ++t)
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int n = 32 * (SN0 + t) + 8 * j + 4 * hf;
                f32x4 v = {0.f, 0.f, 0.f, 0.f};
                if constexpr (LP) {
                    if (from) v = codes_load4(a.init16, a.codes.f16, sbase(sl) + hp * NS + n);
                } else {
                    if (from) v = *reinterpret_cast<const f32x4*>(a.init_state + sbase(sl) + hp * NS + n);
                }
#pragma unroll
                for (int r = 0; r < 4; ++r) dst[t][4 * j + r] = v[r];
            }
    };
    auto store_final = [&](int64_t s, const f32x16 (&src)[NT]) {   // src as the final state of sequence s
        const int64_t sl = cx.slot(s);
        if ((LP ? a.final16 == nullptr : a.final_state == nullptr) || sl < 0) return;
#pragma unroll
        for (int t = 0; t < NT; ++t)
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int n = 32 * (SN0 + t) + 8 * j + 4 * hf;
                const f32x4 v = {src[t][4 * j], src[t][4 * j + 1], src[t][4 * j + 2], src[t][4 * j + 3]};
                if constexpr (LP) codes_store4(a.final16, a.codes, sbase(sl) + hp * NS + n, v);
                else *reinterpret_cast<f32x4*>(a.final_state + sbase(sl) + hp * NS + n) = v;
            }
    };
    // empty sequences in [s0, s1) end with their initial state (zeros without one)
    auto finish_empty = [&](int s0, int s1) {
        for (int e = s0; e < s1; ++e) {
            f32x16 He[NT];
            load_init(e, He);
            store_final(e, He);
        }
    };
    Cursor cur = cx.first();
    finish_empty(cx.s_begin, cur.ok ? cur.s : cx.s_end);
    if (cur.ok) {
        load_init(cur.s, Hs);
    } else {
#pragma unroll
        for (int t = 0; t < NT; ++t) Hs[t] = zero16();
    }
    auto write_h = [&]() {
#pragma unroll
        for (int t = 0; t < NT; ++t)
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                bf16x4 hh, hl;
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    hh[r] = bhi(Hs[t][4 * j + r]);
                    hl[r] = static_cast<bf16>(Hs[t][4 * j + r] - static_cast<float>(hh[r]));
                }
                const int o = soff<kRowB>(hp, 4 * (SN0 + t) + j) + 8 * hf;
                *reinterpret_cast<bf16x4*>(sm.Hh + o) = hh;
                *reinterpret_cast<bf16x4*>(sm.Hl + o) = hl;
            }
    };

    write_h();
    __syncthreads();                                            // chunk 0

    for (int64_t gc = 0; cur.ok; ++gc) {
        const Cursor nx = cx.next(cur);
        const int buf = static_cast<int>(gc & 1);
        const Vec& v = sm.vec[buf];
        const unsigned char* Bt = sm.B[buf];
        const unsigned char* Xt = sm.X[buf];
        const float dec = v.dec;
#pragma unroll
        for (int t = 0; t < NT; ++t) Hs[t] *= dec;

        // token step k (tokens 16k .. 16k+15): H^T[n][p] += sum_j B^T[n][j] (w_j x_j)[p]; steps
        // past the chunk's last token would only add zero weights
        const int valid = cur.valid();
#pragma unroll
        for (int k = 0; k < 8; ++k) {
            const int j0 = 16 * k;
            if (k > 0 && j0 >= valid) break;
            const bf16x8 xf = tr_frag<kRowX>(Xt, trW, trW, j0);
            const f32x4 w0 = *reinterpret_cast<const f32x4*>(&v.wS[j0 + 4 * hf]);
            const f32x4 w1 = *reinterpret_cast<const f32x4*>(&v.wS[j0 + 8 + 4 * hf]);
            float e[8];
#pragma unroll
            for (int s = 0; s < 8; ++s) e[s] = static_cast<float>(xf[s]) * (s < 4 ? w0[s] : w1[s - 4]);
            bf16x8 wh, wl;
            split8(e, wh, wl);
#pragma unroll
            for (int t = 0; t < NT; ++t) {
                const bf16x8 bt = tr_frag<kRowB>(Bt, trB0[t], trB8[t], j0);
                Hs[t] = mfma32(bt, wh, Hs[t]);
                Hs[t] = mfma32(bt, wl, Hs[t]);
            }
        }
        // state snapshot after token (c + 1) * Q - 1 of the sequence when that closes an interval
        if (a.snapshots) {
            float* snap = snapshot_dst(a, cur.s, cur.L, (cur.c + 1) * static_cast<int64_t>(Q), cx.h);
            if (snap) {
#pragma unroll
                for (int t = 0; t < NT; ++t)
#pragma unroll
                    for (int j = 0; j < 4; ++j) {
                        const int n = 32 * (SN0 + t) + 8 * j + 4 * hf;
                        *reinterpret_cast<f32x4*>(snap + hp * NS + n) =
                            f32x4{Hs[t][4 * j], Hs[t][4 * j + 1], Hs[t][4 * j + 2], Hs[t][4 * j + 3]};
                    }
            }
        }
        // the sequence's last chunk: its final state, those of the empty sequences after it, and
        // the next sequence's initial state, which the y waves then use as the carried state.  The
        // next state's loads are issued before the final state's stores, so that waiting for them
        // does not wait for the stores as well (one counter covers both).
        if (!nx.ok || nx.s != cur.s) {
            f32x16 Hn[NT];
            if (nx.ok) load_init(nx.s, Hn);
            store_final(cur.s, Hs);
            if (nx.ok) {
#pragma unroll
                for (int t = 0; t < NT; ++t) Hs[t] = Hn[t];
            }
            finish_empty(cur.s + 1, nx.ok ? nx.s : cx.s_end);
        }
        // the y waves must have read the previous state before it is overwritten
        const int target = 4 * static_cast<int>(gc + 1);
        bool seen = false;
        for (int n = 0; n < a.spin_max; ++n) {
            if (__hip_atomic_load(&sm.hread, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP) >= target) {
                seen = true;
                break;
            }
            __builtin_amdgcn_s_sleep(1);
        }
        if (!seen) {                                // the wait ran out: make it visible in every later output
#pragma unroll
            for (int t = 0; t < NT; ++t)
#pragma unroll
                for (int e = 0; e < 16; ++e) Hs[t][e] = __builtin_nanf("");
        }
        __atomic_signal_fence(__ATOMIC_SEQ_CST);   // the state writes stay after the wait
        write_h();
        __syncthreads();                                        // chunk c + 1
        cur = nx;
    }
}

// ---------------------------------------------------------------------------
// loader wave: the next chunk's x tile and the lower half of its B tile, and its
// per-token vectors.
template <class CX>
__device__ void run_l(Smem& sm, const ScanArgs& a, const CX& cx, const int lane) {
    const float A2 = a.A[cx.h] * kLog2e;
    const bf16* bsrc = cx.Bg + static_cast<int64_t>(cx.grp) * NS;
    const bf16* xsrc = cx.xg + static_cast<int64_t>(cx.h) * P;
    auto load_dt = [&](bf16& d0, bf16& d1, int64_t r0, int valid) {   // rows r0 .. r0 + valid - 1
        const int q0 = 2 * lane < valid ? 2 * lane : valid - 1;
        const int q1 = 2 * lane + 1 < valid ? 2 * lane + 1 : valid - 1;
        d0 = cx.dtg[(r0 + q0) * cx.H + cx.h];
        d1 = cx.dtg[(r0 + q1) * cx.H + cx.h];
    };
    if (lane == 0) sm.hread = 0;
    Cursor cur = cx.first();
    if (cur.ok) {
        bf16 d0, d1;
        const int v0 = cur.valid();
        const int64_t r0 = cur.first_row();
        load_dt(d0, d1, r0, v0);
        // the head's x rows are read by this workgroup only, and y is written once: both streamed
        // (non-temporal), which leaves the caches to the B/C tiles the group's heads share
        dma_rows<kRowX, 0, 16, 2>(sm.X[0], xsrc, cx.xs, r0, 0, v0, lane);
        dma_rows<kRowB, 0, 32>(sm.B[0], bsrc, cx.bcs, r0, 0, v0, lane);
        build_vec(sm.vec[0], d0, d1, A2, v0, lane, a.dtp, cx.h);
    }
    wait_vmem();
    __syncthreads();                                            // chunk 0

    for (int64_t gc = 0; cur.ok; ++gc) {
        const Cursor nx = cx.next(cur);
        const int buf = static_cast<int>(gc & 1);
        if (nx.ok) {
            const int64_t r0 = nx.first_row();
            const int vn = nx.valid();
            bf16 d0, d1;
            load_dt(d0, d1, r0, vn);
            dma_rows<kRowX, 0, 16, 2>(sm.X[buf ^ 1], xsrc, cx.xs, r0, 0, vn, lane);
            dma_rows<kRowB, 0, kYB>(sm.B[buf ^ 1], bsrc, cx.bcs, r0, 0, vn, lane);
            build_vec(sm.vec[buf ^ 1], d0, d1, A2, vn, lane, a.dtp, cx.h);
        }
        wait_vmem();
        __syncthreads();                                        // chunk c + 1
        cur = nx;
    }
}

// First sequence of range r of a.nranges: sequences split evenly for a batch of equal
// sequences; for packed ones, the first sequence that starts at or after token r T / R (T the
// packed rows), so that ranges hold about equal token counts.  Range 0 starts at 0 and range R
// at the end; with a non-decreasing cu_seqlens the ranges partition the sequences.
__device__ int64_t range_start(const ScanArgs& a, int64_t r) {
    const int64_t S = a.batch, R = a.nranges;
    if (r <= 0) return 0;
    if (r >= R) return S;
    if (!a.seq.cu_seqlens) return S * r / R;
    const int64_t t = (a.seqlen * r + R - 1) / R;
    int64_t lo = 0, hi = S;
    while (lo < hi) {
        const int64_t m = (lo + hi) / 2;
        int64_t v = a.seq.cu_seqlens[m];
        v = v < 0 ? 0 : (v > a.seqlen ? a.seqlen : v);
        if (v >= t) hi = m;
        else lo = m + 1;
    }
    return lo;
}

template <typename TY, bool WALK, bool LP>
__global__ __launch_bounds__(kThreads, 1) void chunk_scan_kernel(ScanArgs a) {
    extern __shared__ __align__(16) unsigned char smem_raw[];
    Smem& sm = *reinterpret_cast<Smem*>(smem_raw);
    // XCD-aware numbering: workgroup id % 8 picks the XCD.  XCD k takes heads
    // [k H/8, (k+1) H/8) of every batch entry / sequence range: heads of one group share B
    // and C in that XCD's L2, and every XCD gets an equal share of each sequence
    // (packed batches mix short and long ones).
    int64_t id = blockIdx.x;
    if (a.nheads % 8 == 0) {
        const int64_t hpx = a.nheads / 8, j = id / 8;
        id = (j / hpx) * a.nheads + (id % 8) * hpx + j % hpx;
    }
    Ctx<WALK> cx;
    cx.xg = static_cast<const bf16*>(a.x);
    cx.Bg = static_cast<const bf16*>(a.B);
    cx.Cg = static_cast<const bf16*>(a.C);
    cx.dtg = static_cast<const bf16*>(a.dt);
    cx.xs = a.x_row_stride;
    cx.bcs = a.bc_row_stride;
    const int64_t r = id / a.nheads;
    cx.h = static_cast<int>(id % a.nheads);
    cx.seq = &a.seq;
    cx.seqlen = a.seqlen;
    if (!WALK) {                             // one sequence per workgroup
        cx.s_begin = static_cast<int>(r);
        cx.s_end = static_cast<int>(r + 1);
    } else {
        const int64_t b = range_start(a, r), e = range_start(a, r + 1);
        cx.s_begin = static_cast<int>(b);
        cx.s_end = static_cast<int>(e > b ? e : b);
    }
    cx.H = a.nheads;
    cx.grp = cx.h / (a.nheads / a.ngroups);
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int lane = threadIdx.x & 63;
    // wave w runs on SIMD w % 4; the role split balances MFMAs per SIMD.  The state waves issue
    // ahead of the y wave on their SIMD (their state feeds the next chunk; about 2 % faster than
    // equal priority, while raising the y waves or the loader instead was slower).
    if (wave >= 4 && wave < 7) __builtin_amdgcn_s_setprio(1);
    if (wave == 0) run_y<TY, 0>(sm, a, cx, lane);
    else if (wave == 1) run_y<TY, 1>(sm, a, cx, lane);
    else if (wave == 2) run_y<TY, 2>(sm, a, cx, lane);
    else if (wave == 3) run_y<TY, 3>(sm, a, cx, lane);
    else if (wave == 4) run_s<4, 0, 0, LP>(sm, a, cx, lane);
    else if (wave == 5) run_s<3, 1, 0, LP>(sm, a, cx, lane);
    else if (wave == 6) run_s<1, 1, 3, LP>(sm, a, cx, lane);
    else run_l(sm, a, cx, lane);
}

}  // namespace scan32

bool mfma_scan_supports(int head_dim, int d_state, int chunk) {
    return head_dim == scan32::P && d_state == scan32::NS && chunk == scan32::Q;
}

// Workgroups resident per CU times this: the sequence ranges per head are chosen so that one
// launch has about this many rounds of workgroups.
#ifndef SSD_SCAN_RANGE_ROUNDS
#define SSD_SCAN_RANGE_ROUNDS 1
#endif

// Compute units of the current device (cached per device).
static int64_t device_cus() {
    static std::atomic<int> cache[64];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0) return 256;
    if (dev < 64) {
        const int c = cache[dev].load(std::memory_order_relaxed);
        if (c > 0) return c;
    }
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = 256;
    if (dev < 64) cache[dev].store(n, std::memory_order_relaxed);
    return n;
}

template <typename TY>
static hipError_t mfma_t(const ScanArgs& args, hipStream_t s) {
    if (args.batch * args.nheads == 0) return hipSuccess;
    // One workgroup per (sequence, head) while that fills the chip, or while sequences average
    // more than kWalkChunks chunks (the walking kernel's per-chunk cost is a little higher);
    // past that, each workgroup walks a range of sequences (one CU holds one workgroup), so that
    // a sequence's first chunk is fetched while the previous one's last chunk is computed.
    constexpr int64_t kWalkChunks = 8;
    ScanArgs a = args;
    const int64_t want = (SSD_SCAN_RANGE_ROUNDS * device_cus() + a.nheads - 1) / a.nheads;
    const int64_t rows = a.seq.cu_seqlens ? a.seqlen : a.batch * a.seqlen;   // all sequences' rows
    const bool walk = a.batch > want && rows <= kWalkChunks * scan32::Q * a.batch;
    a.nranges = walk ? want : a.batch;
    // SSD_SCAN_SPIN_MAX (a test hook) shortens the bounded wait, e.g. to 0 to check that running out is seen
    static const int spin_env = [] {
        const char* v = std::getenv("SSD_SCAN_SPIN_MAX");
        return v ? std::atoi(v) : -1;
    }();
    a.spin_max = spin_env >= 0 ? spin_env : scan32::kSpinMax;
    const int64_t blocks = a.nranges * a.nheads;
    const bool lp = a.init16 || a.final16;
    const bool wk = a.nranges < a.batch;
    auto kern = wk ? (lp ? scan32::chunk_scan_kernel<TY, true, true> : scan32::chunk_scan_kernel<TY, true, false>)
                   : (lp ? scan32::chunk_scan_kernel<TY, false, true> : scan32::chunk_scan_kernel<TY, false, false>);
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
