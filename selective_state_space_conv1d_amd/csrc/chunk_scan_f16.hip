// SSD chunked scan for prefill on fp16 MFMA (gfx950): head_dim 64, d_state 128, chunk 128,
// bf16 inputs -- the Ultra-family Mamba layer.
//
// Method (the structured-semiseparable / chunked form of the Mamba-2 scan: "Mamba 与 Nemotron
// 系列模型深度调研", Mamba 架构; the 128-token chunked scan that returns the final state in the
// modeling_nemotron_h.py walk-through, "Prefill 阶段").  Per chunk of Q = 128 tokens, with cs the
// inclusive prefix sum of dt*A in base-2 units:
//   M[i][j] = (C_i . B_j) * exp2(cs_i - cs_j) * dt_j   (j <= i), + D on the diagonal
//   y_i     = sum_j M[i][j] x_j  +  exp2(cs_i) * (C_i . H)
//   H       = exp2(cs_last) * H + sum_j (exp2(cs_last - cs_j) dt_j x_j) (x) B_j
// which is the token recurrence re-associated exactly.
//
// Precision.  Every product runs as ONE v_mfma_f32_32x32x16_f16 with fp32 accumulation.  fp16 has
// an 11-bit significand (8x finer than bf16), so one rounding of each fp32-derived operand (M,
// the decay-weighted x, H) stays well inside the bar, and the bf16 inputs x, B and C convert to
// fp16 exactly.  fp16's range is narrow, so every operand carries an exact power-of-two scale:
//   * B and C: a pre-pass converts each (batch, group, chunk) tile with the scale that puts its
//     largest magnitude in [2^14, 2^15) (exponents eB, eC), and stores what the scan reads: B'^T
//     as the LDS image of its swizzled tile, C' in the y waves' register order, and the causal
//     tiles of C'.B'^T in fp32 (shared by every head of the group, so computed once);
//   * x: the loader wave scales a chunk only when its largest magnitude leaves [2^-8, 2^15)
//     (exponent ex, usually 0);
//   * M, the weighted x and H: scales from bounds computed in scalar arithmetic per chunk
//     (|C.B| <= N max|C| max|B|; decays <= 1; |H| follows bound' = dec bound + sum(w) max|B| max|x|);
// all of which fold into per-token or per-lane factors the kernel computes anyway.  The state
// stays fp32 in registers across chunks; only its copy for C.H is rounded.
//
// Mapping.  One workgroup of 8 waves (two per SIMD: wave w runs on SIMD w % 4) per (batch, head)
// walks the chunks in order, one barrier per chunk.  Everything one chunk reads from LDS was
// written in the chunk before (double buffers), so no wave waits on another inside a chunk:
//   * y waves 0..3: token tile t (tokens 32t .. 32t+31).  C.H for both 32-wide p tiles from the
//     state copy H'; then per causal key tile jt <= t: the pre-pass's C.B^T tile (accumulator
//     rows = key tokens) times the masked decay in registers, converted straight into the next
//     MFMA's operand, and y^T += X^T M^T.  C rows and C.B^T tiles stay in registers, each set
//     reloaded with the next chunk's values right after its last use.
//   * waves 4, 5: the fp32 state H^T of n tiles 0, 1 / 2, 3 (both p tiles), + B^T (w x) per chunk with
//     B^T operands loaded from the pre-pass into registers a chunk ahead, and the fp16 copy H' for the
//     next chunk's C.H.
//   * waves 6, 7: x rows 0..31 / 32..127, loaded three chunks ahead into registers, converted to fp16
//     into LDS one chunk ahead (the two parts share their largest |x| through LDS across a barrier);
//     wave 6 also builds each chunk's per-token vectors and scale exponents.
// The kernel is bound by the vector-memory path of each CU (every head's workgroup reads its group's
// B, C and C.B^T tiles, ~84 KiB per chunk, besides its own x and dt): loads are laid out so that each
// instruction reads whole 1 KiB runs, and are spread over the waves instead of issued in bursts.
// MFMAs per SIMD and chunk: 20 + 32, 24 + 32, 28 + 0, 32 + 0.
// Operands that contract over tokens are LDS transpose reads (ds_read_b64_tr_b16) of row-major
// tiles; 16-byte chunks of each row are XOR-permuted so that row and transpose reads are free of
// bank conflicts.  Workgroups are numbered so that the heads sharing a B/C group sit on one XCD.
#include <utility>

#include "ssd_device.h"
#include "ssd_kernels.h"
#include "state_codes.h"

namespace ssd {
namespace scan16 {

constexpr int Q = 128;    // tokens per chunk
constexpr int P = 64;     // head_dim
constexpr int NS = 128;   // d_state
constexpr int kThreads = 512;
constexpr int kRowB = NS * 2;   // bytes per row of the B and H' tiles
constexpr int kRowX = P * 2;    // bytes per row of the x tile
constexpr int kTile = Q * kRowB;   // bytes of one B (or C) tile: 32 KiB
constexpr float kLog2e = 1.4426950408889634f;

typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef _Float16 f16;
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef unsigned short u16x2 __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) bf16 lds_bf16;
typedef __attribute__((address_space(3))) bf16x4 lds_bf16x4;

// floor(log2 v) for finite v > 0 (an upper bound -127 for subnormals); kNoExp for v == 0
constexpr int kNoExp = -400;
__device__ __forceinline__ int ilog2f(float v) {
    const unsigned u = __float_as_uint(v) & 0x7FFFFFFFu;
    return u == 0 ? kNoExp : static_cast<int>(u >> 23) - 127;
}
__device__ __forceinline__ float ldexp_f(float v, int e) { return __builtin_amdgcn_ldexpf(v, e); }
__device__ __forceinline__ float fexp2(float v) { return __builtin_amdgcn_exp2f(v); }

// Per-chunk quantities, built by the loader wave.  Scale exponents (integers):
//   eB, eC  pre-pass scales of the chunk's B and C tiles (B = B' 2^eB)
//   ex      the chunk's x scale (x = x' 2^ex)
//   sM      lane-factor exponent of M' = M 2^(ex - eM): M' = (C'.B'^T) 2^sM exp2(cs_i - cs_j) dt_j
//   eM      y accumulates in units of 2^eM
//   ew      weighted-x scale: w x = (w' x') 2^ew, wS holding w' = w 2^(ex - ew) (in fp16)
//   sH      the state waves' accumulator units after this chunk (eB + ew)
//   eHc     units of the fp16 state copy H' this chunk reads; eHn: of the copy it writes
struct Vec {
    float cs[Q];        // inclusive prefix sum of dt*A*log2(e)
    float fM[Q];        // off-diagonal column factor exp2(cs_e - cs_j) dt_j, e = last token of j's tile
    float vD[Q];        // diagonal column factor exp2(cs_m - cs_j) dt_j, m = token 15 of j's tile
    float dt[Q];        // dt_j (0 past the chunk's end)
    f16 wS[Q];          // exp2(cs_last - cs_j) dt_j 2^(ex - ew) for real tokens, 0 for padding: w' <= 1, in fp16
    float csE[4];       // cs at the end of each 32-token tile
    float csM[4];       // cs at token 15 of each tile
    int diagOK[4];      // the tile's decay range allows the factored diagonal
    float dec;          // exp2(cs at the last real token): the chunk's decay of H
    float dx;           // D 2^(ex - eM)
    int eB, eC, ex, sM, eM, ew, sH, sHp, eHc, eHn;
    int pad[2];
};

struct Smem {
    unsigned char X[2][Q * kRowX];       // x'[j][p] fp16, double-buffered
    unsigned char H[2][P * kRowB];       // H'[p][n] fp16, double-buffered
    unsigned char stage[4][32 * kRowX];  // private to y wave t: its chunk's bf16 y rows, stored one chunk later
    Vec vec[2];
    float hmax[2];                       // |initial state| maxima of the two state waves
    unsigned xmax[2][2];                 // largest |x| (bf16 bits) of each half of a chunk, by chunk parity
    // fused conv only (the unfused kernel allocates up to Xr): a chunk's raw xBC x rows (3 rows before it,
    // then its 128 rows; bf16, swizzled like X), double-buffered; the head's taps cw[k][ch] (k = 4: bias)
    // and the bounds |bias| <= cbound[0], sum_k |w_k| <= cbound[1] over its channels
    unsigned char Xr[2][(Q + 3) * kRowX];
    float cw[5][P];
    float cbound[2];
};
static_assert(sizeof(Smem) <= 160 * 1024, "LDS budget");
static_assert(sizeof(Vec) % 8 == 0, "8-byte reads of the second vector block");

// LDS swizzle: 256-byte rows XOR their 16-byte chunk index with a 4-bit key of the row, 128-byte
// rows with a 3-bit key (conflict-free row reads of 16 lanes and transpose reads of 32 lanes).
__device__ __forceinline__ int key16(int r) { return ((r & 3) << 2) | ((r >> 2) & 3); }
__device__ __forceinline__ int key8(int r) { return ((r & 3) << 1) | ((r >> 2) & 1); }
template <int RB> __device__ __forceinline__ int rkey(int r) { return RB == 256 ? key16(r) : key8(r); }
template <int RB> __device__ __forceinline__ int soff(int r, int c) { return r * RB + ((c ^ rkey<RB>(r)) << 4); }

__device__ __forceinline__ f32x16 mfma(f16x8 a, f16x8 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x16 zero16() {
    f32x16 z;
#pragma unroll
    for (int i = 0; i < 16; ++i) z[i] = 0.f;
    return z;
}
// 8 fp32 values -> fp16x8 (round to nearest even)
__device__ __forceinline__ f16x8 to_f16x8(const float* v) {
    f16x8 r;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        const f16x2 h = __builtin_convertvector(f32x2{v[2 * k], v[2 * k + 1]}, f16x2);
        r[2 * k] = h[0];
        r[2 * k + 1] = h[1];
    }
    return r;
}
__device__ __forceinline__ unsigned pack_bf16(float a, float b) {
    return __builtin_bit_cast(unsigned, __builtin_convertvector(f32x2{a, b}, bf16x2));
}

// Lane-dependent LDS offsets (see the bf16 MFMA scan for the derivation):
//  * row reads: lane (c32, hf) reads row base + c32, 16-byte chunk 2ks + hf;
//  * transpose reads: within each 16-lane group lane m supplies row first + 4hf + m/4, columns
//    col0 + 16g + 4(m%4) .. +3; the receiving lane (c32, hf) then holds column col0 + c32 at
//    tokens first + 4hf + {0..3}; reads at first and first + 8 give an operand's 8 slots in the
//    row order of a 32x32 accumulator.
struct LaneOff {
    int row[8];
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
    template <int RB> __device__ __forceinline__ int tr(int col0, int h) const {
        return rl * RB + ((((col0 >> 3) + cl) ^ rkey<RB>(rl + 8 * h)) << 4) + hb;
    }
};

__device__ __forceinline__ f16x8 ld16(const unsigned char* p) { return *reinterpret_cast<const f16x8*>(p); }

template <int RB>
__device__ __forceinline__ f16x8 tr_frag(const unsigned char* t, int b0, int b8, int j0) {
    const bf16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)(lds_bf16*)(t + b0 + j0 * RB));
    const bf16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)(lds_bf16*)(t + b8 + (j0 + 8) * RB));
    const f16x4 l = __builtin_bit_cast(f16x4, lo), h = __builtin_bit_cast(f16x4, hi);
    return f16x8{l[0], l[1], l[2], l[3], h[0], h[1], h[2], h[3]};
}

// Row broadcast (DPP row_newbcast): every lane of each 16-lane row receives lane K of that row.  Every
// source lane exists, so bound_ctrl (zero for a missing source) changes nothing; with it and no old value
// the compiler no longer copies a zero into each slot's register before the broadcast (15 moves per tile).
template <int K> __device__ __forceinline__ float row_bcast(float v) {
    return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0x150 + K, 0xF, 0xF, true));
}
// m[k] = (m[k] * f_k) a, f_k = lane k of this lane's row of f: the column factors of an accumulator
// whose slot k sits on the key token that lane k of the row holds the factor of
template <int... K>
__device__ __forceinline__ void scale_cols(f32x16& m, float f, float a, std::integer_sequence<int, K...>) {
    ((m[K] = (m[K] * row_bcast<K>(f)) * a), ...);
}

// Workspace of one call, per (batch, group, chunk) tile index:
//   BT  32 KiB  B'^T in the state waves' register order: n tile t, token step ks, lane l: 16 bytes
//               B'[16ks + 4(l/32) + {0..3, 8..11}][32t + l%32] (the slot order of an MFMA operand whose k
//               runs over tokens);
//   C   32 KiB  C' in the y waves' register order: token tile t, k step ks, lane l: 16 bytes
//               C'[32t + l%32][16ks + 8(l/32) + 0..7];
//   CB  20 KiB  the ten causal 32x32 tiles of (C'.B'^T)^T 2^-kCBShift in fp16 (rows: key tokens j; columns:
//               tokens i), tile (it, jt) at index it(it+1)/2 + jt, the four diagonal tiles zero where j > i;
//               within a tile, accumulator values 8h .. 8h+7 of lane l at 16 (64h + l), so that each 16-byte
//               load of a wave reads 1 KiB in one run;
// then per (batch, head, chunk) the 128 dt values after the dt prologue (fp32, 0 past the sequence end),
// then the (eB, eC) pairs.  C.B^T is the same for every head of a group, so it is computed here once; the
// per-head dt rows replace 128 scattered 2-byte reads (one cache line each) by one 512-byte read.
// |C'.B'^T| < N 2^15 2^15 = 2^37, so the fp16 copy with the shift below stays under 2^14.
constexpr int kCBShift = 23;
constexpr int kDtHeads = 32;                       // most heads per group whose dt the pre-pass reads as rows
constexpr int kDtItems = kDtHeads / 8 * Q / 256;   // 16-byte dt loads per thread
constexpr int kCBBytes = 10 * 2048;
constexpr int64_t kWsTile = 2 * kTile + kCBBytes;
struct WsView {
    unsigned char* tiles;
    float* dts;      // [batch * heads * chunks][Q]
    int2* scales;
    int64_t ntile;   // batch * groups * chunks
    __device__ __host__ unsigned char* btile(int64_t i) const { return tiles + i * kWsTile; }
    __device__ __host__ unsigned char* ctile(int64_t i) const { return tiles + i * kWsTile + kTile; }
    __device__ __host__ unsigned char* cbtile(int64_t i) const { return tiles + i * kWsTile + 2 * kTile; }
};
// workspace bytes for ntile (batch, group, chunk) tiles and nhc (batch, head, chunk) dt rows
__host__ __device__ inline int64_t ws_bytes(int64_t ntile, int64_t nhc) {
    return ntile * kWsTile + nhc * Q * static_cast<int64_t>(sizeof(float)) + ntile * static_cast<int64_t>(sizeof(int2));
}

// ---------------------------------------------------------------------------
// The fused conv (ssd_conv_chunk_scan): the scan reads the conv's input xBC instead of its output and
// computes the causal depthwise conv (width 4) + SiLU itself, in the order and rounding of the conv
// kernel -- bias, then taps 0..3 by fused multiply-adds in fp32, SiLU, nearest-even bf16 -- so that its
// results equal conv-then-scan bit for bit.
struct ConvIn {
    const bf16* w;       // [CD, 4] taps (tap 3 multiplies the current token)
    const bf16* bias;    // [CD], or null
    const bf16* s_in;    // [B, CD, 4] conv state: inputs at tokens -4..-1, or null (zeros)
    bf16* s_out;         // [B, CD, 4] new conv state (inputs at tokens L-4..L-1), or null
    const bf16* xbc;     // [B, L, CD] the conv input, row stride xs
    int64_t xs, cd, hp;  // hp = H P: the first B channel
};

__device__ __forceinline__ float bf16_lo(unsigned u) { return __uint_as_float(u << 16); }
__device__ __forceinline__ float bf16_hi(unsigned u) { return __uint_as_float(u & 0xFFFF0000u); }
__device__ __forceinline__ float conv_silu_bf16(float bias, const float* w, float u0, float u1, float u2, float u3) {
    float acc = bias;
    acc = fmaf(w[0], u0, acc);
    acc = fmaf(w[1], u1, acc);
    acc = fmaf(w[2], u2, acc);
    acc = fmaf(w[3], u3, acc);
    return static_cast<float>(static_cast<bf16>(silu_f(acc)));
}

// Pre-pass conv: rows rb .. rb + 7 of the chunk starting at token tok0 of batch entry b, channels ch .. ch + 7;
// inputs before token 0 come from the conv state; rows at or past `valid` are zeros.
__device__ __forceinline__ void conv8_rows(u32x4 (&o)[8], const ConvIn& cv, int64_t b, int64_t seqlen, int64_t tok0,
                                           int rb, int valid, int64_t ch) {
    float w[8][4], bs[8];
    {
        const u32x4* wp = reinterpret_cast<const u32x4*>(cv.w + ch * 4);
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const u32x4 v = wp[q];                   // channels ch + 2q, ch + 2q + 1
#pragma unroll
            for (int e = 0; e < 2; ++e) {
                w[2 * q + e][0] = bf16_lo(v[2 * e]);
                w[2 * q + e][1] = bf16_hi(v[2 * e]);
                w[2 * q + e][2] = bf16_lo(v[2 * e + 1]);
                w[2 * q + e][3] = bf16_hi(v[2 * e + 1]);
            }
        }
        u32x4 bv = {0, 0, 0, 0};
        if (cv.bias) bv = *reinterpret_cast<const u32x4*>(cv.bias + ch);
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            bs[2 * q] = bf16_lo(bv[q]);
            bs[2 * q + 1] = bf16_hi(bv[q]);
        }
    }
    float u[11][8];                                  // inputs at rows rb - 3 .. rb + 7
#pragma unroll
    for (int j = 0; j < 11; ++j) {
        const int row = rb - 3 + j;
        const int64_t tok = tok0 + row;
        u32x4 v = {0, 0, 0, 0};
        if (row < valid && tok >= 0) {
            v = *reinterpret_cast<const u32x4*>(cv.xbc + (b * seqlen + tok) * cv.xs + ch);
        } else if (row < valid && cv.s_in) {         // tokens -3 .. -1: the conv state
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const unsigned short lo = reinterpret_cast<const unsigned short*>(cv.s_in)[(b * cv.cd + ch + 2 * q) * 4 + 4 + tok];
                const unsigned short hi = reinterpret_cast<const unsigned short*>(cv.s_in)[(b * cv.cd + ch + 2 * q + 1) * 4 + 4 + tok];
                v[q] = static_cast<unsigned>(lo) | (static_cast<unsigned>(hi) << 16);
            }
        }
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            u[j][2 * q] = bf16_lo(v[q]);
            u[j][2 * q + 1] = bf16_hi(v[q]);
        }
    }
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        bf16x8 r;
#pragma unroll
        for (int e = 0; e < 8; ++e)
            r[e] = static_cast<bf16>(rb + j < valid ? conv_silu_bf16(bs[e], w[e], u[j][e], u[j + 1][e], u[j + 2][e], u[j + 3][e])
                                                  : 0.f);
        o[j] = __builtin_bit_cast(u32x4, r);
    }
}

// The new conv state of channel ch: the inputs at tokens L-4 .. L-1 (from the old state where negative)
__device__ __forceinline__ void conv_state_out(const ConvIn& cv, int64_t b, int64_t seqlen, int64_t ch) {
    unsigned short v[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        const int64_t tau = seqlen - 4 + k;
        if (tau >= 0)
            v[k] = reinterpret_cast<const unsigned short*>(cv.xbc)[(b * seqlen + tau) * cv.xs + ch];
        else
            v[k] = cv.s_in ? reinterpret_cast<const unsigned short*>(cv.s_in)[(b * cv.cd + ch) * 4 + 4 + tau] : 0;
    }
    *reinterpret_cast<uint2*>(cv.s_out + (b * cv.cd + ch) * 4) =
        uint2{v[0] | (static_cast<unsigned>(v[1]) << 16), v[2] | (static_cast<unsigned>(v[3]) << 16)};
}

// Packed batches (cu_seqlens): chunk c of sequence s (first row start) takes workspace chunk slot
// s + floor(start / Q) + c.  floor(a / Q) + ceil(L / Q) <= floor((a + L) / Q) + 1 keeps the slots of distinct
// (sequence, chunk) pairs distinct, and below S + ceil(T / Q) for any table clamped into [0, T].
__device__ __forceinline__ int64_t packed_slot0(int64_t s, int64_t start) { return s + start / Q; }
__host__ __device__ inline int64_t packed_slots(int64_t nseq, int64_t rows) { return nseq + (rows + Q - 1) / Q; }

// ---------------------------------------------------------------------------
// Pre-pass: one workgroup of 256 threads per (batch, group, chunk); packed batches: per (group, chunk slot),
// the workgroups of unused slots return at once.  Thread t holds 16-byte pieces
// t + 256k (k < 8) of the B tile and of the C tile (piece i: row i / 16, chunk i % 16); rows past the
// sequence end are zeros.  The scaled fp16 tiles are staged in LDS, from which the four waves write B'^T
// (transpose reads) and compute the causal C'.B'^T tiles (wave w: tiles w, w + 4, w + 8).
// Fused conv: thread t computes channel piece t % 16 of B and of C over rows 8 (t / 16) .. + 7 from
// xBC instead (same pieces, another row order), and the chunk-0 workgroup writes the group's new conv state.
template <bool CONV>
__global__ __launch_bounds__(256) void bc_prep_kernel(const bf16* Bg, const bf16* Cg, int64_t bcs, const bf16* dtg,
                                                      DtParams dtp, int64_t seqlen, int nheads, int ngroups,
                                                      int64_t nchunks, WsView ws, ConvIn cv, int64_t batch, SeqMap seq) {
    __shared__ __align__(16) unsigned char lb[kTile];
    __shared__ __align__(16) unsigned char lc[kTile];
    __shared__ unsigned wmax[2][4];
    const int64_t id = blockIdx.x;
    // batched: id = (b G + g) nchunks + c, rows b seqlen + c Q ..; packed (seqlen = all rows, nchunks = chunk
    // slots): id = g nchunks + slot, the slot's sequence found by bisection (the slots' first indices
    // increase with s)
    int64_t c, b, row0, len;
    int g;
    if (seq.cu_seqlens) {
        g = static_cast<int>(id / nchunks);
        const int64_t slot = id % nchunks;
        int64_t lo = 0, hi = batch;                  // the last s with packed_slot0(s) <= slot, in [lo, hi)
        while (hi - lo > 1) {
            const int64_t m = (lo + hi) / 2;
            int64_t st, ln;
            seq_span(seq.cu_seqlens, m, seqlen, st, ln);
            if (packed_slot0(m, st) <= slot) lo = m; else hi = m;
        }
        b = lo;
        seq_span(seq.cu_seqlens, b, seqlen, row0, len);
        c = slot - packed_slot0(b, row0);
        if (c < 0 || c * Q >= len) return;           // no chunk of any sequence here (uniform: before any barrier)
        row0 += c * Q;
    } else {
        c = id % nchunks;
        const int64_t bg = id / nchunks;
        g = static_cast<int>(bg % ngroups);
        b = bg / ngroups;
        row0 = b * seqlen + c * Q;
        len = seqlen;
    }
    // the workspace dt row of head h for this chunk
    auto hrow = [&](int h) {
        return seq.cu_seqlens ? static_cast<int64_t>(h) * nchunks + id % nchunks : (b * nheads + h) * nchunks + c;
    };
    const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
    const int valid = static_cast<int>(len - c * Q < Q ? len - c * Q : Q);
    // dt, read as whole rows with the B and C tiles: item (token j, heads 8q .. 8q + 7 of the group) is one
    // 16-byte load; tokens past the end read nothing.  Used when the group's heads come in 16-byte pieces (at
    // most kDtHeads of them), else the per-head loop at the end.
    const int hpg = nheads / ngroups;
    const int q8 = hpg >> 3;
    const bool dt_rows = hpg <= kDtHeads && (hpg & 7) == 0 && (nheads & 7) == 0 &&
                         (reinterpret_cast<uintptr_t>(dtg) & 15) == 0;
    u32x4 vdt[kDtItems];
    if (dt_rows) {
#pragma unroll
        for (int k = 0; k < kDtItems; ++k) {
            const int item = t + 256 * k, j = item / (q8 > 0 ? q8 : 1);
            vdt[k] = u32x4{0, 0, 0, 0};
            if (item < Q * q8 && j < valid)
                vdt[k] = *reinterpret_cast<const u32x4*>(dtg + (row0 + j) * nheads + g * hpg + 8 * (item % q8));
        }
    }
    u32x4 vb[8], vc[8];
    // piece k of this thread: row, 16-byte chunk
    auto piece_r = [&](int k) { return CONV ? 8 * (t >> 4) + k : (t + 256 * k) >> 4; };
    auto piece_c = [&](int k) { return CONV ? (t & 15) : ((t + 256 * k) & 15); };
    if constexpr (CONV) {
        const int64_t gn = static_cast<int64_t>(g) * NS + 8 * (t & 15);
        conv8_rows(vb, cv, b, seqlen, c * Q, 8 * (t >> 4), valid, cv.hp + gn);
        conv8_rows(vc, cv, b, seqlen, c * Q, 8 * (t >> 4), valid, cv.hp + static_cast<int64_t>(ngroups) * NS + gn);
    }
    u16x2 mb2 = {0, 0}, mc2 = {0, 0};
#pragma unroll
    for (int k = 0; k < 8; ++k) {
        if constexpr (!CONV) {
            const int r = piece_r(k), cc = piece_c(k);
            vb[k] = u32x4{0, 0, 0, 0};
            vc[k] = u32x4{0, 0, 0, 0};
            if (r < valid) {
                const int64_t off = (row0 + r) * bcs + static_cast<int64_t>(g) * NS + 8 * cc;
                // read by this workgroup only: non-temporal (measured 1-3 % faster; the workspace tiles the
                // scan reads, shared by a group's heads through L2, stay cached: non-temporal there cost 10 %)
                vb[k] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(Bg + off));
                vc[k] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(Cg + off));
            }
        }
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            mb2 = __builtin_elementwise_max(mb2, __builtin_bit_cast(u16x2, vb[k][e] & 0x7FFF7FFFu));
            mc2 = __builtin_elementwise_max(mc2, __builtin_bit_cast(u16x2, vc[k][e] & 0x7FFF7FFFu));
        }
    }
    unsigned mb = max(static_cast<unsigned>(mb2[0]), static_cast<unsigned>(mb2[1]));
    unsigned mc = max(static_cast<unsigned>(mc2[0]), static_cast<unsigned>(mc2[1]));
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) {
        mb = max(mb, static_cast<unsigned>(__shfl_xor(static_cast<int>(mb), off, 64)));
        mc = max(mc, static_cast<unsigned>(__shfl_xor(static_cast<int>(mc), off, 64)));
    }
    if (lane == 0) {
        wmax[0][wave] = mb;
        wmax[1][wave] = mc;
    }
    __syncthreads();
    mb = max(max(wmax[0][0], wmax[0][1]), max(wmax[0][2], wmax[0][3]));
    mc = max(max(wmax[1][0], wmax[1][1]), max(wmax[1][2], wmax[1][3]));
    // exponent of the largest magnitude (bf16 bits): scale it into [2^14, 2^15)
    auto scale_of = [](unsigned m) {
        if (m == 0 || m >= 0x7F80u) return 0;                 // zeros, or inf/nan (left to propagate)
        return static_cast<int>(m >> 7) - 127 - 14;
    };
    const int eB = scale_of(mb), eC = scale_of(mc);
    const int64_t tix = id;   // tile index (b, g, c) in the same order
    unsigned char* bt = ws.btile(tix);
    unsigned char* ct = ws.ctile(tix);
    auto conv = [](const u32x4& v, int e) {
        u32x4 o;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const float lo = ldexp_f(__uint_as_float(v[q] << 16), -e);
            const float hi = ldexp_f(__uint_as_float(v[q] & 0xFFFF0000u), -e);
            o[q] = __builtin_bit_cast(unsigned, __builtin_convertvector(f32x2{lo, hi}, f16x2));
        }
        return o;
    };
#pragma unroll
    for (int k = 0; k < 8; ++k) {
        const int r = piece_r(k), cc = piece_c(k);
        *reinterpret_cast<u32x4*>(lb + soff<kRowB>(r, cc)) = conv(vb[k], eB);
        const u32x4 cv = conv(vc[k], eC);
        *reinterpret_cast<u32x4*>(lc + soff<kRowB>(r, cc)) = cv;
        const int tt = r >> 5, c32 = r & 31, ks = cc >> 1, hf = cc & 1;
        *reinterpret_cast<u32x4*>(ct + (((tt * 8 + ks) * 64) + hf * 32 + c32) * 16) = cv;
    }
    __syncthreads();
    const LaneOff lo(lane);
    const int c32 = lane & 31, hf = lane >> 5;
    {   // B'^T: wave w writes the fragments of n tile w
        const int b0 = lo.tr<kRowB>(32 * wave, 0), b8 = lo.tr<kRowB>(32 * wave, 1);
#pragma unroll
        for (int k = 0; k < 8; ++k)
            *reinterpret_cast<f16x8*>(bt + ((wave * 8 + k) * 64 + lane) * 16) = tr_frag<kRowB>(lb, b0, b8, 16 * k);
    }
    unsigned char* cb = ws.cbtile(tix);
#pragma unroll
    for (int T = wave; T < 10; T += 4) {
        const int it = T >= 6 ? 3 : (T >= 3 ? 2 : (T >= 1 ? 1 : 0));
        const int jt = T - it * (it + 1) / 2;
        f32x16 acc = zero16();
#pragma unroll
        for (int ks = 0; ks < 8; ++ks)
            acc = mfma(ld16(lb + 32 * jt * kRowB + lo.row[ks]), ld16(lc + 32 * it * kRowB + lo.row[ks]), acc);
        if (it == jt) {   // a diagonal tile: zero above the diagonal (key token after the token), the causal mask
#pragma unroll
            for (int e = 0; e < 16; ++e)
                if (8 * (e >> 2) + 4 * (lane >> 5) + (e & 3) > (lane & 31)) acc[e] = 0.f;
        }
        f16x8* dst = reinterpret_cast<f16x8*>(cb + T * 2048) + lane;
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            float v[8];
#pragma unroll
            for (int k = 0; k < 8; ++k) v[k] = ldexp_f(acc[8 * h + k], -kCBShift);
            dst[64 * h] = to_f16x8(v);
        }
    }
    // the dt rows of the group's heads (each store instruction of a wave writes 64-byte runs of 4 rows); else
    // item (head hh, 16-token segment sg) read per element
    if (dt_rows) {
#pragma unroll
        for (int k = 0; k < kDtItems; ++k) {
            const int item = t + 256 * k;
            if (item < Q * q8) {
                const int j = item / q8, h0 = 8 * (item % q8);
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    const unsigned u = vdt[k][e >> 1];
                    const float raw = (e & 1) ? bf16_hi(u) : bf16_lo(u);
                    const int h = g * hpg + h0 + e;
                    ws.dts[hrow(h) * Q + j] = j < valid ? dt_prologue(raw, dtp, h) : 0.f;
                }
            }
        }
    } else for (int item = t; item < hpg * 8; item += 256) {
        const int hh = item >> 3, sg = item & 7, h = g * hpg + hh;
        float v[16];
#pragma unroll
        for (int k = 0; k < 16; ++k) {
            const int j = 16 * sg + k;
            v[k] = j < valid ? dt_prologue(static_cast<float>(dtg[(row0 + j) * nheads + h]), dtp, h) : 0.f;
        }
        f32x4* dst = reinterpret_cast<f32x4*>(ws.dts + hrow(h) * Q + 16 * sg);
#pragma unroll
        for (int k = 0; k < 4; ++k) dst[k] = f32x4{v[4 * k], v[4 * k + 1], v[4 * k + 2], v[4 * k + 3]};
    }
    if (t == 0) ws.scales[tix] = int2{eB, eC};
    if constexpr (CONV) {
        // the group's new conv state, written by the workgroup that read the old one (the state may be
        // updated in place): 128 B channels, then 128 C channels
        if (c == 0 && cv.s_out) {
            __syncthreads();
            const int64_t gch = static_cast<int64_t>(g) * NS + (t & 127);
            conv_state_out(cv, b, seqlen, cv.hp + (t < 128 ? 0 : static_cast<int64_t>(ngroups) * NS) + gch);
        }
    }
}

// ---------------------------------------------------------------------------
struct Ctx {
    const bf16* xg; const bf16* dtg;
    int64_t xs, seqlen, b;   // seqlen: this sequence's rows; b: its batch entry (packed: sequence)
    int64_t rowbase;         // its first token row
    int64_t sslot;           // its state row in init_state / final_state (packed: pool slot; -1: none)
    bool use_init;           // it starts from init_state (else from zeros)
    int H, h, grp, nchunks;
    int64_t tile0;      // workspace tile index of this (batch, group)'s chunk 0
    int64_t hrow0;      // workspace dt row of this (batch, head)'s chunk 0
    WsView ws;
    ConvIn cv;          // fused conv only
    __device__ __forceinline__ int valid(int c) const {
        const int64_t r = seqlen - static_cast<int64_t>(c) * Q;
        return r < Q ? static_cast<int>(r) : Q;
    }
    __device__ __forceinline__ int64_t row0(int c) const { return rowbase + static_cast<int64_t>(c) * Q; }
};

// ---------------------------------------------------------------------------
// Fused conv: the scale of chunk x tile from its raw inputs' largest magnitude (bf16 bits, over the chunk's
// rows and the 3 before them) -- the conv's result is bounded by |bias| + sum_k |w_k| max|u| (fp32 rounding
// and the bf16 rounding of SiLU's result add under 2^-7), and |silu(z)| <= |z| -- with the rule of the
// unfused path applied to that bound.  Returns ex; maxx receives the bound.
__device__ __forceinline__ int conv_scale(const Smem& sm, int slot, float& maxx) {
    const unsigned m = max(sm.xmax[slot][0], sm.xmax[slot][1]);
    const float mu = __uint_as_float(m << 16);
    maxx = (sm.cbound[0] + sm.cbound[1] * mu) * (1.f + 0x1p-7f);
    const int e = ilog2f(maxx);
    return (maxx == 0.f || !(maxx < 3.0e38f)) ? 0 : ((e >= 15 || e < -8) ? e - 14 : 0);
}

// Fused conv: slice w turns rows 16w .. 16w+15 of chunk c1's raw tile into its fp16 x tile
// (x' = bf16(silu(conv)) 2^-ex); lane l takes channels 8 (l % 8) .. + 7 of rows 16w + 2 (l / 8) + {0, 1}.
// The slices each wave takes (-1: none): y waves 0..3, state waves 4, 5 (no registers to spare), loaders
// 6, 7 (they convert nothing in this mode).  The lighter waves take more: timed at 1 x 8192, 256 heads,
// this split runs the fused call in 323 us; one slice per y wave and two per loader, 344 us.
#ifndef SSD_CONV_SLICES
#define SSD_CONV_SLICES {{0, 1, -1}, {2, -1, -1}, {-1, -1, -1}, {-1, -1, -1}, {-1, -1, -1}, {-1, -1, -1}, {3, 4, -1}, {5, 6, 7}}
#endif
constexpr int kConvSlices[8][3] = SSD_CONV_SLICES;
__device__ __forceinline__ void conv_slice(Smem& sm, int wave, int lane, int c1);
template <int W>
__device__ __forceinline__ void conv_slices(Smem& sm, int lane, int c1) {
#pragma unroll
    for (int k = 0; k < 3; ++k)
        if (kConvSlices[W][k] >= 0) conv_slice(sm, kConvSlices[W][k], lane, c1);
}
__device__ __forceinline__ void conv_slice(Smem& sm, int wave, int lane, int c1) {
    float maxx;
    const int ex = conv_scale(sm, c1 & 1, maxx);
    const unsigned char* xr = sm.Xr[c1 & 1];
    unsigned char* xt = sm.X[c1 & 1];
    const int pc = lane & 7, r0 = 16 * wave + 2 * (lane >> 3);
    u32x4 raw[5];                                    // inputs at rows r0 - 3 .. r0 + 1
#pragma unroll
    for (int j = 0; j < 5; ++j) raw[j] = *reinterpret_cast<const u32x4*>(xr + soff<kRowX>(r0 + j, pc));
    float acc[2][8];
    {
        const f32x4 b0 = *reinterpret_cast<const f32x4*>(&sm.cw[4][8 * pc]);
        const f32x4 b1 = *reinterpret_cast<const f32x4*>(&sm.cw[4][8 * pc + 4]);
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[0][e] = acc[1][e] = e < 4 ? b0[e] : b1[e - 4];
    }
    auto u = [&](int j, int e) { return (e & 1) ? bf16_hi(raw[j][e >> 1]) : bf16_lo(raw[j][e >> 1]); };
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        const f32x4 w0 = *reinterpret_cast<const f32x4*>(&sm.cw[k][8 * pc]);
        const f32x4 w1 = *reinterpret_cast<const f32x4*>(&sm.cw[k][8 * pc + 4]);
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const float w = e < 4 ? w0[e] : w1[e - 4];
            acc[0][e] = fmaf(w, u(k, e), acc[0][e]);
            acc[1][e] = fmaf(w, u(k + 1, e), acc[1][e]);
        }
    }
#pragma unroll
    for (int j = 0; j < 2; ++j) {
        float v[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const float o = static_cast<float>(static_cast<bf16>(silu_f(acc[j][e])));
            v[e] = ex == 0 ? o : ldexp_f(o, -ex);
        }
        *reinterpret_cast<f16x8*>(xt + soff<kRowX>(r0 + j, pc)) = to_f16x8(v);
    }
}

// ---------------------------------------------------------------------------
// y wave: token tile IT, both p tiles.
template <typename TY, int IT, bool CONV>
__device__ void run_y(Smem& sm, const ScanArgs& a, const Ctx& cx, const int lane) {
    const int c32 = lane & 31, hf = lane >> 5;
    const int i = 32 * IT + c32;                     // this lane's token within the chunk
    TY* yg = static_cast<TY*>(a.y);
    const LaneOff lo(lane);
    const int trX0 = lo.tr<kRowX>(0, 0), trX1 = lo.tr<kRowX>(32, 0);
    // the key token whose column factor this lane holds for the row broadcasts: slot k = lane % 16 of
    // an accumulator of this half-wave
    const int rb = 8 * ((lane & 15) >> 2) + 4 * hf + (lane & 3);

    // this lane's C' operand of chunk c, k step ks: C'[i][16ks + 8hf .. +7]
    auto c_load = [&](f16x8 (&cr)[8], int c) {
        const unsigned char* src = cx.ws.ctile(cx.tile0 + c) + ((IT * 8) * 64 + lane) * 16;
#pragma unroll
        for (int ks = 0; ks < 8; ++ks) cr[ks] = *reinterpret_cast<const f16x8*>(src + ks * 64 * 16);
    };
    // this lane's 16 values of the pre-pass C'.B'^T tile (IT, jt) of chunk c (fp16, in units of 2^kCBShift)
    struct CbReg { f16x8 h0, h1; };
    auto cb_load = [&](int c, int jt) {
        const f16x8* src = reinterpret_cast<const f16x8*>(cx.ws.cbtile(cx.tile0 + c) + (IT * (IT + 1) / 2 + jt) * 2048) +
                           lane;
        return CbReg{src[0], src[64]};
    };
    auto cb_f32 = [](const CbReg& r) {
        f32x16 m;
#pragma unroll
        for (int k = 0; k < 8; ++k) {
            m[k] = static_cast<float>(r.h0[k]);
            m[8 + k] = static_cast<float>(r.h1[k]);
        }
        return m;
    };
    // bf16 y: each chunk's 32 x 64 block goes to this wave's LDS stage (rows of 128 bytes, 16-byte chunks
    // XOR-permuted), is read back at the next chunk's start as whole rows and stored after that chunk's
    // C.H: 8 rows per store instead of 32 partial ones, and -- since loads and stores share one vector-
    // memory counter, so that a wait for a load also waits for earlier stores -- after the first wait for
    // that chunk's loads, which leaves the stores a whole chunk to complete.  The stores are non-temporal:
    // y is written once, and dirty y lines left in the caches cost the next launch their write-back.
    u32x4 yq[4];                                     // lane l: row 8k + l/8, 16-byte piece l%8
    unsigned char* st = sm.stage[IT];
    int yq_valid = 0;                                // valid tokens of the staged chunk
    TY* yq_row = nullptr;                            // its first y row (null: nothing staged)
    auto stage_read = [&]() {
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            const int r = 8 * k + (lane >> 3), ch = lane & 7;
            yq[k] = *reinterpret_cast<const u32x4*>(st + r * kRowX + ((ch ^ ((r >> 1) & 7)) << 4));
        }
    };
    auto flush_y = [&]() {
        if constexpr (sizeof(TY) == 2) {
            if (yq_row != nullptr) {
#pragma unroll
                for (int k = 0; k < 4; ++k) {
                    const int r = 8 * k + (lane >> 3);
                    if (32 * IT + r < yq_valid)
                        __builtin_nontemporal_store(yq[k], reinterpret_cast<u32x4*>(
                            yq_row + (32 * IT + r) * static_cast<int64_t>(cx.H) * P + 8 * (lane & 7)));
                }
            }
        }
    };
    // rolling prefetch: each register set is reloaded with the next chunk's data right after its last use
    f16x8 cf[8];
    CbReg cb[IT + 1];
    if (cx.nchunks > 0) {
        c_load(cf, 0);
#pragma unroll
        for (int jt = 0; jt <= IT; ++jt) cb[jt] = cb_load(0, jt);
    }
    __syncthreads();                                 // prologue 1
    if constexpr (CONV) {
        if (cx.nchunks > 0) conv_slices<IT>(sm, lane, 0);
    }
    __syncthreads();                                 // chunk 0

    for (int c = 0; c < cx.nchunks; ++c) {
        const int valid = cx.valid(c);
        const int buf = c & 1;
        // the chunk whose values the reloads fetch: the last chunk reloads itself (in bounds, unused), which
        // keeps the loads unconditional and in place
        const int cnext = c + 1 < cx.nchunks ? c + 1 : c;
        // (tokens past a ragged chunk's end are computed like the others, from zero B and C rows and
        // zero dt, and never stored)
        const Vec& v = sm.vec[buf];
        const unsigned char* Xt = sm.X[buf];
        const unsigned char* Ht = sm.H[buf];
        if constexpr (sizeof(TY) == 2) stage_read();
        // per-chunk factors, issued with the C.H operands: cs_i, the tiles' end values, and this lane's
        // column factor of each key tile (off-diagonal fM, diagonal vD) for the row broadcasts
        const float csi = v.cs[i];
        const f32x4 csE = *reinterpret_cast<const f32x4*>(v.csE);
        float fcol[IT + 1];
#pragma unroll
        for (int jt = 0; jt < IT; ++jt) fcol[jt] = v.fM[32 * jt + rb];
        fcol[IT] = v.vD[32 * IT + rb];

        // carried state: y^T[p][i] = sum_n H'[p][n] C'[i][n], p tiles 0 and 1; the fragments are
        // read in batches of 4, two batches ahead of the MFMAs that use them
        f32x16 y0 = zero16(), y1 = zero16();
        {
            auto hfrag = [&](int k) { return ld16(Ht + (k & 1) * 32 * kRowB + lo.row[k >> 1]); };   // k = 2ks + pt
            f16x8 hv[12];
#pragma unroll
            for (int k = 0; k < 8; ++k) hv[k] = hfrag(k);
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                if (g < 2) {
#pragma unroll
                    for (int k = 4 * g + 8; k < 4 * g + 12; ++k) hv[k % 12] = hfrag(k);
                }
                __builtin_amdgcn_sched_barrier(0);
#pragma unroll
                for (int k = 4 * g; k < 4 * (g + 1); ++k) {
                    if (k & 1) y1 = mfma(hv[k % 12], cf[k >> 1], y1);
                    else y0 = mfma(hv[k % 12], cf[k >> 1], y0);
                }
                __builtin_amdgcn_sched_barrier(0);
            }
        }
        flush_y();                                   // the previous chunk's y (C.H waited for every load)
        // the next chunk's C rows: issued after C.H, so that they do not hold up its LDS reads behind
        // the memory traffic every wave starts at the chunk boundary
        c_load(cf, cnext);
        // into the units of y: exp2(cs_i) 2^(eHc + eC - eM)
        const float ey = ldexp_f(fexp2(csi), v.eHc + v.eC - v.eM);
        y0 *= ey;
        y1 *= ey;

        // causal key tiles: the C'.B'^T tile (acc rows = key tokens j, cols = tokens i), M' in
        // registers, y^T[p][i] += sum_j X'^T[p][j] M'^T[j][i]; the X^T operands of the next tile are
        // read while this one is scaled
        const int sM = v.sM + kCBShift;             // m holds C'.B'^T 2^-kCBShift
        auto x_frags = [&](f16x8 (&xr)[4], int jt) {
#pragma unroll
            for (int q = 0; q < 2; ++q) {
                xr[2 * q] = tr_frag<kRowX>(Xt, trX0, trX0, 32 * jt + 16 * q);
                xr[2 * q + 1] = tr_frag<kRowX>(Xt, trX1, trX1, 32 * jt + 16 * q);
            }
        };
        f16x8 xc[4];
        x_frags(xc, 0);
#pragma unroll
        for (int jt = 0; jt <= IT; ++jt) {
            f32x16 m = cb_f32(cb[jt]);   // m[4q + r] = C'_i . B'_jj 2^-kCBShift,  jj = 32jt + 8q + 4hf + r
            __builtin_amdgcn_sched_barrier(0);
            cb[jt] = cb_load(cnext, jt);
            __builtin_amdgcn_sched_barrier(0);
            f16x8 xn[4];
            if (jt < IT) x_frags(xn, jt + 1);
            if (jt < IT) {
                scale_cols(m, fcol[jt], fexp2(csi - csE[jt] + static_cast<float>(sM)),
                           std::make_integer_sequence<int, 16>{});
            } else if (v.diagOK[jt]) {
                const float dx = v.dx;
                scale_cols(m, fcol[jt], fexp2(csi - v.csM[jt] + static_cast<float>(sM)),
                           std::make_integer_sequence<int, 16>{});
#pragma unroll
                for (int k = 0; k < 16; ++k) {      // above the diagonal the pre-pass's tile holds zeros, and
                    const int jj = 32 * jt + 8 * (k >> 2) + 4 * hf + (k & 3);   // both factors are finite there
                    if (jj == i) m[k] += dx;
                }
            } else {                 // steep decay inside the tile: per-element exp2
                const float dx = v.dx;
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const f32x4 cj = *reinterpret_cast<const f32x4*>(&v.cs[32 * jt + 8 * q + 4 * hf]);
                    const f32x4 dj = *reinterpret_cast<const f32x4*>(&v.dt[32 * jt + 8 * q + 4 * hf]);
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        const int jj = 32 * jt + 8 * q + 4 * hf + r;
                        float e = m[4 * q + r] * fexp2(csi - cj[r] + static_cast<float>(sM)) * dj[r];
                        if (jj == i) e += dx;
                        m[4 * q + r] = jj <= i ? e : 0.f;
                    }
                }
            }
#pragma unroll
            for (int q = 0; q < 2; ++q) {
                float mv[8];
#pragma unroll
                for (int s = 0; s < 8; ++s) mv[s] = m[8 * q + s];
                const f16x8 mh = to_f16x8(mv);
                y0 = mfma(xc[2 * q], mh, y0);
                y1 = mfma(xc[2 * q + 1], mh, y1);
            }
            if (jt < IT) {
#pragma unroll
                for (int k = 0; k < 4; ++k) xc[k] = xn[k];
            }
        }

        // y[token i][p] = acc 2^eM.  Lane (c32, hf) holds p = 32pt + 8j + 4hf + r in y_pt[4j + r];
        // swapping j = 1 of the low half-wave with j = 0 of the high one (and 3 with 2) leaves each
        // lane with p = 32pt + 16g + 8hf + {0..7}: two 16-byte pieces per p tile.
        const int eM = v.eM;
        TY* yrow = yg + (cx.row0(c) * cx.H + cx.h) * static_cast<int64_t>(P);
        const int64_t ystr = static_cast<int64_t>(cx.H) * P;
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
                            const float a0 = ldexp_f(yv[8 * g + r], eM), b0 = ldexp_f(yv[8 * g + 4 + r], eM);
                            const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(a0), __float_as_uint(b0),
                                                                             false, false);
                            lo4[r] = sw[0];
                            hi4[r] = sw[1];
                        }
                        *reinterpret_cast<u32x4*>(dst + 32 * pt + 16 * g) = lo4;
                        *reinterpret_cast<u32x4*>(dst + 32 * pt + 16 * g + 4) = hi4;
                    }
                }
            }
        } else {
            // into the stage: lane (c32, hf) holds y[i][32pt + 16g + 8hf .. +7] after the swap
#pragma unroll
            for (int pt = 0; pt < 2; ++pt) {
                const f32x16& yv = pt ? y1 : y0;
#pragma unroll
                for (int g = 0; g < 2; ++g) {
                    u32x4 o;
#pragma unroll
                    for (int h2 = 0; h2 < 2; ++h2) {
                        const unsigned pa = pack_bf16(ldexp_f(yv[8 * g + 2 * h2], eM), ldexp_f(yv[8 * g + 2 * h2 + 1], eM));
                        const unsigned pb = pack_bf16(ldexp_f(yv[8 * g + 4 + 2 * h2], eM),
                                                      ldexp_f(yv[8 * g + 4 + 2 * h2 + 1], eM));
                        const auto sw = __builtin_amdgcn_permlane32_swap(pa, pb, false, false);
                        o[h2] = sw[0];
                        o[2 + h2] = sw[1];
                    }
                    const int ch = 4 * pt + 2 * g + hf;
                    *reinterpret_cast<u32x4*>(st + c32 * kRowX + ((ch ^ ((c32 >> 1) & 7)) << 4)) = o;
                }
            }
            yq_row = yrow;
            yq_valid = valid;
        }
        if constexpr (CONV) {
            if (c + 1 < cx.nchunks) conv_slices<IT>(sm, lane, c + 1);
        }
        __syncthreads();                             // chunk c + 1
    }
    if constexpr (sizeof(TY) == 2) stage_read();
    flush_y();
}

// ---------------------------------------------------------------------------
// state wave SN: n tiles 2SN, 2SN + 1 of both p tiles.  Accumulator u = 2 tt + pt holds
// Hs[u][4q + r] = H[p = 32pt + c32][n = 32(2SN + tt) + 8q + 4hf + r] in units of 2^sH (sH of the last chunk
// processed; 0 for the initial state).  Its B'^T operands come straight from the pre-pass in registers,
// one chunk ahead: each token step's pair is reloaded with the next chunk's right after its MFMAs.
// LP: the initial and final states are 16-bit codes (a separate instantiation, so that the fp32
// kernel carries none of the rounding code)
template <int SN, bool CONV, bool LP>
__device__ __attribute__((always_inline)) void run_s(Smem& sm, const ScanArgs& a, const Ctx& cx, const int lane) {
    const int c32 = lane & 31, hf = lane >> 5;
    const int64_t sbase = (cx.sslot >= 0 ? cx.sslot * cx.H + cx.h : 0) * static_cast<int64_t>(P) * NS;
    const LaneOff lo(lane);
    const int trW0 = lo.tr<kRowX>(0, 0), trW1 = lo.tr<kRowX>(32, 0);
    // element (u, q) of the state: row p, columns n .. n + 3
    auto p_of = [&](int u) { return 32 * (u & 1) + c32; };
    auto n_of = [&](int u, int q) { return 32 * (2 * SN + (u >> 1)) + 8 * q + 4 * hf; };
    f32x16 Hs[4];
    float mx = 0.f;
#pragma unroll
    for (int u = 0; u < 4; ++u)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            f32x4 v4 = {0.f, 0.f, 0.f, 0.f};
            if constexpr (LP) {
                if (a.init16) v4 = codes_load4(a.init16, a.codes.f16, sbase + p_of(u) * NS + n_of(u, q));
            } else {
                if (a.init_state && cx.use_init)
                    v4 = *reinterpret_cast<const f32x4*>(a.init_state + sbase + p_of(u) * NS + n_of(u, q));
            }
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                Hs[u][4 * q + r] = v4[r];
                mx = fmaxf(mx, fabsf(v4[r]));
            }
        }
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) mx = fmaxf(mx, __shfl_xor(mx, off, 64));
    if (lane == 0) sm.hmax[SN] = mx;
    // B'^T operands of chunk c: bq[tt][ks] for n tile 2SN + tt, token step ks
    f16x8 bq[2][8];
    auto b_load = [&](int c, int tt, int ks) {
        return *reinterpret_cast<const f16x8*>(cx.ws.btile(cx.tile0 + c) + (((2 * SN + tt) * 8 + ks) * 64 + lane) * 16);
    };
    if (cx.nchunks > 0) {
#pragma unroll
        for (int ks = 0; ks < 8; ++ks)
#pragma unroll
            for (int tt = 0; tt < 2; ++tt) bq[tt][ks] = b_load(0, tt, ks);
    }
    // fp16 copy of the state in units of 2^e (e.g. H' for the next chunk's C.H), into buffer hb
    auto write_h = [&](int buf, int sh, int e) {
        unsigned char* hb = sm.H[buf];
#pragma unroll
        for (int u = 0; u < 4; ++u)
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                f16x4 h4;
#pragma unroll
                for (int r = 0; r < 4; r += 2) {
                    const f16x2 p2 = __builtin_convertvector(
                        f32x2{ldexp_f(Hs[u][4 * q + r], sh - e), ldexp_f(Hs[u][4 * q + r + 1], sh - e)}, f16x2);
                    h4[r] = p2[0];
                    h4[r + 1] = p2[1];
                }
                *reinterpret_cast<f16x4*>(hb + soff<kRowB>(p_of(u), 4 * (2 * SN + (u >> 1)) + q) + 8 * hf) = h4;
            }
    };
    auto store_state = [&](int sh) {
#pragma unroll
        for (int u = 0; u < 4; ++u)
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const f32x4 v = {ldexp_f(Hs[u][4 * q], sh), ldexp_f(Hs[u][4 * q + 1], sh),
                                 ldexp_f(Hs[u][4 * q + 2], sh), ldexp_f(Hs[u][4 * q + 3], sh)};
                const int64_t e = sbase + p_of(u) * NS + n_of(u, q);
                if constexpr (LP) {
                    // one quad at a time: interleaving the Philox blocks of all 16 quads spills
                    __builtin_amdgcn_sched_barrier(0);
                    codes_store4(a.final16, a.codes, e, v);
                    __builtin_amdgcn_sched_barrier(0);
                } else {
                    *reinterpret_cast<f32x4*>(a.final_state + e) = v;
                }
            }
    };
    __syncthreads();                                 // prologue 1
    {
        const float bound0 = fmaxf(sm.hmax[0], sm.hmax[1]);
        write_h(0, 0, max(ilog2f(bound0), -126) + 1 - 15);
    }
    __syncthreads();                                 // chunk 0

    int sh = 0;                                      // units of Hs
    for (int c = 0; c < cx.nchunks; ++c) {
        const int buf = c & 1;
        const int cnext = c + 1 < cx.nchunks ? c + 1 : c;   // the last chunk reloads itself (unused)
        const Vec& v = sm.vec[buf];
        const unsigned char* Xt = sm.X[buf];
        // H <- dec H, re-expressed in this chunk's units 2^sH (a power-of-two change of units)
        // Units that shrink by more than 2^100 take the change of units per element after the decay, in place.
        const int du = sh - v.sH;
        {
            const float dec = du <= 100 ? ldexp_f(v.dec, du) : v.dec;
#pragma unroll
            for (int u = 0; u < 4; ++u) Hs[u] *= dec;
        }
        if (du > 100) {
#pragma unroll
            for (int u = 0; u < 4; ++u)
#pragma unroll
                for (int e = 0; e < 16; ++e) Hs[u][e] = ldexp_f(Hs[u][e], du);
        }
        sh = v.sH;
        // token step k (tokens 16k .. 16k+15): H^T[n][p] += sum_j B'^T[n][j] (w'_j x'_j)[p].  Steps past a
        // ragged chunk's end add zero weights (w' = 0 there).  The x operands and weights of step k + 2
        // are read from LDS while step k computes (scheduling barriers keep the reads where they are
        // issued: the compiler would otherwise sink them next to their use).
        // The weighted x is one packed fp16 product per pair of values, w'_j x'_j rounded once more after
        // w' itself: both factors are fp16 (|w'| <= 1, |x'| < 2^15), two roundings of 2^-11 each.
        struct Frag {
            f16x8 x0, x1;
            f16x4 w0, w1;
        };
        auto load = [&](Frag& f, int j0) {
            f.x0 = tr_frag<kRowX>(Xt, trW0, trW0, j0);
            f.x1 = tr_frag<kRowX>(Xt, trW1, trW1, j0);
            f.w0 = *reinterpret_cast<const f16x4*>(&v.wS[j0 + 4 * hf]);
            f.w1 = *reinterpret_cast<const f16x4*>(&v.wS[j0 + 8 + 4 * hf]);
        };
        auto wx = [](const f16x8& x, const f16x4& w0, const f16x4& w1) {
            const f16x8 w = __builtin_shufflevector(w0, w1, 0, 1, 2, 3, 4, 5, 6, 7);
            return x * w;
        };
        Frag f[3];
        load(f[0], 0);
        load(f[1], 16);
#pragma unroll
        for (int k = 0; k < 8; ++k) {
            __builtin_amdgcn_sched_barrier(0);
            if (k + 2 < 8) load(f[(k + 2) % 3], 16 * (k + 2));
            __builtin_amdgcn_sched_barrier(0);
            const Frag& g = f[k % 3];
            const f16x8 wx0 = wx(g.x0, g.w0, g.w1), wx1 = wx(g.x1, g.w0, g.w1);
#pragma unroll
            for (int tt = 0; tt < 2; ++tt) {
                Hs[2 * tt] = mfma(bq[tt][k], wx0, Hs[2 * tt]);
                Hs[2 * tt + 1] = mfma(bq[tt][k], wx1, Hs[2 * tt + 1]);
            }
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int tt = 0; tt < 2; ++tt) bq[tt][k] = b_load(cnext, tt, k);
            __builtin_amdgcn_sched_barrier(0);
        }
        if (c + 1 < cx.nchunks) {
            write_h(buf ^ 1, sh, v.eHn);
        } else if (!LP && a.final_state && cx.sslot >= 0) {
            store_state(sh);
        }
        __syncthreads();                             // chunk c + 1
    }
    if constexpr (LP) {
        // after the loop, where its prefetch registers are free for the rounding (sh = 0 without chunks)
        if (a.final16) store_state(sh);
    } else {
        if (cx.nchunks == 0 && a.final_state && cx.sslot >= 0) store_state(0);   // no tokens: the final state is the initial one
    }   // no tokens: the final state is the initial one
}

// ---------------------------------------------------------------------------
// Loader waves 6 and 7: rows 0..31 / 32..127 of each chunk's x tile (wave 6 also builds the vectors,
// so it converts fewer rows).  A chunk's rows are loaded into registers three chunks ahead; two chunks
// ahead each wave takes the largest |x| of its rows and leaves it in LDS; one chunk ahead (after the
// barrier) both read the chunk's maximum, convert their rows to fp16 into the chunk's x tile, and wave 6
// builds the chunk's per-token vectors.  Three register sets rotate (the chunk loop is unrolled by
// three so that they stay registers).
template <int NK>
struct XPart {
    u32x4 v[NK];     // instruction k: lane l holds row r0 + 8k + l/8 of the wave's rows, 16-byte piece l%8
};

template <int NK>
__device__ __forceinline__ void x_load(XPart<NK>& xr, const Ctx& cx, int c, int r0, int lane) {
    const int valid = cx.valid(c);
    const bf16* base = cx.xg + cx.row0(c) * cx.xs + static_cast<int64_t>(cx.h) * P + 8 * (lane & 7);
#pragma unroll
    for (int k = 0; k < NK; ++k) {
        int r = r0 + 8 * k + (lane >> 3);
        r = r < valid ? r : valid - 1;               // past the end: a real row (zero weights)
        xr.v[k] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(base + r * cx.xs));   // read once
    }
}

struct DtRegs {
    f32x2 d;         // dt of tokens 2 lane, 2 lane + 1 (after the prologue; 0 past the end)
    int2 sc;         // (eB, eC) of the chunk
};

__device__ __forceinline__ void dt_load(DtRegs& dr, const Ctx& cx, int c, int lane) {
    dr.d = reinterpret_cast<const f32x2*>(cx.ws.dts + (cx.hrow0 + c) * Q)[lane];
    dr.sc = cx.ws.scales[cx.tile0 + c];
}

// Wave-wide inclusive scans with DPP lane moves (VALU, no LDS round trips): shifts by 1, 2, 4 and 8
// inside each 16-lane row (lanes shifted in from outside the row read 0), then the last lane of rows
// 0 and 2 into rows 1 and 3, then lane 31 into rows 2 and 3.  Valid for operations with identity 0
// on the values involved (sums; maxima of non-negative values).
template <int CTRL, int RMASK, bool BC>
__device__ __forceinline__ unsigned dpp_u(unsigned x) {
    return static_cast<unsigned>(__builtin_amdgcn_update_dpp(0, static_cast<int>(x), CTRL, RMASK, 0xF, BC));
}
template <class OP>
__device__ __forceinline__ unsigned wave_scan_bits(unsigned v, OP op) {
    v = op(v, dpp_u<0x111, 0xF, true>(v));
    v = op(v, dpp_u<0x112, 0xF, true>(v));
    v = op(v, dpp_u<0x114, 0xF, true>(v));
    v = op(v, dpp_u<0x118, 0xF, true>(v));
    v = op(v, dpp_u<0x142, 0xA, false>(v));
    v = op(v, dpp_u<0x143, 0xC, false>(v));
    return v;
}
__device__ __forceinline__ float wave_incl_sum(float v) {
    return __uint_as_float(wave_scan_bits(__float_as_uint(v), [](unsigned a, unsigned b) {
        return __float_as_uint(__uint_as_float(a) + __uint_as_float(b));
    }));
}
__device__ __forceinline__ unsigned wave_max_u(unsigned m) {
    return static_cast<unsigned>(__builtin_amdgcn_readlane(
        static_cast<int>(wave_scan_bits(m, [](unsigned a, unsigned b) { return a > b ? a : b; })), 63));
}
__device__ __forceinline__ float wave_max_f(float m) {      // m >= 0
    return __int_as_float(__builtin_amdgcn_readlane(static_cast<int>(wave_scan_bits(__float_as_uint(m),
        [](unsigned a, unsigned b) { return __float_as_uint(fmaxf(__uint_as_float(a), __uint_as_float(b))); })), 63));
}
__device__ __forceinline__ float wave_sum_f(float m) {
    return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(wave_incl_sum(m)), 63));
}
__device__ __forceinline__ float lane_f(float v, int l) { return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), l)); }
// value of lane 16 (l / 16) + k, for each lane l (k wave-uniform)
__device__ __forceinline__ float row_lane_f(float v, int k, int lane) {
    const float r0 = lane_f(v, k), r1 = lane_f(v, 16 + k), r2 = lane_f(v, 32 + k), r3 = lane_f(v, 48 + k);
    const int row = lane >> 4;
    return row == 0 ? r0 : (row == 1 ? r1 : (row == 2 ? r2 : r3));
}

// largest |x| of a wave's rows, as bf16 bits
template <int NK>
__device__ __forceinline__ unsigned half_max(const XPart<NK>& xr) {
    u16x2 m2 = {0, 0};
#pragma unroll
    for (int k = 0; k < NK; ++k)
#pragma unroll
        for (int e = 0; e < 4; ++e) m2 = __builtin_elementwise_max(m2, __builtin_bit_cast(u16x2, xr.v[k][e] & 0x7FFF7FFFu));
    return wave_max_u(max(static_cast<unsigned>(m2[0]), static_cast<unsigned>(m2[1])));
}

// the chunk's x scale from the largest |x| (bf16 bits): 0 while it lies in [2^-8, 2^15)
__device__ __forceinline__ int x_scale(unsigned mb) {
    const int e = static_cast<int>(mb >> 7) - 127;
    return (mb == 0 || mb >= 0x7F80u) ? 0 : ((e >= 15 || e < -8) ? e - 14 : 0);
}

// a wave's rows -> fp16 x' = x 2^-ex into x tile xt
template <int NK>
__device__ __forceinline__ void x_convert(const XPart<NK>& xr, unsigned char* xt, int r0, int ex, int lane) {
    const int rp = lane >> 3, pc = lane & 7;
    auto convert = [&](auto scale) {
#pragma unroll
        for (int k = 0; k < NK; ++k) {
            u32x4 o;
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const float lo = scale(__uint_as_float(xr.v[k][q] << 16));
                const float hi = scale(__uint_as_float(xr.v[k][q] & 0xFFFF0000u));
                o[q] = __builtin_bit_cast(unsigned, __builtin_convertvector(f32x2{lo, hi}, f16x2));
            }
            *reinterpret_cast<u32x4*>(xt + soff<kRowX>(r0 + 8 * k + rp, pc)) = o;
        }
    };
    if (ex == 0) convert([](float f) { return f; });
    else convert([ex](float f) { return ldexp_f(f, -ex); });
}

// Chunk c's per-token vectors and scale exponents into v.  ex: the chunk's x scale; maxx: its largest |x|
// (or a bound on it);
// bound: the bound on |H| at the chunk's start (updated to the bound at its end); eH, sHp: units of the
// state copy the chunk reads and of the state accumulator before it (updated for the next chunk).
__device__ __forceinline__ void build_vec(const DtRegs& dr, int ex, float maxx, Vec& v, const Ctx& cx, const ScanArgs& a,
                                          int c, int lane, float A2, float Dh, float& bound, int& eH, int& sHp) {
    // per-token vectors (two tokens per lane)
    const int valid = cx.valid(c);
    const int h = cx.h;
    const float d0 = dr.d[0], d1 = dr.d[1];
    const float a0 = d0 * A2, a1 = d1 * A2;
    const float s = wave_incl_sum(a0 + a1);
    const float c1 = s, c0 = s - a1;                  // inclusive sums at tokens 2 lane + 1 and 2 lane
    const int last = valid - 1;
    const float csl = (last & 1) ? lane_f(c1, last >> 1) : lane_f(c0, last >> 1);
    const float ce = row_lane_f(c1, 15, lane);                 // end of this lane's 32-token tile
    const float cm = row_lane_f(c1, 7, lane);                  // token 15 of the tile
    const float cf = row_lane_f(c0, 0, lane);                  // first token of the tile
    const float maxdt = wave_max_f(fmaxf(d0, d1));
    const int eB = dr.sc.x, eC = dr.sc.y;
    const int j0 = 2 * lane, j1 = 2 * lane + 1;
    const float w0 = j0 < valid ? fexp2(csl - c0) * d0 : 0.f;
    const float w1 = j1 < valid ? fexp2(csl - c1) * d1 : 0.f;
    const float sumw = wave_sum_f(w0 + w1);
    // scale exponents (integer arithmetic on bounds)
    const int ldt = max(ilog2f(maxdt), -100);
    const int ebM = max(max(37 + eB + eC + ldt + 1, ilog2f(Dh) + 1) + 1, eB + eC - 45);
    const int eM = ex + ebM - 15;
    const int sM = eB + eC + ex - eM;
    const float sbound = sumw * maxx * ldexp_f(1.f, eB + 15);
    const float dec = fexp2(csl);
    const float bnext = dec * bound + sbound;
    const int lbn = max(ilog2f(bnext), -126);
    const int ew = max(ex + ldt + 1, lbn + 1 - eB - 120);
    v.cs[j0] = c0;
    v.cs[j1] = c1;
    v.dt[j0] = d0;
    v.dt[j1] = d1;
    v.fM[j0] = fexp2(ce - c0) * d0;
    v.fM[j1] = fexp2(ce - c1) * d1;
    const float range = cf - ce;                              // the tile's decay range (>= 0)
    const bool dok = range < 48.f;
    v.vD[j0] = dok ? fexp2(cm - c0) * d0 : 0.f;
    v.vD[j1] = dok ? fexp2(cm - c1) * d1 : 0.f;
    v.wS[j0] = static_cast<f16>(ldexp_f(w0, ex - ew));
    v.wS[j1] = static_cast<f16>(ldexp_f(w1, ex - ew));
    if ((lane & 15) == 15) {
        v.csE[lane >> 4] = c1;
        v.diagOK[lane >> 4] = dok ? 1 : 0;
    }
    if ((lane & 15) == 7) v.csM[lane >> 4] = c1;
    if (lane == 0) {
        v.dec = dec;
        v.dx = ldexp_f(Dh, ex - eM);
        v.eB = eB;
        v.eC = eC;
        v.ex = ex;
        v.sM = sM;
        v.eM = eM;
        v.ew = ew;
        v.sH = eB + ew;
        v.sHp = sHp;
        v.eHc = eH;
        v.eHn = lbn + 1 - 15;
    }
    bound = bnext;
    eH = lbn + 1 - 15;
    sHp = eB + ew;
}

// Loader wave for rows 64 half .. 64 half + 63 (half 0: wave 6, which also builds the vectors; half 1:
// wave 7, which also copies each next chunk's B tile from the pre-pass into LDS).
template <int HALF, bool CONV>
__device__ void run_x(Smem& sm, const ScanArgs& a, const Ctx& cx, const int lane) {
    // wave 6: rows 0..31 (it also builds the vectors), wave 7: 32..127; fused conv (no conversion here,
    // two conv slices each): 0..63 / 64..127
    constexpr int NK = CONV ? 8 : (HALF ? 12 : 4);
    constexpr int R0 = CONV ? 64 * HALF : (HALF ? 32 : 0);
    using XHalf = XPart<NK>;
    const float A2 = a.A[cx.h] * kLog2e;
    const float Dh = a.D ? a.D[cx.h] : 0.f;
    const int nc = cx.nchunks;
    XHalf r0, r1, r2;           // register set m % 3 holds chunk m
    DtRegs d0, d1, d2;
    if (nc > 0) x_load(r0, cx, 0, R0, lane);
    if (nc > 1) x_load(r1, cx, 1, R0, lane);
    if (nc > 2) x_load(r2, cx, 2, R0, lane);
    if constexpr (HALF == 0) {
        if (nc > 0) dt_load(d0, cx, 0, lane);
        if (nc > 1) dt_load(d1, cx, 1, lane);
        if (nc > 2) dt_load(d2, cx, 2, lane);
    }
    // fused conv: a chunk's raw rows into Xr (after the 3 rows before the chunk), and wave 7's share of the
    // next chunk's first rows: rows 125..127 of chunk rp (lanes 40..63 of its last instruction)
    auto raw_write = [&](const XHalf& xr, int slot) {
#pragma unroll
        for (int k = 0; k < NK; ++k)
            *reinterpret_cast<u32x4*>(sm.Xr[slot] + soff<kRowX>(3 + R0 + 8 * k + (lane >> 3), lane & 7)) = xr.v[k];
    };
    auto halo_write = [&](const XHalf& rp, int slot) {
        if constexpr (HALF == 1) {
            if (lane >= 40) *reinterpret_cast<u32x4*>(sm.Xr[slot] + soff<kRowX>((lane >> 3) - 5, lane & 7)) = rp.v[NK - 1];
        }
    };
    // largest |raw| of this wave's rows of a chunk, with (wave 7) the 3 rows before it from the previous chunk
    auto raw_max = [&](const XHalf& xr, const XHalf& rp) {
        unsigned m = half_max(xr);
        if constexpr (HALF == 1) {
            unsigned mh = 0;
            if (lane >= 40) {
                u16x2 m2 = {0, 0};
#pragma unroll
                for (int e = 0; e < 4; ++e) m2 = __builtin_elementwise_max(m2, __builtin_bit_cast(u16x2, rp.v[NK - 1][e] & 0x7FFF7FFFu));
                mh = max(static_cast<unsigned>(m2[0]), static_cast<unsigned>(m2[1]));
            }
            m = max(m, wave_max_u(mh));
        }
        return m;
    };
    if constexpr (CONV) {
        if constexpr (HALF == 0) {
            // the head's taps and bias (lane = channel), their bounds, and chunk 0's 3 earlier rows from the
            // conv state (zeros without one)
            const int64_t ch = static_cast<int64_t>(cx.h) * P + lane;
            const uint2 wv = *reinterpret_cast<const uint2*>(cx.cv.w + ch * 4);
            const float w4[4] = {bf16_lo(wv.x), bf16_hi(wv.x), bf16_lo(wv.y), bf16_hi(wv.y)};
            const float bv = cx.cv.bias ? static_cast<float>(cx.cv.bias[ch]) : 0.f;
#pragma unroll
            for (int k = 0; k < 4; ++k) sm.cw[k][lane] = w4[k];
            sm.cw[4][lane] = bv;
            const float sw = fabsf(w4[0]) + fabsf(w4[1]) + fabsf(w4[2]) + fabsf(w4[3]);
            const float mbias = wave_max_f(fabsf(bv)), msw = wave_max_f(sw);
            if (lane == 0) {
                sm.cbound[0] = mbias;
                sm.cbound[1] = msw * (1.f + 0x1p-20f);
            }
            unsigned short sv[3] = {0, 0, 0};
            if (cx.cv.s_in) {
                const uint2 s4 = *reinterpret_cast<const uint2*>(cx.cv.s_in + (cx.b * cx.cv.cd + ch) * 4);
                sv[0] = static_cast<unsigned short>(s4.x >> 16);
                sv[1] = static_cast<unsigned short>(s4.y & 0xFFFFu);
                sv[2] = static_cast<unsigned short>(s4.y >> 16);
            }
            unsigned mh = 0;
#pragma unroll
            for (int j = 0; j < 3; ++j) {
                *reinterpret_cast<unsigned short*>(sm.Xr[0] + soff<kRowX>(j, lane >> 3) + 2 * (lane & 7)) = sv[j];
                mh = max(mh, static_cast<unsigned>(sv[j] & 0x7FFFu));
            }
            if (nc > 0) {
                const unsigned m = max(half_max(r0), wave_max_u(mh));
                if (lane == 0) sm.xmax[0][0] = m;
            }
        } else if (nc > 0) {
            const unsigned m = half_max(r0);
            if (lane == 0) sm.xmax[0][1] = m;
        }
        if (nc > 0) raw_write(r0, 0);
    } else if (nc > 0) {
        const unsigned m = half_max(r0);
        if (lane == 0) sm.xmax[0][HALF] = m;
    }
    __syncthreads();                                 // prologue 1
    float bound = fmaxf(sm.hmax[0], sm.hmax[1]);
    int eH = max(ilog2f(bound), -126) + 1 - 15;      // units of the initial state copy
    int sHp = 0;
    // the scale of chunk c's x tile and its largest |x| (or a bound on it)
    auto x_scale_of = [&](int c, float& maxx) {
        if constexpr (CONV) {
            return conv_scale(sm, c & 1, maxx);
        } else {
            const unsigned mb = max(sm.xmax[c & 1][0], sm.xmax[c & 1][1]);
            maxx = __uint_as_float(mb << 16);
            return x_scale(mb);
        }
    };
    if (nc > 0) {
        float maxx;
        const int ex = x_scale_of(0, maxx);
        if constexpr (!CONV) x_convert(r0, sm.X[0], R0, ex, lane);
        if constexpr (HALF == 0) build_vec(d0, ex, maxx, sm.vec[0], cx, a, 0, lane, A2, Dh, bound, eH, sHp);
        if (nc > 1) {
            const unsigned m = CONV ? raw_max(r1, r0) : half_max(r1);
            if (lane == 0) sm.xmax[1][HALF] = m;
            if constexpr (CONV) {
                raw_write(r1, 1);
                halo_write(r0, 1);
            }
        }
        if constexpr (CONV) {
            conv_slices<6 + HALF>(sm, lane, 0);
        }
    }
    __syncthreads();                                 // chunk 0
    // chunk c: convert chunk c + 1 (rc, dt in dc) -- fused conv: all waves convolve it from its raw tile --
    // take the maximum of chunk c + 2 (rm; fused conv: and put its raw rows in LDS), load chunk c + 3
    // into the sets chunk c used (rl, dl)
    auto phase = [&](int c, XHalf& rc, DtRegs& dc, XHalf& rm, XHalf& rl, DtRegs& dl) {
        if (c + 1 < nc) {
            float maxx;
            const int ex = x_scale_of(c + 1, maxx);
            if constexpr (!CONV) x_convert(rc, sm.X[(c + 1) & 1], R0, ex, lane);
            if constexpr (HALF == 0) build_vec(dc, ex, maxx, sm.vec[(c + 1) & 1], cx, a, c + 1, lane, A2, Dh, bound, eH, sHp);
        }
        if (c + 2 < nc) {
            const unsigned m = CONV ? raw_max(rm, rc) : half_max(rm);
            if (lane == 0) sm.xmax[c & 1][HALF] = m;
            if constexpr (CONV) {
                raw_write(rm, c & 1);
                halo_write(rc, c & 1);
            }
        }
        if (c + 3 < nc) x_load(rl, cx, c + 3, R0, lane);
        if constexpr (HALF == 0) {
            if (c + 3 < nc) dt_load(dl, cx, c + 3, lane);
        }
        if constexpr (CONV) {
            if (c + 1 < nc) {
                conv_slices<6 + HALF>(sm, lane, c + 1);
            }
        }
        __syncthreads();                             // chunk c + 1
    };
    for (int c = 0; c < nc; c += 3) {
        phase(c, r1, d1, r2, r0, d0);
        if (c + 1 >= nc) break;
        phase(c + 1, r2, d2, r0, r1, d1);
        if (c + 2 >= nc) break;
        phase(c + 2, r0, d0, r1, r2, d2);
    }
    if constexpr (CONV && HALF == 0) {
        // the head's new conv state (this workgroup read the old one)
        if (cx.cv.s_out) conv_state_out(cx.cv, cx.b, cx.seqlen, static_cast<int64_t>(cx.h) * P + lane);
    }
}

template <typename TY, bool CONV, bool LP>
__global__ __launch_bounds__(kThreads, 1) void chunk_scan_kernel(ScanArgs a, WsView ws, ConvIn cv) {
    extern __shared__ __align__(16) unsigned char smem_raw[];
    Smem& sm = *reinterpret_cast<Smem*>(smem_raw);
    // XCD-aware numbering: workgroup id % 8 picks the XCD; XCD k takes heads [k H/8, (k+1) H/8) of
    // every batch entry, so a B/C group's heads share that XCD's L2.
    int64_t id = blockIdx.x;
    if (a.nheads % 8 == 0) {
        const int64_t hpx = a.nheads / 8, j = id / 8;
        id = (j / hpx) * a.nheads + (id % 8) * hpx + j % hpx;
    }
    Ctx cx;
    cx.xg = static_cast<const bf16*>(a.x);
    cx.dtg = static_cast<const bf16*>(a.dt);
    cx.xs = a.x_row_stride;
    cx.b = id / a.nheads;
    cx.h = static_cast<int>(id % a.nheads);
    cx.H = a.nheads;
    cx.grp = cx.h / (a.nheads / a.ngroups);
    if (a.seq.cu_seqlens) {      // packed: sequence b's rows, its workspace chunk slots and its pool slot
        seq_span(a.seq.cu_seqlens, cx.b, a.seqlen, cx.rowbase, cx.seqlen);
        const int64_t ns = packed_slots(a.batch, a.seqlen), s0 = packed_slot0(cx.b, cx.rowbase);
        cx.tile0 = cx.grp * ns + s0;
        cx.hrow0 = cx.h * ns + s0;
        cx.sslot = seq_slot(a.seq.slot_idx, cx.b, a.seq.nslots);
        cx.use_init = cx.sslot >= 0 && a.seq.has_init && a.seq.has_init[cx.b] != 0;
    } else {
        cx.seqlen = a.seqlen;
        cx.rowbase = cx.b * a.seqlen;
        const int64_t nc = (a.seqlen + Q - 1) / Q;
        cx.tile0 = (cx.b * a.ngroups + cx.grp) * nc;
        cx.hrow0 = (cx.b * a.nheads + cx.h) * nc;
        cx.sslot = cx.b;
        cx.use_init = true;
    }
    cx.nchunks = static_cast<int>((cx.seqlen + Q - 1) / Q);
    cx.ws = ws;
    cx.cv = cv;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int lane = threadIdx.x & 63;
    if (wave == 0) run_y<TY, 0, CONV>(sm, a, cx, lane);
    else if (wave == 1) run_y<TY, 1, CONV>(sm, a, cx, lane);
    else if (wave == 2) run_y<TY, 2, CONV>(sm, a, cx, lane);
    else if (wave == 3) run_y<TY, 3, CONV>(sm, a, cx, lane);
    else if (wave == 4) run_s<0, CONV, LP>(sm, a, cx, lane);
    else if (wave == 5) run_s<1, CONV, LP>(sm, a, cx, lane);
    else if (wave == 6) run_x<0, CONV>(sm, a, cx, lane);
    else run_x<1, CONV>(sm, a, cx, lane);
}

// A single sequence longer than kSegRows tokens is scanned in segments of kSegRows, chained through an fp32
// state in the workspace: one segment's pre-pass tiles (210 MB at 8 groups, 256 heads) stay in the
// last-level cache for the scan that reads them, where the whole sequence's would not (measured on the
// 262144-token layer: 6.6 ms in one pass, 5.9 ms in 32768-token segments, the same y and final state).
constexpr int64_t kSegRows = 32768;
// byte offset of the state between segments in the workspace: after one segment's tiles, dt rows and scales
inline int64_t seg_state_off(int64_t nheads, int64_t ngroups) {
    return (ws_bytes(ngroups * (kSegRows / Q), nheads * (kSegRows / Q)) + 15) / 16 * 16;
}

template <typename TY, bool CONV, bool LP>
static hipError_t launch_t(const ScanArgs& a, void* workspace, const ConvIn& cv, hipStream_t s) {
    if (a.batch * a.nheads == 0) return hipSuccess;
    if constexpr (!CONV && !LP) {
        if (a.batch == 1 && !a.seq.cu_seqlens && a.seqlen > kSegRows) {
            float* mid = reinterpret_cast<float*>(static_cast<unsigned char*>(workspace) +
                                                  seg_state_off(a.nheads, a.ngroups));
            for (int64_t r0 = 0; r0 < a.seqlen; r0 += kSegRows) {
                ScanArgs g = a;
                g.seqlen = a.seqlen - r0 < kSegRows ? a.seqlen - r0 : kSegRows;
                g.x = static_cast<const bf16*>(a.x) + r0 * a.x_row_stride;
                g.B = static_cast<const bf16*>(a.B) + r0 * a.bc_row_stride;
                g.C = static_cast<const bf16*>(a.C) + r0 * a.bc_row_stride;
                g.dt = static_cast<const bf16*>(a.dt) + r0 * a.nheads;
                g.y = static_cast<TY*>(a.y) + r0 * a.nheads * static_cast<int64_t>(P);
                g.init_state = r0 == 0 ? a.init_state : mid;
                g.final_state = r0 + g.seqlen >= a.seqlen ? a.final_state : mid;
                const hipError_t e = launch_t<TY, CONV, LP>(g, workspace, cv, s);   // one segment each
                if (e != hipSuccess) return e;
            }
            return hipSuccess;
        }
    }
    // chunks per (batch entry, group), or packed: chunk slots per group (one workspace layout, [G][slot])
    const bool packed = a.seq.cu_seqlens != nullptr;
    const int64_t nc = packed ? packed_slots(a.batch, a.seqlen) : (a.seqlen + Q - 1) / Q;
    const int64_t ntile = (packed ? 1 : a.batch) * a.ngroups * nc;
    const int64_t nhc = (packed ? 1 : a.batch) * a.nheads * nc;
    unsigned char* w = static_cast<unsigned char*>(workspace);
    WsView ws{w, reinterpret_cast<float*>(w + ntile * kWsTile),
              reinterpret_cast<int2*>(w + ntile * kWsTile + nhc * Q * static_cast<int64_t>(sizeof(float))), ntile};
    if (ntile > 0) {
        hipLaunchKernelGGL(bc_prep_kernel<CONV>, dim3(static_cast<uint32_t>(ntile)), dim3(256), 0, s,
                           static_cast<const bf16*>(a.B), static_cast<const bf16*>(a.C), a.bc_row_stride,
                           static_cast<const bf16*>(a.dt), a.dtp, a.seqlen, a.nheads, a.ngroups, nc, ws, cv,
                           a.batch, a.seq);
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    auto kern = chunk_scan_kernel<TY, CONV, LP>;
    const size_t smem = CONV ? sizeof(Smem) : offsetof(Smem, Xr);
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern), hipFuncAttributeMaxDynamicSharedMemorySize,
                                       static_cast<int>(smem));
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(kern, dim3(static_cast<uint32_t>(a.batch * a.nheads)), dim3(kThreads), smem, s, a, ws, cv);
    return hipGetLastError();
}

}  // namespace scan16

bool f16_scan_supports(int head_dim, int d_state, int chunk) {
    return head_dim == scan16::P && d_state == scan16::NS && chunk == scan16::Q;
}

size_t f16_scan_varlen_workspace_bytes(int64_t nseq, int64_t rows, int nheads, int ngroups) {
    const int64_t ns = scan16::packed_slots(nseq, rows);
    return static_cast<size_t>(scan16::ws_bytes(ngroups * ns, nheads * ns));
}

size_t f16_scan_workspace_bytes(int64_t batch, int64_t seqlen, int nheads, int ngroups) {
    const int64_t nc = (seqlen + scan16::Q - 1) / scan16::Q;
    if (batch == 1 && seqlen > scan16::kSegRows) {   // at least one segment's tiles and the state between segments
        const int64_t whole = scan16::ws_bytes(ngroups * nc, nheads * nc);
        const int64_t seg = scan16::seg_state_off(nheads, ngroups) +
                            static_cast<int64_t>(nheads) * scan16::P * scan16::NS * static_cast<int64_t>(sizeof(float));
        return static_cast<size_t>(whole > seg ? whole : seg);
    }
    return static_cast<size_t>(scan16::ws_bytes(batch * ngroups * nc, batch * nheads * nc));
}

hipError_t launch_chunk_scan_f16(const ScanArgs& a, Dt ydt, void* workspace, hipStream_t s) {
    const scan16::ConvIn none{};
    if (a.init16 || a.final16)
        return ydt == Dt::BF16 ? scan16::launch_t<bf16, false, true>(a, workspace, none, s)
                               : scan16::launch_t<float, false, true>(a, workspace, none, s);
    return ydt == Dt::BF16 ? scan16::launch_t<bf16, false, false>(a, workspace, none, s)
                           : scan16::launch_t<float, false, false>(a, workspace, none, s);
}

hipError_t launch_conv_chunk_scan_f16(const ScanArgs& a, Dt ydt, const ConvScanArgs& c, void* workspace,
                                      hipStream_t s) {
    const scan16::ConvIn cv{static_cast<const bf16*>(c.w), static_cast<const bf16*>(c.bias),
                            static_cast<const bf16*>(c.state_in), static_cast<bf16*>(c.state_out),
                            static_cast<const bf16*>(c.xbc), c.xbc_row_stride, c.conv_dim,
                            static_cast<int64_t>(a.nheads) * a.head_dim};
    return ydt == Dt::BF16 ? scan16::launch_t<bf16, true, false>(a, workspace, cv, s)
                           : scan16::launch_t<float, true, false>(a, workspace, cv, s);
}

}  // namespace ssd
