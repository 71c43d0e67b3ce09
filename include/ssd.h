/*
 * ssd.h -- C ABI of libssd: the Mamba-2 selective-SSM mixer hot path on
 * AMD Instinct MI355X (gfx950).
 *
 * Four operations, all asynchronous on the caller's HIP stream:
 *   ssd_conv1d_fwd     causal depthwise conv1d (width 4) + SiLU over the packed
 *                      x|B|C channels of a prefill, with a conv-state halo
 *   ssd_conv1d_update  the same conv for one new token per sequence (decode)
 *   ssd_chunk_scan     the SSD chunked scan of a prefill: y and the fp32 final
 *                      state from x, dt, A, B, C, D and an optional initial state
 *   ssd_state_update   the single-token selective state update (decode)
 *   (ssd_chunk_scan_snapshots: the scan, also storing the state every N tokens;
 *    ssd_chunk_scan_varlen_snapshots: the same for packed sequences, into a snapshot pool)
 * and their serving forms on packed variable-length batches and state pools:
 *   ssd_conv1d_fwd_varlen, ssd_chunk_scan_varlen, ssd_conv1d_update_slots,
 *   ssd_state_update_slots
 * and multi-token (speculative) decode with the accept step:
 *   ssd_state_update_multi, ssd_conv1d_update_multi, ssd_accept_states (or, by recomputation,
 *   ssd_state_update_accept and ssd_conv1d_update_accept)
 * and the decode update on a 16-bit state with stochastic rounding: ssd_state_update_lp,
 * and the gated group RMSNorm of the mixer output: ssd_gated_rmsnorm,
 * and one decode step (conv update + state update) in one launch: ssd_decode_step
 *
 * Sources (web pages, cited by title and section):
 *  [P1] "Mamba 与 Nemotron 系列模型深度调研": "Mamba 架构 / 1. Selective SSM 的直觉"
 *       (state recurrence and output), "状态契约" (state shapes, decode has
 *       seqlen 1 and never scans the cumulative context).
 *  [P2] walk-through of NVIDIA-Nemotron-Labs-Teacher-Chat modeling_nemotron_h.py:
 *       "Prefill 阶段" (causal conv keeps the last 4 conv inputs; 128-token
 *       chunked scan returns the final state, copied into the cache), "Decode
 *       阶段" (conv-state roll; in-place state update), fp32 state cache.
 *  [P3] "MAX 平台 Nemotron-H 混合架构解析": 4.5 (conv_dim = H*P + 2*G*N, channel
 *       order x | B | C), 5.4 (channels-last conv and in-place SSD scan that reads
 *       the initial state and writes the final state to the same slot).
 *
 * Semantics (fp32 arithmetic on the device; g(h) = h / (H/G)):
 *   conv:   v[b,t,c] = silu(bias[c] + sum_{k<4} w[c,k] * u~[b, t-3+k, c]), where
 *           u~ is the input for t >= 0 and conv_state_in[b, c, 4+t] for t in -3..-1;
 *           conv_state_out[b,c,k] = u~[b, L-4+k, c]  (the last 4 inputs).
 *   scan:   per (b,h,p), S = init[b,h,p,:] (or 0); for each token t:
 *             S = exp(dt*A[h]) * S + dt * B[b,t,g(h),:] * x[b,t,h,p]
 *             y[b,t,h,p] = <S, C[b,t,g(h),:]> + D[h] * x[b,t,h,p]
 *           final[b,h,p,:] = S.  The scan reaches this result by 128-token (or
 *           `chunk`) blocks; it equals the recurrence up to rounding.
 *   update: the scan with one token, state updated in place.
 *
 * Ownership: the caller allocates and frees every buffer (device memory);
 * the library allocates nothing and holds no state between calls beyond a
 * per-device cache of the compute-unit count (thread-safe), so calls on
 * different streams are independent.  Nothing synchronises.
 * Errors: every argument is checked on the host before anything is launched;
 * a call that returns an error has launched nothing and written nothing.
 * A launch failure returns SSD_ERR_HIP.  No call throws.
 * Buffers must not overlap unless marked "may alias".
 */
#ifndef SSD_H
#define SSD_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    SSD_OK = 0,
    SSD_ERR_NULL = 1,        /* a required pointer is NULL */
    SSD_ERR_SHAPE = 2,       /* negative size, H % G != 0, stride too small, ... */
    SSD_ERR_DTYPE = 3,       /* unknown dtype code */
    SSD_ERR_ALIGN = 4,       /* pointer not 16-byte aligned / stride not a multiple of 16 bytes */
    SSD_ERR_UNSUPPORTED = 5, /* size outside the compiled instantiations */
    SSD_ERR_WORKSPACE = 6,   /* workspace too small */
    SSD_ERR_HIP = 7          /* the HIP runtime reported an error at launch */
} ssd_status_t;

typedef enum { SSD_F32 = 0, SSD_BF16 = 1, SSD_F16 = 2 /* stored SSM state only */ } ssd_dtype_t;

/* Sizes of one mixer layer.  act_dtype is the element type of the conv input,
 * taps, bias, conv state and output, and of x, B, C and dt.  y_dtype is the
 * element type of y.  A, D and the SSM state are always fp32. */
typedef struct {
    int64_t batch;      /* B >= 0 */
    int64_t seqlen;     /* L >= 0 (prefill calls; the one-token calls ignore it) */
    int32_t nheads;     /* H */
    int32_t head_dim;   /* P: 16, 32, 64 or 128 */
    int32_t ngroups;    /* G, H % G == 0 */
    int32_t d_state;    /* N: 16, 32, 64 or 128 */
    int32_t conv_width; /* K: must be 4 */
    int32_t act_dtype;  /* ssd_dtype_t */
    int32_t y_dtype;    /* ssd_dtype_t */
} ssd_dims_t;

/*
 * Optional dt prologue ([P2] plugin inputs: dt_bias with softplus; the configs
 * draw dt = softplus(N(-2, 1)) directly).  NULL, or all fields zero, uses dt as
 * given.  Otherwise, in fp32, per token and head h:
 *   v = dt + bias[h]                      (bias NULL: + 0)
 *   v = softplus ? log(1 + exp(v)) : v    (returns v itself for v > 20)
 *   v = lo < hi ? min(max(v, lo), hi) : v
 * and the scan or update uses v as dt.
 */
typedef struct {
    const float* bias;  /* [H] fp32 device memory, or NULL */
    int32_t softplus;   /* nonzero: apply softplus after the bias */
    float lo, hi;       /* clamp range; lo >= hi disables the clamp */
} ssd_dt_params_t;

/* Conv channels CD = H*P + 2*G*N. */
int64_t ssd_conv_dim(const ssd_dims_t* d);

/*
 * Prefill conv ([P2] "Prefill 阶段"; [P3] 5.4, channels last, no transposes).
 *  xbc            [B, L, CD] act dtype; token rows xbc_row_stride elements apart
 *                 (>= CD, multiple of 8 elements), batch rows L*xbc_row_stride apart.
 *                 May be a view into a wider in_proj output.
 *  w              [CD, 4]  act dtype; w[c,3] multiplies the newest token.
 *  bias           [CD]     act dtype, or NULL (no bias).
 *  conv_state_in  [B, CD, 4] act dtype, or NULL (zeros: a fresh sequence).
 *  conv_state_out [B, CD, 4] act dtype, or NULL (not written).  May alias
 *                 conv_state_in (in-place cache update).
 *  out            [B, L, CD] contiguous, act dtype.  Must not alias xbc.
 * CD must be a multiple of 8.  L = 0 copies the state through.
 */
ssd_status_t ssd_conv1d_fwd(const ssd_dims_t* d, const void* xbc, int64_t xbc_row_stride,
                            const void* w, const void* bias, const void* conv_state_in,
                            void* conv_state_out, void* out, hipStream_t stream);

/*
 * One-token conv update ([P2] "Decode 阶段": roll the window by one, the new
 * input enters the last slot, then convolve).
 *  xbc        [B, CD] act dtype, rows xbc_row_stride elements apart (>= CD).
 *  w, bias    as ssd_conv1d_fwd.
 *  conv_state [B, CD, 4] act dtype, updated in place.
 *  out        [B, CD] contiguous act dtype.
 */
ssd_status_t ssd_conv1d_update(const ssd_dims_t* d, const void* xbc, int64_t xbc_row_stride,
                               const void* w, const void* bias, void* conv_state, void* out,
                               hipStream_t stream);

/*
 * Workspace bytes with which ssd_chunk_scan runs its fp16 path for these sizes: for bf16 inputs
 * with head_dim 64, d_state 128 and chunk 128, per (batch entry, group, 128-token chunk) 84 KiB
 * + 8 bytes (the chunk's fp16 B^T and C tiles, the causal tiles of C.B^T in fp16, and two
 * power-of-two scale exponents) plus 512 bytes per (batch entry, head, chunk) (dt after the dt
 * prologue); 0 for other sizes, dtypes or chunks, and for a NULL d.
 */
size_t ssd_chunk_scan_workspace_size(const ssd_dims_t* d, int32_t chunk);

/*
 * SSD chunked scan of a prefill ([P1] section 1 for the recurrence; [P2]
 * "Prefill 阶段" for the 128-token chunks and the final state; [P3] 5.4 for
 * the in-place initial/final state).
 *  chunk        64, 128 or 256 (tokens per block; the result does not depend on it
 *               beyond rounding).  L need not be a multiple of chunk.
 *  x            x[b,t,h,p] at x[(b*L + t)*x_row_stride + h*P + p], act dtype.
 *  B, C         B[b,t,g,n] at B[(b*L + t)*bc_row_stride + g*N + n] (same for C).
 *               x, B and C may be views into the conv output (row stride CD).
 *  dt           [B, L, H] act dtype, already positive (no bias, no softplus).
 *  A            [H] fp32 (negative decay rates).  D: [H] fp32 or NULL (no skip).
 *  dt_params    optional dt prologue (see ssd_dt_params_t), or NULL.
 *  init_state   [B, H, P, N] fp32, or NULL (zeros).
 *  final_state  [B, H, P, N] fp32, or NULL (not written).  May alias init_state.
 *  y            [B, L, H, P] contiguous, y dtype.
 *  workspace    NULL (or workspace_bytes 0) runs the bf16 split-operand MFMA scan.  Otherwise a
 *               caller-owned device buffer, 16-byte aligned, overwritten by the call: when
 *               ssd_chunk_scan_workspace_size() is non-zero it must hold at least that many bytes
 *               (else SSD_ERR_WORKSPACE; misaligned: SSD_ERR_ALIGN) and selects the fp16 scan; when
 *               that size is 0 it is ignored.  Both scans meet the same error bound and differ only
 *               in rounding.
 * Row strides are in elements: >= the row's extent, multiples of 8 (bf16) or 4 (fp32).
 * B and L above 2^31 - 1 are rejected (SSD_ERR_SHAPE).
 */
ssd_status_t ssd_chunk_scan(const ssd_dims_t* d, int32_t chunk,
                            const void* x, int64_t x_row_stride,
                            const void* B, const void* C, int64_t bc_row_stride,
                            const void* dt, const float* A, const float* D,
                            const ssd_dt_params_t* dt_params,
                            const float* init_state, float* final_state, void* y,
                            void* workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * The prefill conv fused into the chunked scan ([P3] 5.4, item 2: the conv folded into the
 * scan's launches; [P2] "Prefill 阶段" for what each step computes): the result of
 * ssd_conv1d_fwd(xbc, conv_w, conv_bias, conv_state_in, conv_state_out) followed by
 * ssd_chunk_scan over the x, B and C views of its output with a workspace -- y, final_state and
 * conv_state_out equal that pair's bit for bit -- without writing or re-reading the conv output:
 * x, B and C are convolved from xbc inside the scan.  bf16 activations with head_dim 64,
 * d_state 128 and chunk 128 only (else SSD_ERR_UNSUPPORTED); workspace as for ssd_chunk_scan
 * (ssd_chunk_scan_workspace_size() bytes, required when L > 0).  The rest of the arguments are
 * those of the two calls (conv_state_out may alias conv_state_in, final_state init_state).
 * One difference in rounding: x's power-of-two scale per chunk comes from a bound on the conv's
 * result (|bias| + sum |w| max|input|) rather than from its maximum; both choose 1 while the
 * values lie in [2^-8, 2^15), which is where the bit-for-bit equality holds.
 */
ssd_status_t ssd_conv_chunk_scan(const ssd_dims_t* d, int32_t chunk,
                                 const void* xbc, int64_t xbc_row_stride,
                                 const void* conv_w, const void* conv_bias,
                                 const void* conv_state_in, void* conv_state_out,
                                 const void* dt, const float* A, const float* D,
                                 const ssd_dt_params_t* dt_params,
                                 const float* init_state, float* final_state, void* y,
                                 void* workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * ssd_chunk_scan for callers that cannot allocate device memory: code under HIP graph capture,
 * tight serving loops, harnesses that forbid hipMalloc.  It allocates nothing (no hipMalloc,
 * hipFree or allocating library call): where ssd_chunk_scan would take a workspace (bf16 inputs,
 * head_dim 64, d_state 128, chunk 128) it uses a static 64 MiB device array instead, one per
 * device, held until the process ends -- enough while ssd_chunk_scan_workspace_size() <= 64 MiB
 * (one 8192-token sequence with 8 groups and 256 heads needs 50 MiB); larger sizes return
 * SSD_ERR_WORKSPACE.  Other
 * sizes run the kernels ssd_chunk_scan runs without a workspace.  Results are those of
 * ssd_chunk_scan with a workspace, bit for bit.  Every call on a device shares that device's
 * array (each call overwrites all of it that it reads): calls that overlap on one device, e.g.
 * on two streams, race.  Arguments, layouts and errors are otherwise those of ssd_chunk_scan.
 */
ssd_status_t ssd_chunk_scan_noalloc(const ssd_dims_t* d, int32_t chunk,
                                    const void* x, int64_t x_row_stride,
                                    const void* B, const void* C, int64_t bc_row_stride,
                                    const void* dt, const float* A, const float* D,
                                    const ssd_dt_params_t* dt_params,
                                    const float* init_state, float* final_state, void* y,
                                    hipStream_t stream);

/*
 * ssd_chunk_scan that also stores the state every `interval` tokens ([P2] 部署时如何调这些缓存:
 * one engine's setting writes an SSM state snapshot every N tokens, for prefix caching).
 *  snapshots  [B, L / interval, H, P, N] fp32, 16-byte aligned: entry k is the state after token
 *             (k + 1) * interval - 1 of each batch entry (the same values the final state would
 *             have if the sequence ended there).  May be NULL when L < interval.
 *  interval   a positive multiple of 128.
 * The rest is as for ssd_chunk_scan, except that the workspace is unused (may be NULL).
 */
ssd_status_t ssd_chunk_scan_snapshots(const ssd_dims_t* d, int32_t chunk,
                                      const void* x, int64_t x_row_stride,
                                      const void* B, const void* C, int64_t bc_row_stride,
                                      const void* dt, const float* A, const float* D,
                                      const ssd_dt_params_t* dt_params,
                                      const float* init_state, float* final_state, float* snapshots,
                                      int64_t interval, void* y, void* workspace, size_t workspace_bytes,
                                      hipStream_t stream);

/*
 * ssd_chunk_scan_varlen that also stores states at interval boundaries of each packed
 * sequence into a snapshot pool ([P2] 部署时如何调这些缓存: a state snapshot every N tokens for
 * prefix caching; here for the packed prefill that fills the cache).
 *  snap_pool     [nsnap_slots, H, P, N] fp32, 16-byte aligned; may be NULL when nsnap_slots is 0.
 *  snap_table    [S, max_snaps] int32 (device): entry (s, k) names the pool slot that receives the
 *                state of sequence s after its token (k + 1) * interval - 1.  Negative entries,
 *                entries naming no slot of the pool, and entries with k >= len_s / interval store
 *                nothing.  May be NULL when max_snaps is 0.
 *  interval      a positive multiple of 128.
 * Slots named by the table must be distinct from one another.  y and the state pool are exactly
 * those of ssd_chunk_scan_varlen; the rest is as there.
 */
ssd_status_t ssd_chunk_scan_varlen_snapshots(const ssd_dims_t* d, int32_t chunk, const void* x,
                                             int64_t x_row_stride, const void* B, const void* C,
                                             int64_t bc_row_stride, const void* dt, const float* A, const float* D,
                                             const ssd_dt_params_t* dt_params, const int32_t* cu_seqlens,
                                             const int32_t* slot_idx, const int32_t* has_initial_state,
                                             float* state_pool, int64_t nslots, float* snap_pool,
                                             int64_t nsnap_slots, const int32_t* snap_table, int32_t max_snaps,
                                             int64_t interval, void* y, void* workspace, size_t workspace_bytes,
                                             hipStream_t stream);

/*
 * Single-token selective state update, in place ([P2] "Decode 阶段"; [P1]
 * "状态契约": one token per call, no scan length).
 *  state  [B, H, P, N] fp32, updated in place.
 *  x      x[b,h,p] at x[b*x_row_stride + h*P + p]; B, C: B[b,g,n] at
 *         B[b*bc_row_stride + g*N + n]; act dtype.
 *  dt     [B, H] act dtype.  A [H] fp32; D [H] fp32 or NULL.  dt_params: optional
 *         dt prologue (see ssd_dt_params_t), or NULL.
 *  y      [B, H, P] contiguous, y dtype.
 */
ssd_status_t ssd_state_update(const ssd_dims_t* d, float* state,
                              const void* x, int64_t x_row_stride,
                              const void* B, const void* C, int64_t bc_row_stride,
                              const void* dt, const float* A, const float* D,
                              const ssd_dt_params_t* dt_params, void* y, hipStream_t stream);

/*
 * ---------------------------------------------------------------------------
 * Packed variable-length batches and state pools (serving).  [P2] "Mamba SSM 缓存详解" and
 * "Prefill 阶段": the conv and SSM states live in per-request cache slots that the
 * prefill writes in place.  [P3] 5.4: the kernels read and write the pool slots directly,
 * with no gather or scatter around them.  [P1] "状态契约": decode advances one token per
 * request.
 *
 * For the prefill calls, d->batch is the number of sequences S and d->seqlen is the
 * number of packed token rows T.  Sequence s covers rows [cu_seqlens[s], cu_seqlens[s+1])
 * of every packed tensor.
 *  cu_seqlens         [S + 1] int32, device memory, nondecreasing from 0 to T.  Values
 *                     outside [0, T] are clamped, so a malformed table cannot address
 *                     outside the buffers, but its results are unspecified.
 *  slot_idx           [S] int32 device memory, or NULL for slot s.  A negative slot, or
 *                     one >= nslots, marks padding: the sequence starts from zeros and its
 *                     final state is not stored.  Slots of one call must be distinct.
 *  has_initial_state  [S] int32 device memory, or NULL for all zero.  Nonzero starts
 *                     sequence s from its slot's state; zero starts from zeros.
 *  nslots             Pool entries, >= 0.  A pool may be NULL only when nslots is 0.
 * The tables and pools belong to the caller and are read on the device, in stream order.
 */

/*
 * Varlen prefill conv.
 *  xbc              [T, CD] act dtype, rows xbc_row_stride elements apart.
 *  conv_state_pool  [nslots, CD, 4] act dtype, updated in place.  Each sequence with a
 *                   slot gets its last 4 inputs, taking earlier columns from its old
 *                   state (or zeros) when it has fewer than 4 tokens.
 *  out              [T, CD] contiguous act dtype.  Rows outside every sequence are not written.
 * w, bias and the other rules are as for ssd_conv1d_fwd.  The call makes two launches on
 * `stream`: the per-token pass, then the pass that writes the pool.
 */
ssd_status_t ssd_conv1d_fwd_varlen(const ssd_dims_t* d, const void* xbc, int64_t xbc_row_stride,
                                   const void* w, const void* bias, const int32_t* cu_seqlens,
                                   const int32_t* slot_idx, const int32_t* has_initial_state,
                                   void* conv_state_pool, int64_t nslots, void* out, hipStream_t stream);

/*
 * Varlen SSD chunked scan.  Each sequence is scanned on its own, with chunks starting at
 * its first row.  The result equals ssd_chunk_scan run per sequence.
 *  x, B, C, dt   packed [T, ...] rows with the strides of ssd_chunk_scan (batch stride unused).
 *  state_pool    [nslots, H, P, N] fp32, updated in place: the initial state is read as
 *                has_initial_state says, and the final state is written to every sequence's slot.
 *  y             [T, H, P] contiguous y dtype.
 * chunk, A, D and dt_params as for ssd_chunk_scan; S and T above 2^31 - 1 are rejected (SSD_ERR_SHAPE).
 *  workspace     optional, 16-byte aligned, at least ssd_chunk_scan_varlen_workspace_size bytes: it selects
 *                the fp16 scan (bf16 inputs, head_dim 64, d_state 128, chunk 128), one workgroup per
 *                (sequence, head); a smaller nonzero buffer is SSD_ERR_WORKSPACE.  Without one (NULL or 0
 *                bytes) the bf16 split-operand kernel runs: when sequences x heads exceed what the device
 *                holds at once, one of its workgroups scans a range of consecutive sequences (balanced by
 *                tokens).  Either way sequence states must sit in distinct slots, as for any in-place pool
 *                update.
 */
/*
 * Workspace of the fp16 packed scan (above) for S = d->batch sequences over T = d->seqlen packed rows:
 * per group and per head, the pre-pass's tiles and dt rows for S + ceil(T / 128) chunk slots (chunk c of
 * sequence s, whose first row is r, takes slot s + floor(r / 128) + c).  0 where that scan does not apply
 * (then no workspace is needed).  d may be NULL (returns 0).
 */
size_t ssd_chunk_scan_varlen_workspace_size(const ssd_dims_t* d, int32_t chunk);

ssd_status_t ssd_chunk_scan_varlen(const ssd_dims_t* d, int32_t chunk, const void* x, int64_t x_row_stride,
                                   const void* B, const void* C, int64_t bc_row_stride, const void* dt,
                                   const float* A, const float* D, const ssd_dt_params_t* dt_params,
                                   const int32_t* cu_seqlens,
                                   const int32_t* slot_idx, const int32_t* has_initial_state,
                                   float* state_pool, int64_t nslots, void* y, void* workspace,
                                   size_t workspace_bytes, hipStream_t stream);

/*
 * One-token conv update on a conv-state pool.  Batch entry b uses slot slot_idx[b] of
 * conv_state_pool [nslots, CD, 4].  slot_idx is [B] int32 device memory and required.
 * A padding entry (slot < 0 or >= nslots) is convolved against a zero window and stores no
 * state.  The rest is as for ssd_conv1d_update.
 */
ssd_status_t ssd_conv1d_update_slots(const ssd_dims_t* d, const void* xbc, int64_t xbc_row_stride,
                                     const void* w, const void* bias, const int32_t* slot_idx,
                                     void* conv_state_pool, int64_t nslots, void* out, hipStream_t stream);

/*
 * Single-token state update on a state pool.  Batch entry b updates slot slot_idx[b] of
 * state_pool [nslots, H, P, N] fp32 in place.  slot_idx is [B] int32 device memory and
 * required.  A padding entry starts from a zero state and stores nothing; its y is still
 * written.  The rest is as for ssd_state_update.
 */
ssd_status_t ssd_state_update_slots(const ssd_dims_t* d, float* state_pool, int64_t nslots,
                                    const int32_t* slot_idx, const void* x, int64_t x_row_stride,
                                    const void* B, const void* C, int64_t bc_row_stride, const void* dt,
                                    const float* A, const float* D, const ssd_dt_params_t* dt_params, void* y,
                                    hipStream_t stream);

/*
 * ---------------------------------------------------------------------------
 * Multi-token decode for speculative decoding.  [P1] 状态契约, "MTP / speculative decoding":
 * each candidate token of a request leaves an intermediate recurrent state and conv state;
 * after verification, the state at the request's accepted length has to be written back into
 * its main state, or later decode steps continue from the wrong history.
 *
 * d->batch = B requests, d->seqlen = k candidate tokens per request (0 <= k < 2^31).  Token j
 * of request b is row b*k + j of every per-token tensor.  The multi-token calls only read the
 * main states; ssd_accept_states then writes them.
 *  slot_idx  [B] int32 device memory, or NULL: request b uses entry b of the main states.
 *            With a table, the main states are pools of nslots entries and request b uses
 *            slot slot_idx[b]; a slot < 0 or >= nslots is padding (starts from zeros, and
 *            accept stores nothing for it).
 * A k-token step with every token accepted equals k single-token calls (bitwise, for the same
 * dtypes): the arithmetic per token is that of ssd_conv1d_update and ssd_state_update.
 */

/*
 * k-token SSM update from the request's state (read only).
 *  state         [B or nslots, H, P, N] fp32.  May be NULL only with a slot table and nslots 0.
 *  x             x[b,j,h,p] at x[(b*k + j)*x_row_stride + h*P + p]; B, C: B[b,j,g,n] at
 *                B[(b*k + j)*bc_row_stride + g*N + n]; act dtype.  B and C 16-byte aligned and
 *                bc_row_stride a multiple of 8 (bf16) or 4 (fp32) elements.
 *  dt            [B, k, H] act dtype, contiguous.  A, D, dt_params as ssd_state_update.
 *  inter_states  [B, k, H, P, N] fp32: the state after each token, or NULL (not written).
 *  y             [B, k, H, P] contiguous y dtype.
 */
ssd_status_t ssd_state_update_multi(const ssd_dims_t* d, const float* state, const int32_t* slot_idx,
                                    int64_t nslots, const void* x, int64_t x_row_stride, const void* B,
                                    const void* C, int64_t bc_row_stride, const void* dt, const float* A,
                                    const float* D, const ssd_dt_params_t* dt_params, float* inter_states,
                                    void* y, hipStream_t stream);

/*
 * k-token conv update from the request's conv state (read only).
 *  xbc                [B*k, CD] act dtype, rows xbc_row_stride elements apart (>= CD).
 *  w, bias            as ssd_conv1d_fwd.
 *  conv_state         [B or nslots, CD, 4] act dtype.  NULL only with a slot table and nslots 0.
 *  inter_conv_states  [B, k, CD, 4] act dtype: the window after each token, or NULL.
 *  out                [B, k, CD] contiguous act dtype.
 */
ssd_status_t ssd_conv1d_update_multi(const ssd_dims_t* d, const void* xbc, int64_t xbc_row_stride,
                                     const void* w, const void* bias, const void* conv_state,
                                     const int32_t* slot_idx, int64_t nslots, void* inter_conv_states,
                                     void* out, hipStream_t stream);

/*
 * Accept step.  accept_len [B] int32 device memory: request b keeps its first n tokens, with n
 * clamped to [0, k].  For n >= 1, inter_states[b, n-1] is copied into its state (entry b or
 * slot slot_idx[b]) and inter_conv_states[b, n-1] into its conv state; n = 0 and padding
 * requests leave them unchanged.  Either pair (state, inter_states) or (conv_state,
 * inter_conv_states) may be NULL, not one pointer of a pair.  Slots of one call must be
 * distinct, and the intermediate buffers must not overlap the main states.  B <= 65535.
 * Two launches on `stream` (SSM state, then conv state).
 */
ssd_status_t ssd_accept_states(const ssd_dims_t* d, const int32_t* accept_len, const int32_t* slot_idx,
                               int64_t nslots, float* state, const float* inter_states, void* conv_state,
                               const void* inter_conv_states, hipStream_t stream);

/*
 * ---------------------------------------------------------------------------
 * Reduced-precision state storage.  [P2] 部署时如何调这些缓存: inference engines store the
 * Mamba state cache in fp16 with stochastic rounding driven by a Philox generator (5 rounds).
 * [P3] 5.4: the state pool may be stored in a narrower type while the update accumulates in
 * fp32.  The state is read as 16-bit codes, updated in fp32 exactly as ssd_state_update does,
 * and rounded back:
 *  sr == NULL  round to nearest even.
 *  sr != NULL  stochastic rounding.  Element e of the state array (its flat index in the pool
 *              with a slot table) draws r16 = the 16-bit half (e mod 2), low half first, of word
 *              (e mod 8) / 2 of Philox4x32-R (Salmon, Moraes, Dror, Shaw, SC 2011) with counter
 *              (o mod 2^32, o / 2^32, offset mod 2^32, offset / 2^32), o = e / 8, and key
 *              (seed mod 2^32, seed / 2^32).  With lo the code next to the fp32 value v toward
 *              zero (v itself when representable) and spacing the distance from lo to the next
 *              code away from zero, v is stored as that next code iff
 *              r16 < 65536 * (|v| - |lo|) / spacing, else as lo.  Past the largest finite value
 *              the next code is infinity and the spacing that of the last binade; fp16 values
 *              of magnitude 65536 or more become infinities; NaN and infinite v round to
 *              nearest even.  Use a new offset for every call, or the same numbers repeat.
 */
typedef struct {
    uint64_t seed;     /* Philox key */
    uint64_t offset;   /* Philox counter words 2 and 3 */
    int32_t rounds;    /* Philox rounds, 1..16 */
} ssd_sr_params_t;

/*
 * Single-token state update on a 16-bit state.
 *  state        [B or nslots, H, P, N] codes of state_dtype (SSD_F16 or SSD_BF16), updated in
 *               place, 16-byte aligned.
 *  slot_idx     [B] int32 device memory or NULL, as ssd_state_update_slots (NULL: entry b).
 *  sr           rounding (above); NULL rounds to nearest even.
 *  B, C         16-byte aligned, bc_row_stride a multiple of 8 (bf16) or 4 (fp32) elements.
 * The rest is as for ssd_state_update.
 */
ssd_status_t ssd_state_update_lp(const ssd_dims_t* d, void* state, int32_t state_dtype, const int32_t* slot_idx,
                                 int64_t nslots, const void* x, int64_t x_row_stride, const void* B, const void* C,
                                 int64_t bc_row_stride, const void* dt, const float* A, const float* D,
                                 const ssd_dt_params_t* dt_params, const ssd_sr_params_t* sr, void* y,
                                 hipStream_t stream);

/*
 * The chunked scans with 16-bit state arrays (the modeling_nemotron_h.py walk-through,
 * 部署时如何调这些缓存: an fp16 Mamba state cache with Philox stochastic rounding; [P3] 5.4: the
 * stored state narrower than the fp32 the scan accumulates in).  The initial states are fp16 or
 * bf16 codes (state_dtype SSD_F16 or SSD_BF16, else SSD_ERR_DTYPE), read exactly; the scan runs as
 * in fp32; each final state element is rounded into a code as ssd_state_update_lp rounds
 * (sr NULL: nearest even; else stochastically, element e being its flat index in the array or pool,
 * rounds 1..16 else SSD_ERR_UNSUPPORTED).  The code arrays are 16-byte aligned.
 *  ssd_chunk_scan_lp          init_state / final_state [B, H, P, N] codes, or NULL (zeros / not
 *                             stored); they may alias.  Everything else as ssd_chunk_scan (a
 *                             workspace selects the fp16 scan there too).
 *  ssd_chunk_scan_varlen_lp   state_pool [nslots, H, P, N] codes, read and written in place as
 *                             ssd_chunk_scan_varlen's fp32 pool.
 */
ssd_status_t ssd_chunk_scan_lp(const ssd_dims_t* d, int32_t chunk, const void* x, int64_t x_row_stride,
                               const void* B, const void* C, int64_t bc_row_stride, const void* dt,
                               const float* A, const float* D, const ssd_dt_params_t* dt_params,
                               const void* init_state, void* final_state, int32_t state_dtype,
                               const ssd_sr_params_t* sr, void* y, void* workspace, size_t workspace_bytes,
                               hipStream_t stream);
ssd_status_t ssd_chunk_scan_varlen_lp(const ssd_dims_t* d, int32_t chunk, const void* x, int64_t x_row_stride,
                                      const void* B, const void* C, int64_t bc_row_stride, const void* dt,
                                      const float* A, const float* D, const ssd_dt_params_t* dt_params,
                                      const int32_t* cu_seqlens, const int32_t* slot_idx,
                                      const int32_t* has_initial_state, void* state_pool, int32_t state_dtype,
                                      int64_t nslots, const ssd_sr_params_t* sr, void* y, void* workspace,
                                      size_t workspace_bytes, hipStream_t stream);

/*
 * Gated group RMSNorm of the mixer output ([P3] 5.4, item 4: one fused kernel; the gate is applied
 * before the norm, in fp32, with an fp32 weight).  Per row and group g of gs = H*P/G channels:
 *   v = y * silu(z);  out = v / sqrt(mean over the group of v^2 + eps) * weight.
 *  d          rows = batch * seqlen; the channels are H*P in G groups (gs a multiple of 8).
 *  y          [rows, H*P] y dtype, rows y_row_stride elements apart.
 *  z          [rows, H*P] act dtype, rows z_row_stride elements apart (may be a view into the
 *             in_proj output).
 *  weight     [H*P] fp32.  eps >= 0.
 *  out        [rows, H*P] contiguous act dtype; must not overlap y or z.
 * Row strides keep rows 16-byte aligned; all pointers 16-byte aligned.
 */
ssd_status_t ssd_gated_rmsnorm(const ssd_dims_t* d, const void* y, int64_t y_row_stride, const void* z,
                               int64_t z_row_stride, const float* weight, float eps, void* out, hipStream_t stream);

/*
 * One decode step of the mixer in one launch: ssd_conv1d_update followed by ssd_state_update
 * ([P2] "Decode 阶段"), bitwise equal to the two calls (the conv outputs are rounded to the
 * activation dtype as the conv call stores them).  The conv outputs x, B, C are not written.
 *  xbc             [B, CD] act dtype, rows xbc_row_stride elements apart.
 *  conv_state_in   [B, CD, 4] act dtype, read only.
 *  conv_state_out  [B, CD, 4] act dtype: the rolled windows.  Must not overlap conv_state_in:
 *                  the step reads every group's old window from many workgroups (swap the two
 *                  buffers between steps).
 *  state           [B, H, P, N] fp32, updated in place.
 * w, bias, dt, A, D, dt_params and y as for ssd_conv1d_update and ssd_state_update.
 */
ssd_status_t ssd_decode_step(const ssd_dims_t* d, const void* xbc, int64_t xbc_row_stride, const void* w,
                             const void* bias, const void* conv_state_in, void* conv_state_out, float* state,
                             const void* dt, const float* A, const float* D, const ssd_dt_params_t* dt_params,
                             void* y, hipStream_t stream);

/*
 * Accept step by recomputation: instead of keeping the k intermediate states, apply each request's
 * first n = accept_len[b] (clamped to [0, k]) candidate tokens to its main state in place.  The
 * per-token arithmetic is ssd_state_update_multi's, so the state equals the intermediate state
 * n - 1 bitwise; n = 0 and padding requests are left unchanged.  The inputs are the multi-token
 * call's: x, B, C, dt with its layout and strides (B and C 16-byte aligned).  With it, the
 * multi-token call can run with inter_states NULL.
 */
ssd_status_t ssd_state_update_accept(const ssd_dims_t* d, float* state, const int32_t* slot_idx, int64_t nslots,
                                     const void* x, int64_t x_row_stride, const void* B, const void* C,
                                     int64_t bc_row_stride, const void* dt, const float* A, const float* D,
                                     const ssd_dt_params_t* dt_params, const int32_t* accept_len, hipStream_t stream);

/*
 * The conv counterpart: request b's window becomes the last 4 of (its old window, candidate rows
 * 0 .. n-1 of xbc), in place.  xbc is the multi-token conv call's input [B*k, CD].
 */
ssd_status_t ssd_conv1d_update_accept(const ssd_dims_t* d, const void* xbc, int64_t xbc_row_stride, void* conv_state,
                                      const int32_t* slot_idx, int64_t nslots, const int32_t* accept_len,
                                      hipStream_t stream);

/* Static, human-readable name of a status code. */
const char* ssd_status_string(ssd_status_t s);

#ifdef __cplusplus
}
#endif
#endif /* SSD_H */
