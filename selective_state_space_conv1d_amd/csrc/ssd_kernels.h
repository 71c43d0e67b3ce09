// Internal launch interface between the C ABI (ssd_api.cpp) and the HIP kernels.
// Every launcher assumes its arguments were validated by the ABI layer.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace ssd {

enum class Dt : int { F32 = 0, BF16 = 1 };

// Packed variable-length batches (all NULL / 0 for the fixed-length calls): "batch" counts
// sequences, sequence s covers token rows [cu_seqlens[s], cu_seqlens[s+1]) of the packed
// tensors, and its states are slot slot_idx[s] (NULL: slot s) of the caller's state pools of
// nslots entries.  has_init[s] != 0 (NULL: never) starts sequence s from its slot's state.
struct SeqMap {
    const int32_t* cu_seqlens;
    const int32_t* slot_idx;
    const int32_t* has_init;
    int64_t nslots;
};

// dt prologue: dt <- clamp(softplus(dt + bias[h])) with each step optional (bias NULL,
// softplus 0, lo >= hi skip it).
struct DtParams {
    const float* bias;
    int softplus;
    float lo, hi;
};

struct ConvFwdArgs {
    const void* xbc; int64_t xbc_row_stride;
    const void* w; const void* bias;
    const void* state_in; void* state_out;
    void* out;
    int64_t batch, seqlen, channels;
    SeqMap seq;   // varlen: state_in / state_out are the conv-state pool
};

struct ConvUpdateArgs {
    const void* xbc; int64_t xbc_row_stride;
    const void* w; const void* bias;
    void* state; void* out;
    int64_t batch, channels;
    const int32_t* slot_idx;   // NULL: batch entry b uses state b; else slot slot_idx[b] of nslots
    int64_t nslots;
    void* inter;   // multi-token: [B, k, CD, 4] window after each token, or NULL
    int k;         // multi-token: tokens per request (the state is then read only)
};

// How a state array of 16-bit codes is read and rounded: fp16 or bf16 codes; rounds = 0 rounds to
// nearest even, otherwise stochastically with Philox4x32-(rounds) keyed by seed at offset.
struct Codes {
    bool f16;
    uint64_t seed, offset;
    int rounds;
};

struct ScanArgs {
    const void* x; int64_t x_row_stride;
    const void* B; const void* C; int64_t bc_row_stride;
    const void* dt; const float* A; const float* D;
    const float* init_state; float* final_state;
    void* y;
    int64_t batch, seqlen;
    int nheads, head_dim, ngroups, d_state, chunk;
    SeqMap seq;   // varlen: init_state / final_state are the state pool
    DtParams dtp;
    float* snapshots;        // [B, L / snap_interval, H, P, N]: state after every snap_interval tokens, or NULL;
                             // with snap_table: the snapshot pool [snap_slots, H, P, N]
    int64_t snap_interval;   // a positive multiple of 128 when snapshots is set
    const int32_t* snap_table;   // packed sequences: [S, snap_max] pool slot per (sequence, interval), or NULL
    int64_t snap_max, snap_slots;
    int64_t nranges;         // set by the launcher: sequence ranges per head (workgroups = nranges * nheads)
    int spin_max;            // set by the launcher: iterations of the split scan's bounded LDS-counter wait
    // 16-bit state arrays (init_state and final_state NULL): the initial states as codes, or NULL
    // (zeros), and the final states rounded into codes, or NULL (not stored); may alias
    const uint16_t* init16;
    uint16_t* final16;
    Codes codes;
};

struct UpdateArgs {
    float* state;
    const void* x; int64_t x_row_stride;
    const void* B; const void* C; int64_t bc_row_stride;
    const void* dt; const float* A; const float* D;
    void* y;
    int64_t batch;
    int nheads, head_dim, ngroups, d_state;
    const int32_t* slot_idx;   // NULL: batch entry b uses state b; else slot slot_idx[b] of nslots
    int64_t nslots;
    DtParams dtp;
    float* inter;   // multi-token: [B, k, H, P, N] state after each token, or NULL
    int k;          // multi-token: tokens per request (the state is then read only)
    const int32_t* accept_len;   // multi-token replay: apply the first accept_len[b] tokens in place
};

// Decode update on a 16-bit state (fp16 or bf16 codes): u carries everything but the state.
struct LpUpdateArgs {
    UpdateArgs u;
    void* state;
    bool f16;          // fp16 codes, else bf16
    uint64_t seed, offset;
    int rounds;        // Philox rounds for stochastic rounding; 0: round to nearest even
};

// One decode step (conv update + state update) in one launch: u carries the state update's
// arguments (x, B, C unused: they are the conv's outputs); the conv reads conv_in and writes conv_out.
struct DecodeStepArgs {
    UpdateArgs u;
    const void* xbc; int64_t xbc_row_stride;
    const void* w; const void* bias;
    const void* conv_in; void* conv_out;
};

// Gated group RMSNorm: rows x channels, ngroups groups of channels / ngroups.
struct NormArgs {
    const void* y; int64_t y_row_stride;
    const void* z; int64_t z_row_stride;
    const float* weight; float eps;
    void* out;
    int64_t rows, channels;
    int ngroups;
};

// Accept step of speculative decoding: request b with n = clamp(accept_len[b], 0, k) >= 1 gets
// intermediate state b*k + n - 1 copied into its slot (b without a slot table), for the SSM
// state (state_bytes per request) and the conv state (conv_bytes); NULL pointers skip one.
struct AcceptArgs {
    const int32_t* accept_len;
    const int32_t* slot_idx;
    int64_t nslots, batch;
    int k;
    void* state; const void* inter; int64_t state_bytes;
    void* conv_state; const void* inter_conv; int64_t conv_bytes;
};

hipError_t launch_conv1d_fwd(const ConvFwdArgs& a, Dt act, hipStream_t s);
// varlen prefill conv: the per-token pass, then the conv-state pass
hipError_t launch_conv1d_fwd_varlen(const ConvFwdArgs& a, Dt act, hipStream_t s);
hipError_t launch_conv1d_update(const ConvUpdateArgs& a, Dt act, hipStream_t s);
hipError_t launch_state_update(const UpdateArgs& a, Dt act, Dt ydt, hipStream_t s);
// speculative decode: k tokens per request from a read-only state, then the accept copy
hipError_t launch_state_update_multi(const UpdateArgs& a, Dt act, Dt ydt, hipStream_t s);
hipError_t launch_conv1d_update_multi(const ConvUpdateArgs& a, Dt act, hipStream_t s);
hipError_t launch_state_update_lp(const LpUpdateArgs& a, Dt act, Dt ydt, hipStream_t s);
hipError_t launch_gated_rmsnorm(const NormArgs& a, Dt act, Dt ydt, hipStream_t s);
hipError_t launch_decode_step(const DecodeStepArgs& a, Dt act, Dt ydt, hipStream_t s);
hipError_t launch_accept_states(const AcceptArgs& a, hipStream_t s);
// accept by recomputation: the multi-token update with u.accept_len set, and the conv windows
hipError_t launch_conv1d_update_accept(const ConvUpdateArgs& a, const int32_t* accept_len, Dt act, hipStream_t s);
// MFMA chunk scan: bf16 inputs with (head_dim, d_state, chunk) = (64, 128, 128).
bool mfma_scan_supports(int head_dim, int d_state, int chunk);
hipError_t launch_chunk_scan_mfma(const ScanArgs& a, Dt ydt, hipStream_t s);
// fp16 MFMA chunk scan (pre-pass of B and C into the workspace, then the scan): bf16 inputs with
// (head_dim, d_state, chunk) = (64, 128, 128); workspace of f16_scan_workspace_bytes, 16-byte aligned.
bool f16_scan_supports(int head_dim, int d_state, int chunk);
size_t f16_scan_workspace_bytes(int64_t batch, int64_t seqlen, int nheads, int ngroups);
// packed batches (ScanArgs.seq set): nseq sequences over rows token rows
size_t f16_scan_varlen_workspace_bytes(int64_t nseq, int64_t rows, int nheads, int ngroups);
// the device address and size of the current device's static fp16-scan workspace (looked up once per device)
hipError_t f16_scan_scratch(void** ptr, size_t* bytes);
hipError_t launch_chunk_scan_f16(const ScanArgs& a, Dt ydt, void* workspace, hipStream_t s);
// the fp16 scan with the prefill conv fused in: x, B and C are convolved from xBC inside the scan's launches
struct ConvScanArgs {
    const void* xbc; int64_t xbc_row_stride;
    const void* w; const void* bias;
    const void* state_in; void* state_out;
    int64_t conv_dim;
};
hipError_t launch_conv_chunk_scan_f16(const ScanArgs& a, Dt ydt, const ConvScanArgs& c, void* workspace,
                                      hipStream_t s);
// Generic chunk scan on fp32 FMA (any act dtype, head_dim and d_state <= 128).
hipError_t launch_chunk_scan_fma(const ScanArgs& a, Dt act, Dt ydt, hipStream_t s);

}  // namespace ssd
