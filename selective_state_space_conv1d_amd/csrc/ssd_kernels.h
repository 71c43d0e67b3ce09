// Internal launch interface between the C ABI (ssd_api.cpp) and the HIP kernels.
// Every launcher assumes its arguments were validated by the ABI layer.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace ssd {

enum class Dt : int { F32 = 0, BF16 = 1 };

struct ConvFwdArgs {
    const void* xbc; int64_t xbc_row_stride;
    const void* w; const void* bias;
    const void* state_in; void* state_out;
    void* out;
    int64_t batch, seqlen, channels;
};

struct ConvUpdateArgs {
    const void* xbc; int64_t xbc_row_stride;
    const void* w; const void* bias;
    void* state; void* out;
    int64_t batch, channels;
};

struct ScanArgs {
    const void* x; int64_t x_row_stride;
    const void* B; const void* C; int64_t bc_row_stride;
    const void* dt; const float* A; const float* D;
    const float* init_state; float* final_state;
    void* y;
    int64_t batch, seqlen;
    int nheads, head_dim, ngroups, d_state, chunk;
};

struct UpdateArgs {
    float* state;
    const void* x; int64_t x_row_stride;
    const void* B; const void* C; int64_t bc_row_stride;
    const void* dt; const float* A; const float* D;
    void* y;
    int64_t batch;
    int nheads, head_dim, ngroups, d_state;
};

hipError_t launch_conv1d_fwd(const ConvFwdArgs& a, Dt act, hipStream_t s);
hipError_t launch_conv1d_update(const ConvUpdateArgs& a, Dt act, hipStream_t s);
hipError_t launch_state_update(const UpdateArgs& a, Dt act, Dt ydt, hipStream_t s);
// MFMA chunk scan: bf16 inputs with (head_dim, d_state, chunk) = (64, 128, 128).
bool mfma_scan_supports(int head_dim, int d_state, int chunk);
hipError_t launch_chunk_scan_mfma(const ScanArgs& a, Dt ydt, hipStream_t s);
// Generic chunk scan on fp32 FMA (any act dtype, head_dim and d_state <= 128).
hipError_t launch_chunk_scan_fma(const ScanArgs& a, Dt act, Dt ydt, hipStream_t s);

}  // namespace ssd
