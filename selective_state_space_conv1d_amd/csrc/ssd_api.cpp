// libssd C ABI: argument validation on the host, then one launch per call.
// All checks run before anything is launched, so a failed call has no effect.
#include "../../include/ssd.h"
#include "ssd_kernels.h"

#include <stdint.h>

namespace {

using ssd::Dt;

bool valid_dtype(int32_t d) { return d == SSD_F32 || d == SSD_BF16; }
int elem_size(int32_t d) { return d == SSD_BF16 ? 2 : 4; }
bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
bool pow2_16_128(int32_t v) { return v == 16 || v == 32 || v == 64 || v == 128; }
// row stride (elements) keeps every row start 16-byte aligned
bool stride_ok(int64_t stride, int32_t dt) { return (stride * elem_size(dt)) % 16 == 0; }

ssd_status_t check_dims(const ssd_dims_t* d, bool need_seqlen) {
    if (!d) return SSD_ERR_NULL;
    if (!valid_dtype(d->act_dtype) || !valid_dtype(d->y_dtype)) return SSD_ERR_DTYPE;
    if (d->batch < 0 || (need_seqlen && d->seqlen < 0)) return SSD_ERR_SHAPE;
    if (d->nheads <= 0 || d->head_dim <= 0 || d->ngroups <= 0 || d->d_state <= 0) return SSD_ERR_SHAPE;
    if (d->nheads % d->ngroups != 0) return SSD_ERR_SHAPE;
    if (d->conv_width != 4) return SSD_ERR_UNSUPPORTED;
    return SSD_OK;
}

ssd_status_t hip_status(hipError_t e) { return e == hipSuccess ? SSD_OK : SSD_ERR_HIP; }

ssd::DtParams dt_params_of(const ssd_dt_params_t* p) {
    if (!p) return ssd::DtParams{nullptr, 0, 0.f, 0.f};
    return ssd::DtParams{p->bias, p->softplus, p->lo, p->hi};
}
bool dt_params_ok(const ssd_dt_params_t* p) {
    return !p || !p->bias || (reinterpret_cast<uintptr_t>(p->bias) & 3u) == 0;
}

// Packed variable-length calls: tables and pool present as the sizes require.
ssd_status_t check_seq_tables(const ssd_dims_t* d, const int32_t* cu_seqlens, const void* pool, int64_t nslots) {
    if (nslots < 0) return SSD_ERR_SHAPE;
    if (d->batch > 0 && !cu_seqlens) return SSD_ERR_NULL;
    if (nslots > 0 && !pool) return SSD_ERR_NULL;
    if (pool && !aligned16(pool)) return SSD_ERR_ALIGN;
    return SSD_OK;
}

}  // namespace

extern "C" {

int64_t ssd_conv_dim(const ssd_dims_t* d) {
    if (!d) return -1;
    return static_cast<int64_t>(d->nheads) * d->head_dim + 2LL * d->ngroups * d->d_state;
}

const char* ssd_status_string(ssd_status_t s) {
    switch (s) {
        case SSD_OK: return "ok";
        case SSD_ERR_NULL: return "required pointer is NULL";
        case SSD_ERR_SHAPE: return "invalid shape or stride";
        case SSD_ERR_DTYPE: return "invalid dtype";
        case SSD_ERR_ALIGN: return "pointer or stride not 16-byte aligned";
        case SSD_ERR_UNSUPPORTED: return "size not supported by the compiled kernels";
        case SSD_ERR_WORKSPACE: return "workspace too small";
        case SSD_ERR_HIP: return "HIP runtime error at launch";
    }
    return "unknown status";
}

ssd_status_t ssd_conv1d_fwd(const ssd_dims_t* d, const void* xbc, int64_t xbc_row_stride,
                            const void* w, const void* bias, const void* conv_state_in,
                            void* conv_state_out, void* out, hipStream_t stream) {
    ssd_status_t st = check_dims(d, true);
    if (st != SSD_OK) return st;
    const int64_t CD = ssd_conv_dim(d);
    const bool tokens = d->batch > 0 && d->seqlen > 0;
    if (tokens && (!xbc || !w || !out)) return SSD_ERR_NULL;
    if (CD % 8 != 0) return SSD_ERR_UNSUPPORTED;
    if (tokens && xbc_row_stride < CD) return SSD_ERR_SHAPE;
    if (!stride_ok(xbc_row_stride, d->act_dtype)) return SSD_ERR_ALIGN;
    for (const void* p : {xbc, w, bias, conv_state_in, static_cast<const void*>(conv_state_out),
                          static_cast<const void*>(out)})
        if (p && !aligned16(p)) return SSD_ERR_ALIGN;
    ssd::ConvFwdArgs a{xbc, xbc_row_stride, w, bias, conv_state_in, conv_state_out, out,
                       d->batch, d->seqlen, CD};
    return hip_status(ssd::launch_conv1d_fwd(a, static_cast<Dt>(d->act_dtype), stream));
}

ssd_status_t ssd_conv1d_update(const ssd_dims_t* d, const void* xbc, int64_t xbc_row_stride,
                               const void* w, const void* bias, void* conv_state, void* out,
                               hipStream_t stream) {
    ssd_status_t st = check_dims(d, false);
    if (st != SSD_OK) return st;
    const int64_t CD = ssd_conv_dim(d);
    if (!xbc || !w || !conv_state || !out) return SSD_ERR_NULL;
    if (CD % 8 != 0) return SSD_ERR_UNSUPPORTED;
    if (xbc_row_stride < CD) return SSD_ERR_SHAPE;
    if (!stride_ok(xbc_row_stride, d->act_dtype)) return SSD_ERR_ALIGN;
    for (const void* p : {xbc, w, bias, static_cast<const void*>(conv_state), static_cast<const void*>(out)})
        if (p && !aligned16(p)) return SSD_ERR_ALIGN;
    ssd::ConvUpdateArgs a{xbc, xbc_row_stride, w, bias, conv_state, out, d->batch, CD};
    return hip_status(ssd::launch_conv1d_update(a, static_cast<Dt>(d->act_dtype), stream));
}

ssd_status_t ssd_conv1d_fwd_varlen(const ssd_dims_t* d, const void* xbc, int64_t xbc_row_stride,
                                   const void* w, const void* bias, const int32_t* cu_seqlens,
                                   const int32_t* slot_idx, const int32_t* has_initial_state,
                                   void* conv_state_pool, int64_t nslots, void* out, hipStream_t stream) {
    ssd_status_t st = check_dims(d, true);
    if (st != SSD_OK) return st;
    st = check_seq_tables(d, cu_seqlens, conv_state_pool, nslots);
    if (st != SSD_OK) return st;
    const int64_t CD = ssd_conv_dim(d);
    const bool tokens = d->batch > 0 && d->seqlen > 0;
    if ((tokens || (d->batch > 0 && nslots > 0)) && (!w || (tokens && (!xbc || !out)))) return SSD_ERR_NULL;
    if (CD % 8 != 0) return SSD_ERR_UNSUPPORTED;
    if (tokens && xbc_row_stride < CD) return SSD_ERR_SHAPE;
    if (!stride_ok(xbc_row_stride, d->act_dtype)) return SSD_ERR_ALIGN;
    for (const void* p : {xbc, w, bias, static_cast<const void*>(out)})
        if (p && !aligned16(p)) return SSD_ERR_ALIGN;
    ssd::ConvFwdArgs a{xbc, xbc_row_stride, w, bias, conv_state_pool, conv_state_pool, out,
                       d->batch, d->seqlen, CD, {cu_seqlens, slot_idx, has_initial_state, nslots}};
    return hip_status(ssd::launch_conv1d_fwd_varlen(a, static_cast<Dt>(d->act_dtype), stream));
}

ssd_status_t ssd_conv1d_update_slots(const ssd_dims_t* d, const void* xbc, int64_t xbc_row_stride,
                                     const void* w, const void* bias, const int32_t* slot_idx,
                                     void* conv_state_pool, int64_t nslots, void* out, hipStream_t stream) {
    ssd_status_t st = check_dims(d, false);
    if (st != SSD_OK) return st;
    const int64_t CD = ssd_conv_dim(d);
    if (nslots < 0) return SSD_ERR_SHAPE;
    if (d->batch > 0 && (!xbc || !w || !out || !slot_idx)) return SSD_ERR_NULL;
    if (nslots > 0 && !conv_state_pool) return SSD_ERR_NULL;
    if (CD % 8 != 0) return SSD_ERR_UNSUPPORTED;
    if (xbc_row_stride < CD) return SSD_ERR_SHAPE;
    if (!stride_ok(xbc_row_stride, d->act_dtype)) return SSD_ERR_ALIGN;
    for (const void* p : {xbc, w, bias, static_cast<const void*>(conv_state_pool), static_cast<const void*>(out)})
        if (p && !aligned16(p)) return SSD_ERR_ALIGN;
    ssd::ConvUpdateArgs a{xbc, xbc_row_stride, w, bias, conv_state_pool, out, d->batch, CD, slot_idx, nslots};
    return hip_status(ssd::launch_conv1d_update(a, static_cast<Dt>(d->act_dtype), stream));
}

// The fp16 scan applies to bf16 inputs at (head_dim, d_state, chunk) = (64, 128, 128); its workspace
// holds the pre-pass's fp16 B and C tiles and their scales.
static bool f16_scan_applies(const ssd_dims_t* d, int32_t chunk) {
    return d && d->act_dtype == SSD_BF16 && ssd::f16_scan_supports(d->head_dim, d->d_state, chunk);
}

size_t ssd_chunk_scan_workspace_size(const ssd_dims_t* d, int32_t chunk) {
    if (!f16_scan_applies(d, chunk) || d->batch <= 0 || d->seqlen <= 0 || d->ngroups <= 0 || d->nheads <= 0) return 0;
    return ssd::f16_scan_workspace_bytes(d->batch, d->seqlen, d->nheads, d->ngroups);
}

size_t ssd_chunk_scan_varlen_workspace_size(const ssd_dims_t* d, int32_t chunk) {
    if (!f16_scan_applies(d, chunk) || d->batch <= 0 || d->seqlen <= 0 || d->ngroups <= 0 || d->nheads <= 0) return 0;
    return ssd::f16_scan_varlen_workspace_bytes(d->batch, d->seqlen, d->nheads, d->ngroups);
}

// 16-bit initial / final states of a scan, in place of the fp32 ones
struct States16 {
    const void* init;
    void* fin;
    int32_t dtype;
    const ssd_sr_params_t* sr;
};

static ssd_status_t check_states16(const States16* s16) {
    if (!s16) return SSD_OK;
    if (s16->dtype != SSD_F16 && s16->dtype != SSD_BF16) return SSD_ERR_DTYPE;
    if (s16->sr && (s16->sr->rounds < 1 || s16->sr->rounds > 16)) return SSD_ERR_UNSUPPORTED;
    for (const void* p : {s16->init, static_cast<const void*>(s16->fin)})
        if (p && !aligned16(p)) return SSD_ERR_ALIGN;
    return SSD_OK;
}

static void set_states16(ssd::ScanArgs& a, const States16* s16) {
    if (!s16) return;
    a.init16 = static_cast<const uint16_t*>(s16->init);
    a.final16 = static_cast<uint16_t*>(s16->fin);
    a.codes = ssd::Codes{s16->dtype == SSD_F16, s16->sr ? s16->sr->seed : 0, s16->sr ? s16->sr->offset : 0,
                         s16->sr ? s16->sr->rounds : 0};
}

// the batched scan, with optional state snapshots or 16-bit states (internal linkage)
static ssd_status_t chunk_scan(const ssd_dims_t* d, int32_t chunk, const void* x, int64_t x_row_stride,
                               const void* B, const void* C, int64_t bc_row_stride, const void* dt, const float* A,
                               const float* D, const ssd_dt_params_t* dt_params, const float* init_state,
                               float* final_state, float* snapshots, int64_t interval, void* y, void* workspace,
                               size_t workspace_bytes, hipStream_t stream, const States16* s16 = nullptr) {
    ssd_status_t st = check_dims(d, true);
    if (st != SSD_OK) return st;
    st = check_states16(s16);
    if (st != SSD_OK) return st;
    if (d->batch > INT32_MAX || d->seqlen > INT32_MAX) return SSD_ERR_SHAPE;
    const bool tokens = d->batch > 0 && d->seqlen > 0;
    if (tokens && (!x || !B || !C || !dt || !A || !y)) return SSD_ERR_NULL;
    if (chunk != 64 && chunk != 128 && chunk != 256) return SSD_ERR_UNSUPPORTED;
    if (!pow2_16_128(d->head_dim) || !pow2_16_128(d->d_state)) return SSD_ERR_UNSUPPORTED;
    const int64_t I = static_cast<int64_t>(d->nheads) * d->head_dim;
    const int64_t GN = static_cast<int64_t>(d->ngroups) * d->d_state;
    if (tokens && (x_row_stride < I || bc_row_stride < GN)) return SSD_ERR_SHAPE;
    if (!stride_ok(x_row_stride, d->act_dtype) || !stride_ok(bc_row_stride, d->act_dtype)) return SSD_ERR_ALIGN;
    for (const void* p : {x, B, C, static_cast<const void*>(y), static_cast<const void*>(init_state), static_cast<const void*>(final_state)})
        if (p && !aligned16(p)) return SSD_ERR_ALIGN;
    if ((reinterpret_cast<uintptr_t>(dt) % elem_size(d->act_dtype)) != 0) return SSD_ERR_ALIGN;
    // A workspace selects the fp16 scan: it must then be large enough and 16-byte aligned.  Without
    // one (NULL or 0 bytes) the scan runs on the bf16 split-operand kernel.
    const size_t ws_need = snapshots ? 0 : ssd_chunk_scan_workspace_size(d, chunk);
    const bool use_f16 = ws_need > 0 && workspace && workspace_bytes > 0;
    if (use_f16 && workspace_bytes < ws_need) return SSD_ERR_WORKSPACE;
    if (use_f16 && !aligned16(workspace)) return SSD_ERR_ALIGN;
    if (!dt_params_ok(dt_params)) return SSD_ERR_ALIGN;
    ssd::ScanArgs a{x, x_row_stride, B, C, bc_row_stride, dt, A, D, init_state, final_state, y,
                    d->batch, d->seqlen, d->nheads, d->head_dim, d->ngroups, d->d_state, chunk,
                    {nullptr, nullptr, nullptr, 0}, dt_params_of(dt_params), snapshots, interval};
    set_states16(a, s16);
    const Dt act = static_cast<Dt>(d->act_dtype), ydt = static_cast<Dt>(d->y_dtype);
    if (use_f16) return hip_status(ssd::launch_chunk_scan_f16(a, ydt, workspace, stream));
    if (act == Dt::BF16 && ssd::mfma_scan_supports(d->head_dim, d->d_state, chunk))
        return hip_status(ssd::launch_chunk_scan_mfma(a, ydt, stream));
    return hip_status(ssd::launch_chunk_scan_fma(a, act, ydt, stream));
}

ssd_status_t ssd_chunk_scan(const ssd_dims_t* d, int32_t chunk, const void* x, int64_t x_row_stride,
                            const void* B, const void* C, int64_t bc_row_stride, const void* dt,
                            const float* A, const float* D, const ssd_dt_params_t* dt_params,
                            const float* init_state,
                            float* final_state, void* y, void* workspace, size_t workspace_bytes,
                            hipStream_t stream) {
    return chunk_scan(d, chunk, x, x_row_stride, B, C, bc_row_stride, dt, A, D, dt_params, init_state, final_state,
                      nullptr, 0, y, workspace, workspace_bytes, stream);
}

ssd_status_t ssd_conv_chunk_scan(const ssd_dims_t* d, int32_t chunk, const void* xbc, int64_t xbc_row_stride,
                                 const void* conv_w, const void* conv_bias, const void* conv_state_in,
                                 void* conv_state_out, const void* dt, const float* A, const float* D,
                                 const ssd_dt_params_t* dt_params, const float* init_state, float* final_state,
                                 void* y, void* workspace, size_t workspace_bytes, hipStream_t stream) {
    ssd_status_t st = check_dims(d, true);
    if (st != SSD_OK) return st;
    if (!f16_scan_applies(d, chunk)) return SSD_ERR_UNSUPPORTED;
    if (d->batch > INT32_MAX || d->seqlen > INT32_MAX) return SSD_ERR_SHAPE;
    const int64_t CD = ssd_conv_dim(d);
    const bool tokens = d->batch > 0 && d->seqlen > 0;
    if (tokens && (!xbc || !conv_w || !dt || !A || !y)) return SSD_ERR_NULL;
    if (tokens && xbc_row_stride < CD) return SSD_ERR_SHAPE;
    if (!stride_ok(xbc_row_stride, d->act_dtype)) return SSD_ERR_ALIGN;
    for (const void* p : {xbc, conv_w, conv_bias, conv_state_in, static_cast<const void*>(conv_state_out),
                          static_cast<const void*>(y), static_cast<const void*>(init_state),
                          static_cast<const void*>(final_state)})
        if (p && !aligned16(p)) return SSD_ERR_ALIGN;
    if ((reinterpret_cast<uintptr_t>(dt) % elem_size(d->act_dtype)) != 0) return SSD_ERR_ALIGN;
    if (!dt_params_ok(dt_params)) return SSD_ERR_ALIGN;
    const int64_t I = static_cast<int64_t>(d->nheads) * d->head_dim;
    const int64_t GN = static_cast<int64_t>(d->ngroups) * d->d_state;
    if (!tokens) {
        // no tokens: the conv state and the SSM state are carried through (as conv-then-scan does)
        ssd::ConvFwdArgs ca{xbc, xbc_row_stride, conv_w, conv_bias, conv_state_in, conv_state_out, nullptr,
                            d->batch, d->seqlen, CD};
        st = hip_status(ssd::launch_conv1d_fwd(ca, static_cast<Dt>(d->act_dtype), stream));
        if (st != SSD_OK) return st;
        return chunk_scan(d, chunk, nullptr, I, nullptr, nullptr, GN, nullptr, A, D, dt_params, init_state,
                          final_state, nullptr, 0, y, nullptr, 0, stream);
    }
    const size_t need = ssd_chunk_scan_workspace_size(d, chunk);
    if (!workspace || workspace_bytes < need) return SSD_ERR_WORKSPACE;
    if (!aligned16(workspace)) return SSD_ERR_ALIGN;
    const char* xb = static_cast<const char*>(xbc);
    const size_t es = elem_size(d->act_dtype);
    ssd::ScanArgs a{xbc, xbc_row_stride, xb + I * es, xb + (I + GN) * es, xbc_row_stride, dt, A, D,
                    init_state, final_state, y, d->batch, d->seqlen, d->nheads, d->head_dim, d->ngroups,
                    d->d_state, chunk, {nullptr, nullptr, nullptr, 0}, dt_params_of(dt_params), nullptr, 0};
    const ssd::ConvScanArgs c{xbc, xbc_row_stride, conv_w, conv_bias, conv_state_in, conv_state_out, CD};
    return hip_status(ssd::launch_conv_chunk_scan_f16(a, static_cast<Dt>(d->y_dtype), c, workspace, stream));
}

ssd_status_t ssd_chunk_scan_noalloc(const ssd_dims_t* d, int32_t chunk, const void* x, int64_t x_row_stride,
                                    const void* B, const void* C, int64_t bc_row_stride, const void* dt,
                                    const float* A, const float* D, const ssd_dt_params_t* dt_params,
                                    const float* init_state, float* final_state, void* y, hipStream_t stream) {
    // the fp16 scan's workspace is the static per-device array; the other scans need none
    const size_t need = ssd_chunk_scan_workspace_size(d, chunk);
    void* ws = nullptr;
    size_t ws_bytes = 0;
    if (need > 0) {
        if (ssd::f16_scan_scratch(&ws, &ws_bytes) != hipSuccess) return SSD_ERR_HIP;
        if (need > ws_bytes) return SSD_ERR_WORKSPACE;
    }
    return chunk_scan(d, chunk, x, x_row_stride, B, C, bc_row_stride, dt, A, D, dt_params, init_state, final_state,
                      nullptr, 0, y, ws, ws_bytes, stream);
}

ssd_status_t ssd_chunk_scan_snapshots(const ssd_dims_t* d, int32_t chunk, const void* x, int64_t x_row_stride,
                                      const void* B, const void* C, int64_t bc_row_stride, const void* dt,
                                      const float* A, const float* D, const ssd_dt_params_t* dt_params,
                                      const float* init_state, float* final_state, float* snapshots,
                                      int64_t interval, void* y, void* workspace, size_t workspace_bytes,
                                      hipStream_t stream) {
    if (!d) return SSD_ERR_NULL;
    if (interval <= 0 || interval % 128 != 0) return SSD_ERR_UNSUPPORTED;
    if (d->batch > 0 && d->seqlen >= interval && !snapshots) return SSD_ERR_NULL;
    if (snapshots && !aligned16(snapshots)) return SSD_ERR_ALIGN;
    return chunk_scan(d, chunk, x, x_row_stride, B, C, bc_row_stride, dt, A, D, dt_params, init_state, final_state,
                      snapshots, interval, y, workspace, workspace_bytes, stream);
}

// the packed scan, with optional snapshots into a pool (internal linkage)
static ssd_status_t chunk_scan_varlen(const ssd_dims_t* d, int32_t chunk, const void* x, int64_t x_row_stride,
                                      const void* B, const void* C, int64_t bc_row_stride, const void* dt,
                                      const float* A, const float* D, const ssd_dt_params_t* dt_params,
                                      const int32_t* cu_seqlens, const int32_t* slot_idx,
                                      const int32_t* has_initial_state, float* state_pool, int64_t nslots,
                                      float* snap_pool, int64_t nsnap_slots, const int32_t* snap_table,
                                      int32_t max_snaps, int64_t interval, void* y, void* workspace,
                                      size_t workspace_bytes, hipStream_t stream, const States16* s16 = nullptr) {
    ssd_status_t st = check_dims(d, true);
    if (st != SSD_OK) return st;
    st = check_seq_tables(d, cu_seqlens, s16 ? s16->fin : state_pool, nslots);
    if (st != SSD_OK) return st;
    st = check_states16(s16);
    if (st != SSD_OK) return st;
    if (d->batch > INT32_MAX || d->seqlen > INT32_MAX) return SSD_ERR_SHAPE;
    const bool tokens = d->batch > 0 && d->seqlen > 0;
    if (tokens && (!x || !B || !C || !dt || !A || !y)) return SSD_ERR_NULL;
    if (chunk != 64 && chunk != 128 && chunk != 256) return SSD_ERR_UNSUPPORTED;
    if (!pow2_16_128(d->head_dim) || !pow2_16_128(d->d_state)) return SSD_ERR_UNSUPPORTED;
    const int64_t I = static_cast<int64_t>(d->nheads) * d->head_dim;
    const int64_t GN = static_cast<int64_t>(d->ngroups) * d->d_state;
    if (tokens && (x_row_stride < I || bc_row_stride < GN)) return SSD_ERR_SHAPE;
    if (!stride_ok(x_row_stride, d->act_dtype) || !stride_ok(bc_row_stride, d->act_dtype)) return SSD_ERR_ALIGN;
    for (const void* p : {x, B, C, static_cast<const void*>(y)})
        if (p && !aligned16(p)) return SSD_ERR_ALIGN;
    if ((reinterpret_cast<uintptr_t>(dt) % elem_size(d->act_dtype)) != 0) return SSD_ERR_ALIGN;
    // A workspace selects the fp16 scan (fp32 state pool, no snapshots): it must then be large enough and
    // 16-byte aligned.  Without one the packed scan runs on the bf16 split-operand kernel.
    const size_t ws_need = (snap_table || s16) ? 0 : ssd_chunk_scan_varlen_workspace_size(d, chunk);
    const bool use_f16 = ws_need > 0 && workspace && workspace_bytes > 0;
    if (use_f16 && workspace_bytes < ws_need) return SSD_ERR_WORKSPACE;
    if (use_f16 && !aligned16(workspace)) return SSD_ERR_ALIGN;
    if (d->batch > 0 && !tokens && nslots == 0) return SSD_OK;   // nothing to compute or store
    if (!dt_params_ok(dt_params)) return SSD_ERR_ALIGN;
    ssd::ScanArgs a{x, x_row_stride, B, C, bc_row_stride, dt, A, D, state_pool, state_pool, y,
                    d->batch, d->seqlen, d->nheads, d->head_dim, d->ngroups, d->d_state, chunk,
                    {cu_seqlens, slot_idx, has_initial_state, nslots}, dt_params_of(dt_params)};
    set_states16(a, s16);
    if (snap_table && max_snaps > 0 && nsnap_slots > 0) {   // otherwise no snapshot can be stored
        a.snapshots = snap_pool;
        a.snap_interval = interval;
        a.snap_table = snap_table;
        a.snap_max = max_snaps;
        a.snap_slots = nsnap_slots;
    }
    const Dt act = static_cast<Dt>(d->act_dtype), ydt = static_cast<Dt>(d->y_dtype);
    if (use_f16) return hip_status(ssd::launch_chunk_scan_f16(a, ydt, workspace, stream));
    if (act == Dt::BF16 && ssd::mfma_scan_supports(d->head_dim, d->d_state, chunk))
        return hip_status(ssd::launch_chunk_scan_mfma(a, ydt, stream));
    return hip_status(ssd::launch_chunk_scan_fma(a, act, ydt, stream));
}

ssd_status_t ssd_chunk_scan_varlen(const ssd_dims_t* d, int32_t chunk, const void* x, int64_t x_row_stride,
                                   const void* B, const void* C, int64_t bc_row_stride, const void* dt,
                                   const float* A, const float* D, const ssd_dt_params_t* dt_params,
                                   const int32_t* cu_seqlens,
                                   const int32_t* slot_idx, const int32_t* has_initial_state,
                                   float* state_pool, int64_t nslots, void* y, void* workspace,
                                   size_t workspace_bytes, hipStream_t stream) {
    return chunk_scan_varlen(d, chunk, x, x_row_stride, B, C, bc_row_stride, dt, A, D, dt_params, cu_seqlens,
                             slot_idx, has_initial_state, state_pool, nslots, nullptr, 0, nullptr, 0, 0, y,
                             workspace, workspace_bytes, stream);
}

ssd_status_t ssd_chunk_scan_varlen_snapshots(const ssd_dims_t* d, int32_t chunk, const void* x,
                                             int64_t x_row_stride, const void* B, const void* C,
                                             int64_t bc_row_stride, const void* dt, const float* A, const float* D,
                                             const ssd_dt_params_t* dt_params, const int32_t* cu_seqlens,
                                             const int32_t* slot_idx, const int32_t* has_initial_state,
                                             float* state_pool, int64_t nslots, float* snap_pool,
                                             int64_t nsnap_slots, const int32_t* snap_table, int32_t max_snaps,
                                             int64_t interval, void* y, void* workspace, size_t workspace_bytes,
                                             hipStream_t stream) {
    if (!d) return SSD_ERR_NULL;
    if (interval <= 0 || interval % 128 != 0) return SSD_ERR_UNSUPPORTED;
    if (nsnap_slots < 0 || max_snaps < 0) return SSD_ERR_SHAPE;
    if (nsnap_slots > 0 && !snap_pool) return SSD_ERR_NULL;
    if (d->batch > 0 && max_snaps > 0 && !snap_table) return SSD_ERR_NULL;
    if (snap_pool && !aligned16(snap_pool)) return SSD_ERR_ALIGN;
    return chunk_scan_varlen(d, chunk, x, x_row_stride, B, C, bc_row_stride, dt, A, D, dt_params, cu_seqlens,
                             slot_idx, has_initial_state, state_pool, nslots, snap_pool, nsnap_slots, snap_table,
                             max_snaps, interval, y, workspace, workspace_bytes, stream);
}

ssd_status_t ssd_state_update_slots(const ssd_dims_t* d, float* state_pool, int64_t nslots, const int32_t* slot_idx,
                                    const void* x, int64_t x_row_stride, const void* B, const void* C,
                                    int64_t bc_row_stride, const void* dt, const float* A, const float* D,
                                    const ssd_dt_params_t* dt_params, void* y, hipStream_t stream) {
    ssd_status_t st = check_dims(d, false);
    if (st != SSD_OK) return st;
    if (nslots < 0) return SSD_ERR_SHAPE;
    if (d->batch > 0 && (!x || !B || !C || !dt || !A || !y || !slot_idx)) return SSD_ERR_NULL;
    if (nslots > 0 && !state_pool) return SSD_ERR_NULL;
    if (!pow2_16_128(d->head_dim) || !pow2_16_128(d->d_state)) return SSD_ERR_UNSUPPORTED;
    const int64_t I = static_cast<int64_t>(d->nheads) * d->head_dim;
    const int64_t GN = static_cast<int64_t>(d->ngroups) * d->d_state;
    if (x_row_stride < I || bc_row_stride < GN) return SSD_ERR_SHAPE;
    if (state_pool && !aligned16(state_pool)) return SSD_ERR_ALIGN;
    if (!dt_params_ok(dt_params)) return SSD_ERR_ALIGN;
    ssd::UpdateArgs a{state_pool, x, x_row_stride, B, C, bc_row_stride, dt, A, D, y,
                      d->batch, d->nheads, d->head_dim, d->ngroups, d->d_state, slot_idx, nslots,
                      dt_params_of(dt_params)};
    return hip_status(ssd::launch_state_update(a, static_cast<Dt>(d->act_dtype),
                                               static_cast<Dt>(d->y_dtype), stream));
}

ssd_status_t ssd_state_update(const ssd_dims_t* d, float* state, const void* x, int64_t x_row_stride,
                              const void* B, const void* C, int64_t bc_row_stride, const void* dt,
                              const float* A, const float* D, const ssd_dt_params_t* dt_params, void* y,
                              hipStream_t stream) {
    ssd_status_t st = check_dims(d, false);
    if (st != SSD_OK) return st;
    if (d->batch > 0 && (!state || !x || !B || !C || !dt || !A || !y)) return SSD_ERR_NULL;
    if (!pow2_16_128(d->head_dim) || !pow2_16_128(d->d_state)) return SSD_ERR_UNSUPPORTED;
    const int64_t I = static_cast<int64_t>(d->nheads) * d->head_dim;
    const int64_t GN = static_cast<int64_t>(d->ngroups) * d->d_state;
    if (x_row_stride < I || bc_row_stride < GN) return SSD_ERR_SHAPE;
    if (!aligned16(state)) return SSD_ERR_ALIGN;
    if (!dt_params_ok(dt_params)) return SSD_ERR_ALIGN;
    ssd::UpdateArgs a{state, x, x_row_stride, B, C, bc_row_stride, dt, A, D, y,
                      d->batch, d->nheads, d->head_dim, d->ngroups, d->d_state, nullptr, 0,
                      dt_params_of(dt_params)};
    return hip_status(ssd::launch_state_update(a, static_cast<Dt>(d->act_dtype),
                                               static_cast<Dt>(d->y_dtype), stream));
}

ssd_status_t ssd_state_update_multi(const ssd_dims_t* d, const float* state, const int32_t* slot_idx,
                                    int64_t nslots, const void* x, int64_t x_row_stride, const void* B,
                                    const void* C, int64_t bc_row_stride, const void* dt, const float* A,
                                    const float* D, const ssd_dt_params_t* dt_params, float* inter_states,
                                    void* y, hipStream_t stream) {
    ssd_status_t st = check_dims(d, true);
    if (st != SSD_OK) return st;
    if (nslots < 0 || d->seqlen > INT32_MAX) return SSD_ERR_SHAPE;
    const bool tokens = d->batch > 0 && d->seqlen > 0;
    if (tokens && (!x || !B || !C || !dt || !A || !y)) return SSD_ERR_NULL;
    if (tokens && !state && (!slot_idx || nslots > 0)) return SSD_ERR_NULL;
    if (!pow2_16_128(d->head_dim) || !pow2_16_128(d->d_state)) return SSD_ERR_UNSUPPORTED;
    const int64_t I = static_cast<int64_t>(d->nheads) * d->head_dim;
    const int64_t GN = static_cast<int64_t>(d->ngroups) * d->d_state;
    if (tokens && (x_row_stride < I || bc_row_stride < GN)) return SSD_ERR_SHAPE;
    if (!stride_ok(bc_row_stride, d->act_dtype)) return SSD_ERR_ALIGN;   // B/C are read 4 elements at a time
    for (const void* p : {static_cast<const void*>(state), static_cast<const void*>(inter_states), B, C})
        if (p && !aligned16(p)) return SSD_ERR_ALIGN;
    if (!dt_params_ok(dt_params)) return SSD_ERR_ALIGN;
    ssd::UpdateArgs a{const_cast<float*>(state), x, x_row_stride, B, C, bc_row_stride, dt, A, D, y,
                      d->batch, d->nheads, d->head_dim, d->ngroups, d->d_state, slot_idx, nslots,
                      dt_params_of(dt_params), inter_states, static_cast<int>(d->seqlen)};
    return hip_status(ssd::launch_state_update_multi(a, static_cast<Dt>(d->act_dtype),
                                                     static_cast<Dt>(d->y_dtype), stream));
}

ssd_status_t ssd_conv1d_update_multi(const ssd_dims_t* d, const void* xbc, int64_t xbc_row_stride,
                                     const void* w, const void* bias, const void* conv_state,
                                     const int32_t* slot_idx, int64_t nslots, void* inter_conv_states,
                                     void* out, hipStream_t stream) {
    ssd_status_t st = check_dims(d, true);
    if (st != SSD_OK) return st;
    if (nslots < 0 || d->seqlen > INT32_MAX) return SSD_ERR_SHAPE;
    const int64_t CD = ssd_conv_dim(d);
    const bool tokens = d->batch > 0 && d->seqlen > 0;
    if (tokens && (!xbc || !w || !out)) return SSD_ERR_NULL;
    if (tokens && !conv_state && (!slot_idx || nslots > 0)) return SSD_ERR_NULL;
    if (CD % 8 != 0) return SSD_ERR_UNSUPPORTED;
    if (tokens && xbc_row_stride < CD) return SSD_ERR_SHAPE;
    if (!stride_ok(xbc_row_stride, d->act_dtype)) return SSD_ERR_ALIGN;
    for (const void* p : {xbc, w, bias, conv_state, static_cast<const void*>(inter_conv_states),
                          static_cast<const void*>(out)})
        if (p && !aligned16(p)) return SSD_ERR_ALIGN;
    ssd::ConvUpdateArgs a{xbc, xbc_row_stride, w, bias, const_cast<void*>(conv_state), out, d->batch, CD,
                          slot_idx, nslots, inter_conv_states, static_cast<int>(d->seqlen)};
    return hip_status(ssd::launch_conv1d_update_multi(a, static_cast<Dt>(d->act_dtype), stream));
}

ssd_status_t ssd_state_update_accept(const ssd_dims_t* d, float* state, const int32_t* slot_idx, int64_t nslots,
                                     const void* x, int64_t x_row_stride, const void* B, const void* C,
                                     int64_t bc_row_stride, const void* dt, const float* A, const float* D,
                                     const ssd_dt_params_t* dt_params, const int32_t* accept_len, hipStream_t stream) {
    ssd_status_t st = check_dims(d, true);
    if (st != SSD_OK) return st;
    if (nslots < 0 || d->seqlen > INT32_MAX) return SSD_ERR_SHAPE;
    const bool tokens = d->batch > 0 && d->seqlen > 0 && (!slot_idx || nslots > 0);
    if (tokens && (!x || !B || !C || !dt || !A || !accept_len || !state)) return SSD_ERR_NULL;
    if (!pow2_16_128(d->head_dim) || !pow2_16_128(d->d_state)) return SSD_ERR_UNSUPPORTED;
    const int64_t I = static_cast<int64_t>(d->nheads) * d->head_dim;
    const int64_t GN = static_cast<int64_t>(d->ngroups) * d->d_state;
    if (tokens && (x_row_stride < I || bc_row_stride < GN)) return SSD_ERR_SHAPE;
    if (!stride_ok(bc_row_stride, d->act_dtype)) return SSD_ERR_ALIGN;
    for (const void* p : {static_cast<const void*>(state), B, C})
        if (p && !aligned16(p)) return SSD_ERR_ALIGN;
    if (!dt_params_ok(dt_params)) return SSD_ERR_ALIGN;
    if (!tokens) return SSD_OK;
    ssd::UpdateArgs a{state, x, x_row_stride, B, C, bc_row_stride, dt, A, D, nullptr,
                      d->batch, d->nheads, d->head_dim, d->ngroups, d->d_state, slot_idx, nslots,
                      dt_params_of(dt_params), nullptr, static_cast<int>(d->seqlen), accept_len};
    return hip_status(ssd::launch_state_update_multi(a, static_cast<Dt>(d->act_dtype), static_cast<Dt>(d->act_dtype),
                                                     stream));
}

ssd_status_t ssd_conv1d_update_accept(const ssd_dims_t* d, const void* xbc, int64_t xbc_row_stride, void* conv_state,
                                      const int32_t* slot_idx, int64_t nslots, const int32_t* accept_len,
                                      hipStream_t stream) {
    ssd_status_t st = check_dims(d, true);
    if (st != SSD_OK) return st;
    if (nslots < 0 || d->seqlen > INT32_MAX) return SSD_ERR_SHAPE;
    const int64_t CD = ssd_conv_dim(d);
    const bool tokens = d->batch > 0 && d->seqlen > 0 && (!slot_idx || nslots > 0);
    if (tokens && (!xbc || !conv_state || !accept_len)) return SSD_ERR_NULL;
    if (CD % 8 != 0) return SSD_ERR_UNSUPPORTED;
    if (tokens && xbc_row_stride < CD) return SSD_ERR_SHAPE;
    if (!stride_ok(xbc_row_stride, d->act_dtype)) return SSD_ERR_ALIGN;
    for (const void* p : {xbc, static_cast<const void*>(conv_state)})
        if (p && !aligned16(p)) return SSD_ERR_ALIGN;
    if (!tokens) return SSD_OK;
    ssd::ConvUpdateArgs a{xbc, xbc_row_stride, nullptr, nullptr, conv_state, nullptr, d->batch, CD,
                          slot_idx, nslots, nullptr, static_cast<int>(d->seqlen)};
    return hip_status(ssd::launch_conv1d_update_accept(a, accept_len, static_cast<Dt>(d->act_dtype), stream));
}

ssd_status_t ssd_accept_states(const ssd_dims_t* d, const int32_t* accept_len, const int32_t* slot_idx,
                               int64_t nslots, float* state, const float* inter_states, void* conv_state,
                               const void* inter_conv_states, hipStream_t stream) {
    ssd_status_t st = check_dims(d, true);
    if (st != SSD_OK) return st;
    if (nslots < 0 || d->seqlen > INT32_MAX) return SSD_ERR_SHAPE;
    if (d->batch > 65535) return SSD_ERR_UNSUPPORTED;   // one grid row per request
    if ((state == nullptr) != (inter_states == nullptr)) return SSD_ERR_NULL;
    if ((conv_state == nullptr) != (inter_conv_states == nullptr)) return SSD_ERR_NULL;
    const bool work = d->batch > 0 && d->seqlen > 0 && (state || conv_state) && (!slot_idx || nslots > 0);
    if (work && !accept_len) return SSD_ERR_NULL;
    if (ssd_conv_dim(d) % 8 != 0) return SSD_ERR_UNSUPPORTED;
    for (const void* p : {static_cast<const void*>(state), static_cast<const void*>(inter_states),
                          static_cast<const void*>(conv_state), inter_conv_states})
        if (p && !aligned16(p)) return SSD_ERR_ALIGN;
    if (!work) return SSD_OK;
    const int64_t state_bytes = static_cast<int64_t>(d->nheads) * d->head_dim * d->d_state * 4;
    const int64_t conv_bytes = ssd_conv_dim(d) * 4 * elem_size(d->act_dtype);
    ssd::AcceptArgs a{accept_len, slot_idx, nslots, d->batch, static_cast<int>(d->seqlen),
                      state, inter_states, state_bytes, conv_state, inter_conv_states, conv_bytes};
    return hip_status(ssd::launch_accept_states(a, stream));
}

ssd_status_t ssd_chunk_scan_lp(const ssd_dims_t* d, int32_t chunk, const void* x, int64_t x_row_stride,
                               const void* B, const void* C, int64_t bc_row_stride, const void* dt,
                               const float* A, const float* D, const ssd_dt_params_t* dt_params,
                               const void* init_state, void* final_state, int32_t state_dtype,
                               const ssd_sr_params_t* sr, void* y, void* workspace, size_t workspace_bytes,
                               hipStream_t stream) {
    const States16 s16{init_state, final_state, state_dtype, sr};
    return chunk_scan(d, chunk, x, x_row_stride, B, C, bc_row_stride, dt, A, D, dt_params, nullptr, nullptr,
                      nullptr, 0, y, workspace, workspace_bytes, stream, &s16);
}

ssd_status_t ssd_chunk_scan_varlen_lp(const ssd_dims_t* d, int32_t chunk, const void* x, int64_t x_row_stride,
                                      const void* B, const void* C, int64_t bc_row_stride, const void* dt,
                                      const float* A, const float* D, const ssd_dt_params_t* dt_params,
                                      const int32_t* cu_seqlens, const int32_t* slot_idx,
                                      const int32_t* has_initial_state, void* state_pool, int32_t state_dtype,
                                      int64_t nslots, const ssd_sr_params_t* sr, void* y, void* workspace,
                                      size_t workspace_bytes, hipStream_t stream) {
    const States16 s16{state_pool, state_pool, state_dtype, sr};
    return chunk_scan_varlen(d, chunk, x, x_row_stride, B, C, bc_row_stride, dt, A, D, dt_params, cu_seqlens,
                             slot_idx, has_initial_state, nullptr, nslots, nullptr, 0, nullptr, 0, 0, y, workspace,
                             workspace_bytes, stream, &s16);
}

ssd_status_t ssd_state_update_lp(const ssd_dims_t* d, void* state, int32_t state_dtype, const int32_t* slot_idx,
                                 int64_t nslots, const void* x, int64_t x_row_stride, const void* B, const void* C,
                                 int64_t bc_row_stride, const void* dt, const float* A, const float* D,
                                 const ssd_dt_params_t* dt_params, const ssd_sr_params_t* sr, void* y,
                                 hipStream_t stream) {
    ssd_status_t st = check_dims(d, false);
    if (st != SSD_OK) return st;
    if (state_dtype != SSD_F16 && state_dtype != SSD_BF16) return SSD_ERR_DTYPE;
    if (nslots < 0) return SSD_ERR_SHAPE;
    if (sr && (sr->rounds < 1 || sr->rounds > 16)) return SSD_ERR_UNSUPPORTED;
    if (d->batch > 0 && (!x || !B || !C || !dt || !A || !y)) return SSD_ERR_NULL;
    if (d->batch > 0 && !state && (!slot_idx || nslots > 0)) return SSD_ERR_NULL;
    if (!pow2_16_128(d->head_dim) || !pow2_16_128(d->d_state)) return SSD_ERR_UNSUPPORTED;
    const int64_t I = static_cast<int64_t>(d->nheads) * d->head_dim;
    const int64_t GN = static_cast<int64_t>(d->ngroups) * d->d_state;
    if (x_row_stride < I || bc_row_stride < GN) return SSD_ERR_SHAPE;
    if (I * d->d_state >= (INT64_C(1) << 31)) return SSD_ERR_UNSUPPORTED;   // one state's offsets in 32 bits
    if (!stride_ok(bc_row_stride, d->act_dtype)) return SSD_ERR_ALIGN;   // B/C are read 8 elements at a time
    for (const void* p : {static_cast<const void*>(state), B, C})
        if (p && !aligned16(p)) return SSD_ERR_ALIGN;
    if (!dt_params_ok(dt_params)) return SSD_ERR_ALIGN;
    ssd::LpUpdateArgs a{{nullptr, x, x_row_stride, B, C, bc_row_stride, dt, A, D, y, d->batch, d->nheads,
                         d->head_dim, d->ngroups, d->d_state, slot_idx, slot_idx ? nslots : d->batch,
                         dt_params_of(dt_params)},
                        state, state_dtype == SSD_F16, sr ? sr->seed : 0, sr ? sr->offset : 0, sr ? sr->rounds : 0};
    return hip_status(ssd::launch_state_update_lp(a, static_cast<Dt>(d->act_dtype), static_cast<Dt>(d->y_dtype),
                                                  stream));
}

ssd_status_t ssd_gated_rmsnorm(const ssd_dims_t* d, const void* y, int64_t y_row_stride, const void* z,
                               int64_t z_row_stride, const float* weight, float eps, void* out, hipStream_t stream) {
    ssd_status_t st = check_dims(d, true);
    if (st != SSD_OK) return st;
    const int64_t rows = d->batch * d->seqlen;
    const int64_t I = static_cast<int64_t>(d->nheads) * d->head_dim;
    if (rows > 0 && (!y || !z || !weight || !out)) return SSD_ERR_NULL;
    if ((I / d->ngroups) % 8 != 0 || rows * d->ngroups >= (INT64_C(1) << 32)) return SSD_ERR_UNSUPPORTED;
    if (!(eps >= 0.f)) return SSD_ERR_SHAPE;
    if (rows > 0 && (y_row_stride < I || z_row_stride < I)) return SSD_ERR_SHAPE;
    if (!stride_ok(y_row_stride, d->y_dtype) || !stride_ok(z_row_stride, d->act_dtype)) return SSD_ERR_ALIGN;
    for (const void* p : {y, z, static_cast<const void*>(weight), static_cast<const void*>(out)})
        if (p && !aligned16(p)) return SSD_ERR_ALIGN;
    ssd::NormArgs a{y, y_row_stride, z, z_row_stride, weight, eps, out, rows, I, d->ngroups};
    return hip_status(ssd::launch_gated_rmsnorm(a, static_cast<Dt>(d->act_dtype), static_cast<Dt>(d->y_dtype),
                                                stream));
}

ssd_status_t ssd_decode_step(const ssd_dims_t* d, const void* xbc, int64_t xbc_row_stride, const void* w,
                             const void* bias, const void* conv_state_in, void* conv_state_out, float* state,
                             const void* dt, const float* A, const float* D, const ssd_dt_params_t* dt_params,
                             void* y, hipStream_t stream) {
    ssd_status_t st = check_dims(d, false);
    if (st != SSD_OK) return st;
    const int64_t CD = ssd_conv_dim(d);
    if (d->batch > 0 && (!xbc || !w || !conv_state_in || !conv_state_out || !state || !dt || !A || !y))
        return SSD_ERR_NULL;
    if (!pow2_16_128(d->head_dim) || !pow2_16_128(d->d_state)) return SSD_ERR_UNSUPPORTED;
    if (xbc_row_stride < CD) return SSD_ERR_SHAPE;
    // the old and new conv windows must be distinct buffers (every block reads the old ones)
    const uintptr_t cb = static_cast<uintptr_t>(d->batch) * CD * 4 * elem_size(d->act_dtype);
    const uintptr_t ci = reinterpret_cast<uintptr_t>(conv_state_in), co = reinterpret_cast<uintptr_t>(conv_state_out);
    if (d->batch > 0 && ci < co + cb && co < ci + cb) return SSD_ERR_SHAPE;
    if (state && !aligned16(state)) return SSD_ERR_ALIGN;
    if (!dt_params_ok(dt_params)) return SSD_ERR_ALIGN;
    ssd::DecodeStepArgs a{{state, nullptr, 0, nullptr, nullptr, 0, dt, A, D, y, d->batch, d->nheads, d->head_dim,
                           d->ngroups, d->d_state, nullptr, 0, dt_params_of(dt_params)},
                          xbc, xbc_row_stride, w, bias, conv_state_in, conv_state_out};
    return hip_status(ssd::launch_decode_step(a, static_cast<Dt>(d->act_dtype), static_cast<Dt>(d->y_dtype), stream));
}

}  // extern "C"
