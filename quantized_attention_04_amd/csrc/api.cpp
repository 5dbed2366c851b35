// api.cpp -- the C ABI (include/sage.h): argument validation, device check, dispatch.
#include <hip/hip_runtime.h>
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include <atomic>
#include <climits>
#include <cmath>

#include "../../include/sage.h"
#include "internal.hpp"

namespace {

thread_local char g_detail[512] = "";

sage_status fail(sage_status s, const char* fmt, ...) {
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_detail, sizeof(g_detail), fmt, ap);
    va_end(ap);
    return s;
}

sage_status ok() {
    g_detail[0] = '\0';
    return SAGE_OK;
}

constexpr int kMaxDevices = 64;
std::atomic<int> g_arch[kMaxDevices];  // 0 unknown, 1 gfx950, 2 other

sage_status check_device() {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0) {
        (void)hipGetLastError();
        return fail(SAGE_ERR_DEVICE, "no HIP device is available");
    }
    if (dev >= kMaxDevices) return fail(SAGE_ERR_DEVICE, "device index %d out of range", dev);
    int st = g_arch[dev].load(std::memory_order_relaxed);
    if (st == 0) {
        hipDeviceProp_t prop;
        if (hipGetDeviceProperties(&prop, dev) != hipSuccess) {
            (void)hipGetLastError();
            return fail(SAGE_ERR_DEVICE, "hipGetDeviceProperties failed for device %d", dev);
        }
        st = strncmp(prop.gcnArchName, "gfx950", 6) == 0 ? 1 : 2;
        g_arch[dev].store(st, std::memory_order_relaxed);
        if (st != 1) return fail(SAGE_ERR_DEVICE, "device %d is %s, this library is built for gfx950 only", dev,
                                 prop.gcnArchName);
    }
    if (st != 1) return fail(SAGE_ERR_DEVICE, "device %d is not gfx950", dev);
    return SAGE_OK;
}

sage_status launch_status(hipError_t e, const char* what) {
    if (e != hipSuccess) return fail(SAGE_ERR_HIP, "%s: kernel launch failed: %s", what, hipGetErrorString(e));
    return ok();
}

bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

constexpr int kMaxN = 1 << 28;     // tokens per sequence
constexpr int kMaxSplits = 64;     // key-range splits of one query tile
constexpr int kMaxGridYZ = 65535;  // batch and head grid dimensions

// Shared shape checks.  Returns SAGE_OK or the failing status (with detail set).
sage_status check_shape(int B, int Hq, int Hkv, int Nq, int Nkv, int D) {
    if (B <= 0 || Hq <= 0 || Hkv <= 0 || Nq <= 0 || Nkv <= 0 || D <= 0)
        return fail(SAGE_ERR_INVALID_ARG, "sizes must be positive (B=%d H_qo=%d H_kv=%d Nq=%d Nkv=%d D=%d)", B, Hq,
                    Hkv, Nq, Nkv, D);
    if (Hq % Hkv != 0)
        return fail(SAGE_ERR_INVALID_ARG, "num_qo_heads (%d) must be a multiple of num_kv_heads (%d)", Hq, Hkv);
    if (D > 256) return fail(SAGE_ERR_UNSUPPORTED, "head_dim %d > 256 is not supported", D);
    if (Nq > kMaxN || Nkv > kMaxN) return fail(SAGE_ERR_UNSUPPORTED, "sequence length above %d", kMaxN);
    if (B > kMaxGridYZ || Hq > kMaxGridYZ) return fail(SAGE_ERR_UNSUPPORTED, "batch or head count above %d", kMaxGridYZ);
    const double elems = double(B) * Hq * double(Nq > Nkv ? Nq : Nkv) * 128.0;
    if (elems > 9.0e15) return fail(SAGE_ERR_UNSUPPORTED, "tensor too large");
    return SAGE_OK;
}

int padded_dim(int D) { return D <= 0 || D > 256 ? 0 : (D <= 64 ? 64 : (D <= 128 ? 128 : 256)); }
int nblocks(int N) { return N <= 0 ? 0 : (N + 63) / 64; }

// Packed (variable-length) batches: rows and block slots per head.
int64_t varlen_rows(int total, int B) { return int64_t(total) + 64 * int64_t(B); }
int64_t varlen_slots(int total, int B) { return (varlen_rows(total, B) + 63) / 64; }

sage_status check_varlen(const int32_t* cu_q, const int32_t* cu_k, int B, int Hq, int Hkv, int total_q, int total_kv,
                         int max_q, int max_kv, int D) {
    if (!cu_q || !cu_k) return fail(SAGE_ERR_INVALID_ARG, "cu_seqlens pointers must not be null");
    if (!aligned(cu_q, 4) || !aligned(cu_k, 4)) return fail(SAGE_ERR_INVALID_ARG, "cu_seqlens must be 4-byte aligned");
    if (total_q <= 0 || total_kv <= 0)
        return fail(SAGE_ERR_INVALID_ARG, "total token counts must be positive (total_q=%d total_kv=%d)", total_q,
                    total_kv);
    sage_status s = check_shape(B, Hq, Hkv, max_q, max_kv, D);
    if (s != SAGE_OK) return s;
    if (varlen_rows(total_q, B) > INT32_MAX || varlen_rows(total_kv, B) > INT32_MAX)
        return fail(SAGE_ERR_UNSUPPORTED, "total tokens + 64 * batch above 2^31");
    return SAGE_OK;
}


// Checks shared by every attention call except those of the Q operand (not the shapes).
sage_status check_kv_attn_args(const int8_t* k_i8, const float* k_scale, const void* v_hat, const float* v_scale,
                               void* out, sage_dtype out_dtype, int is_causal, float sm_scale, sage_pv pv,
                               sage_accum accum, int D, const char* what) {
    if (!k_i8 || !k_scale || !v_hat || !out) return fail(SAGE_ERR_INVALID_ARG, "%s: null tensor pointer", what);
    if (out_dtype != SAGE_FP16 && out_dtype != SAGE_BF16)
        return fail(SAGE_ERR_INVALID_ARG, "bad out dtype %d", int(out_dtype));
    if (pv != SAGE_PV_FP16 && pv != SAGE_PV_FP8) return fail(SAGE_ERR_INVALID_ARG, "bad pv mode %d", int(pv));
    if (accum != SAGE_ACC_FP32 && accum != SAGE_ACC_FP16_FP32 && accum != SAGE_ACC_FP16 &&
        accum != SAGE_ACC_FP16_FP32_SPLIT)
        return fail(SAGE_ERR_INVALID_ARG, "bad accum mode %d", int(accum));
    if (is_causal != 0 && is_causal != 1) return fail(SAGE_ERR_INVALID_ARG, "is_causal must be 0 or 1");
    if (!std::isfinite(sm_scale) || !(sm_scale > 0.0f))
        return fail(SAGE_ERR_INVALID_ARG, "sm_scale must be finite and > 0 (got %g)", double(sm_scale));
    if (accum == SAGE_ACC_FP16)
        return fail(SAGE_ERR_UNSUPPORTED, "single-level fp16 PV accumulation is not offered: gfx950 matrix cores "
                                          "accumulate FP16/FP8 products in fp32");
    if (pv == SAGE_PV_FP8 && (!v_scale || !aligned(v_scale, 4)))
        return fail(SAGE_ERR_INVALID_ARG, "%s: FP8 mode needs v_scale", what);
    if (!aligned(k_i8, 16) || !aligned(v_hat, 16) || !aligned(k_scale, 4) || !aligned(out, (D % 4) == 0 ? 8 : 2))
        return fail(SAGE_ERR_INVALID_ARG, "%s: misaligned tensor", what);
    return SAGE_OK;
}

// Checks shared by the dense and the packed attention calls on quantised Q (not the shapes).
sage_status check_attn_args(const int8_t* q_i8, const float* q_scale, const int8_t* k_i8, const float* k_scale,
                            const void* v_hat, const float* v_scale, void* out, sage_dtype out_dtype, int is_causal,
                            float sm_scale, sage_pv pv, sage_accum accum, int D, const char* what) {
    if (!q_i8 || !q_scale) return fail(SAGE_ERR_INVALID_ARG, "%s: null tensor pointer", what);
    sage_status s = check_kv_attn_args(k_i8, k_scale, v_hat, v_scale, out, out_dtype, is_causal, sm_scale, pv, accum,
                                       D, what);
    if (s != SAGE_OK) return s;
    if (!aligned(q_i8, 16) || !aligned(q_scale, 4)) return fail(SAGE_ERR_INVALID_ARG, "%s: misaligned tensor", what);
    return SAGE_OK;
}

// Pointer, dtype and pv checks of the fused Q/K/V quantisation.
sage_status check_qkv_args(const void* q, const void* k, const void* v, sage_dtype dtype, sage_pv pv,
                           const int8_t* q_i8, const float* q_scale, const int8_t* k_i8, const float* k_scale,
                           const float* k_mean, const void* v_hat, const float* v_scale, const char* what) {
    if (!q || !k || !v || !q_i8 || !q_scale || !k_i8 || !k_scale || !k_mean || !v_hat)
        return fail(SAGE_ERR_INVALID_ARG, "%s: null tensor pointer", what);
    if (dtype != SAGE_FP16 && dtype != SAGE_BF16) return fail(SAGE_ERR_INVALID_ARG, "bad dtype %d", int(dtype));
    if (pv != SAGE_PV_FP16 && pv != SAGE_PV_FP8) return fail(SAGE_ERR_INVALID_ARG, "bad pv mode %d", int(pv));
    if (pv == SAGE_PV_FP8 && (!v_scale || !aligned(v_scale, 4)))
        return fail(SAGE_ERR_INVALID_ARG, "%s: FP8 mode needs v_scale", what);
    if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(q_i8, 16) || !aligned(k_i8, 16) ||
        !aligned(v_hat, 16) || !aligned(q_scale, 4) || !aligned(k_scale, 4) || !aligned(k_mean, 4))
        return fail(SAGE_ERR_INVALID_ARG, "%s: tensors must be 16-byte aligned (scales 4-byte)", what);
    return SAGE_OK;
}

}  // namespace

extern "C" {

int sage_abi_version(void) { return SAGE_ABI_VERSION; }

const char* sage_status_string(sage_status s) {
    switch (s) {
    case SAGE_OK: return "SAGE_OK";
    case SAGE_ERR_INVALID_ARG: return "SAGE_ERR_INVALID_ARG: invalid argument";
    case SAGE_ERR_UNSUPPORTED: return "SAGE_ERR_UNSUPPORTED: unsupported configuration";
    case SAGE_ERR_WORKSPACE: return "SAGE_ERR_WORKSPACE: workspace missing or too small";
    case SAGE_ERR_DEVICE: return "SAGE_ERR_DEVICE: no gfx950 device";
    case SAGE_ERR_HIP: return "SAGE_ERR_HIP: HIP launch failure";
    }
    return "unknown sage_status";
}

const char* sage_last_error_detail(void) { return g_detail; }

int sage_padded_dim(int D) { return padded_dim(D); }
int sage_num_blocks(int N) { return nblocks(N); }

size_t sage_quant_qk_workspace_bytes(int B, int H_kv, int Nkv, int D) {
    if (B <= 0 || H_kv <= 0 || Nkv <= 0 || D <= 0 || D > 256) return 0;
    return size_t(B) * size_t(H_kv) * size_t(nblocks(Nkv)) * size_t(D) * sizeof(double);
}

size_t sage_quant_v_workspace_bytes(int B, int H_kv, int D, sage_pv pv) {
    if (B <= 0 || H_kv <= 0 || D <= 0 || D > 256) return 0;
    if (pv != SAGE_PV_FP8) return 0;
    return size_t(B) * size_t(H_kv) * size_t(padded_dim(D)) * sizeof(uint32_t);
}

sage_status sage_quant_qk(const void* q, const void* k, sage_dtype dtype, sage_layout layout, int B, int H_qo,
                          int H_kv, int Nq, int Nkv, int D, int8_t* q_i8, float* q_scale, int8_t* k_i8,
                          float* k_scale, float* k_mean, void* workspace, size_t workspace_bytes, void* stream) {
    if (!q || !k || !q_i8 || !q_scale || !k_i8 || !k_scale || !k_mean)
        return fail(SAGE_ERR_INVALID_ARG, "sage_quant_qk: null tensor pointer");
    if (dtype != SAGE_FP16 && dtype != SAGE_BF16) return fail(SAGE_ERR_INVALID_ARG, "bad dtype %d", int(dtype));
    if (layout != SAGE_HND && layout != SAGE_NHD) return fail(SAGE_ERR_INVALID_ARG, "bad layout %d", int(layout));
    sage_status s = check_shape(B, H_qo, H_kv, Nq, Nkv, D);
    if (s != SAGE_OK) return s;
    if (!aligned(q, 16) || !aligned(k, 16) || !aligned(q_i8, 16) || !aligned(k_i8, 16) || !aligned(q_scale, 4) ||
        !aligned(k_scale, 4) || !aligned(k_mean, 4))
        return fail(SAGE_ERR_INVALID_ARG, "sage_quant_qk: tensors must be 16-byte aligned (scales 4-byte)");
    const size_t need = sage_quant_qk_workspace_bytes(B, H_kv, Nkv, D);
    if (!workspace || workspace_bytes < need || !aligned(workspace, 8))
        return fail(SAGE_ERR_WORKSPACE, "sage_quant_qk: workspace of %zu bytes (8-byte aligned) required, got %zu",
                    need, workspace ? workspace_bytes : size_t(0));
    s = check_device();
    if (s != SAGE_OK) return s;
    sage::QuantQKArgs a{};
    a.q = q;
    a.k = k;
    a.bf16 = dtype == SAGE_BF16;
    a.layout_nhd = layout == SAGE_NHD;
    a.B = B, a.Hq = H_qo, a.Hkv = H_kv, a.Nq = Nq, a.Nkv = Nkv, a.D = D;
    a.q_i8 = q_i8, a.q_scale = q_scale, a.k_i8 = k_i8, a.k_scale = k_scale, a.k_mean = k_mean;
    a.workspace = workspace;
    return launch_status(sage::launch_quant_qk(a, (hipStream_t)stream), "sage_quant_qk");
}

sage_status sage_quant_v(const void* v, sage_dtype dtype, sage_layout layout, int B, int H_kv, int Nkv, int D,
                         sage_pv pv, void* v_hat, float* v_scale, void* workspace, size_t workspace_bytes,
                         void* stream) {
    if (!v || !v_hat) return fail(SAGE_ERR_INVALID_ARG, "sage_quant_v: null tensor pointer");
    if (dtype != SAGE_FP16 && dtype != SAGE_BF16) return fail(SAGE_ERR_INVALID_ARG, "bad dtype %d", int(dtype));
    if (layout != SAGE_HND && layout != SAGE_NHD) return fail(SAGE_ERR_INVALID_ARG, "bad layout %d", int(layout));
    if (pv != SAGE_PV_FP16 && pv != SAGE_PV_FP8) return fail(SAGE_ERR_INVALID_ARG, "bad pv mode %d", int(pv));
    sage_status s = check_shape(B, H_kv, H_kv, Nkv, Nkv, D);
    if (s != SAGE_OK) return s;
    if (!aligned(v, 16) || !aligned(v_hat, 16)) return fail(SAGE_ERR_INVALID_ARG, "sage_quant_v: tensors must be 16-byte aligned");
    if (pv == SAGE_PV_FP8) {
        if (!v_scale || !aligned(v_scale, 4)) return fail(SAGE_ERR_INVALID_ARG, "sage_quant_v: FP8 mode needs v_scale");
        const size_t need = sage_quant_v_workspace_bytes(B, H_kv, D, pv);
        if (!workspace || workspace_bytes < need || !aligned(workspace, 4))
            return fail(SAGE_ERR_WORKSPACE, "sage_quant_v: workspace of %zu bytes required, got %zu", need,
                        workspace ? workspace_bytes : size_t(0));
    }
    s = check_device();
    if (s != SAGE_OK) return s;
    sage::QuantVArgs a{};
    a.v = v;
    a.bf16 = dtype == SAGE_BF16;
    a.layout_nhd = layout == SAGE_NHD;
    a.B = B, a.Hkv = H_kv, a.Nkv = Nkv, a.D = D;
    a.fp8 = pv == SAGE_PV_FP8;
    a.v_hat = v_hat, a.v_scale = v_scale, a.workspace = workspace;
    return launch_status(sage::launch_quant_v(a, (hipStream_t)stream), "sage_quant_v");
}

size_t sage_quant_qkv_workspace_bytes(int B, int H_kv, int Nkv, int D, sage_pv pv) {
    if (B <= 0 || H_kv <= 0 || Nkv <= 0 || D <= 0 || D > 256) return 0;
    if (pv != SAGE_PV_FP16 && pv != SAGE_PV_FP8) return 0;
    return sage::qkv_workspace(B, H_kv, Nkv, D, false, 0, pv == SAGE_PV_FP8).bytes;
}

sage_status sage_quant_qkv(const void* q, const void* k, const void* v, sage_dtype dtype, sage_layout layout, int B,
                           int H_qo, int H_kv, int Nq, int Nkv, int D, sage_pv pv, sage_qk_gran gran, int8_t* q_i8,
                           float* q_scale, int8_t* k_i8, float* k_scale, float* k_mean, void* v_hat, float* v_scale,
                           void* workspace, size_t workspace_bytes, void* stream) {
    if (gran != SAGE_GRAN_BLOCK && gran != SAGE_GRAN_THREAD)
        return fail(SAGE_ERR_INVALID_ARG, "bad quantisation granularity %d", int(gran));
    sage_status s = check_qkv_args(q, k, v, dtype, pv, q_i8, q_scale, k_i8, k_scale, k_mean, v_hat, v_scale,
                                   "sage_quant_qkv");
    if (s != SAGE_OK) return s;
    if (layout != SAGE_HND && layout != SAGE_NHD) return fail(SAGE_ERR_INVALID_ARG, "bad layout %d", int(layout));
    s = check_shape(B, H_qo, H_kv, Nq, Nkv, D);
    if (s != SAGE_OK) return s;
    const size_t need = sage_quant_qkv_workspace_bytes(B, H_kv, Nkv, D, pv);
    if (!workspace || workspace_bytes < need || !aligned(workspace, 8))
        return fail(SAGE_ERR_WORKSPACE, "sage_quant_qkv: workspace of %zu bytes (8-byte aligned) required, got %zu",
                    need, workspace ? workspace_bytes : size_t(0));
    s = check_device();
    if (s != SAGE_OK) return s;
    sage::QuantQKArgs a{};
    a.q = q, a.k = k;
    a.bf16 = dtype == SAGE_BF16;
    a.layout_nhd = layout == SAGE_NHD;
    a.B = B, a.Hq = H_qo, a.Hkv = H_kv, a.Nq = Nq, a.Nkv = Nkv, a.D = D;
    a.q_i8 = q_i8, a.q_scale = q_scale, a.k_i8 = k_i8, a.k_scale = k_scale, a.k_mean = k_mean;
    a.workspace = workspace;
    a.thread_gran = gran == SAGE_GRAN_THREAD;
    sage::QuantVArgs va{};
    va.v = v;
    va.fp8 = pv == SAGE_PV_FP8;
    va.v_hat = v_hat, va.v_scale = v_scale;
    return launch_status(sage::launch_quant_qkv(a, va, (hipStream_t)stream), "sage_quant_qkv");
}

sage_status sage_quant_kv(const void* k, const void* v, sage_dtype dtype, sage_layout layout, int B, int H_kv, int Nkv,
                          int D, sage_pv pv, int8_t* k_i8, float* k_scale, float* k_mean, void* v_hat, float* v_scale,
                          void* workspace, size_t workspace_bytes, void* stream) {
    if (!k || !v || !k_i8 || !k_scale || !k_mean || !v_hat)
        return fail(SAGE_ERR_INVALID_ARG, "sage_quant_kv: null tensor pointer");
    if (dtype != SAGE_FP16 && dtype != SAGE_BF16) return fail(SAGE_ERR_INVALID_ARG, "bad dtype %d", int(dtype));
    if (pv != SAGE_PV_FP16 && pv != SAGE_PV_FP8) return fail(SAGE_ERR_INVALID_ARG, "bad pv mode %d", int(pv));
    if (pv == SAGE_PV_FP8 && (!v_scale || !aligned(v_scale, 4)))
        return fail(SAGE_ERR_INVALID_ARG, "sage_quant_kv: FP8 mode needs v_scale");
    if (!aligned(k, 16) || !aligned(v, 16) || !aligned(k_i8, 16) || !aligned(v_hat, 16) || !aligned(k_scale, 4) ||
        !aligned(k_mean, 4))
        return fail(SAGE_ERR_INVALID_ARG, "sage_quant_kv: tensors must be 16-byte aligned (scales 4-byte)");
    if (layout != SAGE_HND && layout != SAGE_NHD) return fail(SAGE_ERR_INVALID_ARG, "bad layout %d", int(layout));
    sage_status s = check_shape(B, H_kv, H_kv, Nkv, Nkv, D);
    if (s != SAGE_OK) return s;
    const size_t need = sage_quant_qkv_workspace_bytes(B, H_kv, Nkv, D, pv);
    if (!workspace || workspace_bytes < need || !aligned(workspace, 8))
        return fail(SAGE_ERR_WORKSPACE, "sage_quant_kv: workspace of %zu bytes (8-byte aligned) required, got %zu", need,
                    workspace ? workspace_bytes : size_t(0));
    s = check_device();
    if (s != SAGE_OK) return s;
    sage::QuantQKArgs a{};
    a.q = nullptr;  // no Q: the K/V part of sage_quant_qkv's schedule
    a.k = k;
    a.bf16 = dtype == SAGE_BF16;
    a.layout_nhd = layout == SAGE_NHD;
    a.B = B, a.Hq = H_kv, a.Hkv = H_kv, a.Nq = Nkv, a.Nkv = Nkv, a.D = D;
    a.k_i8 = k_i8, a.k_scale = k_scale, a.k_mean = k_mean;
    a.workspace = workspace;
    sage::QuantVArgs va{};
    va.v = v;
    va.fp8 = pv == SAGE_PV_FP8;
    va.v_hat = v_hat, va.v_scale = v_scale;
    return launch_status(sage::launch_quant_qkv(a, va, (hipStream_t)stream), "sage_quant_kv");
}

sage_status sage_attn_fwd_fused_q(const void* q, sage_dtype dtype, sage_layout layout, const int8_t* k_i8,
                                  const float* k_scale, const void* v_hat, const float* v_scale, void* out, int B,
                                  int H_qo, int H_kv, int Nq, int Nkv, int D, int is_causal, float sm_scale, sage_pv pv,
                                  sage_accum accum, int8_t* q_i8_out, float* q_scale_out, void* stream) {
    if (!q) return fail(SAGE_ERR_INVALID_ARG, "sage_attn_fwd_fused_q: null q");
    if (dtype != SAGE_FP16 && dtype != SAGE_BF16) return fail(SAGE_ERR_INVALID_ARG, "bad dtype %d", int(dtype));
    sage_status s = check_kv_attn_args(k_i8, k_scale, v_hat, v_scale, out, dtype, is_causal, sm_scale, pv, accum, D,
                                       "sage_attn_fwd_fused_q");
    if (s != SAGE_OK) return s;
    if (!aligned(q, 16) || (q_i8_out && !aligned(q_i8_out, 16)) || (q_scale_out && !aligned(q_scale_out, 4)))
        return fail(SAGE_ERR_INVALID_ARG, "sage_attn_fwd_fused_q: q and q_i8_out must be 16-byte aligned");
    if (accum == SAGE_ACC_FP16_FP32_SPLIT)
        return fail(SAGE_ERR_UNSUPPORTED, "sage_attn_fwd_fused_q: SAGE_ACC_FP16_FP32_SPLIT is not offered here");
    if (layout != SAGE_HND && layout != SAGE_NHD) return fail(SAGE_ERR_INVALID_ARG, "bad layout %d", int(layout));
    s = check_shape(B, H_qo, H_kv, Nq, Nkv, D);
    if (s != SAGE_OK) return s;
    s = check_device();
    if (s != SAGE_OK) return s;
    sage::AttnArgs a{};
    a.k_i8 = k_i8, a.k_scale = k_scale, a.v_hat = v_hat, a.v_scale = v_scale;
    a.out = out;
    a.out_bf16 = dtype == SAGE_BF16;
    a.out_nhd = layout == SAGE_NHD;
    a.B = B, a.Hq = H_qo, a.Hkv = H_kv, a.Nq = Nq, a.Nkv = Nkv, a.D = D;
    a.causal = is_causal;
    a.sm_scale = sm_scale;
    a.fp8 = pv == SAGE_PV_FP8;
    a.q16 = q;
    a.q_bf16 = dtype == SAGE_BF16;
    a.q_nhd = layout == SAGE_NHD;
    a.q_i8_out = q_i8_out;
    a.q_scale_out = q_scale_out;
    return launch_status(sage::launch_attn_fwd(a, (hipStream_t)stream), "sage_attn_fwd_fused_q");
}

size_t sage_quant_qkv_noalloc_max_bytes(void) { return sage::kNoAllocScratchBytes; }

sage_status sage_quant_qkv_noalloc(const void* q, const void* k, const void* v, sage_dtype dtype, sage_layout layout,
                                   int B, int H_qo, int H_kv, int Nq, int Nkv, int D, sage_pv pv, sage_qk_gran gran,
                                   int8_t* q_i8, float* q_scale, int8_t* k_i8, float* k_scale, float* k_mean,
                                   void* v_hat, float* v_scale, void* stream) {
    if (gran != SAGE_GRAN_BLOCK && gran != SAGE_GRAN_THREAD)
        return fail(SAGE_ERR_INVALID_ARG, "bad quantisation granularity %d", int(gran));
    sage_status s = check_qkv_args(q, k, v, dtype, pv, q_i8, q_scale, k_i8, k_scale, k_mean, v_hat, v_scale,
                                   "sage_quant_qkv_noalloc");
    if (s != SAGE_OK) return s;
    if (layout != SAGE_HND && layout != SAGE_NHD) return fail(SAGE_ERR_INVALID_ARG, "bad layout %d", int(layout));
    s = check_shape(B, H_qo, H_kv, Nq, Nkv, D);
    if (s != SAGE_OK) return s;
    const size_t need = sage_quant_qkv_workspace_bytes(B, H_kv, Nkv, D, pv);
    if (need > sage::kNoAllocScratchBytes)
        return fail(SAGE_ERR_UNSUPPORTED,
                    "sage_quant_qkv_noalloc: these sizes need %zu bytes of workspace, the static scratch holds %zu "
                    "(use sage_quant_qkv with a caller-supplied workspace)",
                    need, sage::kNoAllocScratchBytes);
    s = check_device();
    if (s != SAGE_OK) return s;
    void* ws = nullptr;
    const hipError_t e = sage::noalloc_scratch(&ws);
    if (e != hipSuccess)
        return fail(SAGE_ERR_HIP, "sage_quant_qkv_noalloc: no device address for the static scratch: %s",
                    hipGetErrorString(e));
    sage::QuantQKArgs a{};
    a.q = q, a.k = k;
    a.bf16 = dtype == SAGE_BF16;
    a.layout_nhd = layout == SAGE_NHD;
    a.B = B, a.Hq = H_qo, a.Hkv = H_kv, a.Nq = Nq, a.Nkv = Nkv, a.D = D;
    a.q_i8 = q_i8, a.q_scale = q_scale, a.k_i8 = k_i8, a.k_scale = k_scale, a.k_mean = k_mean;
    a.workspace = ws;
    a.thread_gran = gran == SAGE_GRAN_THREAD;
    sage::QuantVArgs va{};
    va.v = v;
    va.fp8 = pv == SAGE_PV_FP8;
    va.v_hat = v_hat, va.v_scale = v_scale;
    return launch_status(sage::launch_quant_qkv(a, va, (hipStream_t)stream), "sage_quant_qkv_noalloc");
}

sage_status sage_attn_fwd(const int8_t* q_i8, const float* q_scale, const int8_t* k_i8, const float* k_scale,
                          const void* v_hat, const float* v_scale, void* out, sage_dtype out_dtype,
                          sage_layout out_layout, int B, int H_qo, int H_kv, int Nq, int Nkv, int D, int is_causal,
                          float sm_scale, sage_pv pv, sage_accum accum, void* stream) {
    return sage_attn_fwd_g(q_i8, q_scale, k_i8, k_scale, v_hat, v_scale, out, out_dtype, out_layout, B, H_qo, H_kv,
                           Nq, Nkv, D, is_causal, sm_scale, pv, accum, SAGE_GRAN_BLOCK, stream);
}

sage_status sage_attn_fwd_g(const int8_t* q_i8, const float* q_scale, const int8_t* k_i8, const float* k_scale,
                            const void* v_hat, const float* v_scale, void* out, sage_dtype out_dtype,
                            sage_layout out_layout, int B, int H_qo, int H_kv, int Nq, int Nkv, int D, int is_causal,
                            float sm_scale, sage_pv pv, sage_accum accum, sage_qk_gran gran, void* stream) {
    if (gran != SAGE_GRAN_BLOCK && gran != SAGE_GRAN_THREAD)
        return fail(SAGE_ERR_INVALID_ARG, "bad quantisation granularity %d", int(gran));
    if (gran == SAGE_GRAN_THREAD && accum == SAGE_ACC_FP16_FP32_SPLIT)
        return fail(SAGE_ERR_UNSUPPORTED, "SAGE_ACC_FP16_FP32_SPLIT is offered with SAGE_GRAN_BLOCK only");
    sage_status s = check_attn_args(q_i8, q_scale, k_i8, k_scale, v_hat, v_scale, out, out_dtype, is_causal, sm_scale,
                                    pv, accum, D, "sage_attn_fwd");
    if (s != SAGE_OK) return s;
    if (out_layout != SAGE_HND && out_layout != SAGE_NHD)
        return fail(SAGE_ERR_INVALID_ARG, "bad layout %d", int(out_layout));
    s = check_shape(B, H_qo, H_kv, Nq, Nkv, D);
    if (s != SAGE_OK) return s;
    s = check_device();
    if (s != SAGE_OK) return s;
    sage::AttnArgs a{};
    a.q_i8 = q_i8, a.q_scale = q_scale, a.k_i8 = k_i8, a.k_scale = k_scale, a.v_hat = v_hat, a.v_scale = v_scale;
    a.out = out;
    a.out_bf16 = out_dtype == SAGE_BF16;
    a.out_nhd = out_layout == SAGE_NHD;
    a.B = B, a.Hq = H_qo, a.Hkv = H_kv, a.Nq = Nq, a.Nkv = Nkv, a.D = D;
    a.causal = is_causal;
    a.sm_scale = sm_scale;
    a.fp8 = pv == SAGE_PV_FP8;
    a.split_partials = accum == SAGE_ACC_FP16_FP32_SPLIT;
    a.thread_gran = gran == SAGE_GRAN_THREAD;
    return launch_status(sage::launch_attn_fwd(a, (hipStream_t)stream), "sage_attn_fwd");
}

int sage_attn_fwd_split_choice(int B, int H_qo, int Nq, int Nkv, int D, int is_causal, sage_pv pv) {
    (void)is_causal;
    if (B <= 0 || H_qo <= 0 || Nq <= 0 || Nkv <= 0 || D <= 0 || D > 256 || pv != SAGE_PV_FP16) return 1;
    // workgroups of the unsplit launch (128 queries each); a split pays when they leave
    // CUs idle: aim at two workgroups per CU (256 CUs), every split >= 4 key tiles
    const int64_t nwg = int64_t(B) * H_qo * ((Nq + 127) / 128);
    const int nbk = nblocks(Nkv);
    if (nwg >= 384 || nbk < 8) return 1;
    int S = int((512 + nwg - 1) / nwg);
    S = S < nbk / 4 ? S : nbk / 4;
    S = S < 16 ? S : 16;
    if (S <= 1) return 1;
    const int tps = (nbk + S - 1) / S;
    return (nbk + tps - 1) / tps;
}

size_t sage_attn_fwd_split_workspace_bytes(int B, int H_qo, int Nq, int D, int num_splits) {
    if (B <= 0 || H_qo <= 0 || Nq <= 0 || D <= 0 || D > 256 || num_splits <= 1 || num_splits > kMaxSplits) return 0;
    return sage::attn_split_workspace(B, H_qo, Nq, D, num_splits).bytes;
}

sage_status sage_attn_fwd_split(const int8_t* q_i8, const float* q_scale, const int8_t* k_i8, const float* k_scale,
                                const void* v_hat, const float* v_scale, void* out, sage_dtype out_dtype,
                                sage_layout out_layout, int B, int H_qo, int H_kv, int Nq, int Nkv, int D,
                                int is_causal, float sm_scale, sage_pv pv, sage_accum accum, int num_splits,
                                void* workspace, size_t workspace_bytes, void* stream) {
    if (num_splits < 1 || num_splits > kMaxSplits)
        return fail(SAGE_ERR_INVALID_ARG, "num_splits must be in 1..%d (got %d)", kMaxSplits, num_splits);
    if (num_splits == 1)
        return sage_attn_fwd_g(q_i8, q_scale, k_i8, k_scale, v_hat, v_scale, out, out_dtype, out_layout, B, H_qo,
                               H_kv, Nq, Nkv, D, is_causal, sm_scale, pv, accum, SAGE_GRAN_BLOCK, stream);
    sage_status s = check_attn_args(q_i8, q_scale, k_i8, k_scale, v_hat, v_scale, out, out_dtype, is_causal, sm_scale,
                                    pv, accum, D, "sage_attn_fwd_split");
    if (s != SAGE_OK) return s;
    if (out_layout != SAGE_HND && out_layout != SAGE_NHD)
        return fail(SAGE_ERR_INVALID_ARG, "bad layout %d", int(out_layout));
    s = check_shape(B, H_qo, H_kv, Nq, Nkv, D);
    if (s != SAGE_OK) return s;
    if (pv != SAGE_PV_FP16)
        return fail(SAGE_ERR_UNSUPPORTED, "sage_attn_fwd_split: key-range splits are offered with FP16 P.V only (each "
                                          "split's own running maximum would move FP8 P codes)");
    if (accum == SAGE_ACC_FP16_FP32_SPLIT)
        return fail(SAGE_ERR_UNSUPPORTED, "sage_attn_fwd_split: SAGE_ACC_FP16_FP32_SPLIT is not offered with splits");
    const size_t need = sage_attn_fwd_split_workspace_bytes(B, H_qo, Nq, D, num_splits);
    if (!workspace || workspace_bytes < need || !aligned(workspace, 16))
        return fail(SAGE_ERR_WORKSPACE, "sage_attn_fwd_split: workspace of %zu bytes (16-byte aligned) required, got %zu",
                    need, workspace ? workspace_bytes : size_t(0));
    s = check_device();
    if (s != SAGE_OK) return s;
    sage::AttnArgs a{};
    a.q_i8 = q_i8, a.q_scale = q_scale, a.k_i8 = k_i8, a.k_scale = k_scale, a.v_hat = v_hat, a.v_scale = v_scale;
    a.out = out;
    a.out_bf16 = out_dtype == SAGE_BF16;
    a.out_nhd = out_layout == SAGE_NHD;
    a.B = B, a.Hq = H_qo, a.Hkv = H_kv, a.Nq = Nq, a.Nkv = Nkv, a.D = D;
    a.causal = is_causal;
    a.sm_scale = sm_scale;
    a.fp8 = 0;
    a.splits = num_splits;
    a.workspace = workspace;
    return launch_status(sage::launch_attn_fwd(a, (hipStream_t)stream), "sage_attn_fwd_split");
}

sage_status sage_debug_qk_int32(const int8_t* q_i8, const int8_t* k_i8, int B, int H_qo, int H_kv, int Nq, int Nkv,
                                int D, sage_pv pv, const int32_t* tiles, int T, int32_t* out, void* stream) {
    if (!q_i8 || !k_i8 || !tiles || !out) return fail(SAGE_ERR_INVALID_ARG, "sage_debug_qk_int32: null pointer");
    if (pv != SAGE_PV_FP16 && pv != SAGE_PV_FP8) return fail(SAGE_ERR_INVALID_ARG, "bad pv mode %d", int(pv));
    if (T <= 0) return fail(SAGE_ERR_INVALID_ARG, "tile count must be positive");
    sage_status s = check_shape(B, H_qo, H_kv, Nq, Nkv, D);
    if (s != SAGE_OK) return s;
    if (!aligned(q_i8, 16) || !aligned(k_i8, 16) || !aligned(tiles, 4) || !aligned(out, 4))
        return fail(SAGE_ERR_INVALID_ARG, "sage_debug_qk_int32: misaligned tensor");
    s = check_device();
    if (s != SAGE_OK) return s;
    sage::DebugQKArgs a{q_i8, k_i8, B, H_qo, H_kv, Nq, Nkv, D, pv == SAGE_PV_FP8, tiles, T, out};
    return launch_status(sage::launch_debug_qk(a, (hipStream_t)stream), "sage_debug_qk_int32");
}

int64_t sage_varlen_rows(int total, int B) { return total <= 0 || B <= 0 ? 0 : varlen_rows(total, B); }
int64_t sage_varlen_slots(int total, int B) { return total <= 0 || B <= 0 ? 0 : varlen_slots(total, B); }

size_t sage_quant_qk_varlen_workspace_bytes(int B, int H_kv, int total_kv, int D) {
    if (B <= 0 || H_kv <= 0 || total_kv <= 0 || D <= 0 || D > 256) return 0;
    return size_t(H_kv) * size_t(varlen_slots(total_kv, B)) * size_t(D) * sizeof(double);
}

sage_status sage_quant_qk_varlen(const void* q, const void* k, sage_dtype dtype, const int32_t* cu_seqlens_q,
                                 const int32_t* cu_seqlens_kv, int B, int H_qo, int H_kv, int total_q, int total_kv,
                                 int max_seqlen_q, int max_seqlen_kv, int D, int8_t* q_i8, float* q_scale,
                                 int8_t* k_i8, float* k_scale, float* k_mean, void* workspace, size_t workspace_bytes,
                                 void* stream) {
    if (!q || !k || !q_i8 || !q_scale || !k_i8 || !k_scale || !k_mean)
        return fail(SAGE_ERR_INVALID_ARG, "sage_quant_qk_varlen: null tensor pointer");
    if (dtype != SAGE_FP16 && dtype != SAGE_BF16) return fail(SAGE_ERR_INVALID_ARG, "bad dtype %d", int(dtype));
    sage_status s = check_varlen(cu_seqlens_q, cu_seqlens_kv, B, H_qo, H_kv, total_q, total_kv, max_seqlen_q,
                                 max_seqlen_kv, D);
    if (s != SAGE_OK) return s;
    if (!aligned(q, 16) || !aligned(k, 16) || !aligned(q_i8, 16) || !aligned(k_i8, 16) || !aligned(q_scale, 4) ||
        !aligned(k_scale, 4) || !aligned(k_mean, 4))
        return fail(SAGE_ERR_INVALID_ARG, "sage_quant_qk_varlen: tensors must be 16-byte aligned (scales 4-byte)");
    const size_t need = sage_quant_qk_varlen_workspace_bytes(B, H_kv, total_kv, D);
    if (!workspace || workspace_bytes < need || !aligned(workspace, 8))
        return fail(SAGE_ERR_WORKSPACE, "sage_quant_qk_varlen: workspace of %zu bytes (8-byte aligned) required, got %zu",
                    need, workspace ? workspace_bytes : size_t(0));
    s = check_device();
    if (s != SAGE_OK) return s;
    sage::QuantQKArgs a{};
    a.q = q;
    a.k = k;
    a.bf16 = dtype == SAGE_BF16;
    a.B = B, a.Hq = H_qo, a.Hkv = H_kv, a.Nq = max_seqlen_q, a.Nkv = max_seqlen_kv, a.D = D;
    a.cu_q = cu_seqlens_q, a.cu_k = cu_seqlens_kv, a.total_q = total_q, a.total_k = total_kv;
    a.q_i8 = q_i8, a.q_scale = q_scale, a.k_i8 = k_i8, a.k_scale = k_scale, a.k_mean = k_mean;
    a.workspace = workspace;
    return launch_status(sage::launch_quant_qk(a, (hipStream_t)stream), "sage_quant_qk_varlen");
}

sage_status sage_quant_v_varlen(const void* v, sage_dtype dtype, const int32_t* cu_seqlens_kv, int B, int H_kv,
                                int total_kv, int max_seqlen_kv, int D, sage_pv pv, void* v_hat, float* v_scale,
                                void* workspace, size_t workspace_bytes, void* stream) {
    if (!v || !v_hat) return fail(SAGE_ERR_INVALID_ARG, "sage_quant_v_varlen: null tensor pointer");
    if (dtype != SAGE_FP16 && dtype != SAGE_BF16) return fail(SAGE_ERR_INVALID_ARG, "bad dtype %d", int(dtype));
    if (pv != SAGE_PV_FP16 && pv != SAGE_PV_FP8) return fail(SAGE_ERR_INVALID_ARG, "bad pv mode %d", int(pv));
    sage_status s = check_varlen(cu_seqlens_kv, cu_seqlens_kv, B, H_kv, H_kv, total_kv, total_kv, max_seqlen_kv,
                                 max_seqlen_kv, D);
    if (s != SAGE_OK) return s;
    if (!aligned(v, 16) || !aligned(v_hat, 16))
        return fail(SAGE_ERR_INVALID_ARG, "sage_quant_v_varlen: tensors must be 16-byte aligned");
    if (pv == SAGE_PV_FP8) {
        if (!v_scale || !aligned(v_scale, 4))
            return fail(SAGE_ERR_INVALID_ARG, "sage_quant_v_varlen: FP8 mode needs v_scale");
        const size_t need = sage_quant_v_workspace_bytes(B, H_kv, D, pv);
        if (!workspace || workspace_bytes < need || !aligned(workspace, 4))
            return fail(SAGE_ERR_WORKSPACE, "sage_quant_v_varlen: workspace of %zu bytes required, got %zu", need,
                        workspace ? workspace_bytes : size_t(0));
    }
    s = check_device();
    if (s != SAGE_OK) return s;
    sage::QuantVArgs a{};
    a.v = v;
    a.bf16 = dtype == SAGE_BF16;
    a.B = B, a.Hkv = H_kv, a.Nkv = max_seqlen_kv, a.D = D;
    a.cu_k = cu_seqlens_kv, a.total_k = total_kv;
    a.fp8 = pv == SAGE_PV_FP8;
    a.v_hat = v_hat, a.v_scale = v_scale, a.workspace = workspace;
    return launch_status(sage::launch_quant_v(a, (hipStream_t)stream), "sage_quant_v_varlen");
}

size_t sage_quant_qkv_varlen_workspace_bytes(int B, int H_kv, int total_kv, int D, sage_pv pv) {
    if (B <= 0 || H_kv <= 0 || total_kv <= 0 || D <= 0 || D > 256) return 0;
    if (pv != SAGE_PV_FP16 && pv != SAGE_PV_FP8) return 0;
    return sage::qkv_workspace(B, H_kv, 0, D, true, total_kv, pv == SAGE_PV_FP8).bytes;
}

sage_status sage_quant_qkv_varlen(const void* q, const void* k, const void* v, sage_dtype dtype,
                                  const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_kv, int B, int H_qo, int H_kv,
                                  int total_q, int total_kv, int max_seqlen_q, int max_seqlen_kv, int D, sage_pv pv,
                                  sage_qk_gran gran, int8_t* q_i8, float* q_scale, int8_t* k_i8, float* k_scale,
                                  float* k_mean, void* v_hat, float* v_scale, void* workspace, size_t workspace_bytes,
                                  void* stream) {
    if (gran != SAGE_GRAN_BLOCK && gran != SAGE_GRAN_THREAD)
        return fail(SAGE_ERR_INVALID_ARG, "bad quantisation granularity %d", int(gran));
    sage_status s = check_qkv_args(q, k, v, dtype, pv, q_i8, q_scale, k_i8, k_scale, k_mean, v_hat, v_scale,
                                   "sage_quant_qkv_varlen");
    if (s != SAGE_OK) return s;
    s = check_varlen(cu_seqlens_q, cu_seqlens_kv, B, H_qo, H_kv, total_q, total_kv, max_seqlen_q, max_seqlen_kv, D);
    if (s != SAGE_OK) return s;
    const size_t need = sage_quant_qkv_varlen_workspace_bytes(B, H_kv, total_kv, D, pv);
    if (!workspace || workspace_bytes < need || !aligned(workspace, 8))
        return fail(SAGE_ERR_WORKSPACE,
                    "sage_quant_qkv_varlen: workspace of %zu bytes (8-byte aligned) required, got %zu", need,
                    workspace ? workspace_bytes : size_t(0));
    s = check_device();
    if (s != SAGE_OK) return s;
    sage::QuantQKArgs a{};
    a.q = q, a.k = k;
    a.bf16 = dtype == SAGE_BF16;
    a.B = B, a.Hq = H_qo, a.Hkv = H_kv, a.Nq = max_seqlen_q, a.Nkv = max_seqlen_kv, a.D = D;
    a.cu_q = cu_seqlens_q, a.cu_k = cu_seqlens_kv, a.total_q = total_q, a.total_k = total_kv;
    a.q_i8 = q_i8, a.q_scale = q_scale, a.k_i8 = k_i8, a.k_scale = k_scale, a.k_mean = k_mean;
    a.workspace = workspace;
    a.thread_gran = gran == SAGE_GRAN_THREAD;
    sage::QuantVArgs va{};
    va.v = v;
    va.fp8 = pv == SAGE_PV_FP8;
    va.v_hat = v_hat, va.v_scale = v_scale;
    return launch_status(sage::launch_quant_qkv(a, va, (hipStream_t)stream), "sage_quant_qkv_varlen");
}

sage_status sage_quant_kv_varlen(const void* k, const void* v, sage_dtype dtype, const int32_t* cu_seqlens_kv, int B,
                                 int H_kv, int total_kv, int max_seqlen_kv, int D, sage_pv pv, int8_t* k_i8,
                                 float* k_scale, float* k_mean, void* v_hat, float* v_scale, void* workspace,
                                 size_t workspace_bytes, void* stream) {
    if (!k || !v || !k_i8 || !k_scale || !k_mean || !v_hat)
        return fail(SAGE_ERR_INVALID_ARG, "sage_quant_kv_varlen: null tensor pointer");
    if (dtype != SAGE_FP16 && dtype != SAGE_BF16) return fail(SAGE_ERR_INVALID_ARG, "bad dtype %d", int(dtype));
    if (pv != SAGE_PV_FP16 && pv != SAGE_PV_FP8) return fail(SAGE_ERR_INVALID_ARG, "bad pv mode %d", int(pv));
    if (pv == SAGE_PV_FP8 && (!v_scale || !aligned(v_scale, 4)))
        return fail(SAGE_ERR_INVALID_ARG, "sage_quant_kv_varlen: FP8 mode needs v_scale");
    if (!aligned(k, 16) || !aligned(v, 16) || !aligned(k_i8, 16) || !aligned(v_hat, 16) || !aligned(k_scale, 4) ||
        !aligned(k_mean, 4))
        return fail(SAGE_ERR_INVALID_ARG, "sage_quant_kv_varlen: tensors must be 16-byte aligned (scales 4-byte)");
    // the K/V sequences stand for both sides of the shared checks
    sage_status s = check_varlen(cu_seqlens_kv, cu_seqlens_kv, B, H_kv, H_kv, total_kv, total_kv, max_seqlen_kv,
                                 max_seqlen_kv, D);
    if (s != SAGE_OK) return s;
    const size_t need = sage_quant_qkv_varlen_workspace_bytes(B, H_kv, total_kv, D, pv);
    if (!workspace || workspace_bytes < need || !aligned(workspace, 8))
        return fail(SAGE_ERR_WORKSPACE,
                    "sage_quant_kv_varlen: workspace of %zu bytes (8-byte aligned) required, got %zu", need,
                    workspace ? workspace_bytes : size_t(0));
    s = check_device();
    if (s != SAGE_OK) return s;
    sage::QuantQKArgs a{};
    a.q = nullptr;  // no Q: the K/V part of sage_quant_qkv_varlen's schedule
    a.k = k;
    a.bf16 = dtype == SAGE_BF16;
    a.B = B, a.Hq = H_kv, a.Hkv = H_kv, a.Nq = max_seqlen_kv, a.Nkv = max_seqlen_kv, a.D = D;
    a.cu_q = cu_seqlens_kv, a.cu_k = cu_seqlens_kv, a.total_q = total_kv, a.total_k = total_kv;
    a.k_i8 = k_i8, a.k_scale = k_scale, a.k_mean = k_mean;
    a.workspace = workspace;
    sage::QuantVArgs va{};
    va.v = v;
    va.fp8 = pv == SAGE_PV_FP8;
    va.v_hat = v_hat, va.v_scale = v_scale;
    return launch_status(sage::launch_quant_qkv(a, va, (hipStream_t)stream), "sage_quant_kv_varlen");
}

sage_status sage_attn_fwd_varlen_fused_q(const void* q, sage_dtype dtype, const int32_t* cu_seqlens_q,
                                         const int32_t* cu_seqlens_kv, const int8_t* k_i8, const float* k_scale,
                                         const void* v_hat, const float* v_scale, void* out, int B, int H_qo, int H_kv,
                                         int total_q, int total_kv, int max_seqlen_q, int max_seqlen_kv, int D,
                                         int is_causal, float sm_scale, sage_pv pv, sage_accum accum, int8_t* q_i8_out,
                                         float* q_scale_out, void* stream) {
    if (!q) return fail(SAGE_ERR_INVALID_ARG, "sage_attn_fwd_varlen_fused_q: null q");
    if (dtype != SAGE_FP16 && dtype != SAGE_BF16) return fail(SAGE_ERR_INVALID_ARG, "bad dtype %d", int(dtype));
    sage_status s = check_kv_attn_args(k_i8, k_scale, v_hat, v_scale, out, dtype, is_causal, sm_scale, pv, accum, D,
                                       "sage_attn_fwd_varlen_fused_q");
    if (s != SAGE_OK) return s;
    if (!aligned(q, 16) || (q_i8_out && !aligned(q_i8_out, 16)) || (q_scale_out && !aligned(q_scale_out, 4)))
        return fail(SAGE_ERR_INVALID_ARG, "sage_attn_fwd_varlen_fused_q: q and q_i8_out must be 16-byte aligned");
    if (accum == SAGE_ACC_FP16_FP32_SPLIT)
        return fail(SAGE_ERR_UNSUPPORTED, "sage_attn_fwd_varlen_fused_q: SAGE_ACC_FP16_FP32_SPLIT is not offered here");
    s = check_varlen(cu_seqlens_q, cu_seqlens_kv, B, H_qo, H_kv, total_q, total_kv, max_seqlen_q, max_seqlen_kv, D);
    if (s != SAGE_OK) return s;
    s = check_device();
    if (s != SAGE_OK) return s;
    sage::AttnArgs a{};
    a.k_i8 = k_i8, a.k_scale = k_scale, a.v_hat = v_hat, a.v_scale = v_scale;
    a.out = out;
    a.out_bf16 = dtype == SAGE_BF16;
    a.B = B, a.Hq = H_qo, a.Hkv = H_kv, a.Nq = max_seqlen_q, a.Nkv = max_seqlen_kv, a.D = D;
    a.causal = is_causal;
    a.sm_scale = sm_scale;
    a.fp8 = pv == SAGE_PV_FP8;
    a.cu_q = cu_seqlens_q, a.cu_k = cu_seqlens_kv, a.total_q = total_q, a.total_k = total_kv;
    a.q16 = q;
    a.q_bf16 = dtype == SAGE_BF16;
    a.q_i8_out = q_i8_out;
    a.q_scale_out = q_scale_out;
    return launch_status(sage::launch_attn_fwd(a, (hipStream_t)stream), "sage_attn_fwd_varlen_fused_q");
}

sage_status sage_attn_fwd_varlen(const int8_t* q_i8, const float* q_scale, const int8_t* k_i8, const float* k_scale,
                                 const void* v_hat, const float* v_scale, void* out, sage_dtype out_dtype,
                                 const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_kv, int B, int H_qo, int H_kv,
                                 int total_q, int total_kv, int max_seqlen_q, int max_seqlen_kv, int D, int is_causal,
                                 float sm_scale, sage_pv pv, sage_accum accum, void* stream) {
    return sage_attn_fwd_varlen_g(q_i8, q_scale, k_i8, k_scale, v_hat, v_scale, out, out_dtype, cu_seqlens_q,
                                  cu_seqlens_kv, B, H_qo, H_kv, total_q, total_kv, max_seqlen_q, max_seqlen_kv, D,
                                  is_causal, sm_scale, pv, accum, SAGE_GRAN_BLOCK, stream);
}

sage_status sage_attn_fwd_varlen_g(const int8_t* q_i8, const float* q_scale, const int8_t* k_i8, const float* k_scale,
                                   const void* v_hat, const float* v_scale, void* out, sage_dtype out_dtype,
                                   const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_kv, int B, int H_qo,
                                   int H_kv, int total_q, int total_kv, int max_seqlen_q, int max_seqlen_kv, int D,
                                   int is_causal, float sm_scale, sage_pv pv, sage_accum accum, sage_qk_gran gran,
                                   void* stream) {
    if (gran != SAGE_GRAN_BLOCK && gran != SAGE_GRAN_THREAD)
        return fail(SAGE_ERR_INVALID_ARG, "bad quantisation granularity %d", int(gran));
    if (gran == SAGE_GRAN_THREAD && accum == SAGE_ACC_FP16_FP32_SPLIT)
        return fail(SAGE_ERR_UNSUPPORTED, "SAGE_ACC_FP16_FP32_SPLIT is offered with SAGE_GRAN_BLOCK only");
    sage_status s = check_attn_args(q_i8, q_scale, k_i8, k_scale, v_hat, v_scale, out, out_dtype, is_causal, sm_scale,
                                    pv, accum, D, "sage_attn_fwd_varlen");
    if (s != SAGE_OK) return s;
    s = check_varlen(cu_seqlens_q, cu_seqlens_kv, B, H_qo, H_kv, total_q, total_kv, max_seqlen_q, max_seqlen_kv, D);
    if (s != SAGE_OK) return s;
    s = check_device();
    if (s != SAGE_OK) return s;
    sage::AttnArgs a{};
    a.q_i8 = q_i8, a.q_scale = q_scale, a.k_i8 = k_i8, a.k_scale = k_scale, a.v_hat = v_hat, a.v_scale = v_scale;
    a.out = out;
    a.out_bf16 = out_dtype == SAGE_BF16;
    a.B = B, a.Hq = H_qo, a.Hkv = H_kv, a.Nq = max_seqlen_q, a.Nkv = max_seqlen_kv, a.D = D;
    a.causal = is_causal;
    a.sm_scale = sm_scale;
    a.fp8 = pv == SAGE_PV_FP8;
    a.split_partials = accum == SAGE_ACC_FP16_FP32_SPLIT;
    a.cu_q = cu_seqlens_q, a.cu_k = cu_seqlens_kv, a.total_q = total_q, a.total_k = total_kv;
    a.thread_gran = gran == SAGE_GRAN_THREAD;
    return launch_status(sage::launch_attn_fwd(a, (hipStream_t)stream), "sage_attn_fwd_varlen");
}


// ---- microscaling FP4 ---------------------------------------------------------------

size_t sage_quant_mxfp4_workspace_bytes(int B, int H_kv, int Nkv, int D) {
    if (B <= 0 || H_kv <= 0 || Nkv <= 0 || D <= 0 || D > 256) return 0;
    return size_t(B) * size_t(H_kv) * size_t(nblocks(Nkv)) * size_t(D) * sizeof(double);
}

sage_status sage_quant_mxfp4(const void* q, const void* k, const void* v, sage_dtype dtype, sage_layout layout, int B,
                             int H_qo, int H_kv, int Nq, int Nkv, int D, uint8_t* q4, uint8_t* q4_exp, uint8_t* k4,
                             uint8_t* k4_exp, float* k_mean, uint8_t* v4, uint8_t* v4_exp, void* workspace,
                             size_t workspace_bytes, void* stream) {
    if (!q || !k || !v || !q4 || !q4_exp || !k4 || !k4_exp || !k_mean || !v4 || !v4_exp)
        return fail(SAGE_ERR_INVALID_ARG, "sage_quant_mxfp4: null tensor pointer");
    if (dtype != SAGE_FP16 && dtype != SAGE_BF16) return fail(SAGE_ERR_INVALID_ARG, "bad dtype %d", int(dtype));
    if (layout != SAGE_HND && layout != SAGE_NHD) return fail(SAGE_ERR_INVALID_ARG, "bad layout %d", int(layout));
    if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(q4, 16) || !aligned(k4, 16) ||
        !aligned(v4, 16) || !aligned(k_mean, 4))
        return fail(SAGE_ERR_INVALID_ARG, "sage_quant_mxfp4: misaligned tensor");
    sage_status s = check_shape(B, H_qo, H_kv, Nq, Nkv, D);
    if (s != SAGE_OK) return s;
    const size_t need = sage_quant_mxfp4_workspace_bytes(B, H_kv, Nkv, D);
    if (!workspace || workspace_bytes < need || !aligned(workspace, 8))
        return fail(SAGE_ERR_WORKSPACE, "sage_quant_mxfp4: workspace of %zu bytes (8-byte aligned) required, got %zu",
                    need, workspace ? workspace_bytes : size_t(0));
    s = check_device();
    if (s != SAGE_OK) return s;
    sage::QuantMXArgs a{};
    a.q = q, a.k = k, a.v = v;
    a.bf16 = dtype == SAGE_BF16;
    a.layout_nhd = layout == SAGE_NHD;
    a.B = B, a.Hq = H_qo, a.Hkv = H_kv, a.Nq = Nq, a.Nkv = Nkv, a.D = D;
    a.q4 = q4, a.q4_exp = q4_exp, a.k4 = k4, a.k4_exp = k4_exp, a.k_mean = k_mean, a.v4 = v4, a.v4_exp = v4_exp;
    a.workspace = workspace;
    return launch_status(sage::launch_quant_mxfp4(a, (hipStream_t)stream), "sage_quant_mxfp4");
}

sage_status sage_quant_mxfp4_kv(const void* k, const void* v, sage_dtype dtype, sage_layout layout, int B, int H_kv,
                                int Nkv, int D, uint8_t* k4, uint8_t* k4_exp, float* k_mean, uint8_t* v4,
                                uint8_t* v4_exp, void* workspace, size_t workspace_bytes, void* stream) {
    if (!k || !v || !k4 || !k4_exp || !k_mean || !v4 || !v4_exp)
        return fail(SAGE_ERR_INVALID_ARG, "sage_quant_mxfp4_kv: null tensor pointer");
    if (dtype != SAGE_FP16 && dtype != SAGE_BF16) return fail(SAGE_ERR_INVALID_ARG, "bad dtype %d", int(dtype));
    if (layout != SAGE_HND && layout != SAGE_NHD) return fail(SAGE_ERR_INVALID_ARG, "bad layout %d", int(layout));
    if (!aligned(k, 16) || !aligned(v, 16) || !aligned(k4, 16) || !aligned(v4, 16) || !aligned(k_mean, 4))
        return fail(SAGE_ERR_INVALID_ARG, "sage_quant_mxfp4_kv: misaligned tensor");
    sage_status s = check_shape(B, H_kv, H_kv, Nkv, Nkv, D);
    if (s != SAGE_OK) return s;
    const size_t need = sage_quant_mxfp4_workspace_bytes(B, H_kv, Nkv, D);
    if (!workspace || workspace_bytes < need || !aligned(workspace, 8))
        return fail(SAGE_ERR_WORKSPACE, "sage_quant_mxfp4_kv: workspace of %zu bytes (8-byte aligned) required, got %zu",
                    need, workspace ? workspace_bytes : size_t(0));
    s = check_device();
    if (s != SAGE_OK) return s;
    sage::QuantMXArgs a{};
    a.q = nullptr;  // no Q: the K and V part of sage_quant_mxfp4
    a.k = k, a.v = v;
    a.bf16 = dtype == SAGE_BF16;
    a.layout_nhd = layout == SAGE_NHD;
    a.B = B, a.Hq = H_kv, a.Hkv = H_kv, a.Nq = Nkv, a.Nkv = Nkv, a.D = D;
    a.k4 = k4, a.k4_exp = k4_exp, a.k_mean = k_mean, a.v4 = v4, a.v4_exp = v4_exp;
    a.workspace = workspace;
    return launch_status(sage::launch_quant_mxfp4(a, (hipStream_t)stream), "sage_quant_mxfp4_kv");
}

sage_status sage_attn_fwd_mxfp4_fused_q(const void* q, sage_dtype dtype, sage_layout layout, const uint8_t* k4,
                                        const uint8_t* k4_exp, const uint8_t* v4, const uint8_t* v4_exp, void* out,
                                        int B, int H_qo, int H_kv, int Nq, int Nkv, int D, int is_causal,
                                        float sm_scale, uint8_t* q4_out, uint8_t* q4_exp_out, void* stream) {
    if (!q || !k4 || !k4_exp || !v4 || !v4_exp || !out)
        return fail(SAGE_ERR_INVALID_ARG, "sage_attn_fwd_mxfp4_fused_q: null tensor pointer");
    if (dtype != SAGE_FP16 && dtype != SAGE_BF16) return fail(SAGE_ERR_INVALID_ARG, "bad dtype %d", int(dtype));
    if (layout != SAGE_HND && layout != SAGE_NHD) return fail(SAGE_ERR_INVALID_ARG, "bad layout %d", int(layout));
    if (is_causal != 0 && is_causal != 1) return fail(SAGE_ERR_INVALID_ARG, "is_causal must be 0 or 1");
    if (!std::isfinite(sm_scale) || !(sm_scale > 0.0f))
        return fail(SAGE_ERR_INVALID_ARG, "sm_scale must be finite and > 0 (got %g)", double(sm_scale));
    if (!aligned(q, 16) || !aligned(k4, 16) || !aligned(v4, 16) || !aligned(out, (D % 4) == 0 ? 8 : 2) ||
        (q4_out && !aligned(q4_out, 16)))
        return fail(SAGE_ERR_INVALID_ARG, "sage_attn_fwd_mxfp4_fused_q: misaligned tensor");
    sage_status s = check_shape(B, H_qo, H_kv, Nq, Nkv, D);
    if (s != SAGE_OK) return s;
    const int64_t grid = int64_t((Nq + 127) / 128) * H_qo * B;
    if (grid > INT32_MAX) return fail(SAGE_ERR_UNSUPPORTED, "sage_attn_fwd_mxfp4_fused_q: grid too large");
    s = check_device();
    if (s != SAGE_OK) return s;
    sage::AttnMXArgs a{};
    a.k4 = k4, a.k4_exp = k4_exp, a.v4 = v4, a.v4_exp = v4_exp;
    a.out = out;
    a.out_bf16 = dtype == SAGE_BF16;
    a.out_nhd = layout == SAGE_NHD;
    a.B = B, a.Hq = H_qo, a.Hkv = H_kv, a.Nq = Nq, a.Nkv = Nkv, a.D = D;
    a.causal = is_causal;
    a.sm_scale = sm_scale;
    a.q16 = q;
    a.q_bf16 = dtype == SAGE_BF16;
    a.q_nhd = layout == SAGE_NHD;
    a.q4_out = q4_out;
    a.q4_exp_out = q4_exp_out;
    return launch_status(sage::launch_attn_mxfp4(a, (hipStream_t)stream), "sage_attn_fwd_mxfp4_fused_q");
}

size_t sage_quant_mxfp4_varlen_workspace_bytes(int B, int H_kv, int total_kv, int D) {
    if (B <= 0 || H_kv <= 0 || total_kv <= 0 || D <= 0 || D > 256) return 0;
    return size_t(H_kv) * size_t(varlen_slots(total_kv, B)) * size_t(D) * sizeof(double);
}

sage_status sage_quant_mxfp4_varlen(const void* q, const void* k, const void* v, sage_dtype dtype,
                                    const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_kv, int B, int H_qo,
                                    int H_kv, int total_q, int total_kv, int max_seqlen_q, int max_seqlen_kv, int D,
                                    uint8_t* q4, uint8_t* q4_exp, uint8_t* k4, uint8_t* k4_exp, float* k_mean,
                                    uint8_t* v4, uint8_t* v4_exp, void* workspace, size_t workspace_bytes,
                                    void* stream) {
    if (!q || !k || !v || !q4 || !q4_exp || !k4 || !k4_exp || !k_mean || !v4 || !v4_exp)
        return fail(SAGE_ERR_INVALID_ARG, "sage_quant_mxfp4_varlen: null tensor pointer");
    if (dtype != SAGE_FP16 && dtype != SAGE_BF16) return fail(SAGE_ERR_INVALID_ARG, "bad dtype %d", int(dtype));
    if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(q4, 16) || !aligned(k4, 16) ||
        !aligned(v4, 16) || !aligned(k_mean, 4))
        return fail(SAGE_ERR_INVALID_ARG, "sage_quant_mxfp4_varlen: misaligned tensor");
    sage_status s =
        check_varlen(cu_seqlens_q, cu_seqlens_kv, B, H_qo, H_kv, total_q, total_kv, max_seqlen_q, max_seqlen_kv, D);
    if (s != SAGE_OK) return s;
    const size_t need = sage_quant_mxfp4_varlen_workspace_bytes(B, H_kv, total_kv, D);
    if (!workspace || workspace_bytes < need || !aligned(workspace, 8))
        return fail(SAGE_ERR_WORKSPACE,
                    "sage_quant_mxfp4_varlen: workspace of %zu bytes (8-byte aligned) required, got %zu", need,
                    workspace ? workspace_bytes : size_t(0));
    s = check_device();
    if (s != SAGE_OK) return s;
    sage::QuantMXArgs a{};
    a.q = q, a.k = k, a.v = v;
    a.bf16 = dtype == SAGE_BF16;
    a.B = B, a.Hq = H_qo, a.Hkv = H_kv, a.Nq = max_seqlen_q, a.Nkv = max_seqlen_kv, a.D = D;
    a.cu_q = cu_seqlens_q, a.cu_k = cu_seqlens_kv, a.total_q = total_q, a.total_k = total_kv;
    a.q4 = q4, a.q4_exp = q4_exp, a.k4 = k4, a.k4_exp = k4_exp, a.k_mean = k_mean, a.v4 = v4, a.v4_exp = v4_exp;
    a.workspace = workspace;
    return launch_status(sage::launch_quant_mxfp4(a, (hipStream_t)stream), "sage_quant_mxfp4_varlen");
}

sage_status sage_attn_fwd_mxfp4_varlen(const uint8_t* q4, const uint8_t* q4_exp, const uint8_t* k4,
                                       const uint8_t* k4_exp, const uint8_t* v4, const uint8_t* v4_exp, void* out,
                                       sage_dtype out_dtype, const int32_t* cu_seqlens_q,
                                       const int32_t* cu_seqlens_kv, int B, int H_qo, int H_kv, int total_q,
                                       int total_kv, int max_seqlen_q, int max_seqlen_kv, int D, int is_causal,
                                       float sm_scale, void* stream) {
    if (!q4 || !q4_exp || !k4 || !k4_exp || !v4 || !v4_exp || !out)
        return fail(SAGE_ERR_INVALID_ARG, "sage_attn_fwd_mxfp4_varlen: null tensor pointer");
    if (out_dtype != SAGE_FP16 && out_dtype != SAGE_BF16)
        return fail(SAGE_ERR_INVALID_ARG, "bad out dtype %d", int(out_dtype));
    if (is_causal != 0 && is_causal != 1) return fail(SAGE_ERR_INVALID_ARG, "is_causal must be 0 or 1");
    if (!std::isfinite(sm_scale) || !(sm_scale > 0.0f))
        return fail(SAGE_ERR_INVALID_ARG, "sm_scale must be finite and > 0 (got %g)", double(sm_scale));
    if (!aligned(q4, 16) || !aligned(k4, 16) || !aligned(v4, 16) || !aligned(out, (D % 4) == 0 ? 8 : 2))
        return fail(SAGE_ERR_INVALID_ARG, "sage_attn_fwd_mxfp4_varlen: misaligned tensor");
    sage_status s =
        check_varlen(cu_seqlens_q, cu_seqlens_kv, B, H_qo, H_kv, total_q, total_kv, max_seqlen_q, max_seqlen_kv, D);
    if (s != SAGE_OK) return s;
    const int64_t grid = int64_t((max_seqlen_q + 127) / 128) * H_qo * B;
    if (grid > INT32_MAX) return fail(SAGE_ERR_UNSUPPORTED, "sage_attn_fwd_mxfp4_varlen: grid too large");
    s = check_device();
    if (s != SAGE_OK) return s;
    sage::AttnMXArgs a{};
    a.q4 = q4, a.q4_exp = q4_exp, a.k4 = k4, a.k4_exp = k4_exp, a.v4 = v4, a.v4_exp = v4_exp;
    a.out = out;
    a.out_bf16 = out_dtype == SAGE_BF16;
    a.B = B, a.Hq = H_qo, a.Hkv = H_kv, a.Nq = max_seqlen_q, a.Nkv = max_seqlen_kv, a.D = D;
    a.causal = is_causal;
    a.sm_scale = sm_scale;
    a.cu_q = cu_seqlens_q, a.cu_k = cu_seqlens_kv, a.total_q = total_q, a.total_k = total_kv;
    return launch_status(sage::launch_attn_mxfp4(a, (hipStream_t)stream), "sage_attn_fwd_mxfp4_varlen");
}

sage_status sage_attn_fwd_mxfp4(const uint8_t* q4, const uint8_t* q4_exp, const uint8_t* k4, const uint8_t* k4_exp,
                                const uint8_t* v4, const uint8_t* v4_exp, void* out, sage_dtype out_dtype,
                                sage_layout out_layout, int B, int H_qo, int H_kv, int Nq, int Nkv, int D,
                                int is_causal, float sm_scale, void* stream) {
    if (!q4 || !q4_exp || !k4 || !k4_exp || !v4 || !v4_exp || !out)
        return fail(SAGE_ERR_INVALID_ARG, "sage_attn_fwd_mxfp4: null tensor pointer");
    if (out_dtype != SAGE_FP16 && out_dtype != SAGE_BF16)
        return fail(SAGE_ERR_INVALID_ARG, "bad out dtype %d", int(out_dtype));
    if (out_layout != SAGE_HND && out_layout != SAGE_NHD)
        return fail(SAGE_ERR_INVALID_ARG, "bad layout %d", int(out_layout));
    if (is_causal != 0 && is_causal != 1) return fail(SAGE_ERR_INVALID_ARG, "is_causal must be 0 or 1");
    if (!std::isfinite(sm_scale) || !(sm_scale > 0.0f))
        return fail(SAGE_ERR_INVALID_ARG, "sm_scale must be finite and > 0 (got %g)", double(sm_scale));
    if (!aligned(q4, 16) || !aligned(k4, 16) || !aligned(v4, 16) || !aligned(out, (D % 4) == 0 ? 8 : 2))
        return fail(SAGE_ERR_INVALID_ARG, "sage_attn_fwd_mxfp4: misaligned tensor");
    sage_status s = check_shape(B, H_qo, H_kv, Nq, Nkv, D);
    if (s != SAGE_OK) return s;
    const int64_t grid = int64_t((Nq + 127) / 128) * H_qo * B;
    if (grid > INT32_MAX) return fail(SAGE_ERR_UNSUPPORTED, "sage_attn_fwd_mxfp4: grid too large");
    s = check_device();
    if (s != SAGE_OK) return s;
    sage::AttnMXArgs a{};
    a.q4 = q4, a.q4_exp = q4_exp, a.k4 = k4, a.k4_exp = k4_exp, a.v4 = v4, a.v4_exp = v4_exp;
    a.out = out;
    a.out_bf16 = out_dtype == SAGE_BF16;
    a.out_nhd = out_layout == SAGE_NHD;
    a.B = B, a.Hq = H_qo, a.Hkv = H_kv, a.Nq = Nq, a.Nkv = Nkv, a.D = D;
    a.causal = is_causal;
    a.sm_scale = sm_scale;
    return launch_status(sage::launch_attn_mxfp4(a, (hipStream_t)stream), "sage_attn_fwd_mxfp4");
}

}  // extern "C"
