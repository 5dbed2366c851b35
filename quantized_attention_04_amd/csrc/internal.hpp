// internal.hpp -- argument blocks and launchers shared by the host API and the kernels.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace sage {

// Batches are dense (cu_* null: B sequences of Nq / Nkv tokens) or packed (cu_* =
// device prefix sums, Nq / Nkv bound every sequence, total_* tokens in all).
struct QuantQKArgs {
    const void* q;
    const void* k;
    int bf16, layout_nhd;
    int B, Hq, Hkv, Nq, Nkv, D;
    const int32_t* cu_q;
    const int32_t* cu_k;
    int total_q, total_k;
    int8_t* q_i8;
    float* q_scale;
    int8_t* k_i8;
    float* k_scale;
    float* k_mean;
    void* workspace;
    int thread_gran;  // 1: one Q scale per token and one K scale per 32 keys (else per 64)
};

struct QuantVArgs {
    const void* v;
    int bf16, layout_nhd;
    int B, Hkv, Nkv, D;
    const int32_t* cu_k;
    int total_k;
    int fp8;
    void* v_hat;
    float* v_scale;
    void* workspace;
};

struct AttnArgs {
    const int8_t* q_i8;
    const float* q_scale;
    const int8_t* k_i8;
    const float* k_scale;
    const void* v_hat;
    const float* v_scale;
    void* out;
    int out_bf16, out_nhd;
    int B, Hq, Hkv, Nq, Nkv, D;
    int causal;
    float sm_scale;
    int fp8;
    int split_partials;  // the explicit two-level P.V form (fresh fp32 partial per tile + vector add)
    const int32_t* cu_q;
    const int32_t* cu_k;
    int total_q, total_k;
    int thread_gran;  // scales of sage_quant_qkv's per-thread granularity
    int splits;       // > 1: key-range splits (FP16 P.V, block granularity) into workspace
    void* workspace;  // splits > 1: part_o fp16 [B*Hq][Nq][splits][Dp], then part_ml fp32 [..][2]
    // non-null: Q in fp16 / bf16 (q_bf16), layout q_nhd, dense, quantised in the attention
    // prologue (q_i8 / q_scale unused); the codes and scales also go to q_i8_out /
    // q_scale_out where those are non-null
    const void* q16;
    int q_bf16, q_nhd;
    int8_t* q_i8_out;
    float* q_scale_out;
};

// Workspace of the key-range split attention: fp16 per-split outputs [rows][Dp] at byte
// 0, then fp32 (running max, row sum) pairs [rows][2] at byte ml; rows = B*Hq*Nq*splits.
struct SplitWorkspace {
    size_t ml, bytes;
};
inline SplitWorkspace attn_split_workspace(int B, int Hq, int Nq, int D, int splits) {
    const size_t dp = D <= 64 ? 64 : (D <= 128 ? 128 : 256);
    const size_t rows = size_t(B) * size_t(Hq) * size_t(Nq) * size_t(splits);
    return SplitWorkspace{rows * dp * 2, rows * (dp * 2 + 2 * sizeof(float))};
}

// Microscaling FP4: codes and E8M0 exponent bytes of Q, smoothed K and V in the layouts
// of include/sage.h; workspace = the fp64 K block channel sums.  Dense or packed batches
// as for the INT8 path (cu_* null: dense).
struct QuantMXArgs {
    const void* q;
    const void* k;
    const void* v;
    int bf16, layout_nhd;
    int B, Hq, Hkv, Nq, Nkv, D;
    const int32_t* cu_q;
    const int32_t* cu_k;
    int total_q, total_k;
    uint8_t* q4;
    uint8_t* q4_exp;
    uint8_t* k4;
    uint8_t* k4_exp;
    float* k_mean;
    uint8_t* v4;
    uint8_t* v4_exp;
    void* workspace;
};

struct AttnMXArgs {
    const uint8_t* q4;
    const uint8_t* q4_exp;
    const uint8_t* k4;
    const uint8_t* k4_exp;
    const uint8_t* v4;
    const uint8_t* v4_exp;
    void* out;
    int out_bf16, out_nhd;
    int B, Hq, Hkv, Nq, Nkv, D;
    int causal;
    float sm_scale;
    const int32_t* cu_q;
    const int32_t* cu_k;
    int total_q, total_k;
    // non-null: Q in fp16 / bf16 (q_bf16), layout q_nhd, dense, quantised in the attention
    // prologue (q4 / q4_exp unused); codes and exponents also to q4_out / q4_exp_out if set
    const void* q16;
    int q_bf16, q_nhd;
    uint8_t* q4_out;
    uint8_t* q4_exp_out;
};

struct DebugQKArgs {
    const int8_t* q_i8;
    const int8_t* k_i8;
    int B, Hq, Hkv, Nq, Nkv, D;
    int fp8;
    const int32_t* tiles;
    int T;
    int32_t* out;
};

// Workspace of the fused Q/K/V quantisation (byte offsets; total = bytes):
// fp64 K block channel sums [slots][D], then (FP8) fp32 V block channel maxima
// [slots][Dp] and the V channel maxima as float bits [B * H_kv][Dp].  slots = block
// slots of K: B * H_kv * ceil(Nkv / 64) dense, H_kv * ceil((total + 64 B) / 64) packed.
struct QKVWorkspace {
    size_t kpart, vpart, amax, bytes;
};
inline QKVWorkspace qkv_workspace(int B, int Hkv, int Nkv, int D, bool packed, int total_kv, bool fp8) {
    const size_t dp = D <= 64 ? 64 : (D <= 128 ? 128 : 256);
    const size_t slots = packed ? size_t(Hkv) * size_t((int64_t(total_kv) + 64 * int64_t(B) + 63) / 64)
                                : size_t(B) * size_t(Hkv) * size_t((Nkv + 63) / 64);
    QKVWorkspace w;
    w.kpart = 0;
    w.vpart = slots * size_t(D) * sizeof(double);
    w.amax = w.vpart + (fp8 ? slots * dp * sizeof(float) : 0);
    w.bytes = w.amax + (fp8 ? size_t(B) * size_t(Hkv) * dp * sizeof(uint32_t) : 0);
    return w;
}

// Static workspace of sage_quant_qkv_noalloc (quant.hip): its size, and its device
// address on the current device (looked up once per device).
constexpr size_t kNoAllocScratchBytes = size_t(32) << 20;
hipError_t noalloc_scratch(void** ptr);

hipError_t launch_quant_qk(const QuantQKArgs& a, hipStream_t s);
hipError_t launch_quant_qkv(const QuantQKArgs& a, const QuantVArgs& v, hipStream_t s);
hipError_t launch_quant_v(const QuantVArgs& a, hipStream_t s);
hipError_t launch_attn_fwd(const AttnArgs& a, hipStream_t s);
hipError_t launch_debug_qk(const DebugQKArgs& a, hipStream_t s);
hipError_t launch_quant_mxfp4(const QuantMXArgs& a, hipStream_t s);
hipError_t launch_attn_mxfp4(const AttnMXArgs& a, hipStream_t s);

}  // namespace sage
