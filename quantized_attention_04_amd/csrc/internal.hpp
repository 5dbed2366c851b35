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
    int fp8, two_level;
    const int32_t* cu_q;
    const int32_t* cu_k;
    int total_q, total_k;
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

hipError_t launch_quant_qk(const QuantQKArgs& a, hipStream_t s);
hipError_t launch_quant_v(const QuantVArgs& a, hipStream_t s);
hipError_t launch_attn_fwd(const AttnArgs& a, hipStream_t s);
hipError_t launch_debug_qk(const DebugQKArgs& a, hipStream_t s);

}  // namespace sage
