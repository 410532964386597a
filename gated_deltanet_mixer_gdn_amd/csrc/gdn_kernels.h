// gdn_kernels.h - internal interface between the C-ABI layer (gdn_api.cpp) and the
// gfx950 kernels (gdn_conv.hip, gdn_recurrence.hip, gdn_norm.hip).  Not installed,
// not part of the ABI.
#pragma once

#include <hip/hip_runtime_api.h>
#include <stdint.h>

#include "gdn.h"

namespace gdn {

// Head size and conv width the kernels are built for.
constexpr int kS = 128;
constexpr int kDConv = 4;
constexpr int kHist = kDConv - 1;
// The conv kernel: 128-channel heads per 256-thread workgroup (one per half-wave), and
// the consecutive tokens of one sequence a workgroup takes (kConvGroup for calls of
// 8 tokens or more, 4 for 2 to 7, 1 for single-token calls).  h is written with
// streaming stores from kConvStreamBytes of output up (a stream that large will not
// stay in the caches for the next kernel anyway).
constexpr int kConvHeadsPerBlock = 8;
constexpr int kConvGroup = 8;
constexpr long long kConvStreamBytes = 64LL << 20;
// Rows (value heads x tokens) per gated-RMSNorm workgroup: one half-wave per row.
constexpr int kNormRowsPerBlock = 8;

struct ConvParams {
    float* conv;            // pool conv region [n_slots][C][3]
    const int32_t* slots;   // [B] or null
    const int32_t* n_tok;   // [B] or null
    const float* qkv;       // [B][T][C]
    const float* w;         // [C][4]
    float* h;               // [B][T][C]
    uint32_t* flags;        // pool flag word
    long long n_slots;
    int B, T, h_k, n_heads; // n_heads = 2*h_k + h_v (128-channel heads)
    int n_groups;           // token groups per sequence, ceil(T / group)
    int group;              // tokens per group: 1, 4 or kConvGroup
    int persist;            // 0: leave the stored history untouched (speculative window)
    int stream_h;           // 1: h written with streaming (non-temporal) stores
    float eps, qscale;
    // a commit first (else null): the stored history advances by the first n_adv[b] raw
    // rows of adv_qkv [B][adv_T][C] and is stored, and this call's tokens start from it
    const float* adv_qkv;
    const int32_t* n_adv;
    int adv_T;
};

struct StepParams {
    float* state;           // pool state region [n_slots][h_v][128][128]
    const int32_t* slots;
    const int32_t* n_tok;
    const float* h;         // [B][T][C]
    const float* alpha;     // [B][T][h_v]
    const float* beta_logit;
    const float* dt;        // [h_v]
    const float* ssm_a;     // [h_v]
    float* o;               // [B][T][h_v][128], or null: not written
    const float* z;         // fused gated RMSNorm epilogue: [B][T][h_v*128], or null
    const float* norm_w;    // [128]
    float* y;               // [B][T][h_v*128], or null: no epilogue
    // commit only (else null): the pool's conv region and the raw qkv rows [B][T][C]
    // whose first n_tok[b] rows advance the conv history of each sequence
    float* conv;
    const float* adv_qkv;
    uint32_t* flags;
    long long n_slots;
    int B, T, h_k, h_v, group;  // group = h_v / h_k
    int persist;            // 0: leave the state untouched (speculative window)
    int gate_silu;          // epilogue gate: 0 sigmoid(z), 1 z * sigmoid(z)
    float eps;              // RMSNorm epsilon (epilogue only)
    float oscale;           // multiplies the readout o (1, or 1/sqrt(S) when q is unscaled)
};

// Largest GQA group (h_v / h_k) the single-launch decode supports: the conv prologue
// gives one 16-lane row to each of q_j, k_j and the group's value heads.
constexpr int kFusedMaxGroup = 14;

struct FusedParams {
    float* state;           // pool state region
    float* conv;            // pool conv region
    const int32_t* slots;   // [B] or null
    const float* qkv;       // [B][C] raw projections of one token
    const float* w;         // [C][4]
    const float* alpha;     // [B][h_v]
    const float* beta_logit;
    const float* dt;        // [h_v]
    const float* ssm_a;     // [h_v]
    const float* z;         // [B][h_v*128]
    const float* norm_w;    // [128]
    float* y;               // [B][h_v*128] or null (then ys is set)
    float* h;               // [B][C] or null: the conv/SiLU/L2 output, if wanted
    uint16_t* ys;           // y split into bf16 hi / lo in the projections' tiled layout, or null
    int ys_chunks;          // 64-column chunks per row of ys (h_v * 128 / 64)
    uint32_t* flags;
    long long n_slots;
    int B, h_k, h_v, group;
    int gate_silu;
    float eps, qscale, oscale;
};

struct NormParams {
    const float* o;
    const float* z;
    const float* w;
    float* y;
    long long rows;
    float eps;
    int gate_silu;
};

struct ZeroParams {
    float* state;
    float* conv;
    uint32_t* flags;
    const int32_t* slots;   // null: zero everything and clear the flag word
    long long n_slots;
    long long state_f4;     // float4s of state per slot
    long long conv_f4;      // float4s of conv history per slot
    int n;                  // slots listed
};

hipError_t launch_conv_silu_norm(const ConvParams& p, hipStream_t stream);
hipError_t launch_decode_step(const StepParams& p, hipStream_t stream);
hipError_t launch_commit_window(const StepParams& com, const StepParams& win, hipStream_t stream);
hipError_t launch_decode_fused(const FusedParams& p, hipStream_t stream);
hipError_t launch_gated_rmsnorm(const NormParams& p, hipStream_t stream);
hipError_t launch_zero(const ZeroParams& p, hipStream_t stream);

}  // namespace gdn
