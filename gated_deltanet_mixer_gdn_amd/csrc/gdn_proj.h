// gdn_proj.h - internal interface of the alpha / beta projection kernel
// (gdn_proj.hip) for the C-ABI layer.  Not installed, not part of the ABI.
#pragma once

#include <hip/hip_runtime_api.h>
#include <stdint.h>

namespace gdn {

// one workgroup per (kAbRows rows, kAbCols output columns)
constexpr int kAbRows = 4;
constexpr int kAbCols = 8;
// 256-element blocks of n_embd a wave loads at once (a wave takes every 4th block)
constexpr int kAbBlocks = 3;

struct AbParams {
    const float* x;          // [rows][n_embd]
    const uint16_t* w_alpha; // [h_v][n_embd] bf16 bits
    const uint16_t* w_beta;  // [h_v][n_embd] bf16 bits
    float* alpha;            // [rows][h_v]
    float* beta_logit;       // [rows][h_v]
    long long rows;
    int n_embd, h_v;
};

hipError_t launch_ab_project(const AbParams& p, hipStream_t stream);

}  // namespace gdn
