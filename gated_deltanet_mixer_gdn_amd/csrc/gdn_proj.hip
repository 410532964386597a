// gdn_proj.hip - the alpha / beta projections that feed the recurrence: for every
// row r of x (one token of one sequence),
//   alpha[r][i] = sum_e w_alpha[i][e] x[r][e],  beta_logit[r][i] = sum_e w_beta[i][e] x[r][e]
// with bf16 weights and fp32 activations, as the native path of step 5 of
// `gdn_layer` on the "src/core/layer.cpp" page uses (the sigmoid / softplus epilogue
// runs in the recurrence kernels' prologue).  At decode sizes this is a
// bandwidth- and latency-bound GEMV-like pass (96 x 2560 bf16 weights), not a dense
// contraction worth MFMA: activations stay fp32 and products are exact in fp32.
#include "gdn_device.h"
#include "gdn_proj.h"

namespace gdn {

__device__ __forceinline__ float bf16_lo(unsigned u) { return __uint_as_float(u << 16); }
__device__ __forceinline__ float bf16_hi(unsigned u) { return __uint_as_float(u & 0xFFFF0000u); }

__device__ __forceinline__ float wave_sum(float v) { return add_xor32(add_xor16(add_xor8(block8_sum(v)))); }

// One wave per (block of kAbRows rows, group of kAbCols of the 2*h_v output
// columns; columns 0..h_v-1 are alpha, h_v..2h_v-1 beta).  Lane l takes the
// elements 4l + 256m of n_embd, keeps kAbRows x kAbCols partial dot products, and
// the wave sums them; lane r*kAbCols + c writes output (r, c).
__global__ __launch_bounds__(256) void ab_project_kernel(AbParams p) {
    const int wave = threadIdx.x >> 6;
    const int lane = threadIdx.x & 63;
    const int n_out = 2 * p.h_v;
    const int n_groups = (n_out + kAbCols - 1) / kAbCols;
    const long long job = (long long) blockIdx.x * 4 + wave;
    const long long rb = job / n_groups;
    const int grp = (int) (job - rb * n_groups);
    const long long r0 = rb * kAbRows;
    if (r0 >= p.rows) return;   // the whole wave leaves together
    const int K = p.n_embd;

    const uint16_t* wr[kAbCols];
#pragma unroll
    for (int c = 0; c < kAbCols; ++c) {
        const int n = grp * kAbCols + c;
        wr[c] = n < p.h_v ? p.w_alpha + (long long) n * K
                          : (n < n_out ? p.w_beta + (long long) (n - p.h_v) * K : nullptr);
    }
    float acc[kAbRows][kAbCols];
#pragma unroll
    for (int r = 0; r < kAbRows; ++r)
#pragma unroll
        for (int c = 0; c < kAbCols; ++c) acc[r][c] = 0.f;

    for (int e = lane * 4; e < K; e += 256) {
        f4 x[kAbRows];
#pragma unroll
        for (int r = 0; r < kAbRows; ++r)
            x[r] = r0 + r < p.rows ? *(const f4*) (p.x + (r0 + r) * K + e) : f4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int c = 0; c < kAbCols; ++c) {
            if (!wr[c]) continue;
            const uint2 wb = *(const uint2*) (wr[c] + e);
            const f4 w = {bf16_lo(wb.x), bf16_hi(wb.x), bf16_lo(wb.y), bf16_hi(wb.y)};
#pragma unroll
            for (int r = 0; r < kAbRows; ++r) {
                float a = acc[r][c];
                a = __builtin_fmaf(w.x, x[r].x, a);
                a = __builtin_fmaf(w.y, x[r].y, a);
                a = __builtin_fmaf(w.z, x[r].z, a);
                a = __builtin_fmaf(w.w, x[r].w, a);
                acc[r][c] = a;
            }
        }
    }
#pragma unroll
    for (int r = 0; r < kAbRows; ++r)
#pragma unroll
        for (int c = 0; c < kAbCols; ++c) {
            const float v = wave_sum(acc[r][c]);
            const int n = grp * kAbCols + c;
            if (lane == r * kAbCols + c && r0 + r < p.rows && n < n_out) {
                if (n < p.h_v) p.alpha[(r0 + r) * p.h_v + n] = v;
                else p.beta_logit[(r0 + r) * p.h_v + (n - p.h_v)] = v;
            }
        }
}

// ------------------------------------------------------------------ launch
hipError_t launch_ab_project(const AbParams& p, hipStream_t stream) {
    const long long n_groups = (2 * p.h_v + kAbCols - 1) / kAbCols;
    const long long jobs = (p.rows + kAbRows - 1) / kAbRows * n_groups;
    hipLaunchKernelGGL(ab_project_kernel, dim3((unsigned) ((jobs + 3) / 4)), dim3(256), 0, stream, p);
    return hipGetLastError();
}

}  // namespace gdn
