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

// One workgroup per (block of kAbRows rows, group of kAbCols of the 2*h_v output
// columns; columns 0..h_v-1 are alpha, h_v..2h_v-1 beta).  The 4 waves split n_embd
// in 256-element blocks (wave w takes blocks w, w + 4, ...); in a block, lane l takes
// elements 4l..4l+3 and keeps kAbRows x kAbCols partial dot products; the blocks
// are taken kAbBlocks at a time with their loads issued together.  Each wave sums
// its lanes, and wave 0 adds the 4 waves' sums as (w0 + w1) + (w2 + w3).  Rows and
// columns past the end are clamped to the last one (and not stored), the tail of
// n_embd is zeroed by a select, so every load is unconditional.
__global__ __launch_bounds__(256) void ab_project_kernel(AbParams p) {
    __shared__ float part[4][kAbRows * kAbCols];
    const int wave = threadIdx.x >> 6;
    const int lane = threadIdx.x & 63;
    const int n_out = 2 * p.h_v;
    const int n_groups = (n_out + kAbCols - 1) / kAbCols;
    const long long job = blockIdx.x;
    const long long rb = job / n_groups;
    const int grp = (int) (job - rb * n_groups);
    const long long r0 = rb * kAbRows;
    const int K = p.n_embd;

    const float* xr[kAbRows];
#pragma unroll
    for (int r = 0; r < kAbRows; ++r) xr[r] = p.x + min(r0 + r, p.rows - 1) * K;
    const uint16_t* wr[kAbCols];
#pragma unroll
    for (int c = 0; c < kAbCols; ++c) {
        const int n = min(grp * kAbCols + c, n_out - 1);
        wr[c] = n < p.h_v ? p.w_alpha + (long long) n * K : p.w_beta + (long long) (n - p.h_v) * K;
    }
    float acc[kAbRows][kAbCols];
#pragma unroll
    for (int r = 0; r < kAbRows; ++r)
#pragma unroll
        for (int c = 0; c < kAbCols; ++c) acc[r][c] = 0.f;

    // kAbBlocks of this wave's blocks per trip, all loads issued before the arithmetic
    // (one memory round trip per trip; n_embd = 2560 is one trip)
    for (int t0 = 256 * wave; t0 < K; t0 += 1024 * kAbBlocks) {
        f4 x[kAbBlocks][kAbRows];
        uint2 wb[kAbBlocks][kAbCols];
        bool in[kAbBlocks];
#pragma unroll
        for (int u = 0; u < kAbBlocks; ++u) {
            const int e = t0 + 1024 * u + 4 * lane;
            in[u] = e < K;
            const int ec = in[u] ? e : K - 4;
#pragma unroll
            for (int r = 0; r < kAbRows; ++r) x[u][r] = *(const f4*) (xr[r] + ec);
#pragma unroll
            for (int c = 0; c < kAbCols; ++c) wb[u][c] = *(const uint2*) (wr[c] + ec);
        }
#pragma unroll
        for (int u = 0; u < kAbBlocks; ++u)
#pragma unroll
            for (int c = 0; c < kAbCols; ++c) {
                const f4 w = {bf16_lo(wb[u][c].x), bf16_hi(wb[u][c].x), bf16_lo(wb[u][c].y), bf16_hi(wb[u][c].y)};
#pragma unroll
                for (int r = 0; r < kAbRows; ++r) {
                    const f4 xv = in[u] ? x[u][r] : f4{0.f, 0.f, 0.f, 0.f};
                    float a = acc[r][c];
                    a = __builtin_fmaf(w.x, xv.x, a);
                    a = __builtin_fmaf(w.y, xv.y, a);
                    a = __builtin_fmaf(w.z, xv.z, a);
                    a = __builtin_fmaf(w.w, xv.w, a);
                    acc[r][c] = a;
                }
            }
    }
#pragma unroll
    for (int r = 0; r < kAbRows; ++r)
#pragma unroll
        for (int c = 0; c < kAbCols; ++c) {
            const float v = wave_sum(acc[r][c]);
            if (lane == r * kAbCols + c) part[wave][lane] = v;
        }
    __syncthreads();
    if (wave == 0 && lane < kAbRows * kAbCols) {
        const int r = lane / kAbCols, c = lane % kAbCols;
        const int n = grp * kAbCols + c;
        const float v = (part[0][lane] + part[1][lane]) + (part[2][lane] + part[3][lane]);
        if (r0 + r < p.rows && n < n_out) {
            if (n < p.h_v) p.alpha[(r0 + r) * p.h_v + n] = v;
            else p.beta_logit[(r0 + r) * p.h_v + (n - p.h_v)] = v;
        }
    }
}

// ------------------------------------------------------------------ launch
hipError_t launch_ab_project(const AbParams& p, hipStream_t stream) {
    const long long n_groups = (2 * p.h_v + kAbCols - 1) / kAbCols;
    const long long jobs = (p.rows + kAbRows - 1) / kAbRows * n_groups;
    hipLaunchKernelGGL(ab_project_kernel, dim3((unsigned) jobs), dim3(256), 0, stream, p);
    return hipGetLastError();
}

}  // namespace gdn
