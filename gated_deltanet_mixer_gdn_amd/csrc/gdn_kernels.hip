// gdn_kernels.hip - gfx950 kernels of the Gated DeltaNet decode mixer.
//
// Three kernels make one pass of the mixer (the order of the GDN layer's docstring
// on the "include/strata/core/layer.hpp" page, steps 3-7 of `gdn_layer` on the
// "src/core/layer.cpp" page), plus a fill kernel for the state pool:
//
//   conv_silu_norm_kernel  causal depthwise conv + conv-history roll + SiLU on all
//                          C channels + L2 norm of q/k heads + 1/sqrt(S) on q.
//                          One half-wave (32 lanes x 4 channels) per 128-channel
//                          head, so each norm is a half-wave shuffle reduction.
//   decode_step_kernel     beta/gate prologue and the gated delta rule.  One
//                          256-thread workgroup per (sequence, value head); the
//                          64 KiB fp32 state tile is read once with 16-byte
//                          loads into VGPRs (64 floats per thread), kept there
//                          across the call's tokens, and written back once.
//   gated_rmsnorm_kernel   y = rms_norm(o) * w * sigmoid(z), one half-wave per row.
//
// Everything here is bound by HBM traffic except the multi-token recurrence, which
// is bound by the VALU: there is no dense contraction on this path (rank-1 updates
// and matrix-vector products), so no MFMA.
#include <hip/hip_runtime.h>

#include "gdn_kernels.h"

namespace gdn {

typedef float f4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ float sigmoid_f(float x) { return 1.0f / (1.0f + expf(-x)); }

// softplus in fp32: above 20 the log1p term is below half an ulp of x
__device__ __forceinline__ float softplus_f(float x) { return x > 20.0f ? x : log1pf(expf(x)); }

__device__ __forceinline__ f4 sigmoid4(f4 x) {
    return f4{sigmoid_f(x.x), sigmoid_f(x.y), sigmoid_f(x.z), sigmoid_f(x.w)};
}

// Sum over the 32 lanes of a half-wave (lanes 0-31 or 32-63); every lane gets the sum.
__device__ __forceinline__ float halfwave_sum(float v) {
    v += __shfl_xor(v, 16);
    v += __shfl_xor(v, 8);
    v += __shfl_xor(v, 4);
    v += __shfl_xor(v, 2);
    v += __shfl_xor(v, 1);
    return v;
}

__device__ __forceinline__ int read_slot(const int32_t* slots, int b, long long n_slots,
                                         uint32_t* flags, bool report) {
    const int slot = slots ? slots[b] : b;
    if (slot < 0 || (long long) slot >= n_slots) {
        if (report) atomicOr(flags, GDN_FLAG_BAD_SLOT);
        return -1;
    }
    return slot;
}

__device__ __forceinline__ int read_ntok(const int32_t* n_tok, int b, int T, uint32_t* flags,
                                         bool report) {
    if (!n_tok) return T;
    int n = n_tok[b];
    if (n < 0 || n > T) {
        if (report) atomicOr(flags, GDN_FLAG_BAD_NTOK);
        n = n < 0 ? 0 : T;
    }
    return n;
}

// ------------------------------------------------------------------ conv + SiLU + L2
//
// grid.x = B * n_tb (sequence, token block), grid.y = ceil(n_heads / 8); 256 threads.
// Thread (half-wave hw = tid/32, lane l = tid%32) owns channels c0..c0+3 of head
// grid.y*8 + hw, c0 = head*128 + 4l, for the tokens [t0, t0+8) of its block.
// Conv history per channel is held in registers as three float4 over the 4
// channels: x3 (oldest) .. x1 (newest).  Only token block 0 reads or writes the
// stored history; later blocks take their first three history entries from qkv.
__global__ __launch_bounds__(256) void conv_silu_norm_kernel(ConvParams p) {
    const int tid = threadIdx.x;
    const int head = blockIdx.y * 8 + (tid >> 5);
    if (head >= p.n_heads) return;  // whole half-wave leaves together
    const int l = tid & 31;
    const int b = blockIdx.x / p.n_tb;
    const int tb = blockIdx.x - b * p.n_tb;
    const long long C = (long long) p.n_heads * kS;
    const long long c0 = (long long) head * kS + 4 * l;
    const int t0 = tb * kConvTokensPerBlock;
    const int t1 = min(t0 + kConvTokensPerBlock, p.T);
    const long long row0 = (long long) b * p.T;
    const bool reporter = (tid == 0 && blockIdx.y == 0 && tb == 0);

    const int slot = read_slot(p.slots, b, p.n_slots, p.flags, reporter);
    int nt = read_ntok(p.n_tok, b, p.T, p.flags, reporter);
    if (slot < 0) nt = 0;  // unknown slot: no history to read or advance, outputs zero

    const f4 w0 = *(const f4*) (p.w + (c0 + 0) * kDConv);
    const f4 w1 = *(const f4*) (p.w + (c0 + 1) * kDConv);
    const f4 w2 = *(const f4*) (p.w + (c0 + 2) * kDConv);
    const f4 w3 = *(const f4*) (p.w + (c0 + 3) * kDConv);

    f4 x3 = {0.f, 0.f, 0.f, 0.f}, x2 = x3, x1 = x3;  // history, oldest first
    float* X = nullptr;
    if (nt > t0) {
        if (t0 == 0) {
            // [c][j] layout: 12 consecutive floats for channels c0..c0+3
            X = p.conv + ((long long) slot * C + c0) * kHist;
            const f4 a = *(const f4*) (X + 0);
            const f4 m = *(const f4*) (X + 4);
            const f4 z = *(const f4*) (X + 8);
            x3 = f4{a.x, a.w, m.z, z.y};
            x2 = f4{a.y, m.x, m.w, z.z};
            x1 = f4{a.z, m.y, z.x, z.w};
        } else {
            x3 = *(const f4*) (p.qkv + (row0 + t0 - 3) * C + c0);
            x2 = *(const f4*) (p.qkv + (row0 + t0 - 2) * C + c0);
            x1 = *(const f4*) (p.qkv + (row0 + t0 - 1) * C + c0);
        }
    }

    const bool normed = head < 2 * p.h_k;
    const float extra = head < p.h_k ? p.qscale : 1.0f;
    const int t_end = min(t1, nt);
    for (int t = t0; t < t_end; ++t) {
        const f4 x = *(const f4*) (p.qkv + (row0 + t) * C + c0);
        f4 u;
        u.x = w0.x * x3.x + w0.y * x2.x + w0.z * x1.x + w0.w * x.x;
        u.y = w1.x * x3.y + w1.y * x2.y + w1.z * x1.y + w1.w * x.y;
        u.z = w2.x * x3.z + w2.y * x2.z + w2.z * x1.z + w2.w * x.z;
        u.w = w3.x * x3.w + w3.y * x2.w + w3.z * x1.w + w3.w * x.w;
        x3 = x2;
        x2 = x1;
        x1 = x;
        f4 hv = u * sigmoid4(u);
        if (normed) {
            const float ss = halfwave_sum(hv.x * hv.x + hv.y * hv.y + hv.z * hv.z + hv.w * hv.w);
            hv *= extra / sqrtf(ss + p.eps);
        }
        *(f4*) (p.h + (row0 + t) * C + c0) = hv;
    }
    const f4 zero = {0.f, 0.f, 0.f, 0.f};
    for (int t = max(t0, nt); t < t1; ++t) *(f4*) (p.h + (row0 + t) * C + c0) = zero;

    if (t0 == 0 && nt > 0) {
        // the new history is the last three entries of (stored history, tokens 0..nt-1)
        f4 n3, n2, n1;
        if (nt <= t1) {
            n3 = x3;
            n2 = x2;
            n1 = x1;
        } else {  // nt > 8 > 3: all three come from qkv
            n3 = *(const f4*) (p.qkv + (row0 + nt - 3) * C + c0);
            n2 = *(const f4*) (p.qkv + (row0 + nt - 2) * C + c0);
            n1 = *(const f4*) (p.qkv + (row0 + nt - 1) * C + c0);
        }
        *(f4*) (X + 0) = f4{n3.x, n2.x, n1.x, n3.y};
        *(f4*) (X + 4) = f4{n2.y, n1.y, n3.z, n2.z};
        *(f4*) (X + 8) = f4{n1.z, n3.w, n2.w, n1.w};
    }
}

// ------------------------------------------------------------------ gated delta rule
//
// One workgroup of 256 threads per (sequence b, value head i); qk head j = i / group.
// Thread tid owns columns 4*cg..4*cg+3 (cg = tid % 32) of rows 16*rg..16*rg+15
// (rg = tid / 32) of the 128 x 128 state: 16 float4 = 64 VGPRs.  A wave's loads
// cover two 512-byte row segments per instruction.
//
// Per token both column reductions come from ONE pass over the old state:
//   PK[c] = sum_r S[r][c] k[r],  PQ[c] = sum_r S[r][c] q[r],  KQ = k . q
//   d = beta (v - e^g PK);  o = e^g PQ + KQ d;  S <- e^g S + k d^T
// which equals decay -> read -> write -> read of the recurrence in exact
// arithmetic (o = S_new^T q expanded).  Reductions: per-thread partial over 16
// rows, a cross-half-wave shuffle, then 4 waves through LDS: one barrier.
__global__ __launch_bounds__(256) void decode_step_kernel(StepParams p) {
    __shared__ f4 qk_lds[2][64];     // double-buffered: q as 32 float4, then k as 32 float4
    __shared__ f4 red_k[4][32];
    __shared__ f4 red_q[4][32];
    __shared__ float red_kq[4];

    const int tid = threadIdx.x;
    const int cg = tid & 31;
    const int rg = tid >> 5;
    const int wave = tid >> 6;

    // Workgroups are dispatched round-robin over the 8 XCDs; remap so each XCD
    // runs a contiguous range of (sequence, head) pairs and the value heads
    // sharing one q/k read it through the same L2.
    const unsigned nwg = gridDim.x;
    unsigned wid = blockIdx.x;
    if ((nwg & 7u) == 0) wid = (wid & 7u) * (nwg >> 3) + (wid >> 3);
    const int b = (int) (wid / (unsigned) p.h_v);
    const int i = (int) (wid - (unsigned) b * (unsigned) p.h_v);
    const int j = i / p.group;
    const long long C = (long long) (2 * p.h_k + p.h_v) * kS;
    const long long tok0 = (long long) b * p.T;

    const int slot = read_slot(p.slots, b, p.n_slots, p.flags, tid == 0 && i == 0);
    const int nt = slot < 0 ? 0 : read_ntok(p.n_tok, b, p.T, p.flags, tid == 0 && i == 0);

    float* tile = nullptr;
    f4 s[16];
    if (nt > 0) {
        tile = p.state + ((long long) slot * p.h_v + i) * (kS * kS) + (rg * 16) * kS + cg * 4;
#pragma unroll
        for (int m = 0; m < 16; ++m) s[m] = __builtin_nontemporal_load((const f4*) (tile + m * kS));
    }

    const float dt_i = p.dt[i];
    const float a_i = p.ssm_a[i];
    for (int t = 0; t < nt; ++t) {
        const float* ht = p.h + (tok0 + t) * C;
        f4* buf = qk_lds[t & 1];
        if (tid < 64) {
            const long long off = tid < 32 ? (long long) j * kS + tid * 4
                                           : (long long) (p.h_k + j) * kS + (tid - 32) * 4;
            buf[tid] = *(const f4*) (ht + off);
        }
        const f4 v = *(const f4*) (ht + (long long) (2 * p.h_k + i) * kS + cg * 4);
        const long long e = (tok0 + t) * p.h_v + i;
        const float bl = p.beta_logit[e];
        const float al = p.alpha[e];
        __syncthreads();

        const float* qrow = (const float*) buf + rg * 16;
        const float* krow = (const float*) buf + kS + rg * 16;
        f4 pk = {0.f, 0.f, 0.f, 0.f}, pq = pk;
        float kq = 0.f;
#pragma unroll
        for (int m = 0; m < 16; ++m) {
            const float kk = krow[m];
            const float qq = qrow[m];
            pk += s[m] * kk;
            pq += s[m] * qq;
            kq += kk * qq;
        }
        // fold the two row groups of this wave (lanes l and l^32)
        pk.x += __shfl_xor(pk.x, 32);
        pk.y += __shfl_xor(pk.y, 32);
        pk.z += __shfl_xor(pk.z, 32);
        pk.w += __shfl_xor(pk.w, 32);
        pq.x += __shfl_xor(pq.x, 32);
        pq.y += __shfl_xor(pq.y, 32);
        pq.z += __shfl_xor(pq.z, 32);
        pq.w += __shfl_xor(pq.w, 32);
        kq += __shfl_xor(kq, 32);
        if ((tid & 32) == 0) {
            red_k[wave][cg] = pk;
            red_q[wave][cg] = pq;
            if (cg == 0) red_kq[wave] = kq;
        }
        __syncthreads();

        const f4 PK = red_k[0][cg] + red_k[1][cg] + red_k[2][cg] + red_k[3][cg];
        const f4 PQ = red_q[0][cg] + red_q[1][cg] + red_q[2][cg] + red_q[3][cg];
        const float KQ = red_kq[0] + red_kq[1] + red_kq[2] + red_kq[3];
        const float beta = sigmoid_f(bl);
        const float eg = expf(softplus_f(al + dt_i) * a_i);
        const f4 d = beta * (v - eg * PK);
        if (rg == 0) *(f4*) (p.o + e * kS + cg * 4) = eg * PQ + KQ * d;
#pragma unroll
        for (int m = 0; m < 16; ++m) s[m] = eg * s[m] + krow[m] * d;
    }
    if (rg == 0) {
        const f4 zero = {0.f, 0.f, 0.f, 0.f};
        for (int t = nt; t < p.T; ++t) *(f4*) (p.o + ((tok0 + t) * p.h_v + i) * kS + cg * 4) = zero;
    }
    if (nt > 0) {
#pragma unroll
        for (int m = 0; m < 16; ++m) __builtin_nontemporal_store(s[m], (f4*) (tile + m * kS));
    }
}

// ------------------------------------------------------------------ gated RMSNorm
// One half-wave per 128-wide row, 8 rows per workgroup.
__global__ __launch_bounds__(256) void gated_rmsnorm_kernel(NormParams p) {
    const long long row = (long long) blockIdx.x * kNormRowsPerBlock + (threadIdx.x >> 5);
    if (row >= p.rows) return;
    const int l = threadIdx.x & 31;
    const long long off = row * kS + 4 * l;
    const f4 x = *(const f4*) (p.o + off);
    const f4 z = *(const f4*) (p.z + off);
    const f4 w = *(const f4*) (p.w + 4 * l);
    const float ss = halfwave_sum(x.x * x.x + x.y * x.y + x.z * x.z + x.w * x.w);
    const float inv = 1.0f / sqrtf(ss * (1.0f / kS) + p.eps);
    *(f4*) (p.y + off) = x * inv * w * sigmoid4(z);
}

// ------------------------------------------------------------------ pool fill
// slots == null: grid-stride zero of the whole state and conv regions, and the
// flag word.  Otherwise blockIdx.y picks a listed slot and blockIdx.x strides over it.
__global__ __launch_bounds__(256) void zero_kernel(ZeroParams p) {
    const f4 zero = {0.f, 0.f, 0.f, 0.f};
    const long long stride = (long long) gridDim.x * blockDim.x;
    const long long first = (long long) blockIdx.x * blockDim.x + threadIdx.x;
    if (!p.slots) {
        if (first == 0 && blockIdx.y == 0) *p.flags = 0u;
        f4* st = (f4*) p.state;
        f4* cv = (f4*) p.conv;
        const long long ns = p.n_slots * p.state_f4, nc = p.n_slots * p.conv_f4;
        for (long long k = first; k < ns; k += stride) st[k] = zero;
        for (long long k = first; k < nc; k += stride) cv[k] = zero;
        return;
    }
    const int slot = p.slots[blockIdx.y];
    if (slot < 0 || (long long) slot >= p.n_slots) {
        if (first == 0) atomicOr(p.flags, GDN_FLAG_BAD_SLOT);
        return;
    }
    f4* st = (f4*) p.state + (long long) slot * p.state_f4;
    f4* cv = (f4*) p.conv + (long long) slot * p.conv_f4;
    for (long long k = first; k < p.state_f4; k += stride) st[k] = zero;
    for (long long k = first; k < p.conv_f4; k += stride) cv[k] = zero;
}

// ------------------------------------------------------------------ launches
hipError_t launch_conv_silu_norm(const ConvParams& p, hipStream_t stream) {
    const dim3 grid((unsigned) ((long long) p.B * p.n_tb), (unsigned) ((p.n_heads + 7) / 8));
    hipLaunchKernelGGL(conv_silu_norm_kernel, grid, dim3(256), 0, stream, p);
    return hipGetLastError();
}

hipError_t launch_decode_step(const StepParams& p, hipStream_t stream) {
    const dim3 grid((unsigned) ((long long) p.B * p.h_v));
    hipLaunchKernelGGL(decode_step_kernel, grid, dim3(256), 0, stream, p);
    return hipGetLastError();
}

hipError_t launch_gated_rmsnorm(const NormParams& p, hipStream_t stream) {
    const dim3 grid((unsigned) ((p.rows + kNormRowsPerBlock - 1) / kNormRowsPerBlock));
    hipLaunchKernelGGL(gated_rmsnorm_kernel, grid, dim3(256), 0, stream, p);
    return hipGetLastError();
}

hipError_t launch_zero(const ZeroParams& p, hipStream_t stream) {
    const dim3 grid(p.slots ? 64u : 2048u, p.slots ? (unsigned) p.n : 1u);
    hipLaunchKernelGGL(zero_kernel, grid, dim3(256), 0, stream, p);
    return hipGetLastError();
}

}  // namespace gdn
