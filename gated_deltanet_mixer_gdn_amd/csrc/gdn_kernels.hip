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
//   decode_one_kernel      beta/gate prologue and the gated delta rule for one
//                          token.  One 256-thread workgroup per (sequence, value
//                          head); the 64 KiB fp32 state tile is read once with
//                          16-byte loads into VGPRs (64 floats per thread) and
//                          written back once.
//   decode_multi_kernel    the same for T > 1 tokens: the tile stays in VGPRs
//                          for all of them, one wave per 32-column block, no
//                          barrier per token (one with the fused norm).
//   gated_rmsnorm_kernel   y = rms_norm(o) * w * sigmoid(z), one half-wave per row.
//                          The same norm also runs as an optional epilogue of
//                          the recurrence kernels (o need not go through HBM), as
//                          the pages' engine fuses its step with the output norm
//                          (`fused_gdn_step_norm`, step 7 of gdn_layer).
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

// Explicit fused multiply-adds: both recurrence kernels spell out the same operation
// sequence so that a T-token call reproduces T single-token calls bit for bit.
__device__ __forceinline__ f4 fma4(f4 a, f4 b, f4 c) {
    return f4{__builtin_fmaf(a.x, b.x, c.x), __builtin_fmaf(a.y, b.y, c.y), __builtin_fmaf(a.z, b.z, c.z),
              __builtin_fmaf(a.w, b.w, c.w)};
}
__device__ __forceinline__ f4 fma4(f4 a, float b, f4 c) { return fma4(a, f4{b, b, b, b}, c); }
__device__ __forceinline__ f4 fma4(float a, f4 b, f4 c) { return fma4(f4{a, a, a, a}, b, c); }
__device__ __forceinline__ float sumsq4(f4 x) {
    return __builtin_fmaf(x.w, x.w, __builtin_fmaf(x.z, x.z, __builtin_fmaf(x.y, x.y, x.x * x.x)));
}

// Cross-lane partial sums that stay in the VALU (no LDS round trip): DPP for lanes
// inside a 16-lane row, the gfx950 permlane swaps across rows.  Each returns v plus
// its partner's v in every lane; the partners are lane ^ 1, lane ^ 2, lane ^ 8,
// lane ^ 16, lane ^ 32, and for add_half8 the other half of the 8-lane block (after
// add_xor1 and add_xor2 all lanes of a quad hold the same value, so that is the
// other quad).  All lanes of the rows involved must be active.
template <int kCtrl>
__device__ __forceinline__ float add_dpp(float v) {
    return v + __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), kCtrl, 0xf, 0xf, false));
}
__device__ __forceinline__ float add_xor1(float v) { return add_dpp<0xB1>(v); }    // quad_perm [1,0,3,2]
__device__ __forceinline__ float add_xor2(float v) { return add_dpp<0x4E>(v); }    // quad_perm [2,3,0,1]
__device__ __forceinline__ float add_half8(float v) { return add_dpp<0x141>(v); }  // row_half_mirror
__device__ __forceinline__ float add_xor8(float v) { return add_dpp<0x128>(v); }   // row_ror:8
__device__ __forceinline__ float add_xor16(float v) {
    const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ __forceinline__ float add_xor32(float v) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ __forceinline__ f4 add_xor8(f4 v) { return f4{add_xor8(v.x), add_xor8(v.y), add_xor8(v.z), add_xor8(v.w)}; }
__device__ __forceinline__ f4 add_xor16(f4 v) {
    return f4{add_xor16(v.x), add_xor16(v.y), add_xor16(v.z), add_xor16(v.w)};
}
__device__ __forceinline__ f4 add_xor32(f4 v) {
    return f4{add_xor32(v.x), add_xor32(v.y), add_xor32(v.z), add_xor32(v.w)};
}

// Sum over each 8-lane block, then over the 32 lanes of a half-wave (lanes 0-31 or
// 32-63); every lane gets the sum.  The fused norms of the recurrence kernels use
// the same order: 8-lane (32-column) blocks b0..b3, then (b0+b1)+(b2+b3).
__device__ __forceinline__ float block8_sum(float v) { return add_half8(add_xor2(add_xor1(v))); }
__device__ __forceinline__ float halfwave_sum(float v) { return add_xor16(add_xor8(block8_sum(v))); }

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
            const float ss = halfwave_sum(sumsq4(hv));
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
// Both recurrence kernels use the one-pass form of a token's update: with the old
// state S, PK[c] = sum_r S[r][c] k[r], PQ[c] = sum_r S[r][c] q[r] and KQ = k . q,
//   d = beta (v - e^g PK);  o = e^g PQ + KQ d;  S <- e^g S + k d^T
// which equals decay -> read -> write -> read of the recurrence in exact arithmetic
// (o = S_new^T q expanded), so one read of S gives both column reductions.

// The (sequence, value head) a workgroup works on.  Workgroups are dispatched
// round-robin over the 8 XCDs; the remap gives each XCD a contiguous range of
// (sequence, head) pairs, so the value heads sharing one q/k read it through the
// same L2 and each XCD streams one region of the pool.
struct HeadJob {
    int b, i, j, slot, nt;
};

__device__ __forceinline__ HeadJob head_job(const StepParams& p, bool report) {
    const unsigned nwg = gridDim.x;
    unsigned wid = blockIdx.x;
    if ((nwg & 7u) == 0) wid = (wid & 7u) * (nwg >> 3) + (wid >> 3);
    HeadJob h;
    h.b = (int) (wid / (unsigned) p.h_v);
    h.i = (int) (wid - (unsigned) h.b * (unsigned) p.h_v);
    h.j = h.i / p.group;
    h.slot = read_slot(p.slots, h.b, p.n_slots, p.flags, report && h.i == 0);
    h.nt = h.slot < 0 ? 0 : read_ntok(p.n_tok, h.b, p.T, p.flags, report && h.i == 0);
    return h;
}

// Single-token decode (T == 1): bandwidth-bound.  One workgroup of 256 threads per
// (sequence, value head); thread tid owns columns 4*cg..4*cg+3 (cg = tid % 32) of
// rows 16*rg..16*rg+15 (rg = tid / 32): 16 float4 = 64 VGPRs of state.  A wave's
// loads cover two 512-byte row segments per instruction.  Reductions: a per-thread
// partial over 16 rows, a cross-half-wave shuffle, then the 4 waves through LDS with
// one barrier.  kNorm: fused gated-RMSNorm epilogue writing y.
template <bool kNorm>
__global__ __launch_bounds__(256) void decode_one_kernel(StepParams p) {
    __shared__ f4 qk_lds[64];        // q as 32 float4, then k as 32 float4
    __shared__ f4 red_k[4][32];
    __shared__ f4 red_q[4][32];
    __shared__ float red_kq[4];

    const int tid = threadIdx.x;
    const int cg = tid & 31;
    const int rg = tid >> 5;
    const int wave = tid >> 6;
    const HeadJob job = head_job(p, tid == 0);
    const int i = job.i;
    const long long C = (long long) (2 * p.h_k + p.h_v) * kS;
    const long long e = (long long) job.b * p.h_v + i;   // (sequence, token 0, head)

    if (job.nt == 0) {   // no token (or an unknown slot): outputs zero, state untouched
        if (rg == 0) {
            const f4 zero = {0.f, 0.f, 0.f, 0.f};
            if (!kNorm || p.o) *(f4*) (p.o + e * kS + cg * 4) = zero;
            if (kNorm) *(f4*) (p.y + e * kS + cg * 4) = zero;
        }
        return;
    }
    float* tile = p.state + ((long long) job.slot * p.h_v + i) * (kS * kS) + (rg * 16) * kS + cg * 4;
    f4 s[16];
#pragma unroll
    for (int m = 0; m < 16; ++m) s[m] = __builtin_nontemporal_load((const f4*) (tile + m * kS));

    const float* ht = p.h + (long long) job.b * C;
    if (tid < 64) {
        const long long off = tid < 32 ? (long long) job.j * kS + tid * 4
                                       : (long long) (p.h_k + job.j) * kS + (tid - 32) * 4;
        qk_lds[tid] = *(const f4*) (ht + off);
    }
    const f4 v = *(const f4*) (ht + (long long) (2 * p.h_k + i) * kS + cg * 4);
    const float bl = p.beta_logit[e];
    const float al = p.alpha[e];
    __syncthreads();

    const float* qrow = (const float*) qk_lds + rg * 16;
    const float* krow = (const float*) qk_lds + kS + rg * 16;
    f4 pk = {0.f, 0.f, 0.f, 0.f}, pq = pk;
    float kq = 0.f;
#pragma unroll
    for (int m = 0; m < 16; ++m) {
        const float kk = krow[m];
        const float qq = qrow[m];
        pk = fma4(s[m], kk, pk);
        pq = fma4(s[m], qq, pq);
        kq = __builtin_fmaf(kk, qq, kq);
    }
    // fold the two row groups of this wave (lanes l and l^32)
    pk = add_xor32(pk);
    pq = add_xor32(pq);
    kq = add_xor32(kq);
    if ((tid & 32) == 0) {
        red_k[wave][cg] = pk;
        red_q[wave][cg] = pq;
        if (cg == 0) red_kq[wave] = kq;
    }
    __syncthreads();

    // the 8 row groups summed as ((g0+g1)+(g2+g3))+((g4+g5)+(g6+g7))
    const f4 PK = (red_k[0][cg] + red_k[1][cg]) + (red_k[2][cg] + red_k[3][cg]);
    const f4 PQ = (red_q[0][cg] + red_q[1][cg]) + (red_q[2][cg] + red_q[3][cg]);
    const float KQ = (red_kq[0] + red_kq[1]) + (red_kq[2] + red_kq[3]);
    const float beta = sigmoid_f(bl);
    const float eg = expf(softplus_f(al + p.dt[i]) * p.ssm_a[i]);
    const f4 d = beta * fma4(-eg, PK, v);
    if (rg == 0) {
        // lanes 0-31 of wave 0 hold o for the whole head, 4 columns each
        const f4 out = fma4(KQ, d, eg * PQ);
        if (!kNorm || p.o) *(f4*) (p.o + e * kS + cg * 4) = out;
        if (kNorm) {
            // sum of o^2: 8-lane (32-column) blocks first, then ((b0+b1)+(b2+b3))
            const float ss = halfwave_sum(sumsq4(out));
            const float inv = 1.0f / sqrtf(ss * (1.0f / kS) + p.eps);
            const f4 zz = *(const f4*) (p.z + e * kS + cg * 4);
            const f4 wn = *(const f4*) (p.norm_w + cg * 4);
            *(f4*) (p.y + e * kS + cg * 4) = out * inv * wn * sigmoid4(zz);
        }
    }
#pragma unroll
    for (int m = 0; m < 16; ++m) __builtin_nontemporal_store(fma4(krow[m], d, eg * s[m]), (f4*) (tile + m * kS));
}

// Multi-token recurrence (T > 1): the state stays in VGPRs for all the call's tokens
// and the per-token chain is what bounds it.  One workgroup of 4 waves per
// (sequence, value head); wave w owns the 32-column block 32w..32w+31 for ALL 128
// rows: lane l has columns 32w + 4*(l % 8) .. +3 of rows 16*(l / 8) .. +15.  The
// column sums then reduce inside the wave (xor-shuffles over the 8 row groups), the
// q/k rows are staged in a wave-private LDS slot, and each token's inputs are
// loaded one token ahead, so the token loop itself has no barrier.
// kNorm: each wave parks its o columns and its sum of o^2 in an 8-token LDS ring;
// every 8 tokens the workgroup synchronises once and normalises that chunk
// cooperatively (thread -> token tid/32, columns 4*(tid%32)..+3), with the chunk's
// z loaded one chunk ahead.
constexpr int kNormChunk = 8;

template <bool kNorm>
__global__ __launch_bounds__(256) void decode_multi_kernel(StepParams p) {
    __shared__ f4 qk_lds[4][64];                    // per wave: q as 32 float4, then k as 32 float4
    __shared__ f4 o_ring[2][kNormChunk][32];        // [chunk parity][token][float4 column group]
    __shared__ float ss_ring[2][kNormChunk][4];     // [chunk parity][token][wave]

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int cg = lane & 7;
    const int rg = lane >> 3;
    const int col = wave * 32 + cg * 4;
    const HeadJob job = head_job(p, tid == 0);
    const int i = job.i;
    const int nt = job.nt;
    const long long C = (long long) (2 * p.h_k + p.h_v) * kS;
    const long long tok0 = (long long) job.b * p.T;
    const long long q_off = (long long) job.j * kS + (lane & 31) * 4 + (lane < 32 ? 0 : (long long) p.h_k * kS);
    const long long v_off = (long long) (2 * p.h_k + i) * kS + col;
    // chunk normalisation: this thread's token within a chunk and columns
    const int n_tt = tid >> 5;
    const int n_c4 = (tid & 31) * 4;

    float* tile = nullptr;
    f4 s[16];
    if (nt > 0) {
        tile = p.state + ((long long) job.slot * p.h_v + i) * (kS * kS) + (rg * 16) * kS + col;
#pragma unroll
        for (int m = 0; m < 16; ++m) s[m] = __builtin_nontemporal_load((const f4*) (tile + m * kS));
    }
    const float dt_i = p.dt[i];
    const float a_i = p.ssm_a[i];

    // q|k and v of the next token, loaded one token ahead
    f4 qk_n = {0.f, 0.f, 0.f, 0.f}, v_n = qk_n;
    auto fetch = [&](int t) {
        const float* ht = p.h + (tok0 + t) * C;
        qk_n = *(const f4*) (ht + q_off);
        v_n = *(const f4*) (ht + v_off);
    };
    // beta and the decay e^g are the same for the whole head: lane l evaluates them for
    // token t0 + l of a 64-token window, and each token reads its pair with readlane
    float beta_w = 0.f, eg_w = 0.f;
    auto gates = [&](int t0) {
        if (t0 + lane < nt) {
            const long long e = (tok0 + t0 + lane) * p.h_v + i;
            beta_w = sigmoid_f(p.beta_logit[e]);
            eg_w = expf(softplus_f(p.alpha[e] + dt_i) * a_i);
        }
    };
    // z of this thread's token in the next chunk, loaded one chunk ahead
    f4 z_n = {0.f, 0.f, 0.f, 0.f};
    auto fetch_z = [&](int t0c) {
        if (t0c + n_tt < nt) z_n = *(const f4*) (p.z + ((tok0 + t0c + n_tt) * p.h_v + i) * kS + n_c4);
    };
    if (nt > 0) {
        fetch(0);
        if (kNorm) fetch_z(0);
    }

    f4* buf = qk_lds[wave];
    const float* qrow = (const float*) buf + rg * 16;
    const float* krow = (const float*) buf + kS + rg * 16;
    for (int t = 0; t < nt; ++t) {
        if ((t & 63) == 0) gates(t);
        const float beta = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(beta_w), t & 63));
        const float eg = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(eg_w), t & 63));
        buf[lane] = qk_n;
        const f4 v = v_n;
        if (t + 1 < nt) fetch(t + 1);
        // the staging above is wave-private: order it against this wave's reads
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");

        f4 pk = {0.f, 0.f, 0.f, 0.f}, pq = pk;
        float kq = 0.f;
#pragma unroll
        for (int m = 0; m < 16; ++m) {
            const float kk = krow[m];
            const float qq = qrow[m];
            pk = fma4(s[m], kk, pk);
            pq = fma4(s[m], qq, pq);
            kq = __builtin_fmaf(kk, qq, kq);
        }
        // sum over the 8 row groups of the wave (lane bits 3..5):
        // ((g0+g1)+(g2+g3))+((g4+g5)+(g6+g7)), as in the single-token kernel
        pk = add_xor32(add_xor16(add_xor8(pk)));
        pq = add_xor32(add_xor16(add_xor8(pq)));
        kq = add_xor32(add_xor16(add_xor8(kq)));
        const f4 d = beta * fma4(-eg, pk, v);
        const f4 out = fma4(kq, d, eg * pq);
        if ((!kNorm || p.o) && rg == 0) *(f4*) (p.o + ((tok0 + t) * p.h_v + i) * kS + col) = out;
        if (kNorm) {
            const int par = (t / kNormChunk) & 1;
            const int slot8 = t % kNormChunk;
            // sum of o^2 over this wave's 32 columns (lane bits 0..2)
            const float ss = block8_sum(sumsq4(out));
            if (rg == 0) o_ring[par][slot8][wave * 8 + cg] = out;
            if (lane == 0) ss_ring[par][slot8][wave] = ss;
            if (slot8 == kNormChunk - 1 || t == nt - 1) {   // uniform over the workgroup
                __syncthreads();
                const int t0c = t - slot8;
                const f4 zz = z_n;
                if (t0c + kNormChunk < nt) fetch_z(t0c + kNormChunk);
                if (n_tt <= slot8) {
                    const float tot = (ss_ring[par][n_tt][0] + ss_ring[par][n_tt][1]) +
                                      (ss_ring[par][n_tt][2] + ss_ring[par][n_tt][3]);
                    const float inv = 1.0f / sqrtf(tot * (1.0f / kS) + p.eps);
                    const f4 wn = *(const f4*) (p.norm_w + n_c4);
                    *(f4*) (p.y + ((tok0 + t0c + n_tt) * p.h_v + i) * kS + n_c4) =
                        o_ring[par][n_tt][n_c4 / 4] * inv * wn * sigmoid4(zz);
                }
            }
        }
        // re-read k from LDS rather than keeping 16 rows live across the reduction (the
        // fence stops the compiler from reusing the values loaded above)
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
        const f4* k4 = (const f4*) krow;
#pragma unroll
        for (int m4 = 0; m4 < 4; ++m4) {
            const f4 kk = k4[m4];
            s[4 * m4 + 0] = fma4(kk.x, d, eg * s[4 * m4 + 0]);
            s[4 * m4 + 1] = fma4(kk.y, d, eg * s[4 * m4 + 1]);
            s[4 * m4 + 2] = fma4(kk.z, d, eg * s[4 * m4 + 2]);
            s[4 * m4 + 3] = fma4(kk.w, d, eg * s[4 * m4 + 3]);
        }
    }
    if (rg == 0) {
        const f4 zero = {0.f, 0.f, 0.f, 0.f};
        for (int t = nt; t < p.T; ++t) {
            const long long e = ((tok0 + t) * p.h_v + i) * kS + col;
            if (!kNorm || p.o) *(f4*) (p.o + e) = zero;
            if (kNorm) *(f4*) (p.y + e) = zero;
        }
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
    const float ss = halfwave_sum(sumsq4(x));
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
    const bool one = p.T == 1;
    if (p.y) {
        if (one) hipLaunchKernelGGL((decode_one_kernel<true>), grid, dim3(256), 0, stream, p);
        else hipLaunchKernelGGL((decode_multi_kernel<true>), grid, dim3(256), 0, stream, p);
    } else {
        if (one) hipLaunchKernelGGL((decode_one_kernel<false>), grid, dim3(256), 0, stream, p);
        else hipLaunchKernelGGL((decode_multi_kernel<false>), grid, dim3(256), 0, stream, p);
    }
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
