// gdn_device.h - device helpers shared by the gfx950 kernels of the Gated DeltaNet
// decode mixer (gdn_conv.hip, gdn_recurrence.hip, gdn_norm.hip).
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
#pragma once

#include <hip/hip_runtime.h>

#include "gdn_bf16.h"
#include "gdn_kernels.h"

namespace gdn {

typedef float f4 __attribute__((ext_vector_type(4)));
typedef float f2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ float sigmoid_f(float x) { return 1.0f / (1.0f + expf(-x)); }

// softplus in fp32: above 20 the log1p term is below half an ulp of x
__device__ __forceinline__ float softplus_f(float x) { return x > 20.0f ? x : log1pf(expf(x)); }

// The sigmoid of SiLU and of the output gate, per channel: e^-x as 2^(-x log2 e) on the
// hardware exp2 and 1 / (1 + e^-x) on the hardware reciprocal (about 1 ulp each, the
// rounding of -x log2 e adding |x| 2^-24 relative), four instructions where the
// correctly rounded exp and division take about twenty.  Every kernel uses this one,
// so the kernels still agree with one another bit for bit.
__device__ __forceinline__ float sigmoid_hw(float x) {
    return __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(x * -1.44269504088896341f));
}
__device__ __forceinline__ f4 sigmoid4(f4 x) {
    return f4{sigmoid_hw(x.x), sigmoid_hw(x.y), sigmoid_hw(x.z), sigmoid_hw(x.w)};
}

// output gate of the gated RMSNorm: sigmoid(z), or z * sigmoid(z) (SiLU, the earlier
// model of the family); silu is uniform over the launch
__device__ __forceinline__ f4 gate4(f4 z, int silu) {
    const f4 g = sigmoid4(z);
    return silu ? z * g : g;
}

// Explicit fused multiply-adds: both recurrence kernels spell out the same operation
// sequence so that a T-token call reproduces T single-token calls bit for bit.
__device__ __forceinline__ f4 fma4(f4 a, f4 b, f4 c) {
    return f4{__builtin_fmaf(a.x, b.x, c.x), __builtin_fmaf(a.y, b.y, c.y), __builtin_fmaf(a.z, b.z, c.z),
              __builtin_fmaf(a.w, b.w, c.w)};
}
__device__ __forceinline__ f4 fma4(f4 a, float b, f4 c) { return fma4(a, f4{b, b, b, b}, c); }
__device__ __forceinline__ f4 fma4(float a, f4 b, f4 c) { return fma4(f4{a, a, a, a}, b, c); }
// 1 / sqrt(mean of squares + eps) for a 128-wide row from its sum of squares, on the
// hardware reciprocal square root (about 1 ulp; one function for every kernel)
__device__ __forceinline__ float rms_inv(float sum_sq, float eps) {
    return __builtin_amdgcn_rsqf(__builtin_fmaf(sum_sq, 1.0f / kS, eps));
}
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

// Reduce-scatter of the 4 components of v over the lanes lane, lane ^ 16, lane ^ 32 and
// lane ^ 48: each lane ends with the total of one component, added in the order
// add_xor32(add_xor16(.)) adds it, at a third of the instructions (one swap moves a
// component each way).  Which component a lane gets depends only on its lane bits 4
// and 5; scatter_sum4(f4{0, 1, 2, 3}) / 4 names it.  All 64 lanes must be active.
__device__ __forceinline__ float scatter_sum4(f4 v) {
    const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(v.x), __float_as_uint(v.z), false, false);
    const auto b = __builtin_amdgcn_permlane16_swap(__float_as_uint(v.y), __float_as_uint(v.w), false, false);
    const float u = __uint_as_float(a[0]) + __uint_as_float(a[1]);
    const float w = __uint_as_float(b[0]) + __uint_as_float(b[1]);
    const auto c = __builtin_amdgcn_permlane32_swap(__float_as_uint(u), __float_as_uint(w), false, false);
    return __uint_as_float(c[0]) + __uint_as_float(c[1]);
}

// Where the single-launch decode also writes y split for the projections: row `row` of
// a [rows][chunks * 64] activation in the tiled layout of gdn_split_bf16 (tile = 32
// rows x 64 k; fragment (s, lane = i + 32h) of a tile holds the 8 values
// [32R + i][64C + 32h + 8s + j] as bf16, the hi fragment at (2s)*64 + lane and the lo
// fragment at (2s + 1)*64 + lane, in 16-byte units, 512 per tile), columns of value
// head `head` at head*128 ..
struct SplitOut {
    uint16_t* ys;   // null: not written
    int row, chunks, head;
};

// 16-byte slot of the fragment that column group cg (columns 4cg..4cg+3 of the head)
// writes: the pair (cg, cg ^ 1) covers 8 consecutive columns; the even member writes
// their hi fragment, the odd one their lo fragment.
__device__ __forceinline__ long long split_slot(const SplitOut& so, int cg) {
    const int kin = (4 * (cg & ~1)) & 63;            // column of the pair in its 64-chunk
    const long long tile = (long long) (so.row >> 5) * so.chunks + 2 * so.head + ((cg & ~1) >= 16);
    return tile * 512 + (2 * ((kin & 31) >> 3) + (cg & 1)) * 64 + (so.row & 31) + 32 * (kin >> 5);
}

// The 32 lanes of a half-wave hold y columns 4cg..4cg+3 (cg = lane % 32) of one head:
// each pair swaps its 4 values (a DPP move inside the quad) and writes its fragment,
// hi or lo, with the split pass's arithmetic (so the same bits as gdn_split_bf16 of y).
__device__ __forceinline__ void store_split8(const SplitOut& so, int cg, f4 v) {
    auto mate = [](float x) {
        return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0xB1, 0xf, 0xf, false));
    };
    const f4 pv = {mate(v.x), mate(v.y), mate(v.z), mate(v.w)};
    const bool odd = cg & 1;
    const f4 a = odd ? pv : v;   // the pair's first 4 columns
    const f4 c = odd ? v : pv;   // its last 4
    const float x[8] = {a.x, a.y, a.z, a.w, c.x, c.y, c.z, c.w};
    unsigned hi[8], lo[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) split_bf16(x[j], hi[j], lo[j]);
    const unsigned* w = odd ? lo : hi;
    typedef unsigned u4 __attribute__((ext_vector_type(4)));
    const u4 frag = {w[0] | w[1] << 16, w[2] | w[3] << 16, w[4] | w[5] << 16, w[6] | w[7] << 16};
    ((u4*) so.ys)[split_slot(so, cg)] = frag;
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

// Four channels c..c+3 of the causal depthwise conv: their taps (tap 3 multiplies the
// current input) and their last three raw inputs, oldest first, as float4 over the
// four channels.
struct ConvGroup {
    f4 w0, w1, w2, w3;   // taps of channels c, c+1, c+2, c+3
    f4 x3, x2, x1;       // history: x3 oldest, x1 newest

    __device__ __forceinline__ void load_taps(const float* w, long long c) {
        w0 = *(const f4*) (w + (c + 0) * kDConv);
        w1 = *(const f4*) (w + (c + 1) * kDConv);
        w2 = *(const f4*) (w + (c + 2) * kDConv);
        w3 = *(const f4*) (w + (c + 3) * kDConv);
    }
    // the stored history is [c][j]: 12 consecutive floats for channels c..c+3
    __device__ __forceinline__ void load_history(const float* X) {
        set_history(*(const f4*) (X + 0), *(const f4*) (X + 4), *(const f4*) (X + 8));
    }
    // the history from its 12 stored floats (as three float4 loads)
    __device__ __forceinline__ void set_history(f4 a, f4 m, f4 z) {
        x3 = f4{a.x, a.w, m.z, z.y};
        x2 = f4{a.y, m.x, m.w, z.z};
        x1 = f4{a.z, m.y, z.x, z.w};
    }
    __device__ __forceinline__ static void store_history(float* X, f4 n3, f4 n2, f4 n1) {
        *(f4*) (X + 0) = f4{n3.x, n2.x, n1.x, n3.y};
        *(f4*) (X + 4) = f4{n2.y, n1.y, n3.z, n2.z};
        *(f4*) (X + 8) = f4{n1.z, n3.w, n2.w, n1.w};
    }
    // pre-activation of the current input x (taps applied oldest first, as explicit
    // FMAs so every kernel rounds it the same way), then roll x into the history
    __device__ __forceinline__ static float tap4(f4 w, float a, float b, float c, float d) {
        return __builtin_fmaf(w.w, d, __builtin_fmaf(w.z, c, __builtin_fmaf(w.y, b, w.x * a)));
    }
    __device__ __forceinline__ f4 step(f4 x) {
        f4 u;
        u.x = tap4(w0, x3.x, x2.x, x1.x, x.x);
        u.y = tap4(w1, x3.y, x2.y, x1.y, x.y);
        u.z = tap4(w2, x3.z, x2.z, x1.z, x.z);
        u.w = tap4(w3, x3.w, x2.w, x1.w, x.w);
        x3 = x2;
        x2 = x1;
        x1 = x;
        return u;
    }
};

// The conv history of channels c..c+3 after their sequence advances by nt >= 1 tokens:
// entries nt, nt+1, nt+2 of (stored history x3 x2 x1, raw rows 0..nt-1 of xq).  Raw
// values are only moved, so every kernel that advances a history gets the same bits.
__device__ __forceinline__ void advance_history(float* X, const float* xq, long long C, long long c, int nt) {
    ConvGroup old;
    old.load_history(X + c * kHist);
    auto entry = [&](int k) -> f4 {
        return k == 0 ? old.x3 : k == 1 ? old.x2 : k == 2 ? old.x1 : *(const f4*) (xq + (k - 3) * C + c);
    };
    ConvGroup::store_history(X + c * kHist, entry(nt), entry(nt + 1), entry(nt + 2));
}

}  // namespace gdn
