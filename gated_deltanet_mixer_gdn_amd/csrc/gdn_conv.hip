// gdn_conv.hip - conv + SiLU + L2 norm kernel and the state-pool fill kernel.
#include "gdn_device.h"

namespace gdn {

// ------------------------------------------------------------------ conv + SiLU + L2
//
// grid.x = B * n_tb (sequence, token block of tpb tokens),
// grid.y = ceil(n_heads / 16); 256 threads.  A 16-lane row (one DPP row) owns one
// 128-channel head: lane l has the channel groups 4l..4l+3 and 64+4l..64+4l+3, so
// every load and store instruction of the row covers 256 contiguous bytes and the
// head's L2 norm is a 16-lane DPP sum.  Inputs are loaded three tokens ahead.  Only
// token block 0 reads or writes the stored history; later blocks take their first
// three history entries from qkv, so blocks never race on it.  persist = 0 leaves
// the stored history as it was (a speculative window).
// advance_history for channels c..c+3 that also leaves the new history in g
__device__ __forceinline__ void advance_and_keep(ConvGroup& g, float* X, const float* xq, long long C, long long c,
                                                 int nt) {
    ConvGroup old;
    old.load_history(X + c * kHist);
    auto entry = [&](int k) -> f4 {
        return k == 0 ? old.x3 : k == 1 ? old.x2 : k == 2 ? old.x1 : *(const f4*) (xq + (k - 3) * C + c);
    };
    g.x3 = entry(nt);
    g.x2 = entry(nt + 1);
    g.x1 = entry(nt + 2);
    ConvGroup::store_history(X + c * kHist, g.x3, g.x2, g.x1);
}

__global__ __launch_bounds__(256) void conv_silu_norm_kernel(ConvParams p) {
    const int tid = threadIdx.x;
    const int head = blockIdx.y * 16 + (tid >> 4);
    if (head >= p.n_heads) return;  // whole 16-lane rows leave together
    const int l = tid & 15;
    const int b = blockIdx.x / p.n_tb;
    const int tb = blockIdx.x - b * p.n_tb;
    const long long C = (long long) p.n_heads * kS;
    const long long ca = (long long) head * kS + 4 * l;
    const long long cb = ca + 64;
    const int t0 = tb * p.tpb;
    const int t1 = min(t0 + p.tpb, p.T);
    const float* xq = p.qkv + (long long) b * p.T * C;   // this sequence's qkv rows
    float* hq = p.h + (long long) b * p.T * C;
    const bool reporter = (tid == 0 && blockIdx.y == 0 && tb == 0);

    const int slot = read_slot(p.slots, b, p.n_slots, p.flags, reporter);
    int nt = read_ntok(p.n_tok, b, p.T, p.flags, reporter);
    if (slot < 0) nt = 0;  // unknown slot: no history to read or advance, outputs zero
    const int t_end = min(t1, nt);

    ConvGroup ga, gb;
    float* X = p.conv + ((long long) (slot < 0 ? 0 : slot) * C) * kHist;
    bool advanced = false;
    if (p.adv_qkv && tb == 0 && slot >= 0) {
        // the commit of the previous window comes first: its kept rows advance the
        // stored history (kept whatever this call's tokens do), and token 0 below
        // starts from the advanced history, kept in registers
        const int na = read_ntok(p.n_adv, b, p.adv_T, p.flags, reporter);
        if (na > 0) {
            const float* xa = p.adv_qkv + (long long) b * p.adv_T * C;
            advance_and_keep(ga, X, xa, C, ca, na);
            advance_and_keep(gb, X, xa, C, cb, na);
            advanced = true;
        }
    }
    // inputs of tokens t, t + 1 and t + 2, loaded ahead
    f4 xa_1 = {0.f, 0.f, 0.f, 0.f}, xb_1 = xa_1, xa_2 = xa_1, xb_2 = xa_1, xa_3 = xa_1, xb_3 = xa_1;
    if (t_end > t0) {
        ga.load_taps(p.w, ca);
        gb.load_taps(p.w, cb);
        if (t0 == 0) {
            if (!advanced) {
                ga.load_history(X + ca * kHist);
                gb.load_history(X + cb * kHist);
            }
        } else {
            ga.x3 = *(const f4*) (xq + (t0 - 3) * C + ca);
            ga.x2 = *(const f4*) (xq + (t0 - 2) * C + ca);
            ga.x1 = *(const f4*) (xq + (t0 - 1) * C + ca);
            gb.x3 = *(const f4*) (xq + (t0 - 3) * C + cb);
            gb.x2 = *(const f4*) (xq + (t0 - 2) * C + cb);
            gb.x1 = *(const f4*) (xq + (t0 - 1) * C + cb);
        }
        xa_1 = *(const f4*) (xq + t0 * C + ca);
        xb_1 = *(const f4*) (xq + t0 * C + cb);
        if (t0 + 1 < t_end) {
            xa_2 = *(const f4*) (xq + (t0 + 1) * C + ca);
            xb_2 = *(const f4*) (xq + (t0 + 1) * C + cb);
        }
        if (t0 + 2 < t_end) {
            xa_3 = *(const f4*) (xq + (t0 + 2) * C + ca);
            xb_3 = *(const f4*) (xq + (t0 + 2) * C + cb);
        }
    }

    const bool normed = head < 2 * p.h_k;
    const float extra = head < p.h_k ? p.qscale : 1.0f;
    for (int t = t0; t < t_end; ++t) {
        const f4 xa = xa_1, xb = xb_1;
        xa_1 = xa_2;
        xb_1 = xb_2;
        xa_2 = xa_3;
        xb_2 = xb_3;
        if (t + 3 < t_end) {
            xa_3 = *(const f4*) (xq + (t + 3) * C + ca);
            xb_3 = *(const f4*) (xq + (t + 3) * C + cb);
        }
        const f4 ua = ga.step(xa);
        const f4 ub = gb.step(xb);
        f4 ha = ua * sigmoid4(ua);
        f4 hb = ub * sigmoid4(ub);
        if (normed) {
            const float ss = add_xor8(block8_sum(sumsq4(ha) + sumsq4(hb)));
            const float sc = extra / sqrtf(ss + p.eps);
            ha *= sc;
            hb *= sc;
        }
        *(f4*) (hq + t * C + ca) = ha;
        *(f4*) (hq + t * C + cb) = hb;
    }
    const f4 zero = {0.f, 0.f, 0.f, 0.f};
    for (int t = max(t0, nt); t < t1; ++t) {
        *(f4*) (hq + t * C + ca) = zero;
        *(f4*) (hq + t * C + cb) = zero;
    }

    if (t0 == 0 && nt > 0 && p.persist) {
        // the new history is the last three entries of (stored history, tokens 0..nt-1)
        if (nt <= t1) {
            ConvGroup::store_history(X + ca * kHist, ga.x3, ga.x2, ga.x1);
            ConvGroup::store_history(X + cb * kHist, gb.x3, gb.x2, gb.x1);
        } else {  // nt > t1 >= 3: all three come from qkv
            for (int g = 0; g < 2; ++g) {
                const long long c = g ? cb : ca;
                ConvGroup::store_history(X + c * kHist, *(const f4*) (xq + (nt - 3) * C + c),
                                         *(const f4*) (xq + (nt - 2) * C + c),
                                         *(const f4*) (xq + (nt - 1) * C + c));
            }
        }
    }
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

// ------------------------------------------------------------------ launch
hipError_t launch_conv_silu_norm(const ConvParams& p, hipStream_t stream) {
    const dim3 grid((unsigned) ((long long) p.B * p.n_tb), (unsigned) ((p.n_heads + 15) / 16));
    hipLaunchKernelGGL(conv_silu_norm_kernel, grid, dim3(256), 0, stream, p);
    return hipGetLastError();
}

hipError_t launch_zero(const ZeroParams& p, hipStream_t stream) {
    const dim3 grid(p.slots ? 64u : 2048u, p.slots ? (unsigned) p.n : 1u);
    hipLaunchKernelGGL(zero_kernel, grid, dim3(256), 0, stream, p);
    return hipGetLastError();
}

}  // namespace gdn
