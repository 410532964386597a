// gdn_conv.hip - conv + SiLU + L2 norm kernel and the state-pool fill kernel.
#include "gdn_device.h"

namespace gdn {

// ------------------------------------------------------------------ conv + SiLU + L2
//
// The conv reads only raw inputs (the stored history and qkv rows), so its tokens are
// independent and the kernel is laid out as a flat stream over (sequence, token group,
// head block): one 256-thread workgroup takes G consecutive tokens of 8 heads of one
// sequence, and consecutive workgroups take the next head block, then the next token
// group, so the chip sweeps qkv and h in address order (a token-by-token walk per
// workgroup scatters the concurrent accesses and moved the same bytes about 20% slower
// on MI355X).  The workgroup id is remapped so each XCD sweeps one contiguous range,
// where the three rows before a group, which the group before it also read, are still
// in that XCD's L2.
//
// A half-wave (32 lanes) owns one 128-channel head: lane l has the four channels
// 4l..4l+3.  The L2 norm of a q or k head is summed in the order of the single-launch
// decode's prologue (lane l < 16 and lane l + 16 hold the channel groups that prologue
// gives one lane, so their sums of squares are added first, then the 16-lane tree),
// which keeps h bit for bit equal across the two forms.
//
// Only token group 0 of a sequence reads or writes the stored history (and advances it
// first for a commit); later groups take their three history entries from the qkv rows
// before them, so groups never race on it.  persist = 0 leaves the stored history as it
// was (a speculative window).
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

template <int G>
__global__ __launch_bounds__(256) void conv_silu_norm_kernel(ConvParams p) {
    const int tid = threadIdx.x;
    const unsigned nwg = gridDim.x;
    unsigned wid = blockIdx.x;
    if ((nwg & 7u) == 0) wid = (wid & 7u) * (nwg >> 3) + (wid >> 3);
    const int n_hb = (p.n_heads + kConvHeadsPerBlock - 1) / kConvHeadsPerBlock;
    const int hb = (int) (wid % (unsigned) n_hb);
    const int grp = (int) ((wid / (unsigned) n_hb) % (unsigned) p.n_groups);
    const int b = (int) (wid / ((unsigned) n_hb * (unsigned) p.n_groups));
    const int head = hb * kConvHeadsPerBlock + (tid >> 5);
    if (head >= p.n_heads) return;  // whole half-waves leave together
    const long long C = (long long) p.n_heads * kS;
    const long long c = (long long) head * kS + 4 * (tid & 31);
    const int t0 = grp * G;
    const int t1 = min(t0 + G, p.T);
    const float* xq = p.qkv + (long long) b * p.T * C;   // this sequence's qkv rows
    float* hq = p.h + (long long) b * p.T * C;
    const bool reporter = (tid == 0 && hb == 0 && grp == 0);

    const int slot = read_slot(p.slots, b, p.n_slots, p.flags, reporter);
    int nt = read_ntok(p.n_tok, b, p.T, p.flags, reporter);
    if (slot < 0) nt = 0;  // unknown slot: no history to read or advance, outputs zero
    const int t_end = min(t1, nt);

    ConvGroup g;
    float* X = p.conv + ((long long) (slot < 0 ? 0 : slot) * C) * kHist;
    bool advanced = false;
    if (p.adv_qkv && grp == 0 && slot >= 0) {
        // the commit of the previous window comes first: its kept rows advance the
        // stored history (kept whatever this call's tokens do), and token 0 below
        // starts from the advanced history, kept in registers
        const int na = read_ntok(p.n_adv, b, p.adv_T, p.flags, reporter);
        if (na > 0) {
            advance_and_keep(g, X, p.adv_qkv + (long long) b * p.adv_T * C, C, c, na);
            advanced = true;
        }
    }
    if (t_end > t0) {
        g.load_taps(p.w, c);
        if (t0 == 0) {
            if (!advanced) g.load_history(X + c * kHist);
        } else {
            g.x3 = *(const f4*) (xq + (t0 - 3) * C + c);
            g.x2 = *(const f4*) (xq + (t0 - 2) * C + c);
            g.x1 = *(const f4*) (xq + (t0 - 1) * C + c);
        }
        // the group's inputs, all in flight at once; slots past the last token re-read
        // that token's row (in bounds, and no branch around a load, so the array stays
        // in registers)
        f4 x[G];
#pragma unroll
        for (int u = 0; u < G; ++u) x[u] = *(const f4*) (xq + min(t0 + u, t_end - 1) * C + c);
        const bool normed = head < 2 * p.h_k;
        const float extra = head < p.h_k ? p.qscale : 1.0f;
#pragma unroll
        for (int u = 0; u < G; ++u) {
            if (t0 + u >= t_end) break;   // the same in every lane of the workgroup
            const f4 uu = g.step(x[u]);
            f4 hv = uu * sigmoid4(uu);
            if (normed) {
                // lanes l and l ^ 16 hold the prologue's two channel groups of one lane
                const float ss = add_xor8(block8_sum(add_xor16(sumsq4(hv))));
                hv *= extra / sqrtf(ss + p.eps);
            }
            f4* dst = (f4*) (hq + (t0 + u) * C + c);
            if (p.stream_h) __builtin_nontemporal_store(hv, dst);
            else *dst = hv;
        }
    }
    const f4 zero = {0.f, 0.f, 0.f, 0.f};
    for (int t = max(t0, nt); t < t1; ++t) *(f4*) (hq + t * C + c) = zero;

    if (t0 == 0 && nt > 0 && p.persist) {
        // the new history is the last three entries of (stored history, tokens 0..nt-1)
        if (nt <= t1)
            ConvGroup::store_history(X + c * kHist, g.x3, g.x2, g.x1);
        else  // nt > t1 >= 3: all three come from qkv
            ConvGroup::store_history(X + c * kHist, *(const f4*) (xq + (nt - 3) * C + c),
                                     *(const f4*) (xq + (nt - 2) * C + c), *(const f4*) (xq + (nt - 1) * C + c));
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
    const long long n_hb = (p.n_heads + kConvHeadsPerBlock - 1) / kConvHeadsPerBlock;
    const dim3 grid((unsigned) ((long long) p.B * p.n_groups * n_hb));
    switch (p.group) {
    case 1: hipLaunchKernelGGL(conv_silu_norm_kernel<1>, grid, dim3(256), 0, stream, p); break;
    case 4: hipLaunchKernelGGL(conv_silu_norm_kernel<4>, grid, dim3(256), 0, stream, p); break;
    case kConvGroup: hipLaunchKernelGGL(conv_silu_norm_kernel<kConvGroup>, grid, dim3(256), 0, stream, p); break;
    default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

hipError_t launch_zero(const ZeroParams& p, hipStream_t stream) {
    const dim3 grid(p.slots ? 64u : 2048u, p.slots ? (unsigned) p.n : 1u);
    hipLaunchKernelGGL(zero_kernel, grid, dim3(256), 0, stream, p);
    return hipGetLastError();
}

}  // namespace gdn
