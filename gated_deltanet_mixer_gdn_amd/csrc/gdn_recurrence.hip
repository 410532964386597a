// gdn_recurrence.hip - the gated delta-rule recurrence kernels (one token, many tokens).
#include "gdn_device.h"

namespace gdn {

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

// LDS a 256-thread workgroup uses to reduce one head's column sums across its waves.
struct HeadReduce {
    f4 k[4][32];
    f4 q[4][32];
};

// k . q over the 128 rows, the same in every lane of a full wave: lane l multiplies
// rows 2l and 2l+1, then the 64 lane sums are added pairwise across the wave.  Every
// recurrence kernel forms it this way, so they agree bit for bit.  qk: q as 128
// floats, then k as 128 floats.
__device__ __forceinline__ float wave_kq(const float* qk, int lane) {
    const float2 q2 = ((const float2*) qk)[lane];
    const float2 k2 = ((const float2*) (qk + kS))[lane];
    const float part = __builtin_fmaf(k2.y, q2.y, k2.x * q2.x);
    return add_xor32(add_xor16(add_xor8(block8_sum(part))));
}

// One token of one head for a group of 256 threads (tid = the thread's index in the
// group; a larger workgroup runs one such group per head) whose thread tid holds columns
// 4*cg..4*cg+3 (cg = tid % 32) of rows 16*rg..16*rg+15 (rg = tid / 32) of the old
// state in s[] (16 float4 = 64 VGPRs).  qk: q as 32 float4, then k as 32 float4, in
// LDS; v: this thread's 4 columns of v.  Reductions: a per-thread partial over 16
// rows, a cross-half-wave fold, then the 4 waves through LDS (one barrier, so every
// thread must call this).  Lanes 0-31 of wave 0 (rg == 0) then hold o for the whole
// head and write o (if o_row) and the gated RMSNorm y (if kNorm); s[] becomes the new
// state.  The operation sequence is the multi-token kernel's, so the two agree bit
// for bit.
// oscale multiplies o after the readout (1 unless the 1/sqrt(S) is applied there
// rather than to q); gate_silu picks the epilogue's gate.
// y_row may be null; so.ys (if set) also takes y split for the projections.
template <bool kNorm>
__device__ __forceinline__ void head_token_256(f4 (&s)[16], const f4* qk, f4 v, float beta, float eg,
                                               HeadReduce& red, float* o_row, const float* z_row,
                                               const float* norm_w, float* y_row, const SplitOut& so, float eps,
                                               float oscale, int gate_silu, int tid) {
    const int cg = tid & 31;
    const int rg = tid >> 5;
    const int wave = tid >> 6;
    const float* qrow = (const float*) qk + rg * 16;
    const float* krow = (const float*) qk + kS + rg * 16;
    f4 pk = {0.f, 0.f, 0.f, 0.f}, pq = pk;
#pragma unroll
    for (int m = 0; m < 16; ++m) {
        pk = fma4(s[m], krow[m], pk);
        pq = fma4(s[m], qrow[m], pq);
    }
    const float KQ = wave_kq((const float*) qk, tid & 63);
    // fold the two row groups of this wave (lanes l and l^32)
    pk = add_xor32(pk);
    pq = add_xor32(pq);
    if ((tid & 32) == 0) {
        red.k[wave][cg] = pk;
        red.q[wave][cg] = pq;
    }
    __syncthreads();

    // the 8 row groups summed as ((g0+g1)+(g2+g3))+((g4+g5)+(g6+g7))
    const f4 PK = (red.k[0][cg] + red.k[1][cg]) + (red.k[2][cg] + red.k[3][cg]);
    const f4 PQ = (red.q[0][cg] + red.q[1][cg]) + (red.q[2][cg] + red.q[3][cg]);
    const f4 d = beta * fma4(-eg, PK, v);
    if (rg == 0) {
        f4 out = fma4(KQ, d, eg * PQ);
        if (oscale != 1.0f) out *= oscale;
        if (o_row) *(f4*) (o_row + cg * 4) = out;
        if (kNorm) {
            // sum of o^2: 8-lane (32-column) blocks first, then ((b0+b1)+(b2+b3))
            const float ss = halfwave_sum(sumsq4(out));
            const float inv = rms_inv(ss, eps);
            const f4 zz = *(const f4*) (z_row + cg * 4);
            const f4 wn = *(const f4*) (norm_w + cg * 4);
            const f4 yv = out * inv * wn * gate4(zz, gate_silu);
            if (y_row) *(f4*) (y_row + cg * 4) = yv;
            if (so.ys) store_split8(so, cg, yv);
        }
    }
#pragma unroll
    for (int m = 0; m < 16; ++m) s[m] = fma4(krow[m], d, eg * s[m]);
}

__device__ __forceinline__ void load_tile(f4 (&s)[16], const float* tile) {
#pragma unroll
    for (int m = 0; m < 16; ++m) s[m] = __builtin_nontemporal_load((const f4*) (tile + m * kS));
}

__device__ __forceinline__ void store_tile(const f4 (&s)[16], float* tile) {
#pragma unroll
    for (int m = 0; m < 16; ++m) __builtin_nontemporal_store(s[m], (f4*) (tile + m * kS));
}

// Single-token decode (T == 1): bandwidth-bound.  One workgroup of 256 threads per
// (sequence, value head) in the layout of head_token_256; a wave's tile loads cover
// two 512-byte row segments per instruction.  kNorm: fused gated-RMSNorm epilogue.
template <bool kNorm>
__global__ __launch_bounds__(256) void decode_one_kernel(StepParams p) {
    __shared__ f4 qk_lds[64];        // q as 32 float4, then k as 32 float4
    __shared__ HeadReduce red;

    const int tid = threadIdx.x;
    const int cg = tid & 31;
    const int rg = tid >> 5;
    const HeadJob job = head_job(p, tid == 0);
    const int i = job.i;
    const long long C = (long long) (2 * p.h_k + p.h_v) * kS;
    const long long e = (long long) job.b * p.h_v + i;   // (sequence, token 0, head)

    if (job.nt == 0) {   // no token (or an unknown slot): outputs zero, state untouched
        if (rg == 0) {
            const f4 zero = {0.f, 0.f, 0.f, 0.f};
            if (p.o) *(f4*) (p.o + e * kS + cg * 4) = zero;
            if (kNorm) *(f4*) (p.y + e * kS + cg * 4) = zero;
        }
        return;
    }
    float* tile = p.state + ((long long) job.slot * p.h_v + i) * (kS * kS) + (rg * 16) * kS + cg * 4;
    f4 s[16];
    load_tile(s, tile);

    const float* ht = p.h + (long long) job.b * C;
    if (tid < 64) {
        const long long off = tid < 32 ? (long long) job.j * kS + tid * 4
                                       : (long long) (p.h_k + job.j) * kS + (tid - 32) * 4;
        qk_lds[tid] = *(const f4*) (ht + off);
    }
    const f4 v = *(const f4*) (ht + (long long) (2 * p.h_k + i) * kS + cg * 4);
    const float beta = sigmoid_f(p.beta_logit[e]);
    const float eg = expf(softplus_f(p.alpha[e] + p.dt[i]) * p.ssm_a[i]);
    __syncthreads();

    head_token_256<kNorm>(s, qk_lds, v, beta, eg, red, p.o ? p.o + e * kS : nullptr,
                          kNorm ? p.z + e * kS : nullptr, p.norm_w, kNorm ? p.y + e * kS : nullptr,
                          SplitOut{nullptr, 0, 0, 0}, p.eps, p.oscale, p.gate_silu, tid);
    if (p.persist) store_tile(s, tile);
}

// The conv prologue of the single-launch decode for (sequence b, qk head j): 16-lane
// rows run the conv + SiLU + L2 norm exactly as conv_silu_norm_kernel does (row 0:
// q_j, row 1: k_j, row 2+n: v of head g*j+n) into LDS and advance the conv history.
// Threads tid >= 16 * (2 + g) do nothing.  slot >= 0.  The loads (taps, history and
// input of the thread's two channel groups) are a step of their own, so a kernel can
// issue them ahead of its state tile and run the conv while the tile streams in.
struct ConvPrologue {
    ConvGroup ga, gb;   // taps loaded; the history is set in the finishing step
    f4 ha[3], hb[3];    // the stored history as loaded (12 floats per channel group)
    f4 xa, xb;
};

__device__ __forceinline__ long long prologue_channel(const FusedParams& p, int j, int tid) {
    const int crow = tid >> 4;
    const int hd = crow == 0 ? j : crow == 1 ? p.h_k + j : 2 * p.h_k + p.group * j + (crow - 2);
    return (long long) hd * kS + 4 * (tid & 15);
}

// (the two steps below run only in threads tid < 16 * (2 + g); the caller checks)
__device__ __forceinline__ void fused_conv_prologue_load(const FusedParams& p, int b, int j, int slot, int tid,
                                                         ConvPrologue& cp) {
    const long long C = (long long) (2 * p.h_k + p.h_v) * kS;
    const long long ca = prologue_channel(p, j, tid);
    const long long cb = ca + 64;
    const float* X = p.conv + (long long) slot * C * kHist;
    const float* xq = p.qkv + (long long) b * C;
    cp.ga.load_taps(p.w, ca);
    cp.gb.load_taps(p.w, cb);
    for (int u = 0; u < 3; ++u) {
        cp.ha[u] = *(const f4*) (X + ca * kHist + 4 * u);
        cp.hb[u] = *(const f4*) (X + cb * kHist + 4 * u);
    }
    cp.xa = *(const f4*) (xq + ca);
    cp.xb = *(const f4*) (xq + cb);
}

__device__ __forceinline__ void fused_conv_prologue_finish(const FusedParams& p, int b, int j, int slot, int tid,
                                                           ConvPrologue& cp, f4* qk_lds, f4 (*v_lds)[32],
                                                           bool store = true) {
    const int crow = tid >> 4;
    const int cl = tid & 15;
    const long long C = (long long) (2 * p.h_k + p.h_v) * kS;
    const long long ca = prologue_channel(p, j, tid);
    const long long cb = ca + 64;
    float* X = p.conv + (long long) slot * C * kHist;
    cp.ga.set_history(cp.ha[0], cp.ha[1], cp.ha[2]);
    cp.gb.set_history(cp.hb[0], cp.hb[1], cp.hb[2]);
    const f4 ua = cp.ga.step(cp.xa);
    const f4 ub = cp.gb.step(cp.xb);
    f4 ha = ua * sigmoid4(ua);
    f4 hb = ub * sigmoid4(ub);
    if (crow < 2) {
        const float ss = add_xor8(block8_sum(sumsq4(ha) + sumsq4(hb)));
        const float sc = (crow == 0 ? p.qscale : 1.0f) / sqrtf(ss + p.eps);
        ha *= sc;
        hb *= sc;
    }
    if (!store) return;
    ConvGroup::store_history(X + ca * kHist, cp.ga.x3, cp.ga.x2, cp.ga.x1);
    ConvGroup::store_history(X + cb * kHist, cp.gb.x3, cp.gb.x2, cp.gb.x1);
    if (p.h) {
        *(f4*) (p.h + (long long) b * C + ca) = ha;
        *(f4*) (p.h + (long long) b * C + cb) = hb;
    }
    f4* dst = crow < 2 ? qk_lds + 32 * crow : v_lds[crow - 2];
    dst[cl] = ha;
    dst[16 + cl] = hb;
}

__device__ __forceinline__ void fused_conv_prologue(const FusedParams& p, int b, int j, int slot, int tid,
                                                    f4* qk_lds, f4 (*v_lds)[32]) {
    if ((tid >> 4) >= 2 + p.group) return;
    ConvPrologue cp;
    fused_conv_prologue_load(p, b, j, slot, tid, cp);
    fused_conv_prologue_finish(p, b, j, slot, tid, cp, qk_lds, v_lds);
}

// Outputs of the single-launch decode for a sequence with an unknown slot: y (and its
// split) of the group's heads and (if asked for) their h channels are zero; the pool
// is untouched.
__device__ __forceinline__ void fused_zero_outputs(const FusedParams& p, int b, int j, int tid, int nthreads) {
    const int g = p.group;
    const long long C = (long long) (2 * p.h_k + p.h_v) * kS;
    const f4 zero = {0.f, 0.f, 0.f, 0.f};
    for (int u = tid; u < g * 32; u += nthreads) {
        if (p.y) *(f4*) (p.y + ((long long) b * p.h_v + g * j + u / 32) * kS + (u % 32) * 4) = zero;
        if (p.ys) ((f4*) p.ys)[split_slot(SplitOut{p.ys, b, p.ys_chunks, g * j + u / 32}, u % 32)] = zero;
    }
    if (p.h)
        for (int u = tid; u < (2 + g) * 32; u += nthreads) {
            const int crow = u / 32;
            const int hd = crow == 0 ? j : crow == 1 ? p.h_k + j : 2 * p.h_k + g * j + (crow - 2);
            *(f4*) (p.h + (long long) b * C + (long long) hd * kS + (u % 32) * 4) = zero;
        }
}

// The whole mixer for one decode token in one launch.  One workgroup per (sequence b,
// qk head j): it owns the conv channels of q_j, k_j and of the group's value heads
// i = g*j .. g*j+g-1 (g = h_v / h_k), so it is the only reader and writer of their conv
// history.  After the conv prologue the g heads run head_token_256 with the fused
// gated RMSNorm.  Results equal gdn_conv_silu_norm followed by gdn_decode_step_norm
// bit for bit.
//
// decode_fused_par_kernel<G> (g = G <= 3): 256 * G threads, one 256-thread group per
// value head, all G heads at once; every group's tile loads are issued before the
// prologue, so the workgroup streams its G tiles together.
template <int G>
__global__ __launch_bounds__(256 * G) void decode_fused_par_kernel(FusedParams p) {
    __shared__ f4 qk_lds[64];
    __shared__ f4 v_lds[G][32];
    __shared__ HeadReduce red[G];

    const int tid = threadIdx.x;
    const int n = tid >> 8;       // value head g*j + n of this thread's group
    const int lt = tid & 255;
    const int cg = lt & 31;
    const int rg = lt >> 5;
    const unsigned nwg = gridDim.x;
    unsigned wid = blockIdx.x;
    if ((nwg & 7u) == 0) wid = (wid & 7u) * (nwg >> 3) + (wid >> 3);
    const int b = (int) (wid / (unsigned) p.h_k);
    const int j = (int) (wid - (unsigned) b * (unsigned) p.h_k);
    // the same in every lane; said so, the branches below are per wave
    const int slot = __builtin_amdgcn_readfirstlane(read_slot(p.slots, b, p.n_slots, p.flags, tid == 0 && j == 0));
    if (slot < 0) {
        fused_zero_outputs(p, b, j, tid, 256 * G);
        return;
    }
    const int i = G * j + n;
    float* tile = p.state + ((long long) slot * p.h_v + i) * (kS * kS) + (rg * 16) * kS + cg * 4;
    // The waves that run the conv (16-lane rows, 2 + G of them) load its inputs first,
    // then their tile rows, and run the conv while the tiles stream in.  The branch is
    // per wave, so no lane waits on another lane's loads; rows past 2 + G load row
    // 0's inputs and store nothing.
    constexpr int kConvWaves = (16 * (2 + G) + 63) / 64;
    f4 s[16];
    if (__builtin_amdgcn_readfirstlane(tid >> 6) < kConvWaves) {
        const int ctid = (tid >> 4) < 2 + G ? tid : (tid & 15);
        ConvPrologue cp;
        fused_conv_prologue_load(p, b, j, slot, ctid, cp);
        load_tile(s, tile);
        fused_conv_prologue_finish(p, b, j, slot, ctid, cp, qk_lds, v_lds, (tid >> 4) < 2 + G);
    } else {
        load_tile(s, tile);
    }
    const long long e = (long long) b * p.h_v + i;
    const float beta_l = p.beta_logit[e], alpha = p.alpha[e], dt = p.dt[i], a = p.ssm_a[i];
    __syncthreads();
    const float beta = sigmoid_f(beta_l);
    const float eg = expf(softplus_f(alpha + dt) * a);
    head_token_256<true>(s, qk_lds, v_lds[n][cg], beta, eg, red[n], nullptr, p.z + e * kS, p.norm_w,
                         p.y ? p.y + e * kS : nullptr, SplitOut{p.ys, b, p.ys_chunks, i}, p.eps, p.oscale,
                         p.gate_silu, lt);
    store_tile(s, tile);
}

// decode_fused_kernel (any g up to kFusedMaxGroup): 256 threads stepping the g heads
// one after another; head 0's tile loads are issued before the prologue, each later
// head's follow the previous head's stores.
__global__ __launch_bounds__(256) void decode_fused_kernel(FusedParams p) {
    __shared__ f4 qk_lds[64];
    __shared__ f4 v_lds[kFusedMaxGroup][32];
    __shared__ HeadReduce red[2];

    const int tid = threadIdx.x;
    const int cg = tid & 31;
    const int rg = tid >> 5;
    const unsigned nwg = gridDim.x;
    unsigned wid = blockIdx.x;
    if ((nwg & 7u) == 0) wid = (wid & 7u) * (nwg >> 3) + (wid >> 3);
    const int b = (int) (wid / (unsigned) p.h_k);
    const int j = (int) (wid - (unsigned) b * (unsigned) p.h_k);
    const int g = p.group;
    const int slot = read_slot(p.slots, b, p.n_slots, p.flags, tid == 0 && j == 0);
    if (slot < 0) {
        fused_zero_outputs(p, b, j, tid, 256);
        return;
    }
    const float* tile_base = p.state + ((long long) slot * p.h_v + g * j) * (kS * kS) + (rg * 16) * kS + cg * 4;
    f4 s[16];
    load_tile(s, tile_base);
    fused_conv_prologue(p, b, j, slot, tid, qk_lds, v_lds);
    __syncthreads();

    for (int n = 0; n < g; ++n) {
        const int i = g * j + n;
        const long long e = (long long) b * p.h_v + i;
        float* tile = (float*) tile_base + (long long) n * (kS * kS);
        if (n > 0) load_tile(s, tile);
        const float beta = sigmoid_f(p.beta_logit[e]);
        const float eg = expf(softplus_f(p.alpha[e] + p.dt[i]) * p.ssm_a[i]);
        head_token_256<true>(s, qk_lds, v_lds[n][cg], beta, eg, red[n & 1], nullptr, p.z + e * kS, p.norm_w,
                             p.y ? p.y + e * kS : nullptr, SplitOut{p.ys, b, p.ys_chunks, i}, p.eps, p.oscale,
                             p.gate_silu, tid);
        store_tile(s, tile);
    }
}

// Multi-token recurrence (T > 1): the state stays in VGPRs for all the call's tokens
// and the per-token chain is what bounds it.  One workgroup of 4 waves per
// (sequence, value head); wave w owns the 32-column block 32w..32w+31 for ALL 128
// rows: lane l has columns 32w + 4*(l % 8) .. +3 of rows 16*(l / 8) .. +15.  The
// column sums then reduce inside the wave (xor-shuffles over the 8 row groups), the
// q/k rows are staged in a wave-private LDS slot, and each token's inputs are
// loaded one token ahead, so the token loop itself has no barrier.  The k and q
// column sums are reduce-scattered, so each lane ends with the sums of one of its 4
// columns (lanes 8..15 of each row repeat lanes 0..7): it forms delta of that column
// and reads it out, and the deltas are gathered back for the update.
// kNorm: each wave parks its o columns in an 8-token LDS ring; every 8 tokens the
// workgroup synchronises once and normalises that chunk cooperatively (thread ->
// token tid/32, columns 4*(tid%32)..+3, the sum of o^2 over a half-wave in the
// single-token kernel's order), with the chunk's z loaded one chunk ahead.
constexpr int kNormChunk = 8;

// Shared memory of one multi-token workgroup.
struct MultiLds {
    f4 qk[4][64];                        // per wave: q as 32 float4, then k as 32 float4
    f4 o_ring[2][kNormChunk][32];        // [chunk parity][token][float4 column group]
    f4 qk_next[4][2][64];                // per wave: q|k of its two tokens of the next chunk
    float kq[2][kNormChunk];             // [chunk parity][token]: k . q of the chunk's tokens
    f2 gate[4][64];                      // per wave: (beta, e^g) of the 64 tokens of a round
};

// A pointer into LDS (address space 3): its integer value is the 32-bit LDS address,
// unlike a generic pointer to shared memory, whose high bits hold the LDS aperture.
template <typename X>
using lds_ptr = __attribute__((address_space(3))) X*;

// A raw buffer descriptor over memory from `base` on (gfx9 data format word); the
// per-token loads and stores below address it with a lane-constant byte offset, so a new
// token moves only the scalar base.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t buffer_at(const void* base) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, -1, 0x00020000);
}
__device__ __forceinline__ f4 buffer_load_f4(const void* base, unsigned byte_off) {
    typedef unsigned u4 __attribute__((ext_vector_type(4)));
    const u4 v = __builtin_amdgcn_raw_buffer_load_b128(buffer_at(base), (int) byte_off, 0, 0);
    return f4{__uint_as_float(v.x), __uint_as_float(v.y), __uint_as_float(v.z), __uint_as_float(v.w)};
}
__device__ __forceinline__ float buffer_load_f1(const void* base, unsigned byte_off) {
    return __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(buffer_at(base), (int) byte_off, 0, 0));
}
__device__ __forceinline__ void buffer_store_f4(f4 v, void* base, unsigned byte_off) {
    typedef unsigned u4 __attribute__((ext_vector_type(4)));
    const u4 u = {__float_as_uint(v.x), __float_as_uint(v.y), __float_as_uint(v.z), __float_as_uint(v.w)};
    __builtin_amdgcn_raw_buffer_store_b128(u, buffer_at(base), (int) byte_off, 0, 0);
}
__device__ __forceinline__ void buffer_store_f1(float v, void* base, unsigned byte_off) {
    __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(v), buffer_at(base), (int) byte_off, 0, 0);
}

// The token loop of the multi-token recurrence for head (job.b, job.i): tokens 0..nt-1
// of the inputs p describes (rows of h, alpha, beta_logit and z of sequence job.b, T
// per sequence), the state in s[] (in and out).  Outputs of tokens nt..T-1 are written
// as zero.  Every thread of the workgroup calls it.
// keep_state = false: the caller discards s[] afterwards (a speculative window), so
// the last token's state update is skipped; its outputs come from the old state in
// the one-pass form, so they do not change.
// The loop runs in rounds of 64 tokens (one evaluation of beta and e^g per lane, parked
// in the wave's LDS) of kNormChunk-token chunks, unrolled, so a token's slots in LDS are
// immediates; the token count and the row bases are wave-uniform, so loop control and
// addressing stay in scalar registers.  With the norm (kNorm), the workgroup meets once
// per chunk anyway, and for a sequence of more than one chunk each wave also forms there
// k . q of two tokens of the next chunk (wave_kq on the same staged rows, so the same
// bits), which the chunk then reads from LDS instead of every wave forming it for every
// token (kChunkKq: the kernels that store the state after long calls; a single chunk
// keeps the per-token form, as the extra round trip before its first token would cost
// more than it saves).
template <bool kNorm, bool kChunkKq>
__device__ __forceinline__ void multi_tokens(const StepParams& p, const HeadJob& job, int nt_in, f4 (&s)[16],
                                             MultiLds& lds, bool keep_state) {
    f4 (&o_ring)[2][kNormChunk][32] = lds.o_ring;

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int cg = lane & 7;
    const int rg = lane >> 3;
    const int col = wave * 32 + cg * 4;
    const int i = job.i;
    const int nt = __builtin_amdgcn_readfirstlane(nt_in);   // one sequence per workgroup
    const long long C = (long long) (2 * p.h_k + p.h_v) * kS;
    const long long tok0 = (long long) job.b * p.T;
    const long long row_hv = (long long) p.h_v * kS;   // one token's o, z or y row
    // the column of its 4 whose q sum a lane ends with after scatter_sum4
    const int oc = (int) (scatter_sum4(f4{0.f, 1.f, 2.f, 3.f}) * 0.25f);
    const bool reads_out = (lane & 8) == 0;
    // The four lanes (lane & 15) + 16 b, b = 0..3, hold the four columns of one group,
    // column oc_b in row pair b.  The deltas are gathered back in column order with LDS
    // permutes (ds_bpermute, no VALU): component k reads the lane of the row pair b_k
    // whose column is k.
    const int oc0 = __builtin_amdgcn_readlane(oc, 0), oc1 = __builtin_amdgcn_readlane(oc, 16),
              oc2 = __builtin_amdgcn_readlane(oc, 32);
    auto src_of = [&](int k) {
        const int b = oc0 == k ? 0 : oc1 == k ? 1 : oc2 == k ? 2 : 3;
        return ((lane & 15) | (b << 4)) << 2;
    };
    const int gsrc0 = src_of(0), gsrc1 = src_of(1), gsrc2 = src_of(2), gsrc3 = src_of(3);
    auto gather_d = [&](float v) {
        const int x = __float_as_int(v);
        return f4{__int_as_float(__builtin_amdgcn_ds_bpermute(gsrc0, x)),
                  __int_as_float(__builtin_amdgcn_ds_bpermute(gsrc1, x)),
                  __int_as_float(__builtin_amdgcn_ds_bpermute(gsrc2, x)),
                  __int_as_float(__builtin_amdgcn_ds_bpermute(gsrc3, x))};
    };
    // byte offsets inside one token's row of h, and of o
    const unsigned q_off = 4u * (unsigned) (job.j * kS + (lane & 31) * 4 + (lane < 32 ? 0 : p.h_k * kS));
    const unsigned v_off = 4u * (unsigned) ((2 * p.h_k + i) * kS + col + oc);
    const unsigned o_off = 4u * (unsigned) (col + oc);
    const float* h_seq = p.h + tok0 * C;
    float* o_seq = p.o ? p.o + (tok0 * p.h_v + i) * kS : nullptr;
    // chunk normalisation: this thread's token within a chunk and columns
    const int n_tt = tid >> 5;
    const int n_c4 = (tid & 31) * 4;
    const float* z_seq = kNorm ? p.z + (tok0 * p.h_v + i) * kS : nullptr;
    float* y_seq = kNorm ? p.y + (tok0 * p.h_v + i) * kS : nullptr;
    const unsigned zy_off = 4u * (unsigned) n_c4;

    const float dt_i = p.dt[i];
    const float a_i = p.ssm_a[i];
    const int last = nt - 1;
    const bool chunk_kq_on = kNorm && kChunkKq && nt > kNormChunk;   // uniform over the workgroup

    // q|k and v of the next token, loaded one token ahead (past the last token: the
    // last token's row again, so no branch sits around the loads)
    f4 qk_n = {0.f, 0.f, 0.f, 0.f};
    float v_n = 0.f;   // v of the one column (col + oc) whose delta this lane forms
    auto fetch = [&](int t) {
        const float* ht = h_seq + min(t, last) * C;
        qk_n = buffer_load_f4(ht, q_off);
        v_n = buffer_load_f1(ht, v_off);
    };
    // z of this thread's token in the chunk after the current one, loaded one chunk ahead
    f4 z_n = {0.f, 0.f, 0.f, 0.f};
    auto fetch_z = [&](int t0c) { z_n = buffer_load_f4(z_seq + min(t0c + n_tt, last) * row_hv, zy_off); };
    // q|k of this wave's two tokens (2 wave, 2 wave + 1) of the chunk after the current one
    f4 qkp0 = {0.f, 0.f, 0.f, 0.f}, qkp1 = qkp0;
    auto fetch_qkp = [&](int t0c) {
        qkp0 = buffer_load_f4(h_seq + min(t0c + 2 * wave, last) * C, q_off);
        qkp1 = buffer_load_f4(h_seq + min(t0c + 2 * wave + 1, last) * C, q_off);
    };
    // k . q of those two tokens, into kq[par]; the caller's barrier publishes them
    auto chunk_kq = [&](int par) {
        lds.qk_next[wave][0][lane] = qkp0;
        lds.qk_next[wave][1][lane] = qkp1;
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
        const float k0 = wave_kq((const float*) lds.qk_next[wave][0], lane);
        const float k1 = wave_kq((const float*) lds.qk_next[wave][1], lane);
        if (lane == 0) {
            lds.kq[par][2 * wave] = k0;
            lds.kq[par][2 * wave + 1] = k1;
        }
    };
    // the gated RMSNorm of the first n tokens of the chunk that starts at token tc, from
    // o parked in ring parity par; z of the chunk is in zz
    auto norm_chunk = [&](int tc, int par, int n, f4 zz) {
        if (n_tt < n) {   // whole half-waves, as halfwave_sum needs
            const f4 o4 = o_ring[par][n_tt][n_c4 / 4];
            const float inv = rms_inv(halfwave_sum(sumsq4(o4)), p.eps);
            const f4 wn = *(const f4*) (p.norm_w + n_c4);
            buffer_store_f4(o4 * inv * wn * gate4(zz, p.gate_silu), y_seq + (tc + n_tt) * row_hv, zy_off);
        }
    };
    if (nt > 0) {
        fetch(0);
        if (kNorm) fetch_z(0);
        if (chunk_kq_on) {
            fetch_qkp(0);
            chunk_kq(0);
            fetch_qkp(kNormChunk);
            __syncthreads();
        }
    }

    f4* buf = lds.qk[wave];
    const float* qrow = (const float*) buf + rg * 16;
    const float* krow = (const float*) buf + kS + rg * 16;
    const float* ring_lane = (const float*) o_ring + wave * 32 + cg * 4 + oc;
    for (int tg = 0; tg < nt; tg += 64) {
        // beta and the decay e^g are the same for the whole head: lane l evaluates them
        // for token tg + l into the wave's LDS, and each token reads its pair back
        {
            f2 ge = {0.f, 0.f};
            if (tg + lane < nt) {
                const long long e = (tok0 + tg + lane) * p.h_v + i;
                ge.x = sigmoid_f(p.beta_logit[e]);
                ge.y = expf(softplus_f(p.alpha[e] + dt_i) * a_i);
            }
            lds.gate[wave][lane] = ge;
            __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
            __builtin_amdgcn_wave_barrier();
            __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
        }
        const int tg_end = min(tg + 64, nt);
        for (int tc = tg; tc < tg_end; tc += kNormChunk) {
            const int par = (tc / kNormChunk) & 1;
            // this chunk's LDS slots, as 32-bit LDS addresses held in registers once per
            // chunk (the tokens then address them with immediate offsets)
            unsigned ring_addr = (unsigned) (size_t) (lds_ptr<float>) (ring_lane + par * (kNormChunk * 128));
            unsigned gate_addr = (unsigned) (size_t) (lds_ptr<f2>) &lds.gate[wave][tc - tg];
            unsigned kq_addr = (unsigned) (size_t) (lds_ptr<float>) &lds.kq[par][0];
            asm volatile("" : "+v"(ring_addr), "+v"(gate_addr), "+v"(kq_addr));
            const lds_ptr<float> ring_par = (lds_ptr<float>) (size_t) ring_addr;
            const lds_ptr<f2> gate_c = (lds_ptr<f2>) (size_t) gate_addr;
            const lds_ptr<float> kq_c = (lds_ptr<float>) (size_t) kq_addr;
            int u = 0;
#pragma unroll
            for (; u < kNormChunk; ++u) {
                const int t = tc + u;
                if (t >= tg_end) break;   // uniform: only the last chunk stops early
                __builtin_amdgcn_sched_barrier(0);
                const f2 ge = gate_c[u];
                const float beta = ge.x, eg = ge.y;
                buf[lane] = qk_n;
                const float vc = v_n;
                fetch(t + 1);
                // the staging above is wave-private: order it against this wave's reads
                __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
                __builtin_amdgcn_wave_barrier();
                __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");

                f4 pk = {0.f, 0.f, 0.f, 0.f}, pq = pk;
#pragma unroll
                for (int m = 0; m < 16; ++m) {
                    pk = fma4(s[m], krow[m], pk);
                    pq = fma4(s[m], qrow[m], pq);
                }
                const float kq = chunk_kq_on ? kq_c[u] : wave_kq((const float*) buf, lane);
                // column sums over the 8 row groups of the wave (lane bits 3..5):
                // ((g0+g1)+(g2+g3))+((g4+g5)+(g6+g7)), as in the single-token kernel
                const float pkc = scatter_sum4(add_xor8(pk));
                const float pqc = scatter_sum4(add_xor8(pq));
                // delta and readout of column col + oc (the readout scale, when there is
                // one, multiplies after the sum as in the single-token kernel)
                const float dc = beta * __builtin_fmaf(-eg, pkc, vc);
                float out = __builtin_fmaf(kq, dc, eg * pqc);
                if (p.oscale != 1.0f) out *= p.oscale;
                // the deltas of all 4 columns for the update
                const f4 d = gather_d(dc);
                if (o_seq && reads_out) buffer_store_f1(out, o_seq + t * row_hv, o_off);
                if (kNorm) {
                    if (reads_out) ring_par[u * 128] = out;
                    if (u == kNormChunk - 1) {   // a whole chunk: its norm, and k . q of the next
                        const f4 zz = z_n;
                        fetch_z(tc + kNormChunk);
                        if (chunk_kq_on) {
                            chunk_kq(par ^ 1);
                            fetch_qkp(tc + 2 * kNormChunk);
                        }
                        __syncthreads();
                        norm_chunk(tc, par, kNormChunk, zz);
                    }
                }
                if (keep_state || t < last) {
                    // re-read k from LDS rather than keeping 16 rows live across the
                    // reduction (the fence stops the compiler from reusing the values
                    // loaded above)
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
            }
            // the last chunk of the call, cut short: its norm
            if (kNorm && u < kNormChunk) {
                __syncthreads();
                norm_chunk(tc, par, u, z_n);
            }
        }
    }
    if (rg == 0) {
        const f4 zero = {0.f, 0.f, 0.f, 0.f};
        for (int t = nt; t < p.T; ++t) {
            const long long e = ((tok0 + t) * p.h_v + i) * kS + col;
            if (p.o) *(f4*) (p.o + e) = zero;
            if (kNorm) *(f4*) (p.y + e) = zero;
        }
    }
}

// kKeep: the state is stored at the end (p.persist); a speculative window (kKeep false,
// always with the norm) stores nothing and skips its last token's update.
template <bool kNorm, bool kKeep>
__global__ __launch_bounds__(256) void decode_multi_kernel(StepParams p) {
    __shared__ MultiLds lds;
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int rg = lane >> 3;
    const int col = wave * 32 + (lane & 7) * 4;
    const HeadJob job = head_job(p, tid == 0);
    const int i = job.i;
    const int nt = job.nt;
    const long long C = (long long) (2 * p.h_k + p.h_v) * kS;
    const long long tok0 = (long long) job.b * p.T;
    float* tile = nullptr;
    f4 s[16];
    if (nt > 0) {
        tile = p.state + ((long long) job.slot * p.h_v + i) * (kS * kS) + (rg * 16) * kS + col;
#pragma unroll
        for (int m = 0; m < 16; ++m) s[m] = __builtin_nontemporal_load((const f4*) (tile + m * kS));
    }
    if (p.conv && nt > 0 && tid < 96) {
        // commit: while the tile loads, advance the conv history by the nt kept rows,
        // v of this head by every workgroup, q and k of the qk head by the group's
        // first value head only (no other workgroup touches those channels)
        const int part = tid >> 5;   // 0: v of head i, 1: q_j, 2: k_j
        if (part == 0 || i % p.group == 0) {
            const long long head = part == 0 ? 2 * p.h_k + i : part == 1 ? job.j : p.h_k + job.j;
            advance_history(p.conv + (long long) job.slot * C * kHist, p.adv_qkv + tok0 * C, C,
                            head * kS + 4 * (tid & 31), nt);
        }
    }
    multi_tokens<kNorm, kNorm && kKeep>(p, job, nt, s, lds, kKeep);
    if (nt > 0 && kKeep) store_tile(s, tile);
}

// A commit and the next speculative window in one launch, for a decode loop that
// verifies the next drafts right after accepting the last ones.  One workgroup per
// (sequence, value head) reads its state tile once, replays the previous window's
// n_keep accepted tokens from that window's h (com: the commit, no outputs), stores
// the committed tile, and runs the next window's tokens from it in registers (win:
// y out, nothing stored).  The conv launch before this one advanced the history by
// the kept rows and computed the next window's h from it.  With the same token loop
// the results equal gdn_commit followed by gdn_verify_window bit for bit, at one state
// read per round instead of two.
__global__ __launch_bounds__(256) void commit_window_kernel(StepParams com, StepParams win) {
    __shared__ MultiLds lds;
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int rg = lane >> 3;
    const int col = (tid >> 6) * 32 + (lane & 7) * 4;
    const HeadJob job = head_job(win, tid == 0);   // the slot and the window's token count
    const int nk = job.slot < 0 ? 0 : read_ntok(com.n_tok, job.b, com.T, win.flags, tid == 0 && job.i == 0);
    float* tile = nullptr;
    f4 s[16];
    if (nk > 0 || job.nt > 0) {
        tile = win.state + ((long long) job.slot * win.h_v + job.i) * (kS * kS) + (rg * 16) * kS + col;
        load_tile(s, tile);
    }
    if (nk > 0) {
        multi_tokens<false, false>(com, job, nk, s, lds, true);
        store_tile(s, tile);
    }
    multi_tokens<true, false>(win, job, job.nt, s, lds, false);
}

// ------------------------------------------------------------------ launch
hipError_t launch_decode_fused(const FusedParams& p, hipStream_t stream) {
    const dim3 grid((unsigned) ((long long) p.B * p.h_k));
    switch (p.group) {
    case 1: hipLaunchKernelGGL(decode_fused_par_kernel<1>, grid, dim3(256), 0, stream, p); break;
    case 2: hipLaunchKernelGGL(decode_fused_par_kernel<2>, grid, dim3(512), 0, stream, p); break;
    case 3: hipLaunchKernelGGL(decode_fused_par_kernel<3>, grid, dim3(768), 0, stream, p); break;
    default: hipLaunchKernelGGL(decode_fused_kernel, grid, dim3(256), 0, stream, p); break;
    }
    return hipGetLastError();
}

hipError_t launch_commit_window(const StepParams& com, const StepParams& win, hipStream_t stream) {
    hipLaunchKernelGGL(commit_window_kernel, dim3((unsigned) ((long long) win.B * win.h_v)), dim3(256), 0, stream,
                       com, win);
    return hipGetLastError();
}

hipError_t launch_decode_step(const StepParams& p, hipStream_t stream) {
    const dim3 grid((unsigned) ((long long) p.B * p.h_v));
    const bool one = p.T == 1 && !p.conv;   // the commit's history advance lives in the multi-token kernel
    if (!p.y && !p.persist) return hipErrorInvalidValue;   // no caller leaves both out
    if (p.y) {
        if (one) hipLaunchKernelGGL((decode_one_kernel<true>), grid, dim3(256), 0, stream, p);
        else if (p.persist) hipLaunchKernelGGL((decode_multi_kernel<true, true>), grid, dim3(256), 0, stream, p);
        else hipLaunchKernelGGL((decode_multi_kernel<true, false>), grid, dim3(256), 0, stream, p);
    } else {
        if (one) hipLaunchKernelGGL((decode_one_kernel<false>), grid, dim3(256), 0, stream, p);
        else hipLaunchKernelGGL((decode_multi_kernel<false, true>), grid, dim3(256), 0, stream, p);
    }
    return hipGetLastError();
}

}  // namespace gdn
