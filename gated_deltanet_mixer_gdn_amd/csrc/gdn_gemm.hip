// gdn_gemm.hip - the dense projections either side of the mixer: qkv = wqkv x and
// z = attn_gate x before it, out = ssm_out y after it (steps 2, 7 and 8 of
// `gdn_layer` on the "src/core/layer.cpp" page), as plain products with bf16
// weights:
//
//   out[r][j] = sum_e w[j][e] * x[r][e]     x [rows][k] fp32, w [n][k] bf16
//
// At a decode batch this is the one dense contraction around the mixer (rows =
// sequences, k and n in the thousands), so it runs on the matrix cores with
// v_mfma_f32_32x32x16_bf16.  The activations are not rounded to bf16: a first
// pass splits each fp32 value into hi = bf16(x) and lo = bf16(x - hi), and every
// weight tile meets both halves, so the product carries x to within 2^-16 |x|
// and sums in fp32.  The split runs once per activation matrix and serves every
// projection that reads it (qkv and z read the same x), the way the pages'
// engine converts an activation once for the GEMVs that follow.
#include <hip/hip_runtime.h>

#include "gdn_bf16.h"
#include "gdn_gemm.h"

namespace gdn {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f16v __attribute__((ext_vector_type(16)));
typedef float f4v __attribute__((ext_vector_type(4)));
typedef unsigned u4v __attribute__((ext_vector_type(4)));

// ------------------------------------------------------------------ split and pack
// One thread per fragment position (tile, step, lane) of the output layout, so the
// writes of a wave are contiguous; positions outside [rows] x [k] are written as zeros.
__global__ __launch_bounds__(256) void split_bf16_kernel(SplitParams p) {
    const int n_chunks = (int) (pad_up(p.k, kTileK) / kTileK);
    const long long total = pad_up(p.rows, kTileRows) / kTileRows * n_chunks * 256;
    const long long stride = (long long) gridDim.x * blockDim.x;
    for (long long f = (long long) blockIdx.x * blockDim.x + threadIdx.x; f < total; f += stride) {
        const long long tile = f >> 8;
        const int s = (int) (f >> 6) & 3, lane = (int) f & 63;
        const long long row = tile / n_chunks * kTileRows + (lane & 31);
        const int kk = (int) (tile % n_chunks) * kTileK + 32 * (lane >> 5) + 8 * s;
        u4v H = {0u, 0u, 0u, 0u}, L = H;
        if (row < p.rows && kk < p.k) {
            const float* src = p.x + row * p.k + kk;
            const f4v a = *(const f4v*) src;
            const f4v b = *(const f4v*) (src + 4);
            const float v[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
            unsigned hi[8], lo[8];
#pragma unroll
            for (int j = 0; j < 8; ++j) split_bf16(v[j], hi[j], lo[j]);
            H = u4v{hi[0] | hi[1] << 16, hi[2] | hi[3] << 16, hi[4] | hi[5] << 16, hi[6] | hi[7] << 16};
            L = u4v{lo[0] | lo[1] << 16, lo[2] | lo[3] << 16, lo[4] | lo[5] << 16, lo[6] | lo[7] << 16};
        }
        u4v* dst = (u4v*) p.xs + tile * 512 + lane;
        dst[(2 * s) * 64] = H;
        dst[(2 * s + 1) * 64] = L;
    }
}

__global__ __launch_bounds__(256) void pack_bf16_kernel(PackParams p) {
    const int n_chunks = (int) (pad_up(p.k, kTileK) / kTileK);
    const long long total = pad_up(p.n, kTileRows) / kTileRows * n_chunks * 256;
    const long long stride = (long long) gridDim.x * blockDim.x;
    for (long long f = (long long) blockIdx.x * blockDim.x + threadIdx.x; f < total; f += stride) {
        const long long tile = f >> 8;
        const int lane = (int) f & 63;
        const long long col = tile / n_chunks * kTileRows + (lane & 31);
        const int kk = (int) (tile % n_chunks) * kTileK + 32 * (lane >> 5) + 8 * ((int) (f >> 6) & 3);
        u4v v = {0u, 0u, 0u, 0u};
        if (col < p.n && kk < p.k) v = *(const u4v*) (p.w + col * p.k + kk);
        ((u4v*) p.wp)[f] = v;
    }
}

// ------------------------------------------------------------------ projection
//
// Workgroup = 4 waves; wave (wn, wk) computes the (32 WM) x (32 WN) block of out at
// rows m0.., columns n0 + wn*32*WN.., over the k chunks c = wk, wk + KW, ... of the
// tiled operands.  Per chunk a lane loads, for each of its WM row tiles, the hi and
// lo fragment of each of the 4 steps and, for each of its WN column tiles, the
// weight fragment of each step: every load instruction reads 1 KiB of contiguous
// memory.  Accumulator element e of lane (i, h) holds out row 8(e/4) + 4h + e%4,
// column i of the block.  The next chunk is loaded while the current one runs
// (two register sets, loads issued unconditionally so the waits count exactly).
// Waves that split k add their partial blocks through LDS in a fixed order
// (wk = 0, 1, ...), so results do not depend on timing.  Row and column tiles past
// the padded operands are clamped to the last one; their outputs are not stored.
// Workgroups are dispatched to the 8 XCDs round robin; give each XCD a contiguous
// run of tiles, in which the row blocks of one column tile are neighbours and share
// their weight tiles in that XCD's L2.
__device__ __forceinline__ int xcd_tile(int b, int tiles_total) {
    const int per = tiles_total >> 3, extra = tiles_total & 7, xcd = b & 7;
    return xcd * per + min(xcd, extra) + (b >> 3);
}

// Accumulator element e of lane (i, h) holds row 8(e/4) + 4h + e%4, column i of its
// 32 x 32 block; rows past p.rows and columns past p.n are not stored.  The output a
// column belongs to is picked with selects on the uniform range bounds (no indexed
// access to the parameter block).
template <int WM, int WN>
__device__ __forceinline__ void store_blocks(const GemmParams& p, const f16v (&acc)[WM][WN], long long m0, int n0,
                                             int i, int h) {
#pragma unroll
    for (int r = 0; r < WM; ++r)
#pragma unroll
        for (int c = 0; c < WN; ++c) {
            const int col = n0 + 32 * c + i;
            if (col >= p.n) continue;
            float* base = p.out[0];
            int lo = 0, hi = p.c0[1];
#pragma unroll
            for (int o = 1; o < kMaxOuts; ++o)
                if (col >= p.c0[o]) {
                    base = p.out[o];
                    lo = p.c0[o];
                    hi = p.c0[o + 1];
                }
            float* dst = base + (col - lo);
            const long long ld = hi - lo;
#pragma unroll
            for (int e = 0; e < 16; ++e) {
                const long long row = m0 + 32 * r + 8 * (e >> 2) + 4 * h + (e & 3);
                if (row < p.rows) dst[row * ld] = acc[r][c][e];
            }
        }
}

template <int WM, int WN>
struct Frag {
    bf16x8 a[WM][4][2];  // [row tile][step][hi, lo]
    bf16x8 b[WN][4];     // [column tile][step]
};

template <int WM, int WN, int KW>
__global__ __launch_bounds__(256) void project_bf16_kernel(GemmParams p, int tiles_m, int tiles_total, int n_chunks) {
    constexpr int kWavesN = 4 / KW;
    constexpr int BM = 32 * WM;
    constexpr int BN = 32 * WN * kWavesN;
    const int wave = threadIdx.x >> 6;
    const int lane = threadIdx.x & 63;
    const int i = lane & 31;
    const int h = lane >> 5;
    const int wn = wave % kWavesN;
    const int wk = wave / kWavesN;

    // with parts > 1 the grid holds parts x tiles_total workgroups, range-major, so
    // the workgroups on one XCD share a k range and its activation tiles
    const int tq = xcd_tile(blockIdx.x, tiles_total * p.parts);
    const int q = tq / tiles_total;
    const int t = tq - q * tiles_total;
    const int tm = t % tiles_m;
    const int tn = t / tiles_m;
    const long long m0 = (long long) tm * BM;
    const int n0 = tn * BN + wn * 32 * WN;
    const long long last_rt = (p.rows + kTileRows - 1) / kTileRows - 1;
    const int last_ct = (p.n + kTileRows - 1) / kTileRows - 1;
    const int c_first = (int) ((long long) q * n_chunks / p.parts);
    const int c_count = (int) ((long long) (q + 1) * n_chunks / p.parts) - c_first;

    const bf16x8* abase[WM];
#pragma unroll
    for (int r = 0; r < WM; ++r) {
        const long long rt = min((long long) tm * WM + r, last_rt);
        abase[r] = (const bf16x8*) p.xs + rt * n_chunks * 512 + lane;
    }
    const bf16x8* bbase[WN];
#pragma unroll
    for (int c = 0; c < WN; ++c) {
        const long long ct = min(n0 / 32 + c, last_ct);
        bbase[c] = (const bf16x8*) p.wp + ct * n_chunks * 256 + lane;
    }

    auto load = [&](int ch, Frag<WM, WN>& f) {
#pragma unroll
        for (int s = 0; s < 4; ++s) {
#pragma unroll
            for (int r = 0; r < WM; ++r) {
                f.a[r][s][0] = abase[r][ch * 512 + (2 * s) * 64];
                f.a[r][s][1] = abase[r][ch * 512 + (2 * s + 1) * 64];
            }
#pragma unroll
            for (int c = 0; c < WN; ++c) f.b[c][s] = bbase[c][ch * 256 + s * 64];
        }
    };

    f16v acc[WM][WN];
#pragma unroll
    for (int r = 0; r < WM; ++r)
#pragma unroll
        for (int c = 0; c < WN; ++c) acc[r][c] = f16v{};
    auto compute = [&](const Frag<WM, WN>& f) {
#pragma unroll
        for (int s = 0; s < 4; ++s)
#pragma unroll
            for (int r = 0; r < WM; ++r)
#pragma unroll
                for (int c = 0; c < WN; ++c) {
                    acc[r][c] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(f.a[r][s][0], f.b[c][s], acc[r][c], 0, 0, 0);
                    acc[r][c] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(f.a[r][s][1], f.b[c][s], acc[r][c], 0, 0, 0);
                }
    };

    // Two chunks per trip: f0 holds chunk it on entry, f1 is loaded while f0 runs and
    // f0 reloaded while f1 runs.  The scheduling barriers keep the compiler from
    // sinking the loads of the next chunk down to their first use.
    const int cnt = wk < c_count ? (c_count - wk + KW - 1) / KW : 0;
    const int c0 = c_first + wk;
    if (cnt > 0) {
        Frag<WM, WN> f0, f1;
        load(c0, f0);
        int it = 0;
        for (; it + 2 <= cnt; it += 2) {
            load(c0 + KW * (it + 1), f1);
            __builtin_amdgcn_sched_barrier(0);
            compute(f0);
            __builtin_amdgcn_sched_barrier(0);
            load(c0 + KW * min(it + 2, cnt - 1), f0);
            __builtin_amdgcn_sched_barrier(0);
            compute(f1);
            __builtin_amdgcn_sched_barrier(0);
        }
        if (it < cnt) compute(f0);
    }

    if constexpr (KW > 1) {
        constexpr int kVals = WM * WN * 16;
        __shared__ float red[(KW - 1) * kWavesN * kVals * 64];
        if (wk > 0) {
            float* dst = red + ((wk - 1) * kWavesN + wn) * kVals * 64 + lane;
#pragma unroll
            for (int r = 0; r < WM; ++r)
#pragma unroll
                for (int c = 0; c < WN; ++c)
#pragma unroll
                    for (int e = 0; e < 16; ++e) dst[((r * WN + c) * 16 + e) * 64] = acc[r][c][e];
        }
        __syncthreads();
        if (wk > 0) return;
#pragma unroll
        for (int j = 1; j < KW; ++j) {
            const float* src = red + ((j - 1) * kWavesN + wn) * kVals * 64 + lane;
#pragma unroll
            for (int r = 0; r < WM; ++r)
#pragma unroll
                for (int c = 0; c < WN; ++c)
#pragma unroll
                    for (int e = 0; e < 16; ++e) acc[r][c][e] += src[((r * WN + c) * 16 + e) * 64];
        }
    }

    if constexpr (KW == 4) {
        if (p.parts > 1) {
            // one wave per workgroup is left: its block is this k range's partial sum
            float* dst = p.ws + ((long long) t * p.parts + q) * (WM * WN * 16 * 64) + lane;
#pragma unroll
            for (int r = 0; r < WM; ++r)
#pragma unroll
                for (int c = 0; c < WN; ++c)
#pragma unroll
                    for (int e = 0; e < 16; ++e) dst[((r * WN + c) * 16 + e) * 64] = acc[r][c][e];
            return;
        }
    }

    store_blocks<WM, WN>(p, acc, m0, n0, i, h);
}

// Second pass of a k-split launch: one wave per tile adds the tile's partial blocks
// in range order 0, 1, ..., parts - 1 (a fixed order) and stores the tile.
template <int WM, int WN>
__global__ __launch_bounds__(256) void add_parts_kernel(GemmParams p, int tiles_m, int tiles_total) {
    const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
    if (t >= tiles_total) return;
    const int lane = threadIdx.x & 63;
    constexpr int kBlk = WM * WN * 16 * 64;
    const float* src = p.ws + (long long) t * p.parts * kBlk + lane;
    f16v acc[WM][WN];
#pragma unroll
    for (int r = 0; r < WM; ++r)
#pragma unroll
        for (int c = 0; c < WN; ++c)
#pragma unroll
            for (int e = 0; e < 16; ++e) acc[r][c][e] = src[((r * WN + c) * 16 + e) * 64];
    for (int j = 1; j < p.parts; ++j)
#pragma unroll
        for (int r = 0; r < WM; ++r)
#pragma unroll
            for (int c = 0; c < WN; ++c)
#pragma unroll
                for (int e = 0; e < 16; ++e) acc[r][c][e] += src[j * kBlk + ((r * WN + c) * 16 + e) * 64];
    store_blocks<WM, WN>(p, acc, (long long) (t % tiles_m) * 32 * WM, t / tiles_m * 32 * WN, lane & 31, lane >> 5);
}

// The same product with the activation tiles shared through LDS: a workgroup of
// 4 * KG waves, 4 side by side in n and KG groups that take alternate k chunks.  Each
// chunk's WM activation tiles (8 KiB each) are read from memory once per group, by
// its 256 threads with contiguous 16-byte loads, and every wave of the group takes
// its fragments from LDS (lane-order 16-byte reads, no bank conflicts).  Two LDS
// buffers per group alternate; the next chunk's activation share and weight
// fragments are loaded while the current chunk runs and the share is written to
// the other buffer after it.  With KG = 2 the second group's partial blocks are
// added to the first's through LDS at the end (group 0 first, a fixed order).
template <int WM, int WN, int KG>
__global__ __launch_bounds__(256 * KG) void project_lds_kernel(GemmParams p, int tiles_m, int tiles_total,
                                                               int n_chunks) {
    constexpr int BM = 32 * WM;
    constexpr int BN = 128 * WN;
    constexpr int kAbufU4 = 2 * WM * 512;                 // per group
    constexpr int kRedU4 = KG > 1 ? 4 * WM * WN * 16 * 16 : 0;   // 4 waves x acc floats / 4
    constexpr int kLdsU4 = KG * kAbufU4 > kRedU4 ? KG * kAbufU4 : kRedU4;
    __shared__ u4v lds[kLdsU4];
    const int gtid = threadIdx.x;
    const int kg = gtid >> 8;            // k group
    const int tid = gtid & 255;          // thread within the group
    const int wave = tid >> 6;
    const int lane = tid & 63;
    const int i = lane & 31;
    const int h = lane >> 5;
    u4v* abuf = lds + kg * kAbufU4;      // [2][WM][512]

    const int t = xcd_tile(blockIdx.x, tiles_total);
    const int tm = t % tiles_m;
    const int tn = t / tiles_m;
    const long long m0 = (long long) tm * BM;
    const int n0 = tn * BN + wave * 32 * WN;
    const long long last_rt = (p.rows + kTileRows - 1) / kTileRows - 1;
    const int last_ct = (p.n + kTileRows - 1) / kTileRows - 1;

    const u4v* asrc[WM];
#pragma unroll
    for (int r = 0; r < WM; ++r) {
        const long long rt = min((long long) tm * WM + r, last_rt);
        asrc[r] = (const u4v*) p.xs + rt * n_chunks * 512 + tid;
    }
    const bf16x8* bbase[WN];
#pragma unroll
    for (int c = 0; c < WN; ++c) {
        const long long ct = min(n0 / 32 + c, last_ct);
        bbase[c] = (const bf16x8*) p.wp + ct * n_chunks * 256 + lane;
    }

    struct BFrag {
        bf16x8 b[WN][4];
    };
    u4v ash[WM][2];
    auto load_a = [&](int ch) {
#pragma unroll
        for (int r = 0; r < WM; ++r) {
            ash[r][0] = asrc[r][ch * 512];
            ash[r][1] = asrc[r][ch * 512 + 256];
        }
    };
    auto store_a = [&](int buf) {
#pragma unroll
        for (int r = 0; r < WM; ++r) {
            abuf[(buf * WM + r) * 512 + tid] = ash[r][0];
            abuf[(buf * WM + r) * 512 + tid + 256] = ash[r][1];
        }
    };
    auto load_b = [&](int ch, BFrag& f) {
#pragma unroll
        for (int s = 0; s < 4; ++s)
#pragma unroll
            for (int c = 0; c < WN; ++c) f.b[c][s] = bbase[c][ch * 256 + s * 64];
    };

    f16v acc[WM][WN];
#pragma unroll
    for (int r = 0; r < WM; ++r)
#pragma unroll
        for (int c = 0; c < WN; ++c) acc[r][c] = f16v{};
    auto compute = [&](int buf, const BFrag& f) {
#pragma unroll
        for (int s = 0; s < 4; ++s) {
            bf16x8 a[WM][2];
#pragma unroll
            for (int r = 0; r < WM; ++r) {
                a[r][0] = __builtin_bit_cast(bf16x8, abuf[(buf * WM + r) * 512 + (2 * s) * 64 + lane]);
                a[r][1] = __builtin_bit_cast(bf16x8, abuf[(buf * WM + r) * 512 + (2 * s + 1) * 64 + lane]);
            }
#pragma unroll
            for (int r = 0; r < WM; ++r)
#pragma unroll
                for (int c = 0; c < WN; ++c) {
                    acc[r][c] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[r][0], f.b[c][s], acc[r][c], 0, 0, 0);
                    acc[r][c] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[r][1], f.b[c][s], acc[r][c], 0, 0, 0);
                }
        }
    };

    // Group kg takes chunks kg, kg + KG, ...; its j-th chunk lives in its buffer j % 2
    // and f0 / f1 hold the weight fragments of its even / odd ones.  Every group runs
    // the same number of trips (a group past its last chunk reloads that chunk and
    // skips the arithmetic) so all waves meet at the same barriers; every load is
    // issued unconditionally so the compiler's wait counts stay exact.
    const int cnt = (n_chunks + KG - 1) / KG;                   // trips of the longest group
    const int mine = (n_chunks - kg + KG - 1) / KG;              // chunks of this group (>= cnt - 1)
    auto chunk = [&](int j) { return mine > 0 ? kg + KG * min(j, mine - 1) : 0; };
    BFrag f0, f1;
    load_a(chunk(0));
    load_b(chunk(0), f0);
    store_a(0);
    __syncthreads();
    int j = 0;
    for (; j + 2 <= cnt; j += 2) {
        load_a(chunk(j + 1));
        load_b(chunk(j + 1), f1);
        __builtin_amdgcn_sched_barrier(0);
        if (j < mine) compute(0, f0);
        store_a(1);
        __syncthreads();
        load_a(chunk(j + 2));
        load_b(chunk(j + 2), f0);
        __builtin_amdgcn_sched_barrier(0);
        if (j + 1 < mine) compute(1, f1);
        store_a(0);
        __syncthreads();
    }
    if (j < cnt && j < mine) compute(0, f0);

    if constexpr (KG > 1) {
        // group 1 hands its partial blocks to group 0 (the A buffers are free now)
        __syncthreads();
        float* red = (float*) lds + wave * (WM * WN * 16 * 64) + lane;
        if (kg == 1) {
#pragma unroll
            for (int r = 0; r < WM; ++r)
#pragma unroll
                for (int c = 0; c < WN; ++c)
#pragma unroll
                    for (int e = 0; e < 16; ++e) red[((r * WN + c) * 16 + e) * 64] = acc[r][c][e];
        }
        __syncthreads();
        if (kg == 1) return;
#pragma unroll
        for (int r = 0; r < WM; ++r)
#pragma unroll
            for (int c = 0; c < WN; ++c)
#pragma unroll
                for (int e = 0; e < 16; ++e) acc[r][c][e] += red[((r * WN + c) * 16 + e) * 64];
    }
    store_blocks<WM, WN>(p, acc, m0, n0, i, h);
}

// The LDS-shared tile with a deeper pipeline: the 4 waves sit side by side in n, the
// chunk's WM activation tiles go through a ring of three LDS buffers (written once
// per workgroup) and each wave keeps a ring of three register sets of weight
// fragments, so two chunks are in flight while a third is multiplied.  Chunk c lives
// in LDS buffer c % 3 and register set c % 3; the activation share of chunk c + 1 is
// written to LDS after chunk c has been multiplied, one barrier per chunk.  Loads past
// the last chunk reload the last one (never used), so every load is unconditional.
template <int WM, int WN>
__global__ __launch_bounds__(256) void project_ring_kernel(GemmParams p, int tiles_m, int tiles_total, int n_chunks) {
    constexpr int BM = 32 * WM;
    constexpr int BN = 128 * WN;
    __shared__ u4v abuf[3][WM][512];
    const int tid = threadIdx.x;
    const int wave = tid >> 6;
    const int lane = tid & 63;
    const int i = lane & 31;
    const int h = lane >> 5;

    const int t = xcd_tile(blockIdx.x, tiles_total);
    const int tm = t % tiles_m;
    const int tn = t / tiles_m;
    const long long m0 = (long long) tm * BM;
    const int n0 = tn * BN + wave * 32 * WN;
    const long long last_rt = (p.rows + kTileRows - 1) / kTileRows - 1;
    const int last_ct = (p.n + kTileRows - 1) / kTileRows - 1;

    const u4v* asrc[WM];
#pragma unroll
    for (int r = 0; r < WM; ++r) {
        const long long rt = min((long long) tm * WM + r, last_rt);
        asrc[r] = (const u4v*) p.xs + rt * n_chunks * 512 + tid;
    }
    const bf16x8* bbase[WN];
#pragma unroll
    for (int c = 0; c < WN; ++c) {
        const long long ct = min(n0 / 32 + c, last_ct);
        bbase[c] = (const bf16x8*) p.wp + ct * n_chunks * 256 + lane;
    }

    struct AShare {
        u4v v[WM][2];
    };
    struct BFrag {
        bf16x8 b[WN][4];
    };
    const int last = n_chunks - 1;
    auto load = [&](int ch, AShare& a, BFrag& f) {
        ch = min(ch, last);
#pragma unroll
        for (int r = 0; r < WM; ++r) {
            a.v[r][0] = asrc[r][ch * 512];
            a.v[r][1] = asrc[r][ch * 512 + 256];
        }
#pragma unroll
        for (int s = 0; s < 4; ++s)
#pragma unroll
            for (int c = 0; c < WN; ++c) f.b[c][s] = bbase[c][ch * 256 + s * 64];
    };
    auto store_a = [&](int buf, const AShare& a) {
#pragma unroll
        for (int r = 0; r < WM; ++r) {
            abuf[buf][r][tid] = a.v[r][0];
            abuf[buf][r][tid + 256] = a.v[r][1];
        }
    };

    f16v acc[WM][WN];
#pragma unroll
    for (int r = 0; r < WM; ++r)
#pragma unroll
        for (int c = 0; c < WN; ++c) acc[r][c] = f16v{};
    auto compute = [&](int buf, const BFrag& f) {
#pragma unroll
        for (int s = 0; s < 4; ++s) {
            bf16x8 a[WM][2];
#pragma unroll
            for (int r = 0; r < WM; ++r) {
                a[r][0] = __builtin_bit_cast(bf16x8, abuf[buf][r][(2 * s) * 64 + lane]);
                a[r][1] = __builtin_bit_cast(bf16x8, abuf[buf][r][(2 * s + 1) * 64 + lane]);
            }
#pragma unroll
            for (int r = 0; r < WM; ++r)
#pragma unroll
                for (int c = 0; c < WN; ++c) {
                    acc[r][c] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[r][0], f.b[c][s], acc[r][c], 0, 0, 0);
                    acc[r][c] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[r][1], f.b[c][s], acc[r][c], 0, 0, 0);
                }
        }
    };

    // On entry to a trip (c = 0 mod 3): chunk c is in LDS buffer 0 with its weights in
    // f0; chunk c + 1 is loaded (in flight) into a1 / f1.
    AShare a0, a1, a2;
    BFrag f0, f1, f2;
    load(0, a0, f0);
    load(1, a1, f1);
    store_a(0, a0);
    __syncthreads();
    int c = 0;
    for (; c + 3 <= n_chunks; c += 3) {
        load(c + 2, a2, f2);
        __builtin_amdgcn_sched_barrier(0);
        compute(0, f0);
        store_a(1, a1);
        __syncthreads();
        load(c + 3, a0, f0);
        __builtin_amdgcn_sched_barrier(0);
        compute(1, f1);
        store_a(2, a2);
        __syncthreads();
        load(c + 4, a1, f1);
        __builtin_amdgcn_sched_barrier(0);
        compute(2, f2);
        store_a(0, a0);
        __syncthreads();
    }
    if (c < n_chunks) compute(0, f0);
    if (c + 1 < n_chunks) {
        store_a(1, a1);
        __syncthreads();
        compute(1, f1);
    }
    store_blocks<WM, WN>(p, acc, m0, n0, i, h);
}

// the instantiated tile shapes: {wm, wn, kw, lds} (lds = kRing: project_ring_kernel)
constexpr GemmConfig kConfigs[] = {
    {1, 1, 4, 0}, {1, 2, 4, 0}, {2, 1, 4, 0}, {2, 2, 4, 0}, {2, 2, 2, 0},
    {2, 2, 1, 0}, {2, 3, 4, 0}, {2, 3, 2, 0}, {2, 3, 1, 2}, {1, 1, 1, kRing},
};

template <int WM, int WN, int KW>
hipError_t launch_tile(const GemmParams& p, hipStream_t stream) {
    constexpr int BM = 32 * WM, BN = 32 * WN * (4 / KW);
    const long long tm = (p.rows + BM - 1) / BM, tn = ((long long) p.n + BN - 1) / BN;
    hipLaunchKernelGGL((project_bf16_kernel<WM, WN, KW>), dim3((unsigned) (tm * tn * p.parts)), dim3(256), 0, stream, p,
                       (int) tm, (int) (tm * tn), (int) (pad_up(p.k, kTileK) / kTileK));
    if constexpr (KW == 4) {
        if (p.parts > 1) {
            const hipError_t e = hipGetLastError();
            if (e != hipSuccess) return e;
            hipLaunchKernelGGL((add_parts_kernel<WM, WN>), dim3((unsigned) ((tm * tn + 3) / 4)), dim3(256), 0, stream,
                               p, (int) tm, (int) (tm * tn));
        }
    }
    return hipGetLastError();
}

template <int WM, int WN>
hipError_t launch_ring_tile(const GemmParams& p, hipStream_t stream) {
    constexpr int BM = 32 * WM, BN = 128 * WN;
    const long long tm = (p.rows + BM - 1) / BM, tn = ((long long) p.n + BN - 1) / BN;
    hipLaunchKernelGGL((project_ring_kernel<WM, WN>), dim3((unsigned) (tm * tn)), dim3(256), 0, stream, p, (int) tm,
                       (int) (tm * tn), (int) (pad_up(p.k, kTileK) / kTileK));
    return hipGetLastError();
}

template <int WM, int WN, int KG>
hipError_t launch_lds_tile(const GemmParams& p, hipStream_t stream) {
    constexpr int BM = 32 * WM, BN = 128 * WN;
    const long long tm = (p.rows + BM - 1) / BM, tn = ((long long) p.n + BN - 1) / BN;
    hipLaunchKernelGGL((project_lds_kernel<WM, WN, KG>), dim3((unsigned) (tm * tn)), dim3(256 * KG), 0, stream, p,
                       (int) tm, (int) (tm * tn), (int) (pad_up(p.k, kTileK) / kTileK));
    return hipGetLastError();
}

}  // namespace

bool gemm_config_supported(const GemmConfig& c) {
    if (c.parts < 1 || (c.parts > 1 && (c.kw != 4 || c.lds != 0))) return false;
    for (const GemmConfig& k : kConfigs)
        if (k.wm == c.wm && k.wn == c.wn && k.kw == c.kw && k.lds == c.lds) return true;
    return false;
}

long long gemm_workgroups(const GemmParams& p, const GemmConfig& c) {
    const long long bm = 32LL * c.wm, bn = c.lds ? 128LL * c.wn : 32LL * c.wn * (4 / c.kw);
    return (p.rows + bm - 1) / bm * (((long long) p.n + bn - 1) / bn) * c.parts;
}

long long gemm_workspace_bytes(const GemmParams& p, const GemmConfig& c) {
    if (c.parts <= 1) return 0;
    return gemm_workgroups(p, c) * (c.wm * c.wn * 16 * 64 * (long long) sizeof(float));
}

// Up to 64 rows the product is bound by the weight stream, and the tile shapes that
// measured fastest on MI355X for n = 2560 to 16384 are taken by rule: one row tile,
// the k range split over the 4 waves, wider column tiles as n grows (the
// ring-pipelined LDS form for the widest).  A long k range (64 chunks or more) over
// few tiles leaves most of the chip idle and each wave with a long serial chain, so
// there the k range is also split over 2 to 4 workgroups per tile (a second kernel
// adds the partial blocks) until about 192 workgroups run.
//
// Above 64 rows each candidate shape is priced as (rounds of 256 workgroups) x
// (chunks per wave) x (32x32 blocks per wave) x (measured microseconds per
// block-chunk of that shape), plus 8 us for the second kernel of a split launch
// (fitted to graph-replayed timings on MI355X, k = 2560 and 6144, n = 1024 to
// 16384), which keeps the launch from spilling a few workgroups into a second round
// and splits k only where the shorter chains pay for that kernel.
namespace {
struct Priced {
    GemmConfig c;
    double us_per_block_chunk;
    long long min_rows;
};
constexpr Priced kPriced[] = {
    {{2, 2, 1, 0}, 0.245, 65}, {{2, 3, 2, 0}, 0.31, 65}, {{2, 2, 2, 0}, 0.305, 65}, {{2, 2, 4, 0}, 0.33, 65},
    {{2, 3, 4, 0}, 0.38, 65},  {{2, 1, 4, 0}, 0.47, 65}, {{2, 3, 1, 2}, 0.46, 257}, {{1, 1, 1, kRing}, 0.34, 65},
    {{1, 2, 4, 0}, 0.42, 65},  {{1, 1, 4, 0}, 0.65, 65},
};
constexpr double kSplitUs = 8.0;
constexpr int kMaxParts = 4;
constexpr long long kSplitMinChunks = 64;
}  // namespace

GemmConfig choose_gemm_config(long long rows, int k, int n) {
    const long long chunks = pad_up(k, kTileK) / kTileK;
    GemmParams p{};
    p.rows = rows;
    p.n = n;
    if (rows <= 64) {
        GemmConfig c = rows <= 32 ? (n >= 12288 ? GemmConfig{1, 1, 1, kRing}
                                    : n >= 8192 ? GemmConfig{1, 2, 4, 0} : GemmConfig{1, 1, 4, 0})
                                  : (n >= 8192 ? GemmConfig{1, 1, 1, kRing}
                                    : n >= 4096 ? GemmConfig{1, 2, 4, 0} : GemmConfig{1, 1, 4, 0});
        if (chunks >= kSplitMinChunks && c.kw == 4 && c.lds == 0) {
            const long long w0 = gemm_workgroups(p, c);
            if (w0 <= 128) c.parts = (int) std::min<long long>(kMaxParts, (192 + w0 - 1) / w0);
        }
        return c;
    }
    GemmConfig best = kPriced[0].c;
    double best_us = -1.0;
    for (const Priced& q : kPriced) {
        if (rows < q.min_rows) continue;
        const long long split = q.c.lds == kRing ? 1 : q.c.lds ? q.c.lds : q.c.kw;
        const bool can_split = chunks >= kSplitMinChunks && q.c.wm == 1 && q.c.kw == 4 && q.c.lds == 0;
        for (int parts = 1; parts <= (can_split ? kMaxParts : 1); ++parts) {
            GemmConfig c = q.c;
            c.parts = parts;
            const long long rounds = (gemm_workgroups(p, c) + 255) / 256;
            const double us = (double) rounds * (double) ((chunks + split * parts - 1) / (split * parts)) * c.wm *
                                  c.wn * q.us_per_block_chunk + (parts > 1 ? kSplitUs : 0.0);
            if (best_us < 0.0 || us < best_us) {
                best = c;
                best_us = us;
            }
        }
    }
    return best;
}

hipError_t launch_split_bf16(const SplitParams& p, hipStream_t stream) {
    const long long frags = pad_up(p.rows, kTileRows) * pad_up(p.k, kTileK) / 8;
    const long long blocks = std::min<long long>((frags + 255) / 256, 1LL << 16);
    hipLaunchKernelGGL(split_bf16_kernel, dim3((unsigned) blocks), dim3(256), 0, stream, p);
    return hipGetLastError();
}

hipError_t launch_pack_bf16(const PackParams& p, hipStream_t stream) {
    const long long frags = pad_up(p.n, kTileRows) * pad_up(p.k, kTileK) / 8;
    const long long blocks = std::min<long long>((frags + 255) / 256, 1LL << 16);
    hipLaunchKernelGGL(pack_bf16_kernel, dim3((unsigned) blocks), dim3(256), 0, stream, p);
    return hipGetLastError();
}

hipError_t launch_project_bf16(const GemmParams& p, const GemmConfig& c, hipStream_t stream) {
    if (p.parts != c.parts || (c.parts > 1 && (p.ws == nullptr || c.kw != 4 || c.lds != 0)))
        return hipErrorInvalidValue;
#define GDN_TILE(A, B, C) \
    if (!c.lds && c.wm == A && c.wn == B && c.kw == C) return launch_tile<A, B, C>(p, stream);
#define GDN_LDS_TILE(A, B, G) \
    if (c.lds == G && c.wm == A && c.wn == B && c.kw == 1) return launch_lds_tile<A, B, G>(p, stream);
    if (c.lds == kRing && c.wm == 1 && c.wn == 1) return launch_ring_tile<1, 1>(p, stream);
    GDN_TILE(1, 1, 4)
    GDN_TILE(1, 2, 4)
    GDN_TILE(2, 1, 4)
    GDN_TILE(2, 2, 4)
    GDN_TILE(2, 2, 2)
    GDN_TILE(2, 2, 1)
    GDN_TILE(2, 3, 4)
    GDN_TILE(2, 3, 2)
    GDN_LDS_TILE(2, 3, 2)
#undef GDN_TILE
#undef GDN_LDS_TILE
    return hipErrorInvalidValue;
}

}  // namespace gdn
