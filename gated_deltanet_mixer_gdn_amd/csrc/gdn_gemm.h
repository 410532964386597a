// gdn_gemm.h - internal interface of the bf16-weight projection kernels
// (gdn_gemm.hip) for the C-ABI layer.  Not installed, not part of the ABI.
//
// Both operands of a projection live in HBM in the order the matrix-core
// instruction v_mfma_f32_32x32x16_bf16 consumes them, so every load instruction of
// the main loop reads 1 KiB of contiguous memory.  The unit is a tile of 32 rows x
// 64 k: for step s (0..3) of the tile and lane l = i + 32h (i < 32, h < 2), the
// lane's 8 values are element [32R + i][64C + 32h + 8s + j], j = 0..7, and they sit
// at fragment (s, l) of the tile, fragment index s*64 + l, 16 bytes each.
//   packed weights  [n32/32][k64/64] tiles of 4 fragments x 64 lanes x 16 B = 4 KiB
//   split x         [r32/32][k64/64] tiles of 4 steps x (hi, lo) x 64 lanes x 16 B
//                   = 8 KiB; hi fragment (2s) * 64 + l, lo fragment (2s + 1) * 64 + l
// Rows are padded to a multiple of 32 and k to a multiple of 64 with zeros.
#pragma once

#include <hip/hip_runtime_api.h>
#include <stdint.h>

namespace gdn {

constexpr int kTileRows = 32;
constexpr int kTileK = 64;

constexpr long long pad_up(long long v, long long m) { return (v + m - 1) / m * m; }

struct SplitParams {
    const float* x;   // [rows][k]
    uint16_t* xs;     // tiled split layout
    long long rows;
    int k;            // multiple of 8
};

struct PackParams {
    const uint16_t* w;  // [n][k] bf16 bits
    uint16_t* wp;       // tiled layout
    int n, k;           // k a multiple of 8
};

constexpr int kMaxOuts = 4;

// res[r][j] = sum_e w[j][e] * (hi + lo)[r][e]; output o takes the columns
// c0[o] <= j < c0[o + 1] as out[o] [rows][c0[o + 1] - c0[o]] (c0[0] = 0; the entries
// past the last output are n, so their ranges are empty)
//
// parts > 1 (tile shapes with kw = 4 only): the k chunks are split into `parts`
// contiguous ranges, one workgroup per (tile, range), each writing its partial block
// to ws; a second kernel adds a tile's blocks in range order and stores the tile.
struct GemmParams {
    const uint16_t* xs;  // split activations, tiled
    const uint16_t* wp;  // packed weights, tiled
    float* out[kMaxOuts];
    int c0[kMaxOuts + 1];
    long long rows;
    int k, n;
    int parts = 1;
    float* ws = nullptr;   // [tiles][parts][32 WM x 32 WN block] partial sums
};

// Tile shape of one launch: each of the 4 waves of a workgroup computes a
// (32*wm) x (32*wn) block of out; kw waves (1, 2 or 4) share one block and split
// its k range, the other 4/kw waves take neighbouring column blocks.  lds = G > 0
// (kw = 1 only): G groups of 4 such waves take alternate k chunks, and each group's
// activation tiles go through LDS once instead of being read by every wave.
// parts > 1 (kw = 4, lds = 0 only): the k range is also split over `parts`
// workgroups per tile (GemmParams::parts).
struct GemmConfig {
    int wm, wn, kw, lds;
    int parts = 1;
};
// lds value of the ring-pipelined LDS form (4 waves side by side in n, activation
// tiles through a 3-buffer LDS ring, weight fragments in a 3-deep register ring)
constexpr int kRing = 9;

bool gemm_config_supported(const GemmConfig& c);
GemmConfig choose_gemm_config(long long rows, int k, int n);
long long gemm_workgroups(const GemmParams& p, const GemmConfig& c);
// bytes of GemmParams::ws a launch of shape c needs (0 when c.parts == 1)
long long gemm_workspace_bytes(const GemmParams& p, const GemmConfig& c);

// Sets the message gdn_last_error() returns on this host thread (cleared for GDN_OK)
// and returns code; for C-ABI entry points defined outside gdn_api.cpp.
int set_last_error(int code, const char* fn, const char* msg);

hipError_t launch_split_bf16(const SplitParams& p, hipStream_t stream);
hipError_t launch_pack_bf16(const PackParams& p, hipStream_t stream);
hipError_t launch_project_bf16(const GemmParams& p, const GemmConfig& c, hipStream_t stream);

}  // namespace gdn
