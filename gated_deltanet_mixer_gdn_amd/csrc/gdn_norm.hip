// gdn_norm.hip - the gated RMSNorm kernel.
#include "gdn_device.h"

namespace gdn {

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
    const float inv = rms_inv(ss, p.eps);
    *(f4*) (p.y + off) = x * inv * w * gate4(z, p.gate_silu);
}

// ------------------------------------------------------------------ launch
hipError_t launch_gated_rmsnorm(const NormParams& p, hipStream_t stream) {
    const dim3 grid((unsigned) ((p.rows + kNormRowsPerBlock - 1) / kNormRowsPerBlock));
    hipLaunchKernelGGL(gated_rmsnorm_kernel, grid, dim3(256), 0, stream, p);
    return hipGetLastError();
}

}  // namespace gdn
