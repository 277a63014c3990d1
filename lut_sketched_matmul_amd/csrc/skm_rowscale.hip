// Row exponents of the per-row power-of-two prescale (see skm_common.h):
// e[r] = clamp(E - 141, -126, 113), E the biased exponent of the largest
// |value| of row r of a bf16 matrix A [rows][cols]. Computed once per call
// into the caller's workspace for the kernels that convert bf16 activations
// (X of the forward GEMM, dY of dX) to f16 matrix-core operands.
//
// One wave per row; HBM-bound (the row is read once, 2 bytes per element).
#include "skm_common.h"
#include "skm_launch.h"

namespace skm {

namespace {

template <bool VEC>
__global__ void __launch_bounds__(256) k_row_exp(const uint16_t* __restrict__ A, int64_t rows, int64_t cols,
                                                  int32_t* __restrict__ e) {
  const int lane = lane_id();
  const int64_t r = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (r >= rows) return;  // wave-uniform
  const uint16_t* row = A + r * cols;
  uint32_t mx = 0;
  if constexpr (VEC) {
    // rows of a multiple of 8 elements are 16-byte aligned: 8 values per load,
    // four loads in flight per lane
    const int64_t chunks = cols / 8;
    const u32x4* p = reinterpret_cast<const u32x4*>(row);
    int64_t c = lane;
    for (; c + 192 < chunks; c += 256) {
      const u32x4 a = p[c], b = p[c + 64], cc = p[c + 128], dd = p[c + 192];
      uint32_t m0 = absmax8_bf16(a), m1 = absmax8_bf16(b), m2 = absmax8_bf16(cc), m3 = absmax8_bf16(dd);
      m0 = m0 > m1 ? m0 : m1;
      m2 = m2 > m3 ? m2 : m3;
      m0 = m0 > m2 ? m0 : m2;
      mx = mx > m0 ? mx : m0;
    }
    for (; c < chunks; c += 64) {
      const uint32_t m0 = absmax8_bf16(p[c]);
      mx = mx > m0 ? mx : m0;
    }
  } else {
    for (int64_t c = lane; c < cols; c += 64) {
      const uint32_t v = row[c] & 0x7FFFu;
      mx = mx > v ? mx : v;
    }
  }
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) {
    const uint32_t v = (uint32_t)__shfl_xor((int)mx, o, 64);
    mx = mx > v ? mx : v;
  }
  if (lane == 0) e[r] = row_exp_of(mx);
}

}  // namespace

hipError_t launch_row_exp(const void* A, int64_t rows, int64_t cols, int32_t* e, hipStream_t s) {
  const dim3 grid((unsigned)((rows + 3) / 4));
  if (cols % 8 == 0)
    hipLaunchKernelGGL(k_row_exp<true>, grid, dim3(256), 0, s, (const uint16_t*)A, rows, cols, e);
  else
    hipLaunchKernelGGL(k_row_exp<false>, grid, dim3(256), 0, s, (const uint16_t*)A, rows, cols, e);
  return hipGetLastError();
}

}  // namespace skm
