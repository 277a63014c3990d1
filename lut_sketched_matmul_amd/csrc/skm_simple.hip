// Checking aids (index unpack, dequantise) and the fp32 path of the
// sketched-weight matmul.
//
// The fp32 path serves fp32 activations with fp32 tables. It computes with
// fp32 products and fp32 accumulation on the vector ALUs; its sizes are small
// (the method's fp32 use is a debug/reference mode), so the kernels favour a
// fixed, deterministic summation order over speed.
#include "skm_common.h"
#include "skm_launch.h"

namespace skm {

// ---------------------------------------------------------------------------
// unpack: one thread per (row, 32-column unit)
// ---------------------------------------------------------------------------
template <int B>
__global__ void __launch_bounds__(256) k_unpack(const uint8_t* __restrict__ idx_packed, int64_t n, int64_t d,
                                                 uint8_t* __restrict__ out) {
  const int64_t units = d / 32;
  const int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (t >= n * units) return;
  const int64_t i = t / units, u = t % units;
  uint32_t w[B];
  load_unit<B>(idx_packed + i * (d * B / 8), u, w);
  uint32_t o[8];
#pragma unroll
  for (int q = 0; q < 8; ++q) {
    uint32_t v = 0;
#pragma unroll
    for (int r = 0; r < 4; ++r) v |= unit_field<B>(w, 4 * q + r) << (8 * r);
    o[q] = v;
  }
  u32x4* dst = reinterpret_cast<u32x4*>(out + i * d + u * 32);
  dst[0] = u32x4{o[0], o[1], o[2], o[3]};
  dst[1] = u32x4{o[4], o[5], o[6], o[7]};
}

hipError_t launch_unpack(const uint8_t* idx_packed, const Problem& p, uint8_t* idx, hipStream_t s) {
  const int64_t work = p.n * p.units();
  const dim3 grid((unsigned)((work + 255) / 256));
  switch (p.b) {
    case 2: hipLaunchKernelGGL(k_unpack<2>, grid, dim3(256), 0, s, idx_packed, p.n, p.d, idx); break;
    case 3: hipLaunchKernelGGL(k_unpack<3>, grid, dim3(256), 0, s, idx_packed, p.n, p.d, idx); break;
    default: hipLaunchKernelGGL(k_unpack<4>, grid, dim3(256), 0, s, idx_packed, p.n, p.d, idx); break;
  }
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// dequantise: one thread per (row, unit); W keeps the table dtype (exact copy)
// ---------------------------------------------------------------------------
template <int B, typename TL>
__global__ void __launch_bounds__(256) k_dequant(const uint8_t* __restrict__ idx_packed, const TL* __restrict__ lut,
                                                  int64_t n, int64_t d, int gpr, TL* __restrict__ W) {
  constexpr int K = 1 << B;
  const int64_t units = d / 32;
  const int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (t >= n * units) return;
  const int64_t i = t / units, u = t % units;
  const int64_t g = (u * 32) / (d / gpr);
  uint32_t w[B];
  load_unit<B>(idx_packed + i * (d * B / 8), u, w);
  const TL* tab = lut + (i * gpr + g) * K;
  TL* dst = W + i * d + u * 32;
#pragma unroll
  for (int f = 0; f < 32; ++f) dst[f] = tab[unit_field<B>(w, f)];
}

template <typename TL>
static hipError_t dequant_t(const uint8_t* idx, const TL* lut, const Problem& p, TL* W, hipStream_t s) {
  const int64_t work = p.n * p.units();
  const dim3 grid((unsigned)((work + 255) / 256));
  switch (p.b) {
    case 2: hipLaunchKernelGGL((k_dequant<2, TL>), grid, dim3(256), 0, s, idx, lut, p.n, p.d, p.gpr, W); break;
    case 3: hipLaunchKernelGGL((k_dequant<3, TL>), grid, dim3(256), 0, s, idx, lut, p.n, p.d, p.gpr, W); break;
    default: hipLaunchKernelGGL((k_dequant<4, TL>), grid, dim3(256), 0, s, idx, lut, p.n, p.d, p.gpr, W); break;
  }
  return hipGetLastError();
}

hipError_t launch_dequant(const uint8_t* idx, const void* lut, int lut_dtype, const Problem& p, void* W,
                          hipStream_t s) {
  if (lut_dtype == DT_F32) return dequant_t(idx, (const float*)lut, p, (float*)W, s);
  // 16-bit tables are copied bit for bit
  return dequant_t(idx, (const uint16_t*)lut, p, (uint16_t*)W, s);
}

// ---------------------------------------------------------------------------
// zero fill
// ---------------------------------------------------------------------------
__global__ void __launch_bounds__(256) k_zero_f32(float* __restrict__ dst, int64_t count) {
  const int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (t < count) dst[t] = 0.0f;
}

hipError_t launch_zero_f32(float* dst, int64_t count, hipStream_t s) {
  if (count <= 0) return hipSuccess;
  hipLaunchKernelGGL(k_zero_f32, dim3((unsigned)((count + 255) / 256)), dim3(256), 0, s, dst, count);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// fp32 forward: one wave per weight row, TT tokens per pass
// ---------------------------------------------------------------------------
constexpr int F32_TT = 8;

template <int B>
__global__ void __launch_bounds__(256) k_fwd_f32(const float* __restrict__ X, const uint8_t* __restrict__ idx_packed,
                                                  const float* __restrict__ lut, int64_t m, int64_t n, int64_t d,
                                                  int gpr, float* __restrict__ Y) {
  constexpr int K = 1 << B;
  const int64_t row = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= n) return;
  const int lane = lane_id();
  const int64_t units = d / 32, ucols = d / gpr;
  const uint8_t* rp = idx_packed + row * (d * B / 8);
  for (int64_t t0 = 0; t0 < m; t0 += F32_TT) {
    float acc[F32_TT];
#pragma unroll
    for (int tt = 0; tt < F32_TT; ++tt) acc[tt] = 0.0f;
    for (int64_t u = lane; u < units; u += 64) {
      uint32_t w[B];
      load_unit<B>(rp, u, w);
      const float* tab = lut + (row * gpr + (u * 32) / ucols) * K;
#pragma unroll 4
      for (int f = 0; f < 32; ++f) {
        const float wv = tab[unit_field<B>(w, f)];
        const int64_t j = u * 32 + f;
#pragma unroll
        for (int tt = 0; tt < F32_TT; ++tt)
          if (t0 + tt < m) acc[tt] = fmaf(X[(t0 + tt) * d + j], wv, acc[tt]);
      }
    }
#pragma unroll
    for (int tt = 0; tt < F32_TT; ++tt) {
      float v = acc[tt];
#pragma unroll
      for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off, 64);
      if (lane == 0 && t0 + tt < m) Y[(t0 + tt) * n + row] = v;
    }
  }
}

hipError_t launch_fwd_f32(const float* X, const uint8_t* idx, const float* lut, const Problem& p, float* Y,
                          hipStream_t s) {
  const dim3 grid((unsigned)((p.n + 3) / 4));
  switch (p.b) {
    case 2: hipLaunchKernelGGL(k_fwd_f32<2>, grid, dim3(256), 0, s, X, idx, lut, p.m, p.n, p.d, p.gpr, Y); break;
    case 3: hipLaunchKernelGGL(k_fwd_f32<3>, grid, dim3(256), 0, s, X, idx, lut, p.m, p.n, p.d, p.gpr, Y); break;
    default: hipLaunchKernelGGL(k_fwd_f32<4>, grid, dim3(256), 0, s, X, idx, lut, p.m, p.n, p.d, p.gpr, Y); break;
  }
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// fp32 dX: one thread per column j, rows summed in order
// ---------------------------------------------------------------------------
template <int B>
__global__ void __launch_bounds__(256) k_dx_f32(const float* __restrict__ dY, const uint8_t* __restrict__ idx_packed,
                                                 const float* __restrict__ lut, int64_t m, int64_t n, int64_t d,
                                                 int gpr, float* __restrict__ dX) {
  constexpr int K = 1 << B;
  const int64_t j = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (j >= d) return;
  const int64_t g = j / (d / gpr);
  const int64_t rb = d * B / 8;
  const int64_t bit = j * B;
  for (int64_t t0 = 0; t0 < m; t0 += F32_TT) {
    float acc[F32_TT];
#pragma unroll
    for (int tt = 0; tt < F32_TT; ++tt) acc[tt] = 0.0f;
    for (int64_t i = 0; i < n; ++i) {
      const uint8_t* rp = idx_packed + i * rb + (bit >> 3);
      // two bytes cover any field of <= 4 bits (the second byte exists whenever it is needed)
      uint32_t two = rp[0];
      if ((bit & 7) + B > 8) two |= (uint32_t)rp[1] << 8;
      const uint32_t e = (two >> (bit & 7)) & (K - 1);
      const float wv = lut[(i * gpr + g) * K + e];
#pragma unroll
      for (int tt = 0; tt < F32_TT; ++tt)
        if (t0 + tt < m) acc[tt] = fmaf(dY[(t0 + tt) * n + i], wv, acc[tt]);
    }
#pragma unroll
    for (int tt = 0; tt < F32_TT; ++tt)
      if (t0 + tt < m) dX[(t0 + tt) * d + j] = acc[tt];
  }
}

hipError_t launch_dx_f32(const float* dY, const uint8_t* idx, const float* lut, const Problem& p, float* dX,
                         hipStream_t s) {
  const dim3 grid((unsigned)((p.d + 255) / 256));
  switch (p.b) {
    case 2: hipLaunchKernelGGL(k_dx_f32<2>, grid, dim3(256), 0, s, dY, idx, lut, p.m, p.n, p.d, p.gpr, dX); break;
    case 3: hipLaunchKernelGGL(k_dx_f32<3>, grid, dim3(256), 0, s, dY, idx, lut, p.m, p.n, p.d, p.gpr, dX); break;
    default: hipLaunchKernelGGL(k_dx_f32<4>, grid, dim3(256), 0, s, dY, idx, lut, p.m, p.n, p.d, p.gpr, dX); break;
  }
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// fp32 dLUT: one block per (row, group). Each thread bins the gradients of its
// columns into private LDS bins; bins are then summed over threads in order.
// ---------------------------------------------------------------------------
template <int B>
__global__ void __launch_bounds__(256) k_dlut_f32(const float* __restrict__ dY, const float* __restrict__ X,
                                                   const uint8_t* __restrict__ idx_packed, int64_t m, int64_t n,
                                                   int64_t d, int gpr, float* __restrict__ dLUT, int accumulate) {
  constexpr int K = 1 << B;
  __shared__ float bins[K][256];
  const int64_t i = blockIdx.x / gpr;
  const int g = (int)(blockIdx.x % gpr);
  const int tid = threadIdx.x;
#pragma unroll
  for (int c = 0; c < K; ++c) bins[c][tid] = 0.0f;
  const int64_t ucols = d / gpr;
  const int64_t rb = d * B / 8;
  for (int64_t jj = tid; jj < ucols; jj += 256) {
    const int64_t j = g * ucols + jj;
    float gw = 0.0f;
    for (int64_t t = 0; t < m; ++t) gw = fmaf(dY[t * n + i], X[t * d + j], gw);
    const int64_t bit = j * B;
    const uint8_t* rp = idx_packed + i * rb + (bit >> 3);
    uint32_t two = rp[0];
    if ((bit & 7) + B > 8) two |= (uint32_t)rp[1] << 8;
    const uint32_t e = (two >> (bit & 7)) & (K - 1);
    bins[e][tid] += gw;
  }
  __syncthreads();
  if (tid < K) {
    float s = 0.0f;
    for (int t = 0; t < 256; ++t) s += bins[tid][t];
    float* dst = dLUT + (i * gpr + g) * K + tid;
    *dst = accumulate ? (*dst + s) : s;
  }
}

hipError_t launch_dlut_f32(const float* dY, const float* X, const uint8_t* idx, const Problem& p, float* dLUT,
                           int accumulate, hipStream_t s) {
  const dim3 grid((unsigned)(p.n * p.gpr));
  switch (p.b) {
    case 2:
      hipLaunchKernelGGL(k_dlut_f32<2>, grid, dim3(256), 0, s, dY, X, idx, p.m, p.n, p.d, p.gpr, dLUT, accumulate);
      break;
    case 3:
      hipLaunchKernelGGL(k_dlut_f32<3>, grid, dim3(256), 0, s, dY, X, idx, p.m, p.n, p.d, p.gpr, dLUT, accumulate);
      break;
    default:
      hipLaunchKernelGGL(k_dlut_f32<4>, grid, dim3(256), 0, s, dY, X, idx, p.m, p.n, p.d, p.gpr, dLUT, accumulate);
      break;
  }
  return hipGetLastError();
}

}  // namespace skm
