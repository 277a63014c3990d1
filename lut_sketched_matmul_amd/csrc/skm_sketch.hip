// Sketch construction: the tables and the index stream of a layer from its
// dense weights and the factor of its damped inverse Hessian.
//
// SpaLLM section 2.2 ("Weighted Lloyd's algorithm ...", "Learning the
// sketching matrix") and the Sketch to Adapt reply to Concern 1:
//   h_j = 1 / [H^-1]_jj, H^-1 = U^T U (U upper triangular, from the caller)
//   tables: weighted Lloyd's algorithm over the weights of each (row, group),
//           weight j counted with h_j, starting from k centroids spread evenly
//           over [min, max] of the group
//   indices: columns in order, each weight to its nearest table entry, its
//           error err = (w_j - q_j) / U_jj spread over the later columns as
//           w_j' -= err * U_jj' (the update of Frantar et al.)
//
// Kernels: k_col_weights (one thread per column); k_lloyd (one wave per
// (row, group), everything in registers and wave reductions); the mapping in
// blocks of 64 columns: k_map_block runs the sequential sweep of one block
// (four lanes per row, the block's 64 x 64 part of U in LDS) and writes the
// packed indices and the block's errors; k_map_trail applies errors to later
// columns as fp32 rank-k updates (W[:, cols] -= E^T U[rows, cols]), in two
// levels: each 64-column block's errors to the rest of its 512-column outer
// block, each outer block's 512 errors to every column after it. The sum each
// weight receives is the sequential one, in another order.
#include "skm_common.h"
#include "skm_launch.h"

namespace skm {

namespace {

constexpr int MAP_COLS = 64;

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}
__device__ __forceinline__ float wave_min(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v = fminf(v, __shfl_xor(v, o, 64));
  return v;
}
__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
  return v;
}

// [H^-1]_jj = sum_{k <= j} U_kj^2 (U is upper triangular). A block takes 64
// columns; its 4 waves take every 4th row (each lane one column, so a wave
// reads 256 contiguous bytes per row) and the 4 partial sums meet in LDS.
__global__ void __launch_bounds__(256) k_col_weights(const float* __restrict__ U, int64_t d, float* __restrict__ h) {
  __shared__ float part[4][64];
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int64_t j = (int64_t)blockIdx.x * 64 + lane;
  float s = 0.f;
  if (j < d)
    for (int64_t k = w; k <= j; k += 4) {
      const float u = U[k * d + j];
      s += u * u;
    }
  part[w][lane] = s;
  __syncthreads();
  if (w == 0 && j < d) h[j] = 1.f / (((part[0][lane] + part[1][lane]) + part[2][lane]) + part[3][lane]);
}

// one wave per (row, group); K = 2^b centroids
template <int K, typename TL>
__global__ void __launch_bounds__(256) k_lloyd(const float* __restrict__ W, const float* __restrict__ h, int64_t n,
                                                int64_t d, int gpr, int iters, TL* __restrict__ lut) {
  const int lane = threadIdx.x & 63;
  const int64_t wg = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (wg >= n * gpr) return;  // whole waves; no block barriers below
  const int64_t i = wg / gpr;
  const int g = (int)(wg % gpr);
  const int64_t G = d / gpr;
  const float* x = W + i * d + g * G;
  const float* hw = h + g * G;

  float lo = __builtin_inff(), hi = -__builtin_inff();
  for (int64_t j = lane; j < G; j += 64) {
    lo = fminf(lo, x[j]);
    hi = fmaxf(hi, x[j]);
  }
  lo = wave_min(lo);
  hi = wave_max(hi);
  float c[K];
  const float step = (hi - lo) / (float)K;
#pragma unroll
  for (int r = 0; r < K; ++r) c[r] = lo + step * ((float)r + 0.5f);

  for (int it = 0; it < iters; ++it) {
    float sw[K], swx[K];
#pragma unroll
    for (int r = 0; r < K; ++r) sw[r] = swx[r] = 0.f;
    for (int64_t j = lane; j < G; j += 64) {
      const float v = x[j], wt = hw[j];
      // nearest centroid, ties to the lower index
      float best = fabsf(v - c[0]);
      int a = 0;
#pragma unroll
      for (int r = 1; r < K; ++r) {
        const float dr = fabsf(v - c[r]);
        if (dr < best) {
          best = dr;
          a = r;
        }
      }
      const float wx = wt * v;
#pragma unroll
      for (int r = 0; r < K; ++r) {
        sw[r] += a == r ? wt : 0.f;
        swx[r] += a == r ? wx : 0.f;
      }
    }
    bool same = true;
#pragma unroll
    for (int r = 0; r < K; ++r) {
      const float s = wave_sum(sw[r]), sx = wave_sum(swx[r]);
      const float nc = s > 0.f ? sx / s : c[r];  // an empty cluster keeps its centroid
      same = same && nc == c[r];
      c[r] = nc;
    }
    if (same) break;  // wave-uniform: every lane holds the same sums
  }
  if (lane < K) {
    float v = c[0];
#pragma unroll
    for (int r = 1; r < K; ++r) v = lane == r ? c[r] : v;
    lut[wg * K + lane] = from_f32<TL>(v);
  }
}

// One 64-column block of the mapping sweep. Four lanes per row (16 rows per
// wave): lane `sub` of a row holds the row's columns 4 t + sub (t < 16) of the
// block, so the updates of each step split over the four lanes. Column c is
// owned by lane c % 4: a quad broadcast (DPP) hands the owner's weight to the
// other three, each lane scans a quarter of the table and two DPP butterfly
// steps leave the nearest entry (ties to the lower index) in all four. The
// error is (w - q) times 1 / U[c][c] (the reciprocals are taken once per
// block). Reads the compensated weights
// Wc[:, j0 : j0 + cols] (all earlier blocks' errors applied), writes the
// block's packed indices and its errors E [64][n]. The block's part of U sits
// in LDS as [c][sub][t] so a lane's 16 coefficients of a step are contiguous.
template <int OWN>
__device__ __forceinline__ float quad_bcast(float v) {
  constexpr int ctrl = OWN | (OWN << 2) | (OWN << 4) | (OWN << 6);  // quad_perm [OWN, OWN, OWN, OWN]
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), ctrl, 0xF, 0xF, false));
}
template <int CTRL>
__device__ __forceinline__ float quad_perm_f(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL, 0xF, 0xF, false));
}
template <int CTRL>
__device__ __forceinline__ int quad_perm_i(int v) {
  return __builtin_amdgcn_update_dpp(0, v, CTRL, 0xF, 0xF, false);
}
// merge with the quad partner given by CTRL: the partner's entry wins when it
// is nearer, or as near with a lower index
template <int CTRL>
__device__ __forceinline__ void quad_min(float& best, float& q, int& a) {
  const float pb = quad_perm_f<CTRL>(best), pq = quad_perm_f<CTRL>(q);
  const int pa = quad_perm_i<CTRL>(a);
  const bool take = pb < best || (pb == best && pa < a);
  best = take ? pb : best;
  q = take ? pq : q;
  a = take ? pa : a;
}

template <int C, int B, int K>
__device__ __forceinline__ void map_step(float (&w)[16], const float (&t0)[K / 4], const float (&t1)[K / 4],
                                         const float (*ub)[MAP_COLS], const float* rdiag, int sub, int cols,
                                         bool row_ok, int64_t n, int64_t i, float* __restrict__ E,
                                         uint32_t (&pk)[MAP_COLS * B / 32]) {
  if constexpr (C < MAP_COLS) {
    constexpr int T = C / 4, OWN = C % 4;
    if (C < cols) {  // uniform
      // the owner's weight; each lane scans its quarter of the table (entries
      // sub K/4 .. sub K/4 + K/4 - 1), then two butterfly steps over the quad
      const float wv = quad_bcast<OWN>(w[T]);
      float best = fabsf(wv - (C < 32 ? t0[0] : t1[0])), q = C < 32 ? t0[0] : t1[0];
      int a = sub * (K / 4);
#pragma unroll
      for (int e = 1; e < K / 4; ++e) {
        const float tvv = C < 32 ? t0[e] : t1[e];
        const float dr = fabsf(wv - tvv);
        const bool lt = dr < best;
        best = lt ? dr : best;
        q = lt ? tvv : q;
        a = lt ? sub * (K / 4) + e : a;
      }
      quad_min<0xB1>(best, q, a);  // quad_perm [1, 0, 3, 2]
      quad_min<0x4E>(best, q, a);  // quad_perm [2, 3, 0, 1]
      const float err = (wv - q) * rdiag[C];  // the same on all four lanes
      if (sub == OWN && row_ok) E[C * n + i] = err;
      const float* u = ub[C] + sub * 16;
#pragma unroll
      for (int t2 = T + 1; t2 < 16; ++t2) w[t2] -= err * u[t2];
      if (sub > OWN) w[T] -= err * u[T];
      constexpr int p = B * C;
      pk[p >> 5] |= (uint32_t)a << (p & 31);
      if constexpr ((p & 31) + B > 32) pk[(p >> 5) + 1] |= (uint32_t)a >> (32 - (p & 31));
    }
    map_step<C + 1, B, K>(w, t0, t1, ub, rdiag, sub, cols, row_ok, n, i, E, pk);
  }
}

template <int B, typename TL>
__global__ void __launch_bounds__(64) k_map_block(float* __restrict__ Wc, const float* __restrict__ U,
                                                   const TL* __restrict__ lut, int64_t n, int64_t d, int gpr,
                                                   int64_t j0, int cols, uint8_t* __restrict__ idx_packed,
                                                   float* __restrict__ E) {
  constexpr int K = 1 << B;
  __shared__ float ub[MAP_COLS][MAP_COLS];  // [c][sub * 16 + t] = U[j0 + c][j0 + 4 t + sub]
  __shared__ float rdiag[MAP_COLS];         // 1 / U[j0 + c][j0 + c] (the steps multiply)
  for (int e = threadIdx.x; e < MAP_COLS * MAP_COLS; e += 64) {
    const int r = e / MAP_COLS, cc = e % MAP_COLS;
    ub[r][(cc & 3) * 16 + (cc >> 2)] = (r < cols && cc < cols) ? U[(j0 + r) * d + j0 + cc] : 0.f;
  }
  rdiag[threadIdx.x] = threadIdx.x < cols ? 1.f / U[(j0 + threadIdx.x) * d + j0 + threadIdx.x] : 0.f;
  __syncthreads();
  const int sub = threadIdx.x & 3;
  const int64_t i = (int64_t)blockIdx.x * 16 + (threadIdx.x >> 2);
  const bool row_ok = i < n;  // no early exit: the quad broadcasts need every lane
  const int64_t ic = row_ok ? i : n - 1;
  const int64_t G = d / gpr;
  float w[16];
#pragma unroll
  for (int t = 0; t < 16; ++t) {
    const int col = 4 * t + sub;
    w[t] = col < cols ? Wc[ic * d + j0 + col] : 0.f;
  }
  // the block spans at most two groups, split at a multiple of 32 columns;
  // each lane keeps its quarter of both tables
  float t0[K / 4], t1[K / 4];
  const int64_t g0 = j0 / G, g1 = (j0 + 32) / G;
#pragma unroll
  for (int e = 0; e < K / 4; ++e) {
    t0[e] = to_f32(lut[(ic * gpr + g0) * K + sub * (K / 4) + e]);
    t1[e] = to_f32(lut[(ic * gpr + (g1 < gpr ? g1 : g0)) * K + sub * (K / 4) + e]);
  }
  constexpr int WORDS = MAP_COLS * B / 32;
  uint32_t pk[WORDS];
#pragma unroll
  for (int q = 0; q < WORDS; ++q) pk[q] = 0u;
  map_step<0, B, K>(w, t0, t1, ub, rdiag, sub, cols, row_ok, n, i, E, pk);
  if (sub == 0 && row_ok) {
    uint32_t* dst = reinterpret_cast<uint32_t*>(idx_packed + i * (d * B / 8) + j0 * B / 8);
    const int words = cols * B / 32;
#pragma unroll
    for (int q = 0; q < WORDS; ++q)
      if (q < words) dst[q] = pk[q];
  }
}

// Wc[:, c0 : c1] -= E[e0 : e0 + k]^T * U[u0 : u0 + k, c0 : c1] (E is [rows][n],
// k a multiple of 64); 64 x 64 output tiles, 4 x 4 outputs per thread, the
// k rows taken 64 at a time through LDS
__global__ void __launch_bounds__(256) k_map_trail(float* __restrict__ Wc, const float* __restrict__ U,
                                                    const float* __restrict__ E, int64_t n, int64_t d, int64_t u0,
                                                    int k, int64_t cbeg, int64_t cend) {
  __shared__ float es[MAP_COLS][MAP_COLS + 4];  // [k][row]
  __shared__ float us[MAP_COLS][MAP_COLS + 4];  // [k][col]
  const int64_t r0 = (int64_t)blockIdx.y * 64, c0 = cbeg + (int64_t)blockIdx.x * 64;
  const int tid = threadIdx.x;
  const int tr = tid / 16, tc = tid % 16;  // rows tr + 16 a, columns 4 tc + b
  float acc[4][4] = {};
  for (int kb = 0; kb < k; kb += MAP_COLS) {
    for (int e = tid; e < 64 * 64; e += 256) {
      const int kk = e / 64, x = e % 64;  // error kb + kk of row r0 + x; U row u0 + kb + kk, column c0 + x
      es[kk][x] = r0 + x < n ? E[(int64_t)(kb + kk) * n + r0 + x] : 0.f;
      us[kk][x] = c0 + x < cend ? U[(u0 + kb + kk) * d + c0 + x] : 0.f;
    }
    __syncthreads();
#pragma unroll 8
    for (int kk = 0; kk < MAP_COLS; ++kk) {
      float ev[4], uv[4];
#pragma unroll
      for (int a = 0; a < 4; ++a) ev[a] = es[kk][tr + 16 * a];
#pragma unroll
      for (int b = 0; b < 4; ++b) uv[b] = us[kk][4 * tc + b];
#pragma unroll
      for (int a = 0; a < 4; ++a)
#pragma unroll
        for (int b = 0; b < 4; ++b) acc[a][b] += ev[a] * uv[b];
    }
    __syncthreads();
  }
#pragma unroll
  for (int a = 0; a < 4; ++a) {
    const int64_t r = r0 + tr + 16 * a;
    if (r >= n) continue;
#pragma unroll
    for (int b = 0; b < 4; ++b) {
      const int64_t c = c0 + 4 * tc + b;
      if (c < cend) Wc[r * d + c] -= acc[a][b];
    }
  }
}

hipError_t map_trail(float* Wc, const float* U, const float* E, const Problem& p, int64_t u0, int k, int64_t cbeg,
                     int64_t cend, hipStream_t s) {
  const dim3 grid((unsigned)((cend - cbeg + 63) / 64), (unsigned)((p.n + 63) / 64));
  hipLaunchKernelGGL(k_map_trail, grid, dim3(256), 0, s, Wc, U, E, p.n, p.d, u0, k, cbeg, cend);
  return hipGetLastError();
}

// The errors of MAP_OUTER columns are kept (E is [MAP_OUTER][n]): inside an
// outer block each 64-column block updates only the rest of the outer block;
// after it, one rank-MAP_OUTER update brings every later column up to date
// (GPTQ's lazy batches, two levels). The later columns are then read and
// written once per outer block instead of once per 64 columns.
constexpr int MAP_OUTER = 512;

template <int B, typename TL>
hipError_t map_run(float* Wc, const float* U, const TL* lut, const Problem& p, uint8_t* idx, float* E, hipStream_t s) {
  for (int64_t ob = 0; ob < p.d; ob += MAP_OUTER) {
    const int64_t oend = p.d - ob < MAP_OUTER ? p.d : ob + MAP_OUTER;
    for (int64_t j0 = ob; j0 < oend; j0 += MAP_COLS) {
      const int cols = (int)(p.d - j0 < MAP_COLS ? p.d - j0 : MAP_COLS);
      float* Eb = E + (j0 - ob) * p.n;
      hipLaunchKernelGGL((k_map_block<B, TL>), dim3((unsigned)((p.n + 15) / 16)), dim3(64), 0, s, Wc, U, lut, p.n,
                         p.d, p.gpr, j0, cols, idx, Eb);
      const int64_t j1 = j0 + cols;
      if (j1 < oend) {
        const hipError_t e = map_trail(Wc, U, Eb, p, j0, MAP_COLS, j1, oend, s);
        if (e != hipSuccess) return e;
      }
    }
    if (oend < p.d) {
      const hipError_t e = map_trail(Wc, U, E, p, ob, (int)(oend - ob), oend, p.d, s);
      if (e != hipSuccess) return e;
    }
  }
  return hipGetLastError();
}

template <typename TL>
hipError_t lloyd_run(const float* W, const float* h, const Problem& p, int iters, TL* lut, hipStream_t s) {
  const dim3 grid((unsigned)((p.n * p.gpr + 3) / 4));
  switch (p.b) {
    case 2: hipLaunchKernelGGL((k_lloyd<4, TL>), grid, dim3(256), 0, s, W, h, p.n, p.d, p.gpr, iters, lut); break;
    case 3: hipLaunchKernelGGL((k_lloyd<8, TL>), grid, dim3(256), 0, s, W, h, p.n, p.d, p.gpr, iters, lut); break;
    default: hipLaunchKernelGGL((k_lloyd<16, TL>), grid, dim3(256), 0, s, W, h, p.n, p.d, p.gpr, iters, lut); break;
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_col_weights(const float* U, int64_t d, float* h, hipStream_t s) {
  hipLaunchKernelGGL(k_col_weights, dim3((unsigned)((d + 63) / 64)), dim3(256), 0, s, U, d, h);
  return hipGetLastError();
}

hipError_t launch_lloyd(const float* W, const float* h, const Problem& p, int iters, void* lut, int lut_dtype,
                        hipStream_t s) {
  if (lut_dtype == DT_F32) return lloyd_run<float>(W, h, p, iters, (float*)lut, s);
  if (lut_dtype == DT_F16) return lloyd_run<half_t>(W, h, p, iters, (half_t*)lut, s);
  return lloyd_run<bf16_t>(W, h, p, iters, (bf16_t*)lut, s);
}

size_t map_workspace_bytes(int64_t n) { return (size_t)n * MAP_OUTER * sizeof(float); }

template <typename TL>
hipError_t map_dispatch(float* Wc, const float* U, const TL* lut, const Problem& p, uint8_t* idx, float* E,
                        hipStream_t s) {
  switch (p.b) {
    case 2: return map_run<2, TL>(Wc, U, lut, p, idx, E, s);
    case 3: return map_run<3, TL>(Wc, U, lut, p, idx, E, s);
    default: return map_run<4, TL>(Wc, U, lut, p, idx, E, s);
  }
}

hipError_t launch_map(float* Wc, const float* U, const void* lut, int lut_dtype, const Problem& p, uint8_t* idx,
                      float* E, hipStream_t s) {
  if (lut_dtype == DT_F32) return map_dispatch<float>(Wc, U, (const float*)lut, p, idx, E, s);
  if (lut_dtype == DT_F16) return map_dispatch<half_t>(Wc, U, (const half_t*)lut, p, idx, E, s);
  return map_dispatch<bf16_t>(Wc, U, (const bf16_t*)lut, p, idx, E, s);
}

}  // namespace skm
