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
// (one wave per row, a lane per column with its column of the block's part
// of U in registers) and writes the packed indices and the block's errors; k_map_trail applies errors to later
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
// columns; its 16 waves take every 16th row (each lane one column, so a wave
// reads 256 contiguous bytes per row), eight rows' loads in flight at a time,
// and the 16 partial sums meet in LDS in wave order.
constexpr int CW_WAVES = 16, CW_UNROLL = 8;
__global__ void __launch_bounds__(CW_WAVES * 64) k_col_weights(const float* __restrict__ U, int64_t d,
                                                                float* __restrict__ h) {
  __shared__ float part[CW_WAVES][64];
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int64_t j = (int64_t)blockIdx.x * 64 + lane;
  const int64_t jc = j < d ? j : d - 1;
  float s = 0.f;
  // rows up to the block's last column (the lanes past their own column add 0)
  const int64_t kend = ((int64_t)blockIdx.x * 64 + 63 < d ? (int64_t)blockIdx.x * 64 + 63 : d - 1) + 1;
  for (int64_t k0 = w; k0 < kend; k0 += CW_WAVES * CW_UNROLL) {
    float u[CW_UNROLL];
#pragma unroll
    for (int a = 0; a < CW_UNROLL; ++a) {
      const int64_t k = k0 + (int64_t)a * CW_WAVES;
      u[a] = (k < kend && k <= j && j < d) ? U[k * d + jc] : 0.f;
    }
#pragma unroll
    for (int a = 0; a < CW_UNROLL; ++a) s += u[a] * u[a];
  }
  part[w][lane] = s;
  __syncthreads();
  if (w == 0 && j < d) {
    float t = 0.f;
#pragma unroll
    for (int q = 0; q < CW_WAVES; ++q) t += part[q][lane];
    h[j] = 1.f / t;
  }
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

// One 64-column block of the mapping sweep, one wave per row (16 rows per
// block). Lane j holds column j0 + j of the block: its compensated weight
// and its column of the block's part of U, in registers. Lane e also holds
// table entry e % K of the (at most two) groups the block spans, so lanes
// 0 .. K-1 hold every entry once, in order. Step c: the owner's weight
// reaches every lane by readlane; every lane takes its entry's distance, and
// a 4-step DPP min over each 16-lane row leaves the smallest in all lanes;
// the lowest lane holding it (ballot, first set bit) is the nearest entry,
// ties going to the lower index. Every lane then subtracts err * U[c][j]
// from its weight (for j <= c that term is zero or the column is done),
// with err = (w_c - q) / U[c][c] (the reciprocal taken once per block).
// Lane c keeps the step's error and the index goes into scalar registers,
// so the errors E [64][n] and the packed indices are written once, at the
// end. Reads the compensated weights Wc[:, j0 : j0 + cols] (all earlier
// blocks' errors applied).
__device__ __forceinline__ float readlane_f(float v, int l) {
  return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), l));
}
template <int CTRL>
__device__ __forceinline__ float dpp_f(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL, 0xF, 0xF, false));
}

template <int B, typename TL>
__global__ void __launch_bounds__(1024) k_map_block(float* __restrict__ Wc, const float* __restrict__ U,
                                                     const TL* __restrict__ lut, int64_t n, int64_t d, int gpr,
                                                     int64_t j0, int cols, uint8_t* __restrict__ idx_packed,
                                                     float* __restrict__ E) {
  constexpr int K = 1 << B;
  __shared__ float ub[MAP_COLS][MAP_COLS];  // U[j0 + c][j0 + j]
  for (int e = threadIdx.x; e < MAP_COLS * MAP_COLS; e += 1024) {
    const int r = e / MAP_COLS, cc = e % MAP_COLS;
    ub[r][cc] = (r < cols && cc < cols) ? U[(j0 + r) * d + j0 + cc] : 0.f;
  }
  __syncthreads();
  const int lane = (int)(threadIdx.x & 63);
  const int64_t i = (int64_t)blockIdx.x * 16 + (threadIdx.x >> 6);
  if (i >= n) return;  // a whole wave; no barrier follows
  float u[MAP_COLS];
#pragma unroll
  for (int c = 0; c < MAP_COLS; ++c) u[c] = ub[c][lane];
  const float rd = lane < cols ? 1.f / ub[lane][lane] : 0.f;
  float w = lane < cols ? Wc[i * d + j0 + lane] : 0.f;
  // the block spans at most two groups, split at a multiple of 32 columns
  const int64_t G = d / gpr;
  const int64_t g0 = j0 / G, g1 = (j0 + 32) / G;
  const float t0 = to_f32(lut[(i * gpr + g0) * K + (lane % K)]);
  const float t1 = to_f32(lut[(i * gpr + (g1 < gpr ? g1 : g0)) * K + (lane % K)]);
  constexpr int WORDS = MAP_COLS * B / 32;
  uint32_t pk[WORDS];
#pragma unroll
  for (int q = 0; q < WORDS; ++q) pk[q] = 0u;
  float ekeep = 0.f;
#pragma unroll
  for (int c = 0; c < MAP_COLS; ++c) {
    if (c < cols) {  // uniform
      const float tv = c < 32 ? t0 : t1;
      const float wv = readlane_f(w, c);
      const float dist = fabsf(wv - tv);
      float mn = fminf(dist, dpp_f<0xB1>(dist));  // quad_perm [1, 0, 3, 2]
      mn = fminf(mn, dpp_f<0x4E>(mn));             // quad_perm [2, 3, 0, 1]
      mn = fminf(mn, dpp_f<0x141>(mn));            // row_half_mirror
      mn = fminf(mn, dpp_f<0x140>(mn));            // row_mirror
      const int a = __builtin_ctzll(__ballot(dist == mn));  // < K: lane a holds entry a
      const float err = (wv - readlane_f(tv, a)) * readlane_f(rd, c);
      ekeep = lane == c ? err : ekeep;
      w -= err * u[c];
      const int p = B * c;
      pk[p >> 5] |= (uint32_t)a << (p & 31);
      if ((p & 31) + B > 32) pk[(p >> 5) + 1] |= (uint32_t)a >> (32 - (p & 31));
    }
  }
  if (lane < cols) E[(int64_t)lane * n + i] = ekeep;
  const int words = cols * B / 32;
  uint32_t v = 0u;
#pragma unroll
  for (int q = 0; q < WORDS; ++q) v = lane == q ? pk[q] : v;
  if (lane < words) reinterpret_cast<uint32_t*>(idx_packed + i * (d * B / 8) + j0 * B / 8)[lane] = v;
}

// Wc[:, c0 : c1] -= E[e0 : e0 + k]^T * U[u0 : u0 + k, c0 : c1] (E is [rows][n],
// k a multiple of 64) on the matrix cores: 64 x 64 output tiles, each wave a
// 32 x 32 quarter as 2 x 2 v_mfma_f32_16x16x4 tiles; the k rows go through
// LDS 64 at a time as [k][row] and [k][col] (the next 64 loaded into
// registers meanwhile), rows padded to 80 floats so the four k rows of an
// operand read land on distinct banks.
constexpr int TRAIL_LD = 80;
__global__ void __launch_bounds__(256) k_map_trail(float* __restrict__ Wc, const float* __restrict__ U,
                                                    const float* __restrict__ E, int64_t n, int64_t d, int64_t u0,
                                                    int k, int64_t cbeg, int64_t cend) {
  __shared__ float es[MAP_COLS][TRAIL_LD];  // [k][row]
  __shared__ float us[MAP_COLS][TRAIL_LD];  // [k][col]
  const int64_t r0 = (int64_t)blockIdx.y * 64, c0 = cbeg + (int64_t)blockIdx.x * 64;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wr = 32 * (wave >> 1), wc = 32 * (wave & 1);  // the wave's quarter
  const int lr = lane & 15, lk = lane >> 4;               // operand row / column, k within the step
  f32x4 acc[2][2];
#pragma unroll
  for (int a = 0; a < 2; ++a)
#pragma unroll
    for (int b = 0; b < 2; ++b) acc[a][b] = f32x4{0.f, 0.f, 0.f, 0.f};
  // the next 64 k rows are loaded into registers while the current ones are
  // multiplied (thread t: k rows t / 64 + 4 q, row / column t % 64)
  const int x = tid & 63, k4 = tid >> 6;
  const bool rok = r0 + x < n, cok = c0 + x < cend;
  float pe[16], pu[16];
  auto fetch = [&](int kb) {
#pragma unroll
    for (int q = 0; q < 16; ++q) {
      const int kk = k4 + 4 * q;
      pe[q] = rok ? E[(int64_t)(kb + kk) * n + r0 + x] : 0.f;
      pu[q] = cok ? U[(u0 + kb + kk) * d + c0 + x] : 0.f;
    }
  };
  fetch(0);
  for (int kb = 0; kb < k; kb += MAP_COLS) {
#pragma unroll
    for (int q = 0; q < 16; ++q) {
      es[k4 + 4 * q][x] = pe[q];
      us[k4 + 4 * q][x] = pu[q];
    }
    __syncthreads();
    if (kb + MAP_COLS < k) fetch(kb + MAP_COLS);
#pragma unroll 4
    for (int kk = 0; kk < MAP_COLS; kk += 4) {
      float av[2], bv[2];
#pragma unroll
      for (int a = 0; a < 2; ++a) av[a] = es[kk + lk][wr + 16 * a + lr];
#pragma unroll
      for (int b = 0; b < 2; ++b) bv[b] = us[kk + lk][wc + 16 * b + lr];
#pragma unroll
      for (int a = 0; a < 2; ++a)
#pragma unroll
        for (int b = 0; b < 2; ++b) acc[a][b] = __builtin_amdgcn_mfma_f32_16x16x4f32(av[a], bv[b], acc[a][b], 0, 0, 0);
    }
    __syncthreads();
  }
  // lane l holds rows 4 (l / 16) + i, column l % 16 of each 16 x 16 tile
#pragma unroll
  for (int a = 0; a < 2; ++a)
#pragma unroll
    for (int b = 0; b < 2; ++b) {
      const int64_t c = c0 + wc + 16 * b + lr;
      if (c >= cend) continue;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int64_t r = r0 + wr + 16 * a + 4 * lk + i;
        if (r < n) Wc[r * d + c] -= acc[a][b][i];
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
      hipLaunchKernelGGL((k_map_block<B, TL>), dim3((unsigned)((p.n + 15) / 16)), dim3(1024), 0, s, Wc, U, lut, p.n,
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
  hipLaunchKernelGGL(k_col_weights, dim3((unsigned)((d + 63) / 64)), dim3(CW_WAVES * 64), 0, s, U, d, h);
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
