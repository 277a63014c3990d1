// The factor of the damped inverse Hessian that sketch construction uses.
//
// SpaLLM section 2.2 ("Learning the sketching matrix") and the Sketch to
// Adapt reply to Concern 1 map each column to the table with the error update
// of Frantar et al., which needs the upper-triangular U with
//   U^T U = (H + damp * mean(diag H) * I)^-1,   H = X^T X of sample inputs.
// With P the exchange matrix (P i = d-1-i) and P H P = L L^T (L lower
// triangular, the Cholesky factor), H^-1 = (P L^-T P)(P L^-1 P), so
// U = P L^-1 P: one Cholesky factorization and one triangular inverse, both
// in float64, in the flipped index space (A = P H P, padded with the
// identity to a multiple of 64).
//
// Blocked, right-looking, 64 x 64 tiles, T = D / 64 steps; step k:
//   diag:   L_kk = chol(A_kk) and Dinv_k = L_kk^-1 (one workgroup, in LDS)
//   panel:  L_ik = A_ik Dinv_k^T (i > k)  and  X_kj = Dinv_k R_kj (j < k)
//   update: A_ij -= L_ik L_jk^T (k < j <= i)  and  R_pj -= L_pk X_kj (p > k, j <= k)
// where X = L^-1 is built block row by block row from R (R_pj starts at 0,
// X_kk = Dinv_k): the forward substitution L X = I taken right-looking, in
// the same steps as the factorization. The off-diagonal blocks of X are kept
// transposed in the (otherwise unused) upper triangle of A: X(a, b) = A[b][a]
// for a and b in different 64-blocks. Within one launch no tile that is
// written is read by another workgroup.
#include "skm_common.h"
#include "skm_launch.h"

namespace skm {

namespace {

constexpr int HF = 64;       // tile size
constexpr int HK = 32;       // k columns per LDS pass of a tile product
constexpr int HS = HK + 2;   // LDS row stride in doubles (272 bytes: 16 rows on distinct banks)

// ---- mean of the diagonal of H -------------------------------------------
__global__ void __launch_bounds__(256) k_hf_mean(const double* __restrict__ H, int64_t d, double* __restrict__ mean) {
  __shared__ double part[256];
  double s = 0.0;
  for (int64_t i = threadIdx.x; i < d; i += 256) s += H[i * d + i];
  part[threadIdx.x] = s;
  __syncthreads();
  for (int w = 128; w > 0; w >>= 1) {
    if ((int)threadIdx.x < w) part[threadIdx.x] += part[threadIdx.x + w];
    __syncthreads();
  }
  if (threadIdx.x == 0) mean[0] = part[0] / (double)d;
}

// ---- A = P (H + damp mean I) P on the lower triangle, identity padding, zero upper triangle
__global__ void __launch_bounds__(256) k_hf_init(const double* __restrict__ H, int64_t d, int64_t D, double damp,
                                                 const double* __restrict__ mean, double* __restrict__ A) {
  const int64_t e = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (e >= D * D) return;
  const int64_t r = e / D, c = e - r * D;
  double v = 0.0;
  if (r >= c) {
    if (r < d) v = H[(d - 1 - r) * d + (d - 1 - c)] + (r == c ? damp * mean[0] : 0.0);
    else v = r == c ? 1.0 : 0.0;
  }
  A[e] = v;
}

// ---- diag: L_kk = chol(A_kk) in place (lower part), Dinv_k = L_kk^-1 ------
// Thread (a, e) = (t / 16, t % 16) holds the 4 x 4 block of rows 4a .. 4a+3
// and columns 4e .. 4e+3, of L and of X = L^-1 (X starts as I), in
// registers. Column c, in one pass behind one barrier: the 16 threads of
// column block c / 4 publish column c of L and the 16 of row block c / 4 row
// c of X (double-buffered in LDS) beside the pivot g = sqrt(L_cc) and 1 / g,
// which the thread holding L_cc worked out during column c - 1 as soon as that
// entry was final (so the square root and division are off the path from one
// barrier to the next); then for r > c
//   L_rc = L_rc / g,  L_rq -= L_rc L_qc / g (q > c),  X_rq -= L_rc X_cq / g,
// while row c sets L_cc = g and X_cq /= g (right-looking Cholesky, and the
// forward substitution L X = I taken with it; entries of L above the diagonal
// are never read for the result). Each thread reads 12 published values per
// column (its rows' and its columns' entries of column c, its columns' of row
// c), as 16-byte pairs. (Rows of 16 entries per thread needed 32 values per
// column, and that LDS traffic set the pace; one wave holding whole rows,
// with no block barrier, was slower still: the column work then runs on one
// SIMD.)
__device__ __forceinline__ void hf_diag(double* __restrict__ A, int64_t D, int k, double* __restrict__ Dinv) {
  __shared__ __attribute__((aligned(16))) double colb[2][HF], rowb[2][HF];
  __shared__ double piv[2][2];
  const int t = threadIdx.x, a = t >> 4, e = t & 15;
  double* Akk = A + (int64_t)k * HF * D + (int64_t)k * HF;
  double l[4][4], x[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int jj = 0; jj < 4; ++jj) {
      l[i][jj] = Akk[(int64_t)(4 * a + i) * D + 4 * e + jj];
      x[i][jj] = (4 * a + i == 4 * e + jj) ? 1.0 : 0.0;
    }
  if (t == 0) {
    const double g0 = sqrt(l[0][0]);
    piv[0][0] = g0;
    piv[0][1] = 1.0 / g0;
  }
  for (int cc = 0; cc < HF / 4; ++cc) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int c = 4 * cc + j, b = j & 1;
      if (e == cc) {
        colb[b][4 * a + 0] = l[0][j];
        colb[b][4 * a + 1] = l[1][j];
        colb[b][4 * a + 2] = l[2][j];
        colb[b][4 * a + 3] = l[3][j];
      }
      if (a == cc) {
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) rowb[b][4 * e + jj] = x[j][jj];
      }
      __syncthreads();
      const double g = piv[b][0], rg = piv[b][1];
      const double2* cb = reinterpret_cast<const double2*>(&colb[b][0]);
      const double2* rb = reinterpret_cast<const double2*>(&rowb[b][0]);
      const double2 cr0 = cb[2 * a], cr1 = cb[2 * a + 1];  // L_rc (unscaled) of this thread's rows
      const double2 cq0 = cb[2 * e], cq1 = cb[2 * e + 1];  // L_qc (unscaled) of its columns
      const double2 xq0 = rb[2 * e], xq1 = rb[2 * e + 1];  // X_cq (unscaled) of its columns
      const double cr[4] = {cr0.x, cr0.y, cr1.x, cr1.y};
      const double cq[4] = {cq0.x, cq0.y, cq1.x, cq1.y};
      const double xq[4] = {xq0.x, xq0.y, xq1.x, xq1.y};
      // the next pivot first: L_{c+1,c+1} is entry ((c+1) % 4, (c+1) % 4) of
      // block ((c+1) / 4, (c+1) / 4), final once this column is applied
      const int i1 = (j + 1) & 3;
      const int b1 = j == 3 ? cc + 1 : cc;
      if (a == b1 && e == b1 && c + 1 < HF) {
        const double f1 = cr[i1] * rg * rg;
        const double v = l[i1][i1] - f1 * cq[i1];
        const double gn = sqrt(v);
        piv[b ^ 1][0] = gn;
        piv[b ^ 1][1] = 1.0 / gn;
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int r = 4 * a + i;
        if (r > c) {
          const double lrc = cr[i] * rg;
          const double f = lrc * rg;
          if (e == cc) l[i][j] = lrc;
#pragma unroll
          for (int jj = 0; jj < 4; ++jj) {
            if (4 * e + jj > c) l[i][jj] -= f * cq[jj];
            x[i][jj] -= f * xq[jj];
          }
        } else if (r == c) {
          if (e == cc) l[i][j] = g;
#pragma unroll
          for (int jj = 0; jj < 4; ++jj) x[i][jj] *= rg;
        }
      }
    }
  }
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int jj = 0; jj < 4; ++jj) {
      const int r = 4 * a + i, q = 4 * e + jj;
      if (q <= r) Akk[(int64_t)r * D + q] = l[i][jj];
    }
  double* dst = Dinv + (int64_t)k * HF * HF;
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int jj = 0; jj < 4; ++jj) dst[(4 * a + i) * HF + 4 * e + jj] = x[i][jj];
}

// the first diagonal block (the later ones are factored by the update of the
// step before, see k_hf_update)
__global__ void __launch_bounds__(256) k_hf_diag(double* __restrict__ A, int64_t D, int k, double* __restrict__ Dinv) {
  hf_diag(A, D, k, Dinv);
}

// A 64 x 64 matrix M in memory: element (r, c) at m + r * rs + c * cs
struct Tile {
  double* m;
  int64_t rs, cs;
};

// C = beta C + sign (P Q) for 64 x 64 tiles. CCOL: C's columns are contiguous
// (cs == 1), so a thread's 16 outputs sit at rows tr + 16 a, columns tc + 16 b
// with tc running fastest over the threads (coalesced stores); otherwise tr
// does. P is staged as [r][k] and Q as [c][k] (16-byte reads of k pairs).
template <bool CCOL>
__device__ __forceinline__ void tile_mul(Tile C, Tile P, Tile Q, double beta, double sign, double* Ps, double* Qs) {
  const int t = threadIdx.x;
  const int tr = CCOL ? (t >> 4) : (t & 15), tc = CCOL ? (t & 15) : (t >> 4);
  double acc[4][4];
#pragma unroll
  for (int a = 0; a < 4; ++a)
#pragma unroll
    for (int b = 0; b < 4; ++b) acc[a][b] = 0.0;
  for (int k0 = 0; k0 < HF; k0 += HK) {
    // 64 x 32 of P and 32 x 64 of Q, consecutive threads on consecutive addresses
#pragma unroll
    for (int q = 0; q < HF * HK / 256; ++q) {
      const int e = t + 256 * q;
      int r, kk;
      if (P.cs == 1) { r = e >> 5; kk = e & 31; } else { r = e & 63; kk = e >> 6; }
      Ps[r * HS + kk] = P.m[(int64_t)r * P.rs + (int64_t)(k0 + kk) * P.cs];
      int c, k2;
      if (Q.cs == 1) { c = e & 63; k2 = e >> 6; } else { c = e >> 5; k2 = e & 31; }
      Qs[c * HS + k2] = Q.m[(int64_t)(k0 + k2) * Q.rs + (int64_t)c * Q.cs];
    }
    __syncthreads();
#pragma unroll 4
    for (int kk = 0; kk < HK; kk += 2) {
      double2 pv[4], qv[4];
#pragma unroll
      for (int a = 0; a < 4; ++a) pv[a] = *reinterpret_cast<const double2*>(Ps + (tr + 16 * a) * HS + kk);
#pragma unroll
      for (int b = 0; b < 4; ++b) qv[b] = *reinterpret_cast<const double2*>(Qs + (tc + 16 * b) * HS + kk);
#pragma unroll
      for (int a = 0; a < 4; ++a)
#pragma unroll
        for (int b = 0; b < 4; ++b) acc[a][b] = fma(pv[a].x, qv[b].x, fma(pv[a].y, qv[b].y, acc[a][b]));
    }
    __syncthreads();
  }
#pragma unroll
  for (int a = 0; a < 4; ++a)
#pragma unroll
    for (int b = 0; b < 4; ++b) {
      double* dst = C.m + (int64_t)(tr + 16 * a) * C.rs + (int64_t)(tc + 16 * b) * C.cs;
      *dst = (beta != 0.0 ? beta * *dst : 0.0) + sign * acc[a][b];
    }
}

__device__ __forceinline__ Tile blk(double* A, int64_t D, int64_t i, int64_t j) {  // block (i, j) of A as stored
  return Tile{A + i * HF * D + j * HF, D, 1};
}
__device__ __forceinline__ Tile blk_t(double* A, int64_t D, int64_t i, int64_t j) {  // (block (j, i) of A)^T
  return Tile{A + j * HF * D + i * HF, 1, D};
}

// ---- panel of step k: blocks b < T-1-k: L_ik = A_ik Dinv_k^T (i = k+1+b);
// the others: X_kj = Dinv_k R_kj (j = b - (T-1-k)), R_kj and X_kj kept transposed
__global__ void __launch_bounds__(256) k_hf_panel(double* __restrict__ A, int64_t D, int T, int k,
                                                  const double* __restrict__ Dinv) {
  __shared__ __attribute__((aligned(16))) double Ps[HF * HS], Qs[HF * HS];
  double* Dk = const_cast<double*>(Dinv) + (int64_t)k * HF * HF;
  const int b = blockIdx.x, nl = T - 1 - k;
  if (b < nl) {
    const int i = k + 1 + b;
    tile_mul<true>(blk(A, D, i, k), blk(A, D, i, k), Tile{Dk, 1, HF}, 0.0, 1.0, Ps, Qs);
  } else {
    const int j = b - nl;
    tile_mul<false>(blk_t(A, D, k, j), Tile{Dk, HF, 1}, blk_t(A, D, k, j), 0.0, 1.0, Ps, Qs);
  }
}

// ---- update of step k: blocks b < N1: A_ij -= L_ik L_jk^T over the trailing
// lower triangle (k < j <= i); the others: R_pj -= L_pk X_kj (p > k, j <= k).
// Block 0 updates the next diagonal tile A_{k+1,k+1} and then factors and
// inverts it (the diagonal step k+1), while the other blocks are still at
// their tiles: no other block of this launch reads that tile or Dinv_{k+1}.
__global__ void __launch_bounds__(256) k_hf_update(double* __restrict__ A, int64_t D, int T, int k,
                                                   double* __restrict__ Dinv) {
  __shared__ __attribute__((aligned(16))) double Ps[HF * HS], Qs[HF * HS];
  const int64_t m = T - k - 1;
  const int64_t n1 = m * (m + 1) / 2;
  const int64_t b = blockIdx.x;
  if (b < n1) {
    // row ip of the trailing triangle holds ip + 1 tiles
    int64_t ip = (int64_t)((sqrt(8.0 * (double)b + 1.0) - 1.0) * 0.5);
    while ((ip + 1) * (ip + 2) / 2 <= b) ++ip;
    while (ip * (ip + 1) / 2 > b) --ip;
    const int64_t jp = b - ip * (ip + 1) / 2;
    const int64_t i = k + 1 + ip, j = k + 1 + jp;
    tile_mul<true>(blk(A, D, i, j), blk(A, D, i, k), blk_t(A, D, k, j), 1.0, -1.0, Ps, Qs);
    if (b == 0) {
      __syncthreads();  // the tile's stores (other threads') before its factorization reads them
      hf_diag(A, D, k + 1, Dinv);
    }
  } else {
    const int64_t b2 = b - n1;
    const int64_t p = k + 1 + b2 / (k + 1), j = b2 % (k + 1);
    double* Dk = Dinv + (int64_t)k * HF * HF;
    const Tile X = j == k ? Tile{Dk, HF, 1} : blk_t(A, D, k, j);
    tile_mul<false>(blk_t(A, D, p, j), blk(A, D, p, k), X, 1.0, -1.0, Ps, Qs);
  }
}

// ---- U[i][j] = X(d-1-i, d-1-j) for i <= j (fp32), 0 below the diagonal;
// 64 x 64 output tiles, transposed through LDS so that reads and writes are
// both contiguous
__global__ void __launch_bounds__(256) k_hf_out(const double* __restrict__ A, int64_t D, int64_t d,
                                                const double* __restrict__ Dinv, float* __restrict__ U) {
  __shared__ float tileU[HF][HF + 1];
  const int64_t tiles = (d + HF - 1) / HF;
  const int64_t I = blockIdx.x / tiles, J = blockIdx.x % tiles;  // U tile rows I, columns J
  const int t = threadIdx.x;
  // read phase: consecutive threads on consecutive output rows i (source a = d-1-i contiguous)
  for (int e = t; e < HF * HF; e += 256) {
    const int ri = e & 63, cj = e >> 6;
    const int64_t i = I * HF + ri, j = J * HF + cj;
    float v = 0.0f;
    if (i < d && j < d && i <= j) {
      const int64_t a = d - 1 - i, bb = d - 1 - j;  // a >= bb
      if (a / HF == bb / HF) v = (float)Dinv[(a / HF) * HF * HF + (a % HF) * HF + (bb % HF)];
      else v = (float)A[bb * D + a];
    }
    tileU[ri][cj] = v;
  }
  __syncthreads();
  for (int e = t; e < HF * HF; e += 256) {
    const int ri = e >> 6, cj = e & 63;
    const int64_t i = I * HF + ri, j = J * HF + cj;
    if (i < d && j < d) U[i * d + j] = tileU[ri][cj];
  }
}

}  // namespace

size_t hessian_factor_workspace_bytes(int64_t d) {
  const int64_t D = (d + HF - 1) / HF * HF, T = D / HF;
  return (size_t)(D * D + T * HF * HF + 32) * sizeof(double);
}

hipError_t launch_hessian_factor(const double* H, int64_t d, double damp, float* U, void* workspace, hipStream_t s) {
  const int64_t D = (d + HF - 1) / HF * HF;
  const int T = (int)(D / HF);
  double* A = static_cast<double*>(workspace);
  double* Dinv = A + D * D;
  double* mean = Dinv + (int64_t)T * HF * HF;
  hipLaunchKernelGGL(k_hf_mean, dim3(1), dim3(256), 0, s, H, d, mean);
  hipLaunchKernelGGL(k_hf_init, dim3((unsigned)((D * D + 255) / 256)), dim3(256), 0, s, H, d, D, damp, mean, A);
  hipLaunchKernelGGL(k_hf_diag, dim3(1), dim3(256), 0, s, A, D, 0, Dinv);
  for (int k = 0; k < T; ++k) {
    // (the diagonal step k + 1 runs in block 0 of the update of step k)
    const int np = (T - 1 - k) + k;
    if (np > 0) hipLaunchKernelGGL(k_hf_panel, dim3((unsigned)np), dim3(256), 0, s, A, D, T, k, Dinv);
    const int64_t m = T - k - 1;
    const int64_t nu = m * (m + 1) / 2 + m * (k + 1);
    if (nu > 0) hipLaunchKernelGGL(k_hf_update, dim3((unsigned)nu), dim3(256), 0, s, A, D, T, k, Dinv);
  }
  const int64_t tiles = (d + HF - 1) / HF;
  hipLaunchKernelGGL(k_hf_out, dim3((unsigned)(tiles * tiles)), dim3(256), 0, s, A, D, d, Dinv, U);
  return hipGetLastError();
}

}  // namespace skm
