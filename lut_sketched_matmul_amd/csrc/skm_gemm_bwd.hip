// Matrix-core backward kernels of the sketched matmul (gfx950):
//
//   dX[t][j]      = sum_i dY[t][i] W[i][j]                      (k_gemm_dx)
//   dLUT[i][g][c] = sum_{j in g, idx[i][j] = c} sum_t dY[t][i] X[t][j]
//                                                              (k_gemm_dlut)
//
// The table gradient is the corrected Eq. (6) of the "Sketch to Adapt"
// discussion (dL/dw = dL/dy (M X)^T) taken row by row: the gradient of every
// virtual parameter W[i][j] is summed into the table entry it maps to. The
// mapping is frozen ("SpaLLM", section 2.3), so there is no index gradient.
// dX is the chain rule through Y = X W^T, needed to train lower layers.
//
// k_gemm_dx: M = tokens (256), N = columns of dX (256), K = weight rows (32
// per step). The weight tile of 32 rows x 256 columns is dequantised once per
// step into a row-major LDS tile and read with gfx950's transposing LDS reads
// (each MFMA B fragment is 8 consecutive rows of one column). Each step brings
// 32 new rows, so the tables (the groups of the column tile, private copy per
// lane slot) are staged every step: loaded three steps ahead, stored two
// steps ahead. k_gemm_dx64 takes 64 rows per step for groups of >= 256
// columns; with b = 4 it looks its weights up in registers (mm::dequant8_b4)
// from a table loaded with each step's index words.
//
// bf16 dY with f16 tables: each token row of dY is prescaled by 2^-e[t]
// while it is converted to f16 (row exponents from the caller's workspace,
// see skm_common.h) and its dX row is multiplied by 2^e[t] when stored; the
// block takes one conversion for all its rows (none, exponent-field add or
// multiply, mm::block_scale_mode), and its prologue, K loop and store are
// compiled once per conversion.
//
// k_gemm_dlut: one block owns 128 rows x one group. For each chunk of up to
// 512 columns of the group it accumulates the dW = dY^T X tile over all
// tokens (K = 32 tokens per step; the operand tiles are stored as loaded,
// [token][row] and [token][column], and read with gfx950's transposing LDS
// reads), then scatter-adds the tile into LDS bins [row][entry] using the
// chunk's indices staged in LDS. Waves own disjoint (row, bin copy) pairs, so
// the bins need no cross-wave atomics and the sums are deterministic; the
// block stores each gradient entry exactly once (no global atomics).
// k_gemm_dlut_dma (whole 32-token steps, the common case) copies the operand
// tiles from global memory into a three-stage LDS ring with global_load_lds
// instead of staging them through registers.
// When the (row block, group) grid alone has fewer blocks than the GPU has
// CUs (e.g. 4096 rows in one group: 32 blocks), the group's columns are split
// into ranges of whole 512-column chunks and, if that is not enough, the
// tokens into ranges: each block then bins one (column range, token range)
// into a partial table of the caller's workspace, and k_dlut_reduce adds the
// partial tables in range order (deterministic, still no atomics).
#include "skm_gemm_common.h"
#include "skm_launch.h"

namespace skm {

namespace {

using namespace mm;

// LDS buffer index of a K-step, known at compile time (buf_tag) or not (buf_rt)
template <int V> struct buf_tag { static constexpr uint32_t value = V; };
struct buf_rt { uint32_t value; };

// ============================================================================
// dX
// ============================================================================
// 8 waves in a 2 (tokens) x 4 (columns) grid, 128 x 64 outputs per wave (4 x 2
// tiles of v_mfma_f32_32x32x16, 16 MFMAs per step); one block per CU; waves
// 0-3 multiply first and stage second, waves 4-7 the other way round, so the
// two waves of a SIMD overlap. LDS:
//   tables [2][NG groups][T entries][64 lane slots] dwords            at 0
//   A  [2][256 tokens][32 rows] dY in the compute dtype (mm::swz rows)
//   Wt [2][32 rows][256 columns + 32 pad] dequantised weights; the row stride
//      is 16 dwords mod 64 banks so the transposing reads are conflict-free
// Staging roles: weight row r = t % 32 of the step, 16-column chunk t / 32
// (16 weights); 16-byte chunk t % 4 of token rows t / 4 and t / 4 + 128 of dY.
// Lane slot s holds the tables of step row s % 32.
constexpr int DX_BM = 256, DX_BN = 256, DX_BK = 32;
constexpr uint32_t DX_RSB = 256u * 2u + 64u;  // 576
constexpr uint32_t DX_TA = DX_BM * DX_BK * 2u;  // 16384
constexpr uint32_t DX_TB = DX_BK * DX_RSB;      // 18432
template <int NG> struct DxLds {
  static constexpr uint32_t T = 0;
  static constexpr uint32_t A = 2u * NG * 16u * 64u * 4u;
  static constexpr uint32_t B = A + 2u * DX_TA;
  static constexpr uint32_t TOTAL = B + 2u * DX_TB;
};

// Per-token factors 2^e of the block's 256 tokens into LDS at 0 (the table
// area, free once the last K-step's barrier has passed), then the factors of
// four consecutive tokens per read.
__device__ __forceinline__ void dx_factors_to_lds(const int32_t* __restrict__ rexp, int64_t m, int64_t m0, int t) {
  if (t < 256) {
    const int64_t tok = m0 + t < m ? m0 + t : m - 1;
    st_w((uint32_t)t * 4u, __builtin_bit_cast(uint32_t, pow2f(rexp[tok])));
  }
  __syncthreads();
}

template <int B> struct DxStage {
  u32x4 y[2];
  uint32_t w[B == 3 ? 3 : (B == 4 ? 2 : 1)];
};

// 16 weights of half hh of a unit -> 8 words of packed consecutive columns
template <int B>
__device__ __forceinline__ void dx_dequant(const uint32_t* w, int hh, uint32_t gk, uint32_t lane4, uint32_t* o) {
  const uint32_t gk4 = gk * 0x01010101u;
  if constexpr (B == 4) {
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const uint32_t ev = (w[j] & 0x0F0F0F0Fu) | gk4;
      const uint32_t od = ((w[j] >> 4) & 0x0F0F0F0Fu) | gk4;
#pragma unroll
      for (int t = 0; t < 4; ++t) o[4 * j + t] = pack2(ld_h(gaddr(ev, lane4, t)), ld_h(gaddr(od, lane4, t)));
    }
  } else if constexpr (B == 2) {
    const uint32_t ev = (w[0] & 0x0F0F0F0Fu) | gk4;
    const uint32_t od = ((w[0] >> 4) & 0x0F0F0F0Fu) | gk4;
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      o[2 * t] = ld_w(gaddr(ev, lane4, t));
      o[2 * t + 1] = ld_w(gaddr(od, lane4, t));
    }
  } else {
    if (hh) {
#pragma unroll
      for (int t = 0; t < 8; ++t) {
        const uint32_t e0 = unit_field<3>(w, 16 + 2 * t), e1 = unit_field<3>(w, 17 + 2 * t);
        o[t] = pack2(ld_h(((gk + e0) << 8) | lane4), ld_h(((gk + e1) << 8) | lane4));
      }
    } else {
#pragma unroll
      for (int t = 0; t < 8; ++t) {
        const uint32_t e0 = unit_field<3>(w, 2 * t), e1 = unit_field<3>(w, 1 + 2 * t);
        o[t] = pack2(ld_h(((gk + e0) << 8) | lane4), ld_h(((gk + e1) << 8) | lane4));
      }
    }
  }
}

// Table words of one thread for one group: lane slot s = t % 64 (step row
// s % 32), part p = t / 64 covers entries 2p, 2p+1 (b = 4 and the b = 2 pair
// table) or, for p < 4, entries 2p, 2p+1 of the b = 3 table.
template <int B> struct DxLutWord { uint32_t v[B == 2 ? 2 : 1]; };

template <int B, typename TL>
__device__ __forceinline__ void dx_lut_load(DxLutWord<B>& L, const TL* lut, int64_t row, bool ok, int gpr, uint32_t g,
                                            int part) {
  constexpr int K = 1 << B;
  const uint16_t* src = reinterpret_cast<const uint16_t*>(lut) + ((int64_t)row * gpr + g) * K;
  if constexpr (B == 2) {
    const u32x2 v = ok ? *reinterpret_cast<const u32x2*>(src) : u32x2{0u, 0u};
    L.v[0] = v.x;
    L.v[1] = v.y;
  } else if constexpr (B == 3) {
    L.v[0] = (ok && part < 4) ? *reinterpret_cast<const uint32_t*>(src + 2 * part) : 0u;
  } else {
    L.v[0] = ok ? *reinterpret_cast<const uint32_t*>(src + 2 * part) : 0u;
  }
}

template <int B>
__device__ __forceinline__ void dx_lut_store(const DxLutWord<B>& L, uint32_t ebase, int part, uint32_t lane4) {
  if constexpr (B == 2) {
    const uint32_t e[4] = {L.v[0] & 0xFFFFu, L.v[0] >> 16, L.v[1] & 0xFFFFu, L.v[1] >> 16};
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int pe = 2 * part + i;  // pair entry a + 4c
      st_w(((ebase + pe) << 8) | lane4, e[pe & 3] | (e[pe >> 2] << 16));
    }
  } else {
    if (B == 3 && part >= 4) return;
    st_w(((ebase + 2u * part) << 8) | lane4, L.v[0] & 0xFFFFu);
    st_w(((ebase + 2u * part + 1u) << 8) | lane4, L.v[0] >> 16);
  }
}

template <int B, int NG, typename TX, typename TL>
__global__ void __launch_bounds__(512, 1)
k_gemm_dx(const TX* __restrict__ dY, const uint8_t* __restrict__ idx_packed, const TL* __restrict__ lut, int64_t m,
          int64_t n, int64_t d, int gpr, uint32_t ug_magic, int64_t mblocks, float* __restrict__ dX,
          const int32_t* __restrict__ rexp) {
  constexpr bool SC = scaled_pair(__is_same(TX, bf16_t), __is_same(TL, half_t));
  // The block's conversion mode of its activation rows (bf16 with f16 tables:
  // block_scale_mode). Everything after it is compiled once per mode (run<MD>),
  // each copy with its own registers: only the kernel arguments cross the
  // dispatch, so the common mode 0 runs the loop 16-bit operands of the table
  // dtype would, and the modes that convert do not squeeze its registers.
  int mode = 0;
  if constexpr (SC) {
    const int64_t mb0 = (int64_t)(blockIdx.x % mblocks) * DX_BM;
    uint32_t flags = 0u;
#pragma unroll
    for (int c = 0; c < 2; ++c) {
      const int64_t tok = mb0 + 128 * c + (threadIdx.x >> 2);
      flags |= scale_flags_of(rexp[tok < m ? tok : m - 1]);
    }
    mode = block_scale_mode(flags, DxLds<NG>::B + DX_TB);
  }
  auto run = [&](auto md) __attribute__((always_inline)) {
    constexpr int MD = decltype(md)::value;
    typedef mfma32<TL> MF;
    typedef DxLds<NG> LDS;
    constexpr uint32_t T = (uint32_t)tab_entries<B>::value;
    extern __shared__ uint32_t smem[];
    (void)smem;

    const int t = threadIdx.x;
    const int lane = t & 63;
    const int wave = t >> 6;
    const uint32_t lane4 = (uint32_t)lane * 4u;
    const int64_t bm = blockIdx.x % mblocks, bn = blockIdx.x / mblocks;
    const int64_t m0 = bm * DX_BM, n0 = bn * DX_BN;  // token / column tile origins
    const bool vec = (n % 8) == 0;
    const int KS = (int)((n + DX_BK - 1) / DX_BK);   // K-steps over the weight rows

    // ---- dequant role: weight row r of the step, 16-column chunk cc
    const int r = t & 31;
    const int cc = t >> 5;
    const int hh = cc & 1;
    const int64_t jc = n0 + 16 * cc;  // first column of the chunk
    const bool col_ok = jc < d;
    const uint32_t u = (uint32_t)((col_ok ? jc : 0) / 32);
    const uint32_t glo = group_of((uint32_t)(n0 / 32), ug_magic);
    const uint32_t ghi = group_of((uint32_t)((n0 + DX_BN < d ? n0 + DX_BN : d) / 32 - 1), ug_magic);
    const int ng = (int)(ghi - glo + 1);  // groups touched by the column tile (<= NG)
    const uint32_t gsel = col_ok ? group_of(u, ug_magic) - glo : 0u;
    const int64_t rbytes = d * B / 8;
    const uint8_t* ucol = idx_packed + (int64_t)u * (4 * B) + (B == 3 ? 0 : hh * 2 * B);
    const uint32_t b_st = (uint32_t)r * DX_RSB + 32u * (uint32_t)cc;
    // ---- table role: lane slot `lane` (row lane % 32 of a step), part = wave
    const int part = wave;
    // ---- dY role: chunk t % 4 of token rows t / 4 + 128 c
    const TX* yrow[2];
    int ye[2] = {0, 0};  // SC: exponents of the two staged token rows
  #pragma unroll
    for (int c = 0; c < 2; ++c) {
      const int64_t tok = m0 + 128 * c + (t >> 2);
      yrow[c] = dY + (tok < m ? tok : m - 1) * n;
      if constexpr (SC && MD != 0) ye[c] = rexp[tok < m ? tok : m - 1];
    }
    float ysc[2] = {1.0f, 1.0f};
    uint32_t yk[2] = {0u, 0u};
  #pragma unroll
    for (int c = 0; c < (int)(sizeof(ye) / sizeof(ye[0])); ++c) {
      if constexpr (MD == 2) ysc[c] = pow2f(-ye[c]);
      if constexpr (MD == 1) yk[c] = exp_add_word(ye[c]);
    }
    (void)ysc;
    (void)yk;
    const uint32_t a_st0 = swz((uint32_t)(t >> 2), (uint32_t)(t & 3));
    const uint32_t a_st1 = swz((uint32_t)(128 + (t >> 2)), (uint32_t)(t & 3));

    auto load_stage = [&](DxStage<B>& S, int j) {
      const int64_t k0 = (int64_t)j * DX_BK;
      const int64_t e0 = k0 + 8 * (t & 3);
  #pragma unroll
      for (int c = 0; c < 2; ++c) {
        if (vec) {
          const bool in = e0 < n;
          const u32x4 v = *reinterpret_cast<const u32x4*>(yrow[c] + (in ? e0 : 0));
          S.y[c] = in ? v : u32x4{0u, 0u, 0u, 0u};
        } else {
          const uint16_t* p = reinterpret_cast<const uint16_t*>(yrow[c]);
  #pragma unroll
          for (int q = 0; q < 4; ++q) {
            const int64_t i = e0 + 2 * q;
            S.y[c][q] = (i < n ? p[i] : 0u) | ((i + 1 < n ? p[i + 1] : 0u) << 16);
          }
        }
      }
      const int64_t row = k0 + r;
      const uint8_t* src = ucol + (row < n ? row : n - 1) * rbytes;
      if constexpr (B == 4) {
        const u32x2 v = *reinterpret_cast<const u32x2*>(src);
        S.w[0] = v.x;
        S.w[1] = v.y;
      } else if constexpr (B == 2) {
        S.w[0] = *reinterpret_cast<const uint32_t*>(src);
      } else {
        const uint32_t* q = reinterpret_cast<const uint32_t*>(src);
        S.w[0] = q[0];
        S.w[1] = q[1];
        S.w[2] = q[2];
      }
    };
    // dequantise / convert tile j into buffer j & 1 (tables of tile j are in
    // table buffer j & 1)
    auto stage = [&](const DxStage<B>& S, int j, auto md) __attribute__((always_inline)) {
      constexpr int MD = decltype(md)::value;
      const uint32_t buf = (uint32_t)(j & 1);
      const bool ok = (int64_t)j * DX_BK + r < n && col_ok;
      uint32_t o[8];
      dx_dequant<B>(S.w, hh, (buf * NG + gsel) * T, lane4, o);
      const uint32_t bb = LDS::B + buf * DX_TB + b_st;
      const u32x4 z = {0u, 0u, 0u, 0u};
      st_q(bb, ok ? u32x4{o[0], o[1], o[2], o[3]} : z);
      st_q(bb + 16u, ok ? u32x4{o[4], o[5], o[6], o[7]} : z);
      const uint32_t ab = LDS::A + buf * DX_TA;
      if constexpr (SC && MD == 2) {
        st_q(ab + a_st0, cvt_quad_scaled(S.y[0], ysc[0]));
        st_q(ab + a_st1, cvt_quad_scaled(S.y[1], ysc[1]));
      } else if constexpr (SC && MD == 1) {
        st_q(ab + a_st0, cvt_quad<TX, TL>(add_quad(S.y[0], yk[0])));
        st_q(ab + a_st1, cvt_quad<TX, TL>(add_quad(S.y[1], yk[1])));
      } else {
        st_q(ab + a_st0, cvt_quad<TX, TL>(S.y[0]));
        st_q(ab + a_st1, cvt_quad<TX, TL>(S.y[1]));
      }
    };
    DxLutWord<B> LW[NG];
    auto lut_load = [&](int j) {
      const int64_t row = (int64_t)j * DX_BK + (lane & 31);
      const bool ok = row < n;
  #pragma unroll
      for (int gs = 0; gs < NG; ++gs)
        if (gs < ng) dx_lut_load<B, TL>(LW[gs], lut, ok ? row : 0, ok, gpr, glo + gs, part);
    };
    auto lut_store = [&](int j) {
      const uint32_t buf = (uint32_t)(j & 1);
  #pragma unroll
      for (int gs = 0; gs < NG; ++gs)
        if (gs < ng) dx_lut_store<B>(LW[gs], (buf * NG + gs) * T, part, lane4);
    };

    // ---- matrix roles
    const int wm = wave & 1, wn = wave >> 1;
    const uint32_t arow = (uint32_t)(128 * wm + (lane & 31));
    const uint32_t khalf = (uint32_t)(lane >> 5);
    f32x16 acc[4][2];
  #pragma unroll
    for (int i = 0; i < 4; ++i)
  #pragma unroll
      for (int jj = 0; jj < 2; ++jj) zero16(acc[i][jj]);
    auto load_frags = [&](u32x4* fa, u32x4* fb, int k, int ks) {
      const uint32_t buf = (uint32_t)(k & 1);
      const uint32_t ch = (uint32_t)(2 * ks) + khalf;
  #pragma unroll
      for (int i = 0; i < 4; ++i) fa[i] = ld_q(LDS::A + buf * DX_TA + swz(arow + 32u * i, ch));
  #pragma unroll
      for (int jj = 0; jj < 2; ++jj)
        fb[jj] = ld_frag_tr(LDS::B + buf * DX_TB + 16u * ks * DX_RSB + (64u * wn + 32u * jj) * 2u, DX_RSB,
                            (uint32_t)lane);
    };
    auto mfma_step = [&](int k) {
      u32x4 fa0[4], fb0[2], fa1[4], fb1[2];
      load_frags(fa0, fb0, k, 0);
  #pragma unroll
      for (int i = 0; i < 4; ++i)
  #pragma unroll
        for (int jj = 0; jj < 2; ++jj) acc[i][jj] = MF::run(fa0[i], fb0[jj], acc[i][jj]);
      load_frags(fa1, fb1, k, 1);
  #pragma unroll
      for (int i = 0; i < 4; ++i)
  #pragma unroll
        for (int jj = 0; jj < 2; ++jj) acc[i][jj] = MF::run(fa1[i], fb1[jj], acc[i][jj]);
      // first half's 8 reads (4 A + 2 x 2 transposing B), then its MFMAs
      // interleaved with the second half's reads, then the second half's MFMAs
      __builtin_amdgcn_sched_group_barrier(0x100, 8, 0);
  #pragma unroll
      for (int q = 0; q < 4; ++q) {
        __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
        __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
      }
      __builtin_amdgcn_sched_group_barrier(0x008, 8, 0);
      __builtin_amdgcn_sched_barrier(0);
    };
    // staging work of step k: the tables of tile k+2 (loaded during step k-1)
    // go to LDS and those of tile k+3 are loaded; tile k+1 goes from Sn into
    // LDS and Sn is refilled with tile k+3
    auto stage_step = [&](int k, DxStage<B>& Sn, auto md) __attribute__((always_inline)) {
      if (k + 2 < KS) lut_store(k + 2);
      if (k + 3 < KS) lut_load(k + 3);
      if (k + 1 < KS) {
        stage(Sn, k + 1, md);
        if (k + 3 < KS) load_stage(Sn, k + 3);
      }
    };
    const bool mfma_first = wave < 4;
    DxStage<B> S0, S1;
    auto step = [&](int k, DxStage<B>& Sn, auto md) __attribute__((always_inline)) {
      if (mfma_first) {
        mfma_step(k);
        stage_step(k, Sn, md);
      } else {
        stage_step(k, Sn, md);
        __builtin_amdgcn_sched_barrier(0);
        mfma_step(k);
      }
      __syncthreads();
    };

    // ---- prologue: tables of tiles 0 and 1, tile 0 staged, tiles 1 and 2 in
    // registers
    lut_load(0);
    load_stage(S0, 0);
    if (KS > 1) load_stage(S1, 1);
    lut_store(0);
    if (KS > 1) {
      lut_load(1);
      lut_store(1);
    }
    if (KS > 2) lut_load(2);
    __syncthreads();
    stage(S0, 0, md);
    if (KS > 2) load_stage(S0, 2);
    __syncthreads();

    int k = 0;
    for (; k + 1 < KS; k += 2) {
      step(k, S1, md);
      step(k + 1, S0, md);
    }
    if (k < KS) step(k, S1, md);

    if constexpr (SC && MD != 0) dx_factors_to_lds(rexp, m, m0, t);  // block-uniform
  #pragma unroll
    for (int i = 0; i < 4; ++i) {
      f32x4 uq[4] = {};
      if constexpr (SC && MD != 0) {
  #pragma unroll
        for (int q = 0; q < 4; ++q) uq[q] = ld_f4((uint32_t)(128 * wm + 32 * i + 8 * q + 4 * (lane >> 5)) * 4u);
      }
  #pragma unroll
      for (int jj = 0; jj < 2; ++jj) {
        const int64_t col = n0 + 64 * wn + 32 * jj + (lane & 31);
        if (col >= d) continue;
  #pragma unroll
        for (int e = 0; e < 16; ++e) {
          const int64_t tok = m0 + 128 * wm + 32 * i + 8 * (e >> 2) + 4 * (lane >> 5) + (e & 3);
          float v = acc[i][jj][e];
          if constexpr (SC && MD != 0) v *= uq[e >> 2][e & 3];
          if (tok < m) dX[tok * d + col] = v;
        }
      }
    }
  };
  if (!SC || mode == 0) run(mode_tag<0>{});
  else if (mode == 1) run(mode_tag<1>{});
  else run(mode_tag<2>{});
}

// dX with 64 weight rows per step, for groups of >= 256 columns (a 256-column
// tile then touches at most 2 groups). Same roles as k_gemm_dx, but each
// step's dY tile has 128-byte token rows (8 lanes read one row's full cache
// line), each thread dequantises one whole 32-column unit of one weight row
// (lane slot = row of the step, so the table copies are unchanged), every wave
// issues 32 MFMAs per step, and one register stage suffices (the loads of
// tile k+2 have a whole step to arrive). LDS: tables [2][2][T][64] at 0, A
// [2][256 tokens][64 rows] (128-byte rows, mm::swz128), Wt [2][64 rows][256
// columns + 32 pad].
constexpr int D6_BK = 64;
constexpr uint32_t D6_TA = 256u * 64u * 2u;               // 32768
constexpr uint32_t D6_TB = 64u * DX_RSB;                  // 36864
constexpr uint32_t D6_A = 2u * 2u * 16u * 64u * 4u;       // 16384
constexpr uint32_t D6_B = D6_A + 2u * D6_TA;              // 81920
constexpr uint32_t D6_LDS = D6_B + 2u * D6_TB;            // 155648

template <int B> struct Dx6Stage {
  u32x4 y[4];
  uint32_t w[B == 3 ? 3 : (B == 4 ? 4 : 2)];
  uint32_t lut[B == 4 ? 8 : 1];  // b = 4: the row's table for the thread's group
};

template <int B, typename TX, typename TL>
__global__ void __launch_bounds__(512, 1)
k_gemm_dx64(const TX* __restrict__ dY, const uint8_t* __restrict__ idx_packed, const TL* __restrict__ lut,
            int64_t m, int64_t n, int64_t d, int gpr, uint32_t ug_magic, int64_t mblocks, float* __restrict__ dX,
            const int32_t* __restrict__ rexp) {
  constexpr bool SC = scaled_pair(__is_same(TX, bf16_t), __is_same(TL, half_t));
  // The block's conversion mode of its activation rows (bf16 with f16 tables:
  // block_scale_mode). Everything after it is compiled once per mode (run<MD>),
  // each copy with its own registers: only the kernel arguments cross the
  // dispatch, so the common mode 0 runs the loop 16-bit operands of the table
  // dtype would, and the modes that convert do not squeeze its registers.
  int mode = 0;
  if constexpr (SC) {
    const int64_t mb0 = (int64_t)(blockIdx.x % mblocks) * DX_BM;
    uint32_t flags = 0u;
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const int64_t tok = mb0 + 64 * c + (threadIdx.x >> 3);
      flags |= scale_flags_of(rexp[tok < m ? tok : m - 1]);
    }
    mode = block_scale_mode(flags, D6_B + D6_TB);
  }
  auto run = [&](auto md) __attribute__((always_inline)) {
    constexpr int MD = decltype(md)::value;
    typedef mfma32<TL> MF;
    constexpr int NG = 2;
    constexpr uint32_t T = (uint32_t)tab_entries<B>::value;
    extern __shared__ uint32_t smem[];
    (void)smem;

    const int t = threadIdx.x;
    const int lane = t & 63;
    const int wave = t >> 6;
    const uint32_t lane4 = (uint32_t)lane * 4u;
    const int64_t bm = blockIdx.x % mblocks, bn = blockIdx.x / mblocks;
    const int64_t m0 = bm * DX_BM, n0 = bn * DX_BN;
    const bool vec = (n % 8) == 0;
    const int KS = (int)((n + D6_BK - 1) / D6_BK);

    // ---- dequant role: weight row r = lane of the step, unit uu = wave of the
    // column tile (32 columns, 4 * B bytes). b = 4 keeps the tables in
    // registers instead (mm::dequant8_b4); then 4 adjacent lanes take 4
    // adjacent units of one row (64 contiguous index bytes per row), 16 rows
    // per wave.
    const int r = B == 4 ? 16 * (wave & 3) + (lane >> 2) : lane;
    const int uu = B == 4 ? 4 * (wave >> 2) + (lane & 3) : wave;
    const int64_t jc = n0 + 32 * uu;
    const bool col_ok = jc < d;
    const uint32_t u = (uint32_t)((col_ok ? jc : 0) / 32);
    const uint32_t glo = group_of((uint32_t)(n0 / 32), ug_magic);
    const uint32_t ghi = group_of((uint32_t)((n0 + DX_BN < d ? n0 + DX_BN : d) / 32 - 1), ug_magic);
    const int ng = (int)(ghi - glo + 1);
    const uint32_t gsel = col_ok ? group_of(u, ug_magic) - glo : 0u;
    const int64_t rbytes = d * B / 8;
    const uint8_t* ucol = idx_packed + (int64_t)u * (4 * B);
    const uint32_t b_st = (uint32_t)r * DX_RSB + 64u * (uint32_t)uu;
    const int part = wave;
    // ---- dY role: chunk t % 8 of token rows t / 8 + 64 c
    const TX* yrow[4];
    int ye[4] = {0, 0, 0, 0};  // SC: exponents of the four staged token rows
  #pragma unroll
    for (int c = 0; c < 4; ++c) {
      const int64_t tok = m0 + 64 * c + (t >> 3);
      yrow[c] = dY + (tok < m ? tok : m - 1) * n;
      if constexpr (SC && MD != 0) ye[c] = rexp[tok < m ? tok : m - 1];
    }
    float ysc[4] = {1.0f, 1.0f, 1.0f, 1.0f};
    uint32_t yk[4] = {0u, 0u, 0u, 0u};
  #pragma unroll
    for (int c = 0; c < (int)(sizeof(ye) / sizeof(ye[0])); ++c) {
      if constexpr (MD == 2) ysc[c] = pow2f(-ye[c]);
      if constexpr (MD == 1) yk[c] = exp_add_word(ye[c]);
    }
    (void)ysc;
    (void)yk;

    const uint8_t* urow = ucol + (int64_t)r * rbytes;  // row r of step 0
    // b = 4: the table of (row, this thread's group), 16 entries
    const uint32_t gabs = glo + gsel;
    auto load_tab = [&](Dx6Stage<B>& S, int64_t row) {
      if constexpr (B == 4) {
        const u32x4* tp = reinterpret_cast<const u32x4*>(reinterpret_cast<const uint16_t*>(lut) +
                                                          (row * gpr + gabs) * 16);
        const u32x4 a = tp[0], b = tp[1];
        S.lut[0] = a.x; S.lut[1] = a.y; S.lut[2] = a.z; S.lut[3] = a.w;
        S.lut[4] = b.x; S.lut[5] = b.y; S.lut[6] = b.z; S.lut[7] = b.w;
      }
    };
    auto load_stage = [&](Dx6Stage<B>& S, int j) {
      const int64_t k0 = (int64_t)j * D6_BK;
      const int64_t e0 = k0 + 8 * (t & 7);
      if (vec && k0 + D6_BK <= n) {  // wave-uniform: every row of the step exists
  #pragma unroll
        for (int c = 0; c < 4; ++c) S.y[c] = *reinterpret_cast<const u32x4*>(yrow[c] + e0);
        const uint8_t* src = urow + k0 * rbytes;
        if constexpr (B == 4) {
          const u32x4 v = *reinterpret_cast<const u32x4*>(src);
          S.w[0] = v.x; S.w[1] = v.y; S.w[2] = v.z; S.w[3] = v.w;
          load_tab(S, k0 + r);
        } else if constexpr (B == 2) {
          const u32x2 v = *reinterpret_cast<const u32x2*>(src);
          S.w[0] = v.x; S.w[1] = v.y;
        } else {
          const uint32_t* q = reinterpret_cast<const uint32_t*>(src);
          S.w[0] = q[0]; S.w[1] = q[1]; S.w[2] = q[2];
        }
        return;
      }
  #pragma unroll
      for (int c = 0; c < 4; ++c) {
        if (vec) {
          const bool in = e0 < n;
          const u32x4 v = *reinterpret_cast<const u32x4*>(yrow[c] + (in ? e0 : 0));
          S.y[c] = in ? v : u32x4{0u, 0u, 0u, 0u};
        } else {
          const uint16_t* pp = reinterpret_cast<const uint16_t*>(yrow[c]);
  #pragma unroll
          for (int q = 0; q < 4; ++q) {
            const int64_t i = e0 + 2 * q;
            S.y[c][q] = (i < n ? pp[i] : 0u) | ((i + 1 < n ? pp[i + 1] : 0u) << 16);
          }
        }
      }
      const int64_t row = k0 + r;
      const uint8_t* src = ucol + (row < n ? row : n - 1) * rbytes;
      if constexpr (B == 4) {
        const u32x4 v = *reinterpret_cast<const u32x4*>(src);
        S.w[0] = v.x; S.w[1] = v.y; S.w[2] = v.z; S.w[3] = v.w;
        load_tab(S, row < n ? row : n - 1);
      } else if constexpr (B == 2) {
        const u32x2 v = *reinterpret_cast<const u32x2*>(src);
        S.w[0] = v.x; S.w[1] = v.y;
      } else {
        const uint32_t* q = reinterpret_cast<const uint32_t*>(src);
        S.w[0] = q[0]; S.w[1] = q[1]; S.w[2] = q[2];
      }
    };
    // activation chunk c of the thread sits 64 rows = 8 KB after chunk 0 (the
    // swizzle repeats every 16 rows); the buffer (bufc) is known at compile
    // time, so every write is a register plus an immediate
    const uint32_t ast = D6_A + swz128((uint32_t)(t >> 3), (uint32_t)(t & 7));
    const uint32_t bst = D6_B + b_st;
    auto stage = [&](const Dx6Stage<B>& S, int j, auto md, auto bufc) __attribute__((always_inline)) {
      constexpr int MD = decltype(md)::value;
      const uint32_t buf = bufc.value;
      const bool ok = (int64_t)j * D6_BK + r < n && col_ok;
      const u32x4 z = {0u, 0u, 0u, 0u};
      if constexpr (B == 4) {
        // columns of each 8-column chunk in the order of mm::dequant8_b4 (undone
        // when dX is stored)
        mm::Planes16 P;
        mm::planes16(S.lut, P);
  #pragma unroll
        for (int q = 0; q < 4; ++q) st_q(bst + buf * D6_TB + 16u * q, ok ? mm::dequant8_b4(S.w[q], P) : z);
      } else {
      const uint32_t gk = (buf * NG + gsel) * T;
      uint32_t o0[8], o1[8];
      if constexpr (B == 3) {
        dx_dequant<B>(S.w, 0, gk, lane4, o0);
        dx_dequant<B>(S.w, 1, gk, lane4, o1);
      } else {
        dx_dequant<B>(S.w, 0, gk, lane4, o0);
        dx_dequant<B>(S.w + (B == 4 ? 2 : 1), 1, gk, lane4, o1);
      }
      st_q(bst + buf * D6_TB, ok ? u32x4{o0[0], o0[1], o0[2], o0[3]} : z);
      st_q(bst + buf * D6_TB + 16u, ok ? u32x4{o0[4], o0[5], o0[6], o0[7]} : z);
      st_q(bst + buf * D6_TB + 32u, ok ? u32x4{o1[0], o1[1], o1[2], o1[3]} : z);
      st_q(bst + buf * D6_TB + 48u, ok ? u32x4{o1[4], o1[5], o1[6], o1[7]} : z);
      }
  #pragma unroll
      for (int c = 0; c < 4; ++c) {
        const uint32_t a = ast + buf * D6_TA + 8192u * c;
        if constexpr (SC && MD == 2) st_q(a, cvt_quad_scaled(S.y[c], ysc[c]));
        else if constexpr (SC && MD == 1) st_q(a, cvt_quad<TX, TL>(add_quad(S.y[c], yk[c])));
        else st_q(a, cvt_quad<TX, TL>(S.y[c]));
      }
    };
    DxLutWord<B> LW[NG];
    auto lut_load = [&](int j) {
      const int64_t row = (int64_t)j * D6_BK + lane;
      const bool ok = row < n;
  #pragma unroll
      for (int gs = 0; gs < NG; ++gs)
        if (gs < ng) dx_lut_load<B, TL>(LW[gs], lut, ok ? row : 0, ok, gpr, glo + gs, part);
    };
    auto lut_store = [&](int j) {
      const uint32_t buf = (uint32_t)(j & 1);
  #pragma unroll
      for (int gs = 0; gs < NG; ++gs)
        if (gs < ng) dx_lut_store<B>(LW[gs], (buf * NG + gs) * T, part, lane4);
    };

    // ---- matrix roles
    const int wm = wave & 1, wn = wave >> 1;
    const uint32_t arow = (uint32_t)(128 * wm + (lane & 31));
    const uint32_t khalf = (uint32_t)(lane >> 5);
    f32x16 acc[4][2];
  #pragma unroll
    for (int i = 0; i < 4; ++i)
  #pragma unroll
      for (int jj = 0; jj < 2; ++jj) zero16(acc[i][jj]);
    // Read addresses in buffer 0: A fragment rows of quarter ks (fragments 32
    // rows apart are 4 KB apart), and the lane's element of the transposing
    // weight reads (as ld_frag_tr places it). Buffer, quarter and fragment
    // are compile-time offsets added to these registers.
    uint32_t ard[4];
  #pragma unroll
    for (int ks = 0; ks < 4; ++ks) ard[ks] = D6_A + swz128(arow, (uint32_t)(2 * ks) + khalf);
    const uint32_t ls = (uint32_t)lane & 15u;
    const uint32_t btr = D6_B + (8u * ((uint32_t)lane >> 5) + (ls >> 2)) * DX_RSB +
                         (16u * (((uint32_t)lane >> 4) & 1u) + 4u * (ls & 3u)) * 2u + 128u * (uint32_t)wn;
    auto load_frags = [&](u32x4* fa, u32x4* fb, uint32_t buf, int ks) __attribute__((always_inline)) {
  #pragma unroll
      for (int i = 0; i < 4; ++i) fa[i] = ld_q(ard[ks] + buf * D6_TA + 4096u * i);
  #pragma unroll
      for (int jj = 0; jj < 2; ++jj) {
        const uint32_t a = btr + buf * D6_TB + 16u * ks * DX_RSB + 64u * jj;
        const u32x2 lo = ld_tr(a), hi = ld_tr(a + 4u * DX_RSB);
        fb[jj] = u32x4{lo.x, lo.y, hi.x, hi.y};
      }
    };
    // four 16-row quarters: each quarter's fragment reads are interleaved with
    // the previous quarter's MFMAs (raising the wave priority of this phase, as
    // the forward kernels do, measured no change here)
    auto mfma_step = [&](auto bufc) __attribute__((always_inline)) {
      const uint32_t buf = bufc.value;
      u32x4 fa[4][4], fb[4][2];
  #pragma unroll
      for (int ks = 0; ks < 4; ++ks) load_frags(fa[ks], fb[ks], buf, ks);
  #pragma unroll
      for (int ks = 0; ks < 4; ++ks)
  #pragma unroll
        for (int i = 0; i < 4; ++i)
  #pragma unroll
          for (int jj = 0; jj < 2; ++jj) acc[i][jj] = MF::run(fa[ks][i], fb[ks][jj], acc[i][jj]);
      __builtin_amdgcn_sched_group_barrier(0x100, 8, 0);
  #pragma unroll
      for (int ks = 1; ks < 4; ++ks) {
  #pragma unroll
        for (int q = 0; q < 4; ++q) {
          __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
          __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
        }
      }
      __builtin_amdgcn_sched_group_barrier(0x008, 8, 0);
      __builtin_amdgcn_sched_barrier(0);
    };
    Dx6Stage<B> S;
    // staging work of step k: tables of tile k+2 to LDS, tables of tile k+3
    // loaded; tile k+1 from S into LDS, S refilled with tile k+2
    auto stage_step = [&](int k, auto md, auto bufc) __attribute__((always_inline)) {
      if constexpr (B != 4) {
        if (k + 2 < KS) lut_store(k + 2);
        if (k + 3 < KS) lut_load(k + 3);
      }
      if (k + 1 < KS) {
        stage(S, k + 1, md, bufc);
        if (k + 2 < KS) load_stage(S, k + 2);
      }
    };
    const bool mfma_first = wave < 4;

    // ---- prologue
    if constexpr (B != 4) lut_load(0);
    load_stage(S, 0);
    if constexpr (B != 4) {
      lut_store(0);
      if (KS > 1) {
        lut_load(1);
        lut_store(1);
      }
      if (KS > 2) lut_load(2);
      __syncthreads();
    }
    stage(S, 0, md, buf_tag<0>{});
    if (KS > 1) load_stage(S, 1);
    __syncthreads();

    // step k multiplies buffer k & 1 and stages the other (a one-step loop:
    // unrolled by two, with compile-time buffer offsets, it measured slower)
    auto step = [&](int k, auto cur, auto nxt) __attribute__((always_inline)) {
      if (mfma_first) {
        mfma_step(cur);
        stage_step(k, md, nxt);
      } else {
        stage_step(k, md, nxt);
        __builtin_amdgcn_sched_barrier(0);
        mfma_step(cur);
      }
      __syncthreads();
    };
    for (int k = 0; k < KS; ++k) step(k, buf_rt{(uint32_t)(k & 1)}, buf_rt{(uint32_t)((k + 1) & 1)});

    if constexpr (SC && MD != 0) dx_factors_to_lds(rexp, m, m0, t);  // block-uniform
  #pragma unroll
    for (int i = 0; i < 4; ++i) {
      f32x4 uq[4] = {};
      if constexpr (SC && MD != 0) {
  #pragma unroll
        for (int q = 0; q < 4; ++q) uq[q] = ld_f4((uint32_t)(128 * wm + 32 * i + 8 * q + 4 * (lane >> 5)) * 4u);
      }
  #pragma unroll
      for (int jj = 0; jj < 2; ++jj) {
        // b = 4: tile column p holds column (p & ~7) + (2 (p & 3) | (p & 7) >> 2)
        const int p = 64 * wn + 32 * jj + (lane & 31);
        const int pc = B == 4 ? (p & ~7) | ((p & 3) << 1) | ((p >> 2) & 1) : p;
        const int64_t col = n0 + pc;
        if (col >= d) continue;
  #pragma unroll
        for (int e = 0; e < 16; ++e) {
          const int64_t tok = m0 + 128 * wm + 32 * i + 8 * (e >> 2) + 4 * (lane >> 5) + (e & 3);
          float v = acc[i][jj][e];
          if constexpr (SC && MD != 0) v *= uq[e >> 2][e & 3];
          if (tok < m) dX[tok * d + col] = v;
        }
      }
    }
  };
  if (!SC || mode == 0) run(mode_tag<0>{});
  else if (mode == 1) run(mode_tag<1>{});
  else run(mode_tag<2>{});
}

// ============================================================================
// dLUT
// ============================================================================
// 8 waves in a 2 (rows) x 4 (columns) grid, 64 x 128 outputs per wave (2 x 4
// tiles of v_mfma_f32_32x32x16, 16 MFMAs per step); one block per CU. In each
// step waves 0-3 multiply first and then stage the next tiles, waves 4-7 the
// other way round, so the two waves of a SIMD overlap. Operand tiles are
// stored as loaded: Yt[token][row] (dY, 128 values) and Xt[token][col] (X, 512
// values), each row padded by 64 bytes (row stride = 16 dwords mod 64 banks)
// so the 4 rows x 2 column halves read by one 32-lane pass of
// ds_read_b64_tr_b16 fall in distinct banks. The raw tiles of step k+2 are
// loaded into registers during step k.
constexpr int DL_BM = 128, DL_BN = 512, DL_BK = 32;
constexpr uint32_t DL_RSA = 128u * 2u + 64u;                 // 320
constexpr uint32_t DL_RSB = 512u * 2u + 64u;                 // 1088
constexpr uint32_t DL_TA = DL_BK * DL_RSA;                   // 10240
constexpr uint32_t DL_TB = DL_BK * DL_RSB;                   // 34816
constexpr uint32_t DL_STAGE = DL_TA + DL_TB;                 // 45056: one buffer of both tiles
// bins: [4 copies][128 rows][24] fp32 (16 entries used). The row stride of 24
// floats puts rows i and i+4 - the two halves of a wave's scatter - on
// opposite halves of the 64 banks.
constexpr uint32_t DL_BRS = 24;                                   // floats per bin row
constexpr uint32_t DL_BCOPY = 128u * DL_BRS * 4u;                 // 12288 bytes per copy
constexpr uint32_t DL_BINS = 2u * DL_STAGE;                       // 90112
constexpr uint32_t DL_LDS = DL_BINS + 4u * DL_BCOPY;              // 139264
// during binning the chunk's packed indices, [128 rows][64 * B bytes], sit at 0
constexpr uint32_t DL_IRS = 256u;                            // index row stride (b <= 4)

// 8 consecutive 16-bit values p[e0 .. e0+7] (zero at or past `lim`).
// VEC: rows are 16-byte aligned and `lim` is a multiple of 8, so a chunk is
// either wholly inside (one 16-byte load) or wholly outside (zeros).
template <bool VEC, typename TS>
__device__ __forceinline__ u32x4 dl_load8(const TS* rowp, int64_t e0, int64_t lim) {
  if constexpr (VEC) {
    const bool in = e0 < lim;
    const u32x4 v = *reinterpret_cast<const u32x4*>(rowp + (in ? e0 : 0));
    return in ? v : u32x4{0u, 0u, 0u, 0u};
  }
  const uint16_t* p = reinterpret_cast<const uint16_t*>(rowp);
  u32x4 v;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int64_t i = e0 + 2 * q;
    const uint32_t lo = i < lim ? p[i] : 0u;
    const uint32_t hi = i + 1 < lim ? p[i + 1] : 0u;
    v[q] = lo | (hi << 16);
  }
  return v;
}

// field j of the packed row staged at LDS byte address `row`
template <int B>
__device__ __forceinline__ uint32_t dl_field(uint32_t row, uint32_t j) {
  const uint32_t bit = j * (uint32_t)B;
  const uint32_t w = ld_w(row + ((bit >> 5) << 2));
  const uint32_t off = bit & 31u;
  if constexpr (B == 3) {
    if (off > 29u) {
      const uint32_t w2 = ld_w(row + ((bit >> 5) << 2) + 4u);
      return __builtin_amdgcn_alignbit(w2, w, off) & 7u;
    }
  }
  return (w >> off) & ((1u << B) - 1u);
}

// Stage this chunk's packed indices (128 rows x 16*B dwords, columns past the
// group read as 0) at LDS 0, row stride DL_IRS.
template <int B>
__device__ __forceinline__ void dl_stage_indices(const uint8_t* __restrict__ idx_packed, int64_t i0, int64_t n,
                                                 int64_t d, int64_t j0, int64_t jend, int t) {
  const int64_t units = (jend - j0) / 32 < DL_BN / 32 ? (jend - j0) / 32 : DL_BN / 32;
  for (int q = t; q < 128 * 16 * B; q += 512) {
    const int row = q / (16 * B), wd = q % (16 * B);
    const int64_t grow = i0 + row < n ? i0 + row : n - 1;
    const uint32_t* src = reinterpret_cast<const uint32_t*>(idx_packed + grow * (d * B / 8) + j0 * B / 8);
    st_w((uint32_t)row * DL_IRS + (uint32_t)wd * 4u, (wd / B) < units ? src[wd] : 0u);
  }
}

// Scatter-add a wave's finished 64 x 128 dW tile (acc[a][b]: D[i][j] with
// i = 64 wm + 32 a + 8 (e/4) + 4 (lane/32) + e%4, j = 128 wn + 32 b + lane%32)
// into its bin copy at `binbase` ([128 rows][brs] fp32), using the indices
// staged by dl_stage_indices. Branch-free: an entry outside the matrix adds 0
// to a bin that is never stored (rows past n) or to entry 0 (columns past the
// group, whose staged indices are 0). Fully unrolled so that the accumulators
// stay in registers; the scheduling fences keep the index reads from being
// hoisted all at once, and an opaque copy of the lane id keeps the compiler
// from hoisting the 128 bin addresses out of the chunk loop (where they would
// stay live across the K loop).
template <int B>
__device__ __forceinline__ void dl_scatter(const f32x16 (&acc)[2][4], uint32_t lane, int wm, int wn, int64_t i0,
                                           int64_t n, int64_t j0, int64_t jend, uint32_t binbase, uint32_t brs) {
  uint32_t bl = lane;
  asm volatile("" : "+v"(bl));
#pragma unroll
  for (int a = 0; a < 2; ++a)
#pragma unroll
    for (int b = 0; b < 4; ++b) {
      const uint32_t j = 128u * wn + 32u * b + (bl & 31u);
      const bool j_ok = j0 + (int64_t)j < jend;
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const uint32_t i = 64u * wm + 32u * a + 8u * (e >> 2) + 4u * (bl >> 5) + (e & 3);
        const float v = (j_ok && i0 + (int64_t)i < n) ? acc[a][b][e] : 0.0f;
        const uint32_t c = dl_field<B>(i * DL_IRS, j);
        __hip_atomic_fetch_add((lds_f32*)(uintptr_t)(binbase + (i * brs + c) * 4u), v, __ATOMIC_RELAXED,
                               __HIP_MEMORY_SCOPE_WORKGROUP);
        if ((e & 3) == 3) __builtin_amdgcn_sched_barrier(0);
      }
    }
}

// One store per gradient entry of the block's rows and group: the four bin
// copies at `bins` (stride `bcopy` bytes, rows of `brs` floats) summed in a
// fixed order.
template <int B>
__device__ __forceinline__ void dl_store_bins(float* __restrict__ dLUT, int64_t i0, int64_t n, int gpr, int g,
                                              uint32_t bins, uint32_t bcopy, uint32_t brs, int accumulate, int t) {
  constexpr int K = 1 << B;
  for (uint32_t q = (uint32_t)t; q < 128u * (uint32_t)K; q += 512u) {
    const uint32_t i = q / K, c = q % K;
    if (i0 + (int64_t)i >= n) continue;
    float s = 0.0f;
#pragma unroll
    for (int w = 0; w < 4; ++w) s += *(const lds_f32*)(uintptr_t)(bins + (uint32_t)w * bcopy + (i * brs + c) * 4u);
    float* dst = dLUT + ((i0 + i) * gpr + g) * K + c;
    *dst = accumulate ? *dst + s : s;
  }
}

// raw operands of one step for one thread: one dY chunk, four X chunks
struct DlStage {
  u32x4 y;
  u32x4 x[4];
};

template <int B, typename TX, bool VEC>
__global__ void __launch_bounds__(512, 1)
k_gemm_dlut(const TX* __restrict__ dY, const TX* __restrict__ X, const uint8_t* __restrict__ idx_packed, int64_t m,
            int64_t n, int64_t d, int gpr, float* __restrict__ dLUT, int accumulate, int tsplits, int csplits,
            int64_t split_tokens, int64_t split_cols, int64_t part_stride) {
  typedef mfma32<TX> MF;
  extern __shared__ uint32_t smem[];
  (void)smem;

  const int t = threadIdx.x;
  const uint32_t lane = (uint32_t)(t & 63);
  const int wave = t >> 6;
  // split (column range, token range; varying slowest, so an XCD's
  // co-resident blocks share it), then the gpr groups of one row block (same
  // dY strip) share an XCD's L2
  const uint32_t lba = xcd_block(blockIdx.x, gridDim.x);
  const uint32_t nb0 = gridDim.x / (uint32_t)(tsplits * csplits);
  const uint32_t sp = lba / nb0, lb = lba % nb0;
  const uint32_t cr = sp / (uint32_t)tsplits;  // column range of the group
  {
    const int64_t tok0 = (int64_t)(sp % (uint32_t)tsplits) * split_tokens;
    dY += tok0 * n;
    X += tok0 * d;
    m = m - tok0 < split_tokens ? m - tok0 : split_tokens;
    dLUT += (int64_t)sp * part_stride;
  }
  const int64_t i0 = (int64_t)(lb / (uint32_t)gpr) * DL_BM;
  const int g = (int)(lb % (uint32_t)gpr);
  const int64_t G = d / gpr;
  // this block's columns of the group: column range cr (whole chunks)
  const int64_t jg0 = (int64_t)g * G + (int64_t)cr * split_cols;
  const int64_t jend = (int64_t)g * G + G < jg0 + split_cols ? (int64_t)g * G + G : jg0 + split_cols;
  const int KS = (int)((m + DL_BK - 1) / DL_BK);

  for (uint32_t q = (uint32_t)t; q < 4u * DL_BCOPY / 4u; q += 512u) st_w(DL_BINS + q * 4u, 0u);

  // ---- staging roles: dY chunk t (token t / 16, rows 8 (t % 16) ..), X
  // chunks t + 512 h (token c / 64, columns 8 (c % 64) ..)
  const int ytok = t >> 4;
  const int64_t yrow = i0 + 8 * (t & 15);
  const uint32_t y_st = (uint32_t)ytok * DL_RSA + (uint32_t)(t & 15) * 16u;
  // Full steps (all 32 tokens and all rows of the block in range, the chunk's
  // 512 columns inside the row, 16-byte aligned rows) load through pointers
  // that advance by a step's worth of rows; only the others take the clamped,
  // masked path.
  const bool rows_full = VEC && i0 + DL_BM <= n;
  const TX* yfast = dY + (int64_t)ytok * n + yrow;
  auto load_step = [&](DlStage& S, int k, int64_t j0) {
    const int64_t t0 = (int64_t)k * DL_BK;
    // (columns past the block's range but inside the row are read too: binning leaves them out)
    if (rows_full && j0 + DL_BN <= d && t0 + DL_BK <= m) {  // wave-uniform
      S.y = *reinterpret_cast<const u32x4*>(yfast + t0 * n);
      const TX* xb = X + t0 * d + j0 + 8 * (t & 63);
#pragma unroll
      for (int h = 0; h < 4; ++h) S.x[h] = *reinterpret_cast<const u32x4*>(xb + (int64_t)(8 * h + (t >> 6)) * d);
      return;
    }
    const int64_t tok = t0 + ytok;
    const bool ok = tok < m;
    S.y = dl_load8<VEC, TX>(dY + (ok ? tok : 0) * n, yrow, ok ? n : 0);
#pragma unroll
    for (int h = 0; h < 4; ++h) {
      const int c = t + 512 * h;
      const int64_t xt = t0 + (c >> 6);
      const bool xok = xt < m;
      // d and the group width are multiples of 32: a chunk is wholly in or out
      S.x[h] = dl_load8<true, TX>(X + (xok ? xt : 0) * d, j0 + 8 * (c & 63), xok ? jend : 0);
    }
  };
  auto store_step = [&](const DlStage& S, int k) {
    const uint32_t base = (uint32_t)(k & 1) * DL_STAGE;
    st_q(base + y_st, S.y);
#pragma unroll
    for (int h = 0; h < 4; ++h) {
      const uint32_t c = (uint32_t)(t + 512 * h);
      st_q(base + DL_TA + (c >> 6) * DL_RSB + (c & 63u) * 16u, S.x[h]);
    }
  };

  // ---- matrix roles
  const int wm = wave & 1, wn = wave >> 1;
  f32x16 acc[2][4];
  auto mfma_step = [&](int k) {
    const uint32_t base = (uint32_t)(k & 1) * DL_STAGE;
    u32x4 af[2][2], bf[2][4];
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
#pragma unroll
      for (int a = 0; a < 2; ++a)
        af[ks][a] = ld_frag_tr(base + 16u * ks * DL_RSA + (64u * wm + 32u * a) * 2u, DL_RSA, lane);
#pragma unroll
      for (int b = 0; b < 4; ++b)
        bf[ks][b] = ld_frag_tr(base + DL_TA + 16u * ks * DL_RSB + (128u * wn + 32u * b) * 2u, DL_RSB, lane);
    }
#pragma unroll
    for (int ks = 0; ks < 2; ++ks)
#pragma unroll
      for (int a = 0; a < 2; ++a)
#pragma unroll
        for (int b = 0; b < 4; ++b) acc[a][b] = MF::run(af[ks][a], bf[ks][b], acc[a][b]);
    // the first half's 12 reads, then its 8 MFMAs interleaved with the second
    // half's reads, then the second half's MFMAs
    __builtin_amdgcn_sched_group_barrier(0x100, 12, 0);
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
      __builtin_amdgcn_sched_group_barrier(0x100, 3, 0);
    }
    __builtin_amdgcn_sched_group_barrier(0x008, 8, 0);
    __builtin_amdgcn_sched_barrier(0);
  };
  const bool mfma_first = wave < 4;  // the other wave of this SIMD stages first
  DlStage S;
  // step k: multiply tile k; store tile k+1 (in S) into the other buffer and
  // load tile k+2 into S
  auto step = [&](int k, int64_t j0) {
    auto stage_part = [&]() {
      if (k + 1 < KS) {
        store_step(S, k + 1);
        if (k + 2 < KS) load_step(S, k + 2, j0);
      }
    };
    if (mfma_first) {
      mfma_step(k);
      stage_part();
    } else {
      stage_part();
      __builtin_amdgcn_sched_barrier(0);
      mfma_step(k);
    }
    __syncthreads();
  };

  for (int64_t j0 = jg0; j0 < jend; j0 += DL_BN) {
#pragma unroll
    for (int a = 0; a < 2; ++a)
#pragma unroll
      for (int b = 0; b < 4; ++b) zero16(acc[a][b]);
    __syncthreads();  // the previous chunk's binning is done with the staged indices
    load_step(S, 0, j0);
    store_step(S, 0);
    if (KS > 1) load_step(S, 1, j0);
    __syncthreads();
    for (int k = 0; k < KS; ++k) step(k, j0);

    // ---- this chunk's packed indices, then the scatter into this wave's bins
    dl_stage_indices<B>(idx_packed, i0, n, d, j0, jend, t);
    __syncthreads();
    dl_scatter<B>(acc, lane, wm, wn, i0, n, j0, jend, DL_BINS + (uint32_t)wn * DL_BCOPY, DL_BRS);
  }
  __syncthreads();
  dl_store_bins<B>(dLUT, i0, n, gpr, g, DL_BINS, DL_BCOPY, DL_BRS, accumulate, t);
}

// ---------------------------------------------------------------------------
// k_gemm_dlut_dma: k_gemm_dlut's blocks, wave grid and binning, with the
// operand tiles copied from global memory straight into LDS (16-byte
// global_load_lds, two steps ahead into a ring of three stages), so that no
// registers and no LDS store instructions carry them and the waves only
// multiply. A DMA'd tile cannot be padded (a wave's 64 lanes write 1 KB
// contiguously), so its 16-byte chunks are XOR-swizzled instead: chunk c of
// token row r sits at c ^ 4 (r % 4), which puts the 4 rows x 4 chunks of one
// 32-lane pass of ds_read_b64_tr_b16 on 64 distinct banks; each lane of a DMA
// fetches the global chunk that belongs at its slot. The copies are issued
// from asm: given the builtin, the compiler cannot tell the transposing reads
// apart from the copies still in flight and drains every copy before each
// read. Ordering is explicit instead: a wave waits for its own copies of step
// k+1 (vmcnt) before the barrier that ends step k, so after that barrier the
// whole tile of step k+1 is in LDS, and the compiler, which does not count
// the copies, schedules the reads with exact LDS waits between the MFMAs. No
// other global load is in flight while copies are (the counts would be off).
// (Steps of 64 tokens in two stages, half the barriers, were 1-4 % slower;
// reads written as asm blocks that wait for all 12 of a half step were 3-4 %
// slower.)
// Requires m % 32 == 0 (there is no zero fill for tokens) and n % 8 == 0
// (16-byte aligned dY rows). Rows past n and columns past the row are read
// from clamped addresses; they only feed outputs that are not binned.
constexpr uint32_t DD_TA = DL_BK * 256u;              // 8192: dY tile [32 tokens][128 rows]
constexpr uint32_t DD_TB = DL_BK * 1024u;             // 32768: X tile [32 tokens][512 columns]
constexpr uint32_t DD_STAGE = DD_TA + DD_TB;          // 40960
constexpr uint32_t DD_BRS = 16;                       // floats per bin row (b <= 4)
constexpr uint32_t DD_BCOPY = 128u * DD_BRS * 4u;     // 8192
constexpr uint32_t DD_BINS = 3u * DD_STAGE;           // 122880
constexpr uint32_t DD_LDS = DD_BINS + 4u * DD_BCOPY;  // 155648


// 16 bytes per lane from `src` into LDS at `lds` + 16 * lane (lds wave-uniform).
// The copy takes its LDS address from M0 (one wait state after writing it);
// M0 is saved and restored around it, since the compiler may keep a value
// there.
__device__ __forceinline__ void dd_dma16(const void* src, uint32_t lds) {
  uint32_t keep;
  asm volatile(
      "s_mov_b32 %0, m0\n\t"
      "s_mov_b32 m0, %2\n\t"
      "s_nop 0\n\t"
      "global_load_lds_dwordx4 %1, off\n\t"
      "s_mov_b32 m0, %0"
      : "=&s"(keep)
      : "v"(src), "s"(lds)
      : "memory");
}

// raw barrier, with compiler-only fences so that no LDS access moves across it
__device__ __forceinline__ void dd_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// s_waitcnt bounding only the vector-memory counter (gfx9 encoding: vmcnt in
// bits 3:0 and 15:14; expcnt 7 and lgkmcnt 15 mean "no wait")
template <int N>
__device__ __forceinline__ void dd_wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt is a 6-bit field");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

template <int B, typename TX>
__global__ void __launch_bounds__(512, 1)
k_gemm_dlut_dma(const TX* __restrict__ dY, const TX* __restrict__ X, const uint8_t* __restrict__ idx_packed,
                int64_t m, int64_t n, int64_t d, int gpr, int gband, float* __restrict__ dLUT, int accumulate,
                int tsplits, int csplits, int64_t split_tokens, int64_t split_cols, int64_t part_stride) {
  typedef mfma32<TX> MF;
  extern __shared__ uint32_t smem[];  // dynamic LDS only: starts at address 0
  (void)smem;

  const int t = threadIdx.x;
  const uint32_t lane = (uint32_t)(t & 63);
  const int wave = __builtin_amdgcn_readfirstlane(t >> 6);
  // Consecutive logical blocks (one XCD's share, see xcd_block) take one
  // split (varying slowest) and in it `gband` groups of consecutive row
  // blocks: an XCD's co-resident blocks then share dY strips (same row block)
  // and X slabs (same group) in its L2.
  const uint32_t lba = xcd_block(blockIdx.x, gridDim.x);
  const uint32_t nb0 = gridDim.x / (uint32_t)(tsplits * csplits);
  const uint32_t sp = lba / nb0, lb = lba % nb0;
  const uint32_t cr = sp / (uint32_t)tsplits;  // column range of the group
  {
    const int64_t tok0 = (int64_t)(sp % (uint32_t)tsplits) * split_tokens;
    dY += tok0 * n;
    X += tok0 * d;
    m = m - tok0 < split_tokens ? m - tok0 : split_tokens;
    dLUT += (int64_t)sp * part_stride;
  }
  const uint32_t rblocks = nb0 / (uint32_t)gpr;
  const uint32_t gi = lb % (uint32_t)gband, rest = lb / (uint32_t)gband;
  const int64_t i0 = (int64_t)(rest % rblocks) * DL_BM;
  const int g = (int)((rest / rblocks) * (uint32_t)gband + gi);
  const int64_t G = d / gpr;
  // this block's columns of the group: column range cr (whole chunks)
  const int64_t jg0 = (int64_t)g * G + (int64_t)cr * split_cols;
  const int64_t jend = (int64_t)g * G + G < jg0 + split_cols ? (int64_t)g * G + G : jg0 + split_cols;
  const int KS = (int)(m / DL_BK);

  for (uint32_t q = (uint32_t)t; q < 4u * DD_BCOPY / 4u; q += 512u) st_w(DD_BINS + q * 4u, 0u);

  // ---- DMA roles: this wave's token rows 4 wave .. +3. dY: one 1 KB
  // instruction (lane = row (lane / 16) x slot (lane % 16)); X: one
  // instruction per row (lane = slot).
  const uint32_t ycg = (lane & 15u) ^ (((lane >> 4) & 3u) << 2);
  const int64_t yrow = i0 + 8 * (int64_t)ycg <= n - 8 ? i0 + 8 * (int64_t)ycg : n - 8;
  const TX* ysrc = dY + (int64_t)(4u * (uint32_t)wave + (lane >> 4)) * n + yrow;
  const uint32_t ydst = 1024u * (uint32_t)wave;
  const int64_t ystep = (int64_t)DL_BK * n;
  const int64_t xstep = (int64_t)DL_BK * d;
  const TX* xsrc[4];
  auto dma = [&](int k, uint32_t stage) {
    dd_dma16(ysrc + (int64_t)k * ystep, stage + ydst);
#pragma unroll
    for (int h = 0; h < 4; ++h) dd_dma16(xsrc[h] + (int64_t)k * xstep, stage + DD_TA + 1024u * (4u * (uint32_t)wave + h));
  };

  // ---- matrix roles: fragment addresses relative to a stage (the half step's
  // 16-token offset and the +4-row read go into the instruction offsets)
  const int wm = wave & 1, wn = wave >> 1;
  const uint32_t fs = lane & 15u;
  const uint32_t frow = 8u * (lane >> 5) + (fs >> 2);
  const uint32_t fx = (fs >> 2) << 2;  // swizzle of the fragment's rows (frow % 4 == fs / 4)
  const uint32_t fin = 2u * ((lane >> 4) & 1u) + ((fs & 3u) >> 1);
  const uint32_t fw = 8u * (fs & 1u);
  uint32_t fa[2], fb[4];
#pragma unroll
  for (int a = 0; a < 2; ++a) fa[a] = frow * 256u + (((8u * wm + 4u * a + fin) ^ fx) << 4) + fw;
#pragma unroll
  for (int b = 0; b < 4; ++b) fb[b] = DD_TA + frow * 1024u + (((16u * wn + 4u * b + fin) ^ fx) << 4) + fw;

  f32x16 acc[2][4];
  // one half step (16 tokens) of fragments: 12 transposing reads
  auto read_half = [&](uint32_t stage, int ks, u32x4 (&af)[2], u32x4 (&bf)[4]) {
#pragma unroll
    for (int a = 0; a < 2; ++a) {
      const uint32_t p = stage + fa[a] + 16u * 256u * (uint32_t)ks;
      const u32x2 lo = ld_tr(p), hi = ld_tr(p + 4u * 256u);
      af[a] = u32x4{lo.x, lo.y, hi.x, hi.y};
    }
#pragma unroll
    for (int b = 0; b < 4; ++b) {
      const uint32_t p = stage + fb[b] + 16u * 1024u * (uint32_t)ks;
      const u32x2 lo = ld_tr(p), hi = ld_tr(p + 4u * 1024u);
      bf[b] = u32x4{lo.x, lo.y, hi.x, hi.y};
    }
  };
  auto mfma_half = [&](const u32x4 (&af)[2], const u32x4 (&bf)[4]) {
#pragma unroll
    for (int a = 0; a < 2; ++a)
#pragma unroll
      for (int b = 0; b < 4; ++b) acc[a][b] = MF::run(af[a], bf[b], acc[a][b]);
  };
  // a half step's 8 MFMAs interleaved with the other half's 12 reads
  auto interleave = [&]() {
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      __builtin_amdgcn_sched_group_barrier(0x100, 3, 0);
      __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
    }
    __builtin_amdgcn_sched_barrier(0);
  };

  for (int64_t j0 = jg0; j0 < jend; j0 += DL_BN) {
#pragma unroll
    for (int h = 0; h < 4; ++h) {
      const int64_t col = j0 + 8 * (int64_t)(lane ^ ((uint32_t)h << 2));
      xsrc[h] = X + (int64_t)(4u * (uint32_t)wave + h) * d + (col <= d - 8 ? col : d - 8);
    }
#pragma unroll
    for (int a = 0; a < 2; ++a)
#pragma unroll
      for (int b = 0; b < 4; ++b) zero16(acc[a][b]);
    __syncthreads();  // the previous chunk's binning is done with the staged indices
    dma(0, 0u);
    if (KS > 1) {
      dma(1, DD_STAGE);
      dd_wait_vmcnt<5>();
    } else {
      dd_wait_vmcnt<0>();
    }
    dd_barrier();
    // Pipelined across the step barrier: step k's second half of reads runs
    // beside its first half of MFMAs; then every read of stage k has landed
    // (lgkmcnt 0) and this wave's copy of step k+1 (vmcnt), the barrier, and
    // step k+1's first half of reads runs beside step k's second half of
    // MFMAs, so the matrix core has work while the waves meet.
    u32x4 a0[2], b0[4], a1[2], b1[4];
    uint32_t st = 0u;  // stage of step k
    read_half(st, 0, a0, b0);
    for (int k = 0; k < KS; ++k) {
      const uint32_t st2 = st >= DD_STAGE ? st - DD_STAGE : st + 2u * DD_STAGE;  // stage of step k+2
      // (stage k+2 = stage k-1: every wave finished reading it before the last barrier)
      if (k + 2 < KS) dma(k + 2, st2);
      read_half(st, 1, a1, b1);
      mfma_half(a0, b0);
      interleave();
      __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0): every read of stage k has landed
      // this wave's DMA of step k+1 has landed (the one of step k+2 may not)
      if (k + 2 < KS) dd_wait_vmcnt<5>();
      else dd_wait_vmcnt<0>();
      dd_barrier();
      st = st + DD_STAGE == 3u * DD_STAGE ? 0u : st + DD_STAGE;
      // (unconditional, so that the reads interleave with the MFMAs: after
      // the last step they read a stale stage and the values go unused)
      read_half(st, 0, a0, b0);
      mfma_half(a1, b1);
      interleave();
    }
    dd_wait_vmcnt<0>();  // (no copy is in flight here; the compiler does not count them)

    dl_stage_indices<B>(idx_packed, i0, n, d, j0, jend, t);
    __syncthreads();
    dl_scatter<B>(acc, lane, wm, wn, i0, n, j0, jend, DD_BINS + (uint32_t)wn * DD_BCOPY, DD_BRS);
  }
  __syncthreads();
  dl_store_bins<B>(dLUT, i0, n, gpr, g, DD_BINS, DD_BCOPY, DD_BRS, accumulate, t);
}

// ---- launchers ---------------------------------------------------------------

uint32_t ug_magic_of(const Problem& p) {
  const uint32_t ug = (uint32_t)(p.group_cols() / 32);
  return ug == 1 ? 0u : (uint32_t)((((uint64_t)1) << 32) / ug + 1);
}

template <int B, int NG, typename TX, typename TL>
hipError_t dx_launch(const TX* dY, const uint8_t* idx, const TL* lut, const Problem& p, float* dX,
                     const int32_t* rexp, hipStream_t s) {
  const auto kern = k_gemm_dx<B, NG, TX, TL>;
  static const hipError_t prep = prepare_kernel((const void*)kern, DxLds<NG>::TOTAL);
  if (prep != hipSuccess) return prep;
  const int64_t mb = (p.m + DX_BM - 1) / DX_BM;
  const int64_t nb = (p.d + DX_BN - 1) / DX_BN;
  hipLaunchKernelGGL(kern, dim3((unsigned)(mb * nb)), dim3(512), DxLds<NG>::TOTAL, s, dY, idx, lut, p.m, p.n, p.d,
                     p.gpr, ug_magic_of(p), mb, dX, rexp);
  return hipGetLastError();
}

template <int B, typename TX, typename TL>
hipError_t dx_b(const TX* dY, const uint8_t* idx, const TL* lut, const Problem& p, float* dX, const int32_t* rexp,
                hipStream_t s) {
  // a 256-column tile touches at most 2 groups when groups are >= 256 columns
  // wide, at most 8 (one per 32-column unit) otherwise
  if (p.group_cols() >= 256) {
    const auto kern = k_gemm_dx64<B, TX, TL>;
    static const hipError_t prep = prepare_kernel((const void*)kern, D6_LDS);
    if (prep != hipSuccess) return prep;
    const int64_t mb = (p.m + DX_BM - 1) / DX_BM;
    const int64_t nb = (p.d + DX_BN - 1) / DX_BN;
    hipLaunchKernelGGL(kern, dim3((unsigned)(mb * nb)), dim3(512), D6_LDS, s, dY, idx, lut, p.m, p.n, p.d, p.gpr,
                       ug_magic_of(p), mb, dX, rexp);
    return hipGetLastError();
  }
  return dx_launch<B, 8>(dY, idx, lut, p, dX, rexp, s);
}

template <typename TX, typename TL>
hipError_t dx_t(const TX* dY, const uint8_t* idx, const TL* lut, const Problem& p, float* dX, const int32_t* rexp,
                hipStream_t s) {
  switch (p.b) {
    case 2: return dx_b<2>(dY, idx, lut, p, dX, rexp, s);
    case 3: return dx_b<3>(dY, idx, lut, p, dX, rexp, s);
    default: return dx_b<4>(dY, idx, lut, p, dX, rexp, s);
  }
}

// Splits of the table gradient (see the header of this file) when the (row
// block, group) grid has fewer than 256 blocks: first into column ranges of
// whole 512-column chunks of the group (each block still sums every token, so
// the binning is not repeated per token), then, when the chunks alone cannot
// fill the CUs, into token ranges of at least 4 steps of 32 tokens. Each
// count is the one that minimises rounds of 256 blocks times the chunks (or
// steps) per block, the fewer ranges on a tie, with the partial tables
// (parts * n * gpr * 2^b floats) within DLUT_PART_MAX bytes. No range is empty.
constexpr size_t DLUT_PART_MAX = size_t(6) << 20;
struct DlutSplit {
  int tsplits, csplits;
  int64_t tokens;  // tokens per range (a multiple of 32)
  int64_t cols;    // columns per range (a multiple of 512, or the whole group)
  int parts() const { return tsplits * csplits; }
};
// the count in [1, most] minimising ceil(blocks * c / 256) * ceil(units / c)
inline int64_t best_split(int64_t blocks, int64_t units, int64_t most) {
  int64_t best = 1, cost = ((blocks + 255) / 256) * units;
  for (int64_t c = 2; c <= most; ++c) {
    const int64_t k = ((blocks * c + 255) / 256) * ((units + c - 1) / c);
    if (k < cost) {
      cost = k;
      best = c;
    }
  }
  return best;
}
DlutSplit dlut_split_of(const Problem& p) {
  const int64_t nb0 = (p.n + DL_BM - 1) / DL_BM * p.gpr;
  const int64_t steps = (p.m + DL_BK - 1) / DL_BK;
  const int64_t G = p.group_cols();
  if (nb0 >= 256) return {1, 1, steps * DL_BK, G};
  const int64_t want = (256 + nb0 - 1) / nb0;  // ranges that fill the CUs once
  const int64_t nch = (G + DL_BN - 1) / DL_BN;
  const int64_t cap = (int64_t)(DLUT_PART_MAX / ((size_t)(p.n * p.gpr * p.k()) * 4));  // most partial tables
  if (cap < 2) return {1, 1, steps * DL_BK, G};
  int64_t most = nch < 4 * want ? nch : 4 * want;
  int64_t cs = best_split(nb0, nch, most < cap ? most : cap);
  const int64_t per_c = (nch + cs - 1) / cs;
  cs = (nch + per_c - 1) / per_c;
  int64_t ts = 1, per_t = steps;
  if (nb0 * cs < 256 && steps / 4 > 1 && cap / cs > 1) {
    const int64_t tw = (256 + nb0 * cs - 1) / (nb0 * cs);
    most = steps / 4 < 4 * tw ? steps / 4 : 4 * tw;
    ts = best_split(nb0 * cs, steps, most < cap / cs ? most : cap / cs);
    per_t = (steps + ts - 1) / ts;
    ts = (steps + per_t - 1) / per_t;
  }
  return {(int)ts, (int)cs, per_t * DL_BK, cs > 1 ? per_c * DL_BN : G};
}

// dLUT = (accumulate ? dLUT : 0) + sum over the ranges of the partial tables,
// in range order; four entries per thread (the entry count n * gpr * 2^b is a
// multiple of 4)
__global__ void __launch_bounds__(256) k_dlut_reduce(const float* __restrict__ part, int splits, int64_t count,
                                                     float* __restrict__ dLUT, int accumulate) {
  const int64_t q = ((int64_t)blockIdx.x * 256 + threadIdx.x) * 4;
  if (q >= count) return;
  f32x4 s = *reinterpret_cast<const f32x4*>(part + q);
  for (int k = 1; k < splits; ++k) s += *reinterpret_cast<const f32x4*>(part + (int64_t)k * count + q);
  f32x4* dst = reinterpret_cast<f32x4*>(dLUT + q);
  *dst = accumulate ? *dst + s : s;
}

hipError_t dlut_reduce(const float* part, int splits, int64_t count, float* dLUT, int accumulate, hipStream_t s) {
  const int64_t threads = count / 4;
  hipLaunchKernelGGL(k_dlut_reduce, dim3((unsigned)((threads + 255) / 256)), dim3(256), 0, s, part, splits, count,
                     dLUT, accumulate);
  return hipGetLastError();
}

template <int B, typename TX, bool VEC>
hipError_t dlut_launch(const TX* dY, const TX* X, const uint8_t* idx, const Problem& p, float* dLUT, int accumulate,
                       float* part, hipStream_t s) {
  const auto kern = k_gemm_dlut<B, TX, VEC>;
  static const hipError_t prep = prepare_kernel((const void*)kern, DL_LDS);
  if (prep != hipSuccess) return prep;
  const int64_t rb = (p.n + DL_BM - 1) / DL_BM;
  const DlutSplit sp = dlut_split_of(p);
  const int64_t count = p.n * p.gpr * p.k();
  const bool split = sp.parts() > 1;
  hipLaunchKernelGGL(kern, dim3((unsigned)(rb * p.gpr * sp.parts())), dim3(512), DL_LDS, s, dY, X, idx, p.m, p.n,
                     p.d, p.gpr, split ? part : dLUT, split ? 0 : accumulate, sp.tsplits, sp.csplits, sp.tokens,
                     sp.cols, count);
  hipError_t e = hipGetLastError();
  if (e == hipSuccess && split) e = dlut_reduce(part, sp.parts(), count, dLUT, accumulate, s);
  return e;
}

template <int B, typename TX>
hipError_t dlut_dma_launch(const TX* dY, const TX* X, const uint8_t* idx, const Problem& p, float* dLUT,
                           int accumulate, float* part, hipStream_t s) {
  const auto kern = k_gemm_dlut_dma<B, TX>;
  static const hipError_t prep = prepare_kernel((const void*)kern, DD_LDS);
  if (prep != hipSuccess) return prep;
  const int64_t rb = (p.n + DL_BM - 1) / DL_BM;
  // bands of 4 groups (or 2, or 1) in the XCD-local block order
  const int gband = p.gpr % 4 == 0 ? 4 : (p.gpr % 2 == 0 ? 2 : 1);
  const DlutSplit sp = dlut_split_of(p);
  const int64_t count = p.n * p.gpr * p.k();
  const bool split = sp.parts() > 1;
  hipLaunchKernelGGL(kern, dim3((unsigned)(rb * p.gpr * sp.parts())), dim3(512), DD_LDS, s, dY, X, idx, p.m, p.n,
                     p.d, p.gpr, gband, split ? part : dLUT, split ? 0 : accumulate, sp.tsplits, sp.csplits,
                     sp.tokens, sp.cols, count);
  hipError_t e = hipGetLastError();
  if (e == hipSuccess && split) e = dlut_reduce(part, sp.parts(), count, dLUT, accumulate, s);
  return e;
}

template <int B, typename TX>
hipError_t dlut_b(const TX* dY, const TX* X, const uint8_t* idx, const Problem& p, float* dLUT, int accumulate,
                  float* part, hipStream_t s) {
  // DMA staging: whole 32-token steps and 16-byte aligned dY rows
  if (p.m % DL_BK == 0 && p.n % 8 == 0)
    return dlut_dma_launch<B, TX>(dY, X, idx, p, dLUT, accumulate, part, s);
  if (p.n % 8 == 0) return dlut_launch<B, TX, true>(dY, X, idx, p, dLUT, accumulate, part, s);
  return dlut_launch<B, TX, false>(dY, X, idx, p, dLUT, accumulate, part, s);
}

template <typename TX>
hipError_t dlut_t(const TX* dY, const TX* X, const uint8_t* idx, const Problem& p, float* dLUT, int accumulate,
                  float* part, hipStream_t s) {
  switch (p.b) {
    case 2: return dlut_b<2>(dY, X, idx, p, dLUT, accumulate, part, s);
    case 3: return dlut_b<3>(dY, X, idx, p, dLUT, accumulate, part, s);
    default: return dlut_b<4>(dY, X, idx, p, dLUT, accumulate, part, s);
  }
}

}  // namespace

bool gemm_bwd_supported(const Problem& p) { return p.d <= (int64_t(1) << 20); }

size_t dlut_partial_bytes(const Problem& p) {
  const DlutSplit sp = dlut_split_of(p);
  return sp.parts() > 1 ? (size_t)sp.parts() * (size_t)(p.n * p.gpr * p.k()) * 4 : 0;
}

hipError_t launch_gemm_dx(const void* dY, int io_dtype, const uint8_t* idx, const void* lut, int lut_dtype,
                          const Problem& p, float* dX, const int32_t* rexp, hipStream_t s) {
  if (io_dtype == DT_F16 && lut_dtype == DT_F16)
    return dx_t((const half_t*)dY, idx, (const half_t*)lut, p, dX, nullptr, s);
  if (io_dtype == DT_BF16 && lut_dtype == DT_F16)
    return dx_t((const bf16_t*)dY, idx, (const half_t*)lut, p, dX, rexp, s);
  if (io_dtype == DT_F16 && lut_dtype == DT_BF16)
    return dx_t((const half_t*)dY, idx, (const bf16_t*)lut, p, dX, nullptr, s);
  return dx_t((const bf16_t*)dY, idx, (const bf16_t*)lut, p, dX, nullptr, s);
}

hipError_t launch_gemm_dlut(const void* dY, const void* X, int io_dtype, const uint8_t* idx, const Problem& p,
                            float* dLUT, int accumulate, float* part, hipStream_t s) {
  if (io_dtype == DT_F16) return dlut_t((const half_t*)dY, (const half_t*)X, idx, p, dLUT, accumulate, part, s);
  return dlut_t((const bf16_t*)dY, (const bf16_t*)X, idx, p, dLUT, accumulate, part, s);
}

}  // namespace skm
