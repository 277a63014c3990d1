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
// k_gemm_dx: M = tokens (256), N = columns of dX (128), K = weight rows (32
// per step). The weight tile of 32 rows x 128 columns is dequantised once per
// step and written transposed ([column][row]) so each MFMA B fragment is 8
// consecutive rows of one column. Each step brings 32 new rows, so the tables
// (up to 4 groups of the column tile, private copy per lane slot) are staged
// every step, two steps ahead.
//
// k_gemm_dlut: one block owns 128 rows x one group. For each chunk of up to
// 512 columns of the group it accumulates the dW = dY^T X tile over all
// tokens (K = 32 tokens per step; the operand tiles are stored as loaded,
// [token][row] and [token][column], and read with gfx950's transposing LDS
// reads), then scatter-adds the tile into LDS bins [row][entry] using the
// chunk's indices staged in LDS. Waves own disjoint (row, bin copy) pairs, so
// the bins need no cross-wave atomics and the sums are deterministic; the
// block stores each gradient entry exactly once (no global atomics).
#include "skm_gemm_common.h"
#include "skm_launch.h"

namespace skm {

namespace {

using namespace mm;

// ============================================================================
// dX
// ============================================================================
constexpr int DX_BM = 256, DX_BN = 128, DX_BK = 32, DX_NG = 4;
constexpr uint32_t DX_A = 0;                                   // [2][256][32] dY (compute dtype)
constexpr uint32_t DX_B = 2u * DX_BM * DX_BK * 2u;             // 32768: [2][128 cols][32 rows]
constexpr uint32_t DX_T = DX_B + 2u * DX_BN * DX_BK * 2u;      // 49152: tables [2][NG][T][64] dwords
constexpr uint32_t DX_LDS = DX_T + 2u * DX_NG * 16u * 64u * 4u;  // 81920

template <int B> struct DxIdx { uint32_t w[B == 3 ? 3 : (B == 4 ? 2 : 1)]; };

template <int B>
__device__ __forceinline__ void dx_load_idx(DxIdx<B>& I, const uint8_t* rowp, uint32_t u, int hh) {
  if constexpr (B == 4) {
    const u32x2 v = *reinterpret_cast<const u32x2*>(rowp + u * 16u + hh * 8);
    I.w[0] = v.x;
    I.w[1] = v.y;
  } else if constexpr (B == 2) {
    I.w[0] = *reinterpret_cast<const uint32_t*>(rowp + u * 8u + hh * 4);
  } else {
    const uint32_t* p = reinterpret_cast<const uint32_t*>(rowp + u * 12u);
    I.w[0] = p[0];
    I.w[1] = p[1];
    I.w[2] = p[2];
  }
}

// 16 weights of half hh of a unit -> 8 words of packed consecutive columns
template <int B>
__device__ __forceinline__ void dx_dequant(const DxIdx<B>& I, int hh, uint32_t gk, uint32_t lane4, uint32_t* o) {
  const uint32_t gk4 = gk * 0x01010101u;
  if constexpr (B == 4) {
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const uint32_t ev = (I.w[j] & 0x0F0F0F0Fu) | gk4;
      const uint32_t od = ((I.w[j] >> 4) & 0x0F0F0F0Fu) | gk4;
#pragma unroll
      for (int t = 0; t < 4; ++t)
        o[4 * j + t] = pack2(ld_h(gaddr(ev, lane4, t) + DX_T), ld_h(gaddr(od, lane4, t) + DX_T));
    }
  } else if constexpr (B == 2) {
    const uint32_t ev = (I.w[0] & 0x0F0F0F0Fu) | gk4;
    const uint32_t od = ((I.w[0] >> 4) & 0x0F0F0F0Fu) | gk4;
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      o[2 * t] = ld_w(gaddr(ev, lane4, t) + DX_T);
      o[2 * t + 1] = ld_w(gaddr(od, lane4, t) + DX_T);
    }
  } else {
    if (hh) {
#pragma unroll
      for (int t = 0; t < 8; ++t) {
        const uint32_t e0 = unit_field<3>(I.w, 16 + 2 * t), e1 = unit_field<3>(I.w, 17 + 2 * t);
        o[t] = pack2(ld_h((((gk + e0) << 8) | lane4) + DX_T), ld_h((((gk + e1) << 8) | lane4) + DX_T));
      }
    } else {
#pragma unroll
      for (int t = 0; t < 8; ++t) {
        const uint32_t e0 = unit_field<3>(I.w, 2 * t), e1 = unit_field<3>(I.w, 1 + 2 * t);
        o[t] = pack2(ld_h((((gk + e0) << 8) | lane4) + DX_T), ld_h((((gk + e1) << 8) | lane4) + DX_T));
      }
    }
  }
}

// Tables of step rows k0..k0+31, groups glo..glo+ng-1, into buffer tb:
// slot s (lane id) holds row k0 + s%32; wave w writes entries [w*T/4, (w+1)*T/4).
template <int B> struct DxLut { uint32_t v[2]; };

template <int B, typename TL>
__device__ __forceinline__ void dx_load_lut(DxLut<B>& L, const TL* lut, int64_t row, bool row_ok, int gpr, uint32_t g,
                                            int w) {
  constexpr int K = 1 << B;
  const uint16_t* src = reinterpret_cast<const uint16_t*>(lut) + ((int64_t)row * gpr + g) * K;
  if (!row_ok) {
    L.v[0] = L.v[1] = 0u;
    return;
  }
  if constexpr (B == 4) {
    const u32x2 v = *reinterpret_cast<const u32x2*>(src + 4 * w);
    L.v[0] = v.x;
    L.v[1] = v.y;
  } else if constexpr (B == 3) {
    L.v[0] = *reinterpret_cast<const uint32_t*>(src + 2 * w);
    L.v[1] = 0u;
  } else {
    const u32x2 v = *reinterpret_cast<const u32x2*>(src);
    L.v[0] = v.x;
    L.v[1] = v.y;
  }
}

template <int B>
__device__ __forceinline__ void dx_store_lut(const DxLut<B>& L, uint32_t tb, uint32_t gsel, int w, uint32_t lane4) {
  constexpr uint32_t T = (uint32_t)tab_entries<B>::value;
  const uint32_t base = (tb * DX_NG + gsel) * T;
  if constexpr (B == 4) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const uint32_t v = (i & 1) ? (L.v[i >> 1] >> 16) : (L.v[i >> 1] & 0xFFFFu);
      st_w(DX_T + ((base + 4u * w + i) << 8) + lane4, v);
    }
  } else if constexpr (B == 3) {
    st_w(DX_T + ((base + 2u * w) << 8) + lane4, L.v[0] & 0xFFFFu);
    st_w(DX_T + ((base + 2u * w + 1) << 8) + lane4, L.v[0] >> 16);
  } else {
    const uint32_t e[4] = {L.v[0] & 0xFFFFu, L.v[0] >> 16, L.v[1] & 0xFFFFu, L.v[1] >> 16};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int pe = 4 * w + i;
      st_w(DX_T + ((base + pe) << 8) + lane4, e[pe & 3] | (e[pe >> 2] << 16));
    }
  }
}

// dY tile row (32 weight rows starting at k0) of one token -> compute dtype
template <typename TX, typename TC>
__device__ __forceinline__ void dx_load_a(u32x4* a, const TX* dyrow, int64_t k0, int64_t n, bool vec) {
  if (vec && k0 + 32 <= n) {
    const u32x4* p = reinterpret_cast<const u32x4*>(dyrow + k0);
#pragma unroll
    for (int c = 0; c < 4; ++c) a[c] = p[c];
  } else {
    const uint16_t* p = reinterpret_cast<const uint16_t*>(dyrow);
#pragma unroll
    for (int c = 0; c < 4; ++c)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int64_t i0 = k0 + 8 * c + 2 * q;
        const uint32_t lo = i0 < n ? p[i0] : 0u;
        const uint32_t hi = i0 + 1 < n ? p[i0 + 1] : 0u;
        a[c][q] = lo | (hi << 16);
      }
  }
}

template <int B, typename TX, typename TL>
__global__ void __launch_bounds__(256, 1)
k_gemm_dx(const TX* __restrict__ dY, const uint8_t* __restrict__ idx_packed, const TL* __restrict__ lut, int64_t m,
          int64_t n, int64_t d, int gpr, uint32_t ug_magic, int64_t mblocks, float* __restrict__ dX) {
  typedef mfma32<TL> MF;
  constexpr uint32_t T = (uint32_t)tab_entries<B>::value;
  extern __shared__ uint32_t smem[];
  (void)smem;

  const int t = threadIdx.x;
  const int lane = t & 63;
  const int wave = t >> 6;
  const uint32_t lane4 = (uint32_t)lane * 4u;
  const int64_t bm = blockIdx.x % mblocks, bn = blockIdx.x / mblocks;
  const int64_t m0 = bm * DX_BM, n0 = bn * DX_BN;   // token / column tile origins
  const bool vec = (n % 8) == 0;

  // dequant role: weight row r of the step, 16-column chunk c of the tile
  const int r = t & 31;
  const int c = t >> 5;
  const int hh = c & 1;
  const int64_t jc = n0 + 16 * c;                   // first column of the chunk
  const bool col_ok = jc < d;
  const uint32_t u = (uint32_t)((col_ok ? jc : 0) / 32);
  const uint32_t glo = group_of((uint32_t)(n0 / 32), ug_magic);
  const uint32_t ghi = group_of((uint32_t)((n0 + DX_BN < d ? n0 + DX_BN : d) / 32 - 1), ug_magic);
  const uint32_t ng = ghi - glo + 1;                // groups touched by the column tile (<= 4)
  const uint32_t gsel = col_ok ? group_of(u, ug_magic) - glo : 0u;
  // activation role: token row t
  const int64_t gtok = (m0 + t < m) ? m0 + t : m - 1;
  const TX* dyrow = dY + gtok * n;

  const int64_t rb = d * B / 8;
  const uint32_t KS = (uint32_t)((n + DX_BK - 1) / DX_BK);  // K-steps

  auto stage_tables = [&](uint32_t ks, uint32_t tb) {
    const int64_t row = (int64_t)ks * DX_BK + (lane & 31);
    const bool ok = row < n;
    for (uint32_t gs = 0; gs < ng; ++gs) {
      DxLut<B> L;
      dx_load_lut<B, TL>(L, lut, ok ? row : 0, ok, gpr, glo + gs, wave);
      dx_store_lut<B>(L, tb, gs, wave, lane4);
    }
  };
  auto dequant_step = [&](uint32_t ks, uint32_t buf) {
    const int64_t row = (int64_t)ks * DX_BK + r;
    const bool ok = row < n && col_ok;
    uint32_t o[8];
    DxIdx<B> I;
    dx_load_idx<B>(I, idx_packed + (ok ? row : 0) * rb, u, hh);
    dx_dequant<B>(I, hh, ((ks & 1u) * DX_NG + gsel) * T, lane4, o);
    const uint32_t bb = DX_B + buf * (uint32_t)(DX_BN * DX_BK * 2);
#pragma unroll
    for (int f = 0; f < 16; ++f) {
      const uint32_t v = ok ? ((f & 1) ? (o[f >> 1] >> 16) : (o[f >> 1] & 0xFFFFu)) : 0u;
      st_h(bb + swz_elem((uint32_t)(16 * c + f), (uint32_t)r), v);
    }
  };
  auto store_a = [&](const u32x4* a, uint32_t buf) {
    const uint32_t ab = DX_A + buf * (uint32_t)(DX_BM * DX_BK * 2);
#pragma unroll
    for (int q = 0; q < 4; ++q) st_q(ab + swz((uint32_t)t, (uint32_t)q), cvt_quad<TX, TL>(a[q]));
  };

  // ---- prologue
  u32x4 a[4];
  stage_tables(0, 0);
  if (KS > 1) stage_tables(1, 1);
  dx_load_a<TX, TL>(a, dyrow, 0, n, vec);
  __syncthreads();
  dequant_step(0, 0);
  store_a(a, 0);
  __syncthreads();

  f32x16 acc[4][2];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) zero16(acc[i][j]);
  const int wm = wave & 1, wn = wave >> 1;
  const uint32_t arow = (uint32_t)(128 * wm + (lane & 31));
  const uint32_t brow = (uint32_t)(64 * wn + (lane & 31));
  const uint32_t khalf = (uint32_t)(lane >> 5);

  for (uint32_t k = 0; k < KS; ++k) {
    const uint32_t cur = k & 1u;
    const bool more = k + 1 < KS;
    if (more) dx_load_a<TX, TL>(a, dyrow, (int64_t)(k + 1) * DX_BK, n, vec);
    const uint32_t abase = DX_A + cur * (uint32_t)(DX_BM * DX_BK * 2);
    const uint32_t bbase = DX_B + cur * (uint32_t)(DX_BN * DX_BK * 2);
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      const uint32_t ch = (uint32_t)(2 * ks) + khalf;
      u32x4 af[4], bf[2];
#pragma unroll
      for (int i = 0; i < 4; ++i) af[i] = ld_q(abase + swz(arow + 32u * i, ch));
#pragma unroll
      for (int j = 0; j < 2; ++j) bf[j] = ld_q(bbase + swz(brow + 32u * j, ch));
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) acc[i][j] = MF::run(af[i], bf[j], acc[i][j]);
    }
    if (more) {
      dequant_step(k + 1, cur ^ 1u);
      store_a(a, cur ^ 1u);
      if (k + 2 < KS) stage_tables(k + 2, cur);
    }
    __syncthreads();
  }

#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int64_t col = n0 + 64 * wn + 32 * j + (lane & 31);
      if (col >= d) continue;
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int64_t tok = m0 + 128 * wm + 32 * i + 8 * (e >> 2) + 4 * (lane >> 5) + (e & 3);
        if (tok < m) dX[tok * d + col] = acc[i][j][e];
      }
    }
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
constexpr uint32_t DL_BINS = 2u * DL_STAGE;                  // 90112: [4 copies][128 rows][16] fp32
constexpr uint32_t DL_LDS = DL_BINS + 4u * 128u * 16u * 4u;  // 122880
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

// raw operands of one step for one thread: one dY chunk, four X chunks
struct DlStage {
  u32x4 y;
  u32x4 x[4];
};

template <int B, typename TX, bool VEC>
__global__ void __launch_bounds__(512, 1)
k_gemm_dlut(const TX* __restrict__ dY, const TX* __restrict__ X, const uint8_t* __restrict__ idx_packed, int64_t m,
            int64_t n, int64_t d, int gpr, float* __restrict__ dLUT, int accumulate) {
  typedef mfma32<TX> MF;
  constexpr int K = 1 << B;
  extern __shared__ uint32_t smem[];
  (void)smem;

  const int t = threadIdx.x;
  const uint32_t lane = (uint32_t)(t & 63);
  const int wave = t >> 6;
  // the gpr groups of one row block (same dY strip) share an XCD's L2
  const uint32_t lb = xcd_block(blockIdx.x, gridDim.x);
  const int64_t i0 = (int64_t)(lb / (uint32_t)gpr) * DL_BM;
  const int g = (int)(lb % (uint32_t)gpr);
  const int64_t G = d / gpr;
  const int64_t jg0 = (int64_t)g * G;  // first column of the group
  const int64_t jend = jg0 + G;
  const int KS = (int)((m + DL_BK - 1) / DL_BK);

  for (uint32_t q = (uint32_t)t; q < 4u * 128u * 16u; q += 512u) st_w(DL_BINS + q * 4u, 0u);

  // ---- staging roles: dY chunk t (token t / 16, rows 8 (t % 16) ..), X
  // chunks t + 512 h (token c / 64, columns 8 (c % 64) ..)
  const int ytok = t >> 4;
  const int64_t yrow = i0 + 8 * (t & 15);
  const uint32_t y_st = (uint32_t)ytok * DL_RSA + (uint32_t)(t & 15) * 16u;
  auto load_step = [&](DlStage& S, int k, int64_t j0) {
    const int64_t tok = (int64_t)k * DL_BK + ytok;
    const bool ok = tok < m;
    S.y = dl_load8<VEC, TX>(dY + (ok ? tok : 0) * n, yrow, ok ? n : 0);
#pragma unroll
    for (int h = 0; h < 4; ++h) {
      const int c = t + 512 * h;
      const int64_t xt = (int64_t)k * DL_BK + (c >> 6);
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

    // ---- this chunk's packed indices: 128 rows x (16 * B) dwords
    {
      const int64_t units = (jend - j0) / 32 < DL_BN / 32 ? (jend - j0) / 32 : DL_BN / 32;
      for (int q = t; q < 128 * 16 * B; q += 512) {
        const int row = q / (16 * B), wd = q % (16 * B);
        const int64_t grow = i0 + row < n ? i0 + row : n - 1;
        const uint32_t* src = reinterpret_cast<const uint32_t*>(idx_packed + grow * (d * B / 8) + j0 * B / 8);
        st_w((uint32_t)row * DL_IRS + (uint32_t)wd * 4u, (wd / B) < units ? src[wd] : 0u);
      }
    }
    __syncthreads();

    // ---- scatter-add the finished dW tile into this wave's bins
    // D[i][j] of tile (a, b): i = 64 wm + 32 a + 8 (e/4) + 4 (lane/32) + e%4,
    // j = 128 wn + 32 b + lane%32 (fully unrolled so the accumulators stay in
    // registers; the scheduling fences keep the index reads from being
    // hoisted all at once)
    // (an opaque copy of the lane id keeps the compiler from hoisting the 128
    // bin addresses out of the chunk loop, where they would stay live across
    // the K loop)
    uint32_t bl = lane;
    asm volatile("" : "+v"(bl));
    const uint32_t binbase = DL_BINS + (uint32_t)wn * (128u * 16u * 4u);
#pragma unroll
    for (int a = 0; a < 2; ++a)
#pragma unroll
      for (int b = 0; b < 4; ++b) {
        const uint32_t j = 128u * wn + 32u * b + (bl & 31u);
        const bool j_ok = j0 + (int64_t)j < jend;
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          // branch-free: an entry outside the matrix adds 0 to a bin that is
          // never stored (rows past n) or to entry 0 (columns past the group,
          // whose staged indices are 0)
          const uint32_t i = 64u * wm + 32u * a + 8u * (e >> 2) + 4u * (bl >> 5) + (e & 3);
          const float v = (j_ok && i0 + (int64_t)i < n) ? acc[a][b][e] : 0.0f;
          const uint32_t c = dl_field<B>(i * DL_IRS, j);
          __hip_atomic_fetch_add((lds_f32*)(uintptr_t)(binbase + (i * 16u + c) * 4u), v, __ATOMIC_RELAXED,
                                 __HIP_MEMORY_SCOPE_WORKGROUP);
          if ((e & 3) == 3) __builtin_amdgcn_sched_barrier(0);
        }
      }
  }
  __syncthreads();

  // ---- one store per gradient entry (bin copies summed in a fixed order)
  for (uint32_t q = (uint32_t)t; q < 128u * (uint32_t)K; q += 512u) {
    const uint32_t i = q / K, c = q % K;
    if (i0 + (int64_t)i >= n) continue;
    float s = 0.0f;
#pragma unroll
    for (int w = 0; w < 4; ++w)
      s += *(const lds_f32*)(uintptr_t)(DL_BINS + (uint32_t)w * (128u * 16u * 4u) + (i * 16u + c) * 4u);
    float* dst = dLUT + ((i0 + i) * gpr + g) * K + c;
    *dst = accumulate ? *dst + s : s;
  }
}

// ---- launchers ---------------------------------------------------------------

uint32_t ug_magic_of(const Problem& p) {
  const uint32_t ug = (uint32_t)(p.group_cols() / 32);
  return ug == 1 ? 0u : (uint32_t)((((uint64_t)1) << 32) / ug + 1);
}

template <int B, typename TX, typename TL>
hipError_t dx_b(const TX* dY, const uint8_t* idx, const TL* lut, const Problem& p, float* dX, hipStream_t s) {
  const auto kern = k_gemm_dx<B, TX, TL>;
  // more than 64 KB of LDS per block must be requested once per kernel
  static const hipError_t attr =
      hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize, DX_LDS);
  if (attr != hipSuccess) return attr;
  const int64_t mb = (p.m + DX_BM - 1) / DX_BM;
  const int64_t nb = (p.d + DX_BN - 1) / DX_BN;
  hipLaunchKernelGGL(kern, dim3((unsigned)(mb * nb)), dim3(256), DX_LDS, s, dY, idx, lut, p.m, p.n, p.d, p.gpr,
                     ug_magic_of(p), mb, dX);
  return hipGetLastError();
}

template <typename TX, typename TL>
hipError_t dx_t(const TX* dY, const uint8_t* idx, const TL* lut, const Problem& p, float* dX, hipStream_t s) {
  switch (p.b) {
    case 2: return dx_b<2>(dY, idx, lut, p, dX, s);
    case 3: return dx_b<3>(dY, idx, lut, p, dX, s);
    default: return dx_b<4>(dY, idx, lut, p, dX, s);
  }
}

template <int B, typename TX, bool VEC>
hipError_t dlut_launch(const TX* dY, const TX* X, const uint8_t* idx, const Problem& p, float* dLUT, int accumulate,
                       hipStream_t s) {
  const auto kern = k_gemm_dlut<B, TX, VEC>;
  static const hipError_t attr =
      hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize, (int)DL_LDS);
  if (attr != hipSuccess) return attr;
  const int64_t rb = (p.n + DL_BM - 1) / DL_BM;
  hipLaunchKernelGGL(kern, dim3((unsigned)(rb * p.gpr)), dim3(512), DL_LDS, s, dY, X, idx, p.m, p.n, p.d, p.gpr, dLUT,
                     accumulate);
  return hipGetLastError();
}

template <int B, typename TX>
hipError_t dlut_b(const TX* dY, const TX* X, const uint8_t* idx, const Problem& p, float* dLUT, int accumulate,
                  hipStream_t s) {
  if (p.n % 8 == 0) return dlut_launch<B, TX, true>(dY, X, idx, p, dLUT, accumulate, s);
  return dlut_launch<B, TX, false>(dY, X, idx, p, dLUT, accumulate, s);
}

template <typename TX>
hipError_t dlut_t(const TX* dY, const TX* X, const uint8_t* idx, const Problem& p, float* dLUT, int accumulate,
                  hipStream_t s) {
  switch (p.b) {
    case 2: return dlut_b<2>(dY, X, idx, p, dLUT, accumulate, s);
    case 3: return dlut_b<3>(dY, X, idx, p, dLUT, accumulate, s);
    default: return dlut_b<4>(dY, X, idx, p, dLUT, accumulate, s);
  }
}

}  // namespace

bool gemm_bwd_supported(const Problem& p) { return p.d <= (int64_t(1) << 20); }

hipError_t launch_gemm_dx(const void* dY, int io_dtype, const uint8_t* idx, const void* lut, int lut_dtype,
                          const Problem& p, float* dX, hipStream_t s) {
  if (io_dtype == DT_F16 && lut_dtype == DT_F16) return dx_t((const half_t*)dY, idx, (const half_t*)lut, p, dX, s);
  if (io_dtype == DT_BF16 && lut_dtype == DT_F16) return dx_t((const bf16_t*)dY, idx, (const half_t*)lut, p, dX, s);
  if (io_dtype == DT_F16 && lut_dtype == DT_BF16) return dx_t((const half_t*)dY, idx, (const bf16_t*)lut, p, dX, s);
  return dx_t((const bf16_t*)dY, idx, (const bf16_t*)lut, p, dX, s);
}

hipError_t launch_gemm_dlut(const void* dY, const void* X, int io_dtype, const uint8_t* idx, const Problem& p,
                            float* dLUT, int accumulate, hipStream_t s) {
  if (io_dtype == DT_F16) return dlut_t((const half_t*)dY, (const half_t*)X, idx, p, dLUT, accumulate, s);
  return dlut_t((const bf16_t*)dY, (const bf16_t*)X, idx, p, dLUT, accumulate, s);
}

}  // namespace skm
