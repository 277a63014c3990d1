// Matrix-core forward pass Y = X W^T for m > 16 tokens (prefill, training).
//
// At prefill / training sizes the sketched matmul is a dense contraction
// ("SpaLLM", section 2.3: one compressed matmul per layer, single tower), so
// the weights are dequantised tile by tile into LDS and fed to
// v_mfma_f32_32x32x16 (f16 or bf16, fp32 accumulation). W never reaches HBM:
// each block turns its 128 rows x 32 columns of packed indices into a
// 128 x 32 weight tile once per K-step and reuses it for all 256 tokens of
// the block, so the gather cost per multiply-add falls as 1/256.
//
// Block tile: 256 tokens (M) x 128 weight rows (N) x 32 columns (K = one
// 32-column unit, so a K-step never straddles a group). 4 waves in a 2 x 2
// grid, 128 x 64 outputs per wave (4 x 2 MFMA tiles). Double-buffered LDS:
//   A  [2][256 tokens][32 cols] activations in the compute dtype
//   Bt [2][128 rows][32 cols]   dequantised weights
//   tables [2 groups][2 row halves][T entries][64 lanes] dwords
// Rows of A and Bt are 64 bytes with XOR-swizzled 16-byte chunks (mm::swz) so
// the 16 rows of one ds_read_b128 pass land in distinct banks.
//
// Dequantisation roles: thread t owns weight row r = t % 128 and the column
// half hh = t / 128 of each unit (16 weights per K-step). Its table copies sit
// at lane slot t % 64 of its row half, entry-major, so the gathers of one wave
// (64 distinct rows) are conflict-free; the gather address is built by one
// v_perm_b32 as in the decode kernel. Tables are staged one group ahead.
#include "skm_gemm_common.h"
#include "skm_launch.h"

namespace skm {

namespace {

using mm::swz;

constexpr int G_BM = 256;
constexpr int G_BN = 128;
constexpr int G_BK = 32;
constexpr int G_THREADS = 256;

constexpr uint32_t LDS_A = 0;
constexpr uint32_t LDS_B = 2u * G_BM * G_BK * 2u;          // 32768
constexpr uint32_t LDS_T = LDS_B + 2u * G_BN * G_BK * 2u;   // 49152
constexpr uint32_t LDS_TOTAL = LDS_T + 2u * 2u * 16u * 64u * 4u;  // 65536

typedef __attribute__((address_space(3))) uint16_t lds_u16;
typedef __attribute__((address_space(3))) uint32_t lds_u32;
typedef __attribute__((address_space(3))) u32x4 lds_u32x4;

template <int B> struct tab_entries { static constexpr int value = (B == 2) ? 16 : (1 << B); };

template <typename TC> struct mfma32;
template <> struct mfma32<half_t> {
  typedef f16x8 vec;
  static __device__ __forceinline__ f32x16 run(u32x4 a, u32x4 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(vec, a), __builtin_bit_cast(vec, b), c, 0, 0, 0);
  }
};
template <> struct mfma32<bf16_t> {
  typedef bf16x8 vec;
  static __device__ __forceinline__ f32x16 run(u32x4 a, u32x4 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(vec, a), __builtin_bit_cast(vec, b), c, 0, 0, 0);
  }
};


__device__ __forceinline__ uint32_t lds_h(uint32_t a) { return *(const lds_u16*)(uintptr_t)a; }
__device__ __forceinline__ uint32_t lds_w(uint32_t a) { return *(const lds_u32*)(uintptr_t)a; }
__device__ __forceinline__ u32x4 lds_q(uint32_t a) { return *(const lds_u32x4*)(uintptr_t)a; }
__device__ __forceinline__ void st_w(uint32_t a, uint32_t v) { *(lds_u32*)(uintptr_t)a = v; }
__device__ __forceinline__ void st_q(uint32_t a, u32x4 v) { *(lds_u32x4*)(uintptr_t)a = v; }

__device__ __forceinline__ uint32_t gaddr(uint32_t ent, uint32_t lane4, int p) {
  return __builtin_amdgcn_perm(ent, lane4, 0x0C0C0400u | ((4u + (uint32_t)p) << 8));
}
__device__ __forceinline__ uint32_t pack2(uint32_t lo, uint32_t hi) {
  return __builtin_amdgcn_perm(hi, lo, 0x05040100u);
}

// 16-bit activations -> compute dtype, 8 values (same helper as the decode
// kernel; goes through 16-bit integers, see the note there)
template <typename TX, typename TC>
__device__ __forceinline__ u32x4 x_to_tc(u32x4 v) {
  if constexpr (__is_same(TX, TC)) {
    return v;
  } else {
    typedef _Float16 f16x2_t __attribute__((ext_vector_type(2)));
    typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
    u32x4 o;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const uint32_t w = v[q];
      float lo, hi;
      if constexpr (__is_same(TX, bf16_t)) {
        lo = __builtin_bit_cast(float, w << 16);
        hi = __builtin_bit_cast(float, w & 0xFFFF0000u);
      } else {
        lo = (float)__builtin_bit_cast(half_t, (uint16_t)(w & 0xFFFFu));
        hi = (float)__builtin_bit_cast(half_t, (uint16_t)(w >> 16));
      }
      if constexpr (__is_same(TC, half_t)) {
        f16x2_t r;
        r.x = (half_t)lo;
        r.y = (half_t)hi;
        o[q] = __builtin_bit_cast(uint32_t, r);
      } else {
        bf16x2_t r;
        r.x = (bf16_t)lo;
        r.y = (bf16_t)hi;
        o[q] = __builtin_bit_cast(uint32_t, r);
      }
    }
    return o;
  }
}

// ---- per-thread index words of one K-step (the thread's half unit) ----------
template <int B> struct IdxRegs { uint32_t w[B == 3 ? 3 : (B == 4 ? 2 : 1)]; };

template <int B>
__device__ __forceinline__ void load_idx(IdxRegs<B>& I, const uint8_t* rowp, uint32_t k, int hh) {
  if constexpr (B == 4) {
    const u32x2 v = *reinterpret_cast<const u32x2*>(rowp + k * 16u + hh * 8);
    I.w[0] = v.x;
    I.w[1] = v.y;
  } else if constexpr (B == 2) {
    I.w[0] = *reinterpret_cast<const uint32_t*>(rowp + k * 8u + hh * 4);
  } else {
    const uint32_t* p = reinterpret_cast<const uint32_t*>(rowp + k * 12u);
    I.w[0] = p[0];
    I.w[1] = p[1];
    I.w[2] = p[2];
  }
}

// 16 weights (fields 16*HH .. 16*HH+15 of the unit) -> 8 packed dwords
template <int B, int HH>
__device__ __forceinline__ void dequant16(const IdxRegs<B>& I, uint32_t gk, uint32_t lane4, uint32_t* o) {
  const uint32_t gk4 = gk * 0x01010101u;
  if constexpr (B == 4) {
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const uint32_t ev = (I.w[j] & 0x0F0F0F0Fu) | gk4;
      const uint32_t od = ((I.w[j] >> 4) & 0x0F0F0F0Fu) | gk4;
#pragma unroll
      for (int t = 0; t < 4; ++t)
        o[4 * j + t] = pack2(lds_h(gaddr(ev, lane4, t) + LDS_T), lds_h(gaddr(od, lane4, t) + LDS_T));
    }
  } else if constexpr (B == 2) {
    // nibble p of the word is the pair (2p, 2p+1): one pair-table gather each
    const uint32_t ev = (I.w[0] & 0x0F0F0F0Fu) | gk4;
    const uint32_t od = ((I.w[0] >> 4) & 0x0F0F0F0Fu) | gk4;
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      o[2 * t] = lds_w(gaddr(ev, lane4, t) + LDS_T);
      o[2 * t + 1] = lds_w(gaddr(od, lane4, t) + LDS_T);
    }
  } else {
#pragma unroll
    for (int t = 0; t < 8; ++t) {
      const uint32_t e0 = unit_field<3>(I.w, 16 * HH + 2 * t);
      const uint32_t e1 = unit_field<3>(I.w, 16 * HH + 2 * t + 1);
      o[t] = pack2(lds_h((((gk + e0) << 8) | lane4) + LDS_T), lds_h((((gk + e1) << 8) | lane4) + LDS_T));
    }
  }
}

// ---- table staging ------------------------------------------------------------
template <int B> struct LutRegs { uint32_t v[B == 4 ? 4 : 2]; };

template <int B, typename TL>
__device__ __forceinline__ void load_lut(LutRegs<B>& L, const TL* lut, int64_t grow, int gpr, uint32_t g, int hh) {
  constexpr int K = 1 << B;
  const uint16_t* src = reinterpret_cast<const uint16_t*>(lut) + ((int64_t)grow * gpr + g) * K;
  if constexpr (B == 4) {
    const u32x4 v = *reinterpret_cast<const u32x4*>(src + 8 * hh);
    L.v[0] = v.x; L.v[1] = v.y; L.v[2] = v.z; L.v[3] = v.w;
  } else if constexpr (B == 3) {
    const u32x2 v = *reinterpret_cast<const u32x2*>(src + 4 * hh);
    L.v[0] = v.x; L.v[1] = v.y;
  } else {
    const u32x2 v = *reinterpret_cast<const u32x2*>(src);
    L.v[0] = v.x; L.v[1] = v.y;
  }
}

// entry base (in entries) of table buffer tb for this thread's row half
template <int B>
__device__ __forceinline__ uint32_t tab_base(uint32_t tb, uint32_t rowhalf) {
  return (tb * 2u + rowhalf) * (uint32_t)tab_entries<B>::value;
}

template <int B>
__device__ __forceinline__ void store_lut(const LutRegs<B>& L, uint32_t tb, uint32_t rowhalf, int hh, uint32_t lane4) {
  const uint32_t base = tab_base<B>(tb, rowhalf);
  if constexpr (B == 4) {
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const uint32_t v = (i & 1) ? (L.v[i >> 1] >> 16) : (L.v[i >> 1] & 0xFFFFu);
      st_w(LDS_T + ((base + 8u * hh + i) << 8) + lane4, v);
    }
  } else if constexpr (B == 3) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const uint32_t v = (i & 1) ? (L.v[i >> 1] >> 16) : (L.v[i >> 1] & 0xFFFFu);
      st_w(LDS_T + ((base + 4u * hh + i) << 8) + lane4, v);
    }
  } else {
    const uint32_t e[4] = {L.v[0] & 0xFFFFu, L.v[0] >> 16, L.v[1] & 0xFFFFu, L.v[1] >> 16};
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int pe = 8 * hh + i;  // pair entry a + 4c
      st_w(LDS_T + ((base + pe) << 8) + lane4, e[pe & 3] | (e[pe >> 2] << 16));
    }
  }
}

template <int B, typename TX, typename TL>
__global__ void __launch_bounds__(G_THREADS, 2)
k_gemm_fwd(const TX* __restrict__ X, const uint8_t* __restrict__ idx_packed, const TL* __restrict__ lut,
           int64_t m, int64_t n, int64_t d, int gpr, uint32_t ug_magic, int64_t mblocks, TX* __restrict__ Y) {
  typedef mfma32<TL> MF;
  extern __shared__ uint32_t smem[];  // dynamic LDS only: starts at address 0
  (void)smem;

  const int t = threadIdx.x;
  const int lane = t & 63;
  const int wave = t >> 6;
  const uint32_t lane4 = (uint32_t)lane * 4u;
  const int64_t bm = blockIdx.x % mblocks;
  const int64_t bn = blockIdx.x / mblocks;
  const int64_t m0 = bm * G_BM, n0 = bn * G_BN;

  // dequant role
  const int r = t & (G_BN - 1);
  const int hh = t >> 7;                  // wave-uniform
  const uint32_t rowhalf = (uint32_t)(wave & 1);
  const int64_t grow = (n0 + r < n) ? n0 + r : n - 1;
  const uint8_t* rowp = idx_packed + grow * (d * B / 8);
  // activation role: token row t of the tile
  const int64_t gtok = (m0 + t < m) ? m0 + t : m - 1;
  const TX* xrow = X + gtok * d;

  const uint32_t U = (uint32_t)(d / 32);
  auto group_of = [&](uint32_t k) -> uint32_t { return ug_magic ? __umulhi(k, ug_magic) : k; };

  // ---- prologue: tables of group(0), tile 0
  IdxRegs<B> I;
  LutRegs<B> L;
  u32x4 xr[4];
  uint32_t gcur = group_of(0);
  load_lut<B, TL>(L, lut, grow, gpr, gcur, hh);
  load_idx<B>(I, rowp, 0, hh);
#pragma unroll
  for (int c = 0; c < 4; ++c) xr[c] = reinterpret_cast<const u32x4*>(xrow)[c];
  store_lut<B>(L, gcur & 1u, rowhalf, hh, lane4);
  uint32_t gnext = U > 1 ? group_of(1) : gcur;
  if (gnext != gcur) load_lut<B, TL>(L, lut, grow, gpr, gnext, hh);
  __syncthreads();
  {
    uint32_t o[8];
    if (hh) dequant16<B, 1>(I, tab_base<B>(gcur & 1u, rowhalf), lane4, o);
    else dequant16<B, 0>(I, tab_base<B>(gcur & 1u, rowhalf), lane4, o);
    st_q(LDS_B + swz(r, 2 * hh), u32x4{o[0], o[1], o[2], o[3]});
    st_q(LDS_B + swz(r, 2 * hh + 1), u32x4{o[4], o[5], o[6], o[7]});
#pragma unroll
    for (int c = 0; c < 4; ++c) st_q(LDS_A + swz(t, c), x_to_tc<TX, TL>(xr[c]));
    if (gnext != gcur) store_lut<B>(L, gnext & 1u, rowhalf, hh, lane4);
  }
  __syncthreads();

  f32x16 acc[4][2];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.0f;

  const int wm = wave & 1, wn = wave >> 1;
  const uint32_t arow = (uint32_t)(128 * wm + (lane & 31));
  const uint32_t brow = (uint32_t)(64 * wn + (lane & 31));
  const uint32_t khalf = (uint32_t)(lane >> 5);

  for (uint32_t k = 0; k < U; ++k) {
    const uint32_t cur = k & 1u;
    const bool more = k + 1 < U;
    uint32_t g1 = 0, g2 = 0;
    if (more) {
      g1 = group_of(k + 1);
      load_idx<B>(I, rowp, k + 1, hh);
      const u32x4* xp = reinterpret_cast<const u32x4*>(xrow + (int64_t)(k + 1) * 32);
#pragma unroll
      for (int c = 0; c < 4; ++c) xr[c] = xp[c];
      g2 = (k + 2 < U) ? group_of(k + 2) : g1;
      if (g2 != g1) load_lut<B, TL>(L, lut, grow, gpr, g2, hh);
    }
    // ---- MFMAs on buffer cur
    const uint32_t abase = LDS_A + cur * (uint32_t)(G_BM * G_BK * 2);
    const uint32_t bbase = LDS_B + cur * (uint32_t)(G_BN * G_BK * 2);
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      const uint32_t ch = (uint32_t)(2 * ks) + khalf;
      u32x4 af[4], bf[2];
#pragma unroll
      for (int i = 0; i < 4; ++i) af[i] = lds_q(abase + swz(arow + 32u * i, ch));
#pragma unroll
      for (int j = 0; j < 2; ++j) bf[j] = lds_q(bbase + swz(brow + 32u * j, ch));
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) acc[i][j] = MF::run(af[i], bf[j], acc[i][j]);
    }
    // ---- stage tile k+1 into the other buffer
    if (more) {
      const uint32_t nb = cur ^ 1u;
      uint32_t o[8];
      if (hh) dequant16<B, 1>(I, tab_base<B>(g1 & 1u, rowhalf), lane4, o);
      else dequant16<B, 0>(I, tab_base<B>(g1 & 1u, rowhalf), lane4, o);
      const uint32_t bb = LDS_B + nb * (uint32_t)(G_BN * G_BK * 2);
      st_q(bb + swz(r, 2 * hh), u32x4{o[0], o[1], o[2], o[3]});
      st_q(bb + swz(r, 2 * hh + 1), u32x4{o[4], o[5], o[6], o[7]});
      const uint32_t ab = LDS_A + nb * (uint32_t)(G_BM * G_BK * 2);
#pragma unroll
      for (int c = 0; c < 4; ++c) st_q(ab + swz(t, c), x_to_tc<TX, TL>(xr[c]));
      if (g2 != g1) store_lut<B>(L, g2 & 1u, rowhalf, hh, lane4);
    }
    __syncthreads();
  }

  // ---- epilogue: D[i][j] of a 32x32 tile sits in lane j (+32 for the second
  // 4-row band) at register 4*(i/8) + i%4, i.e. row 8*(e/4) + 4*(lane/32) + e%4
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int64_t col = n0 + 64 * wn + 32 * j + (lane & 31);
      if (col >= n) continue;
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int64_t tok = m0 + 128 * wm + 32 * i + 8 * (e >> 2) + 4 * (lane >> 5) + (e & 3);
        if (tok < m) Y[tok * n + col] = from_f32<TX>(acc[i][j][e]);
      }
    }
}

template <int B, typename TX, typename TL>
hipError_t gemm_fwd_b(const TX* X, const uint8_t* idx, const TL* lut, const Problem& p, TX* Y, hipStream_t s) {
  const int64_t mb = (p.m + G_BM - 1) / G_BM;
  const int64_t nb = (p.n + G_BN - 1) / G_BN;
  const uint32_t ug = (uint32_t)(p.group_cols() / 32);
  const uint32_t magic = ug == 1 ? 0u : (uint32_t)((((uint64_t)1) << 32) / ug + 1);
  hipLaunchKernelGGL((k_gemm_fwd<B, TX, TL>), dim3((unsigned)(mb * nb)), dim3(G_THREADS), LDS_TOTAL, s, X, idx, lut,
                     p.m, p.n, p.d, p.gpr, magic, mb, Y);
  return hipGetLastError();
}

template <typename TX, typename TL>
hipError_t gemm_fwd_t(const TX* X, const uint8_t* idx, const TL* lut, const Problem& p, TX* Y, hipStream_t s) {
  switch (p.b) {
    case 2: return gemm_fwd_b<2>(X, idx, lut, p, Y, s);
    case 3: return gemm_fwd_b<3>(X, idx, lut, p, Y, s);
    default: return gemm_fwd_b<4>(X, idx, lut, p, Y, s);
  }
}

}  // namespace

bool gemm_fwd_supported(const Problem& p) {
  // group index by multiply-high is exact while units * units-per-group < 2^32
  return p.d <= (int64_t(1) << 20) && p.n * p.m < (int64_t(1) << 62);
}

hipError_t launch_gemm_fwd(const void* X, int x_dtype, const uint8_t* idx, const void* lut, int lut_dtype,
                           const Problem& p, void* Y, hipStream_t s) {
  if (x_dtype == DT_F16 && lut_dtype == DT_F16)
    return gemm_fwd_t((const half_t*)X, idx, (const half_t*)lut, p, (half_t*)Y, s);
  if (x_dtype == DT_BF16 && lut_dtype == DT_F16)
    return gemm_fwd_t((const bf16_t*)X, idx, (const half_t*)lut, p, (bf16_t*)Y, s);
  if (x_dtype == DT_F16 && lut_dtype == DT_BF16)
    return gemm_fwd_t((const half_t*)X, idx, (const bf16_t*)lut, p, (half_t*)Y, s);
  return gemm_fwd_t((const bf16_t*)X, idx, (const bf16_t*)lut, p, (bf16_t*)Y, s);
}

}  // namespace skm
