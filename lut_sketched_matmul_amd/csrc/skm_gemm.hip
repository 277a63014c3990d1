// Matrix-core forward pass Y = X W^T for m > 16 tokens (prefill, training).
//
// At prefill / training sizes the sketched matmul is a dense contraction
// ("SpaLLM", section 2.3: one compressed matmul per layer, single tower), so
// the weights are dequantised tile by tile into LDS and fed to
// v_mfma_f32_32x32x16 (f16 or bf16, fp32 accumulation). W never reaches HBM:
// each block turns its 256 rows x 32 columns of packed indices into a
// 256 x 32 weight tile once per K-step and reuses it for all 256 tokens of
// the block.
//
// Block tile: 256 tokens (M) x 256 weight rows (N) x 32 columns (K = one
// 32-column unit, so a K-step never straddles a group); 8 waves in a 2 x 4
// grid, 128 x 64 outputs per wave (4 x 2 tiles of v_mfma_f32_32x32x16, 16
// MFMAs per K-step). One block per CU, two waves per SIMD (waves w and w+4).
// In each K-step every wave multiplies tile k from LDS and stages (loads,
// dequantises, converts) its share of tile k+1 into the other LDS buffer;
// waves 0-3 do the matrix work first and waves 4-7 the staging first, so the
// two waves of a SIMD overlap one's MFMAs with the other's vector work.
// LDS (96 KB):
//   tables [2 groups][4 row quarters][T entries][64 lanes] dwords   at 0
//   A  [2][256 tokens][32 cols] activations in the compute dtype     at 32 KB
//   Bt [2][256 rows][32 cols]   dequantised weights                  at 64 KB
// Rows of A and Bt are 64 bytes with XOR-swizzled 16-byte chunks (mm::swz).
//
// Staging roles (b = 2, 3): thread t owns weight row r = t % 256 with column
// half hh = t / 256 (16 weights per K-step), and 16-byte chunk t % 4 of token
// rows t / 4 and t / 4 + 128 (16 activations; the 4 lanes that share a row
// read its 64 bytes together). Its table copy sits at lane slot t % 64 of row
// quarter (t / 64) % 4, entry-major, so the gathers of one wave (64 distinct
// rows) are conflict-free; the gather address is one v_perm_b32.
// b = 4 looks its weights up in registers instead (mm::dequant8_b4, tables
// loaded once per group) and pairs the two threads of a row on adjacent lanes
// (r = t / 2, hh = t % 2); both operands are then staged in that lookup's K
// order within each 8-column chunk.
//
// Pipeline: the raw index words and activations of tile k+3 are loaded into
// registers during K-step k and staged in K-step k+2 (two register stages);
// one barrier per K-step; LDS tables (b = 2, 3) are staged one group ahead
// into the other table buffer.
//
// bf16 activations with f16 tables: each token row is prescaled by 2^-e[t]
// while it is converted (row exponents from the caller's workspace, see
// skm_common.h) and its outputs are multiplied by 2^e[t] before rounding.
// The block takes one conversion for all its rows (block_scale_mode): none
// when every e is 0 (the common case), an exponent-field add, or a multiply;
// the prologue, K loop and store are compiled once per conversion (run<MD>),
// so the common case runs the same loop as 16-bit activations of the table
// dtype would.
#include "skm_gemm_common.h"
#include "skm_launch.h"

namespace skm {

namespace {

using mm::swz;
using mm::swz128;
using mm::gaddr;
using mm::pack2;
using mm::tab_entries;

constexpr int G_BM = 256;
constexpr int G_BN = 256;
constexpr int G_BK = 32;
constexpr int G_THREADS = 512;

constexpr uint32_t A_TILE = G_BM * G_BK * 2u;  // 16 KB
constexpr uint32_t B_TILE = G_BN * G_BK * 2u;  // 16 KB
constexpr uint32_t LDS_T = 0;
constexpr uint32_t LDS_A = 2u * 4u * 16u * 64u * 4u;  // 32768
constexpr uint32_t LDS_B = LDS_A + 2u * A_TILE;       // 65536
constexpr uint32_t LDS_TOTAL = LDS_B + 2u * B_TILE;   // 98304

using mm::ld_h;
using mm::ld_w;
using mm::ld_q;
using mm::st_w;
using mm::st_q;

// ---- per-thread raw operands of one K-step: the thread's half unit of index
// words and its 16 activations ---------------------------------------------
template <int B> struct Stage {
  uint32_t w[B == 3 ? 3 : (B == 4 ? 2 : 1)];
  u32x4 x[2];
};

template <int B, typename TX>
__device__ __forceinline__ void load_stage(Stage<B>& S, const uint8_t* rowp, const TX* const* xrow, uint32_t k,
                                           int hh) {
  if constexpr (B == 4) {
    const u32x2 v = *reinterpret_cast<const u32x2*>(rowp + k * 16u + hh * 8);
    S.w[0] = v.x;
    S.w[1] = v.y;
  } else if constexpr (B == 2) {
    S.w[0] = *reinterpret_cast<const uint32_t*>(rowp + k * 8u + hh * 4);
  } else {
    // the 16 fields of a half unit start at bit 48 for hh = 1: load the whole unit
    const uint32_t* p = reinterpret_cast<const uint32_t*>(rowp + k * 12u);
    S.w[0] = p[0];
    S.w[1] = p[1];
    S.w[2] = p[2];
  }
#pragma unroll
  for (int c = 0; c < 2; ++c) S.x[c] = *reinterpret_cast<const u32x4*>(xrow[c] + (int64_t)k * 32);
}

// 16 weights (fields 16*HH .. 16*HH+15 of the unit) -> 8 packed dwords.
// `tb` is the entry base of the thread's table copy.
template <int B, int HH>
__device__ __forceinline__ void dequant16(const Stage<B>& S, uint32_t tb, uint32_t lane4, uint32_t* o) {
  const uint32_t tb4 = tb * 0x01010101u;
  if constexpr (B == 4) {
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const uint32_t ev = (S.w[j] & 0x0F0F0F0Fu) | tb4;
      const uint32_t od = ((S.w[j] >> 4) & 0x0F0F0F0Fu) | tb4;
#pragma unroll
      for (int t = 0; t < 4; ++t)
        o[4 * j + t] = pack2(ld_h(gaddr(ev, lane4, t) + LDS_T), ld_h(gaddr(od, lane4, t) + LDS_T));
    }
  } else if constexpr (B == 2) {
    // nibble p of the word is the pair (2p, 2p+1): one pair-table gather each
    const uint32_t ev = (S.w[0] & 0x0F0F0F0Fu) | tb4;
    const uint32_t od = ((S.w[0] >> 4) & 0x0F0F0F0Fu) | tb4;
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      o[2 * t] = ld_w(gaddr(ev, lane4, t) + LDS_T);
      o[2 * t + 1] = ld_w(gaddr(od, lane4, t) + LDS_T);
    }
  } else {
#pragma unroll
    for (int t = 0; t < 8; ++t) {
      const uint32_t e0 = unit_field<3>(S.w, 16 * HH + 2 * t);
      const uint32_t e1 = unit_field<3>(S.w, 16 * HH + 2 * t + 1);
      o[t] = pack2(ld_h((((tb + e0) << 8) | lane4) + LDS_T), ld_h((((tb + e1) << 8) | lane4) + LDS_T));
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

// entry base (in entries) of table buffer `buf` for row quarter rq
template <int B>
__device__ __forceinline__ uint32_t tab_base(uint32_t buf, uint32_t rq) {
  return (buf * 4u + rq) * (uint32_t)tab_entries<B>::value;
}

// The thread's half of its row's table (the other half comes from the thread
// with the other hh); the b = 2 pair table is built by both halves.
template <int B>
__device__ __forceinline__ void store_lut(const LutRegs<B>& L, uint32_t base, int hh, uint32_t lane4) {
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

// Store a wave's 128 x 64 outputs (acc[i][jj]: a 32 x 32 tile whose D[r][c]
// sits in lane c (+32 for the second 4-row band) at register 4 (r / 8) + r % 4,
// i.e. row 8 (e / 4) + 4 (lane / 32) + e % 4) rounded to TX. SC: row r of
// the block's 256 tokens is first multiplied by 2^e[r]; the 256 factors go
// through LDS (free after the last K-step's barrier), four tokens per read.
template <typename TX, bool SC>
__device__ __forceinline__ void store_tile(const f32x16 (&acc)[4][2], TX* __restrict__ Y,
                                           const int32_t* __restrict__ rexp, int64_t m, int64_t n, int64_t m0,
                                           int64_t n0, int wm, int wn, int lane, int t) {
  if constexpr (SC) {
    if (t < G_BM) {
      const int64_t tok = m0 + t < m ? m0 + t : m - 1;
      st_w((uint32_t)t * 4u, __builtin_bit_cast(uint32_t, pow2f(rexp[tok])));
    }
    __syncthreads();
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    f32x4 uq[4] = {};
    if constexpr (SC) {
#pragma unroll
      for (int q = 0; q < 4; ++q) uq[q] = mm::ld_f4((uint32_t)(128 * wm + 32 * i + 8 * q + 4 * (lane >> 5)) * 4u);
    }
#pragma unroll
    for (int jj = 0; jj < 2; ++jj) {
      const int64_t col = n0 + 64 * wn + 32 * jj + (lane & 31);
      if (col >= n) continue;
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int64_t tok = m0 + 128 * wm + 32 * i + 8 * (e >> 2) + 4 * (lane >> 5) + (e & 3);
        float v = acc[i][jj][e];
        if constexpr (SC) v *= uq[e >> 2][e & 3];
        if (tok < m) Y[tok * n + col] = from_f32<TX>(v);
      }
    }
  }
}

template <int B, typename TX, typename TL>
__global__ void __launch_bounds__(G_THREADS, 1)
k_gemm_fwd(const TX* __restrict__ X, const uint8_t* __restrict__ idx_packed, const TL* __restrict__ lut,
           int64_t m, int64_t n, int64_t d, int gpr, uint32_t ug_magic, int64_t mblocks, TX* __restrict__ Y,
           const int32_t* __restrict__ rexp) {
  constexpr bool SC = scaled_pair(__is_same(TX, bf16_t), __is_same(TL, half_t));
  // The block's conversion mode of its activation rows (bf16 with f16 tables:
  // block_scale_mode). Everything after it is compiled once per mode (run<MD>),
  // each copy with its own registers: only the kernel arguments cross the
  // dispatch, so the common mode 0 runs the loop 16-bit operands of the table
  // dtype would, and the modes that convert do not squeeze its registers.
  int mode = 0;
  if constexpr (SC) {
    const int64_t mb0 = (int64_t)(blockIdx.x % mblocks) * G_BM;
    uint32_t flags = 0u;
#pragma unroll
    for (int c = 0; c < 2; ++c) {
      const int64_t tok = mb0 + 128 * c + (threadIdx.x >> 2);
      flags |= scale_flags_of(rexp[tok < m ? tok : m - 1]);
    }
    mode = mm::block_scale_mode(flags, LDS_B + B_TILE);
  }
  auto run = [&](auto md) __attribute__((always_inline)) {
    constexpr int MD = decltype(md)::value;
    typedef mm::mfma32<TL> MF;
    extern __shared__ uint32_t smem[];  // dynamic LDS only: starts at address 0
    (void)smem;

    const int t = threadIdx.x;
    const int lane = t & 63;
    const int wave = t >> 6;
    const uint32_t lane4 = (uint32_t)lane * 4u;
    const int64_t bm = blockIdx.x % mblocks;
    const int64_t bn = blockIdx.x / mblocks;
    const int64_t m0 = bm * G_BM, n0 = bn * G_BN;
    const int U = (int)(d / 32);
    auto group_of = [&](int k) -> uint32_t { return mm::group_of((uint32_t)k, ug_magic); };

    // ---- staging state (b = 4: the two threads of a row are adjacent lanes and
    // the tables stay in registers, as in k_gemm_fwd64)
    const int r = B == 4 ? (t >> 1) : (t & 255);
    const int hh = B == 4 ? (t & 1) : (t >> 8);  // wave-uniform for b = 2, 3
    const uint32_t rq = (uint32_t)(wave & 3);    // row quarter of r (b = 2, 3)
    const int64_t grow = (n0 + r < n) ? n0 + r : n - 1;
    const uint8_t* rowp = idx_packed + grow * (d * B / 8);
    const uint16_t* lutrow = reinterpret_cast<const uint16_t*>(lut) + grow * (int64_t)gpr * (1 << B);
    mm::Planes16 P;
    uint32_t Ln[8];
    uint32_t cur_g = 0xFFFFFFFFu;
    auto load_tab = [&](uint32_t g) {
      const u32x4* tp = reinterpret_cast<const u32x4*>(lutrow + g * 16u);
      const u32x4 a = tp[0], b = tp[1];
      Ln[0] = a.x; Ln[1] = a.y; Ln[2] = a.z; Ln[3] = a.w;
      Ln[4] = b.x; Ln[5] = b.y; Ln[6] = b.z; Ln[7] = b.w;
    };
    const TX* xrow[2];
    int xe[2] = {0, 0};  // SC: exponents of the two staged token rows
  #pragma unroll
    for (int c = 0; c < 2; ++c) {
      const int64_t tok = m0 + 128 * c + (t >> 2);
      xrow[c] = X + (tok < m ? tok : m - 1) * d + 8 * (t & 3);
      if constexpr (SC && MD != 0) xe[c] = rexp[tok < m ? tok : m - 1];
    }
    float xsc[2] = {1.0f, 1.0f};
    uint32_t xk[2] = {0u, 0u};
  #pragma unroll
    for (int c = 0; c < (int)(sizeof(xe) / sizeof(xe[0])); ++c) {
      if constexpr (MD == 2) xsc[c] = pow2f(-xe[c]);
      if constexpr (MD == 1) xk[c] = exp_add_word(xe[c]);
    }
    (void)xsc;
    (void)xk;
    const uint32_t b_st0 = swz((uint32_t)r, 2u * hh), b_st1 = swz((uint32_t)r, 2u * hh + 1u);
    const uint32_t a_st0 = swz((uint32_t)(t >> 2), (uint32_t)(t & 3));
    const uint32_t a_st1 = swz((uint32_t)(128 + (t >> 2)), (uint32_t)(t & 3));
    Stage<B> S0, S1;
    LutRegs<B> L;

    // stage tile j (raw operands in S) into LDS buffer j & 1
    auto stage = [&](const Stage<B>& S, int j, auto md) __attribute__((always_inline)) {
      constexpr int MD = decltype(md)::value;
      const uint32_t buf = (uint32_t)(j & 1);
      const uint32_t bb = LDS_B + buf * B_TILE;
      const uint32_t ab = LDS_A + buf * A_TILE;
      if constexpr (B == 4) {
        const uint32_t g = group_of(j);
        if (g != cur_g) {
          mm::planes16(Ln, P);
          cur_g = g;
          load_tab(g + 1 < (uint32_t)gpr ? g + 1 : g);
        }
        st_q(bb + b_st0, mm::dequant8_b4(S.w[0], P));
        st_q(bb + b_st1, mm::dequant8_b4(S.w[1], P));
        if constexpr (SC && MD == 2) {
          st_q(ab + a_st0, mm::cvt_quad_perm_scaled(S.x[0], xsc[0]));
          st_q(ab + a_st1, mm::cvt_quad_perm_scaled(S.x[1], xsc[1]));
        } else if constexpr (SC && MD == 1) {
          st_q(ab + a_st0, mm::cvt_quad_perm<TX, TL>(mm::add_quad(S.x[0], xk[0])));
          st_q(ab + a_st1, mm::cvt_quad_perm<TX, TL>(mm::add_quad(S.x[1], xk[1])));
        } else {
          st_q(ab + a_st0, mm::cvt_quad_perm<TX, TL>(S.x[0]));
          st_q(ab + a_st1, mm::cvt_quad_perm<TX, TL>(S.x[1]));
        }
      } else {
        uint32_t o[8];
        const uint32_t tb = tab_base<B>(group_of(j) & 1u, rq);
        if (hh) dequant16<B, 1>(S, tb, lane4, o);
        else dequant16<B, 0>(S, tb, lane4, o);
        st_q(bb + b_st0, u32x4{o[0], o[1], o[2], o[3]});
        st_q(bb + b_st1, u32x4{o[4], o[5], o[6], o[7]});
        if constexpr (SC && MD == 2) {
          st_q(ab + a_st0, mm::cvt_quad_scaled(S.x[0], xsc[0]));
          st_q(ab + a_st1, mm::cvt_quad_scaled(S.x[1], xsc[1]));
        } else if constexpr (SC && MD == 1) {
          st_q(ab + a_st0, mm::cvt_quad<TX, TL>(mm::add_quad(S.x[0], xk[0])));
          st_q(ab + a_st1, mm::cvt_quad<TX, TL>(mm::add_quad(S.x[1], xk[1])));
        } else {
          st_q(ab + a_st0, mm::cvt_quad<TX, TL>(S.x[0]));
          st_q(ab + a_st1, mm::cvt_quad<TX, TL>(S.x[1]));
        }
      }
    };
    // staging work of K-step k: tile k+1 from Sn into LDS, Sn refilled with
    // tile k+3, tables kept one group ahead (the table of tile k+2's group is
    // in L and goes to LDS now; the table of tile k+3's group is loaded)
    auto stage_step = [&](int k, Stage<B>& Sn, auto md) __attribute__((always_inline)) {
      if (k + 1 >= U) return;
      stage(Sn, k + 1, md);
      if (k + 3 < U) load_stage<B, TX>(Sn, rowp, xrow, (uint32_t)(k + 3), hh);
      if (B != 4 && k + 2 < U) {
        const uint32_t g2 = group_of(k + 2);
        if (g2 != group_of(k + 1)) store_lut<B>(L, tab_base<B>(g2 & 1u, rq), hh, lane4);
        if (k + 3 < U && group_of(k + 3) != g2) load_lut<B, TL>(L, lut, grow, gpr, group_of(k + 3), hh);
      }
    };

    // ---- matrix state
    const int wm = wave & 1, wn = wave >> 1;
    const uint32_t arow = (uint32_t)(128 * wm + (lane & 31));
    const uint32_t brow = (uint32_t)(64 * wn + (lane & 31));
    const uint32_t khalf = (uint32_t)(lane >> 5);
    f32x16 acc[4][2];
  #pragma unroll
    for (int i = 0; i < 4; ++i)
  #pragma unroll
      for (int jj = 0; jj < 2; ++jj) mm::zero16(acc[i][jj]);
    auto load_frags = [&](u32x4* fa, u32x4* fb, int k, int ks) {
      const uint32_t buf = (uint32_t)(k & 1);
      const uint32_t ch = (uint32_t)(2 * ks) + khalf;
  #pragma unroll
      for (int i = 0; i < 4; ++i) fa[i] = ld_q(LDS_A + buf * A_TILE + swz(arow + 32u * i, ch));
  #pragma unroll
      for (int jj = 0; jj < 2; ++jj) fb[jj] = ld_q(LDS_B + buf * B_TILE + swz(brow + 32u * jj, ch));
    };
    // matrix work of K-step k. The scheduling groups issue the first half's
    // fragment reads, then alternate MFMAs of the first half with the second
    // half's reads (each read reuses the registers of an A fragment whose MFMAs
    // have been issued), then the second half's MFMAs.
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
      __builtin_amdgcn_sched_group_barrier(0x100, 6, 0);  // reads of the first half
  #pragma unroll
      for (int i = 0; i < 4; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);  // two MFMAs
        __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);  // one read of the second half
      }
      __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
      __builtin_amdgcn_sched_group_barrier(0x008, 8, 0);
      __builtin_amdgcn_sched_barrier(0);
    };
    const bool mfma_first = wave < 4;  // the other wave of this SIMD stages first
    auto step = [&](int k, Stage<B>& Sn, auto md) __attribute__((always_inline)) {
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

    // ---- prologue: tables of group 0 (group 1's in registers), tile 0 staged,
    // tiles 1 and 2 in registers, then the table of group 1 and of tile 2's
    // group staged / loaded as in a K-step
    if constexpr (B == 4) {
      load_tab(group_of(0));
      load_stage<B, TX>(S0, rowp, xrow, 0, hh);
      if (U > 1) load_stage<B, TX>(S1, rowp, xrow, 1, hh);
      stage(S0, 0, md);
      if (U > 2) load_stage<B, TX>(S0, rowp, xrow, 2, hh);
    } else {
      load_lut<B, TL>(L, lut, grow, gpr, group_of(0), hh);
      load_stage<B, TX>(S0, rowp, xrow, 0, hh);
      if (U > 1) load_stage<B, TX>(S1, rowp, xrow, 1, hh);
      store_lut<B>(L, tab_base<B>(group_of(0) & 1u, rq), hh, lane4);
      const bool new1 = U > 1 && group_of(1) != group_of(0);
      if (new1) load_lut<B, TL>(L, lut, grow, gpr, group_of(1), hh);
      __syncthreads();
      stage(S0, 0, md);
      if (U > 2) load_stage<B, TX>(S0, rowp, xrow, 2, hh);
      if (new1) store_lut<B>(L, tab_base<B>(group_of(1) & 1u, rq), hh, lane4);
      if (U > 2 && group_of(2) != group_of(1)) load_lut<B, TL>(L, lut, grow, gpr, group_of(2), hh);
    }
    __syncthreads();

    // ---- main loop: two K-steps per trip so each register stage keeps its
    // role; an odd last step is peeled
    int k = 0;
    for (; k + 1 < U; k += 2) {
      step(k, S1, md);
      step(k + 1, S0, md);
    }
    if (k < U) step(k, S1, md);

    // ---- epilogue: D[i][j] of a 32x32 tile sits in lane j (+32 for the second
    // 4-row band) at register 4*(i/8) + i%4, i.e. row 8*(e/4) + 4*(lane/32) + e%4
    store_tile<TX, SC && MD != 0>(acc, Y, rexp, m, n, m0, n0, wm, wn, lane, t);
  };
  if (!SC || mode == 0) run(mm::mode_tag<0>{});
  else if (mode == 1) run(mm::mode_tag<1>{});
  else run(mm::mode_tag<2>{});
}

// ---- 64-column K-steps ------------------------------------------------------
// When every group holds an even number of 32-column units, a K-step of two
// units never straddles a group. Then: 128-byte activation rows per step (8
// lanes read one token row's full cache line), each thread dequantises one
// whole unit (32 weights) of its row, every wave issues 32 MFMAs per step,
// and one register stage suffices (tile k+2 is loaded during step k). LDS
// (160 KB): tables as above at 0, A [2][256 tokens][64 cols] and Bt [2][256
// rows][64 cols] in 128-byte rows (mm::swz128).
// For b = 4 the tables stay in registers (mm::dequant8_b4: byte-plane
// lookups with v_perm_b32, about 3 vector instructions per weight, no LDS
// gathers), loaded once per group, and the two threads of a row are adjacent
// lanes, so one index load instruction covers 32 rows x 32 contiguous bytes
// (32 cache lines instead of 64). Both MFMA operands are stored in the K
// order of dequant8_b4 within each 8-column chunk.
constexpr uint32_t A64_TILE = G_BM * 64u * 2u;            // 32768
constexpr uint32_t B64_TILE = G_BN * 64u * 2u;            // 32768
constexpr uint32_t LDS64_A = 2u * 4u * 16u * 64u * 4u;    // 32768
constexpr uint32_t LDS64_B = LDS64_A + 2u * A64_TILE;     // 98304
constexpr uint32_t LDS64_TOTAL = LDS64_B + 2u * B64_TILE; // 163840

// compile-time LDS buffer index of a K-step
template <int V> struct buf_tag { static constexpr uint32_t value = V; };

template <int B> struct Stage64 {
  uint32_t w[B];  // one whole unit
  u32x4 x[4];
};

template <int B, typename TX, typename TL>
__global__ void __launch_bounds__(G_THREADS, 1)
k_gemm_fwd64(const TX* __restrict__ X, const uint8_t* __restrict__ idx_packed, const TL* __restrict__ lut,
             int64_t m, int64_t n, int64_t d, int gpr, uint32_t ug_magic, int64_t mblocks, TX* __restrict__ Y,
             const int32_t* __restrict__ rexp) {
  constexpr bool SC = scaled_pair(__is_same(TX, bf16_t), __is_same(TL, half_t));
  // The block's conversion mode of its activation rows (bf16 with f16 tables:
  // block_scale_mode). Everything after it is compiled once per mode (run<MD>),
  // each copy with its own registers: only the kernel arguments cross the
  // dispatch, so the common mode 0 runs the loop 16-bit operands of the table
  // dtype would, and the modes that convert do not squeeze its registers.
  int mode = 0;
  if constexpr (SC) {
    const int64_t mb0 = (int64_t)(blockIdx.x % mblocks) * G_BM;
    uint32_t flags = 0u;
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const int64_t tok = mb0 + 64 * c + (threadIdx.x >> 3);
      flags |= scale_flags_of(rexp[tok < m ? tok : m - 1]);
    }
    mode = mm::block_scale_mode(flags, LDS64_B + B64_TILE);
  }
  auto run = [&](auto md) __attribute__((always_inline)) {
    constexpr int MD = decltype(md)::value;
    typedef mm::mfma32<TL> MF;
    extern __shared__ uint32_t smem[];
    (void)smem;

    const int t = threadIdx.x;
    const int lane = t & 63;
    const int wave = t >> 6;
    const uint32_t lane4 = (uint32_t)lane * 4u;
    const int64_t bm = blockIdx.x % mblocks;
    const int64_t bn = blockIdx.x / mblocks;
    const int64_t m0 = bm * G_BM, n0 = bn * G_BN;
    const int KS = (int)(d / 64);
    // group of tile j (both of its units are in it)
    auto group_of = [&](int j) -> uint32_t { return mm::group_of((uint32_t)(2 * j), ug_magic); };

    // ---- staging state: weight row r, unit hh of the step; activation chunk
    // t % 8 of token rows t / 8 + 64 c. b = 4 pairs adjacent lanes on one row
    // (32 contiguous index bytes per row and step); the LDS tables of b = 2, 3
    // need hh wave-uniform (threads t and t + 256 fill one lane's table copy).
    const int r = B == 4 ? (t >> 1) : (t & 255);
    const int hh = B == 4 ? (t & 1) : (t >> 8);
    const uint32_t rq = (uint32_t)(wave & 3);  // row quarter of r (b = 2, 3)
    const int64_t grow = (n0 + r < n) ? n0 + r : n - 1;
    const uint8_t* rowp = idx_packed + grow * (d * B / 8) + hh * (4 * B);
    const uint16_t* lutrow = reinterpret_cast<const uint16_t*>(lut) + grow * (int64_t)gpr * (1 << B);
    const TX* xrow[4];
    int xe[4] = {0, 0, 0, 0};  // SC: exponents of the four staged token rows
  #pragma unroll
    for (int c = 0; c < 4; ++c) {
      const int64_t tok = m0 + 64 * c + (t >> 3);
      xrow[c] = X + (tok < m ? tok : m - 1) * d + 8 * (t & 7);
      if constexpr (SC && MD != 0) xe[c] = rexp[tok < m ? tok : m - 1];
    }
    float xsc[4] = {1.0f, 1.0f, 1.0f, 1.0f};
    uint32_t xk[4] = {0u, 0u, 0u, 0u};
  #pragma unroll
    for (int c = 0; c < (int)(sizeof(xe) / sizeof(xe[0])); ++c) {
      if constexpr (MD == 2) xsc[c] = pow2f(-xe[c]);
      if constexpr (MD == 1) xk[c] = exp_add_word(xe[c]);
    }
    (void)xsc;
    (void)xk;
    auto load_stage = [&](Stage64<B>& S, int j) {
      const uint8_t* p = rowp + (int64_t)j * (8 * B);
      if constexpr (B == 4) {
        const u32x4 v = *reinterpret_cast<const u32x4*>(p);
        S.w[0] = v.x; S.w[1] = v.y; S.w[2] = v.z; S.w[3] = v.w;
      } else if constexpr (B == 2) {
        const u32x2 v = *reinterpret_cast<const u32x2*>(p);
        S.w[0] = v.x; S.w[1] = v.y;
      } else {
        const uint32_t* q = reinterpret_cast<const uint32_t*>(p);
        S.w[0] = q[0]; S.w[1] = q[1]; S.w[2] = q[2];
      }
  #pragma unroll
      for (int c = 0; c < 4; ++c) S.x[c] = *reinterpret_cast<const u32x4*>(xrow[c] + (int64_t)j * 64);
    };
    Stage64<B> S;
    // b = 4: the table of the group being staged, as byte planes (P), and the
    // next group's table as loaded (Ln); the group changes every UG/2 steps
    mm::Planes16 P;
    uint32_t Ln[8];
    uint32_t cur_g = 0xFFFFFFFFu;
    auto load_tab = [&](uint32_t g) {
      const u32x4* tp = reinterpret_cast<const u32x4*>(lutrow + g * 16u);
      const u32x4 a = tp[0], b = tp[1];
      Ln[0] = a.x; Ln[1] = a.y; Ln[2] = a.z; Ln[3] = a.w;
      Ln[4] = b.x; Ln[5] = b.y; Ln[6] = b.z; Ln[7] = b.w;
    };
    LutRegs<B> L;
    // LDS write addresses of the thread's four weight chunks and of its first
    // activation chunk (the other three are 64 rows = 8 KB further: the
    // swizzle of a row repeats every 16 rows); the buffer is a compile-time
    // offset, so every write takes its address from one of these registers
    // plus an immediate
    uint32_t bst[4];
  #pragma unroll
    for (int q = 0; q < 4; ++q) bst[q] = LDS64_B + swz128((uint32_t)r, 4u * hh + q);
    const uint32_t ast = LDS64_A + swz128((uint32_t)(t >> 3), (uint32_t)(t & 7));
    auto stage = [&](const Stage64<B>& St, int j, auto md, auto bufc) __attribute__((always_inline)) {
      constexpr int MD = decltype(md)::value;
      constexpr uint32_t buf = decltype(bufc)::value;
      if constexpr (B == 4) {
        // tables in registers; both operands in the K order of dequant8_b4
        const uint32_t g = group_of(j);
        if (g != cur_g) {
          mm::planes16(Ln, P);
          cur_g = g;
          load_tab(g + 1 < (uint32_t)gpr ? g + 1 : g);
        }
  #pragma unroll
        for (int q = 0; q < 4; ++q) st_q(bst[q] + buf * B64_TILE, mm::dequant8_b4(St.w[q], P));
  #pragma unroll
        for (int c = 0; c < 4; ++c) {
          const uint32_t a = ast + buf * A64_TILE + 8192u * c;
          if constexpr (SC && MD == 2) st_q(a, mm::cvt_quad_perm_scaled(St.x[c], xsc[c]));
          else if constexpr (SC && MD == 1) st_q(a, mm::cvt_quad_perm<TX, TL>(mm::add_quad(St.x[c], xk[c])));
          else st_q(a, mm::cvt_quad_perm<TX, TL>(St.x[c]));
        }
      } else {
        const uint32_t tb = tab_base<B>(group_of(j) & 1u, rq);
        uint32_t o0[8], o1[8];
        Stage<B> h0, h1;  // the two half units in the layout dequant16 expects
        if constexpr (B == 2) {
          h0.w[0] = St.w[0];
          h1.w[0] = St.w[1];
        } else {
          h0.w[0] = h1.w[0] = St.w[0];
          h0.w[1] = h1.w[1] = St.w[1];
          h0.w[2] = h1.w[2] = St.w[2];
        }
        dequant16<B, 0>(h0, tb, lane4, o0);
        dequant16<B, 1>(h1, tb, lane4, o1);
        st_q(bst[0] + buf * B64_TILE, u32x4{o0[0], o0[1], o0[2], o0[3]});
        st_q(bst[1] + buf * B64_TILE, u32x4{o0[4], o0[5], o0[6], o0[7]});
        st_q(bst[2] + buf * B64_TILE, u32x4{o1[0], o1[1], o1[2], o1[3]});
        st_q(bst[3] + buf * B64_TILE, u32x4{o1[4], o1[5], o1[6], o1[7]});
  #pragma unroll
        for (int c = 0; c < 4; ++c) {
          const uint32_t a = ast + buf * A64_TILE + 8192u * c;
          if constexpr (SC && MD == 2) st_q(a, mm::cvt_quad_scaled(St.x[c], xsc[c]));
          else if constexpr (SC && MD == 1) st_q(a, mm::cvt_quad<TX, TL>(mm::add_quad(St.x[c], xk[c])));
          else st_q(a, mm::cvt_quad<TX, TL>(St.x[c]));
        }
      }
    };
    // staging work of step k: tile k+1 into the other buffer, S refilled with
    // tile k+2, tables kept one group ahead
    auto stage_step = [&](int k, auto md, auto bufc) __attribute__((always_inline)) {
      if (k + 1 >= KS) return;
      stage(S, k + 1, md, bufc);
      if (k + 2 < KS) {
        load_stage(S, k + 2);
        if constexpr (B != 4) {
          const uint32_t g2 = group_of(k + 2);
          if (g2 != group_of(k + 1)) store_lut<B>(L, tab_base<B>(g2 & 1u, rq), hh, lane4);
          if (k + 3 < KS && group_of(k + 3) != g2) load_lut<B, TL>(L, lut, grow, gpr, group_of(k + 3), hh);
        }
      }
    };

    // ---- matrix state
    const int wm = wave & 1, wn = wave >> 1;
    const uint32_t arow = (uint32_t)(128 * wm + (lane & 31));
    const uint32_t brow = (uint32_t)(64 * wn + (lane & 31));
    const uint32_t khalf = (uint32_t)(lane >> 5);
    f32x16 acc[4][2];
  #pragma unroll
    for (int i = 0; i < 4; ++i)
  #pragma unroll
      for (int jj = 0; jj < 2; ++jj) mm::zero16(acc[i][jj]);
    // fragment read addresses of quarter ks in buffer 0; fragments 32 rows
    // apart are 4 KB apart (the swizzle repeats every 16 rows), and the buffer
    // is a compile-time offset: every read is one of these plus an immediate
    uint32_t ard[4], brd[4];
  #pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      ard[ks] = LDS64_A + swz128(arow, (uint32_t)(2 * ks) + khalf);
      brd[ks] = LDS64_B + swz128(brow, (uint32_t)(2 * ks) + khalf);
    }
    auto load_frags = [&](u32x4* fa, u32x4* fb, uint32_t buf, int ks) __attribute__((always_inline)) {
  #pragma unroll
      for (int i = 0; i < 4; ++i) fa[i] = ld_q(ard[ks] + buf * A64_TILE + 4096u * i);
  #pragma unroll
      for (int jj = 0; jj < 2; ++jj) fb[jj] = ld_q(brd[ks] + buf * B64_TILE + 4096u * jj);
    };
    // The matrix phase runs at raised wave priority, so that while the other
    // wave of the SIMD stages, its vector work does not hold back the next
    // MFMA issue.
    auto mfma_step = [&](auto bufc) __attribute__((always_inline)) {
      constexpr uint32_t buf = decltype(bufc)::value;
      __builtin_amdgcn_s_setprio(1);
      u32x4 fa[4][4], fb[4][2];
  #pragma unroll
      for (int ks = 0; ks < 4; ++ks) load_frags(fa[ks], fb[ks], buf, ks);
  #pragma unroll
      for (int ks = 0; ks < 4; ++ks)
  #pragma unroll
        for (int i = 0; i < 4; ++i)
  #pragma unroll
          for (int jj = 0; jj < 2; ++jj) acc[i][jj] = MF::run(fa[ks][i], fb[ks][jj], acc[i][jj]);
      // each quarter's fragment reads interleaved with the previous quarter's MFMAs
      __builtin_amdgcn_sched_group_barrier(0x100, 6, 0);
  #pragma unroll
      for (int ks = 1; ks < 4; ++ks) {
  #pragma unroll
        for (int q = 0; q < 2; ++q) {
          __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
          __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
        }
  #pragma unroll
        for (int q = 0; q < 2; ++q) {
          __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
          __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
        }
      }
      __builtin_amdgcn_sched_group_barrier(0x008, 8, 0);
      __builtin_amdgcn_sched_barrier(0);
      __builtin_amdgcn_s_setprio(0);
    };
    const bool mfma_first = wave < 4;

    // ---- prologue: tables of tile 0's group (tile 1's in registers if new),
    // tile 0 staged, tile 1 in registers, then tile 1's table staged and tile
    // 2's loaded as in a step
    if constexpr (B == 4) {
      load_tab(group_of(0));
      load_stage(S, 0);
      stage(S, 0, md, buf_tag<0>{});
      if (KS > 1) load_stage(S, 1);
    } else {
      load_lut<B, TL>(L, lut, grow, gpr, group_of(0), hh);
      load_stage(S, 0);
      store_lut<B>(L, tab_base<B>(group_of(0) & 1u, rq), hh, lane4);
      const bool new1 = KS > 1 && group_of(1) != group_of(0);
      if (new1) load_lut<B, TL>(L, lut, grow, gpr, group_of(1), hh);
      __syncthreads();
      stage(S, 0, md, buf_tag<0>{});
      if (KS > 1) load_stage(S, 1);
      if (new1) store_lut<B>(L, tab_base<B>(group_of(1) & 1u, rq), hh, lane4);
      if (KS > 2 && group_of(2) != group_of(1)) load_lut<B, TL>(L, lut, grow, gpr, group_of(2), hh);
    }
    __syncthreads();

    // step k multiplies buffer k & 1 and stages the other; two steps per trip
    // keep both buffer offsets compile-time
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
    int k = 0;
    for (; k + 1 < KS; k += 2) {
      step(k, buf_tag<0>{}, buf_tag<1>{});
      step(k + 1, buf_tag<1>{}, buf_tag<0>{});
    }
    if (k < KS) step(k, buf_tag<0>{}, buf_tag<1>{});
    store_tile<TX, SC && MD != 0>(acc, Y, rexp, m, n, m0, n0, wm, wn, lane, t);
  };
  if (!SC || mode == 0) run(mm::mode_tag<0>{});
  else if (mode == 1) run(mm::mode_tag<1>{});
  else run(mm::mode_tag<2>{});
}

template <int B, typename TX, typename TL>
hipError_t gemm_fwd_b(const TX* X, const uint8_t* idx, const TL* lut, const Problem& p, TX* Y,
                      const int32_t* rexp, hipStream_t s) {
  const int64_t mb = (p.m + G_BM - 1) / G_BM;
  const int64_t nb = (p.n + G_BN - 1) / G_BN;
  const uint32_t ug = (uint32_t)(p.group_cols() / 32);
  const uint32_t magic = ug == 1 ? 0u : (uint32_t)((((uint64_t)1) << 32) / ug + 1);
  if (ug % 2 == 0) {
    const auto kern = k_gemm_fwd64<B, TX, TL>;
    static const hipError_t prep = prepare_kernel((const void*)kern, LDS64_TOTAL);
    if (prep != hipSuccess) return prep;
    hipLaunchKernelGGL(kern, dim3((unsigned)(mb * nb)), dim3(G_THREADS), LDS64_TOTAL, s, X, idx, lut, p.m, p.n,
                       p.d, p.gpr, magic, mb, Y, rexp);
    return hipGetLastError();
  }
  const auto kern = k_gemm_fwd<B, TX, TL>;
  static const hipError_t prep = prepare_kernel((const void*)kern, LDS_TOTAL);
  if (prep != hipSuccess) return prep;
  hipLaunchKernelGGL(kern, dim3((unsigned)(mb * nb)), dim3(G_THREADS), LDS_TOTAL, s, X, idx, lut, p.m, p.n, p.d,
                     p.gpr, magic, mb, Y, rexp);
  return hipGetLastError();
}

template <typename TX, typename TL>
hipError_t gemm_fwd_t(const TX* X, const uint8_t* idx, const TL* lut, const Problem& p, TX* Y, const int32_t* rexp,
                      hipStream_t s) {
  switch (p.b) {
    case 2: return gemm_fwd_b<2>(X, idx, lut, p, Y, rexp, s);
    case 3: return gemm_fwd_b<3>(X, idx, lut, p, Y, rexp, s);
    default: return gemm_fwd_b<4>(X, idx, lut, p, Y, rexp, s);
  }
}

}  // namespace

bool gemm_fwd_supported(const Problem& p) {
  // group index by multiply-high is exact while units * units-per-group < 2^32
  return p.d <= (int64_t(1) << 20) && p.n * p.m < (int64_t(1) << 62);
}

hipError_t launch_gemm_fwd(const void* X, int x_dtype, const uint8_t* idx, const void* lut, int lut_dtype,
                           const Problem& p, void* Y, const int32_t* rexp, hipStream_t s) {
  if (x_dtype == DT_F16 && lut_dtype == DT_F16)
    return gemm_fwd_t((const half_t*)X, idx, (const half_t*)lut, p, (half_t*)Y, nullptr, s);
  if (x_dtype == DT_BF16 && lut_dtype == DT_F16)
    return gemm_fwd_t((const bf16_t*)X, idx, (const half_t*)lut, p, (bf16_t*)Y, rexp, s);
  if (x_dtype == DT_F16 && lut_dtype == DT_BF16)
    return gemm_fwd_t((const half_t*)X, idx, (const bf16_t*)lut, p, (half_t*)Y, nullptr, s);
  return gemm_fwd_t((const bf16_t*)X, idx, (const bf16_t*)lut, p, (bf16_t*)Y, nullptr, s);
}

}  // namespace skm
