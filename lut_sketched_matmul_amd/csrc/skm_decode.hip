// Decode-sized forward pass Y = X W^T for m <= 16 tokens (gfx950).
//
// "SpaLLM" (abstract, section 2.3; Table 5) runs inference as one compressed
// matmul per layer: table lookup plus accumulate, with every weight index
// streamed once per token. At m <= 16 that stream is the whole cost (the
// operation is HBM-bound), so the kernel reads idx_packed exactly once with
// wide loads and spends as few vector-ALU operations per weight as it can.
//
// Mapping onto the matrix cores. One v_mfma_f32_16x16x32 (f16 or bf16) takes
// A = X fragment (16 tokens x 32 columns) and B = W^T fragment (32 columns x
// 16 weight rows). Lane l holds A[token l%16][8 columns] and B[8 columns][row
// l%16] for quarter q = l/16 of the 32 contraction slots. The contraction
// order is free, so quarter q's slots are simply 8 columns of the 32-column
// unit that lane loads: lane (row j, quarter q) of a wave loads unit 4s+q of
// row j with one 16/8/12-byte load (b = 4/2/3) and dequantises it into four B
// fragments; the A fragments are X at the same columns. Padding tokens
// (m < 16) cost matrix-core time only, which this kernel leaves idle anyway;
// the vector ALUs and the LDS do the dequantisation.
//
// Tables. Every lane gathers from its own private copy of its row's tables in
// LDS, laid out entry-major / lane-minor (byte (entry*64 + lane)*4), so the 64
// lanes of a gather hit 64 distinct banks whatever the indices are. With the
// entry number e' = g*T + e in byte 1 of the address, one v_perm_b32 builds a
// gather address from a byte-lane-aligned index field. For b = 4 and b = 3 a
// table entry is one weight (T = 2^b); for b = 2 it is a *pair* of weights
// (T = 16 entries, entry a + 4c holds (LUT[a], LUT[c]) packed as f16x2), so
// one 32-bit gather yields two MFMA operand halves. The copies for the
// block's 16 rows are written once per launch, after the first index loads
// have been issued.
//
// Work split. Block = 16 weight rows x all d columns, NW waves. Wave w handles
// slots s = w, w + NW, ... (slot = 4 units = 128 columns), so the waves of a
// block read adjacent pieces of each row. The NW partial 16x16 tiles are
// summed in LDS in wave order (deterministic) and stored once.
//
// Activations. When m*d <= 32768 the block stages X in LDS once and reads its
// fragments there (below 8 tokens also up to 49152 elements when the grid has
// at most one block per CU and the LDS fits, see
// decode_stages_activations). Otherwise they come from global memory with
// each slot:
// below 8 tokens every lane loads its own fragment (64-byte runs of at most
// m distinct rows). From 8 tokens on such a load spreads over 64 separate
// 16-byte pieces of up to 16 rows, which the load unit handles piece by
// piece, so each wave loads its slot's [16 tokens][256 bytes] with
// neighbouring lanes on neighbouring pieces instead (four fully used 1 KB
// loads), stores them in a private LDS buffer (rows padded by 16 bytes, so
// the fragment reads hit distinct banks) and reads the four fragments back.
// One wave's LDS operations complete in order, so no barrier is involved.
//
// bf16 activations with f16 tables take the per-row prescale of skm_common.h.
// When the activations are staged in LDS, the block finds the exponents
// itself. One table set: the activations are staged unscaled and every wave
// records, beside them, whether any value reaches 2^16 and which rows hold a
// value of at least 2^-2; after the staging barrier every row lying in
// [2^-2, 2^16) (row_exp_of gives 0, the common case) means nothing more is
// done. Otherwise (block-uniform) the block re-reads its activations, finds
// each row's largest magnitude (below), stages them again prescaled and
// passes one more barrier. Several sets: each pass takes that exact path
// directly. The exact path: every lane folds the maxima of its chunks in
// registers; when all of a wave's chunks lie in one row (always for one
// token) a DPP reduction leaves the wave's maximum in one lane, which writes
// it to the wave's own LDS slot, else every lane adds its running maximum
// with an LDS atomic max per run of chunks in one row; one barrier, then each
// lane reduces the slots of the rows it needs. Without staging, the row
// exponents come from the caller's workspace.
#include "skm_common.h"
#include "skm_launch.h"

namespace skm {

namespace {

constexpr int DEC_ROWS = 16;
// slots loaded per batch and wave: a batch of NW waves covers 32 slots
template <int NW> struct dec_pf { static constexpr int value = 32 / NW; };
constexpr int DEC_MAX_ENTRIES = 224;  // table entries per row kept in LDS (entry byte must fit in 8 bits)
constexpr int DEC_LUT_CHUNKS = 2;     // 8-entry table chunks loaded per wave (16 * 2 * 8 >= 224)
constexpr int64_t DEC_XL_MAX = 32768; // m * d elements staged in LDS (64 KB)
constexpr int DEC_XL_CHUNKS = (int)(DEC_XL_MAX / 8 / (8 * 64));  // 16-byte chunks per thread (NW >= 8)
// one table set, at most one 16-row block per CU: up to 96 KB of staged
// activations when the block's LDS still fits
constexpr int64_t DEC_XL_MAX1 = 49152;
constexpr int DEC_XL_CHUNKS1 = (int)(DEC_XL_MAX1 / 8 / (8 * 64));
// unstaged activations: every wave turns its slot's [16 tokens][16 pieces of
// 16 bytes] around in a private LDS buffer, rows padded by one piece
constexpr uint32_t DEC_XT_ROW = 17 * 16;
constexpr uint32_t DEC_XT_WAVE = 16 * DEC_XT_ROW;
constexpr int DEC_XT_MIN_M = 8;  // tokens from which unstaged single-set calls take the turn-around

typedef __attribute__((address_space(3))) uint16_t lds_u16;
typedef __attribute__((address_space(3))) uint32_t lds_u32;

template <typename TC> struct mfma16;
template <> struct mfma16<half_t> {
  typedef f16x8 vec;
  static __device__ __forceinline__ f32x4 run(vec a, vec b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
  }
};
template <> struct mfma16<bf16_t> {
  typedef bf16x8 vec;
  static __device__ __forceinline__ f32x4 run(vec a, vec b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
  }
};

template <bool V> struct btag { static constexpr bool value = V; };

// table entries per group for bit width B (b = 2 stores pairs)
template <int B> struct tab_entries { static constexpr int value = (B == 2) ? 16 : (1 << B); };

// 8 activations (16-bit storage TX) -> packed compute dtype TC, two at a time
// through fp32 (exact widening, then one packed round-to-nearest-even convert)
typedef _Float16 f16x2_t __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

// bf16 -> f16 with every value multiplied by s (a power of two) first
__device__ __forceinline__ u32x4 x_to_tc_scaled(u32x4 v, float s) {
  u32x4 o;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    f16x2_t r;
    r.x = (half_t)(__builtin_bit_cast(float, v[q] << 16) * s);
    r.y = (half_t)(__builtin_bit_cast(float, v[q] & 0xFFFF0000u) * s);
    o[q] = __builtin_bit_cast(uint32_t, r);
  }
  return o;
}

template <typename TX, typename TC>
__device__ __forceinline__ u32x4 x_to_tc(u32x4 v) {
  if constexpr (__is_same(TX, TC)) {
    return v;
  } else {
    u32x4 o;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      float lo, hi;
      if constexpr (__is_same(TX, bf16_t)) {
        lo = __builtin_bit_cast(float, v[q] << 16);
        hi = __builtin_bit_cast(float, v[q] & 0xFFFF0000u);
      } else {
        // (bit-casting the vector element itself to a 2 x f16 vector is
        // miscompiled by this hipcc into a splat of element 0; go through
        // 16-bit integers instead)
        const uint32_t w = v[q];
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

// LDS byte address of byte-lane p of `ent` (entry number) for this lane:
// [lane*4, ent.byte_p, 0, 0]
__device__ __forceinline__ uint32_t gaddr(uint32_t ent, uint32_t lane4, int p) {
  return __builtin_amdgcn_perm(ent, lane4, 0x0C0C0400u | ((4u + (uint32_t)p) << 8));
}

__device__ __forceinline__ uint32_t lds_h(uint32_t addr) { return *(const lds_u16*)(uintptr_t)addr; }
__device__ __forceinline__ uint32_t lds_w(uint32_t addr) { return *(const lds_u32*)(uintptr_t)addr; }
__device__ __forceinline__ uint32_t pack2(uint32_t lo, uint32_t hi) {
  return __builtin_amdgcn_perm(hi, lo, 0x05040100u);
}

// Dequantise MFMA step h (fields 8h..8h+7) of one unit into a packed B fragment.
// gk = this unit's group times the entries per group (all four bytes set).
template <int B>
__device__ __forceinline__ u32x4 dequant_step(const uint32_t* w, int h, uint32_t gk4, uint32_t gk, uint32_t lane4) {
  u32x4 r;
  if constexpr (B == 4) {
    // dword h holds fields 8h..8h+7 as nibbles; even/odd nibbles to byte lanes
    const uint32_t ev = (w[h] & 0x0F0F0F0Fu) | gk4;
    const uint32_t od = ((w[h] >> 4) & 0x0F0F0F0Fu) | gk4;
#pragma unroll
    for (int t = 0; t < 4; ++t) r[t] = pack2(lds_h(gaddr(ev, lane4, t)), lds_h(gaddr(od, lane4, t)));
  } else if constexpr (B == 2) {
    // pair (8h+2t, 8h+2t+1) = nibble t of the 16-bit half h%2 of dword h/2
    const uint32_t half = (h & 1) ? (w[h >> 1] >> 16) : (w[h >> 1] & 0xFFFFu);
    const uint32_t nib = (half & 0x0F0Fu) | ((half & 0xF0F0u) << 12);  // nibbles 0,2 -> bytes 0,1; 1,3 -> 2,3
    const uint32_t ent = nib | gk4;
    r[0] = lds_w(gaddr(ent, lane4, 0));
    r[1] = lds_w(gaddr(ent, lane4, 2));
    r[2] = lds_w(gaddr(ent, lane4, 1));
    r[3] = lds_w(gaddr(ent, lane4, 3));
  } else {
    // 3-bit fields at arbitrary bit offsets: extract, then (gk + e) << 8 | lane*4
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      const uint32_t e0 = unit_field<3>(w, 8 * h + 2 * t);
      const uint32_t e1 = unit_field<3>(w, 8 * h + 2 * t + 1);
      const uint32_t a0 = ((gk + e0) << 8) | lane4;
      const uint32_t a1 = ((gk + e1) << 8) | lane4;
      r[t] = pack2(lds_h(a0), lds_h(a1));
    }
  }
  return r;
}

// Private table copies. Row j = lane%16 of the block; every wave writes whole
// 64-lane entry rows, so each ds_write is conflict-free. The loads are issued
// before the first index loads and stored after them (vmcnt counts in order).
template <int B> struct TabRegs { uint32_t v[2 * DEC_LUT_CHUNKS][4]; };

template <int B, int NW, typename TL>
__device__ __forceinline__ void tab_load(TabRegs<B>& R, const TL* __restrict__ lut, int64_t grow, int gpr, int wave) {
  constexpr int K = 1 << B;
  const uint16_t* src = reinterpret_cast<const uint16_t*>(lut) + grow * (int64_t)gpr * K;
#pragma unroll
  for (int c = 0; c < DEC_LUT_CHUNKS * (16 / NW); ++c) {
    const int ch = wave + NW * c;
    // unconditional loads (a chunk past the row's tables re-reads chunk 0 and
    // is not stored) so that the compiler can count them
    if constexpr (B == 2) {
      // chunk = one group's 4 entries
      const int cc = ch < gpr ? ch : 0;
      const u32x2 v = *reinterpret_cast<const u32x2*>(src + cc * 4);
      R.v[c][0] = v.x;
      R.v[c][1] = v.y;
    } else {
      const int cc = ch * 8 < gpr * K ? ch : 0;
      const u32x4 v = *reinterpret_cast<const u32x4*>(src + cc * 8);
      R.v[c][0] = v.x; R.v[c][1] = v.y; R.v[c][2] = v.z; R.v[c][3] = v.w;
    }
  }
}

template <int B, int NW>
__device__ __forceinline__ void tab_store(const TabRegs<B>& R, uint32_t* tabs, int gpr, int lane, int wave) {
  constexpr int K = 1 << B;
#pragma unroll
  for (int c = 0; c < DEC_LUT_CHUNKS * (16 / NW); ++c) {
    const int ch = wave + NW * c;
    if constexpr (B == 2) {
      if (ch < gpr) {
        const uint32_t e[4] = {R.v[c][0] & 0xFFFFu, R.v[c][0] >> 16, R.v[c][1] & 0xFFFFu, R.v[c][1] >> 16};
#pragma unroll
        for (int cc = 0; cc < 4; ++cc)
#pragma unroll
          for (int a = 0; a < 4; ++a) tabs[(ch * 16 + a + 4 * cc) * 64 + lane] = e[a] | (e[cc] << 16);
      }
    } else {
      if (ch * 8 < gpr * K) {
#pragma unroll
        for (int t = 0; t < 4; ++t) {
          tabs[(ch * 8 + 2 * t) * 64 + lane] = R.v[c][t] & 0xFFFFu;
          tabs[(ch * 8 + 2 * t + 1) * 64 + lane] = R.v[c][t] >> 16;
        }
      }
    }
  }
}

// Sources of one wave's coalesced activation loads (unstaged, one table set):
// load i of a slot brings token min(4i + l/16, m-1) (element offset off[i])
// at columns 128 s + c8, c8 = 8 (l%16), clamped to dcol = d - 8 when the
// row ends inside the slot.
template <typename TX>
struct XtSrc {
  const TX* x = nullptr;
  uint32_t off[4] = {0u, 0u, 0u, 0u};
  uint32_t c8 = 0u;
  uint32_t dcol = 0u;
};

template <int B, typename TX, int PF>
struct SlotRegs {
  uint32_t w[PF][B];
  u32x4 x[PF][4];
  uint32_t gk[PF];
  uint32_t u[PF];
  bool ok[PF];
};

// Issue the index and activation loads of PF slots. Addresses are clamped in
// range instead of masked, and the loads are unconditional (so the compiler
// can count them and wait for one batch while the next is in flight): a slot
// past the last one re-reads the last slot and is skipped by the caller, a
// token row >= m or a weight row >= n only feeds outputs that are never
// stored, and a unit past the row end (RAGGED only) is zeroed by the caller.
// g = u / UG is a multiply-high by the host's magic constant (exact for
// u * UG < 2^32). XT: the activations arrive in load order (see XtSrc) and
// are put into fragment order by the caller.
template <int B, int NW, typename TX, bool RAGGED, bool XL, bool XT, int PF>
__device__ __forceinline__ void load_batch(SlotRegs<B, TX, PF>& R, int64_t s0, int64_t S, uint32_t U,
                                           uint32_t ug_magic, int q, const uint8_t* rowp, const TX* xrow,
                                           const XtSrc<TX>& xt) {
  constexpr int T = tab_entries<B>::value;
#pragma unroll
  for (int p = 0; p < PF; ++p) {
    const int64_t sp = s0 + (int64_t)p * NW;
    const int64_t s = sp < S ? sp : S - 1;
    uint32_t u = 4u * (uint32_t)s + (uint32_t)q;
    if constexpr (RAGGED) {
      R.ok[p] = u < U;
      u = u < U ? u : U - 1u;
    }
    load_unit<B>(rowp, u, R.w[p]);
    R.u[p] = u;
    if constexpr (XT) {
      uint32_t col = 128u * (uint32_t)s + xt.c8;
      if constexpr (RAGGED) col = col < xt.dcol ? col : xt.dcol;
#pragma unroll
      for (int i = 0; i < 4; ++i) R.x[p][i] = *reinterpret_cast<const u32x4*>(xt.x + xt.off[i] + col);
    } else if constexpr (!XL) {
      const u32x4* xp = reinterpret_cast<const u32x4*>(xrow + (int64_t)u * 32);
#pragma unroll
      for (int h = 0; h < 4; ++h) R.x[p][h] = xp[h];
    }
    R.gk[p] = (ug_magic ? __umulhi(u, ug_magic) : u) * T;  // magic 0: one unit per group
  }
}

// s_waitcnt that bounds only the vector-memory counter (gfx9 encoding: vmcnt
// in bits 3:0 and 15:14; expcnt 7 and lgkmcnt 15 mean "no wait").
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt is a 6-bit field");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

template <typename T>
__device__ __forceinline__ u32x4 lds_q16(uint32_t a) {
  return *(const __attribute__((address_space(3))) u32x4*)(uintptr_t)a;
}

// XL: the activations (m x d, converted to the compute dtype) are staged once
// per block in LDS after the tables, and A fragments are read from there;
// otherwise each slot's A fragments are loaded from global memory with its
// index words. The next batch of slots is loaded while the current one is
// being computed (two register sets), except for activations in registers at
// 4 slots per batch.
// MULTI: several table sets over the one index stream ("SpaLLM", section 2.3:
// every adapter is a set of tables in the same format over the frozen
// mapping), token t using set lut_set[t] (clamped into [0, n_sets)). The block
// takes one pass per set that some token uses, in the order of first use:
// stage that set's tables (and, with XL, the activations of that set's tokens
// only, so that a pass stages at most 32768 / d tokens and a set with more
// takes several passes), run the slot loop over all the block's weights
// (after the first pass the index words come from the L2), and keep for each
// output element the result of its token's pass. Each pass costs the set's
// tables and one round of table lookups; the index stream is read from memory
// once. A pass's tables, activations and first index batch are loaded during
// the pass before it.
template <int B, int NW, typename TX, typename TL, bool RAGGED, bool XL, bool XT, bool MULTI>
__global__ void __launch_bounds__(NW * 64)
k_decode(const TX* __restrict__ X, const uint8_t* __restrict__ idx_packed, const TL* __restrict__ lut,
         int m, int64_t n, int64_t d, int gpr, uint32_t ug_magic, uint32_t d_magic, TX* __restrict__ Y,
         const int32_t* __restrict__ lut_set, int n_sets, int64_t set_stride, const int32_t* __restrict__ rexp) {
  // Dynamic LDS only (this kernel has no static LDS, so it starts at address
  // 0): [entries][64 lanes] table dwords, [m][d] activations (XL), the
  // [NW][16][16] fp32 partials; SC with XL: the partials in the activations'
  // place at the end, then the [16 rows][NW waves] largest magnitudes of the
  // staged activation rows and the [NW] range records.
  extern __shared__ uint32_t smem[];
  constexpr int T = tab_entries<B>::value;
  typedef mfma16<TL> MF;
  constexpr bool SC = scaled_pair(__is_same(TX, bf16_t), __is_same(TL, half_t));
  static_assert(!(SC && MULTI && !XL), "prescaled multi-set decode stages its activations");
  // XT (one table set without staging, m >= 8): coalesced activation loads,
  // turned into fragments through a per-wave LDS buffer
  static_assert(!(XT && (XL || MULTI)), "the LDS turn-around serves unstaged single-set calls");

  const int lane = lane_id();
  // wave index as a scalar, so that the slot loop's branches are scalar
  // branches and every path through it is a real path
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int64_t row0 = (int64_t)blockIdx.x * DEC_ROWS;
  const int j = lane & 15;           // weight row within the block (B operand column)
  const int q = lane >> 4;           // contraction quarter
  const int64_t grow = row0 + j;
  const bool row_ok = grow < n;
  const int tok = lane & 15;         // A operand row = token (clamped: rows >= m are never stored)
  const int tokc = tok < m ? tok : m - 1;

  const uint32_t U = (uint32_t)(d / 32);         // units per row
  const int64_t S = (U + 3) / 4;                 // slots per row
  const uint8_t* rowp = idx_packed + (row_ok ? grow : n - 1) * (d * B / 8);
  const TX* xrow = X + (int64_t)tokc * d;
  XtSrc<TX> xts;
  if constexpr (XT) {
    xts.x = X;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int t = 4 * i + (lane >> 4);
      xts.off[i] = (uint32_t)((t < m ? t : m - 1) * d);
    }
    xts.c8 = 8u * (uint32_t)(lane & 15);
    xts.dcol = (uint32_t)d - 8u;
  }
  const uint32_t lane4 = (uint32_t)lane * 4u;
  const uint32_t xl_base = (uint32_t)gpr * T * 256u;  // byte offset of the staged activations
  // activation elements staged (MULTI + XL: one pass's tokens)
  const int64_t xl_elems =
      (int64_t)((MULTI && XL) ? (m < (int)(DEC_XL_MAX / d) ? m : (int)(DEC_XL_MAX / d)) : m) * d;
  // 16-byte activation chunks per thread (the larger staging only runs with 16 waves)
  constexpr int XCH = XL ? ((MULTI || NW < 16) ? DEC_XL_CHUNKS : DEC_XL_CHUNKS1) * 8 / NW : 1;
  // SC + XL: the partials overlay the staged activations (after a barrier
  // at the end), and the magnitude slots [16 rows][NW] and the waves' range
  // records [NW] follow that region (keeping the block's LDS near the f16
  // pair's, so as many blocks fit on a CU)
  const uint32_t xl_bytes = XL ? (uint32_t)((xl_elems + 7) / 8) * 16u : 0u;
  const uint32_t mag_base =
      xl_base + (SC && XL ? (xl_bytes > (uint32_t)NW * 1024u ? xl_bytes : (uint32_t)NW * 1024u)
                          : xl_bytes + (uint32_t)NW * 1024u);
  // SC: e of the activation row (staged row with XL, token otherwise) of lane % 16
  int erow = 0;
  if constexpr (SC && !XL) erow = rexp[(lane & 15) < m ? (lane & 15) : m - 1];

  // MULTI: the block's passes, worked out once in lanes. A pass covers the
  // tokens of one set, at most `cap` of them (with XL the pass stages only its
  // own tokens' activations: cap = min(m, activation elements that fit / d));
  // sets go in order of first use and a set with more than cap tokens takes
  // several passes (chunks of cap tokens in token order). Lane t (< m) holds
  // token t's set and its position in the pass-ordered token list (tokens of
  // earlier sets first, then by rank within the set); lane p holds pass p's
  // set, chunk, first list position and token count; lane i holds the token
  // at list position i.
  const int cap = (MULTI && XL) ? (m < (int)(DEC_XL_MAX / d) ? m : (int)(DEC_XL_MAX / d)) : m;
  int tpos = 0, ps_set = 0, ps_start = 0, ps_cnt = 0, sorted_tok = 0, npass = 1;
  if constexpr (MULTI) {
    const int tl = lane < m ? lane : m - 1;
    const int v = lut_set[tl];
    const int setv = v < 0 ? 0 : (v >= n_sets ? n_sets - 1 : v);
    int rank = 0, ftok = tl;  // rank of token tl in its set; the set's first token
    for (int u = 0; u < m; ++u) {
      const int su = __builtin_amdgcn_readlane(setv, u);
      if (su == setv) {
        rank += u < tl ? 1 : 0;
        ftok = u < ftok ? u : ftok;
      }
    }
    int before = 0, count = 0;  // tokens of sets used earlier; tokens of this set
    for (int u = 0; u < m; ++u) {
      const int fu = __builtin_amdgcn_readlane(ftok, u);
      before += fu < ftok ? 1 : 0;
      count += fu == ftok ? 1 : 0;
    }
    tpos = before + rank;
    const int nch = (lane < m && rank == 0) ? (count + cap - 1) / cap : 0;  // passes of a set, at its first token
    int pbase = 0;
    npass = 0;
    for (int u = 0; u < m; ++u) {
      const int nu = __builtin_amdgcn_readlane(nch, u);
      pbase += u < lane ? nu : 0;
      npass += nu;
    }
    for (int u = 0; u < m; ++u) {
      const int nu = __builtin_amdgcn_readlane(nch, u), bu = __builtin_amdgcn_readlane(pbase, u);
      if (nu > 0 && lane >= bu && lane < bu + nu) {
        ps_set = __builtin_amdgcn_readlane(setv, u);
        const int kc = lane - bu;  // chunk of the set
        ps_start = __builtin_amdgcn_readlane(before, u) + kc * cap;
        const int left = __builtin_amdgcn_readlane(count, u) - kc * cap;
        ps_cnt = left < cap ? left : cap;
      }
    }
    // lane tpos(t) receives t (lanes >= m repeat token m - 1's position and value)
    sorted_tok = __builtin_amdgcn_ds_permute(tpos * 4, tl);
  }
  // the four tokens whose outputs this lane holds (lane l: tokens 4 (l / 16) + r)
  int lpos[4] = {0, 0, 0, 0};
  int apos = 0;  // the token of this lane's A row
  if constexpr (MULTI) {
#pragma unroll
    for (int r = 0; r < 4; ++r) lpos[r] = __shfl(tpos, 4 * q + r < m ? 4 * q + r : m - 1, 64);
    apos = __shfl(tpos, tokc, 64);
  }
  int pass = 0;
  int cur = 0, pstart = 0, pcnt = m;  // this pass: set, first list position, tokens
  auto load_pass = [&](int pp) {
    cur = __builtin_amdgcn_readlane(ps_set, pp);
    pstart = __builtin_amdgcn_readlane(ps_start, pp);
    pcnt = __builtin_amdgcn_readlane(ps_cnt, pp);
  };
  if constexpr (MULTI) load_pass(0);
  // MULTI + XL: one pass's activation loads into registers, unconditional (a
  // chunk with no token of the pass re-reads X[0] and is not stored), so the
  // compiler's load counts stay exact
  auto stage_src = [&](int c, int st, int cnt, bool& ok) -> const TX* {
    const int64_t e = ((int64_t)c * NW * 64 + threadIdx.x) * 8;
    const int slot = (int)__umulhi((uint32_t)e, d_magic);  // e / d
    const int col = (int)(e - (int64_t)slot * d);
    ok = slot < cnt;
    const int t = __shfl(sorted_tok, ok ? st + slot : 0, 64);
    return ok ? X + (int64_t)t * d + col : X;
  };
  f32x4 out = {0.f, 0.f, 0.f, 0.f};
  constexpr int PF = dec_pf<NW>::value;
  SlotRegs<B, TX, PF> R0, R1;
  int64_t s0 = wave;
  TabRegs<B> TR;  // MULTI: after the first pass, loaded during the previous pass
  u32x4 xs[XCH];   // MULTI + XL: likewise the pass's activations
  bool xok[XCH];
  if constexpr (MULTI) {
    // the first pass's loads, issued before the loop so that every pass starts
    // with the same loads in flight, in the same order (tables, activations,
    // first index batch)
    tab_load<B, NW, TL>(TR, lut + (int64_t)cur * set_stride, row_ok ? grow : n - 1, gpr, wave);
    if constexpr (XL) {
#pragma unroll
      for (int c = 0; c < XCH; ++c) xs[c] = *reinterpret_cast<const u32x4*>(stage_src(c, pstart, pcnt, xok[c]));
    }
    load_batch<B, NW, TX, RAGGED, XL, XT, PF>(R0, (int64_t)wave, S, U, ug_magic, q, rowp, xrow, xts);
  }
  while (true) {
  const bool has_next = MULTI && pass + 1 < npass;
  // ---- prologue: table loads, activation loads (XL), first index loads, then
  // the LDS stores of the first two (their loads complete first). MULTI passes
  // find their tables, activations and first index batch loaded.
  if constexpr (!MULTI) {
    // one token of a multi-set call (lut_set given): the tables of its set
    const TL* lut1 = lut;
    if (lut_set) {
      const int v = __builtin_amdgcn_readfirstlane(lut_set[0]);
      lut1 = lut + (int64_t)(v < 0 ? 0 : (v >= n_sets ? n_sets - 1 : v)) * set_stride;
    }
    tab_load<B, NW, TL>(TR, lut1, row_ok ? grow : n - 1, gpr, wave);
  }
  // (a chunk past m*d is neither loaded nor read: giving it a value would
  // merge it with the load at a branch, which waits for the load there)
  auto load_x = [&]() {
#pragma unroll
    for (int c = 0; c < XCH; ++c) {
      const int64_t e = ((int64_t)c * NW * 64 + threadIdx.x) * 8;
      if (e < xl_elems) xs[c] = *reinterpret_cast<const u32x4*>(X + e);
    }
  };
  if constexpr (XL && !MULTI) load_x();
  s0 = wave;
  if constexpr (!MULTI) load_batch<B, NW, TX, RAGGED, XL, XT, PF>(R0, s0, S, U, ug_magic, q, rowp, xrow, xts);
  tab_store<B, NW>(TR, smem, gpr, lane, wave);
  // SC + XL: the exponent of a staged row from the waves' slots (NW maxima)
  auto row_slots_exp = [&](uint32_t row) -> int {
    uint32_t mx = 0;
#pragma unroll
    for (int q = 0; q < NW / 4; ++q) {
      const u32x4 w = lds_q16<TL>(mag_base + (row * NW + 4u * q) * 4u);
#pragma unroll
      for (int k = 0; k < 4; ++k) mx = mx > w[k] ? mx : w[k];
    }
    return row_exp_of(mx);
  };
  // SC + XL, exact path: the largest magnitude of every staged row into the
  // waves' slots, one barrier, then erow for the row of lane % 16
  auto exact_exponents = [&]() {
    // a wave's LDS accesses stay in order, so it zeroes its own slots first;
    // a lane's chunks lie in non-decreasing rows, so it keeps a running
    // maximum and adds it with one atomic max whenever the row changes
    typedef __attribute__((address_space(3))) uint32_t lds_u32_t;
    if (lane < 16) *(lds_u32_t*)(uintptr_t)(mag_base + ((uint32_t)lane * NW + wave) * 4u) = 0u;
    // the row of the wave's first element: when every valid chunk of the
    // wave lies in it, one DPP reduction and one store suffice
    const uint32_t row0 = __umulhi((uint32_t)(64 * wave * 8), d_magic);
    uint32_t run_row = 0u, run_max = 0u;
    bool one_row = true;
#pragma unroll
    for (int c = 0; c < XCH; ++c) {
      const int64_t e = ((int64_t)c * NW * 64 + threadIdx.x) * 8;
      const bool ok = MULTI ? xok[c] : e < xl_elems;
      const uint32_t row = __umulhi((uint32_t)e, d_magic);  // e / d
      if (ok) {
        one_row = one_row && row == row0;
        if (row != run_row && run_max != 0u)
          __hip_atomic_fetch_max((lds_u32_t*)(uintptr_t)(mag_base + (run_row * NW + wave) * 4u), run_max,
                                 __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
        if (row != run_row) run_max = 0u;
        run_row = row;
        const uint32_t v = absmax8_bf16(xs[c]);
        run_max = run_max > v ? run_max : v;
      }
    }
    if (__ballot(!one_row) == 0) {  // wave-uniform: the whole wave's chunks lie in row0
      const uint32_t mx = wave_max_to_lane63(run_max);
      // (mx == 0: no valid chunk, or only zeros; then row0 may lie past the staged rows and the slot stays 0)
      if (lane == 63 && mx != 0u) *(lds_u32_t*)(uintptr_t)(mag_base + (row0 * NW + wave) * 4u) = mx;
    } else if (run_max != 0u) {
      __hip_atomic_fetch_max((lds_u32_t*)(uintptr_t)(mag_base + (run_row * NW + wave) * 4u), run_max,
                             __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
    }
    __syncthreads();
    erow = row_slots_exp((uint32_t)(lane & 15));  // for the outputs of the row of lane % 16
  };
  // stage the activation chunks (prescaled by their rows' exponents, looked
  // up in the slots, or converted as they are)
  auto store_x = [&](auto scaled) {
    int crow = -1, cexp = 0;  // the exponent of the last chunk row looked up
#pragma unroll
    for (int c = 0; c < XCH; ++c) {
      const int64_t e = ((int64_t)c * NW * 64 + threadIdx.x) * 8;
      const bool ok = MULTI ? xok[c] : e < xl_elems;
      if (ok) {
        u32x4 v;
        if constexpr (decltype(scaled)::value) {
          const int row = (int)__umulhi((uint32_t)e, d_magic);  // e / d
          if (row != crow) {
            crow = row;
            cexp = row_slots_exp((uint32_t)row);
          }
          v = x_to_tc_scaled(xs[c], pow2f(-cexp));
        } else {
          v = x_to_tc<TX, TL>(xs[c]);
        }
        *(__attribute__((address_space(3))) u32x4*)(uintptr_t)(xl_base + (uint32_t)e * 2u) = v;
      }
    }
  };
  if constexpr (SC && XL && MULTI) {
    exact_exponents();
    store_x(btag<true>{});
  } else if constexpr (SC && XL) {
    // range record of this wave: bit r = row r holds a magnitude >= 2^-2,
    // bit 31 = some magnitude >= 2^16 (or an infinity or NaN)
    uint32_t rec = 0u;
#pragma unroll
    for (int c = 0; c < XCH; ++c) {
      const int64_t e = ((int64_t)c * NW * 64 + threadIdx.x) * 8;
      if (e < xl_elems) {
        const uint32_t v = absmax8_bf16(xs[c]);
        rec |= (v >= kNoScaleLo ? 1u << __umulhi((uint32_t)e, d_magic) : 0u) | (v >= kNoScaleHi ? 1u << 31 : 0u);
      }
    }
    rec = wave_or_to_lane63(rec);
    if (lane == 63) *(__attribute__((address_space(3))) uint32_t*)(uintptr_t)(mag_base + 64u * NW + wave * 4u) = rec;
    store_x(btag<false>{});
  } else if constexpr (XL) {
    store_x(btag<false>{});
  }
  // Every table and activation load has been consumed by now on the paths
  // that store it; the ones past the row's tables (or past m*d) were issued
  // but not consumed. Waiting for all but the first batch's index loads here
  // (at most 3 loads per slot) settles them on every path, so the compiler's
  // load counting below starts from the first batch alone.
  wait_vmcnt<PF * ((B == 3 ? 3 : 1) + (XL ? 0 : 4))>();
  __syncthreads();
  if constexpr (SC && XL && !MULTI) {
    // every staged row inside [2^-2, 2^16): no prescale (erow stays 0);
    // otherwise (block-uniform) re-read the activations and take the exact path
    uint32_t all = 0u;
#pragma unroll
    for (int q = 0; q < NW / 4; ++q) {
      const u32x4 w = lds_q16<TL>(mag_base + 64u * NW + 16u * q);
      all |= w[0] | w[1] | w[2] | w[3];
    }
    const uint32_t rows = (1u << m) - 1u;  // m <= 16 staged rows
    if ((all >> 31) != 0u || (all & rows) != rows) {
      load_x();
      exact_exponents();
      store_x(btag<true>{});
      __syncthreads();
    }
  }
  // this lane's A row: its token's staged row (MULTI + XL: the token's slot in
  // the pass, or slot 0 for a token outside the pass, whose results are not kept)
  int aslot = tokc;
  if constexpr (MULTI && XL) {
    const bool in = apos >= pstart && apos < pstart + pcnt;
    aslot = in ? apos - pstart : 0;
  }
  const uint32_t xl_row = xl_base + (uint32_t)aslot * (uint32_t)d * 2u;
  if constexpr (MULTI) {
    // the next pass's tables and activations (this pass's again when none is
    // left: the loads stay unconditional), in flight while this pass computes
    const int pn = has_next ? pass + 1 : pass;
    const int sn = __builtin_amdgcn_readlane(ps_set, pn);
    tab_load<B, NW, TL>(TR, lut + (int64_t)sn * set_stride, row_ok ? grow : n - 1, gpr, wave);
    if constexpr (XL) {
      const int stn = __builtin_amdgcn_readlane(ps_start, pn), cnn = __builtin_amdgcn_readlane(ps_cnt, pn);
#pragma unroll
      for (int c = 0; c < XCH; ++c) xs[c] = *reinterpret_cast<const u32x4*>(stage_src(c, stn, cnn, xok[c]));
    }
  }

  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  // XT: this wave's buffer; a lane stores load i at row 4i + l/16, piece
  // l%16, and reads step h of its fragment at row l%16 (its token), piece
  // 4 (l/16) + h: columns 8h.. of unit 4s + q, as a direct load would give
  const uint32_t xt_w = xl_base + (uint32_t)wave * DEC_XT_WAVE;
  const uint32_t xt_st = xt_w + (uint32_t)(lane >> 4) * DEC_XT_ROW + (uint32_t)(lane & 15) * 16u;
  const uint32_t xt_ld = xt_w + (uint32_t)(lane & 15) * DEC_XT_ROW + (uint32_t)(lane >> 4) * 64u;
  (void)xt_st;
  (void)xt_ld;
  // SC without staging: 2^-e of this lane's A row (its token)
  const float xsc = SC && !XL ? pow2f(-erow) : 1.0f;
  (void)xsc;
  // compute(R, first slot, tail): a batch can be partial only when it is a
  // wave's last one (tail = true); full batches carry no early exits, so every
  // path through them consumes all of their loads.
  auto compute = [&](const SlotRegs<B, TX, PF>& Rc, int64_t sb, auto tail) {
#pragma unroll
    for (int p = 0; p < PF; ++p) {
      if (decltype(tail)::value && sb + (int64_t)p * NW >= S) break;  // wave-uniform
      const uint32_t gk = Rc.gk[p];
      const uint32_t gk4 = __builtin_amdgcn_perm(0u, gk, 0u);  // gk < 256 in all four bytes
      // XT: the slot's activations through the wave's buffer (one wave's LDS
      // accesses are carried out in order, so the next slot's stores cannot
      // overtake these loads)
      u32x4 xf[4];
      if constexpr (XT) {
#pragma unroll
        for (int i = 0; i < 4; ++i)
          *(__attribute__((address_space(3))) u32x4*)(uintptr_t)(xt_st + (uint32_t)i * 4u * DEC_XT_ROW) = Rc.x[p][i];
#pragma unroll
        for (int h = 0; h < 4; ++h) xf[h] = lds_q16<TL>(xt_ld + 16u * (uint32_t)h);
      }
#pragma unroll
      for (int h = 0; h < 4; ++h) {
        u32x4 wb = dequant_step<B>(Rc.w[p], h, gk4, gk, lane4);
        // a slot past the row end (only when d/32 is not a multiple of 4) has
        // X = 0; its weights are zeroed too so no table value can leak in
        if constexpr (RAGGED) {
          if (!Rc.ok[p]) wb = u32x4{0u, 0u, 0u, 0u};
        }
        u32x4 xv;
        if constexpr (XL) xv = lds_q16<TL>(xl_row + (Rc.u[p] * 32u + 8u * h) * 2u);
        else if constexpr (SC) xv = x_to_tc_scaled(XT ? xf[h] : Rc.x[p][h], xsc);
        else xv = x_to_tc<TX, TL>(XT ? xf[h] : Rc.x[p][h]);
        if constexpr (RAGGED) {
          if (!Rc.ok[p]) xv = u32x4{0u, 0u, 0u, 0u};
        }
        acc = MF::run(__builtin_bit_cast(typename MF::vec, xv), __builtin_bit_cast(typename MF::vec, wb), acc);
      }
    }
  };
  constexpr int64_t STEP = (int64_t)NW * PF;
  // batches of PF slots this wave computes (at least one, which may be empty
  // when the row has fewer slots than the block has waves)
  const int64_t nb_raw = (S - s0 + STEP - 1) / STEP;
  const int64_t nb = nb_raw > 1 ? nb_raw : 1;
  if constexpr (XL || PF <= 2) {
    // Two register sets: the next batch is loaded while the current one is
    // computed. The loop has one exit and issues its loads unconditionally,
    // so the compiler knows exactly how many loads are younger than the batch
    // it waits for (a load under a condition, or a batch with early exits,
    // makes it wait as if fewer were in flight: every batch would then stall
    // on the next one's first load); the last one or two batches run after it.
    int64_t b = 0;
    for (; b + 2 < nb; b += 2) {
      load_batch<B, NW, TX, RAGGED, XL, XT, PF>(R1, s0 + STEP, S, U, ug_magic, q, rowp, xrow, xts);
      compute(R0, s0, btag<false>{});
      load_batch<B, NW, TX, RAGGED, XL, XT, PF>(R0, s0 + 2 * STEP, S, U, ug_magic, q, rowp, xrow, xts);
      compute(R1, s0 + STEP, btag<false>{});
      s0 += 2 * STEP;
    }
    if (nb - b == 2) {
      load_batch<B, NW, TX, RAGGED, XL, XT, PF>(R1, s0 + STEP, S, U, ug_magic, q, rowp, xrow, xts);
      compute(R0, s0, btag<false>{});
      compute(R1, s0 + STEP, btag<true>{});
    } else {
      compute(R0, s0, btag<true>{});
    }
  } else {
    // activations in registers for 4 slots per batch: one register set (two
    // would halve the waves a SIMD holds)
    for (int64_t b = 0; b + 1 < nb; ++b) {
      compute(R0, s0, btag<false>{});
      s0 += STEP;
      load_batch<B, NW, TX, RAGGED, XL, XT, PF>(R0, s0, S, U, ug_magic, q, rowp, xrow, xts);
    }
    compute(R0, s0, btag<true>{});
  }

  if constexpr (!MULTI) {
    out = acc;
    break;
  } else {
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const bool in = lpos[r] >= pstart && lpos[r] < pstart + pcnt;
      float v = acc[r];
      // SC: the output row's staged row (its position in the pass) carries its exponent
      if constexpr (SC) v *= pow2f(__shfl(erow, in ? lpos[r] - pstart : 0, 64));
      out[r] = in ? v : out[r];
    }
    // the next pass's first index batch (from the L2), issued before the exit
    // test so that every path into the next pass has it in flight (after the
    // last pass it re-reads batch 0, unused); then every wave is done with
    // this pass's tables
    load_batch<B, NW, TX, RAGGED, XL, XT, PF>(R0, (int64_t)wave, S, U, ug_magic, q, rowp, xrow, xts);
    if (!has_next) break;
    load_pass(++pass);
    __syncthreads();
  }
  }  // per-set passes

  // ---- sum the NW partial tiles in wave order, then store Y[token][row]
  // lane l holds D[token 4*(l/16)+r][row l%16]
  // (SC + XL: in the staged activations, once every wave is done with them)
  // (XT: each wave's partials in its own buffer, which only it has used)
  if constexpr (SC && XL) __syncthreads();
  float* red = reinterpret_cast<float*>(smem) + (xl_base + (SC && XL ? 0u : xl_bytes)) / 4u;
  constexpr int RS = XT ? (int)(DEC_XT_WAVE / 4) : 256;  // floats between the waves' partial tiles
#pragma unroll
  for (int r = 0; r < 4; ++r) red[wave * RS + (4 * q + r) * 16 + j] = out[r];
  __syncthreads();
  const int t = threadIdx.x;
  if (t < 256) {
    const int token = t >> 4, rr = t & 15;
    // SC (one set): the token's exponent from lane `token` of this wave
    float u = 1.0f;
    if constexpr (SC && !MULTI) u = pow2f(__shfl(erow, token, 64));
    if (token < m && row0 + rr < n) {
      float sum = 0.0f;
#pragma unroll
      for (int wv = 0; wv < NW; ++wv) sum += red[wv * RS + t];
      if constexpr (SC && !MULTI) sum *= u;
      Y[(int64_t)token * n + row0 + rr] = from_f32<TX>(sum);
    }
  }
}

template <int B, int NW>
size_t decode_lds_bytes(int gpr, int64_t x_elems, bool mags, bool xt) {
  // x_elems is rounded up to whole 16-byte chunks so the partials stay
  // aligned; with the magnitude slots the partials overlay the activations;
  // the waves' transposition buffers (xt) hold their partials
  if (xt) return (size_t)gpr * tab_entries<B>::value * 64 * 4 + (size_t)NW * DEC_XT_WAVE;
  const size_t xb = (size_t)((x_elems + 7) / 8) * 16, pb = (size_t)NW * 256 * 4;
  return (size_t)gpr * tab_entries<B>::value * 64 * 4 + (mags ? (xb > pb ? xb : pb) + (size_t)17 * NW * 4 : xb + pb);
}

// Table sets for the MULTI kernel (a single set: lut_set == nullptr)
struct SetArgs {
  const int32_t* lut_set = nullptr;
  bool select = false;             // one token: the single-set kernel on set lut_set[0]
  int n_sets = 1;
  int64_t set_stride = 0;          // table elements per set
  const int32_t* rexp = nullptr;   // row exponents of X (prescaled pair without staging)
};

template <int B, int NW, typename TX, typename TL, bool RAGGED, bool XL, bool XT>
hipError_t decode_launch(const TX* X, const uint8_t* idx, const TL* lut, const Problem& p, TX* Y, hipStream_t s,
                         uint32_t magic, const SetArgs& sa) {
  constexpr bool SC = scaled_pair(__is_same(TX, bf16_t), __is_same(TL, half_t));
  // MULTI + XL stages one pass's tokens: at most min(m, DEC_XL_MAX / d) of them
  const int64_t xl_m = sa.lut_set && !sa.select && p.m > DEC_XL_MAX / p.d ? DEC_XL_MAX / p.d : p.m;
  const size_t lds = decode_lds_bytes<B, NW>(p.gpr, XL ? xl_m * p.d : 0, SC && XL, XT);
  const dim3 grid((unsigned)((p.n + DEC_ROWS - 1) / DEC_ROWS));
  // element e of the staged activations lies in row e / d = umulhi(e, ceil(2^32 / d)), exact for e * d < 2^32
  // (staged elements number at most 49152 and d <= 49152 when staging)
  const uint32_t d_magic = p.d <= DEC_XL_MAX1 ? (uint32_t)(((uint64_t)1 << 32) / (uint64_t)p.d) + 1u : 0u;
  // (the gathers address the tables with absolute LDS addresses, see gaddr:
  // checked once per kernel, which also raises its LDS limit to 160 KB)
  if (sa.lut_set && !sa.select) {
    if constexpr ((SC && !XL) || XT) {
      return hipErrorNotSupported;  // (the ABI routes no such call here)
    } else {
      const auto kern = k_decode<B, NW, TX, TL, RAGGED, XL, false, true>;
      static const hipError_t prep = prepare_kernel((const void*)kern, 160 * 1024);
      if (prep != hipSuccess) return prep;
      hipLaunchKernelGGL(kern, grid, dim3(NW * 64), lds, s, X, idx, lut, (int)p.m, p.n, p.d, p.gpr, magic, d_magic, Y,
                         sa.lut_set, sa.n_sets, sa.set_stride, sa.rexp);
      return hipGetLastError();
    }
  }
  const auto kern = k_decode<B, NW, TX, TL, RAGGED, XL, XT, false>;
  static const hipError_t prep = prepare_kernel((const void*)kern, 160 * 1024);
  if (prep != hipSuccess) return prep;
  hipLaunchKernelGGL(kern, grid, dim3(NW * 64), lds, s, X, idx, lut, (int)p.m, p.n, p.d, p.gpr, magic, d_magic, Y,
                     sa.lut_set, sa.n_sets, sa.set_stride, sa.rexp);
  return hipGetLastError();
}

template <int B, int NW, typename TX, typename TL>
hipError_t decode_nw(const TX* X, const uint8_t* idx, const TL* lut, const Problem& p, TX* Y, hipStream_t s,
                     uint32_t magic, const SetArgs& sa) {
  // one table set: stage the activations when all m rows fit. Several sets:
  // each pass stages its own tokens, so it suffices that one row fits (with a
  // single set in use, the m rows then take several passes)
  const bool multi = sa.lut_set && !sa.select;
  const bool xl = decode_stages_activations(p, multi, sa.n_sets,
                                            scaled_pair(__is_same(TX, bf16_t), __is_same(TL, half_t)));
  // Unstaged, one set: from 8 tokens on, the coalesced loads and the LDS
  // turn-around cost less than loading fragments directly (whose cost grows
  // with the distinct token rows a load touches); below, the direct loads.
  const bool xt = !xl && !multi && p.m >= DEC_XT_MIN_M;
  if (p.units() % 4 != 0)
    return xl ? decode_launch<B, NW, TX, TL, true, true, false>(X, idx, lut, p, Y, s, magic, sa)
              : (xt ? decode_launch<B, NW, TX, TL, true, false, true>(X, idx, lut, p, Y, s, magic, sa)
                    : decode_launch<B, NW, TX, TL, true, false, false>(X, idx, lut, p, Y, s, magic, sa));
  return xl ? decode_launch<B, NW, TX, TL, false, true, false>(X, idx, lut, p, Y, s, magic, sa)
            : (xt ? decode_launch<B, NW, TX, TL, false, false, true>(X, idx, lut, p, Y, s, magic, sa)
                  : decode_launch<B, NW, TX, TL, false, false, false>(X, idx, lut, p, Y, s, magic, sa));
}

template <int B, typename TX, typename TL>
hipError_t decode_b(const TX* X, const uint8_t* idx, const TL* lut, const Problem& p, TX* Y, hipStream_t s,
                    const SetArgs& sa) {
  const uint32_t ug = (uint32_t)(p.group_cols() / 32);
  // u / ug == umulhi(u, magic) for u * ug < 2^32; ug == 1 is passed as 0
  const uint32_t magic = ug == 1 ? 0u : (uint32_t)((((uint64_t)1) << 32) / ug + 1);
  // Few 16-row blocks (one per CU or less): 16 waves per block for more loads
  // in flight. Many blocks: 8 waves so two or more blocks share a CU and one
  // block's start-up latency hides behind another's work.
  const int64_t blocks = (p.n + DEC_ROWS - 1) / DEC_ROWS;
  const int nw = blocks <= 384 ? 16 : 8;
  if (nw == 16) return decode_nw<B, 16>(X, idx, lut, p, Y, s, magic, sa);
  return decode_nw<B, 8>(X, idx, lut, p, Y, s, magic, sa);
}

template <typename TX, typename TL>
hipError_t decode_t(const TX* X, const uint8_t* idx, const TL* lut, const Problem& p, TX* Y, hipStream_t s,
                    const SetArgs& sa) {
  switch (p.b) {
    case 2: return decode_b<2>(X, idx, lut, p, Y, s, sa);
    case 3: return decode_b<3>(X, idx, lut, p, Y, s, sa);
    default: return decode_b<4>(X, idx, lut, p, Y, s, sa);
  }
}

hipError_t decode_dispatch(const void* X, int x_dtype, const uint8_t* idx, const void* lut, int lut_dtype,
                           const Problem& p, void* Y, hipStream_t s, const SetArgs& sa) {
  if (x_dtype == DT_F16 && lut_dtype == DT_F16)
    return decode_t((const half_t*)X, idx, (const half_t*)lut, p, (half_t*)Y, s, sa);
  if (x_dtype == DT_BF16 && lut_dtype == DT_F16)
    return decode_t((const bf16_t*)X, idx, (const half_t*)lut, p, (bf16_t*)Y, s, sa);
  if (x_dtype == DT_F16 && lut_dtype == DT_BF16)
    return decode_t((const half_t*)X, idx, (const bf16_t*)lut, p, (half_t*)Y, s, sa);
  return decode_t((const bf16_t*)X, idx, (const bf16_t*)lut, p, (bf16_t*)Y, s, sa);
}

}  // namespace

int decode_max_m() { return 16; }

bool decode_stages_activations(const Problem& p, bool multi, int n_sets, bool scaled) {
  // the prescaled multi-set decode always stages (it finds the exponents of
  // the staged rows itself). One set: up to 32768 elements, or, below the
  // token count from which the LDS turn-around runs (staging 72-96 KB per
  // block measured slower than that), up to 49152 when the grid has at most
  // one 16-row block per CU (more LDS per block then costs no occupancy) and
  // tables, activations, 16 partial tiles and the magnitude slots fit in
  // 160 KB.
  if (p.m * p.d <= DEC_XL_MAX) return true;
  if (multi) return (n_sets > 1 || scaled) && p.d <= DEC_XL_MAX;
  const int64_t T = p.b == 2 ? 16 : p.k();
  const int64_t lds = p.gpr * T * 256 + p.m * p.d * 2 + 16 * 1024 + 17 * 16 * 4;
  return p.m < DEC_XT_MIN_M && p.m * p.d <= DEC_XL_MAX1 && (p.n + DEC_ROWS - 1) / DEC_ROWS <= 256 &&
         lds <= 160 * 1024;
}

bool decode_multi_supported(const Problem& p, bool scaled) {
  // the prescaled pair stages its activations in the one-pass-per-set kernel
  // (rows of at most 32768 columns); the set-interleaved kernel (m >= 2)
  // finds its row exponents without staging, and takes every set count when
  // the entries per row fit two cells (a set count above 8 needs that)
  const int64_t E = (int64_t)p.gpr << p.b;
  return decode_supported(p) && (!scaled || p.d <= DEC_XL_MAX || (p.m >= 2 && E <= (p.m > 8 ? 128 : 224)));
}

bool decode_supported(const Problem& p) {
  const int T = p.b == 2 ? 16 : p.k();
  // the magic-number division by units-per-group is exact while U * UG < 2^32
  return p.m >= 1 && p.m <= 16 && (int64_t)p.gpr * T <= DEC_MAX_ENTRIES && p.d <= (int64_t(1) << 20);
}

hipError_t launch_decode(const void* X, int x_dtype, const uint8_t* idx, const void* lut, int lut_dtype,
                         const Problem& p, void* Y, const int32_t* rexp, hipStream_t s) {
  SetArgs sa;
  sa.rexp = rexp;
  return decode_dispatch(X, x_dtype, idx, lut, lut_dtype, p, Y, s, sa);
}

hipError_t launch_decode_multi(const void* X, int x_dtype, const uint8_t* idx, const void* luts, int lut_dtype,
                               const int32_t* lut_set, int n_sets, const Problem& p, void* Y, hipStream_t s) {
  // one set: the single-set decode (every token on set 0); one token: the
  // single-set decode on that token's set (found on the device), when it
  // needs no row exponents from a workspace; else set-interleaved tables
  // whenever they apply; otherwise one pass per set in use
  const bool scaled = x_dtype == DT_BF16 && lut_dtype == DT_F16;
  if (n_sets == 1 && !scaled) return decode_dispatch(X, x_dtype, idx, luts, lut_dtype, p, Y, s, SetArgs{});
  if (p.m == 1 && (!scaled || decode_stages_activations(p, false, 1, true))) {
    SetArgs one;
    one.lut_set = lut_set;
    one.select = true;
    one.n_sets = n_sets;
    one.set_stride = p.n * p.gpr * p.k();
    return decode_dispatch(X, x_dtype, idx, luts, lut_dtype, p, Y, s, one);
  }
  if (decode_sets_supported(p, n_sets, scaled))
    return launch_decode_sets(X, x_dtype, idx, luts, lut_dtype, lut_set, n_sets, p, Y, s);
  SetArgs sa;
  sa.lut_set = lut_set;
  sa.n_sets = n_sets;
  sa.set_stride = p.n * p.gpr * p.k();
  return decode_dispatch(X, x_dtype, idx, luts, lut_dtype, p, Y, s, sa);
}

}  // namespace skm
