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
#include "skm_common.h"
#include "skm_launch.h"

namespace skm {

namespace {

constexpr int DEC_ROWS = 16;
constexpr int DEC_NW = 8;     // waves per block
constexpr int DEC_PF = 4;     // slots loaded per batch and wave
constexpr int DEC_MAX_ENTRIES = 224;  // table entries per row kept in LDS (entry byte must fit in 8 bits)

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

// table entries per group for bit width B (b = 2 stores pairs)
template <int B> struct tab_entries { static constexpr int value = (B == 2) ? 16 : (1 << B); };

// 8 activations (16-bit storage TX) -> packed compute dtype TC, two at a time
// through fp32 (exact widening, then one packed round-to-nearest-even convert)
typedef _Float16 f16x2_t __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

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

// Write this lane's private table copies. Row j = lane%16 of the block; every
// wave writes whole 64-lane entry rows, so each ds_write is conflict-free.
template <int B, typename TL>
__device__ __forceinline__ void fill_tables(uint32_t* tabs, const TL* __restrict__ lut, int64_t grow, bool row_ok,
                                            int gpr, int lane, int wave) {
  constexpr int K = 1 << B;
  const uint16_t* src = reinterpret_cast<const uint16_t*>(lut) + (row_ok ? grow : 0) * (int64_t)gpr * K;
  if constexpr (B == 2) {
    // one group per step: 4 entries -> 16 pairs (a + 4c) = (LUT[a], LUT[c])
    for (int g = wave; g < gpr; g += DEC_NW) {
      u32x2 v = row_ok ? *reinterpret_cast<const u32x2*>(src + g * 4) : u32x2{0u, 0u};
      const uint32_t e[4] = {v.x & 0xFFFFu, v.x >> 16, v.y & 0xFFFFu, v.y >> 16};
#pragma unroll
      for (int c = 0; c < 4; ++c)
#pragma unroll
        for (int a = 0; a < 4; ++a) tabs[(g * 16 + a + 4 * c) * 64 + lane] = e[a] | (e[c] << 16);
    }
  } else {
    // chunks of 8 entries (one 16-byte load; gpr*K is a multiple of 8)
    const int E = gpr * K;
    for (int c = wave; c * 8 < E; c += DEC_NW) {
      u32x4 v = row_ok ? *reinterpret_cast<const u32x4*>(src + c * 8) : u32x4{0u, 0u, 0u, 0u};
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        tabs[(c * 8 + 2 * t) * 64 + lane] = v[t] & 0xFFFFu;
        tabs[(c * 8 + 2 * t + 1) * 64 + lane] = v[t] >> 16;
      }
    }
  }
}

template <int B, typename TX>
struct SlotRegs {
  uint32_t w[DEC_PF][B];
  u32x4 x[DEC_PF][4];
  uint32_t gk[DEC_PF];
  bool ok[DEC_PF];
};

// Issue the index and activation loads of DEC_PF slots. Addresses are clamped
// in range instead of masked: a token row >= m or a weight row >= n only
// feeds outputs that are never stored, and a unit past the row end (RAGGED
// only) is zeroed by the caller. g = u / UG is a multiply-high by the host's
// magic constant (exact for u * UG < 2^32).
template <int B, typename TX, bool RAGGED>
__device__ __forceinline__ void load_batch(SlotRegs<B, TX>& R, int64_t s0, int64_t S, uint32_t U, uint32_t ug_magic,
                                           int q, const uint8_t* rowp, const TX* xrow) {
  constexpr int T = tab_entries<B>::value;
#pragma unroll
  for (int p = 0; p < DEC_PF; ++p) {
    const int64_t s = s0 + (int64_t)p * DEC_NW;
    if (s < S) {  // wave-uniform
      uint32_t u = 4u * (uint32_t)s + (uint32_t)q;
      if constexpr (RAGGED) {
        R.ok[p] = u < U;
        u = u < U ? u : U - 1u;
      }
      load_unit<B>(rowp, u, R.w[p]);
      const u32x4* xp = reinterpret_cast<const u32x4*>(xrow + (int64_t)u * 32);
#pragma unroll
      for (int h = 0; h < 4; ++h) R.x[p][h] = xp[h];
      R.gk[p] = (ug_magic ? __umulhi(u, ug_magic) : u) * T;  // magic 0: one unit per group
    }
  }
}

template <int B, typename TX, typename TL, bool RAGGED>
__global__ void __launch_bounds__(DEC_NW * 64)
k_decode(const TX* __restrict__ X, const uint8_t* __restrict__ idx_packed, const TL* __restrict__ lut,
         int m, int64_t n, int64_t d, int gpr, uint32_t ug_magic, TX* __restrict__ Y) {
  // Dynamic LDS only (this kernel has no static LDS, so it starts at address
  // 0): [entries][64 lanes] table dwords, then the [NW][16][16] fp32 partials.
  extern __shared__ uint32_t smem[];
  constexpr int T = tab_entries<B>::value;
  typedef mfma16<TL> MF;

  const int lane = lane_id();
  const int wave = threadIdx.x >> 6;
  const int64_t row0 = (int64_t)blockIdx.x * DEC_ROWS;
  const int j = lane & 15;           // weight row within the block (B operand column)
  const int q = lane >> 4;           // contraction quarter
  const int64_t grow = row0 + j;
  const bool row_ok = grow < n;
  const int tok = lane & 15;         // A operand row = token
  const bool tok_ok = tok < m;
  (void)tok_ok;

  const uint32_t U = (uint32_t)(d / 32);         // units per row
  const int64_t S = (U + 3) / 4;                 // slots per row
  const uint8_t* rowp = idx_packed + (row_ok ? grow : n - 1) * (d * B / 8);
  const TX* xrow = X + (int64_t)(tok_ok ? tok : m - 1) * d;
  const uint32_t lane4 = (uint32_t)lane * 4u;

  SlotRegs<B, TX> R;
  int64_t s0 = wave;
  // first index loads go out before the tables are staged
  load_batch<B, TX, RAGGED>(R, s0, S, U, ug_magic, q, rowp, xrow);
  fill_tables<B, TL>(smem, lut, grow, row_ok, gpr, lane, wave);
  __syncthreads();
  // the gathers address the tables with absolute LDS addresses (see gaddr)
  if ((uint32_t)(uintptr_t)smem != 0u) return;

  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  while (true) {
#pragma unroll
    for (int p = 0; p < DEC_PF; ++p) {
      if (s0 + (int64_t)p * DEC_NW >= S) break;  // wave-uniform
      const uint32_t gk = R.gk[p];
      const uint32_t gk4 = gk * 0x01010101u;
#pragma unroll
      for (int h = 0; h < 4; ++h) {
        u32x4 wb = dequant_step<B>(R.w[p], h, gk4, gk, lane4);
        // a slot past the row end (only when d/32 is not a multiple of 4) has
        // X = 0; its weights are zeroed too so no table value can leak in
        if constexpr (RAGGED) {
          if (!R.ok[p]) wb = u32x4{0u, 0u, 0u, 0u};
        }
        u32x4 xv = x_to_tc<TX, TL>(R.x[p][h]);
        if constexpr (RAGGED) {
          if (!R.ok[p]) xv = u32x4{0u, 0u, 0u, 0u};
        }
        acc = MF::run(__builtin_bit_cast(typename MF::vec, xv), __builtin_bit_cast(typename MF::vec, wb), acc);
      }
    }
    s0 += (int64_t)DEC_NW * DEC_PF;
    if (s0 >= S) break;
    load_batch<B, TX, RAGGED>(R, s0, S, U, ug_magic, q, rowp, xrow);
  }

  // ---- sum the NW partial tiles in wave order, then store Y[token][row]
  // lane l holds D[token 4*(l/16)+r][row l%16]
  float* red = reinterpret_cast<float*>(smem + gpr * T * 64);
#pragma unroll
  for (int r = 0; r < 4; ++r) red[wave * 256 + (4 * q + r) * 16 + j] = acc[r];
  __syncthreads();
  const int t = threadIdx.x;
  if (t < 256) {
    const int token = t >> 4, rr = t & 15;
    if (token < m && row0 + rr < n) {
      float sum = 0.0f;
#pragma unroll
      for (int wv = 0; wv < DEC_NW; ++wv) sum += red[wv * 256 + t];
      Y[(int64_t)token * n + row0 + rr] = from_f32<TX>(sum);
    }
  }
}

template <int B>
size_t decode_lds_bytes(int gpr) {
  return (size_t)gpr * tab_entries<B>::value * 64 * 4 + (size_t)DEC_NW * 256 * 4;
}

template <int B, typename TX, typename TL>
hipError_t decode_b(const TX* X, const uint8_t* idx, const TL* lut, const Problem& p, TX* Y, hipStream_t s) {
  const dim3 grid((unsigned)((p.n + DEC_ROWS - 1) / DEC_ROWS));
  const dim3 block(DEC_NW * 64);
  const size_t lds = decode_lds_bytes<B>(p.gpr);
  const int m = (int)p.m;
  const uint32_t ug = (uint32_t)(p.group_cols() / 32);
  // u / ug == umulhi(u, magic) for u * ug < 2^32; ug == 1 is passed as 0
  const uint32_t magic = ug == 1 ? 0u : (uint32_t)((((uint64_t)1) << 32) / ug + 1);
  if (p.units() % 4 != 0)
    hipLaunchKernelGGL((k_decode<B, TX, TL, true>), grid, block, lds, s, X, idx, lut, m, p.n, p.d, p.gpr, magic, Y);
  else
    hipLaunchKernelGGL((k_decode<B, TX, TL, false>), grid, block, lds, s, X, idx, lut, m, p.n, p.d, p.gpr, magic, Y);
  return hipGetLastError();
}

template <typename TX, typename TL>
hipError_t decode_t(const TX* X, const uint8_t* idx, const TL* lut, const Problem& p, TX* Y, hipStream_t s) {
  switch (p.b) {
    case 2: return decode_b<2>(X, idx, lut, p, Y, s);
    case 3: return decode_b<3>(X, idx, lut, p, Y, s);
    default: return decode_b<4>(X, idx, lut, p, Y, s);
  }
}

}  // namespace

int decode_max_m() { return 16; }

bool decode_supported(const Problem& p) {
  const int T = p.b == 2 ? 16 : p.k();
  // the magic-number division by units-per-group is exact while U * UG < 2^32
  return p.m >= 1 && p.m <= 16 && (int64_t)p.gpr * T <= DEC_MAX_ENTRIES && p.d <= (int64_t(1) << 20);
}

hipError_t launch_decode(const void* X, int x_dtype, const uint8_t* idx, const void* lut, int lut_dtype,
                         const Problem& p, void* Y, hipStream_t s) {
  if (x_dtype == DT_F16 && lut_dtype == DT_F16)
    return decode_t((const half_t*)X, idx, (const half_t*)lut, p, (half_t*)Y, s);
  if (x_dtype == DT_BF16 && lut_dtype == DT_F16)
    return decode_t((const bf16_t*)X, idx, (const half_t*)lut, p, (bf16_t*)Y, s);
  if (x_dtype == DT_F16 && lut_dtype == DT_BF16)
    return decode_t((const half_t*)X, idx, (const bf16_t*)lut, p, (half_t*)Y, s);
  return decode_t((const bf16_t*)X, idx, (const bf16_t*)lut, p, (bf16_t*)Y, s);
}

}  // namespace skm
