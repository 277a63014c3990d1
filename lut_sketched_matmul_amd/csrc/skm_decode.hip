// Decode-sized forward pass Y = X W^T for m <= 16 tokens (gfx950).
//
// "SpaLLM" (abstract, section 2.3; Table 5) runs inference as one compressed
// matmul per layer: table lookup plus accumulate, with every weight index
// streamed once per token. At m <= 16 that stream is the whole cost (the
// operation is HBM-bound), so the kernel is built around reading idx_packed
// exactly once with wide loads while doing as little work per weight as
// possible.
//
// Mapping onto the matrix cores. One v_mfma_f32_16x16x32 (f16 or bf16) takes
// A = X fragment (16 tokens x 32 columns) and B = W^T fragment (32 columns x
// 16 weight rows). Lane l holds A[token l%16][8 columns] and B[8 columns][row
// l%16] for quarter q = l/16 of the 32 contraction slots. The contraction
// order is free, so quarter q's 8 slots are simply 8 columns of the 32-column
// unit that lane loads: lane (row j, quarter q) of a wave loads unit 4s+q of
// row j with one 16/8/12-byte load (b = 4/2/3) and dequantises it into four B
// fragments; the A fragments are X at the same columns. Padding tokens
// (m < 16) cost matrix-core time only, which is idle in this kernel anyway;
// the vector ALUs and LDS do the dequantisation.
//
// Tables. Every lane gathers from its own private copy of its row's tables in
// LDS, laid out entry-major / lane-minor (dword (g*K + e)*64 + lane), so the
// 64 lanes of any gather hit 64 distinct banks whatever the indices are. The
// copies for the block's 16 rows and all gpr groups are written once at the
// start (they are identical for every wave of the block).
//
// Work split. Block = 16 weight rows x all d columns, NW waves. Wave w handles
// slots s = w, w + NW, ... (slot = 4 units = 128 columns), so the waves of a
// block read adjacent 64-byte pieces of each row. The NW partial 16x16 tiles
// are summed in LDS in wave order (deterministic) and stored once.
#include "skm_common.h"
#include "skm_launch.h"

namespace skm {

namespace {

constexpr int DEC_ROWS = 16;
constexpr int DEC_NW = 8;      // waves per block
constexpr int DEC_PF = 4;      // slots loaded ahead per wave
constexpr int DEC_MAX_TABLE_ENTRIES = 224;  // gpr * 2^b per row kept in LDS (<= 64 KB total)

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

// 8 activations (16-bit storage TX) -> packed compute dtype TC
template <typename TX, typename TC>
__device__ __forceinline__ u32x4 x_to_tc(u32x4 v) {
  if constexpr (__is_same(TX, TC)) {
    return v;
  } else {
    u32x4 o;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const uint32_t lo = convert16<TX, TC>((uint16_t)(v[q] & 0xffffu));
      const uint32_t hi = convert16<TX, TC>((uint16_t)(v[q] >> 16));
      o[q] = lo | (hi << 16);
    }
    return o;
  }
}

template <int B, typename TX, typename TL>
__global__ void __launch_bounds__(DEC_NW * 64)
k_decode(const TX* __restrict__ X, const uint8_t* __restrict__ idx_packed, const TL* __restrict__ lut,
         int m, int64_t n, int64_t d, int gpr, TX* __restrict__ Y) {
  constexpr int K = 1 << B;
  typedef mfma16<TL> MF;
  extern __shared__ uint32_t smem[];
  const int E = gpr * K;             // table entries per row
  uint32_t* tabs = smem;             // [E][64] dwords (low 16 bits used)
  float* red = reinterpret_cast<float*>(smem + E * 64);  // [NW][16 tokens][16 rows]

  const int lane = lane_id();
  const int wave = threadIdx.x >> 6;
  const int64_t row0 = (int64_t)blockIdx.x * DEC_ROWS;
  const int j = lane & 15;           // weight row within the block (B operand column)
  const int q = lane >> 4;           // contraction quarter
  const int64_t grow = row0 + j;
  const bool row_ok = grow < n;

  // ---- private table copies: entry ge of lane l's row goes to dword ge*64 + l
  {
    const uint16_t* src = reinterpret_cast<const uint16_t*>(lut) + (row_ok ? grow : 0) * E;
    for (int ge = wave; ge < E; ge += DEC_NW) tabs[ge * 64 + lane] = row_ok ? (uint32_t)src[ge] : 0u;
  }
  __syncthreads();

  const int64_t U = d / 32;                      // units per row
  const int64_t UG = (d / gpr) / 32;             // units per group
  const int64_t S = (U + 3) / 4;                 // slots per row
  const int64_t rb = d * B / 8;
  const uint8_t* rowp = idx_packed + (row_ok ? grow : 0) * rb;
  const int tok = lane & 15;                     // A operand row = token
  const bool tok_ok = tok < m;
  const TX* xrow = X + (int64_t)(tok_ok ? tok : 0) * d;
  const uint16_t* tab16 = reinterpret_cast<const uint16_t*>(tabs);

  f32x4 acc = {0.f, 0.f, 0.f, 0.f};

  for (int64_t s0 = wave; s0 < S; s0 += (int64_t)DEC_NW * DEC_PF) {
    uint32_t w[DEC_PF][B];
    u32x4 xa[DEC_PF][4];
    int tb[DEC_PF];
    bool uok[DEC_PF];
    // issue every load of DEC_PF slots before using any of them
#pragma unroll
    for (int p = 0; p < DEC_PF; ++p) {
      const int64_t s = s0 + (int64_t)p * DEC_NW;
      const int64_t u = 4 * s + q;
      uok[p] = (s < S) && (u < U);
      if (uok[p] && row_ok) {
        load_unit<B>(rowp, u, w[p]);
      } else {
#pragma unroll
        for (int t = 0; t < B; ++t) w[p][t] = 0u;
      }
      if (uok[p] && tok_ok) {
        const u32x4* xp = reinterpret_cast<const u32x4*>(xrow + u * 32);
#pragma unroll
        for (int h = 0; h < 4; ++h) xa[p][h] = xp[h];
      } else {
#pragma unroll
        for (int h = 0; h < 4; ++h) xa[p][h] = u32x4{0u, 0u, 0u, 0u};
      }
      const int64_t g = uok[p] ? (u / UG) : 0;
      tb[p] = (int)(g * K) * 64 + lane;
    }
#pragma unroll
    for (int p = 0; p < DEC_PF; ++p) {
      if (s0 + (int64_t)p * DEC_NW >= S) break;
#pragma unroll
      for (int h = 0; h < 4; ++h) {
        u32x4 wb;
#pragma unroll
        for (int t = 0; t < 4; ++t) {
          const uint32_t e0 = unit_field<B>(w[p], 8 * h + 2 * t);
          const uint32_t e1 = unit_field<B>(w[p], 8 * h + 2 * t + 1);
          const uint32_t v0 = tab16[2 * (tb[p] + (int)e0 * 64)];
          const uint32_t v1 = tab16[2 * (tb[p] + (int)e1 * 64)];
          wb[t] = v0 | (v1 << 16);
        }
        if (!uok[p]) wb = u32x4{0u, 0u, 0u, 0u};
        const u32x4 xv = x_to_tc<TX, TL>(xa[p][h]);
        acc = MF::run(__builtin_bit_cast(typename MF::vec, xv), __builtin_bit_cast(typename MF::vec, wb), acc);
      }
    }
  }

  // ---- sum the NW partial tiles in wave order, then store Y[token][row]
  // lane l holds D[token 4*(l/16)+r][row l%16]
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

template <typename TX, typename TL>
hipError_t decode_t(const TX* X, const uint8_t* idx, const TL* lut, const Problem& p, TX* Y, hipStream_t s) {
  const dim3 grid((unsigned)((p.n + DEC_ROWS - 1) / DEC_ROWS));
  const dim3 block(DEC_NW * 64);
  const size_t lds = (size_t)p.gpr * p.k() * 64 * 4 + (size_t)DEC_NW * 256 * 4;
  const int m = (int)p.m;
  switch (p.b) {
    case 2: hipLaunchKernelGGL((k_decode<2, TX, TL>), grid, block, lds, s, X, idx, lut, m, p.n, p.d, p.gpr, Y); break;
    case 3: hipLaunchKernelGGL((k_decode<3, TX, TL>), grid, block, lds, s, X, idx, lut, m, p.n, p.d, p.gpr, Y); break;
    default: hipLaunchKernelGGL((k_decode<4, TX, TL>), grid, block, lds, s, X, idx, lut, m, p.n, p.d, p.gpr, Y); break;
  }
  return hipGetLastError();
}

}  // namespace

int decode_max_m() { return 16; }

bool decode_supported(const Problem& p) {
  return p.m >= 1 && p.m <= 16 && (int64_t)p.gpr * p.k() <= DEC_MAX_TABLE_ENTRIES;
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
