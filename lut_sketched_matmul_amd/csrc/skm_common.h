// Device-side building blocks shared by the sketched-matmul kernels (gfx950).
//
// Index layout (the library's reading of the b-bit sketch indices; the pages
// fix only b): row i of idx_packed is one little-endian bitstream, index j at
// bits b*j .. b*j+b-1. The kernels work in 32-column "units": a unit is
// 4*b bytes (b=2: 8 B, b=3: 12 B, b=4: 16 B), always starts on a byte that is
// a multiple of 4*b, and never straddles a group because the group width is a
// multiple of 32 columns.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace skm {

typedef _Float16 half_t;
typedef __bf16 bf16_t;

typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x3 __attribute__((ext_vector_type(3)));

// dtype tags matching skm_dtype in sketch_matmul.h
enum : int { DT_F32 = 0, DT_F16 = 1, DT_BF16 = 2 };

template <int DT> struct dtype_of;
template <> struct dtype_of<DT_F32> { typedef float type; };
template <> struct dtype_of<DT_F16> { typedef half_t type; };
template <> struct dtype_of<DT_BF16> { typedef bf16_t type; };

// ---- 16-bit float bit helpers -------------------------------------------------
// Conversions go through float: f16 <-> f32 and bf16 -> f32 are exact, and
// f32 -> f16 / f32 -> bf16 round to nearest even (hardware cvt instructions).

__device__ __forceinline__ float to_f32(float v) { return v; }
__device__ __forceinline__ float to_f32(half_t v) { return (float)v; }
__device__ __forceinline__ float to_f32(bf16_t v) { return (float)v; }

template <typename T> __device__ __forceinline__ T from_f32(float v);
template <> __device__ __forceinline__ float from_f32<float>(float v) { return v; }
template <> __device__ __forceinline__ half_t from_f32<half_t>(float v) { return (half_t)v; }
template <> __device__ __forceinline__ bf16_t from_f32<bf16_t>(float v) { return (bf16_t)v; }

// 16-bit pattern of a value already in the compute dtype
__device__ __forceinline__ uint16_t bits16(half_t v) { return __builtin_bit_cast(uint16_t, v); }
__device__ __forceinline__ uint16_t bits16(bf16_t v) { return __builtin_bit_cast(uint16_t, v); }

// Convert a 16-bit storage value (given by its bits) to compute dtype TC bits.
template <typename TS, typename TC>
__device__ __forceinline__ uint16_t convert16(uint16_t s) {
  if constexpr (__is_same(TS, TC)) {
    return s;
  } else {
    TS v = __builtin_bit_cast(TS, s);
    return bits16(from_f32<TC>(to_f32(v)));
  }
}

// ---- index extraction --------------------------------------------------------

// Number of 32-bit words in one 32-column unit.
template <int B> struct unit_words { static constexpr int value = B; };

// Field f (0..31) of a unit held in registers w[0..B-1] (little-endian stream).
template <int B>
__device__ __forceinline__ uint32_t unit_field(const uint32_t* w, int f) {
  const int bit = B * f;
  const int word = bit >> 5;
  const int off = bit & 31;
  if (off + B <= 32) {
    return (w[word] >> off) & ((1u << B) - 1u);
  } else {
    // straddles two words (only for B == 3): funnel shift of (w[word+1]:w[word])
    return __builtin_amdgcn_alignbit(w[word + 1], w[word], off) & ((1u << B) - 1u);
  }
}

// Load one unit of row `row_ptr` (unit index u) into w[0..B-1].
template <int B>
__device__ __forceinline__ void load_unit(const uint8_t* __restrict__ row_ptr, int64_t u, uint32_t* w) {
  const uint8_t* p = row_ptr + u * (4 * B);
  if constexpr (B == 4) {
    u32x4 v = *reinterpret_cast<const u32x4*>(p);
    w[0] = v.x; w[1] = v.y; w[2] = v.z; w[3] = v.w;
  } else if constexpr (B == 2) {
    u32x2 v = *reinterpret_cast<const u32x2*>(p);
    w[0] = v.x; w[1] = v.y;
  } else {
    const uint32_t* q = reinterpret_cast<const uint32_t*>(p);
    w[0] = q[0]; w[1] = q[1]; w[2] = q[2];
  }
}

__device__ __forceinline__ int lane_id() { return (int)(threadIdx.x & 63); }

// ---- per-row power-of-two prescale (bf16 activations on f16 matrix cores) ----
// The matrix cores take both operands in one dtype. With bf16 activations and
// f16 tables the activations are converted to f16, whose range is far
// narrower than bf16's (largest 65504, normal values from 2^-14). A bf16 value
// has 8 significant bits, so once inside f16's normal range it converts
// exactly. Each token row therefore gets an exponent e, taken from its largest
// magnitude M (biased exponent field E): the row is multiplied by 2^-e before
// the conversion and each fp32 result of that row by 2^e after the
// contraction (exact: powers of two).
//   * 2^-2 <= M < 2^16 (E in [125, 142]): e = 0. Every bf16 value below 2^16
//     is a finite f16; values from 2^-14 up convert exactly, smaller ones
//     round to f16 subnormals with an absolute error below 2^-23 M.
//   * otherwise e = clamp(E - 141, -126, 113), which puts M into [2^14, 2^15):
//     values down to 2^-31 M convert exactly, smaller ones round to f16
//     subnormals with an error below 2^-38 M.
// Both scale factors are normal fp32 numbers for every e in that range.
constexpr bool scaled_pair(bool x_is_bf16, bool lut_is_f16) { return x_is_bf16 && lut_is_f16; }

__device__ __forceinline__ int row_exp_of(uint32_t absmax_bits) {
  const int E = (int)(absmax_bits >> 7);
  if (E >= 125 && E <= 142) return 0;
  const int e = E - 141;
  return e < -126 ? -126 : (e > 113 ? 113 : e);
}

// Rows of exponent -101 <= e <= 0 (and no others in a block) may be scaled by
// raising the exponent field of every bf16 value by k = -e: exact for normal
// values (their exponent stays <= 142), and a zero or subnormal becomes a
// value below 2^-25, which rounds to f16 zero as its true scaled value does
// (or would round to at most 2^-24). scale_mode_of gives the conversion a
// block uses: 0 none (all e == 0), 1 exponent add (all -101 <= e <= 0),
// 2 multiply by 2^-e.
__device__ __forceinline__ uint32_t scale_flags_of(int e) {
  return (e != 0 ? 1u : 0u) | ((e > 0 || e < -101) ? 2u : 0u);
}
__device__ __forceinline__ int scale_mode_of(uint32_t flags) { return (flags & 2u) ? 2 : (int)(flags & 1u); }
// the word added to a pair of bf16 values (two 16-bit halves) to raise both
// exponent fields by k (no carry leaves either half: the fields stay <= 142)
__device__ __forceinline__ uint32_t exp_add_word(int e) { return ((uint32_t)(-e) << 7) * 0x00010001u; }

// 2^e as fp32 for -126 <= e <= 127
__device__ __forceinline__ float pow2f(int e) { return __builtin_bit_cast(float, (uint32_t)(127 + e) << 23); }

// largest magnitude pattern (|bf16| bits, 15 bits; NaN above infinity) of the
// two bf16 values in a word, and of eight in four words
__device__ __forceinline__ uint32_t absmax2_bf16(uint32_t w) {
  const uint32_t lo = w & 0x7FFFu, hi = (w >> 16) & 0x7FFFu;
  return lo > hi ? lo : hi;
}
// op(v) over the wave, in lane 63, with DPP row shifts and row broadcasts
// (vector ALU only; lanes shifted in from outside a row read 0, the identity
// of an unsigned maximum and of a bitwise or).
template <typename Op>
__device__ __forceinline__ uint32_t wave_reduce_to_lane63(uint32_t v, Op op) {
  v = op(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x111, 0xF, 0xF, true));  // row_shr:1
  v = op(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x112, 0xF, 0xF, true));  // row_shr:2
  v = op(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x114, 0xF, 0xF, true));  // row_shr:4
  v = op(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x118, 0xF, 0xF, true));  // row_shr:8
  v = op(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x142, 0xA, 0xF, true));  // row_bcast:15
  v = op(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x143, 0xC, 0xF, true));  // row_bcast:31
  return v;
}
__device__ __forceinline__ uint32_t wave_max_to_lane63(uint32_t v) {
  return wave_reduce_to_lane63(v, [](uint32_t a, uint32_t b) { return a > b ? a : b; });
}
__device__ __forceinline__ uint32_t wave_or_to_lane63(uint32_t v) {
  return wave_reduce_to_lane63(v, [](uint32_t a, uint32_t b) { return a | b; });
}

// magnitude patterns (|bf16| bits) of 2^-2 and 2^16: rows whose largest
// magnitude lies in [2^-2, 2^16) take no prescale (row_exp_of gives 0)
constexpr uint32_t kNoScaleLo = 125u << 7, kNoScaleHi = 143u << 7;

__device__ __forceinline__ uint32_t absmax8_bf16(u32x4 v) {
  uint32_t a = absmax2_bf16(v[0]), b = absmax2_bf16(v[1]), c = absmax2_bf16(v[2]), d = absmax2_bf16(v[3]);
  a = a > b ? a : b;
  c = c > d ? c : d;
  return a > c ? a : c;
}

}  // namespace skm
