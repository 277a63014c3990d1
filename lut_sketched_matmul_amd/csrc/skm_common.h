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

}  // namespace skm
