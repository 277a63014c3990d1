// Shared pieces of the tiled matrix-core kernels (forward GEMM, dX, dLUT):
// LDS access by absolute address, the swizzled 64-byte row layout, MFMA
// wrappers, activation conversion and the per-lane gather address.
#pragma once

#include "skm_common.h"

namespace skm {
namespace mm {

typedef __attribute__((address_space(3))) uint16_t lds_u16;
typedef __attribute__((address_space(3))) uint32_t lds_u32;
typedef __attribute__((address_space(3))) u32x4 lds_u32x4;
typedef __attribute__((address_space(3))) float lds_f32;

// Kernels that use these helpers allocate only dynamic LDS, which therefore
// starts at address 0, and address it with absolute byte offsets.
__device__ __forceinline__ uint32_t ld_h(uint32_t a) { return *(const lds_u16*)(uintptr_t)a; }
__device__ __forceinline__ uint32_t ld_w(uint32_t a) { return *(const lds_u32*)(uintptr_t)a; }
__device__ __forceinline__ u32x4 ld_q(uint32_t a) { return *(const lds_u32x4*)(uintptr_t)a; }
__device__ __forceinline__ void st_h(uint32_t a, uint32_t v) { *(lds_u16*)(uintptr_t)a = (uint16_t)v; }
__device__ __forceinline__ void st_w(uint32_t a, uint32_t v) { *(lds_u32*)(uintptr_t)a = v; }
__device__ __forceinline__ void st_q(uint32_t a, u32x4 v) { *(lds_u32x4*)(uintptr_t)a = v; }
// four floats (read as a float vector: this hipcc turns a bit-cast of an
// element of a loaded integer vector, indexed in an unrolled loop, into a
// splat of element 0)
typedef __attribute__((address_space(3))) f32x4 lds_f32x4;
__device__ __forceinline__ f32x4 ld_f4(uint32_t a) { return *(const lds_f32x4*)(uintptr_t)a; }

// 64-byte rows of four 16-byte chunks; chunk c of row r is stored at
// c ^ f(r) with f(r) = ((r >> 1) ^ (r >> 2)) & 3. gfx950's LDS serves a
// ds_read_b128 / ds_write_b128 in passes of 16 lanes over 64 banks: rows r,
// r+4, r+8, r+12 start on the same bank, and f gives them four different
// chunks, so 16 consecutive rows at one chunk index touch 16 distinct 16-byte
// bank groups (f is also conflict-free for passes of 8 lanes over 32 banks).
__device__ __forceinline__ uint32_t swz(uint32_t row, uint32_t chunk) {
  return row * 64u + ((chunk ^ (((row >> 1) ^ (row >> 2)) & 3u)) << 4);
}
// 128-byte rows of eight 16-byte chunks: chunk c of row r is stored at
// c ^ ((r >> 1) & 7). Even rows start on bank 0 and odd rows on bank 32, and
// the 8 rows of each parity among 16 consecutive rows get 8 different chunks,
// so one 16-lane ds_read_b128 pass over 16 rows at one chunk index touches all
// 64 banks once.
__device__ __forceinline__ uint32_t swz128(uint32_t row, uint32_t chunk) {
  return row * 128u + ((chunk ^ ((row >> 1) & 7u)) << 4);
}
// byte offset of 16-bit element e (0..31) of row r in the 64-byte layout
__device__ __forceinline__ uint32_t swz_elem(uint32_t row, uint32_t e) {
  return swz(row, e >> 3) + ((e & 7u) << 1);
}

// gather address: lane slot in byte 0, entry number from byte-lane p of `ent`
__device__ __forceinline__ uint32_t gaddr(uint32_t ent, uint32_t lane4, int p) {
  return __builtin_amdgcn_perm(ent, lane4, 0x0C0C0400u | ((4u + (uint32_t)p) << 8));
}
__device__ __forceinline__ uint32_t pack2(uint32_t lo, uint32_t hi) {
  return __builtin_amdgcn_perm(hi, lo, 0x05040100u);
}

template <int B> struct tab_entries { static constexpr int value = (B == 2) ? 16 : (1 << B); };

template <typename TC> struct mfma32;
template <> struct mfma32<half_t> {
  static __device__ __forceinline__ f32x16 run(u32x4 a, u32x4 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, a), __builtin_bit_cast(f16x8, b), c, 0, 0,
                                                  0);
  }
};
template <> struct mfma32<bf16_t> {
  static __device__ __forceinline__ f32x16 run(u32x4 a, u32x4 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b), c, 0,
                                                   0, 0);
  }
};

// Convert two 16-bit values packed in a word from storage TS to compute TC.
// (Goes through 16-bit integers: this hipcc miscompiles a bit-cast of a vector
// element to a 2 x f16 vector into a splat of element 0.)
template <typename TS, typename TC>
__device__ __forceinline__ uint32_t cvt_word(uint32_t w) {
  if constexpr (__is_same(TS, TC)) {
    return w;
  } else {
    typedef _Float16 f16x2_t __attribute__((ext_vector_type(2)));
    typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
    float lo, hi;
    if constexpr (__is_same(TS, bf16_t)) {
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
      return __builtin_bit_cast(uint32_t, r);
    } else {
      bf16x2_t r;
      r.x = (bf16_t)lo;
      r.y = (bf16_t)hi;
      return __builtin_bit_cast(uint32_t, r);
    }
  }
}

template <typename TS, typename TC>
__device__ __forceinline__ u32x4 cvt_quad(u32x4 v) {
  if constexpr (__is_same(TS, TC)) {
    return v;
  } else {
    u32x4 o;
#pragma unroll
    for (int q = 0; q < 4; ++q) o[q] = cvt_word<TS, TC>(v[q]);
    return o;
  }
}

// ---- b = 4 table lookup in registers ------------------------------------
// A 16-entry table of 16-bit values held as byte planes: lo[q] / hi[q] hold
// the low / high bytes of entries 4q..4q+3. One v_perm_b32 picks four bytes
// out of eight by 3-bit selectors, so a plane pair (entries 0-7 or 8-15)
// answers four lookups at once and v_bfi_b32 chooses between the two halves
// by bit 3 of each index.
struct Planes16 { uint32_t lo[4], hi[4]; };

// L[i] holds entries 2i (low half) and 2i+1 (high half)
__device__ __forceinline__ void planes16(const uint32_t* L, Planes16& P) {
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    P.lo[q] = __builtin_amdgcn_perm(L[2 * q + 1], L[2 * q], 0x06040200u);
    P.hi[q] = __builtin_amdgcn_perm(L[2 * q + 1], L[2 * q], 0x07050301u);
  }
}

// bytes k of the result: plane byte selected by the low 3 bits of byte k of
// `sel`, from entries 8..15 where byte k of `mask` is 0xFF, else 0..7
__device__ __forceinline__ uint32_t plane_lookup(const uint32_t* pl, uint32_t sel, uint32_t mask) {
  const uint32_t a = __builtin_amdgcn_perm(pl[1], pl[0], sel);
  const uint32_t b = __builtin_amdgcn_perm(pl[3], pl[2], sel);
  return (mask & b) | (~mask & a);
}

// The 8 weights of one index dword w (4-bit fields f0..f7 from the low end)
// as four packed 16-bit pairs in the K order (f0,f2), (f4,f6), (f1,f3),
// (f5,f7) (see cvt_quad_perm for the matching activation order). The masks
// come from v_perm_b32's sign-replicating selectors 8..11 (top bits of bytes
// 1 and 3 of either source), with bit 3 of each field shifted there.
__device__ __forceinline__ u32x4 dequant8_b4(uint32_t w, const Planes16& P) {
  const uint32_t se = w & 0x07070707u;
  const uint32_t so = (w >> 4) & 0x07070707u;
  const uint32_t me = __builtin_amdgcn_perm(w << 4, w << 12, 0x0B090A08u);
  const uint32_t mo = __builtin_amdgcn_perm(w, w << 8, 0x0B090A08u);
  const uint32_t le = plane_lookup(P.lo, se, me), he = plane_lookup(P.hi, se, me);
  const uint32_t lo = plane_lookup(P.lo, so, mo), ho = plane_lookup(P.hi, so, mo);
  return u32x4{__builtin_amdgcn_perm(he, le, 0x05010400u), __builtin_amdgcn_perm(he, le, 0x07030602u),
               __builtin_amdgcn_perm(ho, lo, 0x05010400u), __builtin_amdgcn_perm(ho, lo, 0x07030602u)};
}

// Two values (fp32) rounded to the compute dtype TC and packed
template <typename TC>
__device__ __forceinline__ uint32_t pack_tc(float lo, float hi) {
  typedef _Float16 f16x2_t __attribute__((ext_vector_type(2)));
  typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
  if constexpr (__is_same(TC, half_t)) {
    f16x2_t r;
    r.x = (half_t)lo;
    r.y = (half_t)hi;
    return __builtin_bit_cast(uint32_t, r);
  } else {
    bf16x2_t r;
    r.x = (bf16_t)lo;
    r.y = (bf16_t)hi;
    return __builtin_bit_cast(uint32_t, r);
  }
}

// 8 activations x0..x7 (16-bit storage TS, two per word) in the compute
// dtype TC and the K order (x0,x2), (x4,x6), (x1,x3), (x5,x7)
template <typename TS, typename TC>
__device__ __forceinline__ u32x4 cvt_quad_perm(u32x4 v) {
  if constexpr (__is_same(TS, TC)) {
    return u32x4{__builtin_amdgcn_perm(v[1], v[0], 0x05040100u), __builtin_amdgcn_perm(v[3], v[2], 0x05040100u),
                 __builtin_amdgcn_perm(v[1], v[0], 0x07060302u), __builtin_amdgcn_perm(v[3], v[2], 0x07060302u)};
  } else {
    float f[8];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      if constexpr (__is_same(TS, bf16_t)) {
        f[2 * q] = __builtin_bit_cast(float, v[q] << 16);
        f[2 * q + 1] = __builtin_bit_cast(float, v[q] & 0xFFFF0000u);
      } else {
        f[2 * q] = (float)__builtin_bit_cast(half_t, (uint16_t)(v[q] & 0xFFFFu));
        f[2 * q + 1] = (float)__builtin_bit_cast(half_t, (uint16_t)(v[q] >> 16));
      }
    }
    return u32x4{pack_tc<TC>(f[0], f[2]), pack_tc<TC>(f[4], f[6]), pack_tc<TC>(f[1], f[3]), pack_tc<TC>(f[5], f[7])};
  }
}

// The prescaled conversions of bf16 activations to f16 operands (the row
// prescale of skm_common.h): every value is multiplied by s = 2^-e of its
// row (exact) and then rounded to f16. cvt_quad_scaled keeps the order,
// cvt_quad_perm_scaled produces the K order of cvt_quad_perm.
__device__ __forceinline__ u32x4 cvt_quad_scaled(u32x4 v, float s) {
  u32x4 o;
#pragma unroll
  for (int q = 0; q < 4; ++q)
    o[q] = pack_tc<half_t>(__builtin_bit_cast(float, v[q] << 16) * s, __builtin_bit_cast(float, v[q] & 0xFFFF0000u) * s);
  return o;
}
// the same with the exponent fields raised by an exp_add_word (block mode 1)
__device__ __forceinline__ u32x4 add_quad(u32x4 v, uint32_t k) {
  return u32x4{v[0] + k, v[1] + k, v[2] + k, v[3] + k};
}

// compile-time tag of a block's prescale mode (0 none, 1 exponent add, 2 multiply)
template <int V> struct mode_tag { static constexpr int value = V; };

// Block-uniform prescale mode (skm_common.h scale_mode_of) from each thread's
// flags: the waves OR their ballots into an LDS word at `word` (an address no
// thread touches before the block's first K-step), two barriers.
__device__ __forceinline__ int block_scale_mode(uint32_t flags, uint32_t word) {
  if (threadIdx.x == 0) st_w(word, 0u);
  __syncthreads();
  const uint64_t b1 = __ballot(flags & 1u), b2 = __ballot(flags & 2u);
  if ((threadIdx.x & 63) == 0 && (b1 | b2))
    __hip_atomic_fetch_or((lds_u32*)(uintptr_t)word, (b1 ? 1u : 0u) | (b2 ? 2u : 0u), __ATOMIC_RELAXED,
                          __HIP_MEMORY_SCOPE_WORKGROUP);
  __syncthreads();
  return scale_mode_of(ld_w(word));
}

__device__ __forceinline__ u32x4 cvt_quad_perm_scaled(u32x4 v, float s) {
  float f[8];
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    f[2 * q] = __builtin_bit_cast(float, v[q] << 16) * s;
    f[2 * q + 1] = __builtin_bit_cast(float, v[q] & 0xFFFF0000u) * s;
  }
  return u32x4{pack_tc<half_t>(f[0], f[2]), pack_tc<half_t>(f[4], f[6]), pack_tc<half_t>(f[1], f[3]),
               pack_tc<half_t>(f[5], f[7])};
}

// Transposed LDS read (gfx950 ds_read_b64_tr_b16). Within each group of 16
// lanes, lane l receives 16-bit element l % 4 of the 8-byte pieces addressed
// by lanes 4j + l/4 of its group, j = 0..3. If lane s of a group points at row
// k0 + s/4, columns c0 + 4 (s % 4) .. +3 of a row-major tile T[k][c], then
// lane l receives T[k0 + j][c0 + l] for j = 0..3: four consecutive k of one
// column, i.e. an MFMA operand quarter from a K-major tile.
typedef short short4_t __attribute__((ext_vector_type(4)));
__device__ __forceinline__ u32x2 ld_tr(uint32_t a) {
  const short4_t v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) short4_t*)(uintptr_t)a);
  return __builtin_bit_cast(u32x2, v);
}

// One 32x32x16 MFMA operand (8 consecutive k of one column per lane) from a
// row-major K-major tile: `tile` is the LDS byte address of T[k0][c0] for the
// fragment's first k row and first column, `rs` the tile's row stride.
// Lane l covers column c0 + l % 32 and k rows k0 + 8 (l / 32) .. +7.
__device__ __forceinline__ u32x4 ld_frag_tr(uint32_t tile, uint32_t rs, uint32_t lane) {
  const uint32_t s = lane & 15u;
  const uint32_t row = 8u * (lane >> 5) + (s >> 2);
  const uint32_t col = 16u * ((lane >> 4) & 1u) + 4u * (s & 3u);
  const uint32_t a = tile + row * rs + col * 2u;
  const u32x2 lo = ld_tr(a), hi = ld_tr(a + 4u * rs);
  return u32x4{lo.x, lo.y, hi.x, hi.y};
}

__device__ __forceinline__ void zero16(f32x16& a) {
#pragma unroll
  for (int e = 0; e < 16; ++e) a[e] = 0.0f;
}

// Workgroups are dispatched round-robin over the 8 XCDs, each with its own L2.
// Renumber them so that each XCD receives a contiguous range of logical block
// ids (a bijection on [0, nblocks)): blocks that share operands are then
// co-resident in one L2 instead of being spread over all eight.
__device__ __forceinline__ uint32_t xcd_block(uint32_t b, uint32_t nblocks) {
  constexpr uint32_t NX = 8;
  const uint32_t q = nblocks / NX, r = nblocks % NX;
  const uint32_t x = b % NX, s = b / NX;
  return x * q + (x < r ? x : r) + s;
}

// group index of unit u: multiply-high by the host's magic (0 = one unit/group)
__device__ __forceinline__ uint32_t group_of(uint32_t u, uint32_t magic) { return magic ? __umulhi(u, magic) : u; }

}  // namespace mm
}  // namespace skm
