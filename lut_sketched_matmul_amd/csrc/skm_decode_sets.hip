// Decode-sized forward pass with one table set per token over one shared
// index stream (gfx950): Y[t][i] = sum_j X[t][j] * LUT_{s(t)}[i][j/G][idx[i][j]]
// for m <= 16 tokens.
//
// "SpaLLM" (section 2.3, multiple adapters): fine-tuned adapters of one base
// model share the frozen mapping and differ only in their tables, so a batch
// of decode tokens from different adapters reads one index stream. What grows
// with the number of sets in a batch is the table lookups: every weight has
// to be looked up once per set in use.
//
// Set-interleaved tables. A block (16 weight rows x all columns) stages the
// tables of the sets its tokens use (at most 16) in LDS, interleaved per
// (entry, row): the 16-byte cell of (entry e, row j) holds entry e of row j
// for 8 set slots, as 16-bit values. One 128-bit LDS read (64-bit for at most
// four sets, 32-bit for two) then looks up one weight for up to 8 sets at
// once, and its address is formed exactly as in the single-set decode: the
// entry number in byte 1, the lane's row constant (16 j) in byte 0, built with
// one v_perm_b32 from a byte-aligned index field. With more than 8 sets a
// second cell per (entry, row) sits 256 bytes above the first (entries then
// 512 bytes apart: the index field is doubled before the perm), read with an
// immediate offset.
//
// Contraction over (column, set parity). One v_mfma_f32_16x16x32 takes K = 32
// contraction slots; here lane (row j, quarter q) puts 4 columns into its 8
// slots, each column twice: slot pair i = (column c_i under set 2p, column
// c_i under set 2p+1). The dword of a looked-up cell that holds sets (2p,
// 2p+1) is exactly that B operand dword, so the lookups feed the matrix cores
// with no repacking. On the A side, token t's activation x[t][c_i] goes into
// the half of the pair that belongs to its set's parity (the other half is
// zero). The MFMA of pair p then yields, for every token t, the product with
// the tables of set slot 2p + parity(t); a token keeps the accumulator of the
// pair that holds its own set (one per pair, selected at the end). The A
// fragment is built once per 4 columns and shared by all pairs.
//
// Which 4 columns go into one MFMA is free as long as A and B agree, so they
// are chosen to match the byte lanes of the index words: b = 4 takes the even
// or the odd nibbles of one index word, b = 2 the fields i, i+4, i+8, i+12 of
// one word, b = 3 four consecutive fields.
//
// Work split as in the single-set decode: wave w handles slots (4 units = 128
// columns) w, w + NW, ..., lane (j, q) loads unit 4s+q of row j with one
// index load, and the A fragments of token t = lane % 16 come from global
// memory through a turn-around: the wave loads the slot's [m tokens][256
// bytes] in groups of four token rows (one 16-byte load per lane and group,
// neighbouring lanes on neighbouring pieces), stores them in a private LDS
// buffer and reads each lane's fragments back (loading per lane, 64 bytes of
// the lane's own token, spreads one load over many rows, which the load
// path serves piece by piece). The waves' partial tiles are summed in LDS in
// wave order (deterministic) and stored once.
//
// Set slots: each wave computes the same schedule from lut_set: set indices
// are clamped into [0, n_sets), the distinct sets are numbered in order of
// first use, and lane k holds the set of slot k.
//
// Blocks have 16 waves, or 8 when the grid has more than 384 blocks (two
// blocks then share a CU and one block's start-up hides behind the other's
// work). With bf16 activations and f16 tables each token row is prescaled
// by a power of two (skm_common.h): the waves find the rows' largest
// magnitudes before the table barrier, the activations are converted scaled
// and the sums scaled back.
#include "skm_common.h"
#include "skm_launch.h"

namespace skm {

namespace {

constexpr int DS_ROWS = 16;     // weight rows per block
// waves per block: 16 when the grid has at most 384 blocks, else 8 (two
// blocks share a CU, so one block's start-up hides behind the other's work)
constexpr int DS_NW_MAX = 16;
constexpr int64_t DS_NW16_MAX_BLOCKS = 384;
constexpr int DS_MAX_ENTRIES = 224;   // table entries per row (entry byte: 8 bits)
constexpr int DS_MAX_ENTRIES2 = 128;  // with two cells per (entry, row): doubled entry byte
// every wave turns its slot's [up to 16 tokens][16 pieces of 16 bytes]
// around in a private LDS buffer, rows padded by one piece (conflict-free
// reads)
constexpr uint32_t DS_XT_ROW = 17 * 16;
constexpr uint32_t DS_XT_WAVE = 16 * DS_XT_ROW;

template <bool V> struct btag_ds { static constexpr bool value = V; };
template <int V> struct ival_ds { static constexpr int value = V; };

typedef __attribute__((address_space(3))) uint32_t ds_u32;
typedef __attribute__((address_space(3))) u32x2 ds_u32x2;
typedef __attribute__((address_space(3))) u32x4 ds_u32x4;

template <typename TC> struct ds_mfma;
template <> struct ds_mfma<half_t> {
  typedef f16x8 vec;
  static __device__ __forceinline__ f32x4 run(vec a, vec b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
  }
};
template <> struct ds_mfma<bf16_t> {
  typedef bf16x8 vec;
  static __device__ __forceinline__ f32x4 run(vec a, vec b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
  }
};

// 8 activations in storage dtype TX -> compute dtype TC (exact widening to
// fp32, then round-to-nearest-even)
template <typename TX, typename TC>
__device__ __forceinline__ u32x4 ds_convert(u32x4 v) {
  if constexpr (__is_same(TX, TC)) {
    return v;
  } else {
    u32x4 o;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const float lo = to_f32(__builtin_bit_cast(TX, (uint16_t)(v[k] & 0xFFFFu)));
      const float hi = to_f32(__builtin_bit_cast(TX, (uint16_t)(v[k] >> 16)));
      o[k] = (uint32_t)bits16(from_f32<TC>(lo)) | ((uint32_t)bits16(from_f32<TC>(hi)) << 16);
    }
    return o;
  }
}

// 8 bf16 activations -> f16 with every value multiplied by sc (a power of two)
// first: the per-row prescale of the (BF16, F16) pair (skm_common.h)
__device__ __forceinline__ u32x4 ds_convert_scaled(u32x4 v, float sc) {
  u32x4 o;
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const float lo = __builtin_bit_cast(float, v[k] << 16) * sc;
    const float hi = __builtin_bit_cast(float, v[k] & 0xFFFF0000u) * sc;
    o[k] = (uint32_t)bits16((half_t)lo) | ((uint32_t)bits16((half_t)hi) << 16);
  }
  return o;
}

// LDS read of one cell: GW sets' 16-bit values, GW / 2 dwords
template <int GW>
__device__ __forceinline__ void ds_cell(uint32_t addr, uint32_t* g) {
  if constexpr (GW == 8) {
    const u32x4 v = *(const ds_u32x4*)(uintptr_t)addr;
    g[0] = v[0]; g[1] = v[1]; g[2] = v[2]; g[3] = v[3];
  } else if constexpr (GW == 4) {
    const u32x2 v = *(const ds_u32x2*)(uintptr_t)addr;
    g[0] = v[0]; g[1] = v[1];
  } else {
    g[0] = *(const ds_u32*)(uintptr_t)addr;
  }
}

// cell address: byte p of `ent` (an entry number, doubled with two cells per
// entry) in byte 1, the lane's row constant jc (16 j) in byte 0
__device__ __forceinline__ uint32_t ds_addr(uint32_t ent, uint32_t jc, int p) {
  return __builtin_amdgcn_perm(ent, jc, 0x0C0C0400u | ((4u + (uint32_t)p) << 8));
}

template <int B, typename TX>
struct DsSlot {
  uint32_t w[B];   // the unit's index words
  u32x4 x[4];      // token (lane % 16)'s 32 activations of the unit
  uint32_t gk;     // first entry of the unit's group (group * 2^b)
  bool ok;         // unit inside the row (RAGGED)
};

// Sources of the coalesced activation loads: load i of a slot brings
// token min(4i + l/16, m-1) (element offset off[i]) at columns 128 s + c8,
// c8 = 8 (l % 16), clamped to dcol = d - 8 when the row ends inside the slot.
template <typename TX>
struct DsXt {
  const TX* x = nullptr;
  uint32_t off[4] = {0u, 0u, 0u, 0u};
  uint32_t c8 = 0u;
  uint32_t dcol = 0u;
};

// Index and activation loads of slot s (clamped to the last slot, and to the
// last unit with RAGGED, so every load is unconditional and in range). The
// wave's XT activation loads cover the slot's [4 XT tokens][128 columns] with
// neighbouring lanes on neighbouring 16-byte pieces.
template <int B, typename TX, bool RAGGED, int XT>
__device__ __forceinline__ void ds_load(DsSlot<B, TX>& R, int64_t s, int64_t S, uint32_t U, uint32_t ug_magic,
                                        int q, const uint8_t* rowp, const DsXt<TX>& xt) {
  const int64_t sc = s < S ? s : S - 1;
  uint32_t u = 4u * (uint32_t)sc + (uint32_t)q;
  R.ok = true;
  if constexpr (RAGGED) {
    R.ok = u < U;
    u = u < U ? u : U - 1u;
  }
  load_unit<B>(rowp, u, R.w);
  uint32_t col = 128u * (uint32_t)sc + xt.c8;
  if constexpr (RAGGED) col = col < xt.dcol ? col : xt.dcol;
#pragma unroll
  for (int i = 0; i < XT; ++i) R.x[i] = *reinterpret_cast<const u32x4*>(xt.x + xt.off[i] + col);
  R.gk = (ug_magic ? __umulhi(u, ug_magic) : u) << B;
}

// GW: sets per cell read (2, 4 or 8); OCT2: a second cell per (entry, row)
// for set slots 8..15 (GW == 8 only).
template <int B, int NW, int GW, bool OCT2, typename TX, typename TL, bool RAGGED, int XT>
__global__ void __launch_bounds__(NW * 64, 16 / NW)
k_decode_sets(const TX* __restrict__ X, const uint8_t* __restrict__ idx_packed, const TL* __restrict__ luts,
              const int32_t* __restrict__ lut_set, int n_sets, int64_t set_stride, int m, int64_t n, int64_t d,
              int gpr, uint32_t ug_magic, TX* __restrict__ Y) {
  // Dynamic LDS only (no static LDS: absolute addresses from 0): the cells
  // [entry][cell][row] of 16 bytes; after the last lookup, the waves'
  // [NW][16][16] fp32 partial tiles in the same place; XT: the waves'
  // activation buffers above both.
  extern __shared__ uint32_t smem[];
  static_assert(NW == 8 || NW == 16, "8 or 16 waves");
  constexpr int NP = (OCT2 ? 16 : GW) / 2;  // set pairs (accumulators)
  constexpr uint32_t ES = OCT2 ? 512u : 256u;  // bytes per entry
  typedef ds_mfma<TL> MF;
  // (BF16, F16): each token row is prescaled by 2^-e before the f16
  // conversion and its results multiplied by 2^e (skm_common.h)
  constexpr bool SC = scaled_pair(__is_same(TX, bf16_t), __is_same(TL, half_t));
  static_assert(GW == 2 || GW == 4 || GW == 8, "cell reads of 2, 4 or 8 sets");
  static_assert(!OCT2 || GW == 8, "a second cell only after a full first one");
  static_assert(XT == 1 || XT == 2 || XT == 4, "turn-around loads: groups of four token rows");

  const int lane = lane_id();
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int64_t row0 = (int64_t)blockIdx.x * DS_ROWS;
  const int j = lane & 15;  // weight row within the block (B operand column)
  const int q = lane >> 4;  // contraction quarter
  const int64_t grow = row0 + j;
  const bool row_ok = grow < n;
  const int tokc = j < m ? j : m - 1;  // A operand row = token (clamped)
  const int E = gpr << B;              // table entries per row

  const uint32_t U = (uint32_t)(d / 32);
  const int64_t S = (U + 3) / 4;  // slots per row
  const uint8_t* rowp = idx_packed + (row_ok ? grow : n - 1) * (d * B / 8);
  DsXt<TX> xts;
  {
    xts.x = X;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int t = 4 * i + q;
      xts.off[i] = (uint32_t)((t < m ? t : m - 1) * d);
    }
    xts.c8 = 8u * (uint32_t)j;
    xts.dcol = (uint32_t)d - 8u;
  }

  // The set indices are loaded first and the first slot's index and
  // activation loads right after them, so that the index stream is under way
  // while the table loads wait for the set indices (the loads complete in
  // order, so waiting for the set indices does not wait for the slot's).
  const int tl = lane < m ? lane : m - 1;
  const int sv = lut_set[tl];
  int64_t s0 = wave;
  DsSlot<B, TX> R0, R1;
  ds_load<B, TX, RAGGED, XT>(R0, s0, S, U, ug_magic, q, rowp, xts);
  ds_load<B, TX, RAGGED, XT>(R1, s0 + NW, S, U, ug_magic, q, rowp, xts);

  // ---- set slots (every wave computes the same)
  const int setv = sv < 0 ? 0 : (sv >= n_sets ? n_sets - 1 : sv);
  int ftok = tl;  // first token on this token's set
  for (int u = 0; u < m; ++u) {
    const int su = __builtin_amdgcn_readlane(setv, u);
    ftok = (su == setv && u < ftok) ? u : ftok;
  }
  const uint64_t firsts = __ballot(lane < m && ftok == lane);
  const int nd = __popcll(firsts);                                    // distinct sets in use
  const int slot = __popcll(firsts & ((1ull << ftok) - 1ull));        // slot of this lane's token
  // lane k: the set of slot k (k < nd), then the last slot's set
  const int pushed = __builtin_amdgcn_ds_permute(slot * 4, setv);
  const int setk = __shfl(pushed, lane < nd ? lane : nd - 1, 64);

  // ---- table loads: unit (cell c, row jj, 4-entry chunk ec); rows vary
  // fastest, so a wave's cell writes cover 256 contiguous bytes per chunk
  constexpr int UPT = 16 / NW;  // units per thread (at most 1024 units: the host checks the count)
  const int EC = E >> 2;
  const int units = (OCT2 ? 2 : 1) * 16 * EC;
  u32x2 tv[UPT][GW];
#pragma unroll
  for (int k = 0; k < UPT; ++k) {
    const int uid0 = (int)threadIdx.x + k * NW * 64;
    const int uid = uid0 < units ? uid0 : units - 1;
    const int jj = uid & 15, ec = (uid >> 4) % EC, c = (uid >> 4) / EC;
    const int64_t tr = row0 + jj < n ? row0 + jj : n - 1;
#pragma unroll
    for (int kk = 0; kk < GW; ++kk) {
      const int sl = c * 8 + kk;
      const int st = __shfl(setk, sl < nd ? sl : nd - 1, 64);
      tv[k][kk] = *reinterpret_cast<const u32x2*>(luts + (int64_t)st * set_stride + tr * E + 4 * ec);
    }
  }
  // cells: entry 4 ec + e of row jj for the set slots of cell c
#pragma unroll
  for (int k = 0; k < UPT; ++k) {
    const int uid = (int)threadIdx.x + k * NW * 64;
    if (uid < units) {
      const int jj = uid & 15, ec = (uid >> 4) % EC, c = (uid >> 4) / EC;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const uint32_t sel = (e & 1) ? 0x07060302u : 0x05040100u;
        uint32_t o[GW / 2];
#pragma unroll
        for (int i = 0; i < GW / 2; ++i)
          o[i] = __builtin_amdgcn_perm(tv[k][2 * i + 1][e >> 1], tv[k][2 * i][e >> 1], sel);
        const uint32_t a = (uint32_t)(4 * ec + e) * ES + (uint32_t)c * 256u + (uint32_t)jj * 16u;
        if constexpr (GW == 8) *(ds_u32x4*)(uintptr_t)a = u32x4{o[0], o[1], o[2], o[3]};
        else if constexpr (GW == 4) *(ds_u32x2*)(uintptr_t)a = u32x2{o[0], o[1]};
        else *(ds_u32*)(uintptr_t)a = o[0];
      }
    }
  }
  // LDS above the cells (or the partial tiles, when larger): the XT buffers,
  // then (SC) the largest magnitude of each token row
  const uint32_t cells = (uint32_t)E * ES;
  const uint32_t above = cells > NW * 1024u ? cells : NW * 1024u;
  const uint32_t rmax = above + NW * DS_XT_WAVE;
  if constexpr (SC) {
    // wave w < m scans token row w (wave-uniform branch)
    // (wave-uniform loop: wave w takes rows w, w + NW)
    for (int tr = wave; tr < m; tr += NW) {
      const TX* xr = X + (int64_t)tr * d;
      uint32_t mx = 0u;
      for (int64_t c = (int64_t)lane * 8; c < d; c += 512) {
        const uint32_t v = absmax8_bf16(*reinterpret_cast<const u32x4*>(xr + c));
        mx = mx > v ? mx : v;
      }
      mx = wave_max_to_lane63(mx);
      if (lane == 63) *(ds_u32*)(uintptr_t)(rmax + (uint32_t)tr * 4u) = mx;
    }
  }
  // every load is consumed by now, the slots' (issued before the table
  // loads) included, or has landed
  __syncthreads();

  const uint32_t jc = (uint32_t)j * 16u;
  // SC: 2^-e of this lane's A row (its token)
  const float xsc = SC ? pow2f(-row_exp_of(*(const ds_u32*)(uintptr_t)(rmax + (uint32_t)tokc * 4u))) : 1.0f;
  (void)xsc;
  // XT: this wave's buffer, above the cells and the partial tiles
  const uint32_t xt_w = above + (uint32_t)wave * DS_XT_WAVE;
  const uint32_t xt_st = xt_w + (uint32_t)q * DS_XT_ROW + (uint32_t)j * 16u;
  const uint32_t xt_ld = xt_w + (uint32_t)tokc * DS_XT_ROW + (uint32_t)q * 64u;
  (void)xt_st;
  (void)xt_ld;
  // A fragment selectors: token's value into the half of its set's parity
  const int par = __shfl(slot, tokc, 64) & 1;
  const uint32_t sel_lo = par ? 0x01000C0Cu : 0x0C0C0100u;
  const uint32_t sel_hi = par ? 0x03020C0Cu : 0x0C0C0302u;

  f32x4 acc[NP];
#pragma unroll
  for (int p = 0; p < NP; ++p) acc[p] = f32x4{0.f, 0.f, 0.f, 0.f};

  // one MFMA chunk: 4 cell addresses (byte p of ent for p = 0..3, or given
  // addresses for b = 3) and the 4 A dwords. NPA (compile time) pairs run
  // without branches, so lookups and MFMAs of successive chunks overlap;
  // pairs past the sets in use read valid (clamped) cells and their
  // accumulators are never selected.
  auto chunk = [&](auto npa, const uint32_t (&addr)[4], const u32x4& a, bool ok) {
    constexpr int NPA = decltype(npa)::value;
    constexpr int P1 = NPA < GW / 2 ? NPA : GW / 2;  // pairs in the first cell
    uint32_t g[4][GW / 2];
#pragma unroll
    for (int i = 0; i < 4; ++i) ds_cell<GW>(addr[i], g[i]);
    u32x4 av = a;
    if constexpr (RAGGED) {
      if (!ok) av = u32x4{0u, 0u, 0u, 0u};
    }
#pragma unroll
    for (int p = 0; p < P1; ++p) {
      u32x4 bv{g[0][p], g[1][p], g[2][p], g[3][p]};
      if constexpr (RAGGED) {
        if (!ok) bv = u32x4{0u, 0u, 0u, 0u};
      }
      acc[p] = MF::run(__builtin_bit_cast(typename MF::vec, av), __builtin_bit_cast(typename MF::vec, bv), acc[p]);
    }
    if constexpr (NPA > 4) {
      // (the second cells' lookups after the first cells' MFMAs: one set of
      // lookup registers at a time)
      __builtin_amdgcn_sched_barrier(0);
      uint32_t g2[4][4];
#pragma unroll
      for (int i = 0; i < 4; ++i) ds_cell<8>(addr[i] + 256u, g2[i]);
#pragma unroll
      for (int p = 0; p < NPA - 4; ++p) {
        u32x4 bv{g2[0][p], g2[1][p], g2[2][p], g2[3][p]};
        if constexpr (RAGGED) {
          if (!ok) bv = u32x4{0u, 0u, 0u, 0u};
        }
        acc[4 + p] = MF::run(__builtin_bit_cast(typename MF::vec, av), __builtin_bit_cast(typename MF::vec, bv),
                             acc[4 + p]);
      }
    }
    // keep the next chunk's lookups behind this one's (bounded registers;
    // the other waves of the SIMD cover the lookup latency)
    if constexpr (GW > 2) __builtin_amdgcn_sched_barrier(0);
  };

  auto compute = [&](auto npa, const DsSlot<B, TX>& Rc, int64_t s, auto tail) {
    if (decltype(tail)::value && s >= S) return;  // wave-uniform
    // a lane stores load i at row 4i + l/16, piece l%16, and reads its
    // token's (row min(l%16, m-1)) pieces 4q..4q+3: unit 4s+q (one wave's
    // LDS accesses are carried out in order)
#pragma unroll
    for (int i = 0; i < XT; ++i) *(ds_u32x4*)(uintptr_t)(xt_st + (uint32_t)i * 4u * DS_XT_ROW) = Rc.x[i];
    // columns 8h..8h+7 of the unit in the compute dtype (dword i = columns
    // 8h + 2i, 8h + 2i + 1), read where first needed
    auto xq = [&](int h) -> u32x4 {
      const u32x4 v = *(const ds_u32x4*)(uintptr_t)(xt_ld + 16u * (uint32_t)h);
      if constexpr (SC) return ds_convert_scaled(v, xsc);
      else return ds_convert<TX, TL>(v);
    };
    const uint32_t gk = OCT2 ? Rc.gk * 2u : Rc.gk;
    const uint32_t gk4 = __builtin_amdgcn_perm(0u, gk, 0u);  // gk (< 256) in all four bytes
    if constexpr (B == 4) {
      // word k: fields 8k..8k+7; even fields (nibbles 0,2,4,6) in bytes 0..3, then odd
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const uint32_t w = Rc.w[k];
        const u32x4 xk = xq(k);
        // columns 8k + 2i (low halves of xk[i]), then 8k + 2i + 1 (high halves)
        {
          const uint32_t ev = OCT2 ? (((w << 1) & 0x1E1E1E1Eu) | gk4) : ((w & 0x0F0F0F0Fu) | gk4);
          const uint32_t ae[4] = {ds_addr(ev, jc, 0), ds_addr(ev, jc, 1), ds_addr(ev, jc, 2), ds_addr(ev, jc, 3)};
          const u32x4 xe{__builtin_amdgcn_perm(0u, xk[0], sel_lo), __builtin_amdgcn_perm(0u, xk[1], sel_lo),
                         __builtin_amdgcn_perm(0u, xk[2], sel_lo), __builtin_amdgcn_perm(0u, xk[3], sel_lo)};
          chunk(npa, ae, xe, Rc.ok);
        }
        {
          const uint32_t od = OCT2 ? (((w >> 3) & 0x1E1E1E1Eu) | gk4) : (((w >> 4) & 0x0F0F0F0Fu) | gk4);
          const uint32_t ao[4] = {ds_addr(od, jc, 0), ds_addr(od, jc, 1), ds_addr(od, jc, 2), ds_addr(od, jc, 3)};
          const u32x4 xo{__builtin_amdgcn_perm(0u, xk[0], sel_hi), __builtin_amdgcn_perm(0u, xk[1], sel_hi),
                         __builtin_amdgcn_perm(0u, xk[2], sel_hi), __builtin_amdgcn_perm(0u, xk[3], sel_hi)};
          chunk(npa, ao, xo, Rc.ok);
        }
      }
    } else if constexpr (B == 2) {
      // word k: fields 16k..16k+15; chunk i: fields 16k + i + 4c in byte c
#pragma unroll
      for (int k = 0; k < 2; ++k) {
        const u32x4 xa = xq(2 * k), xb = xq(2 * k + 1);
        // column 16k + i + 4c = half (i & 1) of local dword 2c + (i >> 1)
        const uint32_t xl[8] = {xa[0], xa[1], xa[2], xa[3], xb[0], xb[1], xb[2], xb[3]};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const uint32_t w = Rc.w[k];
          const uint32_t f = OCT2 ? ((i == 0 ? (w << 1) : (w >> (2 * i - 1))) & 0x06060606u)
                                  : ((w >> (2 * i)) & 0x03030303u);
          const uint32_t ent = f | gk4;
          const uint32_t a[4] = {ds_addr(ent, jc, 0), ds_addr(ent, jc, 1), ds_addr(ent, jc, 2), ds_addr(ent, jc, 3)};
          const uint32_t sl = (i & 1) ? sel_hi : sel_lo;
          const u32x4 xv{__builtin_amdgcn_perm(0u, xl[(i >> 1)], sl), __builtin_amdgcn_perm(0u, xl[2 + (i >> 1)], sl),
                         __builtin_amdgcn_perm(0u, xl[4 + (i >> 1)], sl), __builtin_amdgcn_perm(0u, xl[6 + (i >> 1)], sl)};
          chunk(npa, a, xv, Rc.ok);
        }
      }
    } else {
      // 3-bit fields at any bit offset: chunk h = fields 4h..4h+3
      const uint32_t base = (gk << 8) | jc;
#pragma unroll
      for (int hp = 0; hp < 4; ++hp) {
        const u32x4 xk = xq(hp);
#pragma unroll
        for (int hh = 0; hh < 2; ++hh) {
          const int h = 2 * hp + hh;
          uint32_t a[4];
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const uint32_t e = unit_field<3>(Rc.w, 4 * h + i);
            a[i] = base + (e << (OCT2 ? 9 : 8));
          }
          // columns 4h..4h+3: dwords 2hh, 2hh + 1 of xk
          const u32x4 xv{__builtin_amdgcn_perm(0u, xk[2 * hh], sel_lo), __builtin_amdgcn_perm(0u, xk[2 * hh], sel_hi),
                         __builtin_amdgcn_perm(0u, xk[2 * hh + 1], sel_lo),
                         __builtin_amdgcn_perm(0u, xk[2 * hh + 1], sel_hi)};
          chunk(npa, a, xv, Rc.ok);
        }
      }
    }
  };

  // slots of this wave: at least one (possibly past the row end: skipped)
  const int64_t nb_raw = (S - s0 + NW - 1) / NW;
  const int64_t nb = nb_raw > 1 ? nb_raw : 1;
  // two register sets, two slots in flight, one exit, unconditional loads
  // (exact load counts; the last iteration's loads of slots past the end
  // are clamped and left unused)
  auto run = [&](auto npa) {
    int64_t bi = 0;
    for (; bi + 2 < nb; bi += 2) {
      compute(npa, R0, s0, btag_ds<false>{});
      ds_load<B, TX, RAGGED, XT>(R0, s0 + 2 * NW, S, U, ug_magic, q, rowp, xts);
      compute(npa, R1, s0 + NW, btag_ds<false>{});
      ds_load<B, TX, RAGGED, XT>(R1, s0 + 3 * NW, S, U, ug_magic, q, rowp, xts);
      s0 += 2 * NW;
    }
    compute(npa, R0, s0, btag_ds<true>{});
    if (nb - bi == 2) compute(npa, R1, s0 + NW, btag_ds<true>{});
  };
  // every pair of the capacity (chosen on the host from min(m, n_sets)), in
  // use or not: one branch-free instance of the slot loop
  run(ival_ds<NP>{});

  // ---- each output keeps its token's pair: lane l holds D[token 4q + r][row j]
  f32x4 out = acc[0];
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const int t = 4 * q + r;
    const int pr = __shfl(slot, t < m ? t : m - 1, 64) >> 1;
#pragma unroll
    for (int p = 1; p < NP; ++p) out[r] = pr == p ? acc[p][r] : out[r];
  }
  // partial tiles over the cells, once every wave is done with them; summed
  // in wave order
  __syncthreads();
  float* red = reinterpret_cast<float*>(smem);
#pragma unroll
  for (int r = 0; r < 4; ++r) red[wave * 256 + (4 * q + r) * 16 + j] = out[r];
  __syncthreads();
  const int t = threadIdx.x;
  if (t < 256) {
    const int token = t >> 4, rr = t & 15;
    if (token < m && row0 + rr < n) {
      float sum = 0.0f;
#pragma unroll
      for (int wv = 0; wv < NW; ++wv) sum += red[wv * 256 + t];
      if constexpr (SC) sum *= pow2f(row_exp_of(*(const ds_u32*)(uintptr_t)(rmax + (uint32_t)token * 4u)));
      Y[(int64_t)token * n + row0 + rr] = from_f32<TX>(sum);
    }
  }
}

template <int B, int NW, int GW, bool OCT2, typename TX, typename TL, bool RAGGED, int XT>
hipError_t sets_kernel(const TX* X, const uint8_t* idx, const TL* luts, const int32_t* lut_set, int n_sets,
                       const Problem& p, TX* Y, hipStream_t s, uint32_t magic, size_t lds) {
  const auto kern = k_decode_sets<B, NW, GW, OCT2, TX, TL, RAGGED, XT>;
  static const hipError_t prep = prepare_kernel((const void*)kern, lds);
  if (prep != hipSuccess) return prep;
  const dim3 grid((unsigned)((p.n + DS_ROWS - 1) / DS_ROWS));
  hipLaunchKernelGGL(kern, grid, dim3(NW * 64), lds, s, X, idx, luts, lut_set, n_sets, p.n * ((int64_t)p.gpr << p.b),
                     (int)p.m, p.n, p.d, p.gpr, magic, Y);
  return hipGetLastError();
}

template <int B, int NW, int GW, bool OCT2, typename TX, typename TL>
hipError_t sets_launch(const TX* X, const uint8_t* idx, const TL* luts, const int32_t* lut_set, int n_sets,
                       const Problem& p, TX* Y, hipStream_t s) {
  const uint32_t ug = (uint32_t)(p.group_cols() / 32);
  // u / ug == umulhi(u, magic) for u * ug < 2^32; ug == 1 is passed as 0
  const uint32_t magic = ug == 1 ? 0u : (uint32_t)((((uint64_t)1) << 32) / ug + 1);
  const size_t cells = (size_t)((int64_t)p.gpr << p.b) * (OCT2 ? 512 : 256);
  const size_t part = (size_t)NW * 256 * 4;
  // + the waves' turn-around buffers + 16 row maxima of the (BF16, F16) prescale
  const size_t lds = (cells > part ? cells : part) + (size_t)NW * DS_XT_WAVE + 64;
  const bool ragged = p.units() % 4 != 0;
  // turn-around loads: groups of four token rows, ceil(m / 4) rounded up to 1, 2 or 4
  if (p.m > 8)
    return ragged ? sets_kernel<B, NW, GW, OCT2, TX, TL, true, 4>(X, idx, luts, lut_set, n_sets, p, Y, s, magic, lds)
                  : sets_kernel<B, NW, GW, OCT2, TX, TL, false, 4>(X, idx, luts, lut_set, n_sets, p, Y, s, magic, lds);
  if constexpr (OCT2) {
    return hipErrorNotSupported;  // (more than 8 sets means more than 8 tokens)
  } else {
    if (p.m > 4)
      return ragged ? sets_kernel<B, NW, GW, OCT2, TX, TL, true, 2>(X, idx, luts, lut_set, n_sets, p, Y, s, magic, lds)
                    : sets_kernel<B, NW, GW, OCT2, TX, TL, false, 2>(X, idx, luts, lut_set, n_sets, p, Y, s, magic, lds);
    return ragged ? sets_kernel<B, NW, GW, OCT2, TX, TL, true, 1>(X, idx, luts, lut_set, n_sets, p, Y, s, magic, lds)
                  : sets_kernel<B, NW, GW, OCT2, TX, TL, false, 1>(X, idx, luts, lut_set, n_sets, p, Y, s, magic, lds);
  }
}

template <int B, typename TX, typename TL>
hipError_t sets_b(const TX* X, const uint8_t* idx, const TL* luts, const int32_t* lut_set, int n_sets,
                  const Problem& p, TX* Y, hipStream_t s) {
  const int64_t bound = p.m < n_sets ? p.m : n_sets;  // distinct sets at most
  if ((p.n + DS_ROWS - 1) / DS_ROWS > DS_NW16_MAX_BLOCKS) {
    if (bound <= 2) return sets_launch<B, 8, 2, false>(X, idx, luts, lut_set, n_sets, p, Y, s);
    if (bound <= 4) return sets_launch<B, 8, 4, false>(X, idx, luts, lut_set, n_sets, p, Y, s);
    if (bound <= 8) return sets_launch<B, 8, 8, false>(X, idx, luts, lut_set, n_sets, p, Y, s);
    return sets_launch<B, 8, 8, true>(X, idx, luts, lut_set, n_sets, p, Y, s);
  }
  if (bound <= 2) return sets_launch<B, 16, 2, false>(X, idx, luts, lut_set, n_sets, p, Y, s);
  if (bound <= 4) return sets_launch<B, 16, 4, false>(X, idx, luts, lut_set, n_sets, p, Y, s);
  if (bound <= 8) return sets_launch<B, 16, 8, false>(X, idx, luts, lut_set, n_sets, p, Y, s);
  return sets_launch<B, 16, 8, true>(X, idx, luts, lut_set, n_sets, p, Y, s);
}

template <typename TX, typename TL>
hipError_t sets_t(const TX* X, const uint8_t* idx, const TL* luts, const int32_t* lut_set, int n_sets,
                  const Problem& p, TX* Y, hipStream_t s) {
  switch (p.b) {
    case 2: return sets_b<2>(X, idx, luts, lut_set, n_sets, p, Y, s);
    case 3: return sets_b<3>(X, idx, luts, lut_set, n_sets, p, Y, s);
    default: return sets_b<4>(X, idx, luts, lut_set, n_sets, p, Y, s);
  }
}

}  // namespace

bool decode_sets_supported(const Problem& p, int n_sets, bool scaled) {
  // one token uses one set: the single-pass multi-set decode serves it with
  // the single-set lookups (no parity halves, activations staged)
  // (the (BF16, F16) pair with one set: every token on set 0, still prescaled)
  if (p.m < 2 || p.m > 16 || n_sets < 1 || (n_sets < 2 && !scaled)) return false;
  const int64_t E = (int64_t)p.gpr << p.b;
  const int64_t bound = p.m < n_sets ? p.m : n_sets;
  const int64_t maxe = bound > 8 ? DS_MAX_ENTRIES2 : DS_MAX_ENTRIES;
  // table units (cells x rows x 4-entry chunks): one per thread
  const int64_t units = (bound > 8 ? 2 : 1) * 16 * (E / 4);
  return E <= maxe && units <= DS_NW_MAX * 64 && p.d <= (int64_t(1) << 20);
}

hipError_t launch_decode_sets(const void* X, int x_dtype, const uint8_t* idx, const void* luts, int lut_dtype,
                              const int32_t* lut_set, int n_sets, const Problem& p, void* Y, hipStream_t s) {
  if (x_dtype == DT_F16 && lut_dtype == DT_F16)
    return sets_t((const half_t*)X, idx, (const half_t*)luts, lut_set, n_sets, p, (half_t*)Y, s);
  if (x_dtype == DT_F16 && lut_dtype == DT_BF16)
    return sets_t((const half_t*)X, idx, (const bf16_t*)luts, lut_set, n_sets, p, (half_t*)Y, s);
  if (x_dtype == DT_BF16 && lut_dtype == DT_BF16)
    return sets_t((const bf16_t*)X, idx, (const bf16_t*)luts, lut_set, n_sets, p, (bf16_t*)Y, s);
  return sets_t((const bf16_t*)X, idx, (const half_t*)luts, lut_set, n_sets, p, (bf16_t*)Y, s);  // (BF16, F16)
}

}  // namespace skm
