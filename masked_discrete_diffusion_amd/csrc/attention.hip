// Step attention under the step-causal mask.
//
// The query set of a step is [D | C | R]: rows entering the cache, the masked
// rows decoded now, the registers (page 1, worked example = the paper's
// Figure 3).  D rows see the cache (which already holds D); C and R rows see
// the cache, every C key and every R key.  The keys a block streams are laid
// out in three segments of 64-key tiles: the cache slots [0, S), the C keys,
// the R keys (softmax does not depend on key order).  A D row's visible set is
// the first segment, a C/R row's all three, so the mask is a per-wavefront
// tile bound plus the valid count of a segment's last tile.  Rows are cut into
// 32-row chunks of a single kind.  Keys past a tile's valid count are removed
// by select (scores to -1e30, values to 0), never multiplied by zero, so stale
// slots cannot leak even when they hold NaN.
//
// C and R keys/values are never stored in the cache: a C row is the mask
// token, so its key depends on its position only and its value is the same
// for every C key; a register's key and value are fixed.  Tables built once at
// init hold them in the layouts the tiles need: the keys of the mask token at
// every position and of the registers (key table), the mask token's value
// repeated as 8-key V^T units, and the registers' values transposed.
//
// bf16 path (block = 8 wavefronts = 8 chunks of 32 rows of the query heads of
// one key/value head, over one contiguous range of the tiles):
//   Every tile goes from HBM straight into LDS with global_load_lds_dwordx4
//   (no register staging; per-lane source addresses gather the C keys' rows)
//   through a 4-deep ring, one barrier per tile; LDS rows are padded by 16
//   bytes so the MFMA operand reads are bank-conflict free with compile-time
//   offsets.
//   S^T = K Q^T with v_mfma_f32_32x32x16_bf16 (Q^T in registers, RoPE'd in the
//   prologue), fp32 online softmax with a lazily raised reference maximum
//   (one partner exchange per half-tile for the row max), P split into bf16
//   hi + lo, O^T += V^T P_hi^T + V^T P_lo^T, fp32 out.
//   The key rows of the K operand are permuted so each lane's eight P values
//   of a k-step are eight consecutive keys: the V^T operand is one 16-byte read.
//   When there are fewer (sequence, kv head, chunk group) blocks than compute
//   units, the tiles are split over several blocks; each writes its unscaled
//   partial (O, row reference, row sum) and a second small kernel merges the
//   partials in split order.  (A last-arriving-block merge inside the kernel
//   needs device-scope fences, which write back and invalidate the whole L2
//   of an XCD and cost more than the launch.)  Block ids are remapped so that
//   the blocks of a group sit on one XCD (and L2).
// fp32 path: the same mask with fp32 VALU arithmetic (validation mode).
#include <algorithm>

#include "common.hpp"
#include "kernels.hpp"

namespace mdm {

namespace {

constexpr float kNegInf = -__builtin_inff();
constexpr float kLog2e = 1.4426950408889634f;
// Score of a key a row may not see: finite, so that exp2 of (score - reference)
// is exactly 0 without ever forming inf - inf.
constexpr float kMaskedScore = -1e30f;
constexpr int kAttnWaves = 8;                  // wavefronts per bf16 attention block
constexpr int kAttnThreads = kAttnWaves * 64;
constexpr int kStages = 4;                     // LDS ring depth (tiles) of the bf16 kernel
constexpr int kAhead = 2;                      // tiles loaded ahead of the one being computed

struct RowInfo {
  int id, pos;
};

// Token id and position of query row `row` (D | C | R) of sequence b.
__device__ inline RowInfo query_row(const Geometry& g, const AttnArgs& a, int b, int row) {
  RowInfo ri;
  if (row < a.n_d) {
    ri.id = a.d_tok[(int64_t)b * a.d_stride + row];
    ri.pos = a.d_pos[(int64_t)b * a.d_stride + row];
  } else if (row < a.n_d + a.n_c) {
    ri.id = g.V;
    ri.pos = a.c_pos[(int64_t)b * a.c_stride + (row - a.n_d)];
  } else {
    const int j = row - a.n_d - a.n_c;
    ri.id = g.V + 1 + j;
    ri.pos = g.seq_len + j;
  }
  if (ri.id < 0 || ri.id >= g.table_rows) { flag_error(a.err, kErrTok); ri.id = 0; }
  if (ri.pos < 0 || ri.pos >= g.max_pos) { flag_error(a.err, kErrPos); ri.pos = 0; }
  return ri;
}

// Transient key j (slot S + j): its key-table row.
__device__ inline int transient_krow(const Geometry& g, const AttnArgs& a, int b, int j) {
  if (j < a.n_c) {
    int pos = a.c_pos[(int64_t)b * a.c_stride + j];
    if (pos < 0 || pos >= g.seq_len) { flag_error(a.err, kErrPos); pos = 0; }
    return pos;
  }
  return g.seq_len + (j - a.n_c);
}

// Token id of transient key j: the mask token, then the registers.
__device__ inline int transient_id(const Geometry& g, const AttnArgs& a, int j) {
  return j < a.n_c ? g.V : g.V + 1 + (j - a.n_c);
}

struct ChunkPlan {
  int chunks_d;     // chunks of D rows
  int n_chunks;     // D chunks then C|R chunks
  int per_block;    // chunks (wavefronts) per block
  int blocks;       // chunk groups per (sequence, kv head)
  int ksplit;       // blocks sharing one chunk group's key tiles (bf16 path)
  int real_blocks;  // B * Hkv * blocks * ksplit (the grid may be padded to a multiple of 8)
  int pair;         // bf16: chunk groups of four, wavefronts w and w + 4 split the tiles by parity
};

// Rows [base, end) of chunk ch; is_cr: a chunk of C|R rows (sees every key)
// rather than D rows (see the cache only).
__host__ __device__ inline void chunk_rows(const AttnArgs& a, const ChunkPlan& cp, int rows_per_chunk,
                                           int ch, int& base, int& end, bool& is_cr) {
  if (ch < cp.chunks_d) {
    base = ch * rows_per_chunk;
    end = min(base + rows_per_chunk, a.n_d);
    is_cr = false;
  } else {
    const int cc = ch - cp.chunks_d;
    base = a.n_d + cc * rows_per_chunk;
    end = min(base + rows_per_chunk, a.n_d + a.n_c + a.n_r);
    is_cr = true;
  }
}

// ---------------------------------------------------------------- bf16 MFMA --
// LDS tile layouts, in 16-byte units ("chunks"), rows padded by one unit so
// that MFMA operand reads of 16 consecutive rows hit distinct banks:
//   K   [64 keys][D]:   key r, chunk c at unit r*KU + c,   KU = D/8 + 1
//   V^T [D][64 keys]:   dim d, chunk c at unit d*VU + c,   VU = 8 + 1
// A wave-wide LDS-DMA load fills 64 consecutive units (1 KiB); lane l fills
// unit 64*blk + l with the chunk that belongs there (a pad unit receives an
// in-bounds copy of chunk 0 of its row, never read).  The K blocks and then
// the V^T blocks of a tile are dealt round-robin to the block's wavefronts.
template <int D>
struct AttnTile {
  static constexpr int KT = kKeyTile;
  static constexpr int KC = D / 8;                   // chunks per key row
  static constexpr int KU = KC + 1;                  // units per padded key row
  static constexpr int VC = KT / 8;                  // chunks per V^T row
  static constexpr int VU = VC + 1;
  static constexpr int K_BLOCKS = KT * KU / kWave;   // 1 KiB DMA blocks per K tile
  static constexpr int V_BLOCKS = D * VU / kWave;
  static constexpr int BLOCKS = K_BLOCKS + V_BLOCKS;
  static constexpr int K_ELEMS = KT * KU * 8;        // bf16 elements per K tile
  static constexpr int V_ELEMS = D * VU * 8;
  // DMA loads per loading wavefront per tile: wavefront w issues blocks
  // [w*LPW, w*LPW + LPW); the remaining wavefronts issue none, so every
  // loading wavefront has the same count and the ring waits are constants.
  static constexpr int LPW = (BLOCKS + kAttnWaves - 1) / kAttnWaves;
  static_assert(BLOCKS % LPW == 0, "DMA blocks must split evenly over the loading wavefronts");
  static constexpr int LOADERS = BLOCKS / LPW;
};

// Tile t of a block's key range: segment (0 cache, 1 C keys, 2 registers),
// first key within the segment, number of valid keys (1..64).
struct TileRef {
  int seg, base, valid;
};
__device__ inline TileRef tile_ref(const AttnArgs& a, int T0, int T1, int t) {
  if (t < T0) return TileRef{0, t * kKeyTile, min(kKeyTile, a.S - t * kKeyTile)};
  t -= T0;
  if (t < T1) return TileRef{1, t * kKeyTile, min(kKeyTile, a.n_c - t * kKeyTile)};
  t -= T1;
  return TileRef{2, t * kKeyTile, min(kKeyTile, a.n_r - t * kKeyTile)};
}

// Per-(sequence, kv head) sources of the three segments.
struct KvSrc {
  const uint16_t* kc;     // cache keys [slots][D]
  const uint16_t* vc;     // cache values [slots/64][D][64] (V^T in 64-slot tiles)
  const uint16_t* ktab;   // key table [ktab_rows][D]
  const uint16_t* mvt;    // mask-token value units [D][8]
  const uint16_t* rvt;    // register values [D][r_pad]
  const int* kidx;        // LDS: key-table row of each C key
  int k2row0;             // key-table row of the first segment-2 key (seq_len; 0 in transient mode)
};

// Byte offsets, per lane, of this wavefront's DMA units for a cache tile,
// relative to the tile's first key (K) or its V^T tile (each 64-slot V^T
// tile is one contiguous [D][64] block): K unit (row r, chunk c) -> r*D + 8c,
// V^T unit (dim d, chunk c) -> 64d + 8c (elements, times 2).  A pad unit
// (c = last) loads chunk 0 of its row, never read.
template <int D>
__device__ inline void dma_offsets(int wave, int lane, uint32_t (&off)[AttnTile<D>::LPW]) {
  using T = AttnTile<D>;
#pragma unroll
  for (int i = 0; i < T::LPW; ++i) {
    const int blk = min(wave * T::LPW + i, T::BLOCKS - 1);
    if (blk < T::K_BLOCKS) {
      const int u = blk * kWave + lane;
      const int r = u / T::KU, c = u % T::KU;
      off[i] = 2u * (uint32_t)(r * D + (c < T::KC ? c : 0) * 8);
    } else {
      const int u = (blk - T::K_BLOCKS) * kWave + lane;
      const int d = u / T::VU, c = u % T::VU;
      off[i] = 2u * (uint32_t)(d * kKeyTile + (c < T::VC ? c : 0) * 8);
    }
  }
}

// Issue this wavefront's LDS-DMA loads of one tile (segment, first key base).
// Rows past the valid count load in-bounds rows (spare cache slots, clamped
// C index, key-table padding, zero register columns); select removes them.
template <int D>
__device__ inline void tile_dma(const AttnArgs& a, const Geometry& g, const KvSrc& src, const TileRef& tr,
                                int wave, int lane, const uint32_t (&off)[AttnTile<D>::LPW], uint16_t* ks,
                                uint16_t* vs) {
  using T = AttnTile<D>;
  if (wave >= T::LOADERS) return;
  // C-key and register tiles (at most one or two per block) compute their
  // per-lane offsets here; the opaque copy of the lane id keeps the compiler
  // from hoisting them out of the tile loop, where they would need VGPRs.
  int ln = lane;
  asm volatile("" : "+v"(ln));
  const uint16_t* kbase = tr.seg == 0 ? src.kc + (int64_t)tr.base * D
                                      : src.ktab + (int64_t)(src.k2row0 + tr.base) * D;   // seg 2 (seg 1 below)
  const uint16_t* vbase = src.vc + (int64_t)tr.base * D;                               // seg 0: V^T tile
#pragma unroll
  for (int i = 0; i < T::LPW; ++i) {
    const int blk = wave * T::LPW + i;
    if (blk < T::K_BLOCKS) {
      uint16_t* dst = ks + blk * kWave * 8;
      if (tr.seg != 1) {
        dma16(kbase, off[i], dst);
      } else {
        const int u = blk * kWave + ln;
        const int r = u / T::KU, c = u % T::KU;
        const int row = src.kidx[min(tr.base + r, a.n_c - 1)];
        dma16(src.ktab, 2u * (uint32_t)(row * D + (c < T::KC ? c : 0) * 8), dst);
      }
    } else {
      const int vb = blk - T::K_BLOCKS;
      uint16_t* dst = vs + vb * kWave * 8;
      if (tr.seg == 0) {
        dma16(vbase, off[i], dst);
      } else {
        const int u = vb * kWave + ln;
        const int d = u / T::VU, c = u % T::VU;
        if (tr.seg == 1) dma16(src.mvt, 16u * (uint32_t)d, dst);
        else dma16(src.rvt + tr.base, 2u * (uint32_t)(d * a.r_pad + (c < T::VC ? c : 0) * 8), dst);
      }
    }
  }
}

// The same for a cache tile (the common case), without the per-load segment
// branches: each of this wavefront's loads is a K or a V^T unit block,
// chosen by a select on the block index.
// (LDS addresses as plain integers: a select between two shared-memory
// pointers would be redone with null checks for every load.)
template <int D>
__device__ inline void tile_dma_cache(const KvSrc& src, int base, int wave, const uint32_t (&off)[AttnTile<D>::LPW],
                                      uint32_t ks_lds, uint32_t vs_lds) {
  using T = AttnTile<D>;
  if (wave >= T::LOADERS) return;
  const uint16_t* kbase = src.kc + (int64_t)base * D;
  const uint16_t* vbase = src.vc + (int64_t)base * D;
#pragma unroll
  for (int i = 0; i < T::LPW; ++i) {
    const int blk = wave * T::LPW + i;
    const bool is_k = blk < T::K_BLOCKS;
    const uint32_t dst = is_k ? ks_lds + blk * 1024u : vs_lds + (blk - T::K_BLOCKS) * 1024u;
    dma16_at(is_k ? kbase : vbase, off[i], dst);
  }
}

// Wait for tile i of the ring when `younger` later tiles may stay in flight.
// (kAhead tiles are loaded ahead; the lagging wavefronts still read the
// previous tile's buffer, so a 4-deep ring leaves kAhead = 2.)
template <int LPW>
__device__ inline void ring_wait_tiles(int younger) {
  static_assert(kAhead == 2 && kStages >= kAhead + 2, "waits are spelled out for two tiles ahead");
  if (younger >= 2) ring_wait<LPW>();
  else if (younger == 1) ring_wait<LPW>();
  else ring_wait<0>();
}

// Split p into bf16 hi + lo for a pair of values, packed two per word.
struct HiLo {
  uint32_t hi, lo;
};
__device__ inline HiLo split_pair(float p0, float p1) {
  const uint32_t hi = pack_bf16x2(p0, p1);
  const float h0 = __uint_as_float(hi << 16);
  const float h1 = __uint_as_float(hi & 0xffff0000u);
  return HiLo{hi, pack_bf16x2(p0 - h0, p1 - h1)};
}

// The softmax reference m_ref of a row only moves up when the tile maximum
// exceeds it by more than kRescaleLog2 (in log2 units): probabilities are
// computed as exp2(t - m_ref) <= 2^kRescaleLog2, which fp32 accumulation and
// the bf16 hi/lo split handle exactly as well as values <= 1, and the O and l
// rescale is skipped on almost every tile.  The normalisation at the end
// divides by the same l, so the result is the same softmax.
constexpr float kRescaleLog2 = 8.f;

// Full tiles take a cheaper path: the reference is the row maximum over the
// first full tile and is never raised in the loop, so no branch rescales (and
// redefines) the accumulators there, and no row maximum is taken.  After the
// loop a wavefront checks that its row sums stayed below 2^kOverflowLog2
// (then every p did: p <= 2^50 keeps O = sum p v far inside the fp32 range;
// an infinite or NaN sum fails the check too); if one did not, the block
// recomputes everything on the lazy path above.
constexpr float kOverflowLog2 = 50.f;

// max of three floats.  IEEE maximum (NaN-propagating) needs no canonicalising
// moves in front of MFMA results and becomes one v_maximum3_f32; the compiler
// inserts the MFMA-to-VALU wait states itself.  Scores are finite or -1e30
// (masked) unless the inputs hold NaN, which then propagates.
__device__ inline float max3(float a, float b, float c) {
  return __builtin_elementwise_maximum(__builtin_elementwise_maximum(a, b), c);
}

// Combine a value of lane l with lane l ^ 32 (the other half of the row's
// lanes) through v_permlane32_swap: the swap leaves (own, partner) in lanes
// 0-31 and (partner, own) in lanes 32-63, so max/sum of the pair is the same
// commutative operation on every lane.
__device__ inline float halves_max(float x) {
  const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __builtin_elementwise_maximum(__uint_as_float(sw[0]), __uint_as_float(sw[1]));
}
__device__ inline float halves_sum(float x) {
  const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(sw[0]) + __uint_as_float(sw[1]);
}

// Masking and row maximum (log2 units) of one 32-key half for this lane's row.
template <bool kEdge>
__device__ inline float half_max(floatx16& sv, int key_base, int wlen, int half, float sc) {
  if (kEdge) {
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      const int jj = e / 4, ii = e % 4;
      const int key = key_base + 16 * (jj / 2) + 8 * half + 4 * (jj % 2) + ii;
      sv[e] = key < wlen ? sv[e] : kMaskedScore;
    }
  }
  float mt = max3(sv[0], sv[1], sv[2]);
#pragma unroll
  for (int e = 3; e < 15; e += 2) mt = max3(mt, sv[e], sv[e + 1]);
  return halves_max(max3(mt, sv[15], sv[15])) * sc;
}

// Raise the reference to mt (when above it), rescaling O and l.
template <int NDB>
__device__ inline void rescale(floatx16* acc, float& m_ref, float& l_run, float mt) {
  const float m_new = fmaxf(m_ref, mt);
  const float alpha = __builtin_amdgcn_exp2f(m_ref - m_new);
  l_run *= alpha;
#pragma unroll
  for (int db = 0; db < NDB; ++db)
#pragma unroll
    for (int e = 0; e < 16; ++e) acc[db][e] *= alpha;
  m_ref = m_new;
}

// p = exp2(s * sc - m_ref) in place, their sum added to l.
__device__ inline void half_exp(floatx16& sv, float m_ref, float& l_run, float sc) {
  float lsum = 0.f;
#pragma unroll
  for (int e = 0; e < 16; ++e) {
    sv[e] = __builtin_amdgcn_exp2f(fmaf(sv[e], sc, -m_ref));
    lsum += sv[e];
  }
  l_run += lsum;
}

// O^T += V^T (P_hi + P_lo)^T for one 32-key half (two 16-key k-steps).  The
// V^T operands are read from LDS per k-step (vhalf: first unit of this half in
// this lane's V^T rows); the scheduler hoists the reads as far as registers allow.
template <int D, bool kEdge>
__device__ inline void half_pv(const floatx16& p, const uint16_t* vhalf, floatx16* acc, int key_base, int wlen,
                               int half) {
  using T = AttnTile<D>;
  constexpr int NDB = D / 32;
#pragma unroll
  for (int u = 0; u < 2; ++u) {
    if (u > 0) __builtin_amdgcn_sched_barrier(0);   // one k-step's V operands in flight
    typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
    u32x4 hi, lo;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const HiLo w = split_pair(p[8 * u + 2 * q], p[8 * u + 2 * q + 1]);
      hi[q] = w.hi;
      lo[q] = w.lo;
    }
    const bf16x8 phi = __builtin_bit_cast(bf16x8, hi);
    const bf16x8 plo = __builtin_bit_cast(bf16x8, lo);
    bf16x8 v[NDB];
#pragma unroll
    for (int db = 0; db < NDB; ++db) {
      u16x8 raw = *reinterpret_cast<const u16x8*>(vhalf + (32 * db * T::VU + 2 * u) * 8);
      if (kEdge) {
        const int key0 = key_base + 16 * u + 8 * half;
#pragma unroll
        for (int e = 0; e < 8; ++e) raw[e] = (key0 + e < wlen) ? raw[e] : (uint16_t)0;
      }
      v[db] = __builtin_bit_cast(bf16x8, raw);
    }
#pragma unroll
    for (int db = 0; db < NDB; ++db) acc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(v[db], phi, acc[db], 0, 0, 0);
#pragma unroll
    for (int db = 0; db < NDB; ++db) acc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(v[db], plo, acc[db], 0, 0, 0);
  }
}

// S^T for one 32-key half hk of a tile: lane holds keys 16(jj/2) + 8*half +
// 4(jj%2) + ii of the half for row l32 (K rows permuted, see krow).
template <int D>
__device__ inline floatx16 s_half(const uint16_t* kb, const bf16x8* qf, int hk, int krow, int half) {
  using T = AttnTile<D>;
  constexpr int NKS = D / 16;
  const uint16_t* kbase = kb + ((32 * hk + krow) * T::KU + half) * 8;
  floatx16 sv;
#pragma unroll
  for (int e = 0; e < 16; ++e) sv[e] = 0.f;
  // all eight K operands are read before the MFMA chain: read one by one in
  // front of their MFMAs, every MFMA waited a full LDS latency (same-box C3:
  // attention -2 %)
  bf16x8 kf[NKS];
#pragma unroll
  for (int t = 0; t < NKS; ++t) kf[t] = *reinterpret_cast<const bf16x8*>(kbase + (2 * t) * 8);
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int t = 0; t < NKS; ++t) sv = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf[t], qf[t], sv, 0, 0, 0);
  return sv;
}

// Softmax and O += V P for half hk of a tile.  kEdge: only the first `valid`
// keys count (valid < 64; the rest are removed by select).
template <int D, bool kEdge>
__device__ inline void finish_half(floatx16& sv, const uint16_t* vb, int hk, int valid, floatx16* acc,
                                   float& m_ref, float& l_run, int half, int l32, float sc) {
  using T = AttnTile<D>;
  constexpr int NDB = D / 32;
  const uint16_t* vhalf = vb + (l32 * T::VU + half + 4 * hk) * 8;
  // The rare rescale path repeats the exp and PV code, so that no branch
  // merges two definitions of the accumulators in front of the PV MFMAs.
  const float mt = half_max<kEdge>(sv, 32 * hk, valid, half, sc);
  if (__builtin_expect(__any(mt > m_ref + kRescaleLog2), 0)) {
    rescale<NDB>(acc, m_ref, l_run, mt);
    half_exp(sv, m_ref, l_run, sc);
    half_pv<D, kEdge>(sv, vhalf, acc, 32 * hk, valid, half);
  } else {
    half_exp(sv, m_ref, l_run, sc);
    half_pv<D, kEdge>(sv, vhalf, acc, 32 * hk, valid, half);
  }
}

// Softmax and O += V P for half hk of a full tile at a fixed reference.
template <int D>
__device__ inline void finish_half_fixed(floatx16& sv, const uint16_t* vb, int hk, floatx16* acc, float m_ref,
                                         float& l_run, int half, int l32, float sc) {
  using T = AttnTile<D>;
  const uint16_t* vhalf = vb + (l32 * T::VU + half + 4 * hk) * 8;
  half_exp(sv, m_ref, l_run, sc);
  half_pv<D, false>(sv, vhalf, acc, 32 * hk, kKeyTile, half);
}

// Order in which a block streams its tiles [t_lo, t_lo + n): the full tiles in
// key order, then the partial last tiles of the segments (at most three).
// Softmax does not depend on the order; keeping the partial tiles out of the
// main loop keeps that loop free of masking code and of branches that would
// merge accumulator definitions.
// (Scalar members, read by value: an indexed array, or a select between
// member addresses, would put the struct in scratch memory.)
__device__ inline int order_at(int i, int t_lo, int n_full, int e0, int e1, int e2) {
  if (i >= n_full) {
    const int k = i - n_full;
    return k == 0 ? e0 : (k == 1 ? e1 : e2);
  }
  int t = t_lo + i;
  t += t >= e0;
  t += t >= e1;
  t += t >= e2;
  return t;
}
struct TileOrder {
  int t_lo, n, n_full;
  int e0, e1, e2;          // partial tiles in key order; unused ones are INT_MAX
  __device__ inline int at(int i) const { return order_at(i, t_lo, n_full, e0, e1, e2); }
};

// One ring step: wait for tile i (own loads, then the barrier for everyone's)
// and issue the loads of tile i + kAhead.
template <int D>
__device__ inline void ring_step(const AttnArgs& a, const Geometry& g, const KvSrc& src, const TileOrder ord,
                                 int T0, int T1, const uint32_t (&off)[AttnTile<D>::LPW],
                                 uint16_t (*ks)[AttnTile<D>::K_ELEMS], uint16_t (*vs)[AttnTile<D>::V_ELEMS], int i,
                                 int wave, int lane) {
  using T = AttnTile<D>;
  ring_wait_tiles<T::LPW>(ord.n - 1 - i);
  ring_barrier();
  const int nxt = i + kAhead;
  if (nxt < ord.n) {
    const TileRef tr = tile_ref(a, T0, T1, ord.at(nxt));
    if (tr.seg == 0)
      tile_dma_cache<D>(src, tr.base, wave, off, lds_addr(&ks[0][0]) + (nxt % kStages) * (T::K_ELEMS * 2),
                        lds_addr(&vs[0][0]) + (nxt % kStages) * (T::V_ELEMS * 2));
    else tile_dma<D>(a, g, src, tr, wave, lane, off, ks[nxt % kStages], vs[nxt % kStages]);
  }
}

// The tile loop of one wavefront, in three phases over the block's ring steps:
//  1. the full tiles this wavefront's rows see (the first n_comp of the order;
//     for D rows the full cache tiles, which come first), no masking;
//  2. the remaining full tiles: ring steps only (D rows past the cache);
//  3. the partial tiles, masked, when this wavefront's rows see them.
// LAG = false: both halves of tile i in step i.  LAG = true (the second
// wavefront of each SIMD): step i first finishes the second half of tile i-1
// (scores carried in registers, V still in its ring slot), then the first
// half of tile i, and leaves the second half's scores for the next step.  The
// two wavefronts of a SIMD are then in different phases (one in MFMA, the
// other in softmax VALU work) instead of in lockstep after every barrier.
template <int D, bool LAG, bool FAST>
__device__ inline void tile_loop(const AttnArgs& a, const Geometry& g, const KvSrc& src, const TileOrder ord,
                                 const uint32_t (&off)[AttnTile<D>::LPW], uint16_t (*ks)[AttnTile<D>::K_ELEMS],
                                 uint16_t (*vs)[AttnTile<D>::V_ELEMS], const bf16x8* qf, floatx16* acc, float& m_ref,
                                 float& l_run, int T0, int T1, int n_comp, int w_end, bool active, int wave,
                                 int lane, int krow, int half, int l32, float sc, bool& over) {
  if (FAST && n_comp > 0) {
    // first full tile: both halves' scores set the reference
    ring_step<D>(a, g, src, ord, T0, T1, off, ks, vs, 0, wave, lane);
    floatx16 sv = s_half<D>(ks[0], qf, 0, krow, half);
    floatx16 sv1 = s_half<D>(ks[0], qf, 1, krow, half);
    m_ref = fmaxf(half_max<false>(sv, 0, kKeyTile, half, sc), half_max<false>(sv1, 32, kKeyTile, half, sc));
    finish_half_fixed<D>(sv, vs[0], 0, acc, m_ref, l_run, half, l32, sc);
    if (LAG) {
      for (int i = 1; i < n_comp; ++i) {
        ring_step<D>(a, g, src, ord, T0, T1, off, ks, vs, i, wave, lane);
        finish_half_fixed<D>(sv1, vs[(i - 1) % kStages], 1, acc, m_ref, l_run, half, l32, sc);
        const int cur = i % kStages;
        sv = s_half<D>(ks[cur], qf, 0, krow, half);
        finish_half_fixed<D>(sv, vs[cur], 0, acc, m_ref, l_run, half, l32, sc);
        sv1 = s_half<D>(ks[cur], qf, 1, krow, half);
      }
      finish_half_fixed<D>(sv1, vs[(n_comp - 1) % kStages], 1, acc, m_ref, l_run, half, l32, sc);
    } else {
      finish_half_fixed<D>(sv1, vs[0], 1, acc, m_ref, l_run, half, l32, sc);
      for (int i = 1; i < n_comp; ++i) {
        ring_step<D>(a, g, src, ord, T0, T1, off, ks, vs, i, wave, lane);
        const int cur = i % kStages;
        // both halves' scores first: the second half's MFMAs run under the
        // first half's softmax
        sv = s_half<D>(ks[cur], qf, 0, krow, half);
        sv1 = s_half<D>(ks[cur], qf, 1, krow, half);
        finish_half_fixed<D>(sv, vs[cur], 0, acc, m_ref, l_run, half, l32, sc);
        finish_half_fixed<D>(sv1, vs[cur], 1, acc, m_ref, l_run, half, l32, sc);
      }
    }
  }
  // every p of the fast phase is at most this lane's sum (a NaN fails too)
  if (FAST && n_comp > 0) over = !(l_run < 0x1p50f);
  static_assert(kOverflowLog2 == 50.f, "the bound above is 2^kOverflowLog2");
  if (!FAST && n_comp > 0) {
    if (LAG) {
      ring_step<D>(a, g, src, ord, T0, T1, off, ks, vs, 0, wave, lane);
      floatx16 sv = s_half<D>(ks[0], qf, 0, krow, half);
      finish_half<D, false>(sv, vs[0], 0, kKeyTile, acc, m_ref, l_run, half, l32, sc);
      floatx16 sv_carry = s_half<D>(ks[0], qf, 1, krow, half);
      for (int i = 1; i < n_comp; ++i) {
        ring_step<D>(a, g, src, ord, T0, T1, off, ks, vs, i, wave, lane);
        finish_half<D, false>(sv_carry, vs[(i - 1) % kStages], 1, kKeyTile, acc, m_ref, l_run, half, l32, sc);
        const int cur = i % kStages;
        sv = s_half<D>(ks[cur], qf, 0, krow, half);
        finish_half<D, false>(sv, vs[cur], 0, kKeyTile, acc, m_ref, l_run, half, l32, sc);
        sv_carry = s_half<D>(ks[cur], qf, 1, krow, half);
      }
      finish_half<D, false>(sv_carry, vs[(n_comp - 1) % kStages], 1, kKeyTile, acc, m_ref, l_run, half, l32, sc);
    } else {
      for (int i = 0; i < n_comp; ++i) {
        ring_step<D>(a, g, src, ord, T0, T1, off, ks, vs, i, wave, lane);
        const int cur = i % kStages;
        floatx16 sv = s_half<D>(ks[cur], qf, 0, krow, half);
        finish_half<D, false>(sv, vs[cur], 0, kKeyTile, acc, m_ref, l_run, half, l32, sc);
        sv = s_half<D>(ks[cur], qf, 1, krow, half);
        finish_half<D, false>(sv, vs[cur], 1, kKeyTile, acc, m_ref, l_run, half, l32, sc);
      }
    }
  }
  for (int i = max(n_comp, 0); i < ord.n_full; ++i) ring_step<D>(a, g, src, ord, T0, T1, off, ks, vs, i, wave, lane);
  for (int i = ord.n_full; i < ord.n; ++i) {
    ring_step<D>(a, g, src, ord, T0, T1, off, ks, vs, i, wave, lane);
    const int t = ord.at(i);
    if (!active || t >= w_end) continue;
    const int valid = tile_ref(a, T0, T1, t).valid;
    const int cur = i % kStages;
    floatx16 sv = s_half<D>(ks[cur], qf, 0, krow, half);
    finish_half<D, true>(sv, vs[cur], 0, valid, acc, m_ref, l_run, half, l32, sc);
    sv = s_half<D>(ks[cur], qf, 1, krow, half);
    finish_half<D, true>(sv, vs[cur], 1, valid, acc, m_ref, l_run, half, l32, sc);
  }
}

// Quarter role (blocks of five chunks): wavefronts 4-7 share the fifth chunk,
// wavefront 4 + q taking key half (q & 1) of the tiles of parity (q >> 1), so
// that each SIMD carries 1.25 chunks instead of one SIMD carrying two.  Phases
// as in tile_loop; the first half-tile computed sets the fixed reference.  The
// four partial states are merged at the end of the kernel.
template <int D, bool FAST>
__device__ inline void tile_loop_quarter(const AttnArgs& a, const Geometry& g, const KvSrc& src, const TileOrder ord,
                                         const uint32_t (&off)[AttnTile<D>::LPW],
                                         uint16_t (*ks)[AttnTile<D>::K_ELEMS], uint16_t (*vs)[AttnTile<D>::V_ELEMS],
                                         const bf16x8* qf, floatx16* acc, float& m_ref, float& l_run, int T0, int T1,
                                         int n_comp, int w_end, bool active, int q, int wave, int lane, int krow,
                                         int half, int l32, float sc, bool& over) {
  const int tp = q >> 1, hf = q & 1;
  if (FAST && n_comp > 0) {
    // A half-tile's scores are computed in its own ring step and its softmax
    // and PV in the next one (its V stays in its ring slot: kStages >= kAhead
    // + 2), so that every step gives each SIMD part of the fifth chunk (done
    // in one step, the two SIMDs of that parity carried it alone and the
    // others waited at the barrier: same-box C3, attention -2 %).
    bool have_ref = false;
    floatx16 sv;
    int pend = -1;                        // ring slot of the half-tile whose scores are in sv
    for (int i = 0; i < n_comp; ++i) {
      ring_step<D>(a, g, src, ord, T0, T1, off, ks, vs, i, wave, lane);
      if (pend >= 0) {
        finish_half_fixed<D>(sv, vs[pend], hf, acc, m_ref, l_run, half, l32, sc);
        pend = -1;
      }
      if ((i & 1) != tp) continue;
      const int cur = i % kStages;
      sv = s_half<D>(ks[cur], qf, hf, krow, half);
      if (!have_ref) {
        m_ref = half_max<false>(sv, 32 * hf, kKeyTile, half, sc);
        have_ref = true;
      }
      pend = cur;
    }
    if (pend >= 0) finish_half_fixed<D>(sv, vs[pend], hf, acc, m_ref, l_run, half, l32, sc);
    over = !(l_run < 0x1p50f);
  }
  if (!FAST && n_comp > 0) {
    for (int i = 0; i < n_comp; ++i) {
      ring_step<D>(a, g, src, ord, T0, T1, off, ks, vs, i, wave, lane);
      if ((i & 1) != tp) continue;
      const int cur = i % kStages;
      floatx16 sv = s_half<D>(ks[cur], qf, hf, krow, half);
      finish_half<D, false>(sv, vs[cur], hf, kKeyTile, acc, m_ref, l_run, half, l32, sc);
    }
  }
  for (int i = max(n_comp, 0); i < ord.n_full; ++i) ring_step<D>(a, g, src, ord, T0, T1, off, ks, vs, i, wave, lane);
  for (int i = ord.n_full; i < ord.n; ++i) {
    ring_step<D>(a, g, src, ord, T0, T1, off, ks, vs, i, wave, lane);
    const int t = ord.at(i);
    if (!active || t >= w_end || (i & 1) != tp) continue;
    const int valid = tile_ref(a, T0, T1, t).valid;
    const int cur = i % kStages;
    floatx16 sv = s_half<D>(ks[cur], qf, hf, krow, half);
    finish_half<D, true>(sv, vs[cur], hf, valid, acc, m_ref, l_run, half, l32, sc);
  }
}

// The result of a wavefront: O = acc / l for its rows, or (key split) the
// unscaled partial (O, reference, row sum) that k_attn_combine merges.
// bf16 copies of four consecutive output features (from column col) of query
// row `row` of sequence b for the logits, when it is a C row: hi = the value
// rounded to bf16, lo = the remainder rounded to bf16.
__device__ inline void pack_store4(const AttnArgs& a, const Geometry& g, int b, int row, int col, const floatx4& x) {
  const int c = row - a.n_d;
  if (!a.pack_hi || c < 0 || c >= a.n_c) return;
  const int64_t off = ((int64_t)b * a.n_c + c) * g.hidden + col;
  uint16_t hb[4], lb[4];
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    hb[e] = f32_to_bf16(x[e]);
    lb[e] = f32_to_bf16(x[e] - bf16_to_f32(hb[e]));
  }
  *reinterpret_cast<uint2*>(a.pack_hi + off) =
      uint2{(uint32_t)hb[0] | ((uint32_t)hb[1] << 16), (uint32_t)hb[2] | ((uint32_t)hb[3] << 16)};
  if (a.pack_lo)
    *reinterpret_cast<uint2*>(a.pack_lo + off) =
        uint2{(uint32_t)lb[0] | ((uint32_t)lb[1] << 16), (uint32_t)lb[2] | ((uint32_t)lb[3] << 16)};
}

template <int D>
__device__ inline void write_result(const AttnArgs& a, const Geometry& g, const ChunkPlan& cp, const floatx16* acc,
                                    float m_ref, float l_run, int b, int row, int h, bool rvalid, bool active,
                                    int logical, int wave, int half, int l32) {
  constexpr int NDB = D / 32;
  const float l_tot = halves_sum(l_run);
  const int n_q = a.n_d + a.n_c + a.n_r;
  float* o = a.out + ((int64_t)b * n_q + row) * g.hidden + h * D;
  if (cp.ksplit == 1) {
    if (rvalid) {
      const float inv = 1.f / l_tot;
#pragma unroll
      for (int db = 0; db < NDB; ++db)
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) {
          floatx4 v;
#pragma unroll
          for (int ii = 0; ii < 4; ++ii) v[ii] = acc[db][4 * jj + ii] * inv;
          *reinterpret_cast<floatx4*>(o + 32 * db + 8 * jj + 4 * half) = v;
          pack_store4(a, g, b, row, h * D + 32 * db + 8 * jj + 4 * half, v);
        }
    }
    return;
  }

  // split: publish this block's unscaled partial
  if (!active) return;
  float* po = a.part_o + ((int64_t)logical * kAttnWaves + wave) * 32 * D + l32 * D;
#pragma unroll
  for (int db = 0; db < NDB; ++db)
#pragma unroll
    for (int jj = 0; jj < 4; ++jj) {
      floatx4 v;
#pragma unroll
      for (int ii = 0; ii < 4; ++ii) v[ii] = acc[db][4 * jj + ii];
      *reinterpret_cast<floatx4*>(po + 32 * db + 8 * jj + 4 * half) = v;
    }
  if (half == 0) {
    float* pml = a.part_ml + ((int64_t)logical * kAttnWaves + wave) * 64;
    pml[2 * l32] = m_ref;
    pml[2 * l32 + 1] = l_tot;
  }
}


// Pair mode (chunk groups of four): wavefronts w and w + 4 own the same chunk
// and take the even and the odd tiles of the block's order (parity p = w / 4).
// A ring step covers two tiles, so the two wavefronts of a SIMD compute at the
// same time (one in MFMA while the other is in softmax) instead of four
// wavefronts doing all the work while four only load.  Phases per wavefront:
//  A. pairs of full tiles it computes (fixed reference in the fast pass, the
//     first one peeled to set it; no masking, no branch on the accumulators);
//  B. pairs of full tiles it does not compute (ring steps only);
//  C. the remaining tiles (an odd last full tile and the partial tiles), on
//     the lazily rescaled path.
// The two partial softmax states of a chunk are merged through LDS at the end.
template <int D, bool FAST>
__device__ inline void tile_loop_pair(const AttnArgs& a, const Geometry& g, const KvSrc& src, const TileOrder ord,
                                      const uint32_t (&off)[AttnTile<D>::LPW], uint16_t (*ks)[AttnTile<D>::K_ELEMS],
                                      uint16_t (*vs)[AttnTile<D>::V_ELEMS], const bf16x8* qf, floatx16* acc,
                                      float& m_ref, float& l_run, int T0, int T1, int n_comp, int w_end, bool active,
                                      int parity, int wave, int lane, int krow, int half, int l32, float sc,
                                      bool& over) {
  const int nf2 = ord.n_full / 2;                        // pairs made of two full tiles
  const int c_a = min(nf2, (n_comp - parity + 1) / 2);   // pairs whose tile 2j + p this wavefront computes
  auto pair_ring = [&](int j) {
    ring_step<D>(a, g, src, ord, T0, T1, off, ks, vs, 2 * j, wave, lane);
    if (2 * j + 1 < ord.n) ring_step<D>(a, g, src, ord, T0, T1, off, ks, vs, 2 * j + 1, wave, lane);
  };
  int j = 0;
  if (FAST && c_a > 0) {
    pair_ring(0);
    const int cur = parity % kStages;
    floatx16 sv = s_half<D>(ks[cur], qf, 0, krow, half);
    floatx16 sv1 = s_half<D>(ks[cur], qf, 1, krow, half);
    m_ref = fmaxf(half_max<false>(sv, 0, kKeyTile, half, sc), half_max<false>(sv1, 32, kKeyTile, half, sc));
    finish_half_fixed<D>(sv, vs[cur], 0, acc, m_ref, l_run, half, l32, sc);
    finish_half_fixed<D>(sv1, vs[cur], 1, acc, m_ref, l_run, half, l32, sc);
    for (j = 1; j < c_a; ++j) {
      pair_ring(j);
      const int c = (2 * j + parity) % kStages;
      sv = s_half<D>(ks[c], qf, 0, krow, half);
      sv1 = s_half<D>(ks[c], qf, 1, krow, half);
      finish_half_fixed<D>(sv, vs[c], 0, acc, m_ref, l_run, half, l32, sc);
      finish_half_fixed<D>(sv1, vs[c], 1, acc, m_ref, l_run, half, l32, sc);
    }
    over = !(l_run < 0x1p50f);
  }
  if (!FAST) {
    for (; j < c_a; ++j) {
      pair_ring(j);
      const int c = (2 * j + parity) % kStages;
      floatx16 sv = s_half<D>(ks[c], qf, 0, krow, half);
      finish_half<D, false>(sv, vs[c], 0, kKeyTile, acc, m_ref, l_run, half, l32, sc);
      sv = s_half<D>(ks[c], qf, 1, krow, half);
      finish_half<D, false>(sv, vs[c], 1, kKeyTile, acc, m_ref, l_run, half, l32, sc);
    }
  }
  for (j = max(c_a, 0); j < nf2; ++j) pair_ring(j);
  for (j = nf2; 2 * j < ord.n; ++j) {
    pair_ring(j);
    const int i = 2 * j + parity;
    if (i >= ord.n || !active) continue;
    // one compute path (a branch between two would merge accumulator
    // definitions): an odd last full tile takes the masked path with all keys valid
    const int t = ord.at(i);
    const bool full = i < ord.n_full;
    if (full ? i >= n_comp : t >= w_end) continue;
    const int valid = full ? kKeyTile : tile_ref(a, T0, T1, t).valid;
    const int c = i % kStages;
    floatx16 sv = s_half<D>(ks[c], qf, 0, krow, half);
    finish_half<D, true>(sv, vs[c], 0, valid, acc, m_ref, l_run, half, l32, sc);
    sv = s_half<D>(ks[c], qf, 1, krow, half);
    finish_half<D, true>(sv, vs[c], 1, valid, acc, m_ref, l_run, half, l32, sc);
  }
  if (FAST) over = over || !(l_run < 0x1p50f);
}

// Block: kAttnWaves wavefronts, each owning one 32-row chunk of one query head;
// the chunks of a block belong to query heads of one key/value head, so a
// K/V tile in LDS feeds every chunk of the block.  Tiles stream through a
// kStages-deep LDS-DMA ring: while tile i is computed, tiles i+1 .. i+kStages-2
// are in flight.  Each wavefront waits only for its own loads of tile i
// (vmcnt counts the younger tiles' loads it may leave outstanding), then the
// barrier makes every wavefront's part of tile i visible.
// Merge of the four quarter states of the fifth chunk (wavefronts 4-7) into
// wavefront 4 through LDS (mrg: the free K ring), states added in wavefront
// order; every quarter wavefront leaves with the group's overflow flag (the
// four hold the same rows, so they recompute together or not at all).  Called
// by every wavefront of the block (two barriers).
template <int D>
__device__ inline void quad_merge(float* mrg, floatx16* acc, float& m_ref, float& l_run, bool& over, bool quarter,
                                  int wave, int lane) {
  constexpr int NDB = D / 32, QW = kAttnWaves / 2, SZ = 16 * NDB + 3;
  __syncthreads();
  if (quarter) {
    float* dst = mrg + (int64_t)(wave - QW) * SZ * kWave + lane;
    if (wave > QW) {
#pragma unroll
      for (int db = 0; db < NDB; ++db)
#pragma unroll
        for (int e = 0; e < 16; ++e) dst[(16 * db + e) * kWave] = acc[db][e];
      dst[(16 * NDB) * kWave] = m_ref;
      dst[(16 * NDB + 1) * kWave] = l_run;
    }
    dst[(16 * NDB + 2) * kWave] = over ? 1.f : 0.f;
  }
  __syncthreads();
  if (quarter) {
    bool any = false;
#pragma unroll
    for (int j = 0; j < 4; ++j) any |= mrg[((int64_t)j * SZ + 16 * NDB + 2) * kWave + lane] != 0.f;
    over = any;
    if (wave == QW) {
      float m_new = m_ref;
#pragma unroll
      for (int j = 1; j < 4; ++j) m_new = fmaxf(m_new, mrg[((int64_t)j * SZ + 16 * NDB) * kWave + lane]);
      const float a0 = __builtin_amdgcn_exp2f(m_ref - m_new);
#pragma unroll
      for (int db = 0; db < NDB; ++db)
#pragma unroll
        for (int e = 0; e < 16; ++e) acc[db][e] *= a0;
      l_run *= a0;
#pragma unroll
      for (int j = 1; j < 4; ++j) {
        const float* srcm = mrg + (int64_t)j * SZ * kWave + lane;
        const float aj = __builtin_amdgcn_exp2f(srcm[(16 * NDB) * kWave] - m_new);
#pragma unroll
        for (int db = 0; db < NDB; ++db)
#pragma unroll
          for (int e = 0; e < 16; ++e) acc[db][e] += srcm[(16 * db + e) * kWave] * aj;
        l_run += srcm[(16 * NDB + 1) * kWave] * aj;
      }
      m_ref = m_new;
    }
  }
}

template <int D, bool PAIR, bool QUAD>
__global__ __launch_bounds__(kAttnThreads, 1) void k_attn_bf16(Geometry g, AttnArgs a, ChunkPlan cp) {
  using T = AttnTile<D>;
  constexpr int NKS = D / 16;           // k-steps of the QK^T product
  constexpr int NDB = D / 32;           // 32-row blocks of O^T
  __shared__ __align__(1024) uint16_t ks[kStages][T::K_ELEMS];
  __shared__ __align__(1024) uint16_t vs[kStages][T::V_ELEMS];
  static_assert(!QUAD || 4 * (16 * NDB + 3) * kWave * sizeof(float) <= sizeof(ks), "quarter merge exceeds the K ring");
  __shared__ int kidx[kAttnMaxDecode];

  const int n_grid = gridDim.x;
  const int logical = (blockIdx.x % 8) * (n_grid / 8) + blockIdx.x / 8;
  if (logical >= cp.real_blocks) return;
  const int G = g.H / g.Hkv;
  const int split = logical % cp.ksplit;
  const int group = logical / cp.ksplit;
  const int j = group % cp.blocks;
  const int bk = group / cp.blocks;
  const int kvh = bk % g.Hkv;
  const int b = bk / g.Hkv;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  const int lane = threadIdx.x % kWave;
  const int half = lane / 32;
  const int l32 = lane % 32;

  // chunks [c0, c1) of this (sequence, kv head): chunk c is head c / n_chunks
  // of the group, local chunk c % n_chunks
  const int c0 = j * cp.per_block;
  const int c1 = min(G * cp.n_chunks, c0 + cp.per_block);
  bool any_cr = false;
  for (int c = c0; c < c1; ++c) any_cr |= (c % cp.n_chunks) >= cp.chunks_d;
  const int parity = PAIR ? wave / (kAttnWaves / 2) : 0;
  // QUAD (blocks of five chunks): wavefronts 4-7 share the fifth chunk
  const bool quarter = QUAD && wave >= kAttnWaves / 2;
  const int ch = c0 + (PAIR ? wave % (kAttnWaves / 2) : (quarter ? kAttnWaves / 2 : wave));
  const bool active = ch < c1;
  const int h = kvh * G + (active ? ch / cp.n_chunks : 0);
  int row_base = 0, row_end = 0;
  bool is_cr = false;
  if (active) chunk_rows(a, cp, 32, ch % cp.n_chunks, row_base, row_end, is_cr);
  const int row = row_base + l32;
  const bool rvalid = active && row < row_end;

  // this block's tiles [t_lo, t_hi) of the segmented key range
  const int T0 = (a.S + kKeyTile - 1) / kKeyTile;
  const int T1 = (a.n_c + kKeyTile - 1) / kKeyTile;
  const int T2 = (a.n_r + kKeyTile - 1) / kKeyTile;
  const int kend = any_cr ? T0 + T1 + T2 : T0;
  const int tps = (kend + cp.ksplit - 1) / cp.ksplit;
  const int t_lo = min(kend, split * tps);
  const int n_my = min(kend, t_lo + tps) - t_lo;
  const int w_end = is_cr ? T0 + T1 + T2 : T0;       // tiles this wavefront's rows see

  // key-table rows of the C keys, if this block streams any C tile
  if (T1 > 0 && t_lo < T0 + T1 && t_lo + n_my > T0) {
    for (int jj = threadIdx.x; jj < a.n_c; jj += kAttnThreads) {
      int pos = a.c_pos[(int64_t)b * a.c_stride + jj];
      if (pos < 0 || pos >= g.seq_len) { flag_error(a.err, kErrPos); pos = 0; }
      kidx[jj] = pos;
    }
  }
  __syncthreads();

  KvSrc src;
  src.kc = static_cast<const uint16_t*>(a.kc) + ((int64_t)b * g.Hkv + kvh) * g.slots * D;
  src.vc = static_cast<const uint16_t*>(a.vc) + ((int64_t)b * g.Hkv + kvh) * D * g.slots;
  src.ktab = static_cast<const uint16_t*>(a.ktab) + (int64_t)kvh * a.ktab_rows * D;
  src.mvt = static_cast<const uint16_t*>(a.mvt) + (int64_t)kvh * D * 8;
  src.rvt = static_cast<const uint16_t*>(a.rvt) + (int64_t)kvh * D * a.r_pad;
  src.kidx = kidx;
  src.k2row0 = g.seq_len;
  if (a.tk) {
    // upper layer: the C|R keys of this step, per (sequence, kv head)
    src.ktab = static_cast<const uint16_t*>(a.tk) + ((int64_t)b * g.Hkv + kvh) * a.t_pad * D;
    src.rvt = static_cast<const uint16_t*>(a.tvt) + ((int64_t)b * g.Hkv + kvh) * D * a.t_pad;
    src.k2row0 = 0;
  }

  // stream order: full tiles, then the segments' partial last tiles
  TileOrder ord;
  ord.t_lo = t_lo;
  ord.n = n_my;
  {
    constexpr int kNone = 0x7fffffff;
    const int c0e = (a.S % kKeyTile) ? T0 - 1 : -1;
    const int c1e = (a.n_c % kKeyTile) ? T0 + T1 - 1 : -1;
    const int c2e = (a.n_r % kKeyTile) ? T0 + T1 + T2 - 1 : -1;
    const bool in0 = c0e >= t_lo && c0e < t_lo + n_my;
    const bool in1 = c1e >= t_lo && c1e < t_lo + n_my;
    const bool in2 = c2e >= t_lo && c2e < t_lo + n_my;
    // compact the present ones, in key order
    const int f0 = in0 ? c0e : (in1 ? c1e : (in2 ? c2e : kNone));
    const int f1 = in0 ? (in1 ? c1e : (in2 ? c2e : kNone)) : (in1 && in2 ? c2e : kNone);
    const int f2 = in0 && in1 && in2 ? c2e : kNone;
    ord.e0 = f0;
    ord.e1 = f1;
    ord.e2 = f2;
    ord.n_full = n_my - (int)in0 - (int)in1 - (int)in2;
  }
  // full tiles this wavefront computes: all of them for C|R rows, the full
  // cache tiles (a prefix of the order) for D rows
  int n_comp = 0;
  if (active) {
    if (is_cr) {
      n_comp = ord.n_full;
    } else {
      const bool cache_edge = (a.S % kKeyTile) && T0 - 1 >= t_lo && T0 - 1 < t_lo + n_my;
      n_comp = max(0, min(t_lo + n_my, T0) - t_lo - (cache_edge ? 1 : 0));
    }
  }

  // Q^T fragment (B operand): lane holds row l32, dims 16t + 8*half + 0..7, RoPE'd.
  // C and R rows read the query table (the mask token at the row's position,
  // the registers); D rows read the queries their append wrote, or, if the
  // append did not write them, rotate their table row here.  Loaded before
  // the first tiles are requested: the compiler's wait for the C rows'
  // positions counts only its own loads, so issued after the tile loads it
  // would also wait for those.
  bf16x8 qf[NKS];
  {
    const uint16_t* qrow = nullptr;
    bool rotate = false;
    RowInfo ri = {0, 0};
    if (rvalid) {
      if (row < a.n_d && !a.qbuf) {
        rotate = true;
        ri = query_row(g, a, b, row);
      } else if (row < a.n_d || a.tk) {
        qrow = static_cast<const uint16_t*>(a.qbuf) + (((int64_t)b * g.H + h) * a.qbuf_rows + row) * D;
      } else {
        int pos;
        if (row < a.n_d + a.n_c) {
          pos = a.c_pos[(int64_t)b * a.c_stride + (row - a.n_d)];
          if (pos < 0 || pos >= g.seq_len) { flag_error(a.err, kErrPos); pos = 0; }
        } else {
          pos = g.seq_len + (row - a.n_d - a.n_c);
        }
        qrow = static_cast<const uint16_t*>(a.qtab) + ((int64_t)h * a.qtab_rows + pos) * D;
      }
    }
    if (rotate) {
      const uint16_t* tq = static_cast<const uint16_t*>(a.tq) + (int64_t)ri.id * g.hidden + h * D;
      const float* cs = a.rope_cos + (int64_t)ri.pos * (D / 2);
      const float* sn = a.rope_sin + (int64_t)ri.pos * (D / 2);
#pragma unroll
      for (int t = 0; t < NKS; ++t) {
        const u16x8 raw = *reinterpret_cast<const u16x8*>(tq + 16 * t + 8 * half);
        u16x8 rot;
#pragma unroll
        for (int p = 0; p < 4; ++p) {
          const int pi = 8 * t + 4 * half + p;
          double r0, r1;
          rope_pair(bf16_to_f32(raw[2 * p]), bf16_to_f32(raw[2 * p + 1]), cs[pi], sn[pi], r0, r1);
          rot[2 * p] = f64_to_bf16(r0);
          rot[2 * p + 1] = f64_to_bf16(r1);
        }
        qf[t] = __builtin_bit_cast(bf16x8, rot);
      }
    } else {
#pragma unroll
      for (int t = 0; t < NKS; ++t) {
        u16x8 raw = {0, 0, 0, 0, 0, 0, 0, 0};
        if (qrow) raw = *reinterpret_cast<const u16x8*>(qrow + 16 * t + 8 * half);
        qf[t] = __builtin_bit_cast(bf16x8, raw);
      }
    }
  }

  uint32_t off[T::LPW];
  dma_offsets<D>(wave, lane, off);
  for (int i = 0; i < kAhead && i < n_my; ++i)
    tile_dma<D>(a, g, src, tile_ref(a, T0, T1, ord.at(i)), wave, lane, off, ks[i], vs[i]);

  // Key row of the K operand for this lane within a 32-key sub-tile: output
  // row r = 8jj + 4hh + ii maps to key 16(jj/2) + 8hh + 4(jj%2) + ii.
  const int rj = l32 / 8, rh = (l32 / 4) % 2, ri4 = l32 % 4;
  const int krow = 16 * (rj / 2) + 8 * rh + 4 * (rj % 2) + ri4;

  floatx16 acc[NDB];
#pragma unroll
  for (int db = 0; db < NDB; ++db)
#pragma unroll
    for (int e = 0; e < 16; ++e) acc[db][e] = 0.f;
  float m_ref = -1e30f, l_run = 0.f;     // softmax reference (log2 units) and row sum
  const float sc = kLog2e / sqrtf((float)D);

  // Wavefronts 0-3 take a tile's halves in order within the iteration;
  // wavefronts 4-7 (the second wavefront of each SIMD) run half a tile
  // behind (see tile_loop).
  bool over = false;
  if constexpr (PAIR)
    tile_loop_pair<D, true>(a, g, src, ord, off, ks, vs, qf, acc, m_ref, l_run, T0, T1, n_comp, w_end, active, parity,
                            wave, lane, krow, half, l32, sc, over);
  else if (quarter)
    tile_loop_quarter<D, true>(a, g, src, ord, off, ks, vs, qf, acc, m_ref, l_run, T0, T1, n_comp, w_end, active,
                               wave - kAttnWaves / 2, wave, lane, krow, half, l32, sc, over);
  else if (!QUAD && wave >= kAttnWaves / 2)
    tile_loop<D, true, true>(a, g, src, ord, off, ks, vs, qf, acc, m_ref, l_run, T0, T1, n_comp, w_end, active, wave,
                             lane, krow, half, l32, sc, over);
  else
    tile_loop<D, false, true>(a, g, src, ord, off, ks, vs, qf, acc, m_ref, l_run, T0, T1, n_comp, w_end, active,
                              wave, lane, krow, half, l32, sc, over);
  // the quarter states merge now, so that the vote below needs no state kept
  // across a second pass
  float* const mrg = reinterpret_cast<float*>(&ks[0][0]);
  const bool merged_away = quarter && wave > kAttnWaves / 2;    // state now in wavefront 4
  if constexpr (QUAD) quad_merge<D>(mrg, acc, m_ref, l_run, over, quarter, wave, lane);
  // A score far above its row's first-tile maximum somewhere in the block:
  // stream the tiles again on the lazily rescaled path.
  // Only the wavefronts whose own rows failed the check recompute (the others
  // keep their result and take the ring steps only), so a row's result never
  // depends on the keys other rows see.
  const bool redo = __any(over);
  bool written = false;
  if (__syncthreads_or(over ? 1 : 0)) {
    if constexpr (PAIR) {
      // (selects, not a branch: a branch would merge two definitions of the
      // accumulators); the pair's states merge below, so nothing is written yet
#pragma unroll
      for (int db = 0; db < NDB; ++db)
#pragma unroll
        for (int e = 0; e < 16; ++e) acc[db][e] = redo ? 0.f : acc[db][e];
      m_ref = redo ? -1e30f : m_ref;
      l_run = redo ? 0.f : l_run;
    } else {
      // the wavefronts that keep their result write it now, so that no
      // accumulator stays live across the second pass
      if (!redo && !merged_away) {
        write_result<D>(a, g, cp, acc, m_ref, l_run, b, row, h, rvalid, active, logical, wave, half, l32);
        written = true;
      }
#pragma unroll
      for (int db = 0; db < NDB; ++db)
#pragma unroll
        for (int e = 0; e < 16; ++e) acc[db][e] = 0.f;
      m_ref = -1e30f;
      l_run = 0.f;
    }
    for (int i = 0; i < kAhead && i < n_my; ++i)
      tile_dma<D>(a, g, src, tile_ref(a, T0, T1, ord.at(i)), wave, lane, off, ks[i], vs[i]);
    const int n_redo = redo ? n_comp : 0;
    const bool act_redo = active && redo;
    bool unused = false;
    if constexpr (PAIR)
      tile_loop_pair<D, false>(a, g, src, ord, off, ks, vs, qf, acc, m_ref, l_run, T0, T1, n_redo, w_end, act_redo,
                               parity, wave, lane, krow, half, l32, sc, unused);
    else if (quarter)
      tile_loop_quarter<D, false>(a, g, src, ord, off, ks, vs, qf, acc, m_ref, l_run, T0, T1, n_redo, w_end,
                                  act_redo, wave - kAttnWaves / 2, wave, lane, krow, half, l32, sc, unused);
    else if (!QUAD && wave >= kAttnWaves / 2)
      tile_loop<D, true, false>(a, g, src, ord, off, ks, vs, qf, acc, m_ref, l_run, T0, T1, n_redo, w_end, act_redo,
                                wave, lane, krow, half, l32, sc, unused);
    else
      tile_loop<D, false, false>(a, g, src, ord, off, ks, vs, qf, acc, m_ref, l_run, T0, T1, n_redo, w_end,
                                 act_redo, wave, lane, krow, half, l32, sc, unused);
    if constexpr (QUAD) quad_merge<D>(mrg, acc, m_ref, l_run, unused, quarter, wave, lane);
  }

  if constexpr (PAIR) {
    // merge the odd-tile state of wavefront w + 4 into wavefront w (the ring is
    // free: every wavefront has passed its last ring step)
    constexpr int PW = kAttnWaves / 2;
    float* mrg = reinterpret_cast<float*>(&ks[0][0]);         // [PW][16 NDB + 2][64]
    __syncthreads();
    if (parity == 1) {
      float* dst = mrg + (int64_t)(wave - PW) * (16 * NDB + 2) * kWave + lane;
#pragma unroll
      for (int db = 0; db < NDB; ++db)
#pragma unroll
        for (int e = 0; e < 16; ++e) dst[(16 * db + e) * kWave] = acc[db][e];
      dst[(16 * NDB) * kWave] = m_ref;
      dst[(16 * NDB + 1) * kWave] = l_run;
    }
    __syncthreads();
    if (parity == 1) return;
    const float* srcm = mrg + (int64_t)wave * (16 * NDB + 2) * kWave + lane;
    const float m1 = srcm[(16 * NDB) * kWave], l1 = srcm[(16 * NDB + 1) * kWave];
    const float m_new = fmaxf(m_ref, m1);
    const float a0 = __builtin_amdgcn_exp2f(m_ref - m_new), a1 = __builtin_amdgcn_exp2f(m1 - m_new);
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[db][e] = acc[db][e] * a0 + srcm[(16 * db + e) * kWave] * a1;
    l_run = l_run * a0 + l1 * a1;
    m_ref = m_new;
  }
  if (!written && !merged_away)
    write_result<D>(a, g, cp, acc, m_ref, l_run, b, row, h, rvalid, active, logical, wave, half, l32);
}

// Merge of the key-split partials: one 256-thread block per chunk (blockIdx =
// chunk group * 8 + chunk slot); thread: row tid/8, dims [D/8 * (tid%8), +D/8).
// Splits are folded in split order (fixed arithmetic, independent of which
// block ran first): O = sum_s 2^(m_s - M) O_s / sum_s 2^(m_s - M) l_s,
// M = max_s m_s.  KS >= ksplit bounds the unrolled split loop, so that every
// split's loads are in flight together.
constexpr int kCombineThreads = 256;

template <int D, int KS>
__global__ __launch_bounds__(kCombineThreads) void k_attn_combine(Geometry g, AttnArgs a, ChunkPlan cp) {
  constexpr int QD = D / 8;
  const int group = blockIdx.x / kAttnWaves;
  const int wave = blockIdx.x % kAttnWaves;       // chunk slot of the group (the wavefront that wrote it)
  const int G = g.H / g.Hkv;
  const int j = group % cp.blocks;
  const int bk = group / cp.blocks;
  const int kvh = bk % g.Hkv;
  const int b = bk / g.Hkv;
  const int c0 = j * cp.per_block;
  const int c1 = min(G * cp.n_chunks, c0 + cp.per_block);
  const int ch = c0 + wave;
  if (ch >= c1) return;
  const int h = kvh * G + ch / cp.n_chunks;
  int row_base, row_end;
  bool is_cr;
  chunk_rows(a, cp, 32, ch % cp.n_chunks, row_base, row_end, is_cr);
  const int r = threadIdx.x / 8, part = threadIdx.x % 8;
  const int row = row_base + r;
  if (row >= row_end) return;
  const int64_t slot0 = (int64_t)group * cp.ksplit;
  float2 ml[KS];
  floatx4 v[KS][QD / 4];
#pragma unroll
  for (int s = 0; s < KS; ++s) {
    const int64_t slot = (slot0 + (s < cp.ksplit ? s : 0)) * kAttnWaves + wave;
    ml[s] = *reinterpret_cast<const float2*>(a.part_ml + slot * 64 + 2 * r);
    const floatx4* ps = reinterpret_cast<const floatx4*>(a.part_o + slot * 32 * D + r * D + part * QD);
#pragma unroll
    for (int q = 0; q < QD / 4; ++q) v[s][q] = ps[q];
  }
  float mx = -1e30f;
#pragma unroll
  for (int s = 0; s < KS; ++s)
    if (s < cp.ksplit) mx = fmaxf(mx, ml[s].x);
  floatx4 sum[QD / 4];
#pragma unroll
  for (int q = 0; q < QD / 4; ++q) sum[q] = floatx4{0.f, 0.f, 0.f, 0.f};
  float lsum = 0.f;
#pragma unroll
  for (int s = 0; s < KS; ++s) {
    if (s >= cp.ksplit) break;
    const float w = __builtin_amdgcn_exp2f(ml[s].x - mx);
    lsum = fmaf(w, ml[s].y, lsum);
#pragma unroll
    for (int q = 0; q < QD / 4; ++q)
#pragma unroll
      for (int ii = 0; ii < 4; ++ii) sum[q][ii] = fmaf(w, v[s][q][ii], sum[q][ii]);
  }
  const float inv = 1.f / lsum;
  const int n_q = a.n_d + a.n_c + a.n_r;
  floatx4* o = reinterpret_cast<floatx4*>(a.out + ((int64_t)b * n_q + row) * g.hidden + h * D + part * QD);
#pragma unroll
  for (int q = 0; q < QD / 4; ++q) {
    floatx4 x;
#pragma unroll
    for (int ii = 0; ii < 4; ++ii) x[ii] = sum[q][ii] * inv;
    o[q] = x;
    pack_store4(a, g, b, row, h * D + part * QD + 4 * q, x);
  }
}

// ------------------------------------------------------------- fp32 VALU --
// Block: 64 query rows of one kind x 4 threads per row (each a quarter of d).
template <int D>
__global__ __launch_bounds__(256) void k_attn_f32(Geometry g, AttnArgs a, ChunkPlan cp) {
  constexpr int KT = 32;
  constexpr int QD = D / 4;
  __shared__ float ks[KT][D + 1];
  __shared__ float vs[D][KT + 1];

  const int blk = blockIdx.x;
  const int ch = blk % cp.n_chunks;
  const int bh = blk / cp.n_chunks;
  const int h = bh % g.H;
  const int b = bh / g.H;
  const int kvh = h / (g.H / g.Hkv);
  int row_base, row_end;
  bool is_cr;
  chunk_rows(a, cp, 64, ch, row_base, row_end, is_cr);
  const int wlen = is_cr ? a.S + a.n_c + a.n_r : a.S;
  const int t = threadIdx.x;
  const int qpart = t % 4;
  const int row = row_base + t / 4;
  const bool rvalid = row < row_end;

  float q[QD], o[QD];
  {
    RowInfo ri = {0, 0};
    if (rvalid) ri = query_row(g, a, b, row);
    const float* tq = static_cast<const float*>(a.tq) + (int64_t)ri.id * g.hidden + h * D + qpart * QD;
    const float* cs = a.rope_cos + (int64_t)ri.pos * (D / 2) + qpart * (QD / 2);
    const float* sn = a.rope_sin + (int64_t)ri.pos * (D / 2) + qpart * (QD / 2);
#pragma unroll
    for (int p = 0; p < QD / 2; ++p) {
      double r0, r1;
      const float x0 = rvalid ? tq[2 * p] : 0.f, x1 = rvalid ? tq[2 * p + 1] : 0.f;
      rope_pair(x0, x1, cs[p], sn[p], r0, r1);
      q[2 * p] = (float)r0;
      q[2 * p + 1] = (float)r1;
    }
  }
#pragma unroll
  for (int e = 0; e < QD; ++e) o[e] = 0.f;
  float m_run = -1e30f, l_run = 0.f;
  const float sc = kLog2e / sqrtf((float)D);
  const float* kc = static_cast<const float*>(a.kc) + ((int64_t)b * g.Hkv + kvh) * g.slots * D;
  const float* vc = static_cast<const float*>(a.vc) + ((int64_t)b * g.Hkv + kvh) * D * g.slots;
  const float* ktab = static_cast<const float*>(a.ktab) + (int64_t)kvh * a.ktab_rows * D;
  const float* tv = static_cast<const float*>(a.tv);
  const int kvd = g.Hkv * D;
  const int s_tot = a.S + a.n_c + a.n_r;

  for (int kt = 0; kt < wlen; kt += KT) {
    __syncthreads();
    for (int c = t; c < KT * D; c += blockDim.x) {
      const int kr = c / D, dd = c % D;
      const int slot = kt + kr;
      float x = 0.f;
      if (slot < a.S) x = kc[(int64_t)slot * D + dd];
      else if (slot < s_tot) x = ktab[(int64_t)transient_krow(g, a, b, slot - a.S) * D + dd];
      ks[kr][dd] = x;
    }
    for (int c = t; c < D * KT; c += blockDim.x) {
      const int dd = c / KT, kr = c % KT;
      const int slot = kt + kr;
      float v = 0.f;
      if (slot < a.S) v = vc[((int64_t)(slot / kKeyTile) * D + dd) * kKeyTile + slot % kKeyTile];
      else if (slot < min(s_tot, wlen)) v = tv[(int64_t)transient_id(g, a, slot - a.S) * kvd + kvh * D + dd];
      vs[dd][kr] = v;
    }
    __syncthreads();
    float s[KT];
    float mt = kNegInf;
#pragma unroll
    for (int k = 0; k < KT; ++k) {
      float acc = 0.f;
#pragma unroll
      for (int e = 0; e < QD; ++e) acc = fmaf(q[e], ks[k][qpart * QD + e], acc);
      acc += __shfl_xor(acc, 1);
      acc += __shfl_xor(acc, 2);
      s[k] = (kt + k < wlen) ? acc : kNegInf;
      mt = fmaxf(mt, s[k]);
    }
    const float m_new = fmaxf(m_run, mt);
    const float alpha = exp2f((m_run - m_new) * sc);
    float lsum = 0.f;
#pragma unroll
    for (int k = 0; k < KT; ++k) {
      s[k] = exp2f((s[k] - m_new) * sc);
      lsum += s[k];
    }
    l_run = l_run * alpha + lsum;
    m_run = m_new;
#pragma unroll
    for (int e = 0; e < QD; ++e) {
      float acc = o[e] * alpha;
#pragma unroll
      for (int k = 0; k < KT; ++k) acc = fmaf(s[k], vs[qpart * QD + e][k], acc);
      o[e] = acc;
    }
  }
  if (rvalid) {
    const float inv = 1.f / l_run;
    const int n_q = a.n_d + a.n_c + a.n_r;
    float* out = a.out + ((int64_t)b * n_q + row) * g.hidden + h * D + qpart * QD;
#pragma unroll
    for (int e = 0; e < QD; ++e) out[e] = o[e] * inv;
  }
}

}  // namespace

hipError_t launch_attention(const Geometry& g, const AttnArgs& a, hipStream_t s) {
  const int n_cr = a.n_c + a.n_r;
  const int rows_per_chunk = g.fp32 ? 64 : 32;
  ChunkPlan cp{};
  cp.chunks_d = (a.n_d + rows_per_chunk - 1) / rows_per_chunk;
  cp.n_chunks = cp.chunks_d + (n_cr + rows_per_chunk - 1) / rows_per_chunk;
  if (cp.n_chunks == 0) return hipSuccess;
  if (g.fp32) {
    cp.per_block = 1;
    cp.blocks = cp.n_chunks;
    cp.ksplit = 1;
    cp.real_blocks = g.B * g.H * cp.n_chunks;
    dim3 grid(cp.real_blocks);
    if (g.D == 128) hipLaunchKernelGGL((k_attn_f32<128>), grid, dim3(256), 0, s, g, a, cp);
    else hipLaunchKernelGGL((k_attn_f32<64>), grid, dim3(256), 0, s, g, a, cp);
  } else {
    if (a.n_c > kAttnMaxDecode) return hipErrorInvalidValue;
    const int G = g.H / g.Hkv;
    const int space = G * cp.n_chunks;                 // chunks per (sequence, kv head)
    // One wavefront per SIMD (chunk groups of four) when that still fits one
    // block per compute unit: a block's tile time is set by its busiest SIMD,
    // and row groups need no partial results or combine pass.  Otherwise up
    // to eight chunks (two wavefronts per SIMD) share each streamed tile.
    int nb = (space + kAttnWaves - 1) / kAttnWaves;
    const int nb4 = (space + kAttnWaves / 2 - 1) / (kAttnWaves / 2);
    if (g.B * g.Hkv * nb4 <= kAttnSplitBlocks) nb = nb4;
    cp.blocks = nb;
    cp.per_block = (space + nb - 1) / nb;
    cp.pair = cp.per_block <= kAttnWaves / 2 ? 1 : 0;
    const int groups = g.B * g.Hkv * nb;
    // split the key tiles while the groups leave compute units idle, keeping
    // at least kAttnMinSplitTiles tiles per block (4 when the groups fill at
    // most a quarter of the compute units: C2 3.86 -> 3.77 ms per generation,
    // C3 and C5 unchanged, same box)
    const int tiles = (a.S + kKeyTile - 1) / kKeyTile + (a.n_c + kKeyTile - 1) / kKeyTile +
                      (a.n_r + kKeyTile - 1) / kKeyTile;
    int ks = 1;
    if (groups < kAttnSplitBlocks && a.part_o)
      ks = std::max(1, std::min(std::min(kAttnSplitBlocks / groups, kAttnMaxSplit), tiles / (groups <= kAttnSplitBlocks / 4 ? 4 : kAttnMinSplitTiles)));
    cp.ksplit = ks;
    cp.real_blocks = groups * ks;
    dim3 grid((cp.real_blocks + 7) / 8 * 8);
    // blocks of five chunks: the fifth split over wavefronts 4-7 (QUAD)
    const bool quad = !cp.pair && cp.per_block == kAttnWaves / 2 + 1;
    if (cp.pair) {
      if (g.D == 128) hipLaunchKernelGGL((k_attn_bf16<128, true, false>), grid, dim3(kAttnThreads), 0, s, g, a, cp);
      else hipLaunchKernelGGL((k_attn_bf16<64, true, false>), grid, dim3(kAttnThreads), 0, s, g, a, cp);
    } else if (quad) {
      if (g.D == 128) hipLaunchKernelGGL((k_attn_bf16<128, false, true>), grid, dim3(kAttnThreads), 0, s, g, a, cp);
      else hipLaunchKernelGGL((k_attn_bf16<64, false, true>), grid, dim3(kAttnThreads), 0, s, g, a, cp);
    } else {
      if (g.D == 128) hipLaunchKernelGGL((k_attn_bf16<128, false, false>), grid, dim3(kAttnThreads), 0, s, g, a, cp);
      else hipLaunchKernelGGL((k_attn_bf16<64, false, false>), grid, dim3(kAttnThreads), 0, s, g, a, cp);
    }
    if (ks > 1) {
      const dim3 cgrid(groups * kAttnWaves);
#define MDM_COMBINE(KS)                                                                                 \
  if (g.D == 128) hipLaunchKernelGGL((k_attn_combine<128, KS>), cgrid, dim3(kCombineThreads), 0, s, g, a, cp); \
  else hipLaunchKernelGGL((k_attn_combine<64, KS>), cgrid, dim3(kCombineThreads), 0, s, g, a, cp)
      if (ks <= 2) { MDM_COMBINE(2); }
      else if (ks <= 4) { MDM_COMBINE(4); }
      else { MDM_COMBINE(kAttnMaxSplit); }
#undef MDM_COMBINE
    }
  }
  return hipGetLastError();
}

}  // namespace mdm
