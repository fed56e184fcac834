// Step attention under the step-causal mask.
//
// The query set of a step is [D | C | R]: rows entering the cache, the masked
// rows decoded now, the registers (page 1, worked example = the paper's
// Figure 3).  With keys in append order [cache (incl. D) | C | R], D rows see
// the first S keys and C/R rows see all S + n_C + R keys, so the mask is a
// visible prefix whose length depends only on the row kind.  Rows are cut into
// 32-row chunks of a single kind, so every wavefront has one prefix length and
// the mask is a wave-uniform key bound.  Keys past the bound are removed by
// select (scores to -inf, values to 0), never multiplied by zero, so
// invisible slots cannot leak even when they hold NaN.
//
// Keys in slots [0, S) come from the KV cache.  The C and R keys/values are
// never stored in the cache: a C row is the mask token, so its key depends on
// its position only, and a register's key is fixed; both are read from a key
// table built once at init, and their values are rows of the value table.
//
// bf16 path (block = 8 wavefronts = 8 chunks of 32 rows of the query heads of
// one key/value head):
//   K / V^T tiles of 64 keys go from HBM straight into LDS with
//   global_load_lds_dwordx4 (no register staging) through a 4-deep ring, one
//   barrier per tile; LDS rows are padded by 16 bytes so the MFMA operand
//   reads are bank-conflict free with compile-time offsets.
//   S^T = K Q^T with v_mfma_f32_32x32x16_bf16 (Q^T in registers, RoPE'd in the
//   prologue), fp32 online softmax with a lazily raised reference maximum
//   (one partner exchange per tile for the row max), P split into bf16 hi +
//   lo, O^T += V^T P_hi^T + V^T P_lo^T, fp32 out.
//   The key rows of the K operand are permuted so each lane's eight P values
//   of a k-step are eight consecutive keys: the V^T operand is one 16-byte read.
//   Block ids are remapped so that blocks sharing a head's keys/values sit on
//   the same XCD (and L2).
// fp32 path: the same mask with fp32 VALU arithmetic (validation mode).
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
  int blocks;       // blocks per (sequence, head)
  int real_blocks;  // B * H * blocks (the grid may be padded to a multiple of 8)
};

__host__ __device__ inline void chunk_rows(const AttnArgs& a, const ChunkPlan& cp, int rows_per_chunk,
                                           int ch, int& base, int& end, int& len) {
  if (ch < cp.chunks_d) {
    base = ch * rows_per_chunk;
    end = min(base + rows_per_chunk, a.n_d);
    len = a.S;
  } else {
    const int cc = ch - cp.chunks_d;
    base = a.n_d + cc * rows_per_chunk;
    end = min(base + rows_per_chunk, a.n_d + a.n_c + a.n_r);
    len = a.S + a.n_c + a.n_r;
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
  // DMA loads a wavefront issues per tile
  __host__ __device__ static constexpr int loads_of(int wave) { return (BLOCKS - wave + kAttnWaves - 1) / kAttnWaves; }
};

template <int D>
__device__ inline void tile_dma(const uint16_t* kc, const uint16_t* vc, int slots, int kt, uint16_t* ks,
                                uint16_t* vs) {
  using T = AttnTile<D>;
  const int wave = threadIdx.x / kWave, lane = threadIdx.x % kWave;
#pragma unroll
  for (int i = 0; i < (T::BLOCKS + kAttnWaves - 1) / kAttnWaves; ++i) {
    const int blk = wave + kAttnWaves * i;
    if (blk < T::K_BLOCKS) {
      const int u = blk * kWave + lane;
      const int r = u / T::KU, c = u % T::KU;
      const uint16_t* gk = kc + (int64_t)(kt + r) * D + (c < T::KC ? c : 0) * 8;
      dma16(gk, ks + blk * kWave * 8);
    } else if (blk < T::BLOCKS) {
      const int vb = blk - T::K_BLOCKS;
      const int u = vb * kWave + lane;
      const int d = u / T::VU, c = u % T::VU;
      const uint16_t* gv = vc + (int64_t)d * slots + kt + (c < T::VC ? c : 0) * 8;
      dma16(gv, vs + vb * kWave * 8);
    }
  }
}

// A tile reaching past S: cached slots from the cache, transient slots from the
// key table and the value table, slots past S + n_C + R zero.  Same layout.
// Synchronous: its loads complete (and with them every older load) before return.
template <int D>
__device__ inline void tile_edge(const Geometry& g, const AttnArgs& a, int b, int kvh, const uint16_t* kc,
                                 const uint16_t* vc, int kt, uint16_t* ks, uint16_t* vs) {
  using T = AttnTile<D>;
  const uint16_t* ktab = static_cast<const uint16_t*>(a.ktab) + (int64_t)kvh * a.ktab_rows * D;
  const uint16_t* tv = static_cast<const uint16_t*>(a.tv);
  const int kvd = g.Hkv * D;
  const int s_tot = a.S + a.n_c + a.n_r;
  for (int u = threadIdx.x; u < T::K_BLOCKS * kWave; u += kAttnThreads) {
    const int r = u / T::KU, c = u % T::KU;
    const int slot = kt + r;
    u16x8 v = {0, 0, 0, 0, 0, 0, 0, 0};
    if (c < T::KC) {
      if (slot < a.S) {
        v = *reinterpret_cast<const u16x8*>(kc + (int64_t)slot * D + c * 8);
      } else if (slot < s_tot) {
        const int krow = transient_krow(g, a, b, slot - a.S);
        v = *reinterpret_cast<const u16x8*>(ktab + (int64_t)krow * D + c * 8);
      }
    }
    *reinterpret_cast<u16x8*>(ks + u * 8) = v;
  }
  for (int u = threadIdx.x; u < T::V_BLOCKS * kWave; u += kAttnThreads) {
    const int d = u / T::VU, c = u % T::VU;
    u16x8 v = {0, 0, 0, 0, 0, 0, 0, 0};
    if (c < T::VC) {
      const int slot0 = kt + c * 8;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int sl = slot0 + e;
        if (sl < a.S) v[e] = vc[(int64_t)d * g.slots + sl];
        else if (sl < s_tot) v[e] = tv[(int64_t)transient_id(g, a, sl - a.S) * kvd + kvh * D + d];
      }
    }
    *reinterpret_cast<u16x8*>(vs + u * 8) = v;
  }
}

template <int D>
__device__ inline void tile_fill(const Geometry& g, const AttnArgs& a, int b, int kvh, const uint16_t* kc,
                                 const uint16_t* vc, int kt, uint16_t* ks, uint16_t* vs) {
  if (kt + kKeyTile <= a.S) tile_dma<D>(kc, vc, g.slots, kt, ks, vs);
  else tile_edge<D>(g, a, b, kvh, kc, vc, kt, ks, vs);
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

// max of three floats.  IEEE maximum (NaN-propagating) needs no canonicalising
// moves in front of MFMA results and becomes one v_maximum3_f32; the compiler
// inserts the MFMA-to-VALU wait states itself.  Scores are finite or -1e30
// (masked) unless the inputs hold NaN, which then propagates.
__device__ inline float max3(float a, float b, float c) {
  return __builtin_elementwise_maximum(__builtin_elementwise_maximum(a, b), c);
}

// Softmax of one 32-key half for this lane's row: lazily raise the reference
// (rescaling O and l when a row maximum passes it by more than kRescaleLog2),
// then p = exp2(s * sc - m_ref) in place and their sum added to l.
template <int NDB, bool kEdge>
__device__ inline void half_softmax(floatx16& sv, floatx16* acc, float& m_ref, float& l_run, int key_base,
                                    int wlen, int half, float sc) {
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
  mt = max3(mt, sv[15], __shfl_xor(max3(mt, sv[15], sv[15]), 32)) * sc;
  if (__any(mt > m_ref + kRescaleLog2)) {
    const float m_new = fmaxf(m_ref, mt);
    const float alpha = __builtin_amdgcn_exp2f(m_ref - m_new);
    l_run *= alpha;
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[db][e] *= alpha;
    m_ref = m_new;
  }
  float lsum = 0.f;
#pragma unroll
  for (int e = 0; e < 16; ++e) {
    sv[e] = __builtin_amdgcn_exp2f(fmaf(sv[e], sc, -m_ref));
    lsum += sv[e];
  }
  l_run += lsum;
}

// O^T += V^T (P_hi + P_lo)^T for one 32-key half (two 16-key k-steps).
template <int NDB, bool kEdge>
__device__ inline void half_pv(const floatx16& p, const u16x8 (*vf)[NDB], floatx16* acc, int key_base, int wlen,
                               int half) {
#pragma unroll
  for (int u = 0; u < 2; ++u) {
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
      u16x8 raw = vf[u][db];
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

// One 64-key tile for one wavefront (32 query rows), as two 32-key halves
// pipelined so that each half's softmax (VALU) can run while the other half's
// MFMAs execute: S0, S1 issued; softmax(S0) overlaps S1; PV(0) issued;
// softmax(S1) overlaps PV(0); PV(1).  kEdge: keys at or past wlen are
// removed by select.
template <int D, bool kEdge>
__device__ inline void attn_tile(const uint16_t* kb, const uint16_t* vb, const bf16x8* qf, floatx16* acc,
                                 float& m_ref, float& l_run, int kt, int wlen, int krow, int half, int l32,
                                 float sc) {
  using T = AttnTile<D>;
  constexpr int NKS = D / 16;
  constexpr int NDB = D / 32;
  const uint16_t* kbase = kb + (krow * T::KU + half) * 8;
  const uint16_t* vbase = vb + (l32 * T::VU + half) * 8;
  floatx16 s0, s1;
#pragma unroll
  for (int e = 0; e < 16; ++e) { s0[e] = 0.f; s1[e] = 0.f; }
#pragma unroll
  for (int t = 0; t < NKS; ++t) {
    const bf16x8 k0 = *reinterpret_cast<const bf16x8*>(kbase + (2 * t) * 8);
    const bf16x8 k1 = *reinterpret_cast<const bf16x8*>(kbase + (32 * T::KU + 2 * t) * 8);
    s0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(k0, qf[t], s0, 0, 0, 0);
    s1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(k1, qf[t], s1, 0, 0, 0);
  }
  u16x8 vf[2][NDB];
#pragma unroll
  for (int u = 0; u < 2; ++u)
#pragma unroll
    for (int db = 0; db < NDB; ++db)
      vf[u][db] = *reinterpret_cast<const u16x8*>(vbase + (32 * db * T::VU + 2 * u) * 8);
  half_softmax<NDB, kEdge>(s0, acc, m_ref, l_run, kt, wlen, half, sc);
  half_pv<NDB, kEdge>(s0, vf, acc, kt, wlen, half);
#pragma unroll
  for (int u = 0; u < 2; ++u)
#pragma unroll
    for (int db = 0; db < NDB; ++db)
      vf[u][db] = *reinterpret_cast<const u16x8*>(vbase + (32 * db * T::VU + 4 + 2 * u) * 8);
  half_softmax<NDB, kEdge>(s1, acc, m_ref, l_run, kt + 32, wlen, half, sc);
  half_pv<NDB, kEdge>(s1, vf, acc, kt + 32, wlen, half);
}

// Block: kAttnWaves wavefronts, each owning one 32-row chunk of one query head;
// the chunks of a block belong to query heads of one key/value head, so a
// K/V tile in LDS feeds every chunk of the block.  Tiles stream through a
// kStages-deep LDS-DMA ring: while tile i is computed, tiles i+1 .. i+kStages-2
// are in flight.  Each wavefront waits only for its own loads of tile i
// (vmcnt counts the younger tiles' loads it may leave outstanding), then the
// barrier makes every wavefront's part of tile i visible.
template <int D>
__global__ __launch_bounds__(kAttnThreads, 1) void k_attn_bf16(Geometry g, AttnArgs a, ChunkPlan cp) {
  using T = AttnTile<D>;
  constexpr int KT = kKeyTile;
  constexpr int NKS = D / 16;           // k-steps of the QK^T product
  constexpr int NDB = D / 32;           // 32-row blocks of O^T
  __shared__ __align__(1024) uint16_t ks[kStages][T::K_ELEMS];
  __shared__ __align__(1024) uint16_t vs[kStages][T::V_ELEMS];

  const int n_grid = gridDim.x;
  const int logical = (blockIdx.x % 8) * (n_grid / 8) + blockIdx.x / 8;
  if (logical >= cp.real_blocks) return;
  const int G = g.H / g.Hkv;
  const int j = logical % cp.blocks;
  const int bk = logical / cp.blocks;
  const int kvh = bk % g.Hkv;
  const int b = bk / g.Hkv;
  const int wave = threadIdx.x / kWave;
  const int lane = threadIdx.x % kWave;
  const int half = lane / 32;
  const int l32 = lane % 32;

  // chunks [c0, c1) of this (sequence, kv head): chunk c is head c / n_chunks
  // of the group, local chunk c % n_chunks
  const int c0 = j * cp.per_block;
  const int c1 = min(G * cp.n_chunks, c0 + cp.per_block);
  int kend = 0;
  for (int c = c0; c < c1; ++c) kend = max(kend, (c % cp.n_chunks) >= cp.chunks_d ? a.S + a.n_c + a.n_r : a.S);
  const int ch = c0 + wave;
  const bool active = ch < c1;
  const int h = kvh * G + (active ? ch / cp.n_chunks : 0);
  int row_base = 0, row_end = 0, wlen = 0;
  if (active) chunk_rows(a, cp, 32, ch % cp.n_chunks, row_base, row_end, wlen);
  const int row = row_base + l32;
  const bool rvalid = active && row < row_end;

  const uint16_t* kc = static_cast<const uint16_t*>(a.kc) + ((int64_t)b * g.Hkv + kvh) * g.slots * D;
  const uint16_t* vc = static_cast<const uint16_t*>(a.vc) + ((int64_t)b * g.Hkv + kvh) * D * g.slots;

  const int n_tiles = (kend + KT - 1) / KT;
  for (int t = 0; t < kStages - 1 && t < n_tiles; ++t) tile_fill<D>(g, a, b, kvh, kc, vc, t * KT, ks[t], vs[t]);

  // Q^T fragment (B operand): lane holds row l32, dims 16t + 8*half + 0..7, RoPE'd.
  bf16x8 qf[NKS];
  {
    RowInfo ri = {0, 0};
    if (rvalid) ri = query_row(g, a, b, row);
    const uint16_t* tq = static_cast<const uint16_t*>(a.tq) + (int64_t)ri.id * g.hidden + h * D;
    const float* cs = a.rope_cos + (int64_t)ri.pos * (D / 2);
    const float* sn = a.rope_sin + (int64_t)ri.pos * (D / 2);
#pragma unroll
    for (int t = 0; t < NKS; ++t) {
      u16x8 raw = {0, 0, 0, 0, 0, 0, 0, 0};
      if (rvalid) raw = *reinterpret_cast<const u16x8*>(tq + 16 * t + 8 * half);
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
  }

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
  const int my_loads = T::loads_of(wave);

  for (int t = 0; t < n_tiles; ++t) {
    const int younger = min(kStages - 2, n_tiles - 1 - t);
    ring_wait(younger * my_loads);
    ring_barrier();
    const int nxt = t + kStages - 1;
    if (nxt < n_tiles) tile_fill<D>(g, a, b, kvh, kc, vc, nxt * KT, ks[nxt % kStages], vs[nxt % kStages]);
    const int kt = t * KT;
    if (!active || kt >= wlen) continue;
    const int cur = t % kStages;
    if (kt + KT > wlen) attn_tile<D, true>(ks[cur], vs[cur], qf, acc, m_ref, l_run, kt, wlen, krow, half, l32, sc);
    else attn_tile<D, false>(ks[cur], vs[cur], qf, acc, m_ref, l_run, kt, wlen, krow, half, l32, sc);
  }

  const float l_tot = l_run + __shfl_xor(l_run, 32);
  if (rvalid) {
    const float inv = 1.f / l_tot;
    const int n_q = a.n_d + a.n_c + a.n_r;
    float* o = a.out + ((int64_t)b * n_q + row) * g.hidden + h * D;
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) {
        floatx4 v;
#pragma unroll
        for (int ii = 0; ii < 4; ++ii) v[ii] = acc[db][4 * jj + ii] * inv;
        *reinterpret_cast<floatx4*>(o + 32 * db + 8 * jj + 4 * half) = v;
      }
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
  int row_base, row_end, wlen;
  chunk_rows(a, cp, 64, ch, row_base, row_end, wlen);
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
      if (slot < a.S) v = vc[(int64_t)dd * g.slots + slot];
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
  ChunkPlan cp;
  cp.chunks_d = (a.n_d + rows_per_chunk - 1) / rows_per_chunk;
  cp.n_chunks = cp.chunks_d + (n_cr + rows_per_chunk - 1) / rows_per_chunk;
  if (cp.n_chunks == 0) return hipSuccess;
  if (g.fp32) {
    cp.per_block = 1;
    cp.blocks = cp.n_chunks;
    cp.real_blocks = g.B * g.H * cp.n_chunks;
    dim3 grid(cp.real_blocks);
    if (g.D == 128) hipLaunchKernelGGL((k_attn_f32<128>), grid, dim3(256), 0, s, g, a, cp);
    else hipLaunchKernelGGL((k_attn_f32<64>), grid, dim3(256), 0, s, g, a, cp);
  } else {
    const int G = g.H / g.Hkv;
    const int space = G * cp.n_chunks;                 // chunks per (sequence, kv head)
    const int nb = (space + kAttnWaves - 1) / kAttnWaves;
    cp.blocks = nb;
    cp.per_block = (space + nb - 1) / nb;
    cp.real_blocks = g.B * g.Hkv * nb;
    dim3 grid((cp.real_blocks + 7) / 8 * 8);
    if (g.D == 128) hipLaunchKernelGGL((k_attn_bf16<128>), grid, dim3(kAttnThreads), 0, s, g, a, cp);
    else hipLaunchKernelGGL((k_attn_bf16<64>), grid, dim3(kAttnThreads), 0, s, g, a, cp);
  }
  return hipGetLastError();
}

}  // namespace mdm
