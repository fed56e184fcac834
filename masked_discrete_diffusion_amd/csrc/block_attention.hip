// Training-form step-causal attention: one parallel forward under the block
// mask (bf16 MFMA, head_dim 128).
//
// Page 1, key design 3 (page 3, sections 3.3 and 7.3): training reproduces
// the incremental cache in a single forward.  Every row carries a block id;
// with M clean blocks (the prompt is block 0, clean tokens blocks 1..M), a
// row of clean block i sees the keys of blocks j <= i, and a row of masked
// block i > M sees its own block and every block j <= M, never another masked
// block.  Each masked block's registers are rows of that block.  Block ids are
// labels: rows may come in any order.
//
// Work split: a block of 8 wavefronts takes 8 chunks of 32 query rows of the
// query heads of one key/value head (with grouped heads, the chunks of one
// row range over the group's heads share the block), and streams the 64-key
// tiles that at least one of its chunks sees.  A pre-pass records each key
// tile's block-id range; each wavefront classifies every tile from its rows'
// range as unseen, fully seen or partly seen, so only the tiles on a block
// boundary pay for an element-wise mask.
//
// Per tile: K and V go from HBM to LDS by LDS-DMA (global_load_lds_dwordx4)
// through a 4-deep ring, both in their natural [key][d] layout with 16-byte
// units XOR-swizzled per row.  S^T = K Q^T with v_mfma_f32_32x32x16_bf16 (Q^T
// in registers), fp32 softmax at a fixed reference (each row's maximum over
// the wavefront's first seen tile), P in bf16, O^T += V^T P^T; the scores of
// tile i + 1 are issued next to the softmax of tile i.  A row sum that
// reaches 2^50 (a later score far above the reference) sends the block
// through a second pass with a running maximum, which gives the same softmax.  The V^T operand comes straight from the
// natural-layout V tile through the LDS transpose read ds_read_b64_tr_b16:
// within each 16 lanes, lane j receives element j%4 of the 64-bit words that
// lanes 4e + j/4 addressed (e = 0..3), so lanes that address 4 consecutive
// keys at 4 neighbouring 4-dim groups hand every lane 4 consecutive keys of
// one dim, which is what the MFMA operand wants.
#include <climits>
#include <mutex>

#include "common.hpp"
#include "kernels.hpp"

// Per-tile block-id ranges of mdm_block_attention_static, for callers that
// cannot allocate: 16384 int32 (64 KiB), which every GPU the library runs on
// holds until the process ends.  Host code never passes this name to a kernel
// (in host code it is a host-side stand-in); it uses the device address that
// block_attention_static_scratch() looks up.
static __device__ __align__(256) int32_t scratch[mdm::kStaticRangeInts];

namespace mdm {

namespace {

constexpr int kD = 128;                              // head dim
constexpr int kRB = 1;                                // 32-row MFMA blocks per wavefront
constexpr int kBaWaves = 8 / kRB;                     // wavefronts per block (256 rows)
constexpr int kRowsPerWave = 32 * kRB;
constexpr int kBaThreads = kBaWaves * kWave;
constexpr int kBaStages = 4;                          // LDS ring depth (tiles)
constexpr int kBaAhead = 2;                           // tiles loaded ahead of the one being scored
constexpr int kRowBytes = kD * 2;                     // one K or V row in LDS (16 units, no padding)
constexpr int kTileBytes = kKeyTile * kRowBytes;      // 16 KiB
constexpr int kDmaBlocks = 2 * kTileBytes / 1024;     // 32 wave-wide 1 KiB loads per K+V tile
constexpr int kLpw = kDmaBlocks / kBaWaves;           // loads per wavefront per tile
static_assert(kDmaBlocks % kBaWaves == 0, "K and V loads split evenly over the wavefronts");
static_assert(kBaStages >= kBaAhead + 2, "tiles i (PV) and i + 1 (scores) stay while i + 1 + ahead loads");

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kRefFloor = -3.0e38f;                 // finite start for the reference

enum : int { kUnseen = 0, kSeen = 1, kPartly = 2 };

// Visibility of a key of block kb to a row of block qb (m = number of clean blocks).
__device__ inline bool block_visible(int qb, int kb, int m) { return qb <= m ? kb <= qb : (kb == qb || kb <= m); }

// A wavefront's rows (block ids in [qmin, qmax]) against a key tile (block ids
// in [kmin, kmax]; whole = all 64 keys exist).  Every key a row sees has a
// block id <= the row's, so a tile above qmax is unseen.
__device__ inline int classify(int qmin, int qmax, int kmin, int kmax, int m, bool whole) {
  if (kmin > qmax) return kUnseen;
  int c;
  if (qmax <= m) {
    c = kmax <= qmin ? kSeen : kPartly;
  } else if (qmin > m) {
    if (kmax <= m) c = kSeen;
    else if (kmin > m && (kmax < qmin || kmin > qmax)) return kUnseen;
    else c = (kmin == kmax && qmin == qmax && kmin == qmin) ? kSeen : kPartly;
  } else {
    c = kPartly;
  }
  return (c == kSeen && !whole) ? kPartly : c;
}

// Minimum (MAX = false) or maximum over the wavefront, on every lane.
template <bool MAX>
__device__ inline int wave_ext_i32(int x) {
  auto pick = [](const U2 p) { return MAX ? max((int)p.a, (int)p.b) : min((int)p.a, (int)p.b); };
  x = pick(wave_pair<0>((uint32_t)x));
  x = pick(wave_pair<1>((uint32_t)x));
  x = pick(wave_pair<2>((uint32_t)x));
  x = pick(wave_pair<3>((uint32_t)x));
  x = pick(wave_pair<4>((uint32_t)x));
  return pick(wave_pair<5>((uint32_t)x));
}
__device__ inline int wave_min_i32(int x) { return wave_ext_i32<false>(x); }
__device__ inline int wave_max_i32(int x) { return wave_ext_i32<true>(x); }

// Block-id range of each 64-key tile: ranges[(b * n_tiles + t) * 2 + {0, 1}].
__global__ void __launch_bounds__(kWave) k_tile_ranges(const int32_t* __restrict__ blk, int n, int n_tiles,
                                                      int32_t* __restrict__ ranges) {
  const int t = blockIdx.x, b = blockIdx.y, key = t * kKeyTile + threadIdx.x;
  const bool ok = key < n;
  const int kb = ok ? blk[(int64_t)b * n + key] : 0;
  const int lo = wave_min_i32(ok ? kb : INT_MAX);
  const int hi = wave_max_i32(ok ? kb : INT_MIN);
  if (threadIdx.x == 0) {
    ranges[((int64_t)b * n_tiles + t) * 2] = lo;
    ranges[((int64_t)b * n_tiles + t) * 2 + 1] = hi;
  }
}

typedef short short4v __attribute__((ext_vector_type(4)));
typedef short short8v __attribute__((ext_vector_type(8)));

__device__ inline short4v lds_read_tr(uint32_t addr) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (__attribute__((address_space(3))) short4v*)(uintptr_t)addr);
}
__device__ inline bf16x8 lds_read_b128(uint32_t addr) {
  return *(const __attribute__((address_space(3))) bf16x8*)(uintptr_t)addr;
}

// Per-lane LDS byte offsets of the MFMA operands within a ring slot.
//  K (A operand of S^T = K Q^T, key r of a 32-key half, dims 16t + 8h..+7):
//    row r holds logical unit c at unit c ^ (r & 15).
//  V (A operand of O^T = V^T P^T through the transpose read): row r holds
//    logical unit c at unit c ^ swz_v(r), swz_v(r) = 4(r & 3) + 2((r >> 2) & 1).
//    Lane l addresses key 4(l >> 5) + ((l >> 2) & 3) (+ 8 for the second
//    read, + 16 per k-step, + 32 per half) at dims 32db + 16((l >> 4) & 1) + 4(l & 3).
struct LaneOffsets {
  uint32_t k[8];     // per 16-dim k-step t, first half
  uint32_t v[4];     // per 32-dim block db, first k-step, first read
};
__device__ inline LaneOffsets lane_offsets(int lane) {
  LaneOffsets o;
  const int h = lane >> 5, f = lane & 15;
#pragma unroll
  for (int t = 0; t < 8; ++t) o.k[t] = (uint32_t)((lane & 31) * kRowBytes + 16 * ((2 * t + h) ^ f));
  const int r = 4 * h + ((lane >> 2) & 3);
  const int sw = 4 * (r & 3) + 2 * ((r >> 2) & 1);
  const int c = 2 * ((lane >> 4) & 1) + ((lane & 3) >> 1);
#pragma unroll
  for (int db = 0; db < 4; ++db)
    o.v[db] = (uint32_t)(r * kRowBytes + 16 * ((4 * db + c) ^ sw) + 8 * (lane & 1));
  return o;
}

// Global byte offset (within a tile, rows rs bytes apart) of the 16-byte unit
// that DMA lane `lane` of 1 KiB block `blk` (of the K or V tile) brings to LDS.
__device__ inline uint32_t dma_src(int blk, int lane, bool is_k, int rs, int last_row) {
  const int u = blk * kWave + lane;
  const int r = u >> 4, p = u & 15;
  const int sw = is_k ? (r & 15) : (4 * (r & 3) + 2 * ((r >> 2) & 1));
  return (uint32_t)(min(r, last_row) * rs + 16 * (p ^ sw));
}

// A pointer every lane holds the same value of, in scalar registers.
__device__ inline const uint16_t* uniform_ptr(const uint16_t* p) {
  const uint64_t u = (uint64_t)(uintptr_t)p;
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)u);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(u >> 32));
  return reinterpret_cast<const uint16_t*>((uintptr_t)(((uint64_t)hi << 32) | lo));
}

struct BaCtx {
  const uint16_t* kbase;    // keys of (b, kvh) at row 0
  const uint16_t* vbase;
  int rs;                   // bytes between consecutive rows (H_kv * D * 2)
  int n;
  uint32_t ring_k, ring_v;  // LDS byte addresses of the two rings
};

// Issue this wavefront's DMA loads of tile t into ring slot s.  The first
// half of the wavefronts loads K, the second half V, kLpw wave-wide loads each.
__device__ inline void issue_tile(const BaCtx& c, int t, int s, int wave, const uint32_t (&off)[kLpw], int lane) {
  const bool is_k = wave < kBaWaves / 2;
  const int key0 = __builtin_amdgcn_readfirstlane(t) * kKeyTile;
  const uint16_t* base = uniform_ptr((is_k ? c.kbase : c.vbase) + (int64_t)key0 * (c.rs / 2));
  const uint32_t dst = (is_k ? c.ring_k : c.ring_v) + s * kTileBytes + (wave % (kBaWaves / 2)) * kLpw * 1024;
  if (key0 + kKeyTile <= c.n) {
#pragma unroll
    for (int i = 0; i < kLpw; ++i) dma16_at(base, off[i], dst + i * 1024);
  } else {
    // last, partial tile: rows past n re-read row n-1 (masked later)
    const int last = c.n - 1 - key0;
#pragma unroll
    for (int i = 0; i < kLpw; ++i)
      dma16_at(base, dma_src((wave % (kBaWaves / 2)) * kLpw + i, lane, is_k, c.rs, last), dst + i * 1024);
  }
}

// Wait for a tile's loads (this wavefront's; the barrier covers everyone's)
// when `younger` later tiles of this wavefront may stay in flight.
__device__ inline void wait_tile(int younger) {
  static_assert(kBaAhead == 2, "waits are spelled out for two tiles ahead");
  if (younger >= 1) ring_wait<kLpw>();
  else ring_wait<0>();
}

__device__ inline float max3(float a, float b, float c) {
  return __builtin_elementwise_maximum(__builtin_elementwise_maximum(a, b), c);
}
__device__ inline float halves_max(float x) {
  const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __builtin_elementwise_maximum(__uint_as_float(sw[0]), __uint_as_float(sw[1]));
}
__device__ inline float halves_sum(float x) {
  const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(sw[0]) + __uint_as_float(sw[1]);
}

// Scores of one tile for the wavefront's rows: s[rb][hk] = S^T of row block
// rb (rows 32rb + lane & 31) and 32-key half hk; lane holds keys
// 8j + 4(lane >> 5) + i (e = 4j + i) of the half.  Each K operand read from
// LDS feeds every row block.
typedef floatx16 TileS[kRB][2];
__device__ inline void tile_scores(uint32_t ks, const LaneOffsets& lo, const bf16x8 (&qf)[kRB][8], TileS& s) {
#pragma unroll
  for (int rb = 0; rb < kRB; ++rb)
#pragma unroll
    for (int hk = 0; hk < 2; ++hk)
#pragma unroll
      for (int e = 0; e < 16; ++e) s[rb][hk][e] = 0.f;
#pragma unroll
  for (int t = 0; t < 8; ++t)
#pragma unroll
    for (int hk = 0; hk < 2; ++hk) {
      const bf16x8 kf = lds_read_b128(ks + lo.k[t] + hk * 32 * kRowBytes);
#pragma unroll
      for (int rb = 0; rb < kRB; ++rb) s[rb][hk] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf, qf[rb][t], s[rb][hk], 0, 0, 0);
    }
}

// Scores of keys a row may not see become -inf (exp2 gives exactly 0).
__device__ inline void mask_tile(TileS& s, const int32_t* kblk, int key0, int n, const int (&qb)[kRB], int m) {
  const int h = (__lane_id() >> 5) & 1;
#pragma unroll
  for (int hk = 0; hk < 2; ++hk)
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      const int key = key0 + 32 * hk + 8 * (e / 4) + 4 * h + (e % 4);
      const int kb = kblk[min(key, n - 1)];
#pragma unroll
      for (int rb = 0; rb < kRB; ++rb)
        s[rb][hk][e] = (key < n && block_visible(qb[rb], kb, m)) ? s[rb][hk][e] : -__builtin_inff();
    }
}

__device__ inline float tile_max(const floatx16& s0, const floatx16& s1) {
  float a = max3(s0[0], s0[1], s0[2]), b = max3(s1[0], s1[1], s1[2]);
#pragma unroll
  for (int e = 3; e < 15; e += 2) {
    a = max3(a, s0[e], s0[e + 1]);
    b = max3(b, s1[e], s1[e + 1]);
  }
  return halves_max(max3(a, b, __builtin_elementwise_maximum(s0[15], s1[15])));
}

// p = exp2(s * sc - m_ref) in place; returns their sum.
__device__ inline float exp_half(floatx16& sv, float m_ref, float sc) {
  float sum = 0.f;
#pragma unroll
  for (int e = 0; e < 16; ++e) {
    sv[e] = __builtin_amdgcn_exp2f(fmaf(sv[e], sc, -m_ref));
    sum += sv[e];
  }
  return sum;
}

// O^T += V^T P^T for every row block over the tile in ring slot vs.  K-step
// (hk, u) takes the lane's p values 8u..8u+7 of half hk = keys
// 32hk + 16u + 4(lane >> 5) + {0..3} and 32hk + 16u + 8 + 4(lane >> 5) + {0..3};
// the two transpose reads deliver V at exactly those keys, and each V
// operand feeds every row block.
__device__ inline void tile_pv(const TileS& p, uint32_t vs, const LaneOffsets& lo, floatx16 (&acc)[kRB][4]) {
  typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
#pragma unroll
  for (int hk = 0; hk < 2; ++hk)
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      bf16x8 pb[kRB];
#pragma unroll
      for (int rb = 0; rb < kRB; ++rb) {
        u32x4 w;
#pragma unroll
        for (int q = 0; q < 4; ++q) w[q] = pack_bf16x2(p[rb][hk][8 * u + 2 * q], p[rb][hk][8 * u + 2 * q + 1]);
        pb[rb] = __builtin_bit_cast(bf16x8, w);
      }
#pragma unroll
      for (int db = 0; db < 4; ++db) {
        const uint32_t a = vs + lo.v[db] + (32 * hk + 16 * u) * kRowBytes;
        const short4v r0 = lds_read_tr(a);
        const short4v r1 = lds_read_tr(a + 8 * kRowBytes);
        const bf16x8 vv = __builtin_bit_cast(bf16x8, __builtin_shufflevector(r0, r1, 0, 1, 2, 3, 4, 5, 6, 7));
#pragma unroll
        for (int rb = 0; rb < kRB; ++rb) acc[rb][db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vv, pb[rb], acc[rb][db], 0, 0, 0);
      }
    }
}

// Online softmax of a tile's scores and O += P V with the running row
// maximum as the reference, rescaling O and l on every tile (no branch, so
// no merge of accumulator definitions).  Used by the recompute pass only.
__device__ inline void tile_softmax_pv(TileS& s, uint32_t vs, const LaneOffsets& lo, floatx16 (&acc)[kRB][4],
                                       float (&m_ref)[kRB], float (&l_run)[kRB], float sc) {
#pragma unroll
  for (int rb = 0; rb < kRB; ++rb) {
    const float m_new = fmaxf(m_ref[rb], tile_max(s[rb][0], s[rb][1]) * sc);
    const float alpha = __builtin_amdgcn_exp2f(m_ref[rb] - m_new);
    l_run[rb] *= alpha;
#pragma unroll
    for (int db = 0; db < 4; ++db)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[rb][db][e] *= alpha;
    m_ref[rb] = m_new;
    l_run[rb] += exp_half(s[rb][0], m_ref[rb], sc) + exp_half(s[rb][1], m_ref[rb], sc);
  }
  tile_pv(s, vs, lo, acc);
}

// Fixed-reference variant: p = exp2(s * sc - m_ref) with the reference never
// raised, no maximum taken, no rescale.
__device__ inline void tile_exp_pv_fixed(TileS& s, uint32_t vs, const LaneOffsets& lo, floatx16 (&acc)[kRB][4],
                                         const float (&m_ref)[kRB], float (&l_run)[kRB], float sc) {
#pragma unroll
  for (int rb = 0; rb < kRB; ++rb) l_run[rb] += exp_half(s[rb][0], m_ref[rb], sc) + exp_half(s[rb][1], m_ref[rb], sc);
  tile_pv(s, vs, lo, acc);
}

// A fully seen tile at the fixed reference, in one basic block: the scores
// of both 32-key halves are issued first, then the exp of half 0 runs under
// the MFMAs of half 1, and the exp of half 1 under the PV MFMAs of half 0.
__device__ inline void tile_fixed_fused(uint32_t ks, uint32_t vs, const LaneOffsets& lo, const bf16x8 (&qf)[kRB][8],
                                        floatx16 (&acc)[kRB][4], const float (&m_ref)[kRB], float (&l_run)[kRB],
                                        float sc) {
  typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
  TileS s;
  tile_scores(ks, lo, qf, s);
#pragma unroll
  for (int hk = 0; hk < 2; ++hk)
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      bf16x8 pb[kRB];
#pragma unroll
      for (int rb = 0; rb < kRB; ++rb) {
        float sum = 0.f;
        u32x4 w;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const float p0 = __builtin_amdgcn_exp2f(fmaf(s[rb][hk][8 * u + 2 * q], sc, -m_ref[rb]));
          const float p1 = __builtin_amdgcn_exp2f(fmaf(s[rb][hk][8 * u + 2 * q + 1], sc, -m_ref[rb]));
          sum += p0 + p1;
          w[q] = pack_bf16x2(p0, p1);
        }
        l_run[rb] += sum;
        pb[rb] = __builtin_bit_cast(bf16x8, w);
      }
#pragma unroll
      for (int db = 0; db < 4; ++db) {
        const uint32_t a = vs + lo.v[db] + (32 * hk + 16 * u) * kRowBytes;
        const short4v r0 = lds_read_tr(a);
        const short4v r1 = lds_read_tr(a + 8 * kRowBytes);
        const bf16x8 vv = __builtin_bit_cast(bf16x8, __builtin_shufflevector(r0, r1, 0, 1, 2, 3, 4, 5, 6, 7));
#pragma unroll
        for (int rb = 0; rb < kRB; ++rb)
          acc[rb][db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vv, pb[rb], acc[rb][db], 0, 0, 0);
      }
    }
}

// Row sums stay below 2^kOverflowLog2 on the fixed-reference pass (then
// every p did, and O = sum p v stays far inside fp32); a NaN fails too.
constexpr float kOverflowLog2 = 50.f;

__device__ inline int tile_class(const uint16_t* cls, int t, int wave) {
  return __builtin_amdgcn_readfirstlane((cls[t] >> (2 * wave)) & 3);
}

__global__ void __launch_bounds__(kBaThreads) k_block_attn(BlockAttnArgs a) {
  __shared__ __attribute__((aligned(1024))) uint8_t ring[2 * kBaStages * kTileBytes];
  __shared__ int s_qrange[kBaWaves][2];
  __shared__ uint16_t s_cls[kBlockAttnMaxTiles];
  __shared__ uint16_t s_list[kBlockAttnMaxTiles];
  __shared__ int s_count, s_count_all;

  const int tid = threadIdx.x, lane = tid % kWave;
  const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);
  // Heaviest first over the whole grid: rows later in the sequence see more
  // tiles (clean blocks are causal, masked blocks come last), so the blocks
  // of the last row chunks of every (sequence, kv head) are dispatched
  // first and the light ones fill the tail.
  const int lb = blockIdx.x;
  if (lb >= a.real_blocks) return;
  const int G = a.H / a.Hkv;
  const int n_bh = a.B * a.Hkv;
  const int bh = lb % n_bh;
  const int cb = a.nbk - 1 - lb / n_bh;
  const int b = bh / a.Hkv, kvh = bh % a.Hkv;
  const int n = a.n, n_rc = (n + kRowsPerWave - 1) / kRowsPerWave, n_tiles = (n + kKeyTile - 1) / kKeyTile;
  const int chunk = cb * kBaWaves + wave;
  const int g = chunk % G, rc = chunk / G;
  const bool active = rc < n_rc;
  const int head = kvh * G + g;
  const int32_t* blk = a.blk + (int64_t)b * n;
  const int m = a.n_clean[b];
  int rowc[kRB], qb[kRB];
  bool row_ok[kRB];
#pragma unroll
  for (int rb = 0; rb < kRB; ++rb) {
    const int row = rc * kRowsPerWave + 32 * rb + (lane & 31);
    row_ok[rb] = active && row < n;
    rowc[rb] = min(row, n - 1);
    qb[rb] = blk[rowc[rb]];
  }

  {
    int lo_q = INT_MAX, hi_q = INT_MIN;
#pragma unroll
    for (int rb = 0; rb < kRB; ++rb) {
      lo_q = min(lo_q, row_ok[rb] ? qb[rb] : INT_MAX);
      hi_q = max(hi_q, row_ok[rb] ? qb[rb] : INT_MIN);
    }
    const int qmin = wave_min_i32(lo_q);
    const int qmax = wave_max_i32(hi_q);
    if (lane == 0) {
      s_qrange[wave][0] = active ? qmin : 1;
      s_qrange[wave][1] = active ? qmax : 0;     // empty range: every tile unseen
    }
  }
  __syncthreads();
  const int32_t* rg = a.ranges + (int64_t)b * n_tiles * 2;
  for (int t = tid; t < n_tiles; t += kBaThreads) {
    const int kmin = rg[2 * t], kmax = rg[2 * t + 1];
    const bool whole = (t + 1) * kKeyTile <= n;
    int word = 0;
#pragma unroll
    for (int w = 0; w < kBaWaves; ++w) {
      const int lo = s_qrange[w][0], hi = s_qrange[w][1];
      const int c = lo > hi ? kUnseen : classify(lo, hi, kmin, kmax, m, whole);
      word |= c << (2 * w);
    }
    s_cls[t] = (uint16_t)word;
  }
  __syncthreads();
  // Tile list: first the tiles every active wavefront sees whole (the
  // branch-free main loop), then the remaining tiles some wavefront sees;
  // each part in key order.
  if (wave == 0) {
    uint32_t all = 0;
#pragma unroll
    for (int w = 0; w < kBaWaves; ++w) {
      const bool on = s_qrange[w][0] <= s_qrange[w][1];
      all |= (on ? (uint32_t)kSeen : 0u) << (2 * w);
    }
    int cnt = 0;
    for (int part = 0; part < 2; ++part) {
      for (int t0 = 0; t0 < n_tiles; t0 += kWave) {
        const int t = t0 + lane;
        const uint32_t w = t < n_tiles ? s_cls[t] : 0u;
        const bool pick = part == 0 ? (w == all) : (w != 0 && w != all);
        const uint64_t mask = __ballot(pick);
        const int pos = cnt + __builtin_popcountll(mask & ((1ull << lane) - 1ull));
        if (pick) s_list[pos] = (uint16_t)t;
        cnt += __builtin_popcountll(mask);
      }
      if (part == 0 && lane == 0) s_count_all = cnt;
    }
    if (lane == 0) s_count = cnt;
  }
  __syncthreads();
  const int nt = __builtin_amdgcn_readfirstlane(s_count);
  const int n_all = __builtin_amdgcn_readfirstlane(s_count_all);

  BaCtx c;
  c.rs = a.Hkv * kD * 2;
  c.n = n;
  c.kbase = static_cast<const uint16_t*>(a.k) + ((int64_t)b * n * a.Hkv + kvh) * kD;
  c.vbase = static_cast<const uint16_t*>(a.v) + ((int64_t)b * n * a.Hkv + kvh) * kD;
  c.ring_k = lds_addr(&ring[0]);
  c.ring_v = c.ring_k + kBaStages * kTileBytes;
  uint32_t off[kLpw];
#pragma unroll
  for (int i = 0; i < kLpw; ++i)
    off[i] = dma_src((wave % (kBaWaves / 2)) * kLpw + i, lane, wave < kBaWaves / 2, c.rs, kKeyTile - 1);

  auto start_ring = [&]() {
    for (int i = 0; i < kBaAhead && i < nt; ++i) issue_tile(c, s_list[i], i, wave, off, lane);
  };
  // prologue loads, then Q^T fragments (row, dims 16t + 8(lane >> 5)..+7)
  start_ring();
  bf16x8 qf[kRB][8];
#pragma unroll
  for (int rb = 0; rb < kRB; ++rb) {
    const uint16_t* qrow = static_cast<const uint16_t*>(a.q) + (((int64_t)b * n + rowc[rb]) * a.H + head) * kD;
#pragma unroll
    for (int t = 0; t < 8; ++t) qf[rb][t] = *reinterpret_cast<const bf16x8*>(qrow + 16 * t + 8 * (lane >> 5));
  }
  const LaneOffsets lo = lane_offsets(lane);
  const float sc = kLog2e / sqrtf((float)kD);
  floatx16 acc[kRB][4];
  float m_ref[kRB], l_run[kRB];
  auto reset = [&]() {
#pragma unroll
    for (int rb = 0; rb < kRB; ++rb) {
#pragma unroll
      for (int db = 0; db < 4; ++db)
#pragma unroll
        for (int e = 0; e < 16; ++e) acc[rb][db][e] = 0.f;
      m_ref[rb] = kRefFloor;
      l_run[rb] = 0.f;
    }
  };
  reset();

  // Ring step of tile i: wait for it (own loads, then the barrier for
  // everyone's) and issue tile i + 2.  The barrier also ends every
  // wavefront's use of tile i - 2, whose slot receives tile i + 2.
  auto ring_step = [&](int i) -> int {
    wait_tile(min(nt - 1 - i, kBaAhead - 1));
    ring_barrier();
    if (i + kBaAhead < nt) issue_tile(c, s_list[i + kBaAhead], (i + kBaAhead) % kBaStages, wave, off, lane);
    return tile_class(s_cls, s_list[i], wave);
  };
  // Scores of tile i when this wavefront's rows see it, masked when partly.
  auto scores = [&](int i, int cls, TileS& s) {
    if (cls != kUnseen) {
      tile_scores(c.ring_k + (i % kBaStages) * kTileBytes, lo, qf, s);
      if (cls == kPartly) mask_tile(s, blk, s_list[i] * kKeyTile, n, qb, m);
    }
  };

  // Fast pass.  The reference of each row is the maximum over the
  // wavefront's first tile and is never raised, so no loop carries a rescale
  // branch.  Phase 1: the tiles every wavefront sees whole, one basic block
  // each (the first peeled to set the reference); phase 2: the others.
  TileS sA;
  bool have_ref = false;
  if (n_all > 0) {
    const int cls = ring_step(0);
    scores(0, cls, sA);
#pragma unroll
    for (int rb = 0; rb < kRB; ++rb) m_ref[rb] = tile_max(sA[rb][0], sA[rb][1]) * sc;
    have_ref = true;
    tile_exp_pv_fixed(sA, c.ring_v, lo, acc, m_ref, l_run, sc);
    for (int i = 1; i < n_all; ++i) {
      ring_step(i);
      tile_fixed_fused(c.ring_k + (i % kBaStages) * kTileBytes, c.ring_v + (i % kBaStages) * kTileBytes, lo, qf,
                       acc, m_ref, l_run, sc);
    }
  }
  for (int i = n_all; i < nt; ++i) {
    const int cls = ring_step(i);
    if (cls == kUnseen) continue;
    scores(i, cls, sA);
    if (!have_ref) {
#pragma unroll
      for (int rb = 0; rb < kRB; ++rb) m_ref[rb] = tile_max(sA[rb][0], sA[rb][1]) * sc;
      have_ref = true;
    }
    tile_exp_pv_fixed(sA, c.ring_v + (i % kBaStages) * kTileBytes, lo, acc, m_ref, l_run, sc);
  }
  bool over = false;
#pragma unroll
  for (int rb = 0; rb < kRB; ++rb) over = over || (row_ok[rb] && !(l_run[rb] < 0x1p50f));
  static_assert(kOverflowLog2 == 50.f, "the bound above is 2^kOverflowLog2");
  // A row sum reached the bound (or a row saw no key of its first tile):
  // the tiles stream again and those rows recompute with a running maximum.
  // The barrier of the vote ends every wavefront's use of the ring.
  // Only the wavefronts whose own rows failed recompute; the others keep
  // their result and take the ring steps only.
  const bool redo = __any(over);
  if (__syncthreads_or(over ? 1 : 0)) {
    if (redo) reset();
    start_ring();
    for (int i = 0; i < nt; ++i) {
      int cls = ring_step(i);
      if (!redo) cls = kUnseen;
      scores(i, cls, sA);
      if (cls != kUnseen) tile_softmax_pv(sA, c.ring_v + (i % kBaStages) * kTileBytes, lo, acc, m_ref, l_run, sc);
    }
  }

  // O = acc / l; lane holds dims 32db + 8j + 4(lane >> 5) + i of its row
#pragma unroll
  for (int rb = 0; rb < kRB; ++rb) {
    const float inv = 1.f / halves_sum(l_run[rb]);
    if (row_ok[rb]) {
      float* orow = a.out + (((int64_t)b * n + rc * kRowsPerWave + 32 * rb + (lane & 31)) * a.H + head) * kD +
                    4 * (lane >> 5);
#pragma unroll
      for (int db = 0; db < 4; ++db)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          floatx4 o;
#pragma unroll
          for (int e = 0; e < 4; ++e) o[e] = acc[rb][db][4 * j + e] * inv;
          *reinterpret_cast<floatx4*>(orow + 32 * db + 8 * j) = o;
        }
    }
  }
}

}  // namespace

hipError_t launch_block_attention(BlockAttnArgs a, hipStream_t s) {
  const int n_tiles = (a.n + kKeyTile - 1) / kKeyTile;
  if (a.n <= 0 || n_tiles > kBlockAttnMaxTiles || a.Hkv <= 0 || a.H % a.Hkv) return hipErrorInvalidValue;
  hipLaunchKernelGGL(k_tile_ranges, dim3(n_tiles, a.B), dim3(kWave), 0, s, a.blk, a.n, n_tiles, a.ranges);
  const int G = a.H / a.Hkv;
  const int n_rc = (a.n + kRowsPerWave - 1) / kRowsPerWave;
  a.nbk = (G * n_rc + kBaWaves - 1) / kBaWaves;
  a.real_blocks = a.B * a.Hkv * a.nbk;
  hipLaunchKernelGGL(k_block_attn, dim3(a.real_blocks), dim3(kBaThreads), 0, s, a);
  return hipGetLastError();
}

// Device address of `scratch` on the current device: looked up with
// hipGetSymbolAddress the first time a device is current here, then kept per
// device (each GPU holds its own copy of the array at its own address).
hipError_t block_attention_static_scratch(int32_t** ptr, size_t* n_ints) {
  constexpr int kMaxDevices = 64;
  static std::mutex mu;
  static int32_t* addr[kMaxDevices] = {};
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(mu);
  if (!addr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    addr[dev] = static_cast<int32_t*>(p);
  }
  *ptr = addr[dev];
  *n_ints = kStaticRangeInts;
  return hipSuccess;
}

}  // namespace mdm
