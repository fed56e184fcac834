// Logits for the decoded subset only, with max-probability confidence and
// argmax (page 1, key design 1; page 3, section 3.2).
//
// 1. pack:   fp32 h rows of the decoded subset -> bf16 hi (and lo = bf16(h - hi))
//            in a dense [m_pad][hidden] operand, zero rows past M.
// 2. screen: z^T = W h^T on bf16 MFMA (32x32x16), one 128-column vocab tile by
//            32/64/128 rows per block; the epilogue keeps per (row, tile) the maximum,
//            the sum of exp(z - max) and the three best (value, index) pairs, and
//            never writes the logits (unless asked to, for validation).
//            fp32 mode: the same tile and epilogue with fp32 VALU products.
// 3. decide: per row, combine the tiles (max, sum of exp), re-score the kCand
//            best entries exactly in fp32 from the fp32 h, prove from the
//            screen's error bound that no other column can beat the best of
//            them (re-scoring more where the bound cannot), decide the argmax
//            (lowest index on ties) and the confidence exp(z_best - M) / sum
//            exp(z - M), with the re-scored entries' terms exact.
#include <type_traits>

#include "common.hpp"
#include "kernels.hpp"

namespace mdm {

namespace {

constexpr float kNegInf = -__builtin_inff();
constexpr int kKChunk = 64;        // hidden elements per LDS stage
constexpr int kScreenTargetBlocks = 256;   // split hidden until about this many blocks
constexpr int kSplitMaxRows = 1 << 20;     // split hidden only for steps of at most this many rows
constexpr int kProjWideBlocks = 192;     // projection blocks from which the wide tiles are used

// Per (row, vocabulary tile) summary of screened logits: the maximum, the sum
// of exp(z - max) and the three best (value, index) pairs in rank order
// (larger value first, lower index on equal values).  Every other column of
// the tile ranks after the third, so its screened value is at most v3.
struct Top3 {
  float m;      // running maximum
  float se;     // sum of exp(z - m)
  float v1, v2, v3;
  int i1, i2, i3;
};

__device__ __attribute__((always_inline)) inline Top3 top3_push(Top3 t, float v, int i) {
  if (ranks_before(v, i, t.v1, t.i1)) {
    t.v3 = t.v2; t.i3 = t.i2; t.v2 = t.v1; t.i2 = t.i1; t.v1 = v; t.i1 = i;
  } else if (ranks_before(v, i, t.v2, t.i2)) {
    t.v3 = t.v2; t.i3 = t.i2; t.v2 = v; t.i2 = i;
  } else if (ranks_before(v, i, t.v3, t.i3)) {
    t.v3 = v; t.i3 = i;
  }
  return t;
}

// (max, sum of exp) of two partial sums
__device__ __attribute__((always_inline)) inline void lse_merge(float& m, float& se, float om, float ose) {
  const float nm = fmaxf(m, om);
  se = (m == kNegInf ? 0.f : se * expf(m - nm)) + (om == kNegInf ? 0.f : ose * expf(om - nm));
  m = nm;
}

__device__ __attribute__((always_inline)) inline Top3 top3_merge(Top3 a, Top3 b) {
  Top3 r;
  r.m = fmaxf(a.m, b.m);
  r.se = (a.m == kNegInf ? 0.f : a.se * expf(a.m - r.m)) + (b.m == kNegInf ? 0.f : b.se * expf(b.m - r.m));
  r.v1 = a.v1; r.i1 = a.i1; r.v2 = a.v2; r.i2 = a.i2; r.v3 = a.v3; r.i3 = a.i3;
  r = top3_push(r, b.v1, b.i1);
  r = top3_push(r, b.v2, b.i2);
  r = top3_push(r, b.v3, b.i3);
  return r;
}

__device__ __attribute__((always_inline)) inline Top3 top3_shfl_xor(Top3 t, int mask) {
  Top3 o;
  o.m = __shfl_xor(t.m, mask);
  o.se = __shfl_xor(t.se, mask);
  o.v1 = __shfl_xor(t.v1, mask);
  o.v2 = __shfl_xor(t.v2, mask);
  o.v3 = __shfl_xor(t.v3, mask);
  o.i1 = __shfl_xor(t.i1, mask);
  o.i2 = __shfl_xor(t.i2, mask);
  o.i3 = __shfl_xor(t.i3, mask);
  return o;
}

// Fold a lane's logits into (max, sumexp, top-3): values[n] with indices idx[n].
template <int N>
__device__ __attribute__((always_inline)) inline Top3 summarize(const float* vals, const int* idx) {
  Top3 t;
  t.m = kNegInf; t.se = 0.f;
  t.v1 = t.v2 = t.v3 = kNegInf;
  t.i1 = t.i2 = t.i3 = 0x7fffffff;
#pragma unroll
  for (int e = 0; e < N; ++e) {
    t.m = fmaxf(t.m, vals[e]);
    t = top3_push(t, vals[e], idx[e]);
  }
  if (t.m != kNegInf) {
#pragma unroll
    for (int e = 0; e < N; ++e) t.se += expf(vals[e] - t.m);
  }
  return t;
}

// One 32-byte partial record: {m, se, v1, i1} {v2, i2, v3, i3}.
__device__ __attribute__((always_inline)) inline void store_partial(float* p, Top3 t) {
  floatx4 a = {t.m, t.se, t.v1, __int_as_float(t.i1)};
  floatx4 c = {t.v2, __int_as_float(t.i2), t.v3, __int_as_float(t.i3)};
  reinterpret_cast<floatx4*>(p)[0] = a;
  reinterpret_cast<floatx4*>(p)[1] = c;
}

// ------------------------------------------------------------------ pack --
__global__ __launch_bounds__(256) void k_pack(Geometry g, VocabArgs a, int M) {
  const int64_t n8 = (int64_t)a.m_pad * g.hidden / 8;
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= n8) return;
  const int64_t e0 = i * 8;
  const int m = (int)(e0 / g.hidden);
  const int k = (int)(e0 % g.hidden);
  u16x8 hi = {0, 0, 0, 0, 0, 0, 0, 0}, lo = {0, 0, 0, 0, 0, 0, 0, 0};
  if (m < M) {
    const int b = m / a.n_c, c = m % a.n_c;
    const float* src = a.h + (int64_t)b * a.h_stride + (int64_t)c * g.hidden + k;
    const floatx4 x0 = reinterpret_cast<const floatx4*>(src)[0];
    const floatx4 x1 = reinterpret_cast<const floatx4*>(src)[1];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const float x = e < 4 ? x0[e] : x1[e - 4];
      const uint16_t hb = f32_to_bf16(x);
      hi[e] = hb;
      lo[e] = f32_to_bf16(x - bf16_to_f32(hb));
    }
  }
  reinterpret_cast<u16x8*>(a.hhi)[i] = hi;
  if (a.hlo) reinterpret_cast<u16x8*>(a.hlo)[i] = lo;
}

// ------------------------------------------------------- screen, bf16 MFMA --
// Block: 4 * NG wavefronts; wave w owns vocab columns [32(w%4), +32) of a
// 128-column tile and row blocks (w/4)*RB/NG .. +RB/NG of the 32*RB-row tile
// (NG = 2 gives each SIMD two wavefronts to overlap LDS latency and barriers).
// Hidden is consumed in 64-wide chunks ("stages") that flow from HBM straight
// into LDS (LDS-DMA, issued from asm with explicit waits, see common.hpp)
// through an NST-deep ring: NST-1 stages are in flight while one is
// multiplied, one barrier per stage.  The stream rate is set by the bytes in
// flight, so the ring is as deep as LDS allows (the epilogue's reduction
// buffer reuses it) and a stage has no padding: an LDS row is the 8 16-byte
// units of 64 hidden elements, unit u of row r stored at u ^ ((r >> 1) & 7),
// which spreads the MFMA operand reads of 16 consecutive rows over distinct
// banks.  Every wavefront issues the same number of 1 KiB DMA blocks, so the
// ring waits are constants.
// With n_split > 1 the hidden dimension is split over blockIdx.z: every split
// writes its partial logits and the decision kernel sums them in split order
// (an in-kernel last-block reduction would need device-scope fences, which
// write back and invalidate a whole L2).
template <int RB, int NG, bool kLo>
struct ScreenStage {
  static constexpr int NW = 4 * NG;                                // wavefronts per block
  static constexpr int THREADS = NW * kWave;
  static constexpr int RBW = RB / NG;                              // row blocks per wavefront
  static_assert(RB % NG == 0, "row blocks must split evenly over the row groups");
  static constexpr int RU = kKChunk / 8;                           // 16-byte units per LDS row
  static_assert(RU == 8, "the swizzle assumes 8 units per row");
  static constexpr int W_BLOCKS = kVocabTile * RU / kWave;         // 16
  static constexpr int H_BLOCKS = 32 * RB * RU / kWave;
  static constexpr int BLOCKS = W_BLOCKS + H_BLOCKS * (kLo ? 2 : 1);
  static constexpr int LPW = BLOCKS / NW;                          // loads per wavefront per stage
  static_assert(BLOCKS % NW == 0, "DMA blocks must split evenly over the wavefronts");
  static constexpr int ELEMS = BLOCKS * kWave * 8;                 // bf16 elements per stage
  static constexpr int H_OFF = W_BLOCKS * kWave * 8;               // element offsets in a stage
  static constexpr int L_OFF = H_OFF + H_BLOCKS * kWave * 8;
  static constexpr int FIT = 160 * 1024 / (ELEMS * 2);
  static constexpr int NST = FIT >= 5 ? 5 : FIT;                   // ring depth
  static_assert(NST >= 2, "a stage must fit twice");
  static_assert(NST * ELEMS * 2 >= 4 * 32 * RB * (int)sizeof(Top3), "the reduction buffer reuses the ring");
};

// Physical unit of logical unit u in LDS row r.
__device__ __attribute__((always_inline)) inline int swz(int r, int u) { return u ^ ((r >> 1) & 7); }

// Per-lane byte offsets of this wavefront's DMA units, relative to the
// stage's W base (W row v0) or h base (row m0), and the kind of each slot
// (0 W, 1 h hi, 2 h lo).  Lane l of block blk fills physical unit q = 64 blk
// + l (row q / 8, position q % 8) with the logical unit stored there.
template <class S>
__device__ __attribute__((always_inline)) inline void screen_offsets(int wave, int lane, int hidden, int V, int v0, uint32_t* off, int* kind) {
#pragma unroll
  for (int i = 0; i < S::LPW; ++i) {
    const int blk = wave * S::LPW + i;
    if (blk < S::W_BLOCKS) {
      const int q = blk * kWave + lane;
      const int r = q / S::RU, u = swz(r, q % S::RU);
      off[i] = (uint32_t)((min(v0 + r, V - 1) - v0) * hidden + u * 8) * 2u;
      kind[i] = 0;
    } else {
      const int hb = (blk - S::W_BLOCKS) % S::H_BLOCKS;
      const int q = hb * kWave + lane;
      const int r = q / S::RU, u = swz(r, q % S::RU);
      off[i] = (uint32_t)(r * hidden + u * 8) * 2u;
      kind[i] = blk - S::W_BLOCKS >= S::H_BLOCKS ? 2 : 1;
    }
  }
}

template <class S>
__device__ __attribute__((always_inline)) inline void screen_dma(const uint16_t* wb, const uint16_t* hb, const uint16_t* lb, int wave,
                                  const uint32_t* off, const int* kind, uint32_t stage_lds) {
#pragma unroll
  for (int i = 0; i < S::LPW; ++i) {
    const int blk = wave * S::LPW + i;
    const uint16_t* base = kind[i] == 1 ? hb : (kind[i] == 2 ? lb : wb);
    dma16_at(base, off[i], stage_lds + blk * 1024u);
  }
}

template <int LPW, int AHEAD>
__device__ __attribute__((always_inline)) inline void screen_wait(int younger) {
  static_assert(AHEAD <= 4, "waits are spelled out for up to four stages ahead");
  if (younger >= 3 && AHEAD >= 4) ring_wait<3 * LPW>();
  else if (younger >= 2 && AHEAD >= 3) ring_wait<2 * LPW>();
  else if (younger >= 1 && AHEAD >= 2) ring_wait<LPW>();
  else ring_wait<0>();
}

template <int RB, int NG, bool kLo>
__global__ __launch_bounds__(4 * NG * kWave) void k_screen_bf16(Geometry g, VocabArgs a, int M, int n_split) {
  using S = ScreenStage<RB, NG, kLo>;
  constexpr int MT = 32 * RB;
  constexpr int RBW = S::RBW;
  constexpr int AHEAD = S::NST - 1;
  __shared__ __align__(1024) uint16_t ring[S::NST][S::ELEMS];
  Top3 (*red)[MT] = reinterpret_cast<Top3 (*)[MT]>(&ring[0][0]);   // after the stages are consumed

  const int vt = blockIdx.x;
  const int mt = blockIdx.y;
  const int split = blockIdx.z;
  const int v0 = vt * kVocabTile;
  const int m0 = mt * MT;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  const int wv = wave % 4;                  // vocab block of the tile
  const int rb0 = (wave / 4) * RBW;         // first row block of this wavefront
  const int lane = threadIdx.x % kWave;
  const int half = lane / 32, l32 = lane % 32;
  const int k_len = g.hidden / n_split;
  const int k_beg = split * k_len;
  const int n_chunks = k_len / kKChunk;
  const uint16_t* wrow = static_cast<const uint16_t*>(a.w) + (int64_t)v0 * g.hidden + k_beg;
  const uint16_t* hrow = a.hhi + (int64_t)m0 * g.hidden + k_beg;
  const uint16_t* lrow = kLo ? a.hlo + (int64_t)m0 * g.hidden + k_beg : hrow;

  floatx16 acc[RBW];
#pragma unroll
  for (int rb = 0; rb < RBW; ++rb)
#pragma unroll
    for (int e = 0; e < 16; ++e) acc[rb][e] = 0.f;

  uint32_t off[S::LPW];
  int kind[S::LPW];
  screen_offsets<S>(wave, lane, g.hidden, g.V, v0, off, kind);
  const uint32_t ring_lds = lds_addr(&ring[0][0]);
  for (int c = 0; c < AHEAD && c < n_chunks; ++c)
    screen_dma<S>(wrow + c * kKChunk, hrow + c * kKChunk, lrow + c * kKChunk, wave, off, kind,
                  ring_lds + c * (S::ELEMS * 2));
  // element offsets of this lane's operand rows and units for k-step t:
  // rows 32 wv + l32 (W) and 32 rb0 + l32 (h), logical unit 2t + half
  int woff[kKChunk / 16], hoff[kKChunk / 16];
#pragma unroll
  for (int t = 0; t < kKChunk / 16; ++t) {
    woff[t] = ((32 * wv + l32) * S::RU + swz(l32, 2 * t + half)) * 8;
    hoff[t] = ((32 * rb0 + l32) * S::RU + swz(l32, 2 * t + half)) * 8;
  }
  for (int ci = 0; ci < n_chunks; ++ci) {
    screen_wait<S::LPW, AHEAD>(n_chunks - 1 - ci);
    ring_barrier();
    const int nxt = ci + AHEAD;
    if (nxt < n_chunks)
      screen_dma<S>(wrow + nxt * kKChunk, hrow + nxt * kKChunk, lrow + nxt * kKChunk, wave, off, kind,
                    ring_lds + (nxt % S::NST) * (S::ELEMS * 2));
    // the stage's operands are all read before its MFMAs (one LDS latency per
    // stage instead of one per MFMA)
    const uint16_t* st = ring[ci % S::NST];
    bf16x8 wf[kKChunk / 16], hf[kKChunk / 16][RBW], lf[kKChunk / 16][RBW];
#pragma unroll
    for (int t = 0; t < kKChunk / 16; ++t) {
      wf[t] = *reinterpret_cast<const bf16x8*>(st + woff[t]);
#pragma unroll
      for (int rb = 0; rb < RBW; ++rb) {
        hf[t][rb] = *reinterpret_cast<const bf16x8*>(st + S::H_OFF + hoff[t] + rb * 32 * S::RU * 8);
        if (kLo) lf[t][rb] = *reinterpret_cast<const bf16x8*>(st + S::L_OFF + hoff[t] + rb * 32 * S::RU * 8);
      }
    }
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int t = 0; t < kKChunk / 16; ++t) {
#pragma unroll
      for (int rb = 0; rb < RBW; ++rb) {
        acc[rb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(wf[t], hf[t][rb], acc[rb], 0, 0, 0);
        if (kLo) acc[rb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(wf[t], lf[t][rb], acc[rb], 0, 0, 0);
      }
    }
  }

  // lane holds z for row m0 + 32(rb0 + rb) + l32 and vocab v0 + 32wv + 8jj + 4half + ii
  if (n_split > 1 || a.emit) {
    float* zp = a.zpart;
#pragma unroll
    for (int rb = 0; rb < RBW; ++rb) {
      const int r = m0 + 32 * (rb0 + rb) + l32;
      if (r < M) {
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) {
          const int v = v0 + 32 * wv + 8 * jj + 4 * half;
          floatx4 q = {acc[rb][4 * jj], acc[rb][4 * jj + 1], acc[rb][4 * jj + 2], acc[rb][4 * jj + 3]};
          *reinterpret_cast<floatx4*>(zp + ((int64_t)split * M + r) * a.v_pad + v) = q;
        }
      }
    }
    return;                                   // the decision kernel folds the splits (or the caller reads z)
  }

  __syncthreads();                            // every wavefront is done with the ring
#pragma unroll
  for (int rb = 0; rb < RBW; ++rb) {
    float vals[16];
    int idx[16];
    const int r = m0 + 32 * (rb0 + rb) + l32;
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      const int jj = e / 4, ii = e % 4;
      const int v = v0 + 32 * wv + 8 * jj + 4 * half + ii;
      idx[e] = v;
      vals[e] = v < g.V ? acc[rb][e] : kNegInf;
      if (a.logits && r < M && v < g.V) a.logits[(int64_t)r * g.V + v] = acc[rb][e];
    }
    Top3 t = summarize<16>(vals, idx);
    t = top3_merge(t, top3_shfl_xor(t, 32));
    if (half == 0) red[wv][32 * (rb0 + rb) + l32] = t;
  }
  __syncthreads();
  if (threadIdx.x < MT) {
    const int r = threadIdx.x;
    Top3 t = red[0][r];
#pragma unroll
    for (int w = 1; w < 4; ++w) t = top3_merge(t, red[w][r]);
    const int n_vt = (g.V + kVocabTile - 1) / kVocabTile;
    if (m0 + r < a.m_pad) store_partial(a.partials + ((int64_t)(m0 + r) * n_vt + vt) * 8, t);
  }
}

// ------------------------------------------- screen, wide vocabulary tiles --
// For large vocabularies the h rows are the bigger stream (a 128 x 128 block
// moves the W tile once and its h tile, hi and lo, once per vocab tile), so a
// block takes 512 vocab columns: 8 wavefronts = 4 vocab groups (one 128-column
// partial tile each, 4 MFMA blocks wide) x 2 row groups.  Hidden goes in
// 32-wide stages (LDS rows of 4 16-byte units, unit u of row r stored at
// u ^ ((r >> 2) & 3): conflict-free operand reads), 3-4 stages deep.  Each
// wavefront holds complete 128-column tiles of its rows, so the epilogue's
// per-tile partials need no cross-wavefront reduction.
constexpr int kWideTile = 512;
constexpr int kWideK = 32;

template <int RB, bool kLo>
struct WideStage {
  static constexpr int NW = 8;
  static constexpr int RBW = RB / 2;                              // row blocks per wavefront
  static constexpr int RU = kWideK / 8;                           // units per LDS row
  static constexpr int W_BLOCKS = kWideTile * RU / kWave;         // 32
  static constexpr int H_BLOCKS = 32 * RB * RU / kWave;
  static constexpr int BLOCKS = W_BLOCKS + H_BLOCKS * (kLo ? 2 : 1);
  static constexpr int LPW = BLOCKS / NW;
  static_assert(BLOCKS % NW == 0, "DMA blocks must split evenly over the wavefronts");
  static constexpr int ELEMS = BLOCKS * kWave * 8;
  static constexpr int H_OFF = W_BLOCKS * kWave * 8;
  static constexpr int L_OFF = H_OFF + H_BLOCKS * kWave * 8;
  static constexpr int NST = 160 * 1024 / (ELEMS * 2) >= 4 ? 4 : 160 * 1024 / (ELEMS * 2);
  static_assert(NST >= 3, "the ring must hold three stages");
};

__device__ __attribute__((always_inline)) inline int swz4(int r, int u) { return u ^ ((r >> 2) & 3); }

template <int RB, bool kLo>
__global__ __launch_bounds__(512) void k_screen_wide(Geometry g, VocabArgs a, int M, int n_split) {
  using S = WideStage<RB, kLo>;
  constexpr int RBW = S::RBW;
  constexpr int AHEAD = S::NST - 1;
  __shared__ __align__(1024) uint16_t ring[S::NST][S::ELEMS];

  // 1-D grid, XCD-aware: blocks i and i + 8k run on one XCD, and the row
  // tiles of a 512-column tile take consecutive slots of one XCD, so they
  // stream the same W rows at about the same time and the second read is an
  // L2 hit instead of another pass over HBM (W is 1 GB for a 128k vocabulary).
  const int n_m = (M + 32 * RB - 1) / (32 * RB);
  const int n_vw = (g.V + kWideTile - 1) / kWideTile;
  const int xcd = blockIdx.x % 8, slot = blockIdx.x / 8;
  const int mt = slot % n_m;
  const int vw = (slot / n_m) * 8 + xcd;          // 512-column tile
  if (vw >= n_vw) return;
  const int split = 0;
  const int v0 = vw * kWideTile;
  const int m0 = mt * 32 * RB;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  const int vg = wave % 4;                       // 128-column partial tile of this wavefront
  const int rb0 = (wave / 4) * RBW;
  const int lane = threadIdx.x % kWave;
  const int half = lane / 32, l32 = lane % 32;
  const int k_len = g.hidden / n_split;
  const int k_beg = split * k_len;
  const int n_chunks = k_len / kWideK;
  // W of chunk c (32 columns): row-major rows v0.. at column k_beg + 32 c, or
  // in the tiled copy half (c & 1) of the 64-column runs of the tile's four
  // 128-row tiles (the run of row tile j at j * hidden * 128 elements), so
  // that each stage reads four contiguous 8 KB pieces instead of 512 rows'
  // 64-byte pieces 8 KB apart (C5: 57.4 -> 54.9 ms per generation)
  const bool tiled = a.wt != nullptr;
  const uint16_t* wrow = tiled ? a.wt + (int64_t)(v0 / kVocabTile) * g.hidden * kVocabTile + (int64_t)k_beg * kVocabTile
                               : static_cast<const uint16_t*>(a.w) + (int64_t)v0 * g.hidden + k_beg;
  const int wstep = tiled ? kVocabTile * kWideK : kWideK;
  const uint16_t* hrow = a.hhi + (int64_t)m0 * g.hidden + k_beg;
  const uint16_t* lrow = kLo ? a.hlo + (int64_t)m0 * g.hidden + k_beg : hrow;

  floatx16 acc[4][RBW];
#pragma unroll
  for (int vb = 0; vb < 4; ++vb)
#pragma unroll
    for (int rb = 0; rb < RBW; ++rb)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[vb][rb][e] = 0.f;

  // DMA units: lane l of block blk fills physical unit q = 64 blk + l
  uint32_t off[S::LPW];
  int kind[S::LPW];
#pragma unroll
  for (int i = 0; i < S::LPW; ++i) {
    const int blk = wave * S::LPW + i;
    if (blk < S::W_BLOCKS) {
      const int q = blk * kWave + lane;
      const int r = q / S::RU, u = swz4(r, q % S::RU);
      off[i] = tiled ? (uint32_t)((r / kVocabTile) * g.hidden * kVocabTile + (r % kVocabTile) * 32 + u * 8) * 2u
                     : (uint32_t)((min(v0 + r, g.V - 1) - v0) * g.hidden + u * 8) * 2u;
      kind[i] = 0;
    } else {
      const int hb = (blk - S::W_BLOCKS) % S::H_BLOCKS;
      const int q = hb * kWave + lane;
      const int r = q / S::RU, u = swz4(r, q % S::RU);
      off[i] = (uint32_t)(r * g.hidden + u * 8) * 2u;
      kind[i] = blk - S::W_BLOCKS >= S::H_BLOCKS ? 2 : 1;
    }
  }
  const uint32_t ring_lds = lds_addr(&ring[0][0]);
  // With one row tile, each 512-column tile walks the hidden dimension from
  // its own starting chunk: at any moment the blocks read W at different
  // offsets within its 8 KB rows instead of all at the same one, which
  // spreads the stream over more HBM channels (measured at 128k columns:
  // 64-row steps 253 -> 218 us).  With two row tiles the pair that shares a
  // column tile keeps the plain order (measured faster: their W reads meet
  // in the cache).  Only the order of the hidden sum changes.
  const int rot = n_m == 1 ? (int)(((unsigned)vw * 37u) % (unsigned)n_chunks) : 0;
  auto issue = [&](int c, uint32_t stage) {
    const int cr = c + rot < n_chunks ? c + rot : c + rot - n_chunks;
#pragma unroll
    for (int i = 0; i < S::LPW; ++i) {
      const int blk = wave * S::LPW + i;
      const uint16_t* base = kind[i] == 1 ? hrow + cr * kWideK : (kind[i] == 2 ? lrow + cr * kWideK : wrow + cr * wstep);
      dma16_at(base, off[i], stage + blk * 1024u);
    }
  };
  for (int c = 0; c < AHEAD && c < n_chunks; ++c) issue(c, ring_lds + c * (S::ELEMS * 2));
  // operand element offsets for k-step t (2 per stage): logical unit 2t + half
  int woff[2], hoff[2];
#pragma unroll
  for (int t = 0; t < 2; ++t) {
    woff[t] = ((128 * vg + l32) * S::RU + swz4(l32, 2 * t + half)) * 8;
    hoff[t] = ((32 * rb0 + l32) * S::RU + swz4(l32, 2 * t + half)) * 8;
  }
  for (int ci = 0; ci < n_chunks; ++ci) {
    screen_wait<S::LPW, AHEAD>(n_chunks - 1 - ci);
    ring_barrier();
    const int nxt = ci + AHEAD;
    if (nxt < n_chunks) issue(nxt, ring_lds + (nxt % S::NST) * (S::ELEMS * 2));
    const uint16_t* st = ring[ci % S::NST];
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      bf16x8 wf[4];
#pragma unroll
      for (int vb = 0; vb < 4; ++vb) wf[vb] = *reinterpret_cast<const bf16x8*>(st + woff[t] + vb * 32 * S::RU * 8);
#pragma unroll
      for (int rb = 0; rb < RBW; ++rb) {
        const bf16x8 hf = *reinterpret_cast<const bf16x8*>(st + S::H_OFF + hoff[t] + rb * 32 * S::RU * 8);
#pragma unroll
        for (int vb = 0; vb < 4; ++vb)
          acc[vb][rb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(wf[vb], hf, acc[vb][rb], 0, 0, 0);
        if (kLo) {
          const bf16x8 lf = *reinterpret_cast<const bf16x8*>(st + S::L_OFF + hoff[t] + rb * 32 * S::RU * 8);
#pragma unroll
          for (int vb = 0; vb < 4; ++vb)
            acc[vb][rb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(wf[vb], lf, acc[vb][rb], 0, 0, 0);
        }
      }
    }
  }

  // lane holds z for row m0 + 32(rb0 + rb) + l32 and vocab v0 + 128 vg + 32 vb + 8jj + 4half + ii
  const int vt = vw * (kWideTile / kVocabTile) + vg;      // 128-column tile index
  if (n_split > 1 || a.emit) {
#pragma unroll
    for (int vb = 0; vb < 4; ++vb)
#pragma unroll
      for (int rb = 0; rb < RBW; ++rb) {
        const int r = m0 + 32 * (rb0 + rb) + l32;
        if (r < M) {
#pragma unroll
          for (int jj = 0; jj < 4; ++jj) {
            const int v = v0 + 128 * vg + 32 * vb + 8 * jj + 4 * half;
            if (v < a.v_pad) {
              floatx4 q = {acc[vb][rb][4 * jj], acc[vb][rb][4 * jj + 1], acc[vb][rb][4 * jj + 2],
                           acc[vb][rb][4 * jj + 3]};
              *reinterpret_cast<floatx4*>(a.zpart + ((int64_t)split * M + r) * a.v_pad + v) = q;
            }
          }
        }
      }
    return;
  }
  const int n_vt = (g.V + kVocabTile - 1) / kVocabTile;
#pragma unroll
  for (int rb = 0; rb < RBW; ++rb) {
    const int r = m0 + 32 * (rb0 + rb) + l32;
    Top3 tt;
#pragma unroll
    for (int vb = 0; vb < 4; ++vb) {
      float vals[16];
      int idx[16];
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int jj = e / 4, ii = e % 4;
        const int v = v0 + 128 * vg + 32 * vb + 8 * jj + 4 * half + ii;
        idx[e] = v;
        vals[e] = v < g.V ? acc[vb][rb][e] : kNegInf;
        if (a.logits && r < M && v < g.V) a.logits[(int64_t)r * g.V + v] = acc[vb][rb][e];
      }
      const Top3 t = summarize<16>(vals, idx);
      tt = vb == 0 ? t : top3_merge(tt, t);
    }
    tt = top3_merge(tt, top3_shfl_xor(tt, 32));
    if (half == 0 && vt < n_vt && r < a.m_pad) store_partial(a.partials + ((int64_t)r * n_vt + vt) * 8, tt);
  }
}

// Insert (v, i) into the rank-ordered top-3 with selects only (no branches:
// the lanes of the reduce push different values).
__device__ __attribute__((always_inline)) inline Top3 top3_push_sel(Top3 t, float v, int i) {
  const bool b1 = ranks_before(v, i, t.v1, t.i1);
  const bool b2 = ranks_before(v, i, t.v2, t.i2);
  const bool b3 = ranks_before(v, i, t.v3, t.i3);
  const float n3 = b2 ? t.v2 : (b3 ? v : t.v3);
  const int j3 = b2 ? t.i2 : (b3 ? i : t.i3);
  const float n2 = b1 ? t.v1 : (b2 ? v : t.v2);
  const int j2 = b1 ? t.i1 : (b2 ? i : t.i2);
  t.v1 = b1 ? v : t.v1;
  t.i1 = b1 ? i : t.i1;
  t.v2 = n2; t.i2 = j2;
  t.v3 = n3; t.i3 = j3;
  return t;
}

// Fold the hidden-split partial logits of one 128-vocab tile for 32 rows:
// thread t: row t/8, vocab columns 16(t%8) .. +16; splits summed in order,
// every split's loads issued before the sums (up to 4 splits).
__global__ __launch_bounds__(256) void k_screen_reduce(Geometry g, VocabArgs a, int M, int n_split) {
  const int vt = blockIdx.x;
  const int r = blockIdx.y * 32 + threadIdx.x / 8;
  const int rr = min(r, M - 1);
  const int c0 = vt * kVocabTile + 16 * (threadIdx.x % 8);
  floatx4 zp[4][4];
#pragma unroll
  for (int sp = 0; sp < 4; ++sp) {
    const floatx4* z = reinterpret_cast<const floatx4*>(a.zpart + ((int64_t)min(sp, n_split - 1) * M + rr) * a.v_pad + c0);
#pragma unroll
    for (int q = 0; q < 4; ++q) zp[sp][q] = z[q];
  }
  float vals[16];
  int idx[16];
#pragma unroll
  for (int q = 0; q < 4; ++q)
#pragma unroll
    for (int ii = 0; ii < 4; ++ii) {
      float z = zp[0][q][ii];
#pragma unroll
      for (int sp = 1; sp < 4; ++sp) z = sp < n_split ? z + zp[sp][q][ii] : z;
      const int v = c0 + 4 * q + ii;
      idx[4 * q + ii] = v;
      if (a.logits && r < M && v < g.V) a.logits[(int64_t)r * g.V + v] = z;
      vals[4 * q + ii] = v < g.V ? z : kNegInf;
    }
  Top3 t;
  t.m = kNegInf; t.se = 0.f;
  t.v1 = t.v2 = t.v3 = kNegInf;
  t.i1 = t.i2 = t.i3 = 0x7fffffff;
#pragma unroll
  for (int e = 0; e < 16; ++e) {
    t.m = fmaxf(t.m, vals[e]);
    t = top3_push_sel(t, vals[e], idx[e]);
  }
  if (t.m != kNegInf) {
#pragma unroll
    for (int e = 0; e < 16; ++e) t.se += expf(vals[e] - t.m);
  }
#pragma unroll
  for (int mask = 1; mask < 8; mask <<= 1) {
    const Top3 o = top3_shfl_xor(t, mask);
    lse_merge(t.m, t.se, o.m, o.se);
    t = top3_push_sel(t, o.v1, o.i1);
    t = top3_push_sel(t, o.v2, o.i2);
    t = top3_push_sel(t, o.v3, o.i3);
  }
  const int n_vt = (g.V + kVocabTile - 1) / kVocabTile;
  if (threadIdx.x % 8 == 0 && r < M) store_partial(a.partials + ((int64_t)r * n_vt + vt) * 8, t);
}

// ------------------------------------------------------------ screen, fp32 --
// Block: 128 vocab x 32 rows; thread t owns vocab {t%32 + 32q} and rows 4(t/32)+0..3.
__global__ __launch_bounds__(256) void k_screen_f32(Geometry g, VocabArgs a, int M) {
  constexpr int KC = 32;
  constexpr int RT = 32;
  __shared__ float ws[kVocabTile][KC + 1];
  __shared__ float hs[RT][KC + 1];
  const int vt = blockIdx.x, mt = blockIdx.y;
  const int v0 = vt * kVocabTile, m0 = mt * RT;
  const int t = threadIdx.x;
  const int tv = t % 32, tr = t / 32;
  const float* w = static_cast<const float*>(a.w);
  float acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = 0.f;
  for (int k0 = 0; k0 < g.hidden; k0 += KC) {
    __syncthreads();
    for (int c = t; c < kVocabTile * KC; c += blockDim.x) {
      const int vr = c / KC, kk = c % KC;
      const int v = min(v0 + vr, g.V - 1);
      ws[vr][kk] = w[(int64_t)v * g.hidden + k0 + kk];
    }
    for (int c = t; c < RT * KC; c += blockDim.x) {
      const int r = c / KC, kk = c % KC;
      const int m = m0 + r;
      float x = 0.f;
      if (m < M) {
        const int b = m / a.n_c, cc = m % a.n_c;
        x = a.h[(int64_t)b * a.h_stride + (int64_t)cc * g.hidden + k0 + kk];
      }
      hs[r][kk] = x;
    }
    __syncthreads();
#pragma unroll 8
    for (int kk = 0; kk < KC; ++kk) {
      float wv[4], hv[4];
#pragma unroll
      for (int q = 0; q < 4; ++q) wv[q] = ws[tv + 32 * q][kk];
#pragma unroll
      for (int i = 0; i < 4; ++i) hv[i] = hs[4 * tr + i][kk];
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int q = 0; q < 4; ++q) acc[i][q] = fmaf(hv[i], wv[q], acc[i][q]);
    }
  }
  const int n_vt = (g.V + kVocabTile - 1) / kVocabTile;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int r = m0 + 4 * tr + i;
    float vals[4];
    int idx[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int v = v0 + tv + 32 * q;
      idx[q] = v;
      vals[q] = v < g.V ? acc[i][q] : kNegInf;
      if (a.logits && r < M && v < g.V) a.logits[(int64_t)r * g.V + v] = acc[i][q];
    }
    Top3 tt = summarize<4>(vals, idx);
#pragma unroll
    for (int mask = 1; mask < 32; mask <<= 1) tt = top3_merge(tt, top3_shfl_xor(tt, mask));
    if (tv == 0 && r < a.m_pad) store_partial(a.partials + ((int64_t)r * n_vt + vt) * 8, tt);
  }
}

// ---------------------------------------------------- decide (merge) --
// One 256-thread block per row.  The decision is the argmax of
// the exact fp32 logits z = h W^T over the whole vocabulary, which the screen
// only approximates; the kernel makes that exact as follows.
//
// 1. Fold the tiles' (max, sum of exp) and take the kCand best of the tiles'
//    top-3 entries (and the next one, v_next).
// 2. Re-score the kCand candidates exactly in fp32 from the fp32 h (each lane
//    a fixed slice of hidden, fixed-order wavefront sum).  z* = best exact.
// 3. Every column that was not re-scored has a screened value of at most
//    D = max(v_next, v3 of each tile whose three entries were all candidates).
//    A screened value differs from the exact logit by at most
//      eps_s = (||h - h_s||_2 + gamma(n_s) ||h_s||_2) * max_v ||W_v||_2
//    (h_s = the screen's rounded copy of h, n_s its accumulation depth;
//    Cauchy-Schwarz), and a re-scored one by eps_e = gamma(n_e) ||h|| max||W_v||.
//    If D + eps_s < z* - eps_e no other column can win.  Otherwise (rare) every
//    tile entry whose screened value reaches tau = z* - eps_e - eps_s is
//    re-scored too, and every column of a tile whose third entry reaches tau
//    (its unseen columns may), after which nothing outside the re-scored set
//    can reach z*.
// 4. conf = exp(z* - M) / sum exp(z - M) over the screened terms, with the
//    re-scored candidates' terms replaced by their exact ones (in double).
// Optional per-row certificate (trace) and per-context counters record the
// rows that needed step 3's extra re-scoring and the rows whose two best exact
// logits lie within 2 eps_e of each other (a tie at fp32 precision).
struct Cand {
  float v;
  int i;
};

template <typename WT>
struct W8;
template <>
struct W8<uint16_t> {
  static __device__ __attribute__((always_inline)) inline void load(const uint16_t* p, float* out) {
    const u16x8 r = *reinterpret_cast<const u16x8*>(p);
#pragma unroll
    for (int e = 0; e < 8; ++e) out[e] = bf16_to_f32(r[e]);
  }
};
template <>
struct W8<float> {
  static __device__ __attribute__((always_inline)) inline void load(const float* p, float* out) {
    const floatx4 a = reinterpret_cast<const floatx4*>(p)[0];
    const floatx4 b = reinterpret_cast<const floatx4*>(p)[1];
#pragma unroll
    for (int e = 0; e < 4; ++e) { out[e] = a[e]; out[4 + e] = b[e]; }
  }
};

// A rank-ordered candidate list, passed and returned by value (an array
// behind a pointer or reference would be kept in memory).
struct CandList {
  Cand c[kCand];
};

// Insert (v, i) into the sorted list (rank order), dropping the last; selects only.
__device__ __attribute__((always_inline)) inline CandList cand_insert(CandList l, float v, int i) {
#pragma unroll
  for (int k = 0; k < kCand; ++k) {
    const bool sw = ranks_before(v, i, l.c[k].v, l.c[k].i);
    const float tv = l.c[k].v;
    const int ti = l.c[k].i;
    l.c[k].v = sw ? v : tv;
    l.c[k].i = sw ? i : ti;
    v = sw ? tv : v;
    i = sw ? ti : i;
  }
  return l;
}

// (max, sum of exp) over the whole wavefront
__device__ __attribute__((always_inline)) inline void wave_lse(float& m, float& se) {
  static_assert(kWave == 64, "wave");
#define MDM_LSE_STEP(S)                                                   \
  {                                                                       \
    const U2 pm = wave_pair<S>(__float_as_uint(m));                       \
    const U2 ps = wave_pair<S>(__float_as_uint(se));                      \
    float m0 = __uint_as_float(pm.a), s0 = __uint_as_float(ps.a);          \
    lse_merge(m0, s0, __uint_as_float(pm.b), __uint_as_float(ps.b));       \
    m = m0;                                                               \
    se = s0;                                                              \
  }
  MDM_LSE_STEP(0) MDM_LSE_STEP(1) MDM_LSE_STEP(2) MDM_LSE_STEP(3) MDM_LSE_STEP(4) MDM_LSE_STEP(5)
#undef MDM_LSE_STEP
}

__device__ __attribute__((always_inline)) inline float wave_max(float x) {
#pragma unroll
  for (int s = 0; s < 6; ++s) {
    const int o = __shfl_xor(__float_as_int(x), 1 << s);
    x = fmaxf(x, __int_as_float(o));
  }
  return x;
}

// Unmasking in a pre-generated order, fused into the decision (page 3,
// section 3.2: every decoded position is unmasked): the decided token of row
// m = (b, c) is written at its candidate position in the dense sequence.
__device__ __attribute__((always_inline)) inline void unmask_order(const Geometry& g, const VocabArgs& a, int m, int tok) {
  const int b = m / a.n_c, cc = m % a.n_c;
  const int pos = a.cand_pos[(int64_t)b * a.cand_stride + cc];
  if (pos < 0 || pos >= g.seq_len) flag_error(a.err, kErrPos);
  else if (a.seq_tokens) a.seq_tokens[(int64_t)b * g.seq_len + pos] = tok;
}

// gamma(n) = n u / (1 - n u), u = 2^-24: the bound on the relative error of a
// sum of n fp32 roundings
__device__ __attribute__((always_inline)) inline float gamma_f32(float n) {
  const float nu = n * 5.9604645e-8f;
  return nu / (1.f - nu);
}

// Raw 8 elements of a row (16 bytes of bf16 or 32 of fp32) and their values;
// loaded and read through free functions taking and returning values.
template <typename WT>
struct Raw8;
template <>
struct Raw8<uint16_t> {
  u16x8 r;
};
template <>
struct Raw8<float> {
  floatx4 a, b;
};
__device__ __attribute__((always_inline)) inline Raw8<uint16_t> raw8_load(const uint16_t* p) {
  Raw8<uint16_t> x;
  x.r = *reinterpret_cast<const u16x8*>(p);
  return x;
}
__device__ __attribute__((always_inline)) inline Raw8<float> raw8_load(const float* p) {
  Raw8<float> x;
  x.a = reinterpret_cast<const floatx4*>(p)[0];
  x.b = reinterpret_cast<const floatx4*>(p)[1];
  return x;
}
__device__ __attribute__((always_inline)) inline float raw8_at(Raw8<uint16_t> x, int e) { return bf16_to_f32(x.r[e]); }
__device__ __attribute__((always_inline)) inline float raw8_at(Raw8<float> x, int e) { return e < 4 ? x.a[e] : x.b[e - 4]; }

// Lane l's slice of a hidden row: elements [8l + 512j, +8) for j < NIT; the
// addresses are clamped into the row (every load is issued unconditionally)
// and elements past the row are zero.
template <int NIT>
__device__ __attribute__((always_inline)) inline void load_h_slice(const float* row, int lane, int hidden, float (&x)[NIT][8]) {
  Raw8<float> raw[NIT];
#pragma unroll
  for (int j = 0; j < NIT; ++j) raw[j] = raw8_load(row + min(8 * lane + 512 * j, hidden - 8));
#pragma unroll
  for (int j = 0; j < NIT; ++j) {
    const bool ok = 8 * lane + 512 * j < hidden;
#pragma unroll
    for (int e = 0; e < 8; ++e) x[j][e] = ok ? raw8_at(raw[j], e) : 0.f;
  }
}

// Exact fp32 logit of vocabulary column `col` from the wavefront's slices of h:
// lane l takes elements [8l + 512j, +8) in order, the lanes' sums are added in
// a fixed tree (the same order as the candidates' re-score).
template <typename WT, int NIT>
__device__ __attribute__((always_inline)) inline float wave_dot(const float (&hr)[NIT][8], const WT* w, int col, int lane, int hidden) {
  const WT* row = w + (int64_t)col * hidden;
  Raw8<WT> raw[NIT];
#pragma unroll
  for (int j = 0; j < NIT; ++j) raw[j] = raw8_load(row + min(8 * lane + 512 * j, hidden - 8));
  float acc = 0.f;
#pragma unroll
  for (int j = 0; j < NIT; ++j)
#pragma unroll
    for (int e = 0; e < 8; ++e) acc = fmaf(hr[j][e], raw8_at(raw[j], e), acc);
  return group_sum<6>(acc);
}

// Best and runner-up (rank order) of the exact logits seen, updated by value.
struct Best2 {
  float zb;
  int ib;
  float zr;
  int ir;
};
__device__ __attribute__((always_inline)) inline Best2 best2_take(Best2 t, float z, int col) {
  const bool first = ranks_before(z, col, t.zb, t.ib);
  const bool second = !first && ranks_before(z, col, t.zr, t.ir);
  Best2 o;
  o.zr = first ? t.zb : (second ? z : t.zr);
  o.ir = first ? t.ib : (second ? col : t.ir);
  o.zb = first ? z : t.zb;
  o.ib = first ? col : t.ib;
  return o;
}

// Two columns at once (both rows' loads in flight together), each summed
// exactly as wave_dot sums it.
template <typename WT, int NIT>
__device__ __attribute__((always_inline)) inline void wave_dot2(const float (&hr)[NIT][8], const WT* w, int c0, int c1,
                                                                int lane, int hidden, float& z0, float& z1) {
  const WT* row0 = w + (int64_t)c0 * hidden;
  const WT* row1 = w + (int64_t)c1 * hidden;
  Raw8<WT> raw0[NIT], raw1[NIT];
#pragma unroll
  for (int j = 0; j < NIT; ++j) {
    raw0[j] = raw8_load(row0 + min(8 * lane + 512 * j, hidden - 8));
    raw1[j] = raw8_load(row1 + min(8 * lane + 512 * j, hidden - 8));
  }
  float a0 = 0.f, a1 = 0.f;
#pragma unroll
  for (int j = 0; j < NIT; ++j)
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      a0 = fmaf(hr[j][e], raw8_at(raw0[j], e), a0);
      a1 = fmaf(hr[j][e], raw8_at(raw1[j], e), a1);
    }
  z0 = group_sum<6>(a0);
  z1 = group_sum<6>(a1);
}

template <typename WT, int NIT, bool kLo>
__global__ __launch_bounds__(256) void k_decide(Geometry g, VocabArgs a, int M) {
  constexpr bool kF32 = sizeof(WT) == 4;
  __shared__ float s_lse[4][2];
  __shared__ Cand s_c[4][kCand + 1];
  __shared__ float s_red[4][2];
  const int tid = threadIdx.x;
  const int wave = tid / kWave, lane = tid % kWave;
  const int m = blockIdx.x;
  constexpr int tw = kVocabTile;            // vocabulary columns per partial record
  const int n_vt = (g.V + tw - 1) / tw;
  const float* part = a.partials + (int64_t)m * n_vt * 8;
  const WT* w = static_cast<const WT*>(a.w);
  const int b = m / a.n_c, cc = m % a.n_c;
  const float* hrow = a.h + (int64_t)b * a.h_stride + (int64_t)cc * g.hidden;
  const float wmax = *a.wmax;               // loaded early: used after the re-score

  // lane l's slice of h, elements [8l + 512 j, +8) in every wavefront (the
  // layout of every exact re-score below); loaded first, its latency overlaps
  // the fold
  float hr[NIT][8];
  load_h_slice<NIT>(hrow, lane, g.hidden, hr);

  // 1. fold the tiles: (max, sum of exp) and the kCand + 1 best entries
  __shared__ Cand s_best[kCand + 1];
  __shared__ float s_m, s_se;
  if (n_vt <= kWave) {
    // one tile per lane of wavefront 0: its three entries are already in rank order
    if (wave == 0) {
      const int t = min(lane, n_vt - 1);
      const floatx4 p0 = reinterpret_cast<const floatx4*>(part + t * 8)[0];
      const floatx4 p1 = reinterpret_cast<const floatx4*>(part + t * 8)[1];
      const bool own = lane < n_vt;
      float lm = own ? p0[0] : kNegInf, lse = own ? p0[1] : 0.f;
      Cand h3[3] = {{own ? p0[2] : kNegInf, own ? __float_as_int(p0[3]) : 0x7fffffff},
                    {own ? p1[0] : kNegInf, own ? __float_as_int(p1[1]) : 0x7fffffff},
                    {own ? p1[2] : kNegInf, own ? __float_as_int(p1[3]) : 0x7fffffff}};
      wave_lse(lm, lse);
#pragma unroll
      for (int k = 0; k <= kCand; ++k) {
        float bv = h3[0].v;
        int bi = h3[0].i;
        group_argmax<6>(bv, bi);
        if (lane == 0) s_best[k] = Cand{bv, bi};
        const bool pop = bi == h3[0].i && bi != 0x7fffffff;
        h3[0].v = pop ? h3[1].v : h3[0].v; h3[0].i = pop ? h3[1].i : h3[0].i;
        h3[1].v = pop ? h3[2].v : h3[1].v; h3[1].i = pop ? h3[2].i : h3[1].i;
        h3[2].v = pop ? kNegInf : h3[2].v; h3[2].i = pop ? 0x7fffffff : h3[2].i;
      }
      if (lane == 0) { s_m = lm; s_se = lse; }
    }
  } else {
    // several tiles per thread (large vocabularies): sorted insertion, then a
    // block merge of the wavefronts' top-(kCand + 1)
    float lm = kNegInf, lse = 0.f;
    CandList cl;
#pragma unroll
    for (int k = 0; k < kCand; ++k) { cl.c[k].v = kNegInf; cl.c[k].i = 0x7fffffff; }
    // four tiles per thread and pass, every load issued before any is used
    for (int t0 = 0; t0 < n_vt; t0 += 1024) {
      floatx4 p0[4], p1[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int t = min(t0 + u * 256 + tid, n_vt - 1);
        p0[u] = reinterpret_cast<const floatx4*>(part + t * 8)[0];
        p1[u] = reinterpret_cast<const floatx4*>(part + t * 8)[1];
      }
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        if (t0 + u * 256 + tid < n_vt) {
          lse_merge(lm, lse, p0[u][0], p0[u][1]);
          cl = cand_insert(cl, p0[u][2], __float_as_int(p0[u][3]));
          cl = cand_insert(cl, p1[u][0], __float_as_int(p1[u][1]));
          cl = cand_insert(cl, p1[u][2], __float_as_int(p1[u][3]));
        }
      }
    }
    wave_lse(lm, lse);
#pragma unroll
    for (int k = 0; k <= kCand; ++k) {
      float bv = cl.c[0].v;
      int bi = cl.c[0].i;
      group_argmax<6>(bv, bi);
      if (lane == 0) s_c[wave][k] = Cand{bv, bi};
      const bool pop = bi == cl.c[0].i && bi != 0x7fffffff;
#pragma unroll
      for (int q = 0; q < kCand - 1; ++q) {
        cl.c[q].v = pop ? cl.c[q + 1].v : cl.c[q].v;
        cl.c[q].i = pop ? cl.c[q + 1].i : cl.c[q].i;
      }
      cl.c[kCand - 1].v = pop ? kNegInf : cl.c[kCand - 1].v;
      cl.c[kCand - 1].i = pop ? 0x7fffffff : cl.c[kCand - 1].i;
    }
    if (lane == 0) { s_lse[wave][0] = lm; s_lse[wave][1] = lse; }
    __syncthreads();
    if (wave == 0) {
      // block top-(kCand + 1) from the 4 x (kCand + 1) wavefront entries
      // (indices are distinct: each column lives in one tile)
      float cv = kNegInf;
      int ci = 0x7fffffff;
      if (lane < 4 * (kCand + 1)) { cv = s_c[lane / (kCand + 1)][lane % (kCand + 1)].v; ci = s_c[lane / (kCand + 1)][lane % (kCand + 1)].i; }
#pragma unroll
      for (int k = 0; k <= kCand; ++k) {
        float bv = cv;
        int bi = ci;
        group_argmax<6>(bv, bi);
        if (lane == 0) s_best[k] = Cand{bv, bi};
        const bool pop = ci == bi && ci != 0x7fffffff;
        cv = pop ? kNegInf : cv;
        ci = pop ? 0x7fffffff : ci;
      }
      if (lane == 0) {
        float m0 = s_lse[0][0], se0 = s_lse[0][1];
#pragma unroll
        for (int q = 1; q < 4; ++q) lse_merge(m0, se0, s_lse[q][0], s_lse[q][1]);
        s_m = m0; s_se = se0;
      }
    }
  }
  __syncthreads();
  float bestv[kCand + 1];
  int besti[kCand + 1];
#pragma unroll
  for (int k = 0; k <= kCand; ++k) { bestv[k] = s_best[k].v; besti[k] = s_best[k].i; }
  const float lm = s_m, lse = s_se;

  // 2. exact fp32 logits of the candidates: wavefront w re-scores candidates
  //    2w and 2w + 1 (both rows' loads in flight together), in the one
  //    summation order every exact re-score of this kernel uses, so that equal
  //    W rows give bit-identical logits and exact ties go to the lowest index;
  //    every wavefront also forms |h|^2 and |h - h_screen|^2 over its slices
  static_assert(kCand == 8, "two candidates per wavefront");
  float hh = 0.f, dd = 0.f;
  {
    const int ca = besti[2 * wave], cb = besti[2 * wave + 1];
    float za, zb2;
    wave_dot2<WT, NIT>(hr, w, (ca >= 0 && ca < g.V) ? ca : 0, (cb >= 0 && cb < g.V) ? cb : 0, lane, g.hidden, za,
                       zb2);
#pragma unroll
    for (int j = 0; j < NIT; ++j)
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float x = hr[j][e];
        hh = fmaf(x, x, hh);
        if constexpr (!kF32) {
          const float hi = bf16_to_f32(f32_to_bf16(x));
          float r = x - hi;                  // exact (x and hi share the leading bits)
          if constexpr (kLo) r -= bf16_to_f32(f32_to_bf16(r));
          dd = fmaf(r, r, dd);
        }
      }
    hh = group_sum<6>(hh);                   // the same in every wavefront
    dd = group_sum<6>(dd);
    if (lane == 0) {
      s_red[wave][0] = za;
      s_red[wave][1] = zb2;
    }
  }
  __shared__ int s_rescan;
  __syncthreads();
  if (wave != 0) {
    // wavefronts 1-3 are needed again only for the rare block re-scan, which
    // wavefront 0 announces after the barrier below
    __syncthreads();
    if (!s_rescan) return;
  }
  // the exact logits and bounds (the same values in every wavefront that gets here)
  float ze[kCand];
#pragma unroll
  for (int k = 0; k < kCand; ++k) ze[k] = (besti[k] >= 0 && besti[k] < g.V) ? s_red[k / 2][k % 2] : kNegInf;
  // error bounds (rounded up by a small factor for the fp32 evaluation of the norms)
  const float hn = sqrtf(hh) * 1.0001f;
  // accumulation depth of a screened logit: sequential fp32 FMAs (fp32 screen);
  // for the MFMA screen every 32x32x16 step is counted as 17 roundings of up
  // to 2u each (products of bf16 values are exact in fp32; the order and
  // rounding inside an MFMA are not relied on), plus the split sums
  const float n_s = kF32 ? (float)g.hidden + 8.f
                         : 2.f * ((float)(g.hidden / 16) * 17.f * (kLo ? 2.f : 1.f) + 8.f + (float)a.n_split);
  const float eps_s = (sqrtf(dd) * 1.0001f + gamma_f32(n_s) * hn * 1.01f) * wmax;
  // every re-score: 8 NIT sequential FMAs per lane and 6 tree levels (counted as 8)
  const float eps_e = gamma_f32(8.f * NIT + 8.f) * hn * wmax;

  int tb = 0;                        // tracked by value: no indexing by tb
  float zbest = ze[0];
  int ibest = besti[0];
#pragma unroll
  for (int k = 1; k < kCand; ++k)
    if (ranks_before(ze[k], besti[k], zbest, ibest)) { tb = k; zbest = ze[k]; ibest = besti[k]; }

  // 3. the bound on every column left out, and the re-scoring it may call for
  float dmax = bestv[kCand];
  int ctile[kCand];                         // each candidate's tile (one division each, not one per pair)
#pragma unroll
  for (int k = 0; k < kCand; ++k) ctile[k] = besti[k] / tw;
#pragma unroll
  for (int k = 0; k < kCand; ++k) {
    int same = 0;
#pragma unroll
    for (int q = 0; q < kCand; ++q) same += (ctile[q] == ctile[k]) ? 1 : 0;
    // a tile with all three entries among the candidates: its other columns rank after its third
    bool last = true;
#pragma unroll
    for (int q = k + 1; q < kCand; ++q) last = last && (ctile[q] != ctile[k]);
    if (same == 3 && last && besti[k] != 0x7fffffff) dmax = fmaxf(dmax, bestv[k]);
  }
  const bool rescan = dmax != kNegInf && dmax + eps_s >= zbest - eps_e;   // uniform over the block
  if (wave == 0) {
    if (lane == 0) s_rescan = rescan ? 1 : 0;
    __syncthreads();                        // pairs with the barrier wavefronts 1-3 wait at
  }
  int flags = 0;
  float zrun = kNegInf;              // runner-up exact logit among everything re-scored
  int irun = 0x7fffffff;
#pragma unroll
  for (int k = 0; k < kCand; ++k)
    if (k != tb && ranks_before(ze[k], besti[k], zrun, irun)) { zrun = ze[k]; irun = besti[k]; }
  // conf sum relative to the screened maximum lm: exact minus screened terms of
  // the re-scored entries (double, one term per lane, fixed-order sum)
  double extra = 0.0;
  {
    float zk = kNegInf, sk = 0.f;           // lane k < kCand takes candidate k
#pragma unroll
    for (int k = 0; k < kCand; ++k) {
      zk = lane == k ? ze[k] : zk;
      sk = lane == k ? bestv[k] : sk;
    }
    const double term = zk == kNegInf ? 0.0 : exp((double)zk - (double)lm) - exp((double)sk - (double)lm);
#pragma unroll
    for (int k = 0; k < kCand; ++k) extra += __shfl(term, k);
  }

  if (rescan) {
    // Rare.  Every wavefront scans the tile records in order (the same values
    // in each) and takes its turn at the work: the single entries at or above
    // tau go to the wavefronts in turn (entry e to wavefront e mod 4), and the
    // columns of a tile whose third entry reaches tau (its unseen columns may)
    // are shared out two at a time (columns 2w, 2w + 1, 2w + 8, ... to
    // wavefront w).  Every re-score is a wavefront dot (lane l taking elements
    // [8l + 512j, +8), the candidates' order, so eps_e bounds it).  Each
    // wavefront keeps its own best, runner-up and sum of exact-minus-screened
    // terms; wavefront 0 merges them in wavefront order.
    __shared__ Cand s_rb[4][2];
    __shared__ double s_rx[4];
    flags |= 1;
    const float tau = zbest - eps_e - eps_s;
    float dafter = kNegInf;
    // this wavefront's tallies: wavefront 0 starts from the candidates'
    Best2 t2 = wave == 0 ? Best2{zbest, ibest, zrun, irun} : Best2{kNegInf, 0x7fffffff, kNegInf, 0x7fffffff};
    double ex = wave == 0 ? extra : 0.0;
    int turn = 0;                              // single entries seen so far (uniform)
    for (int t0 = 0; t0 < n_vt; t0 += kWave) {
      const int t = t0 + lane;
      float v[3] = {kNegInf, kNegInf, kNegInf};
      int ix[3] = {0x7fffffff, 0x7fffffff, 0x7fffffff};
      if (t < n_vt) {
        const floatx4 p0 = reinterpret_cast<const floatx4*>(part + t * 8)[0];
        const floatx4 p1 = reinterpret_cast<const floatx4*>(part + t * 8)[1];
        v[0] = p0[2]; ix[0] = __float_as_int(p0[3]);
        v[1] = p1[0]; ix[1] = __float_as_int(p1[1]);
        v[2] = p1[2]; ix[2] = __float_as_int(p1[3]);
      }
      const bool full = t < n_vt && v[2] >= tau;
      if (!full) dafter = fmaxf(dafter, v[2]);          // the tile's unseen columns
#pragma unroll
      for (int q = 0; q < 3; ++q) {
        bool is_cand = false;
#pragma unroll
        for (int k = 0; k < kCand; ++k) is_cand = is_cand || (besti[k] == ix[q]);
        const bool want = v[q] >= tau && !is_cand && ix[q] >= 0 && ix[q] < g.V;
        if (!want && !is_cand) dafter = fmaxf(dafter, v[q]);
        uint64_t mask = __ballot(want);       // the same in every wavefront
        while (mask) {
          const int src = __builtin_ctzll(mask);
          mask &= mask - 1;
          const int col = __shfl(ix[q], src);
          const float scr = __shfl(v[q], src);
          if ((turn & 3) == wave) {
            const float z = wave_dot<WT, NIT>(hr, w, col, lane, g.hidden);
            ex += exp((double)z - (double)lm) - exp((double)scr - (double)lm);
            t2 = best2_take(t2, z, col);
          }
          ++turn;
        }
      }
      uint64_t fmask = __ballot(full);        // the same in every wavefront
      while (fmask) {
        flags |= 2;
        const int src = __builtin_ctzll(fmask);
        fmask &= fmask - 1;
        const int tile = t0 + src;
        // the tile's three entries were re-scored above (all reach tau) or are
        // candidates; its other columns are re-scored here, their screened
        // terms staying in the conf sum (only the decision uses them)
        const int e0 = __shfl(ix[0], src), e1 = __shfl(ix[1], src), e2 = __shfl(ix[2], src);
        for (int j = 2 * wave; j < tw; j += 8) {
          const int c0 = tile * tw + j, c1 = c0 + 1;
          float z0, z1;
          wave_dot2<WT, NIT>(hr, w, min(c0, g.V - 1), min(c1, g.V - 1), lane, g.hidden, z0, z1);
          bool ok0 = c0 < g.V && c0 != e0 && c0 != e1 && c0 != e2;
          bool ok1 = j + 1 < tw && c1 < g.V && c1 != e0 && c1 != e1 && c1 != e2;
#pragma unroll
          for (int k = 0; k < kCand; ++k) { ok0 = ok0 && besti[k] != c0; ok1 = ok1 && besti[k] != c1; }
          if (ok0) t2 = best2_take(t2, z0, c0);
          if (ok1) t2 = best2_take(t2, z1, c1);
        }
      }
    }
    if (lane == 0) {
      s_rb[wave][0] = Cand{t2.zb, t2.ib};
      s_rb[wave][1] = Cand{t2.zr, t2.ir};
      s_rx[wave] = ex;
    }
    __syncthreads();
    if (wave != 0) return;
#pragma unroll
    for (int q = 1; q < 4; ++q) {
#pragma unroll
      for (int r = 0; r < 2; ++r)
        if (s_rb[q][r].i != 0x7fffffff) t2 = best2_take(t2, s_rb[q][r].v, s_rb[q][r].i);
      ex += s_rx[q];
    }
    zbest = t2.zb; ibest = t2.ib; zrun = t2.zr; irun = t2.ir; extra = ex;
    dmax = wave_max(dafter);
  }
  if (zrun != kNegInf && zbest - zrun <= 2.f * eps_e) flags |= 4;
  if (dmax == kNegInf || dmax + eps_s < zbest - eps_e) flags |= 8;

  // 4. confidence = exp(z* - lm) / (sum of exp(z - lm)): screened terms with
  //    the re-scored entries' terms replaced by their exact ones
  if (lane == 0) {
    const double tot = (lm == kNegInf ? 0.0 : (double)lse) + extra;
    a.conf[m] = (float)(exp((double)zbest - (double)lm) / tot);
    a.token[m] = ibest;
    if (a.cand_pos) unmask_order(g, a, m, ibest);
    if (a.trace) {
      floatx4 t0 = {zbest, __int_as_float(ibest), zrun, __int_as_float(irun)};
      floatx4 t1 = {dmax, eps_s, eps_e, __int_as_float(flags)};
      reinterpret_cast<floatx4*>(a.trace + (int64_t)m * 8)[0] = t0;
      reinterpret_cast<floatx4*>(a.trace + (int64_t)m * 8)[1] = t1;
    }
    if (a.stats) {
      if (flags & 1) atomicAdd(&a.stats[0], 1u);
      if (flags & 2) atomicAdd(&a.stats[1], 1u);
      if (flags & 4) atomicAdd(&a.stats[2], 1u);
    }
  }
}

template <typename WT, bool kLo>
hipError_t launch_decide_lo(const Geometry& g, const VocabArgs& a, int M, hipStream_t s) {
  const dim3 grid(M), block(256);
  const int nit = (g.hidden + 511) / 512;
  if (nit <= 1) hipLaunchKernelGGL((k_decide<WT, 1, kLo>), grid, block, 0, s, g, a, M);
  else if (nit <= 2) hipLaunchKernelGGL((k_decide<WT, 2, kLo>), grid, block, 0, s, g, a, M);
  else if (nit <= 4) hipLaunchKernelGGL((k_decide<WT, 4, kLo>), grid, block, 0, s, g, a, M);
  else if (nit <= 8) hipLaunchKernelGGL((k_decide<WT, 8, kLo>), grid, block, 0, s, g, a, M);
  else hipLaunchKernelGGL((k_decide<WT, 16, kLo>), grid, block, 0, s, g, a, M);
  return hipGetLastError();
}

template <typename WT>
hipError_t launch_decide(const Geometry& g, const VocabArgs& a, int M, hipStream_t s) {
  if constexpr (!std::is_same<WT, float>::value)
    if (a.hlo) return launch_decide_lo<WT, true>(g, a, M, s);
  return launch_decide_lo<WT, false>(g, a, M, s);
}

// The tiled copy of W (VocabArgs::wt): block (c, rt) writes the 16 KB run of
// row tile rt and 64-column chunk c, unit q = (h, r, u) of the run holding
// W[128 rt + r][64 c + 32 h + 8 u .. +8] (zero past V); stores contiguous.
__global__ __launch_bounds__(256) void k_tile_w(Geometry g, const uint16_t* w, uint16_t* wt) {
  const int c = blockIdx.x, rt = blockIdx.y;
  uint16_t* dst = wt + ((int64_t)rt * (g.hidden / kKChunk) + c) * (kVocabTile * kKChunk);
  for (int q = threadIdx.x; q < kVocabTile * kKChunk / 8; q += 256) {
    const int h = q >> 9, r = (q >> 2) & 127, u = q & 3;
    const int row = rt * kVocabTile + r;
    u16x8 x;
#pragma unroll
    for (int e = 0; e < 8; ++e) x[e] = 0;
    if (row < g.V) x = *reinterpret_cast<const u16x8*>(w + (int64_t)row * g.hidden + c * kKChunk + h * 32 + u * 8);
    *reinterpret_cast<u16x8*>(dst + q * 8) = x;
  }
}

// max_v ||W_v||_2 (rounded up) into *out: one wavefront per vocabulary row
template <typename WT>
__global__ __launch_bounds__(256) void k_row_norm_max(Geometry g, const WT* w, float* out) {
  const int row = blockIdx.x * 4 + threadIdx.x / kWave, lane = threadIdx.x % kWave;
  if (row >= g.V) return;
  float acc = 0.f;
  for (int e0 = 8 * lane; e0 < g.hidden; e0 += 512) {
    float wv[8];
    W8<WT>::load(w + (int64_t)row * g.hidden + e0, wv);
#pragma unroll
    for (int e = 0; e < 8; ++e) acc = fmaf(wv[e], wv[e], acc);
  }
  acc = group_sum<6>(acc);
  // the fp32 sum of squares is within gamma(hidden/64 + 6) of exact: round up
  const float nrm = sqrtf(acc * (1.f + gamma_f32((float)(g.hidden / 64 + 8)))) * 1.00001f;
  if (lane == 0) atomicMax(reinterpret_cast<unsigned*>(out), __float_as_uint(nrm));
}

}  // namespace

hipError_t launch_vocab(const Geometry& g, const VocabArgs& a, hipStream_t s) {
  const int M = g.B * a.n_c;
  if (M <= 0) return hipSuccess;
  const int n_vt = (g.V + kVocabTile - 1) / kVocabTile;
  if (g.fp32) {
    dim3 grid(n_vt, (M + 31) / 32);
    hipLaunchKernelGGL(k_screen_f32, grid, dim3(256), 0, s, g, a, M);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    VocabArgs da = a;
    da.n_split = 1;
    return launch_decide<float>(g, da, M, s);
  }
  const int n_wide = (g.V + kWideTile - 1) / kWideTile;
  int rb = M <= 32 ? 1 : (M <= 64 ? 2 : 4);
  // hi + lo steps of 129-192 rows on a large vocabulary: three 64-row tiles
  // (768 blocks) instead of two 128-row tiles padded to 256 rows (C5 55.9 ->
  // 54.9 ms per generation; 64-row tiles for the 65-128 or 193-256-row steps
  // measured slower)
  if (a.hlo && M > 128 && M <= 192 && n_wide >= 128) rb = 2;
  // bf16(h) steps of 65-256 rows below the wide regime: 32-row tiles for
  // 65-128 rows and 64-row tiles for 129-256 rows (192-256 blocks either way)
  // without a hidden split, so no split-reduce launch.  Same box, per
  // generation: 129-256 rows C3 7.62 -> 7.57 and 7.90 -> 7.75, C4 6.86 ->
  // 6.77 and 7.10 -> 6.84 ms; 65-128 rows on top C3 7.77 -> 7.73, C4 6.89 ->
  // 6.83 ms (64-row tiles there gained less; 32-row tiles for 33-64 rows, or
  // 64-row tiles up to 320 or 384 rows, measured no gain or slower).
  const bool unsplit = !a.hlo && M > 64 && M <= 256 && n_wide * ((M + 127) / 128) < kScreenTargetBlocks * 7 / 8;
  if (unsplit) rb = M <= 128 ? 1 : 2;
  const int mt_rows = 32 * rb;
  const int m_tiles = (M + mt_rows - 1) / mt_rows;
  // wide vocabulary tiles when they alone give (nearly) a block per compute unit
  const bool wide = (rb == 4 || (rb == 2 && a.hlo)) && n_wide * m_tiles >= kScreenTargetBlocks * 7 / 8;
  VocabArgs pa = a;
  pa.m_pad = ((M + 63) / 64) * 64;
  if (m_tiles * mt_rows > pa.m_pad) pa.m_pad = m_tiles * mt_rows;
  if (wide) {
    hipError_t ew;
    if (!a.prepacked) {
      const int64_t n8w = (int64_t)pa.m_pad * g.hidden / 8;
      hipLaunchKernelGGL(k_pack, dim3((unsigned)((n8w + 255) / 256)), dim3(256), 0, s, g, pa, M);
      ew = hipGetLastError();
      if (ew != hipSuccess) return ew;
    }
    dim3 wgrid((unsigned)(((n_wide + 7) / 8) * 8 * m_tiles));
    if (rb == 4) {
      if (a.hlo) hipLaunchKernelGGL((k_screen_wide<4, true>), wgrid, dim3(512), 0, s, g, pa, M, 1);
      else hipLaunchKernelGGL((k_screen_wide<4, false>), wgrid, dim3(512), 0, s, g, pa, M, 1);
    } else {
      hipLaunchKernelGGL((k_screen_wide<2, true>), wgrid, dim3(512), 0, s, g, pa, M, 1);
    }
    ew = hipGetLastError();
    if (ew != hipSuccess) return ew;
    pa.n_split = 1;
    return launch_decide<uint16_t>(g, pa, M, s);
  }
  int n_split = 1;
  const int chunks = g.hidden / kKChunk;
  while (!unsplit && n_split < 4 && M <= kSplitMaxRows && n_vt * m_tiles * n_split * 2 <= kScreenTargetBlocks &&
         chunks % (n_split * 2) == 0 &&
         (int64_t)n_split * 2 * M * pa.v_pad * 4 <= a.zpart_bytes)
    n_split *= 2;
  hipError_t e;
  if (!a.prepacked) {
    const int64_t n8 = (int64_t)pa.m_pad * g.hidden / 8;
    hipLaunchKernelGGL(k_pack, dim3((unsigned)((n8 + 255) / 256)), dim3(256), 0, s, g, pa, M);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  dim3 grid(n_vt, m_tiles, n_split);
#define MDM_SCREEN(RB, NG)                                                                              \
  if (a.hlo) hipLaunchKernelGGL((k_screen_bf16<RB, NG, true>), grid, dim3(ScreenStage<RB, NG, true>::THREADS), 0, s, \
                                g, pa, M, n_split);                                                      \
  else hipLaunchKernelGGL((k_screen_bf16<RB, NG, false>), grid, dim3(ScreenStage<RB, NG, false>::THREADS), 0, s,     \
                          g, pa, M, n_split)
  if (rb == 1) { MDM_SCREEN(1, 1); }
  else if (rb == 2) { MDM_SCREEN(2, 2); }
  else { MDM_SCREEN(4, 2); }
#undef MDM_SCREEN
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  // split partial logits are summed in split order by the reduce launch,
  // whose grid spreads the sums over the vocabulary tiles
  if (n_split > 1) {
    hipLaunchKernelGGL(k_screen_reduce, dim3(n_vt, (M + 31) / 32), dim3(256), 0, s, g, pa, M, n_split);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    pa.n_split = n_split;              // the accumulation depth of the screened values
    pa.zpart = nullptr;                // the decision reads the reduced tile records
    return launch_decide<uint16_t>(g, pa, M, s);
  }
  pa.n_split = n_split;
  return launch_decide<uint16_t>(g, pa, M, s);
}

hipError_t launch_row_norm_max(const Geometry& g, const void* w, float* out, hipStream_t s) {
  const dim3 grid((g.V + 3) / 4), block(256);
  if (g.fp32) hipLaunchKernelGGL((k_row_norm_max<float>), grid, block, 0, s, g, static_cast<const float*>(w), out);
  else hipLaunchKernelGGL((k_row_norm_max<uint16_t>), grid, block, 0, s, g, static_cast<const uint16_t*>(w), out);
  return hipGetLastError();
}

hipError_t launch_tile_w(const Geometry& g, const void* w, uint16_t* wt, hipStream_t s) {
  static_assert(kVocabTile == 128 && kKChunk == 64 && kWideK == 32 && kWideTile == 4 * kVocabTile,
                "the tiled copy's run layout");
  if (g.fp32 || g.hidden % kKChunk) return hipErrorInvalidValue;
  const dim3 grid(g.hidden / kKChunk, (unsigned)(tiled_w_elems(g.V, g.hidden) / ((size_t)kVocabTile * g.hidden)));
  hipLaunchKernelGGL(k_tile_w, grid, dim3(256), 0, s, g, static_cast<const uint16_t*>(w), wt);
  return hipGetLastError();
}

hipError_t launch_project(const Geometry& g, const ProjArgs& p, hipStream_t s) {
  const int M = g.B * p.n_q;
  if (M <= 0) return hipSuccess;
  // the screen as a plain product: "vocabulary" = the N projection rows
  Geometry gp = g;
  gp.V = (g.H + 2 * g.Hkv) * g.D;
  VocabArgs va{};
  va.w = p.w;
  va.h = p.h;
  va.h_stride = p.h_stride;
  va.n_c = p.n_q;
  va.hhi = p.hhi;
  va.hlo = p.hlo;
  va.zpart = p.z;
  va.v_pad = p.n_pad;
  va.emit = 1;
  const int rb = M <= 32 ? 1 : (M <= 64 ? 2 : 4);
  const int mt_rows = 32 * rb;
  const int m_tiles = (M + mt_rows - 1) / mt_rows;
  va.m_pad = m_tiles * mt_rows;
  const int64_t n8 = (int64_t)va.m_pad * g.hidden / 8;
  hipLaunchKernelGGL(k_pack, dim3((unsigned)((n8 + 255) / 256)), dim3(256), 0, s, gp, va, M);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  // Large steps take the 512-column tiles of the wide screen (each h operand
  // read from LDS feeds four MFMA blocks instead of one) once they alone give
  // at least kProjWideBlocks blocks; below that the 128-column tiles keep
  // every compute unit busy.  Same-box two-layer C3 generations: 26.1 against
  // 26.9 ms at 192 blocks, 26.2 at 128, 27.7 at 64.
  const int n_wide = gp.V / kWideTile;
  if (rb == 4 && gp.V % kWideTile == 0 && n_wide * m_tiles >= kProjWideBlocks) {
    hipLaunchKernelGGL((k_screen_wide<4, true>), dim3((unsigned)(((n_wide + 7) / 8) * 8 * m_tiles)), dim3(512), 0, s,
                       gp, va, M, 1);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    return launch_rope_scatter(g, p, M, s);
  }
  dim3 grid(p.n_pad / kVocabTile, m_tiles, 1);
  if (rb == 1) hipLaunchKernelGGL((k_screen_bf16<1, 1, true>), grid, dim3(ScreenStage<1, 1, true>::THREADS), 0, s, gp, va, M, 1);
  else if (rb == 2) hipLaunchKernelGGL((k_screen_bf16<2, 2, true>), grid, dim3(ScreenStage<2, 2, true>::THREADS), 0, s, gp, va, M, 1);
  else hipLaunchKernelGGL((k_screen_bf16<4, 2, true>), grid, dim3(ScreenStage<4, 2, true>::THREADS), 0, s, gp, va, M, 1);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  return launch_rope_scatter(g, p, M, s);
}

}  // namespace mdm
