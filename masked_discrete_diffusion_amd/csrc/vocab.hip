// Logits for the decoded subset only, with max-probability confidence and
// argmax (page 1, key design 1; page 3, section 3.2).
//
// 1. pack:   fp32 h rows of the decoded subset -> bf16 hi (and lo = bf16(h - hi))
//            in a dense [m_pad][hidden] operand, zero rows past M.
// 2. screen: z^T = W h^T on bf16 MFMA (32x32x16), one 128-column vocab tile by
//            32/64/128 rows per block; the epilogue keeps per (row, tile) the maximum,
//            the sum of exp(z - max) and the two best (value, index) pairs, and
//            never writes the logits (unless asked to, for validation).
//            fp32 mode: the same tile and epilogue with fp32 VALU products.
// 3. merge:  per row, combine the tiles (max, sum of exp), take the kTopK best
//            candidates, recompute their logits exactly in fp32 from the fp32 h,
//            decide the argmax among them (lowest index on ties) and the
//            confidence exp(z_best - M) / sum exp(z - M), with the candidates'
//            screened terms replaced by their exact ones.
#include "common.hpp"
#include "kernels.hpp"

namespace mdm {

namespace {

constexpr float kNegInf = -__builtin_inff();
constexpr int kKChunk = 64;        // hidden elements per LDS stage
constexpr int kScreenTargetBlocks = 256;   // split hidden until about this many blocks

struct Top2 {
  float m;      // running maximum
  float se;     // sum of exp(z - m)
  float v1, v2;
  int i1, i2;
};

__device__ inline void top2_push(Top2& t, float v, int i) {
  if (ranks_before(v, i, t.v1, t.i1)) {
    t.v2 = t.v1; t.i2 = t.i1; t.v1 = v; t.i1 = i;
  } else if (ranks_before(v, i, t.v2, t.i2)) {
    t.v2 = v; t.i2 = i;
  }
}

__device__ inline Top2 top2_merge(const Top2& a, const Top2& b) {
  Top2 r;
  r.m = fmaxf(a.m, b.m);
  r.se = (a.m == kNegInf ? 0.f : a.se * expf(a.m - r.m)) + (b.m == kNegInf ? 0.f : b.se * expf(b.m - r.m));
  r.v1 = a.v1; r.i1 = a.i1; r.v2 = a.v2; r.i2 = a.i2;
  top2_push(r, b.v1, b.i1);
  top2_push(r, b.v2, b.i2);
  return r;
}

__device__ inline Top2 top2_shfl_xor(const Top2& t, int mask) {
  Top2 o;
  o.m = __shfl_xor(t.m, mask);
  o.se = __shfl_xor(t.se, mask);
  o.v1 = __shfl_xor(t.v1, mask);
  o.v2 = __shfl_xor(t.v2, mask);
  o.i1 = __shfl_xor(t.i1, mask);
  o.i2 = __shfl_xor(t.i2, mask);
  return o;
}

// Fold a lane's logits into (max, sumexp, top2): values[n] with indices idx[n].
template <int N>
__device__ inline Top2 summarize(const float* vals, const int* idx) {
  Top2 t;
  t.m = kNegInf; t.se = 0.f; t.v1 = kNegInf; t.v2 = kNegInf; t.i1 = 0x7fffffff; t.i2 = 0x7fffffff;
#pragma unroll
  for (int e = 0; e < N; ++e) {
    t.m = fmaxf(t.m, vals[e]);
    top2_push(t, vals[e], idx[e]);
  }
  if (t.m != kNegInf) {
#pragma unroll
    for (int e = 0; e < N; ++e) t.se += expf(vals[e] - t.m);
  }
  return t;
}

__device__ inline void store_partial(float* p, const Top2& t) {
  floatx4 a = {t.m, t.se, t.v1, __int_as_float(t.i1)};
  floatx4 c = {t.v2, __int_as_float(t.i2), 0.f, 0.f};
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
// writes its partial logits and k_screen_reduce sums them in split order and
// runs the epilogue (a separate launch: an in-kernel last-block reduction
// needs device-scope fences, which write back and invalidate a whole L2).
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
  static_assert(NST * ELEMS * 2 >= 4 * 32 * RB * (int)sizeof(float) * 6, "the reduction buffer reuses the ring");
};

// Physical unit of logical unit u in LDS row r.
__device__ inline int swz(int r, int u) { return u ^ ((r >> 1) & 7); }

// Per-lane byte offsets of this wavefront's DMA units, relative to the
// stage's W base (W row v0) or h base (row m0), and the kind of each slot
// (0 W, 1 h hi, 2 h lo).  Lane l of block blk fills physical unit q = 64 blk
// + l (row q / 8, position q % 8) with the logical unit stored there.
template <class S>
__device__ inline void screen_offsets(int wave, int lane, int hidden, int V, int v0, uint32_t* off, int* kind) {
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
__device__ inline void screen_dma(const uint16_t* wb, const uint16_t* hb, const uint16_t* lb, int wave,
                                  const uint32_t* off, const int* kind, uint32_t stage_lds) {
#pragma unroll
  for (int i = 0; i < S::LPW; ++i) {
    const int blk = wave * S::LPW + i;
    const uint16_t* base = kind[i] == 1 ? hb : (kind[i] == 2 ? lb : wb);
    dma16_at(base, off[i], stage_lds + blk * 1024u);
  }
}

template <int LPW, int AHEAD>
__device__ inline void screen_wait(int younger) {
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
  Top2 (*red)[MT] = reinterpret_cast<Top2 (*)[MT]>(&ring[0][0]);   // after the stages are consumed

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
    const uint16_t* st = ring[ci % S::NST];
#pragma unroll
    for (int t = 0; t < kKChunk / 16; ++t) {
      const bf16x8 wf = *reinterpret_cast<const bf16x8*>(st + woff[t]);
#pragma unroll
      for (int rb = 0; rb < RBW; ++rb) {
        const bf16x8 hf = *reinterpret_cast<const bf16x8*>(st + S::H_OFF + hoff[t] + rb * 32 * S::RU * 8);
        acc[rb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(wf, hf, acc[rb], 0, 0, 0);
        if (kLo) {
          const bf16x8 lf = *reinterpret_cast<const bf16x8*>(st + S::L_OFF + hoff[t] + rb * 32 * S::RU * 8);
          acc[rb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(wf, lf, acc[rb], 0, 0, 0);
        }
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
    return;                                   // k_screen_reduce folds the splits (or the caller reads z)
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
    Top2 t = summarize<16>(vals, idx);
    t = top2_merge(t, top2_shfl_xor(t, 32));
    if (half == 0) red[wv][32 * (rb0 + rb) + l32] = t;
  }
  __syncthreads();
  if (threadIdx.x < MT) {
    const int r = threadIdx.x;
    Top2 t = red[0][r];
#pragma unroll
    for (int w = 1; w < 4; ++w) t = top2_merge(t, red[w][r]);
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

__device__ inline int swz4(int r, int u) { return u ^ ((r >> 2) & 3); }

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
  const uint16_t* wrow = static_cast<const uint16_t*>(a.w) + (int64_t)v0 * g.hidden + k_beg;
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
      off[i] = (uint32_t)((min(v0 + r, g.V - 1) - v0) * g.hidden + u * 8) * 2u;
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
  auto issue = [&](int c, uint32_t stage) {
#pragma unroll
    for (int i = 0; i < S::LPW; ++i) {
      const int blk = wave * S::LPW + i;
      const uint16_t* base = kind[i] == 1 ? hrow : (kind[i] == 2 ? lrow : wrow);
      dma16_at(base + c * kWideK, off[i], stage + blk * 1024u);
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
  if (n_split > 1) {
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
    Top2 tt;
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
      const Top2 t = summarize<16>(vals, idx);
      tt = vb == 0 ? t : top2_merge(tt, t);
    }
    tt = top2_merge(tt, top2_shfl_xor(tt, 32));
    if (half == 0 && vt < n_vt && r < a.m_pad) store_partial(a.partials + ((int64_t)r * n_vt + vt) * 8, tt);
  }
}

// Fold the hidden-split partial logits of one 128-vocab tile for 32 rows:
// thread t: row t/8, vocab columns 16(t%8) .. +16; splits summed in order.
__global__ __launch_bounds__(256) void k_screen_reduce(Geometry g, VocabArgs a, int M, int n_split) {
  const int vt = blockIdx.x;
  const int r = blockIdx.y * 32 + threadIdx.x / 8;
  const int c0 = vt * kVocabTile + 16 * (threadIdx.x % 8);
  float vals[16];
  int idx[16];
#pragma unroll
  for (int e = 0; e < 16; ++e) vals[e] = 0.f;
  if (r < M) {
    for (int sp = 0; sp < n_split; ++sp) {
      const floatx4* z = reinterpret_cast<const floatx4*>(a.zpart + ((int64_t)sp * M + r) * a.v_pad + c0);
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const floatx4 v = z[q];
#pragma unroll
        for (int ii = 0; ii < 4; ++ii) vals[4 * q + ii] += v[ii];
      }
    }
  }
#pragma unroll
  for (int e = 0; e < 16; ++e) {
    const int v = c0 + e;
    idx[e] = v;
    if (a.logits && r < M && v < g.V) a.logits[(int64_t)r * g.V + v] = vals[e];
    if (v >= g.V) vals[e] = kNegInf;
  }
  Top2 t = summarize<16>(vals, idx);
#pragma unroll
  for (int mask = 1; mask < 8; mask <<= 1) t = top2_merge(t, top2_shfl_xor(t, mask));
  const int n_vt = (g.V + kVocabTile - 1) / kVocabTile;
  if (threadIdx.x % 8 == 0 && r < a.m_pad) store_partial(a.partials + ((int64_t)r * n_vt + vt) * 8, t);
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
    Top2 tt = summarize<4>(vals, idx);
#pragma unroll
    for (int mask = 1; mask < 32; mask <<= 1) tt = top2_merge(tt, top2_shfl_xor(tt, mask));
    if (tv == 0 && r < a.m_pad) store_partial(a.partials + ((int64_t)r * n_vt + vt) * 8, tt);
  }
}

// ----------------------------------------------------- merge and re-score --
// One block (4 wavefronts) per row: the threads fold the tiles' (max, sum of
// exp, top-2) partials, the block keeps the kTopK best candidates, and all
// threads re-score the candidates together exactly in fp32 from the fp32 h
// (each thread a slice of hidden for every candidate, then a fixed-order
// reduction).
struct Cand {
  float v;
  int i;
};

template <typename WT>
struct W8;
template <>
struct W8<uint16_t> {
  static __device__ inline void load(const uint16_t* p, float* out) {
    const u16x8 r = *reinterpret_cast<const u16x8*>(p);
#pragma unroll
    for (int e = 0; e < 8; ++e) out[e] = bf16_to_f32(r[e]);
  }
};
template <>
struct W8<float> {
  static __device__ inline void load(const float* p, float* out) {
    const floatx4 a = reinterpret_cast<const floatx4*>(p)[0];
    const floatx4 b = reinterpret_cast<const floatx4*>(p)[1];
#pragma unroll
    for (int e = 0; e < 4; ++e) { out[e] = a[e]; out[4 + e] = b[e]; }
  }
};

__device__ inline void cand_insert(Cand* c, float v, int i) {
#pragma unroll
  for (int k = 0; k < kTopK; ++k) {
    if (ranks_before(v, i, c[k].v, c[k].i)) {
      const Cand t = c[k];
      c[k].v = v; c[k].i = i;
      v = t.v; i = t.i;
    }
  }
}

// (max, sum of exp) of two partial sums
__device__ inline void lse_merge(float& m, float& se, float om, float ose) {
  const float nm = fmaxf(m, om);
  se = (m == kNegInf ? 0.f : se * expf(m - nm)) + (om == kNegInf ? 0.f : ose * expf(om - nm));
  m = nm;
}

// (max, sum of exp) over the whole wavefront
__device__ inline void wave_lse(float& m, float& se) {
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

// Unmasking in a pre-generated order, fused into the merge (page 3, section
// 3.2: every decoded position is unmasked): the decided token of row
// m = (b, c) is written at its candidate position in the dense sequence.
__device__ inline void unmask_order(const Geometry& g, const VocabArgs& a, int m, int tok) {
  const int b = m / a.n_c, cc = m % a.n_c;
  const int pos = a.cand_pos[(int64_t)b * a.cand_stride + cc];
  if (pos < 0 || pos >= g.seq_len) flag_error(a.err, kErrPos);
  else if (a.seq_tokens) a.seq_tokens[(int64_t)b * g.seq_len + pos] = tok;
}

// 4. decision and confidence (wave 0).  The exact logit replaces the screened
//    term of each candidate in the sum of exp; the double exps are taken one
//    per lane and summed by lane 0 in a fixed order.
template <typename WT>
__device__ inline void merge_decide(const Geometry& g, const VocabArgs& a, int m, int lane, const float* bestv,
                                    const int* besti, const float* s_m, const float* s_se,
                                    const float (*s_dot)[kTopK]) {
  float bm = s_m[0], bse = s_se[0];
  for (int wv = 1; wv < 4; ++wv) lse_merge(bm, bse, s_m[wv], s_se[wv]);
  float ze[kTopK];
#pragma unroll
  for (int k = 0; k < kTopK; ++k) {
    const bool ok = besti[k] >= 0 && besti[k] < g.V;
    ze[k] = ok ? ((s_dot[0][k] + s_dot[1][k]) + (s_dot[2][k] + s_dot[3][k])) : kNegInf;
  }
  int tb = 0;
#pragma unroll
  for (int k = 1; k < kTopK; ++k)
    if (ranks_before(ze[k], besti[k], ze[tb], besti[tb])) tb = k;
  double mx = bm;
#pragma unroll
  for (int k = 0; k < kTopK; ++k)
    if (ze[k] != kNegInf) mx = fmax(mx, (double)ze[k]);
  // lane 0: the screened sum; lane 1+k: exact term k; lane 1+kTopK+k: screened term k
  double arg = (double)bm - mx;
#pragma unroll
  for (int k = 0; k < kTopK; ++k) {
    if (lane == 1 + k) arg = (double)ze[k] - mx;
    if (lane == 1 + kTopK + k) arg = (double)bestv[k] - mx;
  }
  const double ex = exp(arg);
  double terms[2 * kTopK + 1];
#pragma unroll
  for (int q = 0; q <= 2 * kTopK; ++q) terms[q] = __shfl(ex, q);
  if (lane == 0) {
    double tot = (double)bse * terms[0];
#pragma unroll
    for (int k = 0; k < kTopK; ++k) {
      if (ze[k] == kNegInf) continue;
      tot += terms[1 + k] - terms[1 + kTopK + k];
    }
    double et = terms[1];
#pragma unroll
    for (int k = 1; k < kTopK; ++k)
      if (tb == k) et = terms[1 + k];
    a.conf[m] = (float)(et / tot);
    a.token[m] = besti[tb];
    if (a.cand_pos) unmask_order(g, a, m, besti[tb]);
  }
}

template <typename WT>
__global__ __launch_bounds__(256) void k_merge(Geometry g, VocabArgs a, int M, int n_split) {
  __shared__ float s_m[4], s_se[4];
  __shared__ Cand s_c[4][kTopK];
  __shared__ float s_dot[4][kTopK];
  const int m = blockIdx.x;
  const int wave = threadIdx.x / kWave, lane = threadIdx.x % kWave;
  const int n_vt = (g.V + kVocabTile - 1) / kVocabTile;
  const float* part = a.partials + (int64_t)m * n_vt * 8;

  // 1. fold the tiles: (max, sum of exp) and each lane's kTopK best
  float lm = kNegInf, lse = 0.f;
  Cand c[kTopK];
#pragma unroll
  for (int k = 0; k < kTopK; ++k) { c[k].v = kNegInf; c[k].i = 0x7fffffff; }
  if (n_split > 1) {
    // hidden was split over blocks and not reduced: sum this row's partial
    // logits in split order (the screened logits), 16 columns per thread at a time
    for (int c0 = 16 * threadIdx.x; c0 < g.V; c0 += 16 * blockDim.x) {
      float vals[16];
      int idx[16];
#pragma unroll
      for (int e = 0; e < 16; ++e) vals[e] = 0.f;
      for (int sp = 0; sp < n_split; ++sp) {
        const floatx4* z = reinterpret_cast<const floatx4*>(a.zpart + ((int64_t)sp * M + m) * a.v_pad + c0);
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const floatx4 v = z[q];
#pragma unroll
          for (int ii = 0; ii < 4; ++ii) vals[4 * q + ii] += v[ii];
        }
      }
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int v = c0 + e;
        idx[e] = v;
        if (a.logits && v < g.V) a.logits[(int64_t)m * g.V + v] = vals[e];
        if (v >= g.V) vals[e] = kNegInf;
      }
      const Top2 t = summarize<16>(vals, idx);
      lse_merge(lm, lse, t.m, t.se);
#pragma unroll
      for (int e = 0; e < 16; ++e) cand_insert(c, vals[e], idx[e]);
    }
  } else {
    for (int tile = threadIdx.x; tile < n_vt; tile += blockDim.x) {
      const floatx4 p0 = reinterpret_cast<const floatx4*>(part + tile * 8)[0];
      const floatx4 p1 = reinterpret_cast<const floatx4*>(part + tile * 8)[1];
      lse_merge(lm, lse, p0[0], p0[1]);
      cand_insert(c, p0[2], __float_as_int(p0[3]));
      cand_insert(c, p1[0], __float_as_int(p1[1]));
    }
  }
  wave_lse(lm, lse);
  // wave top-K: K rounds of a (value desc, index asc) argmax; the owner pops
#pragma unroll
  for (int k = 0; k < kTopK; ++k) {
    float bv = c[0].v;
    int bi = c[0].i;
    group_argmax<6>(bv, bi);
    if (lane == 0) s_c[wave][k] = Cand{bv, bi};
    if (bi == c[0].i && bi != 0x7fffffff) {
#pragma unroll
      for (int q = 0; q < kTopK - 1; ++q) c[q] = c[q + 1];
      c[kTopK - 1].v = kNegInf;
      c[kTopK - 1].i = 0x7fffffff;
    }
  }
  if (lane == 0) { s_m[wave] = lm; s_se[wave] = lse; }
  __syncthreads();

  // 2. block top-K, taken by every wave from the 4 x kTopK wave candidates in
  //    lanes 0..15 (indices are distinct: each vocab column lives in one tile)
  float bestv[kTopK];
  int besti[kTopK];
  {
    float cv = kNegInf;
    int ci = 0x7fffffff;
    if (lane < 4 * kTopK) { cv = s_c[lane / kTopK][lane % kTopK].v; ci = s_c[lane / kTopK][lane % kTopK].i; }
#pragma unroll
    for (int k = 0; k < kTopK; ++k) {
      float bv = cv;
      int bi = ci;
      group_argmax<4>(bv, bi);
      bestv[k] = __int_as_float(__builtin_amdgcn_readfirstlane(__float_as_int(bv)));
      besti[k] = __builtin_amdgcn_readfirstlane(bi);
      if (ci == besti[k] && ci != 0x7fffffff) { cv = kNegInf; ci = 0x7fffffff; }
    }
  }

  // 3. exact fp32 logits of the candidates: thread t takes hidden elements
  //    [8t + 2048j, +8) for all kTopK candidates, so the h row is read once;
  //    then a fixed-order sum (lanes, then waves)
  const int b = m / a.n_c, cc = m % a.n_c;
  const float* hrow = a.h + (int64_t)b * a.h_stride + (int64_t)cc * g.hidden;
  const WT* w = static_cast<const WT*>(a.w);
  const WT* wr[kTopK];
#pragma unroll
  for (int k = 0; k < kTopK; ++k) {
    const bool ok = besti[k] >= 0 && besti[k] < g.V;
    wr[k] = w + (int64_t)(ok ? besti[k] : 0) * g.hidden;
  }
  float dot[kTopK];
#pragma unroll
  for (int k = 0; k < kTopK; ++k) dot[k] = 0.f;
#pragma unroll 2
  for (int e0 = 8 * threadIdx.x; e0 < g.hidden; e0 += 8 * 256) {
    const floatx4 h0 = reinterpret_cast<const floatx4*>(hrow + e0)[0];
    const floatx4 h1 = reinterpret_cast<const floatx4*>(hrow + e0)[1];
#pragma unroll
    for (int k = 0; k < kTopK; ++k) {
      float wv[8];
      W8<WT>::load(wr[k] + e0, wv);
#pragma unroll
      for (int e = 0; e < 4; ++e) dot[k] = fmaf(h0[e], wv[e], dot[k]);
#pragma unroll
      for (int e = 0; e < 4; ++e) dot[k] = fmaf(h1[e], wv[4 + e], dot[k]);
    }
  }
#pragma unroll
  for (int k = 0; k < kTopK; ++k) dot[k] = group_sum<6>(dot[k]);
  if (lane == 0)
#pragma unroll
    for (int k = 0; k < kTopK; ++k) s_dot[wave][k] = dot[k];
  __syncthreads();
  if (wave == 0) merge_decide<WT>(g, a, m, lane, bestv, besti, s_m, s_se, s_dot);
}


}  // namespace

hipError_t launch_vocab(const Geometry& g, const VocabArgs& a, hipStream_t s) {
  const int M = g.B * a.n_c;
  if (M <= 0) return hipSuccess;
  const int n_vt = (g.V + kVocabTile - 1) / kVocabTile;
  const dim3 merge_grid(M);
  if (g.fp32) {
    dim3 grid(n_vt, (M + 31) / 32);
    hipLaunchKernelGGL(k_screen_f32, grid, dim3(256), 0, s, g, a, M);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL((k_merge<float>), merge_grid, dim3(256), 0, s, g, a, M, 1);
    return hipGetLastError();
  }
  const int rb = M <= 32 ? 1 : (M <= 64 ? 2 : 4);
  const int mt_rows = 32 * rb;
  const int m_tiles = (M + mt_rows - 1) / mt_rows;
  const int n_wide = (g.V + kWideTile - 1) / kWideTile;
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
    hipLaunchKernelGGL((k_merge<uint16_t>), merge_grid, dim3(256), 0, s, g, pa, M, 1);
    return hipGetLastError();
  }
  int n_split = 1;
  const int chunks = g.hidden / kKChunk;
  while (n_split < 8 && n_vt * m_tiles * n_split * 2 <= kScreenTargetBlocks && chunks % (n_split * 2) == 0 &&
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
  // a two-way split is summed by the merge itself (two partial rows per
  // merge row); wider splits of fewer rows go through the reduce launch,
  // whose grid spreads the sums over the vocabulary tiles
  const bool fold = n_split == 2;
  if (n_split > 1 && !fold) {
    hipLaunchKernelGGL(k_screen_reduce, dim3(n_vt, (M + 31) / 32), dim3(256), 0, s, g, pa, M, n_split);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL((k_merge<uint16_t>), merge_grid, dim3(256), 0, s, g, pa, M, fold ? n_split : 1);
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
  dim3 grid(p.n_pad / kVocabTile, m_tiles, 1);
  if (rb == 1) hipLaunchKernelGGL((k_screen_bf16<1, 1, true>), grid, dim3(ScreenStage<1, 1, true>::THREADS), 0, s, gp, va, M, 1);
  else if (rb == 2) hipLaunchKernelGGL((k_screen_bf16<2, 2, true>), grid, dim3(ScreenStage<2, 2, true>::THREADS), 0, s, gp, va, M, 1);
  else hipLaunchKernelGGL((k_screen_bf16<4, 2, true>), grid, dim3(ScreenStage<4, 2, true>::THREADS), 0, s, gp, va, M, 1);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  return launch_rope_scatter(g, p, M, s);
}

}  // namespace mdm
