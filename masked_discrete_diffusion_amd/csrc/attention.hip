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
// bf16 path (per wavefront: 32 query rows of one head):
//   S^T = K Q^T with v_mfma_f32_32x32x16_bf16 (K from LDS, Q^T in registers),
//   fp32 online softmax (one partner exchange per 64-key tile for the row max),
//   P split into bf16 hi + lo, O^T += V^T P_hi^T + V^T P_lo^T (V^T from LDS),
//   fp32 output.  The key rows of the K operand are permuted so that each
//   lane's eight P values for a k-step are eight consecutive keys, which makes
//   the V^T operand a single 16-byte LDS read.
// fp32 path: the same mask with fp32 VALU arithmetic (validation mode).
#include "common.hpp"
#include "kernels.hpp"

namespace mdm {

namespace {

constexpr float kNegInf = -__builtin_inff();
constexpr float kLog2e = 1.4426950408889634f;

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

struct ChunkPlan {
  int chunks_d;    // chunks of D rows
  int n_chunks;    // D chunks then C|R chunks
  int per_block;   // chunks (wavefronts) per block
  int blocks;      // blocks per (sequence, head)
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
template <int D>
__global__ __launch_bounds__(512) void k_attn_bf16(Geometry g, AttnArgs a, ChunkPlan cp) {
  constexpr int KT = kKeyTile;          // 64 keys per LDS stage
  constexpr int KPAD = D + 8;           // K row stride in LDS (elements): conflict-free b128 reads
  constexpr int VPAD = KT + 8;          // V^T row stride in LDS (elements)
  constexpr int NKS = D / 16;           // k-steps of the QK^T product
  constexpr int NDB = D / 32;           // 32-row blocks of O^T
  __shared__ __align__(16) uint16_t ks[KT * KPAD];
  __shared__ __align__(16) uint16_t vs[D * VPAD];

  const int blk = blockIdx.x;
  const int j = blk % cp.blocks;
  const int bh = blk / cp.blocks;
  const int h = bh % g.H;
  const int b = bh / g.H;
  const int kvh = h / (g.H / g.Hkv);
  const int wave = threadIdx.x / kWave;
  const int lane = threadIdx.x % kWave;
  const int half = lane / 32;
  const int l32 = lane % 32;

  const int ch0 = j * cp.per_block;
  const int ch_last = min(cp.n_chunks, ch0 + cp.per_block) - 1;
  const int kend = (ch_last >= cp.chunks_d) ? a.S + a.n_c + a.n_r : a.S;
  const int ch = ch0 + wave;
  const bool active = ch < cp.n_chunks;
  int row_base = 0, row_end = 0, wlen = 0;
  if (active) chunk_rows(a, cp, 32, ch, row_base, row_end, wlen);
  const int row = row_base + l32;
  const bool rvalid = active && row < row_end;

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
  float m_run = -1e30f, l_run = 0.f;
  const float sc = kLog2e / sqrtf((float)D);

  const uint16_t* kc = static_cast<const uint16_t*>(a.kc) + ((int64_t)b * g.Hkv + kvh) * g.slots * D;
  const uint16_t* vc = static_cast<const uint16_t*>(a.vc) + ((int64_t)b * g.Hkv + kvh) * D * g.slots;

  for (int kt = 0; kt < kend; kt += KT) {
    __syncthreads();
    for (int c = threadIdx.x; c < KT * D / 8; c += blockDim.x) {
      const int kr = c / (D / 8), kcol = c % (D / 8);
      *reinterpret_cast<u16x8*>(ks + kr * KPAD + kcol * 8) =
          *reinterpret_cast<const u16x8*>(kc + (int64_t)(kt + kr) * D + kcol * 8);
    }
    for (int c = threadIdx.x; c < D * KT / 8; c += blockDim.x) {
      const int dr = c / (KT / 8), kcol = c % (KT / 8);
      *reinterpret_cast<u16x8*>(vs + dr * VPAD + kcol * 8) =
          *reinterpret_cast<const u16x8*>(vc + (int64_t)dr * g.slots + kt + kcol * 8);
    }
    __syncthreads();
    if (!active || kt >= wlen) continue;

    floatx16 s[2];
#pragma unroll
    for (int sub = 0; sub < 2; ++sub) {
#pragma unroll
      for (int e = 0; e < 16; ++e) s[sub][e] = 0.f;
#pragma unroll
      for (int t = 0; t < NKS; ++t) {
        const bf16x8 kf = *reinterpret_cast<const bf16x8*>(ks + (sub * 32 + krow) * KPAD + 16 * t + 8 * half);
        s[sub] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf, qf[t], s[sub], 0, 0, 0);
      }
    }
    const bool edge = kt + KT > wlen;
    float mt = kNegInf;
#pragma unroll
    for (int sub = 0; sub < 2; ++sub)
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int jj = e / 4, ii = e % 4;
        const int key = kt + 32 * sub + 16 * (jj / 2) + 8 * half + 4 * (jj % 2) + ii;
        float v = s[sub][e];
        if (edge && key >= wlen) v = kNegInf;
        s[sub][e] = v;
        mt = fmaxf(mt, v);
      }
    mt = fmaxf(mt, __shfl_xor(mt, 32));
    const float m_new = fmaxf(m_run, mt);
    const float alpha = exp2f((m_run - m_new) * sc);
    const float msc = m_new * sc;
    float lsum = 0.f;
#pragma unroll
    for (int sub = 0; sub < 2; ++sub)
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const float p = exp2f(fmaf(s[sub][e], sc, -msc));
        s[sub][e] = p;
        lsum += p;
      }
    l_run = l_run * alpha + lsum;
    m_run = m_new;
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[db][e] *= alpha;

#pragma unroll
    for (int sub = 0; sub < 2; ++sub)
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        u16x8 hi, lo;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const float p = s[sub][8 * u + e];
          const uint16_t hb = f32_to_bf16(p);
          hi[e] = hb;
          lo[e] = f32_to_bf16(p - bf16_to_f32(hb));
        }
        const bf16x8 phi = __builtin_bit_cast(bf16x8, hi);
        const bf16x8 plo = __builtin_bit_cast(bf16x8, lo);
        const int key0 = kt + 32 * sub + 16 * u + 8 * half;
#pragma unroll
        for (int db = 0; db < NDB; ++db) {
          u16x8 vraw = *reinterpret_cast<const u16x8*>(vs + (32 * db + l32) * VPAD + 32 * sub + 16 * u + 8 * half);
          if (edge) {
#pragma unroll
            for (int e = 0; e < 8; ++e) vraw[e] = (key0 + e < wlen) ? vraw[e] : (uint16_t)0;
          }
          const bf16x8 vf = __builtin_bit_cast(bf16x8, vraw);
          acc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf, phi, acc[db], 0, 0, 0);
          acc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf, plo, acc[db], 0, 0, 0);
        }
      }
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

  for (int kt = 0; kt < wlen; kt += KT) {
    __syncthreads();
    for (int c = t; c < KT * D; c += blockDim.x) {
      const int kr = c / D, dd = c % D;
      ks[kr][dd] = kc[(int64_t)(kt + kr) * D + dd];
    }
    for (int c = t; c < D * KT; c += blockDim.x) {
      const int dd = c / KT, kr = c % KT;
      const float v = vc[(int64_t)dd * g.slots + kt + kr];
      vs[dd][kr] = (kt + kr < wlen) ? v : 0.f;
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
    dim3 grid(g.B * g.H * cp.n_chunks);
    if (g.D == 128) hipLaunchKernelGGL((k_attn_f32<128>), grid, dim3(256), 0, s, g, a, cp);
    else hipLaunchKernelGGL((k_attn_f32<64>), grid, dim3(256), 0, s, g, a, cp);
  } else {
    const int max_waves = 8;
    const int nb = (cp.n_chunks + max_waves - 1) / max_waves;
    cp.blocks = nb;
    cp.per_block = (cp.n_chunks + nb - 1) / nb;
    dim3 grid(g.B * g.H * nb);
    dim3 block(kWave * cp.per_block);
    if (g.D == 128) hipLaunchKernelGGL((k_attn_bf16<128>), grid, block, 0, s, g, a, cp);
    else hipLaunchKernelGGL((k_attn_bf16<64>), grid, block, 0, s, g, a, cp);
  }
  return hipGetLastError();
}

}  // namespace mdm
