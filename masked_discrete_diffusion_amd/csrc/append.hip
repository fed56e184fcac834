// KV append: gather key/value rows from the folded tables by token id, rotate
// keys by RoPE at each row's explicit position id, and store them into the
// cache (keys [slot][d]; values transposed [d][slot] so the attention kernel
// streams them key-contiguous).  Used for committed rows (the prompt prefetch
// and the tokens decoded at the previous step) and, once at init, for the keys
// of the mask token at every position and of the registers (page 3, section
// 3.2; page 1, worked example = the paper's Figure 3).
#include "common.hpp"
#include "kernels.hpp"

namespace mdm {

namespace {

constexpr int kRowsPerBlock = 32;

template <typename T>
struct Elem;
template <>
struct Elem<uint16_t> {
  static __device__ float load(const uint16_t* p, int i) { return bf16_to_f32(p[i]); }
  static __device__ uint16_t from_f64(double x) { return f64_to_bf16(x); }
};
template <>
struct Elem<float> {
  static __device__ float load(const float* p, int i) { return p[i]; }
  static __device__ float from_f64(double x) { return (float)x; }
};

template <typename T>
struct Vec16;
template <>
struct Vec16<uint16_t> {   // 16 bf16 = two 16-byte units
  static __device__ inline void load(const uint16_t* p, float* out) {
    const u16x8 x0 = reinterpret_cast<const u16x8*>(p)[0];
    const u16x8 x1 = reinterpret_cast<const u16x8*>(p)[1];
#pragma unroll
    for (int e = 0; e < 8; ++e) { out[e] = bf16_to_f32(x0[e]); out[8 + e] = bf16_to_f32(x1[e]); }
  }
};
template <>
struct Vec16<float> {
  static __device__ inline void load(const float* p, float* out) {
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const floatx4 x = reinterpret_cast<const floatx4*>(p)[q];
#pragma unroll
      for (int e = 0; e < 4; ++e) out[4 * q + e] = x[e];
    }
  }
};

// RoPE of kEpt consecutive elements (kEpt/2 interleaved pairs) from src to dst.
template <typename T, int kEpt>
__device__ inline void rope_store(const T* src, T* dst, const float* cs, const float* sn) {
  static_assert(kEpt % 16 == 0 || kEpt == 8, "kEpt");
  float x[kEpt];
  if constexpr (kEpt >= 16) {
#pragma unroll
    for (int q = 0; q < kEpt / 16; ++q) Vec16<T>::load(src + 16 * q, x + 16 * q);
  } else {
#pragma unroll
    for (int e = 0; e < kEpt; ++e) x[e] = Elem<T>::load(src, e);
  }
  T y[kEpt];
#pragma unroll
  for (int p = 0; p < kEpt / 2; ++p) {
    double r0d, r1d;
    rope_pair(x[2 * p], x[2 * p + 1], cs[p], sn[p], r0d, r1d);
    y[2 * p] = Elem<T>::from_f64(r0d);
    y[2 * p + 1] = Elem<T>::from_f64(r1d);
  }
  if constexpr (sizeof(T) == 2) {
#pragma unroll
    for (int q = 0; q < kEpt / 8; ++q) {
      u16x8 v;
#pragma unroll
      for (int e = 0; e < 8; ++e) v[e] = y[8 * q + e];
      reinterpret_cast<u16x8*>(dst)[q] = v;
    }
  } else {
#pragma unroll
    for (int q = 0; q < kEpt / 4; ++q) {
      floatx4 v;
#pragma unroll
      for (int e = 0; e < 4; ++e) v[e] = y[4 * q + e];
      reinterpret_cast<floatx4*>(dst)[q] = v;
    }
  }
}

// Block: 32 rows of one (sequence, kv head); thread: row t/8, elements
// [D/8 * (t%8), +D/8).  Writes the keys, the transposed values and, with qout,
// the queries of the kv head's G query heads.
template <typename T, int D>
__global__ __launch_bounds__(256) void k_append(Geometry g, AppendArgs a) {
  constexpr int kEpt = D / 8;                 // elements per thread (8 threads per row)
  __shared__ T vs[kRowsPerBlock][D + 2];
  const int b = blockIdx.z;
  const int kvh = blockIdx.y;
  const int r0 = blockIdx.x * kRowsPerBlock;
  const int n_rows = a.n_a + a.n_reg;
  const int t = threadIdx.x;
  const int lr = t / 8, part = t % 8;
  const int r = r0 + lr;
  const bool valid = r < n_rows;

  int id = 0, pos = 0;
  if (valid) {
    if (r < a.n_a) {
      id = a.tok ? a.tok[(int64_t)b * a.stride + r] : g.V;
      pos = a.pos ? a.pos[(int64_t)b * (a.pos_stride ? a.pos_stride : a.stride) + r] : r;
    } else {
      const int j = r - a.n_a;
      id = g.V + 1 + j;
      pos = g.seq_len + j;
    }
    if (id < 0 || id >= g.table_rows) { flag_error(a.err, kErrTok); id = 0; }
    // sequence rows sit at 0..seq_len-1; only the register rows may use the
    // positions after the sequence
    const int pos_end = r < a.n_a ? g.seq_len : g.max_pos;
    if (pos < 0 || pos >= pos_end) { flag_error(a.err, kErrPos); pos = 0; }
  }

  const T* tv = static_cast<const T*>(a.tv);
  T* vc = static_cast<T*>(a.vc);
  const int slot = a.slot0 + r;
  if (valid && (a.kc || a.qout)) {
    float cs[kEpt / 2], sn[kEpt / 2];
    const float* cp = a.rope_cos + (int64_t)pos * (D / 2) + part * (kEpt / 2);
    const float* sp = a.rope_sin + (int64_t)pos * (D / 2) + part * (kEpt / 2);
#pragma unroll
    for (int q = 0; q < kEpt / 8; ++q) {
      const floatx4 c4 = reinterpret_cast<const floatx4*>(cp)[q];
      const floatx4 s4 = reinterpret_cast<const floatx4*>(sp)[q];
#pragma unroll
      for (int e = 0; e < 4; ++e) { cs[4 * q + e] = c4[e]; sn[4 * q + e] = s4[e]; }
    }
    const int64_t head_base = ((int64_t)b * g.Hkv + kvh) * g.slots;
    if (a.kc)
      rope_store<T, kEpt>(static_cast<const T*>(a.tk) + ((int64_t)id * g.Hkv + kvh) * D + part * kEpt,
                          static_cast<T*>(a.kc) + (head_base + slot) * D + part * kEpt, cs, sn);
    if (a.qout) {
      const int G = g.H / g.Hkv;
      for (int gi = 0; gi < G; ++gi) {
        const int h = kvh * G + gi;
        rope_store<T, kEpt>(static_cast<const T*>(a.tq) + ((int64_t)id * g.H + h) * D + part * kEpt,
                            static_cast<T*>(a.qout) + (((int64_t)b * g.H + h) * a.q_rows + r) * D + part * kEpt,
                            cs, sn);
      }
    }
  }
  if (valid) {
    if (vc) {
      const T* vsrc = tv + ((int64_t)id * g.Hkv + kvh) * D + part * kEpt;
#pragma unroll
      for (int e = 0; e < kEpt; ++e) vs[lr][part * kEpt + e] = vsrc[e];
    }
    if (a.cache_pos && kvh == 0 && part == 0) {
      a.cache_pos[(int64_t)b * g.slots + slot] = pos;
      a.cache_tok[(int64_t)b * g.slots + slot] = id;
    }
  }
  if (!vc) return;
  __syncthreads();
  // transposed value store in 64-slot tiles ([slot tile][d][64]): for each d,
  // the block's rows are consecutive slots of one or two tiles
  const int rows_here = min(kRowsPerBlock, n_rows - r0);
  T* vhead = vc + ((int64_t)b * g.Hkv + kvh) * D * g.slots;
#pragma unroll
  for (int e0 = 0; e0 < D * kRowsPerBlock; e0 += 256) {
    const int e = e0 + t;
    const int dd = e / kRowsPerBlock, rr = e % kRowsPerBlock;
    const int sl = a.slot0 + r0 + rr;
    if (rr < rows_here) vhead[((int64_t)(sl / kKeyTile) * D + dd) * kKeyTile + sl % kKeyTile] = vs[rr][dd];
  }
}

// One thread per (kv head, dim, j): j < 8 fills the mask token's value unit,
// every j < r_pad fills one register column (zero past R).
__global__ __launch_bounds__(256) void k_value_tables(Geometry g, const uint16_t* tv, uint16_t* mvt, uint16_t* rvt,
                                                      int r_pad) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t n = (int64_t)g.Hkv * g.D * r_pad;
  if (i >= n) return;
  const int j = (int)(i % r_pad);
  const int col = (int)(i / r_pad);              // kvh * D + d
  const int64_t kvd = (int64_t)g.Hkv * g.D;
  if (j < 8) mvt[(int64_t)col * 8 + j] = tv[(int64_t)g.V * kvd + col];
  rvt[i] = j < g.R ? tv[(int64_t)(g.V + 1 + j) * kvd + col] : (uint16_t)0;
}

// Upper layers: the projected rows z [M][n_pad] (fp32, row m = (b, r) with
// r < n_q) become RoPE'd bf16 queries and keys and bf16 values, scattered to
// where the layer's attention reads them (see ProjArgs).  Thread: 8
// consecutive features of one row (a 16-byte unit of the output).
__global__ __launch_bounds__(256) void k_rope_scatter(Geometry g, ProjArgs a) {
  const int m = blockIdx.y;
  const int b = m / a.n_q, r = m % a.n_q;
  const int unit = blockIdx.x * blockDim.x + threadIdx.x;
  const int D = g.D, hd = g.H * g.D, kd = g.Hkv * g.D;
  if (unit * 8 >= hd + kd) return;
  const int n0 = unit * 8;
  int pos;
  if (r < a.n_d) pos = a.d_pos[(int64_t)b * a.d_stride + r];
  else if (r < a.n_d + a.n_c) pos = a.c_pos[(int64_t)b * a.c_stride + (r - a.n_d)];
  else pos = g.seq_len + (r - a.n_d - a.n_c);
  if (pos < 0 || pos >= g.max_pos) { flag_error(a.err, kErrPos); pos = 0; }
  const float* zr = a.z + (int64_t)m * a.n_pad + n0;
  const floatx4 x0 = reinterpret_cast<const floatx4*>(zr)[0];
  const floatx4 x1 = reinterpret_cast<const floatx4*>(zr)[1];
  const float x[8] = {x0[0], x0[1], x0[2], x0[3], x1[0], x1[1], x1[2], x1[3]};
  u16x8 y;
  {
    const int j = (n0 < hd ? n0 : n0 - hd) % D;            // first dim (even): pairs j/2 .. j/2 + 3
    const float* cs = a.rope_cos + (int64_t)pos * (D / 2) + j / 2;
    const float* sn = a.rope_sin + (int64_t)pos * (D / 2) + j / 2;
#pragma unroll
    for (int p = 0; p < 4; ++p) {
      double r0, r1;
      rope_pair(x[2 * p], x[2 * p + 1], cs[p], sn[p], r0, r1);
      y[2 * p] = f64_to_bf16(r0);
      y[2 * p + 1] = f64_to_bf16(r1);
    }
    if (n0 < hd) {
      const int h = n0 / D;
      *reinterpret_cast<u16x8*>(static_cast<uint16_t*>(a.qbuf) + (((int64_t)b * g.H + h) * a.qbuf_rows + r) * D + j) = y;
      return;
    }
    const int kvh = (n0 - hd) / D;
    uint16_t* dst = r < a.n_d
        ? static_cast<uint16_t*>(a.kc) + (((int64_t)b * g.Hkv + kvh) * g.slots + a.slot0 + r) * D + j
        : static_cast<uint16_t*>(a.tk) + (((int64_t)b * g.Hkv + kvh) * a.t_pad + (r - a.n_d)) * D + j;
    *reinterpret_cast<u16x8*>(dst) = y;
  }
}

__global__ void k_fill_i32(int32_t* p, int32_t v, int n) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) p[i] = v;
}

}  // namespace

hipError_t launch_append(const Geometry& g, const AppendArgs& a, hipStream_t s) {
  const int n_rows = a.n_a + a.n_reg;
  if (n_rows <= 0) return hipSuccess;
  dim3 grid((n_rows + kRowsPerBlock - 1) / kRowsPerBlock, g.Hkv, g.B);
  if (g.fp32) {
    if (g.D == 128) hipLaunchKernelGGL((k_append<float, 128>), grid, dim3(256), 0, s, g, a);
    else hipLaunchKernelGGL((k_append<float, 64>), grid, dim3(256), 0, s, g, a);
  } else {
    if (g.D == 128) hipLaunchKernelGGL((k_append<uint16_t, 128>), grid, dim3(256), 0, s, g, a);
    else hipLaunchKernelGGL((k_append<uint16_t, 64>), grid, dim3(256), 0, s, g, a);
  }
  return hipGetLastError();
}

hipError_t launch_value_tables(const Geometry& g, const void* tv, void* mvt, void* rvt, int r_pad, hipStream_t s) {
  const int64_t n = (int64_t)g.Hkv * g.D * r_pad;
  hipLaunchKernelGGL(k_value_tables, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, g,
                     static_cast<const uint16_t*>(tv), static_cast<uint16_t*>(mvt), static_cast<uint16_t*>(rvt),
                     r_pad);
  return hipGetLastError();
}

// Upper layers, values: block = 32 consecutive query rows of one sequence x
// 64 value features, staged in LDS so that the transposed stores (the cache's
// 64-slot value tiles for D rows, tvt for C|R rows) write each feature's
// consecutive rows together instead of one 2-byte store per line.
constexpr int kVsRows = 32, kVsFeat = 64;

__global__ __launch_bounds__(256) void k_value_scatter(Geometry g, ProjArgs a) {
  __shared__ uint16_t vs[kVsRows][kVsFeat + 2];
  const int f0 = blockIdx.x * kVsFeat;                    // first value feature (kv head * D + dim)
  const int r0 = blockIdx.y * kVsRows;
  const int b = blockIdx.z;
  const int hd = g.H * g.D, kd = g.Hkv * g.D;
  const int t = threadIdx.x;
  {
    const int lr = t / 8, u = t % 8;                      // row, 8-feature unit
    const int r = r0 + lr;
    if (r < a.n_q) {
      const float* zr = a.z + (int64_t)(b * a.n_q + r) * a.n_pad + hd + kd + f0 + 8 * u;
      const floatx4 x0 = reinterpret_cast<const floatx4*>(zr)[0];
      const floatx4 x1 = reinterpret_cast<const floatx4*>(zr)[1];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        vs[lr][8 * u + e] = f32_to_bf16(x0[e]);
        vs[lr][8 * u + 4 + e] = f32_to_bf16(x1[e]);
      }
    }
  }
  __syncthreads();
  const int rr = t % kVsRows;
  const int r = r0 + rr;
  if (r >= a.n_q) return;
#pragma unroll
  for (int i = 0; i < kVsFeat * kVsRows / 256; ++i) {
    const int ff = t / kVsRows + i * (256 / kVsRows);     // feature within the block
    const int f = f0 + ff;
    const int kvh = f / g.D, j = f % g.D;
    if (r < a.n_d) {
      const int slot = a.slot0 + r;
      static_cast<uint16_t*>(a.vc)[((((int64_t)b * g.Hkv + kvh) * (g.slots / kKeyTile) + slot / kKeyTile) * g.D + j) *
                                       kKeyTile + slot % kKeyTile] = vs[rr][ff];
    } else {
      static_cast<uint16_t*>(a.tvt)[(((int64_t)b * g.Hkv + kvh) * g.D + j) * a.t_pad + (r - a.n_d)] = vs[rr][ff];
    }
  }
}

hipError_t launch_rope_scatter(const Geometry& g, const ProjArgs& a, int M, hipStream_t s) {
  const int units = (g.H + g.Hkv) * g.D / 8;                 // queries and keys
  hipLaunchKernelGGL(k_rope_scatter, dim3((units + 255) / 256, M), dim3(256), 0, s, g, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int kd = g.Hkv * g.D;
  hipLaunchKernelGGL(k_value_scatter, dim3(kd / kVsFeat, (a.n_q + kVsRows - 1) / kVsRows, g.B), dim3(256), 0, s, g, a);
  return hipGetLastError();
}

hipError_t launch_fill_i32(int32_t* p, int32_t v, int n, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  hipLaunchKernelGGL(k_fill_i32, dim3((n + 255) / 256), dim3(256), 0, s, p, v, n);
  return hipGetLastError();
}

}  // namespace mdm
