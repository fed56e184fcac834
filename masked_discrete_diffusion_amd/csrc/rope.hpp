// RoPE'd row stores shared by the cache append and the fused commit of the
// logits merge: elements are widened exactly to float, rotated in double
// (rope_pair) and rounded once to the storage type.
#pragma once

#include "common.hpp"

namespace mdm {

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

}  // namespace mdm
