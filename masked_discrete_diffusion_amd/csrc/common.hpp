// Device helpers shared by the sparse-step kernels (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mdm {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float floatx16 __attribute__((ext_vector_type(16)));
typedef float floatx4 __attribute__((ext_vector_type(4)));
typedef uint16_t u16x8 __attribute__((ext_vector_type(8)));
typedef float floatx2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

constexpr int kWave = 64;
constexpr int kKeyTile = 64;       // keys per LDS stage in attention; cache slots are a multiple
constexpr int kVocabTile = 128;    // vocab columns per screening tile (one partial per tile)
constexpr int kCand = 8;           // candidates re-scored exactly per row

// Error bits of the device flag word.
constexpr int kErrTok = 1;
constexpr int kErrPos = 2;

__device__ __attribute__((always_inline)) inline void flag_error(int* err, int bit) {
  if (err) atomicOr(err, bit);
}

// bf16 bit pattern -> float (exact).
__device__ __attribute__((always_inline)) inline float bf16_to_f32(uint16_t b) { return __uint_as_float(((uint32_t)b) << 16); }

// float -> bf16 bit pattern, round to nearest even (hardware conversion on gfx950).
__device__ __attribute__((always_inline)) inline uint16_t f32_to_bf16(float f) {
  __bf16 h = (__bf16)f;
  return __builtin_bit_cast(uint16_t, h);
}

// Two floats -> packed bf16 pair (first in the low half), round to nearest even.
__device__ __attribute__((always_inline)) inline uint32_t pack_bf16x2(float a, float b) {
  const floatx2 f = {a, b};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f, bf16x2));
}

// double -> bf16 bit pattern, round to nearest even in ONE step (no detour via
// fp32, which could round twice).  Keeps the top 7 of the 52 stored mantissa
// bits: add just under half of the dropped 45 bits plus the kept lsb, then
// truncate; a carry into the exponent is the correct result.  Inputs are
// finite and in the normal range of bf16 (O(1) activations); the truncated
// double is then exactly representable in fp32 and in bf16.
__device__ __attribute__((always_inline)) inline uint16_t f64_to_bf16(double x) {
  uint64_t u = (uint64_t)__double_as_longlong(x);
  const uint64_t lsb = (u >> 45) & 1ull;
  u += ((1ull << 44) - 1ull) + lsb;
  u &= ~((1ull << 45) - 1ull);
  float f = (float)__longlong_as_double((long long)u);
  return (uint16_t)(__float_as_uint(f) >> 16);
}

// RoPE of one interleaved pair (x0, x1) by the angle whose fp32 cos/sin are c, s.
// Evaluated in double: x (bf16 or fp32) times c or s (fp32) is exact in double,
// so each component rounds once; contraction into fma cannot change it.
__device__ __attribute__((always_inline)) inline void rope_pair(float x0, float x1, float c, float s, double& r0, double& r1) {
  const double dx0 = x0, dx1 = x1, dc = c, ds = s;
  r0 = dx0 * dc - dx1 * ds;
  r1 = dx0 * ds + dx1 * dc;
}

// Strict "a ranks before b" for (value, index) candidates: larger value first,
// lower index on equal values.
__device__ __attribute__((always_inline)) inline bool ranks_before(float va, int ia, float vb, int ib) {
  return va > vb || (va == vb && ia < ib);
}

// ---- wavefront all-reduce without LDS ------------------------------------------
// wave_pair<S>(x) returns this lane's value and its step-S partner's as {a, b},
// in an order that may differ between the two partners.  Steps 0..5 pair the
// lanes 1 apart and 2 apart (DPP quad permutes), across the two halves of each
// 8 and each 16 lanes (DPP row half-mirror, row mirror), 16 apart
// (v_permlane16_swap) and 32 apart (v_permlane32_swap).  After steps 0..s
// every lane holds the result over its aligned group of 2^(s+1) lanes; with a
// symmetric combining function both partners compute identical bits, so the
// result is deterministic and uniform over the group.
struct U2 {
  uint32_t a, b;
};
template <int S>
__device__ __attribute__((always_inline)) inline U2 wave_pair(uint32_t x) {
  static_assert(S >= 0 && S <= 5, "step");
  if constexpr (S == 0) return {x, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0xB1, 0xF, 0xF, false)};
  else if constexpr (S == 1) return {x, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x4E, 0xF, 0xF, false)};
  else if constexpr (S == 2) return {x, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x141, 0xF, 0xF, false)};
  else if constexpr (S == 3) return {x, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x140, 0xF, 0xF, false)};
  else if constexpr (S == 4) {
    const auto r = __builtin_amdgcn_permlane16_swap(x, x, false, false);
    return {(uint32_t)r[0], (uint32_t)r[1]};
  } else {
    const auto r = __builtin_amdgcn_permlane32_swap(x, x, false, false);
    return {(uint32_t)r[0], (uint32_t)r[1]};
  }
}

// Sum over aligned groups of 2^N lanes (N <= 6): steps 0..N-1.
template <int N>
__device__ __attribute__((always_inline)) inline float group_sum(float x) {
  if constexpr (N > 0) {
    x = group_sum<N - 1>(x);
    const U2 p = wave_pair<N - 1>(__float_as_uint(x));
    x = __uint_as_float(p.a) + __uint_as_float(p.b);
  }
  return x;
}

// (value desc, index asc) best pair over aligned groups of 2^N lanes.
template <int N>
__device__ __attribute__((always_inline)) inline void group_argmax(float& v, int& i) {
  if constexpr (N > 0) {
    group_argmax<N - 1>(v, i);
    const U2 pv = wave_pair<N - 1>(__float_as_uint(v));
    const U2 pi = wave_pair<N - 1>((uint32_t)i);
    const float va = __uint_as_float(pv.a), vb = __uint_as_float(pv.b);
    const int ia = (int)pi.a, ib = (int)pi.b;
    const bool tb = ranks_before(vb, ib, va, ia);
    v = tb ? vb : va;
    i = tb ? ib : ia;
  }
}

// ---- LDS-DMA rings -----------------------------------------------------------
// A wave-wide global_load_lds_dwordx4 writes 64 consecutive 16-byte units of
// LDS starting at `lds_block` (uniform); lane l's 16 bytes come from
// base + off_l (base uniform, in SGPRs; off_l a per-lane byte offset) and
// land in unit l.
//
// Issued from inline asm on purpose: the compiler treats an LDS-DMA load it
// can see as a pending write to any LDS it cannot prove disjoint, and then
// waits for vmcnt(0) in front of the next LDS read, which drains the whole
// ring on every tile.  Hidden from it, the load is ordered by the explicit
// ring_wait / ring_barrier below (both memory clobbers), and the compiler's
// own vmcnt waits for its loads only become stricter (the counter retires in
// issue order).  M0 holds the LDS base; nothing else in these kernels uses M0,
// and one wait state separates its write from the load.
__device__ __attribute__((always_inline)) inline void dma16_at(const void* base, uint32_t off, uint32_t lds) {
  lds = __builtin_amdgcn_readfirstlane(lds);
  asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %1" ::"v"(off), "s"(base), "s"(lds)
               : "memory");
}
// LDS byte address of a pointer into shared memory.
__device__ __attribute__((always_inline)) inline uint32_t lds_addr(const void* p) {
  return (uint32_t)(uintptr_t)(const void __attribute__((address_space(3)))*)p;
}
__device__ __attribute__((always_inline)) inline void dma16(const void* base, uint32_t off, void* lds_block) { dma16_at(base, off, lds_addr(lds_block)); }

// Wait until at most N of this wavefront's vector-memory operations are in
// flight, and its LDS operations are done.  vmcnt retires in issue order, so
// with N = (loads this wave issued after tile i) it waits exactly for tile i.
template <int N>
__device__ __attribute__((always_inline)) inline void ring_wait() {
  static_assert(N >= 0 && N < 64, "vmcnt immediate out of range");
  asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)" ::"n"(N) : "memory");
}

// Workgroup barrier without the release fence of __syncthreads (that fence
// would wait for every LDS-DMA load in flight); waits are explicit, above.
__device__ __attribute__((always_inline)) inline void ring_barrier() {
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

}  // namespace mdm
