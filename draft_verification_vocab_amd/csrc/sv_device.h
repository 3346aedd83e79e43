// Device helpers shared by the verify and build kernels (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace sv {

constexpr int kWave = 64;
constexpr int kOct = 8;                 // elements per lane per load group ("octet")
constexpr int kTile = kWave * kOct;     // 512 elements: granularity of the draw's CDF

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));

// ---------------------------------------------------------------- bf16 / fp32
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

template <bool NT>
__device__ __forceinline__ u32x4 ld16(const void* p) {
  if constexpr (NT) return __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
  else return *reinterpret_cast<const u32x4*>(p);
}

template <bool NT>
__device__ __forceinline__ u32x2 ld8(const void* p) {
  if constexpr (NT) return __builtin_nontemporal_load(reinterpret_cast<const u32x2*>(p));
  else return *reinterpret_cast<const u32x2*>(p);
}

// Element e of a logit row as fp32 (exact widening).
__device__ __forceinline__ float logit_at(const float* row, long e) { return row[e]; }
__device__ __forceinline__ float logit_at(const uint16_t* row, long e) {
  return __uint_as_float(static_cast<uint32_t>(row[e]) << 16);
}

// Octet o (elements 8o..8o+7) of a logit row.  vec: the whole octet is in
// range and 16-byte aligned, load it with vector loads; otherwise load the
// elements one by one and pad past V with `pad`.
template <bool NT>
__device__ __forceinline__ void load_octet(const uint16_t* row, long o, long V, bool vec,
                                           float pad, float v[8]) {
  if (vec) {
    u32x4 w = ld16<NT>(row + o * 8);
    v[0] = bf16_lo(w.x); v[1] = bf16_hi(w.x); v[2] = bf16_lo(w.y); v[3] = bf16_hi(w.y);
    v[4] = bf16_lo(w.z); v[5] = bf16_hi(w.z); v[6] = bf16_lo(w.w); v[7] = bf16_hi(w.w);
  } else {
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      long e = o * 8 + j;
      v[j] = e < V ? logit_at(row, e) : pad;
    }
  }
}

template <bool NT>
__device__ __forceinline__ void load_octet(const float* row, long o, long V, bool vec,
                                           float pad, float v[8]) {
  if (vec) {
    u32x4 a = ld16<NT>(row + o * 8);
    u32x4 b = ld16<NT>(row + o * 8 + 4);
    v[0] = __uint_as_float(a.x); v[1] = __uint_as_float(a.y);
    v[2] = __uint_as_float(a.z); v[3] = __uint_as_float(a.w);
    v[4] = __uint_as_float(b.x); v[5] = __uint_as_float(b.y);
    v[6] = __uint_as_float(b.z); v[7] = __uint_as_float(b.w);
  } else {
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      long e = o * 8 + j;
      v[j] = e < V ? row[e] : pad;
    }
  }
}

// ---------------------------------------------------------------- wave ops
__device__ __forceinline__ int lane_id() { return __lane_id(); }

__device__ __forceinline__ double wave_sum(double x) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) x += __shfl_xor(x, off);
  return x;  // every lane holds the same total (butterfly order is fixed)
}

__device__ __forceinline__ float wave_max(float x) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) x = fmaxf(x, __shfl_xor(x, off));
  return x;
}

// Inclusive prefix sum over the 64 lanes (Hillis-Steele, fixed order).
__device__ __forceinline__ double wave_inclusive_scan(double x) {
  const int l = lane_id();
#pragma unroll
  for (int off = 1; off < kWave; off <<= 1) {
    double y = __shfl_up(x, off);
    if (l >= off) x += y;
  }
  return x;
}

// (value, index) lexicographic max: larger value wins, equal values keep the
// lower index.  An index of INT32_MAX means "no element".
__device__ __forceinline__ void argmax_combine(float& m, int& g, float m2, int g2) {
  if (m2 > m || (m2 == m && g2 < g) || (g == INT32_MAX && g2 != INT32_MAX)) { m = m2; g = g2; }
}

__device__ __forceinline__ void wave_argmax(float& m, int& g) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) {
    float m2 = __shfl_xor(m, off);
    int g2 = __shfl_xor(g, off);
    argmax_combine(m, g, m2, g2);
  }
}

// 2^x for an fp64 argument x <= 0 with fp32 accuracy: 2^floor(x) exactly,
// times the hardware fp32 exponential of the fraction (relative error ~1e-7,
// that of every per-element exponential of the row statistics), at a few
// instructions instead of the ~40 of an fp64 exp2.  Used to bring partial
// sums of exponentials to a common reference.
__device__ __forceinline__ double exp2_split(double x) {
  if (!(x > -1074.0)) return 0.0;             // also -inf and NaN
  const double n = floor(x);
  return ldexp((double)__builtin_amdgcn_exp2f((float)(x - n)), (int)n);
}

__device__ __forceinline__ void flag_error(int32_t* device_error, int bit) {
  if (device_error) atomicOr(device_error, bit);
}

// ---------------------------------------------------------------- coherent access
// Agent-scope relaxed atomic stores and loads bypass the non-coherent
// per-CU vector cache (and are kept coherent across the XCDs' L2 caches by
// the gfx94x/gfx950 memory model), so a wave that rewrites values and reads
// them back, or reads values another launch wrote, never sees a stale cached
// copy; wait_stores_performed makes a wave wait until its stores are done.
// None of them needs a cache write-back or invalidate instruction.
template <typename T>
__device__ __forceinline__ void st_coherent(T* p, T v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
template <typename T>
__device__ __forceinline__ T ld_coherent(T* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void wait_stores_performed() {
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  __builtin_amdgcn_s_waitcnt(0x0F70);   // vmcnt(0), expcnt / lgkmcnt untouched
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
}

}  // namespace sv
