// Row statistics and CDF-tile helpers shared by the verify, drafter and tree
// kernels (gfx950, wave64): the per-slice max / argmax / sum of exponentials,
// the quad layout of CDF tiles, and the search for a drawn token inside one
// CDF tile (octet layout in the drafter, quad layout in the verify draw and
// the tree walk).
#pragma once

#include <math.h>

#include "../../include/spec_verify.h"
#include "sv_device.h"

namespace sv {

struct Partial {
  float m;       // max of the slice (-inf if every element is -inf)
  int g;         // greedy: lowest index attaining m
  double acc;    // sampling: sum over the slice of 2^((z - m) * c)
};

enum Mode { GREEDY = 0, SAMPLE = 1, MIXED = 2 };   // MIXED: per-sequence temperature

// Exponent scale c = log2(e) / T of a sequence's temperature T, or 0 for a
// greedy sequence: T = 0, or a temperature that is negative, NaN, infinite or
// so small that c itself overflows fp32 (`bad` is then set).
__device__ __forceinline__ float seq_scale(float T, bool& bad) {
  bad = false;
  if (T == 0.f) return 0.f;
  const float c = (float)(1.4426950408889634 / (double)T);
  if (!(T > 0.f) || !isfinite(T) || !isfinite(c)) {
    bad = true;
    return 0.f;
  }
  return c;
}

constexpr int kTileLoads = 4;           // wave-wide 512-element loads per CDF tile
constexpr int kTileElems = kTile * kTileLoads;
constexpr int kMaxTiles = SV_MAX_V / kTileElems;

// ---------------------------------------------------------------- raw octets
// One octet in the registers it was loaded into, so that a step can issue all
// of its loads before converting any of them.
template <typename LT> struct Raw;
template <> struct Raw<uint16_t> { u32x4 w; };
template <> struct Raw<float> { u32x4 a, b; };

template <bool NT>
__device__ __forceinline__ void raw_load(const uint16_t* row, long o, Raw<uint16_t>& r) {
  r.w = ld16<NT>(row + o * 8);
}
template <bool NT>
__device__ __forceinline__ void raw_load(const float* row, long o, Raw<float>& r) {
  r.a = ld16<NT>(row + o * 8);
  r.b = ld16<NT>(row + o * 8 + 4);
}
__device__ __forceinline__ void unpack(const Raw<uint16_t>& r, float v[8]) {
  v[0] = bf16_lo(r.w.x); v[1] = bf16_hi(r.w.x); v[2] = bf16_lo(r.w.y); v[3] = bf16_hi(r.w.y);
  v[4] = bf16_lo(r.w.z); v[5] = bf16_hi(r.w.z); v[6] = bf16_lo(r.w.w); v[7] = bf16_hi(r.w.w);
}
__device__ __forceinline__ void unpack(const Raw<float>& r, float v[8]) {
  v[0] = __uint_as_float(r.a.x); v[1] = __uint_as_float(r.a.y);
  v[2] = __uint_as_float(r.a.z); v[3] = __uint_as_float(r.a.w);
  v[4] = __uint_as_float(r.b.x); v[5] = __uint_as_float(r.b.y);
  v[6] = __uint_as_float(r.b.z); v[7] = __uint_as_float(r.b.w);
}

// ---------------------------------------------------------------- quad layout
// Element layout of the CDF tiles of the verify draw and the tree walk.  A
// wave load g covers the 512 elements [512 g, 512 g + 512) of a row; lane l
// holds the quads (4 consecutive elements) starting at 512 g + 4 l (half 0)
// and 512 g + 256 + 4 l (half 1), so each load instruction of the wave reads
// one contiguous block: 512 B of bf16 logits, 1 KB of fp32 q.  (With one
// 8-element octet per lane the fp32 loads of a lane are two 16-byte loads 32
// bytes apart: the draw of B=1024, K=7, V=151936 bf16 took 160 instead of
// 151 us.)
template <typename LT> struct Quad;
template <> struct Quad<uint16_t> { u32x2 w; };
template <> struct Quad<float> { u32x4 w; };

template <bool NT>
__device__ __forceinline__ void load_quad(const uint16_t* row, long e, Quad<uint16_t>& q) {
  q.w = ld8<NT>(row + e);
}
template <bool NT>
__device__ __forceinline__ void load_quad(const float* row, long e, Quad<float>& q) {
  q.w = ld16<NT>(row + e);
}
__device__ __forceinline__ void unpack(const Quad<uint16_t>& q, float v[4]) {
  v[0] = bf16_lo(q.w.x); v[1] = bf16_hi(q.w.x); v[2] = bf16_lo(q.w.y); v[3] = bf16_hi(q.w.y);
}
__device__ __forceinline__ void unpack(const Quad<float>& q, float v[4]) {
  v[0] = __uint_as_float(q.w.x); v[1] = __uint_as_float(q.w.y);
  v[2] = __uint_as_float(q.w.z); v[3] = __uint_as_float(q.w.w);
}
// An empty statement that claims to change a loaded quad: placed after a
// group of loads and before their first use, it makes every load of the group
// go out before the first wait (without it the compiler may wait for each
// load before issuing the next one).
template <typename LT>
__device__ __forceinline__ void hold(Quad<LT>& q) {
  asm volatile("" : "+v"(q.w));
}

// ---------------------------------------------------------------- row-slice state
struct SliceState {
  float best = -INFINITY;   // greedy: running max ...
  int idx = INT32_MAX;      // ... and the lowest index attaining it
  float mref = -INFINITY;   // sampling: running max ...
  float R = -1e30f;         // ... its exponent mref*c (log2 units, fp32) ...
  double acc = 0.0;         // ... and the sum of 2^(z*c - R) so far
};

__device__ __forceinline__ float tree_sum8(const float e[8]) {
  return ((e[0] + e[1]) + (e[2] + e[3])) + ((e[4] + e[5]) + (e[6] + e[7]));
}

// Fold N octets (at octet indices o0, o0 + OSTRIDE, ...) into the state.  The
// octets arrive in increasing index order, so "strictly greater" keeps the
// lowest index of a maximum.  RANGED: some of the elements may lie at or past
// V (padding of a ragged row) and must not be taken as the argmax.  Without
// it every element is in the row and the greedy search names a candidate by
// its slot u*8 + j in the step (< 64, so every select takes an inline
// constant and no register), one independent compare/select chain per octet
// joined by a minimum: one compare and one select per element.  The ranged
// form adds a 64-bit index and bound test, ~3x the instructions, and a search
// runs on most steps because some lane of the wave almost always finds a new
// maximum.
// Element offset of slot j (0..7) of an 8-element group from the group's
// first octet o0: the octet's own elements, or (QUAD) lane l's two quads at
// 4 l and 256 + 4 l of the wave's 512-element block starting at octet o0.
// Either way the offsets grow with j, so a thread still meets its elements
// in increasing index order.
template <bool QUAD>
__device__ __forceinline__ int slot_elem(int j, int l) {
  if constexpr (QUAD) return j < 4 ? 4 * l + j : 252 + 4 * l + j;
  else return j;
}

template <int MODE, int N, int OSTRIDE, bool RANGED = true, bool QUAD = false>
__device__ __forceinline__ void fold(SliceState& s, float (&v)[N][8], long o0, long V, float c,
                                     int l = 0) {
  float mt = v[0][0];
#pragma unroll
  for (int u = 0; u < N; ++u)
#pragma unroll
    for (int j = 0; j < 8; ++j) mt = fmaxf(mt, v[u][j]);
  if constexpr (MODE == GREEDY) {
    if (mt > s.best || s.idx == INT32_MAX) {
      int found = INT32_MAX;
      if constexpr (RANGED) {
#pragma unroll
        for (int u = N - 1; u >= 0; --u)
#pragma unroll
          for (int j = 7; j >= 0; --j) {
            const long e = (o0 + (long)u * OSTRIDE) * 8 + slot_elem<QUAD>(j, l);
            if (e < V && v[u][j] == mt) found = (int)e;
          }
      } else {
        static_assert(N * 8 <= 64, "slot numbers must stay inline constants");
        int slot = 64;
#pragma unroll
        for (int u = 0; u < N; ++u) {
          int su = 64;
#pragma unroll
          for (int j = 7; j >= 0; --j)
            if (v[u][j] == mt) su = u * 8 + j;
          slot = min(slot, su);
        }
        if (slot < 64)
          found = (int)(o0 * 8) + (slot >> 3) * (OSTRIDE * 8) + slot_elem<QUAD>(slot & 7, l);
      }
      if (found != INT32_MAX) { s.best = mt; s.idx = found; }
    }
  } else {
    if (mt > s.mref) {
      const float Rn = mt * c;
      s.acc *= (double)__builtin_amdgcn_exp2f(s.R - Rn);
      s.R = Rn;
      s.mref = mt;
    }
    float part = 0.f;
#pragma unroll
    for (int u = 0; u < N; ++u) {
      float e[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) e[j] = __builtin_amdgcn_exp2f(fmaf(v[u][j], c, -s.R));
      part += tree_sum8(e);
    }
    s.acc += (double)part;
  }
}

// One slice [o_lo, o_hi) of octets of one row -> one Partial (returned by
// thread 0) by a workgroup of THREADS threads; sm_f / sm_i / sm_d hold one
// entry per wave.  VEC: V is a multiple of 8 and the rows are 16-byte
// aligned, so the steady-state loop has no branches and issues all of a
// step's loads before using any.  NT: non-temporal loads, for data read
// exactly once (measured 10% faster than cached loads on gfx950).  RANGED:
// keep the bound-tested greedy search under VEC as well (same result); the
// drafter kernel uses it: with the short search its sampled path measured
// 11% slower, although that path's instructions stay the same; only the
// kernel's scalar register count changes (98 -> 74).
template <typename LT, int MODE, bool VEC, int THREADS, bool NT = true, bool RANGED = false>
__device__ __forceinline__ Partial slice_stats(const LT* row, long o_lo, long o_hi, long V, float c,
                               float* sm_f, int* sm_i, double* sm_d) {
  constexpr int U = 16 / sizeof(LT);    // octets per step: 128 bytes in flight per thread
  const int t = threadIdx.x;
  SliceState st;
  long base = o_lo + t;
  if constexpr (VEC && sizeof(LT) == 4) {
    // fp32 rows: the quad layout, so that each load instruction of a wave
    // reads one contiguous kilobyte (with one octet per lane a lane's two
    // 16-byte loads were 32 bytes apart, and the row kernel read fp32 logits
    // at 6.1 TB/s against 6.9 TB/s for bf16).  The wave steps together while
    // its whole block of each of the step's U wave loads lies in the slice;
    // the rest of the slice goes through the per-octet loops below.
    const int l = lane_id();
    long wbase = base - l;                  // the wave's first octet of the step
    for (; wbase + (kWave - 1) + (long)(U - 1) * THREADS < o_hi; wbase += (long)U * THREADS) {
      Quad<LT> qa[U], qb[U];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const long e = (wbase + (long)u * THREADS) * 8 + 4 * l;
        load_quad<NT>(row, e, qa[u]);
        load_quad<NT>(row, e + kTile / 2, qb[u]);
      }
      float v[U][8];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        unpack(qa[u], &v[u][0]);
        unpack(qb[u], &v[u][4]);
      }
      fold<MODE, U, THREADS, RANGED, true>(st, v, wbase, V, c, l);
    }
    base = wbase + l;
  }
  if constexpr (VEC) {
    for (; base + (long)(U - 1) * THREADS < o_hi; base += (long)U * THREADS) {
      Raw<LT> raw[U];
#pragma unroll
      for (int u = 0; u < U; ++u) raw_load<NT>(row, base + (long)u * THREADS, raw[u]);
      float v[U][8];
#pragma unroll
      for (int u = 0; u < U; ++u) unpack(raw[u], v[u]);
      fold<MODE, U, THREADS, RANGED>(st, v, base, V, c);
    }
    for (; base < o_hi; base += THREADS) {
      Raw<LT> raw;
      raw_load<false>(row, base, raw);
      float v[1][8];
      unpack(raw, v[0]);
      fold<MODE, 1, THREADS, RANGED>(st, v, base, V, c);
    }
  } else {
    for (; base < o_hi; base += THREADS) {
      float v[1][8];
      load_octet<false>(row, base, V, false, -INFINITY, v[0]);
      fold<MODE, 1, THREADS>(st, v, base, V, c);
    }
  }

  Partial P{-INFINITY, INT32_MAX, 0.0};
  const int w = t / kWave, l = lane_id();
  if constexpr (MODE == GREEDY) {
    float best = st.best;
    int idx = st.idx;
    wave_argmax(best, idx);
    if (l == 0) { sm_f[w] = best; sm_i[w] = idx; }
    __syncthreads();
    if (t == 0) {
      P.m = sm_f[0];
      P.g = sm_i[0];
      for (int i = 1; i < (THREADS / kWave); ++i) argmax_combine(P.m, P.g, sm_f[i], sm_i[i]);
    }
  } else {
    float M = wave_max(st.mref);
    if (l == 0) sm_f[w] = M;
    __syncthreads();
    M = sm_f[0];
    for (int i = 1; i < (THREADS / kWave); ++i) M = fmaxf(M, sm_f[i]);
    // rescale this thread's sum from its reference R to M*c (fp64)
    const double mine = st.acc == 0.0 ? 0.0 : st.acc * exp2((double)st.R - (double)M * (double)c);
    const double ws = wave_sum(mine);
    if (l == 0) sm_d[w] = ws;
    __syncthreads();
    if (t == 0) {
      double s = sm_d[0];
      for (int i = 1; i < (THREADS / kWave); ++i) s += sm_d[i];
      P.m = M; P.g = 0; P.acc = s;
    }
  }
  return P;
}

__device__ __forceinline__ float wave_sum_f(float x) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) x += __shfl_xor(x, off);
  return x;
}

// q(x) of a drafted row from its drafter logit z(x) and its descriptor: the
// fp32 operations the drafter kernel uses to write q.
__device__ __forceinline__ float drafter_q(const sv_draft_row& d, float z, long e) {
  return d.c > 0.f ? __builtin_amdgcn_exp2f(fmaf(z, d.c, -d.mc)) * d.inv_s
                   : (e == (long)d.argmax ? 1.f : 0.f);
}

// The token drawn inside one CDF tile.  Lane l holds the masses r[sl][0..7]
// of octet (tile * kTileLoads + sl) * 64 + l; tpre is the running total before
// the tile and target = u * S.  Returns (on every lane) the first element
// whose running total exceeds target; with `fallback`, or when rounding
// leaves no crossing in the tile, its last element with positive mass (0 if
// it has none).  Running totals are fp64.
__device__ __forceinline__ int pick_in_tile(const float (&r)[kTileLoads][8], long tile,
                                            double tpre, double target, bool fallback) {
  const int l = lane_id();
  int pick = -1, lastpos = -1;
  double lrun0 = tpre;               // running total before the current wave load
#pragma unroll
  for (int sl = 0; sl < kTileLoads; ++sl) {
    const long o = ((long)tile * kTileLoads + sl) * kWave + l;
    int lastj = -1;
    for (int j = 7; j >= 0; --j) if (r[sl][j] > 0.f) { lastj = (int)(o * 8 + j); break; }
    const unsigned long long anyp = __ballot(lastj >= 0);
    if (anyp) lastpos = __shfl(lastj, 63 - __clzll((long long)anyp));
    if (fallback || pick >= 0) continue;
    const double ls = (double)tree_sum8(r[sl]);
    const double lincl = wave_inclusive_scan(ls);
    double lexcl = __shfl_up(lincl, 1);
    if (l == 0) lexcl = 0.0;
    const unsigned long long cross = __ballot(lrun0 + lincl > target);
    if (cross) {
      const int src = __ffsll((long long)cross) - 1;
      int mine = -1;
      if (l == src) {
        double lrun = lrun0 + lexcl;
        for (int j = 0; j < 8; ++j) {
          lrun += (double)r[sl][j];
          if (r[sl][j] > 0.f && lrun > target) { mine = (int)(o * 8 + j); break; }
        }
        if (mine < 0)
          for (int j = 7; j >= 0; --j) if (r[sl][j] > 0.f) { mine = (int)(o * 8 + j); break; }
      }
      const unsigned long long got = __ballot(mine >= 0);
      pick = got ? __shfl(mine, __ffsll((long long)got) - 1) : lastpos;
      if (pick < 0) pick = 0;
    }
    lrun0 += __shfl(lincl, kWave - 1);
  }
  // rounding left u*S at or past the tile's total: its last positive element
  if (pick < 0) pick = lastpos >= 0 ? lastpos : 0;
  return pick;
}

// The token drawn inside CDF tile `tile` of a row whose masses this lane
// holds in the quad layout (r[sl][4 h + j]: element 512 g + 256 h + 4 l + j
// of wave load g = tile * kTileLoads + sl).  The
// halves of the wave loads are walked in vocabulary order; tpre is the
// running total before the tile and target = u * S.  Returns (on every lane)
// the first element whose running total exceeds target; with `fallback`, or
// when rounding leaves no crossing in the tile, its last element with
// positive mass (0 if it has none).  Running totals are fp64.
__device__ __forceinline__ int pick_in_quad_tile(const float (&r)[kTileLoads][8], long tile,
                                                 double tpre, double target, bool fallback) {
  const int l = lane_id();
  int pick = -1, lastpos = -1;
  double run0 = tpre;                // running total before the current half
#pragma unroll
  for (int sl = 0; sl < kTileLoads; ++sl) {
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const long e0 = (tile * kTileLoads + sl) * (long)kTile + h * (kTile / 2) + 4 * l;
      const float* m = &r[sl][4 * h];
      int lastj = -1;
      for (int j = 3; j >= 0; --j) if (m[j] > 0.f) { lastj = (int)(e0 + j); break; }
      const unsigned long long anyp = __ballot(lastj >= 0);
      if (anyp) lastpos = __shfl(lastj, 63 - __clzll((long long)anyp));
      if (fallback || pick >= 0) continue;
      const double ls = (double)((m[0] + m[1]) + (m[2] + m[3]));
      const double lincl = wave_inclusive_scan(ls);
      double lexcl = __shfl_up(lincl, 1);
      if (l == 0) lexcl = 0.0;
      const unsigned long long cross = __ballot(run0 + lincl > target);
      if (cross) {
        const int src = __ffsll((long long)cross) - 1;
        int mine = -1;
        if (l == src) {
          double lrun = run0 + lexcl;
          for (int j = 0; j < 4; ++j) {
            lrun += (double)m[j];
            if (m[j] > 0.f && lrun > target) { mine = (int)(e0 + j); break; }
          }
          if (mine < 0)
            for (int j = 3; j >= 0; --j) if (m[j] > 0.f) { mine = (int)(e0 + j); break; }
        }
        const unsigned long long got = __ballot(mine >= 0);
        pick = got ? __shfl(mine, __ffsll((long long)got) - 1) : lastpos;
        if (pick < 0) pick = 0;
      }
      run0 += __shfl(lincl, kWave - 1);
    }
  }
  // rounding left u*S at or past the tile's total: its last positive element
  if (pick < 0) pick = lastpos >= 0 ? lastpos : 0;
  return pick;
}

}  // namespace sv
