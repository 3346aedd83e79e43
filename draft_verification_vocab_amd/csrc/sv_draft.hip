// Drafter-output sampling for gfx950: the P-EAGLE drafter's K prediction rows
// per sequence -> the K draft tokens and the drafter distribution q that the
// next verify tests them against (P-EAGLE / TorchSpec blog summary, section
// 并行架构的核心创新: one drafter forward predicts all K drafts; "Project 14 -
// speculative decoding inference server", section 架构: the drafter proposes,
// the target verifies).
//
// One workgroup per draft (b, k); no workgroup hands anything to another.
//   sweep 1  streams the drafter logit row once and keeps, for every
//            2048-element CDF tile, its max and its sum of exponentials at the
//            sequence's temperature (LDS); the row's max and sum follow from
//            them.  With temperature 0 (greedy) it finds the lowest-index
//            argmax instead.
//   sweep 2  only when q is requested: streams the row again and writes
//            q = softmax(z / T) as fp32;
//   locate   one wave finds the tile whose running mass first exceeds u,
//            rescans that one tile and writes the token.
// A sampled bf16 row of up to 155648 logits (V a multiple of 8) with q
// requested is instead held in the workgroup's registers: read once, and the
// row max, the tile masses and q all come from the registers, so the row is
// fetched once rather than twice.  That form is bound by the q writes, which
// are two thirds of its bytes: at 1024 x 7 x 151936 it takes 1.34 ms
// (1.37 ms with the second read), while a bare kernel that only reads the
// same rows and writes them back as fp32 takes 1.38 ms (1.61 ms with
// non-temporal stores), and writes alone run at about 5.7 TB/s.
// Without q the row is read once with one exponential per element.  Greedy
// rows need no exponentials: q is the one-hot of the argmax.
// The q rows are written with non-temporal stores: the next verify reads only
// a few of their elements and one row per sequence.
#include "sv_device.h"
#include "sv_internal.h"
#include "sv_rowstats.h"

namespace sv {

// Workgroup size: 512 threads when q is written (measured 1.49 vs 1.83 ms
// with 256 at 1024 x 7 x 151936), 256 when only tokens are drawn.
template <bool WQ> constexpr int draft_threads() { return WQ ? 512 : 256; }
constexpr int kDraftTilesPerStep = 2;  // sweep 1: CDF tiles per wave in flight
// Row-resident sampled rows (RES = the workgroup size): wave w holds CDF
// tiles w, w + W, w + 2W, ... (W waves), each as 8 quads of four bf16 logits
// per lane (2 VGPRs a quad), up to kResTiles tiles, so V <= 76 * 2048 = 155648.
constexpr int kResTiles = 76;
constexpr long kResMaxV = (long)kResTiles * kTileElems;
constexpr int kResThreads = 512;      // 1024 threads (5 slots a wave) measured the same
template <int THREADS> constexpr int res_slots() {
  return (kResTiles + THREADS / kWave - 1) / (THREADS / kWave);
}
constexpr int kQuadsPerTileLane = kTileElems / 4 / kWave;   // 8
constexpr int kTileQuads = kTileElems / 4;

typedef float f32x4 __attribute__((ext_vector_type(4)));

struct DraftArgs {
  const void* logits;          // [n_rows][V]
  const int32_t* row_index;    // [B*K] or null (row b*K + k)
  long n_rows;
  const float* uniforms;       // [B*K]; null only when every row is greedy
  const float* temperatures;   // [B] or null (the scalar below)
  float temperature;
  int B, K, V;
  int32_t* out_tokens;         // [B*K]
  float* out_probs;            // [B*K][V] or null
  sv_draft_row* out_desc;      // [B*K] or null
  int32_t* device_error;
};

// q of one octet of a sampled row: 2^(z c - Mc) * inv_s.
__device__ __forceinline__ void q_octet(const float z[8], float c, float Mc, float inv_s,
                                        float q[8]) {
#pragma unroll
  for (int j = 0; j < 8; ++j) q[j] = __builtin_amdgcn_exp2f(fmaf(z[j], c, -Mc)) * inv_s;
}

// q of the kTileLoads octets of tile t seen by this lane (octet
// (t * kTileLoads + sl) * 64 + lane).  Octets past the row give q = 0.
template <typename LT, bool VEC>
__device__ __forceinline__ void tile_q(const LT* zrow, int t, long V, long nocts, float c, float Mc,
                                       float inv_s, float (&q)[kTileLoads][8]) {
  const int l = lane_id();
  if constexpr (VEC) {
    Raw<LT> raw[kTileLoads];
#pragma unroll
    for (int sl = 0; sl < kTileLoads; ++sl) {
      const long o = ((long)t * kTileLoads + sl) * kWave + l;
      raw_load<false>(zrow, o < nocts ? o : nocts - 1, raw[sl]);
    }
#pragma unroll
    for (int sl = 0; sl < kTileLoads; ++sl) {
      const long o = ((long)t * kTileLoads + sl) * kWave + l;
      float z[8];
      unpack(raw[sl], z);
      if (o >= nocts)
#pragma unroll
        for (int j = 0; j < 8; ++j) z[j] = -INFINITY;
      q_octet(z, c, Mc, inv_s, q[sl]);
    }
  } else {
#pragma unroll
    for (int sl = 0; sl < kTileLoads; ++sl) {
      const long o = ((long)t * kTileLoads + sl) * kWave + l;
      float z[8];
      load_octet<false>(zrow, o, V, false, -INFINITY, z);
      q_octet(z, c, Mc, inv_s, q[sl]);
    }
  }
}

// Store octet o of a q row (VEC: two 16-byte non-temporal stores).
template <bool VEC>
__device__ __forceinline__ void store_q(float* qrow, long o, long V, const float q[8]) {
  if constexpr (VEC) {
    f32x4* p = reinterpret_cast<f32x4*>(qrow + o * 8);
    __builtin_nontemporal_store(f32x4{q[0], q[1], q[2], q[3]}, p);
    __builtin_nontemporal_store(f32x4{q[4], q[5], q[6], q[7]}, p + 1);
  } else {
#pragma unroll
    for (int j = 0; j < 8; ++j)
      if (o * 8 + j < V) __builtin_nontemporal_store(q[j], qrow + o * 8 + j);
  }
}

// Four consecutive logits (quad qd = elements 4qd .. 4qd+3), cached loads:
// sweep 2 re-reads the row sweep 1 has just read.
__device__ __forceinline__ void quad_at(const uint16_t* row, long qd, float z[4]) {
  const uint2 w = reinterpret_cast<const uint2*>(row)[qd];
  z[0] = __uint_as_float(w.x << 16); z[1] = __uint_as_float(w.x & 0xffff0000u);
  z[2] = __uint_as_float(w.y << 16); z[3] = __uint_as_float(w.y & 0xffff0000u);
}
__device__ __forceinline__ void quad_at(const float* row, long qd, float z[4]) {
  const f32x4 v = reinterpret_cast<const f32x4*>(row)[qd];
  z[0] = v.x; z[1] = v.y; z[2] = v.z; z[3] = v.w;
}

constexpr int kQuadsPerLane = 8;   // one 2048-element step per wave

// Sweep 2 of a sampled row with VEC (V a multiple of 8, rows 16-byte
// aligned): q = 2^(z c - Mc) * inv_s, element for element as q_octet
// computes it, with lane l of a wave on quad base + j*64 + l, so that each
// 16-byte non-temporal store instruction writes 1 KB of contiguous q.  (With
// one octet per lane, a store instruction writes 16-byte pieces with 16-byte
// gaps, and 10% more bytes reached HBM than q holds.)
template <typename LT, int WAVES>
__device__ __forceinline__ void write_q_quads(const LT* zrow, float* qrow, long V, float c,
                                              float Mc, float inv_s) {
  const long nquads = V / 4;
  const int w = threadIdx.x / kWave, l = lane_id();
  for (long base = (long)w * kWave * kQuadsPerLane; base < nquads;
       base += (long)WAVES * kWave * kQuadsPerLane) {
    float z[kQuadsPerLane][4];
#pragma unroll
    for (int j = 0; j < kQuadsPerLane; ++j) {
      const long qd = base + (long)j * kWave + l;
      quad_at(zrow, qd < nquads ? qd : nquads - 1, z[j]);
    }
#pragma unroll
    for (int j = 0; j < kQuadsPerLane; ++j) {
      const long qd = base + (long)j * kWave + l;
      f32x4 q;
      q.x = __builtin_amdgcn_exp2f(fmaf(z[j][0], c, -Mc)) * inv_s;
      q.y = __builtin_amdgcn_exp2f(fmaf(z[j][1], c, -Mc)) * inv_s;
      q.z = __builtin_amdgcn_exp2f(fmaf(z[j][2], c, -Mc)) * inv_s;
      q.w = __builtin_amdgcn_exp2f(fmaf(z[j][3], c, -Mc)) * inv_s;
      if (qd < nquads) __builtin_nontemporal_store(q, reinterpret_cast<f32x4*>(qrow) + qd);
    }
  }
}

// Whole q row: the one-hot of g (g < 0: all zero), stores only; with VEC one
// contiguous 16-byte quad per lane and store instruction, as above.
template <bool VEC, int THREADS>
__device__ void store_one_hot(float* qrow, long V, long nocts, int g) {
  if constexpr (VEC) {
    const long nquads = V / 4;
    for (long qd = threadIdx.x; qd < nquads; qd += THREADS) {
      const long e = qd * 4;
      const f32x4 q{e == g ? 1.f : 0.f, e + 1 == g ? 1.f : 0.f, e + 2 == g ? 1.f : 0.f,
                    e + 3 == g ? 1.f : 0.f};
      __builtin_nontemporal_store(q, reinterpret_cast<f32x4*>(qrow) + qd);
    }
  } else {
    for (long o = threadIdx.x; o < nocts; o += THREADS) {
      float q[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) q[j] = (o * 8 + j == g) ? 1.f : 0.f;
      store_q<VEC>(qrow, o, V, q);
    }
  }
}

// The max m and the sum s of 2^(z c - m c) of one bf16 CDF tile that a wave
// holds as kQuadsPerTileLane packed quads per lane (quad k * 64 + l of the
// tile in v[k] of lane l; quads past the row hold -inf).  Each lane sums its
// 32 exponentials pairwise, then the wave sums the lanes.  Both the streamed
// and the row-resident passes over bf16 rows use it, so the tile masses, and
// with them the drawn tokens, do not depend on whether q is written.
__device__ __forceinline__ void quad_tile_stats(const u32x2* v, float c, float& m, float& s) {
  float mx = -INFINITY;
#pragma unroll
  for (int k = 0; k < kQuadsPerTileLane; ++k)
    mx = fmaxf(mx, fmaxf(fmaxf(bf16_lo(v[k].x), bf16_hi(v[k].x)),
                         fmaxf(bf16_lo(v[k].y), bf16_hi(v[k].y))));
  mx = wave_max(mx);
  float ls = 0.f;
  if (mx != -INFINITY) {
    const float R = mx * c;
    float e8[kQuadsPerTileLane];
#pragma unroll
    for (int k = 0; k < kQuadsPerTileLane; ++k)
      e8[k] = (__builtin_amdgcn_exp2f(fmaf(bf16_lo(v[k].x), c, -R)) +
               __builtin_amdgcn_exp2f(fmaf(bf16_hi(v[k].x), c, -R))) +
              (__builtin_amdgcn_exp2f(fmaf(bf16_lo(v[k].y), c, -R)) +
               __builtin_amdgcn_exp2f(fmaf(bf16_hi(v[k].y), c, -R)));
    ls = tree_sum8(e8);
  }
  m = mx;
  s = wave_sum_f(ls);
}

// Sweep 1 of a sampled row: the max m_t and the sum s_t of 2^(z c - m_t c)
// of every CDF tile, one wave per tile (kDraftTilesPerStep tiles in flight).
// NT: non-temporal loads, for a row that is not read again (without q);
// with q, sweep 2 reads the row again at once and cached loads serve it.
// Vectorised bf16 rows are loaded as packed quads (quad_tile_stats).
template <typename LT, bool VEC, int WAVES, bool NT>
__device__ __forceinline__ void tile_stats(const LT* zrow, long V, long nocts, int T_tiles, float c,
                                           float* tile_m, float* tile_s) {
  const int w = threadIdx.x / kWave, l = lane_id();
  if constexpr (VEC && sizeof(LT) == 2) {
    const int nquads = (int)(V / 4);
    const u32x2* zq = reinterpret_cast<const u32x2*>(zrow);
    for (int t0 = w * kDraftTilesPerStep; t0 < T_tiles; t0 += WAVES * kDraftTilesPerStep) {
      u32x2 v[kDraftTilesPerStep][kQuadsPerTileLane];
#pragma unroll
      for (int j = 0; j < kDraftTilesPerStep; ++j)
#pragma unroll
        for (int k = 0; k < kQuadsPerTileLane; ++k) {
          const int qd = (t0 + j) * kTileQuads + k * kWave + l;
          v[j][k] = ld8<NT>(zq + min(qd, nquads - 1));
        }
#pragma unroll
      for (int j = 0; j < kDraftTilesPerStep; ++j) {
#pragma unroll
        for (int k = 0; k < kQuadsPerTileLane; ++k)
          if ((t0 + j) * kTileQuads + k * kWave + l >= nquads)
            v[j][k] = u32x2{0xff80ff80u, 0xff80ff80u};
        float m, st;
        quad_tile_stats(v[j], c, m, st);
        if (l == 0 && t0 + j < T_tiles) { tile_m[t0 + j] = m; tile_s[t0 + j] = st; }
      }
    }
    return;
  }
  for (int t0 = w * kDraftTilesPerStep; t0 < T_tiles; t0 += WAVES * kDraftTilesPerStep) {
    float z[kDraftTilesPerStep][kTileLoads][8];
    if constexpr (VEC) {
      Raw<LT> raw[kDraftTilesPerStep][kTileLoads];
#pragma unroll
      for (int j = 0; j < kDraftTilesPerStep; ++j)
#pragma unroll
        for (int sl = 0; sl < kTileLoads; ++sl) {
          const long o = ((long)(t0 + j) * kTileLoads + sl) * kWave + l;
          raw_load<NT>(zrow, o < nocts ? o : nocts - 1, raw[j][sl]);
        }
#pragma unroll
      for (int j = 0; j < kDraftTilesPerStep; ++j)
#pragma unroll
        for (int sl = 0; sl < kTileLoads; ++sl) {
          const long o = ((long)(t0 + j) * kTileLoads + sl) * kWave + l;
          unpack(raw[j][sl], z[j][sl]);
          if (o >= nocts)
#pragma unroll
            for (int e = 0; e < 8; ++e) z[j][sl][e] = -INFINITY;
        }
    } else {
#pragma unroll
      for (int j = 0; j < kDraftTilesPerStep; ++j)
#pragma unroll
        for (int sl = 0; sl < kTileLoads; ++sl) {
          const long o = ((long)(t0 + j) * kTileLoads + sl) * kWave + l;
          load_octet<false>(zrow, o, V, false, -INFINITY, z[j][sl]);
        }
    }
#pragma unroll
    for (int j = 0; j < kDraftTilesPerStep; ++j) {
      float m = -INFINITY;
#pragma unroll
      for (int sl = 0; sl < kTileLoads; ++sl)
#pragma unroll
        for (int e = 0; e < 8; ++e) m = fmaxf(m, z[j][sl][e]);
      m = wave_max(m);
      float ls = 0.f;
      if (m != -INFINITY) {
        const float R = m * c;
#pragma unroll
        for (int sl = 0; sl < kTileLoads; ++sl) {
          float e8[8];
#pragma unroll
          for (int e = 0; e < 8; ++e) e8[e] = __builtin_amdgcn_exp2f(fmaf(z[j][sl][e], c, -R));
          ls += tree_sum8(e8);
        }
      }
      const float st = wave_sum_f(ls);
      if (l == 0 && t0 + j < T_tiles) { tile_m[t0 + j] = m; tile_s[t0 + j] = st; }
    }
  }
}

// The row-resident path keeps each quad packed (two VGPRs for four bf16
// logits) and unpacks it again in every pass; this empty statement, which
// claims to change the packed words, keeps the compiler from holding the
// unpacked fp32 values (twice the registers) from one pass to the next.
template <int N>
__device__ __forceinline__ void keep_packed(u32x2 (&raw)[N]) {
#pragma unroll
  for (int j = 0; j < N; ++j) asm volatile("" : "+v"(raw[j].x), "+v"(raw[j].y));
}

// WQ: q is written (out_probs non-null).  RES (a workgroup size, or 0):
// sampled rows are held in registers (bf16, VEC, WQ, V <= kResMaxV).
template <typename LT, bool VEC, bool WQ, int RES = 0>
__global__ __launch_bounds__(RES ? RES : draft_threads<WQ>()) void draft_sample_kernel(DraftArgs A) {
  constexpr int THREADS = RES ? RES : draft_threads<WQ>();
  constexpr int WAVES = THREADS / kWave;
  static_assert(!RES || (WQ && VEC && sizeof(LT) == 2), "row-resident rows: bf16 with q written");
  __shared__ float sm_f[WAVES];
  __shared__ int sm_i[WAVES];
  __shared__ double sm_d[WAVES];
  __shared__ Partial stats;
  __shared__ float tile_m[kMaxTiles];
  __shared__ float tile_s[kMaxTiles];
  __shared__ double row_S;

  const long r = blockIdx.x;                    // b * K + k
  const int b = (int)(r / A.K);
  const long V = A.V;
  const long nocts = (V + 7) / 8;
  const int t = threadIdx.x, w = t / kWave, l = lane_id();
  float* qrow = WQ ? A.out_probs + r * V : nullptr;

  const long ri = A.row_index ? (long)A.row_index[r] : r;
  if (ri < 0 || ri >= A.n_rows) {
    if (t == 0) {
      flag_error(A.device_error, SV_DEVERR_ROW_INDEX);
      A.out_tokens[r] = -1;
      if (A.out_desc) A.out_desc[r] = sv_draft_row{0.f, 0.f, 0.f, -1};   // q = 0
    }
    if constexpr (WQ) store_one_hot<VEC, THREADS>(qrow, V, nocts, -1);
    return;
  }
  const LT* zrow = static_cast<const LT*>(A.logits) + ri * V;

  bool bad;
  float c = seq_scale(A.temperatures ? A.temperatures[b] : A.temperature, bad);
  if (bad && t == 0) flag_error(A.device_error, SV_DEVERR_TEMPERATURE);
  const bool greedy = c == 0.f;
  if (greedy) c = 1.f;

  if (greedy) {
    // lowest-index argmax; q is its one-hot
    const Partial P = slice_stats<LT, GREEDY, VEC, THREADS, !WQ, true>(zrow, 0, nocts, V, c,
                                                                     sm_f, sm_i, sm_d);
    if (t == 0) stats = P;
    __syncthreads();
    const int g = stats.g == INT32_MAX ? 0 : stats.g;
    if (t == 0) {
      A.out_tokens[r] = g;
      if (A.out_desc) A.out_desc[r] = sv_draft_row{0.f, 0.f, 0.f, g};      // q = one-hot(g)
    }
    if constexpr (WQ) store_one_hot<VEC, THREADS>(qrow, V, nocts, g);
    return;
  }

  const int T_tiles = (int)((V + kTileElems - 1) / kTileElems);
  // RES: the row, once, into registers: slot i of wave w is tile w + W i, lane
  // l holding its quads k * 64 + l (k < 8).  All loads are issued back to back
  // (addresses past the row clamped to its last quad); then quads past the
  // row, all in the last tile, are set to bf16 -inf, which adds nothing.
  // Whether a slot's tile lies wholly inside the row is uniform across the
  // wave.
  constexpr int SLOTS = RES ? res_slots<THREADS>() : 1;
  constexpr int NQ = SLOTS * kQuadsPerTileLane;
  const int nquads = (int)(V / 4);
  const int wv = __builtin_amdgcn_readfirstlane(w);
  u32x2 raw[NQ];
  if constexpr (RES) {
    const u32x2* zq = reinterpret_cast<const u32x2*>(zrow);
#pragma unroll
    for (int j = 0; j < NQ; ++j) {
      const int qd = (wv + WAVES * (j / kQuadsPerTileLane)) * kTileQuads +
                     (j % kQuadsPerTileLane) * kWave + l;
      raw[j] = ld8<true>(zq + min(qd, nquads - 1));
    }
    keep_packed(raw);
#pragma unroll
    for (int i = 0; i < SLOTS; ++i) {
      const int q0 = (wv + WAVES * i) * kTileQuads;
      if (q0 + kTileQuads > nquads) {                // uniform
#pragma unroll
        for (int k = 0; k < kQuadsPerTileLane; ++k)
          if (q0 + k * kWave + l >= nquads)
            raw[i * kQuadsPerTileLane + k] = u32x2{0xff80ff80u, 0xff80ff80u};
      }
    }
    // sweep 1 from the registers: the tile statistics tile_stats computes
#pragma unroll
    for (int i = 0; i < SLOTS; ++i) {
      const int tile = wv + WAVES * i;
      if (tile < T_tiles) {                          // uniform
        float m, st;
        quad_tile_stats(raw + i * kQuadsPerTileLane, c, m, st);
        if (l == 0) { tile_m[tile] = m; tile_s[tile] = st; }
      }
    }
  } else {
    // sweep 1: per-tile max and sum of exponentials
    tile_stats<LT, VEC, WAVES, !WQ>(zrow, V, nocts, T_tiles, c, tile_m, tile_s);
  }
  __syncthreads();
  // row max M; tile masses w_t = s_t 2^(m_t c - M c) replace s_t; row sum S
  if (w == 0) {
    float M = -INFINITY;
    for (int i = l; i < T_tiles; i += kWave) M = fmaxf(M, tile_m[i]);
    M = wave_max(M);
    double part = 0.0;
    for (int i = l; i < T_tiles; i += kWave) {
      const float mt = tile_m[i];
      const float wt = mt == -INFINITY ? 0.f
          : (float)((double)tile_s[i] * exp2((double)(mt * c) - (double)M * (double)c));
      tile_s[i] = wt;
      part += (double)wt;
    }
    const double St = wave_sum(part);
    if (l == 0) { row_S = St; stats.m = M; }
  }
  __syncthreads();
  const float M = stats.m;
  const double S = row_S;
  // p = 2^(z c - Mc32) * inv_s, where Mc32 is M*c rounded to fp32 and inv_s
  // folds that rounding back in
  const float Mc = M * c;
  const float inv_s = (float)(exp2((double)Mc - (double)M * (double)c) / S);
  if (t == 0 && A.out_desc) A.out_desc[r] = sv_draft_row{c, Mc, inv_s, -1};

  if constexpr (RES) {
    // q from the registers, each element as the descriptor recomputes it
    keep_packed(raw);
    f32x4* qv = reinterpret_cast<f32x4*>(qrow);
#pragma unroll
    for (int i = 0; i < SLOTS; ++i) {
      const int q0 = (wv + WAVES * i) * kTileQuads;
      const bool whole = q0 + kTileQuads <= nquads;  // uniform
      if (q0 >= nquads) continue;                    // uniform
#pragma unroll
      for (int k = 0; k < kQuadsPerTileLane; ++k) {
        const u32x2 v = raw[i * kQuadsPerTileLane + k];
        const int qd = q0 + k * kWave + l;
        if (whole || qd < nquads) {
          const f32x4 q{__builtin_amdgcn_exp2f(fmaf(bf16_lo(v.x), c, -Mc)) * inv_s,
                        __builtin_amdgcn_exp2f(fmaf(bf16_hi(v.x), c, -Mc)) * inv_s,
                        __builtin_amdgcn_exp2f(fmaf(bf16_lo(v.y), c, -Mc)) * inv_s,
                        __builtin_amdgcn_exp2f(fmaf(bf16_hi(v.y), c, -Mc)) * inv_s};
          __builtin_nontemporal_store(q, qv + qd);
        }
      }
    }
  } else if constexpr (WQ) {
    // sweep 2: write q
    if constexpr (VEC) {
      write_q_quads<LT, WAVES>(zrow, qrow, V, c, Mc, inv_s);
    } else {
      for (int tile = w; tile < T_tiles; tile += WAVES) {
        float q[kTileLoads][8];
        tile_q<LT, VEC>(zrow, tile, V, nocts, c, Mc, inv_s, q);
#pragma unroll
        for (int sl = 0; sl < kTileLoads; ++sl) {
          const long o = ((long)tile * kTileLoads + sl) * kWave + l;
          if (o < nocts) store_q<VEC>(qrow, o, V, q[sl]);
        }
      }
    }
  }
  if (w != 0) return;

  // locate, in units of q (tile masses / S): the tile holding u (lanes own
  // contiguous runs of tiles), then the element inside it from the q values
  const int per = (T_tiles + kWave - 1) / kWave;
  const int lo = min(T_tiles, l * per), hi = min(T_tiles, (l + 1) * per);
  const double invS = 1.0 / S;
  double part = 0.0;
  for (int i = lo; i < hi; ++i) part += (double)tile_s[i] * invS;
  const double incl = wave_inclusive_scan(part);
  const double target = (double)A.uniforms[r] * __shfl(incl, kWave - 1);
  double run = __shfl_up(incl, 1);
  if (l == 0) run = 0.0;
  int hit = -1, last = -1;
  double pre = 0.0;
  for (int i = lo; i < hi; ++i) {
    const double wt = (double)tile_s[i] * invS;
    if (wt > 0.0) last = i;
    const double nxt = run + wt;
    if (hit < 0 && nxt > target) { hit = i; pre = run; }
    run = nxt;
  }
  int tile;
  bool fallback = false;
  const unsigned long long any = __ballot(hit >= 0);
  if (any) {
    const int src = __ffsll((long long)any) - 1;
    tile = __shfl(hit, src);
    pre = __shfl(pre, src);
  } else {
    // rounding left the target at or past the total: the last tile with mass
    const unsigned long long anyp = __ballot(last >= 0);
    tile = anyp ? __shfl(last, 63 - __clzll((long long)anyp)) : 0;
    fallback = true;
  }
  float q[kTileLoads][8];
  tile_q<LT, VEC>(zrow, tile, V, nocts, c, Mc, inv_s, q);
  const int pick = pick_in_tile(q, tile, pre, target, fallback);
  if (l == 0) A.out_tokens[r] = pick;
}

hipError_t launch_draft(const DraftLaunch& L, hipStream_t stream) {
  DraftArgs A;
  A.logits = L.logits;
  A.row_index = L.row_index;
  A.n_rows = L.n_rows;
  A.uniforms = L.uniforms;
  A.temperatures = L.temperatures;
  A.temperature = L.temperature;
  A.B = L.B; A.K = L.K; A.V = L.V;
  A.out_tokens = L.out_tokens;
  A.out_probs = L.out_probs;
  A.out_desc = L.out_desc;
  A.device_error = L.device_error;
  const dim3 grid((unsigned)((long)L.B * L.K));
  const bool wq = L.out_probs != nullptr;
  const dim3 block(wq ? draft_threads<true>() : draft_threads<false>());
  trace_before(stream, SV_KERNEL_DRAFT_SAMPLE);
#define SV_DRAFT(LT, VEC, WQ) \
  hipLaunchKernelGGL((draft_sample_kernel<LT, VEC, WQ>), grid, block, 0, stream, A)
  if (L.bf16) {
    if (L.vec && wq && (long)L.V <= kResMaxV)
      hipLaunchKernelGGL((draft_sample_kernel<uint16_t, true, true, kResThreads>), grid,
                         dim3(kResThreads), 0, stream, A);
    else if (L.vec) { if (wq) SV_DRAFT(uint16_t, true, true); else SV_DRAFT(uint16_t, true, false); }
    else { if (wq) SV_DRAFT(uint16_t, false, true); else SV_DRAFT(uint16_t, false, false); }
  } else {
    if (L.vec) { if (wq) SV_DRAFT(float, true, true); else SV_DRAFT(float, true, false); }
    else { if (wq) SV_DRAFT(float, false, true); else SV_DRAFT(float, false, false); }
  }
#undef SV_DRAFT
  const hipError_t err = hipGetLastError();
  trace_after(stream, SV_KERNEL_DRAFT_SAMPLE);
  return err;
}

}  // namespace sv
