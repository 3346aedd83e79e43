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

// Sweep 1 of a sampled row: the max m_t and the sum s_t of 2^(z c - m_t c)
// of every CDF tile, one wave per tile (kDraftTilesPerStep tiles in flight).
// NT: non-temporal loads, for a row that is not read again (without q);
// with q, sweep 2 reads the row again at once and cached loads serve it.
template <typename LT, bool VEC, int WAVES, bool NT>
__device__ __forceinline__ void tile_stats(const LT* zrow, long V, long nocts, int T_tiles, float c,
                                           float* tile_m, float* tile_s) {
  const int w = threadIdx.x / kWave, l = lane_id();
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

// WQ: q is written (out_probs non-null).
template <typename LT, bool VEC, bool WQ>
__global__ __launch_bounds__(draft_threads<WQ>()) void draft_sample_kernel(DraftArgs A) {
  constexpr int THREADS = draft_threads<WQ>();
  constexpr int WAVES = THREADS / kWave;
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

  // sweep 1: per-tile max and sum of exponentials
  const int T_tiles = (int)((V + kTileElems - 1) / kTileElems);
  tile_stats<LT, VEC, WAVES, !WQ>(zrow, V, nocts, T_tiles, c, tile_m, tile_s);
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
    const double S = wave_sum(part);
    if (l == 0) { row_S = S; stats.m = M; }
  }
  __syncthreads();
  const float M = stats.m;
  const double S = row_S;
  // p = 2^(z c - Mc32) * inv_s, where Mc32 is M*c rounded to fp32 and inv_s
  // folds that rounding back in
  const float Mc = M * c;
  const float inv_s = (float)(exp2((double)Mc - (double)M * (double)c) / S);
  if (t == 0 && A.out_desc) A.out_desc[r] = sv_draft_row{c, Mc, inv_s, -1};

  // sweep 2 (only when q is requested): write q
  if constexpr (WQ) {
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
    if (L.vec) { if (wq) SV_DRAFT(uint16_t, true, true); else SV_DRAFT(uint16_t, true, false); }
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
