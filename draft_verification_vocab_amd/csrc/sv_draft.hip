// Drafter-output sampling for gfx950: the P-EAGLE drafter's K prediction rows
// per sequence -> the K draft tokens and the drafter distribution q that the
// next verify tests them against (P-EAGLE / TorchSpec blog summary, section
// 并行架构的核心创新: one drafter forward predicts all K drafts; "Project 14 -
// speculative decoding inference server", section 架构: the drafter proposes,
// the target verifies).
//
// One workgroup per draft (b, k); no workgroup hands anything to another.
//   sweep 1  streams the drafter logit row and reduces it to its max and sum
//            of exponentials at the sequence's temperature, or to its
//            lowest-index argmax when that temperature is 0 (greedy);
//   sweep 2  streams the row again, writes q = softmax(z / T) as fp32 and
//            keeps the mass of every 2048-element CDF tile in LDS;
//   locate   one wave finds the tile whose running total first exceeds u * S,
//            rescans that tile and writes the token.
// Greedy rows skip sweep 2's loads: q is the one-hot of the argmax.
// The q rows are written with non-temporal stores: the next verify reads only
// a few of their elements and one row per sequence.
#include "sv_device.h"
#include "sv_internal.h"
#include "sv_rowstats.h"

namespace sv {

constexpr int kDraftThreads = 512;      // 8 waves
constexpr int kDraftWaves = kDraftThreads / kWave;

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

// Whole q row: the one-hot of g (g < 0: all zero), stores only.
template <bool VEC>
__device__ void store_one_hot(float* qrow, long V, long nocts, int g) {
  for (long o = threadIdx.x; o < nocts; o += kDraftThreads) {
    float q[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) q[j] = (o * 8 + j == g) ? 1.f : 0.f;
    store_q<VEC>(qrow, o, V, q);
  }
}

template <typename LT, bool VEC>
__global__ __launch_bounds__(kDraftThreads) void draft_sample_kernel(DraftArgs A) {
  __shared__ float sm_f[kDraftWaves];
  __shared__ int sm_i[kDraftWaves];
  __shared__ double sm_d[kDraftWaves];
  __shared__ Partial stats;
  __shared__ float tsum[kMaxTiles];

  const long r = blockIdx.x;                    // b * K + k
  const int b = (int)(r / A.K);
  const long V = A.V;
  const long nocts = (V + 7) / 8;
  const int t = threadIdx.x, w = t / kWave, l = lane_id();
  float* qrow = A.out_probs ? A.out_probs + r * V : nullptr;

  const long ri = A.row_index ? (long)A.row_index[r] : r;
  if (ri < 0 || ri >= A.n_rows) {
    if (t == 0) {
      flag_error(A.device_error, SV_DEVERR_ROW_INDEX);
      A.out_tokens[r] = -1;
    }
    if (qrow) store_one_hot<VEC>(qrow, V, nocts, -1);
    return;
  }
  const LT* zrow = static_cast<const LT*>(A.logits) + ri * V;

  float T = A.temperatures ? A.temperatures[b] : A.temperature;
  float c = 1.f;
  bool greedy = T == 0.f;
  if (!greedy) {
    c = (float)(1.4426950408889634 / (double)T);
    if (!(T > 0.f) || !isfinite(T) || !isfinite(c)) {
      if (t == 0) flag_error(A.device_error, SV_DEVERR_TEMPERATURE);
      greedy = true;
      c = 1.f;
    }
  }

  // sweep 1: row statistics (greedy -> argmax; sampling -> max, sum of 2^(zc - Mc))
  Partial P;
  if (greedy) P = slice_stats<LT, GREEDY, VEC, kDraftThreads>(zrow, 0, nocts, V, c, sm_f, sm_i, sm_d);
  else P = slice_stats<LT, SAMPLE, VEC, kDraftThreads>(zrow, 0, nocts, V, c, sm_f, sm_i, sm_d);
  if (t == 0) stats = P;
  __syncthreads();
  P = stats;

  if (greedy) {
    const int g = P.g == INT32_MAX ? 0 : P.g;
    if (t == 0) A.out_tokens[r] = g;
    if (qrow) store_one_hot<VEC>(qrow, V, nocts, g);
    return;
  }

  // sweep 2: q and the CDF tile masses.  p = 2^(z c - Mc32) * inv_s, where
  // Mc32 is M*c rounded to fp32 and inv_s folds that rounding back in.
  const float Mc = P.m * c;
  const float inv_s = (float)(exp2((double)Mc - (double)P.m * (double)c) / P.acc);
  const int T_tiles = (int)((V + kTileElems - 1) / kTileElems);
  for (int tile = w; tile < T_tiles; tile += kDraftWaves) {
    float q[kTileLoads][8];
    tile_q<LT, VEC>(zrow, tile, V, nocts, c, Mc, inv_s, q);
    float ls = 0.f;
#pragma unroll
    for (int sl = 0; sl < kTileLoads; ++sl) {
      const long o = ((long)tile * kTileLoads + sl) * kWave + l;
      if (qrow && o < nocts) store_q<VEC>(qrow, o, V, q[sl]);
      ls += tree_sum8(q[sl]);
    }
    const float ts = wave_sum_f(ls);
    if (l == 0) tsum[tile] = ts;
  }
  __syncthreads();
  if (w != 0) return;

  // locate: the tile holding u * S (lanes own contiguous runs of tiles) ...
  const int per = (T_tiles + kWave - 1) / kWave;
  const int lo = min(T_tiles, l * per), hi = min(T_tiles, (l + 1) * per);
  double part = 0.0;
  for (int i = lo; i < hi; ++i) part += (double)tsum[i];
  const double incl = wave_inclusive_scan(part);
  const double S = __shfl(incl, kWave - 1);
  const double target = (double)A.uniforms[r] * S;
  double run = __shfl_up(incl, 1);
  if (l == 0) run = 0.0;
  int hit = -1, last = -1;
  double pre = 0.0;
  for (int i = lo; i < hi; ++i) {
    const float ts = tsum[i];
    if (ts > 0.f) last = i;
    const double nxt = run + (double)ts;
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
    // rounding left u*S at or past the total: the last tile with positive mass
    const unsigned long long anyp = __ballot(last >= 0);
    tile = anyp ? __shfl(last, 63 - __clzll((long long)anyp)) : 0;
    fallback = true;
  }
  // ... then the element inside it, from the same q values
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
  A.device_error = L.device_error;
  const dim3 grid((unsigned)((long)L.B * L.K)), block(kDraftThreads);
  trace_before(stream, SV_KERNEL_DRAFT_SAMPLE);
  if (L.bf16) {
    if (L.vec) hipLaunchKernelGGL((draft_sample_kernel<uint16_t, true>), grid, block, 0, stream, A);
    else hipLaunchKernelGGL((draft_sample_kernel<uint16_t, false>), grid, block, 0, stream, A);
  } else {
    if (L.vec) hipLaunchKernelGGL((draft_sample_kernel<float, true>), grid, block, 0, stream, A);
    else hipLaunchKernelGGL((draft_sample_kernel<float, false>), grid, block, 0, stream, A);
  }
  const hipError_t err = hipGetLastError();
  trace_after(stream, SV_KERNEL_DRAFT_SAMPLE);
  return err;
}

}  // namespace sv
