// Batched speculative verify-and-accept for gfx950.
//
// verify_rows: one workgroup per (sequence b, logit row k, vocabulary split
// s).  Each workgroup streams its slice of row k from HBM once and reduces it
// to a partial: the max and its lowest index (greedy), or the max and the sum
// of exponentials relative to it (sampling).  Nothing else: no workgroup of
// this kernel waits for or hands anything to another.
//
// The accept scan: one wave per sequence (one lane per row) combines the
// sequence's partials, tests every draft in parallel and takes the first
// rejection from a wave ballot.  Greedy verify runs it in verify_accept,
// which writes the argmax of row a as the new token.
//
// verify_draw (sampling, mixed batches): C workgroups per sequence each run
// the accept scan (chunk 0 writes its outputs and leaves a, max and sum of
// row a for the locate kernel), then take a contiguous chunk of row a and
// store the mass r = max(0, p_a - q_a) (or p_K for the bonus token) of each
// 2048-element tile in it.
// verify_locate: one wave per sequence finds the tile whose running total
// first exceeds u * S, rescans that one tile and writes the token.  With one
// draw workgroup per sequence (C = 1) that workgroup keeps the tile masses in
// LDS and runs the same search itself, and no locate kernel is launched.
// Every hand-off between workgroups goes through a kernel boundary.
//
// The verify flow is that of "Project 14 - speculative decoding inference
// server", section 架构 (architecture): accept the prefix, resample the
// rejected suffix.  The bitmask form of the accept scan follows the rskf.cn
// survey, section 3.3 (DFlash): one bit per draft instead of a branch per
// draft; here the bits come from a wave64 ballot.
#include <math.h>

#include "sv_device.h"
#include "sv_internal.h"
#include "sv_rowstats.h"

namespace sv {

struct ScanResult {  // outcome of a sequence's accept scan
  int a;             // accepted drafts
  int g_a;           // greedy: argmax of row a
  float M_a;         // max of row a
  float c;           // the sequence's exponent scale; 0 = greedy (nothing to draw)
  double s_a;        // sampling: sum over row a of 2^((z - M_a) * c)
};

constexpr int kThreads = 256;           // 4 waves
constexpr int kWaves = kThreads / kWave;
constexpr int kMaxSplits = 16;          // workgroups per logit row at most
constexpr int kTileUnroll = 1;          // draw: tiles per wave per step
constexpr int kLevelSlots = 64;         // early exit: ranges after the first (<= 6 for K < 64)
// Early exit: gate kernels from these batch sizes on (below, ranges with the
// scan in every workgroup).  GPU time per call at K = 7, V = 151936 bf16,
// inline against listed: greedy 30.5 / 34.5 us at B = 64 (V = 201088), 39.7 /
// 36.8 at B = 128, 81.6 / 49.0 at B = 256; sampled 63.6 / 68.9 at B = 64,
// 84.6 / 91.1 at B = 128, 125.1 / 125.2 at B = 256, 187.8 / 181.5 at B = 512,
// 326.7 / 312.1 at B = 1024 (mixed batches alike).
constexpr int kListedMinBatchGreedy = 128;
constexpr int kListedMinBatchSampled = 512;

// ---------------------------------------------------------------- workspace
// scan results [B] | tile sums [B][T] | partials [B][K+1][S] |
// early-exit range counters [kLevelSlots] and sequence list [B]
struct Layout {
  size_t info, tile, partials, levels, total;
  int S, C, T;
  int Sg;            // splits of the greedy early-exit form (partials sized for max(S, Sg))
};

static inline size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

int verify_splits(int B, int K, int V) {
  const long rows = (long)B * (K + 1);
  const long octets = (V + 7) / 8;
  long s = (2048 + rows - 1) / rows;
  s = s < kMaxSplits ? s : kMaxSplits;
  long cap = octets / 256;
  if (s > cap) s = cap;
  return s < 1 ? 1 : (int)s;
}

// Splits per row of the greedy early-exit form: at least as many as the full
// call's, and enough that the few rows of a later range still spread over
// the chip (about 4096 workgroups for the first range).  A greedy row's
// maximum and lowest argmax do not depend on the split, so its outputs are
// those of the full call.
static int greedy_ee_splits(int B, int K, int V) {
  const int S = verify_splits(B, K, V);
  long s = (4096 + (long)B - 1) / (B > 0 ? B : 1);
  if (s > kMaxSplits) s = kMaxSplits;
  const long cap = ((long)V + 7) / 8 / 256;
  if (s > cap) s = cap;
  return s > S ? (int)s : S;
}

// Draw workgroups per sequence (for the batches below 256 sequences, and
// mixed batches; see launch_verify for the rest): about one round of
// resident workgroups over the whole chip (256 CUs x 5 resident draw
// workgroups of 4 waves), since
// every workgroup first waits on its sequence's accept scan.  Measured draw
// times (V=151936 bf16 unless noted): B=64 (V=201088) 21 us at 20 chunks vs
// 29 us at 64; B=128 27 vs 35 us at 32; B=256 45 vs 51 us at 16; B=1024
// 154-156 us for every count from 1 to 6.
constexpr long kDrawWorkgroups = 1280;

// In a mixed batch the greedy sequences' workgroups stop after the scan, so
// at least 4 chunks per sequence let the sampled sequences' rows spread over
// the CUs those leave idle (B=1024 with 199 greedy sequences: draw + locate
// 144 us at 4 chunks, 149 us for the draw alone at one workgroup per
// sequence).
static int draw_chunks(int B, int V, bool mixed = false) {
  const long tiles = (V + kTileElems - 1) / kTileElems;
  long c = (kDrawWorkgroups + B / 2) / B;
  if (mixed && c < 4) c = 4;
  if (c > tiles) c = tiles;
  return c < 1 ? 1 : (int)c;
}

static Layout layout(int B, int K, int V) {
  Layout L;
  L.S = verify_splits(B, K, V);
  L.Sg = greedy_ee_splits(B, K, V);
  L.C = draw_chunks(B, V);
  L.T = (V + kTileElems - 1) / kTileElems;
  size_t off = 0;
  L.info = off;     off = align256(off + (size_t)B * sizeof(ScanResult));
  L.tile = off;     off = align256(off + (size_t)B * L.T * sizeof(float));
  L.partials = off; off = align256(off + (size_t)B * (K + 1) * (L.S > L.Sg ? L.S : L.Sg) * sizeof(Partial));
  L.levels = off;   off = align256(off + (kLevelSlots + (size_t)B) * sizeof(int32_t));
  L.total = off;
  return L;
}

size_t verify_workspace_bytes(int B, int K, int V) { return layout(B, K, V).total; }

RowPartials row_partials(void* workspace, int B, int K, int V) {
  const Layout lay = layout(B, K, V);
  return RowPartials{reinterpret_cast<char*>(workspace) + lay.partials, lay.S};
}

struct RowsArgs {
  const void* logits;
  const float* temperatures;  // mixed: [B] per-sequence temperatures
  float c;                 // log2(e) / T   (sampling)
  int K, V, S;
  long octets;             // ceil(V / 8)
  Partial* partials;       // [B][K+1][S]
};

struct ScanArgs {          // what an accept scan reads and writes
  const void* logits;
  const float* temperatures;  // mixed: [B]
  const void* dlogits;        // q from the drafter logits: [d_rows][V]
  long d_rows;
  const int32_t* drows;       // [B*K] or null (row b*K + k)
  const sv_draft_row* ddesc;  // [B*K]
  const float* draft_probs;
  const int32_t* draft_tokens;
  const float* uniforms;
  float c;
  int B, K, V, S;
  Partial* partials;       // [B][K+1][S]
  ScanResult* info;        // [B] written by verify_draw, read by verify_locate
  int32_t* out_tokens;
  int32_t* out_num_accepted;
  float* out_p_draft;
  int32_t* device_error;
  int prefix_only;         // early exit: rows past the first rejection hold no statistics
  int* level_counts;       // early exit: the gates' counters [kLevelSlots] and their
                           // sequence list [B], cleared by the call's last kernel (else null)
};

// The call's last kernel leaves the early-exit counters and list zero for the
// next call: workgroup 0 clears the counters, and the thread that `owns`
// sequence b its list entry.
__device__ __forceinline__ void clear_level_state(const ScanArgs& A, int b, bool owns) {
  if (!A.level_counts) return;
  if (blockIdx.x == 0 && threadIdx.x < kLevelSlots) A.level_counts[threadIdx.x] = 0;
  if (owns) A.level_counts[kLevelSlots + b] = 0;
}

struct DrawArgs {
  ScanArgs sc;
  int C, T;
  float* tile_sums;        // [B][T]
};

// ----------------------------------------------------------------------------
template <typename LT, int MODE, bool VEC>
__global__ __launch_bounds__(kThreads) void verify_rows(RowsArgs A) {
  __shared__ float sm_f[kWaves];
  __shared__ int sm_i[kWaves];
  __shared__ double sm_d[kWaves];

  const int S = A.S;
  const long V = A.V;
  const long unit = blockIdx.x;                 // ((b * (K+1)) + k) * S + s
  const int s = (int)(unit % S);
  const long rowi = unit / S;                   // b * (K+1) + k
  const LT* row = static_cast<const LT*>(A.logits) + rowi * V;
  const long o_lo = (long)s * A.octets / S, o_hi = (long)(s + 1) * A.octets / S;

  Partial P;
  if constexpr (MODE == MIXED) {
    // the sequence's own rule; uniform across the workgroup
    bool bad;
    const float c = seq_scale(A.temperatures[rowi / (A.K + 1)], bad);
    if (c == 0.f) P = slice_stats<LT, GREEDY, VEC, kThreads>(row, o_lo, o_hi, V, 1.f, sm_f, sm_i, sm_d);
    else P = slice_stats<LT, SAMPLE, VEC, kThreads>(row, o_lo, o_hi, V, c, sm_f, sm_i, sm_d);
  } else {
    P = slice_stats<LT, MODE, VEC, kThreads>(row, o_lo, o_hi, V, A.c, sm_f, sm_i, sm_d);
  }
  if (threadIdx.x == 0) A.partials[unit] = P;   // read by the next kernel
}

// ----------------------------------------------------------------------------
// Accept scan of sequence b by one full wave (lane k holds row k <= K).
// Combines the S partials of each row, tests every draft, finds the first
// rejection with a ballot.  With `write` it writes the accepted prefix, the
// -1 padding, num_accepted and p_k(d_k); the new token is written by the
// caller (greedy: g_a; sampling: the draw).
template <typename LT, int MODE, bool QL = false>
__device__ __forceinline__ ScanResult accept_scan(const ScanArgs& A, int b, bool write, float c) {
  const int K = A.K, S = A.S;
  const long V = A.V;
  const int k = lane_id();
  const Partial* Pb = A.partials + (long)b * (K + 1) * S;
  float M = -INFINITY;
  int g = INT32_MAX;
  double s_k = 0.0;
  if (k <= K) {
    // all of the row's partials are loaded at once (S <= kMaxSplits), so the
    // scan waits for one load latency, not S of them
    Partial pk[kMaxSplits];
#pragma unroll
    for (int j = 0; j < kMaxSplits; ++j)
      if (j < S) pk[j] = Pb[k * S + j];
    if constexpr (MODE == GREEDY) {
#pragma unroll
      for (int j = 0; j < kMaxSplits; ++j)
        if (j < S && (j == 0 || pk[j].m > M)) { M = pk[j].m; g = pk[j].g; }
    } else {
#pragma unroll
      for (int j = 0; j < kMaxSplits; ++j)
        if (j < S) M = fmaxf(M, pk[j].m);
#pragma unroll
      for (int j = 0; j < kMaxSplits; ++j)
        if (j < S && pk[j].acc != 0.0)
          s_k += pk[j].acc * exp2_split(((double)pk[j].m - (double)M) * (double)c);
    }
  }
  int d = -1;
  bool rej = false;
  float pdraft = 0.f;
  if (k < K) {
    d = A.draft_tokens[(long)b * K + k];
    const bool valid = d >= 0 && d < V;
    if constexpr (MODE == GREEDY) {
      rej = !(valid && d == g);
      pdraft = rej ? 0.f : 1.f;           // the T -> 0 limit of p_k(d_k)
    } else {
      double px = 0.0;
      if (valid) {
        const LT* zr = static_cast<const LT*>(A.logits) + ((long)b * (K + 1) + k) * V;
        const float zx = logit_at(zr, d);
        px = exp2(((double)zx - (double)M) * (double)c) / s_k;
        double qx;
        if constexpr (QL) {
          // q_k(x) recomputed from drafter row r with the drafter's operations
          const long j = (long)b * K + k;
          const long r = A.drows ? (long)A.drows[j] : j;
          if (r >= 0 && r < A.d_rows) {
            qx = (double)drafter_q(A.ddesc[j], logit_at(static_cast<const LT*>(A.dlogits) + r * V, d), d);
          } else {
            qx = 0.0;
            if (write) flag_error(A.device_error, SV_DEVERR_ROW_INDEX);
          }
        } else {
          qx = (double)A.draft_probs[((long)b * K + k) * V + d];
        }
        const double ratio = qx > 0.0 ? px / qx : (px > 0.0 ? INFINITY : 0.0);
        rej = !((double)A.uniforms[(long)b * (K + 1) + k] < ratio);
      } else {
        rej = true;
      }
      pdraft = (float)px;
    }
    if (write && !valid) flag_error(A.device_error, SV_DEVERR_DRAFT_TOKEN);
  }
  const unsigned long long rejmask = __ballot(k < K && rej);
  ScanResult r;
  r.a = rejmask ? __ffsll((long long)rejmask) - 1 : K;
  r.g_a = __shfl(g, r.a);
  r.M_a = __shfl(M, r.a);
  r.s_a = __shfl(s_k, r.a);
  r.c = MODE == SAMPLE ? c : 0.f;
  if (write) {
    if (k <= K && k != r.a) A.out_tokens[(long)b * (K + 1) + k] = k < r.a ? d : -1;
    if (k == 0) A.out_num_accepted[b] = r.a;
    if (k < K && A.out_p_draft)
      A.out_p_draft[(long)b * K + k] = A.prefix_only && k > r.a ? 0.f : pdraft;
  }
  return r;
}

// The row partials of sequence b are consumed: clear them (one wave), so the
// workspace ends all zero.
__device__ __forceinline__ void clear_partials(const ScanArgs& A, int b) {
  Partial* Pb = A.partials + (long)b * (A.K + 1) * A.S;
  for (int i = lane_id(); i < (A.K + 1) * A.S; i += kWave) Pb[i] = Partial{0.f, 0, 0.0};
}

// Greedy verify: one wave per sequence runs the accept scan and writes g_a as
// the new token.  (Sampling and mixed batches run the scan inside verify_draw.)
template <typename LT>
__global__ __launch_bounds__(kThreads) void verify_accept(ScanArgs A) {
  const int b = blockIdx.x * kWaves + threadIdx.x / kWave;
  const int l = lane_id();
  clear_level_state(A, b, b < A.B && l == 0);
  if (b >= A.B) return;
  const ScanResult r = accept_scan<LT, GREEDY>(A, b, true, 1.f);
  if (l == 0) A.out_tokens[(long)b * (A.K + 1) + r.a] = r.g_a;
  clear_partials(A, b);
}

// The accept scan of sequence b as the draw needs it, by one full wave.  Every
// draw workgroup of b runs it (it reads the row partials and two values per
// draft, a few hundred bytes); the workgroup of chunk 0 (`write`) also writes
// the accept outputs, the greedy token of a greedy sequence of a mixed batch,
// and the result for verify_locate.
template <typename LT, int MODE, bool QL>
__device__ __forceinline__ ScanResult draw_scan(const ScanArgs& A, int b, bool write,
                                                bool handoff) {
  ScanResult r;
  if constexpr (MODE == MIXED) {
    bool bad;
    const float c = seq_scale(A.temperatures[b], bad);
    if (write && bad && lane_id() == 0) flag_error(A.device_error, SV_DEVERR_TEMPERATURE);
    if (c == 0.f) {
      r = accept_scan<LT, GREEDY>(A, b, write, 1.f);          // r.c = 0: nothing to draw
      if (write && lane_id() == 0) A.out_tokens[(long)b * (A.K + 1) + r.a] = r.g_a;
    } else {
      r = accept_scan<LT, SAMPLE, QL>(A, b, write, c);
    }
  } else {
    r = accept_scan<LT, SAMPLE, QL>(A, b, write, A.c);
  }
  if (handoff && lane_id() == 0) A.info[b] = r;              // read by verify_locate
  return r;
}

// ----------------------------------------------------------------------------
// Early exit: the statistics of rows k0 .. k1-1 of every sequence whose
// drafts 0..k0-1 were all accepted.  A draft is tested only if every earlier
// one was accepted (speculative sampling's acceptance is sequential: Project
// 14, 架构), so the rows past a sequence's first rejection never enter its
// outputs.  The launches cover the draft positions in ranges [0,1), [1,2),
// [2,4), [4,8), ...: one launch per position would make every deep position
// cost a full row pass by a single workgroup (~21 us at V = 151936), while a
// range reads, for the few sequences still undecided, some rows that turn
// out not to be needed.
//
// verify_level_gate (before every range but the first): one wave per
// sequence runs the accept scan over the statistics written by the earlier
// launches, with the arithmetic of the final scan, so both take the same
// decisions, and appends b to the range's list when the first rejection
// lies at or past k0 (rows from k0 on hold no statistics yet, and sit at or
// past k0, so their lanes cannot move a first rejection that lies before
// it).  The list's order follows the atomics; it decides only which
// workgroup of the range computes which row, not any value.
template <typename LT, int MODE, bool QL>
__global__ __launch_bounds__(kThreads) void verify_level_gate(ScanArgs sc, int k0, int* count,
                                                              int32_t* list) {
  const int b = blockIdx.x * kWaves + threadIdx.x / kWave;
  if (b >= sc.B) return;
  int a;
  if constexpr (MODE == GREEDY) a = accept_scan<LT, GREEDY>(sc, b, false, 1.f).a;
  else a = draw_scan<LT, MODE, QL>(sc, b, false, false).a;
  if (lane_id() == 0 && a >= k0) {
    const int slot = atomicAdd(count, 1);
    if (slot < sc.B) list[slot] = b;           // always, unless the workspace was left dirty
  }
}

// verify_rows_level: the row statistics of one range.  Work item i is
// (sequence i / (n S), row k0 + i / S % n, split i % S), over
//   kAllSeqs  every sequence, one workgroup per item (the first range);
//   kListed   the gate's list: the grid covers every sequence, as the host
//             does not know the list's length at launch, and a workgroup
//             past the listed items returns at once (measured 2-3 us faster
//             per sampled call than a grid of at most 2048 workgroups
//             striding over the items, whose loop cost ~30 VGPRs);
//   kInline   every sequence, one workgroup per item, whose wave 0 first runs
//             the gate's scan itself and returns when the sequence is decided
//             (small batches: one launch per range instead of two, at the
//             cost of a scan in every workgroup of the range).
// Batches of many sequences take kListed with finer greedy splits (S from
// greedy_ee_splits), so that the few rows of a later range spread over more
// workgroups; a sampled row keeps the full call's split, on which its sum's
// rounding depends.
constexpr int kAllSeqs = 0, kListed = 1, kInline = 2;
template <typename LT, int MODE, bool VEC, int THREADS>
__device__ __forceinline__ void level_item(const RowsArgs& A, int b, int k, int s, float* sm_f,
                                           int* sm_i, double* sm_d) {
  const int S = A.S;
  const long V = A.V;
  const long rowi = (long)b * (A.K + 1) + k;
  const LT* row = static_cast<const LT*>(A.logits) + rowi * V;
  const long o_lo = (long)s * A.octets / S, o_hi = (long)(s + 1) * A.octets / S;
  Partial P;
  if constexpr (MODE == MIXED) {
    bool bad;
    const float c = seq_scale(A.temperatures[b], bad);
    if (c == 0.f) P = slice_stats<LT, GREEDY, VEC, THREADS>(row, o_lo, o_hi, V, 1.f, sm_f, sm_i, sm_d);
    else P = slice_stats<LT, SAMPLE, VEC, THREADS>(row, o_lo, o_hi, V, c, sm_f, sm_i, sm_d);
  } else {
    P = slice_stats<LT, MODE, VEC, THREADS>(row, o_lo, o_hi, V, A.c, sm_f, sm_i, sm_d);
  }
  if (threadIdx.x == 0) A.partials[rowi * S + s] = P;   // read by the next launches
}

template <typename LT, int MODE, bool VEC, int FORM, bool QL = false>
__global__ __launch_bounds__(kThreads) void verify_rows_level(RowsArgs A, ScanArgs sc, int k0,
                                                            int k1, const int* count,
                                                            const int32_t* list) {
  __shared__ float sm_f[kWaves];
  __shared__ int sm_i[kWaves];
  __shared__ double sm_d[kWaves];
  const int S = A.S;
  const int n = k1 - k0;
  if constexpr (FORM != kListed) {
    const int i = blockIdx.x;
    const int b = i / (n * S);
    if constexpr (FORM == kInline) {
      __shared__ int s_go;
      if (threadIdx.x < kWave) {
        int a;
        if constexpr (MODE == GREEDY) a = accept_scan<LT, GREEDY>(sc, b, false, 1.f).a;
        else a = draw_scan<LT, MODE, QL>(sc, b, false, false).a;
        if (threadIdx.x == 0) s_go = a >= k0;
      }
      __syncthreads();
      if (!s_go) return;
    }
    level_item<LT, MODE, VEC, kThreads>(A, b, k0 + i / S % n, i % S, sm_f, sm_i, sm_d);
  } else {
    const int i = blockIdx.x;                  // < B n S: list entry i / (n S) exists
    if (i >= *count * n * S) return;           // count: written by the gate
    const int b = list[i / (n * S)];
    if ((unsigned)b >= (unsigned)sc.B) return; // only a workspace left dirty could hold one
    level_item<LT, MODE, VEC, kThreads>(A, b, k0 + i / S % n, i % S, sm_f, sm_i, sm_d);
  }
}

// ----------------------------------------------------------------------------
// Everything the draw needs about sequence b's row a.
template <typename LT>
struct DrawRow {
  const LT* zrow;
  const float* qrow;       // dense q row a (null for the bonus draw or with QL)
  const LT* dzrow;         // QL: drafter logit row of draft a (null: q = 0)
  sv_draft_row desc;       // QL: its descriptor
  bool residual;           // a < K: draw from max(0, p - q); else the bonus from p
  float c, Mc32, inv_s;
  int a;
};

template <typename LT, bool QL>
__device__ __forceinline__ DrawRow<LT> draw_row(const DrawArgs& A, int b, const ScanResult& scan) {
  const int K = A.sc.K;
  const long V = A.sc.V;
  DrawRow<LT> r;
  r.a = scan.a;
  r.zrow = static_cast<const LT*>(A.sc.logits) + ((long)b * (K + 1) + scan.a) * V;
  r.residual = scan.a < K;
  r.qrow = nullptr;
  r.dzrow = nullptr;
  r.desc = sv_draft_row{0.f, 0.f, 0.f, -1};
  if (r.residual) {
    const long j = (long)b * K + scan.a;
    if constexpr (QL) {
      const long row = A.sc.drows ? (long)A.sc.drows[j] : j;
      if (row >= 0 && row < A.sc.d_rows) {
        r.dzrow = static_cast<const LT*>(A.sc.dlogits) + row * V;
        r.desc = A.sc.ddesc[j];
      }
    } else {
      r.qrow = A.sc.draft_probs + j * V;
    }
  }
  r.c = scan.c;                               // 0: a greedy sequence of a mixed batch
  // p = 2^(z*c - M*c) / s.  Mc32 is M*c rounded to fp32; the rounding is
  // folded into the scale so that p keeps the fp64 reference exactly.
  r.Mc32 = scan.M_a * r.c;
  r.inv_s = r.c == 0.f ? 0.f
      : (float)(exp2((double)r.Mc32 - (double)scan.M_a * (double)r.c) / scan.s_a);
  return r;
}

// Masses of this lane's 8 elements of wave load g of the draw row (the quad
// layout: r[4 h + j] is element 512 g + 256 h + 4 l + j): max(0,
// p - q) (residual) or p.  q comes from the dense q row, or (QL) from the
// drafter logit row and descriptor.  Every row here is read once per step:
// non-temporal loads (measured over whole sampled steps at B=1024,
// V=151936: 541 us, against 546 us with cached logit loads, whose 311 MB
// evict from the Infinity Cache the hidden states the build reads next, and
// 550 us with cached q loads).  VEC: V is a multiple of 8 and the rows 16-byte
// aligned, so a quad lies wholly inside or wholly past the row; a quad past
// it loads from the row's start and is masked.
template <typename LT, bool VEC, bool QL>
__device__ __forceinline__ void wave_load_mass(const DrawRow<LT>& R, long g, long V,
                                               bool residual, float r[8]) {
  const int l = lane_id();
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const long e = g * kTile + h * (kTile / 2) + 4 * l;   // 512 g + 256 h + 4 l
    float z[4], q[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) q[j] = 0.f;
    if constexpr (VEC) {
      const bool in = e < V;
      const long ec = in ? e : 0;
      Quad<LT> qz;
      load_quad<true>(R.zrow, ec, qz);
      unpack(qz, z);
      if (residual) {
        if constexpr (QL) {
          if (R.dzrow) {
            Quad<LT> qd;
            load_quad<true>(R.dzrow, ec, qd);
            float dz[4];
            unpack(qd, dz);
#pragma unroll
            for (int j = 0; j < 4; ++j) q[j] = drafter_q(R.desc, dz[j], ec + j);
          }
        } else {
          Quad<float> qq;
          load_quad<true>(R.qrow, ec, qq);
          unpack(qq, q);
        }
      }
      if (!in) {
#pragma unroll
        for (int j = 0; j < 4; ++j) { z[j] = -INFINITY; q[j] = 0.f; }
      }
    } else {
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const long ej = e + j;
        z[j] = ej < V ? logit_at(R.zrow, ej) : -INFINITY;
        if (residual && ej < V) {
          if constexpr (QL) {
            if (R.dzrow) q[j] = drafter_q(R.desc, logit_at(R.dzrow, ej), ej);
          } else {
            q[j] = R.qrow[ej];
          }
        }
      }
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const float p = __builtin_amdgcn_exp2f(fmaf(z[j], R.c, -R.Mc32)) * R.inv_s;
      r[4 * h + j] = residual ? fmaxf(0.f, p - q[j]) : p;
    }
  }
}

// Mass of tile t seen by one lane: the sum of its masses in the tile's
// kTileLoads wave loads.
template <typename LT, bool VEC, bool QL>
__device__ __forceinline__ float lane_tile_mass(const DrawRow<LT>& R, bool residual, int t,
                                                long V) {
  float ls = 0.f;
#pragma unroll
  for (int sl = 0; sl < kTileLoads; ++sl) {
    float r[8];
    wave_load_mass<LT, VEC, QL>(R, (long)t * kTileLoads + sl, V, residual, r);
    ls += tree_sum8(r);
  }
  return ls;
}

// The token drawn from row a of one sequence by one wave, given the row's T
// tile masses: lane l holds the masses of its contiguous run of tiles [lo,
// hi) in ts (loaded by the caller).  u * S (S = the sum of the masses) picks
// the tile, then the element inside it (pick_in_quad_tile).  In the rare case
// that the residual has no mass (the drafter row sums to more than p_a) the
// wave recomputes every tile mass of p_a into `masses` (global memory with
// agent-coherent stores and loads, or LDS) and draws from p_a.
struct TileChoice {
  int tile;            // the CDF tile that holds u * S
  int residual;        // the masses are those of the residual (else of p: the bonus,
                       // or a residual that has no mass)
  int fallback;        // rounding left u * S at or past the total: the tile's last
                       // element with positive mass
  double pre;          // running total before the tile
  double target;       // u * S
};

template <typename LT, bool VEC, bool QL, bool IN_LDS>
__device__ __forceinline__ TileChoice locate_tile(const DrawRow<LT>& R, float u, int T, long V,
                                                  float (&ts)[kMaxTiles / kWave], float* masses) {
  constexpr int kPer = kMaxTiles / kWave;
  const int l = lane_id();
  const int per = (T + kWave - 1) / kWave;
  const int lo = min(T, l * per), hi = min(T, (l + 1) * per);
  bool residual = R.residual;
  double part = 0.0;
#pragma unroll
  for (int j = 0; j < kPer; ++j) part += (double)ts[j];
  double incl = wave_inclusive_scan(part);
  double S = __shfl(incl, kWave - 1);
  if (residual && !(S > 0.0)) {
    residual = false;
    for (int t = 0; t < T; ++t) {
      const float m = wave_sum_f(lane_tile_mass<LT, VEC, QL>(R, false, t, V));
      if (l == 0) {
        if constexpr (IN_LDS) masses[t] = m;
        else st_coherent(&masses[t], m);
      }
    }
    if constexpr (!IN_LDS) wait_stores_performed();
    part = 0.0;
#pragma unroll
    for (int j = 0; j < kPer; ++j) {
      if constexpr (IN_LDS) ts[j] = lo + j < hi ? masses[lo + j] : 0.f;
      else ts[j] = lo + j < hi ? ld_coherent(&masses[lo + j]) : 0.f;
      part += (double)ts[j];
    }
    incl = wave_inclusive_scan(part);
    S = __shfl(incl, kWave - 1);
  }
  const double target = (double)u * S;

  // the tile that holds u * S
  double run = __shfl_up(incl, 1);
  if (l == 0) run = 0.0;
  int hit = -1, last = -1;
  double pre = 0.0;
#pragma unroll
  for (int j = 0; j < kPer; ++j) {
    if (lo + j >= hi) break;
    if (ts[j] > 0.f) last = lo + j;
    const double nxt = run + (double)ts[j];
    if (hit < 0 && nxt > target) { hit = lo + j; pre = run; }
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
  return TileChoice{tile, residual ? 1 : 0, fallback ? 1 : 0, pre, target};
}

// The drawn token inside the chosen tile: its kTileLoads wave loads are
// loaded again (all at once) and walked.
template <typename LT, bool VEC, bool QL>
__device__ __forceinline__ int pick_in_choice(const DrawRow<LT>& R, const TileChoice& ch, long V) {
  float r[kTileLoads][8];
#pragma unroll
  for (int sl = 0; sl < kTileLoads; ++sl)
    wave_load_mass<LT, VEC, QL>(R, (long)ch.tile * kTileLoads + sl, V, ch.residual != 0, r[sl]);
  return pick_in_quad_tile(r, ch.tile, ch.pre, ch.target, ch.fallback != 0);
}

template <typename LT, bool VEC, bool QL, bool IN_LDS>
__device__ __forceinline__ int locate_in_masses(const DrawRow<LT>& R, float u, int T, long V,
                                                float (&ts)[kMaxTiles / kWave], float* masses) {
  const TileChoice ch = locate_tile<LT, VEC, QL, IN_LDS>(R, u, T, V, ts, masses);
  return pick_in_choice<LT, VEC, QL>(R, ch, V);
}

// Rows of at most as many CDF tiles as a draw workgroup has waves: wave w
// computes the masses of tile w once and keeps them in registers; wave 0
// chooses the tile from their sums (in LDS), and the wave holding that tile
// walks it without loading it again (unless the residual had no mass and
// the choice fell back to p, whose masses wave 0 loads).  Lanes hold the
// tile sums as locate_in_masses reads them (one tile per lane here), so the
// choice and the token are those of that function.
template <typename LT, bool VEC, bool QL, int THREADS>
__device__ __forceinline__ void draw_from_tiles_in_registers(const DrawRow<LT>& R, float u, int T,
                                                             long V, float* s_tsum,
                                                             TileChoice* s_choice,
                                                             int32_t* out_token) {
  constexpr int kPer = kMaxTiles / kWave;
  const int w = threadIdx.x / kWave, l = lane_id();
  float r[kTileLoads][8];
  if (w < T) {
    float ls = 0.f;
#pragma unroll
    for (int sl = 0; sl < kTileLoads; ++sl) {
      wave_load_mass<LT, VEC, QL>(R, (long)w * kTileLoads + sl, V, R.residual, r[sl]);
      ls += tree_sum8(r[sl]);
    }
    const float ts = wave_sum_f(ls);
    if (l == 0) s_tsum[w] = ts;
  }
  __syncthreads();
  if (w == 0) {
    float ts[kPer];
#pragma unroll
    for (int j = 0; j < kPer; ++j) ts[j] = j == 0 && l < T ? s_tsum[l] : 0.f;
    const TileChoice ch = locate_tile<LT, VEC, QL, true>(R, u, T, V, ts, s_tsum);
    if (l == 0) *s_choice = ch;
    if (ch.residual != (R.residual ? 1 : 0)) {
      const int pick = pick_in_choice<LT, VEC, QL>(R, ch, V);
      if (l == 0) *out_token = pick;
    }
  }
  __syncthreads();
  const TileChoice ch = *s_choice;
  if (ch.residual == (R.residual ? 1 : 0) && w == ch.tile) {
    const int pick = pick_in_quad_tile(r, ch.tile, ch.pre, ch.target, ch.fallback != 0);
    if (l == 0) *out_token = pick;
  }
}

// verify_draw: wave 0 of every workgroup runs sequence b's accept scan
// (chunk 0 writes its outputs); then chunk cidx of b computes the mass of
// each of its tiles.  A tile is kTileLoads consecutive 512-element wave
// loads; each lane sums its octets of the tile before one wave reduction.
// With several chunks per sequence the masses go to the workspace for
// verify_locate.  With one (C = 1: large batches, or rows of one tile) the
// workgroup holds every mass of row a in LDS and wave 0 draws the token
// itself, so no locate kernel runs; the workgroup is then the only reader of
// the sequence's row partials and clears them after its scan.
//
// REG (rows of at most THREADS / 64 CDF tiles, one workgroup per sequence):
// the tiles stay in registers and the token is drawn without loading any of
// them again (draw_from_tiles_in_registers).
template <typename LT, int MODE, bool VEC, bool QL, int THREADS = kThreads, bool REG = false>
__global__ __launch_bounds__(THREADS) void verify_draw(DrawArgs A) {
  constexpr int kDrawWaves = THREADS / kWave;
  __shared__ ScanResult scan;
  __shared__ float s_tsum[kMaxTiles];
  const int C = A.C, T = A.T;
  const int b = blockIdx.x / C, cidx = blockIdx.x % C;
  const bool whole = C == 1;
  const long V = A.sc.V;
  clear_level_state(A.sc, b, cidx == 0 && threadIdx.x == 0);
  if (threadIdx.x < kWave) {
    const ScanResult r = draw_scan<LT, MODE, QL>(A.sc, b, cidx == 0, !whole);
    if (whole) clear_partials(A.sc, b);
    if (threadIdx.x == 0) scan = r;
  }
  __syncthreads();
  const DrawRow<LT> R = draw_row<LT, QL>(A, b, scan);
  if (R.c == 0.f) return;                     // greedy: its token is already written
  if constexpr (REG) {
    __shared__ TileChoice s_choice;
    const int K = A.sc.K;
    draw_from_tiles_in_registers<LT, VEC, QL, THREADS>(
        R, A.sc.uniforms[(long)b * (K + 1) + K], T, V, s_tsum, &s_choice,
        &A.sc.out_tokens[(long)b * (K + 1) + R.a]);
    return;
  }
  const bool residual = R.residual;
  float* tsum_g = A.tile_sums + (long)b * T;
  const int t_lo = (int)((long)cidx * T / C), t_hi = (int)((long)(cidx + 1) * T / C);
  const int w = threadIdx.x / kWave, l = lane_id();
  for (int t0 = t_lo + w * kTileUnroll; t0 < t_hi; t0 += kDrawWaves * kTileUnroll) {
    float ls[kTileUnroll];
#pragma unroll
    for (int j = 0; j < kTileUnroll; ++j)
      ls[j] = lane_tile_mass<LT, VEC, QL>(R, residual, t0 + j, V);
#pragma unroll
    for (int j = 0; j < kTileUnroll; ++j) {
      const float ts = wave_sum_f(ls[j]);
      if (l == 0 && t0 + j < t_hi) {
        if (whole) s_tsum[t0 + j] = ts;
        else tsum_g[t0 + j] = ts;             // read by verify_locate
      }
    }
  }
  if (!whole) return;
  __syncthreads();
  if (w != 0) return;
  constexpr int kPer = kMaxTiles / kWave;
  const int per = (T + kWave - 1) / kWave;
  const int lo = min(T, l * per), hi = min(T, (l + 1) * per);
  float ts[kPer];
#pragma unroll
  for (int j = 0; j < kPer; ++j) ts[j] = lo + j < hi ? s_tsum[lo + j] : 0.f;
  const int K = A.sc.K;
  const int pick = locate_in_masses<LT, VEC, QL, true>(
      R, A.sc.uniforms[(long)b * (K + 1) + K], T, V, ts, s_tsum);
  if (l == 0) A.sc.out_tokens[(long)b * (K + 1) + R.a] = pick;
}

// verify_locate: one wave per sequence draws the token from the tile masses
// the draw kernel's workgroups stored (batches with several workgroups per
// sequence).
template <typename LT, bool VEC, bool QL>
__global__ __launch_bounds__(kThreads) void verify_locate(DrawArgs A) {
  constexpr int kPer = kMaxTiles / kWave;     // tiles per lane at most
  const int b = blockIdx.x * kWaves + threadIdx.x / kWave;
  if (b >= A.sc.B) return;
  const int T = A.T, K = A.sc.K;
  const long V = A.sc.V;
  const int l = lane_id();
  float* tsum_g = A.tile_sums + (long)b * T;
  // this sequence's tile masses, lanes owning contiguous runs of tiles; the
  // loads go out before the scan result is read.  They are agent-coherent
  // loads: the rare path rewrites the masses from this wave and reads them
  // back.
  const int per = (T + kWave - 1) / kWave;
  const int lo = min(T, l * per), hi = min(T, (l + 1) * per);
  float ts[kPer];
#pragma unroll
  for (int j = 0; j < kPer; ++j) ts[j] = lo + j < hi ? ld_coherent(&tsum_g[lo + j]) : 0.f;
  const DrawRow<LT> R = draw_row<LT, QL>(A, b, A.sc.info[b]);   // written by verify_draw
  clear_partials(A.sc, b);                    // every draw workgroup of b has read them
  if (R.c == 0.f) {                           // greedy: nothing to draw
    if (l == 0) A.sc.info[b] = ScanResult{0, 0, 0.f, 0.f, 0.0};
    return;
  }
  const int pick = locate_in_masses<LT, VEC, QL, false>(
      R, A.sc.uniforms[(long)b * (K + 1) + K], T, V, ts, tsum_g);
  if (l == 0) A.sc.out_tokens[(long)b * (K + 1) + R.a] = pick;
  // leave this sequence's part of the workspace cleared
  for (int i = l; i < T; i += kWave) st_coherent(&tsum_g[i], 0.f);
  if (l == 0) A.sc.info[b] = ScanResult{0, 0, 0.f, 0.f, 0.0};
}

// ----------------------------------------------------------------------------
hipError_t launch_row_stats(const void* logits, int bf16, int vec, int sample, float c,
                            const float* temperatures, int B, int K, int V, void* workspace,
                            int trace_id, hipStream_t stream) {
  const Layout lay = layout(B, K, V);
  RowsArgs R;
  R.logits = logits;
  R.temperatures = temperatures;
  R.c = c;
  R.K = K; R.V = V; R.S = lay.S;
  R.octets = (V + 7) / 8;
  R.partials = reinterpret_cast<Partial*>(static_cast<char*>(workspace) + lay.partials);
  const dim3 grid1((unsigned)((long)B * (K + 1) * lay.S)), block(kThreads);
  trace_before(stream, trace_id);
#define SV_ROWS(LT, MODE, VEC) hipLaunchKernelGGL((verify_rows<LT, MODE, VEC>), grid1, block, 0, stream, R)
  if (bf16) {
    if (temperatures) { if (vec) SV_ROWS(uint16_t, MIXED, true); else SV_ROWS(uint16_t, MIXED, false); }
    else if (sample) { if (vec) SV_ROWS(uint16_t, SAMPLE, true); else SV_ROWS(uint16_t, SAMPLE, false); }
    else { if (vec) SV_ROWS(uint16_t, GREEDY, true); else SV_ROWS(uint16_t, GREEDY, false); }
  } else {
    if (temperatures) { if (vec) SV_ROWS(float, MIXED, true); else SV_ROWS(float, MIXED, false); }
    else if (sample) { if (vec) SV_ROWS(float, SAMPLE, true); else SV_ROWS(float, SAMPLE, false); }
    else { if (vec) SV_ROWS(float, GREEDY, true); else SV_ROWS(float, GREEDY, false); }
  }
#undef SV_ROWS
  const hipError_t err = hipGetLastError();
  trace_after(stream, trace_id);
  return err;
}

hipError_t launch_verify(const VerifyLaunch& L, hipStream_t stream) {
  const Layout lay = layout(L.B, L.K, L.V);
  char* ws = static_cast<char*>(L.workspace);
  const int mode = L.mixed ? MIXED : (L.sample ? SAMPLE : GREEDY);
  const float c = mode == SAMPLE ? (float)(1.4426950408889634 / (double)L.temperature) : 1.0f;
  Partial* partials = reinterpret_cast<Partial*>(ws + lay.partials);
  const dim3 block(kThreads);
  const int rows_id = mode == MIXED ? SV_KERNEL_VERIFY_MIXED_ROWS
                    : mode == SAMPLE ? SV_KERNEL_VERIFY_SAMPLE_ROWS : SV_KERNEL_VERIFY_GREEDY_ROWS;

  // early exit: gate kernels and listed ranges for large batches (the
  // greedy form then splits rows finer than the full call), ranges that run
  // the gate's scan in every workgroup below
  const bool listed =
      L.early_exit && L.B >= (mode == GREEDY ? kListedMinBatchGreedy : kListedMinBatchSampled);
  const int S = listed && mode == GREEDY ? lay.Sg : lay.S;
  RowsArgs R;
  R.logits = L.logits;
  R.temperatures = L.temperatures;
  R.c = c;
  R.K = L.K; R.V = L.V; R.S = S;
  R.octets = (L.V + 7) / 8;
  R.partials = partials;

  const bool ql = L.dlogits != nullptr;       // q from the drafter logits (sampling)
  ScanArgs sc;
  sc.logits = L.logits;
  sc.temperatures = L.temperatures;
  sc.dlogits = L.dlogits;
  sc.d_rows = L.d_rows;
  sc.drows = L.drows;
  sc.ddesc = L.ddesc;
  sc.draft_probs = L.draft_probs;
  sc.draft_tokens = L.draft_tokens;
  sc.uniforms = L.uniforms;
  sc.c = c;
  sc.B = L.B; sc.K = L.K; sc.V = L.V; sc.S = S;
  sc.partials = partials;
  sc.out_tokens = L.out_tokens;
  sc.out_num_accepted = L.out_num_accepted;
  sc.out_p_draft = L.out_p_draft;
  sc.device_error = L.device_error;
  sc.info = reinterpret_cast<ScanResult*>(ws + lay.info);
  sc.prefix_only = L.early_exit;
  sc.level_counts = L.early_exit ? reinterpret_cast<int*>(ws + lay.levels) : nullptr;

#define SV_BY_MODE(M, LT) \
  do { \
    if (mode == MIXED) M(LT, MIXED); \
    else if (mode == SAMPLE) M(LT, SAMPLE); \
    else M(LT, GREEDY); \
  } while (0)
  hipError_t err = hipSuccess;
  if (L.early_exit) {
    // draft positions [0,1), [1,2), [2,4), [4,8), ...; before each range but
    // the first a gate lists the sequences still undecided
    int* counts = sc.level_counts;
    int32_t* list = reinterpret_cast<int32_t*>(counts + kLevelSlots);
    const dim3 grid_gate((unsigned)((L.B + kWaves - 1) / kWaves));
#define SV_GATE(LT, MODE) \
  do { \
    if (MODE != GREEDY && ql) hipLaunchKernelGGL((verify_level_gate<LT, MODE, true>), grid_gate, block, 0, stream, sc, k0, cnt, list); \
    else hipLaunchKernelGGL((verify_level_gate<LT, MODE, false>), grid_gate, block, 0, stream, sc, k0, cnt, list); \
  } while (0)
#define SV_LEVEL_FORM(LT, MODE, FORM, QL) \
  do { \
    if (L.vec) hipLaunchKernelGGL((verify_rows_level<LT, MODE, true, FORM, QL>), gridl, block, 0, stream, R, sc, k0, k1, cnt, list); \
    else hipLaunchKernelGGL((verify_rows_level<LT, MODE, false, FORM, QL>), gridl, block, 0, stream, R, sc, k0, k1, cnt, list); \
  } while (0)
#define SV_LEVEL(LT, MODE) \
  do { \
    if (k0 == 0) SV_LEVEL_FORM(LT, MODE, kAllSeqs, false); \
    else if (listed) SV_LEVEL_FORM(LT, MODE, kListed, false); \
    else if (MODE != GREEDY && ql) SV_LEVEL_FORM(LT, MODE, kInline, true); \
    else SV_LEVEL_FORM(LT, MODE, kInline, false); \
  } while (0)
    for (int k0 = 0, level = 0; k0 <= L.K && err == hipSuccess; ++level) {
      const int k1 = k0 == 0 ? 1 : (2 * k0 < L.K + 1 ? 2 * k0 : L.K + 1);
      int* cnt = k0 == 0 ? nullptr : counts + (level - 1);
      if (k0 > 0 && listed) {
        trace_before(stream, rows_id);
        if (L.bf16) SV_BY_MODE(SV_GATE, uint16_t);
        else SV_BY_MODE(SV_GATE, float);
        err = hipGetLastError();
        trace_after(stream, rows_id);
        if (err != hipSuccess) break;
      }
      // one workgroup per item of every sequence (listed ranges: those past
      // the list return at once)
      const dim3 gridl((unsigned)((long)L.B * (k1 - k0) * S));
      trace_before(stream, rows_id);
      if (L.bf16) SV_BY_MODE(SV_LEVEL, uint16_t);
      else SV_BY_MODE(SV_LEVEL, float);
      err = hipGetLastError();
      trace_after(stream, rows_id);
      k0 = k1;
    }
#undef SV_LEVEL
#undef SV_LEVEL_FORM
#undef SV_GATE
  } else {
    const dim3 grid1((unsigned)((long)L.B * (L.K + 1) * lay.S));
    trace_before(stream, rows_id);
#define SV_ROWS(LT, MODE) \
  do { \
    if (L.vec) hipLaunchKernelGGL((verify_rows<LT, MODE, true>), grid1, block, 0, stream, R); \
    else hipLaunchKernelGGL((verify_rows<LT, MODE, false>), grid1, block, 0, stream, R); \
  } while (0)
    if (L.bf16) SV_BY_MODE(SV_ROWS, uint16_t);
    else SV_BY_MODE(SV_ROWS, float);
#undef SV_ROWS
    err = hipGetLastError();
    trace_after(stream, rows_id);
  }
#undef SV_BY_MODE
  if (err != hipSuccess) return err;

  const dim3 grid_acc((unsigned)((L.B + kWaves - 1) / kWaves));
  if (mode == GREEDY) {
    trace_before(stream, SV_KERNEL_VERIFY_GREEDY_ACCEPT);
    if (L.bf16) hipLaunchKernelGGL((verify_accept<uint16_t>), grid_acc, block, 0, stream, sc);
    else hipLaunchKernelGGL((verify_accept<float>), grid_acc, block, 0, stream, sc);
    err = hipGetLastError();
    trace_after(stream, SV_KERNEL_VERIFY_GREEDY_ACCEPT);
    return err;
  }

  // sampling and mixed batches: the draw kernel runs the accept scan itself
  DrawArgs D;
  D.sc = sc;
  D.C = mode == MIXED ? draw_chunks(L.B, L.V, true) : lay.C;
  D.T = lay.T;
  D.tile_sums = reinterpret_cast<float*>(ws + lay.tile);
  // Rows of at most 8 CDF tiles (V <= 16384), or 16 (V <= 32768) when the
  // rows are vectorised (and not fp32 rows with q from the drafter logits,
  // whose 1024-thread form would spill): one workgroup per sequence with a
  // wave per tile draws the token from tiles kept in registers.
  const bool reg16 = L.vec && !(ql && !L.bf16);
  if (lay.T <= 8 || (lay.T <= 16 && reg16)) {
    D.C = 1;
    const int th = lay.T <= 4 ? kThreads : lay.T <= 8 ? 2 * kThreads : 4 * kThreads;
    const dim3 grid3((unsigned)L.B);
#define SV_DRAW_REG(LT, VEC, TH) \
  do { \
    if (mode == MIXED && ql) hipLaunchKernelGGL((verify_draw<LT, MIXED, VEC, true, TH, true>), grid3, dim3(TH), 0, stream, D); \
    else if (mode == MIXED) hipLaunchKernelGGL((verify_draw<LT, MIXED, VEC, false, TH, true>), grid3, dim3(TH), 0, stream, D); \
    else if (ql) hipLaunchKernelGGL((verify_draw<LT, SAMPLE, VEC, true, TH, true>), grid3, dim3(TH), 0, stream, D); \
    else hipLaunchKernelGGL((verify_draw<LT, SAMPLE, VEC, false, TH, true>), grid3, dim3(TH), 0, stream, D); \
  } while (0)
#define SV_DRAW_REG_SMALL(LT, VEC) \
  do { \
    if (th == kThreads) SV_DRAW_REG(LT, VEC, kThreads); \
    else SV_DRAW_REG(LT, VEC, 2 * kThreads); \
  } while (0)
    trace_before(stream, SV_KERNEL_VERIFY_SAMPLE_DRAW);
    if (th == 4 * kThreads) {                // vectorised rows only (reg16)
      constexpr int TH = 4 * kThreads;
      if (L.bf16) SV_DRAW_REG(uint16_t, true, TH);
      else if (mode == MIXED) hipLaunchKernelGGL((verify_draw<float, MIXED, true, false, TH, true>), grid3, dim3(TH), 0, stream, D);
      else hipLaunchKernelGGL((verify_draw<float, SAMPLE, true, false, TH, true>), grid3, dim3(TH), 0, stream, D);
    } else if (L.bf16) {
      if (L.vec) SV_DRAW_REG_SMALL(uint16_t, true); else SV_DRAW_REG_SMALL(uint16_t, false);
    } else {
      if (L.vec) SV_DRAW_REG_SMALL(float, true); else SV_DRAW_REG_SMALL(float, false);
    }
#undef SV_DRAW_REG_SMALL
#undef SV_DRAW_REG
    err = hipGetLastError();
    trace_after(stream, SV_KERNEL_VERIFY_SAMPLE_DRAW);
    return err;
  }
  // From B = 256 (every CU gets a sequence) one workgroup per sequence draws
  // the token itself: measured at V = 151936 bf16 (wall time of the sampled
  // verify) 146 against 154 us at B = 256 and 277 against 285 us at B = 512;
  // at B = 128 the two are equal, and below that the chunked draw with its
  // locate kernel is faster (B = 64: 54 against 59 us).  The workgroup is as
  // wide as lets every draw workgroup be resident at once (the draw holds 5
  // waves per SIMD, 20 per CU): 16 waves up to B = 256, 8 up to B = 512, 4
  // above.  Draw kernel at V = 151936 bf16, 1024 / 512 / 256 threads:
  // 46.8 / 48.3 / 61.2 us at B = 256, 70.3 / 67.6 / 71.3 at B = 384,
  // 83.9 / 81.4 / 82.4 at B = 512, 106.4 / 119.6 / 101.3 at B = 640,
  // 118.8 / 125.5 / 115.4 at B = 768.
  const bool one = mode != MIXED && D.C > 1 && L.B >= 256;
  const int dthreads = !one ? kThreads : L.B <= 256 ? 4 * kThreads : L.B <= 512 ? 2 * kThreads : kThreads;
  if (one) D.C = 1;
  const dim3 grid3((unsigned)((long)L.B * D.C));
#define SV_DRAW_KERNELS(LAUNCH) \
  do { \
    if (L.bf16) { \
      if (L.vec) { if (ql) LAUNCH(uint16_t, true, true); else LAUNCH(uint16_t, true, false); } \
      else { if (ql) LAUNCH(uint16_t, false, true); else LAUNCH(uint16_t, false, false); } \
    } else { \
      if (L.vec) { if (ql) LAUNCH(float, true, true); else LAUNCH(float, true, false); } \
      else { if (ql) LAUNCH(float, false, true); else LAUNCH(float, false, false); } \
    } \
  } while (0)
#define SV_DRAW(LT, VEC, QL) \
  do { \
    if (mode == MIXED) hipLaunchKernelGGL((verify_draw<LT, MIXED, VEC, QL>), grid3, block, 0, stream, D); \
    else if (dthreads == 4 * kThreads) hipLaunchKernelGGL((verify_draw<LT, SAMPLE, VEC, QL, 4 * kThreads>), grid3, dim3(4 * kThreads), 0, stream, D); \
    else if (dthreads == 2 * kThreads) hipLaunchKernelGGL((verify_draw<LT, SAMPLE, VEC, QL, 2 * kThreads>), grid3, dim3(2 * kThreads), 0, stream, D); \
    else hipLaunchKernelGGL((verify_draw<LT, SAMPLE, VEC, QL>), grid3, block, 0, stream, D); \
  } while (0)
#define SV_LOCATE(LT, VEC, QL) hipLaunchKernelGGL((verify_locate<LT, VEC, QL>), grid_acc, block, 0, stream, D)
  trace_before(stream, SV_KERNEL_VERIFY_SAMPLE_DRAW);
  SV_DRAW_KERNELS(SV_DRAW);
  err = hipGetLastError();
  trace_after(stream, SV_KERNEL_VERIFY_SAMPLE_DRAW);
  if (err != hipSuccess || D.C == 1) return err;     // C = 1: the draw drew the tokens
  trace_before(stream, SV_KERNEL_VERIFY_SAMPLE_LOCATE);
  SV_DRAW_KERNELS(SV_LOCATE);
#undef SV_LOCATE
#undef SV_DRAW
#undef SV_DRAW_KERNELS
  err = hipGetLastError();
  trace_after(stream, SV_KERNEL_VERIFY_SAMPLE_LOCATE);
  return err;
}

}  // namespace sv
