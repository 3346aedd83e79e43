// Draft-tree verification for gfx950.  "Project 14 - speculative decoding
// inference server", section 概念: P-EAGLE's parallel speculation forms deeper
// draft trees; the target verifies every node in one forward, giving one
// logit row per node (row 0 = the root, the last committed token).
//
// Row statistics of all B * (N+1) rows come from the verify row kernel (one
// pass over every logit), or, in the early-exit form, are computed by the
// walk for the nodes it visits.  One workgroup per sequence walks the tree
// (in a mixed batch each tree by its own temperature):
//   greedy   move to the lowest-index child whose token is the row's argmax;
//            emit the argmax when none matches;
//   sampled  test the children of the current node in index order against
//            the residual r_m = max(0, p - w_m q) / S_m (w_0 = 0, S_0 = 1;
//            after a rejection w_{m+1} = w_m + S_m and S_{m+1} is the mass of
//            the new residual, one workgroup pass over the node's row) --
//            the normalise-and-subtract recursion of rejection sampling over
//            independently drafted candidates, written so that one pass per
//            rejection suffices; an accepted child becomes the current node;
//            when every child is rejected, or the node is a leaf, the new
//            token is drawn from the residual by inverse CDF (tile masses in
//            LDS, then the in-tile search the chain draw uses, over the same
//            quad layout of elements across lanes).
//            q comes from the dense draft rows, or (QL) is recomputed from
//            the drafter's logit row of the node and its descriptor with the
//            drafter kernel's own fp32 operations (drafter_q), which reads
//            V * 2 bytes per pass instead of V * 4 for bf16 logits.
// All threads of a workgroup take the same decisions from the same values,
// so the workgroup-wide passes sit in uniform control flow.
#include <type_traits>

#include "sv_device.h"
#include "sv_internal.h"
#include "sv_rowstats.h"

namespace sv {

// Workgroup size: the sampled walk spends its time in workgroup passes over
// a row (at 256 trees x 16 rows x 151936: 119 us with 512 threads, 181 with
// 256; 1024 would be 106 but spills registers); the greedy walk only reads
// partials.
// A greedy walk that computes its rows' statistics itself (LAZY) is a chain
// of whole-row passes by one workgroup, so it takes the widest workgroup.
template <int MODE, bool LAZY = false>
constexpr int tree_threads() { return MODE != GREEDY ? 512 : (LAZY ? 1024 : 256); }
constexpr int kTreeSplits = 16;        // workgroups per row at most (the row kernel's limit)

struct TreeArgs {
  TreeLaunch L;
  Partial* partials;       // [B][N+1][S]
  int S;
  float c;                 // log2(e) / T (sampled)
};

// Where the q of the current node comes from: its dense row, or (QL) its
// drafter logit row and descriptor.  An invalid drafter row index (valid =
// false) reads the node's target row instead with the descriptor {c = 0,
// argmax = -1}, whose q is 0 everywhere, so the loads never depend on it.
template <typename LT>
struct TreeQ {
  const float* qrow;
  const LT* dzrow;
  sv_draft_row desc;
  bool valid;
};

template <typename LT, bool QL>
__device__ __forceinline__ float tree_q_at(const TreeQ<LT>& Q, long x) {
  if constexpr (QL) return drafter_q(Q.desc, logit_at(Q.dzrow, x), x);
  else return Q.qrow[x];
}

// The packed quads of G wave loads of a tile as this lane loads them (VEC):
// the target logits, and with RESID the q quads (fp32) or the drafter logit
// quads (QL).
template <typename LT, bool QL, int G>
struct TileQuads {
  Quad<LT> z[G][2];
  Quad<typename std::conditional<QL, LT, float>::type> q[G][2];
};

// Residual masses of this lane's elements of CDF tile t in the quad layout
// (r[sl][4 h + j]: element 512 g + 256 h + 4 l + j of wave load g = t *
// kTileLoads + sl): max(0, p - w q) with p = 2^(z c - Mc) * inv_s
// (RESID = false: p).  A pass is bound by load latency (one workgroup per
// tree), so a tile's loads are issued together and held (`hold`) before any
// is used, and RESID is a template argument so that no load sits behind a
// run-time branch: with the q loads behind one, and without the hold, the
// compiler waited for each load before issuing the next (at 256 trees x 16
// rows x 151936 bf16 the walk took 102 us with dense q, and 170 us with q
// from drafter logits, against 95 and 96 us gathered).  Cached loads: a
// node's rows are read again for every rejection at that node.  VEC: V is a multiple of 8 and the rows 16-byte aligned, so a
// quad lies wholly inside or wholly past the row; a quad past it loads from
// the row's start and is masked.
template <typename LT, bool VEC, bool QL, bool RESID>
__device__ __forceinline__ void tile_residual(const LT* zrow, const TreeQ<LT>& Q, int t, long V,
                                              float c, float Mc, float inv_s, float w,
                                              float (&r)[kTileLoads][8]) {
  const int l = lane_id();
  if constexpr (VEC) {
    // wave loads gathered G at a time (all of the tile, or half of it for
    // fp32 rows with q from drafter logits, whose two fp32 quads per
    // element group would not fit the registers)
    constexpr int G = QL && sizeof(LT) == 4 ? kTileLoads / 2 : kTileLoads;
#pragma unroll
    for (int s0 = 0; s0 < kTileLoads; s0 += G) {
      TileQuads<LT, QL, G> tq;
#pragma unroll
      for (int g = 0; g < G; ++g)
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          const long e = ((long)t * kTileLoads + s0 + g) * kTile + h * (kTile / 2) + 4 * l;
          const long ec = e < V ? e : 0;
          load_quad<false>(zrow, ec, tq.z[g][h]);
          if constexpr (RESID) {
            if constexpr (QL) load_quad<false>(Q.dzrow, ec, tq.q[g][h]);
            else load_quad<false>(Q.qrow, ec, tq.q[g][h]);
          }
        }
#pragma unroll
      for (int g = 0; g < G; ++g)
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          hold(tq.z[g][h]);
          if constexpr (RESID) hold(tq.q[g][h]);
        }
#pragma unroll
      for (int g = 0; g < G; ++g)
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          const int sl = s0 + g;
          const long e = ((long)t * kTileLoads + sl) * kTile + h * (kTile / 2) + 4 * l;
          const bool in = e < V;
          float z[4], q[4];
          unpack(tq.z[g][h], z);
#pragma unroll
          for (int j = 0; j < 4; ++j) q[j] = 0.f;
          if constexpr (RESID) {
            if constexpr (QL) {
              // drafter_q, with its choice (c > 0: exponential; else
              // one-hot) taken once per quad: it is the same for the row
              float dz[4];
              unpack(tq.q[g][h], dz);
              if (Q.desc.c > 0.f) {
#pragma unroll
                for (int j = 0; j < 4; ++j)
                  q[j] = __builtin_amdgcn_exp2f(fmaf(dz[j], Q.desc.c, -Q.desc.mc)) * Q.desc.inv_s;
              } else {
#pragma unroll
                for (int j = 0; j < 4; ++j) q[j] = (int)e + j == Q.desc.argmax ? 1.f : 0.f;
              }
            } else {
              unpack(tq.q[g][h], q);
            }
          }
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            if (!in) { z[j] = -INFINITY; q[j] = 0.f; }
            const float p = __builtin_amdgcn_exp2f(fmaf(z[j], c, -Mc)) * inv_s;
            r[sl][4 * h + j] = RESID ? fmaxf(0.f, fmaf(-w, q[j], p)) : p;
          }
        }
    }
  } else {
#pragma unroll
    for (int sl = 0; sl < kTileLoads; ++sl)
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const long e = ((long)t * kTileLoads + sl) * kTile + h * (kTile / 2) + 4 * l;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const long ej = e + j;
          const float z = ej < V ? logit_at(zrow, ej) : -INFINITY;
          const float q = RESID && ej < V ? tree_q_at<LT, QL>(Q, ej) : 0.f;
          const float p = __builtin_amdgcn_exp2f(fmaf(z, c, -Mc)) * inv_s;
          r[sl][4 * h + j] = RESID ? fmaxf(0.f, fmaf(-w, q, p)) : p;
        }
      }
  }
}

// Tile masses of the residual into tsum (LDS); returns the fp64 total, the
// same on every thread.  Called in uniform control flow.  (Two tiles in
// flight per wave, the next tile's loads issued before the current one is
// reduced, measured slower at 256 trees x 16 rows x 151936 bf16: 101-102
// against 95.5-98 us with one buffer copied into the other, 102-103 against
// 94.5-95 us with two buffers swapping roles, whose loads the compiler did
// keep in flight during the reduction.)
template <typename LT, bool VEC, bool QL, bool RESID, int WAVES>
__device__ __forceinline__ double residual_tiles(const LT* zrow, const TreeQ<LT>& Q, float w,
                                                 long V, int T_tiles, float c, float Mc,
                                                 float inv_s, float* tsum, double* red) {
  const int wv = threadIdx.x / kWave, l = lane_id();
  double part = 0.0;
  for (int t = wv; t < T_tiles; t += WAVES) {
    float r[kTileLoads][8];
    tile_residual<LT, VEC, QL, RESID>(zrow, Q, t, V, c, Mc, inv_s, w, r);
    float ls = 0.f;
#pragma unroll
    for (int sl = 0; sl < kTileLoads; ++sl) ls += tree_sum8(r[sl]);
    const float ts = wave_sum_f(ls);
    if (l == 0) tsum[t] = ts;
    part += (double)ts;
  }
  if (l == 0) red[wv] = part;
  __syncthreads();
  double tot = 0.0;
  for (int i = 0; i < WAVES; ++i) tot += red[i];
  __syncthreads();
  return tot;
}

// LAZY: the statistics of a node's row are computed by the walk itself when
// it reaches the node (one workgroup pass, `slice_stats` over the whole row),
// so only the rows of the visited nodes are read; otherwise they come from
// the row kernel's partials of every row.  MIXED: each tree by its own
// temperature, greedily when it is 0 (or invalid: flagged), as the chain
// verify treats a mixed batch.
template <typename LT, int MODE, bool VEC, bool QL = false, bool LAZY = false>
__global__ __launch_bounds__((tree_threads<MODE, LAZY>())) void tree_walk(TreeArgs A) {
  constexpr int THREADS = tree_threads<MODE, LAZY>();
  constexpr int WAVES = THREADS / kWave;
  __shared__ int s_par[SV_MAX_K + 1];
  __shared__ int s_tok[SV_MAX_K + 1];
  __shared__ float tsum[kMaxTiles];
  __shared__ double red[WAVES];
  __shared__ float sm_f[LAZY ? WAVES : 1];
  __shared__ int sm_i[LAZY ? WAVES : 1];
  __shared__ double sm_d[LAZY ? WAVES : 1];
  __shared__ Partial s_stat;

  const TreeLaunch& L = A.L;
  const int b = blockIdx.x, N = L.N, t = threadIdx.x, S = A.S;
  const long V = L.V;
  const int T_tiles = (int)((V + kTileElems - 1) / kTileElems);
  if (t < N) {
    // node i = t + 1: its parent must precede it and its token lie in [0, V)
    const int par = L.parents[(long)b * N + t];
    const int tok = L.tokens[(long)b * N + t];
    const bool ok = par >= 0 && par <= t && tok >= 0 && tok < V;
    if (!ok) flag_error(L.device_error, SV_DEVERR_TREE);
    s_par[t + 1] = ok ? par : -1;          // an invalid node is nobody's child
    s_tok[t + 1] = tok;
  }
  __syncthreads();

  const LT* zb = static_cast<const LT*>(L.logits) + (long)b * (N + 1) * V;
  Partial* Pb = A.partials + (long)b * (N + 1) * S;
  int32_t* out = L.out_tokens + (long)b * (N + 1);
  int32_t* path = L.out_path + (long)b * (N + 1);
  float c = A.c;
  bool greedy = MODE == GREEDY;
  if constexpr (MODE == MIXED) {
    bool bad;
    c = seq_scale(L.temperatures[b], bad);
    if (bad && t == 0) flag_error(L.device_error, SV_DEVERR_TEMPERATURE);
    greedy = c == 0.f;
  }
  int cur = 0, depth = 0;
  for (;;) {
    float M = -INFINITY;
    int g = INT32_MAX;
    double s = 0.0;
    if constexpr (LAZY) {
      // statistics of row cur by one pass of the workgroup, then shared
      const LT* row = zb + (long)cur * V;
      const long oct = (V + 7) / 8;
      Partial P;
      if constexpr (MODE == MIXED) {
        if (greedy) P = slice_stats<LT, GREEDY, VEC, THREADS>(row, 0, oct, V, 1.f, sm_f, sm_i, sm_d);
        else P = slice_stats<LT, SAMPLE, VEC, THREADS>(row, 0, oct, V, c, sm_f, sm_i, sm_d);
      } else {
        P = slice_stats<LT, MODE, VEC, THREADS>(row, 0, oct, V, c, sm_f, sm_i, sm_d);
      }
      if (t == 0) s_stat = P;
      __syncthreads();
      M = s_stat.m;
      g = s_stat.g;
      s = s_stat.acc;
      __syncthreads();                     // s_stat is written again at the next node
    } else {
      // statistics of row cur from its S partials (same order on every
      // thread), all of them loaded at once (at most kTreeSplits)
      Partial pk[kTreeSplits];
#pragma unroll
      for (int j = 0; j < kTreeSplits; ++j)
        if (j < S) pk[j] = Pb[cur * S + j];
      if (greedy) {
#pragma unroll
        for (int j = 0; j < kTreeSplits; ++j)
          if (j < S && (j == 0 || pk[j].m > M)) { M = pk[j].m; g = pk[j].g; }
      } else {
#pragma unroll
        for (int j = 0; j < kTreeSplits; ++j)
          if (j < S) M = fmaxf(M, pk[j].m);
#pragma unroll
        for (int j = 0; j < kTreeSplits; ++j)
          if (j < S && pk[j].acc != 0.0)
            s += pk[j].acc * exp2_split(((double)pk[j].m - (double)M) * (double)c);
      }
    }
    const LT* zrow = zb + (long)cur * V;
    int nxt = -1;
    if (greedy) {
      if (g < 0 || g >= V) g = 0;          // a NaN row: any in-range token
      for (int i = 1; i <= N; ++i)
        if (s_par[i] == cur && s_tok[i] == g) { nxt = i; break; }
      if (nxt < 0) {
        if (t == 0) out[depth] = g;
        break;
      }
    } else {
      TreeQ<LT> Q{nullptr, zrow, sv_draft_row{0.f, 0.f, 0.f, -1}, true};
      if constexpr (QL) {
        const long j = (long)b * (N + 1) + cur;
        const long row = L.drows ? (long)L.drows[j] : j;
        Q.valid = row >= 0 && row < L.d_rows;
        if (Q.valid) {
          Q.dzrow = static_cast<const LT*>(L.dlogits) + row * V;
          Q.desc = L.ddesc[j];
        }
      } else {
        Q.qrow = L.draft_probs + ((long)b * (N + 1) + cur) * V;
      }
      bool flagged = false;                // one flag per invalid drafter row
      // p = 2^(z c - Mc) * inv_s; Mc is M*c rounded to fp32, folded into inv_s
      const float Mc = M * c;
      const float inv_s = (float)(exp2((double)Mc - (double)M * (double)c) / s);
      double w = 0.0, Sr = 1.0;            // residual r = max(0, p - w q) / Sr
      bool tiles = false;                  // tsum holds the current residual's tiles
      // one call site for the workgroup pass: after each rejection (the new
      // residual's mass), and before the final draw when tsum is not current
      for (int i = 1;; ++i) {
        while (i <= N && s_par[i] != cur) ++i;
        bool final_pass = false;
        if (i <= N) {
          const int x = s_tok[i];
          const double px = exp2(((double)logit_at(zrow, x) - (double)M) * (double)c) / s;
          if (QL && !Q.valid && !flagged) {
            if (t == 0) flag_error(L.device_error, SV_DEVERR_ROW_INDEX);
            flagged = true;
          }
          const double qx = (double)tree_q_at<LT, QL>(Q, x);
          const double R = fmax(0.0, px - w * qx);
          const double ratio = qx > 0.0 ? R / (Sr * qx) : (R > 0.0 ? INFINITY : 0.0);
          if ((double)L.uniforms[(long)b * (N + 1) + i] < ratio) { nxt = i; break; }
          w += Sr;
        } else {
          if (tiles) break;                // tsum already holds the residual
          final_pass = true;               // w = 0 here: the tiles of p
        }
        const double tot =
            w > 0.0 ? residual_tiles<LT, VEC, QL, true, WAVES>(zrow, Q, (float)w, V, T_tiles, c,
                                                               Mc, inv_s, tsum, red)
                    : residual_tiles<LT, VEC, QL, false, WAVES>(zrow, Q, (float)w, V, T_tiles, c,
                                                                Mc, inv_s, tsum, red);
        if (final_pass) break;
        Sr = tot;
        tiles = true;
        if (!(Sr > 0.0)) { w = 0.0; Sr = 1.0; tiles = false; }   // empty residual: back to p
      }
      if (nxt < 0) {
        // final draw from the residual (p when w = 0) with u[0]
        const bool residual = w > 0.0;
        if (t < kWave) {
          const int l = t;
          const int per = (T_tiles + kWave - 1) / kWave;
          const int lo = min(T_tiles, l * per), hi = min(T_tiles, (l + 1) * per);
          double part = 0.0;
          for (int k = lo; k < hi; ++k) part += (double)tsum[k];
          const double incl = wave_inclusive_scan(part);
          const double target = (double)L.uniforms[(long)b * (N + 1)] * __shfl(incl, kWave - 1);
          double run = __shfl_up(incl, 1);
          if (l == 0) run = 0.0;
          int hit = -1, last = -1;
          double pre = 0.0;
          for (int k = lo; k < hi; ++k) {
            const float ts = tsum[k];
            if (ts > 0.f) last = k;
            const double nx = run + (double)ts;
            if (hit < 0 && nx > target) { hit = k; pre = run; }
            run = nx;
          }
          int tile;
          bool fallback = false;
          const unsigned long long any = __ballot(hit >= 0);
          if (any) {
            const int src = __ffsll((long long)any) - 1;
            tile = __shfl(hit, src);
            pre = __shfl(pre, src);
          } else {
            const unsigned long long anyp = __ballot(last >= 0);
            tile = anyp ? __shfl(last, 63 - __clzll((long long)anyp)) : 0;
            fallback = true;
          }
          float r[kTileLoads][8];
          if (residual)
            tile_residual<LT, VEC, QL, true>(zrow, Q, tile, V, c, Mc, inv_s, (float)w, r);
          else
            tile_residual<LT, VEC, QL, false>(zrow, Q, tile, V, c, Mc, inv_s, (float)w, r);
          const int pick = pick_in_quad_tile(r, tile, pre, target, fallback);
          if (l == 0) out[depth] = pick;
        }
        break;
      }
    }
    if (t == 0) {
      out[depth] = s_tok[nxt];
      path[depth] = nxt;
    }
    ++depth;
    cur = nxt;
  }
  for (int j = depth + 1 + t; j <= N; j += THREADS) out[j] = -1;
  for (int j = depth + t; j <= N; j += THREADS) path[j] = -1;
  if (t == 0) L.out_num_accepted[b] = depth;
  // the partials are consumed: clear them so the workspace ends all zero
  if constexpr (!LAZY)
    for (int i = t; i < (N + 1) * S; i += THREADS) Pb[i] = Partial{0.f, 0, 0.0};
}

hipError_t launch_tree(const TreeLaunch& L, hipStream_t stream) {
  const bool sample = L.temperature > 0.f;
  const float c = sample ? (float)(1.4426950408889634 / (double)L.temperature) : 1.0f;
  const bool mixed = L.temperatures != nullptr;
  hipError_t err = hipSuccess;
  if (!L.lazy)
    err = launch_row_stats(L.logits, L.bf16, L.vec, sample, c, L.temperatures, L.B, L.N, L.V,
                           L.workspace, SV_KERNEL_TREE_ROWS, stream);
  if (err != hipSuccess) return err;
  const RowPartials rp = row_partials(L.workspace, L.B, L.N, L.V);
  TreeArgs A{L, static_cast<Partial*>(rp.partials), rp.S, c};
  const dim3 grid((unsigned)L.B);
  const dim3 block(sample || mixed ? tree_threads<SAMPLE>()
                                   : (L.lazy ? tree_threads<GREEDY, true>() : tree_threads<GREEDY>()));
  const bool ql = sample && L.dlogits != nullptr;
  trace_before(stream, SV_KERNEL_TREE_WALK);
#define SV_TREE(LT, MODE, QL) \
  do { \
    if (L.lazy) { \
      if (L.vec) hipLaunchKernelGGL((tree_walk<LT, MODE, true, QL, true>), grid, block, 0, stream, A); \
      else hipLaunchKernelGGL((tree_walk<LT, MODE, false, QL, true>), grid, block, 0, stream, A); \
    } else { \
      if (L.vec) hipLaunchKernelGGL((tree_walk<LT, MODE, true, QL>), grid, block, 0, stream, A); \
      else hipLaunchKernelGGL((tree_walk<LT, MODE, false, QL>), grid, block, 0, stream, A); \
    } \
  } while (0)
  if (L.bf16) {
    if (mixed) SV_TREE(uint16_t, MIXED, false);
    else if (ql) SV_TREE(uint16_t, SAMPLE, true);
    else if (sample) SV_TREE(uint16_t, SAMPLE, false);
    else SV_TREE(uint16_t, GREEDY, false);
  } else {
    if (mixed) SV_TREE(float, MIXED, false);
    else if (ql) SV_TREE(float, SAMPLE, true);
    else if (sample) SV_TREE(float, SAMPLE, false);
    else SV_TREE(float, GREEDY, false);
  }
#undef SV_TREE
  err = hipGetLastError();
  trace_after(stream, SV_KERNEL_TREE_WALK);
  return err;
}

}  // namespace sv
