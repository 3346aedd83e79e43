/*
 * spec_verify.h - C ABI of the speculative-decoding hot path on one MI355X.
 *
 * Two steps of a decode round with draft tokens:
 *   1. verify-and-accept: per sequence, softmax over the target's K+1 logit
 *      rows, the greedy argmax-match or p/q rejection test on the K drafts,
 *      the first-rejection prefix length, then the residual max(0, p - q)
 *      resample or the bonus token.  Source: "Project 14 - speculative
 *      decoding inference server" (ai-engineering.com.cn), section 架构
 *      (architecture): the target checks the k drafts in one forward, keeps
 *      the accepted prefix and resamples the rejected suffix; section 概念
 *      (concepts): an accepted prefix replaces the greedy path.
 *   2. the P-EAGLE parallel-draft batch: MASK rows for the multi-token
 *      prediction positions 2..K, remapped positions, h_shared broadcast into
 *      the MASK rows, PADDING_SLOT_ID = -1 for the KV slots of rejected
 *      tokens.  Source: the P-EAGLE / TorchSpec blog summary
 *      (blog.hotdry.top), sections 并行架构的核心创新 (parallel architecture)
 *      and TorchSpec 集成与工程优化 (engineering).
 *
 * Conventions shared by every call
 *   - Every tensor argument is a DEVICE pointer on the current HIP device,
 *     owned by the caller; the verify, build, drafter and metrics calls
 *     allocate no device memory, keep no state between calls and never
 *     synchronise.  (The step graph and the kernel tracer at the end of this
 *     file create HIP graph, stream and event objects, which they hold until
 *     destroyed.)  All work is enqueued on `stream` (a hipStream_t; NULL =
 *     the default stream) in issue order.
 *   - Arrays are dense and row-major with the shapes given below.
 *   - Arguments are validated on the host before anything is enqueued: on an
 *     error the call returns a nonzero sv_status and touches no memory.
 *     SV_ERR_HIP means a launch was rejected by the runtime; faults inside a
 *     kernel surface at the caller's next synchronisation.
 *   - `device_error` (optional, may be NULL) is one int32 in device memory;
 *     kernels OR SV_DEVERR_* bits into it when they meet data that breaks a
 *     precondition.  Such data is handled safely as documented per bit.
 *   - Results are deterministic: the same inputs give bitwise-identical
 *     outputs on every run (no floating-point atomics).
 *   - Calls on one stream run in order; calls that share a workspace must not
 *     run concurrently on different streams.
 */
#ifndef SPEC_VERIFY_H
#define SPEC_VERIFY_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define SV_API __attribute__((visibility("default")))

typedef enum {
  SV_OK = 0,
  SV_ERR_NULL = 1,      /* a required pointer is NULL                          */
  SV_ERR_SHAPE = 2,     /* B, K, V, H, block sizes or table width out of range */
  SV_ERR_DTYPE = 3,     /* dtype code not supported by this call               */
  SV_ERR_VALUE = 4,     /* scalar out of range (temperature <= 0 or not finite)*/
  SV_ERR_WORKSPACE = 5, /* workspace NULL or smaller than required             */
  SV_ERR_ALIGN = 6,     /* pointer not aligned to its element size             */
  SV_ERR_HIP = 7,       /* the HIP runtime rejected a launch                   */
  SV_ERR_SCRATCH = 8    /* the call needs more scratch than the no-allocation
                           entry point holds (SV_NOALLOC_SCRATCH_BYTES)         */
} sv_status;

typedef enum {
  SV_F32 = 0,   /* IEEE binary32                                            */
  SV_BF16 = 1,  /* bfloat16 (upper half of a binary32)                      */
  SV_F16 = 2    /* IEEE binary16: accepted where data is only copied (hidden) */
} sv_dtype;

/* Bits OR-ed into *device_error. */
#define SV_DEVERR_DRAFT_TOKEN 1   /* a draft token outside [0, V): that draft is rejected
                                     (greedy: mismatch; sampling: ratio 0) and its
                                     out_draft_target_prob entry is 0                  */
#define SV_DEVERR_ACCEPT_COUNT 2  /* num_accepted outside [0, K]: clamped into range    */
#define SV_DEVERR_BLOCK_TABLE 4   /* a position past the block table, or a negative
                                     block id: that row gets slot -1                   */
#define SV_DEVERR_ROW_INDEX 8     /* spec_draft_sample: a row index outside
                                     [0, n_rows): that draft gets token -1 and an
                                     all-zero q row                                    */
#define SV_DEVERR_TREE 32         /* spec_verify_tree: a node whose parent does not
                                     precede it or whose token is outside [0, V): the
                                     node is treated as absent                         */
#define SV_DEVERR_TEMPERATURE 16  /* a per-sequence temperature that is negative, NaN,
                                     infinite or too small for log2(e)/T to be a
                                     finite fp32 (T < ~4.24e-39): that sequence is
                                     treated as greedy (T = 0)                         */

/* Limits (a call outside them returns SV_ERR_SHAPE). */
#define SV_MAX_B (1 << 20)        /* sequences per call                               */
#define SV_MAX_K 63               /* drafts per sequence (K+1 rows fit one wavefront) */
#define SV_MAX_V (1 << 19)        /* vocabulary size                                  */
#define SV_PADDING_SLOT_ID (-1)   /* slot of rows that must not write the KV cache    */

/*
 * How one drafted row's distribution q is recomputed from the drafter's
 * logits z (see spec_draft_sample and spec_verify_sample_lq):
 *   c > 0:  q(x) = exp2(fma(z(x), c, -mc)) * inv_s, evaluated in fp32 (c =
 *           log2(e) / T, mc = max(z) * c, inv_s = 1 / sum of the exponentials);
 *   c = 0:  q(x) = 1 if x == argmax else 0 (greedy drafting; argmax = -1: q = 0).
 * These are the same fp32 operations spec_draft_sample uses to write q, so a
 * recomputed q(x) equals the stored one bit for bit.
 */
typedef struct sv_draft_row {
  float c;
  float mc;
  float inv_s;
  int32_t argmax;
} sv_draft_row;

/* Human-readable name of a status code (static storage; never NULL). */
SV_API const char* sv_status_string(int status);

/* Bytes of device workspace spec_verify_greedy / spec_verify_sample need for
 * this (B, K, V).  The workspace must be zero-filled once after allocation;
 * every call leaves it zero-filled again, so it can be reused (and captured
 * in a graph) without clearing.  Returns 0 for invalid shapes. */
SV_API size_t spec_verify_workspace_bytes(int B, int K, int V);

/*
 * Greedy verify.  Source: "Project 14", section 概念 (concepts): the target
 * checks the drafts in one forward and the accepted prefix replaces its own
 * greedy continuation, so the emitted tokens are the target's greedy path.
 * For sequence b, g_k = the lowest index of the maximum of logit row k.  a_b = the first k < K with draft_tokens[b][k] != g_k, or K.
 * Emitted tokens: the a_b accepted drafts, then c_b = g_{a_b}.
 *
 *   target_logits    [B][K+1][V], dtype SV_F32 or SV_BF16; row k is the
 *                    target's distribution for the token after verify slot k
 *                    (slot 0 = last committed token, slot i = draft i-1).
 *   draft_tokens     [B][K] int32.
 *   out_tokens       [B][K+1] int32: d[0..a-1], c, then -1 up to K.
 *   out_num_accepted [B] int32, in [0, K].
 *   workspace        spec_verify_workspace_bytes(B, K, V) bytes (see above).
 * Ties: the lowest index wins.  NaN logits, or a row of only -inf, give an
 * unspecified but in-range token.  B = 0 is a no-op.  1 <= V <= SV_MAX_V,
 * 0 <= K <= SV_MAX_K.  Two kernels are enqueued: row statistics, then the
 * accept scan.
 */
SV_API sv_status spec_verify_greedy(const void* target_logits, int logits_dtype,
                                    const int32_t* draft_tokens,
                                    int B, int K, int V,
                                    int32_t* out_tokens, int32_t* out_num_accepted,
                                    void* workspace, size_t workspace_bytes,
                                    int32_t* device_error, void* stream);

/*
 * Sampled verify (rejection sampling against the drafter's distribution).
 * Source: "Project 14", section 架构 (architecture): accept the verified
 * prefix, resample the rejected suffix; the rskf.cn survey, sections 1 and
 * 2.2: the output follows the target's distribution exactly.
 * p_k = softmax(row k / T); q_k = draft_probs[b][k] used as given.
 * Draft k is accepted iff u[b][k] < p_k(x)/q_k(x), x = draft_tokens[b][k]
 * (q_k(x) = 0: accepted iff p_k(x) > 0).  a_b = the first rejected k, or K.
 * If a_b < K the new token is drawn from r = max(0, p_a - q_a) (from p_a if
 * r sums to 0); if a_b = K it is the bonus token drawn from p_K.  The draw is
 * the smallest v whose running total of r in vocabulary order exceeds
 * u[b][K] * sum(r) (inverse CDF with the last uniform).
 *
 *   target_logits    [B][K+1][V], SV_F32 or SV_BF16.
 *   draft_probs      [B][K][V] fp32, the drafter's probabilities of each draft.
 *   draft_tokens     [B][K] int32, d[b][k] drawn from draft_probs[b][k].
 *   uniforms         [B][K+1] fp32 in [0, 1): [:, k<K] tests, [:, K] the draw.
 *   temperature      > 0 and finite, with log2(e)/T finite in fp32 (T >= ~4.24e-39;
 *                    smaller values return SV_ERR_VALUE); applies to the target
 *                    logits only.
 *   out_tokens, out_num_accepted: as for spec_verify_greedy.
 *   out_draft_target_prob  optional [B][K] fp32: p_k(d[b][k]) for every k
 *                    (NULL = not written).
 * Arithmetic: fp32 exponentials, fp64 accumulation of every sum and of the
 * acceptance ratio; results agree with an fp64 evaluation except when a
 * decision lies within ~1e-6 of its threshold.  A logit whose |z|*log2(e)/T
 * exceeds the fp32 range (possible only for T within a few powers of ten of
 * the lower limit above) gives an unspecified but in-range token, like a NaN
 * logit.  Three kernels are enqueued:
 * row statistics; the accept scan with the residual / bonus masses of row a;
 * the draw of the new token from them.  When one workgroup covers each
 * sequence's row a (B >= 256, or rows of at most 8 CDF tiles of 2048
 * elements, 16 for 16-byte-aligned rows with V a multiple of 8) the second
 * kernel also draws the token and two kernels are enqueued.
 */
SV_API sv_status spec_verify_sample(const void* target_logits, int logits_dtype,
                                    const float* draft_probs,
                                    const int32_t* draft_tokens,
                                    const float* uniforms, float temperature,
                                    int B, int K, int V,
                                    int32_t* out_tokens, int32_t* out_num_accepted,
                                    float* out_draft_target_prob,
                                    void* workspace, size_t workspace_bytes,
                                    int32_t* device_error, void* stream);

/*
 * spec_verify_sample without a workspace argument, for callers that cannot
 * allocate device memory: code under HIP graph capture, serving loops that
 * must not allocate, harnesses that forbid hipMalloc.  Arguments, results and
 * kernels are those of spec_verify_sample; the workspace is a fixed array of
 * SV_NOALLOC_SCRATCH_BYTES in device memory that the library holds on each
 * GPU it runs on until the process ends.  A call whose
 * spec_verify_workspace_bytes(B, K, V) exceeds that size returns
 * SV_ERR_SCRATCH and enqueues nothing.  The call allocates no memory: the
 * first call on a device looks the array up and enqueues one fill kernel
 * that clears it on `stream`; the verify kernels leave it all zero again.
 * Every call on one GPU shares that GPU's array: calls that overlap in time
 * on one GPU (different streams or threads without ordering between them)
 * race and give undefined results; calls on one stream are ordered.
 */
#define SV_NOALLOC_SCRATCH_BYTES ((size_t)8 << 20)
SV_API size_t spec_verify_noalloc_scratch_bytes(void);   /* SV_NOALLOC_SCRATCH_BYTES */
SV_API sv_status spec_verify_sample_noalloc(const void* target_logits, int logits_dtype,
                                            const float* draft_probs,
                                            const int32_t* draft_tokens,
                                            const float* uniforms, float temperature,
                                            int B, int K, int V,
                                            int32_t* out_tokens, int32_t* out_num_accepted,
                                            float* out_draft_target_prob,
                                            int32_t* device_error, void* stream);

/*
 * Sampled verify that takes the drafter's distributions as its logits plus a
 * per-row descriptor (from spec_draft_sample) instead of a dense [B][K][V]
 * q: q_k(x) is recomputed where the method needs it -- at each draft token
 * and along row a for the residual draw.  Results are those of
 * spec_verify_sample with draft_probs = the q that spec_draft_sample would
 * have written (bit for bit).  It spares the dense q's write and halves the
 * draw's drafter-row read (bf16 logits instead of fp32 q).
 *   drafter_logits   [n_drafter_rows][V], same dtype as target_logits.
 *   drafter_rows     optional [B][K] int32: the drafter row of draft k of
 *                    sequence b (NULL: row b*K + k, needs n_drafter_rows >= B*K);
 *                    a row outside [0, n_drafter_rows) sets SV_DEVERR_ROW_INDEX
 *                    and counts as q = 0.
 *   drafter_desc     [B][K] sv_draft_row, as written by spec_draft_sample for
 *                    the same rows (desc b*K+k describes draft k of sequence b).
 *   Other arguments as for spec_verify_sample.  The kernels are enqueued as
 *                    for spec_verify_sample.
 */
SV_API sv_status spec_verify_sample_lq(const void* target_logits, int logits_dtype,
                                       const void* drafter_logits, int64_t n_drafter_rows,
                                       const int32_t* drafter_rows,
                                       const sv_draft_row* drafter_desc,
                                       const int32_t* draft_tokens,
                                       const float* uniforms, float temperature,
                                       int B, int K, int V,
                                       int32_t* out_tokens, int32_t* out_num_accepted,
                                       float* out_draft_target_prob,
                                       void* workspace, size_t workspace_bytes,
                                       int32_t* device_error, void* stream);

/*
 * Verify of a mixed serving batch: sequence b follows the greedy rule of
 * spec_verify_greedy when temperatures[b] = 0, and the rejection sampling of
 * spec_verify_sample at temperature temperatures[b] when it is > 0, all in
 * one launch sequence.  Source: "Project 14", section 架构 (one server
 * verifies every running request's drafts in a single target pass, each
 * request with its own sampling settings) and section 概念 (the greedy path).
 *   target_logits, draft_probs, draft_tokens, uniforms, out_tokens,
 *   out_num_accepted, workspace: as for spec_verify_sample; the draft_probs
 *                    rows and uniforms of greedy sequences are not read.
 *   temperatures     [B] fp32 device array.  A value that is negative, NaN,
 *                    infinite or too small for log2(e)/T to be a finite fp32
 *                    sets SV_DEVERR_TEMPERATURE and verifies that sequence greedily.
 *   out_draft_target_prob  optional [B][K]: p_k(d[b][k]) for sampled
 *                    sequences; for greedy ones 1 where d[b][k] is row k's
 *                    lowest-index argmax and 0 elsewhere (the T -> 0 limit).
 * Results equal those of spec_verify_greedy / spec_verify_sample on each
 * sequence alone.  The same kernels as spec_verify_sample are enqueued (the
 * separate locate kernel whenever V > 2048, at every batch size); the draw
 * and locate kernels stop after the accept scan for greedy sequences.
 */
SV_API sv_status spec_verify_mixed(const void* target_logits, int logits_dtype,
                                   const float* draft_probs, const int32_t* draft_tokens,
                                   const float* uniforms, const float* temperatures,
                                   int B, int K, int V,
                                   int32_t* out_tokens, int32_t* out_num_accepted,
                                   float* out_draft_target_prob,
                                   void* workspace, size_t workspace_bytes,
                                   int32_t* device_error, void* stream);

/*
 * Early-exit forms of spec_verify_greedy, spec_verify_sample and
 * spec_verify_mixed.  Drafts are tested in order and the first rejection
 * ends a sequence's round ("Project 14", section 架构: the verified prefix
 * is kept and the rest resampled), so the target rows past it never enter
 * the sequence's outputs.  These forms compute row statistics over the
 * draft positions in ranges [0,1), [1,2), [2,4), [4,8), ... (one launch
 * each), a range only for the sequences whose drafts before it were all
 * accepted (a gate kernel before each range but the first lists them),
 * then run the usual accept scan and draw: a sequence that accepts a drafts
 * has at most 2a+1 of its K+1 logit rows read (all of them only when a
 * range reaches past its first rejection), at the cost of about
 * 2 log2(K+1) more launches.  Arguments, validation, workspace and device
 * flags are those of the corresponding call; out_tokens and
 * out_num_accepted are identical to its outputs bit for bit (a sampled
 * row's statistics are computed by the same arithmetic; a greedy row's
 * maximum and lowest argmax do not depend on how the row is split, and the
 * greedy form splits rows finer).  out_draft_target_prob
 * [b][k] equals the full call's value for k <= num_accepted[b] and is 0
 * past it.  The launches per call are the gates and row-statistics kernels
 * of the ranges, then the kernels that follow them in the full call.  The ranges
 * are dependent launches: for small batches, bound by latency, these forms
 * are slower than the full calls; they pay for large batches, bound by the
 * bytes of the logits.
 */
SV_API sv_status spec_verify_greedy_early_exit(const void* target_logits, int logits_dtype,
                                               const int32_t* draft_tokens, int B, int K, int V,
                                               int32_t* out_tokens, int32_t* out_num_accepted,
                                               void* workspace, size_t workspace_bytes,
                                               int32_t* device_error, void* stream);
SV_API sv_status spec_verify_sample_early_exit(const void* target_logits, int logits_dtype,
                                               const float* draft_probs,
                                               const int32_t* draft_tokens, const float* uniforms,
                                               float temperature, int B, int K, int V,
                                               int32_t* out_tokens, int32_t* out_num_accepted,
                                               float* out_draft_target_prob, void* workspace,
                                               size_t workspace_bytes, int32_t* device_error,
                                               void* stream);
SV_API sv_status spec_verify_mixed_early_exit(const void* target_logits, int logits_dtype,
                                              const float* draft_probs,
                                              const int32_t* draft_tokens, const float* uniforms,
                                              const float* temperatures, int B, int K, int V,
                                              int32_t* out_tokens, int32_t* out_num_accepted,
                                              float* out_draft_target_prob, void* workspace,
                                              size_t workspace_bytes, int32_t* device_error,
                                              void* stream);

/*
 * A mixed serving batch (as spec_verify_mixed: per-sequence temperatures,
 * 0 = greedy) whose drafter distributions are handed over as drafter logits
 * plus row descriptors (as spec_verify_sample_lq).  Results equal those of
 * spec_verify_mixed with draft_probs = the q that spec_draft_sample would have
 * written for those rows (bit for bit).  Sources: "Project 14", section 架构
 * (one verify pass over every request, each with its own sampling settings).
 *   temperatures     [B] fp32 device array, as for spec_verify_mixed (bad
 *                    values: SV_DEVERR_TEMPERATURE, verified greedily); the
 *                    drafter rows and descriptors of greedy sequences are not
 *                    read.
 *   Other arguments as for spec_verify_sample_lq.  The kernels are enqueued
 *   as for spec_verify_mixed.
 */
SV_API sv_status spec_verify_mixed_lq(const void* target_logits, int logits_dtype,
                                      const void* drafter_logits, int64_t n_drafter_rows,
                                      const int32_t* drafter_rows,
                                      const sv_draft_row* drafter_desc,
                                      const int32_t* draft_tokens,
                                      const float* uniforms, const float* temperatures,
                                      int B, int K, int V,
                                      int32_t* out_tokens, int32_t* out_num_accepted,
                                      float* out_draft_target_prob,
                                      void* workspace, size_t workspace_bytes,
                                      int32_t* device_error, void* stream);

/*
 * Early-exit forms of spec_verify_sample_lq and spec_verify_mixed_lq: the
 * row statistics only up to each sequence's first rejection, as
 * spec_verify_sample_early_exit does for the dense q.  Arguments, validation
 * and results as the corresponding call, out_draft_target_prob 0 past
 * num_accepted[b].
 */
SV_API sv_status spec_verify_sample_lq_early_exit(
    const void* target_logits, int logits_dtype, const void* drafter_logits,
    int64_t n_drafter_rows, const int32_t* drafter_rows, const sv_draft_row* drafter_desc,
    const int32_t* draft_tokens, const float* uniforms, float temperature, int B, int K, int V,
    int32_t* out_tokens, int32_t* out_num_accepted, float* out_draft_target_prob,
    void* workspace, size_t workspace_bytes, int32_t* device_error, void* stream);
SV_API sv_status spec_verify_mixed_lq_early_exit(
    const void* target_logits, int logits_dtype, const void* drafter_logits,
    int64_t n_drafter_rows, const int32_t* drafter_rows, const sv_draft_row* drafter_desc,
    const int32_t* draft_tokens, const float* uniforms, const float* temperatures, int B, int K,
    int V, int32_t* out_tokens, int32_t* out_num_accepted, float* out_draft_target_prob,
    void* workspace, size_t workspace_bytes, int32_t* device_error, void* stream);

/*
 * Verification of a draft tree per sequence.  "Project 14", section 概念:
 * P-EAGLE's parallel speculation forms deeper draft trees (the pages give no
 * tree shape; any shape of up to SV_MAX_K nodes is accepted).  Node 0 is the
 * root (the last committed token); nodes 1..N have parents[b][i-1] < i and
 * tokens[b][i-1]; target logit row n (n = 0..N) is the target's distribution
 * after node n.
 *   temperature = 0 (greedy): from the root, move to the lowest-index child
 *     whose token is the lowest-index argmax of the current row; when none
 *     matches, emit that argmax.
 *   temperature > 0 (sampled): draft_probs row n is the distribution node n's
 *     children were drawn from, independently.  With r = softmax(row / T) of
 *     the current node, its children are tested in index order: child x is
 *     accepted iff uniforms[b][i] < r(x) / q(x) (q(x) = 0: iff r(x) > 0); a
 *     rejection replaces r by max(0, r - q) normalised (by p if that is all
 *     zero).  An accepted child becomes the current node; when every child is
 *     rejected, or at a leaf, the new token is the inverse-CDF draw from r
 *     with uniforms[b][0].  With one child per node this is spec_verify_sample.
 *   target_logits    [B][N+1][V], SV_F32 or SV_BF16.
 *   draft_probs      [B][N+1][V] fp32 (sampled; NULL allowed when greedy).
 *   parents, tokens  [B][N] int32 (bad nodes: SV_DEVERR_TREE, treated as absent).
 *   uniforms         [B][N+1] fp32 in [0, 1) (sampled).
 *   out_tokens       [B][N+1]: the accepted path's tokens, the new token, -1.
 *   out_path         [B][N+1]: the accepted node indices, then -1.
 *   out_num_accepted [B]: the accepted path length.
 *   workspace        spec_verify_workspace_bytes(B, N, V) bytes, zeroed once.
 * 0 <= N <= SV_MAX_K.  Two kernels are enqueued: the row statistics of all
 * B*(N+1) rows, then one workgroup per sequence walks its tree (each
 * rejection costs that workgroup one pass over the node's row).
 */
SV_API sv_status spec_verify_tree(const void* target_logits, int logits_dtype,
                                  const float* draft_probs, const int32_t* parents,
                                  const int32_t* tokens, const float* uniforms, float temperature,
                                  int B, int N, int V,
                                  int32_t* out_tokens, int32_t* out_path,
                                  int32_t* out_num_accepted,
                                  void* workspace, size_t workspace_bytes,
                                  int32_t* device_error, void* stream);

/*
 * Sampled tree verification that takes the drafter's distributions as its
 * logits plus a per-node descriptor (from spec_draft_sample), as
 * spec_verify_sample_lq does for chains: q row n (the distribution node n's
 * children were drawn from) is recomputed from drafter logit row
 * drafter_rows[b][n] with descriptor drafter_desc[b][n] where the walk needs
 * it (at each child's token, and along the node's row for a residual pass).
 * Results are those of spec_verify_tree with draft_probs = the q that
 * spec_draft_sample would have written for those rows (bit for bit).  Each
 * residual pass then reads the node's drafter logit row (V * 2 bytes for
 * bf16) instead of its fp32 q row (V * 4).  Source: as spec_verify_tree
 * ("Project 14", section 概念).
 *   drafter_logits   [n_drafter_rows][V], same dtype as target_logits.
 *   drafter_rows     optional [B][N+1] int32 (NULL: row b*(N+1) + n, needs
 *                    n_drafter_rows >= B*(N+1)); a row outside
 *                    [0, n_drafter_rows) that the walk uses sets
 *                    SV_DEVERR_ROW_INDEX and counts as q = 0.
 *   drafter_desc     [B][N+1] sv_draft_row, 16-byte aligned.
 *   temperature      > 0 (sampling only); other arguments as for
 *                    spec_verify_tree.  The same two kernels are enqueued.
 */
SV_API sv_status spec_verify_tree_lq(const void* target_logits, int logits_dtype,
                                     const void* drafter_logits, int64_t n_drafter_rows,
                                     const int32_t* drafter_rows,
                                     const sv_draft_row* drafter_desc,
                                     const int32_t* parents, const int32_t* tokens,
                                     const float* uniforms, float temperature,
                                     int B, int N, int V,
                                     int32_t* out_tokens, int32_t* out_path,
                                     int32_t* out_num_accepted,
                                     void* workspace, size_t workspace_bytes,
                                     int32_t* device_error, void* stream);

/*
 * Early-exit forms of spec_verify_tree and spec_verify_tree_lq: no row
 * kernel; the walk computes the statistics of a node's row (one workgroup
 * pass) when it reaches the node, so only the rows of the nodes on the
 * accepted path and of the node where the walk stops are read, instead of
 * all B*(N+1).  Same arguments, validation, workspace and flags as the
 * corresponding call; the outcomes are those of the same definitions (the
 * greedy walk's bit for bit), while a row's sum of exponentials is added in
 * a different order than the row kernel's, so a sampled decision within
 * rounding of its threshold may differ from the full call's (the 1e-6
 * near-tie rule).  The walks are one workgroup per tree: these forms pay
 * for batches of at least about one tree per CU.
 */
SV_API sv_status spec_verify_tree_early_exit(const void* target_logits, int logits_dtype,
                                             const float* draft_probs, const int32_t* parents,
                                             const int32_t* tokens, const float* uniforms,
                                             float temperature, int B, int N, int V,
                                             int32_t* out_tokens, int32_t* out_path,
                                             int32_t* out_num_accepted, void* workspace,
                                             size_t workspace_bytes, int32_t* device_error,
                                             void* stream);

/*
 * Tree verification of a mixed serving batch: tree b is walked greedily when
 * temperatures[b] = 0 and by rejection sampling at temperatures[b] when it is
 * > 0, as spec_verify_mixed treats a chain batch ("Project 14", section 架构:
 * each request with its own sampling settings in one target pass; section
 * 概念: trees).  Arguments as spec_verify_tree with temperatures [B] fp32 in
 * place of the scalar temperature; draft_probs and uniforms are required
 * (the rows of greedy trees are not read).  A temperature that is negative,
 * NaN, infinite or too small for log2(e)/T to be a finite fp32 sets
 * SV_DEVERR_TEMPERATURE and walks that tree greedily.  Results equal those
 * of spec_verify_tree on each tree alone at its temperature.  The
 * _early_exit form is that of spec_verify_tree_early_exit.  These take the
 * dense q; the drafter-logit tree calls take one temperature for the batch.
 */
SV_API sv_status spec_verify_tree_mixed(const void* target_logits, int logits_dtype,
                                        const float* draft_probs, const int32_t* parents,
                                        const int32_t* tokens, const float* uniforms,
                                        const float* temperatures, int B, int N, int V,
                                        int32_t* out_tokens, int32_t* out_path,
                                        int32_t* out_num_accepted, void* workspace,
                                        size_t workspace_bytes, int32_t* device_error,
                                        void* stream);
SV_API sv_status spec_verify_tree_mixed_early_exit(
    const void* target_logits, int logits_dtype, const float* draft_probs,
    const int32_t* parents, const int32_t* tokens, const float* uniforms,
    const float* temperatures, int B, int N, int V, int32_t* out_tokens, int32_t* out_path,
    int32_t* out_num_accepted, void* workspace, size_t workspace_bytes, int32_t* device_error,
    void* stream);
SV_API sv_status spec_verify_tree_lq_early_exit(
    const void* target_logits, int logits_dtype, const void* drafter_logits,
    int64_t n_drafter_rows, const int32_t* drafter_rows, const sv_draft_row* drafter_desc,
    const int32_t* parents, const int32_t* tokens, const float* uniforms, float temperature,
    int B, int N, int V, int32_t* out_tokens, int32_t* out_path, int32_t* out_num_accepted,
    void* workspace, size_t workspace_bytes, int32_t* device_error, void* stream);

/*
 * P-EAGLE drafter batch.  Source: the P-EAGLE / TorchSpec blog summary,
 * section 并行架构的核心创新 (one drafter forward predicts all K drafts
 * from the NTP row and K-1 MASK rows carrying h_shared) and section TorchSpec
 * 集成与工程优化 (the batch is rebuilt on the GPU: copy, insert MASK slots,
 * remap positions, PADDING_SLOT_ID = -1 for rejected tokens, hidden states
 * broadcast by a dedicated copy).  Each sequence b owns the 2K rows
 * [2Kb, 2Kb+2K).
 * With a = num_accepted[b], c = verify_out_tokens[b][a], L = start_pos[b]
 * (position of verify slot 0) and h[i] = target_hidden row b*(K+1)+i (the
 * target's hidden state at verify slot i):
 *
 *   row a' = 0..a-1   id verify_out_tokens[b][r]   pos L+r     hidden h[r]      slot(L+r)
 *   row a             id c (the new token)         pos L+a     hidden h[a]      slot(L+a)
 *   row a+m, m=1..K-1 id mask_token_id             pos L+a+m   hidden h_shared  slot(L+a+m)
 *   row a+K+j,        id draft_tokens[b][a+j]      pos L+a+1+j hidden h[a+1+j]  -1
 *     j=0..K-a-1
 *
 * slot(p) = block_table[b][p / block_size] * block_size + p % block_size.
 * out_sample_rows[b][k] = 2Kb + a + k: the NTP row and the K-1 MASK rows whose
 * drafter outputs are the next K drafts.
 *
 *   verify_out_tokens [B][K+1] int32 and num_accepted [B] int32, as written by
 *                    spec_verify_* (they may still be in flight on `stream`).
 *   draft_tokens     [B][K] int32.        start_pos [B] int64.
 *   block_table      [B][max_blocks_per_seq] int32 page ids.
 *   target_hidden    [B*(K+1)][H], h_shared [H]: elements of hidden_dtype
 *                    (SV_BF16, SV_F16 or SV_F32), copied bit for bit.
 *   out_input_ids [B*2K] int32, out_positions [B*2K] int64,
 *   out_slot_mapping [B*2K] int64, out_hidden [B*2K][H], out_sample_rows
 *   optional [B][K] int32.
 * 1 <= K <= SV_MAX_K, H >= 1, block_size >= 1, max_blocks_per_seq >= 1.
 */
SV_API sv_status peagle_build_draft_batch(const int32_t* verify_out_tokens,
                                          const int32_t* num_accepted,
                                          const int32_t* draft_tokens,
                                          const int64_t* start_pos,
                                          const int32_t* block_table,
                                          int max_blocks_per_seq, int block_size,
                                          const void* target_hidden, const void* h_shared,
                                          int hidden_dtype, int32_t mask_token_id,
                                          int B, int K, int H,
                                          int32_t* out_input_ids, int64_t* out_positions,
                                          int64_t* out_slot_mapping, void* out_hidden,
                                          int32_t* out_sample_rows,
                                          int32_t* device_error, void* stream);

/*
 * Drafter-output sampling: the P-EAGLE drafter's K prediction rows per
 * sequence (the NTP row and the K-1 MASK rows, out_sample_rows above) become
 * the K draft tokens and the drafter distribution q of the next verify.
 * Source: the P-EAGLE / TorchSpec blog summary, section 并行架构的核心创新
 * (one drafter forward predicts all K drafts); "Project 14", section 架构 (the
 * drafter proposes k tokens that the target verifies).
 * For draft k of sequence b, z = drafter_logits row row_index[b][k] (or row
 * b*K + k when row_index is NULL) and T_b = temperatures[b] (or the scalar
 * temperature when temperatures is NULL):
 *   T_b > 0:  q = softmax(z / T_b); the token is the smallest v whose running
 *             total of q in vocabulary order exceeds uniforms[b][k] * sum(q)
 *             (inverse CDF, never a token with q = 0);
 *   T_b = 0:  greedy drafting: the token is the lowest-index argmax of z and
 *             q is one-hot at it.
 *   drafter_logits   [n_rows][V], SV_F32 or SV_BF16.
 *   row_index        optional [B][K] int32 in [0, n_rows), e.g. out_sample_rows
 *                    of peagle_build_draft_batch; NULL needs n_rows >= B*K.
 *   uniforms         [B][K] fp32 in [0, 1); may be NULL only when temperature
 *                    is 0 and temperatures is NULL (every draft greedy).
 *   temperature      finite, >= 0 (0 = greedy).
 *   temperatures     optional [B] fp32 device array overriding `temperature`
 *                    per sequence (bad values: SV_DEVERR_TEMPERATURE).
 *   out_draft_tokens [B][K] int32, the draft_tokens of the next verify.
 *   out_draft_probs  optional [B][K][V] fp32, the draft_probs of the next
 *                    verify (NULL = not written).
 *   out_row_desc     optional [B][K] sv_draft_row: what spec_verify_sample_lq
 *                    needs to recompute q from the drafter logits instead of
 *                    reading a dense q (NULL = not written).
 * 1 <= K <= SV_MAX_K, 1 <= V <= SV_MAX_V; B = 0 is a no-op.  Arithmetic as in
 * spec_verify_sample (fp32 exponentials, fp64 running totals).  One kernel is
 * enqueued; no workspace is needed.
 */
SV_API sv_status spec_draft_sample(const void* drafter_logits, int logits_dtype, int64_t n_rows,
                                   const int32_t* row_index, const float* uniforms,
                                   float temperature, const float* temperatures,
                                   int B, int K, int V,
                                   int32_t* out_draft_tokens, float* out_draft_probs,
                                   sv_draft_row* out_row_desc,
                                   int32_t* device_error, void* stream);

/*
 * Acceptance metrics, accumulated on the device.  `metrics` is an array of
 * spec_accept_metrics_words(K) uint64 counters in device memory, zeroed by the
 * caller once; every call adds one verify call's counts:
 *   [SV_METRICS_STEPS]     calls
 *   [SV_METRICS_ROUNDS]    rounds (one sequence in one call)
 *   [SV_METRICS_PROPOSED]  drafts proposed (K per round)
 *   [SV_METRICS_ACCEPTED]  drafts accepted (sum of num_accepted)
 *   [SV_METRICS_EMITTED]   tokens emitted (accepted + the new token per round)
 *   [SV_METRICS_HIST + a]  rounds that accepted exactly a drafts, a = 0..K
 * Acceptance length (mean accepted drafts per round, P-EAGLE / TorchSpec blog
 * summary, section 监控与调优建议) = ACCEPTED / ROUNDS; tokens per round =
 * EMITTED / ROUNDS; draft acceptance rate = ACCEPTED / PROPOSED ("Project 14",
 * section 使用它, reports acceptance rate and accepted tokens per step); the
 * histogram gives the acceptance rate at each draft position.  Counts are
 * integers added with atomics, so totals are exact and order-independent.
 * num_accepted [B] int32 as written by spec_verify_* (values outside [0, K]
 * set SV_DEVERR_ACCEPT_COUNT and are clamped).  1 <= K <= SV_MAX_K.  B = 0 is a
 * no-op.  One kernel is enqueued.
 */
#define SV_METRICS_STEPS 0
#define SV_METRICS_ROUNDS 1
#define SV_METRICS_PROPOSED 2
#define SV_METRICS_ACCEPTED 3
#define SV_METRICS_EMITTED 4
#define SV_METRICS_HIST 5
SV_API size_t spec_accept_metrics_words(int K);  /* SV_METRICS_HIST + K + 1; 0 if K is invalid */
SV_API sv_status spec_accept_metrics(const int32_t* num_accepted, int B, int K, uint64_t* metrics,
                                     int32_t* device_error, void* stream);

/*
 * One decode step captured once as a HIP graph and replayed with a single
 * launch: the verify call (greedy, sampled or mixed), then, optionally, the
 * P-EAGLE build from its outputs and the acceptance metrics.  Every buffer and
 * shape is fixed at capture (static maximum shapes, as serving engines
 * capture their graphs per batch size and extend the capture range by
 * K x max_num_seqs for the drafter batch: P-EAGLE / TorchSpec blog summary,
 * section TorchSpec 集成与工程优化); each replay reads whatever the buffers
 * hold at that time.  The buffers must stay allocated while the graph exists.
 * Fields mirror the arguments of the calls above; the build is skipped when
 * out_hidden is NULL and the metrics when metrics is NULL.  With
 * drafter_logits set (sample / mixed only) the captured verify is
 * spec_verify_sample_lq or spec_verify_mixed_lq on drafter_logits,
 * n_drafter_rows, drafter_rows and drafter_desc, and draft_probs must be NULL
 * (SV_ERR_VALUE otherwise; SV_ERR_VALUE too for drafter_logits in greedy
 * mode).  early_exit != 0 captures the _early_exit form of the verify (row
 * statistics only up to each sequence's first rejection).  Argument errors
 * of the captured calls are returned by sv_step_graph_create, which then
 * creates nothing.  Kernel tracing is paused during capture.
 */
#define SV_STEP_GREEDY 0
#define SV_STEP_SAMPLE 1
#define SV_STEP_MIXED 2
typedef struct sv_step_desc {
  int mode;                               /* SV_STEP_*                          */
  const void* target_logits;
  int logits_dtype;
  const float* draft_probs;               /* sample / mixed                      */
  const int32_t* draft_tokens;
  const float* uniforms;                  /* sample / mixed                      */
  float temperature;                      /* sample                              */
  const float* temperatures;              /* mixed                               */
  int B, K, V;
  int32_t* out_tokens;
  int32_t* out_num_accepted;
  float* out_draft_target_prob;           /* optional                            */
  void* workspace;
  size_t workspace_bytes;
  const int64_t* start_pos;               /* build                               */
  const int32_t* block_table;
  int max_blocks_per_seq, block_size;
  const void* target_hidden;
  const void* h_shared;
  int hidden_dtype;
  int32_t mask_token_id;
  int H;
  int32_t* out_input_ids;
  int64_t* out_positions;
  int64_t* out_slot_mapping;
  void* out_hidden;                       /* NULL: no build                      */
  int32_t* out_sample_rows;               /* optional                            */
  uint64_t* metrics;                      /* NULL: no metrics                    */
  int32_t* device_error;                  /* optional                            */
  const void* drafter_logits;             /* NULL: dense draft_probs             */
  int64_t n_drafter_rows;                 /* with drafter_logits                 */
  const int32_t* drafter_rows;            /* optional, with drafter_logits       */
  const sv_draft_row* drafter_desc;       /* with drafter_logits                 */
  int early_exit;                         /* 0: full verify; else _early_exit    */
} sv_step_desc;

typedef struct sv_step_graph sv_step_graph;   /* opaque */
SV_API sv_status sv_step_graph_create(const sv_step_desc* desc, sv_step_graph** out);
SV_API sv_status sv_step_graph_launch(sv_step_graph* graph, void* stream);
SV_API void sv_step_graph_destroy(sv_step_graph* graph);

/*
 * Kernel tracing, a profiling aid.  While tracing is on for the calling host
 * thread, every kernel the library enqueues whose id is set in `kernel_mask`
 * (bit i = kernel id i; ~0u = all) is bracketed by two HIP timing events
 * recorded on the kernel's own stream, for up to `capacity` launches (later
 * launches are not traced).  After the stream has completed, entry i gives
 * the kernel's id and its duration in milliseconds.  sv_trace_begin creates
 * the events (it may be called again to start over); sv_trace_end destroys
 * them.  Tracing adds two event records per traced launch and nothing else.
 * sv_trace_enable(0) pauses an active trace (launches enqueued meanwhile are
 * neither traced nor counted against `capacity`) and sv_trace_enable(1)
 * resumes it, so that a caller can trace a sample of a loop's launches; it
 * does nothing when no trace is active.
 */
#define SV_KERNEL_VERIFY_GREEDY_ROWS 0   /* spec_verify_greedy: row max / argmax         */
#define SV_KERNEL_VERIFY_SAMPLE_ROWS 1   /* spec_verify_sample: row max / sum of exp     */
#define SV_KERNEL_VERIFY_SAMPLE_DRAW 2   /* spec_verify_sample / _mixed / _lq: the accept
                                            scan, then residual / bonus tile masses      */
#define SV_KERNEL_PEAGLE_BUILD 3         /* peagle_build_draft_batch                     */
#define SV_KERNEL_VERIFY_GREEDY_ACCEPT 4 /* spec_verify_greedy: accept scan              */
#define SV_KERNEL_VERIFY_SAMPLE_LOCATE 5 /* spec_verify_sample / _mixed / _lq: locate the
                                            drawn token                                  */
#define SV_KERNEL_DRAFT_SAMPLE 6         /* spec_draft_sample                            */
#define SV_KERNEL_VERIFY_MIXED_ROWS 7    /* spec_verify_mixed: row statistics            */
#define SV_KERNEL_ACCEPT_METRICS 8       /* spec_accept_metrics                          */
#define SV_KERNEL_TREE_ROWS 9            /* spec_verify_tree: row statistics             */
#define SV_KERNEL_TREE_WALK 10           /* spec_verify_tree: the walk down the tree     */

SV_API const char* sv_kernel_name(int kernel_id);
SV_API sv_status sv_trace_begin(int capacity, unsigned kernel_mask); /* SV_ERR_VALUE if capacity < 1 */
SV_API int sv_trace_count(void);                     /* launches traced so far         */
SV_API sv_status sv_trace_read(int i, int* kernel_id, float* ms);  /* waits for entry i */
SV_API void sv_trace_end(void);
SV_API void sv_trace_enable(int on);                 /* pause (0) / resume (1)        */

#ifdef __cplusplus
}
#endif

#endif /* SPEC_VERIFY_H */
