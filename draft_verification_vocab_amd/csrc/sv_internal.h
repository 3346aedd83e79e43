// Host-side launch descriptors shared by the C ABI and the kernel files.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "../../include/spec_verify.h"

namespace sv {

struct VerifyLaunch {
  const void* logits;
  const float* draft_probs;      // sampling only
  const int32_t* draft_tokens;
  const float* uniforms;         // sampling only
  float temperature;             // sampling only
  int B, K, V;
  int bf16;                      // logits are bf16 (else fp32)
  int sample;                    // rejection sampling (else greedy)
  int mixed;                     // per-sequence temperatures (overrides sample)
  const float* temperatures;     // mixed: [B]
  // q from the drafter logits (sampling only): dlogits != NULL
  const void* dlogits;           // [d_rows][V], same dtype as logits
  long d_rows;
  const int32_t* drows;          // [B*K] or NULL (row b*K + k)
  const sv_draft_row* ddesc;     // [B*K]
  int vec;                       // 16-byte vector loads are legal for every row
  int32_t* out_tokens;
  int32_t* out_num_accepted;
  float* out_p_draft;            // may be NULL
  void* workspace;
  int32_t* device_error;         // may be NULL
  // statistics only of the rows up to the first rejection, one launch per
  // draft position (spec_verify_*_early_exit)
  int early_exit = 0;
};

struct BuildLaunch {
  const int32_t* verify_out_tokens;
  const int32_t* num_accepted;
  const int32_t* draft_tokens;
  const int64_t* start_pos;
  const int32_t* block_table;
  int max_blocks, block_size;
  const void* target_hidden;
  const void* h_shared;
  int elem_bytes;                // 2 or 4
  int vec;                       // rows are 16-byte aligned multiples of 16 bytes
  int32_t mask_token_id;
  int B, K, H;
  int32_t* out_input_ids;
  int64_t* out_positions;
  int64_t* out_slot_mapping;
  void* out_hidden;
  int32_t* out_sample_rows;      // may be NULL
  int32_t* device_error;         // may be NULL
};

struct DraftLaunch {
  const void* logits;            // [n_rows][V]
  const int32_t* row_index;      // [B*K] or NULL
  long n_rows;
  const float* uniforms;         // [B*K]
  const float* temperatures;     // [B] or NULL
  float temperature;
  int B, K, V;
  int bf16;
  int vec;                       // 16-byte vector loads / stores are legal for every row
  int32_t* out_tokens;
  float* out_probs;              // may be NULL
  sv_draft_row* out_desc;        // may be NULL
  int32_t* device_error;         // may be NULL
};

struct TreeLaunch {
  const void* logits;            // [B][N+1][V]
  const float* draft_probs;      // [B][N+1][V] (sampled, dense q)
  const void* dlogits;           // q from drafter logits instead: [d_rows][V], same dtype
  long d_rows;
  const int32_t* drows;          // optional [B][N+1] drafter row of node n (else b*(N+1)+n)
  const sv_draft_row* ddesc;     // [B][N+1] descriptors of those rows
  const int32_t* parents;        // [B][N]
  const int32_t* tokens;         // [B][N]
  const float* uniforms;         // [B][N+1] (sampled)
  float temperature;             // 0 = greedy
  int B, N, V;
  int bf16;
  int vec;
  int32_t* out_tokens;           // [B][N+1]
  int32_t* out_path;             // [B][N+1]
  int32_t* out_num_accepted;     // [B]
  void* workspace;
  int32_t* device_error;
  // row statistics computed by the walk for the nodes it visits only
  // (spec_verify_tree*_early_exit), instead of by the row kernel for all
  int lazy = 0;
  // per-tree temperatures (spec_verify_tree_mixed*): tree b greedy when 0,
  // else sampled at its own; NULL: `temperature` for every tree
  const float* temperatures = nullptr;
};

// The row-statistics partials of a verify workspace: [B][K+1][S] entries.
struct RowPartials {
  void* partials;
  int S;
};

int verify_splits(int B, int K, int V);
RowPartials row_partials(void* workspace, int B, int K, int V);
// Row statistics of B*(K+1) rows into the workspace's partials: greedy,
// sampled at scale c, or (temperatures != NULL) each sequence by its own rule.
hipError_t launch_row_stats(const void* logits, int bf16, int vec, int sample, float c,
                            const float* temperatures, int B, int K, int V, void* workspace,
                            int trace_id, hipStream_t stream);
hipError_t launch_tree(const TreeLaunch& L, hipStream_t stream);

// Kernel tracing (per host thread): bracket a launch with events on its stream.
void trace_before(hipStream_t stream, int kernel_id);
void trace_after(hipStream_t stream, int kernel_id);
size_t verify_workspace_bytes(int B, int K, int V);
// Argument checks and launches of spec_verify_greedy / _sample / _mixed
// (sample: 0, 1, 2) and their _early_exit forms; launch = false checks every
// argument but the workspace and enqueues nothing.
sv_status verify_common(const void* logits, int dtype, const float* draft_probs,
                        const int32_t* draft_tokens, const float* uniforms, float temperature,
                        const float* temperatures, int sample, int B, int K, int V,
                        int32_t* out_tokens, int32_t* out_num_accepted, float* out_p_draft,
                        void* workspace, size_t workspace_bytes, int32_t* device_error,
                        void* stream, bool launch, bool early_exit = false);
hipError_t launch_verify(const VerifyLaunch& L, hipStream_t stream);
hipError_t launch_build(const BuildLaunch& L, hipStream_t stream);
hipError_t launch_draft(const DraftLaunch& L, hipStream_t stream);
hipError_t launch_metrics(const int32_t* num_accepted, int B, int K, uint64_t* metrics,
                          int32_t* device_error, hipStream_t stream);

// Pause kernel tracing on this host thread for the lifetime of the object
// (graph capture records no timing events).
struct TracePause {
  TracePause();
  ~TracePause();
  bool was_on;
};

}  // namespace sv
