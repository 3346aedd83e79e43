// C ABI of libspecverify: host-side validation, then the call's kernel
// launches.  Nothing here reads device memory or synchronises (except
// sv_trace_read, which waits for the traced launch it reports); on any
// validation error a call returns before touching the GPU.
#include <math.h>
#include <stdint.h>

#include <vector>

#include "sv_internal.h"

namespace sv {

// ---------------------------------------------------------------- tracing
namespace {
struct Tracer {
  bool on = false;
  bool pending = false;           // trace_before recorded an event for the next launch
  unsigned mask = ~0u;
  int cap = 0, count = 0;
  std::vector<hipEvent_t> ev;     // 2 per traced launch
  std::vector<int> ids;
  void destroy() {
    for (hipEvent_t e : ev) (void)hipEventDestroy(e);
    ev.clear();
    ids.clear();
    on = pending = false;
    cap = count = 0;
  }
  ~Tracer() { destroy(); }
};
thread_local Tracer tracer;
}  // namespace

void trace_before(hipStream_t stream, int kernel_id) {
  tracer.pending = tracer.on && tracer.count < tracer.cap && ((tracer.mask >> kernel_id) & 1u);
  if (tracer.pending) (void)hipEventRecord(tracer.ev[2 * tracer.count], stream);
}

TracePause::TracePause() : was_on(tracer.on) { tracer.on = false; }
TracePause::~TracePause() { tracer.on = was_on; }

void trace_after(hipStream_t stream, int kernel_id) {
  if (tracer.pending) {
    (void)hipEventRecord(tracer.ev[2 * tracer.count + 1], stream);
    tracer.ids[tracer.count++] = kernel_id;
    tracer.pending = false;
  }
}

}  // namespace sv

namespace {

inline bool aligned(const void* p, size_t n) { return (reinterpret_cast<uintptr_t>(p) % n) == 0; }

constexpr long kMaxB = SV_MAX_B;    // sequences per call

sv_status check_verify_shape(int B, int K, int V) {
  if (B < 0 || B > kMaxB || K < 0 || K > SV_MAX_K || V < 1 || V > SV_MAX_V) return SV_ERR_SHAPE;
  return SV_OK;
}

}  // namespace

extern "C" {

SV_API const char* sv_status_string(int status) {
  switch (status) {
    case SV_OK: return "ok";
    case SV_ERR_NULL: return "a required pointer is NULL";
    case SV_ERR_SHAPE: return "shape argument out of range";
    case SV_ERR_DTYPE: return "unsupported dtype";
    case SV_ERR_VALUE: return "scalar argument out of range";
    case SV_ERR_WORKSPACE: return "workspace missing or too small";
    case SV_ERR_ALIGN: return "pointer not aligned to its element size";
    case SV_ERR_HIP: return "HIP launch failed";
    case SV_ERR_SCRATCH: return "call needs more scratch than the no-allocation entry point holds";
    default: return "unknown status";
  }
}

SV_API const char* sv_kernel_name(int kernel_id) {
  switch (kernel_id) {
    case SV_KERNEL_VERIFY_GREEDY_ROWS: return "verify_greedy_rows";
    case SV_KERNEL_VERIFY_SAMPLE_ROWS: return "verify_sample_rows";
    case SV_KERNEL_VERIFY_SAMPLE_DRAW: return "verify_sample_draw";
    case SV_KERNEL_PEAGLE_BUILD: return "peagle_build";
    case SV_KERNEL_VERIFY_GREEDY_ACCEPT: return "verify_greedy_accept";
    case SV_KERNEL_VERIFY_SAMPLE_LOCATE: return "verify_sample_locate";
    case SV_KERNEL_DRAFT_SAMPLE: return "draft_sample";
    case SV_KERNEL_VERIFY_MIXED_ROWS: return "verify_mixed_rows";
    case SV_KERNEL_ACCEPT_METRICS: return "accept_metrics";
    case SV_KERNEL_TREE_ROWS: return "tree_rows";
    case SV_KERNEL_TREE_WALK: return "tree_walk";
    default: return "unknown";
  }
}

SV_API sv_status sv_trace_begin(int capacity, unsigned kernel_mask) {
  if (capacity < 1) return SV_ERR_VALUE;
  sv::tracer.destroy();
  sv::tracer.ev.resize(2 * (size_t)capacity);
  for (auto& e : sv::tracer.ev) {
    if (hipEventCreate(&e) != hipSuccess) {
      e = nullptr;
      sv::tracer.destroy();
      return SV_ERR_HIP;
    }
  }
  sv::tracer.ids.assign(capacity, -1);
  sv::tracer.cap = capacity;
  sv::tracer.count = 0;
  sv::tracer.mask = kernel_mask;
  sv::tracer.on = true;
  return SV_OK;
}

SV_API int sv_trace_count(void) { return sv::tracer.count; }

SV_API sv_status sv_trace_read(int i, int* kernel_id, float* ms) {
  if (!kernel_id || !ms) return SV_ERR_NULL;
  if (i < 0 || i >= sv::tracer.count) return SV_ERR_VALUE;
  hipEvent_t e0 = sv::tracer.ev[2 * i], e1 = sv::tracer.ev[2 * i + 1];
  if (hipEventSynchronize(e1) != hipSuccess) return SV_ERR_HIP;
  if (hipEventElapsedTime(ms, e0, e1) != hipSuccess) return SV_ERR_HIP;
  *kernel_id = sv::tracer.ids[i];
  return SV_OK;
}

SV_API void sv_trace_end(void) { sv::tracer.destroy(); }

SV_API void sv_trace_enable(int on) {
  if (sv::tracer.cap > 0) sv::tracer.on = on != 0;
}

SV_API size_t spec_verify_workspace_bytes(int B, int K, int V) {
  if (check_verify_shape(B, K, V) != SV_OK) return 0;
  if (B == 0) return 0;
  return sv::verify_workspace_bytes(B, K, V);
}

}  // extern "C"

namespace sv {

// sample: 0 greedy, 1 one temperature, 2 per-sequence temperatures (mixed).
// launch = false: validate every argument but the workspace and enqueue
// nothing (the no-allocation entry point checks its call before it sets up
// its scratch).
sv_status verify_common(const void* logits, int dtype, const float* draft_probs,
                        const int32_t* draft_tokens, const float* uniforms, float temperature,
                        const float* temperatures, int sample, int B, int K, int V,
                        int32_t* out_tokens, int32_t* out_num_accepted, float* out_p_draft,
                        void* workspace, size_t workspace_bytes, int32_t* device_error,
                        void* stream, bool launch, bool early_exit) {
  sv_status st = check_verify_shape(B, K, V);
  if (st != SV_OK) return st;
  if (dtype != SV_F32 && dtype != SV_BF16) return SV_ERR_DTYPE;
  if (sample == 1 && !(temperature > 0.0f && isfinite(temperature) &&
                       isfinite((float)(1.4426950408889634 / (double)temperature))))
    return SV_ERR_VALUE;
  if (B == 0) return SV_OK;
  if (sample == 2 && !temperatures) return SV_ERR_NULL;
  if (temperatures && !aligned(temperatures, 4)) return SV_ERR_ALIGN;
  if (!logits || !out_tokens || !out_num_accepted || (K > 0 && !draft_tokens)) return SV_ERR_NULL;
  if (sample && (!uniforms || (K > 0 && !draft_probs))) return SV_ERR_NULL;
  if (launch && !workspace) return SV_ERR_WORKSPACE;
  if (launch && workspace_bytes < sv::verify_workspace_bytes(B, K, V)) return SV_ERR_WORKSPACE;
  const size_t esz = dtype == SV_BF16 ? 2 : 4;
  if (!aligned(logits, esz) || !aligned(out_tokens, 4) || !aligned(out_num_accepted, 4) ||
      (draft_tokens && !aligned(draft_tokens, 4)) || (launch && !aligned(workspace, 16)) ||
      (device_error && !aligned(device_error, 4)))
    return SV_ERR_ALIGN;
  if (sample && (!aligned(uniforms, 4) || (draft_probs && !aligned(draft_probs, 4)) ||
                 (out_p_draft && !aligned(out_p_draft, 4))))
    return SV_ERR_ALIGN;
  if ((long)B * (K + 1) * sv::verify_splits(B, K, V) > 0x7fffffffL) return SV_ERR_SHAPE;
  if (!launch) return SV_OK;

  sv::VerifyLaunch L;
  L.logits = logits;
  L.draft_probs = draft_probs;
  L.draft_tokens = draft_tokens;
  L.uniforms = uniforms;
  L.temperature = temperature;
  L.B = B; L.K = K; L.V = V;
  L.bf16 = dtype == SV_BF16;
  L.sample = sample != 0;
  L.mixed = sample == 2;
  L.temperatures = sample == 2 ? temperatures : nullptr;
  L.dlogits = nullptr;
  L.d_rows = 0;
  L.drows = nullptr;
  L.ddesc = nullptr;
  L.vec = (V % 8 == 0) && aligned(logits, 16) && (!sample || !draft_probs || aligned(draft_probs, 16));
  L.out_tokens = out_tokens;
  L.out_num_accepted = out_num_accepted;
  L.out_p_draft = sample ? out_p_draft : nullptr;
  L.workspace = workspace;
  L.device_error = device_error;
  L.early_exit = early_exit ? 1 : 0;
  return sv::launch_verify(L, static_cast<hipStream_t>(stream)) == hipSuccess ? SV_OK : SV_ERR_HIP;
}

// spec_verify_sample_lq (temperatures null: the scalar temperature) and
// spec_verify_mixed_lq (per-sequence temperatures), and their _early_exit
// forms.
sv_status verify_lq(const void* target_logits, int logits_dtype, const void* drafter_logits,
                    int64_t n_drafter_rows, const int32_t* drafter_rows,
                    const sv_draft_row* drafter_desc, const int32_t* draft_tokens,
                    const float* uniforms, float temperature, const float* temperatures, int B,
                    int K, int V, int32_t* out_tokens, int32_t* out_num_accepted,
                    float* out_draft_target_prob, void* workspace, size_t workspace_bytes,
                    int32_t* device_error, void* stream, bool early_exit) {
  sv_status st = check_verify_shape(B, K, V);
  if (st != SV_OK) return st;
  if (n_drafter_rows < 0 || n_drafter_rows > 0x7fffffffL) return SV_ERR_SHAPE;
  if (!drafter_rows && n_drafter_rows < (int64_t)B * K) return SV_ERR_SHAPE;
  if (logits_dtype != SV_F32 && logits_dtype != SV_BF16) return SV_ERR_DTYPE;
  const bool mixed = temperatures != nullptr;
  if (!mixed && !(temperature > 0.0f && isfinite(temperature) &&
                  isfinite((float)(1.4426950408889634 / (double)temperature))))
    return SV_ERR_VALUE;
  if (B == 0) return SV_OK;
  if (!target_logits || !out_tokens || !out_num_accepted || !uniforms) return SV_ERR_NULL;
  if (K > 0 && (!draft_tokens || !drafter_logits || !drafter_desc)) return SV_ERR_NULL;
  if (!workspace || workspace_bytes < verify_workspace_bytes(B, K, V)) return SV_ERR_WORKSPACE;
  const size_t esz = logits_dtype == SV_BF16 ? 2 : 4;
  if (!aligned(target_logits, esz) || !aligned(out_tokens, 4) || !aligned(out_num_accepted, 4) ||
      !aligned(uniforms, 4) || !aligned(workspace, 16) ||
      (draft_tokens && !aligned(draft_tokens, 4)) ||
      (drafter_logits && !aligned(drafter_logits, esz)) ||
      (drafter_rows && !aligned(drafter_rows, 4)) ||
      (drafter_desc && !aligned(drafter_desc, 16)) ||
      (temperatures && !aligned(temperatures, 4)) ||
      (out_draft_target_prob && !aligned(out_draft_target_prob, 4)) ||
      (device_error && !aligned(device_error, 4)))
    return SV_ERR_ALIGN;
  if ((long)B * (K + 1) * verify_splits(B, K, V) > 0x7fffffffL) return SV_ERR_SHAPE;
  VerifyLaunch L;
  L.logits = target_logits;
  L.draft_probs = nullptr;
  L.draft_tokens = draft_tokens;
  L.uniforms = uniforms;
  L.temperature = mixed ? 1.0f : temperature;
  L.B = B; L.K = K; L.V = V;
  L.bf16 = logits_dtype == SV_BF16;
  L.sample = 1;
  L.mixed = mixed ? 1 : 0;
  L.temperatures = temperatures;
  // a valid pointer for K = 0 (nothing is read from it then)
  L.dlogits = drafter_logits ? drafter_logits : target_logits;
  L.d_rows = (long)n_drafter_rows;
  L.drows = drafter_rows;
  L.ddesc = drafter_desc;
  L.vec = (V % 8 == 0) && aligned(target_logits, 16) &&
          (!drafter_logits || aligned(drafter_logits, 16));
  L.out_tokens = out_tokens;
  L.out_num_accepted = out_num_accepted;
  L.out_p_draft = out_draft_target_prob;
  L.workspace = workspace;
  L.device_error = device_error;
  L.early_exit = early_exit ? 1 : 0;
  return launch_verify(L, static_cast<hipStream_t>(stream)) == hipSuccess ? SV_OK : SV_ERR_HIP;
}

// spec_verify_tree / spec_verify_tree_lq, and their _early_exit forms (lazy:
// the walk computes the statistics of the rows it visits).
// temperatures != NULL: per-tree temperatures (spec_verify_tree_mixed*), the
// scalar temperature unused.
sv_status tree_dense(const void* target_logits, int logits_dtype, const float* draft_probs,
                     const int32_t* parents, const int32_t* tokens, const float* uniforms,
                     float temperature, const float* temperatures, int B, int N, int V,
                     int32_t* out_tokens, int32_t* out_path, int32_t* out_num_accepted,
                     void* workspace, size_t workspace_bytes, int32_t* device_error,
                     void* stream, bool lazy) {
  sv_status st = check_verify_shape(B, N, V);
  if (st != SV_OK) return st;
  if (logits_dtype != SV_F32 && logits_dtype != SV_BF16) return SV_ERR_DTYPE;
  const bool mixed = temperatures != nullptr;
  if (!mixed && !(temperature >= 0.0f && isfinite(temperature))) return SV_ERR_VALUE;
  const bool sample = mixed || temperature > 0.0f;
  if (!mixed && sample && !isfinite((float)(1.4426950408889634 / (double)temperature)))
    return SV_ERR_VALUE;
  if (B == 0) return SV_OK;
  if (mixed && !aligned(temperatures, 4)) return SV_ERR_ALIGN;
  if (!target_logits || !out_tokens || !out_path || !out_num_accepted) return SV_ERR_NULL;
  if (N > 0 && (!parents || !tokens)) return SV_ERR_NULL;
  if (sample && (!draft_probs || !uniforms)) return SV_ERR_NULL;
  if (!workspace || workspace_bytes < sv::verify_workspace_bytes(B, N, V)) return SV_ERR_WORKSPACE;
  const size_t esz = logits_dtype == SV_BF16 ? 2 : 4;
  if (!aligned(target_logits, esz) || !aligned(out_tokens, 4) || !aligned(out_path, 4) ||
      !aligned(out_num_accepted, 4) || !aligned(workspace, 16) ||
      (parents && !aligned(parents, 4)) || (tokens && !aligned(tokens, 4)) ||
      (draft_probs && !aligned(draft_probs, 4)) || (uniforms && !aligned(uniforms, 4)) ||
      (device_error && !aligned(device_error, 4)))
    return SV_ERR_ALIGN;
  if ((long)B * (N + 1) * sv::verify_splits(B, N, V) > 0x7fffffffL) return SV_ERR_SHAPE;
  sv::TreeLaunch L;
  L.logits = target_logits;
  L.draft_probs = sample ? draft_probs : nullptr;
  L.dlogits = nullptr;
  L.d_rows = 0;
  L.drows = nullptr;
  L.ddesc = nullptr;
  L.parents = parents;
  L.tokens = tokens;
  L.uniforms = uniforms;
  L.temperature = mixed ? 1.0f : temperature;
  L.temperatures = temperatures;
  L.B = B; L.N = N; L.V = V;
  L.bf16 = logits_dtype == SV_BF16;
  L.vec = (V % 8 == 0) && aligned(target_logits, 16) &&
          (!sample || aligned(draft_probs, 16));
  L.out_tokens = out_tokens;
  L.out_path = out_path;
  L.out_num_accepted = out_num_accepted;
  L.workspace = workspace;
  L.device_error = device_error;
  L.lazy = lazy ? 1 : 0;
  return sv::launch_tree(L, static_cast<hipStream_t>(stream)) == hipSuccess ? SV_OK : SV_ERR_HIP;
}

sv_status tree_lq(const void* target_logits, int logits_dtype, const void* drafter_logits,
                  int64_t n_drafter_rows, const int32_t* drafter_rows,
                  const sv_draft_row* drafter_desc, const int32_t* parents,
                  const int32_t* tokens, const float* uniforms, float temperature, int B, int N,
                  int V, int32_t* out_tokens, int32_t* out_path, int32_t* out_num_accepted,
                  void* workspace, size_t workspace_bytes, int32_t* device_error, void* stream,
                  bool lazy) {
  sv_status st = check_verify_shape(B, N, V);
  if (st != SV_OK) return st;
  if (n_drafter_rows < 0 || n_drafter_rows > 0x7fffffffL) return SV_ERR_SHAPE;
  if (!drafter_rows && n_drafter_rows < (int64_t)B * (N + 1)) return SV_ERR_SHAPE;
  if (logits_dtype != SV_F32 && logits_dtype != SV_BF16) return SV_ERR_DTYPE;
  if (!(temperature > 0.0f && isfinite(temperature) &&
        isfinite((float)(1.4426950408889634 / (double)temperature))))
    return SV_ERR_VALUE;
  if (B == 0) return SV_OK;
  if (!target_logits || !out_tokens || !out_path || !out_num_accepted || !uniforms ||
      !drafter_logits || !drafter_desc)
    return SV_ERR_NULL;
  if (N > 0 && (!parents || !tokens)) return SV_ERR_NULL;
  if (!workspace || workspace_bytes < sv::verify_workspace_bytes(B, N, V)) return SV_ERR_WORKSPACE;
  const size_t esz = logits_dtype == SV_BF16 ? 2 : 4;
  if (!aligned(target_logits, esz) || !aligned(drafter_logits, esz) || !aligned(out_tokens, 4) ||
      !aligned(out_path, 4) || !aligned(out_num_accepted, 4) || !aligned(workspace, 16) ||
      !aligned(uniforms, 4) || !aligned(drafter_desc, 16) ||
      (drafter_rows && !aligned(drafter_rows, 4)) || (parents && !aligned(parents, 4)) ||
      (tokens && !aligned(tokens, 4)) || (device_error && !aligned(device_error, 4)))
    return SV_ERR_ALIGN;
  if ((long)B * (N + 1) * sv::verify_splits(B, N, V) > 0x7fffffffL) return SV_ERR_SHAPE;
  sv::TreeLaunch L;
  L.logits = target_logits;
  L.draft_probs = nullptr;
  L.dlogits = drafter_logits;
  L.d_rows = (long)n_drafter_rows;
  L.drows = drafter_rows;
  L.ddesc = drafter_desc;
  L.parents = parents;
  L.tokens = tokens;
  L.uniforms = uniforms;
  L.temperature = temperature;
  L.B = B; L.N = N; L.V = V;
  L.bf16 = logits_dtype == SV_BF16;
  L.vec = (V % 8 == 0) && aligned(target_logits, 16) && aligned(drafter_logits, 16);
  L.out_tokens = out_tokens;
  L.out_path = out_path;
  L.out_num_accepted = out_num_accepted;
  L.workspace = workspace;
  L.device_error = device_error;
  L.lazy = lazy ? 1 : 0;
  return sv::launch_tree(L, static_cast<hipStream_t>(stream)) == hipSuccess ? SV_OK : SV_ERR_HIP;
}

}  // namespace sv

extern "C" {

SV_API sv_status spec_verify_greedy(const void* target_logits, int logits_dtype,
                                    const int32_t* draft_tokens, int B, int K, int V,
                                    int32_t* out_tokens, int32_t* out_num_accepted,
                                    void* workspace, size_t workspace_bytes,
                                    int32_t* device_error, void* stream) {
  return sv::verify_common(target_logits, logits_dtype, nullptr, draft_tokens, nullptr, 1.0f,
                           nullptr, 0, B, K, V, out_tokens, out_num_accepted, nullptr, workspace,
                           workspace_bytes, device_error, stream, true);
}

SV_API sv_status spec_verify_sample(const void* target_logits, int logits_dtype,
                                    const float* draft_probs, const int32_t* draft_tokens,
                                    const float* uniforms, float temperature, int B, int K, int V,
                                    int32_t* out_tokens, int32_t* out_num_accepted,
                                    float* out_draft_target_prob, void* workspace,
                                    size_t workspace_bytes, int32_t* device_error, void* stream) {
  return sv::verify_common(target_logits, logits_dtype, draft_probs, draft_tokens, uniforms,
                           temperature, nullptr, 1, B, K, V, out_tokens, out_num_accepted,
                           out_draft_target_prob, workspace, workspace_bytes, device_error, stream,
                           true);
}

SV_API sv_status spec_verify_sample_lq(const void* target_logits, int logits_dtype,
                                       const void* drafter_logits, int64_t n_drafter_rows,
                                       const int32_t* drafter_rows,
                                       const sv_draft_row* drafter_desc,
                                       const int32_t* draft_tokens, const float* uniforms,
                                       float temperature, int B, int K, int V,
                                       int32_t* out_tokens, int32_t* out_num_accepted,
                                       float* out_draft_target_prob, void* workspace,
                                       size_t workspace_bytes, int32_t* device_error,
                                       void* stream) {
  return sv::verify_lq(target_logits, logits_dtype, drafter_logits, n_drafter_rows,
                       drafter_rows, drafter_desc, draft_tokens, uniforms, temperature, nullptr,
                       B, K, V, out_tokens, out_num_accepted, out_draft_target_prob,
                       workspace, workspace_bytes, device_error, stream, false);
}

SV_API sv_status spec_verify_mixed_lq(const void* target_logits, int logits_dtype,
                                      const void* drafter_logits, int64_t n_drafter_rows,
                                      const int32_t* drafter_rows,
                                      const sv_draft_row* drafter_desc,
                                      const int32_t* draft_tokens, const float* uniforms,
                                      const float* temperatures, int B, int K, int V,
                                      int32_t* out_tokens, int32_t* out_num_accepted,
                                      float* out_draft_target_prob, void* workspace,
                                      size_t workspace_bytes, int32_t* device_error,
                                      void* stream) {
  if (B > 0 && !temperatures) return SV_ERR_NULL;
  // B = 0 with no temperatures validates as a uniform call and returns OK
  return sv::verify_lq(target_logits, logits_dtype, drafter_logits, n_drafter_rows,
                       drafter_rows, drafter_desc, draft_tokens, uniforms, 1.0f, temperatures,
                       B, K, V, out_tokens, out_num_accepted, out_draft_target_prob, workspace,
                       workspace_bytes, device_error, stream, false);
}

SV_API sv_status spec_verify_sample_lq_early_exit(
    const void* target_logits, int logits_dtype, const void* drafter_logits,
    int64_t n_drafter_rows, const int32_t* drafter_rows, const sv_draft_row* drafter_desc,
    const int32_t* draft_tokens, const float* uniforms, float temperature, int B, int K, int V,
    int32_t* out_tokens, int32_t* out_num_accepted, float* out_draft_target_prob,
    void* workspace, size_t workspace_bytes, int32_t* device_error, void* stream) {
  return sv::verify_lq(target_logits, logits_dtype, drafter_logits, n_drafter_rows,
                       drafter_rows, drafter_desc, draft_tokens, uniforms, temperature, nullptr,
                       B, K, V, out_tokens, out_num_accepted, out_draft_target_prob, workspace,
                       workspace_bytes, device_error, stream, true);
}

SV_API sv_status spec_verify_mixed_lq_early_exit(
    const void* target_logits, int logits_dtype, const void* drafter_logits,
    int64_t n_drafter_rows, const int32_t* drafter_rows, const sv_draft_row* drafter_desc,
    const int32_t* draft_tokens, const float* uniforms, const float* temperatures, int B, int K,
    int V, int32_t* out_tokens, int32_t* out_num_accepted, float* out_draft_target_prob,
    void* workspace, size_t workspace_bytes, int32_t* device_error, void* stream) {
  if (B > 0 && !temperatures) return SV_ERR_NULL;
  return sv::verify_lq(target_logits, logits_dtype, drafter_logits, n_drafter_rows,
                       drafter_rows, drafter_desc, draft_tokens, uniforms, 1.0f, temperatures,
                       B, K, V, out_tokens, out_num_accepted, out_draft_target_prob, workspace,
                       workspace_bytes, device_error, stream, true);
}

SV_API sv_status spec_verify_mixed(const void* target_logits, int logits_dtype,
                                   const float* draft_probs, const int32_t* draft_tokens,
                                   const float* uniforms, const float* temperatures, int B, int K,
                                   int V, int32_t* out_tokens, int32_t* out_num_accepted,
                                   float* out_draft_target_prob, void* workspace,
                                   size_t workspace_bytes, int32_t* device_error, void* stream) {
  return sv::verify_common(target_logits, logits_dtype, draft_probs, draft_tokens, uniforms, 1.0f,
                           temperatures, 2, B, K, V, out_tokens, out_num_accepted,
                           out_draft_target_prob, workspace, workspace_bytes, device_error, stream,
                           true);
}

SV_API sv_status spec_verify_greedy_early_exit(const void* target_logits, int logits_dtype,
                                               const int32_t* draft_tokens, int B, int K, int V,
                                               int32_t* out_tokens, int32_t* out_num_accepted,
                                               void* workspace, size_t workspace_bytes,
                                               int32_t* device_error, void* stream) {
  return sv::verify_common(target_logits, logits_dtype, nullptr, draft_tokens, nullptr, 1.0f,
                           nullptr, 0, B, K, V, out_tokens, out_num_accepted, nullptr, workspace,
                           workspace_bytes, device_error, stream, true, true);
}

SV_API sv_status spec_verify_sample_early_exit(const void* target_logits, int logits_dtype,
                                               const float* draft_probs,
                                               const int32_t* draft_tokens, const float* uniforms,
                                               float temperature, int B, int K, int V,
                                               int32_t* out_tokens, int32_t* out_num_accepted,
                                               float* out_draft_target_prob, void* workspace,
                                               size_t workspace_bytes, int32_t* device_error,
                                               void* stream) {
  return sv::verify_common(target_logits, logits_dtype, draft_probs, draft_tokens, uniforms,
                           temperature, nullptr, 1, B, K, V, out_tokens, out_num_accepted,
                           out_draft_target_prob, workspace, workspace_bytes, device_error, stream,
                           true, true);
}

SV_API sv_status spec_verify_mixed_early_exit(const void* target_logits, int logits_dtype,
                                              const float* draft_probs,
                                              const int32_t* draft_tokens, const float* uniforms,
                                              const float* temperatures, int B, int K, int V,
                                              int32_t* out_tokens, int32_t* out_num_accepted,
                                              float* out_draft_target_prob, void* workspace,
                                              size_t workspace_bytes, int32_t* device_error,
                                              void* stream) {
  return sv::verify_common(target_logits, logits_dtype, draft_probs, draft_tokens, uniforms, 1.0f,
                           temperatures, 2, B, K, V, out_tokens, out_num_accepted,
                           out_draft_target_prob, workspace, workspace_bytes, device_error, stream,
                           true, true);
}

SV_API sv_status peagle_build_draft_batch(const int32_t* verify_out_tokens,
                                          const int32_t* num_accepted, const int32_t* draft_tokens,
                                          const int64_t* start_pos, const int32_t* block_table,
                                          int max_blocks_per_seq, int block_size,
                                          const void* target_hidden, const void* h_shared,
                                          int hidden_dtype, int32_t mask_token_id, int B, int K,
                                          int H, int32_t* out_input_ids, int64_t* out_positions,
                                          int64_t* out_slot_mapping, void* out_hidden,
                                          int32_t* out_sample_rows, int32_t* device_error,
                                          void* stream) {
  if (B < 0 || B > kMaxB || K < 1 || K > SV_MAX_K || H < 1 || block_size < 1 ||
      max_blocks_per_seq < 1)
    return SV_ERR_SHAPE;
  if (hidden_dtype != SV_F32 && hidden_dtype != SV_BF16 && hidden_dtype != SV_F16)
    return SV_ERR_DTYPE;
  if (B == 0) return SV_OK;
  if (!verify_out_tokens || !num_accepted || !draft_tokens || !start_pos || !block_table ||
      !target_hidden || !h_shared || !out_input_ids || !out_positions || !out_slot_mapping ||
      !out_hidden)
    return SV_ERR_NULL;
  const int esz = hidden_dtype == SV_F32 ? 4 : 2;
  if (!aligned(verify_out_tokens, 4) || !aligned(num_accepted, 4) || !aligned(draft_tokens, 4) ||
      !aligned(start_pos, 8) || !aligned(block_table, 4) || !aligned(target_hidden, esz) ||
      !aligned(h_shared, esz) || !aligned(out_input_ids, 4) || !aligned(out_positions, 8) ||
      !aligned(out_slot_mapping, 8) || !aligned(out_hidden, esz) ||
      (out_sample_rows && !aligned(out_sample_rows, 4)) ||
      (device_error && !aligned(device_error, 4)))
    return SV_ERR_ALIGN;
  const long row_bytes = (long)H * esz;
  sv::BuildLaunch L;
  L.verify_out_tokens = verify_out_tokens;
  L.num_accepted = num_accepted;
  L.draft_tokens = draft_tokens;
  L.start_pos = start_pos;
  L.block_table = block_table;
  L.max_blocks = max_blocks_per_seq;
  L.block_size = block_size;
  L.target_hidden = target_hidden;
  L.h_shared = h_shared;
  L.elem_bytes = esz;
  L.vec = row_bytes % 16 == 0 && aligned(target_hidden, 16) && aligned(h_shared, 16) &&
          aligned(out_hidden, 16);
  L.mask_token_id = mask_token_id;
  L.B = B; L.K = K; L.H = H;
  L.out_input_ids = out_input_ids;
  L.out_positions = out_positions;
  L.out_slot_mapping = out_slot_mapping;
  L.out_hidden = out_hidden;
  L.out_sample_rows = out_sample_rows;
  L.device_error = device_error;
  return sv::launch_build(L, static_cast<hipStream_t>(stream)) == hipSuccess ? SV_OK : SV_ERR_HIP;
}

SV_API sv_status spec_draft_sample(const void* drafter_logits, int logits_dtype, int64_t n_rows,
                                   const int32_t* row_index, const float* uniforms,
                                   float temperature, const float* temperatures, int B, int K,
                                   int V, int32_t* out_draft_tokens, float* out_draft_probs,
                                   sv_draft_row* out_row_desc, int32_t* device_error,
                                   void* stream) {
  if (B < 0 || B > kMaxB || K < 1 || K > SV_MAX_K || V < 1 || V > SV_MAX_V || n_rows < 0 ||
      n_rows > 0x7fffffffL)
    return SV_ERR_SHAPE;
  if (!row_index && n_rows < (int64_t)B * K) return SV_ERR_SHAPE;
  if (logits_dtype != SV_F32 && logits_dtype != SV_BF16) return SV_ERR_DTYPE;
  if (!(temperature >= 0.0f && isfinite(temperature))) return SV_ERR_VALUE;
  if (temperature > 0.0f && !isfinite((float)(1.4426950408889634 / (double)temperature)))
    return SV_ERR_VALUE;
  if (B == 0) return SV_OK;
  if (!drafter_logits || !out_draft_tokens) return SV_ERR_NULL;
  if (!uniforms && (temperature != 0.0f || temperatures)) return SV_ERR_NULL;
  const size_t esz = logits_dtype == SV_BF16 ? 2 : 4;
  if (!aligned(drafter_logits, esz) || !aligned(out_draft_tokens, 4) ||
      (row_index && !aligned(row_index, 4)) || (uniforms && !aligned(uniforms, 4)) ||
      (temperatures && !aligned(temperatures, 4)) ||
      (out_draft_probs && !aligned(out_draft_probs, 4)) ||
      (out_row_desc && !aligned(out_row_desc, 16)) || (device_error && !aligned(device_error, 4)))
    return SV_ERR_ALIGN;
  sv::DraftLaunch L;
  L.logits = drafter_logits;
  L.row_index = row_index;
  L.n_rows = (long)n_rows;
  L.uniforms = uniforms;
  L.temperatures = temperatures;
  L.temperature = temperature;
  L.B = B; L.K = K; L.V = V;
  L.bf16 = logits_dtype == SV_BF16;
  L.vec = (V % 8 == 0) && aligned(drafter_logits, 16) &&
          (!out_draft_probs || aligned(out_draft_probs, 16));
  L.out_tokens = out_draft_tokens;
  L.out_probs = out_draft_probs;
  L.out_desc = out_row_desc;
  L.device_error = device_error;
  return sv::launch_draft(L, static_cast<hipStream_t>(stream)) == hipSuccess ? SV_OK : SV_ERR_HIP;
}

SV_API sv_status spec_verify_tree(const void* target_logits, int logits_dtype,
                                  const float* draft_probs, const int32_t* parents,
                                  const int32_t* tokens, const float* uniforms, float temperature,
                                  int B, int N, int V, int32_t* out_tokens, int32_t* out_path,
                                  int32_t* out_num_accepted, void* workspace,
                                  size_t workspace_bytes, int32_t* device_error, void* stream) {
  return sv::tree_dense(target_logits, logits_dtype, draft_probs, parents, tokens, uniforms,
                        temperature, nullptr, B, N, V, out_tokens, out_path, out_num_accepted,
                        workspace, workspace_bytes, device_error, stream, false);
}

SV_API sv_status spec_verify_tree_early_exit(const void* target_logits, int logits_dtype,
                                             const float* draft_probs, const int32_t* parents,
                                             const int32_t* tokens, const float* uniforms,
                                             float temperature, int B, int N, int V,
                                             int32_t* out_tokens, int32_t* out_path,
                                             int32_t* out_num_accepted, void* workspace,
                                             size_t workspace_bytes, int32_t* device_error,
                                             void* stream) {
  return sv::tree_dense(target_logits, logits_dtype, draft_probs, parents, tokens, uniforms,
                        temperature, nullptr, B, N, V, out_tokens, out_path, out_num_accepted,
                        workspace, workspace_bytes, device_error, stream, true);
}

SV_API sv_status spec_verify_tree_mixed(const void* target_logits, int logits_dtype,
                                        const float* draft_probs, const int32_t* parents,
                                        const int32_t* tokens, const float* uniforms,
                                        const float* temperatures, int B, int N, int V,
                                        int32_t* out_tokens, int32_t* out_path,
                                        int32_t* out_num_accepted, void* workspace,
                                        size_t workspace_bytes, int32_t* device_error,
                                        void* stream) {
  if (B > 0 && !temperatures) return SV_ERR_NULL;
  return sv::tree_dense(target_logits, logits_dtype, draft_probs, parents, tokens, uniforms,
                        1.0f, temperatures, B, N, V, out_tokens, out_path, out_num_accepted,
                        workspace, workspace_bytes, device_error, stream, false);
}

SV_API sv_status spec_verify_tree_mixed_early_exit(
    const void* target_logits, int logits_dtype, const float* draft_probs,
    const int32_t* parents, const int32_t* tokens, const float* uniforms,
    const float* temperatures, int B, int N, int V, int32_t* out_tokens, int32_t* out_path,
    int32_t* out_num_accepted, void* workspace, size_t workspace_bytes, int32_t* device_error,
    void* stream) {
  if (B > 0 && !temperatures) return SV_ERR_NULL;
  return sv::tree_dense(target_logits, logits_dtype, draft_probs, parents, tokens, uniforms,
                        1.0f, temperatures, B, N, V, out_tokens, out_path, out_num_accepted,
                        workspace, workspace_bytes, device_error, stream, true);
}

SV_API sv_status spec_verify_tree_lq(const void* target_logits, int logits_dtype,
                                     const void* drafter_logits, int64_t n_drafter_rows,
                                     const int32_t* drafter_rows,
                                     const sv_draft_row* drafter_desc, const int32_t* parents,
                                     const int32_t* tokens, const float* uniforms,
                                     float temperature, int B, int N, int V,
                                     int32_t* out_tokens, int32_t* out_path,
                                     int32_t* out_num_accepted, void* workspace,
                                     size_t workspace_bytes, int32_t* device_error,
                                     void* stream) {
  return sv::tree_lq(target_logits, logits_dtype, drafter_logits, n_drafter_rows, drafter_rows,
                     drafter_desc, parents, tokens, uniforms, temperature, B, N, V, out_tokens,
                     out_path, out_num_accepted, workspace, workspace_bytes, device_error, stream,
                     false);
}

SV_API sv_status spec_verify_tree_lq_early_exit(
    const void* target_logits, int logits_dtype, const void* drafter_logits,
    int64_t n_drafter_rows, const int32_t* drafter_rows, const sv_draft_row* drafter_desc,
    const int32_t* parents, const int32_t* tokens, const float* uniforms, float temperature,
    int B, int N, int V, int32_t* out_tokens, int32_t* out_path, int32_t* out_num_accepted,
    void* workspace, size_t workspace_bytes, int32_t* device_error, void* stream) {
  return sv::tree_lq(target_logits, logits_dtype, drafter_logits, n_drafter_rows, drafter_rows,
                     drafter_desc, parents, tokens, uniforms, temperature, B, N, V, out_tokens,
                     out_path, out_num_accepted, workspace, workspace_bytes, device_error, stream,
                     true);
}

SV_API size_t spec_accept_metrics_words(int K) {
  if (K < 1 || K > SV_MAX_K) return 0;
  return (size_t)SV_METRICS_HIST + K + 1;
}

SV_API sv_status spec_accept_metrics(const int32_t* num_accepted, int B, int K, uint64_t* metrics,
                                     int32_t* device_error, void* stream) {
  if (B < 0 || B > kMaxB || K < 1 || K > SV_MAX_K) return SV_ERR_SHAPE;
  if (B == 0) return SV_OK;
  if (!num_accepted || !metrics) return SV_ERR_NULL;
  if (!aligned(num_accepted, 4) || !aligned(metrics, 8) ||
      (device_error && !aligned(device_error, 4)))
    return SV_ERR_ALIGN;
  return sv::launch_metrics(num_accepted, B, K, metrics, device_error,
                            static_cast<hipStream_t>(stream)) == hipSuccess ? SV_OK : SV_ERR_HIP;
}

}  // extern "C"

// ---------------------------------------------------------------- step graphs
struct sv_step_graph {
  hipGraph_t graph;
  hipGraphExec_t exec;
  hipStream_t capture_stream;
};

namespace {

// The step's verify call, on the dense q or on the drafter logits, full or
// early exit (each call validates its own arguments).
sv_status enqueue_verify(const sv_step_desc* d, hipStream_t s) {
  const bool ee = d->early_exit != 0;
  if (d->drafter_logits) {
    auto* lq = d->mode == SV_STEP_SAMPLE
        ? (ee ? spec_verify_sample_lq_early_exit : spec_verify_sample_lq) : nullptr;
    if (lq)
      return lq(d->target_logits, d->logits_dtype, d->drafter_logits, d->n_drafter_rows,
                d->drafter_rows, d->drafter_desc, d->draft_tokens, d->uniforms, d->temperature,
                d->B, d->K, d->V, d->out_tokens, d->out_num_accepted, d->out_draft_target_prob,
                d->workspace, d->workspace_bytes, d->device_error, s);
    auto* mlq = ee ? spec_verify_mixed_lq_early_exit : spec_verify_mixed_lq;
    return mlq(d->target_logits, d->logits_dtype, d->drafter_logits, d->n_drafter_rows,
               d->drafter_rows, d->drafter_desc, d->draft_tokens, d->uniforms, d->temperatures,
               d->B, d->K, d->V, d->out_tokens, d->out_num_accepted, d->out_draft_target_prob,
               d->workspace, d->workspace_bytes, d->device_error, s);
  }
  switch (d->mode) {
    case SV_STEP_GREEDY:
      return (ee ? spec_verify_greedy_early_exit : spec_verify_greedy)(
          d->target_logits, d->logits_dtype, d->draft_tokens, d->B, d->K, d->V, d->out_tokens,
          d->out_num_accepted, d->workspace, d->workspace_bytes, d->device_error, s);
    case SV_STEP_SAMPLE:
      return (ee ? spec_verify_sample_early_exit : spec_verify_sample)(
          d->target_logits, d->logits_dtype, d->draft_probs, d->draft_tokens, d->uniforms,
          d->temperature, d->B, d->K, d->V, d->out_tokens, d->out_num_accepted,
          d->out_draft_target_prob, d->workspace, d->workspace_bytes, d->device_error, s);
    default:
      return (ee ? spec_verify_mixed_early_exit : spec_verify_mixed)(
          d->target_logits, d->logits_dtype, d->draft_probs, d->draft_tokens, d->uniforms,
          d->temperatures, d->B, d->K, d->V, d->out_tokens, d->out_num_accepted,
          d->out_draft_target_prob, d->workspace, d->workspace_bytes, d->device_error, s);
  }
}

// The calls of one step, in order, on stream s (each validates its arguments).
sv_status enqueue_step(const sv_step_desc* d, hipStream_t s) {
  sv_status st = enqueue_verify(d, s);
  if (st != SV_OK) return st;
  if (d->out_hidden) {
    st = peagle_build_draft_batch(d->out_tokens, d->out_num_accepted, d->draft_tokens,
                                  d->start_pos, d->block_table, d->max_blocks_per_seq,
                                  d->block_size, d->target_hidden, d->h_shared, d->hidden_dtype,
                                  d->mask_token_id, d->B, d->K, d->H, d->out_input_ids,
                                  d->out_positions, d->out_slot_mapping, d->out_hidden,
                                  d->out_sample_rows, d->device_error, s);
    if (st != SV_OK) return st;
  }
  if (d->metrics)
    st = spec_accept_metrics(d->out_num_accepted, d->B, d->K, d->metrics, d->device_error, s);
  return st;
}

}  // namespace

extern "C" {

SV_API sv_status sv_step_graph_create(const sv_step_desc* desc, sv_step_graph** out) {
  if (!desc || !out) return SV_ERR_NULL;
  *out = nullptr;
  if (desc->mode != SV_STEP_GREEDY && desc->mode != SV_STEP_SAMPLE && desc->mode != SV_STEP_MIXED)
    return SV_ERR_VALUE;
  // q from the drafter logits replaces the dense q, and only for sampling
  if (desc->drafter_logits && (desc->mode == SV_STEP_GREEDY || desc->draft_probs))
    return SV_ERR_VALUE;
  if (desc->metrics && (desc->K < 1 || desc->K > SV_MAX_K)) return SV_ERR_SHAPE;
  hipStream_t s = nullptr;
  if (hipStreamCreateWithFlags(&s, hipStreamNonBlocking) != hipSuccess) return SV_ERR_HIP;
  sv::TracePause pause;
  if (hipStreamBeginCapture(s, hipStreamCaptureModeThreadLocal) != hipSuccess) {
    (void)hipStreamDestroy(s);
    return SV_ERR_HIP;
  }
  const sv_status st = enqueue_step(desc, s);
  hipGraph_t g = nullptr;
  const hipError_t e = hipStreamEndCapture(s, &g);
  hipGraphExec_t x = nullptr;
  if (st != SV_OK || e != hipSuccess || !g ||
      hipGraphInstantiate(&x, g, nullptr, nullptr, 0) != hipSuccess) {
    if (g) (void)hipGraphDestroy(g);
    (void)hipStreamDestroy(s);
    return st != SV_OK ? st : SV_ERR_HIP;
  }
  *out = new sv_step_graph{g, x, s};
  return SV_OK;
}

SV_API sv_status sv_step_graph_launch(sv_step_graph* graph, void* stream) {
  if (!graph) return SV_ERR_NULL;
  return hipGraphLaunch(graph->exec, static_cast<hipStream_t>(stream)) == hipSuccess ? SV_OK
                                                                                     : SV_ERR_HIP;
}

SV_API void sv_step_graph_destroy(sv_step_graph* graph) {
  if (!graph) return;
  (void)hipGraphExecDestroy(graph->exec);
  (void)hipGraphDestroy(graph->graph);
  (void)hipStreamDestroy(graph->capture_stream);
  delete graph;
}

}  // extern "C"
