// spec_verify_sample_noalloc: the sampled verify with its workspace taken
// from a fixed array in device memory instead of a caller's buffer, for
// callers that cannot allocate device memory.
//
// `scratch` is a file-scope __device__ array: every GPU the library runs on
// holds its own copy, at its own address, until the process ends.  In host
// code the name `scratch` is only a host-side stand-in, so the host never
// passes it to a kernel: it looks the device address up once per device with
// hipGetSymbolAddress and passes that address instead.  The verify kernels
// leave their workspace all zero when they finish, so the array stays zero
// between calls; it is cleared once, by a fill kernel enqueued on the first
// call's stream, before the first use on each device.
#include <mutex>

#include "sv_internal.h"

namespace {

constexpr size_t kScratchBytes = SV_NOALLOC_SCRATCH_BYTES;
constexpr int kMaxDevices = 64;

__device__ __align__(256) unsigned char scratch[kScratchBytes];

__global__ __launch_bounds__(256) void clear_scratch(uint4* p, size_t n) {
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n;
       i += (size_t)gridDim.x * blockDim.x)
    p[i] = make_uint4(0u, 0u, 0u, 0u);
}

std::mutex g_mutex;
void* g_scratch[kMaxDevices];   // device address of `scratch` on device i, once looked up

// This device's scratch address; the first call on a device looks it up and
// enqueues the fill kernel that clears the array on `stream`.
sv_status device_scratch(hipStream_t stream, void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return SV_ERR_HIP;
  std::lock_guard<std::mutex> lock(g_mutex);
  if (!g_scratch[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return SV_ERR_HIP;
    hipLaunchKernelGGL(clear_scratch, dim3(256), dim3(256), 0, stream,
                       static_cast<uint4*>(p), kScratchBytes / sizeof(uint4));
    if (hipGetLastError() != hipSuccess) return SV_ERR_HIP;
    g_scratch[dev] = p;
  }
  *out = g_scratch[dev];
  return SV_OK;
}

}  // namespace

extern "C" {

SV_API size_t spec_verify_noalloc_scratch_bytes(void) { return kScratchBytes; }

SV_API sv_status spec_verify_sample_noalloc(const void* target_logits, int logits_dtype,
                                            const float* draft_probs,
                                            const int32_t* draft_tokens, const float* uniforms,
                                            float temperature, int B, int K, int V,
                                            int32_t* out_tokens, int32_t* out_num_accepted,
                                            float* out_draft_target_prob,
                                            int32_t* device_error, void* stream) {
  // every argument is checked before anything is enqueued
  sv_status st = sv::verify_common(target_logits, logits_dtype, draft_probs, draft_tokens,
                                   uniforms, temperature, nullptr, 1, B, K, V, out_tokens,
                                   out_num_accepted, out_draft_target_prob, nullptr, 0,
                                   device_error, stream, false);
  if (st != SV_OK || B == 0) return st;
  if (sv::verify_workspace_bytes(B, K, V) > kScratchBytes) return SV_ERR_SCRATCH;
  void* ws = nullptr;
  const hipStream_t s = static_cast<hipStream_t>(stream);
  st = device_scratch(s, &ws);
  if (st != SV_OK) return st;
  return sv::verify_common(target_logits, logits_dtype, draft_probs, draft_tokens, uniforms,
                           temperature, nullptr, 1, B, K, V, out_tokens, out_num_accepted,
                           out_draft_target_prob, ws, kScratchBytes, device_error, stream, true);
}

}  // extern "C"
