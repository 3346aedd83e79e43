// The HBM read rate a plain streaming kernel reaches on this GPU: the
// practical ceiling the row-statistics kernels are compared with, beside the
// nominal 8 TB/s.  Not part of the verify library: bench.py loads it from its
// own shared object to time it over the same device buffer as the workload.
//
// Each of kBlocks workgroups of 256 threads reads one contiguous chunk of
// 16-byte vectors, kInFlight loads per thread before any is used, and folds
// them into a value that is kept live without being stored.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
constexpr int kThreads = 256;
constexpr int kInFlight = 8;
constexpr int kBlocks = 8192;

template <bool NT>
__global__ __launch_bounds__(kThreads) void stream_read(const u32x4* x, long nvec, long per_block) {
  const long lo = (long)blockIdx.x * per_block;
  const long hi = lo + per_block < nvec ? lo + per_block : nvec;
  unsigned acc = 0;
  long i = lo + threadIdx.x;
  for (; i + (long)(kInFlight - 1) * kThreads < hi; i += (long)kInFlight * kThreads) {
    u32x4 v[kInFlight];
#pragma unroll
    for (int u = 0; u < kInFlight; ++u)
      v[u] = NT ? __builtin_nontemporal_load(x + i + u * kThreads) : x[i + u * kThreads];
#pragma unroll
    for (int u = 0; u < kInFlight; ++u) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
  }
  for (; i < hi; i += kThreads) {
    const u32x4 v = NT ? __builtin_nontemporal_load(x + i) : x[i];
    acc ^= v.x ^ v.y ^ v.z ^ v.w;
  }
  asm volatile("" : : "v"(acc));        // the loads must not be dropped
}

}  // namespace

// Read `bytes` bytes at device address `data` once (bytes > 0, a multiple of
// 16, data 16-byte aligned), with non-temporal loads when non_temporal != 0,
// on `stream` (a hipStream_t; NULL = the null stream).  Returns 0 when the
// launch was enqueued, 1 for invalid arguments (nothing launched), 2 when the
// launch failed.
extern "C" __attribute__((visibility("default"))) int svc_stream_read(const void* data,
                                                                      int64_t bytes,
                                                                      int non_temporal,
                                                                      void* stream) {
  if (!data || bytes <= 0 || bytes % 16 || reinterpret_cast<uintptr_t>(data) % 16) return 1;
  const long nvec = bytes / 16;
  const long per = (nvec + kBlocks - 1) / kBlocks;
  const long blocks = (nvec + per - 1) / per;
  const u32x4* x = static_cast<const u32x4*>(data);
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (non_temporal)
    hipLaunchKernelGGL(stream_read<true>, dim3((unsigned)blocks), dim3(kThreads), 0, s, x, nvec, per);
  else
    hipLaunchKernelGGL(stream_read<false>, dim3((unsigned)blocks), dim3(kThreads), 0, s, x, nvec, per);
  return hipGetLastError() == hipSuccess ? 0 : 2;
}
