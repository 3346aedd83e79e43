// On-device acceptance metrics: integer counters accumulated across verify
// calls, so a serving loop can report acceptance without a host round trip
// per step.  The quantities are those the pages watch: the acceptance length
// (P-EAGLE / TorchSpec blog summary, section 监控与调优建议: mean accepted
// drafts per speculation round) and the acceptance rate and accepted tokens
// per step of the decode log ("Project 14", section 使用它).
//
// Each workgroup builds a histogram of its accept counts in LDS, then adds
// the histogram and the totals derived from it to the global counters with
// 64-bit integer atomics (exact, so the totals do not depend on the order).
#include "sv_device.h"
#include "sv_internal.h"

namespace sv {

constexpr int kMetricsThreads = 256;
constexpr int kMaxMetricsBlocks = 256;

struct MetricsArgs {
  const int32_t* num_accepted;
  int B, K;
  unsigned long long* metrics;   // [SV_METRICS_HIST + K + 1]
  int32_t* device_error;
};

__device__ __forceinline__ unsigned long long wave_sum_u64(unsigned long long x) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) x += __shfl_xor(x, off);
  return x;
}

__global__ __launch_bounds__(kMetricsThreads) void accept_metrics_kernel(MetricsArgs A) {
  __shared__ unsigned int hist[SV_MAX_K + 1];
  const int t = threadIdx.x, K = A.K;
  for (int i = t; i <= K; i += kMetricsThreads) hist[i] = 0;
  __syncthreads();
  for (long b = (long)blockIdx.x * kMetricsThreads + t; b < A.B;
       b += (long)gridDim.x * kMetricsThreads) {
    int a = A.num_accepted[b];
    if (a < 0 || a > K) {
      flag_error(A.device_error, SV_DEVERR_ACCEPT_COUNT);
      a = a < 0 ? 0 : K;
    }
    atomicAdd(&hist[a], 1u);
  }
  __syncthreads();
  if (t <= K && hist[t]) atomicAdd(&A.metrics[SV_METRICS_HIST + t], (unsigned long long)hist[t]);
  if (t < kWave) {
    // rounds and accepted drafts of this workgroup, from its histogram
    unsigned long long rounds = 0, accepted = 0;
    for (int i = t; i <= K; i += kWave) {
      rounds += hist[i];
      accepted += (unsigned long long)i * hist[i];
    }
    rounds = wave_sum_u64(rounds);
    accepted = wave_sum_u64(accepted);
    if (t == 0 && rounds) {
      atomicAdd(&A.metrics[SV_METRICS_ROUNDS], rounds);
      atomicAdd(&A.metrics[SV_METRICS_PROPOSED], rounds * (unsigned long long)K);
      atomicAdd(&A.metrics[SV_METRICS_ACCEPTED], accepted);
      atomicAdd(&A.metrics[SV_METRICS_EMITTED], accepted + rounds);
    }
    if (t == 0 && blockIdx.x == 0) atomicAdd(&A.metrics[SV_METRICS_STEPS], 1ull);
  }
}

hipError_t launch_metrics(const int32_t* num_accepted, int B, int K, uint64_t* metrics,
                          int32_t* device_error, hipStream_t stream) {
  MetricsArgs A{num_accepted, B, K, reinterpret_cast<unsigned long long*>(metrics), device_error};
  long blocks = ((long)B + kMetricsThreads - 1) / kMetricsThreads;
  if (blocks < 1) blocks = 1;
  if (blocks > kMaxMetricsBlocks) blocks = kMaxMetricsBlocks;
  trace_before(stream, SV_KERNEL_ACCEPT_METRICS);
  hipLaunchKernelGGL(accept_metrics_kernel, dim3((unsigned)blocks), dim3(kMetricsThreads), 0,
                     stream, A);
  const hipError_t err = hipGetLastError();
  trace_after(stream, SV_KERNEL_ACCEPT_METRICS);
  return err;
}

}  // namespace sv
