// Bandwidth ceilings of plain kernels on this GPU, which the library's
// kernels are compared with beside the nominal 8 TB/s.  Not part of the
// verify library: bench.py loads them from their own shared object and times
// them over the same device buffers as the workload.
//
//   stream_read  the HBM read rate: each of kBlocks workgroups of 256 threads
//                reads one contiguous chunk of 16-byte vectors, kInFlight
//                loads per thread before any is used, folded into a value
//                that is kept live without being stored.
//   rows_to_f32  the bytes of drafter sampling with q and no arithmetic: one
//                512-thread workgroup per output row reads a gathered bf16
//                row and writes it back as fp32 (16-byte loads, two 16-byte
//                stores per lane and step).
//   write_rows   writes alone: one 512-thread workgroup per fp32 row,
//                16-byte stores.
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

constexpr int kRowThreads = 512;
typedef float f32x4 __attribute__((ext_vector_type(4)));

template <bool NT>
__device__ __forceinline__ void store4(f32x4* p, f32x4 v) {
  if (NT) __builtin_nontemporal_store(v, p); else *p = v;
}

template <bool NT>
__global__ __launch_bounds__(kRowThreads) void rows_to_f32(const uint16_t* src,
                                                           const int32_t* row_index,
                                                           long n_src_rows, float* out, int V) {
  const long r = blockIdx.x;
  const long ri = row_index[r];
  if (ri < 0 || ri >= n_src_rows) return;
  const u32x4* s = reinterpret_cast<const u32x4*>(src + ri * V);
  f32x4* d = reinterpret_cast<f32x4*>(out + r * V);
  const int nocts = V / 8;
  for (int o = threadIdx.x; o < nocts; o += kRowThreads) {
    const u32x4 w = __builtin_nontemporal_load(s + o);
    store4<NT>(d + 2 * o, f32x4{__uint_as_float(w.x << 16), __uint_as_float(w.x & 0xffff0000u),
                                __uint_as_float(w.y << 16), __uint_as_float(w.y & 0xffff0000u)});
    store4<NT>(d + 2 * o + 1, f32x4{__uint_as_float(w.z << 16), __uint_as_float(w.z & 0xffff0000u),
                                    __uint_as_float(w.w << 16), __uint_as_float(w.w & 0xffff0000u)});
  }
}

template <bool NT>
__global__ __launch_bounds__(kRowThreads) void write_rows(float* out, int V) {
  f32x4* d = reinterpret_cast<f32x4*>(out + (long)blockIdx.x * V);
  const f32x4 v{0.f, 0.25f, 0.5f, 0.75f};
  const int nquads = V / 4;
  for (int i = threadIdx.x; i < nquads; i += kRowThreads) store4<NT>(d + i, v);
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

// Rows r < n_rows of `out` ([n_rows][V] fp32) = the bf16 rows row_index[r] of
// `src` ([n_src_rows][V] bf16) converted to fp32 (a row index outside
// [0, n_src_rows) leaves that output row unwritten); non-temporal stores when
// non_temporal != 0.  V a multiple of 8, src and out 16-byte aligned.
// Returns 0 when enqueued, 1 for invalid arguments, 2 when the launch failed.
extern "C" __attribute__((visibility("default"))) int svc_rows_to_f32(
    const void* src, const int32_t* row_index, int64_t n_src_rows, float* out, int64_t n_rows,
    int V, int non_temporal, void* stream) {
  if (!src || !row_index || !out || n_rows <= 0 || n_rows > 0x7fffffffL || n_src_rows <= 0 ||
      V <= 0 || V % 8 || reinterpret_cast<uintptr_t>(src) % 16 ||
      reinterpret_cast<uintptr_t>(out) % 16 || reinterpret_cast<uintptr_t>(row_index) % 4)
    return 1;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const uint16_t* z = static_cast<const uint16_t*>(src);
  if (non_temporal)
    hipLaunchKernelGGL(rows_to_f32<true>, dim3((unsigned)n_rows), dim3(kRowThreads), 0, s, z,
                       row_index, (long)n_src_rows, out, V);
  else
    hipLaunchKernelGGL(rows_to_f32<false>, dim3((unsigned)n_rows), dim3(kRowThreads), 0, s, z,
                       row_index, (long)n_src_rows, out, V);
  return hipGetLastError() == hipSuccess ? 0 : 2;
}

// Fill `out` ([n_rows][V] fp32) with a constant pattern, one workgroup per
// row; non-temporal stores when non_temporal != 0.  V a multiple of 4, out
// 16-byte aligned.  Returns as svc_rows_to_f32.
extern "C" __attribute__((visibility("default"))) int svc_write_rows(float* out, int64_t n_rows,
                                                                     int V, int non_temporal,
                                                                     void* stream) {
  if (!out || n_rows <= 0 || n_rows > 0x7fffffffL || V <= 0 || V % 4 ||
      reinterpret_cast<uintptr_t>(out) % 16)
    return 1;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (non_temporal)
    hipLaunchKernelGGL(write_rows<true>, dim3((unsigned)n_rows), dim3(kRowThreads), 0, s, out, V);
  else
    hipLaunchKernelGGL(write_rows<false>, dim3((unsigned)n_rows), dim3(kRowThreads), 0, s, out, V);
  return hipGetLastError() == hipSuccess ? 0 : 2;
}
