// P-EAGLE parallel-draft batch construction for gfx950.
//
// Per sequence (a accepted drafts, K drafts, new token c, verify slot 0 at
// position L) the drafter batch has 2K rows:
//   0..a-1 accepted, a NTP, a+1..a+K-1 MASK, a+K..2K-1 rejected (slot -1).
// Every target hidden row h[i] (i = 0..K) lands in exactly one output row:
// row i when i <= a (accepted or NTP), row i+K-1 when i > a (rejected), and
// in every case at position L+i.  h_shared fills the K-1 MASK rows.
//
// One wavefront per source row (b, i), four per workgroup.  The wave starts
// loading h[i] (and h_shared when 1 <= i <= K-1) before it knows a, so the
// hidden-row loads overlap the metadata loads; then it stores h[i] into its
// output row and, for 1 <= i <= K-1, h_shared into MASK row a+i, and lanes 0
// and 1 write those rows' token id, position and KV slot.  Fusing the
// metadata rebuild with the hidden copy is one launch instead of the separate
// copy / scatter / insert / pad / mask / remap operations and the dedicated
// broadcast copy that the P-EAGLE / TorchSpec blog summary describes (section
// TorchSpec 集成与工程优化).
//
// The hidden rows are written with non-temporal stores: the drafter reads
// them in a later launch, and ordinary stores leave ~60 MB of dirty lines in
// the memory-side cache that the next verify step's scattered row reads then
// evict, which was measured to slow that step's residual-draw kernel by ~18%.
#include "sv_device.h"
#include "sv_internal.h"

namespace sv {

constexpr int kBuildThreads = 256;
constexpr int kWavesPerBlock = kBuildThreads / kWave;
constexpr int kCopyUnroll = 8;          // 16-byte vectors per lane per step

struct BuildArgs {
  BuildLaunch L;
  long units;   // B * (K+1) source rows
};

__device__ __forceinline__ int64_t kv_slot(const BuildLaunch& L, int b, int64_t pos) {
  const int64_t blk = pos / L.block_size;
  const bool ok = pos >= 0 && blk < L.max_blocks;
  const int32_t page = ok ? L.block_table[(long)b * L.max_blocks + blk] : -1;
  if (ok && page >= 0) return (int64_t)page * L.block_size + pos % L.block_size;
  flag_error(L.device_error, SV_DEVERR_BLOCK_TABLE);
  return SV_PADDING_SLOT_ID;
}

__global__ __launch_bounds__(kBuildThreads) void build_kernel(BuildArgs A) {
  const BuildLaunch& L = A.L;
  const long unit = (long)blockIdx.x * kWavesPerBlock + threadIdx.x / kWave;
  if (unit >= A.units) return;
  const int K = L.K;
  const int b = (int)(unit / (K + 1));
  const int i = (int)(unit % (K + 1));
  const int l = lane_id();
  const bool mask_row = i >= 1 && i <= K - 1;   // this wave also writes MASK row a+i
  const long row_bytes = (long)L.H * L.elem_bytes;
  const char* src = static_cast<const char*>(L.target_hidden) + unit * row_bytes;
  const char* hs = static_cast<const char*>(L.h_shared);
  char* out = static_cast<char*>(L.out_hidden);
  const long base_row = (long)b * 2 * K;

  if (L.vec) {
    const long nvec = row_bytes / 16;
    const u32x4* s = reinterpret_cast<const u32x4*>(src);
    const u32x4* h = reinterpret_cast<const u32x4*>(hs);
    // first step's loads go out before the accept count is known
    u32x4 vs[kCopyUnroll], vh[kCopyUnroll];
#pragma unroll
    for (int j = 0; j < kCopyUnroll; ++j) {
      const long e = l + (long)j * kWave;
      if (e < nvec) {
        vs[j] = s[e];
        if (mask_row) vh[j] = h[e];
      }
    }
    int a = L.num_accepted[b];
    if (a < 0 || a > K) {
      if (l == 0 && i == 0) flag_error(L.device_error, SV_DEVERR_ACCEPT_COUNT);
      a = a < 0 ? 0 : K;
    }
    const long dst_row = base_row + (i <= a ? i : i + K - 1);
    u32x4* d = reinterpret_cast<u32x4*>(out + dst_row * row_bytes);
    u32x4* dm = reinterpret_cast<u32x4*>(out + (base_row + a + i) * row_bytes);
    for (long e0 = 0;; e0 += (long)kCopyUnroll * kWave) {
#pragma unroll
      for (int j = 0; j < kCopyUnroll; ++j) {
        const long e = e0 + l + (long)j * kWave;
        if (e < nvec) {
          __builtin_nontemporal_store(vs[j], d + e);
          if (mask_row) __builtin_nontemporal_store(vh[j], dm + e);
        }
      }
      const long next = e0 + (long)kCopyUnroll * kWave;
      if (next >= nvec) break;
#pragma unroll
      for (int j = 0; j < kCopyUnroll; ++j) {
        const long e = next + l + (long)j * kWave;
        if (e < nvec) {
          vs[j] = s[e];
          if (mask_row) vh[j] = h[e];
        }
      }
    }
    if (l < 2) {
      // lanes 0 / 1: metadata of the source row / of the MASK row
      const int64_t Lpos = L.start_pos[b];
      if (l == 0) {
        int token;
        int64_t slot;
        if (i <= a) {
          token = L.verify_out_tokens[(long)b * (K + 1) + i];
          slot = kv_slot(L, b, Lpos + i);
        } else {
          token = L.draft_tokens[(long)b * K + i - 1];
          slot = SV_PADDING_SLOT_ID;
        }
        L.out_input_ids[dst_row] = token;
        L.out_positions[dst_row] = Lpos + i;
        L.out_slot_mapping[dst_row] = slot;
      } else if (mask_row) {
        const long mrow = base_row + a + i;
        L.out_input_ids[mrow] = L.mask_token_id;
        L.out_positions[mrow] = Lpos + a + i;
        L.out_slot_mapping[mrow] = kv_slot(L, b, Lpos + a + i);
      }
    }
    if (L.out_sample_rows && i == 0 && l < K)
      L.out_sample_rows[(long)b * K + l] = (int32_t)(base_row + a + l);
    return;
  }

  // element-wise path (rows not a multiple of 16 bytes, or unaligned)
  int a = L.num_accepted[b];
  if (a < 0 || a > K) {
    if (l == 0 && i == 0) flag_error(L.device_error, SV_DEVERR_ACCEPT_COUNT);
    a = a < 0 ? 0 : K;
  }
  const long dst_row = base_row + (i <= a ? i : i + K - 1);
  const long mrow = base_row + a + i;
  if (L.elem_bytes == 4) {
    const uint32_t* s = reinterpret_cast<const uint32_t*>(src);
    const uint32_t* h = reinterpret_cast<const uint32_t*>(hs);
    uint32_t* d = reinterpret_cast<uint32_t*>(out + dst_row * row_bytes);
    uint32_t* dm = reinterpret_cast<uint32_t*>(out + mrow * row_bytes);
    for (long e = l; e < L.H; e += kWave) {
      __builtin_nontemporal_store(s[e], d + e);
      if (mask_row) __builtin_nontemporal_store(h[e], dm + e);
    }
  } else {
    const uint16_t* s = reinterpret_cast<const uint16_t*>(src);
    const uint16_t* h = reinterpret_cast<const uint16_t*>(hs);
    uint16_t* d = reinterpret_cast<uint16_t*>(out + dst_row * row_bytes);
    uint16_t* dm = reinterpret_cast<uint16_t*>(out + mrow * row_bytes);
    for (long e = l; e < L.H; e += kWave) {
      __builtin_nontemporal_store(s[e], d + e);
      if (mask_row) __builtin_nontemporal_store(h[e], dm + e);
    }
  }
  const int64_t Lpos = L.start_pos[b];
  if (l == 0) {
    int token;
    int64_t slot;
    if (i <= a) {
      token = L.verify_out_tokens[(long)b * (K + 1) + i];
      slot = kv_slot(L, b, Lpos + i);
    } else {
      token = L.draft_tokens[(long)b * K + i - 1];
      slot = SV_PADDING_SLOT_ID;
    }
    L.out_input_ids[dst_row] = token;
    L.out_positions[dst_row] = Lpos + i;
    L.out_slot_mapping[dst_row] = slot;
  } else if (l == 1 && mask_row) {
    L.out_input_ids[mrow] = L.mask_token_id;
    L.out_positions[mrow] = Lpos + a + i;
    L.out_slot_mapping[mrow] = kv_slot(L, b, Lpos + a + i);
  }
  if (L.out_sample_rows && i == 0 && l < K)
    L.out_sample_rows[(long)b * K + l] = (int32_t)(base_row + a + l);
}

hipError_t launch_build(const BuildLaunch& L, hipStream_t stream) {
  BuildArgs A;
  A.L = L;
  A.units = (long)L.B * (L.K + 1);
  const unsigned blocks = (unsigned)((A.units + kWavesPerBlock - 1) / kWavesPerBlock);
  trace_before(stream, SV_KERNEL_PEAGLE_BUILD);
  hipLaunchKernelGGL(build_kernel, dim3(blocks), dim3(kBuildThreads), 0, stream, A);
  const hipError_t err = hipGetLastError();
  trace_after(stream, SV_KERNEL_PEAGLE_BUILD);
  return err;
}

}  // namespace sv
