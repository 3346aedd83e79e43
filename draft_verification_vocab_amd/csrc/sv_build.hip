// P-EAGLE parallel-draft batch construction for gfx950.
//
// One wavefront per output row of the drafter batch (2K rows per sequence),
// four rows per workgroup.  Every lane derives the row's role from the
// sequence's accept count (a handful of scalar loads that hit the same
// addresses), lane 0 writes the row's token id, position and KV slot, and the
// whole wave copies the row's hidden state (a target hidden row, or h_shared
// for MASK rows) with 16-byte loads and stores.  Fusing the metadata rebuild
// with the hidden copy is one launch instead of the separate copy / scatter /
// insert / pad / mask / remap operations and the dedicated broadcast copy that
// the P-EAGLE / TorchSpec blog summary describes (section TorchSpec 集成与工程优化).
// Row layout (per sequence, a = accepted drafts, K drafts):
//   0..a-1 accepted, a NTP, a+1..a+K-1 MASK, a+K..2K-1 rejected (slot -1).
#include "sv_device.h"
#include "sv_internal.h"

namespace sv {

constexpr int kBuildThreads = 256;
constexpr int kRowsPerBlock = kBuildThreads / kWave;

struct BuildArgs {
  BuildLaunch L;
  long rows;   // B * 2K
};

__device__ __forceinline__ void copy_row(const void* src, void* dst, long row_bytes, bool vec,
                                         int elem_bytes) {
  const int l = lane_id();
  if (vec) {
    const u32x4* s = static_cast<const u32x4*>(src);
    u32x4* d = static_cast<u32x4*>(dst);
    const long n = row_bytes / 16;
    for (long i = l; i < n; i += kWave) d[i] = s[i];
  } else if (elem_bytes == 4) {
    const uint32_t* s = static_cast<const uint32_t*>(src);
    uint32_t* d = static_cast<uint32_t*>(dst);
    for (long i = l; i < row_bytes / 4; i += kWave) d[i] = s[i];
  } else {
    const uint16_t* s = static_cast<const uint16_t*>(src);
    uint16_t* d = static_cast<uint16_t*>(dst);
    for (long i = l; i < row_bytes / 2; i += kWave) d[i] = s[i];
  }
}

__global__ __launch_bounds__(kBuildThreads) void build_kernel(BuildArgs A) {
  const BuildLaunch& L = A.L;
  const long row = (long)blockIdx.x * kRowsPerBlock + threadIdx.x / kWave;
  if (row >= A.rows) return;
  const int K = L.K;
  const int b = (int)(row / (2 * K));
  const int i = (int)(row % (2 * K));
  int a = L.num_accepted[b];
  if (a < 0 || a > K) {
    if (lane_id() == 0 && i == 0) flag_error(L.device_error, SV_DEVERR_ACCEPT_COUNT);
    a = a < 0 ? 0 : K;
  }
  const int64_t Lpos = L.start_pos[b];
  // role of row i
  int token;
  int64_t pos;
  int hslot;        // verify slot whose hidden row is copied; -1 = h_shared
  bool pad = false;
  if (i < a) {
    token = L.verify_out_tokens[(long)b * (K + 1) + i];
    pos = Lpos + i;
    hslot = i;
  } else if (i == a) {
    token = L.verify_out_tokens[(long)b * (K + 1) + a];
    pos = Lpos + a;
    hslot = a;
  } else if (i < a + K) {
    token = L.mask_token_id;
    pos = Lpos + i;
    hslot = -1;
  } else {
    const int j = i - a - K;
    token = L.draft_tokens[(long)b * K + a + j];
    pos = Lpos + a + 1 + j;
    hslot = a + 1 + j;
    pad = true;
  }
  if (lane_id() == 0) {
    int64_t slot = SV_PADDING_SLOT_ID;
    if (!pad) {
      const int64_t blk = pos / L.block_size;
      bool okb = pos >= 0 && blk < L.max_blocks;
      int32_t page = okb ? L.block_table[(long)b * L.max_blocks + blk] : -1;
      if (okb && page >= 0) slot = (int64_t)page * L.block_size + pos % L.block_size;
      else flag_error(L.device_error, SV_DEVERR_BLOCK_TABLE);
    }
    L.out_input_ids[row] = token;
    L.out_positions[row] = pos;
    L.out_slot_mapping[row] = slot;
  }
  if (L.out_sample_rows && i == 0 && lane_id() < K)
    L.out_sample_rows[(long)b * K + lane_id()] = (int32_t)(row + a + lane_id());
  const long row_bytes = (long)L.H * L.elem_bytes;
  const char* src = hslot < 0
      ? static_cast<const char*>(L.h_shared)
      : static_cast<const char*>(L.target_hidden) + ((long)b * (K + 1) + hslot) * row_bytes;
  char* dst = static_cast<char*>(L.out_hidden) + row * row_bytes;
  copy_row(src, dst, row_bytes, L.vec != 0, L.elem_bytes);
}

hipError_t launch_build(const BuildLaunch& L, hipStream_t stream) {
  BuildArgs A;
  A.L = L;
  A.rows = (long)L.B * 2 * L.K;
  const unsigned blocks = (unsigned)((A.rows + kRowsPerBlock - 1) / kRowsPerBlock);
  trace_before(stream);
  hipLaunchKernelGGL(build_kernel, dim3(blocks), dim3(kBuildThreads), 0, stream, A);
  const hipError_t err = hipGetLastError();
  trace_after(stream, SV_KERNEL_PEAGLE_BUILD);
  return err;
}

}  // namespace sv
