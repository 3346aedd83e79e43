// The P-EAGLE drafter batch built the way the pages build it -- a metadata
// kernel, then a separate copy of the hidden rows (P-EAGLE / TorchSpec blog
// summary, section TorchSpec 集成与工程优化: the batch is rebuilt on the GPU
// and the hidden states are broadcast by a dedicated copy) -- as the
// comparison for the library's one fused build kernel.  Not part of the
// verify library: bench.py times it beside peagle_build_draft_batch, and the
// profiling run hands both to the HBM byte counters.
//
//   meta_kernel  one thread per verify slot (b, i): the row's id, position
//                and slot, the MASK row it seeds, out_sample_rows, and a
//                source -> destination row map in a scratch buffer;
//   copy_kernel  one wave per verify slot copies target_hidden row (b, i)
//                to its destination through the map, and h_shared to the
//                MASK row, 16-byte non-temporal stores.
// Same outputs as peagle_build_draft_batch, bit for bit, for valid inputs
// (0 <= num_accepted <= K, bf16 hidden rows).
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

struct SplitArgs {
  const int32_t* out_tokens;   // [B][K+1]
  const int32_t* acc;          // [B]
  const int32_t* drafts;       // [B][K]
  const int64_t* start_pos;    // [B]
  const int32_t* table;        // [B][max_blocks]
  int max_blocks, block_size;
  const uint16_t* hidden;      // [B*(K+1)][H]
  const uint16_t* h_shared;    // [H]
  int mask_id, B, K, H;
  int32_t* ids; int64_t* pos; int64_t* slots; uint16_t* out_hidden; int32_t* sample_rows;
  int32_t* row_map;            // [B*(K+1)] destination of verify slot (b, i)
  int32_t* mask_map;           // [B*(K+1)] MASK row seeded by (b, i), or -1
};

__device__ int64_t slot_of(const SplitArgs& p, int b, int64_t q) {
  const int64_t blk = q / p.block_size;
  const bool ok = q >= 0 && blk < p.max_blocks;
  const int32_t page = ok ? p.table[(long)b * p.max_blocks + blk] : -1;
  return (ok && page >= 0) ? (int64_t)page * p.block_size + q % p.block_size : -1;
}

__global__ __launch_bounds__(256) void meta_kernel(SplitArgs p) {
  const long unit = (long)blockIdx.x * 256 + threadIdx.x;
  if (unit >= (long)p.B * (p.K + 1)) return;
  const int K = p.K, b = (int)(unit / (K + 1)), i = (int)(unit % (K + 1));
  int a = p.acc[b];
  a = a < 0 ? 0 : (a > K ? K : a);
  const long base = (long)b * 2 * K;
  // slot i <= a: accepted prefix and new token at row i; slot i > a: the
  // rejected draft i-1 at row i + K - 1 with no cache slot
  const long dst = base + (i <= a ? i : i + K - 1);
  const int64_t L = p.start_pos[b];
  p.ids[dst] = i <= a ? p.out_tokens[(long)b * (K + 1) + i] : p.drafts[(long)b * K + i - 1];
  p.pos[dst] = L + i;
  p.slots[dst] = i <= a ? slot_of(p, b, L + i) : -1;
  p.row_map[unit] = (int32_t)dst;
  const bool mask_row = i >= 1 && i <= K - 1;            // slot i seeds MASK row a + i
  p.mask_map[unit] = mask_row ? (int32_t)(base + a + i) : -1;
  if (mask_row) {
    p.ids[base + a + i] = p.mask_id;
    p.pos[base + a + i] = L + a + i;
    p.slots[base + a + i] = slot_of(p, b, L + a + i);
  }
  if (i == 0 && p.sample_rows)
    for (int k = 0; k < K; ++k) p.sample_rows[(long)b * K + k] = (int32_t)(base + a + k);
}

__global__ __launch_bounds__(256) void copy_kernel(SplitArgs p) {
  const long unit = (long)blockIdx.x * 4 + threadIdx.x / 64;
  if (unit >= (long)p.B * (p.K + 1)) return;
  const int l = threadIdx.x & 63;
  const long nvec = (long)p.H * 2 / 16;
  const u32x4* s = reinterpret_cast<const u32x4*>(p.hidden + unit * p.H);
  const u32x4* h = reinterpret_cast<const u32x4*>(p.h_shared);
  const int dst = p.row_map[unit], mdst = p.mask_map[unit];
  u32x4* d = reinterpret_cast<u32x4*>(p.out_hidden + (long)dst * p.H);
  u32x4* dm = reinterpret_cast<u32x4*>(p.out_hidden + (long)(mdst < 0 ? 0 : mdst) * p.H);
  for (long e = l; e < nvec; e += 64) {
    __builtin_nontemporal_store(s[e], d + e);
    if (mdst >= 0) __builtin_nontemporal_store(h[e], dm + e);
  }
}

bool aligned(const void* p, uintptr_t n) { return reinterpret_cast<uintptr_t>(p) % n == 0; }

}  // namespace

// The two-kernel build.  Arguments as peagle_build_draft_batch (bf16 hidden
// rows only, H a multiple of 8), plus row_maps: a device scratch buffer of
// 2 * B * (K+1) int32 that the metadata kernel fills and the copy kernel
// reads.  Returns 0 when both kernels were enqueued on `stream`, 1 for
// invalid arguments (nothing launched), 2 when a launch failed.
extern "C" __attribute__((visibility("default"))) int svc_build_split(
    const int32_t* verify_out_tokens, const int32_t* num_accepted, const int32_t* draft_tokens,
    const int64_t* start_pos, const int32_t* block_table, int max_blocks_per_seq, int block_size,
    const void* target_hidden, const void* h_shared, int32_t mask_token_id, int B, int K, int H,
    int32_t* out_input_ids, int64_t* out_positions, int64_t* out_slot_mapping, void* out_hidden,
    int32_t* out_sample_rows, int32_t* row_maps, void* stream) {
  if (B <= 0 || K < 1 || K > 63 || H <= 0 || H % 8 || max_blocks_per_seq < 1 || block_size < 1)
    return 1;
  if (!verify_out_tokens || !num_accepted || !draft_tokens || !start_pos || !block_table ||
      !target_hidden || !h_shared || !out_input_ids || !out_positions || !out_slot_mapping ||
      !out_hidden || !row_maps)
    return 1;
  if (!aligned(target_hidden, 16) || !aligned(h_shared, 16) || !aligned(out_hidden, 16)) return 1;
  SplitArgs p;
  p.out_tokens = verify_out_tokens; p.acc = num_accepted; p.drafts = draft_tokens;
  p.start_pos = start_pos; p.table = block_table;
  p.max_blocks = max_blocks_per_seq; p.block_size = block_size;
  p.hidden = static_cast<const uint16_t*>(target_hidden);
  p.h_shared = static_cast<const uint16_t*>(h_shared);
  p.mask_id = mask_token_id; p.B = B; p.K = K; p.H = H;
  p.ids = out_input_ids; p.pos = out_positions; p.slots = out_slot_mapping;
  p.out_hidden = static_cast<uint16_t*>(out_hidden); p.sample_rows = out_sample_rows;
  const long units = (long)B * (K + 1);
  p.row_map = row_maps; p.mask_map = row_maps + units;
  hipStream_t s = static_cast<hipStream_t>(stream);
  hipLaunchKernelGGL(meta_kernel, dim3((unsigned)((units + 255) / 256)), dim3(256), 0, s, p);
  if (hipGetLastError() != hipSuccess) return 2;
  hipLaunchKernelGGL(copy_kernel, dim3((unsigned)((units + 3) / 4)), dim3(256), 0, s, p);
  return hipGetLastError() == hipSuccess ? 0 : 2;
}
