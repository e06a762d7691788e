// Internal launch interface between the C-ABI layer (fa_api.cpp) and the
// kernel translation units.  Arguments arrive here already validated.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace fa {

struct FwdArgs {
  const void* Q;
  const void* K;
  const void* V;
  void* O;
  float* LSE;
  int B, H, N, d;   // N: query rows per head
  float scale;
  bool causal;
  int dtype;        // 0 = fp32, 1 = bf16
  hipStream_t stream;
  int Nk = 0;       // key/value rows per head (0: same as N)
  long long delta = 0;   // q_offset - k_offset: key j is visible to row i iff j <= i + delta
  // O and LSE hold a running result on entry, which this block is merged
  // into (contiguous layout only)
  bool accumulate = false;
  // paged prefill: K/V are pools read through a block table, Q/O/LSE are
  // packed [total_q, H, ...] with per-sequence start offsets; B is the number
  // of sequences and N the longest chunk
  bool paged = false;
  const int32_t* table = nullptr;
  const int32_t* q_start = nullptr;
  const int32_t* seq_lens = nullptr;
  int KVH = 0, max_blocks = 0, num_blocks = 0;
  int total_q = 0;   // rows of the packed Q/O/LSE
};

struct MergeArgs {
  const void* Oa;
  const float* La;
  const void* Ob;
  const float* Lb;
  void* O;
  float* L;
  long long rows;   // B * H * N
  int d;
  int dtype;
  hipStream_t stream;
};

struct BwdArgs {
  const void* Q;
  const void* K;
  const void* V;
  const void* O;
  const void* dO;
  const float* LSE;
  float* dQ;
  float* dK;
  float* dV;
  float* Dvec;  // workspace: [B, H, N] fp32
  int B, H, N, d;
  float scale;
  bool causal;
  hipStream_t stream;
  int dtype = 1;   // 1 = bf16, 2 = fp16 inputs
};

struct DecodeArgs {
  const void* q;
  const void* k_pool;
  const void* v_pool;
  const int32_t* block_table;
  const int32_t* seq_lens;
  int block_size, num_seqs, H, d, max_blocks_per_seq, num_blocks;
  float scale;
  void* o;
  float* lse;
  float* part;      // workspace: partial (m, l, o[d]) per (slot, head), then block prefix sums
  int units;        // shares of the block stream (kDecodeUnits)
  hipStream_t stream;
  int KVH = 0;      // key/value heads in the pools (0: same as H)
  int dtype = 1;    // 1 = bf16, 2 = fp16
};

struct AppendArgs {
  const void* k_new;      // [num_seqs, KVH, d]
  const void* v_new;
  void* k_pool;           // [num_blocks, block_size, KVH, d]
  void* v_pool;
  int32_t* block_table;   // [num_seqs, max_blocks_per_seq]
  int32_t* seq_lens;      // [num_seqs]
  const int32_t* free_list;
  int32_t* free_count;    // device scalar, updated
  int32_t* n_failed;      // device scalar, written
  int32_t* slot_map;      // workspace [num_seqs]: pool slot written, or -1
  int num_seqs, block_size, max_blocks_per_seq, num_blocks, free_capacity;
  int row_bytes;          // bytes of one token's K (or V) row: KVH * d * element size
  hipStream_t stream;
};

hipError_t launch_fwd(const FwdArgs& a);
hipError_t launch_merge(const MergeArgs& a);
hipError_t launch_bwd(const BwdArgs& a);
hipError_t launch_decode(const DecodeArgs& a);
// Device address, on the current device, of the allocation-free decode's
// static scratch (kNoAllocScratchBytes); taken once per device.
hipError_t noalloc_scratch(void** ptr);
hipError_t launch_append(const AppendArgs& a);

// Heads per group for xcd_grouped over a grid of `heads` heads whose tiles
// each stream bytes_per_head of operands: the largest divisor g of heads / 8
// whose g heads' operands fit in one XCD's 4 MiB L2 (at least 1).  0 when
// heads is not a positive multiple of 8: the plain XCD blocking is used then.
inline int xcd_group(long long heads, long long bytes_per_head) {
  if (heads <= 0 || heads % 8 != 0) return 0;
  const long long hpx = heads / 8;
  int g = 1;
  for (long long c = 2; c <= hpx; ++c)
    if (hpx % c == 0 && c * bytes_per_head <= (4ll << 20)) g = (int)c;
  return g;
}

// Decode work split shared by the workspace query and the launcher: the
// concatenated 16-token block stream of all sequences is cut into kDecodeUnits
// equal shares (fewer when there are fewer blocks), one per workgroup (per
// head group), so every workgroup has the same work whatever the lengths.  A
// share writes one partial result per sequence piece it covers, in slot
// (share + sequence), so at most kDecodeUnits + num_seqs - 1 slots are used.
// 256 is one share per compute unit of an MI355X: at H = 32 every workgroup
// of the grid is resident at once and has the same work.
#ifndef FA_DECODE_UNITS
#define FA_DECODE_UNITS 256
#endif
constexpr int kDecodeUnits = FA_DECODE_UNITS;
// workspace bytes: per slot and head (m, l, d output values) in fp32, then the
// num_seqs + 1 block prefix sums (int64)
// Bytes of the static scratch behind fa_paged_decode_gqa_noalloc.
constexpr size_t kNoAllocScratchBytes = (size_t)32 << 20;
inline size_t decode_partials_floats(int num_seqs, int H, int d) {
  return ((size_t)kDecodeUnits + num_seqs) * H * (size_t)(d + 2);
}

}  // namespace fa
