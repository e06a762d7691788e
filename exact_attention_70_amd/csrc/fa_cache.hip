// Paged KV-cache append for gfx950: one new token's K and V per sequence,
// written through the block table, with blocks taken on demand from a stack
// of free physical blocks.
//
// Method: CMU 10-423 L17-L18 notes, section "Decoding: PagedAttention" (the
// KV cache is cut into fixed-size token blocks stored non-contiguously; a
// block table maps logical to physical blocks; blocks are allocated only when
// needed and reclaimed when unused), and HPC notes "07-16 afternoon", section
// "Prefill, Decode and inference scheduling" (the runtime keeps each
// sequence's length and block mapping; a finished request hands its blocks
// back for reuse).
//
// append_alloc_kernel (one workgroup): sequence s appends at t = seq_lens[s].
//   When t is a multiple of block_size its blocks are full and it needs a new
//   one.  The sequences that need one are ranked in sequence order (ballot and
//   popcount inside a wave, per-wave counts across the workgroup), and the one
//   of rank r takes free_list[free_count - 1 - r]: the stack is popped in
//   sequence order.  It writes the table entry, the pool slot the token goes
//   to (slot_map, -1 when nothing is appended) and the new length; then the
//   new stack height and the number of sequences that could not append (table
//   full, stack empty, or an out-of-range block id).
// append_copy_kernel: copies each appending sequence's K and V rows into its
//   slot, 16 bytes per thread.
#include "fa_device.h"
#include "fa_internal.h"

namespace fa {

namespace {

constexpr int kAllocThreads = 1024;
constexpr int kAllocWaves = kAllocThreads / 64;

__global__ __launch_bounds__(kAllocThreads) void append_alloc_kernel(
    int32_t* __restrict__ block_table, int32_t* __restrict__ seq_lens,
    const int32_t* __restrict__ free_list, int32_t* __restrict__ free_count,
    int32_t* __restrict__ n_failed, int32_t* __restrict__ slot_map, int num_seqs, int block_size,
    int max_blocks_per_seq, int num_blocks, int free_capacity) {
  __shared__ int wave_cnt[kAllocWaves];
  __shared__ int wave_fail[kAllocWaves];
  __shared__ int sh_top;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  if (tid == 0) sh_top = min(max(free_count[0], 0), free_capacity);
  __syncthreads();
  const int top = sh_top;                               // stack height at entry
  const long long cap = (long long)max_blocks_per_seq * block_size;
  int taken = 0, failed_total = 0;                      // uniform across the workgroup
  for (int s0 = 0; s0 < num_seqs; s0 += kAllocThreads) {
    const int s = s0 + tid;
    const bool live = s < num_seqs;
    const int t = live ? seq_lens[s] : 0;
    const bool room = live && t >= 0 && (long long)t < cap;
    const bool need = room && (t % block_size == 0);
    const uint64_t m = __builtin_amdgcn_ballot_w64(need);
    const int in_wave = __builtin_popcountll(m & ((1ull << lane) - 1ull));
    if (lane == 0) wave_cnt[wave] = __builtin_popcountll(m);
    __syncthreads();
    int before = 0, chunk = 0;
#pragma unroll
    for (int w = 0; w < kAllocWaves; ++w) {
      before += (w < wave) ? wave_cnt[w] : 0;
      chunk += wave_cnt[w];
    }
    const int rank = taken + before + in_wave;          // among all needing sequences so far
    int slot = -1;
    if (need) {
      if (rank < top) {
        const int phys = free_list[top - 1 - rank];
        if ((unsigned)phys < (unsigned)num_blocks) {
          block_table[(size_t)s * max_blocks_per_seq + t / block_size] = phys;
          slot = phys * block_size;
        }
      }
    } else if (room) {
      const int phys = block_table[(size_t)s * max_blocks_per_seq + t / block_size];
      if ((unsigned)phys < (unsigned)num_blocks) slot = phys * block_size + t % block_size;
    }
    if (live) {
      slot_map[s] = slot;
      if (slot >= 0) seq_lens[s] = t + 1;
    }
    const uint64_t fm = __builtin_amdgcn_ballot_w64(live && slot < 0);
    if (lane == 0) wave_fail[wave] = __builtin_popcountll(fm);
    __syncthreads();
    int fails = 0;
#pragma unroll
    for (int w = 0; w < kAllocWaves; ++w) fails += wave_fail[w];
    taken += chunk;
    failed_total += fails;
    __syncthreads();                                    // wave_cnt / wave_fail reused next chunk
  }
  if (tid == 0) {
    free_count[0] = top - min(taken, top);
    n_failed[0] = failed_total;
  }
}

__global__ __launch_bounds__(256) void append_copy_kernel(
    const u32x4* __restrict__ k_new, const u32x4* __restrict__ v_new, u32x4* __restrict__ k_pool,
    u32x4* __restrict__ v_pool, const int32_t* __restrict__ slot_map, int num_seqs, int row16,
    long long total_slots) {
  const long long gid = (long long)blockIdx.x * 256 + threadIdx.x;
  const long long s = gid / row16;
  const int c = (int)(gid % row16);
  if (s >= num_seqs) return;
  const long long slot = slot_map[s];
  if (slot < 0 || slot >= total_slots) return;
  k_pool[slot * row16 + c] = k_new[s * row16 + c];
  v_pool[slot * row16 + c] = v_new[s * row16 + c];
}

}  // namespace

hipError_t launch_append(const AppendArgs& a) {
  hipLaunchKernelGGL(append_alloc_kernel, dim3(1), dim3(kAllocThreads), 0, a.stream, a.block_table,
                     a.seq_lens, a.free_list, a.free_count, a.n_failed, a.slot_map, a.num_seqs,
                     a.block_size, a.max_blocks_per_seq, a.num_blocks, a.free_capacity);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int row16 = a.row_bytes / 16;
  const long long threads = (long long)a.num_seqs * row16;
  hipLaunchKernelGGL(append_copy_kernel, dim3((unsigned)((threads + 255) / 256)), dim3(256), 0,
                     a.stream, (const u32x4*)a.k_new, (const u32x4*)a.v_new, (u32x4*)a.k_pool,
                     (u32x4*)a.v_pool, a.slot_map, a.num_seqs, row16,
                     (long long)a.num_blocks * a.block_size);
  return hipGetLastError();
}

}  // namespace fa
