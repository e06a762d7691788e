// Paged single-token decode for gfx950.
//
// Method: CMU 10-423 L17-L18 notes, section "Decoding: PagedAttention" (the KV
// cache is cut into fixed-size token blocks stored non-contiguously; a block
// table maps logical to physical blocks; the kernel computes block by block)
// and HPC notes "07-16 afternoon", section "Prefill, Decode and inference
// scheduling" (a decode step feeds one token whose query reads every cached
// K/V of its sequence, so the step is bound by memory bandwidth).  The split
// over pieces of the KV stream is merged with the rescaling rule of the online softmax
// (HPC notes, section "Long context and sequence parallelism").
//
// Pool layout [num_blocks, block_size = 16, KVH, d], d = 64 or 128: one physical block
// is a contiguous 16 * KVH * 2d-byte chunk, so a workgroup that reads all
// heads of a block streams contiguous memory.  With grouped-query attention
// (KVH < H; HPC notes, "Prefill, Decode and inference scheduling", KV-cache
// size) consecutive query heads share one cached head: their lanes load the
// same bytes, which the vector L1 merges, so HBM traffic per token falls by
// H / KVH.
//
// Work split: the 16-token blocks of all sequences, taken one after another,
//   are cut into equal shares (prefix sums of the block counts come from a
//   one-workgroup scan), one share per workgroup and head group.  A share
//   covers pieces of one or more sequences and writes one partial result per
//   piece, so every workgroup has the same work whatever the lengths: no
//   last, nearly empty round of workgroups.
// Partial kernel: workgroup = (share, group of heads); a lane owns 8 of a
//   head's d values, so d / 8 lanes serve a head and a wave 64 / (d / 8)
//   heads (4 at d = 128, 8 at d = 64).  Per sequence piece it covers, at
//   H = 32, d = 128 every 16-token block is read as one contiguous 128 KiB
//   stream.  Per 16-token block: 16-byte loads of K and V
//   rows through a buffer resource over that physical block (an out-of-range
//   block id therefore reads zeros instead of faulting), the token stride in
//   the wave-uniform offset, with the non-temporal hint (each cached byte is
//   read once per step; on MI355X the hint took the 64 x 32 x 128 decode
//   from 392 to 360 us); q.k partial dot products reduced across the head's
//   lanes with DPP, one online-softmax update per block, and the P V
//   accumulation.  K and V are separate load batches: the scores of block t
//   run while V_t streams in, and K_{t+1} streams in while V_t is accumulated.
//   Writes (m, l, unnormalised o).
// Grouped-query partial kernel (G = H / KVH in {2, 4, 8}): a wave serves one
//   cached head and the G query heads that read it, so each cached row is
//   loaded once.  Lane = (token phase tq = lane / (d / 8), 8 of the d
//   values); the TQ = 64 / (d / 8) phases take interleaved tokens
//   (TQ i + tq), so one 16-byte load instruction brings TQ token rows (4 at
//   d = 128, 8 at d = 64).  Each lane scores its rows against all G queries
//   (packed two-element dot products, reduced across the row's lanes with
//   DPP); the weights of two rows, rounded to the element type, meet the V
//   values of those rows in one two-element dot product per d.  The running
//   max is shared by the phases; their denominators and outputs stay
//   separate until the piece ends, when cross-phase exchanges combine them.
// Merge kernel: one wave per (sequence, head) combines its pieces, found
//   from the prefix sums.
//   Throughput is bound by HBM: the flops per byte are ~1.
#include <mutex>

#include "fa_device.h"
#include "fa_internal.h"

namespace fa {

namespace {

constexpr int kDecBS = 16;
constexpr int kDecThreads = 512;
// Head dims 64 and 128: a lane owns 8 of a row's d values, so D / 8 lanes
// cover a row, a wave serves 64 / (D / 8) heads (4 at d = 128, 8 at d = 64)
// and a workgroup 8 times that (32: whole 8 KiB token rows at H = 32, d = 128).
template <int D>
struct DecShape {
  static_assert(D == 64 || D == 128, "head dim 64 or 128");
  static constexpr int kLanesPerRow = D / 8;
  static constexpr int kHeadsPerWave = 64 / kLanesPerRow;
  static constexpr int kHeadsPerGroup = (kDecThreads / 64) * kHeadsPerWave;
};

// prefix[s] = 16-token blocks of sequences 0 .. s-1, a sequence's length
// clamped to [0, max_blocks_per_seq * 16]; prefix[num_seqs] = all blocks.
// One workgroup of 256 threads scans the lengths 256 at a time.
__global__ __launch_bounds__(256) void decode_prefix_kernel(const int32_t* __restrict__ seq_lens,
                                                            int num_seqs, int max_blocks_per_seq,
                                                            long long* __restrict__ prefix) {
  __shared__ long long part[256];
  const int t = threadIdx.x;
  long long carry = 0;
  for (int base = 0; base < num_seqs; base += 256) {
    const int sq = base + t;
    long long nb = 0;
    if (sq < num_seqs) {
      const int len = min(seq_lens[sq], max_blocks_per_seq * kDecBS);
      nb = len > 0 ? (len + kDecBS - 1) / kDecBS : 0;
    }
    part[t] = nb;
    __syncthreads();
#pragma unroll
    for (int off = 1; off < 256; off <<= 1) {
      const long long v = t >= off ? part[t - off] : 0;
      __syncthreads();
      part[t] += v;
      __syncthreads();
    }
    if (sq < num_seqs) prefix[sq + 1] = carry + part[t];
    carry += part[255];
    __syncthreads();
  }
  if (t == 0) prefix[0] = 0;
}

// Shares actually used: kDecodeUnits, or one per block when there are fewer
// blocks, so that no share is empty.
__device__ __forceinline__ int decode_shares(const long long* prefix, int num_seqs, int units) {
  const long long tb = prefix[num_seqs];
  return (int)min((long long)units, tb);
}

// Share g of G takes blocks [g TB / G, (g + 1) TB / G) of the concatenated
// block stream (TB blocks in all) and calls f(s, first block, end block) for
// every sequence piece in it, blocks counted within the sequence.
template <class F>
__device__ __forceinline__ void for_each_piece(const long long* prefix, int num_seqs, int g, int G,
                                               F f) {
  const long long tb = prefix[num_seqs];
  const long long lo = (long long)g * tb / G, hi = (long long)(g + 1) * tb / G;
  // the first sequence ending after block lo (binary search on the prefix sums)
  int a = 0, b = num_seqs;
  while (a < b) {
    const int m = (a + b) >> 1;
    if (prefix[m + 1] > lo) b = m;
    else a = m + 1;
  }
  for (int sq = a; sq < num_seqs; ++sq) {
    const long long p0 = prefix[sq], p1 = prefix[sq + 1];
    if (p0 >= hi) break;
    if (p1 > p0) f(sq, (int)(max(lo, p0) - p0), (int)(min(hi, p1) - p0));
  }
}

// One sequence piece (tokens [t_begin, t_end) of sequence s) for this
// workgroup's group of heads; writes the partial result into slot `slot`.
template <class E, int D>
__device__ __forceinline__ void decode_piece(
    const typename E::elem* __restrict__ q, const typename E::elem* __restrict__ k_pool,
    const typename E::elem* __restrict__ v_pool, const int32_t* __restrict__ block_table, int H,
    int KVH, int max_blocks_per_seq, int num_blocks, float scale_log2, float* __restrict__ part_o,
    float* __restrict__ part_ml, int s, int t_begin, int t_end, size_t slot) {
  // H query heads; the pools hold KVH key/value heads and query head h reads
  // cached head h / (H / KVH)
  const int hg = blockIdx.y;
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  using S = DecShape<D>;
  constexpr int LPR = S::kLanesPerRow;
  const int head = hg * S::kHeadsPerGroup + wave * S::kHeadsPerWave + lane / LPR;
  const int ch = lane % LPR;                         // which 8 of the D values
  const bool head_ok = head < H;
  const int hh = head_ok ? head : 0;
  const int kvh = hh / (H / KVH);                   // the cached head this query head reads

  const uint32_t blk_bytes = (uint32_t)kDecBS * KVH * D * 2;
  const uint32_t row_off = (uint32_t)(kvh * D + ch * 8) * 2;   // within one token row
  const uint32_t tok_stride = (uint32_t)KVH * D * 2;

  // this lane's 8 query values, fp32
  float qv[8];
  {
    const auto rq = make_rsrc(q + (size_t)s * H * D, (uint32_t)H * D * 2);
    const u32x4 w = bload16(rq, (uint32_t)(hh * D + ch * 8) * 2);   // this query head
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      qv[2 * e] = E::lo(w[e]);
      qv[2 * e + 1] = E::hi(w[e]);
    }
  }

  float m_run = kNegInf, l_run = 0.f;
  float acc[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) acc[e] = 0.f;

  const int32_t* table = block_table + (size_t)s * max_blocks_per_seq;
  // K of a block and V of a block are separate load batches: the scores of
  // block t run while V_t streams in, and K_{t+1} streams in while V_t is
  // accumulated, so every compute phase has the next batch in flight.
  auto block_rsrc = [&](int t0, __amdgpu_buffer_rsrc_t& rk, __amdgpu_buffer_rsrc_t& rv) {
    const int32_t phys = table[t0 / kDecBS];
    const bool phys_ok = (uint32_t)phys < (uint32_t)num_blocks;
    const size_t boff = (size_t)(phys_ok ? phys : 0) * kDecBS * KVH * D;
    rk = make_rsrc(k_pool + boff, phys_ok ? blk_bytes : 0u);
    rv = make_rsrc(v_pool + boff, phys_ok ? blk_bytes : 0u);
  };
  u32x4 kr[kDecBS], vr[kDecBS];
  __amdgpu_buffer_rsrc_t rk, rv;
  block_rsrc(t_begin, rk, rv);
#pragma unroll
  for (int u = 0; u < kDecBS; ++u) kr[u] = bload16s_nt(rk, row_off, u * tok_stride);
#pragma unroll
  for (int u = 0; u < kDecBS; ++u) vr[u] = bload16s_nt(rv, row_off, u * tok_stride);
  for (int t0 = t_begin; t0 < t_end; t0 += kDecBS) {
    const bool more = t0 + kDecBS < t_end;
    __amdgpu_buffer_rsrc_t rk2 = rk, rv2 = rv;
    if (more) block_rsrc(t0 + kDecBS, rk2, rv2);
    const int n_valid = min(kDecBS, t_end - t0);
    float sc[kDecBS];
    float mx = kNegInf;
#pragma unroll
    for (int u = 0; u < kDecBS; ++u) {
      float part = 0.f;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        part = fmaf(qv[2 * e], E::lo(kr[u][e]), part);
        part = fmaf(qv[2 * e + 1], E::hi(kr[u][e]), part);
      }
      float x = group_sum<LPR>(part) * scale_log2;
      if (u >= n_valid) x = kNegInf;
      sc[u] = x;
      mx = fmaxf(mx, x);
    }
    if (more) {
#pragma unroll
      for (int u = 0; u < kDecBS; ++u) kr[u] = bload16s_nt(rk2, row_off, u * tok_stride);
    }
    const float m_new = fmaxf(m_run, mx);
    const float alpha = fast_exp2(m_run - m_new);
    m_run = m_new;
    float rs = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[e] *= alpha;
#pragma unroll
    for (int u = 0; u < kDecBS; ++u) {
      const float pu = fast_exp2(sc[u] - m_new);
      rs += pu;
      if (u < n_valid) {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          acc[2 * e] = fmaf(pu, E::lo(vr[u][e]), acc[2 * e]);
          acc[2 * e + 1] = fmaf(pu, E::hi(vr[u][e]), acc[2 * e + 1]);
        }
      }
    }
    l_run = l_run * alpha + rs;
    if (more) {
#pragma unroll
      for (int u = 0; u < kDecBS; ++u) vr[u] = bload16s_nt(rv2, row_off, u * tok_stride);
    }
    rk = rk2;
    rv = rv2;
  }
  if (!head_ok) return;
  const size_t entry = slot * H + head;
  u32x4 w0, w1;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    w0[e] = as_u32(acc[e]);
    w1[e] = as_u32(acc[4 + e]);
  }
  *(u32x4*)(part_o + entry * D + ch * 8) = w0;
  *(u32x4*)(part_o + entry * D + ch * 8 + 4) = w1;
  if (ch == 0) {
    part_ml[entry * 2] = m_run;
    part_ml[entry * 2 + 1] = l_run;
  }
}

template <class E, int D>
__global__ __launch_bounds__(kDecThreads, 1) void decode_partial_kernel(
    const typename E::elem* __restrict__ q, const typename E::elem* __restrict__ k_pool,
    const typename E::elem* __restrict__ v_pool, const int32_t* __restrict__ block_table,
    const int32_t* __restrict__ seq_lens, int H, int KVH, int max_blocks_per_seq, int num_blocks,
    float scale_log2, float* __restrict__ part_o, float* __restrict__ part_ml,
    const long long* __restrict__ prefix, int num_seqs, int units) {
  const int G = decode_shares(prefix, num_seqs, units);
  const int g = blockIdx.x;
  if (g >= G) return;
  if ((int)blockIdx.y * DecShape<D>::kHeadsPerGroup +
          (int)(threadIdx.x >> 6) * DecShape<D>::kHeadsPerWave >= H)
    return;
  for_each_piece(prefix, num_seqs, g, G, [&](int sq, int b0, int b1) {
    const int len = min(seq_lens[sq], max_blocks_per_seq * kDecBS);
    decode_piece<E, D>(q, k_pool, v_pool, block_table, H, KVH, max_blocks_per_seq, num_blocks,
                    scale_log2, part_o, part_ml, sq, b0 * kDecBS, min(len, b1 * kDecBS),
                    (size_t)g + sq);
  });
}

constexpr int kGqaWaves = 4;   // cached heads per workgroup

template <class E, int G, int D>
__device__ __forceinline__ void decode_gqa_piece(
    const typename E::elem* __restrict__ q, const typename E::elem* __restrict__ k_pool,
    const typename E::elem* __restrict__ v_pool, const int32_t* __restrict__ block_table, int H,
    int KVH, int max_blocks_per_seq, int num_blocks, float scale_log2, float* __restrict__ part_o,
    float* __restrict__ part_ml, int s, int t_begin, int t_end, size_t slot) {
  constexpr int CH = D / 8;              // lanes per cached row (8 d values each)
  constexpr int TQ = 64 / CH;            // token phases: rows one load instruction brings
  constexpr int NI = (G <= 4 ? 8 : 4) * 4 / TQ;   // token rows per lane per step
  constexpr int STEP = TQ * NI;          // tokens per step: whole blocks
  constexpr int NB = STEP / kDecBS;      // blocks per step
  constexpr int RPB = kDecBS / TQ;       // a lane's rows per block
  static_assert(STEP % kDecBS == 0, "a step is whole blocks");
  static_assert(NI % 2 == 0, "rows are weighted in pairs");
  const int lane = threadIdx.x & 63;
  const int kvh = __builtin_amdgcn_readfirstlane(blockIdx.y * kGqaWaves + (threadIdx.x >> 6));
  if (kvh >= KVH) return;                           // no cached head for this wave
  const int tq = lane / CH;                         // token phase within TQ consecutive tokens
  const int ch = lane % CH;                         // which 8 of the D values

  const uint32_t blk_bytes = (uint32_t)kDecBS * KVH * D * 2;
  const uint32_t tok_stride = (uint32_t)KVH * D * 2;
  // row (TQ i + tq) of a step: block i / RPB, slot TQ (i % RPB) + tq
  const uint32_t lane_off = tq * tok_stride + (uint32_t)(kvh * D + ch * 8) * 2;

  // the G query heads' 8 values of this lane, packed pairs
  u32x4 qv[G];
  {
    const auto rq = make_rsrc(q + (size_t)s * H * D, (uint32_t)H * D * 2);
#pragma unroll
    for (int j = 0; j < G; ++j) qv[j] = bload16(rq, (uint32_t)((kvh * G + j) * D + ch * 8) * 2);
  }

  float m_run[G], l_run[G], acc[G][8];
#pragma unroll
  for (int j = 0; j < G; ++j) {
    m_run[j] = kNegInf;
    l_run[j] = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[j][e] = 0.f;
  }

  const int32_t* table = block_table + (size_t)s * max_blocks_per_seq;
  // resources over the NB blocks of the step starting at t0; a block past the
  // piece (or an out-of-range id) gets an empty resource and reads zeros
  auto step_rsrc = [&](int t0, __amdgpu_buffer_rsrc_t (&rk)[NB], __amdgpu_buffer_rsrc_t (&rv)[NB])
      __attribute__((always_inline)) {
#pragma unroll
    for (int b = 0; b < NB; ++b) {
      const int tb = t0 + b * kDecBS;
      const int32_t phys = tb < t_end ? table[tb / kDecBS] : -1;
      const bool ok = (uint32_t)phys < (uint32_t)num_blocks;
      const size_t boff = (size_t)(ok ? phys : 0) * kDecBS * KVH * D;
      rk[b] = make_rsrc(k_pool + boff, ok ? blk_bytes : 0u);
      rv[b] = make_rsrc(v_pool + boff, ok ? blk_bytes : 0u);
    }
  };
  auto load_rows = [&](const __amdgpu_buffer_rsrc_t (&r)[NB], u32x4 (&dst)[NI])
      __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < NI; ++i)
      dst[i] = bload16s_nt(r[i / RPB], lane_off, (i % RPB) * TQ * tok_stride);
  };

  // One step over tokens [t0, t0 + STEP): K of the next step streams in while
  // the softmax runs, V of the next step while this step's V is accumulated.
  // MASKED: some rows lie past t_end; they are excluded by selects, so pad
  // slots (which may hold NaN) never reach the sums.
  u32x4 kr[NI], vr[NI];
  __amdgpu_buffer_rsrc_t rk[NB], rv[NB];
  step_rsrc(t_begin, rk, rv);
  load_rows(rk, kr);
  load_rows(rv, vr);
  auto step = [&](int t0, auto masked) __attribute__((always_inline)) {
    constexpr bool MASKED = decltype(masked)::value;
    const bool more = t0 + STEP < t_end;
    __amdgpu_buffer_rsrc_t rk2[NB], rv2[NB];
    if (more) step_rsrc(t0 + STEP, rk2, rv2);
    float sc[NI][G];
    float mx[G];
#pragma unroll
    for (int j = 0; j < G; ++j) mx[j] = kNegInf;
#pragma unroll
    for (int i = 0; i < NI; ++i) {
      const bool valid = !MASKED || t0 + TQ * i + tq < t_end;
#pragma unroll
      for (int j = 0; j < G; ++j) {
        float part = 0.f;
#pragma unroll
        for (int e = 0; e < 4; ++e) part = E::dot2(qv[j][e], kr[i][e], part);
        float x = group_sum<CH>(part) * scale_log2;
        if constexpr (MASKED) x = valid ? x : kNegInf;
        sc[i][j] = x;
        mx[j] = fmaxf(mx[j], x);
      }
    }
    if (more) load_rows(rk2, kr);
    float alpha[G], m_new[G];
#pragma unroll
    for (int j = 0; j < G; ++j) {
      float m = mx[j];
#pragma unroll
      for (int off = CH; off < 64; off *= 2)          // the step's max over all TQ phases
        m = fmaxf(m, __shfl_xor(m, off, 64));
      m_new[j] = fmaxf(m_run[j], m);
      alpha[j] = fast_exp2(m_run[j] - m_new[j]);
      m_run[j] = m_new[j];
      l_run[j] *= alpha[j];
#pragma unroll
      for (int e = 0; e < 8; ++e) acc[j][e] *= alpha[j];
    }
    // rows of masked tokens become zeros (pad slots may hold NaN, and a zero
    // weight times NaN is NaN)
    if constexpr (MASKED) {
#pragma unroll
      for (int i = 0; i < NI; ++i)
        if (t0 + TQ * i + tq >= t_end) vr[i] = u32x4{0u, 0u, 0u, 0u};
    }
    // Two rows at a time: the pair's weights, rounded to the element type
    // (as the forward rounds P), weight the pair of V values of each d
    // through one two-element dot product; the denominator sums the same
    // rounded weights.
#pragma unroll
    for (int i = 0; i < NI; i += 2) {
      uint32_t vp[8];   // (row i, row i + 1) values of each of the lane's 8 d
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        vp[2 * w] = __builtin_amdgcn_perm(vr[i + 1][w], vr[i][w], 0x05040100u);
        vp[2 * w + 1] = __builtin_amdgcn_perm(vr[i + 1][w], vr[i][w], 0x07060302u);
      }
#pragma unroll
      for (int j = 0; j < G; ++j) {
        const uint32_t pk = E::pack(fast_exp2(sc[i][j] - m_new[j]),    // 0 for a masked row
                                    fast_exp2(sc[i + 1][j] - m_new[j]));
        l_run[j] = E::dot2(pk, E::kOnes, l_run[j]);
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[j][e] = E::dot2(pk, vp[e], acc[j][e]);
      }
    }
    if (more) load_rows(rv2, vr);
  };
  using Plain = std::integral_constant<bool, false>;
  using Masked = std::integral_constant<bool, true>;
  int t0 = t_begin;
  for (; t0 + STEP <= t_end; t0 += STEP) step(t0, Plain{});
  if (t0 < t_end) step(t0, Masked{});

  // combine the TQ phases' denominators and outputs
#pragma unroll
  for (int j = 0; j < G; ++j) {
#pragma unroll
    for (int off = CH; off < 64; off *= 2) {
      l_run[j] += __shfl_xor(l_run[j], off, 64);
#pragma unroll
      for (int e = 0; e < 8; ++e) acc[j][e] += __shfl_xor(acc[j][e], off, 64);
    }
  }
  // phase j % TQ writes query head kvh * G + j
#pragma unroll
  for (int j = 0; j < G; ++j) {
    if (tq != j % TQ) continue;
    const size_t entry = slot * H + kvh * G + j;
    u32x4 w0, w1;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      w0[e] = as_u32(acc[j][e]);
      w1[e] = as_u32(acc[j][4 + e]);
    }
    *(u32x4*)(part_o + entry * D + ch * 8) = w0;
    *(u32x4*)(part_o + entry * D + ch * 8 + 4) = w1;
    if (ch == 0) {
      part_ml[entry * 2] = m_run[j];
      part_ml[entry * 2 + 1] = l_run[j];
    }
  }
}

template <class E, int G, int D>
__global__ __launch_bounds__(kGqaWaves * 64) void decode_gqa_partial_kernel(
    const typename E::elem* __restrict__ q, const typename E::elem* __restrict__ k_pool,
    const typename E::elem* __restrict__ v_pool, const int32_t* __restrict__ block_table,
    const int32_t* __restrict__ seq_lens, int H, int KVH, int max_blocks_per_seq, int num_blocks,
    float scale_log2, float* __restrict__ part_o, float* __restrict__ part_ml,
    const long long* __restrict__ prefix, int num_seqs, int units) {
  const int shares = decode_shares(prefix, num_seqs, units);
  const int g = blockIdx.x;
  if (g >= shares) return;
  if ((int)blockIdx.y * kGqaWaves + (int)(threadIdx.x >> 6) >= KVH) return;   // no cached head
  for_each_piece(prefix, num_seqs, g, shares, [&](int sq, int b0, int b1) {
    const int len = min(seq_lens[sq], max_blocks_per_seq * kDecBS);
    decode_gqa_piece<E, G, D>(q, k_pool, v_pool, block_table, H, KVH, max_blocks_per_seq, num_blocks,
                           scale_log2, part_o, part_ml, sq, b0 * kDecBS, min(len, b1 * kDecBS),
                           (size_t)g + sq);
  });
}

// One wave per (sequence, head): rescale every piece's (m, l, o) to the
// common maximum and sum.  Lanes take the pieces' (m, l) in parallel for
// the maximum and the weights; then each of the first D / 2 lanes owns 2 of
// the D output values and sums the pieces' contributions with the weights
// broadcast from the lane that computed them.
__device__ __forceinline__ float wave_max(float x) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) x = fmaxf(x, __shfl_xor(x, off, 64));
  return x;
}
__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) x += __shfl_xor(x, off, 64);
  return x;
}

template <class E, int D>
__global__ __launch_bounds__(256) void decode_merge_kernel(
    const float* __restrict__ part_o, const float* __restrict__ part_ml,
    const long long* __restrict__ prefix, int num_seqs, int H, int units,
    typename E::elem* __restrict__ o, float* __restrict__ lse) {
  const int gw = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (gw >= num_seqs * H) return;
  const int lane = threadIdx.x & 63;
  const int s = gw / H, head = gw % H;
  const long long bs0 = prefix[s], bs1 = prefix[s + 1];   // this sequence's blocks
  const bool owner = 2 * lane < D;    // this lane owns output values 2 lane, 2 lane + 1
  if (bs1 <= bs0) {   // invalid length: defined output, nothing read
    if (owner) *(uint32_t*)(o + ((size_t)s * H + head) * D + 2 * lane) = 0u;
    if (lane == 0) lse[(size_t)s * H + head] = kNegInf;
    return;
  }
  // the shares holding this sequence's first and last block: share g holds
  // block b iff g is the largest share with g TB / G <= b
  const long long tb = prefix[num_seqs];
  const int G = decode_shares(prefix, num_seqs, units);
  const int g0 = (int)(((bs0 + 1) * G + tb - 1) / tb - 1);
  const int g1 = (int)((bs1 * G + tb - 1) / tb - 1);
  const int np = g1 - g0 + 1;          // pieces p = 0 .. np - 1 in slots g0 + p + s
  const size_t base = ((size_t)g0 + s) * H + head;
  float m_star = kNegInf;
  for (int p = lane; p < np; p += 64) m_star = fmaxf(m_star, part_ml[(base + (size_t)p * H) * 2]);
  m_star = wave_max(m_star);
  float L = 0.f, a0 = 0.f, a1 = 0.f;
  for (int p0 = 0; p0 < np; p0 += 64) {
    // this lane's piece p0 + lane: weight and its share of the denominator
    float w = 0.f;
    if (p0 + lane < np) {
      const size_t e = base + (size_t)(p0 + lane) * H;
      w = fast_exp2(part_ml[e * 2] - m_star);
      L = fmaf(w, part_ml[e * 2 + 1], L);
    }
    const int cnt = min(64, np - p0);
#pragma unroll 4
    for (int q = 0; q < cnt; ++q) {
      const float wq = __shfl(w, q, 64);
      if (owner) {
        const size_t e = base + (size_t)(p0 + q) * H;
        const float2 v = *(const float2*)(part_o + e * D + 2 * lane);
        a0 = fmaf(wq, v.x, a0);
        a1 = fmaf(wq, v.y, a1);
      }
    }
  }
  L = wave_sum(L);
  const float inv = 1.f / L;
  if (owner) *(uint32_t*)(o + ((size_t)s * H + head) * D + 2 * lane) = E::pack(a0 * inv, a1 * inv);
  if (lane == 0) lse[(size_t)s * H + head] = (m_star + fast_log2(L)) * kLn2;
}

}  // namespace

template <class E, int D>
hipError_t launch_decode_ed(const DecodeArgs& a) {
  using T = typename E::elem;
  const size_t n_floats = decode_partials_floats(a.num_seqs, a.H, D);
  const size_t n_entries = n_floats / (D + 2);
  float* part_o = a.part;
  float* part_ml = a.part + n_entries * D;
  long long* prefix = reinterpret_cast<long long*>(a.part + n_floats);
  hipLaunchKernelGGL(decode_prefix_kernel, dim3(1), dim3(256), 0, a.stream, a.seq_lens,
                     a.num_seqs, a.max_blocks_per_seq, prefix);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int KVH = a.KVH > 0 ? a.KVH : a.H;
  const int g = a.H / KVH;
  // grouped heads with a group size the grouped kernel is built for
  if (g == 2 || g == 4 || g == 8) {
    dim3 grid(a.units, (KVH + kGqaWaves - 1) / kGqaWaves);
    auto kern = g == 2 ? decode_gqa_partial_kernel<E, 2, D>
              : g == 4 ? decode_gqa_partial_kernel<E, 4, D> : decode_gqa_partial_kernel<E, 8, D>;
    hipLaunchKernelGGL(kern, grid, dim3(kGqaWaves * 64), 0, a.stream, (const T*)a.q,
                       (const T*)a.k_pool, (const T*)a.v_pool, a.block_table, a.seq_lens, a.H, KVH,
                       a.max_blocks_per_seq, a.num_blocks, a.scale * kLog2e, part_o, part_ml,
                       prefix, a.num_seqs, a.units);
  } else {
    constexpr int HPG = DecShape<D>::kHeadsPerGroup;
    dim3 grid(a.units, (a.H + HPG - 1) / HPG);
    hipLaunchKernelGGL((decode_partial_kernel<E, D>), grid, dim3(kDecThreads), 0, a.stream,
                       (const T*)a.q, (const T*)a.k_pool, (const T*)a.v_pool, a.block_table,
                       a.seq_lens, a.H, KVH, a.max_blocks_per_seq, a.num_blocks,
                       a.scale * kLog2e, part_o, part_ml, prefix, a.num_seqs, a.units);
  }
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int waves = a.num_seqs * a.H;
  hipLaunchKernelGGL((decode_merge_kernel<E, D>), dim3((waves + 3) / 4), dim3(256), 0, a.stream,
                     part_o, part_ml, prefix, a.num_seqs, a.H, a.units, (T*)a.o, a.lse);
  return hipGetLastError();
}

template <class E>
hipError_t launch_decode_e(const DecodeArgs& a) {
  return a.d == 64 ? launch_decode_ed<E, 64>(a) : launch_decode_ed<E, 128>(a);
}

hipError_t launch_decode(const DecodeArgs& a) {
  return a.dtype == 2 ? launch_decode_e<F16>(a) : launch_decode_e<Bf16>(a);
}

// ---------------------------------------------------------------------------
// Static scratch of the allocation-free decode: the same partials and prefix
// sums the workspace holds, in a file-scope device array that every GPU the
// library runs on keeps for the life of the process.  In host code `scratch`
// names a host-side stand-in, not device memory: its device address is taken
// once per device with hipGetSymbolAddress (with that device current) and only
// that address is handed to kernels.  Every decode kernel fully writes what it
// later reads (prefix sums, then each piece's partial), so nothing needs
// clearing between calls.
namespace {
__device__ __align__(256) unsigned char scratch[kNoAllocScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};
}  // namespace

hipError_t noalloc_scratch(void** ptr) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (p == nullptr) return hipErrorInvalidSymbol;
    g_scratch_ptr[dev] = p;
  }
  *ptr = g_scratch_ptr[dev];
  return hipSuccess;
}

}  // namespace fa
