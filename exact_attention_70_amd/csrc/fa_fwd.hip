// Attention forward for gfx950: tiled Q K^T on the matrix cores, online
// softmax, P V on the matrix cores, one pass over K/V per query tile.
//
// Method: dcwnkz.com GPU/FlashAttention explainer, section "FlashAttention"
// (tile along N so every block fits in on-chip memory; softmax per block with
// a running maximum and denominator; rescale the accumulated numerator and
// denominator by exp(m_old - m_new) when a block raises the maximum; divide
// once at the end; never revisit a block), and CMU 10-423 L17-L18 notes,
// sections "Prerequisite 2: online softmax" and "FlashAttention itself"
// (tiling + online softmax fused so the scores and probabilities never reach
// HBM).  The tiling itself is this file's own design for CDNA4.
//
// Work decomposition (bf16 kernel)
//   * one workgroup = 4 or 8 waves = a 128- or 256-row query tile of one
//     (batch, head) (8 waves for long sequences, causal tiles then paired);
//     wave w owns query rows [32w, 32w + 32) of the tile and keeps them in
//     registers as the B operands of S^T = K Q^T (loaded once from HBM).
//   * K/V stream through LDS in 64-key tiles by buffer-to-LDS DMA, one tile
//     ahead of use, in two-slot rings (V one tile behind K).  Rows are stored
//     with an XOR swizzle of their 16-byte chunks so that both the K operand
//     reads and the transposing V reads (ds_read_b64_tr_b16) are free of LDS
//     bank conflicts.
//   * each wave computes S^T = K Q^T (keys x its 32 queries) so that every
//     lane holds the scores of ONE query: the row max and row sum are
//     in-lane reductions plus one exchange with the other half-wave.
//   * the probabilities P^T are rounded to bf16 and fed straight back as the
//     B operand of O^T += V^T P^T, whose A operand (V^T) comes from transpose
//     reads of the row-major V tile.
//   * software pipeline: iteration j runs the matrix ops of S_j interleaved
//     with the exponentials of tile j-1, then P_{j-1} V_{j-1} with the rest of
//     those exponentials.  The probabilities are taken against a per-row
//     reference maximum that moves (and rescales the accumulated output) only
//     when a probability could exceed 2^kSlack, which the running probability
//     sum reveals without a per-tile maximum (see kSlack).  At d = 64 most
//     launches use a one-stage loop instead (each tile's scores, probabilities
//     and P V in turn), whose smaller register set lets more waves share a
//     SIMD (see SIMPLE).
//   * causal: key tiles entirely above the diagonal are never visited; only
//     tiles that straddle the diagonal (or the ragged end) are masked, in a
//     separate tail of the loop.
//   * workgroups are ordered heaviest-first within each head and mapped so
//     that one head's query tiles share an XCD (and its L2).
#include <algorithm>

#include "fa_device.h"
#include "fa_internal.h"
#include <type_traits>

namespace fa {

namespace {

constexpr int kBNDefault = 64;   // keys per K/V tile
constexpr int kOneStageMaxKeys = 4096;   // d = 64 rows up to this many keys: one-stage loop

constexpr int kKLead = 3;        // K operand reads in flight ahead of their matrix op
constexpr int kVLead = 2;        // V operand read pairs in flight ahead of their matrix op
// Probabilities are exp2(score * scale * log2(e) - m_ref) against a per-row
// reference m_ref and stay <= 2^kSlack: the reference moves (to the row's
// exact maximum over the tile at hand) only when a lane's running probability
// sum over a tile exceeds 2^kSlack, which every larger probability would cause.
constexpr float kSlack = 8.f;
constexpr float kSlackPow = 256.f;   // 2^kSlack

// Paged K/V source of a prefill: sequence s's queries are rows
// [q_start[s], q_start[s+1]) of the packed Q/O/LSE, its seq_lens[s] cached
// tokens (the chunk's own included) live in 16-token blocks of the pools
// [num_blocks, 16, KVH, D] named by block_table[s, :].
struct PagedKV {
  const int32_t* table;
  const int32_t* q_start;
  const int32_t* seq_lens;
  int H, KVH, max_blocks, num_blocks;
  int total_q;          // rows of the packed Q/O/LSE
  uint32_t pool_bytes;  // bytes of one pool when at most 2^31 (one resource per pool), else 0
  int num_seqs;
};

// Up to this many sequences, a prefill takes them longest first.
constexpr int kOrderSeqs = 64;

// The sequence at position p of a prefill's work order, and its chunk's first
// packed row, chunk length and cached length.  With at most kOrderSeqs
// sequences the order is by the keys an average query tile of the chunk reads
// (cached tokens minus half the chunk), most first, ties by index, so that the
// workgroups of the longest sequences start first rather than leave a tail
// behind them; lane i of the wave reads sequence i's entries and ranks it
// against the others, so the ranking costs no memory round trip beyond the
// one that fetches the chosen sequence's entries.  With more sequences they
// keep their own order.
struct SeqPick {
  int seq, q_begin, q_end, len;
};
__device__ __forceinline__ SeqPick pick_sequence(const PagedKV& pg, int p, int lane) {
  if (pg.num_seqs > kOrderSeqs)
    return SeqPick{p, pg.q_start[p], pg.q_start[p + 1], pg.seq_lens[p]};
  const bool live = lane < pg.num_seqs;
  const int qb = live ? pg.q_start[lane] : 0;
  const int qe = live ? pg.q_start[lane + 1] : 0;
  const int L = live ? pg.seq_lens[lane] : 0;
  const int key = L - (qe - qb) / 2;
  int rank = 0;
  for (int j = 0; j < pg.num_seqs; ++j) {
    const int kj = __builtin_amdgcn_readlane(key, j);
    rank += (kj > key || (kj == key && j < lane)) ? 1 : 0;
  }
  // the ranks of the live lanes are 0 .. num_seqs - 1, each once
  const unsigned long long hit = __ballot(live && rank == p);
  const int s = hit ? (int)__builtin_ctzll(hit) : p;
  return SeqPick{s, __builtin_amdgcn_readlane(qb, s), __builtin_amdgcn_readlane(qe, s),
                 __builtin_amdgcn_readlane(L, s)};
}

// Physical ids of the four 16-token blocks one 64-key tile spans (-1: past
// the sequence's table row).
struct TileIds {
  int b[4];
};

// Copy key rows [row0, row0 + ROWS) of one cached head of a paged sequence
// into a swizzled LDS tile.  The tile's four block ids arrive in `ids`
// (read from the table ahead of time).  Every transfer
// instruction covers RPI rows of a single block (RPI divides 16, row0 is a
// multiple of ROWS), so it gets a buffer resource over that physical block,
// sized to stop at the sequence's last valid token: slots past the length,
// bad block ids and rows past the table all read as zeros.
template <int D, int ROWS, int NWAVES, typename T>
__device__ __forceinline__ void dma_rows_paged(const T* pool, TileIds ids, int n_tok, int num_blocks,
                                               int kvh, int KVH, unsigned char* lds, int row0,
                                               int wave, int lane) {
  constexpr int DCH = D / 8;
  constexpr int RPI = 64 / DCH;
  constexpr int NI = ROWS / RPI;
  static_assert(16 % RPI == 0 && NI % NWAVES == 0, "instruction rows must stay inside a block");
  static_assert(ROWS == 64, "a tile spans four blocks");
  const uint32_t row_bytes = (uint32_t)KVH * D * 2;
#pragma unroll
  for (int ii = 0; ii < NI / NWAVES; ++ii) {
    const int ins = ii * NWAVES + wave;
    const int bi = (ins * RPI) >> 4;                // block of this instruction within the tile
    const int b = (row0 >> 4) + bi;
    const int phys = bi == 0 ? ids.b[0] : bi == 1 ? ids.b[1] : bi == 2 ? ids.b[2] : ids.b[3];
    const int valid = min(16, n_tok - (b << 4));    // tokens of this block inside the sequence
    const bool ok = (unsigned)phys < (unsigned)num_blocks && valid > 0;
    const auto r = make_rsrc(pool + (size_t)(ok ? phys : 0) * 16 * KVH * D,
                             ok ? (uint32_t)valid * row_bytes : 0u);
    const int rr = ins * RPI + lane / DCH;          // LDS row written by this lane
    const int c = (lane % DCH) ^ tile_swz<D>(rr);
    const int slot = (row0 + rr) & 15;
    dma16(r, lds + ins * 1024, (uint32_t)((slot * KVH + kvh) * D + c * 8) * 2);
  }
}

// dma_rows_paged through one buffer resource over the whole pool (pools of
// at most 2 GiB): every lane's offset is its row's place in its physical
// block, or 2^31, past the pool (which reads zeros), for a slot past the
// sequence's last token or a block id outside the pool.  No per-block
// resources are built, so the transfers cost a few vector operations per
// instruction instead of scalar address arithmetic per block.
template <int D, int ROWS, int NWAVES>
__device__ __forceinline__ void dma_rows_paged_flat(__amdgpu_buffer_rsrc_t pool, TileIds ids,
                                                    int n_tok, int num_blocks, int kvh, int KVH,
                                                    unsigned char* lds, int row0, int wave,
                                                    int lane) {
  constexpr int DCH = D / 8;
  constexpr int RPI = 64 / DCH;
  constexpr int NI = ROWS / RPI;
  static_assert(16 % RPI == 0 && NI % NWAVES == 0, "instruction rows must stay inside a block");
  static_assert(ROWS == 64, "a tile spans four blocks");
  const uint32_t blk_bytes = (uint32_t)16 * KVH * D * 2;
  // the tile's four block bases, once per call: an id outside the pool maps
  // to 2^31, past the pool (the flat path serves pools of at most 2^31
  // bytes), and stays there with the lane's in-block offset added
  uint32_t base[4];
#pragma unroll
  for (int q = 0; q < 4; ++q)
    base[q] = (unsigned)ids.b[q] < (unsigned)num_blocks ? (uint32_t)ids.b[q] * blk_bytes : 0x80000000u;
  // with the wave index known to be below NWAVES, each instruction's block
  // is a constant (or a choice of two) instead of a select over all four
  __builtin_assume(wave >= 0 && wave < NWAVES);
#pragma unroll
  for (int ii = 0; ii < NI / NWAVES; ++ii) {
    const int ins = ii * NWAVES + wave;
    const int bi = (ins * RPI) >> 4;                // block of this instruction within the tile
    const uint32_t bb = bi == 0 ? base[0] : bi == 1 ? base[1] : bi == 2 ? base[2] : base[3];
    const int rr = ins * RPI + lane / DCH;          // LDS row written by this lane
    const int tok = row0 + rr;
    const int c = (lane % DCH) ^ tile_swz<D>(rr);
    const uint32_t off = bb + (uint32_t)(((tok & 15) * KVH + kvh) * D + c * 8) * 2;
    dma16(pool, lds + ins * 1024, tok < n_tok ? off : 0x80000000u);
  }
}

// True when every probability pair g (key block g / 4), issued in slot
// g * pslots / npair, precedes the first P V op that reads its block (slot
// nq + (g / 4) * dt).
constexpr bool probs_before_use(int npair, int pslots, int nq, int dt) {
  for (int g = 0; g < npair; ++g)
    if (g * pslots / npair >= nq + (g / 4) * dt) return false;
  return true;
}

// Whether the first P V op of key block kb must first check the probability
// sum: true when some probability pair of block kb was issued after the last
// check (pairs issued in slots before a check are covered by it; pair g is
// issued in slot g * pslots / npair, and block b's first P V op sits in slot
// nq + b * dt).
constexpr bool check_before_block(int kb, int npair, int pslots, int nq, int dt) {
  int checked = 0;
  for (int b = 0; b <= kb; ++b) {
    const bool need = (4 * b + 3) * pslots / npair >= checked;
    if (b == kb) return need;
    if (need) checked = nq + b * dt;
  }
  return false;
}

template <class E, int D, bool CAUSAL, int BN, int OCC, bool PAGED = false, bool PAIRED = false,
          int NW = 4, bool FLAT = false, bool SIMPLE = false>
__global__ __launch_bounds__(64 * NW, OCC) void fwd_bf16_kernel(
    const typename E::elem* __restrict__ Q, const typename E::elem* __restrict__ K,
    const typename E::elem* __restrict__ V, typename E::elem* __restrict__ O,
    float* __restrict__ LSE, int N, int Nk, int delta, float scale_log2, int n_qtiles, PagedKV pg,
    int hgroup, int acc, int snake) {
  // scale_log2 = scale * log2(e): scores are handled in base 2.  N query rows
  // and Nk key rows per head; with CAUSAL, key j is visible to row i iff
  // j <= i + delta.  PAGED: one (sequence, head) per bh; N, Nk and delta are
  // that sequence's chunk length, cached length and cached length - chunk.
  // hgroup > 0: workgroups map to tiles by xcd_grouped with that group size.
  // acc != 0 (contiguous layout only): O and LSE hold on entry the running
  // result over other keys, and the epilogue merges this block's result into
  // them by the rescale rule instead of overwriting them.
  // PAIRED (causal only): the workgroup runs rank r (long) and then rank
  // n_qtiles - 1 - r (short) of one head, so every workgroup has the same work
  // and pays the per-tile start-up once per two tiles.  The long tiles of a
  // head start together and share its key stream in L2 (running the short
  // tile first staggered them and raised the reads from 1.46x to 1.70x the
  // bytes of Q, K and V).  The host pairs only when the paired grid still
  // fills the chip.  NW waves of 32 query rows each share every K/V tile the
  // workgroup streams through LDS.
  // SIMPLE (contiguous): one stage per K/V tile (scores, then
  // probabilities, then P V, all of the same tile) instead of the two-stage
  // pipeline that overlaps one tile's scores with the previous tile's
  // probabilities; it holds one score array instead of two, so more waves
  // fit on a SIMD.
  constexpr int BM = 32 * NW;            // query rows per workgroup
  constexpr int KSTEPS = D / 16;         // matrix k-steps over the head dim
  constexpr int DT = D / 32;             // 32-row tiles of O^T
  constexpr int TILE = BN * D * 2;       // bytes of one K or V tile
  constexpr int NSUB = BN / 32;          // 32-key sub-tiles per tile
  constexpr int NU = BN / 16;            // 16-key matrix k-steps of the P V product
  // Two-slot rings for K and for V, four separate objects so that reads of one
  // slot are never made to wait for transfers into another.
  __shared__ __attribute__((aligned(1024))) unsigned char sK0[TILE];
  __shared__ __attribute__((aligned(1024))) unsigned char sK1[TILE];
  __shared__ __attribute__((aligned(1024))) unsigned char sV0[TILE];
  __shared__ __attribute__((aligned(1024))) unsigned char sV1[TILE];

  static_assert(!PAIRED || (CAUSAL && !PAGED), "pairing is for the contiguous causal forward");
  static_assert(!SIMPLE || !PAGED, "the one-stage loop is for the contiguous forward");

  int tile0, tile1 = 0, npass = 1;
  if constexpr (PAIRED) {
    const int n_ranks = (n_qtiles + 1) / 2;
    const int t = hgroup > 0 ? xcd_grouped(blockIdx.x, n_ranks, hgroup)
                             : xcd_remap(blockIdx.x, gridDim.x);
    const int r = t % n_ranks, base = t / n_ranks * n_qtiles;
    tile0 = base + r;
    tile1 = base + n_qtiles - 1 - r;
    npass = tile1 != tile0 ? 2 : 1;
  } else {
    // snake != 0 (grouped order, whole grid resident, 32 k slots per XCD):
    // compute unit j of an XCD holds that XCD's slots j, j + 32, j + 64, ...,
    // so every other round of 32 slots is taken in reverse, and each unit
    // gets long and short tiles instead of all long or all short ones
    int b = blockIdx.x;
    if (snake) {
      const int xs = b >> 3, r = xs >> 5, p = xs & 31;
      b = (((r & 1) ? (r << 5) + 31 - p : xs) << 3) | (b & 7);
    }
    tile0 = hgroup > 0 ? xcd_grouped(b, n_qtiles, hgroup) : xcd_remap(b, gridDim.x);
  }
  // The softmax takes its maximum over raw scores and folds the scale into one
  // multiply-add, which needs a positive multiplier: for a negative scale,
  // each pass negates its Q (exact in bf16) and uses |scale|.  Masked scores
  // are -inf before that multiply, and -inf * 0 is NaN, so a zero scale is
  // raised to the smallest normal float: masked keys stay at -inf, and every
  // finite score below 2^99 in magnitude still gets probability exactly 1.
  const bool neg_scale = scale_log2 < 0.f;
  scale_log2 = fmaxf(fabsf(scale_log2), __FLT_MIN__);
  for (int pass = 0; pass < npass; ++pass) {
    if (pass) __syncthreads();                      // the first tile's LDS reads are done
    const int tile = pass ? tile1 : tile0;
    int tid = threadIdx.x;
    // paired: hide the thread index from loop-invariant code motion, so that
    // addresses derived from it are formed in each pass instead of being held
    // in registers across both
    if constexpr (PAIRED) asm volatile("" : "+v"(tid));
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // uniform: scalar addressing
    const int l32 = lane & 31;
    const int half = lane >> 5;
    const int bh = tile / n_qtiles;
    const int qt = CAUSAL ? (n_qtiles - 1 - tile % n_qtiles) : (tile % n_qtiles);
    const int q0 = qt * BM;

    // row strides of Q/O (elements) and LSE: one head's rows are contiguous, or
    // interleaved with the other heads in the packed layout of a prefill
    const int qstride = PAGED ? pg.H * D : D;
    const int lstride = PAGED ? pg.H : 1;
    size_t head_off, lse_off;
    uint32_t head_bytes, lse_bytes;
    int qrow0 = 0;                                    // packed row of the chunk's first query
    const int32_t* table_row = nullptr;
    int kvh = 0;
    if constexpr (PAGED) {
      // workgroups of head position x run on XCD x % 8; query heads that read
      // one cached head are consecutive, so the position is transposed over
      // the 8 XCDs to keep a cached head's query heads on one XCD (one L2)
      const int hx = bh % pg.H;
      const int h = (pg.H & 7) == 0 ? (hx & 7) * (pg.H >> 3) + (hx >> 3) : hx;
      const SeqPick sp = pick_sequence(pg, bh / pg.H, lane);
      const int seq = sp.seq, qs = sp.q_begin;
      N = sp.q_end - qs;
      // a length past the table row is clamped to the row's capacity (as the
      // decode does), so a corrupt length costs at most one row of blocks
      Nk = min(sp.len, pg.max_blocks * 16);
      delta = Nk - N;                                 // the chunk is the sequence's last tokens
      // a chunk outside the packed rows (malformed offsets) is skipped; so is a
      // query tile past the chunk
      if (qs < 0 || q0 >= N || qs > pg.total_q - N) return;
      qrow0 = qs;
      // resources over the whole packed tensors, from this head's column on:
      // nothing outside them is touched whatever the offsets say; rows past the
      // chunk (the next sequence's) are never stored
      head_off = (size_t)h * D;
      head_bytes = (uint32_t)(((size_t)pg.total_q * pg.H - h) * D * 2);
      lse_off = (size_t)h;
      lse_bytes = (uint32_t)(((size_t)pg.total_q * pg.H - h) * 4);
      table_row = pg.table + (size_t)seq * pg.max_blocks;
      kvh = h / (pg.H / pg.KVH);
    } else {
      head_off = (size_t)bh * (size_t)N * D;
      head_bytes = (uint32_t)N * D * 2;
      lse_off = (size_t)bh * N;
      lse_bytes = (uint32_t)N * 4;
    }
    const size_t khead_off = (size_t)bh * (size_t)Nk * D;
    const uint32_t khead_bytes = (uint32_t)Nk * D * 2;
    const auto rQ = make_rsrc(Q + head_off, head_bytes);
    // paged: one resource over each whole pool when FLAT, else none (each
    // transfer builds one over its block)
    const uint32_t kv_bytes = PAGED ? (FLAT ? pg.pool_bytes : 0u) : khead_bytes;
    const auto rK = make_rsrc(K + (PAGED ? 0 : khead_off), kv_bytes);
    const auto rV = make_rsrc(V + (PAGED ? 0 : khead_off), kv_bytes);
    const auto rO = make_rsrc(O + head_off, head_bytes);
    const auto rL = make_rsrc(LSE + lse_off, lse_bytes);
    // Paged: a tile's block ids are read from the table one iteration before
    // the transfers that use them (ids_v: tile j, ids_k: tile j+1, ids_f: tile
    // j+2, read during iteration j), so no transfer waits on a table read.  The
    // read index is clamped into the row (max_blocks >= 1) and entries past it
    // become -1, which the transfer turns into zeros.
    auto tile_ids = [&](int t) __attribute__((always_inline)) {
      TileIds r{{-1, -1, -1, -1}};
      if constexpr (PAGED) {
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int b = 4 * t + q;
          const int v = table_row[min(b, pg.max_blocks - 1)];
          r.b[q] = b < pg.max_blocks ? v : -1;
        }
      }
      return r;
    };
    TileIds ids_v = tile_ids(0), ids_k = tile_ids(1), ids_f = ids_k;
    // after a barrier (which has waited for the reads): the ids move to scalar
    // registers, leaving only the ids in flight in vector registers
    auto rotate_ids = [&]() __attribute__((always_inline)) {
      ids_v = ids_k;
#pragma unroll
      for (int q = 0; q < 4; ++q) ids_k.b[q] = __builtin_amdgcn_readfirstlane(ids_f.b[q]);
    };
    auto dma_k = [&](unsigned char* dst, int row0) __attribute__((always_inline)) {
      if constexpr (PAGED && FLAT)
        dma_rows_paged_flat<D, BN, NW>(rK, row0 == 0 ? ids_v : ids_k, Nk, pg.num_blocks, kvh,
                                       pg.KVH, dst, row0, wave, lane);
      else if constexpr (PAGED)
        dma_rows_paged<D, BN, NW>(K, row0 == 0 ? ids_v : ids_k, Nk, pg.num_blocks, kvh,
                                             pg.KVH, dst, row0, wave, lane);
      else
        dma_rows<D, BN, NW>(rK, dst, row0, wave, lane);
    };
    auto dma_v = [&](unsigned char* dst, int row0) __attribute__((always_inline)) {
      if constexpr (PAGED && FLAT)
        dma_rows_paged_flat<D, BN, NW>(rV, ids_v, Nk, pg.num_blocks, kvh, pg.KVH, dst, row0,
                                       wave, lane);
      else if constexpr (PAGED)
        dma_rows_paged<D, BN, NW>(V, ids_v, Nk, pg.num_blocks, kvh, pg.KVH, dst, row0,
                                             wave, lane);
      else
        dma_rows<D, BN, NW>(rV, dst, row0, wave, lane);
    };

    const int kv_end = CAUSAL ? min(Nk, q0 + BM + delta) : Nk;
    const int n_kv = kv_end > 0 ? (kv_end + BN - 1) / BN : 0;
    // tiles [0, n_full) need no masking for any row of this workgroup
    const int n_full = min(CAUSAL ? max(0, q0 + delta + 1) / BN : n_kv, Nk / BN);
    if (n_kv == 0) {
      // no row of this tile sees any key: empty softmax, O = 0 and LSE = -inf
      // (merged into a running result, an empty block changes nothing)
      const int row = q0 + tid / 2;
      if (!acc && tid < 2 * BM && (!PAGED || row < N)) {
        const uint32_t prow = (uint32_t)(qrow0 + row);
#pragma unroll
        for (int c = 0; c < D / 16; ++c)
          bstore16(u32x4{0u, 0u, 0u, 0u}, rO, (prow * qstride + (tid & 1) * (D / 2) + 8 * c) * 2);
        if ((tid & 1) == 0) bstore4f(kNegInf, rL, prow * lstride * 4);
      }
      continue;
    }

    // ---- this wave's query rows, straight from HBM into B-operand registers;
    //      K_0 and V_0 into ring slot 0
    dma_k(sK0, 0);
    dma_v(sV0, 0);
    const int my_q_row = q0 + wave * 32 + l32;
    u32x4 qf[KSTEPS];
#pragma unroll
    for (int s = 0; s < KSTEPS; ++s)
      qf[s] = bload16(rQ, ((uint32_t)(qrow0 + my_q_row) * qstride + 16 * s + 8 * half) * 2);
    if (neg_scale) {
#pragma unroll
      for (int s = 0; s < KSTEPS; ++s) qf[s] = qf[s] ^ 0x80008000u;
    }
    barrier_all();                                    // K_0, V_0 landed

    const int my_q = q0 + wave * 32 + l32;            // this lane's query row
    // transpose-read geometry of the V^T operand (see tile_off / ds_read_tr16)
    const int tr_row = 4 * half + ((lane & 15) >> 2);
    const int tr_col = 16 * ((lane >> 4) & 1) + 4 * (lane & 3);

    f32x16 o[DT];
#pragma unroll
    for (int t = 0; t < DT; ++t) o[t] = zero16();
    float m_run = kNegInf;   // reference maximum of scale*log2(e)*score (see kSlack)
    float neg_m = 0.f;       // -m_run, or 0 while the row has seen no key (m_run = -inf)
    float thr = 0.f;         // probability-sum threshold: 2^kSlack, or 0 while m_run = -inf
    float l_run = 0.f;       // this lane's share of the running denominator
    // Four-wave workgroups run two to a CU, so a SIMD's two waves belong to
    // different workgroups and the older one would win every issue tie.  The
    // wave priority tracks progress through an iteration instead (3 at its
    // start, 2 after the score ops, 1 halfway through the P V ops, 0 at the
    // end), so the wave that is behind is served first (4-5% faster at
    // B8 H12 N1024 d64 and B4 H16 N2048 d128).  Eight-wave workgroups hold
    // both waves of a SIMD behind one barrier, where it measured 2% slower.
    constexpr bool kProgressPrio = NW == 4;
    constexpr int NQ = NSUB * KSTEPS;     // matrix ops of S = K Q^T per tile
    constexpr int NP = DT * NU;           // matrix ops of O^T += V^T P^T per tile
    constexpr int KLEAD = kKLead;
    constexpr int VLEAD = kVLead;
    // Issue schedule of one iteration's vector work over its NQ + NP matrix-op
    // slots (S ops first, then P V ops ordered key block by key block).  The
    // probabilities of the previous tile come in NPAIR pairs, key block kb
    // being pairs [4kb, 4kb + 4); they are spread evenly over the first PSLOTS
    // slots, so block kb is done before the first P V op that reads it (slot
    // NQ + kb * DT).
    constexpr int NPAIR = NSUB * 8;
    constexpr int PSLOTS = NQ + NP - DT;
    static_assert(NPAIR == 4 * NU, "four probability pairs per key block");
    static_assert(probs_before_use(NPAIR, PSLOTS, NQ, DT), "a key block's probabilities come late");

    // Per-lane byte offsets of the operand reads inside a tile.  The swizzle
    // makes them differ per k-step (K) and per column block (V); sub-tile,
    // row-block and ring-slot offsets are compile-time constants added on top,
    // which the LDS instructions take as immediates.  The offsets are re-pinned
    // every iteration so they stay the only live copies.
    uint32_t kofs[KSTEPS], vofs[DT][2];
#pragma unroll
    for (int k = 0; k < KSTEPS; ++k) kofs[k] = tile_off<D>(l32, 2 * k + half);
#pragma unroll
    for (int t = 0; t < DT; ++t) {
      const int col = t * 32 + tr_col;
      vofs[t][0] = tile_off<D>(tr_row, col >> 3) + (col & 7) * 2;
      vofs[t][1] = tile_off<D>(tr_row + 8, col >> 3) + (col & 7) * 2;
    }
    auto pin_offsets = [&]() {
#pragma unroll
      for (int k = 0; k < KSTEPS; ++k) asm volatile("" : "+v"(kofs[k]));
#pragma unroll
      for (int t = 0; t < DT; ++t) asm volatile("" : "+v"(vofs[t][0]), "+v"(vofs[t][1]));
    };
    auto k_operand = [&](const unsigned char* sK, int idx) {
      const int t = idx / KSTEPS, k = idx % KSTEPS;
      return *(const u32x4*)(sK + kofs[k] + t * 32 * D * 2);
    };
    auto v_operand = [&](const unsigned char* sV, int idx) {
      const int t = idx / NU, u = idx % NU;
      const u32x2 lo = ds_read_tr16(sV + vofs[t][0] + u * 16 * D * 2);
      const u32x2 hi = ds_read_tr16(sV + vofs[t][1] + u * 16 * D * 2);
      const u32x4 a = {lo[0], lo[1], hi[0], hi[1]};
      return a;
    };
    // keys beyond this lane's row (causal) or beyond N become -inf
    auto mask = [&](f32x16 (&s)[NSUB], int kb) {
      const int lim = min(CAUSAL ? my_q + delta : Nk - 1, Nk - 1) - kb - 4 * half;
#pragma unroll
      for (int t = 0; t < NSUB; ++t)
#pragma unroll
        for (int i = 0; i < 16; ++i)
          if (t * 32 + 8 * (i >> 2) + (i & 3) > lim) s[t][i] = kNegInf;
    };
    // The row's maximum of a score tile, scaled to base 2 (both half-waves
    // hold keys of the same query rows, so they agree on it).
    auto tile_max = [&](const f32x16 (&s)[NSUB]) {
      float mx = kNegInf;
#pragma unroll
      for (int t = 0; t < NSUB; ++t)
#pragma unroll
        for (int i = 0; i < 16; i += 2) mx = fmaxf(mx, fmaxf(s[t][i], s[t][i + 1]));
      return half_max(mx) * scale_log2;
    };
    auto set_ref = [&](float m) {
      m_run = m;
      neg_m = m == kNegInf ? 0.f : -m;
      thr = m == kNegInf ? 0.f : kSlackPow;
    };
    // Probability pair g (keys of score registers s[g/8][2(g%8)], +1) against
    // the current reference, rounded to the element type; the denominator sums
    // the rounded values, so numerator and denominator see the same numbers.
    auto prob_pair = [&](const f32x16 (&s)[NSUB], u32x4 (&pb)[NU], float& rs, const int g)
        __attribute__((always_inline)) {
      const int t = g / 8, i = 2 * (g % 8);
      const float p0 = fast_exp2(fmaf(s[t][i], scale_log2, neg_m));
      const float p1 = fast_exp2(fmaf(s[t][i + 1], scale_log2, neg_m));
      const uint32_t pk = E::pack(p0, p1);
      rs = E::dot2(pk, E::kOnes, rs);
      pb[2 * t + (i >> 3)][(i & 7) >> 1] = pk;
    };
    // Rare path, taken by the whole wave when some lane's probability sum over
    // the pairs taken so far passed its threshold (a probability may exceed
    // 2^kSlack, or the row saw its first key).  Every row whose maximum over
    // the tile lies above its reference moves the reference there, rescales
    // the output and denominator accumulated so far by exp2(m_old - m_new)
    // (output already holding part of this tile included: all of it is on the
    // old reference), and the pairs already taken (issued in slots < upto) are
    // taken again.  Afterwards every probability of the tile is <= 1.
    auto raise_ref = [&](const f32x16 (&s)[NSUB], u32x4 (&pb)[NU], float& rs, const int upto)
        __attribute__((always_inline)) {
      const float cand = tile_max(s);
      if (cand > m_run) {
        const float alpha = fast_exp2(m_run - cand);   // 0 while m_run = -inf
#pragma unroll
        for (int t = 0; t < DT; ++t)
#pragma unroll
          for (int i = 0; i < 16; ++i) o[t][i] *= alpha;
        l_run *= alpha;
        set_ref(cand);
      }
      rs = 0.f;
#pragma unroll
      for (int g = 0; g < NPAIR; ++g)
        if (g * PSLOTS / NPAIR < upto) prob_pair(s, pb, rs, g);
    };
    auto over = [&](float rs) { return __builtin_amdgcn_ballot_w64(rs > thr) != 0; };

    // prologue: S_0, its max; K_1 streams meanwhile
    f32x16 sa[NSUB], sb[NSUB];
    if constexpr (!SIMPLE) {
    if constexpr (PAGED) ids_f = tile_ids(2);
    if (n_kv > 1) dma_k(sK1, BN);
    {
#pragma unroll
      for (int t = 0; t < NSUB; ++t) sa[t] = zero16();
#pragma unroll
      for (int idx = 0; idx < NQ; ++idx)
        sa[idx / KSTEPS] = E::mfma(k_operand(sK0, idx), qf[idx % KSTEPS], sa[idx / KSTEPS]);
      if (0 >= n_full) mask(sa, 0);
      set_ref(tile_max(sa));
    }
    __syncthreads();
    if constexpr (PAGED) rotate_ids();
    }

    // Iteration j: S_j = K_j Q^T on the matrix cores interleaved with the
    // probabilities P_{j-1} (exponentials), then O^T += V_{j-1}^T P_{j-1}^T
    // with the rest of them.  Before the first P V op of a key block whose
    // probabilities have not all been checked, the probability sum is tested
    // against the threshold (raise_ref on the rare hit).  K_j is in slot j&1,
    // V_{j-1} in slot (j-1)&1; K_{j+1} and V_j stream into the other slots.
    auto iter = [&](const int j, const unsigned char* kcur, unsigned char* knxt,
                    const unsigned char* vprev, unsigned char* vcur, f32x16 (&so)[NSUB],
                    f32x16 (&sn)[NSUB], auto masked) {
      pin_offsets();
      if constexpr (kProgressPrio) __builtin_amdgcn_s_setprio(3);
      if constexpr (PAGED) ids_f = tile_ids(j + 2);
      if (j + 1 < n_kv) dma_k(knxt, (j + 1) * BN);
      dma_v(vcur, j * BN);
      u32x4 pb[NU];
      float rs = 0.f;
      u32x4 ka[KLEAD];
#pragma unroll
      for (int x = 0; x < KLEAD; ++x) ka[x] = k_operand(kcur, (x % NSUB) * KSTEPS + x / NSUB);
#pragma unroll
      for (int t = 0; t < NSUB; ++t) sn[t] = zero16();
      // probability pair g of the previous tile (scores so), in the slot the
      // schedule gives it
      auto probs = [&](const int slot) __attribute__((always_inline)) {
#pragma unroll
        for (int g = 0; g < NPAIR; ++g)
          if (g * PSLOTS / NPAIR == slot) prob_pair(so, pb, rs, g);
      };
      // the NSUB accumulator chains in turn (op idx: sub-tile idx % NSUB,
      // k-step idx / NSUB): a matrix op does not wait for the result of the
      // one issued just before it (2% faster than one chain after the other)
      auto kidx = [](int idx) { return (idx % NSUB) * KSTEPS + idx / NSUB; };
#pragma unroll
      for (int idx = 0; idx < NQ; ++idx) {
        const u32x4 a = ka[idx % KLEAD];
        if (idx + KLEAD < NQ) ka[idx % KLEAD] = k_operand(kcur, kidx(idx + KLEAD));
        sn[idx % NSUB] = E::mfma(a, qf[idx / NSUB], sn[idx % NSUB]);
        probs(idx);
      }
      if constexpr (decltype(masked)::value) mask(sn, j * BN);
      if constexpr (kProgressPrio) __builtin_amdgcn_s_setprio(2);
      // P V op ip reads key block ip / DT and writes output column block ip % DT
      auto vidx = [](int ip) { return (ip % DT) * NU + ip / DT; };
      u32x4 va[VLEAD];
#pragma unroll
      for (int x = 0; x < VLEAD; ++x) va[x] = v_operand(vprev, vidx(x));
#pragma unroll
      for (int ip = 0; ip < NP; ++ip) {
        if (ip % DT == 0 && check_before_block(ip / DT, NPAIR, PSLOTS, NQ, DT))
          if (__builtin_expect(over(rs), 0)) raise_ref(so, pb, rs, NQ + ip);
        const u32x4 a = va[ip % VLEAD];
        if (ip + VLEAD < NP) va[ip % VLEAD] = v_operand(vprev, vidx(ip + VLEAD));
        o[ip % DT] = E::mfma(a, pb[ip / DT], o[ip % DT]);
        probs(NQ + ip);
        if constexpr (kProgressPrio)
          if (ip == NP / 2) __builtin_amdgcn_s_setprio(1);
      }
      if constexpr (kProgressPrio) __builtin_amdgcn_s_setprio(0);
      l_run += rs;
      __syncthreads();
      if constexpr (PAGED) rotate_ids();
    };
    using Plain = std::integral_constant<bool, false>;
    using Masked = std::integral_constant<bool, true>;
    int j = 1;
    const int n_plain = max(1, min(n_full, n_kv));   // iterations [1, n_plain) need no mask
    if constexpr (!SIMPLE)
    for (; j + 1 < n_plain; j += 2) {
      iter(j, sK1, sK0, sV0, sV1, sa, sb, Plain{});
      iter(j + 1, sK0, sK1, sV1, sV0, sb, sa, Plain{});
    }
    // epilogue: P V of the last tile (its V sits in slot (n_kv-1)&1, its
    // scores in sa when n_kv-1 is even, else sb)
    auto last_pv = [&](const f32x16 (&sl)[NSUB], const unsigned char* vl) {
      u32x4 pb[NU];
      float rs = 0.f;
#pragma unroll
      for (int g = 0; g < NPAIR; ++g) prob_pair(sl, pb, rs, g);
      if (over(rs)) raise_ref(sl, pb, rs, PSLOTS);
      l_run += rs;
#pragma unroll
      for (int idx = 0; idx < NP; ++idx)
        o[idx / NU] = E::mfma(v_operand(vl, idx), pb[idx % NU], o[idx / NU]);
    };
    // The rest (at most one unmasked tile plus the tiles that straddle the
    // diagonal or the ragged end) runs with the mask on.  j is odd here, so
    // pairs keep the ring slots and score arrays static.  Causal: no row of
    // this wave sees a key past tile n_wave - 1 (its last row's diagonal), so
    // the wave computes up to that tile only; for the workgroup's remaining
    // tiles it just issues its share of the transfers and joins the barriers.
    // n_wave >= n_plain, as the unmasked tiles are seen by every row.
    int n_wave = n_kv;
    if constexpr (CAUSAL) {
      const int last_key = q0 + wave * 32 + 31 + delta;   // last key a row of the wave sees
      n_wave = min(n_kv, last_key >= 0 ? last_key / BN + 1 : 1);
    }
    if constexpr (SIMPLE) {
      // One stage per tile: S_j, its probabilities, then P_j V_j, with K_j
      // and V_j in slot j & 1 while tile j + 1 streams into the other slots.
      // A wave overlaps nothing of its own, but needs one score array instead
      // of two, which lets three (4-wave workgroups) or four (8-wave) waves share a SIMD
      // to hide each other's waits.
      auto simple_iter = [&](const int jj, const unsigned char* kc, const unsigned char* vc,
                             unsigned char* kn, unsigned char* vn) __attribute__((always_inline)) {
        if (jj + 1 < n_kv) {
          dma_k(kn, (jj + 1) * BN);
          dma_v(vn, (jj + 1) * BN);
        }
        if (jj < n_wave) {
          pin_offsets();
          if constexpr (kProgressPrio) __builtin_amdgcn_s_setprio(3);
          auto kidx = [](int idx) { return (idx % NSUB) * KSTEPS + idx / NSUB; };
          u32x4 ka[KLEAD];
#pragma unroll
          for (int x = 0; x < KLEAD; ++x) ka[x] = k_operand(kc, kidx(x));
#pragma unroll
          for (int idx = 0; idx < NQ; ++idx) {
            const u32x4 a = ka[idx % KLEAD];
            if (idx + KLEAD < NQ) ka[idx % KLEAD] = k_operand(kc, kidx(idx + KLEAD));
            sa[idx % NSUB] = E::mfma(a, qf[idx / NSUB], idx < NSUB ? zero16() : sa[idx % NSUB]);
          }
          if (jj >= n_full) mask(sa, jj * BN);
          if (jj == 0) set_ref(tile_max(sa));
          if constexpr (kProgressPrio) __builtin_amdgcn_s_setprio(1);
          last_pv(sa, vc);
          if constexpr (kProgressPrio) __builtin_amdgcn_s_setprio(0);
        }
        __syncthreads();
      };
      for (int jj = 0; jj < n_kv; jj += 2) {
        simple_iter(jj, sK0, sV0, sK1, sV1);
        if (jj + 1 < n_kv) simple_iter(jj + 1, sK1, sV1, sK0, sV0);
      }
    } else {
    for (; j + 1 < n_wave; j += 2) {
      iter(j, sK1, sK0, sV0, sV1, sa, sb, Masked{});
      iter(j + 1, sK0, sK1, sV1, sV0, sb, sa, Masked{});
    }
    if (j < n_wave) {
      iter(j, sK1, sK0, sV0, sV1, sa, sb, Masked{});
      last_pv(sb, sV1);          // last tile j is odd
    } else {
      last_pv(sa, sV0);          // last tile j-1 is even
    }
    // transfers and barriers of tiles [n_wave, n_kv): K_{i+1} into slot
    // (i+1)&1 and V_i into slot i&1, as iteration i issues them
    auto idle_iter = [&](const int i, unsigned char* knxt, unsigned char* vcur) {
      if constexpr (PAGED) ids_f = tile_ids(i + 2);
      if (i + 1 < n_kv) dma_k(knxt, (i + 1) * BN);
      dma_v(vcur, i * BN);
      __syncthreads();
      if constexpr (PAGED) rotate_ids();
    };
    int i = n_wave;
    if (i < n_kv && (i & 1)) idle_iter(i++, sK0, sV1);
    for (; i + 1 < n_kv; i += 2) {
      idle_iter(i, sK1, sV0);
      idle_iter(i + 1, sK0, sV1);
    }
    if (i < n_kv) idle_iter(i, sK1, sV0);
    }

    // ---- epilogue: O = O^T / l, LSE = ln(sum exp) = (m + log2 l) ln 2
    const float l_tot = half_sum(l_run);
    // a row that saw no key (l = 0) gets O = 0 and LSE = -inf
    float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
    float lse_out = l_tot > 0.f ? (m_run + fast_log2(l_tot)) * kLn2 : kNegInf;
    // acc: weights of the running result (a) and of this block (b) in base 2,
    // w = exp2(LSE2 - max); O = c_a O_a + c_b O_b with c = w / (w_a + w_b),
    // LSE = max + log2(w_a + w_b); a side at -inf weighs nothing
    float ca = 0.f;
    if (acc) {
      const float la = bload4f(rL, (uint32_t)(qrow0 + my_q) * lstride * 4);
      const float la2 = la * kLog2e;
      const float lb2 = l_tot > 0.f ? m_run + fast_log2(l_tot) : kNegInf;
      const float M = fmaxf(la2, lb2);
      const bool empty = M == kNegInf;
      const float wa = empty ? 0.f : fast_exp2(la2 - M);
      const float wb = empty ? 0.f : fast_exp2(lb2 - M);
      const float itot = empty ? 0.f : 1.f / (wa + wb);
      ca = wa * itot;
      inv *= wb * itot;
      // a block of weight 0 leaves the running LSE exactly as it was
      lse_out = empty ? kNegInf : wb == 0.f ? la : (M + fast_log2(wa + wb)) * kLn2;
    }
    // O leaves through LDS so that every store instruction writes whole rows:
    // a lane holds one query's values spread over the head dim, and storing
    // them directly would write 16-byte pieces of 32 rows per instruction.
    // Each wave stages its 32 x D tile (swizzled 16-byte chunks) in a quarter
    // of the K/V rings, once every wave is done reading them, and then stores
    // it row-major with 16 bytes per lane.
    constexpr int CPR = D * 2 / 16;       // 16-byte chunks per row
    constexpr int RPS = 64 / CPR;         // rows per store instruction
    constexpr int SW = 32 * D * 2;        // staging bytes per wave (half a ring slot)
    static_assert(2 * SW == TILE && NW <= 8, "two waves' staging per ring slot");
    barrier_lds();
    unsigned char* stage = ((wave >> 1) == 0 ? sK0 : (wave >> 1) == 1 ? sK1
                            : (wave >> 1) == 2 ? sV0 : sV1) + (wave & 1) * SW;
    // the lane index again, hidden from the optimizer: values derived from it
    // here are formed here rather than held across the loop
    int elane = threadIdx.x & 63;
    asm volatile("" : "+v"(elane));
    const int el32 = elane & 31, ehalf = elane >> 5;
#pragma unroll
    for (int t = 0; t < DT; ++t)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        u32x2 w;
        w[0] = E::pack(o[t][4 * g] * inv, o[t][4 * g + 1] * inv);
        w[1] = E::pack(o[t][4 * g + 2] * inv, o[t][4 * g + 3] * inv);
        const int c = t * 4 + g;          // chunk of d0 = t * 32 + 8 * g + 4 * half
        *(u32x2*)(stage + el32 * (D * 2) + ((c ^ (el32 % CPR)) << 4) + 8 * ehalf) = w;
      }
    if (!acc) {
#pragma unroll
      for (int k = 0; k < 32 / RPS; ++k) {
        const int r = k * RPS + elane / CPR, c = elane % CPR;
        const u32x4 w = *(const u32x4*)(stage + r * (D * 2) + ((c ^ (r % CPR)) << 4));
        const int row = q0 + wave * 32 + r;
        if (!PAGED || row < N) bstore16(w, rO, ((uint32_t)(qrow0 + row) * qstride + 8 * c) * 2);
      }
    } else {
      // the running rows first (all loads in flight together), then
      // c_a O_a + (c_b O_b as staged), with c_a of row r from lane r
      u32x4 old[32 / RPS];
#pragma unroll
      for (int k = 0; k < 32 / RPS; ++k) {
        const int r = k * RPS + elane / CPR, c = elane % CPR;
        old[k] = bload16(rO, ((uint32_t)(qrow0 + q0 + wave * 32 + r) * qstride + 8 * c) * 2);
      }
#pragma unroll
      for (int k = 0; k < 32 / RPS; ++k) {
        const int r = k * RPS + elane / CPR, c = elane % CPR;
        const u32x4 w = *(const u32x4*)(stage + r * (D * 2) + ((c ^ (r % CPR)) << 4));
        const float car = __builtin_bit_cast(
            float, __builtin_amdgcn_ds_bpermute(r << 2, __builtin_bit_cast(int, ca)));
        // a running row of weight 0 (LSE -inf on entry) is not read into the
        // result, whatever its O holds
        if (car == 0.f) old[k] = u32x4{0u, 0u, 0u, 0u};
        u32x4 m;
#pragma unroll
        for (int e = 0; e < 4; ++e)
          m[e] = E::pack(fmaf(car, E::lo(old[k][e]), E::lo(w[e])),
                         fmaf(car, E::hi(old[k][e]), E::hi(w[e])));
        bstore16(m, rO, ((uint32_t)(qrow0 + q0 + wave * 32 + r) * qstride + 8 * c) * 2);
      }
    }
    if (half == 0 && (!PAGED || my_q < N))
      bstore4f(lse_out, rL, (uint32_t)(qrow0 + my_q) * lstride * 4);
  }
}

// ---------------------------------------------------------------------------
// fp32 forward: same tiling idea with the fp32 matrix instruction
// (v_mfma_f32_32x32x2f32).  One workgroup = one wave = 32 query rows; K/V
// tiles of 32 keys in LDS.  Both matrix operands take one element per lane,
// so no transposed copy of V is needed.

constexpr int kF32BM = 32;
constexpr int kF32BN = 32;

template <int D>
__global__ __launch_bounds__(64) void fwd_f32_kernel(
    const float* __restrict__ Q, const float* __restrict__ K, const float* __restrict__ V,
    float* __restrict__ O, float* __restrict__ LSE, int N, int Nk, int delta, float scale_log2,
    int causal, int n_qtiles, int acc) {
  constexpr int KSTEPS = D / 2;
  constexpr int DT = D / 32;
  constexpr int PAD = 1;                         // one-float row pad: conflict-free column reads
  __shared__ float sK[kF32BN][D + PAD];
  __shared__ float sV[kF32BN][D + PAD];

  const int lane = threadIdx.x;
  const int l32 = lane & 31;
  const int half = lane >> 5;
  const int tile = blockIdx.x;
  const int bh = tile / n_qtiles;
  const int q0 = (tile % n_qtiles) * kF32BM;
  const size_t head_off = (size_t)bh * (size_t)N * D;
  const size_t khead_off = (size_t)bh * (size_t)Nk * D;
  const uint32_t head_bytes = (uint32_t)N * D * 4;
  const uint32_t khead_bytes = (uint32_t)Nk * D * 4;
  const auto rQ = make_rsrc(Q + head_off, head_bytes);
  const auto rK = make_rsrc(K + khead_off, khead_bytes);
  const auto rV = make_rsrc(V + khead_off, khead_bytes);
  const auto rO = make_rsrc(O + head_off, head_bytes);
  const auto rL = make_rsrc(LSE + (size_t)bh * N, (uint32_t)N * 4);

  const int my_q = q0 + l32;
  // B operand of S^T = K Q^T: lane holds Q[my_q][2k + half]
  float qf[KSTEPS];
#pragma unroll
  for (int k = 0; k < KSTEPS; ++k) qf[k] = bload4f(rQ, (uint32_t)(my_q * D + 2 * k + half) * 4);

  f32x16 o[DT];
#pragma unroll
  for (int t = 0; t < DT; ++t) o[t] = zero16();
  float m_run = kNegInf, l_run = 0.f;

  const int kv_end = causal ? min(Nk, q0 + kF32BM + delta) : Nk;   // may be <= 0: no key
  for (int kb = 0; kb < kv_end; kb += kF32BN) {
    __syncthreads();
    for (int e = lane; e < kF32BN * D / 4; e += 64) {
      const int row = e / (D / 4), c4 = e % (D / 4);
      const u32x4 kv4 = bload16(rK, (uint32_t)((kb + row) * D + c4 * 4) * 4);
      const u32x4 vv4 = bload16(rV, (uint32_t)((kb + row) * D + c4 * 4) * 4);
#pragma unroll
      for (int x = 0; x < 4; ++x) {
        sK[row][c4 * 4 + x] = as_f32(kv4[x]);
        sV[row][c4 * 4 + x] = as_f32(vv4[x]);
      }
    }
    __syncthreads();

    f32x16 s = zero16();
#pragma unroll
    for (int k = 0; k < KSTEPS; ++k) s = mfma_f32(sK[l32][2 * k + half], qf[k], s);

    float mx = kNegInf;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int key = kb + 8 * (i >> 2) + 4 * half + (i & 3);
      float x = s[i] * scale_log2;
      if ((causal && key > my_q + delta) || key >= Nk) x = kNegInf;
      s[i] = x;
      mx = fmaxf(mx, x);
    }
    mx = half_max(mx);
    const float m_new = fmaxf(m_run, mx);
    const float m_use = (m_new == kNegInf) ? 0.f : m_new;
    const float alpha = fast_exp2(m_run - m_use);
    m_run = m_new;
    float rs = 0.f;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      s[i] = fast_exp2(s[i] - m_use);
      rs += s[i];
    }
    l_run = l_run * alpha + rs;
#pragma unroll
    for (int t = 0; t < DT; ++t)
#pragma unroll
      for (int i = 0; i < 16; ++i) o[t][i] *= alpha;
    // O^T[d][q] += sum_key V[key][d] P^T[key][q]; k-step i pairs the keys
    // held in register i by the two half-waves.
#pragma unroll
    for (int t = 0; t < DT; ++t)
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int key = 8 * (i >> 2) + 4 * half + (i & 3);
        o[t] = mfma_f32(sV[key][t * 32 + l32], s[i], o[t]);
      }
  }

  const float l_tot = half_sum(l_run);
  float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;   // no visible key: O = 0
  float lse_out = l_tot > 0.f ? (m_run + fast_log2(l_tot)) * kLn2 : kNegInf;
  float ca = 0.f;   // acc: the running result's weight (as in the 16-bit kernel)
  if (acc) {
    const float la = bload4f(rL, (uint32_t)my_q * 4);
    const float la2 = la * kLog2e;
    const float lb2 = l_tot > 0.f ? m_run + fast_log2(l_tot) : kNegInf;
    const float M = fmaxf(la2, lb2);
    const bool empty = M == kNegInf;
    const float wa = empty ? 0.f : fast_exp2(la2 - M);
    const float wb = empty ? 0.f : fast_exp2(lb2 - M);
    const float itot = empty ? 0.f : 1.f / (wa + wb);
    ca = wa * itot;
    inv *= wb * itot;
    lse_out = empty ? kNegInf : wb == 0.f ? la : (M + fast_log2(wa + wb)) * kLn2;
  }
#pragma unroll
  for (int t = 0; t < DT; ++t)
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const int d0 = t * 32 + 8 * g + 4 * half;
      const uint32_t off = (uint32_t)(my_q * D + d0) * 4;
      u32x4 w;
      if (acc) {
        u32x4 old = bload16(rO, off);
        if (ca == 0.f) old = u32x4{0u, 0u, 0u, 0u};   // weight 0: O not read in
#pragma unroll
        for (int x = 0; x < 4; ++x) w[x] = as_u32(fmaf(ca, as_f32(old[x]), o[t][4 * g + x] * inv));
      } else {
#pragma unroll
        for (int x = 0; x < 4; ++x) w[x] = as_u32(o[t][4 * g + x] * inv);
      }
      bstore16(w, rO, off);
    }
  if (half == 0) bstore4f(lse_out, rL, (uint32_t)my_q * 4);
}

// ---------------------------------------------------------------------------
// Empty result for query rows that see no key at all: O = 0, LSE = -inf.
template <typename T>
__global__ __launch_bounds__(256) void fill_empty_kernel(T* __restrict__ O, float* __restrict__ LSE,
                                                         long long rows, int d) {
  const long long n = rows * d;
  for (long long i = (long long)blockIdx.x * 256 + threadIdx.x; i < n; i += (long long)gridDim.x * 256)
    O[i] = T(0.f);
  for (long long r = (long long)blockIdx.x * 256 + threadIdx.x; r < rows; r += (long long)gridDim.x * 256)
    LSE[r] = kNegInf;
}

// ---------------------------------------------------------------------------
// Merge of two partial results over disjoint key sets (the rescale rule):
// M = max(LSE_a, LSE_b), w = exp(LSE - M), O = (w_a O_a + w_b O_b) / (w_a + w_b),
// LSE = M + ln(w_a + w_b); a side at LSE = -inf weighs nothing.  One thread
// handles 16 bytes of a row; a row's threads sit in one wave, so the output
// may be the same buffer as either input.  Every O byte is touched once, so
// the 16-byte loads and stores carry the non-temporal hint: streamed data
// then does not displace other lines from the caches (on MI355X this took
// the merge of 32 x 8192 rows of d = 128 from 50 to 36 us).
template <typename T>
struct Traits16 { using type = Bf16; };
template <>
struct Traits16<_Float16> { using type = F16; };

template <typename T, int D>
__global__ __launch_bounds__(256) void merge_kernel(const T* Oa, const float* La, const T* Ob,
                                                    const float* Lb, T* O, float* L, long long rows) {
  constexpr int EPT = 16 / sizeof(T);      // elements per thread
  constexpr int TPR = D / EPT;             // threads per row (<= 32)
  const long long gid = (long long)blockIdx.x * 256 + threadIdx.x;
  const long long row = gid / TPR;
  const int c = (int)(gid % TPR);
  if (row >= rows) return;
  const float la = La[row], lb = Lb[row];
  const float M = fmaxf(la, lb);
  const bool empty = M == kNegInf;
  const float wa = empty ? 0.f : fast_exp2((la - M) * kLog2e);
  const float wb = empty ? 0.f : fast_exp2((lb - M) * kLog2e);
  const float tot = wa + wb;
  const float inv = empty ? 0.f : 1.f / tot;
  const float ca = wa * inv, cb = wb * inv;
  const long long off = row * D + (long long)c * EPT;
  u32x4 a = __builtin_nontemporal_load((const u32x4*)(Oa + off));
  u32x4 b = __builtin_nontemporal_load((const u32x4*)(Ob + off));
  // a side of weight 0 is not read into the result, whatever its O holds
  if (ca == 0.f) a = u32x4{0u, 0u, 0u, 0u};
  if (cb == 0.f) b = u32x4{0u, 0u, 0u, 0u};
  u32x4 r;
  if constexpr (sizeof(T) == 2) {
#pragma unroll
    for (int e = 0; e < 4; ++e)
    {
      using E = typename Traits16<T>::type;
      r[e] = E::pack(ca * E::lo(a[e]) + cb * E::lo(b[e]), ca * E::hi(a[e]) + cb * E::hi(b[e]));
    }
  } else {
#pragma unroll
    for (int e = 0; e < 4; ++e) r[e] = as_u32(ca * as_f32(a[e]) + cb * as_f32(b[e]));
  }
  __builtin_nontemporal_store(r, (u32x4*)(O + off));
  if (c == 0) L[row] = empty ? kNegInf : M + fast_log2(tot) * kLn2;
}

// Launch shape of the contiguous 16-bit forward: waves per workgroup (32
// query rows each) and whether causal tiles are paired.
struct FwdPlan {
  int nw;
  bool paired;
};

FwdPlan fwd_plan(long long heads, int N, bool causal) {
  // Long sequences take 256-row workgroups, which halve the K/V tile
  // transfers and LDS writes per flop, as long as the grid still gives every
  // compute unit a workgroup; causal tiles are then always paired.  Below
  // that, 128-row workgroups, paired when the paired grid keeps four
  // workgroups per compute unit.
  const long long t8 = (N + 255) / 256, t4 = (N + 127) / 128;
  if (N >= 4096 && heads * (causal ? (t8 + 1) / 2 : t8) >= 256) return FwdPlan{8, causal};
  return FwdPlan{4, causal && heads * ((t4 + 1) / 2) >= 4 * 256};
}

template <class E, int D, bool CAUSAL, int NW, bool PAIRED>
hipError_t launch_bf16_as(const FwdArgs& a, int Nk, int delta) {
  using T = typename E::elem;
  constexpr int BM = 32 * NW;
  const int n_qtiles = (a.N + BM - 1) / BM;
  const long long units = (long long)a.B * a.H * (PAIRED ? (n_qtiles + 1) / 2 : n_qtiles);
  // causal tiles differ in length: interleave heads so long tiles start first
  const int hg = CAUSAL ? xcd_group((long long)a.B * a.H, (long long)Nk * D * 4) : 0;
  // d = 64 in 8-wave workgroups: the one-stage loop (124 registers), so two
  // workgroups share a CU, four waves per SIMD: 3-9% faster than the
  // two-stage loop at B1-B4 H32-H64 N4096-N16384
  if constexpr (D == 64 && NW == 8) {
    hipLaunchKernelGGL((fwd_bf16_kernel<E, D, CAUSAL, kBNDefault, 4, false, PAIRED, 8, false, true>),
                       dim3((int)units), dim3(64 * NW), 0, a.stream, (const T*)a.Q, (const T*)a.K,
                       (const T*)a.V, (T*)a.O, a.LSE, a.N, Nk, delta, a.scale * kLog2e, n_qtiles,
                       PagedKV{}, hg, a.accumulate ? 1 : 0, 0);
    return hipGetLastError();
  }
  // d = 64 with at most 4096 keys: the one-stage loop at three waves per
  // SIMD (122 registers), 3-18% faster on such shapes (B8 H32 N2048 causal
  // 215 -> 198 us); longer rows keep the two-stage loop
  if constexpr (D == 64 && NW == 4 && !PAIRED) {
    if (Nk <= kOneStageMaxKeys) {
      // three workgroups per CU: a grid of at most 768 is resident at once
      const int snake = hg > 0 && units % 256 == 0 && units <= 3 * 256;
      hipLaunchKernelGGL((fwd_bf16_kernel<E, D, CAUSAL, kBNDefault, 3, false, false, 4, false, true>),
                         dim3((int)units), dim3(64 * NW), 0, a.stream, (const T*)a.Q, (const T*)a.K,
                         (const T*)a.V, (T*)a.O, a.LSE, a.N, Nk, delta, a.scale * kLog2e, n_qtiles,
                         PagedKV{}, hg, a.accumulate ? 1 : 0, snake);
      return hipGetLastError();
    }
  }
  // two waves per SIMD whatever the workgroup size
  hipLaunchKernelGGL((fwd_bf16_kernel<E, D, CAUSAL, kBNDefault, 8 / NW, false, PAIRED, NW>),
                     dim3((int)units), dim3(64 * NW), 0, a.stream, (const T*)a.Q, (const T*)a.K,
                     (const T*)a.V, (T*)a.O, a.LSE, a.N, Nk, delta, a.scale * kLog2e, n_qtiles,
                     PagedKV{}, hg, a.accumulate ? 1 : 0, 0);
  return hipGetLastError();
}

template <class E, int D, bool CAUSAL>
hipError_t launch_bf16(const FwdArgs& a, int Nk, int delta) {
  const FwdPlan p = fwd_plan((long long)a.B * a.H, a.N, CAUSAL);
  if constexpr (CAUSAL) {
    // d = 64 rows of at most 4096 keys take the unpaired one-stage kernel
    // even where 4-wave tiles would pair: 7-15% faster at B16-B64 H12-H16
    // N512-N1024 (three workgroups per CU balance the tile lengths well)
    const bool one_stage = D == 64 && p.nw == 4 && Nk <= kOneStageMaxKeys;
    if (p.paired && !one_stage)
      return p.nw == 8 ? launch_bf16_as<E, D, true, 8, true>(a, Nk, delta)
                       : launch_bf16_as<E, D, true, 4, true>(a, Nk, delta);
  }
  return p.nw == 8 ? launch_bf16_as<E, D, CAUSAL, 8, false>(a, Nk, delta)
                   : launch_bf16_as<E, D, CAUSAL, 4, false>(a, Nk, delta);
}

template <class E, int D, bool CAUSAL>
hipError_t launch_paged(const FwdArgs& a) {
  using T = typename E::elem;
  constexpr int NW = 4;                                // 128 query rows per workgroup
  const int n_qtiles = (a.N + 32 * NW - 1) / (32 * NW);  // a.N: the longest chunk
  const int grid = a.B * a.H * n_qtiles;                // a.B: the number of sequences
  // pools of at most 2 GiB are read through one resource each (offsets of
  // 2^31 then read zeros)
  const unsigned long long pool_bytes = (unsigned long long)a.num_blocks * 16 * a.KVH * D * 2;
  const bool flat = pool_bytes <= 0x80000000ull;
  const PagedKV pg{a.table,      a.q_start,    a.seq_lens,  a.H,
                   a.KVH,        a.max_blocks, a.num_blocks, a.total_q,
                   flat ? (uint32_t)pool_bytes : 0u, a.B};
  // the query heads of one cached head share its K/V stream in one L2 (the
  // kernel keeps them on one XCD when H is a multiple of 8)
  const long long share = (a.H % 8 == 0) ? a.H / a.KVH : 1;
  const int hg =
      CAUSAL ? xcd_group((long long)a.B * a.H, (long long)a.max_blocks * 16 * D * 4 / share) : 0;
  if (flat)
    hipLaunchKernelGGL((fwd_bf16_kernel<E, D, CAUSAL, kBNDefault, 2, true, false, NW, true>),
                       dim3(grid), dim3(64 * NW), 0, a.stream, (const T*)a.Q, (const T*)a.K,
                       (const T*)a.V, (T*)a.O, a.LSE, 0, 0, 0, a.scale * kLog2e, n_qtiles, pg, hg, 0, 0);
  else
    hipLaunchKernelGGL((fwd_bf16_kernel<E, D, CAUSAL, kBNDefault, 2, true, false, NW>), dim3(grid),
                       dim3(64 * NW), 0, a.stream, (const T*)a.Q, (const T*)a.K, (const T*)a.V,
                       (T*)a.O, a.LSE, 0, 0, 0, a.scale * kLog2e, n_qtiles, pg, hg, 0, 0);
  return hipGetLastError();
}

template <class E>
hipError_t launch_paged_e(const FwdArgs& a) {
  if (a.d == 64) return a.causal ? launch_paged<E, 64, true>(a) : launch_paged<E, 64, false>(a);
  return a.causal ? launch_paged<E, 128, true>(a) : launch_paged<E, 128, false>(a);
}

template <class E>
hipError_t launch_16(const FwdArgs& a, int Nk, int delta, bool causal) {
  if (a.d == 64)
    return causal ? launch_bf16<E, 64, true>(a, Nk, delta) : launch_bf16<E, 64, false>(a, Nk, delta);
  return causal ? launch_bf16<E, 128, true>(a, Nk, delta) : launch_bf16<E, 128, false>(a, Nk, delta);
}

template <int D>
hipError_t launch_f32(const FwdArgs& a, int Nk, int delta, bool causal) {
  const int n_qtiles = (a.N + kF32BM - 1) / kF32BM;
  const int grid = a.B * a.H * n_qtiles;
  hipLaunchKernelGGL((fwd_f32_kernel<D>), dim3(grid), dim3(64), 0, a.stream,
                     (const float*)a.Q, (const float*)a.K, (const float*)a.V, (float*)a.O, a.LSE,
                     a.N, Nk, delta, a.scale * kLog2e, causal ? 1 : 0, n_qtiles, a.accumulate ? 1 : 0);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_fwd(const FwdArgs& a) {
  if (a.paged) return a.dtype == 2 ? launch_paged_e<F16>(a) : launch_paged_e<Bf16>(a);
  const int Nk = a.Nk > 0 ? a.Nk : a.N;
  bool causal = a.causal;
  // every key at or before every query: the mask is void
  if (causal && a.delta >= (long long)Nk - 1) causal = false;
  if (causal && a.delta + a.N - 1 < 0) {
    // no query sees any key: merged into a running result, nothing changes
    if (a.accumulate) return hipSuccess;
    const long long rows = (long long)a.B * a.H * a.N;
    const long long n = rows * a.d;
    const int grid = (int)std::min<long long>((n + 255) / 256, 65536);
    if (a.dtype == 1)
      hipLaunchKernelGGL((fill_empty_kernel<__bf16>), dim3(grid), dim3(256), 0, a.stream,
                         (__bf16*)a.O, a.LSE, rows, a.d);
    else if (a.dtype == 2)
      hipLaunchKernelGGL((fill_empty_kernel<_Float16>), dim3(grid), dim3(256), 0, a.stream,
                         (_Float16*)a.O, a.LSE, rows, a.d);
    else
      hipLaunchKernelGGL((fill_empty_kernel<float>), dim3(grid), dim3(256), 0, a.stream,
                         (float*)a.O, a.LSE, rows, a.d);
    return hipGetLastError();
  }
  const int delta = causal ? (int)a.delta : 0;   // |delta| < max(N, Nk) here
  if (a.dtype == 1) return launch_16<Bf16>(a, Nk, delta, causal);
  if (a.dtype == 2) return launch_16<F16>(a, Nk, delta, causal);
  return a.d == 64 ? launch_f32<64>(a, Nk, delta, causal) : launch_f32<128>(a, Nk, delta, causal);
}

hipError_t launch_merge(const MergeArgs& a) {
  const int tpr = a.d * (a.dtype != 0 ? 2 : 4) / 16;
  const long long threads = a.rows * tpr;
  const unsigned grid = (unsigned)((threads + 255) / 256);
  if (a.dtype == 1) {
    if (a.d == 64)
      hipLaunchKernelGGL((merge_kernel<__bf16, 64>), dim3(grid), dim3(256), 0, a.stream,
                         (const __bf16*)a.Oa, a.La, (const __bf16*)a.Ob, a.Lb, (__bf16*)a.O, a.L, a.rows);
    else
      hipLaunchKernelGGL((merge_kernel<__bf16, 128>), dim3(grid), dim3(256), 0, a.stream,
                         (const __bf16*)a.Oa, a.La, (const __bf16*)a.Ob, a.Lb, (__bf16*)a.O, a.L, a.rows);
  } else if (a.dtype == 2) {
    if (a.d == 64)
      hipLaunchKernelGGL((merge_kernel<_Float16, 64>), dim3(grid), dim3(256), 0, a.stream,
                         (const _Float16*)a.Oa, a.La, (const _Float16*)a.Ob, a.Lb, (_Float16*)a.O,
                         a.L, a.rows);
    else
      hipLaunchKernelGGL((merge_kernel<_Float16, 128>), dim3(grid), dim3(256), 0, a.stream,
                         (const _Float16*)a.Oa, a.La, (const _Float16*)a.Ob, a.Lb, (_Float16*)a.O,
                         a.L, a.rows);
  } else {
    if (a.d == 64)
      hipLaunchKernelGGL((merge_kernel<float, 64>), dim3(grid), dim3(256), 0, a.stream,
                         (const float*)a.Oa, a.La, (const float*)a.Ob, a.Lb, (float*)a.O, a.L, a.rows);
    else
      hipLaunchKernelGGL((merge_kernel<float, 128>), dim3(grid), dim3(256), 0, a.stream,
                         (const float*)a.Oa, a.La, (const float*)a.Ob, a.Lb, (float*)a.O, a.L, a.rows);
  }
  return hipGetLastError();
}

}  // namespace fa

