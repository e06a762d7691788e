// Attention backward with recomputation for gfx950 (bf16 in, fp32 gradients).
//
// Method: CMU 10-423 L17-L18 notes, section "FlashAttention itself" (never
// store the attention matrix; recompute the needed block in the backward
// pass) and the dcwnkz.com explainer, recomputation technique (trade extra
// arithmetic for memory traffic).  Each tile of P is rebuilt as
// exp(scale * Q K^T - LSE) from the forward's per-row log-sum-exp, so no
// max/sum pass is repeated and nothing of size N x N is written.  The
// gradients are the chain rule of O = softmax(S) V, S = scale Q K^T:
//   dV = P^T dO,  dP = dO V^T,  D_i = sum_d dO_id O_id,  dS = P o (dP - D),
//   dQ = scale dS K,  dK = scale dS^T Q.
//
// Two kernels, both on the caller's stream, deterministic (no atomics):
//   1. bwd_dq:   workgroup = 128 queries (wave = 32; two workgroups per CU,
//      three at d = 64); loops over 64-key K/V tiles;
//      recomputes S^T = K Q^T and dP^T = V dO^T (each lane then holds one
//      query's row, so LSE_i and D_i are per-lane scalars) and accumulates
//      dQ^T += K^T dS^T.  Within a tile the exponentials run between the dP
//      matrix ops, and each 16-key step's dS feeds its dQ ops at once.  Its
//      prologue forms D_i = rowsum(dO o O) and -LSE_i log2(e) for its rows
//      and writes them into the workspace for the second kernel.
//   2. bwd_dkdv: workgroup = 128 keys (wave = 32 keys); loops over 64-row
//      query tiles; recomputes S = Q K^T and dP = dO V^T with this wave's K
//      and V rows held in registers, and accumulates dV^T += dO^T P and
//      dK^T += Q^T dS on the matrix cores.  Q, dO, LSE and D tiles stream into
//      LDS by buffer->LDS transfers through a three-slot ring, one tile ahead;
//      Q^T and dO^T come from transpose reads.  Each 32-key block has a dV
//      wave and a dK wave on one SIMD (P passes between them through LDS),
//      so one wave's exponentials run beside the other's matrix ops.
// Causal: tiles wholly above the diagonal are skipped; straddling tiles masked.
#include "fa_device.h"
#include "fa_internal.h"
#include <type_traits>

namespace fa {

namespace {

constexpr int kThreads = 256;

// Direct buffer -> LDS copy of one dword per lane (lane i lands at lds + 4 i).
__device__ __forceinline__ void dma4(__amdgpu_buffer_rsrc_t r, void* lds, uint32_t off) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void*)lds, 4, (int)off, 0, 0, 0);
}

// Transpose-read operand (lane: one column of a 32-row tile of a row-major bf16
// tile, 8 consecutive rows 16u + 8a + 4h + c): two ds_read_b64_tr_b16 reads.
// The row order matches the C-layout of a 32 x 32 score tile, so the result
// pairs slot-for-slot with a C-layout tile fed back as the B operand.
template <int D>
__device__ __forceinline__ u32x4 tr_operand(const unsigned char* tile, int u, int t, int lane) {
  const int half = lane >> 5;
  const int row = 16 * u + 4 * half + ((lane & 15) >> 2);
  const int col = t * 32 + 16 * ((lane >> 4) & 1) + 4 * (lane & 3);
  const u32x2 lo = ds_read_tr16(tile + tile_off<D>(row, col >> 3) + (col & 7) * 2);
  const u32x2 hi = ds_read_tr16(tile + tile_off<D>(row + 8, col >> 3) + (col & 7) * 2);
  return u32x4{lo[0], lo[1], hi[0], hi[1]};
}

// ---------------------------------------------------------------- dK, dV
// Workgroup = 128 keys, eight waves.  Each 32-key block has a dV wave (waves
// 0-3) and a dK wave (waves 4-7), so a wave holds one of the two gradient
// accumulators and one of K, V, and two waves share every SIMD.  64-row query
// tiles (Q, dO, -LSE log2 e, D) stream into a three-slot LDS ring by
// buffer->LDS transfers, one tile ahead.  Iteration i:
//   dV wave: dV^T += dO^T P of tile i-1 (its P kept in registers), then for
//            tile i S = Q K^T (rows = queries, columns = the block's keys) and
//            P = exp2(scale log2(e) S - LSE log2(e)), rounded to the element
//            type (as P is for P V in the forward) and handed to the block's
//            dK wave through LDS;
//   dK wave: for tile i-1 dP = dO V^T, dS = P o (dP - D) with that P, and
//            dK^T += Q^T dS.
// So one wave's exponentials run beside the other's matrix ops: matrix,
// matrix, vector for the dV wave against matrix, vector, matrix for the dK
// wave.  dO^T and Q^T come from transpose reads.  Both waves issue 32 matrix
// ops per tile.  P passes through two LDS buffers (by tile parity), so the
// dK wave reads tile i-1's while the dV wave writes tile i's and the roles
// meet at one barrier per iteration.
constexpr int kKvBN = 128;   // keys per workgroup
constexpr int kKvBQ = 64;    // queries per inner tile
constexpr int kKvWaves = 8;

template <class E, int D, bool CAUSAL>
__global__ __launch_bounds__(kKvWaves * 64, 1) void bwd_dkdv_kernel(
    const typename E::elem* __restrict__ Q, const typename E::elem* __restrict__ K,
    const typename E::elem* __restrict__ V, const typename E::elem* __restrict__ dO,
    const float* __restrict__ NL, const float* __restrict__ Dvec,
    float* __restrict__ dK, float* __restrict__ dV, int N, float scale, float scale_log2,
    int n_ktiles, int hgroup) {
  constexpr int KSTEPS = D / 16;
  constexpr int DT = D / 32;
  constexpr int TILE = kKvBQ * D * 2;
  constexpr int NU = kKvBQ / 16;           // 16-query k-steps of the dV / dK products
  constexpr int NA = 2 * KSTEPS;           // matrix ops of S (or dP) per tile
  constexpr int NC = NU * DT;              // matrix ops of dV (or dK) per tile
  constexpr int LEAD = 4;                  // operand reads in flight ahead of their matrix op
  __shared__ __attribute__((aligned(1024))) unsigned char sQ0[TILE], sQ1[TILE], sQ2[TILE];
  __shared__ __attribute__((aligned(1024))) unsigned char sO0[TILE], sO1[TILE], sO2[TILE];
  __shared__ __attribute__((aligned(256))) float sL0[kKvBQ], sL1[kKvBQ], sL2[kKvBQ];
  __shared__ __attribute__((aligned(256))) float sD0[kKvBQ], sD1[kKvBQ], sD2[kKvBQ];
  // P of tile i for key block b: sP[i & 1][b][k-step][lane] (16 bytes per
  // lane and k-step, lane-contiguous:
  // conflict-free 16-byte writes and reads).  Two buffers let the dV wave
  // write tile i's P while the dK wave still reads tile i-1's.
  // One object indexed by the tile's parity, not two chosen by a select: a
  // pointer chosen between two objects may point at either, so the compiler
  // cannot tell it from the ring slots and made the P accesses wait for every
  // transfer in flight (the next tile's included).
  __shared__ __attribute__((aligned(1024))) u32x4 sP[2][4][NU][64];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const bool dk_wave = wave >= 4;
  const int blk = wave & 3;                       // this wave's 32-key block
  const int l32 = lane & 31, half = lane >> 5;
  const int tile = hgroup > 0 ? xcd_grouped(blockIdx.x, n_ktiles, hgroup)
                             : xcd_remap(blockIdx.x, gridDim.x);
  const int bh = tile / n_ktiles;
  const int kb = (tile % n_ktiles) * kKvBN;       // low key tiles see the most queries
  const int my_k = kb + blk * 32 + l32;           // this lane's key (C-layout column)

  const size_t head_off = (size_t)bh * (size_t)N * D;
  const uint32_t head_bytes = (uint32_t)N * D * 2;
  const auto rQ = make_rsrc(Q + head_off, head_bytes);
  const auto rK = make_rsrc(K + head_off, head_bytes);
  const auto rV = make_rsrc(V + head_off, head_bytes);
  const auto rdO = make_rsrc(dO + head_off, head_bytes);
  const auto rL = make_rsrc(NL + (size_t)bh * N, (uint32_t)N * 4);
  const auto rD = make_rsrc(Dvec + (size_t)bh * N, (uint32_t)N * 4);
  const auto rdK = make_rsrc(dK + head_off, (uint32_t)N * D * 4);
  const auto rdV = make_rsrc(dV + head_off, (uint32_t)N * D * 4);

  const int q_first = CAUSAL ? kb : 0;            // earlier queries see none of these keys
  const int n_q = (N - q_first + kKvBQ - 1) / kKvBQ;
  // the ring slot of tile i is i % 3; slots are separate objects so that reads
  // of one are never made to wait for transfers into another
  auto slotQ = [&](auto c) -> unsigned char* {
    if constexpr (decltype(c)::value == 0) return sQ0;
    else if constexpr (decltype(c)::value == 1) return sQ1;
    else return sQ2;
  };
  auto slotO = [&](auto c) -> unsigned char* {
    if constexpr (decltype(c)::value == 0) return sO0;
    else if constexpr (decltype(c)::value == 1) return sO1;
    else return sO2;
  };
  auto slotL = [&](auto c) -> float* {
    if constexpr (decltype(c)::value == 0) return sL0;
    else if constexpr (decltype(c)::value == 1) return sL1;
    else return sL2;
  };
  auto slotD = [&](auto c) -> float* {
    if constexpr (decltype(c)::value == 0) return sD0;
    else if constexpr (decltype(c)::value == 1) return sD1;
    else return sD2;
  };
  // Tiles past the end read as zeros (buffer range check); q0 stays far
  // below 2^31 / (2 D) for any N the library accepts.
  auto load = [&](int i, auto c) __attribute__((always_inline)) {
    const int q0 = q_first + i * kKvBQ;
    dma_rows<D, kKvBQ, kKvWaves>(rQ, slotQ(c), q0, wave, lane);
    dma_rows<D, kKvBQ, kKvWaves>(rdO, slotO(c), q0, wave, lane);
    dma4(rL, slotL(c), (uint32_t)(q0 + lane) * 4);
    dma4(rD, slotD(c), (uint32_t)(q0 + lane) * 4);
  };
  load(0, std::integral_constant<int, 0>{});

  // this wave's 32 keys as B operands (B[k = d][n = key]): K rows for S in a
  // dV wave, V rows for dP in a dK wave
  u32x4 kv[KSTEPS];
  {
    const auto& r = dk_wave ? rV : rK;
#pragma unroll
    for (int s = 0; s < KSTEPS; ++s) kv[s] = bload16(r, (uint32_t)(my_k * D + 16 * s + 8 * half) * 2);
  }
  f32x16 acc[DT];   // dV^T (dV wave) or dK^T (dK wave)
#pragma unroll
  for (int t = 0; t < DT; ++t) acc[t] = zero16();
  // per-lane LDS byte offsets: 16-byte row reads (per k-step) and transpose
  // reads (per 32-column block); sub-tile / row-block offsets are compile-time
  // immediates on top.  Re-pinned every tile.
  uint32_t rofs[KSTEPS], tofs[DT][2];
#pragma unroll
  for (int k = 0; k < KSTEPS; ++k) rofs[k] = tile_off<D>(l32, 2 * k + half);
  {
    const int row = 4 * half + ((lane & 15) >> 2);
#pragma unroll
    for (int t = 0; t < DT; ++t) {
      const int col = t * 32 + 16 * ((lane >> 4) & 1) + 4 * (lane & 3);
      tofs[t][0] = tile_off<D>(row, col >> 3) + (col & 7) * 2;
      tofs[t][1] = tile_off<D>(row + 8, col >> 3) + (col & 7) * 2;
    }
  }
  auto pin_offsets = [&]() __attribute__((always_inline)) {
#pragma unroll
    for (int k = 0; k < KSTEPS; ++k) asm volatile("" : "+v"(rofs[k]));
#pragma unroll
    for (int t = 0; t < DT; ++t) asm volatile("" : "+v"(tofs[t][0]), "+v"(tofs[t][1]));
  };
  barrier_all();

  // S (dV wave) or dP (dK wave) of a tile: rows = queries, columns = keys;
  // operand idx: 32-query sub-tile idx % 2, k-step idx / 2 (two accumulator
  // chains in turn)
  auto stage_a = [&](const unsigned char* rows, f32x16 (&s)[2]) __attribute__((always_inline)) {
    u32x4 ring[LEAD];
#pragma unroll
    for (int x = 0; x < LEAD; ++x)
      ring[x] = *(const u32x4*)(rows + rofs[x / 2] + (x % 2) * 32 * D * 2);
#pragma unroll
    for (int idx = 0; idx < NA; ++idx) {
      const u32x4 a = ring[idx % LEAD];
      if (idx + LEAD < NA) {
        const int nx = idx + LEAD;
        ring[idx % LEAD] = *(const u32x4*)(rows + rofs[nx / 2] + (nx % 2) * 32 * D * 2);
      }
      const int sub = idx % 2, k = idx / 2;
      s[sub] = E::mfma(a, kv[k], k == 0 ? zero16() : s[sub]);
    }
  };
  // acc^T += cols^T B with cols^T from transpose reads; op idx: k-step idx / DT,
  // column block idx % DT
  auto stage_c = [&](const unsigned char* cols, const u32x4 (&b)[NU]) __attribute__((always_inline)) {
    auto op = [&](int idx) {
      const int u = idx / DT, t = idx % DT;
      const u32x2 lo = ds_read_tr16(cols + tofs[t][0] + u * 16 * D * 2);
      const u32x2 hi = ds_read_tr16(cols + tofs[t][1] + u * 16 * D * 2);
      return u32x4{lo[0], lo[1], hi[0], hi[1]};
    };
    u32x4 ring[LEAD];
#pragma unroll
    for (int x = 0; x < LEAD; ++x) ring[x] = op(x);
#pragma unroll
    for (int idx = 0; idx < NC; ++idx) {
      const u32x4 a = ring[idx % LEAD];
      if (idx + LEAD < NC) ring[idx % LEAD] = op(idx + LEAD);
      acc[idx % DT] = E::mfma(a, b[idx / DT], acc[idx % DT]);
    }
  };
  // score element e of this lane: sub-tile e / 16, C-layout register e % 16,
  // query row sub * 32 + 8 g + 4 half + x of the tile; its pair sits in word
  // (g & 1) * 2 + (x >> 1) of B-operand k-step 2 sub + (g >> 1)

  // dV wave: S and P of tile i in ring slot c into pb, and to the dK wave
  auto dv_probs = [&](int i, auto c, u32x4 (&pb)[NU]) __attribute__((always_inline)) {
    pin_offsets();
    const int q0 = q_first + i * kKvBQ;
    f32x16 s[2];
    stage_a(slotQ(c), s);
    const float* sL = slotL(c);
    // keys past a query (causal) or queries past N get P = 0
    const bool masked = (CAUSAL && q0 < kb + blk * 32 + 31) || q0 + kKvBQ > N;
    auto probs = [&](auto mk) __attribute__((always_inline)) {
      f32x4 nl4;
      float pv0 = 0.f;
#pragma unroll
      for (int e = 0; e < 32; ++e) {
        const int sub = e / 16, i2 = e % 16, g = i2 / 4, x = i2 % 4;
        const int r0 = sub * 32 + 8 * g + 4 * half;
        if (x == 0) nl4 = *(const f32x4*)(sL + r0);
        float p = fast_exp2(fmaf(s[sub][i2], scale_log2, nl4[x]));
        if constexpr (decltype(mk)::value) {
          const int q = q0 + r0 + x;
          if ((CAUSAL && my_k > q) || q >= N) p = 0.f;
        }
        if (x & 1) pb[2 * sub + (g >> 1)][(g & 1) * 2 + (x >> 1)] = E::pack(pv0, p);
        else pv0 = p;
      }
    };
    if (masked) probs(std::integral_constant<bool, true>{});
    else probs(std::integral_constant<bool, false>{});
#pragma unroll
    for (int u = 0; u < NU; ++u) sP[i & 1][blk][u][lane] = pb[u];
  };
  // dK wave: tile j (one behind) in ring slot c, with that tile's P in pb
  auto dk_tile = [&](auto c, const u32x4 (&pb)[NU]) __attribute__((always_inline)) {
    pin_offsets();
    f32x16 dp[2];
    stage_a(slotO(c), dp);
    u32x4 db[NU];
    const float* sD = slotD(c);
    f32x4 d4;
    float dv0 = 0.f;
#pragma unroll
    for (int e = 0; e < 32; ++e) {
      const int sub = e / 16, i2 = e % 16, g = i2 / 4, x = i2 % 4;
      const int r0 = sub * 32 + 8 * g + 4 * half;
      if (x == 0) d4 = *(const f32x4*)(sD + r0);
      const uint32_t w = pb[2 * sub + (g >> 1)][(g & 1) * 2 + (x >> 1)];
      const float p = (x & 1) ? E::hi(w) : E::lo(w);
      const float ds = p * (dp[sub][i2] - d4[x]);
      if (x & 1) db[2 * sub + (g >> 1)][(g & 1) * 2 + (x >> 1)] = E::pack(dv0, ds);
      else dv0 = ds;
    }
    stage_c(slotQ(c), db);
  };
  // iteration i: tile i + 1 streams into slot (i + 1) % 3 (which held tile
  // i - 2, finished last iteration); tile i sits in slot i % 3 and tile i - 1
  // in slot (i + 2) % 3.  The dV wave writes the P of tile i into the buffer
  // of i's parity while the dK wave reads that of tile i - 1 from the other,
  // so the two roles meet only at the barrier that closes an iteration (with
  // a single P buffer a mid-iteration barrier kept the matrix pipe idle while
  // the dK wave read P, about a quarter of each iteration).  The two roles
  // run separate loops (so that neither carries the other's registers) with
  // the same barriers.
  auto run = [&](auto body) __attribute__((always_inline)) {
    auto iter = [&](int i, auto c) __attribute__((always_inline)) {
      constexpr int C = decltype(c)::value;
      // issued every iteration (past the end it reads zeros)
      load(i + 1, std::integral_constant<int, (C + 1) % 3>{});
      body(i, c, std::integral_constant<int, (C + 2) % 3>{});
      barrier_all();   // tile i + 1 landed; P of tile i written; slot of tile i - 1 free
    };
    using C0 = std::integral_constant<int, 0>;
    using C1 = std::integral_constant<int, 1>;
    using C2 = std::integral_constant<int, 2>;
    int i = 0;
    for (; i + 2 <= n_q; i += 3) {
      iter(i, C0{});
      iter(i + 1, C1{});
      iter(i + 2, C2{});
    }
    if (i <= n_q) iter(i, C0{});
    if (i + 1 <= n_q) iter(i + 1, C1{});
  };
  if (!dk_wave) {
    u32x4 pkeep[NU];   // P of the previous tile
    run([&](int i, auto c, auto cprev) __attribute__((always_inline)) {
      if (i >= 1) {
        pin_offsets();
        stage_c(slotO(cprev), pkeep);
      }
      if (i < n_q) dv_probs(i, c, pkeep);
    });
  } else {
    run([&](int i, auto c, auto cprev) __attribute__((always_inline)) {
      if (i >= 1) {
        u32x4 pb[NU];
#pragma unroll
        for (int u = 0; u < NU; ++u) pb[u] = sP[(i & 1) ^ 1][blk][u][lane];
        dk_tile(cprev, pb);
      }
    });
  }

  // store: lane holds key my_k, rows d = 32t + 8g + 4*half + (0..3).  Once
  // the last transfers have landed and every wave is done with the rings, each
  // wave stages its 32 x D tile in one ring slot or P buffer (sQ0..2 and sP[0]
  // for the dV waves, sO0..2 and sP[1] for the dK waves) and stores it as whole
  // rows.
  static_assert(32 * D * 4 == TILE, "one wave's fp32 tile per ring slot");
  static_assert(sizeof(sP[0]) >= 32 * D * 4, "one wave's fp32 tile per P buffer");
  barrier_all();
  unsigned char* stage =
      dk_wave ? (blk == 0 ? sO0 : blk == 1 ? sO1 : blk == 2 ? sO2 : (unsigned char*)sP[1])
              : (blk == 0 ? sQ0 : blk == 1 ? sQ1 : blk == 2 ? sQ2 : (unsigned char*)sP[0]);
  store_rows_f32<D, DT>(acc, dk_wave ? scale : 1.f, stage, dk_wave ? rdK : rdV,
                        kb + blk * 32, lane);
}

// ---------------------------------------------------------------- dQ
// Workgroup = 128 queries (wave = 32, Q and dO rows in registers as B
// operands); loops over 64-key K/V tiles streamed into LDS, double-buffered.
// Per tile and wave: S^T = K Q^T and dP^T = V dO^T (each lane holds one
// query's row, so LSE_i and D_i are per-lane scalars), dS^T = P^T o (dP^T - D),
// dQ^T += K^T dS^T with K^T from transpose reads.
constexpr int kQBM = 128;   // queries per workgroup
constexpr int kQBN = 64;    // keys per tile

// The dQ kernel runs first and also forms, for its rows, D = rowsum(dO o O)
// and -LSE log2(e), which it writes for the dK/dV kernel: each lane holds half
// of its row's dO as B operands, loads the same half of O, and the two halves
// meet in one cross-lane exchange.
// d = 64 fits in 168 registers (160-166), so three workgroups share a CU
// (the d = 64 backward 1-7% faster); d = 128 needs all 256 for two.
template <class E, int D, bool CAUSAL>
__global__ __launch_bounds__(kThreads, (D == 64 ? 3 : 2)) void bwd_dq_kernel(
    const typename E::elem* __restrict__ Q, const typename E::elem* __restrict__ K,
    const typename E::elem* __restrict__ V, const typename E::elem* __restrict__ O,
    const typename E::elem* __restrict__ dO, const float* __restrict__ LSE,
    float* __restrict__ Dvec, float* __restrict__ NLvec,
    float* __restrict__ dQ, int N, float scale, float scale_log2, int n_qtiles, int hgroup) {
  constexpr int KSTEPS = D / 16;
  constexpr int DT = D / 32;
  constexpr int TILE = kQBN * D * 2;
  __shared__ __attribute__((aligned(1024))) unsigned char sK0[TILE];
  __shared__ __attribute__((aligned(1024))) unsigned char sK1[TILE];
  __shared__ __attribute__((aligned(1024))) unsigned char sV0[TILE];
  __shared__ __attribute__((aligned(1024))) unsigned char sV1[TILE];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int l32 = lane & 31, half = lane >> 5;
  const int tile = hgroup > 0 ? xcd_grouped(blockIdx.x, n_qtiles, hgroup)
                             : xcd_remap(blockIdx.x, gridDim.x);
  const int bh = tile / n_qtiles;
  const int qt = CAUSAL ? (n_qtiles - 1 - tile % n_qtiles) : (tile % n_qtiles);
  const int q0 = qt * kQBM;
  const int my_q = q0 + wave * 32 + l32;
  const int wave_qlast = q0 + wave * 32 + 31;

  const size_t head_off = (size_t)bh * (size_t)N * D;
  const uint32_t head_bytes = (uint32_t)N * D * 2;
  const auto rQ = make_rsrc(Q + head_off, head_bytes);
  const auto rK = make_rsrc(K + head_off, head_bytes);
  const auto rV = make_rsrc(V + head_off, head_bytes);
  const auto rdO = make_rsrc(dO + head_off, head_bytes);
  const auto rO = make_rsrc(O + head_off, head_bytes);
  const auto rL = make_rsrc(LSE + (size_t)bh * N, (uint32_t)N * 4);
  const auto rD = make_rsrc(Dvec + (size_t)bh * N, (uint32_t)N * 4);
  const auto rNL = make_rsrc(NLvec + (size_t)bh * N, (uint32_t)N * 4);
  const auto rdQ = make_rsrc(dQ + head_off, (uint32_t)N * D * 4);

  const int kv_end = CAUSAL ? min(N, q0 + kQBM) : N;
  const int n_kv = (kv_end + kQBN - 1) / kQBN;
  auto load = [&](int j, unsigned char* sK, unsigned char* sV) {
    dma_rows<D, kQBN, kThreads / 64>(rK, sK, j * kQBN, wave, lane);
    dma_rows<D, kQBN, kThreads / 64>(rV, sV, j * kQBN, wave, lane);
  };
  load(0, sK0, sV0);
  u32x4 qf[KSTEPS], dof[KSTEPS];
  float Di = 0.f;
  {
    u32x4 of[KSTEPS];
#pragma unroll
    for (int s = 0; s < KSTEPS; ++s) {
      qf[s] = bload16(rQ, (uint32_t)(my_q * D + 16 * s + 8 * half) * 2);
      dof[s] = bload16(rdO, (uint32_t)(my_q * D + 16 * s + 8 * half) * 2);
      of[s] = __builtin_amdgcn_raw_buffer_load_b128(rO, (int)((my_q * D + 16 * s + 8 * half) * 2),
                                                    0, kCpolNT);   // O is read once
    }
#pragma unroll
    for (int s = 0; s < KSTEPS; ++s)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        Di = fmaf(E::lo(of[s][e]), E::lo(dof[s][e]), Di);
        Di = fmaf(E::hi(of[s][e]), E::hi(dof[s][e]), Di);
      }
    Di = half_sum(Di);                // with the other half of the row's head dim
  }
  const float neg_lse2 = -bload4f(rL, (uint32_t)my_q * 4) * kLog2e;
  if (half == 0) {                    // rows past N fall outside the resources
    bstore4f(Di, rD, (uint32_t)my_q * 4);
    bstore4f(neg_lse2, rNL, (uint32_t)my_q * 4);
  }
  f32x16 dq[DT];
#pragma unroll
  for (int t = 0; t < DT; ++t) dq[t] = zero16();
  barrier_all();

  // Per-lane LDS byte offsets: row reads per k-step and transpose reads per
  // 32-column block (the swizzle repeats every 16 rows, so sub-tile and
  // key-step offsets are compile-time immediates on top).  Re-pinned every
  // tile so they stay the only live copies.
  uint32_t rofs[KSTEPS], tofs[DT][2];
#pragma unroll
  for (int k = 0; k < KSTEPS; ++k) rofs[k] = tile_off<D>(l32, 2 * k + half);
  {
    const int row = 4 * half + ((lane & 15) >> 2);
#pragma unroll
    for (int t = 0; t < DT; ++t) {
      const int col = t * 32 + 16 * ((lane >> 4) & 1) + 4 * (lane & 3);
      tofs[t][0] = tile_off<D>(row, col >> 3) + (col & 7) * 2;
      tofs[t][1] = tile_off<D>(row + 8, col >> 3) + (col & 7) * 2;
    }
  }
  auto pin_offsets = [&]() __attribute__((always_inline)) {
#pragma unroll
    for (int k = 0; k < KSTEPS; ++k) asm volatile("" : "+v"(rofs[k]));
#pragma unroll
    for (int t = 0; t < DT; ++t) asm volatile("" : "+v"(tofs[t][0]), "+v"(tofs[t][1]));
  };
  constexpr int NS = 2 * KSTEPS;   // matrix ops of S^T (and of dP^T) per tile
  constexpr int LEAD = 3;          // operand reads in flight ahead of their matrix op
  // row-major operand idx of a 64-key tile: 32-key sub-tile idx % 2, k-step idx / 2
  auto row_operand = [&](const unsigned char* tile, int idx) __attribute__((always_inline)) {
    return *(const u32x4*)(tile + rofs[idx / 2] + (idx % 2) * 32 * D * 2);
  };
  auto tr_op = [&](const unsigned char* tile, int u, int t) __attribute__((always_inline)) {
    const u32x2 lo = ds_read_tr16(tile + tofs[t][0] + u * 16 * D * 2);
    const u32x2 hi = ds_read_tr16(tile + tofs[t][1] + u * 16 * D * 2);
    return u32x4{lo[0], lo[1], hi[0], hi[1]};
  };

  // One 64-key tile in three overlapping stages:
  //   A: S^T = K Q^T (the two 32-key sub-tiles' chains in turn);
  //   B: dP^T = V dO^T, sub-tile 0's chain and then sub-tile 1's, with the
  //      probabilities P^T = exp2(scale log2(e) S^T - LSE log2(e)) replacing
  //      the scores between sub-tile 0's ops;
  //   C: per 16-key step u, dS^T = P^T o (dP^T - D) for the step's scores,
  //      then its DT products dQ^T += K^T dS^T; the two steps of sub-tile 0
  //      run between sub-tile 1's dP ops (the backward 1% faster than after them).
  auto compute = [&](int j, const unsigned char* sK, const unsigned char* sV) {
    const int kb = j * kQBN;
    if (CAUSAL && kb > wave_qlast) return;         // whole tile above this wave's diagonal
    pin_offsets();
    // Two workgroups share a CU, so a SIMD's two waves belong to different
    // workgroups; the wave priority tracks progress through the tile (3, then
    // 2 after the S ops, 1 after the dP ops, 0 at the end) so the wave that
    // is behind is served first rather than the older one (4% faster).
    __builtin_amdgcn_s_setprio(3);
    f32x16 s[2], dp[2];
    {
      u32x4 ring[LEAD];
#pragma unroll
      for (int x = 0; x < LEAD; ++x) ring[x] = row_operand(sK, x);
#pragma unroll
      for (int idx = 0; idx < NS; ++idx) {
        const u32x4 a = ring[idx % LEAD];
        if (idx + LEAD < NS) ring[idx % LEAD] = row_operand(sK, idx + LEAD);
        const int t = idx % 2, k = idx / 2;
        s[t] = E::mfma(a, qf[k], k == 0 ? zero16() : s[t]);
      }
    }
    __builtin_amdgcn_s_setprio(2);
    const bool need_mask = (CAUSAL && kb + kQBN - 1 > q0 + wave * 32) || (kb + kQBN > N);
    const int lim = min(CAUSAL ? my_q : N - 1, N - 1) - kb - 4 * half;
    // 16-key step u: dS^T of its scores, then its DT products into dQ^T
    auto cstep = [&](int u) __attribute__((always_inline)) {
      const int t = u / 2, i0 = (u % 2) * 8;
      u32x4 db;
#pragma unroll
      for (int i = i0; i < i0 + 8; i += 2) {
        float p0 = s[t][i], p1 = s[t][i + 1];
        if (need_mask) {
          if (t * 32 + 8 * (i >> 2) + (i & 3) > lim) p0 = 0.f;
          if (t * 32 + 8 * ((i + 1) >> 2) + ((i + 1) & 3) > lim) p1 = 0.f;
        }
        db[(i & 7) >> 1] = E::pack(p0 * (dp[t][i] - Di), p1 * (dp[t][i + 1] - Di));
      }
#pragma unroll
      for (int t2 = 0; t2 < DT; ++t2) dq[t2] = E::mfma(tr_op(sK, u, t2), db, dq[t2]);
    };
    {
      // dP^T sub-tile 0's chain first, with the exponentials of both
      // sub-tiles between its ops; then sub-tile 1's chain, with the dS and
      // dQ products of sub-tile 0's two 16-key steps between its ops
      auto vop = [&](int idx) { return row_operand(sV, 2 * (idx % KSTEPS) + idx / KSTEPS); };
      u32x4 ring[LEAD];
#pragma unroll
      for (int x = 0; x < LEAD; ++x) ring[x] = vop(x);
#pragma unroll
      for (int idx = 0; idx < NS; ++idx) {
        const u32x4 a = ring[idx % LEAD];
        if (idx + LEAD < NS) ring[idx % LEAD] = vop(idx + LEAD);
        const int t = idx / KSTEPS, k = idx % KSTEPS;
        dp[t] = E::mfma(a, dof[k], k == 0 ? zero16() : dp[t]);
        if (idx < KSTEPS) {
#pragma unroll
          for (int e = 0; e < 32; ++e)
            if (e * KSTEPS / 32 == idx)
              s[e / 16][e % 16] = fast_exp2(fmaf(s[e / 16][e % 16], scale_log2, neg_lse2));
        } else if (idx == KSTEPS) {
          cstep(0);
        } else if (idx == KSTEPS + KSTEPS / 2) {
          cstep(1);
        }
      }
    }
    __builtin_amdgcn_s_setprio(1);
    cstep(2);
    cstep(3);
    __builtin_amdgcn_s_setprio(0);
  };
  for (int j = 0; j < n_kv; j += 2) {
    if (j + 1 < n_kv) load(j + 1, sK1, sV1);
    compute(j, sK0, sV0);
    barrier_all();
    if (j + 1 < n_kv) {
      if (j + 2 < n_kv) load(j + 2, sK0, sV0);
      compute(j + 1, sK1, sV1);
      barrier_all();
    }
  }

  // dQ rows through LDS as whole-row stores (one ring slot per wave)
  static_assert(32 * D * 4 == TILE, "one wave's fp32 tile per ring slot");
  barrier_all();
  unsigned char* stage = wave == 0 ? sK0 : wave == 1 ? sK1 : wave == 2 ? sV0 : sV1;
  store_rows_f32<D, DT>(dq, scale, stage, rdQ, q0 + wave * 32, lane);
}

template <class E, int D, bool CAUSAL>
hipError_t launch(const BwdArgs& a) {
  using T = typename E::elem;
  const long long rows = (long long)a.B * a.H * a.N;
  float* NLvec = a.Dvec + rows;   // -LSE log2(e), after D in the workspace
  const float sl2 = a.scale * kLog2e;
  // causal tiles differ in length: interleave heads so long tiles start first
  // (each tile streams two [N, d] operands of its head)
  const int hg = CAUSAL ? xcd_group((long long)a.B * a.H, (long long)a.N * D * 4) : 0;
  // dQ first: it also writes D and -LSE log2(e), which the dK/dV kernel reads
  const int n_qt = (a.N + kQBM - 1) / kQBM;
  hipLaunchKernelGGL((bwd_dq_kernel<E, D, CAUSAL>), dim3(a.B * a.H * n_qt), dim3(kThreads), 0,
                     a.stream, (const T*)a.Q, (const T*)a.K, (const T*)a.V, (const T*)a.O,
                     (const T*)a.dO, a.LSE, a.Dvec, NLvec, a.dQ, a.N, a.scale, sl2, n_qt, hg);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int n_kt = (a.N + kKvBN - 1) / kKvBN;
  hipLaunchKernelGGL((bwd_dkdv_kernel<E, D, CAUSAL>), dim3(a.B * a.H * n_kt), dim3(kKvWaves * 64), 0,
                     a.stream, (const T*)a.Q, (const T*)a.K, (const T*)a.V, (const T*)a.dO, NLvec, a.Dvec, a.dK, a.dV, a.N, a.scale, sl2, n_kt, hg);
  return hipGetLastError();
}

template <class E>
hipError_t launch_e(const BwdArgs& a) {
  if (a.d == 64) return a.causal ? launch<E, 64, true>(a) : launch<E, 64, false>(a);
  return a.causal ? launch<E, 128, true>(a) : launch<E, 128, false>(a);
}

}  // namespace

hipError_t launch_bwd(const BwdArgs& a) {
  return a.dtype == 2 ? launch_e<F16>(a) : launch_e<Bf16>(a);
}

}  // namespace fa
