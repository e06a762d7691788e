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
// Three kernels, all on the caller's stream, deterministic (no atomics):
//   1. bwd_dot:  D_i = rowsum(dO o O) into the workspace.
//   2. bwd_dkdv: workgroup = 128 keys (wave = 32 keys); loops over 32-row
//      query tiles; recomputes S = Q K^T and dP = dO V^T with this wave's K
//      and V rows held in registers, and accumulates dV^T += dO^T P and
//      dK^T += Q^T dS on the matrix cores.  Q and dO tiles are staged in LDS
//      both row-major and transposed.
//   3. bwd_dq:   workgroup = 128 queries (wave = 32); loops over 64-key tiles;
//      recomputes S^T = K Q^T and dP^T = V dO^T (each lane then holds one
//      query's row, so LSE_i and D_i are per-lane scalars) and accumulates
//      dQ^T += K^T dS^T.
// Causal: tiles wholly above the diagonal are skipped; straddling tiles masked.
#include "fa_device.h"
#include "fa_internal.h"

namespace fa {

namespace {

constexpr int kThreads = 256;

// ---------------------------------------------------------------- D = rowsum(dO o O)
template <int D>
__global__ __launch_bounds__(kThreads) void bwd_dot_kernel(const __bf16* __restrict__ O,
                                                           const __bf16* __restrict__ dO,
                                                           float* __restrict__ Dvec,
                                                           long long rows) {
  constexpr int LPR = D / 8;                      // lanes per row, 8 values each
  const long long row = (long long)blockIdx.x * (kThreads / LPR) + threadIdx.x / LPR;
  const int c = threadIdx.x % LPR;
  const bool ok = row < rows;
  const long long r = ok ? row : 0;
  const u32x4 a = *(const u32x4*)(O + r * D + c * 8);
  const u32x4 b = *(const u32x4*)(dO + r * D + c * 8);
  float acc = 0.f;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    acc = fmaf(bf16lo(a[e]), bf16lo(b[e]), acc);
    acc = fmaf(bf16hi(a[e]), bf16hi(b[e]), acc);
  }
  acc = group_sum<LPR>(acc);
  if (ok && c == 0) Dvec[row] = acc;
}

// ---------------------------------------------------------------- dK, dV
constexpr int kKvBN = 128;   // keys per workgroup (32 per wave)
constexpr int kKvBM = 32;    // queries per inner tile

template <int D, bool CAUSAL>
__global__ __launch_bounds__(kThreads, 1) void bwd_dkdv_kernel(
    const __bf16* __restrict__ Q, const __bf16* __restrict__ K, const __bf16* __restrict__ V,
    const __bf16* __restrict__ dO, const float* __restrict__ LSE, const float* __restrict__ Dvec,
    float* __restrict__ dK, float* __restrict__ dV, int N, float scale, float scale_log2,
    int n_ktiles) {
  constexpr int DCH = D / 8;
  constexpr int KSTEPS = D / 16;
  constexpr int DT = D / 32;
  constexpr int ITEMS = (kKvBM / 4) * DCH;         // (4-row group, chunk) items per tensor
  constexpr int TILE = kKvBM * D * 2;              // bytes of one 32 x D bf16 tile
  __shared__ __attribute__((aligned(16))) unsigned char smem[4 * TILE + 2 * kKvBM * 4];
  unsigned char* const sQ = smem;                  // row-major [32][D]
  unsigned char* const sdO = smem + TILE;          // row-major [32][D]
  unsigned char* const sQt = smem + 2 * TILE;      // transposed [D][32]
  unsigned char* const sdOt = smem + 3 * TILE;     // transposed [D][32]
  float* const sL = (float*)(smem + 4 * TILE);     // LSE * log2(e) of the tile's rows
  float* const sD = sL + kKvBM;                    // D of the tile's rows

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int l32 = lane & 31, half = lane >> 5;
  const int tile = xcd_remap(blockIdx.x, gridDim.x);
  const int bh = tile / n_ktiles;
  const int kt = CAUSAL ? (tile % n_ktiles) : (tile % n_ktiles);   // low tiles do the most work
  const int kb = kt * kKvBN;
  const int my_k = kb + wave * 32 + l32;          // this lane's key (C-layout column)

  const size_t head_off = (size_t)bh * (size_t)N * D;
  const uint32_t head_bytes = (uint32_t)N * D * 2;
  const auto rQ = make_rsrc(Q + head_off, head_bytes);
  const auto rK = make_rsrc(K + head_off, head_bytes);
  const auto rV = make_rsrc(V + head_off, head_bytes);
  const auto rdO = make_rsrc(dO + head_off, head_bytes);
  const auto rL = make_rsrc(LSE + (size_t)bh * N, (uint32_t)N * 4);
  const auto rD = make_rsrc(Dvec + (size_t)bh * N, (uint32_t)N * 4);
  const auto rdK = make_rsrc(dK + head_off, (uint32_t)N * D * 4);
  const auto rdV = make_rsrc(dV + head_off, (uint32_t)N * D * 4);

  // this wave's 32 keys as B operands: B[k = d][n = key] = K[key][d]
  bf16x8 kf[KSTEPS], vf[KSTEPS];
#pragma unroll
  for (int s = 0; s < KSTEPS; ++s) {
    kf[s] = as_bf16x8(bload16(rK, (uint32_t)(my_k * D + 16 * s + 8 * half) * 2));
    vf[s] = as_bf16x8(bload16(rV, (uint32_t)(my_k * D + 16 * s + 8 * half) * 2));
  }

  f32x16 dk[DT], dv[DT];
#pragma unroll
  for (int t = 0; t < DT; ++t) {
    dk[t] = zero16();
    dv[t] = zero16();
  }

  // loader role: threads [0, ITEMS) stage Q, [128, 128 + ITEMS) stage dO
  const int role = tid >> 7;                       // 0: Q, 1: dO
  const int item = tid & 127;
  const bool loader = item < ITEMS;
  const int lc = item % DCH, lg = item / DCH;      // chunk, 4-row group

  const int q_first = CAUSAL ? kb : 0;             // queries before kb see none of these keys
  const int wave_k0 = kb + wave * 32;
  for (int q0 = q_first; q0 < N; q0 += kKvBM) {
    u32x4 rows[4];
    if (loader) {
      const auto& r = role ? rdO : rQ;
#pragma unroll
      for (int i = 0; i < 4; ++i)
        rows[i] = bload16(r, (uint32_t)((q0 + 4 * lg + i) * D + lc * 8) * 2);
    }
    float lv = 0.f, dvv = 0.f;
    if (tid < kKvBM) {
      lv = bload4f(rL, (uint32_t)(q0 + tid) * 4) * kLog2e;
      dvv = bload4f(rD, (uint32_t)(q0 + tid) * 4);
    }
    __syncthreads();                               // previous tile consumed
    if (loader) {
      unsigned char* nat = role ? sdO : sQ;
      unsigned char* tr = role ? sdOt : sQt;
#pragma unroll
      for (int i = 0; i < 4; ++i) *(u32x4*)(nat + rm_off<D>(4 * lg + i, lc)) = rows[i];
      u32x2 cols[8];
      transpose4x8(rows, cols);
      const int p = kpos(4 * lg) >> 2;
#pragma unroll
      for (int j = 0; j < 8; ++j) *(u32x2*)(tr + tr32_piece_off(lc * 8 + j, p)) = cols[j];
    }
    if (tid < kKvBM) {
      sL[tid] = lv;
      sD[tid] = dvv;
    }
    __syncthreads();

    if (CAUSAL && q0 + kKvBM - 1 < wave_k0) continue;    // every query precedes every key

    // S = Q K^T and dP = dO V^T: rows = queries, columns = this wave's keys
    f32x16 s = zero16(), dp = zero16();
#pragma unroll
    for (int k = 0; k < KSTEPS; ++k) {
      const bf16x8 aq = *(const bf16x8*)(sQ + rm_off<D>(l32, 2 * k + half));
      const bf16x8 ado = *(const bf16x8*)(sdO + rm_off<D>(l32, 2 * k + half));
      s = mfma_bf16(aq, kf[k], s);
      dp = mfma_bf16(ado, vf[k], dp);
    }
    const bool need_mask = (CAUSAL && q0 < wave_k0 + 31) || (q0 + kKvBM > N);
    bf16x8 pb[2], dsb[2];
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const int r0 = 8 * g + 4 * half;             // first of this lane's 4 query rows
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int i = 4 * g + e;
        const int qrow = q0 + r0 + e;
        float p = fast_exp2(s[i] * scale_log2 - sL[r0 + e]);
        if (need_mask && ((CAUSAL && my_k > qrow) || qrow >= N)) p = 0.f;
        const float ds = p * (dp[i] - sD[r0 + e]);
        pb[i >> 3][i & 7] = (__bf16)p;
        dsb[i >> 3][i & 7] = (__bf16)ds;
      }
    }
    // dV^T += dO^T P ; dK^T += Q^T dS   (contraction over the 32 queries)
#pragma unroll
    for (int t = 0; t < DT; ++t)
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        const bf16x8 adot = *(const bf16x8*)(sdOt + tr32_chunk_off(t * 32 + l32, 2 * u + half));
        const bf16x8 aqt = *(const bf16x8*)(sQt + tr32_chunk_off(t * 32 + l32, 2 * u + half));
        dv[t] = mfma_bf16(adot, pb[u], dv[t]);
        dk[t] = mfma_bf16(aqt, dsb[u], dk[t]);
      }
  }

  // store: lane holds key my_k, rows d = 32t + 8g + 4*half + (0..3)
#pragma unroll
  for (int t = 0; t < DT; ++t)
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const int d0 = t * 32 + 8 * g + 4 * half;
      u32x4 wk, wv;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        wk[e] = as_u32(dk[t][4 * g + e] * scale);
        wv[e] = as_u32(dv[t][4 * g + e]);
      }
      bstore16(wk, rdK, (uint32_t)(my_k * D + d0) * 4);
      bstore16(wv, rdV, (uint32_t)(my_k * D + d0) * 4);
    }
}

// ---------------------------------------------------------------- dQ
constexpr int kQBM = 128;   // queries per workgroup (32 per wave)
constexpr int kQBN = 64;    // keys per tile

template <int D, bool CAUSAL>
__global__ __launch_bounds__(kThreads, 1) void bwd_dq_kernel(
    const __bf16* __restrict__ Q, const __bf16* __restrict__ K, const __bf16* __restrict__ V,
    const __bf16* __restrict__ dO, const float* __restrict__ LSE, const float* __restrict__ Dvec,
    float* __restrict__ dQ, int N, float scale, float scale_log2, int n_qtiles) {
  constexpr int DCH = D / 8;
  constexpr int KSTEPS = D / 16;
  constexpr int DT = D / 32;
  constexpr int STAGE_ROUNDS = kQBM * DCH / kThreads;
  constexpr int K_ROUNDS = kQBN * DCH / kThreads;
  constexpr int T_ITEMS = (kQBN / 4) * DCH;
  constexpr int T_ROUNDS = (T_ITEMS + kThreads - 1) / kThreads;
  constexpr int TILE = kQBN * D * 2;
  constexpr int STAGE = kQBM * D * 2;
  constexpr int SMEM = (STAGE > 3 * TILE) ? STAGE : 3 * TILE;
  __shared__ __attribute__((aligned(16))) unsigned char smem[SMEM];
  unsigned char* const sK = smem;                  // row-major [64][D]
  unsigned char* const sV = smem + TILE;           // row-major [64][D]
  unsigned char* const sKt = smem + 2 * TILE;      // transposed [D][64]

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int l32 = lane & 31, half = lane >> 5;
  const int tile = xcd_remap(blockIdx.x, gridDim.x);
  const int bh = tile / n_qtiles;
  const int qt = CAUSAL ? (n_qtiles - 1 - tile % n_qtiles) : (tile % n_qtiles);
  const int q0 = qt * kQBM;
  const int my_q = q0 + wave * 32 + l32;

  const size_t head_off = (size_t)bh * (size_t)N * D;
  const uint32_t head_bytes = (uint32_t)N * D * 2;
  const auto rQ = make_rsrc(Q + head_off, head_bytes);
  const auto rK = make_rsrc(K + head_off, head_bytes);
  const auto rV = make_rsrc(V + head_off, head_bytes);
  const auto rdO = make_rsrc(dO + head_off, head_bytes);
  const auto rL = make_rsrc(LSE + (size_t)bh * N, (uint32_t)N * 4);
  const auto rD = make_rsrc(Dvec + (size_t)bh * N, (uint32_t)N * 4);
  const auto rdQ = make_rsrc(dQ + head_off, (uint32_t)N * D * 4);

  // stage Q then dO through LDS (coalesced), keep this wave's rows as B operands
  bf16x8 qf[KSTEPS], dof[KSTEPS];
#pragma unroll
  for (int pass = 0; pass < 2; ++pass) {
    const auto& r = pass ? rdO : rQ;
    u32x4 st[STAGE_ROUNDS];
#pragma unroll
    for (int i = 0; i < STAGE_ROUNDS; ++i) {
      const int row = i * (kThreads / DCH) + tid / DCH, c = tid % DCH;
      st[i] = bload16(r, (uint32_t)((q0 + row) * D + c * 8) * 2);
    }
    __syncthreads();
#pragma unroll
    for (int i = 0; i < STAGE_ROUNDS; ++i) {
      const int row = i * (kThreads / DCH) + tid / DCH, c = tid % DCH;
      *(u32x4*)(smem + rm_off<D>(row, c)) = st[i];
    }
    __syncthreads();
#pragma unroll
    for (int s = 0; s < KSTEPS; ++s) {
      const bf16x8 v = *(const bf16x8*)(smem + rm_off<D>(wave * 32 + l32, 2 * s + half));
      if (pass) dof[s] = v; else qf[s] = v;
    }
  }
  const float lse2 = bload4f(rL, (uint32_t)my_q * 4) * kLog2e;
  const float Di = bload4f(rD, (uint32_t)my_q * 4);

  f32x16 dq[DT];
#pragma unroll
  for (int t = 0; t < DT; ++t) dq[t] = zero16();

  const int kv_end = CAUSAL ? min(N, q0 + kQBM) : N;
  const int n_kv = (kv_end + kQBN - 1) / kQBN;
  const int wave_qlast = q0 + wave * 32 + 31;

  u32x4 kreg[K_ROUNDS], vreg[K_ROUNDS], treg[T_ROUNDS][4];
  auto load = [&](int kb) {
#pragma unroll
    for (int r = 0; r < K_ROUNDS; ++r) {
      const int row = r * (kThreads / DCH) + tid / DCH, c = tid % DCH;
      kreg[r] = bload16(rK, (uint32_t)((kb + row) * D + c * 8) * 2);
      vreg[r] = bload16(rV, (uint32_t)((kb + row) * D + c * 8) * 2);
    }
#pragma unroll
    for (int r = 0; r < T_ROUNDS; ++r) {
      const int it = r * kThreads + tid;
      const int c = it % DCH, g = it / DCH;
      if (it < T_ITEMS) {
#pragma unroll
        for (int i = 0; i < 4; ++i)
          treg[r][i] = bload16(rK, (uint32_t)((kb + 4 * g + i) * D + c * 8) * 2);
      }
    }
  };
  auto store = [&]() {
#pragma unroll
    for (int r = 0; r < K_ROUNDS; ++r) {
      const int row = r * (kThreads / DCH) + tid / DCH, c = tid % DCH;
      *(u32x4*)(sK + rm_off<D>(row, c)) = kreg[r];
      *(u32x4*)(sV + rm_off<D>(row, c)) = vreg[r];
    }
#pragma unroll
    for (int r = 0; r < T_ROUNDS; ++r) {
      const int it = r * kThreads + tid;
      const int c = it % DCH, g = it / DCH;
      if (it < T_ITEMS) {
        u32x2 cols[8];
        transpose4x8(treg[r], cols);
        const int p = kpos(4 * g) >> 2;
#pragma unroll
        for (int j = 0; j < 8; ++j) *(u32x2*)(sKt + tr_piece_off(c * 8 + j, p)) = cols[j];
      }
    }
  };

  load(0);
  for (int j = 0; j < n_kv; ++j) {
    const int kb = j * kQBN;
    __syncthreads();
    store();
    __syncthreads();
    if (j + 1 < n_kv) load(kb + kQBN);
    if (CAUSAL && kb > wave_qlast) continue;

    // S^T = K Q^T, dP^T = V dO^T : rows = keys, column = this lane's query
    f32x16 s[2], dp[2];
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      s[t] = zero16();
      dp[t] = zero16();
#pragma unroll
      for (int k = 0; k < KSTEPS; ++k) {
        const bf16x8 ak = *(const bf16x8*)(sK + rm_off<D>(t * 32 + l32, 2 * k + half));
        const bf16x8 av = *(const bf16x8*)(sV + rm_off<D>(t * 32 + l32, 2 * k + half));
        s[t] = mfma_bf16(ak, qf[k], s[t]);
        dp[t] = mfma_bf16(av, dof[k], dp[t]);
      }
    }
    const bool need_mask = (CAUSAL && kb + kQBN - 1 > q0 + wave * 32) || (kb + kQBN > N);
    bf16x8 dsb[4];
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        float p = fast_exp2(s[t][i] * scale_log2 - lse2);
        if (need_mask) {
          const int key = kb + t * 32 + 8 * (i >> 2) + 4 * half + (i & 3);
          if ((CAUSAL && key > my_q) || key >= N) p = 0.f;
        }
        dsb[2 * t + (i >> 3)][i & 7] = (__bf16)(p * (dp[t][i] - Di));
      }
    // dQ^T += K^T dS^T
#pragma unroll
    for (int t = 0; t < DT; ++t)
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const bf16x8 a = *(const bf16x8*)(sKt + tr_chunk_off(t * 32 + l32, 2 * u + half));
        dq[t] = mfma_bf16(a, dsb[u], dq[t]);
      }
  }

#pragma unroll
  for (int t = 0; t < DT; ++t)
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const int d0 = t * 32 + 8 * g + 4 * half;
      u32x4 w;
#pragma unroll
      for (int e = 0; e < 4; ++e) w[e] = as_u32(dq[t][4 * g + e] * scale);
      bstore16(w, rdQ, (uint32_t)(my_q * D + d0) * 4);
    }
}

template <int D, bool CAUSAL>
hipError_t launch(const BwdArgs& a) {
  const long long rows = (long long)a.B * a.H * a.N;
  constexpr int rows_per_block = kThreads / (D / 8);
  hipLaunchKernelGGL((bwd_dot_kernel<D>), dim3((unsigned)((rows + rows_per_block - 1) / rows_per_block)),
                     dim3(kThreads), 0, a.stream, (const __bf16*)a.O, (const __bf16*)a.dO, a.Dvec,
                     rows);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const float sl2 = a.scale * kLog2e;
  const int n_kt = (a.N + kKvBN - 1) / kKvBN;
  hipLaunchKernelGGL((bwd_dkdv_kernel<D, CAUSAL>), dim3(a.B * a.H * n_kt), dim3(kThreads), 0,
                     a.stream, (const __bf16*)a.Q, (const __bf16*)a.K, (const __bf16*)a.V,
                     (const __bf16*)a.dO, a.LSE, a.Dvec, a.dK, a.dV, a.N, a.scale, sl2, n_kt);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int n_qt = (a.N + kQBM - 1) / kQBM;
  hipLaunchKernelGGL((bwd_dq_kernel<D, CAUSAL>), dim3(a.B * a.H * n_qt), dim3(kThreads), 0,
                     a.stream, (const __bf16*)a.Q, (const __bf16*)a.K, (const __bf16*)a.V,
                     (const __bf16*)a.dO, a.LSE, a.Dvec, a.dQ, a.N, a.scale, sl2, n_qt);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_bwd(const BwdArgs& a) {
  if (a.d == 64) return a.causal ? launch<64, true>(a) : launch<64, false>(a);
  return a.causal ? launch<128, true>(a) : launch<128, false>(a);
}

}  // namespace fa
