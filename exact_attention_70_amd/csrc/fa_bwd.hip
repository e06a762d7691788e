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
//   2. bwd_dkdv: workgroup = 128 keys (wave = 32 keys); loops over 64-row
//      query tiles; recomputes S = Q K^T and dP = dO V^T with this wave's K
//      and V rows held in registers, and accumulates dV^T += dO^T P and
//      dK^T += Q^T dS on the matrix cores.  Q, dO, LSE and D tiles stream into
//      LDS by buffer->LDS transfers; Q^T and dO^T come from transpose reads.
//   3. bwd_dq:   workgroup = 128 queries (wave = 32); loops over 64-key K/V tiles;
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

// Direct buffer -> LDS copy of one dword per lane (lane i lands at lds + 4 i).
__device__ __forceinline__ void dma4(__amdgpu_buffer_rsrc_t r, void* lds, uint32_t off) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void*)lds, 4, (int)off, 0, 0, 0);
}

// Transpose-read operand (lane: one column of a 32-row tile of a row-major bf16
// tile, 8 consecutive rows 16u + 8a + 4h + c): two ds_read_b64_tr_b16 reads.
// The row order matches the C-layout of a 32 x 32 score tile, so the result
// pairs slot-for-slot with a C-layout tile fed back as the B operand.
template <int D>
__device__ __forceinline__ bf16x8 tr_operand(const unsigned char* tile, int u, int t, int lane) {
  const int half = lane >> 5;
  const int row = 16 * u + 4 * half + ((lane & 15) >> 2);
  const int col = t * 32 + 16 * ((lane >> 4) & 1) + 4 * (lane & 3);
  const u32x2 lo = ds_read_tr16(tile + tile_off<D>(row, col >> 3) + (col & 7) * 2);
  const u32x2 hi = ds_read_tr16(tile + tile_off<D>(row + 8, col >> 3) + (col & 7) * 2);
  return as_bf16x8(u32x4{lo[0], lo[1], hi[0], hi[1]});
}

// ---------------------------------------------------------------- dK, dV
// Workgroup = 128 keys (wave = 32 keys, held in registers as B operands);
// loops over 64-row query tiles streamed into LDS (Q, dO, LSE, D) by
// buffer->LDS transfers, double-buffered.  Per tile and wave:
//   S = Q K^T, dP = dO V^T (rows = queries, columns = this wave's keys),
//   P = exp(scale S - LSE), dS = P o (dP - D),
//   dV^T += dO^T P, dK^T += Q^T dS  (dO^T and Q^T from transpose reads).
constexpr int kKvBN = 128;   // keys per workgroup
constexpr int kKvBQ = 64;    // queries per inner tile

template <int D, bool CAUSAL>
__global__ __launch_bounds__(kThreads, 1) void bwd_dkdv_kernel(
    const __bf16* __restrict__ Q, const __bf16* __restrict__ K, const __bf16* __restrict__ V,
    const __bf16* __restrict__ dO, const float* __restrict__ LSE, const float* __restrict__ Dvec,
    float* __restrict__ dK, float* __restrict__ dV, int N, float scale, float scale_log2,
    int n_ktiles) {
  constexpr int KSTEPS = D / 16;
  constexpr int DT = D / 32;
  constexpr int TILE = kKvBQ * D * 2;
  __shared__ __attribute__((aligned(1024))) unsigned char sQ0[TILE];
  __shared__ __attribute__((aligned(1024))) unsigned char sQ1[TILE];
  __shared__ __attribute__((aligned(1024))) unsigned char sO0[TILE];
  __shared__ __attribute__((aligned(1024))) unsigned char sO1[TILE];
  __shared__ __attribute__((aligned(256))) float sL0[kKvBQ];
  __shared__ __attribute__((aligned(256))) float sL1[kKvBQ];
  __shared__ __attribute__((aligned(256))) float sD0[kKvBQ];
  __shared__ __attribute__((aligned(256))) float sD1[kKvBQ];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int l32 = lane & 31, half = lane >> 5;
  const int tile = xcd_remap(blockIdx.x, gridDim.x);
  const int bh = tile / n_ktiles;
  const int kb = (tile % n_ktiles) * kKvBN;       // low key tiles see the most queries
  const int wave_k0 = kb + wave * 32;
  const int my_k = wave_k0 + l32;                 // this lane's key (C-layout column)

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

  const int q_first = CAUSAL ? kb : 0;            // earlier queries see none of these keys
  const int n_q = (N - q_first + kKvBQ - 1) / kKvBQ;
  auto load = [&](int i, unsigned char* sQ, unsigned char* sO, float* sL, float* sD) {
    const int q0 = q_first + i * kKvBQ;
    dma_rows<D, kKvBQ, kThreads / 64>(rQ, sQ, q0, wave, lane);
    dma_rows<D, kKvBQ, kThreads / 64>(rdO, sO, q0, wave, lane);
    if (wave == 0) dma4(rL, sL, (uint32_t)(q0 + lane) * 4);
    if (wave == 1) dma4(rD, sD, (uint32_t)(q0 + lane) * 4);
  };
  load(0, sQ0, sO0, sL0, sD0);

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
  barrier_all();

  auto compute = [&](int i, const unsigned char* sQ, const unsigned char* sO, const float* sL,
                     const float* sD) {
    const int q0 = q_first + i * kKvBQ;
    if (CAUSAL && q0 + kKvBQ - 1 < wave_k0) return;        // every query precedes every key
    f32x16 s[2], dp[2];
#pragma unroll
    for (int sub = 0; sub < 2; ++sub) {
#pragma unroll
      for (int k = 0; k < KSTEPS; ++k) {
        const bf16x8 aq = *(const bf16x8*)(sQ + tile_off<D>(sub * 32 + l32, 2 * k + half));
        const bf16x8 ao = *(const bf16x8*)(sO + tile_off<D>(sub * 32 + l32, 2 * k + half));
        s[sub] = mfma_bf16(aq, kf[k], k == 0 ? zero16() : s[sub]);
        dp[sub] = mfma_bf16(ao, vf[k], k == 0 ? zero16() : dp[sub]);
      }
    }
    const bool need_mask = (CAUSAL && q0 < wave_k0 + 31) || (q0 + kKvBQ > N);
    u32x4 pb[4], db[4];
#pragma unroll
    for (int sub = 0; sub < 2; ++sub)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int r0 = sub * 32 + 8 * g + 4 * half;   // first of this lane's 4 query rows
        const f32x4 lse4 = *(const f32x4*)(sL + r0);
        const f32x4 d4 = *(const f32x4*)(sD + r0);
        float pv[4], dsv[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int i = 4 * g + e;
          float p = fast_exp2(fmaf(s[sub][i], scale_log2, -lse4[e] * kLog2e));
          if (need_mask && ((CAUSAL && my_k > q0 + r0 + e) || q0 + r0 + e >= N)) p = 0.f;
          pv[e] = p;
          dsv[e] = p * (dp[sub][i] - d4[e]);
        }
        const int u = 2 * sub + (g >> 1), w = (g & 1) * 2;   // B-operand k-step and word
        pb[u][w] = pack_bf16(pv[0], pv[1]);
        pb[u][w + 1] = pack_bf16(pv[2], pv[3]);
        db[u][w] = pack_bf16(dsv[0], dsv[1]);
        db[u][w + 1] = pack_bf16(dsv[2], dsv[3]);
      }
    // dV^T += dO^T P ; dK^T += Q^T dS   (contraction over the 64 queries)
#pragma unroll
    for (int u = 0; u < 4; ++u)
#pragma unroll
      for (int t = 0; t < DT; ++t) {
        dv[t] = mfma_bf16(tr_operand<D>(sO, u, t, lane), as_bf16x8(pb[u]), dv[t]);
        dk[t] = mfma_bf16(tr_operand<D>(sQ, u, t, lane), as_bf16x8(db[u]), dk[t]);
      }
  };
  for (int i = 0; i < n_q; i += 2) {
    if (i + 1 < n_q) load(i + 1, sQ1, sO1, sL1, sD1);
    compute(i, sQ0, sO0, sL0, sD0);
    barrier_all();
    if (i + 1 < n_q) {
      if (i + 2 < n_q) load(i + 2, sQ0, sO0, sL0, sD0);
      compute(i + 1, sQ1, sO1, sL1, sD1);
      barrier_all();
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
// Workgroup = 128 queries (wave = 32, Q and dO rows in registers as B
// operands); loops over 64-key K/V tiles streamed into LDS, double-buffered.
// Per tile and wave: S^T = K Q^T and dP^T = V dO^T (each lane holds one
// query's row, so LSE_i and D_i are per-lane scalars), dS^T = P^T o (dP^T - D),
// dQ^T += K^T dS^T with K^T from transpose reads.
constexpr int kQBM = 128;   // queries per workgroup
constexpr int kQBN = 64;    // keys per tile

template <int D, bool CAUSAL>
__global__ __launch_bounds__(kThreads, 2) void bwd_dq_kernel(
    const __bf16* __restrict__ Q, const __bf16* __restrict__ K, const __bf16* __restrict__ V,
    const __bf16* __restrict__ dO, const float* __restrict__ LSE, const float* __restrict__ Dvec,
    float* __restrict__ dQ, int N, float scale, float scale_log2, int n_qtiles) {
  constexpr int KSTEPS = D / 16;
  constexpr int DT = D / 32;
  constexpr int TILE = kQBN * D * 2;
  __shared__ __attribute__((aligned(1024))) unsigned char sK0[TILE];
  __shared__ __attribute__((aligned(1024))) unsigned char sK1[TILE];
  __shared__ __attribute__((aligned(1024))) unsigned char sV0[TILE];
  __shared__ __attribute__((aligned(1024))) unsigned char sV1[TILE];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int l32 = lane & 31, half = lane >> 5;
  const int tile = xcd_remap(blockIdx.x, gridDim.x);
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
  const auto rL = make_rsrc(LSE + (size_t)bh * N, (uint32_t)N * 4);
  const auto rD = make_rsrc(Dvec + (size_t)bh * N, (uint32_t)N * 4);
  const auto rdQ = make_rsrc(dQ + head_off, (uint32_t)N * D * 4);

  const int kv_end = CAUSAL ? min(N, q0 + kQBM) : N;
  const int n_kv = (kv_end + kQBN - 1) / kQBN;
  auto load = [&](int j, unsigned char* sK, unsigned char* sV) {
    dma_rows<D, kQBN, kThreads / 64>(rK, sK, j * kQBN, wave, lane);
    dma_rows<D, kQBN, kThreads / 64>(rV, sV, j * kQBN, wave, lane);
  };
  load(0, sK0, sV0);
  bf16x8 qf[KSTEPS], dof[KSTEPS];
#pragma unroll
  for (int s = 0; s < KSTEPS; ++s) {
    qf[s] = as_bf16x8(bload16(rQ, (uint32_t)(my_q * D + 16 * s + 8 * half) * 2));
    dof[s] = as_bf16x8(bload16(rdO, (uint32_t)(my_q * D + 16 * s + 8 * half) * 2));
  }
  const float neg_lse2 = -bload4f(rL, (uint32_t)my_q * 4) * kLog2e;
  const float Di = bload4f(rD, (uint32_t)my_q * 4);
  f32x16 dq[DT];
#pragma unroll
  for (int t = 0; t < DT; ++t) dq[t] = zero16();
  barrier_all();

  auto compute = [&](int j, const unsigned char* sK, const unsigned char* sV) {
    const int kb = j * kQBN;
    if (CAUSAL && kb > wave_qlast) return;         // whole tile above this wave's diagonal
    f32x16 s[2], dp[2];
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
      for (int k = 0; k < KSTEPS; ++k) {
        const bf16x8 ak = *(const bf16x8*)(sK + tile_off<D>(t * 32 + l32, 2 * k + half));
        const bf16x8 av = *(const bf16x8*)(sV + tile_off<D>(t * 32 + l32, 2 * k + half));
        s[t] = mfma_bf16(ak, qf[k], k == 0 ? zero16() : s[t]);
        dp[t] = mfma_bf16(av, dof[k], k == 0 ? zero16() : dp[t]);
      }
    const bool need_mask = (CAUSAL && kb + kQBN - 1 > q0 + wave * 32) || (kb + kQBN > N);
    const int lim = min(CAUSAL ? my_q : N - 1, N - 1) - kb - 4 * half;
    u32x4 db[4];
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
      for (int i = 0; i < 16; i += 2) {
        float p0 = fast_exp2(fmaf(s[t][i], scale_log2, neg_lse2));
        float p1 = fast_exp2(fmaf(s[t][i + 1], scale_log2, neg_lse2));
        if (need_mask) {
          if (t * 32 + 8 * (i >> 2) + (i & 3) > lim) p0 = 0.f;
          if (t * 32 + 8 * ((i + 1) >> 2) + ((i + 1) & 3) > lim) p1 = 0.f;
        }
        db[2 * t + (i >> 3)][(i & 7) >> 1] = pack_bf16(p0 * (dp[t][i] - Di), p1 * (dp[t][i + 1] - Di));
      }
    // dQ^T += K^T dS^T  (contraction over the 64 keys)
#pragma unroll
    for (int u = 0; u < 4; ++u)
#pragma unroll
      for (int t = 0; t < DT; ++t) dq[t] = mfma_bf16(tr_operand<D>(sK, u, t, lane), as_bf16x8(db[u]), dq[t]);
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
