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
//   * one workgroup = 4 waves = a 128-row query tile of one (batch, head);
//     wave w owns query rows [32w, 32w + 32) of the tile.
//   * the query tile is staged once through LDS with coalesced 16-byte loads,
//     then each wave keeps its rows in registers as matrix B operands.
//   * K/V are streamed in 64-key tiles: 16-byte coalesced global loads into
//     registers one tile ahead, then written to LDS (K row-major, V
//     transposed) for the four waves to share.
//   * each wave computes S^T = K Q^T (keys x its 32 queries) so that every
//     lane holds the scores of ONE query: the row max and row sum are
//     in-lane reductions plus one exchange with the other half-wave.
//   * the probabilities P^T are rounded to bf16 and fed straight back as the
//     B operand of O^T += V^T P^T; V is stored transposed with the key order
//     permuted to match the C-layout of the score tile.
//   * causal: key tiles entirely above the diagonal are never visited; only
//     tiles that straddle the diagonal (or the ragged end) are masked.
//   * workgroups are ordered heaviest-first within each head and mapped so
//     that one head's query tiles share an XCD (and its L2).
#include "fa_device.h"
#include "fa_internal.h"

namespace fa {

namespace {

constexpr int kBM = 128;   // query rows per workgroup
constexpr int kBN = 64;    // keys per K/V tile
constexpr int kThreads = 256;

template <int D, bool CAUSAL>
__global__ __launch_bounds__(kThreads, 2) void fwd_bf16_kernel(
    const __bf16* __restrict__ Q, const __bf16* __restrict__ K, const __bf16* __restrict__ V,
    __bf16* __restrict__ O, float* __restrict__ LSE, int N, float scale_log2, int n_qtiles) {
  constexpr int DCH = D / 8;             // 16-byte chunks per row
  constexpr int KSTEPS = D / 16;         // matrix k-steps over the head dim
  constexpr int DT = D / 32;             // 32-row tiles of O^T
  constexpr int Q_ROUNDS = kBM * DCH / kThreads;
  constexpr int K_ROUNDS = kBN * DCH / kThreads;
  constexpr int V_ITEMS = (kBN / 4) * DCH;          // (4-key group, d chunk) items
  constexpr int V_ROUNDS = (V_ITEMS + kThreads - 1) / kThreads;
  constexpr int K_BYTES = kBN * D * 2;
  constexpr int V_BYTES = D * kBN * 2;
  constexpr int Q_BYTES = kBM * D * 2;
  constexpr int SMEM = (Q_BYTES > K_BYTES + V_BYTES) ? Q_BYTES : (K_BYTES + V_BYTES);
  __shared__ __attribute__((aligned(16))) unsigned char smem[SMEM];
  unsigned char* const sK = smem;
  unsigned char* const sV = smem + K_BYTES;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int l32 = lane & 31;
  const int half = lane >> 5;

  const int tile = xcd_remap(blockIdx.x, gridDim.x);
  const int bh = tile / n_qtiles;
  const int qt = CAUSAL ? (n_qtiles - 1 - tile % n_qtiles) : (tile % n_qtiles);
  const int q0 = qt * kBM;

  const size_t head_off = (size_t)bh * (size_t)N * D;
  const uint32_t head_bytes = (uint32_t)N * D * 2;
  const auto rQ = make_rsrc(Q + head_off, head_bytes);
  const auto rK = make_rsrc(K + head_off, head_bytes);
  const auto rV = make_rsrc(V + head_off, head_bytes);
  const auto rO = make_rsrc(O + head_off, head_bytes);
  const auto rL = make_rsrc(LSE + (size_t)bh * N, (uint32_t)N * 4);

  // ---- stage the query tile through LDS, keep this wave's rows in registers
  {
    u32x4 qv[Q_ROUNDS];
#pragma unroll
    for (int r = 0; r < Q_ROUNDS; ++r) {
      const int row = r * (kThreads / DCH) + tid / DCH, c = tid % DCH;
      qv[r] = bload16(rQ, (uint32_t)((q0 + row) * D + c * 8) * 2);
    }
#pragma unroll
    for (int r = 0; r < Q_ROUNDS; ++r) {
      const int row = r * (kThreads / DCH) + tid / DCH, c = tid % DCH;
      *(u32x4*)(smem + rm_off<D>(row, c)) = qv[r];
    }
  }
  __syncthreads();
  bf16x8 qf[KSTEPS];
#pragma unroll
  for (int s = 0; s < KSTEPS; ++s)
    qf[s] = *(const bf16x8*)(smem + rm_off<D>(wave * 32 + l32, 2 * s + half));

  const int kv_end = CAUSAL ? min(N, q0 + kBM) : N;
  const int n_kv = (kv_end + kBN - 1) / kBN;
  const int my_q = q0 + wave * 32 + l32;          // this lane's query row
  const int wave_qlast = q0 + wave * 32 + 31;     // last query row of this wave

  // ---- K/V prefetch registers (one tile ahead)
  u32x4 kreg[K_ROUNDS];
  u32x4 vreg[V_ROUNDS][4];
  auto load_kv = [&](int kb) {
#pragma unroll
    for (int r = 0; r < K_ROUNDS; ++r) {
      const int row = r * (kThreads / DCH) + tid / DCH, c = tid % DCH;
      kreg[r] = bload16(rK, (uint32_t)((kb + row) * D + c * 8) * 2);
    }
#pragma unroll
    for (int r = 0; r < V_ROUNDS; ++r) {
      const int item = r * kThreads + tid;
      const int c = item % DCH, g = item / DCH;
      if (item < V_ITEMS) {
#pragma unroll
        for (int i = 0; i < 4; ++i)
          vreg[r][i] = bload16(rV, (uint32_t)((kb + 4 * g + i) * D + c * 8) * 2);
      }
    }
  };
  auto store_kv = [&]() {
#pragma unroll
    for (int r = 0; r < K_ROUNDS; ++r) {
      const int row = r * (kThreads / DCH) + tid / DCH, c = tid % DCH;
      *(u32x4*)(sK + rm_off<D>(row, c)) = kreg[r];
    }
#pragma unroll
    for (int r = 0; r < V_ROUNDS; ++r) {
      const int item = r * kThreads + tid;
      const int c = item % DCH, g = item / DCH;
      if (item < V_ITEMS) {
        u32x2 cols[8];
        transpose4x8(vreg[r], cols);
        const int p = kpos(4 * g) >> 2;
#pragma unroll
        for (int j = 0; j < 8; ++j) *(u32x2*)(sV + tr_piece_off(c * 8 + j, p)) = cols[j];
      }
    }
  };

  f32x16 o[DT];
#pragma unroll
  for (int t = 0; t < DT; ++t) o[t] = zero16();
  float m_run = kNegInf;   // running max of scale*log2(e)*score
  float l_run = 0.f;       // this lane's share of the running denominator

  load_kv(0);
  for (int j = 0; j < n_kv; ++j) {
    const int kb = j * kBN;
    __syncthreads();                 // previous tile fully consumed
    store_kv();
    __syncthreads();
    if (j + 1 < n_kv) load_kv(kb + kBN);

    if (CAUSAL && kb > wave_qlast) continue;   // whole tile above this wave's diagonal

    // S^T = K Q^T for two 32-key sub-tiles
    f32x16 s[2];
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      s[t] = zero16();
#pragma unroll
      for (int k = 0; k < KSTEPS; ++k) {
        const bf16x8 a = *(const bf16x8*)(sK + rm_off<D>(t * 32 + l32, 2 * k + half));
        s[t] = mfma_bf16(a, qf[k], s[t]);
      }
    }

    // online softmax over this lane's 32 scores (one query row)
    const bool need_mask = (CAUSAL && kb + kBN - 1 > q0 + wave * 32) || (kb + kBN > N);
    float mx = kNegInf;
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        float x = s[t][i] * scale_log2;
        if (need_mask) {
          const int key = kb + t * 32 + 8 * (i >> 2) + 4 * half + (i & 3);
          if ((CAUSAL && key > my_q) || key >= N) x = kNegInf;
        }
        s[t][i] = x;
        mx = fmaxf(mx, x);
      }
    mx = fmaxf(mx, swap_half(mx));
    const float m_new = fmaxf(m_run, mx);
    const float m_use = (m_new == kNegInf) ? 0.f : m_new;
    const float alpha = fast_exp2(m_run - m_use);
    m_run = m_new;
    float rs = 0.f;
    bf16x8 pb[4];
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
      for (int i = 0; i < 16; i += 2) {
        const float p0 = fast_exp2(s[t][i] - m_use);
        const float p1 = fast_exp2(s[t][i + 1] - m_use);
        rs += p0 + p1;
        const bf16x2 pk = {(__bf16)p0, (__bf16)p1};
        pb[2 * t + (i >> 3)][i & 7] = pk[0];
        pb[2 * t + (i >> 3)][(i & 7) + 1] = pk[1];
      }
    l_run = l_run * alpha + rs;
#pragma unroll
    for (int t = 0; t < DT; ++t)
#pragma unroll
      for (int i = 0; i < 16; ++i) o[t][i] *= alpha;

    // O^T += V^T P^T
#pragma unroll
    for (int t = 0; t < DT; ++t)
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const bf16x8 a = *(const bf16x8*)(sV + tr_chunk_off(t * 32 + l32, 2 * u + half));
        o[t] = mfma_bf16(a, pb[u], o[t]);
      }
  }

  // ---- epilogue: O = O^T / l, LSE = ln(sum exp) = (m + log2 l) ln 2
  const float l_tot = l_run + swap_half(l_run);
  const float inv = 1.f / l_tot;
#pragma unroll
  for (int t = 0; t < DT; ++t)
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const int d0 = t * 32 + 8 * g + 4 * half;
      u32x2 w;
      w[0] = pack_bf16(o[t][4 * g] * inv, o[t][4 * g + 1] * inv);
      w[1] = pack_bf16(o[t][4 * g + 2] * inv, o[t][4 * g + 3] * inv);
      bstore8(w, rO, (uint32_t)(my_q * D + d0) * 2);
    }
  if (half == 0) bstore4f((m_run + fast_log2(l_tot)) * kLn2, rL, (uint32_t)my_q * 4);
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
    float* __restrict__ O, float* __restrict__ LSE, int N, float scale_log2, int causal,
    int n_qtiles) {
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
  const uint32_t head_bytes = (uint32_t)N * D * 4;
  const auto rQ = make_rsrc(Q + head_off, head_bytes);
  const auto rK = make_rsrc(K + head_off, head_bytes);
  const auto rV = make_rsrc(V + head_off, head_bytes);
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

  const int kv_end = causal ? min(N, q0 + kF32BM) : N;
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
      if ((causal && key > my_q) || key >= N) x = kNegInf;
      s[i] = x;
      mx = fmaxf(mx, x);
    }
    mx = fmaxf(mx, swap_half(mx));
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

  const float l_tot = l_run + swap_half(l_run);
  const float inv = 1.f / l_tot;
#pragma unroll
  for (int t = 0; t < DT; ++t)
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const int d0 = t * 32 + 8 * g + 4 * half;
      u32x4 w;
#pragma unroll
      for (int x = 0; x < 4; ++x) w[x] = as_u32(o[t][4 * g + x] * inv);
      bstore16(w, rO, (uint32_t)(my_q * D + d0) * 4);
    }
  if (half == 0) bstore4f((m_run + fast_log2(l_tot)) * kLn2, rL, (uint32_t)my_q * 4);
}

template <int D, bool CAUSAL>
hipError_t launch_bf16(const FwdArgs& a) {
  const int n_qtiles = (a.N + kBM - 1) / kBM;
  const int grid = a.B * a.H * n_qtiles;
  hipLaunchKernelGGL((fwd_bf16_kernel<D, CAUSAL>), dim3(grid), dim3(kThreads), 0, a.stream,
                     (const __bf16*)a.Q, (const __bf16*)a.K, (const __bf16*)a.V, (__bf16*)a.O,
                     a.LSE, a.N, a.scale * kLog2e, n_qtiles);
  return hipGetLastError();
}

template <int D>
hipError_t launch_f32(const FwdArgs& a) {
  const int n_qtiles = (a.N + kF32BM - 1) / kF32BM;
  const int grid = a.B * a.H * n_qtiles;
  hipLaunchKernelGGL((fwd_f32_kernel<D>), dim3(grid), dim3(64), 0, a.stream,
                     (const float*)a.Q, (const float*)a.K, (const float*)a.V, (float*)a.O, a.LSE,
                     a.N, a.scale * kLog2e, a.causal ? 1 : 0, n_qtiles);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_fwd(const FwdArgs& a) {
  if (a.dtype == 1) {
    if (a.d == 64) return a.causal ? launch_bf16<64, true>(a) : launch_bf16<64, false>(a);
    return a.causal ? launch_bf16<128, true>(a) : launch_bf16<128, false>(a);
  }
  return a.d == 64 ? launch_f32<64>(a) : launch_f32<128>(a);
}

}  // namespace fa
