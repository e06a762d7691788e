// C-ABI entry points of libfa: argument validation, workspace sizing and
// dispatch to the kernel launchers.  Nothing here computes attention; every
// arithmetic step runs in the HIP kernels.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdlib>
#include <cstring>
#include <vector>

#include "../../include/fa.h"
#include "fa_internal.h"

static_assert(fa::kNoAllocScratchBytes == (size_t)FA_NOALLOC_SCRATCH_BYTES,
              "the header states the static scratch size");

namespace {

constexpr int kMaxN = 1 << 20;

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

int hip_status(hipError_t e) { return e == hipSuccess ? FA_OK : FA_ERR_HIP; }

bool debug_checks() {
  const char* s = std::getenv("FA_DEBUG");
  return s != nullptr && s[0] != '\0' && s[0] != '0';
}

size_t round_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

// Per-head byte sizes must fit the 32-bit range of a buffer resource.
bool head_fits(long long N, long long d, long long elem) { return N * d * elem < (1LL << 31); }

// Global positions handed to fa_fwd_offset (their difference must not overflow).
constexpr long long kMaxOffset = 1LL << 60;

// Two equal-length buffers overlap without being the same buffer.
bool partial_overlap(const void* x, const void* y, size_t bytes) {
  const auto a = reinterpret_cast<uintptr_t>(x), b = reinterpret_cast<uintptr_t>(y);
  return a != b && a < b + bytes && b < a + bytes;
}

}  // namespace

extern "C" {

const char* fa_status_string(int status) {
  switch (status) {
    case FA_OK: return "FA_OK";
    case FA_ERR_NULL: return "FA_ERR_NULL: a required pointer is NULL";
    case FA_ERR_SHAPE: return "FA_ERR_SHAPE: invalid size";
    case FA_ERR_DTYPE: return "FA_ERR_DTYPE: unknown dtype code";
    case FA_ERR_UNSUPPORTED: return "FA_ERR_UNSUPPORTED: configuration not implemented";
    case FA_ERR_ALIGN: return "FA_ERR_ALIGN: tensor pointer not 16-byte aligned";
    case FA_ERR_WORKSPACE: return "FA_ERR_WORKSPACE: workspace missing or too small";
    case FA_ERR_INVALID: return "FA_ERR_INVALID: invalid contents or overlapping buffers";
    case FA_ERR_HIP: return "FA_ERR_HIP: HIP runtime error";
    case FA_ERR_SCRATCH:
      return "FA_ERR_SCRATCH: the call needs more than the library's static scratch "
             "(FA_NOALLOC_SCRATCH_BYTES); use the workspace entry point";
    default: return "unknown libfa status";
  }
}

int fa_version(void) { return 100; }

namespace {
int fwd_offset_impl(const void* Q, const void* K, const void* V, void* O, float* LSE, int B, int H,
                    int Nq, int Nk, int d, long long q_offset, long long k_offset, float scale,
                    int causal, int dtype, void* stream, bool accumulate) {
  if (dtype != FA_DT_F32 && dtype != FA_DT_BF16 && dtype != FA_DT_F16) return FA_ERR_DTYPE;
  if (B < 0 || H < 1 || Nq < 1 || Nq > kMaxN || Nk < 1 || Nk > kMaxN || d < 1) return FA_ERR_SHAPE;
  if (q_offset < -kMaxOffset || q_offset > kMaxOffset || k_offset < -kMaxOffset ||
      k_offset > kMaxOffset)
    return FA_ERR_SHAPE;
  if (!std::isfinite(scale)) return FA_ERR_SHAPE;
  if (d != 64 && d != 128) return FA_ERR_UNSUPPORTED;
  const int elem = dtype == FA_DT_F32 ? 4 : 2;
  if (!head_fits(Nq, d, elem) || !head_fits(Nk, d, elem)) return FA_ERR_SHAPE;
  if ((long long)B * H * ((Nq + 31) / 32) >= (1LL << 31)) return FA_ERR_SHAPE;
  if (B == 0) return FA_OK;
  if (!Q || !K || !V || !O || !LSE) return FA_ERR_NULL;
  if (!aligned16(Q) || !aligned16(K) || !aligned16(V) || !aligned16(O) || !aligned16(LSE))
    return FA_ERR_ALIGN;
  fa::FwdArgs a{Q, K, V, O, LSE, B, H, Nq, d, scale, causal != 0, dtype,
                reinterpret_cast<hipStream_t>(stream)};
  a.Nk = Nk;
  a.delta = q_offset - k_offset;
  a.accumulate = accumulate;
  return hip_status(fa::launch_fwd(a));
}
}  // namespace

int fa_fwd_offset(const void* Q, const void* K, const void* V, void* O, float* LSE, int B, int H,
                  int Nq, int Nk, int d, long long q_offset, long long k_offset, float scale,
                  int causal, int dtype, void* stream) {
  return fwd_offset_impl(Q, K, V, O, LSE, B, H, Nq, Nk, d, q_offset, k_offset, scale, causal,
                         dtype, stream, false);
}

int fa_fwd_offset_accumulate(const void* Q, const void* K, const void* V, void* O, float* LSE,
                             int B, int H, int Nq, int Nk, int d, long long q_offset,
                             long long k_offset, float scale, int causal, int dtype,
                             void* stream) {
  return fwd_offset_impl(Q, K, V, O, LSE, B, H, Nq, Nk, d, q_offset, k_offset, scale, causal,
                         dtype, stream, true);
}

int fa_fwd(const void* Q, const void* K, const void* V, void* O, float* LSE, int B, int H, int N,
           int d, float scale, int causal, int dtype, void* stream) {
  return fa_fwd_offset(Q, K, V, O, LSE, B, H, N, N, d, 0, 0, scale, causal, dtype, stream);
}

int fa_merge(const void* O_a, const float* LSE_a, const void* O_b, const float* LSE_b, void* O,
             float* LSE, int B, int H, int N, int d, int dtype, void* stream) {
  if (dtype != FA_DT_F32 && dtype != FA_DT_BF16 && dtype != FA_DT_F16) return FA_ERR_DTYPE;
  if (B < 0 || H < 1 || N < 1 || N > kMaxN || d < 1) return FA_ERR_SHAPE;
  if (d != 64 && d != 128) return FA_ERR_UNSUPPORTED;
  if (B == 0) return FA_OK;
  if (!O_a || !LSE_a || !O_b || !LSE_b || !O || !LSE) return FA_ERR_NULL;
  if (!aligned16(O_a) || !aligned16(O_b) || !aligned16(O) || !aligned16(LSE_a) ||
      !aligned16(LSE_b) || !aligned16(LSE))
    return FA_ERR_ALIGN;
  const long long rows = (long long)B * H * N;
  const size_t obytes = (size_t)rows * d * (dtype == FA_DT_F32 ? 4 : 2);   // bf16 / fp16: 2
  const size_t lbytes = (size_t)rows * sizeof(float);
  // outputs may be exactly an input buffer (in-place accumulation), never a shifted overlap
  if (partial_overlap(O, O_a, obytes) || partial_overlap(O, O_b, obytes) ||
      partial_overlap(LSE, LSE_a, lbytes) || partial_overlap(LSE, LSE_b, lbytes))
    return FA_ERR_INVALID;
  fa::MergeArgs a{O_a, LSE_a, O_b, LSE_b, O, LSE, rows, d, dtype,
                  reinterpret_cast<hipStream_t>(stream)};
  return hip_status(fa::launch_merge(a));
}

size_t fa_bwd_workspace_size(int B, int H, int N, int d) {
  (void)d;
  if (B <= 0 || H <= 0 || N <= 0) return 0;
  // D_i and -LSE_i log2(e), fp32 [B, H, N] each
  return round_up(2 * (size_t)B * H * N * sizeof(float), 256);
}

int fa_bwd(const void* Q, const void* K, const void* V, const void* O, const void* dO,
           const float* LSE, float* dQ, float* dK, float* dV, int B, int H, int N, int d,
           float scale, int causal, int dtype, void* workspace, size_t workspace_bytes,
           void* stream) {
  if (dtype != FA_DT_F32 && dtype != FA_DT_BF16 && dtype != FA_DT_F16) return FA_ERR_DTYPE;
  if (B < 0 || H < 1 || N < 1 || N > kMaxN || d < 1) return FA_ERR_SHAPE;
  if (!std::isfinite(scale)) return FA_ERR_SHAPE;
  if (dtype == FA_DT_F32) return FA_ERR_UNSUPPORTED;   // 16-bit inputs only
  if (d != 64 && d != 128) return FA_ERR_UNSUPPORTED;
  if (!head_fits(N, d, 4)) return FA_ERR_SHAPE;
  // one workgroup per 128-row tile of every head in each of the two kernels
  if ((long long)B * H * ((N + 127) / 128) >= (1LL << 31)) return FA_ERR_SHAPE;
  if (B == 0) return FA_OK;
  if (!Q || !K || !V || !O || !dO || !LSE || !dQ || !dK || !dV) return FA_ERR_NULL;
  if (!workspace || workspace_bytes < fa_bwd_workspace_size(B, H, N, d)) return FA_ERR_WORKSPACE;
  const void* ptrs[] = {Q, K, V, O, dO, LSE, dQ, dK, dV, workspace};
  for (const void* p : ptrs)
    if (!aligned16(p)) return FA_ERR_ALIGN;
  fa::BwdArgs a{Q, K, V, O, dO, LSE, dQ, dK, dV, static_cast<float*>(workspace),
                B, H, N, d, scale, causal != 0, reinterpret_cast<hipStream_t>(stream)};
  a.dtype = dtype;
  return hip_status(fa::launch_bwd(a));
}

size_t fa_paged_decode_workspace_size(int num_seqs, int H, int d, int max_blocks_per_seq,
                                      int block_size) {
  if (num_seqs <= 0 || H <= 0 || d <= 0 || max_blocks_per_seq <= 0 || block_size <= 0) return 0;
  // per (slot, head): m, l, then d output values (fp32); then the num_seqs + 1
  // block prefix sums (int64)
  return round_up(fa::decode_partials_floats(num_seqs, H, d) * sizeof(float) +
                      ((size_t)num_seqs + 1) * sizeof(long long),
                  256);
}

namespace {

// Argument checks shared by the decode entry points, before any device work:
// FA_OK to go on, or the status to return (1: a no-op, num_seqs == 0).
int check_decode_args(const void* q, const void* k_pool, const void* v_pool,
                      const int32_t* block_table, const int32_t* seq_lens, int block_size,
                      int num_seqs, int H, int KVH, int d, int max_blocks_per_seq, int num_blocks,
                      float scale, void* o, float* lse, int dtype) {
  if (dtype != FA_DT_F32 && dtype != FA_DT_BF16 && dtype != FA_DT_F16) return FA_ERR_DTYPE;
  if (num_seqs < 0 || H < 1 || KVH < 1 || d < 1 || max_blocks_per_seq < 1 || num_blocks < 1 ||
      block_size < 1)
    return FA_ERR_SHAPE;
  if (H % KVH != 0) return FA_ERR_SHAPE;
  // (sequence, head) pairs are counted in 32-bit integers by the launches
  if ((long long)num_seqs * H >= (1LL << 30)) return FA_ERR_SHAPE;
  if (!std::isfinite(scale)) return FA_ERR_SHAPE;
  if (dtype == FA_DT_F32 || block_size != 16 || (d != 64 && d != 128)) return FA_ERR_UNSUPPORTED;
  const long long block_bytes = (long long)block_size * KVH * d * 2;
  if (block_bytes >= (1LL << 31)) return FA_ERR_SHAPE;
  if ((long long)max_blocks_per_seq * block_size > kMaxN) return FA_ERR_SHAPE;
  if (num_seqs == 0) return 1;
  if (!q || !k_pool || !v_pool || !block_table || !seq_lens || !o || !lse)
    return FA_ERR_NULL;
  const void* ptrs[] = {q, k_pool, v_pool, o, lse};
  for (const void* p : ptrs)
    if (!aligned16(p)) return FA_ERR_ALIGN;
  if ((reinterpret_cast<uintptr_t>(block_table) & 3u) || (reinterpret_cast<uintptr_t>(seq_lens) & 3u))
    return FA_ERR_ALIGN;
  return FA_OK;
}

}  // namespace

int fa_paged_decode_gqa(const void* q, const void* k_pool, const void* v_pool,
                        const int32_t* block_table, const int32_t* seq_lens, int block_size,
                        int num_seqs, int H, int KVH, int d, int max_blocks_per_seq, int num_blocks,
                        float scale, void* o, float* lse, int dtype, void* workspace,
                        size_t workspace_bytes, void* stream) {
  const int chk = check_decode_args(q, k_pool, v_pool, block_table, seq_lens, block_size, num_seqs,
                                    H, KVH, d, max_blocks_per_seq, num_blocks, scale, o, lse, dtype);
  if (chk == 1) return FA_OK;
  if (chk != FA_OK) return chk;
  const size_t need =
      fa_paged_decode_workspace_size(num_seqs, H, d, max_blocks_per_seq, block_size);
  if (!workspace || workspace_bytes < need) return FA_ERR_WORKSPACE;
  if (!aligned16(workspace)) return FA_ERR_ALIGN;
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  if (debug_checks()) {
    std::vector<int32_t> tbl((size_t)num_seqs * max_blocks_per_seq), lens(num_seqs);
    if (hipMemcpyAsync(lens.data(), seq_lens, lens.size() * 4, hipMemcpyDeviceToHost, st) !=
            hipSuccess ||
        hipMemcpyAsync(tbl.data(), block_table, tbl.size() * 4, hipMemcpyDeviceToHost, st) !=
            hipSuccess ||
        hipStreamSynchronize(st) != hipSuccess)
      return FA_ERR_HIP;
    for (int s = 0; s < num_seqs; ++s) {
      const int L = lens[s];
      if (L < 1 || (long long)L > (long long)max_blocks_per_seq * block_size) return FA_ERR_INVALID;
      const int nb = (L + block_size - 1) / block_size;
      for (int b = 0; b < nb; ++b) {
        const int32_t p = tbl[(size_t)s * max_blocks_per_seq + b];
        if (p < 0 || p >= num_blocks) return FA_ERR_INVALID;
      }
    }
  }
  fa::DecodeArgs a{q, k_pool, v_pool, block_table, seq_lens, block_size, num_seqs, H, d,
                   max_blocks_per_seq, num_blocks, scale, o, lse,
                   static_cast<float*>(workspace), fa::kDecodeUnits, st};
  a.KVH = KVH;
  a.dtype = dtype;
  return hip_status(fa::launch_decode(a));
}

int fa_paged_decode_gqa_noalloc(const void* q, const void* k_pool, const void* v_pool,
                                const int32_t* block_table, const int32_t* seq_lens,
                                int block_size, int num_seqs, int H, int KVH, int d,
                                int max_blocks_per_seq, int num_blocks, float scale, void* o,
                                float* lse, int dtype, void* stream) {
  const int chk = check_decode_args(q, k_pool, v_pool, block_table, seq_lens, block_size, num_seqs,
                                    H, KVH, d, max_blocks_per_seq, num_blocks, scale, o, lse, dtype);
  if (chk == 1) return FA_OK;
  if (chk != FA_OK) return chk;
  if (fa_paged_decode_workspace_size(num_seqs, H, d, max_blocks_per_seq, block_size) >
      fa::kNoAllocScratchBytes)
    return FA_ERR_SCRATCH;
  void* scratch = nullptr;
  const hipError_t e = fa::noalloc_scratch(&scratch);
  if (e != hipSuccess) return FA_ERR_HIP;
  fa::DecodeArgs a{q, k_pool, v_pool, block_table, seq_lens, block_size, num_seqs, H, d,
                   max_blocks_per_seq, num_blocks, scale, o, lse,
                   static_cast<float*>(scratch), fa::kDecodeUnits,
                   reinterpret_cast<hipStream_t>(stream)};
  a.KVH = KVH;
  a.dtype = dtype;
  return hip_status(fa::launch_decode(a));
}

int fa_paged_decode(const void* q, const void* k_pool, const void* v_pool,
                    const int32_t* block_table, const int32_t* seq_lens, int block_size,
                    int num_seqs, int H, int d, int max_blocks_per_seq, int num_blocks,
                    float scale, void* o, float* lse, int dtype, void* workspace,
                    size_t workspace_bytes, void* stream) {
  return fa_paged_decode_gqa(q, k_pool, v_pool, block_table, seq_lens, block_size, num_seqs, H, H,
                             d, max_blocks_per_seq, num_blocks, scale, o, lse, dtype, workspace,
                             workspace_bytes, stream);
}

int fa_paged_prefill(const void* q, const int32_t* q_start, const void* k_pool, const void* v_pool,
                     const int32_t* block_table, const int32_t* seq_lens, int num_seqs,
                     int total_q, int H, int KVH, int d, int block_size, int max_blocks_per_seq,
                     int num_blocks, int max_q_len, float scale, int causal, void* o, float* lse,
                     int dtype, void* stream) {
  if (dtype != FA_DT_F32 && dtype != FA_DT_BF16 && dtype != FA_DT_F16) return FA_ERR_DTYPE;
  if (num_seqs < 0 || total_q < 0 || H < 1 || KVH < 1 || d < 1 || block_size < 1 ||
      max_blocks_per_seq < 1 || num_blocks < 1 || max_q_len < 1 || max_q_len > kMaxN)
    return FA_ERR_SHAPE;
  // the packed tensors are addressed through 32-bit buffer offsets (plus the
  // rows a last query tile reads past the end)
  if (((long long)total_q + 128) * H * d * 2 >= (1LL << 31)) return FA_ERR_SHAPE;
  if (H % KVH != 0 || !std::isfinite(scale)) return FA_ERR_SHAPE;
  if (dtype == FA_DT_F32 || block_size != 16 || (d != 64 && d != 128)) return FA_ERR_UNSUPPORTED;
  if ((long long)max_q_len * H * d * 2 >= (1LL << 31)) return FA_ERR_SHAPE;
  if ((long long)max_blocks_per_seq * block_size > kMaxN) return FA_ERR_SHAPE;
  if ((long long)block_size * KVH * d * 2 >= (1LL << 31)) return FA_ERR_SHAPE;
  if ((long long)num_seqs * H * ((max_q_len + 127) / 128) >= (1LL << 31)) return FA_ERR_SHAPE;
  if (num_seqs == 0 || total_q == 0) return FA_OK;
  if (!q || !q_start || !k_pool || !v_pool || !block_table || !seq_lens || !o || !lse)
    return FA_ERR_NULL;
  const void* ptrs[] = {q, k_pool, v_pool, o};
  for (const void* p : ptrs)
    if (!aligned16(p)) return FA_ERR_ALIGN;
  const void* ints[] = {q_start, block_table, seq_lens, lse};
  for (const void* p : ints)
    if (reinterpret_cast<uintptr_t>(p) & 3u) return FA_ERR_ALIGN;
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  if (debug_checks()) {
    // chunk offsets ascend with chunks <= max_q_len, each chunk fits inside its
    // sequence's cached tokens, and every block the sequence uses is in the pool
    std::vector<int32_t> starts(num_seqs + 1), lens(num_seqs),
        tbl((size_t)num_seqs * max_blocks_per_seq);
    if (hipMemcpyAsync(starts.data(), q_start, starts.size() * 4, hipMemcpyDeviceToHost, st) !=
            hipSuccess ||
        hipMemcpyAsync(lens.data(), seq_lens, lens.size() * 4, hipMemcpyDeviceToHost, st) !=
            hipSuccess ||
        hipMemcpyAsync(tbl.data(), block_table, tbl.size() * 4, hipMemcpyDeviceToHost, st) !=
            hipSuccess ||
        hipStreamSynchronize(st) != hipSuccess)
      return FA_ERR_HIP;
    if (starts[0] != 0 || starts[num_seqs] > total_q) return FA_ERR_INVALID;
    for (int s = 0; s < num_seqs; ++s) {
      const int n = starts[s + 1] - starts[s], L = lens[s];
      if (n < 0 || n > max_q_len || L < n || (long long)L > (long long)max_blocks_per_seq * block_size)
        return FA_ERR_INVALID;
      for (int b = 0; b < (L + block_size - 1) / block_size; ++b) {
        const int32_t p = tbl[(size_t)s * max_blocks_per_seq + b];
        if (p < 0 || p >= num_blocks) return FA_ERR_INVALID;
      }
    }
  }
  fa::FwdArgs a{q, k_pool, v_pool, o, lse, num_seqs, H, max_q_len, d, scale, causal != 0, dtype, st};
  a.paged = true;
  a.table = block_table;
  a.q_start = q_start;
  a.seq_lens = seq_lens;
  a.KVH = KVH;
  a.max_blocks = max_blocks_per_seq;
  a.num_blocks = num_blocks;
  a.total_q = total_q;
  return hip_status(fa::launch_fwd(a));
}

size_t fa_paged_kv_append_workspace_size(int num_seqs) {
  if (num_seqs <= 0) return 0;
  return round_up((size_t)num_seqs * sizeof(int32_t), 256);   // the per-sequence slot map
}

int fa_paged_kv_append(const void* k_new, const void* v_new, void* k_pool, void* v_pool,
                       int32_t* block_table, int32_t* seq_lens, const int32_t* free_list,
                       int32_t* free_count, int32_t* n_failed, int num_seqs, int KVH, int d,
                       int block_size, int max_blocks_per_seq, int num_blocks, int free_capacity,
                       int dtype, void* workspace, size_t workspace_bytes, void* stream) {
  if (dtype != FA_DT_F32 && dtype != FA_DT_BF16 && dtype != FA_DT_F16) return FA_ERR_DTYPE;
  if (num_seqs < 0 || KVH < 1 || d < 1 || block_size < 1 || max_blocks_per_seq < 1 ||
      num_blocks < 1 || free_capacity < 0)
    return FA_ERR_SHAPE;
  const long long row_bytes = (long long)KVH * d * (dtype == FA_DT_F32 ? 4 : 2);
  if (row_bytes % 16 != 0 || row_bytes >= (1LL << 31)) return FA_ERR_UNSUPPORTED;
  if ((long long)num_blocks * block_size >= (1LL << 31)) return FA_ERR_SHAPE;
  if ((long long)max_blocks_per_seq * block_size > (1LL << 30)) return FA_ERR_SHAPE;
  if (num_seqs == 0) return FA_OK;
  if (!k_new || !v_new || !k_pool || !v_pool || !block_table || !seq_lens || !free_count ||
      !n_failed || (free_capacity > 0 && !free_list))
    return FA_ERR_NULL;
  if (!aligned16(k_new) || !aligned16(v_new) || !aligned16(k_pool) || !aligned16(v_pool) ||
      !aligned16(workspace))
    return FA_ERR_ALIGN;
  const void* ints[] = {block_table, seq_lens, free_list, free_count, n_failed};
  for (const void* p : ints)
    if (reinterpret_cast<uintptr_t>(p) & 3u) return FA_ERR_ALIGN;
  if (!workspace || workspace_bytes < fa_paged_kv_append_workspace_size(num_seqs))
    return FA_ERR_WORKSPACE;
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  if (debug_checks()) {
    // lengths within the table, stack height within the list, stack ids in the pool
    std::vector<int32_t> lens(num_seqs), fl(free_capacity > 0 ? free_capacity : 0);
    int32_t fc = 0;
    if (hipMemcpyAsync(lens.data(), seq_lens, lens.size() * 4, hipMemcpyDeviceToHost, st) !=
            hipSuccess ||
        hipMemcpyAsync(&fc, free_count, 4, hipMemcpyDeviceToHost, st) != hipSuccess ||
        (!fl.empty() && hipMemcpyAsync(fl.data(), free_list, fl.size() * 4,
                                       hipMemcpyDeviceToHost, st) != hipSuccess) ||
        hipStreamSynchronize(st) != hipSuccess)
      return FA_ERR_HIP;
    for (int s = 0; s < num_seqs; ++s)
      if (lens[s] < 0 || (long long)lens[s] > (long long)max_blocks_per_seq * block_size)
        return FA_ERR_INVALID;
    if (fc < 0 || fc > free_capacity) return FA_ERR_INVALID;
    for (int i = 0; i < fc; ++i)
      if (fl[i] < 0 || fl[i] >= num_blocks) return FA_ERR_INVALID;
  }
  fa::AppendArgs a{k_new, v_new, k_pool, v_pool, block_table, seq_lens, free_list, free_count,
                   n_failed, static_cast<int32_t*>(workspace), num_seqs, block_size,
                   max_blocks_per_seq, num_blocks, free_capacity, (int)row_bytes, st};
  return hip_status(fa::launch_append(a));
}

}  // extern "C"
