/*
 * libfa -- exact scaled-dot-product attention for AMD Instinct MI355X (gfx950).
 *
 * C ABI.  Every tensor argument is a DEVICE pointer owned by the caller; the
 * library never allocates, frees or retains caller memory.  Scratch memory
 * comes through an explicit workspace argument whose minimum size the
 * *_workspace_size queries return; the one exception is
 * fa_paged_decode_gqa_noalloc, which uses a fixed static device buffer of the
 * library's own instead (see there).  No other call keeps device state
 * between calls.
 *
 * Synchrony: each call validates its arguments on the host, enqueues its
 * kernels on `stream` (a hipStream_t passed as void*, NULL = the null stream)
 * and returns without synchronising.  Outputs are valid once the caller has
 * synchronised that stream.  Calls are stateless and may be made from several
 * host threads at once.
 *
 * Errors: status codes only; no C++ exception crosses this boundary.  Shapes,
 * dtypes, null pointers, alignment and workspace size are validated BEFORE
 * anything is launched, so a call that fails validation writes nothing.  A
 * launch failure reported by the HIP runtime maps to FA_ERR_HIP.  B == 0,
 * num_seqs == 0 or (prefill) total_q == 0 is a no-op that returns FA_OK.
 *
 * Layouts (row-major, contiguous): Q, K, V, O, dO and the fp32 gradients are
 * [B, H, N, d]; LSE is [B, H, N] fp32.  This is the [batch, heads, seq,
 * head_dim] order of the HPC notes "07-16 afternoon: distributed LLM training
 * and inference", section "Autoregressive language model inference" (the
 * tensor-shape walk-through, where Q K^T gives [B, heads, S, S] scores and
 * the softmax-weighted V gives [B, heads, S, head_dim]).  Every tensor
 * pointer must be 16-byte aligned.
 *
 * Score convention: s_ij = scale * (q_i . k_j).  With causal != 0, key j is
 * visible to query i iff j <= i (each position sees itself and the tokens
 * before it; same notes and section, on the causal mask).  LSE_i is the
 * natural log of sum over visible j of exp(s_ij).
 */
#ifndef LIBFA_FA_H
#define LIBFA_FA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  FA_OK = 0,
  FA_ERR_NULL = -1,        /* a required pointer is NULL                          */
  FA_ERR_SHAPE = -2,       /* a size is negative, zero where not allowed, or too big */
  FA_ERR_DTYPE = -3,       /* dtype code is not one of fa_dtype                    */
  FA_ERR_UNSUPPORTED = -4, /* valid but not implemented (head_dim, block_size, ...) */
  FA_ERR_ALIGN = -5,       /* a tensor pointer is not 16-byte aligned             */
  FA_ERR_WORKSPACE = -6,   /* workspace missing or smaller than the query returns */
  FA_ERR_INVALID = -7,     /* block_table / seq_lens invalid (FA_DEBUG=1), or overlapping buffers */
  FA_ERR_HIP = -8,         /* the HIP runtime reported an error                   */
  FA_ERR_SCRATCH = -9      /* needs more than the static scratch of a *_noalloc call */
} fa_status;

/* Element formats.  FA_DT_F16 is IEEE half: the explainer's mixed-precision
 * example is fp16 inputs with 32-bit matrix accumulation (dcwnkz.com
 * explainer, mixed-precision technique), and its softmax appendix shows why
 * the maximum must be subtracted first (e^12 already overflows fp16). */
typedef enum { FA_DT_F32 = 0, FA_DT_BF16 = 1, FA_DT_F16 = 2 } fa_dtype;

/* Human-readable name of a status code (static string, never NULL). */
const char* fa_status_string(int status);

/* Library version as MAJOR*10000 + MINOR*100 + PATCH. */
int fa_version(void);

/*
 * fa_fwd -- attention forward, FlashAttention-style.
 *
 * Computes O = softmax(scale * Q K^T [masked]) V and LSE per query row, as
 * defined in the dcwnkz.com GPU/FlashAttention explainer, section
 * "FlashAttention" (scores Q K^T, softmax, weighted sum of V), by scanning
 * K/V in tiles with an online softmax: a running maximum and running
 * denominator per row, with the partial output rescaled by
 * exp(m_old - m_new) whenever the maximum grows (same section, worked
 * example; CMU 10-423 L17-L18 notes, sections "Prerequisite 2: online
 * softmax" and "FlashAttention itself").  The N x N matrix never reaches
 * memory.
 *
 *   Q, K, V  in   [B,H,N,d], dtype `dtype` (FA_DT_BF16, FA_DT_F16 or FA_DT_F32)
 *   O        out  [B,H,N,d], same dtype as the inputs (16-bit: round-to-nearest-even)
 *   LSE      out  [B,H,N] fp32, natural-log log-sum-exp of the visible scaled scores
 *   B, H, N  >= 0, >= 1, >= 1 (B == 0 is a no-op); N <= 1<<20
 *   d        64 or 128 (else FA_ERR_UNSUPPORTED)
 *   scale    finite, of either sign or zero; multiplies the raw scores (1/sqrt(d) in
 *            the usual setting).  scale * q.k must stay inside the fp32 range.
 *            scale = 0 gives every visible key the same weight.
 *   causal   0 = every key visible; non-zero = key j visible to query i iff j <= i
 *
 * 16-bit inputs (bf16, fp16) are multiplied on the matrix cores with fp32
 * accumulation; the softmax weights are rounded to the input format before
 * the P V product.  fp32 inputs are multiplied with fp32 matrix instructions
 * throughout.
 */
int fa_fwd(const void* Q, const void* K, const void* V, void* O, float* LSE,
           int B, int H, int N, int d, float scale, int causal, int dtype, void* stream);

/*
 * fa_fwd_offset -- attention forward of one query block against one key/value
 * block whose rows carry global positions: query row i of the block sits at
 * q_offset + i and key row j at k_offset + j.  This is the per-step kernel of
 * ring attention (HPC notes "07-16 afternoon", section "Long context and
 * sequence parallelism"; CS231N L11 notes, context-parallel part): each rank
 * keeps its query block and meets the key/value blocks of the ring one by
 * one, combining the partial results with fa_merge.  It is also the
 * bottom-right-aligned causal forward of a prefill chunk (q_offset = Nk - Nq,
 * k_offset = 0).
 *
 *   Q        in   [B,H,Nq,d];  K, V in [B,H,Nk,d]; dtype `dtype`
 *   O        out  [B,H,Nq,d], same dtype;  LSE out [B,H,Nq] fp32
 *   Nq, Nk   1 .. 1<<20;  d 64 or 128
 *   q_offset, k_offset  global positions, |offset| <= 2^60 (else FA_ERR_SHAPE)
 *   causal   0 = every key visible; non-zero = key j visible to query i iff
 *            k_offset + j <= q_offset + i
 *
 * A query row that sees no key of the block gets O = 0 and LSE = -inf (the
 * online softmax's starting state), which fa_merge treats as weight 0.  With
 * Nq == Nk and equal offsets this is fa_fwd; arithmetic as for fa_fwd.
 */
int fa_fwd_offset(const void* Q, const void* K, const void* V, void* O, float* LSE,
                  int B, int H, int Nq, int Nk, int d, long long q_offset, long long k_offset,
                  float scale, int causal, int dtype, void* stream);

/*
 * fa_merge -- combine two partial attention results for the same queries
 * over disjoint key sets, by the rescale rule of the online softmax (HPC
 * notes "07-16 afternoon", section "Long context and sequence parallelism":
 * rescale the old accumulators by exp(m_old - m_new) before adding a block):
 *   M = max(LSE_a, LSE_b),  w = exp(LSE - M),
 *   O = (w_a O_a + w_b O_b) / (w_a + w_b),  LSE = M + ln(w_a + w_b).
 * A side with LSE = -inf weighs nothing; if both are -inf, O = 0, LSE = -inf.
 *
 *   O_a, O_b, O   [B,H,N,d] dtype `dtype` (16-bit results round to nearest even)
 *   LSE_a, LSE_b, LSE  [B,H,N] fp32
 *   O may be the same buffer as O_a or O_b, and LSE the same as LSE_a or
 *   LSE_b (in-place accumulation); a partial overlap returns FA_ERR_INVALID.
 *   d 64 or 128.  All pointers 16-byte aligned.
 */
int fa_merge(const void* O_a, const float* LSE_a, const void* O_b, const float* LSE_b,
             void* O, float* LSE, int B, int H, int N, int d, int dtype, void* stream);

/*
 * fa_fwd_offset_accumulate -- one ring-attention step in one call: the
 * forward of fa_fwd_offset for this key/value block, merged at once into a
 * running result by the rule of fa_merge (HPC notes "07-16 afternoon",
 * section "Long context and sequence parallelism").  Equivalent to
 * fa_fwd_offset into a temporary followed by fa_merge(O, LSE, temporary ->
 * O, LSE), without the temporary: the block's output never reaches HBM.
 *
 *   Q, K, V, B, H, Nq, Nk, d, offsets, scale, causal, dtype: as fa_fwd_offset
 *   O        in/out [B,H,Nq,d] dtype `dtype`: on entry the running output over
 *            the key blocks merged so far, on return the output over those
 *            blocks and this one (16-bit results round to nearest even)
 *   LSE      in/out [B,H,Nq] fp32, likewise; a row at -inf on entry has no
 *            keys yet and its O is not read into the result
 *
 * A row that sees no key of this block keeps its running result (its weight
 * is 0).  Errors as fa_fwd_offset; on an error nothing is written.
 */
int fa_fwd_offset_accumulate(const void* Q, const void* K, const void* V, void* O, float* LSE,
                             int B, int H, int Nq, int Nk, int d, long long q_offset,
                             long long k_offset, float scale, int causal, int dtype,
                             void* stream);

/*
 * fa_bwd_workspace_size -- bytes of workspace fa_bwd needs for this shape:
 * two fp32 [B,H,N] row vectors, D_i = sum_d dO_id O_id and -LSE_i log2(e),
 * rounded up to 256 bytes.
 */
size_t fa_bwd_workspace_size(int B, int H, int N, int d);

/*
 * fa_bwd -- attention backward with recomputation.
 *
 * Gradients of a loss L through O = softmax(S) V, S = scale * Q K^T, given
 * dO = dL/dO.  Following the recomputation principle of the CMU 10-423
 * L17-L18 notes (section "FlashAttention itself": never store the attention
 * matrix, recompute the needed block in the backward pass), each tile of
 * P = exp(S - LSE) is rebuilt from Q, K and the forward's LSE; nothing of
 * size N x N is stored.  The chain rule written out:
 *   dV = P^T dO;  dP = dO V^T;  D_i = sum_d dO_id O_id;  dS = P o (dP - D);
 *   dQ = scale dS K;  dK = scale dS^T Q.
 *
 *   Q, K, V, O, dO  in   [B,H,N,d] bf16 or fp16, per `dtype` (O is the forward's output)
 *   LSE             in   [B,H,N] fp32 from fa_fwd with the same scale/causal
 *   dQ, dK, dV      out  [B,H,N,d] fp32 (fully overwritten)
 *   d               64 or 128; dtype FA_DT_BF16 or FA_DT_F16 (16-bit inputs)
 *   workspace       device buffer of >= fa_bwd_workspace_size() bytes, 16-B aligned
 *   B * H * ceil(N / 128) < 2^31 (workgroups per kernel), else FA_ERR_SHAPE
 * The result is deterministic (no atomics).
 */
int fa_bwd(const void* Q, const void* K, const void* V, const void* O, const void* dO,
           const float* LSE, float* dQ, float* dK, float* dV,
           int B, int H, int N, int d, float scale, int causal, int dtype,
           void* workspace, size_t workspace_bytes, void* stream);

/*
 * fa_paged_decode_workspace_size -- bytes of workspace fa_paged_decode needs.
 * The 16-token blocks of all sequences, taken one after another, are split
 * into 256 equal shares, one per compute unit of an MI355X (one per block
 * when there are fewer blocks).  The
 * workspace holds a partial result (running max, running denominator and
 * unnormalised output row, fp32) per head for each piece of a sequence that a
 * share covers, at most 256 + num_seqs of them, followed by num_seqs + 1
 * int64 block counts.  The size does not depend on max_blocks_per_seq or
 * block_size, which are validated as for the decode call.
 */
size_t fa_paged_decode_workspace_size(int num_seqs, int H, int d, int max_blocks_per_seq,
                                      int block_size);

/*
 * fa_paged_decode -- one decode step over a paged KV cache.
 *
 * The KV cache is cut into fixed-size token blocks stored non-contiguously in
 * a shared pool; a per-sequence block table maps logical block b to a
 * physical block, and the attention kernel computes block by block (CMU
 * 10-423 L17-L18 notes, section "Decoding: PagedAttention").  Each sequence
 * feeds one new query token, which attends to all of its cached tokens,
 * itself included (HPC notes, section "Prefill, Decode and inference
 * scheduling").  Token t of sequence s is slot t % block_size of physical
 * block block_table[s, t / block_size].  The blocks of all sequences are
 * cut into equal shares of work; a sequence split over several shares has
 * its partial (max, denominator, output) triples merged by the rescaling
 * rule of the online softmax (HPC notes, section "Long context and sequence
 * parallelism").
 *
 *   q            in   [num_seqs, H, d] bf16 or fp16, per `dtype`
 *   k_pool/v_pool in  [num_blocks, block_size, H, d], same dtype
 *   block_table  in   [num_seqs, max_blocks_per_seq] int32 physical block ids;
 *                     entries past a sequence's last block are never read
 *   seq_lens     in   [num_seqs] int32, 1 <= seq_lens[s] <= max_blocks_per_seq*block_size
 *   o            out  [num_seqs, H, d], same dtype
 *   lse          out  [num_seqs, H] fp32 (natural log)
 *   block_size   16 (else FA_ERR_UNSUPPORTED); d 64 or 128 (else FA_ERR_UNSUPPORTED)
 *   H            >= 1 (any count; a wave's lanes past H idle); num_seqs * H < 2^30
 *                (else FA_ERR_SHAPE)
 *   workspace    >= fa_paged_decode_workspace_size() bytes, 16-B aligned
 * The contents of block_table and seq_lens are trusted like a page table.
 * With the environment variable FA_DEBUG=1 they are copied to the host and
 * checked first (0 <= entry < num_blocks for every block a sequence uses,
 * 1 <= seq_len <= max_blocks_per_seq*block_size); a violation returns
 * FA_ERR_INVALID and launches nothing.  Without FA_DEBUG an out-of-range
 * entry reads zeros instead of faulting.
 */
int fa_paged_decode(const void* q, const void* k_pool, const void* v_pool,
                    const int32_t* block_table, const int32_t* seq_lens, int block_size,
                    int num_seqs, int H, int d, int max_blocks_per_seq, int num_blocks,
                    float scale, void* o, float* lse, int dtype,
                    void* workspace, size_t workspace_bytes, void* stream);

/*
 * fa_paged_decode_gqa -- fa_paged_decode with grouped-query attention: the
 * pools hold KVH key/value heads, fewer than the H query heads, and query
 * head h reads cached head h / (H / KVH) (consecutive query heads share one
 * cached head; HPC notes, section "Prefill, Decode and inference scheduling":
 * with grouped-query attention kv_heads < query heads and the KV cache shrinks
 * accordingly).  One cached byte then serves H / KVH query heads.
 *
 *   k_pool/v_pool in  [num_blocks, block_size, KVH, d], dtype `dtype`
 *   KVH          >= 1 and divides H (else FA_ERR_SHAPE)
 * Every other argument, the workspace size (fa_paged_decode_workspace_size
 * with the query head count H) and the error behaviour are those of
 * fa_paged_decode, which is this call with KVH = H.
 */
int fa_paged_decode_gqa(const void* q, const void* k_pool, const void* v_pool,
                        const int32_t* block_table, const int32_t* seq_lens, int block_size,
                        int num_seqs, int H, int KVH, int d, int max_blocks_per_seq,
                        int num_blocks, float scale, void* o, float* lse, int dtype,
                        void* workspace, size_t workspace_bytes, void* stream);

/*
 * fa_paged_decode_gqa_noalloc -- fa_paged_decode_gqa for callers that cannot
 * allocate device memory: code under HIP graph capture, tight serving loops,
 * and harnesses that forbid hipMalloc.  It takes no workspace: the partial
 * results and block counts that fa_paged_decode_gqa keeps in its workspace go
 * to a static device buffer of FA_NOALLOC_SCRATCH_BYTES inside the library,
 * one per GPU, held from the first such call on that GPU until the process
 * ends.  The call allocates nothing (no hipMalloc, no allocating library
 * routine); its first call on a GPU looks up that GPU's buffer address.
 *
 * Arguments, layouts, arithmetic and results are those of fa_paged_decode_gqa
 * (KVH = H for plain multi-head decode).  A call whose workspace requirement
 * (fa_paged_decode_workspace_size) exceeds FA_NOALLOC_SCRATCH_BYTES returns
 * FA_ERR_SCRATCH and launches nothing: at H = 32, d = 128 that is about 1,750
 * sequences.  The FA_DEBUG host-side table check is not made (it would copy
 * the table to the host).
 *
 * Every call on one GPU shares that GPU's buffer, which keeps the last call's
 * contents (nothing in it needs clearing: each call writes what it reads).
 * Calls that overlap on one GPU -- on different streams, or from different
 * host threads without ordering -- race on the buffer and give undefined
 * results; serialise them (one stream, or events).
 */
#define FA_NOALLOC_SCRATCH_BYTES (32u << 20)
int fa_paged_decode_gqa_noalloc(const void* q, const void* k_pool, const void* v_pool,
                                const int32_t* block_table, const int32_t* seq_lens,
                                int block_size, int num_seqs, int H, int KVH, int d,
                                int max_blocks_per_seq, int num_blocks, float scale, void* o,
                                float* lse, int dtype, void* stream);

/*
 * fa_paged_prefill -- the forward of a chunk of new queries per sequence over
 * a paged KV cache (chunked prefill).  Prefill processes a prompt's tokens
 * together and builds the cache (HPC notes, section "Prefill, Decode and
 * inference scheduling"); the cache is read through the block table, block by
 * block (CMU 10-423 L17-L18 notes, section "Decoding: PagedAttention").
 *
 * Sequence s has seq_lens[s] cached tokens, the chunk's own K/V included
 * (append them first, e.g. with fa_paged_kv_append); its chunk is the last
 * n_s = q_start[s+1] - q_start[s] tokens, so with `causal` query r of the
 * chunk sees keys j <= seq_lens[s] - n_s + r (bottom-right alignment: the
 * offset rule of fa_fwd_offset with q_offset = seq_lens[s] - n_s).  Query
 * head h reads cached head h / (H / KVH).
 *
 *   q            in   [total_q, H, d] packed rows of all chunks, dtype bf16/fp16
 *   q_start      in   [num_seqs + 1] int32, q_start[0] = 0, ascending, <= total_q;
 *                     a chunk not inside [0, total_q) is skipped (its rows are
 *                     not written), so malformed offsets never reach memory
 *                     outside q, o and lse
 *   total_q      rows of q, o and lse; (total_q + 128) * H * d * 2 < 2^31
 *   k_pool/v_pool in  [num_blocks, 16, KVH, d], same dtype
 *   block_table  in   [num_seqs, max_blocks_per_seq] int32
 *   seq_lens     in   [num_seqs] int32, n_s <= seq_lens[s] <= max_blocks_per_seq*16;
 *                     a larger value is taken as max_blocks_per_seq*16 (as in decode)
 *   max_q_len    >= every n_s (sizes the launch), <= 1<<20
 *   o            out  [total_q, H, d], same dtype;  lse out [total_q, H] fp32
 *   block_size 16, d 64 or 128, KVH divides H (else FA_ERR_UNSUPPORTED / FA_ERR_SHAPE)
 * Cached slots past a sequence's length and out-of-range block ids read as
 * zeros.  With FA_DEBUG=1 the offsets, lengths and used table entries are
 * checked on the host first (FA_ERR_INVALID, nothing launched).  Arithmetic
 * as for fa_fwd.
 */
int fa_paged_prefill(const void* q, const int32_t* q_start, const void* k_pool, const void* v_pool,
                     const int32_t* block_table, const int32_t* seq_lens, int num_seqs,
                     int total_q, int H, int KVH, int d, int block_size, int max_blocks_per_seq,
                     int num_blocks, int max_q_len, float scale, int causal, void* o, float* lse,
                     int dtype, void* stream);

/*
 * fa_paged_kv_append_workspace_size -- bytes of workspace fa_paged_kv_append
 * needs: one int32 pool-slot index per sequence, rounded up to 256 bytes.
 */
size_t fa_paged_kv_append_workspace_size(int num_seqs);

/*
 * fa_paged_kv_append -- write one new token's K and V for every sequence into
 * a paged KV cache, taking blocks on demand from a stack of free blocks.
 *
 * Blocks are allocated only when needed (CMU 10-423 L17-L18 notes, section
 * "Decoding: PagedAttention"); the runtime keeps each sequence's length and
 * block mapping (HPC notes, section "Prefill, Decode and inference
 * scheduling").  Sequence s writes its token at position t = seq_lens[s]:
 *   - when t is a multiple of block_size (its blocks are full), it takes the
 *     block on top of the free stack, free_list[*free_count - 1], and stores
 *     it in block_table[s, t / block_size]; sequences take blocks in sequence
 *     order, so the stack is popped as if they were served one by one;
 *   - the token's K and V rows go to slot t % block_size of the sequence's
 *     block table[s, t / block_size], and seq_lens[s] becomes t + 1.
 * A sequence whose table is full (t >= max_blocks_per_seq * block_size), that
 * needs a block when the stack is empty, or whose block id is outside the
 * pool is left unchanged (nothing written) and counted in *n_failed.
 *
 *   k_new, v_new   in     [num_seqs, KVH, d], dtype `dtype` (bf16, fp16 or fp32)
 *   k_pool, v_pool in/out [num_blocks, block_size, KVH, d], same dtype
 *   block_table    in/out [num_seqs, max_blocks_per_seq] int32
 *   seq_lens       in/out [num_seqs] int32
 *   free_list      in     [free_capacity] int32 physical ids; entries
 *                         [0, *free_count) are the stack, top last
 *   free_count     in/out device int32 scalar: stack height, reduced by the
 *                         blocks taken
 *   n_failed       out    device int32 scalar
 *   KVH * d * element size must be a multiple of 16 bytes (else
 *   FA_ERR_UNSUPPORTED); num_blocks * block_size < 2^31.
 *   workspace      >= fa_paged_kv_append_workspace_size(num_seqs) bytes.
 * num_seqs == 0 is a no-op that writes nothing.  All device pointers are the
 * caller's; tensor pointers 16-byte aligned, int32 pointers 4-byte aligned.
 * With FA_DEBUG=1 the lengths, the stack height and the stack's ids are
 * checked on the host first (FA_ERR_INVALID, nothing launched).  Calls are
 * ordered on `stream`; two calls that share a pool must not overlap.
 */
int fa_paged_kv_append(const void* k_new, const void* v_new, void* k_pool, void* v_pool,
                       int32_t* block_table, int32_t* seq_lens, const int32_t* free_list,
                       int32_t* free_count, int32_t* n_failed, int num_seqs, int KVH, int d,
                       int block_size, int max_blocks_per_seq, int num_blocks, int free_capacity,
                       int dtype, void* workspace, size_t workspace_bytes, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* LIBFA_FA_H */
