// Device-side helpers shared by the libfa kernels (gfx950 / CDNA4, wave64).
//
// Matrix-core conventions used throughout (v_mfma_f32_32x32x16_bf16):
//   A operand (32 x 16): lane l supplies row (l % 32), eight k values (slot j, half l / 32)
//   B operand (16 x 32): lane l supplies column (l % 32), eight k values (slot j, half l / 32)
//   C/D (32 x 32 fp32):  lane l, register i holds column (l % 32),
//                        row 8*(i/4) + 4*(l/32) + (i%4)
// The contraction pairs A's (half, slot) with B's (half, slot), so any
// relabelling of k applied identically to both operands gives the same
// product; the kernels use this to feed a C-layout tile back in as a B
// operand without moving data between lanes.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fa {

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8;
typedef __attribute__((__vector_size__(2 * sizeof(__bf16)))) __bf16 bf16x2;
typedef __attribute__((__vector_size__(16 * sizeof(float)))) float f32x16;
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

// Bit reinterpretation goes through these by-value helpers only.  hipcc
// miscompiles __builtin_bit_cast whose operand is an element of a vector
// (e.g. bit_cast<float>(v[i])): it reads the wrong element, and the
// optimizer then narrows the vector load feeding it.
__device__ __forceinline__ float as_f32(uint32_t u) { return __builtin_bit_cast(float, u); }
__device__ __forceinline__ uint32_t as_u32(float f) { return __builtin_bit_cast(uint32_t, f); }
__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 v) { return __builtin_bit_cast(bf16x8, v); }
__device__ __forceinline__ u32x4 as_u32x4(bf16x8 v) { return __builtin_bit_cast(u32x4, v); }

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kNegInf = -__builtin_huge_valf();

// Buffer resource word 3 for raw (untyped, stride 0) buffers on gfx9-family parts.
constexpr int kRsrcWord3 = 0x00020000;

// A buffer resource over [base, base + bytes).  Loads outside the range return
// zero and stores outside it are dropped, which is how ragged tails are handled
// (and why an indexing slip cannot touch memory outside the tensor).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, (int)bytes, kRsrcWord3);
}

__device__ __forceinline__ u32x4 bload16(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_amdgcn_raw_buffer_load_b128(r, (int)off, 0, 0);
}
// Cache-policy operand of a buffer access: bit 1 is the non-temporal hint
// (NT) on gfx950, for data that is read or written once.
constexpr int kCpolNT = 2;
// 16-byte streaming load at a per-lane offset plus a wave-uniform (scalar)
// offset, with the non-temporal hint: for bytes read exactly once (the cached
// keys and values of a decode step), so they do not displace reused lines.
__device__ __forceinline__ u32x4 bload16s_nt(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff) {
  return __builtin_amdgcn_raw_buffer_load_b128(r, (int)voff, (int)soff, kCpolNT);
}
__device__ __forceinline__ u32x2 bload8(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_amdgcn_raw_buffer_load_b64(r, (int)off, 0, 0);
}
__device__ __forceinline__ float bload4f(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return as_f32(__builtin_amdgcn_raw_buffer_load_b32(r, (int)off, 0, 0));
}
__device__ __forceinline__ void bstore16(u32x4 v, __amdgpu_buffer_rsrc_t r, uint32_t off) {
  __builtin_amdgcn_raw_buffer_store_b128(v, r, (int)off, 0, 0);
}
__device__ __forceinline__ void bstore16_nt(u32x4 v, __amdgpu_buffer_rsrc_t r, uint32_t off) {
  __builtin_amdgcn_raw_buffer_store_b128(v, r, (int)off, 0, kCpolNT);
}
__device__ __forceinline__ void bstore8(u32x2 v, __amdgpu_buffer_rsrc_t r, uint32_t off) {
  __builtin_amdgcn_raw_buffer_store_b64(v, r, (int)off, 0, 0);
}
__device__ __forceinline__ void bstore4f(float v, __amdgpu_buffer_rsrc_t r, uint32_t off) {
  __builtin_amdgcn_raw_buffer_store_b32(as_u32(v), r, (int)off, 0, 0);
}

__device__ __forceinline__ f32x16 mfma_bf16(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x16 mfma_f32(float a, float b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x2f32(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ f32x16 zero16() {
  f32x16 z;
#pragma unroll
  for (int i = 0; i < 16; ++i) z[i] = 0.f;
  return z;
}

// fp32 -> packed bf16 pair, round-to-nearest-even (v_cvt_pk_bf16_f32).
__device__ __forceinline__ uint32_t pack_bf16(float lo, float hi) {
  bf16x2 h = {(__bf16)lo, (__bf16)hi};
  return __builtin_bit_cast(uint32_t, h);
}

__device__ __forceinline__ float bf16lo(uint32_t u) { return as_f32(u << 16); }
__device__ __forceinline__ float bf16hi(uint32_t u) { return as_f32(u & 0xffff0000u); }

// 16-bit input formats.  Operands travel as raw 16-byte register patterns
// (u32x4, eight values); the format decides the matrix instruction, the
// rounding of fp32 results back to 16 bits (round to nearest even), the
// widening of a packed pair, and a two-element dot product.
typedef __attribute__((__vector_size__(8 * sizeof(_Float16)))) _Float16 f16x8;
typedef __attribute__((__vector_size__(2 * sizeof(_Float16)))) _Float16 f16x2;

struct Bf16 {
  using elem = __bf16;
  static constexpr int code = 1;
  __device__ static __forceinline__ f32x16 mfma(u32x4 a, u32x4 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                   __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
  }
  __device__ static __forceinline__ uint32_t pack(float lo, float hi) { return pack_bf16(lo, hi); }
  __device__ static __forceinline__ float lo(uint32_t u) { return bf16lo(u); }
  __device__ static __forceinline__ float hi(uint32_t u) { return bf16hi(u); }
  // lo(a) * lo(b) + hi(a) * hi(b) + c, fp32 accumulation
  __device__ static __forceinline__ float dot2(uint32_t a, uint32_t b, float c) {
    return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, a),
                                           __builtin_bit_cast(bf16x2, b), c, false);
  }
  static constexpr uint32_t kOnes = 0x3f803f80u;   // the pair (1, 1)
};

struct F16 {
  using elem = _Float16;
  static constexpr int code = 2;
  __device__ static __forceinline__ f32x16 mfma(u32x4 a, u32x4 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, a),
                                                  __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
  }
  __device__ static __forceinline__ uint32_t pack(float lo, float hi) {
    f16x2 h = {(_Float16)lo, (_Float16)hi};
    return __builtin_bit_cast(uint32_t, h);
  }
  __device__ static __forceinline__ float lo(uint32_t u) {
    return (float)__builtin_bit_cast(_Float16, (uint16_t)(u & 0xffffu));
  }
  __device__ static __forceinline__ float hi(uint32_t u) {
    return (float)__builtin_bit_cast(_Float16, (uint16_t)(u >> 16));
  }
  __device__ static __forceinline__ float dot2(uint32_t a, uint32_t b, float c) {
    return __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2, a), __builtin_bit_cast(f16x2, b), c,
                                  false);
  }
  static constexpr uint32_t kOnes = 0x3c003c00u;
};

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float fast_log2(float x) { return __builtin_amdgcn_logf(x); }

// x of the lane 32 positions away (the other half of the wave), and the sum
// and maximum over lanes l and l ^ 32, which both halves get alike.  The lane
// index is formed by an asm block at each call, so the compiler can neither
// compute it once and hold it (or spill it) across a kernel nor merge calls.
// (v_permlane32_swap would need no index, but this compiler folds its two
// results into one when both are used.)
__device__ __forceinline__ float swap_half(float x) {
  int l;
  asm volatile("v_mbcnt_lo_u32_b32 %0, -1, 0\n\tv_mbcnt_hi_u32_b32 %0, -1, %0" : "=v"(l));
  return __builtin_bit_cast(float,
                            __builtin_amdgcn_ds_bpermute((l ^ 32) << 2, __builtin_bit_cast(int, x)));
}
__device__ __forceinline__ float half_sum(float x) { return x + swap_half(x); }
__device__ __forceinline__ float half_max(float x) { return fmaxf(x, swap_half(x)); }

// Workgroup barriers for LDS producer/consumer phases.  barrier_lds() waits
// only for this wave's LDS accesses (so buffer->LDS transfers it issued may
// still be in flight); barrier_all() also waits for its outstanding vector
// memory operations, which includes those transfers.  The "memory" clobber
// keeps the compiler from moving memory accesses across either barrier.
__device__ __forceinline__ void barrier_lds() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}
__device__ __forceinline__ void barrier_all() {
  asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)\n\ts_barrier" ::: "memory");
}
// Barrier after this wave's vector-memory operations older than its last N
// have completed: with buffer->LDS transfers issued in order, a tile issued
// N operations ago has landed (for every wave, once all pass the barrier)
// while the newest transfers keep streaming.
template <int N>
__device__ __forceinline__ void barrier_vm() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  asm volatile("s_waitcnt vmcnt(%0)\n\ts_barrier" ::"n"(N) : "memory");
}

// barrier_vm<N> that also waits for all of this wave's LDS accesses.
template <int N>
__device__ __forceinline__ void barrier_vm_lds() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)\n\ts_barrier" ::"n"(N) : "memory");
}

// Map the hardware workgroup id to a logical tile id so that consecutive
// logical tiles land on the same XCD: the dispatcher hands workgroups to the
// 8 XCDs round-robin, so hardware id b runs on XCD b % 8.  The map is a
// bijection on [0, n) for any n.
__device__ __forceinline__ int xcd_remap(int b, int n) {
  const int q = n >> 3, r = n & 7;
  const int xcd = b & 7, slot = b >> 3;
  return (xcd < r) ? xcd * (q + 1) + slot : r * (q + 1) + (xcd - r) * q + slot;
}

// Map hardware workgroup id b to a logical tile head * n_ranks + rank, for a
// grid of heads * n_ranks workgroups with heads a multiple of 8 and rank 0 the
// longest tile of a head.  Head h runs on XCD h % 8, so its tiles share that
// XCD's L2.  Each XCD takes its heads in groups of g (g divides heads / 8) and
// walks a group rank by rank, so the long tiles of every head in the group
// start before the short ones of any of them.  Bijective under those
// conditions, which the host checks before passing g > 0.
__device__ __forceinline__ int xcd_grouped(int b, int n_ranks, int g) {
  const int xcd = b & 7, slot = b >> 3;
  const int grp = slot / (g * n_ranks), s = slot % (g * n_ranks);
  const int u = grp * g + s % g;                 // the XCD's u-th head: xcd + 8u
  return (xcd + 8 * u) * n_ranks + s / g;
}

// --------------------------------------------------------------------------
// LDS tile layouts.  gfx950's LDS serves 256 bytes per clock as 64 banks of 4
// bytes.  Rows are stored unpadded and 16-byte chunks are XOR-swizzled so that
// each clock's worth of a matrix-operand read touches 64 distinct banks.

// Every bf16 tile is stored row-major [rows][D] with one swizzle that serves
// both kinds of operand read:
//   * 16-byte reads (A/B operands): a 16-lane clock reads the same chunk of 16
//     consecutive rows, which must land on 16 distinct 16-byte bank positions;
//   * transpose reads (ds_read_b64_tr_b16, for V^T, dO^T, Q^T, K^T operands): a
//     32-lane clock reads a 64-byte span (four chunks, 4-aligned) of each of 4
//     consecutive rows, which must land in 4 distinct 64-byte bank windows.
// D = 128 (16 chunks = 256 bytes per row): f(r) = (r & 3) << 2 | (r >> 2) & 3.
// D = 64 (8 chunks; two rows share the 256-byte bank space):
//   f(r) = ((r >> 1) & 1) << 2 | (r >> 2) & 3.
template <int D>
__device__ __forceinline__ int tile_swz(int r) {
  return (D == 128) ? (((r & 3) << 2) | ((r >> 2) & 3))
                    : ((((r >> 1) & 1) << 2) | ((r >> 2) & 3));
}
template <int D>
__device__ __forceinline__ uint32_t tile_off(int r, int c) {       // 16-byte chunk c of row r
  return (uint32_t)(r * (D * 2) + ((c ^ tile_swz<D>(r)) << 4));
}

// Transposed [D][BN] bf16 tile holding a BN = 64 key tile column-wise.  Keys
// are stored in a permuted order inside every group of 16: key k sits at
// position k with bits 2 and 3 swapped, which makes the eight keys a lane
// needs for one P V matrix step (keys 8a + 4h + c, a,c in {0,1}x{0..3}, see
// the C-layout above) contiguous.  Returns the byte offset of the 8-byte
// piece holding positions [4p, 4p + 4) of row d.
__device__ __forceinline__ int kpos(int k) {
  return (k & ~12) | ((k & 4) << 1) | ((k & 8) >> 1);
}
__device__ __forceinline__ uint32_t tr_chunk_off(int d, int c) {   // 16-byte chunk c of row d
  return (uint32_t)(d * 128 + ((c ^ ((d ^ (d >> 3)) & 7)) << 4));
}
__device__ __forceinline__ uint32_t tr_piece_off(int d, int p) {   // 8-byte piece p of row d
  return tr_chunk_off(d, p >> 1) + ((p & 1) << 3);
}

// Transposed [D][32] bf16 tile (32 keys or queries per row, 64-byte rows, four
// 16-byte chunks, same key permutation as above).
__device__ __forceinline__ uint32_t tr32_chunk_off(int d, int c) {
  return (uint32_t)(d * 64 + ((c ^ ((d >> 1) & 3)) << 4));
}
__device__ __forceinline__ uint32_t tr32_piece_off(int d, int p) {
  return tr32_chunk_off(d, p >> 1) + ((p & 1) << 3);
}

// LDS address-space pointers for the direct global->LDS and transpose-read
// instructions.
typedef __attribute__((address_space(3))) void lds_void;
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;

// Direct buffer -> LDS copy: lane i's 16 bytes (at byte offset `off` inside the
// resource; zeros when out of range) land at lds_base + 16 * i.  lds_base must
// be wave-uniform.
__device__ __forceinline__ void dma16(__amdgpu_buffer_rsrc_t r, void* lds_base, uint32_t off) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void*)lds_base, 16, (int)off, 0, 0, 0);
}

// Transpose read (ds_read_b64_tr_b16).  Within each 16-lane group, lane j
// receives element (j mod 4) of the four 16-bit values addressed by lanes
// 4k + j/4, for k = 0..3.
__device__ __forceinline__ u32x2 ds_read_tr16(const void* lds_addr) {
  const s16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)lds_addr);
  return __builtin_bit_cast(u32x2, v);
}

// Copy rows [row0, row0 + ROWS) of a [N][D] bf16 tensor into an LDS tile by
// direct buffer->LDS transfers.  Each instruction moves 1 KiB (64 lanes x 16
// bytes) into consecutive LDS bytes; the lane->source mapping applies the tile's
// chunk swizzle, so the LDS image is the swizzled row-major layout.
template <int D, int ROWS, int NWAVES>
__device__ __forceinline__ void dma_rows(__amdgpu_buffer_rsrc_t r, unsigned char* lds, int row0,
                                         int wave, int lane) {
  constexpr int DCH = D / 8;
  constexpr int RPI = 64 / DCH;             // rows per instruction
  constexpr int NI = ROWS / RPI;            // instructions per tile
  static_assert(NI % (NWAVES) == 0, "tile rows must split evenly over the waves");
#pragma unroll
  for (int ii = 0; ii < NI / (NWAVES); ++ii) {
    const int ins = ii * (NWAVES) + wave;
    const int rr = ins * RPI + lane / DCH;  // LDS row written by this lane
    const int pc = lane % DCH;              // physical chunk written by this lane
    const int c = pc ^ tile_swz<D>(rr);
    dma16(r, lds + ins * 1024, (uint32_t)((row0 + rr) * D + c * 8) * 2);
  }
}

// Store a wave's 32 x D fp32 accumulator tile (MFMA C layout: lane l holds
// row l % 32 and, in register 4g + e of 32-column block t, column
// 32t + 8g + 4(l / 32) + e), scaled by `mul`, as whole rows: the tile is
// staged in `stage` (32 * D * 4 bytes of LDS that no other wave touches) with
// swizzled 16-byte chunks, then stored 16 bytes per lane, each instruction
// covering whole rows.  Row r goes to byte (row0 + r) * D * 4 of `r_out`.
// The stores carry the non-temporal hint: the gradients are written once.
template <int D, int DT>
__device__ __forceinline__ void store_rows_f32(const f32x16 (&acc)[DT], float mul,
                                               unsigned char* stage, __amdgpu_buffer_rsrc_t r_out,
                                               int row0, int lane) {
  constexpr int CPR = D / 4;            // 16-byte chunks per row
  constexpr int RPS = 64 / CPR;         // rows per store instruction
  const int l32 = lane & 31, half = lane >> 5;
#pragma unroll
  for (int t = 0; t < DT; ++t)
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      u32x4 w;
#pragma unroll
      for (int e = 0; e < 4; ++e) w[e] = as_u32(acc[t][4 * g + e] * mul);
      const int c = t * 8 + 2 * g + half;
      *(u32x4*)(stage + l32 * (D * 4) + ((c ^ (l32 & 15)) << 4)) = w;
    }
#pragma unroll
  for (int k = 0; k < 32 / RPS; ++k) {
    const int r = k * RPS + lane / CPR, c = lane % CPR;
    const u32x4 w = *(const u32x4*)(stage + r * (D * 4) + ((c ^ (r & 15)) << 4));
    bstore16_nt(w, r_out, (uint32_t)((row0 + r) * D + 4 * c) * 4);
  }
}

template <int CTRL>
__device__ __forceinline__ float dpp_f32(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), CTRL,
                                                            0xF, 0xF, true));
}

// Sum over groups of N lanes (N = 4, 8 or 16, aligned) with DPP; every lane of
// a group receives the group total.
template <int N>
__device__ __forceinline__ float group_sum(float x) {
  x += dpp_f32<0xB1>(x);                       // quad_perm [1,0,3,2]
  x += dpp_f32<0x4E>(x);                       // quad_perm [2,3,0,1]
  if constexpr (N >= 8) x += dpp_f32<0x141>(x);    // row_half_mirror
  if constexpr (N >= 16) x += dpp_f32<0x140>(x);   // row_mirror
  return x;
}

// Transpose a 4 (keys) x 8 (d) bf16 block held as four 16-byte rows into
// eight 8-byte columns: out[j] holds keys 0..3 of column j.
__device__ __forceinline__ void transpose4x8(const u32x4 (&in)[4], u32x2 (&out)[8]) {
#pragma unroll
  for (int w = 0; w < 4; ++w) {
    // column 2w takes the low halves, column 2w+1 the high halves
    out[2 * w][0] = __builtin_amdgcn_perm(in[1][w], in[0][w], 0x05040100u);
    out[2 * w][1] = __builtin_amdgcn_perm(in[3][w], in[2][w], 0x05040100u);
    out[2 * w + 1][0] = __builtin_amdgcn_perm(in[1][w], in[0][w], 0x07060302u);
    out[2 * w + 1][1] = __builtin_amdgcn_perm(in[3][w], in[2][w], 0x07060302u);
  }
}

}  // namespace fa
