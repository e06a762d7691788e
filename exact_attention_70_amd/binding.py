"""Thin ctypes binding of libfa.

Argument marshalling only: every step of the attention computation runs in
the HIP kernels behind the C ABI declared in include/fa.h.  torch is used for
device memory (output and workspace allocation) and for the current HIP
stream.  If the shared library is missing or fails to load, every entry point
raises; there is no fallback implementation.
"""
from __future__ import annotations

import ctypes
import math
import os

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libfa.so")

FA_DT_F32 = 0
FA_DT_BF16 = 1
FA_DT_F16 = 2

EXPORTED = ("fa_status_string", "fa_version", "fa_fwd", "fa_fwd_offset", "fa_merge",
            "fa_fwd_offset_accumulate",
            "fa_bwd_workspace_size", "fa_bwd", "fa_paged_decode_workspace_size", "fa_paged_decode",
            "fa_paged_decode_gqa", "fa_paged_decode_gqa_noalloc",
            "fa_paged_kv_append_workspace_size", "fa_paged_kv_append", "fa_paged_prefill")

# bytes of the static scratch behind fa_paged_decode_gqa_noalloc (FA_NOALLOC_SCRATCH_BYTES)
NOALLOC_SCRATCH_BYTES = 32 << 20

_lib = None


class LibfaError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {status_string(status)} ({status})")


def load_library(path: str | None = None) -> ctypes.CDLL:
    """Load libfa.so (once) and declare the C signatures.

    The in-tree library is used unless ``path`` or the LIBFA_PATH environment
    variable names another build of the same C ABI.
    """
    global _lib
    if _lib is not None and path is None:
        return _lib
    p = path or os.environ.get("LIBFA_PATH") or LIB_PATH
    if not os.path.exists(p):
        raise RuntimeError(f"libfa shared library not found at {p}; build it with "
                           "`python -m exact_attention_70_amd.build` (hipcc, gfx950)")
    lib = ctypes.CDLL(p)
    vp, i, f, sz = ctypes.c_void_p, ctypes.c_int, ctypes.c_float, ctypes.c_size_t
    lib.fa_status_string.argtypes = [i]
    lib.fa_status_string.restype = ctypes.c_char_p
    lib.fa_version.argtypes = []
    lib.fa_version.restype = i
    lib.fa_fwd.argtypes = [vp, vp, vp, vp, vp, i, i, i, i, f, i, i, vp]
    lib.fa_fwd.restype = i
    ll = ctypes.c_longlong
    lib.fa_fwd_offset.argtypes = [vp, vp, vp, vp, vp, i, i, i, i, i, ll, ll, f, i, i, vp]
    lib.fa_fwd_offset.restype = i
    lib.fa_fwd_offset_accumulate.argtypes = [vp, vp, vp, vp, vp, i, i, i, i, i, ll, ll, f, i, i, vp]
    lib.fa_fwd_offset_accumulate.restype = i
    lib.fa_merge.argtypes = [vp, vp, vp, vp, vp, vp, i, i, i, i, i, vp]
    lib.fa_merge.restype = i
    lib.fa_bwd_workspace_size.argtypes = [i, i, i, i]
    lib.fa_bwd_workspace_size.restype = sz
    lib.fa_bwd.argtypes = [vp] * 9 + [i, i, i, i, f, i, i, vp, sz, vp]
    lib.fa_bwd.restype = i
    lib.fa_paged_decode_workspace_size.argtypes = [i, i, i, i, i]
    lib.fa_paged_decode_workspace_size.restype = sz
    lib.fa_paged_decode.argtypes = [vp, vp, vp, vp, vp, i, i, i, i, i, i, f, vp, vp, i, vp, sz, vp]
    lib.fa_paged_decode.restype = i
    lib.fa_paged_decode_gqa.argtypes = [vp, vp, vp, vp, vp, i, i, i, i, i, i, i, f, vp, vp, i, vp, sz,
                                        vp]
    lib.fa_paged_decode_gqa.restype = i
    lib.fa_paged_decode_gqa_noalloc.argtypes = [vp, vp, vp, vp, vp] + [i] * 7 + [f, vp, vp, i, vp]
    lib.fa_paged_decode_gqa_noalloc.restype = i
    lib.fa_paged_kv_append_workspace_size.argtypes = [i]
    lib.fa_paged_kv_append_workspace_size.restype = sz
    lib.fa_paged_kv_append.argtypes = [vp] * 9 + [i] * 8 + [vp, sz, vp]
    lib.fa_paged_kv_append.restype = i
    lib.fa_paged_prefill.argtypes = [vp] * 6 + [i] * 9 + [f, i, vp, vp, i, vp]
    lib.fa_paged_prefill.restype = i
    if path is None:
        _lib = lib
    return lib


def status_string(status: int) -> str:
    return load_library().fa_status_string(int(status)).decode()


def _check(status: int, where: str):
    if status != 0:
        raise LibfaError(status, where)


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(device) -> ctypes.c_void_p:
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.bfloat16:
        return FA_DT_BF16
    if t.dtype == torch.float16:
        return FA_DT_F16
    if t.dtype == torch.float32:
        return FA_DT_F32
    raise TypeError(f"libfa supports bf16, fp16 and fp32 tensors, got {t.dtype}")


def _need_cuda(*ts):
    for t in ts:
        if not (isinstance(t, torch.Tensor) and t.is_cuda and t.is_contiguous()):
            raise ValueError("libfa expects contiguous device tensors")


def _want(t, shape, dtype, device, name):
    """The kernels index every tensor by the shapes they are told, so a tensor
    of another shape, type or device would be read or written out of bounds:
    refuse it here, before any pointer reaches the library."""
    if not (isinstance(t, torch.Tensor) and t.is_cuda and t.is_contiguous()):
        raise ValueError(f"{name} must be a contiguous device tensor")
    if tuple(t.shape) != tuple(shape) or t.dtype != dtype or t.device != device:
        raise ValueError(f"{name} must be {tuple(shape)} {dtype} on {device}, got "
                         f"{tuple(t.shape)} {t.dtype} on {t.device}")
    return t


def _workspace(ws, nbytes, device):
    if ws is None:
        return torch.empty(max(nbytes, 16), dtype=torch.uint8, device=device)
    _need_cuda(ws)
    if ws.device != device:
        raise ValueError(f"workspace must be on {device}")
    return ws


def _nbytes(t) -> int:
    return t.numel() * t.element_size()


def _check_pool(k_pool, v_pool, like, block_size, KVH, d):
    if k_pool.dim() != 4 or k_pool.shape[1] != block_size or k_pool.shape[2:] != (KVH, d):
        raise ValueError(f"k_pool must be [num_blocks, {block_size}, {KVH}, {d}], got "
                         f"{tuple(k_pool.shape)}")
    _want(k_pool, tuple(k_pool.shape), like.dtype, like.device, "k_pool")
    _want(v_pool, tuple(k_pool.shape), like.dtype, like.device, "v_pool")


def fwd(q, k, v, *, causal: bool, scale: float | None = None, out=None, lse=None):
    """O, LSE = attention(q, k, v) for [B, H, N, d] device tensors (bf16, fp16 or fp32)."""
    _need_cuda(q, k, v)
    B, H, N, d = q.shape
    if k.shape != q.shape or v.shape != q.shape or k.dtype != q.dtype or v.dtype != q.dtype:
        raise ValueError("q, k, v must share shape [B, H, N, d] and dtype")
    scale = 1.0 / math.sqrt(d) if scale is None else float(scale)
    o = torch.empty_like(q) if out is None else _want(out, q.shape, q.dtype, q.device, "out")
    l = (torch.empty((B, H, N), dtype=torch.float32, device=q.device) if lse is None
         else _want(lse, (B, H, N), torch.float32, q.device, "lse"))
    st = load_library().fa_fwd(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(l), B, H, N, d, scale,
                               int(bool(causal)), _dtype_code(q), _stream(q.device))
    _check(st, "fa_fwd")
    return o, l


def fwd_offset(q, k, v, *, q_offset: int, k_offset: int, causal: bool, scale: float | None = None,
               out=None, lse=None):
    """O, LSE of a query block [B, H, Nq, d] against a key/value block [B, H, Nk, d]
    whose rows sit at global positions q_offset + i and k_offset + j."""
    _need_cuda(q, k, v)
    B, H, Nq, d = q.shape
    Nk = k.shape[2]
    if (k.shape[:2] != q.shape[:2] or k.shape[3] != d or v.shape != k.shape
            or k.dtype != q.dtype or v.dtype != q.dtype):
        raise ValueError("q [B,H,Nq,d], k and v [B,H,Nk,d] must share B, H, d and dtype")
    scale = 1.0 / math.sqrt(d) if scale is None else float(scale)
    o = torch.empty_like(q) if out is None else _want(out, q.shape, q.dtype, q.device, "out")
    l = (torch.empty((B, H, Nq), dtype=torch.float32, device=q.device) if lse is None
         else _want(lse, (B, H, Nq), torch.float32, q.device, "lse"))
    st = load_library().fa_fwd_offset(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(l), B, H, Nq, Nk, d,
                                      int(q_offset), int(k_offset), scale, int(bool(causal)),
                                      _dtype_code(q), _stream(q.device))
    _check(st, "fa_fwd_offset")
    return o, l


def fwd_offset_accumulate(q, k, v, o, lse, *, q_offset: int, k_offset: int, causal: bool,
                          scale: float | None = None):
    """Merge the attention of q [B, H, Nq, d] against the key/value block k, v
    [B, H, Nk, d] (rows at global positions q_offset + i, k_offset + j) into the
    running result o [B, H, Nq, d], lse [B, H, Nq] (fp32), in place."""
    _need_cuda(q, k, v, o, lse)
    B, H, Nq, d = q.shape
    Nk = k.shape[2]
    if (k.shape[:2] != q.shape[:2] or k.shape[3] != d or v.shape != k.shape
            or k.dtype != q.dtype or v.dtype != q.dtype):
        raise ValueError("q [B,H,Nq,d], k and v [B,H,Nk,d] must share B, H, d and dtype")
    _want(o, q.shape, q.dtype, q.device, "o")
    _want(lse, (B, H, Nq), torch.float32, q.device, "lse")
    scale = 1.0 / math.sqrt(d) if scale is None else float(scale)
    st = load_library().fa_fwd_offset_accumulate(
        _ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), B, H, Nq, Nk, d, int(q_offset),
        int(k_offset), scale, int(bool(causal)), _dtype_code(q), _stream(q.device))
    _check(st, "fa_fwd_offset_accumulate")
    return o, lse


def merge(o_a, lse_a, o_b, lse_b, *, out=None, lse_out=None):
    """Combine two partial results over disjoint key sets; ``out``/``lse_out`` may
    be ``o_a``/``lse_a`` (or the b side) for in-place accumulation."""
    _need_cuda(o_a, o_b, lse_a, lse_b)
    B, H, N, d = o_a.shape
    if o_b.shape != o_a.shape or o_b.dtype != o_a.dtype or lse_a.shape != (B, H, N) \
            or lse_b.shape != (B, H, N):
        raise ValueError("partials must share [B, H, N, d] / [B, H, N] shapes and dtype")
    if lse_a.dtype != torch.float32 or lse_b.dtype != torch.float32:
        raise ValueError("lse_a and lse_b must be float32")
    o = torch.empty_like(o_a) if out is None else _want(out, o_a.shape, o_a.dtype, o_a.device, "out")
    l = (torch.empty_like(lse_a) if lse_out is None
         else _want(lse_out, (B, H, N), torch.float32, o_a.device, "lse_out"))
    st = load_library().fa_merge(_ptr(o_a), _ptr(lse_a), _ptr(o_b), _ptr(lse_b), _ptr(o), _ptr(l),
                                 B, H, N, d, _dtype_code(o_a), _stream(o_a.device))
    _check(st, "fa_merge")
    return o, l


def bwd_workspace_size(B, H, N, d) -> int:
    return int(load_library().fa_bwd_workspace_size(B, H, N, d))


def bwd(q, k, v, o, do, lse, *, causal: bool, scale: float | None = None, workspace=None,
        grads=None):
    """dQ, dK, dV (fp32) of attention given the forward's O and LSE and dO."""
    _need_cuda(q, k, v, o, do, lse)
    B, H, N, d = q.shape
    for t, name in ((k, "k"), (v, "v"), (o, "o"), (do, "do")):
        _want(t, q.shape, q.dtype, q.device, name)
    _want(lse, (B, H, N), torch.float32, q.device, "lse")
    scale = 1.0 / math.sqrt(d) if scale is None else float(scale)
    if grads is None:
        grads = tuple(torch.empty((B, H, N, d), dtype=torch.float32, device=q.device)
                      for _ in range(3))
    dq, dk, dv = (_want(g, (B, H, N, d), torch.float32, q.device, n)
                  for g, n in zip(grads, ("dq", "dk", "dv")))
    workspace = _workspace(workspace, bwd_workspace_size(B, H, N, d), q.device)
    st = load_library().fa_bwd(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(do), _ptr(lse), _ptr(dq),
                               _ptr(dk), _ptr(dv), B, H, N, d, scale, int(bool(causal)),
                               _dtype_code(q), _ptr(workspace), _nbytes(workspace),
                               _stream(q.device))
    _check(st, "fa_bwd")
    return dq, dk, dv


def paged_decode_workspace_size(num_seqs, H, d, max_blocks_per_seq, block_size) -> int:
    return int(load_library().fa_paged_decode_workspace_size(num_seqs, H, d, max_blocks_per_seq,
                                                             block_size))


def paged_decode(q, k_pool, v_pool, block_table, seq_lens, *, block_size: int,
                 scale: float | None = None, workspace=None, out=None, lse=None):
    """o [S, H, d] bf16 and lse [S, H] fp32 of one decode step over a paged KV pool.

    The pools are [num_blocks, block_size, KVH, d]; KVH < H (grouped-query
    attention) calls fa_paged_decode_gqa, KVH == H fa_paged_decode.
    """
    _need_cuda(q, k_pool, v_pool, block_table, seq_lens)
    S, H, d = q.shape
    num_blocks, KVH = k_pool.shape[0], k_pool.shape[2]
    mbps = block_table.shape[1]
    _check_pool(k_pool, v_pool, q, block_size, KVH, d)
    _want(block_table, (S, mbps), torch.int32, q.device, "block_table")
    _want(seq_lens, (S,), torch.int32, q.device, "seq_lens")
    scale = 1.0 / math.sqrt(d) if scale is None else float(scale)
    o = torch.empty_like(q) if out is None else _want(out, q.shape, q.dtype, q.device, "out")
    l = (torch.empty((S, H), dtype=torch.float32, device=q.device) if lse is None
         else _want(lse, (S, H), torch.float32, q.device, "lse"))
    workspace = _workspace(workspace, paged_decode_workspace_size(S, H, d, mbps, block_size),
                           q.device)
    lib = load_library()
    if KVH == H:
        st = lib.fa_paged_decode(
            _ptr(q), _ptr(k_pool), _ptr(v_pool), _ptr(block_table), _ptr(seq_lens), block_size, S,
            H, d, mbps, num_blocks, scale, _ptr(o), _ptr(l), _dtype_code(q), _ptr(workspace),
            _nbytes(workspace), _stream(q.device))
        _check(st, "fa_paged_decode")
    else:
        st = lib.fa_paged_decode_gqa(
            _ptr(q), _ptr(k_pool), _ptr(v_pool), _ptr(block_table), _ptr(seq_lens), block_size, S,
            H, KVH, d, mbps, num_blocks, scale, _ptr(o), _ptr(l), _dtype_code(q), _ptr(workspace),
            _nbytes(workspace), _stream(q.device))
        _check(st, "fa_paged_decode_gqa")
    return o, l


def paged_decode_noalloc(q, k_pool, v_pool, block_table, seq_lens, *, block_size: int,
                         scale: float | None = None, out=None, lse=None):
    """paged_decode through fa_paged_decode_gqa_noalloc: no workspace, the
    library's static per-GPU scratch instead.  With ``out`` and ``lse`` given,
    the call allocates nothing at all."""
    _need_cuda(q, k_pool, v_pool, block_table, seq_lens)
    S, H, d = q.shape
    num_blocks, KVH = k_pool.shape[0], k_pool.shape[2]
    mbps = block_table.shape[1]
    _check_pool(k_pool, v_pool, q, block_size, KVH, d)
    _want(block_table, (S, mbps), torch.int32, q.device, "block_table")
    _want(seq_lens, (S,), torch.int32, q.device, "seq_lens")
    scale = 1.0 / math.sqrt(d) if scale is None else float(scale)
    o = torch.empty_like(q) if out is None else _want(out, q.shape, q.dtype, q.device, "out")
    l = (torch.empty((S, H), dtype=torch.float32, device=q.device) if lse is None
         else _want(lse, (S, H), torch.float32, q.device, "lse"))
    st = load_library().fa_paged_decode_gqa_noalloc(
        _ptr(q), _ptr(k_pool), _ptr(v_pool), _ptr(block_table), _ptr(seq_lens), block_size, S, H,
        KVH, d, mbps, num_blocks, scale, _ptr(o), _ptr(l), _dtype_code(q), _stream(q.device))
    _check(st, "fa_paged_decode_gqa_noalloc")
    return o, l


def paged_kv_append(k_new, v_new, k_pool, v_pool, block_table, seq_lens, free_list, free_count,
                    n_failed, *, block_size: int, workspace=None):
    """Write one token's K/V per sequence into the paged pools (in place), taking
    blocks from the free stack on demand.  ``free_count`` and ``n_failed`` are
    one-element int32 device tensors; every argument is updated in place."""
    _need_cuda(k_new, v_new, k_pool, v_pool, block_table, seq_lens, free_list, free_count,
               n_failed)
    S, KVH, d = k_new.shape
    dev = k_new.device
    _want(v_new, k_new.shape, k_new.dtype, dev, "v_new")
    _check_pool(k_pool, v_pool, k_new, block_size, KVH, d)
    if block_table.dim() != 2 or block_table.shape[0] != S:
        raise ValueError("block_table must be [S, max_blocks_per_seq]")
    _want(block_table, tuple(block_table.shape), torch.int32, dev, "block_table")
    _want(seq_lens, (S,), torch.int32, dev, "seq_lens")
    _want(free_list, (free_list.numel(),), torch.int32, dev, "free_list")
    _want(free_count, (1,), torch.int32, dev, "free_count")
    _want(n_failed, (1,), torch.int32, dev, "n_failed")
    lib = load_library()
    workspace = _workspace(workspace, int(lib.fa_paged_kv_append_workspace_size(S)), dev)
    st = lib.fa_paged_kv_append(
        _ptr(k_new), _ptr(v_new), _ptr(k_pool), _ptr(v_pool), _ptr(block_table), _ptr(seq_lens),
        _ptr(free_list), _ptr(free_count), _ptr(n_failed), S, KVH, d, block_size,
        block_table.shape[1], k_pool.shape[0], free_list.numel(), _dtype_code(k_new),
        _ptr(workspace), _nbytes(workspace), _stream(k_new.device))
    _check(st, "fa_paged_kv_append")


def paged_prefill(q, q_start, k_pool, v_pool, block_table, seq_lens, *, block_size: int,
                  max_q_len: int, causal: bool = True, scale: float | None = None, out=None,
                  lse=None):
    """o [total_q, H, d] and lse [total_q, H] of chunked prefill over a paged cache."""
    _need_cuda(q, q_start, k_pool, v_pool, block_table, seq_lens)
    T, H, d = q.shape
    S = seq_lens.numel()
    KVH = k_pool.shape[2]
    _check_pool(k_pool, v_pool, q, block_size, KVH, d)
    _want(q_start, (S + 1,), torch.int32, q.device, "q_start")
    _want(seq_lens, (S,), torch.int32, q.device, "seq_lens")
    if block_table.dim() != 2 or block_table.shape[0] != S:
        raise ValueError("block_table must be [S, max_blocks_per_seq]")
    _want(block_table, tuple(block_table.shape), torch.int32, q.device, "block_table")
    scale = 1.0 / math.sqrt(d) if scale is None else float(scale)
    o = torch.empty_like(q) if out is None else _want(out, q.shape, q.dtype, q.device, "out")
    l = (torch.empty((T, H), dtype=torch.float32, device=q.device) if lse is None
         else _want(lse, (T, H), torch.float32, q.device, "lse"))
    st = load_library().fa_paged_prefill(
        _ptr(q), _ptr(q_start), _ptr(k_pool), _ptr(v_pool), _ptr(block_table), _ptr(seq_lens), S, T,
        H, KVH, d, block_size, block_table.shape[1], k_pool.shape[0], int(max_q_len), scale,
        int(bool(causal)), _ptr(o), _ptr(l), _dtype_code(q), _stream(q.device))
    _check(st, "fa_paged_prefill")
    return o, l
