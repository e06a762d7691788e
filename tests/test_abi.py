"""C-ABI checks that need no GPU: the library loads, exports every function
include/fa.h declares, and rejects invalid arguments on the host before any
launch (these calls return before touching the HIP runtime)."""
import ctypes
import os
import re

import pytest

from exact_attention_70_amd import binding as libfa

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "fa.h")

OK, ERR_NULL, ERR_SHAPE, ERR_DTYPE, ERR_UNSUP, ERR_ALIGN, ERR_WS, ERR_INVALID, ERR_HIP = \
    0, -1, -2, -3, -4, -5, -6, -7, -8

# fake but 16-byte aligned, non-null addresses: every call below fails host
# validation before anything could dereference them
P = ctypes.c_void_p(0x10000)
P2 = ctypes.c_void_p(0x20000)
MIS = ctypes.c_void_p(0x10008)


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(fa_[a-z_0-9]+)\s*\(", text)))


@pytest.fixture(scope="module")
def lib():
    return libfa.load_library()


def test_header_declares_the_boundary():
    names = declared_functions()
    for n in ("fa_fwd", "fa_fwd_offset", "fa_fwd_offset_accumulate", "fa_merge", "fa_bwd",
              "fa_paged_decode",
              "fa_paged_decode_gqa", "fa_paged_kv_append", "fa_paged_kv_append_workspace_size",
              "fa_paged_prefill",
              "fa_bwd_workspace_size", "fa_paged_decode_workspace_size", "fa_status_string",
              "fa_version"):
        assert n in names


def test_every_declared_symbol_is_exported(lib):
    for name in declared_functions():
        assert hasattr(lib, name), name
    assert set(declared_functions()) == set(libfa.EXPORTED)


def test_status_strings(lib):
    for code in (OK, ERR_NULL, ERR_SHAPE, ERR_DTYPE, ERR_UNSUP, ERR_ALIGN, ERR_WS, ERR_INVALID,
                 ERR_HIP):
        s = libfa.status_string(code)
        assert s.startswith("FA_") or code == OK
    assert libfa.status_string(12345) == "unknown libfa status"
    assert lib.fa_version() >= 100


def fwd(lib, q=P, k=P, v=P, o=P2, lse=P2, B=1, H=1, N=64, d=64, scale=0.125, causal=1, dt=1):
    return lib.fa_fwd(q, k, v, o, lse, B, H, N, d, scale, causal, dt, None)


def test_fwd_validation(lib):
    assert fwd(lib, dt=7) == ERR_DTYPE
    assert fwd(lib, H=0) == ERR_SHAPE
    assert fwd(lib, N=0) == ERR_SHAPE
    assert fwd(lib, B=-1) == ERR_SHAPE
    assert fwd(lib, N=(1 << 20) + 1) == ERR_SHAPE
    assert fwd(lib, scale=float("nan")) == ERR_SHAPE
    assert fwd(lib, scale=float("inf")) == ERR_SHAPE
    assert fwd(lib, d=96) == ERR_UNSUP
    assert fwd(lib, d=256) == ERR_UNSUP
    assert fwd(lib, q=None) == ERR_NULL
    assert fwd(lib, lse=None) == ERR_NULL
    assert fwd(lib, v=MIS) == ERR_ALIGN
    assert fwd(lib, o=MIS) == ERR_ALIGN
    # B == 0 is a no-op (nothing is touched, so even NULL pointers are fine)
    assert fwd(lib, B=0, q=None, k=None, v=None, o=None, lse=None) == OK


def fwd_off(lib, q=P, k=P, v=P, o=P2, lse=P2, B=1, H=1, Nq=64, Nk=96, d=64, qo=0, ko=0, scale=0.125,
            causal=1, dt=1):
    return lib.fa_fwd_offset(q, k, v, o, lse, B, H, Nq, Nk, d, qo, ko, scale, causal, dt, None)


def test_fwd_offset_validation(lib):
    assert fwd_off(lib, dt=3) == ERR_DTYPE
    assert fwd_off(lib, Nq=0) == ERR_SHAPE
    assert fwd_off(lib, Nk=0) == ERR_SHAPE
    assert fwd_off(lib, Nk=(1 << 20) + 1) == ERR_SHAPE
    assert fwd_off(lib, qo=(1 << 60) + 1) == ERR_SHAPE
    assert fwd_off(lib, ko=-(1 << 60) - 1) == ERR_SHAPE
    assert fwd_off(lib, scale=float("nan")) == ERR_SHAPE
    assert fwd_off(lib, d=80) == ERR_UNSUP
    assert fwd_off(lib, k=None) == ERR_NULL
    assert fwd_off(lib, v=MIS) == ERR_ALIGN
    # B == 0 is a no-op even with NULL pointers
    assert fwd_off(lib, B=0, q=None, k=None, v=None, o=None, lse=None) == OK


def fwd_acc(lib, q=P, k=P, v=P, o=P2, lse=P2, B=1, H=1, Nq=64, Nk=96, d=64, qo=0, ko=0,
            scale=0.125, causal=1, dt=1):
    return lib.fa_fwd_offset_accumulate(q, k, v, o, lse, B, H, Nq, Nk, d, qo, ko, scale, causal,
                                        dt, None)


def test_fwd_offset_accumulate_validation(lib):
    """The fused ring step takes the arguments of fa_fwd_offset (O and LSE in
    and out) and refuses the same things, before any launch."""
    assert fwd_acc(lib, dt=3) == ERR_DTYPE
    assert fwd_acc(lib, Nq=0) == ERR_SHAPE
    assert fwd_acc(lib, Nk=(1 << 20) + 1) == ERR_SHAPE
    assert fwd_acc(lib, qo=(1 << 60) + 1) == ERR_SHAPE
    assert fwd_acc(lib, scale=float("inf")) == ERR_SHAPE
    assert fwd_acc(lib, d=96) == ERR_UNSUP
    assert fwd_acc(lib, lse=None) == ERR_NULL
    assert fwd_acc(lib, o=MIS) == ERR_ALIGN
    assert fwd_acc(lib, B=0, q=None, k=None, v=None, o=None, lse=None) == OK


def merge(lib, oa=P, la=P, ob=P2, lb=P2, o=ctypes.c_void_p(0x40000), l=ctypes.c_void_p(0x80000),
          B=1, H=2, N=64, d=64, dt=1):
    return lib.fa_merge(oa, la, ob, lb, o, l, B, H, N, d, dt, None)


def test_merge_validation(lib):
    assert merge(lib, dt=9) == ERR_DTYPE
    assert merge(lib, N=0) == ERR_SHAPE
    assert merge(lib, H=0) == ERR_SHAPE
    assert merge(lib, d=32) == ERR_UNSUP
    assert merge(lib, ob=None) == ERR_NULL
    assert merge(lib, lb=MIS) == ERR_ALIGN
    # an output shifted into an input (not the same buffer) is refused
    assert merge(lib, o=ctypes.c_void_p(0x10000 + 64)) == ERR_INVALID
    assert merge(lib, l=ctypes.c_void_p(0x20000 + 16)) == ERR_INVALID
    assert merge(lib, B=0, oa=None, la=None, ob=None, lb=None, o=None, l=None) == OK


def test_bwd_validation(lib):
    ws = lib.fa_bwd_workspace_size(2, 3, 100, 128)
    assert ws >= 2 * (2 * 3 * 100 * 4) and ws % 256 == 0
    assert lib.fa_bwd_workspace_size(0, 3, 100, 128) == 0

    def bwd(dt=1, d=128, N=100, ws_ptr=P2, ws_bytes=ws, dq=P2, B=2, H=3, scale=0.1):
        return lib.fa_bwd(P, P, P, P, P, P, dq, P2, P2, B, H, N, d, scale, 1, dt, ws_ptr,
                          ws_bytes, None)
    assert bwd(dt=0) == ERR_UNSUP          # fp32 backward not provided
    assert bwd(dt=5) == ERR_DTYPE
    assert bwd(d=80) == ERR_UNSUP
    assert bwd(N=0) == ERR_SHAPE
    assert bwd(ws_ptr=None) == ERR_WS
    assert bwd(ws_bytes=ws - 1) == ERR_WS
    assert bwd(dq=None) == ERR_NULL
    assert bwd(dq=MIS) == ERR_ALIGN
    assert bwd(scale=float("nan")) == ERR_SHAPE
    # workgroup counts past 2^31 are refused before the workspace is looked at
    assert bwd(B=1 << 12, H=1 << 12, N=128 * 128) == ERR_SHAPE
    assert bwd(B=0) == OK


def test_decode_validation(lib):
    ws = lib.fa_paged_decode_workspace_size(64, 32, 128, 256, 16)
    # partials of 256 shares of the block stream plus one per sequence, 32
    # heads, (m, l, 128 outputs) fp32 each; then 65 int64 prefix sums
    assert ws >= (256 + 64) * 32 * 130 * 4 + 65 * 8
    assert ws % 256 == 0
    assert lib.fa_paged_decode_workspace_size(0, 32, 128, 256, 16) == 0

    def dec(bs=16, S=4, H=32, d=128, mbps=8, nb=40, dt=1, ws_ptr=P2, ws_bytes=None,
            table=P, q=P):
        wsb = lib.fa_paged_decode_workspace_size(max(S, 1), H, d, mbps, bs) if ws_bytes is None \
            else ws_bytes
        return lib.fa_paged_decode(q, P, P, table, P, bs, S, H, d, mbps, nb, 0.1, P2, P2, dt,
                                   ws_ptr, wsb, None)
    assert dec(bs=32) == ERR_UNSUP
    assert dec(d=96) == ERR_UNSUP
    assert dec(d=64, S=0) == OK                  # head dims 64 and 128
    assert dec(H=6, S=0) == OK                   # any head count
    assert dec(dt=0) == ERR_UNSUP
    assert dec(dt=3) == ERR_DTYPE
    assert dec(nb=0) == ERR_SHAPE
    assert dec(mbps=0) == ERR_SHAPE
    assert dec(ws_ptr=None) == ERR_WS
    assert dec(ws_bytes=16) == ERR_WS
    assert dec(table=None) == ERR_NULL
    assert dec(q=MIS) == ERR_ALIGN
    assert dec(table=ctypes.c_void_p(0x10002)) == ERR_ALIGN
    assert dec(S=0) == OK


def test_python_binding_refuses_host_tensors():
    import torch
    x = torch.zeros(1, 1, 4, 64, dtype=torch.bfloat16)
    with pytest.raises(ValueError):
        libfa.fwd(x, x, x, causal=True)


def gqa(lib, H=32, KVH=8, d=128, bs=16, dt=1, S=4, q=P):
    ws = lib.fa_paged_decode_workspace_size(S, H, d, 8, bs)
    return lib.fa_paged_decode_gqa(q, P, P, P, P, bs, S, H, KVH, d, 8, 100, 0.1, P2, P2, dt, P2, ws,
                                   None)


def test_paged_decode_gqa_validation(lib):
    assert gqa(lib, KVH=0) == ERR_SHAPE
    assert gqa(lib, KVH=5) == ERR_SHAPE          # must divide H
    assert gqa(lib, KVH=64) == ERR_SHAPE
    assert gqa(lib, d=80) == ERR_UNSUP
    assert gqa(lib, q=None) == ERR_NULL
    assert gqa(lib, S=0, q=None) == OK
    assert gqa(lib, S=1 << 25, H=32, KVH=8) == ERR_SHAPE    # num_seqs * H >= 2^30


def noalloc(lib, H=32, KVH=32, d=128, bs=16, dt=1, S=4, q=P):
    return lib.fa_paged_decode_gqa_noalloc(q, P, P, P, P, bs, S, H, KVH, d, 8, 100, 0.1, P2, P2, dt,
                                           None)


def test_paged_decode_noalloc_validation(lib):
    """The allocation-free decode checks its arguments like the workspace
    decode, and refuses a call whose partials exceed its static scratch
    (FA_NOALLOC_SCRATCH_BYTES) before any device work."""
    ERR_SCRATCH = -9
    assert "FA_ERR_SCRATCH" in libfa.status_string(ERR_SCRATCH)
    assert noalloc(lib, KVH=5) == ERR_SHAPE
    assert noalloc(lib, d=32) == ERR_UNSUP
    assert noalloc(lib, bs=8) == ERR_UNSUP
    assert noalloc(lib, dt=3) == ERR_DTYPE
    assert noalloc(lib, q=None) == ERR_NULL
    assert noalloc(lib, q=MIS) == ERR_ALIGN
    assert noalloc(lib, S=0, q=None) == OK
    # the largest sequence count whose workspace fits the scratch, and one more
    fits = max(s for s in range(1, 4000)
               if lib.fa_paged_decode_workspace_size(s, 32, 128, 8, 16) <= libfa.NOALLOC_SCRATCH_BYTES)
    assert 1500 < fits < 2000
    assert noalloc(lib, S=fits + 1) == ERR_SCRATCH
    assert noalloc(lib, S=4000, H=64, KVH=8) == ERR_SCRATCH


def append(lib, S=4, KVH=8, d=128, bs=16, mbps=8, nb=100, cap=10, dt=1, kn=P, ws=P2, wsb=None,
           fl=P, fc=P):
    wsb = lib.fa_paged_kv_append_workspace_size(S) if wsb is None else wsb
    return lib.fa_paged_kv_append(kn, P, P, P, P, P, fl, fc, P, S, KVH, d, bs, mbps, nb, cap, dt,
                                  ws, wsb, None)


def test_paged_kv_append_validation(lib):
    assert lib.fa_paged_kv_append_workspace_size(10) == 256
    assert lib.fa_paged_kv_append_workspace_size(0) == 0
    assert append(lib, dt=4) == ERR_DTYPE
    assert append(lib, KVH=0) == ERR_SHAPE
    assert append(lib, cap=-1) == ERR_SHAPE
    assert append(lib, nb=1 << 28) == ERR_SHAPE          # slots past 2^31
    assert append(lib, KVH=1, d=4) == ERR_UNSUP          # 8-byte rows
    assert append(lib, kn=None) == ERR_NULL
    assert append(lib, fl=None) == ERR_NULL              # a stack with capacity needs a list
    assert append(lib, kn=MIS) == ERR_ALIGN
    assert append(lib, fc=ctypes.c_void_p(0x10002)) == ERR_ALIGN
    assert append(lib, wsb=16) == ERR_WS
    assert append(lib, S=0, kn=None) == OK


def prefill(lib, S=3, T=96, H=8, KVH=2, d=128, bs=16, mq=64, dt=1, q=P, causal=1):
    return lib.fa_paged_prefill(q, P, P, P, P, P, S, T, H, KVH, d, bs, 8, 100, mq, 0.1, causal, P2,
                                P2, dt, None)


def test_paged_prefill_validation(lib):
    assert prefill(lib, dt=9) == ERR_DTYPE
    assert prefill(lib, mq=0) == ERR_SHAPE
    assert prefill(lib, KVH=3) == ERR_SHAPE
    assert prefill(lib, dt=0) == ERR_UNSUP
    assert prefill(lib, bs=32) == ERR_UNSUP
    assert prefill(lib, d=96) == ERR_UNSUP
    assert prefill(lib, q=None) == ERR_NULL
    assert prefill(lib, q=MIS) == ERR_ALIGN
    assert prefill(lib, S=0, q=None) == OK
    assert prefill(lib, T=-1) == ERR_SHAPE
    assert prefill(lib, T=1 << 20, H=32) == ERR_SHAPE    # packed rows past 32-bit offsets
    assert prefill(lib, T=0, q=None) == OK
