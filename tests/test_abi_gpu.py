"""C-ABI behaviour with real device buffers: failed validation writes nothing,
empty inputs are no-ops on every entry point, and the binding raises on
error status."""
import ctypes

import pytest
import torch

from exact_attention_70_amd import binding

pytestmark = pytest.mark.gpu


def test_misaligned_pointer_rejected_and_nothing_written(gpu):
    buf = torch.randn(1, 1, 65, 64, device=gpu).to(torch.bfloat16)
    q = buf.flatten()[1:1 + 64 * 64].view(1, 1, 64, 64)     # 2-byte offset: misaligned
    k = torch.randn(1, 1, 64, 64, device=gpu).to(torch.bfloat16)
    o = torch.full((1, 1, 64, 64), 7.0, device=gpu).to(torch.bfloat16)
    lse = torch.full((1, 1, 64), 7.0, device=gpu)
    with pytest.raises(binding.LibfaError) as ei:
        binding.fwd(q, k, k, causal=True, out=o, lse=lse)
    assert ei.value.status == -5
    torch.cuda.synchronize()
    assert bool((o.float() == 7.0).all()) and bool((lse == 7.0).all())


def test_zero_batch_is_noop(gpu):
    lib = binding.load_library()
    o = torch.full((4,), 3.0, device=gpu)
    st = lib.fa_fwd(None, None, None, ctypes.c_void_p(o.data_ptr()), None, 0, 2, 16, 64, 0.1, 1, 1,
                    None)
    torch.cuda.synchronize()
    assert st == 0 and bool((o == 3.0).all())


def test_empty_inputs_are_noops_on_every_entry_point(gpu):
    """B == 0 (fa_fwd_offset, fa_merge, fa_bwd), num_seqs == 0 (decode, GQA
    decode, prefill, KV append) and total_q == 0 (prefill) return FA_OK and
    write nothing: every output and in/out argument points at sentinels that
    keep their values."""
    lib = binding.load_library()
    bf = binding.FA_DT_BF16
    f = torch.full((1024,), 3.0, device=gpu)
    n = torch.full((64,), 5, dtype=torch.int32, device=gpu)
    fp, np_ = ctypes.c_void_p(f.data_ptr()), ctypes.c_void_p(n.data_ptr())
    ws = torch.zeros(4096, dtype=torch.uint8, device=gpu)
    wp = ctypes.c_void_p(ws.data_ptr())
    st = {
        "fa_fwd_offset": lib.fa_fwd_offset(fp, fp, fp, fp, fp, 0, 2, 64, 64, 64, 0, 0, 0.1, 1, bf,
                                           None),
        "fa_merge": lib.fa_merge(fp, fp, fp, fp, fp, fp, 0, 2, 64, 64, bf, None),
        "fa_bwd": lib.fa_bwd(fp, fp, fp, fp, fp, fp, fp, fp, fp, 0, 2, 64, 64, 0.1, 1, bf, wp,
                             4096, None),
        "fa_paged_decode": lib.fa_paged_decode(fp, fp, fp, np_, np_, 16, 0, 4, 128, 1, 1, 0.1,
                                               fp, fp, bf, wp, 4096, None),
        "fa_paged_decode_gqa": lib.fa_paged_decode_gqa(fp, fp, fp, np_, np_, 16, 0, 4, 2, 128, 1,
                                                       1, 0.1, fp, fp, bf, wp, 4096, None),
        "fa_paged_prefill (num_seqs 0)": lib.fa_paged_prefill(
            fp, np_, fp, fp, np_, np_, 0, 0, 4, 2, 128, 16, 1, 1, 1, 0.1, 1, fp, fp, bf, None),
        "fa_paged_prefill (total_q 0)": lib.fa_paged_prefill(
            fp, np_, fp, fp, np_, np_, 3, 0, 4, 2, 128, 16, 1, 1, 1, 0.1, 1, fp, fp, bf, None),
        "fa_paged_kv_append": lib.fa_paged_kv_append(fp, fp, fp, fp, np_, np_, np_, np_, np_, 0,
                                                     2, 128, 16, 1, 1, 4, bf, wp, 4096, None),
    }
    torch.cuda.synchronize()
    assert all(v == 0 for v in st.values()), st
    assert bool((f == 3.0).all()) and bool((n == 5).all())
    assert bool((ws == 0).all())


def test_unsupported_head_dim_raises(gpu):
    x = torch.zeros(1, 1, 8, 96, device=gpu, dtype=torch.bfloat16)
    with pytest.raises(binding.LibfaError) as ei:
        binding.fwd(x, x, x, causal=False)
    assert ei.value.status == -4


def test_bwd_workspace_too_small_raises(gpu):
    x = torch.zeros(1, 1, 64, 64, device=gpu, dtype=torch.bfloat16)
    lse = torch.zeros(1, 1, 64, device=gpu)
    ws = torch.empty(16, dtype=torch.uint8, device=gpu)
    with pytest.raises(binding.LibfaError) as ei:
        binding.bwd(x, x, x, x, x, lse, causal=True, workspace=ws)
    assert ei.value.status == -6


def test_binding_refuses_mismatched_tensors(gpu):
    """Plain pointers cross the C ABI, so the binding refuses tensors whose
    shape, type or device differ from what the call implies; nothing runs."""
    q = torch.zeros(1, 2, 64, 64, device=gpu, dtype=torch.bfloat16)
    o_short = torch.full((1, 2, 32, 64), 5.0, device=gpu).to(torch.bfloat16)
    with pytest.raises(ValueError):
        binding.fwd(q, q, q, causal=True, out=o_short)
    with pytest.raises(ValueError):
        binding.fwd(q, q, q, causal=True, lse=torch.zeros(1, 2, 64, device=gpu, dtype=torch.bfloat16))
    lse = torch.zeros(1, 2, 64, device=gpu)
    with pytest.raises(ValueError):
        binding.bwd(q, q, q, q, q[:, :1].contiguous(), lse, causal=True)
    with pytest.raises(ValueError):
        binding.bwd(q, q, q, q, q, lse, causal=True,
                    grads=tuple(torch.empty(1, 2, 64, 64, device=gpu, dtype=torch.bfloat16)
                                for _ in range(3)))
    qd = torch.zeros(2, 4, 128, device=gpu, dtype=torch.bfloat16)
    pool = torch.zeros(3, 16, 4, 128, device=gpu, dtype=torch.bfloat16)
    lens = torch.tensor([5, 7], device=gpu, dtype=torch.int32)
    with pytest.raises(ValueError):
        binding.paged_decode(qd, pool, pool, torch.zeros(2, 1, device=gpu, dtype=torch.int64), lens,
                             block_size=16)
    with pytest.raises(ValueError):
        binding.paged_decode(qd, pool.float(), pool.float(),
                             torch.zeros(2, 1, device=gpu, dtype=torch.int32), lens, block_size=16)
    torch.cuda.synchronize()
    assert bool((o_short.float() == 5.0).all())


def test_workspace_size_counts_bytes(gpu):
    """A workspace of another element type is sized by its bytes."""
    g = torch.Generator(device=gpu).manual_seed(3)
    q, k, v, do = (torch.randn(1, 2, 128, 64, device=gpu, generator=g).to(torch.bfloat16)
                   for _ in range(4))
    o, lse = binding.fwd(q, k, v, causal=True)
    ref = binding.bwd(q, k, v, o, do, lse, causal=True)
    ws = torch.empty(binding.bwd_workspace_size(1, 2, 128, 64) // 4, device=gpu)   # float32
    got = binding.bwd(q, k, v, o, do, lse, causal=True, workspace=ws)
    torch.cuda.synchronize()
    for a, b in zip(ref, got):
        assert torch.equal(a, b)


def test_concurrent_streams_match_serial(gpu):
    """The library keeps no device state between calls: a backward and a paged
    decode issued on two streams at once, each with its own workspace, give
    bit-identical results to the same calls run one after the other."""
    import workloads
    x = workloads.attention_inputs(1, 4, 700, 128, "bf16", seed=9500, with_do=True)
    q, k, v, do = (x[n].to(gpu) for n in ("q", "k", "v", "do"))
    o, lse = binding.fwd(q, k, v, causal=True)
    p = workloads.paged_inputs(40, 32, 128, 16, 1, 3000, seed=9501, kv_heads=8)
    pd = {n: (t.to(gpu) if isinstance(t, torch.Tensor) else t) for n, t in p.items()}

    def run_bwd():
        return binding.bwd(q, k, v, o, do, lse, causal=True)

    def run_dec():
        return binding.paged_decode(pd["q"], pd["k_pool"], pd["v_pool"], pd["block_table"],
                                    pd["seq_lens"], block_size=16)
    torch.cuda.synchronize()
    ref_b, ref_d = run_bwd(), run_dec()
    torch.cuda.synchronize()
    s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()      # default priority
    s1.wait_stream(torch.cuda.current_stream())
    s2.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s1):
        got_b = run_bwd()
    with torch.cuda.stream(s2):
        got_d = run_dec()
    torch.cuda.synchronize()
    for a, b in zip(ref_b + ref_d, got_b + got_d):
        assert torch.equal(a, b)

