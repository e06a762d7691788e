"""GPU parity of chunked prefill over a paged KV cache (fa_paged_prefill)
against the fp64 oracle on the same seeded inputs.

Tolerance: max-abs 2e-2 on O and LSE for bf16, 1e-2 for fp16 (the bounds of
the contiguous forward for those formats).  Pad slots past each sequence's
length hold NaN, which must never reach the result.
"""
import math

import numpy as np
import pytest
import torch

import oracle
import workloads
from conftest import max_abs
from exact_attention_70_amd import binding

pytestmark = pytest.mark.gpu

TOL = {"bf16": 2e-2, "f16": 1e-2}


def _run(gpu, lens, chunks, H, kvh, d, dtype, seed, causal=True, rows=None):
    p = workloads.paged_inputs(len(lens), H, d, 16, 1, max(lens), seed=seed, dtype=dtype,
                               seq_lens=lens, kv_heads=kvh, pad_value=float("nan"))
    qq = workloads.prefill_queries(chunks, H, d, dtype, seed=seed + 1)
    pd = {k: (v.to(gpu) if isinstance(v, torch.Tensor) else v) for k, v in p.items()}
    o, lse = binding.paged_prefill(qq["q"].to(gpu), qq["q_start"].to(gpu), pd["k_pool"],
                                   pd["v_pool"], pd["block_table"], pd["seq_lens"], block_size=16,
                                   max_q_len=max(chunks), causal=causal, scale=d ** -0.5)
    torch.cuda.synchronize()
    ro, rl = oracle.paged_prefill(qq["q"], qq["q_start"], p["k_pool"], p["v_pool"],
                                  p["block_table"], p["seq_lens"], 16, d ** -0.5, causal)
    go, gl = o.double().cpu().numpy(), lse.double().cpu().numpy()
    if rows is not None:
        go, gl, ro, rl = go[rows], gl[rows], ro[rows], rl[rows]
    assert np.all(np.isfinite(go)) and np.all(np.isfinite(gl))
    assert max_abs(go, ro) <= TOL[dtype]
    assert max_abs(gl, rl) <= TOL[dtype]


LENS = [1, 17, 64, 100, 200, 300]
CHUNKS = [1, 17, 10, 64, 129, 300]       # single token, whole sequence, partial chunks


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("kvh", [8, 2])
def test_paged_prefill_matches_oracle(gpu, dtype, d, kvh):
    _run(gpu, LENS, CHUNKS, 8, kvh, d, dtype, seed=7000 + d + kvh)


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
@pytest.mark.parametrize("d", [64, 128])
def test_paged_prefill_noncausal(gpu, dtype, d):
    _run(gpu, LENS, CHUNKS, 8, 4, d, dtype, seed=7100 + d, causal=False)


def test_paged_prefill_long_chunks_gqa(gpu):
    """The benchmark's prefill shape: eight sequences with 1024-token chunks
    over 1500..4000 cached tokens, 32 query heads on 8 cached heads; every row
    and head."""
    lens = [1500, 2048, 2500, 3000, 3333, 3700, 4000, 1024]
    chunks = [1024] * 8
    _run(gpu, lens, chunks, 32, 8, 128, "bf16", seed=7200)


@pytest.mark.parametrize("n_seqs", [64, 65])
def test_paged_prefill_many_sequences_in_any_order(gpu, n_seqs):
    """Workgroups take the sequences of a call longest first (by the keys an
    average query tile reads) when there are at most 64 of them, and in their
    own order beyond: 64 and 65 sequences whose lengths, chunk lengths and tie
    patterns are mixed (equal keys included), every row checked."""
    rng = np.random.default_rng(7300 + n_seqs)
    lens = [int(x) for x in rng.integers(1, 400, n_seqs)]
    lens[3] = lens[7] = 250                       # equal keys: ties broken by index
    chunks = [int(rng.integers(1, L + 1)) for L in lens]
    chunks[3] = chunks[7] = 40
    _run(gpu, lens, chunks, 8, 4, 128, "bf16", seed=7300 + n_seqs)


def test_paged_prefill_longest_sequences_last(gpu):
    """Sequences in ascending order of work, so that the longest-first order
    reverses them; causal and non-causal."""
    lens = [40, 90, 200, 333, 500, 700]
    chunks = [40, 64, 100, 129, 200, 256]
    _run(gpu, lens, chunks, 8, 2, 64, "bf16", seed=7350)
    _run(gpu, lens, chunks, 8, 2, 64, "bf16", seed=7351, causal=False)


def test_paged_prefill_zero_scale_closed_form(gpu):
    """scale = 0: chunk row r of a sequence with L cached tokens and an n-token
    chunk sees keys 0 .. L - n + r, all with the same weight, so its output is
    the mean of those V rows (read through the block table here) and its LSE
    the log of their count.  Pad slots hold NaN."""
    lens, chunks, H, kvh, d = [17, 100, 300], [17, 10, 129], 8, 2, 128
    p = workloads.paged_inputs(len(lens), H, d, 16, 1, max(lens), seed=7300, seq_lens=lens,
                               kv_heads=kvh, pad_value=float("nan"))
    qq = workloads.prefill_queries(chunks, H, d, seed=7301)
    pd = {k: (v.to(gpu) if isinstance(v, torch.Tensor) else v) for k, v in p.items()}
    o, lse = binding.paged_prefill(qq["q"].to(gpu), qq["q_start"].to(gpu), pd["k_pool"],
                                   pd["v_pool"], pd["block_table"], pd["seq_lens"], block_size=16,
                                   max_q_len=max(chunks), causal=True, scale=0.0)
    torch.cuda.synchronize()
    o, lse = o.double().cpu(), lse.double().cpu()
    start = 0
    for s, (L, n) in enumerate(zip(lens, chunks)):
        t = torch.arange(L)
        v = p["v_pool"][p["block_table"][s, t // 16].long(), t % 16].double()   # [L, kvh, d]
        cum = torch.cumsum(v, 0) / torch.arange(1, L + 1, dtype=torch.float64)[:, None, None]
        last = torch.arange(L - n, L)                           # last visible key of each row
        ref = cum[last].repeat_interleave(H // kvh, dim=1)      # query head h reads h // g
        assert max_abs(o[start:start + n].numpy(), ref.numpy()) <= TOL["bf16"], s
        ref_l = np.log(last.double().numpy() + 1)[:, None].repeat(H, 1)
        assert max_abs(lse[start:start + n].numpy(), ref_l) <= 1e-3, s
        start += n


def test_paged_prefill_debug_validation(gpu, monkeypatch):
    """FA_DEBUG=1: a chunk longer than its sequence is refused before launch."""
    p = workloads.paged_inputs(2, 4, 128, 16, 1, 40, seed=7300, seq_lens=[10, 40], kv_heads=4)
    qq = workloads.prefill_queries([11, 5], 4, 128, seed=7301)
    pd = {k: (v.to(gpu) if isinstance(v, torch.Tensor) else v) for k, v in p.items()}
    monkeypatch.setenv("FA_DEBUG", "1")
    with pytest.raises(binding.LibfaError) as e:
        binding.paged_prefill(qq["q"].to(gpu), qq["q_start"].to(gpu), pd["k_pool"], pd["v_pool"],
                              pd["block_table"], pd["seq_lens"], block_size=16, max_q_len=11)
    assert e.value.status == -7


def test_paged_prefill_chunks_outside_the_packed_rows_are_skipped(gpu):
    """Offsets are trusted like a page table, but a chunk that does not lie
    inside [0, total_q) is skipped rather than read or written out of bounds:
    here the second chunk claims 195 rows from row 5 and the third starts past
    the end.  The first chunk is still computed; the other rows keep what the
    output held."""
    lens = [20, 30, 40]
    p = workloads.paged_inputs(3, 4, 128, 16, 1, 40, seed=7400, seq_lens=lens, kv_heads=2)
    qq = workloads.prefill_queries([5, 7], 4, 128, seed=7401)          # 12 packed rows
    q_start = torch.tensor([0, 5, 200, 12], dtype=torch.int32)
    pd = {k: (v.to(gpu) if isinstance(v, torch.Tensor) else v) for k, v in p.items()}
    out = torch.full((12, 4, 128), 3.0, device=gpu).to(torch.bfloat16)
    lse = torch.full((12, 4), 3.0, device=gpu)
    binding.paged_prefill(qq["q"].to(gpu), q_start.to(gpu), pd["k_pool"], pd["v_pool"],
                          pd["block_table"], pd["seq_lens"], block_size=16, max_q_len=8,
                          scale=128 ** -0.5, out=out, lse=lse)
    torch.cuda.synchronize()
    ro, rl = oracle.paged_prefill(qq["q"][:5], torch.tensor([0, 5]), p["k_pool"], p["v_pool"],
                                  p["block_table"][:1], p["seq_lens"][:1], 16, 128 ** -0.5, True)
    assert max_abs(out[:5].double().cpu().numpy(), ro) <= TOL["bf16"]
    assert max_abs(lse[:5].double().cpu().numpy(), rl) <= TOL["bf16"]
    assert bool((out[5:].float() == 3.0).all()) and bool((lse[5:] == 3.0).all())


def test_paged_prefill_length_past_the_table_is_clamped(gpu):
    """A sequence length beyond its table row (max_blocks_per_seq * 16 tokens)
    is taken as the row's capacity, as the decode takes it: the kernel reads
    at most the row's blocks.  Sequence 1 claims 2^30 tokens with a 7-block
    row; its chunk is computed over the row's 112 slots (pad slots hold finite
    draws here), sequence 0 is unaffected."""
    lens, chunks, H, kvh, d = [40, 100], [8, 10], 4, 2, 128
    p = workloads.paged_inputs(2, H, d, 16, 1, max(lens), seed=7500, seq_lens=lens, kv_heads=kvh)
    qq = workloads.prefill_queries(chunks, H, d, seed=7501)
    mb = p["block_table"].shape[1]
    assert mb * 16 == 112
    bad = p["seq_lens"].clone()
    bad[1] = 1 << 30
    pd = {k: (v.to(gpu) if isinstance(v, torch.Tensor) else v) for k, v in p.items()}
    o, lse = binding.paged_prefill(qq["q"].to(gpu), qq["q_start"].to(gpu), pd["k_pool"],
                                   pd["v_pool"], pd["block_table"], bad.to(gpu), block_size=16,
                                   max_q_len=max(chunks), scale=d ** -0.5)
    torch.cuda.synchronize()
    clamped = torch.tensor([lens[0], mb * 16], dtype=torch.int32)
    ro, rl = oracle.paged_prefill(qq["q"], qq["q_start"], p["k_pool"], p["v_pool"],
                                  p["block_table"], clamped, 16, d ** -0.5, True)
    assert max_abs(o.double().cpu().numpy(), ro) <= TOL["bf16"]
    assert max_abs(lse.double().cpu().numpy(), rl) <= TOL["bf16"]


@pytest.mark.parametrize("d", [64, 128])
def test_paged_prefill_pool_above_2gib(gpu, d):
    """Pools of at most 2 GiB are read through one buffer resource each;
    larger ones through one resource per physical block.  This case takes
    the second path: the blocks the sequences use sit at the top of a pool
    of more than 2 GiB (32 cached heads), the rest of which is never
    written.  Pad slots hold NaN."""
    lens, chunks, H, kvh = [17, 100, 300], [17, 10, 129], 32, 32
    p = workloads.paged_inputs(len(lens), H, d, 16, 1, max(lens), seed=7600 + d, seq_lens=lens,
                               kv_heads=kvh, pad_value=float("nan"))
    qq = workloads.prefill_queries(chunks, H, d, seed=7601 + d)
    n_small = p["k_pool"].shape[0]
    blk_bytes = 16 * kvh * d * 2
    n_big = (2 ** 31) // blk_bytes + 64                     # just past 2 GiB per pool
    top = n_big - 1
    big_k = torch.empty((n_big, 16, kvh, d), dtype=torch.bfloat16, device=gpu)
    big_v = torch.empty_like(big_k)
    ids = torch.arange(n_small)
    big_k[(top - ids).to(gpu)] = p["k_pool"].to(gpu)
    big_v[(top - ids).to(gpu)] = p["v_pool"].to(gpu)
    table = p["block_table"].clone()
    table = torch.where(table >= 0, top - table, table)   # block i lives at top - i
    o, lse = binding.paged_prefill(qq["q"].to(gpu), qq["q_start"].to(gpu), big_k, big_v,
                                   table.to(gpu), p["seq_lens"].to(gpu), block_size=16,
                                   max_q_len=max(chunks), scale=d ** -0.5)
    torch.cuda.synchronize()
    ro, rl = oracle.paged_prefill(qq["q"], qq["q_start"], p["k_pool"], p["v_pool"],
                                  p["block_table"], p["seq_lens"], 16, d ** -0.5, True)
    go, gl = o.double().cpu().numpy(), lse.double().cpu().numpy()
    assert np.all(np.isfinite(go)) and np.all(np.isfinite(gl))
    assert max_abs(go, ro) <= TOL["bf16"]
    assert max_abs(gl, rl) <= TOL["bf16"]
    del big_k, big_v
    torch.cuda.empty_cache()
