"""GPU parity of the ring-attention step: fa_fwd_offset (a query block against a
key/value block at global offsets) and fa_merge (the rescale rule combining
partial results), against the fp64 oracle on the same seeded inputs.

Tolerances as for fa_fwd: max-abs 2e-2 on O and LSE for bf16, 1e-5 for fp32.
Rows that see no key must come out exactly O = 0, LSE = -inf.
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

TOL = {"bf16": 2e-2, "f32": 1e-5}

# (Nq, Nk, q_offset, k_offset): equal and unequal lengths; the key block
# straddling the queries, behind them (every key visible), ahead of them
# (leading rows see nothing), entirely ahead (no row sees anything)
OFFSET_CASES = [
    (130, 200, 0, 0), (130, 200, 100, 0), (200, 130, 0, 100), (257, 64, 0, 300),
    (64, 300, 1000, 0), (1, 1, 5, 5), (129, 63, 63, 1), (300, 257, 2, 0), (65, 129, 0, 64),
    # far-apart and extreme positions: every key visible, none visible, and
    # offsets at the -2^60 limit whose difference (-30) empties the first rows
    (130, 200, 1 << 40, 0), (130, 200, 0, 1 << 40), (100, 150, -(1 << 60), -(1 << 60) + 30),
]


def _inputs(Nq, Nk, d, dtype, seed, B=1, H=3):
    x = workloads.attention_inputs(B, H, Nq, d, dtype, seed=seed, N_k=Nk)
    return x


def _check_offset(gpu, x, qo, ko, causal, scale, tol, heads=None, rows=None):
    q, k, v = (x[n].to(gpu) for n in "qkv")
    o, lse = binding.fwd_offset(q, k, v, q_offset=qo, k_offset=ko, causal=causal, scale=scale)
    torch.cuda.synchronize()
    o, lse = o.float().cpu(), lse.cpu()
    ref = oracle.attention_forward(x["q"], x["k"], x["v"], scale, causal, heads=heads, rows=rows,
                                   q_offset=qo, k_offset=ko)
    for (b, h), (ro, rl) in ref.items():
        go, gl = o[b, h].double().numpy(), lse[b, h].double().numpy()
        if rows is not None:
            go, gl = go[rows], gl[rows]
        empty = rl == -np.inf
        assert np.all(gl[empty] == -np.inf), "rows with no visible key must have LSE = -inf"
        assert np.all(go[empty] == 0.0), "rows with no visible key must have O = 0"
        assert np.all(np.isfinite(gl[~empty])) and np.all(np.isfinite(go))
        if (~empty).any():
            assert max_abs(go[~empty], ro[~empty]) <= tol
            assert max_abs(gl[~empty], rl[~empty]) <= tol
    return o, lse


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("case", OFFSET_CASES)
def test_fwd_offset_causal(gpu, dtype, d, case):
    Nq, Nk, qo, ko = case
    x = _inputs(Nq, Nk, d, dtype, seed=3000 + Nq + 7 * Nk + d)
    _check_offset(gpu, x, qo, ko, True, 1.0 / math.sqrt(d), TOL[dtype])


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_fwd_offset_noncausal_ignores_offsets(gpu, dtype):
    x = _inputs(100, 170, 128, dtype, seed=3100)
    _check_offset(gpu, x, -50, 400, False, 0.09, TOL[dtype])


def test_fwd_offset_equal_offsets_match_fwd(gpu):
    """Equal offsets and lengths: identical to fa_fwd, bit for bit."""
    x = _inputs(333, 333, 128, "bf16", seed=3200, B=2, H=2)
    q, k, v = (x[n].to(gpu) for n in "qkv")
    o1, l1 = binding.fwd(q, k, v, causal=True)
    o2, l2 = binding.fwd_offset(q, k, v, q_offset=777, k_offset=777, causal=True)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


def _partials(gpu, dtype, B=2, H=3, N=150, d=128, seed=3300):
    """Two realistic partials: one query block against two key blocks, with
    offsets chosen so some rows see nothing in one block and some in both."""
    x = workloads.attention_inputs(B, H, N, d, dtype, seed=seed, N_k=2 * N)
    q, k, v = (x[n].to(gpu) for n in "qkv")
    ka, va, kb, vb = k[:, :, :N].contiguous(), v[:, :, :N].contiguous(), \
        k[:, :, N:].contiguous(), v[:, :, N:].contiguous()
    qo = N + 40          # block a (keys 0..N-1) fully visible; block b partly
    oa, la = binding.fwd_offset(q, ka, va, q_offset=qo, k_offset=0, causal=True)
    ob, lb = binding.fwd_offset(q, kb, vb, q_offset=qo, k_offset=N, causal=True)
    # and a row range that sees nothing in either: mark by hand
    la[:, :, :3] = -math.inf
    oa[:, :, :3] = 0
    lb[:, :, :5] = -math.inf
    ob[:, :, :5] = 0
    torch.cuda.synchronize()
    return x, qo, (oa, la, ob, lb)


@pytest.mark.parametrize("dtype", ["bf16", "f16", "f32"])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("inplace", [False, True])
def test_merge_matches_oracle(gpu, dtype, d, inplace):
    _, _, (oa, la, ob, lb) = _partials(gpu, dtype, d=d)
    ref_o, ref_l = oracle.merge_partials(oracle.to_f64(oa), oracle.to_f64(la),
                                         oracle.to_f64(ob), oracle.to_f64(lb))
    if inplace:
        o, l = binding.merge(oa, la, ob, lb, out=oa, lse_out=la)
        assert o.data_ptr() == oa.data_ptr() and l.data_ptr() == la.data_ptr()
    else:
        o, l = binding.merge(oa, la, ob, lb)
    torch.cuda.synchronize()
    go, gl = o.double().cpu().numpy(), l.double().cpu().numpy()
    empty = ref_l == -np.inf
    assert empty.sum() > 0 and np.all(gl[empty] == -np.inf) and np.all(go[empty] == 0)
    tol = {"bf16": 1e-2, "f16": 1e-2, "f32": 1e-5}[dtype]
    assert max_abs(go[~empty], ref_o[~empty]) <= tol
    assert max_abs(gl[~empty], ref_l[~empty]) <= 1e-5


@pytest.mark.parametrize("d", [64, 128])
def test_ring_of_two_ranks_equals_full_causal(gpu, d):
    """Two ranks, each with a 512-row query block, meet the key/value blocks in
    ring order and merge: the result equals causal attention over the whole
    1024-token sequence (fa_fwd and the oracle)."""
    n, H = 512, 4
    x = workloads.attention_inputs(1, H, 2 * n, d, "bf16", seed=3400 + d)
    q, k, v = (x[t].to(gpu) for t in "qkv")
    full_o, full_l = binding.fwd(q, k, v, causal=True)
    outs = []
    for r in range(2):
        qr = q[:, :, r * n:(r + 1) * n].contiguous()
        acc_o = acc_l = None
        for step in range(2):
            src = (r - step) % 2            # the block this rank holds at this step
            kb = k[:, :, src * n:(src + 1) * n].contiguous()
            vb = v[:, :, src * n:(src + 1) * n].contiguous()
            po, pl = binding.fwd_offset(qr, kb, vb, q_offset=r * n, k_offset=src * n, causal=True)
            if acc_o is None:
                acc_o, acc_l = po, pl
            else:
                binding.merge(acc_o, acc_l, po, pl, out=acc_o, lse_out=acc_l)
        outs.append((acc_o, acc_l))
    torch.cuda.synchronize()
    ring_o = torch.cat([o for o, _ in outs], dim=2).float().cpu()
    ring_l = torch.cat([l for _, l in outs], dim=2).cpu()
    # same as the one-shot kernel up to bf16 rounding: the partial outputs are
    # stored in bf16, and each denominator sums bf16-rounded weights (relative
    # error <= 2^-9 per term) against a different reference maximum, so the two
    # LSEs may differ by up to ln(1 + 2^-8) ~ 4e-3
    assert (ring_o - full_o.float().cpu()).abs().max().item() <= 2e-2
    assert (ring_l - full_l.cpu()).abs().max().item() <= 4e-3
    ref = oracle.attention_forward(x["q"], x["k"], x["v"], 1.0 / math.sqrt(d), True, heads=[(0, 1)])
    ro, rl = ref[(0, 1)]
    assert max_abs(ring_o[0, 1].double().numpy(), ro) <= 2e-2
    assert max_abs(ring_l[0, 1].double().numpy(), rl) <= 2e-2


def test_ring_step_long_context_block(gpu):
    """One rank's non-diagonal step at the long-context shape: 32 heads x 8192
    queries against the 8192-token key/value block just before them (every key
    visible).  Every head and row against the oracle."""
    c = workloads.LONG_CONTEXT
    x = workloads.attention_inputs(c.B, c.H, c.N, c.d, c.dtype, seed=workloads.LONG_CONTEXT.seed + 1)
    _check_offset(gpu, x, c.N, 0, True, c.scale, TOL["bf16"])


@pytest.mark.parametrize("Nq,Nk,qo,ko", [(4100, 4100, 1000, 0), (4100, 4096, 0, 1000)])
def test_fwd_offset_256_row_workgroups(gpu, Nq, Nk, qo, ko):
    """Offset blocks long enough for 256-row workgroups with paired tiles: the
    diagonal moved 1000 keys back (every row sees keys before it), and 1000
    keys ahead (the first 1000 rows see nothing; whole tiles are empty)."""
    x = _inputs(Nq, Nk, 128, "bf16", seed=3600 + qo, H=32)
    rows = np.unique(np.r_[0:3, 254:258, 998:1003, 2047:2050, 4095:Nq])
    _check_offset(gpu, x, qo, ko, True, 128 ** -0.5, TOL["bf16"], heads=[(0, 0), (0, 31)],
                  rows=rows)


def test_fwd_offset_paired_d64_long_keys(gpu):
    """d = 64 queries over more than 4096 keys with many heads: 128-row
    workgroups with paired causal tiles (the one-stage kernel stops at 4096
    keys); every row sees the 4000 keys before its own block."""
    x = _inputs(1100, 5000, 64, "bf16", seed=3700, B=8, H=32)
    rows = np.unique(np.r_[0:3, 127:130, 549:552, 1023:1026, 1097:1100])
    _check_offset(gpu, x, 3900, 0, True, 64 ** -0.5, TOL["bf16"], heads=[(0, 0), (7, 31), (3, 17)],
                  rows=rows)


# ---------------------------------------------------------------- fused step
# fa_fwd_offset_accumulate: the forward of one key/value block merged at once
# into a running result.  A contiguous key block split in two (A, then B at
# k_offset + n1) must give attention over the whole block, the rows that see
# no key of either half coming out O = 0, LSE = -inf.
ACC_CASES = [c for c in OFFSET_CASES if c[1] >= 2]


@pytest.mark.parametrize("dtype", ["bf16", "f16", "f32"])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("case", ACC_CASES)
def test_fwd_offset_accumulate_two_halves(gpu, dtype, d, case):
    Nq, Nk, qo, ko = case
    x = _inputs(Nq, Nk, d, dtype, seed=3700 + Nq + 7 * Nk + d)
    q, k, v = (x[n].to(gpu) for n in "qkv")
    n1 = max(1, Nk // 3)
    ka, va = k[:, :, :n1].contiguous(), v[:, :, :n1].contiguous()
    kb, vb = k[:, :, n1:].contiguous(), v[:, :, n1:].contiguous()
    scale = 1.0 / math.sqrt(d)
    o, lse = binding.fwd_offset(q, ka, va, q_offset=qo, k_offset=ko, causal=True, scale=scale)
    binding.fwd_offset_accumulate(q, kb, vb, o, lse, q_offset=qo, k_offset=ko + n1, causal=True,
                                  scale=scale)
    torch.cuda.synchronize()
    ref = oracle.attention_forward(x["q"], x["k"], x["v"], scale, True, q_offset=qo, k_offset=ko)
    tol = {"bf16": 2e-2, "f16": 2e-2, "f32": 1e-5}[dtype]
    for (b, h), (ro, rl) in ref.items():
        go, gl = o[b, h].double().cpu().numpy(), lse[b, h].double().cpu().numpy()
        empty = rl == -np.inf
        assert np.all(gl[empty] == -np.inf) and np.all(go[empty] == 0.0)
        assert np.all(np.isfinite(gl[~empty])) and np.all(np.isfinite(go))
        if (~empty).any():
            assert max_abs(go[~empty], ro[~empty]) <= tol
            assert max_abs(gl[~empty], rl[~empty]) <= tol


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_fwd_offset_accumulate_weightless_sides(gpu, dtype):
    """A running row at LSE = -inf is not read into the result (its O may hold
    NaN): it comes out bit-identical to fa_fwd_offset of the block alone.  A
    row that sees no key of the block keeps its running O and LSE bit for bit."""
    Nq, Nk, d = 200, 300, 128
    x = _inputs(Nq, Nk, d, dtype, seed=3800)
    q, k, v = (x[n].to(gpu) for n in "qkv")
    qo, ko = 100, 150            # key j visible to row i iff j <= i - 50: rows 0..49 see none
    o_blk, l_blk = binding.fwd_offset(q, k, v, q_offset=qo, k_offset=ko, causal=True)
    run_o = torch.randn(q.shape, device=gpu).to(q.dtype)
    run_l = torch.randn(l_blk.shape, device=gpu)
    run_o[:, :, 60:90] = float("nan")
    run_l[:, :, 60:90] = -math.inf
    o, l = run_o.clone(), run_l.clone()
    binding.fwd_offset_accumulate(q, k, v, o, l, q_offset=qo, k_offset=ko, causal=True)
    torch.cuda.synchronize()
    assert torch.equal(o[:, :, 60:90], o_blk[:, :, 60:90])
    assert torch.equal(l[:, :, 60:90], l_blk[:, :, 60:90])
    assert torch.equal(o[:, :, :50], run_o[:, :, :50]) and torch.equal(l[:, :, :50], run_l[:, :, :50])
    assert bool(torch.isfinite(o).all()) and bool(torch.isfinite(l).all())
    # everything else is the merge of the two
    ref_o, ref_l = oracle.merge_partials(oracle.to_f64(run_o[:, :, 90:]), oracle.to_f64(run_l[:, :, 90:]),
                                         oracle.to_f64(o_blk[:, :, 90:]), oracle.to_f64(l_blk[:, :, 90:]))
    tol = 2e-2 if dtype == "bf16" else 1e-5
    assert max_abs(o[:, :, 90:].double().cpu().numpy(), ref_o) <= tol
    assert max_abs(l[:, :, 90:].double().cpu().numpy(), ref_l) <= 1e-5


def test_fwd_offset_accumulate_empty_block_is_a_no_op(gpu):
    """A key block wholly ahead of every query leaves the running result as it was."""
    x = _inputs(130, 200, 128, "bf16", seed=3900)
    q, k, v = (x[n].to(gpu) for n in "qkv")
    run_o = torch.randn(q.shape, device=gpu).to(q.dtype)
    run_l = torch.randn(q.shape[:3], device=gpu)
    o, l = run_o.clone(), run_l.clone()
    binding.fwd_offset_accumulate(q, k, v, o, l, q_offset=0, k_offset=1 << 40, causal=True)
    torch.cuda.synchronize()
    assert torch.equal(o, run_o) and torch.equal(l, run_l)


@pytest.mark.parametrize("d", [64, 128])
def test_ring_of_four_ranks_fused_steps(gpu, d):
    """Four ranks of 256 queries each meet the key/value blocks in ring order,
    fa_fwd for the diagonal block then fa_fwd_offset_accumulate for each later
    one: the result equals causal attention over the 1024-token sequence."""
    n, R, H = 256, 4, 3
    x = workloads.attention_inputs(1, H, R * n, d, "bf16", seed=4000 + d)
    q, k, v = (x[t].to(gpu) for t in "qkv")
    outs = []
    for r in range(R):
        qr = q[:, :, r * n:(r + 1) * n].contiguous()
        kr, vr = k[:, :, r * n:(r + 1) * n].contiguous(), v[:, :, r * n:(r + 1) * n].contiguous()
        acc_o, acc_l = binding.fwd(qr, kr, vr, causal=True)
        for step in range(1, R):
            src = (r - step) % R
            kb = k[:, :, src * n:(src + 1) * n].contiguous()
            vb = v[:, :, src * n:(src + 1) * n].contiguous()
            binding.fwd_offset_accumulate(qr, kb, vb, acc_o, acc_l, q_offset=r * n,
                                          k_offset=src * n, causal=True)
        outs.append((acc_o, acc_l))
    torch.cuda.synchronize()
    ring_o = torch.cat([o for o, _ in outs], dim=2).float().cpu()
    ring_l = torch.cat([l for _, l in outs], dim=2).cpu()
    ref = oracle.attention_forward(x["q"], x["k"], x["v"], 1.0 / math.sqrt(d), True)
    for (b, h), (ro, rl) in ref.items():
        assert max_abs(ring_o[b, h].double().numpy(), ro) <= 2e-2
        assert max_abs(ring_l[b, h].double().numpy(), rl) <= 2e-2


def test_ring_step_long_context_fused(gpu):
    """The long-context ring step (32 heads x 8192 queries against the 8192
    keys just before them) accumulated into the diagonal block's result:
    every head and row against the oracle over all 16384 keys."""
    c = workloads.LONG_CONTEXT
    x = workloads.attention_inputs(c.B, c.H, 2 * c.N, c.d, c.dtype, seed=c.seed + 2)
    q, k, v = (x[t].to(gpu) for t in "qkv")
    q2 = q[:, :, c.N:].contiguous()
    k1, v1 = k[:, :, :c.N].contiguous(), v[:, :, :c.N].contiguous()
    k2, v2 = k[:, :, c.N:].contiguous(), v[:, :, c.N:].contiguous()
    o, l = binding.fwd(q2, k2, v2, causal=True, scale=c.scale)
    binding.fwd_offset_accumulate(q2, k1, v1, o, l, q_offset=c.N, k_offset=0, causal=True,
                                  scale=c.scale)
    torch.cuda.synchronize()
    ref = oracle.attention_forward(x["q"], x["k"], x["v"], c.scale, True,
                                   rows=np.arange(c.N, 2 * c.N))
    o, l = o.double().cpu().numpy(), l.double().cpu().numpy()
    for (b, h), (ro, rl) in ref.items():
        assert max_abs(o[b, h], ro) <= 2e-2
        assert max_abs(l[b, h], rl) <= 2e-2


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("Nq,Nk,qo,ko", [(4100, 4100, 1000, 0), (4100, 4096, 0, 1000)])
def test_fwd_offset_accumulate_256_row_workgroups(gpu, Nq, Nk, qo, ko, d):
    """The fused step on the paired 256-row causal kernel (at d = 64 its
    one-stage form, four waves per SIMD): the key block split in two halves,
    the second accumulated into the first's result, against the oracle over
    the whole block on sampled heads and rows."""
    x = _inputs(Nq, Nk, d, "bf16", seed=4100 + qo + d, H=32)
    q, k, v = (x[n].to(gpu) for n in "qkv")
    n1 = Nk // 2
    scale = d ** -0.5
    o, lse = binding.fwd_offset(q, k[:, :, :n1].contiguous(), v[:, :, :n1].contiguous(),
                                q_offset=qo, k_offset=ko, causal=True, scale=scale)
    binding.fwd_offset_accumulate(q, k[:, :, n1:].contiguous(), v[:, :, n1:].contiguous(), o, lse,
                                  q_offset=qo, k_offset=ko + n1, causal=True, scale=scale)
    torch.cuda.synchronize()
    rows = np.unique(np.r_[0:3, 254:258, 998:1003, 2047:2052, 3095:3100, 4095:Nq])
    ref = oracle.attention_forward(x["q"], x["k"], x["v"], scale, True, heads=[(0, 0), (0, 31)],
                                   rows=rows, q_offset=qo, k_offset=ko)
    for (b, h), (ro, rl) in ref.items():
        go, gl = o[b, h].double().cpu().numpy()[rows], lse[b, h].double().cpu().numpy()[rows]
        empty = rl == -np.inf
        assert np.all(gl[empty] == -np.inf) and np.all(go[empty] == 0.0)
        if (~empty).any():
            assert max_abs(go[~empty], ro[~empty]) <= 2e-2
            assert max_abs(gl[~empty], rl[~empty]) <= 2e-2
