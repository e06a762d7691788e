"""GPU forward parity: fa_fwd against the fp64 oracle on the same seeded inputs.

Tolerances (max-abs): O <= 2e-2 for bf16 inputs, <= 1e-5 for fp32 inputs; the
same bound is used for LSE.  Sizes span several tiles with ragged tails; the
full-size workloads (small fp32, GPT-2-shaped, long-context) are checked on
every head and row; the longest sequence the library accepts and the other
launch variants are checked on sampled heads and rows.
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


def _gpu_fwd(gpu, x, causal, scale):
    q, k, v = (x[n].to(gpu) for n in "qkv")
    o, lse = binding.fwd(q, k, v, causal=causal, scale=scale)
    torch.cuda.synchronize()
    return o.float().cpu(), lse.cpu()


def _check(x, o, lse, causal, scale, tol, heads=None, rows=None):
    ref = oracle.attention_forward(x["q"], x["k"], x["v"], scale, causal, heads=heads, rows=rows)
    worst_o = worst_l = 0.0
    for (b, h), (ro, rl) in ref.items():
        go = o[b, h].double().numpy()
        gl = lse[b, h].double().numpy()
        if rows is not None:
            go, gl = go[rows], gl[rows]
        assert np.all(np.isfinite(go)) and np.all(np.isfinite(gl))
        worst_o = max(worst_o, max_abs(go, ro))
        worst_l = max(worst_l, max_abs(gl, rl))
    assert worst_o <= tol, f"O max-abs {worst_o}"
    assert worst_l <= tol, f"LSE max-abs {worst_l}"
    return worst_o, worst_l


SMALL_N = [1, 2, 3, 17, 63, 64, 65, 127, 128, 129, 255, 300]


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("N", SMALL_N)
def test_fwd_small_shapes(gpu, dtype, d, causal, N):
    x = workloads.attention_inputs(2, 3, N, d, dtype, seed=1000 + N + d + causal)
    scale = 1.0 / math.sqrt(d)
    o, lse = _gpu_fwd(gpu, x, causal, scale)
    _check(x, o, lse, causal, scale, TOL[dtype])


def test_fwd_fp32_b1h2n256d64_noncausal(gpu):
    c = workloads.FP32_SMALL
    x = workloads.attention_inputs(c.B, c.H, c.N, c.d, c.dtype, seed=workloads.FP32_SMALL.seed)
    o, lse = _gpu_fwd(gpu, x, c.causal, c.scale)
    _check(x, o, lse, c.causal, c.scale, TOL["f32"])


def test_fwd_gpt2_shape_b8h12n1024d64_causal(gpu):
    c = workloads.GPT2_SHAPE
    x = workloads.attention_inputs(c.B, c.H, c.N, c.d, c.dtype, seed=workloads.GPT2_SHAPE.seed,
                                   in_scale=c.in_scale)
    o, lse = _gpu_fwd(gpu, x, c.causal, c.scale)
    _check(x, o, lse, c.causal, c.scale, TOL["bf16"])


def test_fwd_gpt2_shape_unscaled_inputs_stress(gpu):
    """Same shape without the 1/sqrt(d) input scaling: peakier softmax rows."""
    c = workloads.GPT2_SHAPE
    x = workloads.attention_inputs(c.B, c.H, c.N, c.d, c.dtype, seed=workloads.GPT2_SHAPE.seed + 50)
    o, lse = _gpu_fwd(gpu, x, c.causal, c.scale)
    _check(x, o, lse, c.causal, c.scale, TOL["bf16"], heads=[(b, h) for b in (0, 7) for h in range(12)])


def test_fwd_long_context_b1h32n8192d128_whole(gpu):
    """The benchmarked long-context launch (256-row paired workgroups), every
    head and every row against the oracle."""
    c = workloads.LONG_CONTEXT
    x = workloads.attention_inputs(c.B, c.H, c.N, c.d, c.dtype, seed=workloads.LONG_CONTEXT.seed)
    o, lse = _gpu_fwd(gpu, x, c.causal, c.scale)
    worst_o, worst_l = _check(x, o, lse, c.causal, c.scale, TOL["bf16"])
    print(f"long context B1 H32 N8192 d128: O max-abs {worst_o:.3e}, LSE max-abs {worst_l:.3e}")


def test_fwd_maximum_length_sampled(gpu):
    """The longest sequence the library accepts (N = 2^20, one head, d = 128),
    where the 32-bit buffer offsets reach 256 MiB per head: rows at tile edges,
    the middle, the last rows and random rows against the oracle."""
    N = 1 << 20
    x = workloads.attention_inputs(1, 1, N, 128, "bf16", seed=71000)
    o, lse = _gpu_fwd(gpu, x, True, 128 ** -0.5)
    rng = np.random.default_rng(5)
    rows = np.unique(np.concatenate([[0, 1, 127, 128, N // 2, N - 129, N - 128, N - 2, N - 1],
                                     rng.integers(0, N, 7)]))
    _check(x, o, lse, True, 128 ** -0.5, TOL["bf16"], rows=rows)


# Long sequences with enough heads run in 256-row workgroups (causal ones with
# a long and a short query tile per workgroup).  4096 rows is a whole number of
# such tiles; 4100 leaves a ragged 4-row tile and an odd tile count, so one
# workgroup runs the middle tile alone.
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [True, False])
@pytest.mark.parametrize("N", [4096, 4100])
def test_fwd_256_row_workgroups_sampled(gpu, d, causal, N):
    H = 32 if causal else 16
    x = workloads.attention_inputs(1, H, N, d, "bf16", seed=72000 + N + d + causal)
    scale = d ** -0.5
    o, lse = _gpu_fwd(gpu, x, causal, scale)
    _check(x, o, lse, causal, scale, TOL["bf16"], heads=[(0, H - 1)])
    rng = np.random.default_rng(N + d)
    rows = np.unique(np.concatenate([[0, 1, 127, 128, 255, 256, 257, 2047, 2048, 2049, 3839,
                                      3840, 4095], np.arange(4096, N), rng.integers(0, N, 20)]))
    _check(x, o, lse, causal, scale, TOL["bf16"], rows=rows)


# Shorter sequences with many heads run in 128-row workgroups with paired
# causal tiles, once the paired grid still leaves four workgroups per compute
# unit (heads x ceil(query tiles / 2) >= 1024); at d = 64 only above 4096 keys
# (shorter rows take the unpaired one-stage kernel, as the next test checks;
# the paired d = 64 kernel is covered by an offset block in the ring tests).
# 1900 rows leave a ragged tile and an odd tile count (one workgroup runs the
# middle tile alone); one case takes a negative scale.
@pytest.mark.parametrize("B,H,N,d,sign", [(8, 16, 2048, 128, 1), (8, 16, 1900, 128, -1)])
def test_fwd_paired_128_row_workgroups_sampled(gpu, B, H, N, d, sign):
    x = workloads.attention_inputs(B, H, N, d, "bf16", seed=73000 + N + d)
    scale = sign * d ** -0.5
    o, lse = _gpu_fwd(gpu, x, True, scale)
    _check(x, o, lse, True, scale, TOL["bf16"], heads=[(0, 0), (B - 1, H - 1)])
    rng = np.random.default_rng(N + d)
    rows = np.unique(np.concatenate([[0, 1, 127, 128, 129, N // 2, N - 1],
                                     rng.integers(0, N, 20)]))
    _check(x, o, lse, True, scale, TOL["bf16"], rows=rows)


# d = 64 rows of at most 4096 keys: the unpaired one-stage kernel at three
# workgroups per compute unit, also where 128-row tiles would pair; 768
# workgroups (a whole grid resident at once) take the reversed-round order.
@pytest.mark.parametrize("B,H,N,causal", [(8, 32, 1000, True), (8, 12, 1024, True),
                                          (2, 12, 1024, False), (64, 12, 128, True),
                                          (8, 32, 1100, True), (1, 16, 4000, True)])
def test_fwd_one_stage_d64_sampled(gpu, B, H, N, causal):
    d = 64
    x = workloads.attention_inputs(B, H, N, d, "bf16", seed=74000 + N + B)
    scale = d ** -0.5
    o, lse = _gpu_fwd(gpu, x, causal, scale)
    _check(x, o, lse, causal, scale, TOL["bf16"], heads=[(0, 0), (B - 1, H - 1), (B // 2, H // 2)])
    rng = np.random.default_rng(N + B)
    rows = np.unique(np.concatenate([[0, 1, 63, 64, 127, 128, N // 2, N - 1],
                                     rng.integers(0, N, 16)]))
    _check(x, o, lse, causal, scale, TOL["bf16"], rows=rows[rows < N])


def test_fwd_deterministic(gpu):
    x = workloads.attention_inputs(2, 4, 777, 128, "bf16", seed=77)
    a = _gpu_fwd(gpu, x, True, 0.0884)
    b = _gpu_fwd(gpu, x, True, 0.0884)
    assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1])


def test_fwd_closed_forms(gpu):
    """Q = 0: uniform weights (O_i = mean of V_0..V_i, LSE_i = ln(i+1)); causal row 0 = V_0."""
    x = workloads.attention_inputs(1, 2, 200, 64, "bf16", seed=88)
    x["q"] = torch.zeros_like(x["q"])
    o, lse = _gpu_fwd(gpu, x, True, 0.125)
    v = x["v"].double()
    mean = torch.cumsum(v, dim=2) / torch.arange(1, 201, dtype=torch.float64)[None, None, :, None]
    assert max_abs(o.double().numpy(), mean.numpy()) <= 2e-2
    assert max_abs(lse.double().numpy(), np.log(np.arange(1, 201))[None, None, :]) <= 1e-5
    assert torch.equal(o[:, :, 0], x["v"][:, :, 0].float())


# scale = 0 gives every visible key the same weight: causal O_i is the mean of
# V_0..V_i and LSE_i = ln(i + 1); non-causal rows all get the mean of V and
# ln(N).  On the paired 256-row launch (32 heads x 4100 rows), the 128-row
# launch with a ragged last key tile, and the fp32 forward.
@pytest.mark.parametrize("B,H,N,d,causal,dtype", [
    (1, 32, 4100, 128, True, "bf16"), (2, 3, 300, 64, True, "bf16"), (2, 3, 300, 128, False, "bf16"),
    (2, 3, 300, 128, True, "f32"), (2, 3, 300, 64, False, "f32"),
])
def test_fwd_zero_scale_closed_form(gpu, B, H, N, d, causal, dtype):
    x = workloads.attention_inputs(B, H, N, d, dtype, seed=74000 + N + d)
    o, lse = _gpu_fwd(gpu, x, causal, 0.0)
    v = x["v"].double()
    if causal:
        cnt = torch.arange(1, N + 1, dtype=torch.float64)
        mean = torch.cumsum(v, dim=2) / cnt[None, None, :, None]
    else:
        cnt = torch.full((N,), float(N), dtype=torch.float64)
        mean = v.mean(dim=2, keepdim=True).expand_as(v)
    assert max_abs(o.double().numpy(), mean.numpy()) <= (2e-2 if dtype == "bf16" else 1e-5)
    assert max_abs(lse.double().numpy(), np.log(cnt.numpy())[None, None, :]) <= 1e-3


def test_fwd_on_side_stream(gpu):
    x = workloads.attention_inputs(1, 2, 130, 128, "bf16", seed=99)
    ref = _gpu_fwd(gpu, x, True, 0.09)
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        q, k, v = (x[n].to(gpu) for n in "qkv")
        o, lse = binding.fwd(q, k, v, causal=True, scale=0.09)
    s.synchronize()
    assert torch.equal(o.float().cpu(), ref[0]) and torch.equal(lse.cpu(), ref[1])


# Scores that climb tile after tile move every row's running maximum again and
# again.  Per 64-key tile the rise in base-2 units is scale*align*ramp*log2(e):
# ~14 makes the accumulated output rescale on every tile, ~4 keeps the old
# reference with probabilities up to 2^4, and a falling ramp never moves it.
# The oracle's max-subtracted softmax is exact in all three cases.
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("rise", [14.0, 4.0, -6.0])
def test_fwd_running_max_moves(gpu, d, causal, rise):
    N, align = 520, 4.0
    scale = 1.0 / math.sqrt(d)
    ramp = rise / (scale * align * math.log2(math.e))
    x = workloads.ramp_inputs(1, 2, N, d, "bf16", seed=4242 + d, align=align, ramp=ramp)
    o, lse = _gpu_fwd(gpu, x, causal, scale)
    _check(x, o, lse, causal, scale, TOL["bf16"])


# One key far above the rest, placed in each of the four 16-key blocks of a
# 64-key tile after the first: the kernels take a tile's probabilities against
# the reference they hold, check the running probability sum before the first
# product of a key block that uses unchecked probabilities, and on a hit move
# the reference and rescale what they have accumulated, part of the current
# tile included.  A rise of 20 (base 2) gives probabilities near 2^20; 150
# overflows exp2 to inf before the move.  The oracle's max-subtracted softmax
# is exact either way.
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("key", [64 + 5, 128 + 20, 192 + 40, 256 + 60, 300 + 63])
@pytest.mark.parametrize("rise", [20.0, 150.0])
def test_fwd_reference_moves_mid_tile(gpu, d, causal, key, rise):
    N, align = 400, 4.0
    scale = 1.0 / math.sqrt(d)
    spike = rise / (scale * align * math.log2(math.e))
    x = workloads.spike_inputs(1, 2, N, d, "bf16", seed=5151 + key, align=align, spike=spike,
                               keys=[key])
    o, lse = _gpu_fwd(gpu, x, causal, scale)
    _check(x, o, lse, causal, scale, TOL["bf16"])


# Spikes in several tiles, in rising order, on the long-sequence launch
# (256-row workgroups, paired causal tiles): the reference moves several
# times per row, in both passes of a paired workgroup.  That launch needs at
# least 256 workgroups: 16 tiles of 256 rows per head, paired to 8 when causal,
# so 32 heads (causal) or 16 (non-causal).
@pytest.mark.parametrize("causal", [False, True])
def test_fwd_reference_moves_long(gpu, causal):
    B, H, N, d = 1, (32 if causal else 16), 4096, 128
    scale = 1.0 / math.sqrt(d)
    keys = [70, 1000, 2047, 2100, 4000]
    x = workloads.spike_inputs(B, H, N, d, "bf16", seed=5252, align=4.0,
                               spike=30.0 / (scale * 4.0 * math.log2(math.e)), keys=keys)
    # rising spikes: each later key scores higher than the one before
    for i, j in enumerate(keys):
        x["k"][:, :, j, :] *= 1.0 + 0.25 * i
    o, lse = _gpu_fwd(gpu, x, causal, scale)
    rows = [0, 69, 70, 71, 999, 1000, 1500, 2047, 2099, 2100, 3000, 3999, 4000, 4095]
    _check(x, o, lse, causal, scale, TOL["bf16"], rows=rows)
