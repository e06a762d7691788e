"""GPU parity with a negative softmax scale on every entry point that takes one.

The library accepts any finite scale.  A negative one turns the largest dot
products into the smallest scores, so the softmax's maximum comes from other
keys than with the usual positive scale.  Each kernel handles the sign in its
own way: the 16-bit forward negates Q once and takes |scale| (the maximum is
taken over raw scores), while the fp32 forward, the backward, the decode and
the prefill multiply by the signed scale before any maximum.

Tolerances are those of the positive-scale parity tests: O and LSE max-abs
2e-2 (bf16), 1e-5 (fp32 forward); gradients 5e-2.
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
TOL_GRAD = 5e-2


def _check_fwd(x, o, lse, causal, scale, tol, heads=None, rows=None, q_offset=0, k_offset=0):
    ref = oracle.attention_forward(x["q"], x["k"], x["v"], scale, causal, heads=heads, rows=rows,
                                   q_offset=q_offset, k_offset=k_offset)
    for (b, h), (ro, rl) in ref.items():
        go, gl = o[b, h].double().numpy(), lse[b, h].double().numpy()
        if rows is not None:
            go, gl = go[rows], gl[rows]
        assert np.all(np.isfinite(go)) and np.all(np.isfinite(gl))
        assert max_abs(go, ro) <= tol, (b, h)
        assert max_abs(gl, rl) <= tol, (b, h)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("N", [65, 300])
def test_fwd_negative_scale(gpu, dtype, d, causal, N):
    x = workloads.attention_inputs(1, 2, N, d, dtype, seed=81000 + N + d + causal)
    scale = -1.5 / math.sqrt(d)
    q, k, v = (x[n].to(gpu) for n in "qkv")
    o, lse = binding.fwd(q, k, v, causal=causal, scale=scale)
    torch.cuda.synchronize()
    _check_fwd(x, o.float().cpu(), lse.cpu(), causal, scale, TOL[dtype])


def test_fwd_negative_scale_256_row_workgroups(gpu):
    """The paired 256-row workgroups that long causal sequences launch."""
    H, N, d = 32, 4100, 128
    x = workloads.attention_inputs(1, H, N, d, "bf16", seed=81100)
    scale = -(d ** -0.5)
    q, k, v = (x[n].to(gpu) for n in "qkv")
    o, lse = binding.fwd(q, k, v, causal=True, scale=scale)
    torch.cuda.synchronize()
    rows = np.array([0, 1, 255, 256, 2047, 2048, 4095, 4096, 4099])
    _check_fwd(x, o.float().cpu(), lse.cpu(), True, scale, TOL["bf16"], heads=[(0, 7)],
               rows=rows)


def test_fwd_offset_negative_scale(gpu):
    x = workloads.attention_inputs(1, 3, 200, 128, "bf16", seed=81200, N_k=333)
    scale = -0.1
    q, k, v = (x[n].to(gpu) for n in "qkv")
    o, lse = binding.fwd_offset(q, k, v, q_offset=400, k_offset=250, causal=True, scale=scale)
    torch.cuda.synchronize()
    _check_fwd(x, o.float().cpu(), lse.cpu(), True, scale, TOL["bf16"], q_offset=400,
               k_offset=250)


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
def test_bwd_negative_scale(gpu, d, causal):
    x = workloads.attention_inputs(1, 2, 200, d, "bf16", seed=81300 + d + causal, with_do=True)
    scale = -1.0 / math.sqrt(d)
    q, k, v, do = (x[n].to(gpu) for n in ("q", "k", "v", "do"))
    o, lse = binding.fwd(q, k, v, causal=causal, scale=scale)
    dq, dk, dv = binding.bwd(q, k, v, o, do, lse, causal=causal, scale=scale)
    torch.cuda.synchronize()
    ref = oracle.attention_backward(x["q"], x["k"], x["v"], x["do"], scale, causal)
    got = {"dq": dq.cpu(), "dk": dk.cpu(), "dv": dv.cpu()}
    for (b, h), r in ref.items():
        for name in ("dq", "dk", "dv"):
            g = got[name][b, h].double().numpy()
            assert np.all(np.isfinite(g)), name
            assert max_abs(g, r[name]) <= TOL_GRAD, (name, b, h)


@pytest.mark.parametrize("kvh", [32, 8])
def test_paged_decode_negative_scale(gpu, kvh):
    """Multi-head (32 cached heads) and grouped-query (8) decode; pad slots NaN."""
    lens = [1, 16, 17, 300, 1000, 2049]
    p = workloads.paged_inputs(len(lens), 32, 128, 16, 1, max(lens), seed=81400 + kvh,
                               seq_lens=lens, kv_heads=kvh, pad_value=float("nan"))
    scale = -(128 ** -0.5)
    pd = {k: (v.to(gpu) if isinstance(v, torch.Tensor) else v) for k, v in p.items()}
    o, lse = binding.paged_decode(pd["q"], pd["k_pool"], pd["v_pool"], pd["block_table"],
                                  pd["seq_lens"], block_size=16, scale=scale)
    torch.cuda.synchronize()
    ro, rl = oracle.paged_decode(p["q"], p["k_pool"], p["v_pool"], p["block_table"], p["seq_lens"],
                                 16, scale)
    go, gl = o.double().cpu().numpy(), lse.double().cpu().numpy()
    assert np.all(np.isfinite(go)) and np.all(np.isfinite(gl))
    assert max_abs(go, ro) <= TOL["bf16"] and max_abs(gl, rl) <= TOL["bf16"]


def test_paged_prefill_negative_scale(gpu):
    lens, chunks = [17, 100, 300], [17, 10, 129]
    p = workloads.paged_inputs(len(lens), 8, 128, 16, 1, max(lens), seed=81500, seq_lens=lens,
                               kv_heads=2, pad_value=float("nan"))
    qq = workloads.prefill_queries(chunks, 8, 128, seed=81501)
    scale = -(128 ** -0.5)
    pd = {k: (v.to(gpu) if isinstance(v, torch.Tensor) else v) for k, v in p.items()}
    o, lse = binding.paged_prefill(qq["q"].to(gpu), qq["q_start"].to(gpu), pd["k_pool"],
                                   pd["v_pool"], pd["block_table"], pd["seq_lens"], block_size=16,
                                   max_q_len=max(chunks), causal=True, scale=scale)
    torch.cuda.synchronize()
    ro, rl = oracle.paged_prefill(qq["q"], qq["q_start"], p["k_pool"], p["v_pool"],
                                  p["block_table"], p["seq_lens"], 16, scale, True)
    go, gl = o.double().cpu().numpy(), lse.double().cpu().numpy()
    assert np.all(np.isfinite(go)) and np.all(np.isfinite(gl))
    assert max_abs(go, ro) <= TOL["bf16"] and max_abs(gl, rl) <= TOL["bf16"]
