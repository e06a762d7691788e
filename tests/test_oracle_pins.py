"""Pins of the fp64 oracle to facts outside itself (CPU only).

Each check ties the oracle to something the pages print, a closed form, an
invariant of the mathematics, or a 50-digit brute force of the literal
definition.  The planted-mistake tests at the end swap one step of the oracle
for a plausible wrong version (dropped term, wrong sign, wrong index,
transposed operand) and show that the pin suite then fails.
"""
import json
import math
import os

import numpy as np
import pytest
import scipy.special
import torch

import oracle
from oracle import attention as A
from oracle import brute
import workloads

RNG = np.random.default_rng(12345)


def _golden(golden_dir, name):
    with open(os.path.join(golden_dir, name)) as f:
        return json.load(f)


# ----------------------------------------------------------- printed examples

def check_worked_example(gold):
    s = np.array(gold["scores_reading"])
    _, traj = A.online_softmax(s, gold["block_size"])
    pr, tol = gold["printed"], gold["printed_tolerance"]
    assert abs(traj[0]["l"] - pr["block1_denominator"]) <= tol
    assert traj[1]["m"] == pr["running_max_after_block2"]
    assert abs(traj[1]["l"] - pr["denominator_after_block2"]) <= tol
    assert traj[2]["m"] == pr["running_max_after_block3"]
    assert abs(traj[2]["alpha"] - math.exp(pr["rescale_factor_exponent_at_block3"])) <= 1e-15
    assert abs(traj[2]["l"] - pr["final_denominator"]) <= tol


def test_worked_example_trajectory(golden_dir):
    check_worked_example(_golden(golden_dir, "online_softmax_worked_example.json"))


def test_worked_example_online_equals_one_shot(golden_dir):
    gold = _golden(golden_dir, "online_softmax_worked_example.json")
    s = np.array(gold["scores_reading"])
    vals = RNG.standard_normal((6, 5))
    online, _ = A.online_softmax(s, 2, vals)
    p, _, _ = A.safe_softmax(s[None, :])
    np.testing.assert_allclose(online, p[0] @ vals, rtol=0, atol=1e-12)
    w, _ = A.online_softmax(s, 2)
    exact = [float(x) for x in brute.softmax_decimal(s)]
    np.testing.assert_allclose(w, exact, rtol=0, atol=1e-14)


def test_appendix_safe_softmax(golden_dir):
    gold = _golden(golden_dir, "safe_softmax_appendix.json")
    s = np.array(gold["scores"])
    assert abs(math.exp(12.0) - gold["printed_exp12"]) <= gold["printed_exp12_tolerance"]
    # the direct form overflows in fp16, the max-subtracted form does not
    with np.errstate(over="ignore"):
        e12_16 = np.float16(np.exp(np.float32(12.0)))
    assert np.isinf(e12_16) and np.float16(gold["printed_fp16_max"]) == np.finfo(np.float16).max
    sub16 = np.exp((s - s.max()).astype(np.float16))
    assert np.all(np.isfinite(sub16))
    p, m, l = A.safe_softmax(s[None, :])
    exact = [float(x) for x in brute.softmax_decimal(s)]
    np.testing.assert_allclose(p[0], exact, rtol=0, atol=1e-15)
    assert m[0] == 12.0


def test_numpy_exercise_three_chunks_vs_scipy():
    """CMU notes, self-study section: online softmax over a long vector in three chunks vs scipy."""
    x = RNG.standard_normal(3001) * 6.0
    w, traj = A.online_softmax(x, 1001)
    assert len(traj) == 3
    np.testing.assert_allclose(w, scipy.special.softmax(x), rtol=1e-12, atol=1e-300)


def test_online_equals_one_shot_every_block_size():
    for n in (1, 2, 7, 16):
        x = RNG.standard_normal(n) * 4.0
        vals = RNG.standard_normal((n, 3))
        p, _, _ = A.safe_softmax(x[None, :])
        for b in range(1, n + 1):
            res, traj = A.online_softmax(x, b, vals)
            np.testing.assert_allclose(res, p[0] @ vals, rtol=0, atol=1e-13)
            assert traj[-1]["m"] == x.max()


def test_blockwise_softmaxes_cannot_simply_be_added():
    """HPC notes, long-context section: per-block softmaxes do not sum to the global one."""
    x = np.array([1.0, 2.0, 5.0, 0.5])
    naive = np.concatenate([A.safe_softmax(x[None, :2])[0][0], A.safe_softmax(x[None, 2:])[0][0]])
    p, _, _ = A.safe_softmax(x[None, :])
    assert np.max(np.abs(naive - p[0])) > 0.1
    w, _ = A.online_softmax(x, 2)
    np.testing.assert_allclose(w, p[0], atol=1e-15)


# ------------------------------------------------------- forward: brute force

def check_forward_vs_decimal(seed=0):
    rng = np.random.default_rng(seed)
    for (n, d, causal) in ((1, 1, False), (3, 2, True), (5, 3, False), (6, 3, True), (4, 2, False)):
        q, k, v = (rng.standard_normal((n, d)) * 1.5 for _ in range(3))
        v = rng.standard_normal((n, d + 1))
        scale = 1.0 / math.sqrt(d)
        o, lse = A.attention_forward_head(q, k, v, scale, causal)
        Od, Ld = brute.attention_decimal(q, k, v, scale, causal)
        np.testing.assert_allclose(o, np.array(Od, dtype=float), rtol=0, atol=1e-13)
        np.testing.assert_allclose(lse, np.array(Ld, dtype=float), rtol=0, atol=1e-13)


def test_forward_vs_decimal_brute_force():
    check_forward_vs_decimal()


def check_forward_large_scores():
    """Scores far beyond exp's float64 range: max subtraction keeps the result exact."""
    q = np.array([[30.0, 0.0], [0.0, 30.0]])
    k = np.array([[30.0, 0.0], [0.0, 29.0]])
    v = np.array([[1.0, 2.0], [3.0, 4.0]])
    o, lse = A.attention_forward_head(q, k, v, 1.0, False)
    # row 0: scores (900, 0) -> weight 1 on key 0; row 1: scores (0, 870) -> key 1
    np.testing.assert_allclose(o, [[1.0, 2.0], [3.0, 4.0]], atol=1e-300)
    np.testing.assert_allclose(lse, [900.0, 870.0], rtol=1e-15)


def test_forward_large_scores_stay_finite():
    check_forward_large_scores()


# ----------------------------------------------------------- forward invariants

def check_forward_invariants(seed=1):
    rng = np.random.default_rng(seed)
    n, d = 37, 8
    scale = 1.0 / math.sqrt(d)
    q, k, v = (rng.standard_normal((n, d)) for _ in range(3))
    for causal in (False, True):
        rows = np.arange(n)
        s = np.where(A.visible(rows, n, causal), A.scores(q, k, scale), -np.inf)
        p, m, l = A.safe_softmax(s)
        np.testing.assert_allclose(p.sum(axis=1), 1.0, rtol=0, atol=1e-14)
        o, lse = A.attention_forward_head(q, k, v, scale, causal)
        for i in range(n):
            vis = np.arange(n) <= i if causal else np.ones(n, bool)
            lo, hi = v[vis].min(axis=0), v[vis].max(axis=0)
            assert np.all(o[i] >= lo - 1e-13) and np.all(o[i] <= hi + 1e-13)
            si = scale * q[i] @ k[vis].T
            assert lse[i] >= si.max() - 1e-13
            assert lse[i] <= si.max() + math.log(vis.sum()) + 1e-13
    # key permutation invariance (non-causal): permute K and V rows together
    perm = rng.permutation(n)
    o1, l1 = A.attention_forward_head(q, k, v, scale, False)
    o2, l2 = A.attention_forward_head(q, k[perm], v[perm], scale, False)
    np.testing.assert_allclose(o1, o2, atol=1e-13)
    np.testing.assert_allclose(l1, l2, atol=1e-13)
    # Q = 0: uniform weights over visible keys
    z = np.zeros_like(q)
    oc, lc = A.attention_forward_head(z, k, v, scale, True)
    np.testing.assert_allclose(oc, np.cumsum(v, axis=0) / np.arange(1, n + 1)[:, None], atol=1e-13)
    np.testing.assert_allclose(lc, np.log(np.arange(1, n + 1)), atol=1e-13)
    on, ln_ = A.attention_forward_head(z, k, v, scale, False)
    np.testing.assert_allclose(on, np.broadcast_to(v.mean(axis=0), on.shape), atol=1e-13)
    np.testing.assert_allclose(ln_, math.log(n), atol=1e-13)
    # causal row 0 sees only key 0: O_0 = V_0, LSE_0 = scale q0.k0
    oc, lc = A.attention_forward_head(q, k, v, scale, True)
    np.testing.assert_array_equal(oc[0], v[0])
    np.testing.assert_allclose(lc[0], scale * q[0] @ k[0], rtol=1e-15)
    # causal last row sees every key: equals the non-causal last row
    onc, lnc = A.attention_forward_head(q, k, v, scale, False)
    np.testing.assert_allclose(oc[-1], onc[-1], atol=1e-14)
    # N = 1: O = V
    o1, l1 = A.attention_forward_head(q[:1], k[:1], v[:1], scale, False)
    np.testing.assert_array_equal(o1, v[:1])
    # a row subset equals the same rows of the full result
    sub = np.array([0, 5, 36, 17])
    os_, ls_ = A.attention_forward_head(q, k, v, scale, True, rows=sub)
    np.testing.assert_allclose(os_, oc[sub], atol=0)
    np.testing.assert_allclose(ls_, lc[sub], atol=0)


def test_forward_invariants():
    check_forward_invariants()


def check_forward_row_chunks(seed=2):
    """The row chunking of the forward changes nothing but peak memory.

    N = 2100 keys puts the default budget at 1997 rows per chunk, so a head is
    two chunks, the second ragged.  Closed forms hold on every row of both:
    Q = 0 gives uniform weights (causal O_i = mean of V_0..V_i, LSE_i =
    ln(i + 1); non-causal O_i = mean of V, LSE_i = ln N), and causal row 0 sees
    only key 0 (O_0 = V_0).  Budgets of one, two and five rows per chunk
    (ragged last chunks) give what one chunk over all rows gives, also for a
    key block ahead of some queries, whose first rows see no key at all.
    """
    rng = np.random.default_rng(seed)
    n, d = 2100, 4
    k, v = rng.standard_normal((n, d)), rng.standard_normal((n, d))
    z = np.zeros((n, d))
    assert len(list(A._row_chunks(np.arange(n), n))) == 2
    oc, lc = A.attention_forward_head(z, k, v, 0.5, True)
    np.testing.assert_allclose(oc, np.cumsum(v, axis=0) / np.arange(1, n + 1)[:, None],
                               rtol=0, atol=1e-12)
    np.testing.assert_allclose(lc, np.log(np.arange(1, n + 1)), rtol=0, atol=1e-12)
    on, ln_ = A.attention_forward_head(z, k, v, 0.5, False)
    np.testing.assert_allclose(on, np.broadcast_to(v.mean(axis=0), on.shape), rtol=0, atol=1e-12)
    np.testing.assert_allclose(ln_, math.log(n), rtol=0, atol=1e-12)
    q = rng.standard_normal((n, d))
    oq, lq = A.attention_forward_head(q, k, v, 0.5, True)
    np.testing.assert_array_equal(oq[0], v[0])
    np.testing.assert_allclose(lq[0], 0.5 * q[0] @ k[0], rtol=1e-15)
    # small heads under tiny budgets against a single chunk
    m_, d_ = 37, 3
    qs, ks, vs = (rng.standard_normal((m_, d_)) for _ in range(3))
    for causal, q_off in ((False, 0), (True, 0), (True, -10)):
        whole = A.attention_forward_head(qs, ks, vs, 0.7, causal, q_offset=q_off,
                                         budget_elems=1 << 30)
        for budget in (1, 2 * m_, 5 * m_ + 3):
            part = A.attention_forward_head(qs, ks, vs, 0.7, causal, q_offset=q_off,
                                            budget_elems=budget)
            np.testing.assert_allclose(part[0], whole[0], rtol=0, atol=1e-14)
            np.testing.assert_array_equal(np.isinf(part[1]), np.isinf(whole[1]))
            fin = np.isfinite(whole[1])
            np.testing.assert_allclose(part[1][fin], whole[1][fin], rtol=0, atol=1e-14)
        if q_off < 0:
            # rows 0..9 sit before key 0: empty softmax
            assert np.all(whole[0][:10] == 0) and np.all(whole[1][:10] == -np.inf)
            assert np.all(np.isfinite(whole[1][10:]))


def test_forward_row_chunks():
    check_forward_row_chunks()


def test_forward_batched_matches_per_head():
    x = workloads.attention_inputs(2, 3, 19, 8, "bf16", seed=5)
    res = A.attention_forward(x["q"], x["k"], x["v"], 0.3, True, workers=4)
    for (b, h), (o, lse) in res.items():
        q, k, v = (A.to_f64(x[n][b, h]) for n in "qkv")
        o2, l2 = A.attention_forward_head(q, k, v, 0.3, True)
        np.testing.assert_array_equal(o, o2)
        np.testing.assert_array_equal(lse, l2)


def test_f16_inputs_converted_exactly():
    x = workloads.attention_inputs(1, 1, 4, 8, "f16", seed=9, in_scale=300.0)
    f = A.to_f64(x["q"])
    assert x["q"].dtype == torch.float16
    assert np.array_equal(f, x["q"].float().double().numpy())
    assert np.abs(f).max() > 256            # values beyond bf16's 8-bit mantissa steps survive


def test_bf16_inputs_converted_exactly():
    x = workloads.attention_inputs(1, 1, 4, 8, "bf16", seed=9)
    f = A.to_f64(x["q"])
    assert np.array_equal(f, x["q"].float().double().numpy())
    assert f.dtype == np.float64


# --------------------------------------------------------------------- backward

def check_backward_vs_fd(seed=2):
    rng = np.random.default_rng(seed)
    for (n, d, causal) in ((3, 2, True), (4, 3, False), (5, 2, True)):
        q, k, v, do = (rng.standard_normal((n, d)) for _ in range(4))
        scale = 1.0 / math.sqrt(d)
        g = A.attention_backward_head(q, k, v, do, scale, causal)
        fd = brute.grads_fd_decimal(q, k, v, do, scale, causal)
        for name in ("dq", "dk", "dv"):
            np.testing.assert_allclose(g[name], fd[name], rtol=0, atol=1e-9)


def test_backward_vs_decimal_finite_differences():
    check_backward_vs_fd()


def check_backward_invariants(seed=3):
    rng = np.random.default_rng(seed)
    n, d = 23, 8
    scale = 1.0 / math.sqrt(d)
    q, k, v, do = (rng.standard_normal((n, d)) for _ in range(4))
    for causal in (False, True):
        g = A.attention_backward_head(q, k, v, do, scale, causal)
        np.testing.assert_allclose(g["dv"].sum(axis=0), do.sum(axis=0), atol=1e-12)
        np.testing.assert_allclose(g["dk"].sum(axis=0), 0.0, atol=1e-12)
        o, lse = A.attention_forward_head(q, k, v, scale, causal)
        np.testing.assert_allclose(g["o"], o, atol=1e-14)
        np.testing.assert_allclose(g["lse"], lse, atol=1e-14)
        if causal:
            assert np.all(np.abs(g["dq"][0]) <= 1e-15)
            # the last key is seen only by the last query
            p_last = 1.0 / np.exp(lse[-1] - scale * q[-1] @ k[-1])
            np.testing.assert_allclose(g["dv"][-1], p_last * do[-1], atol=1e-14)


def test_backward_invariants():
    check_backward_invariants()


# ------------------------------------------------------------------ paged decode

# ---------------------------------------- offset blocks and merged partials

# (Nq, Nk, d, q_offset, k_offset): rows ahead of, straddling and behind the
# key block, including rows that see no key at all
OFFSET_CASES = ((3, 4, 2, 0, 2), (4, 3, 3, 5, 0), (5, 5, 2, 0, 0), (3, 5, 2, 2, 0), (2, 3, 2, 0, 7),
                (4, 2, 1, 1, 3))


def check_offset_vs_decimal(seed=5):
    """Offset causal attention against the 50-digit literal definition."""
    rng = np.random.default_rng(seed)
    for (nq, nk, d, qo, ko) in OFFSET_CASES:
        q = rng.standard_normal((nq, d)) * 1.5
        k = rng.standard_normal((nk, d)) * 1.5
        v = rng.standard_normal((nk, d + 1))
        scale = 1.0 / math.sqrt(d)
        o, lse = A.attention_forward_head(q, k, v, scale, True, q_offset=qo, k_offset=ko)
        Od, Ld = brute.attention_decimal(q, k, v, scale, True, q_offset=qo, k_offset=ko)
        np.testing.assert_allclose(o, np.array(Od, dtype=float), rtol=0, atol=1e-13)
        for got, want in zip(lse, Ld):
            if want is None:
                assert got == -np.inf
            else:
                assert abs(got - float(want)) <= 1e-13


def check_offset_reductions(seed=6):
    """Offsets that put every key at or before every query give plain
    (non-causal) attention; equal offsets give the ordinary causal case."""
    rng = np.random.default_rng(seed)
    q, k, v = (rng.standard_normal((6, 3)) for _ in range(3))
    o_nc, l_nc = A.attention_forward_head(q, k, v, 0.7, False)
    o_far, l_far = A.attention_forward_head(q, k, v, 0.7, True, q_offset=105, k_offset=100)
    np.testing.assert_array_equal(o_far, o_nc)
    np.testing.assert_array_equal(l_far, l_nc)
    o_c, l_c = A.attention_forward_head(q, k, v, 0.7, True)
    o_eq, l_eq = A.attention_forward_head(q, k, v, 0.7, True, q_offset=9, k_offset=9)
    np.testing.assert_array_equal(o_eq, o_c)
    np.testing.assert_array_equal(l_eq, l_c)
    # a key block entirely after every query: nothing visible
    o_none, l_none = A.attention_forward_head(q, k, v, 0.7, True, q_offset=0, k_offset=6)
    assert np.all(o_none == 0) and np.all(l_none == -np.inf)


def check_merge(seed=7):
    """Attention over a key set equals the merge of its parts (any split), the
    empty partial is the identity, and the merge is symmetric and associative."""
    rng = np.random.default_rng(seed)
    nq, nk, d = 7, 11, 3
    q = rng.standard_normal((nq, d)) * 2.0
    k = rng.standard_normal((nk, d)) * 2.0
    v = rng.standard_normal((nk, d))
    for causal, qo in ((True, 0), (True, 4), (True, -3), (False, 0)):
        full = A.attention_forward_head(q, k, v, 0.6, causal, q_offset=qo)
        for cut in (1, 5, 10):
            a = A.attention_forward_head(q, k[:cut], v[:cut], 0.6, causal, q_offset=qo, k_offset=0)
            b = A.attention_forward_head(q, k[cut:], v[cut:], 0.6, causal, q_offset=qo, k_offset=cut)
            o, l = A.merge_partials(a[0], a[1], b[0], b[1])
            np.testing.assert_allclose(o, full[0], rtol=0, atol=1e-13)
            fin = np.isfinite(full[1])
            np.testing.assert_allclose(l[fin], full[1][fin], rtol=0, atol=1e-13)
            assert np.all(l[~fin] == -np.inf) and np.all(o[~fin] == 0)
            o2, l2 = A.merge_partials(b[0], b[1], a[0], a[1])
            np.testing.assert_allclose(o2, o, rtol=0, atol=1e-15)
            np.testing.assert_allclose(l2, l, rtol=0, atol=1e-15)
        # three parts in either grouping
        p1, p2, p3 = (A.attention_forward_head(q, k[s:e], v[s:e], 0.6, causal, q_offset=qo, k_offset=s)
                      for s, e in ((0, 3), (3, 8), (8, nk)))
        left = A.merge_partials(*A.merge_partials(p1[0], p1[1], p2[0], p2[1]), p3[0], p3[1])
        right = A.merge_partials(p1[0], p1[1], *A.merge_partials(p2[0], p2[1], p3[0], p3[1]))
        np.testing.assert_allclose(left[0], full[0], rtol=0, atol=1e-13)
        np.testing.assert_allclose(right[0], full[0], rtol=0, atol=1e-13)
    x = A.attention_forward_head(q, k, v, 0.6, False)
    empty = (np.zeros_like(x[0]), np.full_like(x[1], -np.inf))
    o, l = A.merge_partials(x[0], x[1], *empty)
    np.testing.assert_array_equal(o, x[0])
    np.testing.assert_array_equal(l, x[1])
    o, l = A.merge_partials(*empty, *empty)
    assert np.all(o == 0) and np.all(l == -np.inf)


def test_offset_attention_vs_decimal_brute_force():
    check_offset_vs_decimal()


def test_offset_attention_reductions():
    check_offset_reductions()


def test_merge_of_partials():
    check_merge()


def _all_offset_pins():
    check_offset_vs_decimal()
    check_offset_reductions()
    check_merge()


def _scatter_to_pool(Kc, Vc, lens, block_size, H, d, seed):
    """Build a paged pool from contiguous per-sequence K/V by an independent route."""
    rng = np.random.default_rng(seed)
    nblk = [-(-L // block_size) for L in lens]
    total = sum(nblk) + 3
    perm = rng.permutation(total)
    kp = rng.standard_normal((total, block_size, H, d))
    vp = rng.standard_normal((total, block_size, H, d))
    table = -np.ones((len(lens), max(nblk)), dtype=np.int32)
    off = 0
    for s, L in enumerate(lens):
        for t in range(L):
            b, slot = divmod(t, block_size)
            if slot == 0:
                table[s, b] = perm[off]
                off += 1
            kp[table[s, b], slot] = Kc[s][t]
            vp[table[s, b], slot] = Vc[s][t]
    return kp, vp, table


def check_decode(seed=4):
    rng = np.random.default_rng(seed)
    H, d, bs = 3, 4, 4
    lens = [1, 4, 5, 11]
    Kc = [rng.standard_normal((L, H, d)) for L in lens]
    Vc = [rng.standard_normal((L, H, d)) for L in lens]
    q = rng.standard_normal((len(lens), H, d))
    scale = 0.5
    kp, vp, table = _scatter_to_pool(Kc, Vc, lens, bs, H, d, seed)
    o, lse = A.paged_decode(q, kp, vp, table, np.array(lens), bs, scale)
    for s, L in enumerate(lens):
        for h in range(H):
            Od, Ld = brute.attention_decimal(q[s, h][None], Kc[s][:, h], Vc[s][:, h], scale, False)
            np.testing.assert_allclose(o[s, h], np.array(Od[0], dtype=float), atol=1e-13)
            np.testing.assert_allclose(lse[s, h], float(Ld[0]), atol=1e-13)
    np.testing.assert_array_equal(o[0], Vc[0][0])     # seq_len 1: o = v_0
    # a second, different placement gives the same result
    kp2, vp2, table2 = _scatter_to_pool(Kc, Vc, lens, bs, H, d, seed + 100)
    o2, lse2 = A.paged_decode(q, kp2, vp2, table2, np.array(lens), bs, scale)
    np.testing.assert_allclose(o2, o, atol=1e-15)
    # equals the last row of a causal forward whose final query is q
    s = 3
    for h in range(H):
        qq = np.concatenate([rng.standard_normal((lens[s] - 1, d)), q[s, h][None]])
        of, lf = A.attention_forward_head(qq, Kc[s][:, h], Vc[s][:, h], scale, True)
        np.testing.assert_allclose(of[-1], o[s, h], atol=1e-14)
        np.testing.assert_allclose(lf[-1], lse[s, h], atol=1e-14)
    # pad slots past the length never enter the result
    kp_nan, vp_nan = kp.copy(), vp.copy()
    for s, L in enumerate(lens):
        if L % bs:
            p = table[s, L // bs]
            kp_nan[p, L % bs:] = np.nan
            vp_nan[p, L % bs:] = np.nan
    o3, lse3 = A.paged_decode(q, kp_nan, vp_nan, table, np.array(lens), bs, scale)
    np.testing.assert_array_equal(o3, o)
    np.testing.assert_array_equal(lse3, lse)


def test_paged_decode_pins():
    check_decode()


def test_paged_decode_on_generated_pool_with_nan_pads():
    p = workloads.paged_inputs(5, 2, 8, 16, 1, 40, seed=11, pad_value=float("nan"))
    o, lse = A.paged_decode(p["q"], p["k_pool"], p["v_pool"], p["block_table"], p["seq_lens"],
                            16, 0.35)
    assert np.all(np.isfinite(o)) and np.all(np.isfinite(lse))


# ------------------------------------------- grouped-query decode and append

def check_gqa_decode(seed=8):
    """Query head h reads cached head h // (H / KVH): against the 50-digit
    definition per head, and equal to multi-head decode over pools whose heads
    are repeated group-wise."""
    rng = np.random.default_rng(seed)
    H, d, bs = 6, 4, 4
    lens = [1, 5, 9]
    for KVH in (1, 2, 3, 6):
        g = H // KVH
        Kc = [rng.standard_normal((L, KVH, d)) for L in lens]
        Vc = [rng.standard_normal((L, KVH, d)) for L in lens]
        q = rng.standard_normal((len(lens), H, d))
        kp, vp, table = _scatter_to_pool(Kc, Vc, lens, bs, KVH, d, seed + KVH)
        o, lse = A.paged_decode(q, kp, vp, table, np.array(lens), bs, 0.4)
        for s_, L in enumerate(lens):
            for h in range(H):
                Od, Ld = brute.attention_decimal(q[s_, h][None], Kc[s_][:, h // g], Vc[s_][:, h // g],
                                                 0.4, False)
                np.testing.assert_allclose(o[s_, h], np.array(Od[0], dtype=float), atol=1e-13)
                np.testing.assert_allclose(lse[s_, h], float(Ld[0]), atol=1e-13)
        o_rep, lse_rep = A.paged_decode(q, np.repeat(kp, g, axis=2), np.repeat(vp, g, axis=2), table,
                                        np.array(lens), bs, 0.4)
        np.testing.assert_allclose(o_rep, o, atol=1e-15)
        np.testing.assert_allclose(lse_rep, lse, atol=1e-15)


def _paged_state(lens, bs, max_blocks, kvh, d, extra, seed):
    """A paged cache holding ``lens`` tokens per sequence plus ``extra`` free
    blocks, built by an independent scatter; returns contiguous copies too."""
    rng = np.random.default_rng(seed)
    Kc = [rng.standard_normal((L, kvh, d)) for L in lens]
    Vc = [rng.standard_normal((L, kvh, d)) for L in lens]
    used = sum(-(-L // bs) for L in lens)
    total = used + extra
    perm = rng.permutation(total)
    kp = rng.standard_normal((total, bs, kvh, d))
    vp = rng.standard_normal((total, bs, kvh, d))
    table = -np.ones((len(lens), max_blocks), dtype=np.int64)
    off = 0
    for s_, L in enumerate(lens):
        for t in range(L):
            b, slot = divmod(t, bs)
            if slot == 0:
                table[s_, b] = perm[off]
                off += 1
            kp[table[s_, b], slot] = Kc[s_][t]
            vp[table[s_, b], slot] = Vc[s_][t]
    free = perm[off:].copy()
    return kp, vp, table, free, Kc, Vc, rng


def check_paged_append(seed=9):
    """Appending tokens one step at a time: every sequence then holds exactly
    its old tokens followed by the new ones (read back through the table),
    blocks come off the top of the free stack in sequence order only at block
    boundaries, no block is shared, and full tables or an empty stack leave a
    sequence unchanged."""
    bs, kvh, d, max_blocks = 4, 2, 3, 3
    lens = [0, 3, 4, 7, 8, 11]
    kp, vp, table, free, Kc, Vc, rng = _paged_state(lens, bs, max_blocks, kvh, d, 4, seed)
    lens = np.array(lens)
    top = len(free)
    for step in range(3):
        kn = rng.standard_normal((len(lens), kvh, d))
        vn = rng.standard_normal((len(lens), kvh, d))
        r = A.paged_append(kp, vp, table, lens, free, top, kn, vn, bs)
        expect_fail = 0
        pops = []
        for s_ in range(len(lens)):
            t = int(lens[s_])
            if t >= bs * max_blocks or (t % bs == 0 and top - len(pops) == 0):
                expect_fail += 1
                assert r["seq_lens"][s_] == t
                continue
            if t % bs == 0:
                pops.append(s_)
            Kc[s_] = np.concatenate([Kc[s_], kn[s_][None]])
            Vc[s_] = np.concatenate([Vc[s_], vn[s_][None]])
            assert r["seq_lens"][s_] == t + 1
        assert r["n_failed"] == expect_fail
        assert r["free_count"] == top - len(pops)
        for i, s_ in enumerate(pops):                 # stack order: top first
            assert r["block_table"][s_, int(lens[s_]) // bs] == free[top - 1 - i]
        kp, vp, table, lens, top = r["k_pool"], r["v_pool"], r["block_table"], r["seq_lens"], r["free_count"]
        owned = []
        for s_, L in enumerate(lens):
            np.testing.assert_array_equal(A.gather_tokens(kp, table[s_], int(L), bs), Kc[s_])
            np.testing.assert_array_equal(A.gather_tokens(vp, table[s_], int(L), bs), Vc[s_])
            owned += list(table[s_, :-(-int(L) // bs)])
        assert len(owned) == len(set(owned))
        assert not set(owned) & set(free[:top].tolist())
    assert expect_fail >= 1                            # the sequence at capacity


def check_paged_prefill(seed=10):
    """A prefill chunk over a paged cache equals: the offset forward over the
    same tokens laid out contiguously (built by an independent scatter), plain
    causal attention when the chunk is the whole sequence, the paged decode
    when the chunk is one token, and the 50-digit definition."""
    rng = np.random.default_rng(seed)
    H, KVH, d, bs = 4, 2, 3, 4
    lens = [1, 5, 9, 12]
    chunks = [1, 3, 9, 4]                    # the last 'chunk' tokens of each sequence are queries
    Kc = [rng.standard_normal((L, KVH, d)) for L in lens]
    Vc = [rng.standard_normal((L, KVH, d)) for L in lens]
    kp, vp, table = _scatter_to_pool(Kc, Vc, lens, bs, KVH, d, seed)
    starts = np.concatenate([[0], np.cumsum(chunks)])
    q = rng.standard_normal((starts[-1], H, d))
    o, lse = A.paged_prefill(q, starts, kp, vp, table, np.array(lens), bs, 0.45)
    for s_, (L, n) in enumerate(zip(lens, chunks)):
        a, b = starts[s_], starts[s_ + 1]
        for h in range(H):
            g = h // (H // KVH)
            # the 50-digit definition with the chunk at the end of the sequence
            Od, Ld = brute.attention_decimal(q[a:b, h], Kc[s_][:, g], Vc[s_][:, g], 0.45, True,
                                             q_offset=L - n, k_offset=0)
            np.testing.assert_allclose(o[a:b, h], np.array(Od, dtype=float), atol=1e-13)
            np.testing.assert_allclose(lse[a:b, h], np.array(Ld, dtype=float), atol=1e-13)
            if n == L:      # the whole sequence: ordinary causal attention
                of, lf = A.attention_forward_head(q[a:b, h], Kc[s_][:, g], Vc[s_][:, g], 0.45, True)
                np.testing.assert_allclose(o[a:b, h], of, atol=1e-14)
        if n == 1:          # one new token: the paged decode
            od, ld = A.paged_decode(q[a:b], kp, vp, table[s_:s_ + 1], np.array([L]), bs, 0.45)
            np.testing.assert_allclose(o[a:b], od, atol=1e-14)
            np.testing.assert_allclose(lse[a:b], ld, atol=1e-14)


def test_paged_prefill_pins():
    check_paged_prefill()


def test_gqa_decode_pins():
    check_gqa_decode()


def test_paged_append_pins():
    check_paged_append()


def _all_paged_pins():
    check_decode()
    check_gqa_decode()
    check_paged_append()
    check_paged_prefill()


# ---------------------------------------------------------- planted mistakes

def _all_forward_pins(golden_dir):
    check_forward_vs_decimal()
    check_forward_large_scores()
    check_forward_invariants()
    check_forward_row_chunks()


def _all_backward_pins():
    check_backward_vs_fd()
    check_backward_invariants()


_orig = {n: getattr(A, n) for n in ("scores", "visible", "safe_softmax", "attend", "lse_of",
                                      "grad_v", "grad_p", "row_dot", "grad_s", "grad_q",
                                      "grad_k", "gather_tokens", "online_softmax")}


def _bad_safe_softmax_axis(s):
    m = np.max(s, axis=-1, keepdims=True)
    e = np.exp(s - m)
    l = np.sum(e, axis=0, keepdims=True)   # normalises the wrong axis
    return e / l, m[..., 0], np.sum(e, axis=-1)


def _bad_safe_softmax_nomax(s):
    e = np.exp(s)                          # no max subtraction
    l = np.sum(e, axis=-1, keepdims=True)
    return e / l, np.zeros(s.shape[:-1]), l[..., 0]


def _row_chunks_short(rows, nk, budget_elems=A.ROW_CHUNK_ELEMS):
    step = max(1, budget_elems // max(1, nk))
    for i in range(0, len(rows), step):
        yield rows[i:i + step - 1] if step > 1 else rows[i:i + 1][:0]   # drops a row per chunk


_REAL_FORWARD_HEAD = A.attention_forward_head


def _forward_head_pos_frozen(q, k, v, scale, causal, rows=None, q_offset=0, k_offset=0,
                             budget_elems=A.ROW_CHUNK_ELEMS):
    """The chunked forward with its output index never advancing past chunk 0."""
    nq, nk = q.shape[0], k.shape[0]
    rows = np.arange(nq) if rows is None else np.asarray(rows, dtype=np.int64)
    o = np.zeros((len(rows), v.shape[1]))
    lse = np.full((len(rows),), -np.inf)
    for r in A._row_chunks(rows, nk, budget_elems):
        vis = A.visible(r, nk, causal, q_offset, k_offset)
        some = vis.any(axis=1)
        if some.any():
            rs = r[some]
            s = np.where(vis[some], A.scores(q[rs], k, scale), -np.inf)
            p, m, l = A.safe_softmax(s)
            idx = np.nonzero(some)[0]                 # pos missing
            o[idx] = A.attend(p, v)
            lse[idx] = A.lse_of(m, l)
    return o, lse


def _forward_head_step_doubled(q, k, v, scale, causal, rows=None, q_offset=0, k_offset=0,
                               budget_elems=A.ROW_CHUNK_ELEMS):
    """The chunked forward with its output index advancing twice per chunk."""
    nq = q.shape[0]
    rows = np.arange(nq) if rows is None else np.asarray(rows, dtype=np.int64)
    o = np.zeros((len(rows), v.shape[1]))
    lse = np.full((len(rows),), -np.inf)
    pos = 0
    for r in A._row_chunks(rows, k.shape[0], budget_elems):
        if pos >= len(rows):
            break
        oc, lc = _REAL_FORWARD_HEAD(q, k, v, scale, causal, rows=r, q_offset=q_offset,
                                    k_offset=k_offset, budget_elems=1 << 40)
        n_ = min(len(r), len(rows) - pos)
        o[pos:pos + n_], lse[pos:pos + n_] = oc[:n_], lc[:n_]
        pos += 2 * len(r)
    return o, lse


FORWARD_MUTANTS = {
    "row_chunks_drop_row": ("_row_chunks", _row_chunks_short),
    "row_chunks_pos_frozen": ("attention_forward_head", _forward_head_pos_frozen),
    "row_chunks_step_doubled": ("attention_forward_head", _forward_head_step_doubled),
    "scale_dropped": ("scores", lambda q, k, scale: q @ k.T),
    "scale_squared": ("scores", lambda q, k, scale: scale * scale * (q @ k.T)),
    "transposed_scores": ("scores", lambda q, k, scale: scale * (k @ q.T) if q.shape == k.shape
                          else scale * (q @ k.T)[:, ::-1]),
    "causal_strict": ("visible", lambda rows, nk, causal, qo=0, ko=0:
                      (np.arange(nk)[None, :] + ko < np.asarray(rows)[:, None] + qo)
                      | (not causal) | (np.asarray(rows)[:, None] == 0) & (np.arange(nk)[None, :] == 0)),
    "causal_reversed": ("visible", lambda rows, nk, causal, qo=0, ko=0:
                        (np.arange(nk)[None, :] + ko >= np.asarray(rows)[:, None] + qo) | (not causal)),
    "causal_ignored": ("visible", lambda rows, nk, causal, qo=0, ko=0: np.ones((len(rows), nk), bool)),
    "softmax_wrong_axis": ("safe_softmax", _bad_safe_softmax_axis),
    "softmax_no_max": ("safe_softmax", _bad_safe_softmax_nomax),
    "values_reversed": ("attend", lambda p, v: p @ v[::-1]),
    "lse_sign": ("lse_of", lambda m, l: m - np.log(l)),
    "lse_no_max": ("lse_of", lambda m, l: np.log(l)),
}

def _merge_plain_average(o_a, lse_a, o_b, lse_b):
    return 0.5 * (np.asarray(o_a) + np.asarray(o_b)), np.maximum(lse_a, lse_b)


def _merge_inverted_weights(o_a, lse_a, o_b, lse_b):
    M = np.maximum(lse_a, lse_b)
    w_a, w_b = np.exp(M - lse_a), np.exp(M - lse_b)
    return (w_a[..., None] * o_a + w_b[..., None] * o_b) / (w_a + w_b)[..., None], M + np.log(w_a + w_b)


def _merge_lse_of_max_only(o_a, lse_a, o_b, lse_b):
    o, _ = _REAL_MERGE(o_a, lse_a, o_b, lse_b)
    return o, np.maximum(lse_a, lse_b)


def _merge_unnormalised(o_a, lse_a, o_b, lse_b):
    M = np.maximum(lse_a, lse_b)
    w_a, w_b = np.exp(lse_a - M), np.exp(lse_b - M)
    return w_a[..., None] * o_a + w_b[..., None] * o_b, M + np.log(w_a + w_b)


_REAL_MERGE = A.merge_partials

OFFSET_MUTANTS = {
    "offset_ignored": ("visible", lambda rows, nk, causal, qo=0, ko=0:
                       (np.arange(nk)[None, :] <= np.asarray(rows)[:, None]) | (not causal)),
    "offset_swapped": ("visible", lambda rows, nk, causal, qo=0, ko=0:
                       (np.arange(nk)[None, :] + qo <= np.asarray(rows)[:, None] + ko) | (not causal)),
    "offset_one_late": ("visible", lambda rows, nk, causal, qo=0, ko=0:
                        (np.arange(nk)[None, :] + ko < np.asarray(rows)[:, None] + qo) | (not causal)),
    "merge_plain_average": ("merge_partials", _merge_plain_average),
    "merge_inverted_weights": ("merge_partials", _merge_inverted_weights),
    "merge_lse_of_max_only": ("merge_partials", _merge_lse_of_max_only),
    "merge_unnormalised": ("merge_partials", _merge_unnormalised),
}

BACKWARD_MUTANTS = {
    "dv_untransposed": ("grad_v", lambda p, do: p @ do),
    "dp_wrong_operand": ("grad_p", lambda do, v: do @ v[::-1].T),
    "D_dropped": ("grad_s", lambda p, dp, D: p * dp),
    "D_sign": ("grad_s", lambda p, dp, D: p * (dp + D[:, None])),
    "D_from_wrong_axis": ("row_dot", lambda do, o: np.sum(do * o, axis=1)[::-1]),
    "dq_scale_dropped": ("grad_q", lambda ds, k, scale: ds @ k),
    "dq_transposed": ("grad_q", lambda ds, k, scale: scale * (ds.T @ k)),
    "dk_untransposed": ("grad_k", lambda ds, q, scale: scale * (ds @ q)),
}


def _gather_off_by_one(pool, table_row, length, block_size):
    t = np.arange(length)
    tbl = np.asarray(table_row).astype(np.int64)
    return A.to_f64(np.asarray(pool)[tbl[(t + 1) // block_size % max(1, (length + block_size - 1) // block_size)],
                                     (t + 1) % block_size])


def _gather_logical(pool, table_row, length, block_size):
    t = np.arange(length)
    return A.to_f64(np.asarray(pool)[t // block_size, t % block_size])


def _gather_one_extra(pool, table_row, length, block_size):
    return _orig["gather_tokens"](pool, table_row, min(length + 1, block_size * int(np.sum(np.asarray(table_row) >= 0))),
                                  block_size)


_REAL_APPEND = A.paged_append


def _append_variant(kind):
    """paged_append with one planted mistake."""
    def f(k_pool, v_pool, block_table, seq_lens, free_list, free_count, k_new, v_new, block_size):
        kp, vp = A.to_f64(k_pool).copy(), A.to_f64(v_pool).copy()
        table = np.array(block_table, dtype=np.int64)
        lens = np.array(seq_lens, dtype=np.int64)
        free = np.array(free_list, dtype=np.int64)
        kn, vn = A.to_f64(k_new), A.to_f64(v_new)
        top, bottom, failed = int(free_count), 0, 0
        for s_ in range(table.shape[0]):
            t = int(lens[s_])
            b, slot = t // block_size, t % block_size
            if kind == "slot_next":
                slot = (t + 1) % block_size
            if b >= table.shape[1]:
                failed += 1
                continue
            boundary = (t % block_size == 1) if kind == "alloc_one_late" else (t % block_size == 0)
            if boundary:
                if top - bottom == 0:
                    failed += 1
                    continue
                if kind == "pop_bottom":
                    table[s_, b] = free[bottom]
                    bottom += 1
                else:
                    top -= 1
                    table[s_, b] = free[top]
            phys = table[s_, b]
            kp[phys, slot] = kn[s_]
            vp[phys, slot] = vn[s_]
            if kind != "len_not_advanced":
                lens[s_] = t + 1
        return {"k_pool": kp, "v_pool": vp, "block_table": table, "seq_lens": lens,
                "free_count": top - bottom, "n_failed": failed}
    return f


def _prefill_top_aligned(q, q_start, k_pool, v_pool, block_table, seq_lens, block_size, scale,
                         causal=True, seqs=None, workers=None):
    """paged_prefill with the chunk's queries placed at positions 0.. (top-left
    alignment) instead of at the end of the sequence."""
    lens = np.asarray(seq_lens)
    starts = np.asarray(q_start)
    n = starts[1:] - starts[:-1]
    return _REAL_PREFILL(q, q_start, k_pool, v_pool, block_table, n, block_size, scale, causal,
                         seqs, workers) if np.all(n == lens) else _prefill_shift(
        q, starts, k_pool, v_pool, block_table, lens, block_size, scale)


def _prefill_shift(q, starts, k_pool, v_pool, block_table, lens, block_size, scale):
    H = q.shape[1]
    KVH = k_pool.shape[2]
    o = np.zeros((q.shape[0], H, v_pool.shape[3]))
    lse = np.full((q.shape[0], H), -np.inf)
    for s_ in range(len(lens)):
        a, b = int(starts[s_]), int(starts[s_ + 1])
        K = A.gather_tokens(k_pool, block_table[s_], int(lens[s_]), block_size)
        V = A.gather_tokens(v_pool, block_table[s_], int(lens[s_]), block_size)
        for h in range(H):
            g = A.kv_head_of(h, H, KVH)
            o[a:b, h], lse[a:b, h] = A.attention_forward_head(A.to_f64(q)[a:b, h], K[:, g], V[:, g],
                                                              scale, True)
    return o, lse


_REAL_PREFILL = A.paged_prefill

PAGED_MUTANTS = {
    "prefill_top_left_aligned": ("paged_prefill", _prefill_top_aligned),
    "gqa_modulo_heads": ("kv_head_of", lambda h, H, kvh: h % kvh),
    "gqa_reversed_groups": ("kv_head_of", lambda h, H, kvh: kvh - 1 - h // (H // kvh)),
    "append_pops_bottom": ("paged_append", _append_variant("pop_bottom")),
    "append_alloc_one_late": ("paged_append", _append_variant("alloc_one_late")),
    "append_slot_next": ("paged_append", _append_variant("slot_next")),
    "append_len_not_advanced": ("paged_append", _append_variant("len_not_advanced")),
}

DECODE_MUTANTS = {
    "slot_off_by_one": ("gather_tokens", _gather_off_by_one),
    "logical_block_ids": ("gather_tokens", _gather_logical),
    "reads_pad_slot": ("gather_tokens", _gather_one_extra),
}


def test_pins_pass_on_unmodified_oracle(golden_dir):
    _all_offset_pins()
    _all_paged_pins()
    _all_forward_pins(golden_dir)
    _all_backward_pins()
    check_decode()


@pytest.mark.parametrize("mutant", sorted(FORWARD_MUTANTS))
def test_forward_pins_catch_planted_mistake(mutant, monkeypatch, golden_dir):
    name, fn = FORWARD_MUTANTS[mutant]
    monkeypatch.setattr(A, name, fn)
    with pytest.raises((AssertionError, ValueError, FloatingPointError)):
        with np.errstate(all="ignore"):
            _all_forward_pins(golden_dir)


@pytest.mark.parametrize("mutant", sorted(OFFSET_MUTANTS))
def test_offset_pins_catch_planted_mistake(mutant, monkeypatch):
    name, fn = OFFSET_MUTANTS[mutant]
    monkeypatch.setattr(A, name, fn)
    with pytest.raises((AssertionError, ValueError, FloatingPointError)):
        with np.errstate(all="ignore"):
            _all_offset_pins()


@pytest.mark.parametrize("mutant", sorted(BACKWARD_MUTANTS))
def test_backward_pins_catch_planted_mistake(mutant, monkeypatch):
    name, fn = BACKWARD_MUTANTS[mutant]
    monkeypatch.setattr(A, name, fn)
    with pytest.raises((AssertionError, ValueError)):
        _all_backward_pins()


@pytest.mark.parametrize("mutant", sorted(PAGED_MUTANTS))
def test_paged_pins_catch_planted_mistake(mutant, monkeypatch):
    name, fn = PAGED_MUTANTS[mutant]
    monkeypatch.setattr(A, name, fn)
    with pytest.raises((AssertionError, ValueError, IndexError)):
        with np.errstate(all="ignore"):
            _all_paged_pins()


@pytest.mark.parametrize("mutant", sorted(DECODE_MUTANTS))
def test_decode_pins_catch_planted_mistake(mutant, monkeypatch):
    name, fn = DECODE_MUTANTS[mutant]
    monkeypatch.setattr(A, name, fn)
    with pytest.raises((AssertionError, ValueError, IndexError)):
        with np.errstate(all="ignore"):
            check_decode()


def _online_no_rescale(s, block, values=None):
    s = np.asarray(s, dtype=np.float64)
    n = s.shape[0]
    vals = np.eye(n) if values is None else np.asarray(values, dtype=np.float64)
    m, l, acc, traj = -math.inf, 0.0, np.zeros(vals.shape[1:]), []
    for start in range(0, n, block):
        blk = s[start:start + block]
        m = max(m, float(np.max(blk)))
        e = np.exp(blk - m)
        l = l + float(np.sum(e))           # forgets to rescale the old state
        acc = acc + e @ vals[start:start + block]
        traj.append({"m": m, "l": l, "alpha": 1.0})
    return acc / l, traj


def test_worked_example_catches_missing_rescale(monkeypatch, golden_dir):
    monkeypatch.setattr(A, "online_softmax", _online_no_rescale)
    with pytest.raises(AssertionError):
        check_worked_example(_golden(golden_dir, "online_softmax_worked_example.json"))
