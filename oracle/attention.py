"""fp64 CPU oracle for exact attention, its gradients and paged decode.

TEST INFRASTRUCTURE ONLY.  Nothing in the library imports this module; only
the test suite, the smoke check and the benchmark's CPU-baseline leg call it.
It shares no code with the HIP path: the only thing both sides have in common
is the seeded input generator in ``workloads``.

What is computed, and where the pages state it
-----------------------------------------------
* Attention (dcwnkz.com GPU/FlashAttention explainer, section "FlashAttention",
  its recap of the attention mechanism; and the HPC notes "07-16 afternoon",
  section "Autoregressive language model inference", tensor-shape walk-through):
  raw scores are the q.k dot products (i.e. Q K^T), softmax turns each row into
  weights that sum to 1, and the output is the weight-sum of the value rows.
  Shapes [B, heads, S, S] for scores and [B, heads, S, head_dim] for outputs.
  With grouped-query attention the cache holds fewer key/value heads than
  there are query heads (HPC notes, "Prefill, Decode and inference
  scheduling", KV-cache size); consecutive query heads share one.
  The scale factor on the scores is an argument (the pages never print one);
  the workloads use 1/sqrt(head_dim).
* Safe softmax in three passes (CMU 10-423 L17-L18 notes, section "Prerequisite
  2: online softmax"; explainer, appendix on softmax): pass 1 takes the row
  maximum, pass 2 sums exp(s - max), pass 3 divides.
* Causal mask (HPC notes, section "Autoregressive language model inference"):
  position i sees only itself and the tokens before it, i.e. key j is visible
  to query i iff j <= i.
* Online softmax (explainer, "FlashAttention" worked example; HPC notes,
  section "Long context and sequence parallelism"): blocks are scanned once,
  keeping a running maximum m, a running denominator l and an unnormalised
  weighted sum A; when a block raises the maximum, A and l are multiplied by
  exp(m_old - m_new) before the block is added.  This is used only to pin the
  worked example; the attention oracle itself is the plain definition above.
* Backward: the pages give only the principle (recompute the attention block
  instead of storing it; CMU notes, section "FlashAttention itself").  The
  oracle is the chain rule of O = softmax(S) V with S = scale * Q K^T, written
  out: dV = P^T dO, dP = dO V^T, D_i = sum_d dO_id O_id, dS = P o (dP - D),
  dQ = scale dS K, dK = scale dS^T Q.
* Paged decode (CMU notes, section "Decoding: PagedAttention"; HPC notes,
  section "Prefill, Decode and inference scheduling"): the KV cache is cut into
  fixed-size token blocks stored non-contiguously; a block table maps a
  sequence's logical block b to a physical block.  A decode step feeds one new
  query token that attends to every cached token of its sequence, itself
  included.  Token t of sequence s lives in physical block
  block_table[s, t // block_size], slot t % block_size.

* Offset blocks and merging partial results (HPC notes, section "Long context
  and sequence parallelism"; CS231N L11 notes, context-parallel part, ring
  attention): a rank holds a block of queries and meets the key/value blocks
  of the other ranks one at a time.  Rows carry global positions: query i of
  the block sits at q_offset + i, key j at k_offset + j, and the causal rule
  compares global positions.  Two partial results over disjoint key sets
  combine by the same rescale rule as the online softmax: with LSE = m + ln l,
  the weights are exp(LSE_a - M) and exp(LSE_b - M) for M = max(LSE_a, LSE_b).
  A query that sees no key of a block gets O = 0 and LSE = -inf there (the
  online softmax's starting state m = -inf, l = 0), which the merge treats as
  contributing nothing.

LSE is the natural log of the softmax denominator over the visible scaled
scores: LSE_i = m_i + ln(l_i).

Every routine works in float64 on values converted exactly from the storage
dtype (bf16 and fp32 embed exactly in fp64).
"""
from __future__ import annotations

import math
import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np

try:  # keep BLAS single-threaded inside the worker pool
    from threadpoolctl import threadpool_limits
except Exception:  # pragma: no cover
    threadpool_limits = None

__all__ = [
    "to_f64", "scores", "visible", "safe_softmax", "attend", "lse_of",
    "online_softmax", "attention_forward_head", "attention_forward",
    "attention_backward_head", "attention_backward", "gather_tokens",
    "paged_decode", "grad_v", "grad_p", "row_dot", "grad_s", "grad_q", "grad_k",
    "merge_partials", "kv_head_of", "paged_append", "paged_prefill",
]


def to_f64(x) -> np.ndarray:
    """Exact conversion of a torch tensor (any float dtype incl. bf16) or array to float64."""
    if hasattr(x, "detach"):
        import torch  # local: torch is only needed to read bf16 storage
        return x.detach().to("cpu", torch.float64).numpy()
    return np.asarray(x, dtype=np.float64)


# ---------------------------------------------------------------- forward steps

def scores(q: np.ndarray, k: np.ndarray, scale: float) -> np.ndarray:
    """Raw attention scores s_ij = scale * sum_d q_id k_jd (the Q K^T product)."""
    return scale * (q @ k.T)


def visible(rows: np.ndarray, nk: int, causal: bool, q_offset: int = 0,
            k_offset: int = 0) -> np.ndarray:
    """Boolean [len(rows), nk]: key j visible to query i.

    All keys without the causal rule; with it, key j (global position
    k_offset + j) is visible to query i (global position q_offset + i) iff
    k_offset + j <= q_offset + i.
    """
    cols = np.arange(nk, dtype=np.int64) + int(k_offset)
    if not causal:
        return np.ones((len(rows), nk), dtype=bool)
    return cols[None, :] <= (np.asarray(rows, dtype=np.int64) + int(q_offset))[:, None]


def safe_softmax(s: np.ndarray):
    """Row softmax by the three passes of safe softmax.

    Masked entries are -inf in ``s``; every row must have at least one finite
    entry.  Returns (p, m, l) with p = exp(s - m) / l.
    """
    m = np.max(s, axis=-1, keepdims=True)          # pass 1: row maximum
    e = np.exp(s - m)                              # exp(-inf) = 0 for masked keys
    l = np.sum(e, axis=-1, keepdims=True)          # pass 2: denominator
    return e / l, m[..., 0], l[..., 0]             # pass 3: normalise


def attend(p: np.ndarray, v: np.ndarray) -> np.ndarray:
    """Output rows: the p-weighted sum of the value rows (P V)."""
    return p @ v


def lse_of(m: np.ndarray, l: np.ndarray) -> np.ndarray:
    return m + np.log(l)


def online_softmax(s: np.ndarray, block: int, values: np.ndarray | None = None):
    """Blockwise online softmax of one score vector, as in the worked example.

    Scans ``s`` in blocks of ``block`` entries, never revisiting a block.  State:
    running max m, running denominator l, unnormalised accumulator A = sum of
    exp(s_j - m) * values_j.  When a block raises the max, the old A and l are
    multiplied by exp(m_old - m_new) first.  With ``values`` None the identity
    is used, so the final A / l is the weight vector itself.

    Returns (result, trajectory) with trajectory a list of per-block dicts
    {m, l, alpha} giving the state after each block.
    """
    s = np.asarray(s, dtype=np.float64)
    n = s.shape[0]
    vals = np.eye(n) if values is None else np.asarray(values, dtype=np.float64)
    m = -math.inf
    l = 0.0
    acc = np.zeros(vals.shape[1:], dtype=np.float64)
    traj = []
    for start in range(0, n, block):
        blk = s[start:start + block]
        m_new = max(m, float(np.max(blk)))
        alpha = 0.0 if m == -math.inf else math.exp(m - m_new)
        e = np.exp(blk - m_new)
        l = alpha * l + float(np.sum(e))
        acc = alpha * acc + e @ vals[start:start + block]
        traj.append({"m": m_new, "l": l, "alpha": alpha})
        m = m_new
    return acc / l, traj


ROW_CHUNK_ELEMS = 1 << 22   # score entries held at once per head (32 MiB of fp64)


def _row_chunks(rows: np.ndarray, nk: int, budget_elems: int = ROW_CHUNK_ELEMS):
    """Consecutive pieces of ``rows``, each of at most max(1, budget_elems // nk) rows."""
    step = max(1, budget_elems // max(1, nk))
    for i in range(0, len(rows), step):
        yield rows[i:i + step]


def attention_forward_head(q, k, v, scale: float, causal: bool, rows=None, q_offset: int = 0,
                           k_offset: int = 0, budget_elems: int = ROW_CHUNK_ELEMS):
    """Exact attention for one (batch, head).

    q [Nq, d], k [Nk, d], v [Nk, dv] float64.  ``rows`` selects a subset of the
    query rows (default: all).  ``q_offset`` / ``k_offset`` are the global
    positions of the first query / key row (they matter only for the causal
    rule).  Returns (O [len(rows), dv], LSE [len(rows)]); a row with no visible
    key gets O = 0 and LSE = -inf.  Rows are processed in chunks of at most
    ``budget_elems`` score entries to bound memory; each row is independent,
    so the chunking changes nothing but the peak memory.
    """
    nq, nk = q.shape[0], k.shape[0]
    rows = np.arange(nq) if rows is None else np.asarray(rows, dtype=np.int64)
    o = np.zeros((len(rows), v.shape[1]), dtype=np.float64)
    lse = np.full((len(rows),), -np.inf, dtype=np.float64)
    pos = 0                                        # output index of the chunk's first row
    for r in _row_chunks(rows, nk, budget_elems):
        vis = visible(r, nk, causal, q_offset, k_offset)
        some = vis.any(axis=1)                     # rows that see at least one key
        if some.any():
            rs = r[some]
            s = np.where(vis[some], scores(q[rs], k, scale), -np.inf)
            p, m, l = safe_softmax(s)
            idx = pos + np.nonzero(some)[0]
            o[idx] = attend(p, v)
            lse[idx] = lse_of(m, l)
        pos += len(r)
    return o, lse


def _usable_cpus() -> int:
    try:
        return len(os.sched_getaffinity(0))
    except (AttributeError, OSError):
        return os.cpu_count() or 1


def _pool_map(fn, items, workers):
    # default: one thread per usable core, at most 16 (each holds up to a few
    # hundred MiB of fp64 score chunks)
    workers = workers or min(len(items), _usable_cpus(), 16)
    if workers <= 1 or len(items) <= 1:
        return [fn(x) for x in items]
    if threadpool_limits is None:
        with ThreadPoolExecutor(max_workers=workers) as ex:
            return list(ex.map(fn, items))
    with threadpool_limits(limits=1), ThreadPoolExecutor(max_workers=workers) as ex:
        return list(ex.map(fn, items))


def attention_forward(q, k, v, scale: float, causal: bool, heads=None, rows=None,
                      workers: int | None = None, q_offset: int = 0, k_offset: int = 0):
    """Exact attention over [B, H, Nq, d] queries and [B, H, Nk, d] keys/values.

    ``heads`` is an optional list of (b, h) pairs to compute (default all);
    ``rows`` an optional list of query rows within each head; ``q_offset`` /
    ``k_offset`` the global positions of the first query / key row.  Returns
    {(b, h): (O, LSE)} with float64 arrays.
    """
    B, H = q.shape[0], q.shape[1]
    heads = [(b, h) for b in range(B) for h in range(H)] if heads is None else list(heads)

    def one(bh):
        b, h = bh
        return attention_forward_head(to_f64(q[b, h]), to_f64(k[b, h]), to_f64(v[b, h]),
                                      scale, causal, rows, q_offset, k_offset)
    return dict(zip(heads, _pool_map(one, heads, workers)))


def merge_partials(o_a, lse_a, o_b, lse_b):
    """Combine two partial attention results over disjoint key sets.

    o_* [..., dv] are normalised partial outputs and lse_* [...] their
    log-sum-exps.  By the rescale rule: M = max(LSE_a, LSE_b), weights
    w = exp(LSE - M), O = (w_a O_a + w_b O_b) / (w_a + w_b), LSE = M + ln(w_a + w_b).
    A side with LSE = -inf has weight 0; if both are -inf the result is O = 0,
    LSE = -inf.
    """
    o_a, o_b = np.asarray(o_a, dtype=np.float64), np.asarray(o_b, dtype=np.float64)
    lse_a, lse_b = np.asarray(lse_a, dtype=np.float64), np.asarray(lse_b, dtype=np.float64)
    M = np.maximum(lse_a, lse_b)
    empty = M == -np.inf
    Ms = np.where(empty, 0.0, M)
    w_a = np.where(lse_a == -np.inf, 0.0, np.exp(lse_a - Ms))
    w_b = np.where(lse_b == -np.inf, 0.0, np.exp(lse_b - Ms))
    tot = w_a + w_b
    safe = np.where(empty, 1.0, tot)
    o = (w_a[..., None] * o_a + w_b[..., None] * o_b) / safe[..., None]
    o = np.where(empty[..., None], 0.0, o)
    lse = np.where(empty, -np.inf, Ms + np.log(safe))
    return o, lse


# --------------------------------------------------------------- backward steps

def grad_v(p, do):
    """dV = P^T dO."""
    return p.T @ do


def grad_p(do, v):
    """dP = dO V^T."""
    return do @ v.T


def row_dot(do, o):
    """D_i = sum_d dO_id O_id (equal to sum_j P_ij dP_ij)."""
    return np.sum(do * o, axis=1)


def grad_s(p, dp, D):
    """Softmax backward: dS = P o (dP - D_i)."""
    return p * (dp - D[:, None])


def grad_q(ds, k, scale):
    """dQ = scale * dS K."""
    return scale * (ds @ k)


def grad_k(ds, q, scale):
    """dK = scale * dS^T Q."""
    return scale * (ds.T @ q)


def attention_backward_head(q, k, v, do, scale: float, causal: bool):
    """Gradients of L = sum(O o dO) for one (batch, head), float64, full N x N.

    Returns dict with o, lse (the oracle's own forward), dq, dk, dv.
    """
    nq, nk = q.shape[0], k.shape[0]
    rows = np.arange(nq)
    s = np.where(visible(rows, nk, causal), scores(q, k, scale), -np.inf)
    p, m, l = safe_softmax(s)
    o = attend(p, v)
    dv = grad_v(p, do)
    dp = grad_p(do, v)
    D = row_dot(do, o)
    ds = grad_s(p, dp, D)
    return {"o": o, "lse": lse_of(m, l), "dq": grad_q(ds, k, scale),
            "dk": grad_k(ds, q, scale), "dv": dv, "D": D}


def attention_backward(q, k, v, do, scale: float, causal: bool, heads=None,
                       workers: int | None = None):
    """Per-head gradients over [B, H, N, d] inputs; returns {(b, h): dict}."""
    B, H = q.shape[0], q.shape[1]
    heads = [(b, h) for b in range(B) for h in range(H)] if heads is None else list(heads)

    def one(bh):
        b, h = bh
        return attention_backward_head(to_f64(q[b, h]), to_f64(k[b, h]), to_f64(v[b, h]),
                                       to_f64(do[b, h]), scale, causal)
    return dict(zip(heads, _pool_map(one, heads, workers)))


# ------------------------------------------------------------------ paged decode

def gather_tokens(pool, table_row, length: int, block_size: int):
    """The ``length`` cached tokens of one sequence, in logical order.

    Token t is slot t % block_size of physical block table_row[t // block_size].
    ``pool`` is [num_blocks, block_size, H, d]; returns float64 [length, H, d].
    """
    t = np.arange(length)
    tbl = np.asarray(table_row).astype(np.int64)
    phys = tbl[t // block_size]
    slot = t % block_size
    if hasattr(pool, "detach"):
        import torch
        return to_f64(pool[torch.from_numpy(phys), torch.from_numpy(slot)])
    return to_f64(np.asarray(pool)[phys, slot])


def kv_head_of(h: int, H: int, kv_heads: int) -> int:
    """Grouped-query attention: query head h reads key/value head h // (H / kv_heads)
    (consecutive query heads share one cached head)."""
    return h // (H // kv_heads)


def paged_decode(q, k_pool, v_pool, block_table, seq_lens, block_size: int, scale: float,
                 seqs=None, workers: int | None = None):
    """Single-query attention of each sequence's new token over its cached tokens.

    q [S, H, d]; pools [num_blocks, block_size, KVH, d] with H a multiple of
    KVH (KVH = H is plain multi-head attention); block_table [S, max_blocks];
    seq_lens [S].  Returns (o [len(seqs), H, d], lse [len(seqs), H]) float64.
    """
    table = np.asarray(block_table.numpy() if hasattr(block_table, "numpy") else block_table)
    lens = np.asarray(seq_lens.numpy() if hasattr(seq_lens, "numpy") else seq_lens)
    seqs = list(range(table.shape[0])) if seqs is None else list(seqs)
    H = q.shape[1]
    KVH = k_pool.shape[2]
    assert H % KVH == 0

    def one(s):
        L = int(lens[s])
        K = gather_tokens(k_pool, table[s], L, block_size)
        V = gather_tokens(v_pool, table[s], L, block_size)
        qs = to_f64(q[s])
        o = np.empty((H, V.shape[2]))
        lse = np.empty((H,))
        for h in range(H):
            g = kv_head_of(h, H, KVH)
            oh, lh = attention_forward_head(qs[h:h + 1], K[:, g], V[:, g], scale, False)
            o[h], lse[h] = oh[0], lh[0]
        return o, lse
    res = _pool_map(one, seqs, workers)
    return np.stack([r[0] for r in res]), np.stack([r[1] for r in res])


def paged_append(k_pool, v_pool, block_table, seq_lens, free_list, free_count: int, k_new, v_new,
                 block_size: int):
    """Append one new token's K/V to every sequence of a paged cache.

    Blocks are taken only when needed (CMU notes, "Decoding: PagedAttention";
    HPC notes, "Prefill, Decode and inference scheduling": the runtime keeps
    each sequence's length and block mapping).  Sequences are visited in
    order.  Sequence s writes its token at position t = seq_lens[s]: when t is
    a multiple of block_size the sequence's blocks are full, so the block
    on top of the free stack, free_list[free_count - 1], is popped into
    block_table[s, t // block_size].  The token goes to slot t % block_size of
    that block and seq_lens[s] becomes t + 1.  A sequence that is at its table's
    capacity, or needs a block when the stack is empty, is left unchanged and
    counted as failed.

    Inputs are not modified.  Returns a dict with float64 pools, int64 table,
    lens, the new free_count and n_failed.
    """
    kp = to_f64(k_pool).copy()
    vp = to_f64(v_pool).copy()
    table = np.array(block_table.numpy() if hasattr(block_table, "numpy") else block_table,
                     dtype=np.int64)
    lens = np.array(seq_lens.numpy() if hasattr(seq_lens, "numpy") else seq_lens, dtype=np.int64)
    free = np.array(free_list.numpy() if hasattr(free_list, "numpy") else free_list, dtype=np.int64)
    kn, vn = to_f64(k_new), to_f64(v_new)
    top = int(free_count)
    failed = 0
    for s in range(table.shape[0]):
        t = int(lens[s])
        b, slot = t // block_size, t % block_size
        if b >= table.shape[1]:
            failed += 1
            continue
        if slot == 0:
            if top == 0:
                failed += 1
                continue
            top -= 1
            table[s, b] = free[top]
        phys = table[s, b]
        kp[phys, slot] = kn[s]
        vp[phys, slot] = vn[s]
        lens[s] = t + 1
    return {"k_pool": kp, "v_pool": vp, "block_table": table, "seq_lens": lens,
            "free_count": top, "n_failed": failed}


def paged_prefill(q, q_start, k_pool, v_pool, block_table, seq_lens, block_size: int, scale: float,
                  causal: bool = True, seqs=None, workers: int | None = None):
    """Prefill of a chunk of new queries per sequence over a paged KV cache.

    Sequence s holds seq_lens[s] cached tokens (its chunk's own K/V included)
    through its block table; its chunk has q_start[s+1] - q_start[s] queries,
    packed as rows of q [total_q, H, d], and they are the sequence's last
    tokens: query r of the chunk sits at position seq_lens[s] - n_s + r, so the
    causal rule is the offset one with q_offset = seq_lens[s] - n_s, k_offset 0
    (HPC notes, "Prefill, Decode and inference scheduling": prefill builds the
    cache for a whole prompt at once).  Query head h reads cached head
    kv_head_of(h, H, KVH).  Returns (o [total_q, H, d], lse [total_q, H]) for
    the rows of ``seqs`` (default all), float64.
    """
    table = np.asarray(block_table.numpy() if hasattr(block_table, "numpy") else block_table)
    lens = np.asarray(seq_lens.numpy() if hasattr(seq_lens, "numpy") else seq_lens)
    starts = np.asarray(q_start.numpy() if hasattr(q_start, "numpy") else q_start)
    seqs = list(range(table.shape[0])) if seqs is None else list(seqs)
    H, d = q.shape[1], q.shape[2]
    KVH = k_pool.shape[2]
    qf = to_f64(q)
    o = np.zeros((qf.shape[0], H, v_pool.shape[3]))
    lse = np.full((qf.shape[0], H), -np.inf)

    def one(s):
        L = int(lens[s])
        a, b = int(starts[s]), int(starts[s + 1])
        K = gather_tokens(k_pool, table[s], L, block_size)
        V = gather_tokens(v_pool, table[s], L, block_size)
        res = []
        for h in range(H):
            g = kv_head_of(h, H, KVH)
            res.append(attention_forward_head(qf[a:b, h], K[:, g], V[:, g], scale, causal,
                                              q_offset=L - (b - a), k_offset=0))
        return a, b, res
    for a, b, res in _pool_map(one, seqs, workers):
        for h, (oh, lh) in enumerate(res):
            o[a:b, h], lse[a:b, h] = oh, lh
    return o, lse
