"""Seeded synthetic inputs for exact attention and paged decode.

This module only draws random numbers, casts them to the storage dtype and
arranges them in the layouts the library expects.  It holds none of the
attention arithmetic: both the fp64 oracle (test infrastructure) and the HIP
path read their inputs from here, so that both sides see bit-identical values.

Layouts follow the problem statement of the HPC notes "07-16 afternoon:
distributed LLM training and inference" (section "Autoregressive language
model inference", the tensor-shape walk-through): Q, K, V, O are
[B, heads, S, head_dim].  The paged KV pool follows
the PagedAttention description in the CMU 10-423 L17-L18 notes (section
"Decoding: PagedAttention"): fixed-size token blocks stored non-contiguously
and addressed through a per-sequence block table.

Every tensor returned here lives on the CPU.  Values are drawn as fp32
N(0, 1), optionally multiplied by a constant, then rounded to the storage
dtype with round-to-nearest-even (torch's cast).
"""
from __future__ import annotations

import math
from dataclasses import dataclass

import torch

__all__ = [
    "AttnConfig", "DecodeConfig", "FP32_SMALL", "GPT2_SHAPE", "LONG_CONTEXT", "FWD_BWD", "DECODE",
    "WORKLOADS", "attention_inputs", "paged_inputs", "prefill_queries", "ramp_inputs", "spike_inputs",
]

_TORCH_DTYPES = {"f32": torch.float32, "bf16": torch.bfloat16, "f16": torch.float16}


@dataclass(frozen=True)
class AttnConfig:
    name: str
    B: int
    H: int
    N: int
    d: int
    dtype: str            # "f32" | "bf16"
    causal: bool
    in_scale: float = 1.0  # multiplies the N(0,1) draws before the cast
    grads: bool = False    # also draw dO
    seed: int = 0          # seed of the workload's draws

    @property
    def scale(self) -> float:
        return 1.0 / math.sqrt(self.d)


@dataclass(frozen=True)
class DecodeConfig:
    name: str
    num_seqs: int
    H: int
    d: int
    block_size: int
    min_len: int
    max_len: int
    dtype: str = "bf16"
    seed: int = 0          # seed of the workload's draws

    @property
    def scale(self) -> float:
        return 1.0 / math.sqrt(self.d)

    @property
    def max_blocks_per_seq(self) -> int:
        return -(-self.max_len // self.block_size)


# The benchmark's workloads, each named by what it is.  FP32_SMALL is the
# small fp32 case the oracle finishes in well under a second; GPT2_SHAPE,
# LONG_CONTEXT and FWD_BWD are forward/backward shapes; DECODE is single-token
# decode over a paged cache.  Each carries the seed its inputs are drawn from.
FP32_SMALL = AttnConfig("noncausal_f32_b1_h2_n256_d64", 1, 2, 256, 64, "f32", False, seed=70001)
GPT2_SHAPE = AttnConfig("causal_bf16_b8_h12_n1024_d64", 8, 12, 1024, 64, "bf16", True,
                        in_scale=1.0 / 8.0, seed=70002)
LONG_CONTEXT = AttnConfig("causal_bf16_b1_h32_n8192_d128", 1, 32, 8192, 128, "bf16", True,
                          seed=70003)
FWD_BWD = AttnConfig("causal_fwdbwd_bf16_b4_h16_n2048_d128", 4, 16, 2048, 128, "bf16", True,
                     grads=True, seed=70004)
DECODE = DecodeConfig("paged_decode_bf16_s64_h32_d128_bs16", 64, 32, 128, 16, 128, 4096,
                      seed=70005)
WORKLOADS = {w.name: w for w in (FP32_SMALL, GPT2_SHAPE, LONG_CONTEXT, FWD_BWD, DECODE)}


def _gen(seed: int) -> torch.Generator:
    g = torch.Generator(device="cpu")
    g.manual_seed(int(seed))
    return g


def attention_inputs(B: int, H: int, N: int, d: int, dtype: str = "bf16", *,
                     seed: int, in_scale: float = 1.0, with_do: bool = False,
                     N_k: int | None = None) -> dict:
    """Draw Q, K, V (and dO) in order from one generator.

    Returns CPU tensors in the storage dtype, contiguous [B, H, S, d].
    ``N_k`` (default N) sets the key/value length.
    """
    tdt = _TORCH_DTYPES[dtype]
    g = _gen(seed)
    nk = N if N_k is None else N_k
    out = {}
    for name, n in (("q", N), ("k", nk), ("v", nk)) + ((("do", N),) if with_do else ()):
        x = torch.randn((B, H, n, d), generator=g, dtype=torch.float32)
        if in_scale != 1.0:
            x = x * in_scale
        out[name] = x.to(tdt).contiguous()
    return out


def ramp_inputs(B: int, H: int, N: int, d: int, dtype: str = "bf16", *, seed: int,
                align: float, ramp: float, noise: float = 0.1) -> dict:
    """Q, K, V whose scores grow along the key axis.

    Every query and key shares a component along one fixed unit direction e:
    q_i = noise*z + align*e and k_j = noise*z + ramp*(j/64)*e, so the score of
    key j rises by about scale*align*ramp per 64 keys (one key tile of the
    kernels) and every row's maximum keeps moving to later keys.  ``ramp`` < 0
    makes it fall instead.  V is plain N(0, 1).  CPU tensors, storage dtype.
    """
    tdt = _TORCH_DTYPES[dtype]
    g = _gen(seed)
    e = torch.randn(d, generator=g, dtype=torch.float32)
    e = e / e.norm()
    q = noise * torch.randn((B, H, N, d), generator=g, dtype=torch.float32) + align * e
    pos = torch.arange(N, dtype=torch.float32).view(1, 1, N, 1) / 64.0
    k = noise * torch.randn((B, H, N, d), generator=g, dtype=torch.float32) + ramp * pos * e
    v = torch.randn((B, H, N, d), generator=g, dtype=torch.float32)
    return {"q": q.to(tdt).contiguous(), "k": k.to(tdt).contiguous(), "v": v.to(tdt).contiguous()}


def spike_inputs(B: int, H: int, N: int, d: int, dtype: str = "bf16", *, seed: int,
                 align: float, spike: float, keys: list, noise: float = 0.1) -> dict:
    """Q, K, V where a few chosen keys score far above all others.

    q_i = noise*z + align*e and k_j = noise*z + spike*e for j in ``keys``
    (noise*z alone otherwise), with e one fixed unit direction: the chosen keys
    score about scale*align*spike above the rest for every query.  V is plain
    N(0, 1).  CPU tensors, storage dtype.
    """
    tdt = _TORCH_DTYPES[dtype]
    g = _gen(seed)
    e = torch.randn(d, generator=g, dtype=torch.float32)
    e = e / e.norm()
    q = noise * torch.randn((B, H, N, d), generator=g, dtype=torch.float32) + align * e
    k = noise * torch.randn((B, H, N, d), generator=g, dtype=torch.float32)
    for j in keys:
        k[:, :, j, :] += spike * e
    v = torch.randn((B, H, N, d), generator=g, dtype=torch.float32)
    return {"q": q.to(tdt).contiguous(), "k": k.to(tdt).contiguous(), "v": v.to(tdt).contiguous()}


def paged_inputs(num_seqs: int, H: int, d: int, block_size: int, min_len: int, max_len: int,
                 *, seed: int, dtype: str = "bf16", pad_value: float | None = None,
                 seq_lens: list | None = None, extra_blocks: int = 0,
                 kv_heads: int | None = None) -> dict:
    """Draw a paged KV pool with randomly permuted physical block placement.

    Draw order: seq_lens ~ U{min_len..max_len}; a permutation of the physical
    block ids; k_pool; v_pool; q.  Physical ids are handed out in (sequence,
    logical block) order from the permutation.  ``block_table`` entries past a
    sequence's last block are -1.  ``pad_value`` (e.g. NaN) overwrites the
    token slots past each sequence's length inside its last block, which the
    decode must never read into its result.  ``extra_blocks`` adds unused
    physical blocks to the pool; they are returned as ``free_list`` (int32, the
    rest of the permutation) with ``free_count`` entries.  ``kv_heads`` (default
    H) is the number of key/value heads the pools hold; q always has H heads.
    """
    tdt = _TORCH_DTYPES[dtype]
    g = _gen(seed)
    if seq_lens is None:
        lens = torch.randint(min_len, max_len + 1, (num_seqs,), generator=g, dtype=torch.int64)
    else:
        lens = torch.tensor(seq_lens, dtype=torch.int64)
        assert lens.numel() == num_seqs
    nblk = [(int(n) + block_size - 1) // block_size for n in lens.tolist()]
    max_blocks = max(-(-max_len // block_size), max(nblk) if nblk else 0)
    total = sum(nblk) + int(extra_blocks)
    perm = torch.randperm(total, generator=g, dtype=torch.int64)
    table = torch.full((num_seqs, max_blocks), -1, dtype=torch.int32)
    off = 0
    for s, nb in enumerate(nblk):
        table[s, :nb] = perm[off:off + nb].to(torch.int32)
        off += nb
    kvh = H if kv_heads is None else int(kv_heads)
    shape = (total, block_size, kvh, d)
    k_pool = _randn_chunked(shape, g, tdt)
    v_pool = _randn_chunked(shape, g, tdt)
    q = torch.randn((num_seqs, H, d), generator=g, dtype=torch.float32).to(tdt)
    if pad_value is not None:
        for s, n in enumerate(lens.tolist()):
            r = n % block_size
            if r:
                p = int(table[s, nblk[s] - 1])
                k_pool[p, r:] = pad_value
                v_pool[p, r:] = pad_value
    free = perm[off:].to(torch.int32).contiguous()
    return {"q": q.contiguous(), "k_pool": k_pool, "v_pool": v_pool,
            "block_table": table.contiguous(), "seq_lens": lens.to(torch.int32).contiguous(),
            "block_size": block_size, "num_blocks": total, "max_blocks_per_seq": max_blocks,
            "free_list": free, "free_count": int(free.numel()), "kv_heads": kvh}


def prefill_queries(chunks: list, H: int, d: int, dtype: str = "bf16", *, seed: int) -> dict:
    """Packed query rows of a chunked prefill: q [sum(chunks), H, d] drawn
    N(0, 1) in one go, and q_start [len(chunks) + 1] int32 (prefix sums of the
    chunk lengths).  CPU tensors, storage dtype."""
    g = _gen(seed)
    starts = [0]
    for n in chunks:
        starts.append(starts[-1] + int(n))
    q = torch.randn((starts[-1], H, d), generator=g, dtype=torch.float32).to(_TORCH_DTYPES[dtype])
    return {"q": q.contiguous(), "q_start": torch.tensor(starts, dtype=torch.int32)}


def _randn_chunked(shape, g, tdt, chunk_rows: int = 512) -> torch.Tensor:
    """N(0,1) draws of ``shape`` filled along dim 0 in chunks (bounded fp32 temporaries)."""
    out = torch.empty(shape, dtype=tdt)
    for i in range(0, shape[0], chunk_rows):
        j = min(shape[0], i + chunk_rows)
        out[i:j] = torch.randn((j - i,) + tuple(shape[1:]), generator=g, dtype=torch.float32).to(tdt)
    return out
