"""Benchmark of the libfa hot path on one MI355X.

One step = one pass of the whole hot path over synthetic inputs of the
benchmark shapes:
  * fa_fwd   causal bf16 B=1 H=32 N=8192 d=128   (the headline: TFLOP/s, % MFMA peak)
  * the same forward with fp16 inputs
  * fa_fwd   causal bf16 B=8 H=12 N=1024 d=64
  * fa_fwd + fa_bwd causal bf16 B=4 H=16 N=2048 d=128
  * fa_paged_decode bf16 64 seqs x H=32 x d=128, lengths U[128,4096], 16-token blocks
  * the same decode with 8 cached key/value heads (grouped-query attention)
    and one paged KV append of a token per sequence
  * chunked prefill over a paged cache: 8 sequences x 1024 new tokens
  * one ring-attention step at the long-context shape: fa_fwd_offset of the
    8192 queries against the previous 8192-token block, then fa_merge
Inputs are resident in HBM before timing starts.  Each call is bracketed by
HIP events on the stream it runs on; `value` is the headline forward's
algorithmic TFLOP/s (causal pairs only) over its average kernel time.

The CPU baseline times the fp64 oracle on a bounded sample of the headline
workload on the host's cores.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu-baseline]
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0      # MI355X dense bf16 matrix peak (published)
PEAK_HBM_GBS = 8000.0          # MI355X HBM3E peak (published)


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def causal_flops(B, H, N, d):
    return 4 * B * H * d * (N * (N + 1) // 2)


def source_hash(*names):
    h = hashlib.sha256()
    for n in names:
        with open(os.path.join(ROOT, "exact_attention_70_amd", "csrc", n), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def load_traffic(kernel_key, src_hash):
    """HBM bytes per launch from committed rocprofv3 counter runs, if still current."""
    p = os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(p):
        return None
    try:
        rec = json.load(open(p)).get(kernel_key)
    except Exception:
        return None
    if not rec or rec.get("source_hash") != src_hash:
        return None
    return rec.get("bytes_per_launch")


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--only", default="",
                    help="comma list of parts to run: fwd_c3, fwd_c3_f16, fwd_c2, fwd_c4, bwd_c4, "
                         "decode_c5, "
                         "decode_gqa_c5 (8 cached heads), append_c5 (paged KV append), "
                         "prefill_gqa (chunked prefill over a paged cache), "
                         "ring_c3 (offset forward + merge of one ring step), copy_calib (a 1 GiB "
                         "device copy used to scale the HBM-traffic counters)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only: --gpus {args.gpus} is not supported "
              "(the kernels run on a single MI355X; see DESIGN.md for how the path would shard)",
              file=sys.stderr)
        sys.exit(2)

    import torch
    import workloads
    from exact_attention_70_amd import binding

    binding.load_library()
    dev = torch.device("cuda:0")
    only = set(x for x in args.only.split(",") if x)

    def want(name):
        return not only or name in only

    # ------------------------------------------------------------ inputs (untimed)
    c3, c2, c4, c5 = (workloads.CONFIGS[i] for i in (3, 2, 4, 5))
    parts = {}
    if want("fwd_c3"):
        x = workloads.attention_inputs(c3.B, c3.H, c3.N, c3.d, "bf16", seed=workloads.seed_for(3))
        q, k, v = (x[n].to(dev) for n in "qkv")
        o = torch.empty_like(q)
        lse = torch.empty(c3.B, c3.H, c3.N, device=dev)
        parts["fwd_c3"] = dict(fn=lambda: binding.fwd(q, k, v, causal=True, scale=c3.scale, out=o,
                                                       lse=lse),
                               flops=causal_flops(c3.B, c3.H, c3.N, c3.d))
    if want("fwd_c3_f16"):
        # the headline forward with fp16 inputs (same draws, cast to fp16)
        xh = workloads.attention_inputs(c3.B, c3.H, c3.N, c3.d, "f16", seed=workloads.seed_for(3))
        qh, kh, vh = (xh[n].to(dev) for n in "qkv")
        oh = torch.empty_like(qh)
        lseh = torch.empty(c3.B, c3.H, c3.N, device=dev)
        parts["fwd_c3_f16"] = dict(fn=lambda: binding.fwd(qh, kh, vh, causal=True, scale=c3.scale,
                                                           out=oh, lse=lseh),
                                   flops=causal_flops(c3.B, c3.H, c3.N, c3.d))
    if want("ring_c3"):
        # one rank's non-diagonal ring step at the long-context shape: its 8192
        # queries (global rows 8192..16383) against the previous 8192-token
        # key/value block (every key visible), merged into the running result
        xr = x if want("fwd_c3") else workloads.attention_inputs(c3.B, c3.H, c3.N, c3.d, "bf16",
                                                                 seed=workloads.seed_for(3))
        qr, kr, vr = (xr[n].to(dev) for n in "qkv")
        po = torch.empty_like(qr)
        pl = torch.empty(c3.B, c3.H, c3.N, device=dev)
        acc_o, acc_l = binding.fwd(qr, kr, vr, causal=True, scale=c3.scale)   # diagonal block
        parts["ring_c3_fwd"] = dict(fn=lambda: binding.fwd_offset(
            qr, kr, vr, q_offset=c3.N, k_offset=0, causal=True, scale=c3.scale, out=po, lse=pl),
            flops=4 * c3.B * c3.H * c3.N * c3.N * c3.d)
        parts["ring_c3_merge"] = dict(fn=lambda: binding.merge(acc_o, acc_l, po, pl, out=acc_o,
                                                                lse_out=acc_l),
                                      bytes=3 * acc_o.numel() * 2 + 3 * acc_l.numel() * 4)
    if want("fwd_c2"):
        x2 = workloads.attention_inputs(c2.B, c2.H, c2.N, c2.d, "bf16", seed=workloads.seed_for(2),
                                        in_scale=c2.in_scale)
        q2, k2, v2 = (x2[n].to(dev) for n in "qkv")
        o2 = torch.empty_like(q2)
        lse2 = torch.empty(c2.B, c2.H, c2.N, device=dev)
        parts["fwd_c2"] = dict(fn=lambda: binding.fwd(q2, k2, v2, causal=True, scale=c2.scale,
                                                       out=o2, lse=lse2),
                               flops=causal_flops(c2.B, c2.H, c2.N, c2.d))
    if want("fwd_c4") or want("bwd_c4"):
        x4 = workloads.attention_inputs(c4.B, c4.H, c4.N, c4.d, "bf16", seed=workloads.seed_for(4),
                                        with_do=True)
        q4, k4, v4, do4 = (x4[n].to(dev) for n in ("q", "k", "v", "do"))
        o4 = torch.empty_like(q4)
        lse4 = torch.empty(c4.B, c4.H, c4.N, device=dev)
        grads = tuple(torch.empty(q4.shape, dtype=torch.float32, device=dev) for _ in range(3))
        ws4 = torch.empty(binding.bwd_workspace_size(c4.B, c4.H, c4.N, c4.d), dtype=torch.uint8,
                          device=dev)
        f4 = causal_flops(c4.B, c4.H, c4.N, c4.d)
        parts["fwd_c4"] = dict(fn=lambda: binding.fwd(q4, k4, v4, causal=True, scale=c4.scale,
                                                       out=o4, lse=lse4), flops=f4)
        parts["bwd_c4"] = dict(fn=lambda: binding.bwd(q4, k4, v4, o4, do4, lse4, causal=True,
                                                       scale=c4.scale, workspace=ws4, grads=grads),
                               flops=int(2.5 * f4), flops_2x=2 * f4)
    if want("decode_c5"):
        p = workloads.paged_inputs(c5.num_seqs, c5.H, c5.d, c5.block_size, c5.min_len, c5.max_len,
                                   seed=workloads.seed_for(5))
        pd = {kk: (vv.to(dev) if isinstance(vv, torch.Tensor) else vv) for kk, vv in p.items()}
        od = torch.empty_like(pd["q"])
        lsed = torch.empty(c5.num_seqs, c5.H, device=dev)
        wsd = torch.empty(binding.paged_decode_workspace_size(c5.num_seqs, c5.H, c5.d,
                                                              p["max_blocks_per_seq"], 16),
                          dtype=torch.uint8, device=dev)
        tokens = int(p["seq_lens"].long().sum())
        kv_bytes = tokens * c5.H * c5.d * 2 * 2
        parts["decode_c5"] = dict(fn=lambda: binding.paged_decode(
            pd["q"], pd["k_pool"], pd["v_pool"], pd["block_table"], pd["seq_lens"], block_size=16,
            scale=c5.scale, workspace=wsd, out=od, lse=lsed), bytes=kv_bytes, tokens=tokens)
    if want("decode_gqa_c5") or want("append_c5"):
        # the same sequences with 8 cached heads for the 32 query heads, and
        # enough free blocks for every timed append step
        pg = workloads.paged_inputs(c5.num_seqs, c5.H, c5.d, c5.block_size, c5.min_len,
                                    c5.max_len, seed=workloads.seed_for(5), kv_heads=8,
                                    extra_blocks=4 * c5.num_seqs)
        pgd = {kk: (vv.to(dev) if isinstance(vv, torch.Tensor) else vv) for kk, vv in pg.items()}
        tokens_g = int(pg["seq_lens"].long().sum())
        if want("decode_gqa_c5"):
            og = torch.empty_like(pgd["q"])
            lseg = torch.empty(c5.num_seqs, c5.H, device=dev)
            wsg = torch.empty(binding.paged_decode_workspace_size(c5.num_seqs, c5.H, c5.d,
                                                                  pg["max_blocks_per_seq"], 16),
                              dtype=torch.uint8, device=dev)
            parts["decode_gqa_c5"] = dict(fn=lambda: binding.paged_decode(
                pgd["q"], pgd["k_pool"], pgd["v_pool"], pgd["block_table"], pgd["seq_lens"],
                block_size=16, scale=c5.scale, workspace=wsg, out=og, lse=lseg),
                bytes=tokens_g * 8 * c5.d * 2 * 2, tokens=tokens_g)
        if want("append_c5"):
            ga = torch.Generator().manual_seed(workloads.seed_for(5) + 1)
            kn = torch.randn((c5.num_seqs, 8, c5.d), generator=ga).to(torch.bfloat16).to(dev)
            vn = torch.randn((c5.num_seqs, 8, c5.d), generator=ga).to(torch.bfloat16).to(dev)
            fc = torch.tensor([pg["free_count"]], dtype=torch.int32, device=dev)
            nf = torch.zeros(1, dtype=torch.int32, device=dev)
            # lengths and the free stack advance on every call (state of a real decode loop)
            lens_a = pgd["seq_lens"].clone()
            table_a = pgd["block_table"].clone()
            parts["append_c5"] = dict(fn=lambda: binding.paged_kv_append(
                kn, vn, pgd["k_pool"], pgd["v_pool"], table_a, lens_a, pgd["free_list"], fc, nf,
                block_size=16), bytes=2 * 2 * kn.numel() * 2)
    if want("prefill_gqa"):
        # chunked prefill: 8 sequences, a 1024-token chunk each at the end of
        # 1500..4000 cached tokens, 32 query heads on 8 cached heads
        lens_p = [1500, 2048, 2500, 3000, 3333, 3700, 4000, 1024]
        pp = workloads.paged_inputs(len(lens_p), c5.H, c5.d, 16, 1, max(lens_p),
                                    seed=workloads.seed_for(5) + 2, seq_lens=lens_p, kv_heads=8)
        qp = workloads.prefill_queries([1024] * len(lens_p), c5.H, c5.d, seed=workloads.seed_for(5) + 3)
        ppd = {kk: (vv.to(dev) if isinstance(vv, torch.Tensor) else vv) for kk, vv in pp.items()}
        qpd, qsd = qp["q"].to(dev), qp["q_start"].to(dev)
        op = torch.empty_like(qpd)
        lsep = torch.empty(qpd.shape[0], c5.H, device=dev)
        pairs = sum(sum(L - 1024 + r + 1 for r in range(1024)) for L in lens_p)
        parts["prefill_gqa"] = dict(fn=lambda: binding.paged_prefill(
            qpd, qsd, ppd["k_pool"], ppd["v_pool"], ppd["block_table"], ppd["seq_lens"],
            block_size=16, max_q_len=1024, scale=c5.scale, out=op, lse=lsep),
            flops=4 * c5.H * c5.d * pairs)
    if "copy_calib" in only:
        # plain device copy of known size: the HBM-traffic counters of the kernels
        # are scaled by what the same counters read for this copy
        src = torch.empty(256 << 20, dtype=torch.float32, device=dev)      # 1 GiB
        src.fill_(1.0)
        dst = torch.empty_like(src)
        parts["copy_calib"] = dict(fn=lambda: dst.copy_(src), bytes=2 * src.numel() * 4)
    torch.cuda.synchronize()
    log(f"inputs ready: {list(parts)}")

    order = [n for n in ("fwd_c3", "fwd_c3_f16", "fwd_c2", "fwd_c4", "bwd_c4", "decode_c5",
                         "decode_gqa_c5",
                         "append_c5", "prefill_gqa", "ring_c3_fwd", "ring_c3_merge", "copy_calib")
             if n in parts]
    for _ in range(args.warmup):
        for n in order:
            parts[n]["fn"]()
    torch.cuda.synchronize()
    log("warmup done")

    evs = {n: [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
               for _ in range(args.steps)] for n in order}
    t_start = torch.cuda.Event(enable_timing=True)
    t_end = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t_start.record()
    for s in range(args.steps):
        for n in order:
            a, b = evs[n][s]
            a.record()
            parts[n]["fn"]()
            b.record()
    t_end.record()
    torch.cuda.synchronize()
    total_ms = t_start.elapsed_time(t_end)
    log("timed steps done")

    res = {}
    for n in order:
        ts = sorted(a.elapsed_time(b) for a, b in evs[n])
        avg = sum(ts) / len(ts)
        r = {"avg_ms": round(avg, 5), "median_ms": round(ts[len(ts) // 2], 5),
             "min_ms": round(ts[0], 5)}
        if "flops" in parts[n]:
            r["tflops"] = round(parts[n]["flops"] / (avg * 1e-3) / 1e12, 2)
            r["frac_mfma_peak"] = round(r["tflops"] / PEAK_BF16_TFLOPS, 4)
            if "flops_2x" in parts[n]:
                r["tflops_2x_convention"] = round(parts[n]["flops_2x"] / (avg * 1e-3) / 1e12, 2)
        if "bytes" in parts[n]:
            r["gbs"] = round(parts[n]["bytes"] / (avg * 1e-3) / 1e9, 1)
            r["frac_hbm_peak"] = round(r["gbs"] / PEAK_HBM_GBS, 4)
        res[n] = r
        log(n, r)

    cpu = None
    if not args.no_cpu_baseline and "fwd_c3" in parts:
        import oracle
        workers = min(os.cpu_count() or 1, 16)
        # whole passes of the fp64 oracle over the headline workload (all 32
        # heads, every row) until at least 10 s of host work, at most 8 passes
        passes, dt = 0, 0.0
        while passes < 8 and (passes == 0 or dt < 10.0):
            t0 = time.perf_counter()
            oracle.attention_forward(x["q"], x["k"], x["v"], c3.scale, True, workers=workers)
            dt += time.perf_counter() - t0
            passes += 1
        fl = passes * causal_flops(c3.B, c3.H, c3.N, c3.d)
        cpu = {"value": round(fl / dt / 1e12, 6), "unit": "TFLOP/s", "cores": workers,
               "kind": "oracle",
               "sample": f"fp64 oracle forward over the whole causal B=1 H=32 N=8192 d=128 "
                         f"workload, {passes} pass(es), {dt:.1f} s wall on {workers} threads"}
        log("cpu baseline", cpu)

    head = res.get("fwd_c3")
    src = source_hash("fa_fwd.hip", "fa_device.h")
    roof = None
    if head is not None:
        traffic = load_traffic("fwd_c3", src)
        roof = {"bound": "mfma", "achieved": head["tflops"], "peak": PEAK_BF16_TFLOPS,
                "unit": "TFLOP/s", "frac": head["frac_mfma_peak"], "traffic": traffic,
                "kernel": "fwd_bf16_kernel<128,causal>", "source_hash": src}
    dec = res.get("decode_c5")
    roof_dec = None
    if dec is not None:
        roof_dec = {"bound": "hbm", "achieved": dec["gbs"], "peak": PEAK_HBM_GBS, "unit": "GB/s",
                    "frac": dec["frac_hbm_peak"],
                    "traffic": load_traffic("decode_c5",
                                            source_hash("fa_decode.hip", "fa_device.h")),
                    "kernel": "decode_partial_kernel + decode_merge_kernel"}
    out = {
        "metric": "fwd attention TFLOP/s (causal bf16, % of MFMA dense bf16 peak); "
                  "paged-decode GB/s in parts.decode_c5",
        "value": head["tflops"] if head else None,
        "unit": "TFLOP/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(total_ms / args.steps, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16", "data": "synthetic (seeded N(0,1))",
        "config": {"workload": "causal bf16 attention forward B=1 H=32 N=8192 d=128 "
                               "(one step also runs fwd B=8 H=12 N=1024 d=64, fwd+bwd "
                               "B=4 H=16 N=2048 d=128, paged decode 64x32x128 with 32 and "
                               "with 8 cached heads, a paged KV append, and one "
                               "ring-attention step: offset fwd + merge at 32x8192x128)",
                   "global_batch": 1, "seq_len": 8192, "parallelism": "single-gpu"},
        "roofline": roof,
        "roofline_decode": roof_dec,
        "parts": res,
        "cpu_baseline": cpu,
    }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
