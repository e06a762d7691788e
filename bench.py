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
    8192 queries against the previous 8192-token block, then fa_merge; and the
    same step as one fa_fwd_offset_accumulate call
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

# benchmark parts, named by what they run and their shapes
P_APPEND = "append_s64kv8d128"
P_BWD4 = "bwd_causal_b4h16n2048d128"
P_COPY = "copy_calib"
P_GEMM = "ref_gemm_bf16_m8192n8192k8192"
P_GEMM_ZERO = "ref_gemm_bf16_m8192n8192k8192_zero_inputs"
P_READ = "ref_rowmax_bf16_4gib"
P_DEC = "decode_s64h32d128"
P_DEC_GQA = "decode_gqa_s64h32kv8d128"
P_FWD = "fwd_causal_b1h32n8192d128"
P_FWD16 = "fwd_causal_f16_b1h32n8192d128"
P_FWD_ZERO = "fwd_causal_b1h32n8192d128_zero_inputs"
P_FWD4 = "fwd_causal_b4h16n2048d128"
P_FWD_GPT2 = "fwd_causal_b8h12n1024d64"
P_PREFILL = "prefill_gqa_s8x1024h32kv8d128"
P_RING = "ring_h32n8192d128"
P_RING_FWD = "ring_fwd_h32n8192d128"
P_RING_MERGE = "ring_merge_h32n8192d128"
P_RING_FUSED = "ring_fused_h32n8192d128"


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


def load_trace_time(kernel_key, src_hash):
    """Average kernel duration (us) of a part from the committed rocprofv3
    kernel trace, if that trace was taken from the current sources."""
    p = os.path.join(ROOT, "profiles", "kernel_times.json")
    if not os.path.exists(p):
        return None
    try:
        rec = json.load(open(p)).get(kernel_key)
    except Exception:
        return None
    if not rec or rec.get("source_hash") != src_hash:
        return None
    return rec.get("avg_us")


def host_cpu():
    """The host's CPU model and core counts (logical CPUs, and those this
    process may run on)."""
    model = None
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    try:
        usable = len(os.sched_getaffinity(0))
    except (AttributeError, OSError):
        usable = os.cpu_count() or 1
    return {"model": model, "logical_cpus": os.cpu_count(), "usable_cpus": usable}


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
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--only", default="",
                    help="comma list of parts to run: fwd_causal_b1h32n8192d128, "
                         "fwd_causal_f16_b1h32n8192d128, fwd_causal_b8h12n1024d64, "
                         "fwd_causal_b4h16n2048d128, bwd_causal_b4h16n2048d128, "
                         "decode_s64h32d128, decode_gqa_s64h32kv8d128 (8 cached heads), "
                         "append_s64kv8d128 (paged KV append), prefill_gqa_s8x1024h32kv8d128 "
                         "(chunked prefill over a paged cache), ring_h32n8192d128 (offset "
                         "forward + merge of one ring step, and the fused step), ref_gemm_bf16_m8192n8192k8192 (the "
                         "vendor library's bf16 GEMM on random operands, a reference point), copy_calib (a 1 GiB device copy "
                         "used to scale the HBM-traffic counters); and, to show how the rate depends on the "
                         "operand data, fwd_causal_b1h32n8192d128_zero_inputs and "
                         "ref_gemm_bf16_m8192n8192k8192_zero_inputs (the same work on all-zero inputs); "
                         "ref_rowmax_bf16_4gib (the library's row maximum over 4 GiB of bf16, a plain "
                         "streaming read for comparison with the decode). "
                         "The reference and zero-input parts run only when named here.")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only: --gpus {args.gpus} is not supported "
              "(the kernels run on a single MI355X; no multi-GPU path is built)",
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
    longctx, gpt2 = workloads.LONG_CONTEXT, workloads.GPT2_SHAPE
    fwdbwd, dec = workloads.FWD_BWD, workloads.DECODE
    parts = {}
    if want(P_FWD):
        x = workloads.attention_inputs(longctx.B, longctx.H, longctx.N, longctx.d, "bf16",
                                       seed=longctx.seed)
        q, k, v = (x[n].to(dev) for n in "qkv")
        o = torch.empty_like(q)
        lse = torch.empty(longctx.B, longctx.H, longctx.N, device=dev)
        parts[P_FWD] = dict(fn=lambda: binding.fwd(q, k, v, causal=True, scale=longctx.scale,
                                                   out=o, lse=lse),
                            flops=causal_flops(longctx.B, longctx.H, longctx.N, longctx.d))
    if want(P_FWD16):
        # the headline forward with fp16 inputs (same draws, cast to fp16)
        xh = workloads.attention_inputs(longctx.B, longctx.H, longctx.N, longctx.d, "f16",
                                        seed=longctx.seed)
        qh, kh, vh = (xh[n].to(dev) for n in "qkv")
        oh = torch.empty_like(qh)
        lseh = torch.empty(longctx.B, longctx.H, longctx.N, device=dev)
        parts[P_FWD16] = dict(fn=lambda: binding.fwd(qh, kh, vh, causal=True, scale=longctx.scale,
                                                     out=oh, lse=lseh),
                              flops=causal_flops(longctx.B, longctx.H, longctx.N, longctx.d))
    if want(P_RING):
        # one rank's non-diagonal ring step at the long-context shape: its 8192
        # queries (global rows 8192..16383) against the previous 8192-token
        # key/value block (every key visible), merged into the running result
        xr = x if want(P_FWD) else workloads.attention_inputs(
            longctx.B, longctx.H, longctx.N, longctx.d, "bf16", seed=longctx.seed)
        qr, kr, vr = (xr[n].to(dev) for n in "qkv")
        po = torch.empty_like(qr)
        pl = torch.empty(longctx.B, longctx.H, longctx.N, device=dev)
        acc_o, acc_l = binding.fwd(qr, kr, vr, causal=True, scale=longctx.scale)   # diagonal block
        parts[P_RING_FWD] = dict(fn=lambda: binding.fwd_offset(
            qr, kr, vr, q_offset=longctx.N, k_offset=0, causal=True, scale=longctx.scale, out=po,
            lse=pl),
            flops=4 * longctx.B * longctx.H * longctx.N * longctx.N * longctx.d)
        # the merge reads the partial the offset forward has just written: a
        # 512 MiB fill between the two (outside the timed region) evicts it
        # from the 256 MiB Infinity Cache, so the rate is the HBM rate
        flush = torch.empty(128 << 20, dtype=torch.float32, device=dev)
        parts[P_RING_MERGE] = dict(fn=lambda: binding.merge(acc_o, acc_l, po, pl, out=acc_o,
                                                            lse_out=acc_l),
                                   pre=lambda: flush.fill_(0.5),
                                   bytes=3 * acc_o.numel() * 2 + 3 * acc_l.numel() * 4)
        # the same step in one call: the block's forward merged into the
        # running result in its epilogue (the running result read from HBM,
        # as after the fill)
        fo, fl = acc_o.clone(), acc_l.clone()
        parts[P_RING_FUSED] = dict(fn=lambda: binding.fwd_offset_accumulate(
            qr, kr, vr, fo, fl, q_offset=longctx.N, k_offset=0, causal=True, scale=longctx.scale),
            pre=lambda: flush.fill_(0.5),
            flops=4 * longctx.B * longctx.H * longctx.N * longctx.N * longctx.d)
    if want(P_FWD_GPT2):
        x2 = workloads.attention_inputs(gpt2.B, gpt2.H, gpt2.N, gpt2.d, "bf16", seed=gpt2.seed,
                                        in_scale=gpt2.in_scale)
        q2, k2, v2 = (x2[n].to(dev) for n in "qkv")
        o2 = torch.empty_like(q2)
        lse2 = torch.empty(gpt2.B, gpt2.H, gpt2.N, device=dev)
        parts[P_FWD_GPT2] = dict(fn=lambda: binding.fwd(q2, k2, v2, causal=True, scale=gpt2.scale,
                                                        out=o2, lse=lse2),
                                 flops=causal_flops(gpt2.B, gpt2.H, gpt2.N, gpt2.d))
    if want(P_FWD4) or want(P_BWD4):
        x4 = workloads.attention_inputs(fwdbwd.B, fwdbwd.H, fwdbwd.N, fwdbwd.d, "bf16",
                                        seed=fwdbwd.seed, with_do=True)
        q4, k4, v4, do4 = (x4[n].to(dev) for n in ("q", "k", "v", "do"))
        o4 = torch.empty_like(q4)
        lse4 = torch.empty(fwdbwd.B, fwdbwd.H, fwdbwd.N, device=dev)
        grads = tuple(torch.empty(q4.shape, dtype=torch.float32, device=dev) for _ in range(3))
        ws4 = torch.empty(binding.bwd_workspace_size(fwdbwd.B, fwdbwd.H, fwdbwd.N, fwdbwd.d),
                          dtype=torch.uint8, device=dev)
        f4 = causal_flops(fwdbwd.B, fwdbwd.H, fwdbwd.N, fwdbwd.d)
        parts[P_FWD4] = dict(fn=lambda: binding.fwd(q4, k4, v4, causal=True, scale=fwdbwd.scale,
                                                    out=o4, lse=lse4), flops=f4)
        parts[P_BWD4] = dict(fn=lambda: binding.bwd(q4, k4, v4, o4, do4, lse4, causal=True,
                                                    scale=fwdbwd.scale, workspace=ws4,
                                                    grads=grads),
                             flops=int(2.5 * f4), flops_2x=2 * f4)
    if want(P_DEC):
        p = workloads.paged_inputs(dec.num_seqs, dec.H, dec.d, dec.block_size, dec.min_len,
                                   dec.max_len, seed=dec.seed)
        pd = {kk: (vv.to(dev) if isinstance(vv, torch.Tensor) else vv) for kk, vv in p.items()}
        od = torch.empty_like(pd["q"])
        lsed = torch.empty(dec.num_seqs, dec.H, device=dev)
        wsd = torch.empty(binding.paged_decode_workspace_size(dec.num_seqs, dec.H, dec.d,
                                                              p["max_blocks_per_seq"], 16),
                          dtype=torch.uint8, device=dev)
        tokens = int(p["seq_lens"].long().sum())
        kv_bytes = tokens * dec.H * dec.d * 2 * 2
        parts[P_DEC] = dict(fn=lambda: binding.paged_decode(
            pd["q"], pd["k_pool"], pd["v_pool"], pd["block_table"], pd["seq_lens"], block_size=16,
            scale=dec.scale, workspace=wsd, out=od, lse=lsed), bytes=kv_bytes, tokens=tokens)
    if want(P_DEC_GQA) or want(P_APPEND):
        # the same sequences with 8 cached heads for the 32 query heads, and
        # enough free blocks for every timed append step
        pg = workloads.paged_inputs(dec.num_seqs, dec.H, dec.d, dec.block_size, dec.min_len,
                                    dec.max_len, seed=dec.seed, kv_heads=8,
                                    extra_blocks=4 * dec.num_seqs)
        pgd = {kk: (vv.to(dev) if isinstance(vv, torch.Tensor) else vv) for kk, vv in pg.items()}
        tokens_g = int(pg["seq_lens"].long().sum())
        if want(P_DEC_GQA):
            og = torch.empty_like(pgd["q"])
            lseg = torch.empty(dec.num_seqs, dec.H, device=dev)
            wsg = torch.empty(binding.paged_decode_workspace_size(dec.num_seqs, dec.H, dec.d,
                                                                  pg["max_blocks_per_seq"], 16),
                              dtype=torch.uint8, device=dev)
            parts[P_DEC_GQA] = dict(fn=lambda: binding.paged_decode(
                pgd["q"], pgd["k_pool"], pgd["v_pool"], pgd["block_table"], pgd["seq_lens"],
                block_size=16, scale=dec.scale, workspace=wsg, out=og, lse=lseg),
                bytes=tokens_g * 8 * dec.d * 2 * 2, tokens=tokens_g)
        if want(P_APPEND):
            ga = torch.Generator().manual_seed(dec.seed + 1)
            kn = torch.randn((dec.num_seqs, 8, dec.d), generator=ga).to(torch.bfloat16).to(dev)
            vn = torch.randn((dec.num_seqs, 8, dec.d), generator=ga).to(torch.bfloat16).to(dev)
            fc = torch.tensor([pg["free_count"]], dtype=torch.int32, device=dev)
            nf = torch.zeros(1, dtype=torch.int32, device=dev)
            # lengths and the free stack advance on every call (state of a real decode loop)
            lens_a = pgd["seq_lens"].clone()
            table_a = pgd["block_table"].clone()
            parts[P_APPEND] = dict(fn=lambda: binding.paged_kv_append(
                kn, vn, pgd["k_pool"], pgd["v_pool"], table_a, lens_a, pgd["free_list"], fc, nf,
                block_size=16), bytes=2 * 2 * kn.numel() * 2)
    if want(P_PREFILL):
        # chunked prefill: 8 sequences, a 1024-token chunk each at the end of
        # 1500..4000 cached tokens, 32 query heads on 8 cached heads
        lens_p = [1500, 2048, 2500, 3000, 3333, 3700, 4000, 1024]
        pp = workloads.paged_inputs(len(lens_p), dec.H, dec.d, 16, 1, max(lens_p),
                                    seed=dec.seed + 2, seq_lens=lens_p, kv_heads=8)
        qp = workloads.prefill_queries([1024] * len(lens_p), dec.H, dec.d, seed=dec.seed + 3)
        ppd = {kk: (vv.to(dev) if isinstance(vv, torch.Tensor) else vv) for kk, vv in pp.items()}
        qpd, qsd = qp["q"].to(dev), qp["q_start"].to(dev)
        op = torch.empty_like(qpd)
        lsep = torch.empty(qpd.shape[0], dec.H, device=dev)
        pairs = sum(sum(L - 1024 + r + 1 for r in range(1024)) for L in lens_p)
        parts[P_PREFILL] = dict(fn=lambda: binding.paged_prefill(
            qpd, qsd, ppd["k_pool"], ppd["v_pool"], ppd["block_table"], ppd["seq_lens"],
            block_size=16, max_q_len=1024, scale=dec.scale, out=op, lse=lsep),
            flops=4 * dec.H * dec.d * pairs)
    if P_COPY in only:
        # plain device copy of known size: the HBM-traffic counters of the kernels
        # are scaled by what the same counters read for this copy
        src = torch.empty(256 << 20, dtype=torch.float32, device=dev)      # 1 GiB
        src.fill_(1.0)
        dst = torch.empty_like(src)
        parts[P_COPY] = dict(fn=lambda: dst.copy_(src), bytes=2 * src.numel() * 4)
    if P_GEMM in only:
        # reference point, not the hot path: the vendor library's dense bf16
        # GEMM on N(0,1) operands (torch.mm on contiguous 2-D tensors), whose
        # rate on this data bounds what a matrix-bound kernel can expect
        gen = torch.Generator(device="cpu").manual_seed(70100)
        ga = torch.randn(8192, 8192, generator=gen).to(torch.bfloat16).to(dev)
        gb = torch.randn(8192, 8192, generator=gen).to(torch.bfloat16).to(dev)
        gc = torch.empty(8192, 8192, dtype=torch.bfloat16, device=dev)
        parts[P_GEMM] = dict(fn=lambda: torch.mm(ga, gb, out=gc), flops=2 * 8192 ** 3)
    if P_READ in only:
        # reference point, not the hot path: a plain streaming read by the
        # vendor library (torch.amax over rows of a 4 GiB bf16 tensor)
        rx = torch.ones(1 << 31, dtype=torch.bfloat16, device=dev).view(-1, 4096)
        parts[P_READ] = dict(fn=lambda: torch.amax(rx, dim=1), bytes=rx.numel() * 2)
    if P_GEMM_ZERO in only:
        za = torch.zeros(8192, 8192, dtype=torch.bfloat16, device=dev)
        zb = torch.zeros_like(za)
        zc = torch.empty_like(za)
        parts[P_GEMM_ZERO] = dict(fn=lambda: torch.mm(za, zb, out=zc), flops=2 * 8192 ** 3)
    if P_FWD_ZERO in only:
        # the headline forward's instructions on all-zero Q, K, V: matrix
        # operands that never toggle draw less power, so the clock runs higher
        zq = torch.zeros(longctx.B, longctx.H, longctx.N, longctx.d, dtype=torch.bfloat16,
                         device=dev)
        zk, zv, zo = torch.zeros_like(zq), torch.zeros_like(zq), torch.empty_like(zq)
        zl = torch.empty(longctx.B, longctx.H, longctx.N, device=dev)
        parts[P_FWD_ZERO] = dict(fn=lambda: binding.fwd(zq, zk, zv, causal=True,
                                                        scale=longctx.scale, out=zo, lse=zl),
                                 flops=causal_flops(longctx.B, longctx.H, longctx.N, longctx.d))
    torch.cuda.synchronize()
    log(f"inputs ready: {list(parts)}")

    order = [n for n in (P_FWD, P_FWD16, P_FWD_GPT2, P_FWD4, P_BWD4, P_DEC, P_DEC_GQA, P_APPEND,
                         P_PREFILL, P_RING_FWD, P_RING_MERGE, P_RING_FUSED, P_COPY, P_GEMM,
                         P_FWD_ZERO, P_GEMM_ZERO, P_READ)
             if n in parts]
    for _ in range(args.warmup):
        for n in order:
            if "pre" in parts[n]:
                parts[n]["pre"]()
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
            if "pre" in parts[n]:
                parts[n]["pre"]()
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
    if not args.no_cpu_baseline and P_FWD in parts:
        import oracle
        hc = host_cpu()
        # one worker thread per usable core, at most 16 (one GPU's share of the
        # host on the machines this runs on)
        workers = max(1, min(hc["usable_cpus"], 16))
        # whole passes of the fp64 oracle over the headline workload (all 32
        # heads, every row) until at least 10 s of host work, at most 8 passes
        passes, dt = 0, 0.0
        while passes < 8 and (passes == 0 or dt < 10.0):
            t0 = time.perf_counter()
            oracle.attention_forward(x["q"], x["k"], x["v"], longctx.scale, True, workers=workers)
            dt += time.perf_counter() - t0
            passes += 1
        fl = passes * causal_flops(longctx.B, longctx.H, longctx.N, longctx.d)
        cpu = {"value": round(fl / dt / 1e12, 6), "unit": "TFLOP/s", "cores": workers,
               "kind": "oracle", "host_cpu_model": hc["model"],
               "host_logical_cpus": hc["logical_cpus"], "host_usable_cpus": hc["usable_cpus"],
               "sample": f"fp64 oracle forward over the whole causal B=1 H=32 N=8192 d=128 "
                         f"workload, {passes} pass(es), {dt:.1f} s wall on {workers} threads"}
        log("cpu baseline", cpu)

    head = res.get(P_FWD)
    src = source_hash("fa_fwd.hip", "fa_device.h")
    roof = None
    if head is not None:
        traffic = load_traffic(P_FWD, src)
        roof = {"bound": "mfma", "achieved": head["tflops"], "peak": PEAK_BF16_TFLOPS,
                "unit": "TFLOP/s", "frac": head["frac_mfma_peak"], "traffic": traffic,
                "kernel": "fwd_bf16_kernel<d=128, causal, 8 waves, paired tiles>",
                "source_hash": src}
        # the same fraction from the committed rocprofv3 trace's average
        # duration of this kernel (null once the sources have changed)
        t_us = load_trace_time(P_FWD, src)
        if t_us:
            fl = parts[P_FWD]["flops"]
            roof["trace_avg_us"] = t_us
            roof["frac_from_trace"] = round(fl / (t_us * 1e-6) / 1e12 / PEAK_BF16_TFLOPS, 4)
    dec_res = res.get(P_DEC)
    roof_dec = None
    if dec_res is not None:
        roof_dec = {"bound": "hbm", "achieved": dec_res["gbs"], "peak": PEAK_HBM_GBS, "unit": "GB/s",
                    "frac": dec_res["frac_hbm_peak"],
                    "traffic": load_traffic(P_DEC,
                                            source_hash("fa_decode.hip", "fa_device.h")),
                    "kernel": "decode_partial_kernel + decode_merge_kernel"}
    out = {
        "metric": "fwd attention TFLOP/s & %MFMA peak; paged-decode GB/s & %HBM peak",
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
                               "ring-attention step: offset fwd + merge, and fused, at "
                               "32x8192x128)",
                   "global_batch": 1, "seq_len": 8192, "parallelism": "single-gpu"},
        "roofline": roof,
        "roofline_decode": roof_dec,
        "parts": res,
        "cpu_baseline": cpu,
    }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
