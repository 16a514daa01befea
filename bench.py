#!/usr/bin/env python3
"""Benchmark of the one-GPU join-agg path on MI355X.

A step is one pass of the LLaMA-shaped block (batch 4, seq 2048, d 4096, 32
heads of 128, ffn 11008, bf16) through libja: RMSNorm, the 2x2x2 QKV
contraction join-agg, the tokens->heads repartition, causal attention with
the online-softmax aggregation, heads->tokens, the output projection with the
residual add applied to its aggregated blocks, RMSNorm, the gate-and-up
contraction with SwiGLU applied to its aggregated blocks, and the down
contraction with the second residual add (`--workload block_unfused`: the
adds and SwiGLU as launches of their own).  Inputs are seeded synthetic
tensors already resident in HBM in the blockings the operators need.

Prints one JSON line.  `value` is the block's join-agg throughput (all
contraction and attention flops of a step / step time).  `roofline` is for
the dominant kernel (the bf16 MFMA contraction), timed with HIP events on
the stream the steps run on.  `cpu_baseline` times the CPU oracle on a
bounded token sample of the same block.

    python bench.py [--steps K] [--warmup W] [--workload block|block_unfused|configs|ffn|attention|norm_swiglu|copy]

The non-block workloads print per-operator diagnostics (and `copy` the HBM
copy ceiling); only `block` prints the contract line.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "join-agg TFLOP/s & % MFMA peak; LLaMA-7B-shape block ms, 1 MI355X"
PEAK_BF16_TFLOPS = 2516.6  # 256 CUs x 2.4 GHz x 4096 dense bf16 flop/clk/CU
PEAK_HBM_GBS = 8000.0


def _eq(n, q):
    base, extra = divmod(n, q)
    p = [0]
    for i in range(q):
        p.append(p[-1] + base + (i < extra))
    return p


def _bits_to_dev(bits, dtype: str = "bf16"):
    import numpy as np
    import torch

    t = torch.from_numpy(np.ascontiguousarray(bits).view(np.int16).ravel())
    return t.view(torch.float16 if dtype == "f16" else torch.bfloat16).cuda()


def _stats(ms_list):
    """mean, median, min, max and the half-width of a 95% confidence interval
    of the mean (normal approximation) of per-iteration times."""
    import numpy as np

    a = np.asarray(ms_list, dtype=np.float64)
    half = 1.96 * a.std(ddof=1) / np.sqrt(len(a)) if len(a) > 1 else 0.0
    return {"mean": round(float(a.mean()), 4), "median": round(float(np.median(a)), 4),
            "min": round(float(a.min()), 4), "max": round(float(a.max()), 4), "ci95": round(float(half), 4),
            "n": int(len(a))}


def _timed(launch, steps, flush=None):
    """Per-iteration times (ms) of `launch`, each between its own event pair
    on the current stream; `flush` (not timed) runs before every iteration."""
    import torch

    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
    for e0, e1 in evs:
        if flush is not None:
            flush()
        e0.record()
        launch()
        e1.record()
    torch.cuda.synchronize()
    return [e0.elapsed_time(e1) for e0, e1 in evs]


_SNAPSHOT = None


def _device_snapshot():
    """Clock and power lines of rocm-smi, read once by a child process before
    this process touches the GPU."""
    global _SNAPSHOT
    if _SNAPSHOT is not None:
        return _SNAPSHOT or None
    import subprocess

    try:
        out = subprocess.run(["rocm-smi", "--showclocks", "--showpower"], capture_output=True, text=True,
                             timeout=30).stdout
    except (OSError, subprocess.SubprocessError):
        return None
    keep = [ln.strip() for ln in out.splitlines() if "sclk" in ln or "mclk" in ln or "Power" in ln]
    _SNAPSHOT = keep[:8]
    return _SNAPSHOT or None


def _mean_ms(pairs):
    return sum(s.elapsed_time(e) for s, e in pairs) / max(1, len(pairs))


def cpu_baseline_block(inp, batch, seq, dm, heads, ffn, target_s=12.0, fused=True):
    """Time the oracle (as it stands) on the first n tokens of batch 0 of the
    same block (its fused or unfused rounding points); n is grown (at most
    16x per probe) until one run takes about target_s seconds."""
    import numpy as np

    import oracle

    f = {k: oracle.bf16_to_f64(v) for k, v in inp.items()}
    hd = dm // heads

    def flops(n):
        # the GPU value's convention: attention counted over the kept
        # (query block, key block) tuples of 128-blocks, so token s is
        # charged for the (s // 128 + 1) * 128 keys of its kept blocks
        per_tok = 2.0 * (dm * 3 * dm + dm * dm + 3 * dm * ffn)
        att = sum(2 * 2.0 * (s // 128 + 1) * 128 * hd * heads for s in range(n))
        return n * per_tok + att

    n, dt = 8, 0.0
    while True:
        toks = list(range(n))
        t0 = time.perf_counter()
        oracle.llama_block_tokens(f["x"], f["g1"], f["w_qkv"], f["w_o"], f["g2"], f["w_gate"], f["w_up"],
                                  f["w_down"], batch, seq, heads, toks, fused=fused)
        dt = time.perf_counter() - t0
        if dt >= target_s * 0.7 or n >= seq:
            break
        n = min(seq, 16 * n, max(n * 2, int(n * target_s / max(dt, 1e-3))))
    return {"value": flops(n) / dt / 1e12, "unit": "TFLOP/s", "cores": oracle.num_threads(), "kind": "oracle",
            "cpu": _cpu_model(),
            "sample": "float64 oracle block forward on tokens 0..%d of batch 0 (%.1f GFLOP counted as the GPU value "
                      "counts them, over kept 128-block tuples; %.2f s)" % (n - 1, flops(n) / 1e9, dt)}


def _cpu_model():
    try:
        for ln in open("/proc/cpuinfo"):
            if ln.startswith("model name"):
                return ln.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def _gemm_traffic():
    """HBM-side bytes per contraction launch from the committed counter record
    (FETCH_SIZE and WRITE_SIZE, scaled by a plain copy's readings), or None
    when the kernel's sources changed since the counters were taken."""
    import hashlib

    path = os.path.join(ROOT, "profiles", "gemm_bf16_block_traffic.json")
    try:
        rec = json.load(open(path))
        h = hashlib.sha256()
        for f in rec["sources"]:
            h.update(open(os.path.join(ROOT, f), "rb").read())
    except (OSError, ValueError, KeyError):
        return None
    if h.hexdigest() != rec["sources_sha256"]:
        return None
    return rec["read_bytes_per_launch"] + rec["write_bytes_per_launch"]


# the measured block (LLaMA-7B-shaped, multi-head attention) and the pages'
# own LLaMA-3-8B-like block (grouped-query attention, 32 query over 8
# key-value heads, FFN 14,336) at 8 sequences of 1,024 tokens
BLOCKS = {
    "block": dict(name="llama7b_shaped_block", batch=4, seq=2048, dm=4096, heads=32, kv_heads=32, ffn=11008),
    "block_gqa": dict(name="llama3_8b_shaped_block_gqa", batch=8, seq=1024, dm=4096, heads=32, kv_heads=8,
                      ffn=14336),
    # the same blocks in IEEE half (the pages run their blocks in FP16), and the pages' single-sequence
    # workloads of the LLaMA-3-8B-like block: 1,024 and 8,192 tokens
    "block_f16": dict(name="llama7b_shaped_block_f16", batch=4, seq=2048, dm=4096, heads=32, kv_heads=32,
                      ffn=11008, dtype="f16"),
    "block_gqa_f16": dict(name="llama3_8b_shaped_block_gqa_f16", batch=8, seq=1024, dm=4096, heads=32, kv_heads=8,
                          ffn=14336, dtype="f16"),
    "block_gqa_1k_f16": dict(name="llama3_8b_shaped_block_gqa_1x1024_f16", batch=1, seq=1024, dm=4096, heads=32,
                             kv_heads=8, ffn=14336, dtype="f16"),
    "block_gqa_8k_f16": dict(name="llama3_8b_shaped_block_gqa_1x8192_f16", batch=1, seq=8192, dm=4096, heads=32,
                             kv_heads=8, ffn=14336, dtype="f16"),
}
# each block also runs with the residual adds and SwiGLU as separate 1:1
# join launches (every projection written) instead of fused into the
# contractions that produce their inputs
BLOCKS.update({k + "_unfused": dict(v, fused=False) for k, v in list(BLOCKS.items())})
# the LLaMA-7B-shaped block with attention on head-major relations: the two
# re-indexing repartitions (tokens -> heads, heads -> tokens) around it
BLOCKS["block_heads"] = dict(BLOCKS["block"], name="llama7b_shaped_block_head_major", layout="heads")


def bench_block(args):
    import torch

    from tensor_relational_join_amd import synth
    from tensor_relational_join_amd.block import LlamaBlock
    from tensor_relational_join_amd.device import alloc

    from tensor_relational_join_amd.binding import JA_BF16, JA_F16

    cfg = BLOCKS[args.workload]
    batch, seq, dm, heads, kv, ffn = (cfg[k] for k in ("batch", "seq", "dm", "heads", "kv_heads", "ffn"))
    fused = cfg.get("fused", True)
    dt = cfg.get("dtype", "bf16")
    blk = LlamaBlock(batch, seq, dm, heads, ffn, kv_heads=kv, fused=fused, dtype=JA_F16 if dt == "f16" else JA_BF16,
                     layout=cfg.get("layout", "tokens"))
    GEMMS = blk.gemms
    inp = synth.llama_block_inputs(5, batch, seq, dm, ffn, qkv_cols=blk.qkv_cols, dtype=dt)
    x = blk.materialize(_bits_to_dev(inp["x"], dt), blk.x_rel)
    w = {k: blk.materialize(_bits_to_dev(inp[k], dt), rel) for k, rel in blk.w_rel.items()}
    w["g1"] = blk.materialize(_bits_to_dev(inp["g1"], dt), blk.g_rel)
    w["g2"] = blk.materialize(_bits_to_dev(inp["g2"], dt), blk.ops["norm2"].in_rels[1])
    y = alloc(blk.y_rel)
    flops = blk.flops()
    total_flops = sum(flops.values())

    for _ in range(args.warmup):
        blk.forward(x, w, y)
    torch.cuda.synchronize()
    # timed region 1: K steps back to back, one event pair around all of them
    s0, s1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    s0.record()
    for _ in range(args.steps):
        blk.forward(x, w, y)
    s1.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms = s0.elapsed_time(s1) / args.steps
    # per-step distribution: the same K steps, an event pair around each
    step_stats = _stats(_timed(lambda: blk.forward(x, w, y), args.steps))
    # timed region 2: the same K steps with an event pair around every step of the path
    ev = {}
    torch.cuda.synchronize()
    for _ in range(args.steps):
        blk.forward(x, w, y, events=ev)
    torch.cuda.synchronize()
    step_ms = {k: _mean_ms(v) for k, v in ev.items()}
    gemm_ms = sum(step_ms[k] for k in GEMMS)
    gemm_flops = sum(flops[k] for k in GEMMS)
    achieved = gemm_flops / len(GEMMS) / (gemm_ms / len(GEMMS) / 1e3) / 1e12
    nbytes = blk.step_bytes()
    parts = {}
    for k in step_ms:
        d = {"ms": round(step_ms[k], 4)}
        if k in flops:
            d["tflops"] = round(flops[k] / (step_ms[k] / 1e3) / 1e12, 1)
            d["frac_mfma_peak"] = round(d["tflops"] / PEAK_BF16_TFLOPS, 3)
        if k in nbytes:
            d["gbs"] = round(nbytes[k] / (step_ms[k] / 1e3) / 1e9, 1)
            d["frac_hbm_peak"] = round(d["gbs"] / PEAK_HBM_GBS, 3)
        parts[k] = d
    value = total_flops / (ms / 1e3) / 1e12
    out = {
        "metric": METRIC, "value": round(value, 2), "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms, 4), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": dt, "data": "synthetic",
        "config": {"workload": cfg["name"], "batch": batch, "seq_len": seq, "d_model": dm,
                   "heads": heads, "kv_heads": kv, "head_dim": 128, "ffn": ffn, "parallelism": "single GPU",
                   "adds_and_swiglu": "fused into the contractions" if fused else "separate launches",
                   "attention_layout": ("token-major (no repartition)" if blk.layout == "tokens"
                                        else "head-major (repartitions around attention)")},
        "frac_mfma_peak": round(value / PEAK_BF16_TFLOPS, 4),
        "block_gflop": round(total_flops / 1e9, 1),
        "wall_ms_per_step": round(wall / args.steps * 1e3, 4),
        "step_ms": step_stats,
        "roofline": {"kernel": "gemm_bf16_dma_kernel (contraction join-agg, fused SUM%s)" %
                               (" and 1:1-join epilogues" if fused else ""), "bound": "mfma",
                     "achieved": round(achieved, 1), "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(achieved / PEAK_BF16_TFLOPS, 4), "traffic": _gemm_traffic(),
                     "traffic_unit": "bytes per launch (L2 memory side, rocprofv3 FETCH_SIZE + WRITE_SIZE)",
                     "launches_per_step": len(GEMMS), "gflop_per_launch": round(gemm_flops / len(GEMMS) / 1e9, 1),
                     "avg_launch_ms": round(gemm_ms / len(GEMMS), 4)},
        "parts": parts,
    }
    blk.close()
    return out, inp


def bench_kernel(args):
    """Single-operator workloads at the configs' sizes (diagnostics and
    profiling): tiny = ij,jk->ik 64^3 fp32 (2x2x2); ffn = bd,df->bf
    2048x4096x11008 (2x4x4), fused and unfused (ja_kernel then ja_agg);
    attention = [4,32,2048,128] causal, 128-blocks; norm_swiglu = RMSNorm
    [8192,4096] (d by 8) + SwiGLU [8192,11008] (f by 8); configs = all of
    them; gqa = grouped-query causal attention, 32 query heads over 8
    key-value heads, head_dim 128, one 8,192-token sequence, 8 x 1,024
    tokens and one 131,072-token sequence.  Inputs are seeded torch draws with the configs' distributions."""
    import torch

    from tensor_relational_join_amd import synth
    from tensor_relational_join_amd.device import Op, alloc

    if args.workload == "copy":
        # the library's own streaming copy of 1 GiB: the calibration point of
        # the FETCH_SIZE / WRITE_SIZE counters (bytes known exactly)
        from tensor_relational_join_amd import binding as B

        n = 1 << 30
        src = torch.empty(n // 2, dtype=torch.int16, device="cuda").random_()
        dst = torch.empty_like(src)
        stream = torch.cuda.current_stream().cuda_stream
        for _ in range(args.warmup):
            B.ja_calibrate_copy(src.data_ptr(), dst.data_ptr(), n, stream)
        torch.cuda.synchronize()
        s0, s1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        s0.record()
        for _ in range(args.steps):
            B.ja_calibrate_copy(src.data_ptr(), dst.data_ptr(), n, stream)
        s1.record()
        torch.cuda.synchronize()
        ms = s0.elapsed_time(s1) / args.steps
        gbs = 2.0 * n / (ms / 1e3) / 1e9
        return {"workload": "copy", "kernel": "ja::copy_kernel", "bytes_read": n, "bytes_written": n,
                "steps": args.steps, "ms": round(ms, 4), "gbs": round(gbs, 1),
                "frac_hbm_peak": round(gbs / PEAK_HBM_GBS, 3)}
    runs = []  # (name, launch, flops, bytes, ops to close)
    want = ["tiny", "ffn", "ffn_unfused", "attention", "rmsnorm", "swiglu", "repart"] if args.workload == "configs" else \
        {"ffn": ["ffn"], "attention": ["attention"], "norm_swiglu": ["rmsnorm", "swiglu"],
         "gqa": ["gqa_8k", "gqa_8x1k", "gqa_128k"], "f16": ["ffn_f16", "attention_f16"]}[args.workload]

    def tensors(op, seed, stds):
        torch.manual_seed(seed)
        ins = [alloc(r) for r in op.in_rels]
        for t, (mean, std) in zip(ins, stds):
            t.normal_(mean, std)
        return ins, alloc(op.out_rel)

    from tensor_relational_join_amd.binding import JA_F32

    if "tiny" in want:  # ij,jk->ik 64^3 fp32 U[-1, 1], every letter split in 2: 8 tuples, 4 segments
        sp = {c: _eq(64, 2) for c in "ijk"}
        op = Op("ij,jk->ik", "contract", sp, in_dtypes=[JA_F32, JA_F32], out_dtype=JA_F32)
        torch.manual_seed(1)
        ins = [alloc(r).uniform_(-1, 1) for r in op.in_rels]
        out = alloc(op.out_rel)
        runs.append(("tiny_fp32_2x2x2", lambda op=op, ins=ins, out=out: op.run(ins, out), 2.0 * 64 ** 3,
                     4.0 * 3 * 64 * 64, [op]))
    if "ffn" in want or "ffn_unfused" in want:  # bd,df->bf 2048x4096x11008, b by 2, d by 4, f by 4
        sp = {"b": _eq(2048, 2), "d": _eq(4096, 4), "f": _eq(11008, 4)}
        op = Op("bd,df->bf", "contract", sp)
        ins, out = tensors(op, 2, [(0.0, 1.0), (0.0, 0.02)])
        fl = 2.0 * 2048 * 4096 * 11008
        by = 2.0 * (2048 * 4096 + 4096 * 11008 + 2048 * 11008)
        if "ffn" in want:  # the op is closed after its last use
            runs.append(("ffn_contract", lambda op=op, ins=ins, out=out: op.run(ins, out), fl, by,
                         [] if "ffn_unfused" in want else [op]))
        if "ffn_unfused" in want:
            part = op.partial_buffer()

            def unfused(op=op, ins=ins, out=out, part=part):
                op.kernel(ins, part)
                op.agg(part, out)
            # the unfused path also writes and reads every fp32 partial (32 blocks of 1024 x 2752)
            runs.append(("ffn_unfused_kernel_then_agg", unfused, fl, by + 2 * 4.0 * part.numel(), [op]))
    if "ffn_f16" in want:  # the FFN contraction with IEEE half relations (fp32 accumulation)
        from tensor_relational_join_amd.binding import JA_F16

        sp = {"b": _eq(2048, 2), "d": _eq(4096, 4), "f": _eq(11008, 4)}
        op = Op("bd,df->bf", "contract", sp, in_dtypes=[JA_F16, JA_F16], out_dtype=JA_F16)
        ins, out = tensors(op, 2, [(0.0, 1.0), (0.0, 0.02)])
        runs.append(("ffn_contract_f16", lambda op=op, ins=ins, out=out: op.run(ins, out),
                     2.0 * 2048 * 4096 * 11008, 2.0 * (2048 * 4096 + 4096 * 11008 + 2048 * 11008), [op]))
    if "attention_f16" in want:  # [4, 32, 2048, 128] causal, 128-blocks, IEEE half Q, K, V, O
        from tensor_relational_join_amd.binding import JA_F16

        sp = {"b": _eq(4, 4), "h": _eq(32, 32), "s": _eq(2048, 16), "t": _eq(2048, 16), "d": [0, 128]}
        op = Op("bhsd,bhtd,bhtd->bhsd", "attention", sp, "causal=s,t", in_dtypes=[JA_F16] * 3, out_dtype=JA_F16)
        ins, out = tensors(op, 3, [(0.0, 1.0)] * 3)
        runs.append(("attention_f16", lambda op=op, ins=ins, out=out: op.run(ins, out),
                     2 * 2.0 * 128 * 128 * 128 * 136 * 128, 2.0 * 4 * 4 * 32 * 2048 * 128, [op]))
    if "attention" in want:  # [4, 32, 2048, 128] causal, 128-blocks: 17,408 tuples
        sp = {"b": _eq(4, 4), "h": _eq(32, 32), "s": _eq(2048, 16), "t": _eq(2048, 16), "d": [0, 128]}
        op = Op("bhsd,bhtd,bhtd->bhsd", "attention", sp, "causal=s,t")
        ins, out = tensors(op, 3, [(0.0, 1.0)] * 3)
        runs.append(("attention", lambda op=op, ins=ins, out=out: op.run(ins, out),
                     2 * 2.0 * 128 * 128 * 128 * 136 * 128, 2.0 * 4 * 4 * 32 * 2048 * 128, [op]))
    for name, nb, seq in (("gqa_8k", 1, 8192), ("gqa_8x1k", 8, 1024), ("gqa_128k", 1, 131072)):
        if name not in want:
            continue
        # grouped-query causal attention, 32 query heads over 8 key-value heads (4 per group),
        # head_dim 128, 128-blocks on s and t: Q, O [nb, 8, 4, seq, 128], K, V [nb, 8, seq, 128]
        nblk = seq // 128
        sp = {"b": _eq(nb, nb), "g": _eq(8, 8), "r": [0, 4], "s": _eq(seq, nblk), "t": _eq(seq, nblk), "d": [0, 128]}
        op = Op("bgrsd,bgtd,bgtd->bgrsd", "attention", sp, "causal=s,t")
        ins, out = tensors(op, 5, [(0.0, 1.0)] * 3)
        fl = 2 * 2.0 * 128 ** 3 * (nblk * (nblk + 1) // 2) * 32 * nb
        by = 2.0 * (2 * nb * 32 * seq * 128 + 2 * nb * 8 * seq * 128)
        runs.append((name, lambda op=op, ins=ins, out=out: op.run(ins, out), fl, by, [op]))
    if "rmsnorm" in want:  # x [8192, 4096], d by 8, eps 1e-6, gain N(1, 0.1)
        op = Op("rd,d->rd", "rmsnorm", {"r": [0, 8192], "d": _eq(4096, 8)}, "eps=1e-6")
        ins, out = tensors(op, 4, [(0.0, 1.0), (1.0, 0.1)])
        runs.append(("rmsnorm", lambda op=op, ins=ins, out=out: op.run(ins, out), None,
                     2.0 * (2 * 8192 * 4096 + 4096), [op]))
    if "swiglu" in want:  # g, u [8192, 11008], f by 8, 1:1 join
        op = Op("rf,rf->rf", "swiglu", {"r": [0, 8192], "f": _eq(11008, 8)})
        ins, out = tensors(op, 4, [(0.0, 1.0)] * 2)
        runs.append(("swiglu", lambda op=op, ins=ins, out=out: op.run(ins, out), None, 2.0 * 3 * 8192 * 11008,
                     [op]))
    if "repart" in want:
        # the LLaMA-7B-shaped block's re-indexing repartitions around head-major attention: the QKV projection's
        # output [8192, 12288] in 2 x 2 blocks viewed as [3, 4, 32, 2048, 128] in 128-row head blocks (402.7 MB
        # moved), and attention's output back to [8192, 4096] in 2 x 2 blocks (134.2 MB)
        from tensor_relational_join_amd import binding as B
        from tensor_relational_join_amd.device import Repart

        for name, src, dst, view in (
                ("repart_to_heads", B.Relation((8192, 12288), nblk=(2, 2), dtype=B.JA_BF16),
                 B.Relation((3, 4, 32, 2048, 128), nblk=(3, 4, 32, 16, 1), dtype=B.JA_BF16),
                 B.make_view((4, 2048, 3, 32, 128), (2, 0, 3, 1, 4))),
                ("repart_to_tokens", B.Relation((4, 32, 2048, 128), nblk=(4, 32, 16, 1), dtype=B.JA_BF16),
                 B.Relation((8192, 4096), nblk=(2, 2), dtype=B.JA_BF16),
                 B.make_view((4, 32, 2048, 128), (0, 2, 1, 3)))):
            rp = Repart(src, dst, view)
            torch.manual_seed(6)
            a, b = alloc(src).normal_(0.0, 1.0), alloc(dst)
            runs.append((name, lambda rp=rp, a=a, b=b: rp.run(a, b), None, 2.0 * 2 * a.numel(), [rp]))
    res = {}
    # cold runs: reading 512 MiB between iterations evicts the 256 MB Infinity
    # Cache (a read leaves clean lines, so the timed kernel writes nothing back)
    scratch = torch.ones(1 << 28, dtype=torch.int16, device="cuda")
    for name, launch, fl, by, ops in runs:
        for _ in range(args.warmup):
            launch()
        torch.cuda.synchronize()
        s0, s1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        s0.record()
        for _ in range(args.steps):
            launch()
        s1.record()
        torch.cuda.synchronize()
        ms = s0.elapsed_time(s1) / args.steps
        # at least 100 timed iterations where a kernel is short, about 2 s of timing otherwise
        nstep = max(args.steps, min(100, int(2000.0 / max(ms, 1e-3))))
        d = {"ms": round(ms, 4), "warm": _stats(_timed(launch, nstep)),
             "cold": _stats(_timed(launch, min(nstep, 30), flush=lambda: scratch.max()))}
        if fl:
            d["tflops"] = round(fl / (ms / 1e3) / 1e12, 2)
            d["frac_mfma_peak"] = round(d["tflops"] / PEAK_BF16_TFLOPS, 3)
        if by:
            d["gbs"] = round(by / (ms / 1e3) / 1e9, 1)
            d["frac_hbm_peak"] = round(d["gbs"] / PEAK_HBM_GBS, 3)
            d["cold_gbs"] = round(by / (d["cold"]["median"] / 1e3) / 1e9, 1)
        if fl:
            d["cold_tflops"] = round(fl / (d["cold"]["median"] / 1e3) / 1e12, 2)
        res[name] = d
        for op in ops:
            op.close()
    if args.workload == "configs" and not args.no_cpu_baseline:
        for name, cpu in _cpu_configs().items():
            if name in res:
                res[name]["cpu_oracle"] = cpu
    del scratch
    return {"workload": args.workload, "steps": args.steps, "warmup": args.warmup, "device": _device_snapshot(),
            "results": res}


def _cpu_configs():
    """The float64 oracle (as it stands) on the configs' own inputs, timed on
    the host cores beside the GPU runs: cfg1 median of 5 runs, cfg2 one run
    of the full contraction, cfg3 the full causal attention, cfg4 one run
    each."""
    import numpy as np

    import oracle

    rng = np.random.default_rng(0)
    out = {}

    def timed(fn, reps=1):
        ts = []
        for _ in range(reps):
            t0 = time.perf_counter()
            fn()
            ts.append(time.perf_counter() - t0)
        return float(np.median(ts)) * 1e3

    a, b = rng.uniform(-1, 1, (64, 64)), rng.uniform(-1, 1, (64, 64))
    out["tiny_fp32_2x2x2"] = timed(lambda: oracle.matmul(a, b), 5)
    x, wt = rng.standard_normal((2048, 4096)), rng.standard_normal((4096, 11008)) * 0.02
    out["ffn_contract"] = timed(lambda: oracle.matmul(x, wt))
    q = [rng.standard_normal((4, 32, 2048, 128)) for _ in range(3)]
    out["attention"] = timed(lambda: oracle.attention(q[0], q[1], q[2], 1.0 / np.sqrt(128.0), True))
    xr, gn = rng.standard_normal((8192, 4096)), rng.normal(1.0, 0.1, 4096)
    out["rmsnorm"] = timed(lambda: oracle.rmsnorm(xr, gn, 1e-6))
    g, u = rng.standard_normal((8192, 11008)), rng.standard_normal((8192, 11008))
    out["swiglu"] = timed(lambda: oracle.swiglu(g, u))
    threads = oracle.num_threads()
    return {k: {"ms": round(v, 2), "cores": threads, "kind": "oracle"} for k, v in out.items()}


def _copy_ceiling(nbytes_moved, steps, cold=True):
    """The library's own streaming copy (ja_calibrate_copy) moving
    `nbytes_moved` bytes per launch (half read, half written), timed per
    launch on the current stream; cold: each launch after a 512 MiB read that
    evicts the 256 MB Infinity Cache."""
    import torch

    from tensor_relational_join_amd import binding as B

    n = nbytes_moved // 2 // 16 * 16
    src = torch.empty(n // 2, dtype=torch.int16, device="cuda").random_()
    dst = torch.empty_like(src)
    stream = torch.cuda.current_stream().cuda_stream
    launch = lambda: B.ja_calibrate_copy(src.data_ptr(), dst.data_ptr(), n, stream)  # noqa: E731
    for _ in range(3):
        launch()
    torch.cuda.synchronize()
    assert torch.equal(src, dst)
    scratch = torch.ones(1 << 28, dtype=torch.int16, device="cuda") if cold else None
    st = _stats(_timed(launch, steps, flush=(lambda: scratch.max()) if cold else None))
    gbs = 2 * n / (st["median"] / 1e3) / 1e9
    return {"bytes_moved": 2 * n, "ms": st, "gbs": round(gbs, 1), "frac_hbm_peak": round(gbs / PEAK_HBM_GBS, 3)}


def bench_ceilings(args):
    """The two ceilings the kernels are compared against beside the published
    peaks: the library's own streaming copy (HBM; at 2 GiB moved and at the
    byte counts of the RMSNorm and SwiGLU configs, cold and warm) and a loop
    of nothing but bf16 MFMAs (matrix cores, no memory traffic), each timed
    per launch."""
    import torch

    from tensor_relational_join_amd import binding as B

    copies = {}
    for name, nb in (("2GiB", 1 << 31), ("rmsnorm_bytes", 2 * (2 * 8192 * 4096 + 4096)),
                     ("swiglu_bytes", 2 * 3 * 8192 * 11008)):
        copies[name + "_cold"] = _copy_ceiling(nb, max(args.steps, 30), cold=True)
        copies[name + "_warm"] = _copy_ceiling(nb, max(args.steps, 30), cold=False)
    wgs, iters = 256 * 8, 4096
    sink = torch.empty(wgs * 256, dtype=torch.float32, device="cuda")
    stream = torch.cuda.current_stream().cuda_stream
    fl = B.ja_calibrate_mfma(wgs, iters, sink.data_ptr(), stream)
    for _ in range(args.warmup):
        B.ja_calibrate_mfma(wgs, iters, sink.data_ptr(), stream)
    mf = _stats(_timed(lambda: B.ja_calibrate_mfma(wgs, iters, sink.data_ptr(), stream), args.steps))
    mfma_tflops = fl / (mf["median"] / 1e3) / 1e12
    return {"workload": "ceilings", "steps": args.steps, "warmup": args.warmup, "device": _device_snapshot(),
            "copy": copies,
            "mfma_loop": {"flops": fl, "ms": mf, "tflops": round(mfma_tflops, 1),
                          "frac_mfma_peak": round(mfma_tflops / PEAK_BF16_TFLOPS, 3),
                          "implied_clock_ghz": round(mfma_tflops / PEAK_BF16_TFLOPS * 2.4, 3)}}


def configs_summary(args):
    """The single-operator configurations measured in the default run, one
    compact entry each: back-to-back, warm-median and cold-median ms, the rate
    (TFLOP/s for the contractions and attention, GB/s for the memory-bound
    operators) of the cold median and its fraction of the published peak, and
    the float64 oracle's time on the host cores beside it."""
    cfg = argparse.Namespace(workload="configs", steps=20, warmup=3, no_cpu_baseline=args.no_cpu_baseline)
    res = bench_kernel(cfg)["results"]
    names = {"tiny_fp32_2x2x2": "cfg1 ij,jk->ik 64^3 fp32 2x2x2",
             "ffn_contract": "cfg2 bd,df->bf 2048x4096x11008 bf16 2x4x4",
             "ffn_unfused_kernel_then_agg": "cfg2 unfused (ja_kernel fp32 partials, then ja_agg SUM)",
             "attention": "cfg3 causal attention [4,32,2048,128] bf16, 128-blocks",
             "rmsnorm": "cfg4a RMSNorm [8192,4096] bf16, d by 8",
             "swiglu": "cfg4b SwiGLU [8192,11008] bf16, f by 8",
             "repart_to_heads": "repartition [8192,12288] 2x2 -> [3,4,32,2048,128] head blocks (tokens to heads view)",
             "repart_to_tokens": "repartition [4,32,2048,128] head blocks -> [8192,4096] 2x2 (heads to tokens view)"}
    out = {}
    for k, d in res.items():
        e = {"what": names.get(k, k), "ms": d["ms"], "warm_median_ms": d["warm"]["median"],
             "cold_median_ms": d["cold"]["median"]}
        if "cold_tflops" in d and k != "tiny_fp32_2x2x2":
            e["cold_tflops"] = d["cold_tflops"]
            e["cold_frac_mfma_peak"] = round(d["cold_tflops"] / PEAK_BF16_TFLOPS, 3)
        elif "cold_gbs" in d and k != "tiny_fp32_2x2x2":
            e["cold_gbs"] = d["cold_gbs"]
            e["cold_frac_hbm_peak"] = round(d["cold_gbs"] / PEAK_HBM_GBS, 3)
        if "cpu_oracle" in d:
            e["cpu_oracle_ms"] = d["cpu_oracle"]["ms"]
            e["cpu_oracle_cores"] = d["cpu_oracle"]["cores"]
        out[k] = e
    return out


def bench_join(args):
    """The join step on the device (ja_djoin_run: grid enumeration, join
    predicate, group-by order, CSR segments) against the host join
    (ja_join, timed on the host) on the same decompositions: the
    [4, 32, 2048, 128] causal attention grid (128-blocks), a 131,072-token
    causal grid over 8 heads (1,024 query and key blocks), and the pages'
    packed example (4,096 positions, sequences ending at 1,024, 2,560 and
    4,096) over 32 heads.  Algorithmic bytes: records and segment offsets
    written once, split points read once."""
    import torch

    from tensor_relational_join_amd import binding as B
    from tensor_relational_join_amd.device import DeviceJoin

    cases = [
        ("attention_4x32x2048_causal", "bhsd,bhtd,bhtd->bhsd", "causal=s,t",
         {"b": _eq(4, 4), "h": _eq(32, 32), "s": _eq(2048, 16), "t": _eq(2048, 16), "d": [0, 128]}),
        ("causal_131072_tokens_8_heads", "bhsd,bhtd,bhtd->bhsd", "causal=s,t",
         {"b": [0, 1], "h": _eq(8, 8), "s": _eq(131072, 1024), "t": _eq(131072, 1024), "d": [0, 128]}),
        ("packed_4096_32_heads", "bhsd,bhtd,bhtd->bhsd", "packed=1024,2560,4096;causal=s,t",
         {"b": [0, 1], "h": _eq(32, 32), "s": [0, 1024, 2560, 4096], "t": [0, 1024, 2560, 4096], "d": [0, 128]}),
    ]
    res = {}
    for name, einsum, params, sp in cases:
        dj = DeviceJoin(einsum, "attention", {c: len(v) - 1 for c, v in sp.items()},
                        {c: v[-1] for c, v in sp.items()}, params)
        splits = torch.tensor([x for c in dj.letters for x in sp[c]], dtype=torch.int64, device="cuda")
        for _ in range(args.warmup):
            dj.run(splits)
        torch.cuda.synchronize()
        s0, s1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        s0.record()
        for _ in range(args.steps):
            dj.run(splits)
        s1.record()
        torch.cuda.synchronize()
        ms = s0.elapsed_time(s1) / args.steps
        nt, ns, status = (int(v) for v in dj.counts.cpu())
        nl = len(dj.letters)
        by = 4.0 * nt * nl + 8.0 * (ns + 1) + 8.0 * splits.numel()
        # the host join of the same decomposition
        spec = B.ja_spec_create(einsum, "attention", params)
        dec = B.ja_decomp_create(spec, [sp[c][-1] for c in dj.letters], [len(sp[c]) - 1 for c in dj.letters],
                                 [sp[c] for c in dj.letters])
        reps, t0 = 0, time.perf_counter()
        while reps < 3 or time.perf_counter() - t0 < 0.5:
            B.ja_tuples_destroy(B.ja_join(spec, dec))
            reps += 1
        host_ms = (time.perf_counter() - t0) / reps * 1e3
        B.ja_decomp_destroy(dec)
        B.ja_spec_destroy(spec)
        cells = 1
        for v in sp.values():
            cells *= len(v) - 1
        res[name] = {"cells": cells, "tuples": nt, "segments": ns, "status": status, "ms": round(ms, 4),
                     "mtuples_per_s": round(nt / (ms / 1e3) / 1e6, 1), "gbs": round(by / (ms / 1e3) / 1e9, 1),
                     "frac_hbm_peak": round(by / (ms / 1e3) / 1e9 / PEAK_HBM_GBS, 4),
                     "host_join_ms": round(host_ms, 3), "speedup_vs_host": round(host_ms / ms, 1)}
        dj.close()
    return {"workload": "join", "steps": args.steps, "warmup": args.warmup, "results": res}


def _pearson(xs, ys):
    import numpy as np

    x, y = np.asarray(xs, dtype=np.float64), np.asarray(ys, dtype=np.float64)
    if len(x) < 3 or x.std() == 0 or y.std() == 0:
        return None
    return float(np.corrcoef(x, y)[0, 1])


def bench_plans(args):
    """The logical optimizer's plans run on one GPU (an analogue of the
    pages' section 6 Experiments 3 and 5): for each graph, the optimizer's
    plan, the greedy plan, the plan chosen with the device-time model and 20
    random plans on p = 8, each timed (every operator plus every repartition
    between operators; computation inputs already in the blockings their
    consumers ask for), with the Pearson correlations of the measured time
    with the communication-cost proxy and with the device-time model.
    Graphs: the pages' matrix chains B, (M1 M2)((M3 M4) M5) with dimensions
    9,216 / 20,480 / 5,120 / 20,480 / 5,120 / 9,216, and C, M1 (M2 M3) with
    10,240 x 12,288 x 32,768 x 2,048; and the LLaMA-7B-shaped pre-norm FFN
    with its residual (8,192 tokens, d 4,096, FFN 11,008); and the whole
    LLaMA-7B-shaped block (batch 4 x 2,048 tokens, 32 heads of 128, FFN
    11,008) with its head views, for which the LlamaBlock class's hand
    decompositions are timed too (under "hand").  bf16, N(0, 1) inputs scaled
    by 1/sqrt(fan-in) (the block's weights N(0, 0.02^2))."""
    import torch

    from tensor_relational_join_amd.binding import JA_PLAN_DEVICE, JA_PLAN_GREEDY, JA_PLAN_OPTIMAL, JA_PLAN_RANDOM
    from tensor_relational_join_amd.graph import Graph, PlannedRun

    def chain_b():
        g = Graph()
        d = [9216, 20480, 5120, 20480, 5120, 9216]
        m = [g.input((d[i], d[i + 1])) for i in range(5)]
        p_ = g.op("ab,bc->ac", "contract", [m[0], m[1]])
        q = g.op("cd,de->ce", "contract", [m[2], m[3]])
        r = g.op("ce,ef->cf", "contract", [q, m[4]])
        g.op("ac,cf->af", "contract", [p_, r])
        return g

    def chain_c():
        g = Graph()
        m = [g.input(s) for s in ((10240, 12288), (12288, 32768), (32768, 2048))]
        x = g.op("bc,cd->bd", "contract", [m[1], m[2]])
        g.op("ab,bd->ad", "contract", [m[0], x])
        return g

    def ffn():
        g = Graph()
        T, D, F = 8192, 4096, 11008
        x, gn, wg, wu, wd = g.input((T, D)), g.input((D,)), g.input((D, F)), g.input((D, F)), g.input((F, D))
        h = g.op("rd,d->rd", "rmsnorm", [x, gn], "eps=1e-6")
        a = g.op("td,df->tf", "contract", [h, wg])
        b = g.op("td,df->tf", "contract", [h, wu])
        s_ = g.op("rf,rf->rf", "swiglu", [a, b])
        dn = g.op("tf,fd->td", "contract", [s_, wd])
        g.op("rd,rd->rd", "add", [dn, x])
        return g

    def block():
        # the LLaMA-7B-shaped block (batch 4 x 2048, d 4096, 32 heads, FFN 11008) with views around attention
        from tensor_relational_join_amd.graph import llama_block_graph

        g, _ = llama_block_graph(4, 2048, 4096, 32, 11008)
        return g

    p, nrand = 8, 20
    res = {}
    for name, make in (("chain_b", chain_b), ("chain_c", chain_c), ("ffn_llama7b", ffn), ("llama7b_block", block)):
        g = make()
        torch.manual_seed(11)
        dense = {}
        for t, shape in enumerate(g.shapes):
            if g.producer[t] is not None or t in g.views:
                continue
            x = torch.empty(shape, dtype=torch.bfloat16, device="cuda")
            if len(shape) == 1:  # the RMSNorm gain
                x.normal_(1.0, 0.1)
            elif name in ("ffn_llama7b", "llama7b_block") and t == 0:  # the activations
                x.normal_()
            elif name == "llama7b_block":  # the block's weights
                x.normal_(0.0, 0.02)
            else:  # a matrix of a chain or a weight: N(0, 1 / fan-in)
                x.normal_(0.0, float(shape[0]) ** -0.5)
            dense[t] = x
        plans = [("optimal", JA_PLAN_OPTIMAL, 0), ("greedy", JA_PLAN_GREEDY, 0), ("device", JA_PLAN_DEVICE, 0)] + \
                [("random", JA_PLAN_RANDOM, s) for s in range(nrand)]
        if name == "llama7b_block":  # the LlamaBlock class's hand decompositions (unfused), beside the selectors
            plans.append(("hand", None, 0))
        rows = []
        for label, mode, seed in plans:
            splits = None
            if label == "hand":
                from tensor_relational_join_amd.graph import llama_block_hand_splits

                splits = llama_block_hand_splits(g, 4, 2048)
                plan = [{c: len(v) - 1 for c, v in sp.items()} for sp in splits]
            else:
                _, plan = g.plan(p, mode, seed)
            cost = sum(g.cost(plan))
            model_us = g.device_time(plan)
            run = PlannedRun(g, plan, splits=splits)
            try:
                run.load(dense)
                for _ in range(args.warmup):
                    run.run()
                torch.cuda.synchronize()
                e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                e0.record()
                for _ in range(args.steps):
                    run.run()
                e1.record()
                torch.cuda.synchronize()
                ms = e0.elapsed_time(e1) / args.steps
                rows.append({"plan": label, "seed": seed, "cost": cost, "model_ms": round(model_us / 1e3, 4),
                             "ms": round(ms, 4),
                             "repartitions": len(run.reparts),
                             "intervals": ["".join("%s%d" % (c, v) for c, v in sp.items()) for sp in plan]})
            finally:
                run.close()
        rnd = [r for r in rows if r["plan"] == "random"]
        hand = [r for r in rows if r["plan"] == "hand"]
        if hand:
            res.setdefault("hand", {})[name] = hand[0]
        rows = [r for r in rows if r["plan"] != "hand"]
        res[name] = {"p": p, "optimal": rows[0], "greedy": rows[1], "device": rows[2],
                     "random_ms_median": float(sorted(r["ms"] for r in rnd)[len(rnd) // 2]),
                     "random_ms_best": min(r["ms"] for r in rnd),
                     "pearson_cost_vs_ms": _pearson([r["cost"] for r in rows], [r["ms"] for r in rows]),
                     "pearson_model_vs_ms": _pearson([r["model_ms"] for r in rows], [r["ms"] for r in rows]),
                     "plans": rows[3:]}
    return {"workload": "plans", "steps": args.steps, "warmup": args.warmup, "results": res}


def bench_varlen(args):
    """Causal grouped-query attention over a packed batch whose sequence
    ends are device data (32 query heads over 8 key-value heads, head_dim
    128, 16 sequences summing to 16,384 tokens, lengths drawn on the GPU from
    a fixed seed): one step is ja_dattn_run -- the device-side join, the
    table-building kernels and the attention kernel, no host round trip.
    Beside it, the same cuts planned on the host (join and tables built by the
    CPU, uploaded, then the attention kernel), timed as host planning plus
    the kernel."""
    import torch

    from tensor_relational_join_amd.device import DeviceAttention, Op

    G, R, S, nseq = 8, 4, 16384, 16
    gen = torch.Generator(device="cuda").manual_seed(17)
    cuts = torch.randperm(S - 1, generator=gen, device="cuda")[: nseq - 1] + 1
    ends = torch.cat([torch.zeros(1, dtype=torch.int64, device="cuda"), cuts.sort().values,
                      torch.full((1,), S, dtype=torch.int64, device="cuda")])
    t = lambda lo, hi: torch.tensor([lo, hi], dtype=torch.int64, device="cuda")  # noqa: E731
    gsp = torch.tensor(_eq(G, G), dtype=torch.int64, device="cuda")
    splits = torch.cat([t(0, 1), gsp, t(0, R), ends, t(0, 128), ends])  # letters b g r s d t
    da = DeviceAttention("bgrsd,bgtd,bgtd->bgrsd", {"b": 1, "g": G, "r": 1, "s": nseq, "d": 1, "t": nseq},
                         {"b": 1, "g": G, "r": R, "s": S, "d": 128, "t": S})
    Q = torch.empty(G * R * S * 128, dtype=torch.bfloat16, device="cuda").normal_(generator=gen)
    K = torch.empty(G * S * 128, dtype=torch.bfloat16, device="cuda").normal_(generator=gen)
    V = torch.empty_like(K).normal_(generator=gen)
    O = torch.empty_like(Q)
    for _ in range(args.warmup):
        da.run(splits, Q, K, V, O)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(args.steps):
        da.run(splits, Q, K, V, O)
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / args.steps
    e = ends.cpu().tolist()
    lens = [b - a for a, b in zip(e[:-1], e[1:])]
    flops = sum(2 * 2.0 * 128 * L * (L + 1) / 2 for L in lens) * G * R
    da.close()
    # the same cuts planned on the host, per step
    sp = {"b": [0, 1], "g": _eq(G, G), "r": [0, R], "s": e, "d": [0, 128], "t": e}
    t0 = time.perf_counter()
    op = Op("bgrsd,bgtd,bgtd->bgrsd", "attention", sp, "packed=device;causal=s,t")
    host_plan_ms = (time.perf_counter() - t0) * 1e3
    ins = [torch.empty(r.nbytes // 2, dtype=torch.bfloat16, device="cuda").normal_(generator=gen) for r in op.in_rels]
    out = torch.empty(op.out_rel.nbytes // 2, dtype=torch.bfloat16, device="cuda")
    for _ in range(args.warmup):
        op.run(ins, out)
    torch.cuda.synchronize()
    e0.record()
    for _ in range(args.steps):
        op.run(ins, out)
    e1.record()
    torch.cuda.synchronize()
    kernel_ms = e0.elapsed_time(e1) / args.steps
    op.close()
    return {"workload": "varlen", "steps": args.steps, "warmup": args.warmup,
            "results": {"device_planned_ms": round(ms, 4), "tflops": round(flops / (ms / 1e3) / 1e12, 1),
                        "host_planned_kernel_ms": round(kernel_ms, 4), "host_plan_ms": round(host_plan_ms, 3),
                        "sequence_lengths": lens}}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="block",
                    choices=sorted(BLOCKS) + ["configs", "ffn",
                             "attention", "norm_swiglu", "gqa", "copy", "join", "plans", "f16", "varlen",
                             "ceilings"])
    ap.add_argument("--no-cpu-baseline", action="store_true")
    args = ap.parse_args()
    if args.gpus != 1:
        print("bench.py measures one GPU only: the library has no multi-GPU path (every kernel runs on one "
              "GPU's share); run with --gpus 1", file=sys.stderr)
        sys.exit(2)
    _device_snapshot()  # before anything initialises the GPU in this process
    import torch

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(2)
    if args.workload == "join":
        print(json.dumps(bench_join(args)))
        return
    if args.workload == "plans":
        print(json.dumps(bench_plans(args)))
        return
    if args.workload == "varlen":
        print(json.dumps(bench_varlen(args)))
        return
    if args.workload == "ceilings":
        print(json.dumps(bench_ceilings(args)))
        return
    if args.workload not in BLOCKS:
        print(json.dumps(bench_kernel(args)))
        return
    out, inp = bench_block(args)
    out["device"] = _device_snapshot()
    if args.workload == "block":
        # the single-operator configurations and the copy ceiling, in the same run
        out["configs"] = configs_summary(args)
        out["copy_ceiling_cold"] = _copy_ceiling(1 << 31, 20, cold=True)["gbs"]
    if args.workload in ("block", "block_unfused") and not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline_block(inp, 4, 2048, 4096, 32, 11008,
                                                 fused=BLOCKS[args.workload].get("fused", True))
    print(json.dumps(out))


if __name__ == "__main__":
    main()
