#!/usr/bin/env python3
"""Decode throughput of the 48-layer DF-SSM model (Mamba-2 1.3B shape) on one
MI355X.

Default workload (the headline): batch 1.  Seeded synthetic weights (1-bit
scaffold + int8 LoRA r=16, int8 tied embedding / LM head, vocab 50288), a
16-token seeded prompt prefilled, then greedy decoding.  The timed region is
one launch of the persistent decode kernel that runs every timed token (all
48 layers, the LM head and the argmax fed back on the device).

Prints one JSON line: tokens/s, the roofline of that kernel (HIP-event time of
the launch, algorithmic bytes per token x tokens), and the CPU oracle timed on
a bounded sample of the same workload.

--workload decode-b32, decode-b512 and prefill-8x2048 measure the batched
path instead (32 or 512 sequences decoding after an 8-token prefill; a
prefill of 8 x 2048 tokens); their lines carry step-level rooflines.
"""
import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0  # MI355X HBM3E, GB/s
PAGES_B512_TOKS = 5081.0  # decode tokens/s at batch 512 (A100), the pages' only absolute throughput

# HBM bytes per decoded token of the persistent kernel, from rocprofv3 counter
# passes (FETCH_SIZE, then WRITE_SIZE, KiB per dispatch) over a 64-token launch,
# each scaled by what the same counter reads for a plain 1 GiB device copy
# (FETCH_SIZE reads 0.5 GiB for it: factor 2.0; WRITE_SIZE reads 1 GiB: 1.0).
# Valid only for the kernel sources they were taken from (hash below).
COUNTED_TRAFFIC = {
    "sources_sha256": "b68bd94ac8ac099661d2cbd6b2c0a4d0646b64e458d23916619ab4acd2180158",
    "fetch_bytes_per_token": 461281474,
    "write_bytes_per_token": 118426844,
}
KERNEL_SOURCES = ("bit_quantized_mamba_amd/csrc/persistent.hip", "bit_quantized_mamba_amd/csrc/persistent.h",
                  "bit_quantized_mamba_amd/csrc/common.h")


def kernel_sources_sha256():
    import hashlib
    h = hashlib.sha256()
    for f in KERNEL_SOURCES:
        with open(os.path.join(ROOT, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def algorithmic_bytes(s):
    """Bytes each decode-step kernel must move at batch 1 (reads + writes)."""
    dm, di, N, H, P, V, r = s.d_model, s.d_inner, s.d_state, s.n_heads, s.headdim, s.vocab, s.rank
    dp, cd, K = s.d_in_proj, s.conv_dim, s.d_conv
    f = 4
    k = {}
    k["in_proj"] = (dp * dm // 8 + dp * f + dp * r + dp * f      # bits, row scale, LoRA up + scale
                    + (dm // 32) * 8 * 4 + 3 * f + r * f          # bit planes, qsum/s, t
                    + cd * K * f + cd * f                          # conv weight, bias
                    + 2 * (K - 1) * cd * f                         # conv state read + write
                    + (di + H) * f + cd * f)                       # z, dt_raw, conv output
    k["ssm"] = (2 * H * P * N * f                                 # state read + write
                + cd * f + (di + H) * f + 3 * H * f + di * f)      # x,B,C; z, dt; A_log,dt_bias,D; gated y
    k["out_proj"] = (dm * di // 8 + dm * f + dm * r + dm * f + (di // 32) * 8 * 4 + 3 * f + r * f
                     + 2 * dm * f)                                 # residual read + write
    k["lm_head"] = V * dm + V * f + V * f + dm                    # E, sE, logits, qf
    k["norm_quant"] = dm * f + dm * f + r * dm + dm + (dm // 32) * 8 * 4 + (r + 3) * f
    return k


def step_bytes(s):
    """Algorithmic HBM bytes of one batch-1 decode step of the whole model."""
    dm, di, N, H, P, V, r = s.d_model, s.d_inner, s.d_state, s.n_heads, s.headdim, s.vocab, s.rank
    dp, cd, K = s.d_in_proj, s.conv_dim, s.d_conv
    f = 4
    per_layer = (dp * dm // 8 + dm * di // 8                      # scaffold bits
                 + (dp + dm) * f                                   # scaffold row scales
                 + r * (dm + dp + di + dm)                         # LoRA int8
                 + (2 * r + dp + dm) * f                           # LoRA scales
                 + cd * (K + 1) * f                                # conv weight + bias
                 + K * cd * f                                      # conv state: read K-1 columns, write 1
                 + 2 * H * P * N * f                               # SSM state read + write
                 + (3 * H + dm + di) * f)                          # A_log, dt_bias, D, norm weights
    once = V * dm + V * f + dm * f + dm + V * f                    # LM head + scales, final norm, embed row, logits
    return s.n_layer * per_layer + once


def batched_step_bytes(s, B):
    """Algorithmic HBM bytes of one batch-B decode step: weights once, state and logits per sequence."""
    dm, di, N, H, P, V, r = s.d_model, s.d_inner, s.d_state, s.n_heads, s.headdim, s.vocab, s.rank
    dp, cd, K = s.d_in_proj, s.conv_dim, s.d_conv
    f = 4
    weights = s.n_layer * (dp * dm // 8 + dm * di // 8 + (dp + dm) * f + r * (dm + dp + di + dm)
                           + (2 * r + dp + dm) * f + cd * (K + 1) * f + (3 * H + dm + di) * f) \
        + V * dm + V * f + dm * f
    per_seq = s.n_layer * (K * cd * f + 2 * H * P * N * f) + dm + V * f
    return weights + B * per_seq


def prefill_work(s, B, T):
    """int8 matrix-core ops of the scaffold + LoRA GEMMs and fp32 flops of the scan for a B x T prefill."""
    M = B * T
    dm, di, dp, r = s.d_model, s.d_inner, s.d_in_proj, s.rank
    gemm_ops = 2 * M * s.n_layer * (dp * dm + dm * di + r * (dm + dp + di + dm))
    scan_flops = 5 * s.n_heads * s.headdim * s.d_state * M * s.n_layer
    return gemm_ops, scan_flops


def bench_batched(args):
    import torch
    import synth
    from bit_quantized_mamba_amd import Engine

    s = synth.FULL_1P3B
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    stream = torch.cuda.current_stream()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    common = {"n_gpus": 1, "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
              "dtype": "int8/1-bit weights, int32 accumulation, f32 state", "data": "synthetic (seeded weights and tokens)",
              "cpu_baseline": None}
    if args.workload in ("decode-b32", "decode-b512"):
        B, T = (32, 8) if args.workload == "decode-b32" else (512, 8)
        seed = synth.SEED_BASE + 3
        eng = Engine.from_shape(s, max_batch=B, device=0)
        eng.load_synthetic(seed)
        toks = synth.gen_tokens(seed, 0, B * T, s.vocab).reshape(B, T)
        _, nxt = eng.prefill(torch.from_numpy(toks.astype("int32")).to(dev))
        tok = nxt.clone()
        out = torch.empty((max(args.steps, args.warmup, 1), B), dtype=torch.int32, device=dev)
        if args.warmup:
            eng.generate(tok, args.warmup, out=out, use_graph=True)
        torch.cuda.synchronize()
        e0.record(stream)
        eng.generate(tok, args.steps, out=out, use_graph=True)
        e1.record(stream)
        torch.cuda.synchronize()
        eng.check()
        ms = e0.elapsed_time(e1)
        sb = batched_step_bytes(s, B)
        gbs = sb * args.steps / (ms / 1e3) / 1e9
        res = {"metric": f"decode tokens/s, batch={B}, 48-layer 1.3B shape; % of HBM roofline",
               "value": round(B * args.steps / (ms / 1e3), 1), "unit": "tokens/s", "steps": args.steps,
               "warmup": args.warmup, "ms_per_step": round(ms / args.steps, 4),
               "config": {"workload": f"DF-SSM 48-layer 1.3B shape, batch {B}, 8-token prefill then greedy decode "
                                      f"of {args.steps} steps (one hipGraph replay per step)", "batch": B},
               "roofline": {"bound": "hbm", "scope": "whole step", "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS,
                            "unit": "GB/s", "frac": round(gbs / HBM_PEAK_GBS, 4), "traffic": None,
                            "bytes_per_step": sb}}
        if B == 512:
            # the pages' one absolute throughput: ~5,081 tokens/s at batch 512 on an A100
            # (same model shape; other hardware, context rather than a target)
            res["vs_baseline"] = round(res["value"] / PAGES_B512_TOKS, 3)
            res["baseline"] = {"value": PAGES_B512_TOKS, "unit": "tokens/s", "hardware": "A100",
                               "note": "the pages' batch-512 decode figure"}
    else:
        B, T = 8, 2048
        seed = synth.SEED_BASE + 4
        eng = Engine.from_shape(s, max_batch=B, device=0)
        eng.load_synthetic(seed)
        toks = torch.from_numpy(synth.gen_tokens(seed, 0, B * T, s.vocab).reshape(B, T).astype("int32")).to(dev)
        for _ in range(max(args.warmup, 1)):
            eng.reset_state(B)
            eng.prefill(toks)
        torch.cuda.synchronize()
        reps = max(1, args.steps)
        tot = 0.0
        for _ in range(reps):
            eng.reset_state(B)
            torch.cuda.synchronize()
            e0.record(stream)
            eng.prefill(toks)
            e1.record(stream)
            torch.cuda.synchronize()
            tot += e0.elapsed_time(e1)
        eng.check()
        ms = tot / reps
        gops, sflops = prefill_work(s, B, T)
        res = {"metric": "prefill tokens/s, 8 x 2048 tokens, 48-layer 1.3B shape",
               "value": round(B * T / (ms / 1e3), 1), "unit": "tokens/s", "steps": reps, "warmup": args.warmup,
               "ms_per_step": round(ms, 3),
               "config": {"workload": "DF-SSM 48-layer 1.3B shape, prefill of 8 sequences x 2048 tokens from a "
                                      "zero state (last-position logits)", "batch": B, "seq_len": T},
               # the GEMMs (int8 matrix cores) and the scan (fp32 matrix cores) run one after the
               # other, so the bound is the sum of their times at peak; the scan's work is the
               # recurrence's own flop count, whatever form computes it
               "roofline": {"bound": "mfma", "scope": "whole prefill",
                            "int8_gemm_TOPs": round(gops / 1e12, 2), "scan_TFLOPs": round(sflops / 1e12, 2),
                            "int8_peak_TOPS": 5000.0, "fp32_peak_TFLOPS": 157.3,
                            "bound_ms": round((gops / 5000e12 + sflops / 157.3e12) * 1e3, 2),
                            "frac": round((gops / 5000e12 + sflops / 157.3e12) * 1e3 / ms, 4)}}
    eng.close()
    out = dict(common)
    out.update(res)
    print(json.dumps(out))


def cpu_baseline(shape, seed, prompt, budget_s):
    """The CPU oracle decoding the same model, timed on a bounded number of steps."""
    import numpy as np
    import oracle
    import synth
    t0 = time.perf_counter()
    om = oracle.Model(shape, synth.gen_model(shape, seed))
    st = oracle.State(shape)
    setup = time.perf_counter() - t0
    tok = int(prompt[0])
    steps = 0
    t0 = time.perf_counter()
    while True:
        tok, _, _ = om.decode_step(st, tok)
        steps += 1
        el = time.perf_counter() - t0
        if el >= budget_s or steps >= 1000:
            break
    return {"value": round(steps / el, 3), "unit": "tokens/s", "cores": oracle.num_threads(), "kind": "oracle",
            "sample": f"{steps} greedy decode steps of the 48-layer model at batch 1 from a zero state "
                      f"({el:.1f} s; weight generation {setup:.1f} s not timed); plain C, fp64, OpenMP over rows"}


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=256, help="timed greedy decode steps")
    ap.add_argument("--warmup", type=int, default=16, help="untimed decode steps before the timed region")
    ap.add_argument("--cpu-seconds", type=float, default=15.0, help="time budget of the CPU oracle sample")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--kernel-breakdown", action="store_true",
                    help="also time each kernel of the per-layer (multi-kernel) path")
    ap.add_argument("--path", choices=["auto", "kernels", "persistent", "gemm"], default="auto")
    ap.add_argument("--workload", choices=["decode-b1", "decode-b32", "decode-b512", "prefill-8x2048"],
                    default="decode-b1")
    ap.add_argument("--copy-probe-mib", type=int, default=0,
                    help="after the timed region, run one plain device copy (read + write) of this many MiB, "
                         "a known-size reference for the HBM byte counters of a profiler run")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py: this build runs on one GPU only (the decode path is per-sequence data-parallel; "
              f"see the sharding notes); --gpus {args.gpus} is not supported", file=sys.stderr)
        sys.exit(2)

    if args.workload != "decode-b1":
        bench_batched(args)
        return

    import torch
    import synth
    from bit_quantized_mamba_amd import Engine

    s = synth.FULL_1P3B
    seed = synth.SEED_BASE + 2
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    eng = Engine.from_shape(s, max_batch=1, device=0)
    eng.set_path(args.path)
    eng.load_synthetic(seed)
    prompt = synth.gen_tokens(seed, 0, 16, s.vocab)
    _, nxt = eng.prefill(torch.from_numpy(prompt[None].astype("int32")).to(dev))
    tok = nxt.clone()
    out = torch.empty((max(args.steps, args.warmup, 1), 1), dtype=torch.int32, device=dev)
    if args.warmup:
        eng.generate(tok, args.warmup, out=out, use_graph=True)
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    eng.generate(tok, args.steps, out=out, use_graph=True)
    e1.record(stream)
    torch.cuda.synchronize()
    eng.check()
    if args.copy_probe_mib > 0:
        n = args.copy_probe_mib * (1 << 20) // 4
        src = torch.ones(n, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        torch.mul(src, 1.0, out=dst)  # elementwise: reads n*4 bytes, writes n*4 bytes
        torch.cuda.synchronize()
        del src, dst
    ms = e0.elapsed_time(e1)
    ms_per_step = ms / args.steps
    value = args.steps / (ms / 1e3)
    sb = step_bytes(s)
    step_gbs = sb / (ms_per_step / 1e3) / 1e9

    # The timed region is one launch of the persistent decode kernel (all steps
    # in one kernel) on the auto/persistent path, so its HIP-event time is that
    # kernel's duration; its algorithmic bytes are steps x the step's bytes.
    persistent = args.path in ("auto", "persistent")
    roofline = None
    if persistent:
        achieved = sb * args.steps / (ms / 1e3) / 1e9
        traffic = None
        if kernel_sources_sha256() == COUNTED_TRAFFIC["sources_sha256"]:
            traffic = int((COUNTED_TRAFFIC["fetch_bytes_per_token"] + COUNTED_TRAFFIC["write_bytes_per_token"])
                          * args.steps)
        roofline = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                    "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": traffic,
                    "kernel": "decode_persistent_kernel", "bytes_per_launch": sb * args.steps,
                    "us_per_launch": round(ms * 1e3, 1)}
    kernels = {}
    if args.kernel_breakdown or not persistent:
        ab = algorithmic_bytes(s)
        per_step = {"in_proj": s.n_layer, "ssm": s.n_layer, "out_proj": s.n_layer, "lm_head": 1,
                    "norm_quant": 2 * s.n_layer + 1}
        for name in ("in_proj", "ssm", "out_proj", "lm_head", "norm_quant"):
            iters = 960 if name != "lm_head" else 64
            us = eng.time_kernel(name, 1, iters)
            gbs = ab[name] / (us * 1e-6) / 1e9
            kernels[name] = {"us_per_launch": round(us, 3), "launches_per_step": per_step[name],
                             "us_per_step": round(us * per_step[name], 2), "bytes_per_launch": ab[name],
                             "GB/s": round(gbs, 1)}
        if not persistent:
            dom = max(kernels, key=lambda k: kernels[k]["us_per_step"])
            kd = kernels[dom]
            achieved = kd["bytes_per_launch"] / (kd["us_per_launch"] * 1e-6) / 1e9
            roofline = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                        "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": None, "kernel": dom}
        eng.reset_state(1)

    result = {
        "metric": "decode tokens/s, batch=1, 48-layer 1.3B shape; % of HBM roofline",
        "value": round(value, 2),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "int8/1-bit weights, int32 accumulation, f32 state",
        "data": "synthetic (seeded weights and tokens)",
        "config": {"workload": "DF-SSM 48-layer Mamba-2 1.3B shape (d_model 2048, d_inner 4096, d_state 128, "
                               "64 heads, vocab 50288), batch 1, 16-token prefill then greedy decode of "
                               f"{args.steps} tokens",
                   "batch": 1, "prefill": 16,
                   "path": "persistent kernel, one launch for all timed tokens" if persistent else
                           ("per-layer kernels" if args.path == "kernels" else "batched GEMM path")
                           + ", one hipGraph replay per token"},
        "roofline": roofline,
        "step_roofline": {"bound": "hbm", "bytes_per_step": sb, "achieved": round(step_gbs, 1),
                          "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": round(step_gbs / HBM_PEAK_GBS, 4)},
        "kernels": kernels,
        "cpu_baseline": None,
    }
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(s, seed, prompt, args.cpu_seconds)
    eng.close()
    print(json.dumps(result))


if __name__ == "__main__":
    main()
