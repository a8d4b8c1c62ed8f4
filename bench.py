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
--workload tiny-decode (the 2-layer test stack, us/token over 64 tokens),
layer-1p3b-hot and layer-1p3b-cold (one 1.3B-shaped layer stepped 1000 times
on fp16 inputs; cold cycles 64 layer copies) measure the two small workloads
(use --steps 64 / --steps 1000).
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
    "sources_sha256": "7d6f23ed2288ae67b164c6f50683114adfd5a6fbf372422f38c7153b87ae6b7c",
    "fetch_bytes_per_token": 461728520,
    "write_bytes_per_token": 118426855,
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


def layer_step_bytes(s):
    """Algorithmic HBM bytes of one single-layer decode step at batch 1 (one layer's weights, its conv
    state read of 3 columns and write of 1, its SSM state read and written, the fp16 input and fp32 output)."""
    dm, di, N, H, P, r = s.d_model, s.d_inner, s.d_state, s.n_heads, s.headdim, s.rank
    dp, cd, K = s.d_in_proj, s.conv_dim, s.d_conv
    f = 4
    return (dp * dm // 8 + dm * di // 8 + (dp + dm) * f + r * (dm + dp + di + dm) + (2 * r + dp + dm) * f
            + cd * (K + 1) * f + K * cd * f + 2 * H * P * N * f + (3 * H + dm + di) * f + dm * 2 + dm * f)


PHASES = ["residual hop + norm statistics", "quantise", "wait for LoRA down", "in_proj rows", "conv",
          "B/C hop", "SSM + publish", "gated-output hop + norm statistics", "out_proj rows + publish"]


def phase_profile(eng, tok, n_tokens, s):
    """Per-phase durations of the persistent batch-1 kernel (device timestamps at 10 points of every layer of
    every workgroup, 100 MHz clock): median, mean, 90th percentile and the mean over layers of the slowest
    workgroup, for layers 1 .. L-2; plus, per hop, how far the publishers are spread and how long after the
    last publisher the median receiver has the values."""
    import numpy as np
    prof = eng.profile_persistent(tok, n_tokens, n_tokens)
    p = prof.cpu().numpy().astype(np.int64)  # [T][L+1][G][10]
    L = s.n_layer
    ns = 10.0
    d = np.diff(p[:, 1:L - 1, :, :], axis=-1) * ns
    out = {"tokens": n_tokens, "phases_ns": {}}
    for k, nm in enumerate(PHASES):
        x = d[..., k]
        out["phases_ns"][nm] = {"median": float(np.median(x)), "mean": round(float(x.mean()), 1),
                                "p90": float(np.percentile(x, 90)),
                                "slowest_wg": round(float(x.max(axis=2).mean()), 1)}
    lp = (p[:, 2:L - 1, :, 0] - p[:, 1:L - 2, :, 0]) * ns
    out["layer_period_ns"] = {"median": float(np.median(lp)), "mean": round(float(lp.mean()), 1)}
    e9 = (p[:, 2:L - 1, :, 0] - p[:, 1:L - 2, :, 9]) * ns
    out["layer_turnaround_ns"] = {"median": float(np.median(e9)), "mean": round(float(e9.mean()), 1)}

    def hop(pl, pe, rl, re):
        pub, rec = p[:, pl, :, pe], p[:, rl, :, re]
        last = pub.max(axis=1)
        return (np.mean(last - pub.min(axis=1)) * ns, np.mean(np.median(rec, axis=1) - last) * ns)

    for name, (pe, rl_off, re) in {"residual": (9, 1, 1), "B/C": (5, 0, 6), "gated output": (7, 0, 8)}.items():
        v = np.array([hop(l, pe, l + rl_off, re) for l in range(1, L - 2)])
        out.setdefault("hops_ns", {})[name] = {"publisher_spread": round(float(v[:, 0].mean()), 1),
                                               "last_publisher_to_median_receiver": round(float(v[:, 1].mean()), 1)}
    hd = np.diff(p[:, L, :, :5], axis=-1) * ns
    out["lm_head_ns"] = {nm: float(np.median(hd[..., i]))
                         for i, nm in enumerate(["residual hop", "quantise", "logits + local argmax", "argmax hop"])}
    out["token_period_us"] = round(float(np.median((p[1:, 0, :, 0] - p[:-1, 0, :, 0]) * ns)) / 1000, 2)
    return out


def host_facts():
    """CPU model name (from /proc/cpuinfo), OMP_NUM_THREADS and the usable cores of this host."""
    model = None
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    return {"cpu_model": model, "OMP_NUM_THREADS": os.environ.get("OMP_NUM_THREADS"),
            "nproc": len(os.sched_getaffinity(0)) if hasattr(os, "sched_getaffinity") else os.cpu_count()}


def bench_small(args):
    """The tiny 2-layer model's batch-1 decode (64 greedy tokens in one persistent launch) or one
    1.3B-shaped layer stepped 1000 times on fp16 inputs (hot: one layer; cold: 64 layer copies
    cycled, more than the 256 MB Infinity Cache)."""
    import numpy as np
    import torch
    import synth
    from bit_quantized_mamba_amd import Engine

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    stream = torch.cuda.current_stream()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    common = {"n_gpus": 1, "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
              "dtype": "int8/1-bit weights, int32 accumulation, f32 state", "data": "synthetic (seeded weights and tokens)",
              "cpu_baseline": None}
    if args.workload == "tiny-decode":
        s = synth.TINY
        seed = synth.SEED_BASE
        n = args.steps
        eng = Engine.from_shape(s, max_batch=1, device=0)
        eng.load_synthetic(seed)
        tok = torch.from_numpy(synth.gen_tokens(seed, 0, 1, s.vocab).astype("int32")).to(dev)
        out = torch.empty((max(n, args.warmup, 1), 1), dtype=torch.int32, device=dev)
        if args.warmup:
            eng.generate(tok, args.warmup, out=out)
        eng.reset_state(1)
        torch.cuda.synchronize()
        e0.record(stream)
        eng.generate(tok, n, out=out)
        e1.record(stream)
        torch.cuda.synchronize()
        eng.check()
        ms = e0.elapsed_time(e1)
        sb = step_bytes(s)
        gbs = sb * n / (ms / 1e3) / 1e9
        res = {"metric": "decode us/token, batch=1, 2-layer test stack (d_model 256)",
               "value": round(ms * 1e3 / n, 3), "unit": "us/token", "higher_is_better": False, "steps": n,
               "warmup": args.warmup, "ms_per_step": round(ms / n, 5),
               "config": {"workload": f"DF-SSM 2-layer test stack (d_model 256, d_inner 512, d_state 16, headdim 32, "
                                      f"vocab 1024), batch 1, {n} greedy tokens in one persistent launch", "batch": 1},
               # 0.64 MB per token stays in the caches: the HBM fraction is not a meaningful bound here
               "roofline": {"bound": "hbm", "scope": "cache-resident (0.64 MB/token): fraction not meaningful",
                            "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                            "frac": round(gbs / HBM_PEAK_GBS, 5), "traffic": None, "bytes_per_token": sb}}
    else:
        cold = args.workload == "layer-1p3b-cold"
        base = synth.LAYER_1P3B
        copies = 64 if cold else 1
        s = synth.Shape(n_layer=copies, d_model=base.d_model, d_inner=base.d_inner, d_state=base.d_state,
                        headdim=base.headdim, vocab=base.vocab)
        seed = synth.SEED_BASE + 1
        n = args.steps
        eng = Engine.from_shape(s, max_batch=1, device=0)
        eng.load_synthetic(seed)
        h16 = synth.gen_fp16_normal(seed, 1, n * s.d_model).reshape(n, 1, s.d_model)
        hin = torch.from_numpy(h16).to(dev)
        hout = torch.empty((n, 1, s.d_model), dtype=torch.float32, device=dev)
        # one HIP graph of all n steps (inputs already in HBM), replayed once per timing
        g = torch.cuda.CUDAGraph()
        eng.reset_state(1)
        torch.cuda.synchronize()
        cap = torch.cuda.Stream()
        with torch.cuda.stream(cap):
            with torch.cuda.graph(g, stream=cap):
                for i in range(n):
                    eng.layer_step_f16(i % copies, hin[i], hout[i], stream=cap)
        for _ in range(max(args.warmup, 1)):
            g.replay()
        torch.cuda.synchronize()
        eng.reset_state(1)
        torch.cuda.synchronize()
        e0.record(stream)
        g.replay()
        e1.record(stream)
        torch.cuda.synchronize()
        eng.check()
        ms = e0.elapsed_time(e1)
        sb = layer_step_bytes(s)
        gbs = sb * n / (ms / 1e3) / 1e9
        res = {"metric": "single-layer step us/step, batch=1, 1.3B layer shape" + (", cold (64 layer copies)" if cold
                                                                                  else ", hot"),
               "value": round(ms * 1e3 / n, 3), "unit": "us/step", "higher_is_better": False, "steps": n,
               "warmup": args.warmup, "ms_per_step": round(ms / n, 5),
               "config": {"workload": f"one Mamba-2 1.3B-shaped DF-SSM layer (d_model 2048, d_inner 4096, "
                                      f"d_state 128), batch 1, {n} steps on seeded fp16 N(0,1) inputs, state "
                                      f"carried, per-layer kernels replayed as one HIP graph"
                                      + (f", layer i % {copies} of {copies} copies (working set beyond the "
                                         f"Infinity Cache)" if cold else ""), "batch": 1},
               "roofline": {"bound": "hbm", "scope": "whole step", "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS,
                            "unit": "GB/s", "frac": round(gbs / HBM_PEAK_GBS, 4), "traffic": None,
                            "bytes_per_step": sb}}
    eng.close()
    out = dict(common)
    out.update(res)
    print(json.dumps(out))


def bench_codec(args):
    """The density-field state codec on the 48-layer model: pack / unpack / in-place round trip of the SSM
    state of 32 sequence slots (after an 8-token prefill), HIP-event timed; and the greedy tokens and final
    logits of a batch-1 decode with the codec applied at every 64-token boundary against one without."""
    import numpy as np
    import torch
    import synth
    from bit_quantized_mamba_amd import Engine

    s = synth.FULL_1P3B
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    stream = torch.cuda.current_stream()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    B, T = 32, 8
    seed = synth.SEED_BASE + 3
    eng = Engine.from_shape(s, max_batch=B, device=0)
    eng.load_synthetic(seed)
    toks = synth.gen_tokens(seed, 0, B * T, s.vocab).reshape(B, T)
    eng.prefill(torch.from_numpy(toks.astype("int32")).to(dev))
    field, scale = eng.state_pack(0, B)
    rows = B * s.n_layer * s.n_heads * s.headdim
    fp32_bytes = rows * s.d_state * 4
    packed_bytes = rows * (s.d_state // 2 + 4)
    reps = max(1, args.steps)
    times = {}
    for name, fn in (("pack", lambda: eng.state_pack(0, B)), ("unpack", lambda: eng.state_unpack(field, scale, 0)),
                     ("roundtrip", lambda: eng.state_roundtrip(0, B))):
        for _ in range(max(args.warmup, 1)):
            fn()
        torch.cuda.synchronize()
        e0.record(stream)
        for _ in range(reps):
            fn()
        e1.record(stream)
        torch.cuda.synchronize()
        times[name] = e0.elapsed_time(e1) / reps
    eng.check()
    eng.close()
    moved = {"pack": fp32_bytes + packed_bytes, "unpack": packed_bytes + fp32_bytes, "roundtrip": 2 * fp32_bytes}
    gbs = {k: moved[k] / (times[k] / 1e3) / 1e9 for k in times}
    # drift: batch-1 greedy decode of 256 tokens, codec at every 64-token boundary or not
    seed1 = synth.SEED_BASE + 2
    runs = []
    for codec in (False, True):
        e = Engine.from_shape(s, max_batch=1, device=0)
        e.load_synthetic(seed1)
        prompt = synth.gen_tokens(seed1, 0, 16, s.vocab)
        _, nxt = e.prefill(torch.from_numpy(prompt[None].astype("int32")).to(dev))
        tok = nxt.clone()
        outs = []
        for _ in range(4):
            outs.append(e.generate(tok, 64).cpu().numpy()[:, 0])
            if codec:
                e.state_roundtrip(0, 1)
        lg, _ = e.decode_step(tok)
        runs.append((np.concatenate(outs), lg.cpu().numpy()[0].astype(np.float64)))
        e.check()
        e.close()
    (ta, la), (tb, lb) = runs
    same = ta == tb
    prefix = int(np.argmin(same)) if not same.all() else len(same)
    rms = float(np.sqrt(np.mean(la * la)))
    res = {"metric": "density-field state codec: pack GB/s over 32 sequences' SSM state, 48-layer 1.3B shape",
           "value": round(gbs["pack"], 1), "unit": "GB/s", "higher_is_better": True, "steps": reps,
           "warmup": args.warmup, "ms_per_step": round(times["pack"], 4),
           "config": {"workload": "DF-SSM 48-layer 1.3B shape, SSM state of 32 sequences after an 8-token prefill "
                                  "(3.2 GB fp32) packed to 4 cells per value + a row scale", "batch": B},
           "roofline": {"bound": "hbm", "scope": "pack kernel", "achieved": round(gbs["pack"], 1),
                        "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": round(gbs["pack"] / HBM_PEAK_GBS, 4),
                        "traffic": None, "bytes_per_launch": moved["pack"]},
           "codec": {"ms": {k: round(v, 4) for k, v in times.items()}, "GB/s": {k: round(v, 1) for k, v in gbs.items()},
                     "fp32_state_bytes": fp32_bytes, "packed_bytes": packed_bytes,
                     "ratio": round(fp32_bytes / packed_bytes, 3)},
           "drift_batch1": {"tokens": int(len(ta)), "identical_prefix": prefix, "agreement": round(float(same.mean()), 4),
                            "final_logits_max_rel_err": round(float(np.max(np.abs(lb - la)) / max(rms, 1e-30)), 4),
                            "note": "greedy decode, codec at every 64-token boundary vs none"}}
    out = {"n_gpus": 1, "scaling": "weak", "vs_baseline": None, "dtype": "f32 state -> 4-bit density field",
           "data": "synthetic (seeded weights and tokens)", "cpu_baseline": None}
    out.update(res)
    print(json.dumps(out))


def bench_reference(args):
    """Reference rates of this GPU for the kernels' bounds, printed as one JSON line: the vendor int8 and bf16
    GEMMs (torch._int_mm, torch.matmul) on the prefill's scaffold shapes, plain device copy / in-place scale /
    fill bandwidth, and the scaffold GEMM here (dfssm_k_gemm, no acc output) on the in_proj shape over K."""
    import torch
    from bit_quantized_mamba_amd import call, _dp, _stream

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    g = torch.Generator(device=dev)
    g.manual_seed(1)

    def timed(fn, reps=10):
        for _ in range(3):
            fn()
        torch.cuda.synchronize()
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(reps):
            fn()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / reps * 1e3  # us

    out = {"metric": "reference rates of this GPU (vendor GEMMs, device copies) and the scaffold GEMM over K",
           "n_gpus": 1, "data": "synthetic (seeded)", "gemm": [], "hbm": {}, "k_sweep_in_proj": []}
    for (M, N, K) in [(16384, 8512, 2048), (16384, 2048, 4096)]:
        a = torch.randint(-127, 128, (M, K), dtype=torch.int8, device=dev, generator=g)
        b = torch.randint(-127, 128, (N, K), dtype=torch.int8, device=dev, generator=g).t()
        us_i8 = timed(lambda: torch._int_mm(a, b))
        a16 = torch.randn((M, K), dtype=torch.bfloat16, device=dev, generator=g)
        b16 = torch.randn((K, N), dtype=torch.bfloat16, device=dev, generator=g)
        us_bf = timed(lambda: a16 @ b16)
        out["gemm"].append({"M": M, "N": N, "K": K, "int_mm_us": round(us_i8, 1),
                            "int_mm_TOPs": round(2 * M * N * K / us_i8 / 1e6, 1),
                            "bf16_matmul_us": round(us_bf, 1)})
        del a, b, a16, b16
    x = torch.ones(1 << 27, dtype=torch.float32, device=dev)  # 0.54 GB
    y = torch.empty_like(x)
    nb = x.numel() * 4
    out["hbm"] = {"bytes": nb,
                  "copy_GBs": round(2 * nb / timed(lambda: y.copy_(x)) / 1e3, 0),
                  "inplace_scale_GBs": round(2 * nb / timed(lambda: x.mul_(1.0)) / 1e3, 0),
                  "fill_GBs": round(nb / timed(lambda: y.fill_(0.0)) / 1e3, 0)}
    del x, y
    M, N = 16384, 8512
    for K in (256, 512, 1024, 2048, 4096):
        bits = torch.randint(-2**31, 2**31 - 1, (N, K // 32), dtype=torch.int32, device=dev, generator=g)
        sw = torch.rand(N, device=dev, generator=g) * 0.04 + 0.01
        A = torch.randint(-127, 128, (16, K), dtype=torch.int8, device=dev, generator=g)
        sA = torch.full((16,), 1e-3, device=dev)
        Bm = torch.randint(-127, 128, (N, 16), dtype=torch.int8, device=dev, generator=g)
        sB = torch.full((N,), 1e-3, device=dev)
        q = torch.randint(-127, 128, (M, K), dtype=torch.int8, device=dev, generator=g)
        s = torch.rand(M, device=dev, generator=g) * 0.01
        yk = torch.empty((M, N), dtype=torch.float32, device=dev)
        us = timed(lambda: call("dfssm_k_gemm", _dp(bits), _dp(sw), _dp(A), _dp(sA), _dp(Bm), _dp(sB), K, N,
                                _dp(q), _dp(s), M, None, _dp(yk), _stream(None)))
        out["k_sweep_in_proj"].append({"K": K, "us_per_call_incl_operand_prep": round(us, 1)})
        del bits, A, Bm, q, yk
    print(json.dumps(out))


def bench_host(args):
    """Batch-1 greedy decode of the 48-layer model on the host CPU backend (libdfssm_host.so):
    16-token prompt, untimed warmup steps, then timed steps; the memory roofline is priced against
    this host's measured copy rate with the same threads, and the CPU oracle is timed beside it."""
    import numpy as np
    import synth
    from bit_quantized_mamba_amd.host import HostEngine

    s = synth.FULL_1P3B
    seed = synth.SEED_BASE + 2
    facts = host_facts()
    threads = min(16, facts["nproc"] or 1)
    eng = HostEngine.from_shape(s, max_batch=1, threads=threads)
    eng.load_synthetic(seed)
    prompt = synth.gen_tokens(seed, 0, 16, s.vocab)
    steps, warmup = min(args.steps, 128), min(args.warmup, 8)
    rates = {}
    isas = ["portable", "auto"]
    for isa in isas:
        eng.set_isa(isa)
        eng.reset_state(1)
        _, nxt = eng.prefill(prompt[None])
        tok = nxt.copy()
        if warmup:
            eng.generate(tok, warmup)
        t0 = time.perf_counter()
        eng.generate(tok, steps if isa == "auto" else max(8, steps // 8))
        el = time.perf_counter() - t0
        rates[eng.isa] = (steps if isa == "auto" else max(8, steps // 8)) / el
        if isa == "auto":
            ms = el / steps * 1e3
    value = rates[eng.isa]
    copy = eng.copy_rate(1 << 30, 5)
    per_token = step_bytes(s)
    achieved = per_token * value / 1e9
    res = {
        "metric": "decode tokens/s, batch=1, 48-layer 1.3B shape, host CPU backend; % of the host's copy rate",
        "value": round(value, 2), "unit": "tokens/s", "n_gpus": 0, "steps": steps, "warmup": warmup,
        "ms_per_step": round(ms, 3), "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "int8/1-bit weights, int32 accumulation, f32 state", "data": "synthetic (seeded weights and tokens)",
        "config": {"workload": f"DF-SSM 48-layer 1.3B shape, batch 1, 16-token prefill then greedy decode of "
                               f"{steps} tokens on the host CPU backend ({eng.isa}, {threads} threads)",
                   "batch": 1, "prefill": 16, "threads": threads},
        "roofline": {"bound": "host memory", "achieved": round(achieved, 1), "peak": round(copy, 1), "unit": "GB/s",
                     "frac": round(achieved / copy, 4), "traffic": None,
                     "peak_kind": "measured copy rate (read + write) of this host with the same threads",
                     "bytes_per_token": per_token},
        "paths_tokens_per_s": {k: round(v, 2) for k, v in rates.items()},
        "cpu_baseline": None,
    }
    if not args.no_cpu_baseline:
        res["cpu_baseline"] = cpu_baseline(s, seed, prompt, args.cpu_seconds)
        res["vs_oracle"] = round(value / res["cpu_baseline"]["value"], 2)
    eng.close()
    print(json.dumps(res))


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
            "host": host_facts(),
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
    ap.add_argument("--workload", choices=["decode-b1", "decode-b32", "decode-b512", "prefill-8x2048",
                                           "tiny-decode", "layer-1p3b-hot", "layer-1p3b-cold", "state-codec",
                                           "reference-rates", "host-decode"],
                    default="decode-b1")
    ap.add_argument("--phase-profile", type=int, default=0, metavar="TOKENS",
                    help="after the timed region, decode this many tokens with the persistent kernel's phase "
                         "timestamps and print their summary to stderr (batch 1)")
    ap.add_argument("--copy-probe-mib", type=int, default=0,
                    help="after the timed region, run one plain device copy (read + write) of this many MiB, "
                         "a known-size reference for the HBM byte counters of a profiler run")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py: this build runs on one GPU only (the decode path is per-sequence data-parallel; "
              f"see the sharding notes); --gpus {args.gpus} is not supported", file=sys.stderr)
        sys.exit(2)

    if args.workload == "state-codec":
        bench_codec(args)
        return
    if args.workload == "reference-rates":
        bench_reference(args)
        return
    if args.workload == "host-decode":
        bench_host(args)
        return
    if args.workload in ("tiny-decode", "layer-1p3b-hot", "layer-1p3b-cold"):
        bench_small(args)
        return
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
    if args.phase_profile > 0:
        print(json.dumps({"phase_profile": phase_profile(eng, tok, args.phase_profile, s)}), file=sys.stderr)
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
                    "us_per_launch": round(ms * 1e3, 1),
                    # what limits the launch below its HBM bound (measured, not derived from this run)
                    "limiter": {"what": "all-to-all exchanges between the 256 workgroups: 3 per layer, 1 per token "
                                        "for the argmax, each one device-coherent store -> load round trip plus the "
                                        "wait for the slowest publisher",
                                "us_per_exchange_alone": [1.7, 2.0],
                                "exchanges_per_token": 3 * s.n_layer + 1,
                                "us_per_layer": round(ms * 1e3 / args.steps / s.n_layer, 2)}}
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
