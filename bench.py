#!/usr/bin/env python3
"""Benchmark of the Hymba hybrid-head layer forward on one MI355X.

Workload (value): prefill of one bf16 layer, batch 8 x 2048 tokens plus 128 meta
tokens, d_model 2048, 16 q heads x 128 with 4 kv heads, full causal attention, SSM
inner dim 4096 with state 16.  A step is one whole pass of the layer (in_proj,
attention, x_proj, dt_proj, selective scan, norm + fusion, out_proj) over the batch;
inputs and weights are resident in HBM.  tokens/s counts the 8 x 2048 real tokens.

Also reported: decode of the same layer shape with a 1024-key sliding window,
batch 128, ring cache of 1024 slots plus 128 meta entries, 256 consecutive steps
timed as one span (tokens/s = 128 * 256 / span); the per-stage HIP-event timings; the
roofline of the dominant kernel; and the CPU oracle timed on a bounded sample.

Usage: python bench.py [--steps K] [--warmup W] [--gpus 1]
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "hybrid-layer prefill tokens/s + decode tokens/s on 1 MI355X; % MFMA/HBM peak"
PEAK_BF16_TFLOPS = 2500.0     # MI355X dense bf16 MFMA
PEAK_HBM_GBS = 8000.0          # MI355X HBM3E
PEAK_VALU_TFLOPS = 157.3       # MI355X fp32 vector (256 CU x 2.4 GHz x 256 flop/clk)
# The exponential rate has no published figure: bench.py measures it on the GPU it runs on
# (hymba_op_probe kind 0: independent v_exp_f32 chains) and holds the scan's exponentials
# against that measurement.
EXP_TPS = {"value": None}      # 10^12 exponentials per second, set by measure_ceilings()


def measure_ceilings(hy, torch, dev):
    """This GPU's practical ceilings, each the best of three timed launches of a library
    probe: the v_exp_f32 rate (independent chains), the dense bf16 MFMA rate (a pure
    v_mfma_f32_32x32x16_bf16 loop) and a streaming read of 2 GiB.  Context for the
    rooflines, which use the published peaks; the exponential rate is also the peak the
    scan's exponentials are held to."""
    out = torch.empty(8192 * 256, dtype=torch.float32, device=dev)
    src = torch.empty(2 << 30, dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream()

    def best(fn):
        fn()
        ts = []
        for _ in range(3):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            fn()
            e1.record(stream)
            e1.synchronize()
            ts.append(e0.elapsed_time(e1) * 1e-3)
        return min(ts)

    blocks, it_exp, it_mfma = 8192, 2048, 256
    # the MFMA probe again on operands with the layer's distributions (activations N(0,1),
    # weights N(0, 0.02)), changing every instruction as in a GEMM's k loop
    half = 64 * 8 * 256 * 8  # bf16 values per operand set
    gen = torch.Generator(device=dev)
    gen.manual_seed(12)
    ops = torch.cat([torch.randn(half, generator=gen, device=dev),
                     torch.randn(half, generator=gen, device=dev) * 0.02]).to(torch.bfloat16)
    t_exp = best(lambda: hy.hymba_op_probe(0, blocks, it_exp, None, 0, out, stream))
    t_mfma = best(lambda: hy.hymba_op_probe(1, blocks, it_mfma, None, 0, out, stream))
    t_mfma_data = best(lambda: hy.hymba_op_probe(3, blocks, it_mfma // 2, ops,
                                                 ops.numel() * 2, out, stream))
    t_read = best(lambda: hy.hymba_op_probe(2, 0, 0, src, src.numel(), out, stream))
    exps = blocks * 256 * it_exp * 8
    flops = blocks * 4 * 4 * it_mfma * 32 * 32 * 16 * 2
    flops_data = blocks * 4 * 8 * (it_mfma // 2) * 32 * 32 * 16 * 2
    res = {"exp_tps": round(exps / t_exp / 1e12, 2), "unit_exp": "10^12 exp/s",
           "mfma_bf16_tflops": round(flops / t_mfma / 1e12, 1),
           "mfma_bf16_layer_data_tflops": round(flops_data / t_mfma_data / 1e12, 1),
           "read_gbs": round(src.numel() / t_read / 1e9, 1),
           "probes": "hymba_op_probe kinds 0 (8192 x 256 lanes x 8 chains x 2048 exp2), "
                     "1 (8192 x 4 waves x 4 chains x 256 MFMA 32x32x16 bf16), "
                     "3 (the same MFMA loop, 8 x 128 per wave, on N(0,1) x N(0,0.02) bf16 "
                     "operands that change every instruction), "
                     "2 (streaming read of 2 GiB); best of 3 launches each"}
    EXP_TPS["value"] = res["exp_tps"]
    del out, src, ops
    torch.cuda.empty_cache()
    log(f"[bench] ceilings: exp {res['exp_tps']} T/s, MFMA bf16 {res['mfma_bf16_tflops']} "
        f"TFLOP/s ({res['mfma_bf16_layer_data_tflops']} on the layer's operand distributions), "
        f"read {res['read_gbs']} GB/s")
    return res


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--decode-steps", type=int, default=256)
    ap.add_argument("--no-decode", action="store_true")
    ap.add_argument("--no-stack", action="store_true",
                    help="skip the 16-layer partial-SWA vs all-global stack comparison")
    ap.add_argument("--no-head-ssm", action="store_true",
                    help="skip the layer variants (Mamba-2 head, group-norm fusion, block)")
    ap.add_argument("--no-long", action="store_true",
                    help="skip the layer-pair (B=4, L=8192) and long-context (L=32768) "
                         "prefill workloads")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seqs", type=int, default=8,
                    help="sequences of the prefill workload the CPU oracle runs (8 = all)")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="BYTES",
                    help="after the prefill pass, copy BYTES once with the library's copy "
                         "kernel (the known-size reference for HBM byte counters)")
    return ap.parse_args()


def scan_channels(N):
    """Channels per workgroup of the bf16 scan (one per lane of a wave, for every N)."""
    return 64


def deferred_norm(dims):
    """The library applies the branch norms inside out_proj for bf16 layers whose scan
    has the fused dt projection (dt_rank 64 or 128, d_state 16..128)."""
    return (dims.dtype == "bf16" and dims.dt_rank in (64, 128) and
            dims.d_state in (4, 8, 16, 32, 64, 128) and
            dims.d_inner % scan_channels(dims.d_state) == 0 and dims.q_width % 128 == 0)


def stage_work(dims, B, L):
    """Algorithmic work per prefill launch of each stage (flops or bytes)."""
    M, d, Di, N, R = dims.n_meta, dims.d_model, dims.d_inner, dims.d_state, dims.dt_rank
    rows = M + B * L
    qw = dims.q_width
    W = dims.window
    pairs_seq = sum(min(i + 1, W) if W > 0 else i + 1 for i in range(L)) + L * M
    pairs_meta = M * (M + 1) // 2
    attn_flops = 4 * dims.head_dim * dims.n_q_heads * (B * pairs_seq + pairs_meta)
    return {
        # the batch-shared meta rows go through in_proj, the scan and out_proj in
        # launches of their own
        "meta": ("mfma", 2.0 * M * (dims.n_in + dims.f_width) * d),
        "in_proj": ("mfma", 2.0 * B * L * dims.n_in * d),
        "attn": ("mfma", float(attn_flops)),
        "x_proj": ("mfma", 2.0 * rows * dims.n_xproj * Di),
        "dt_proj": ("mfma", 2.0 * rows * Di * R),
        # bytes: x, G, y (bf16) per (row, channel), delta (bf16) and B, C (fp32) per row,
        # h once; dt is computed in the scan and never stored.  The scan stage is the
        # launch over the B*L sequence rows (the meta rows are scanned once, in "meta")
        "scan": ("hbm", float(B * L * (Di * 6 + 2 * R + 8 * N) + B * Di * N * 4)),
        # bytes: bf16 prefill with the fused scan derives two factors per row from the
        # partial sums of squares (read), writes them, and rescales the meta rows of F in
        # place (out_proj applies the factors); otherwise the pass reads O and Y_ssm and
        # writes F
        "norm": ("hbm", float(rows * (dims.n_q_heads + Di // scan_channels(N)) * 4 + rows * 8 +
                              M * (qw + Di) * 2 * 2) if deferred_norm(dims) else
                 float(rows * (qw + Di) * 2 * 2)),
        "out_proj": ("mfma", 2.0 * B * L * dims.f_width * d),
    }


def roofline_entry(bound, work, avg_ms):
    if bound == "mfma":
        achieved = work / (avg_ms * 1e-3) / 1e12
        return {"bound": "mfma", "achieved": round(achieved, 2), "peak": PEAK_BF16_TFLOPS,
                "unit": "TFLOP/s", "frac": round(achieved / PEAK_BF16_TFLOPS, 4)}
    achieved = work / (avg_ms * 1e-3) / 1e9
    return {"bound": "hbm", "achieved": round(achieved, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
            "frac": round(achieved / PEAK_HBM_GBS, 4)}


def traffic_for(kernel_stage):
    """HBM bytes per launch measured by rocprofv3 counters (profiles/traffic.json), only
    while the kernel source it was taken on is unchanged."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(path):
        return None
    try:
        rec = json.load(open(path)).get(kernel_stage)
    except (OSError, ValueError):
        return None
    if not rec:
        return None
    h = hashlib.sha256()
    for name in rec["sources"]:
        src = os.path.join(ROOT, "hybrid_attention_ssm_proj_amd", "csrc", name)
        if not os.path.exists(src):
            return None
        h.update(open(src, "rb").read())
    return rec["bytes_per_launch"] if h.hexdigest()[:16] == rec["source_sha"] else None


def stage_pass(hy, torch, step, steps, mask):
    """Run `steps` steps with the stage timers in `mask` on; per-stage average launch time."""
    torch.cuda.synchronize()
    for i in range(len(hy.STAGES)):
        hy.hymba_timer_read(i)
    hy.hymba_timer_enable(mask)
    for _ in range(steps):
        step()
    torch.cuda.synchronize()
    hy.hymba_timer_enable(0)
    out = {}
    for i, name in enumerate(hy.STAGES):
        ms, n = hy.hymba_timer_read(i)
        if n:
            out[name] = {"avg_ms": ms / n, "per_step": n // steps}
    return out


def cpu_baseline(seqs):
    """The oracle (fp64 numpy) on `seqs` sequences of the prefill workload (2048 tokens
    plus the 128 meta tokens each)."""
    import numpy as np
    import oracle as orc
    from synth import CASES, gen_layer_weights, gen_activations
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:  # threadpoolctl missing: report the affinity size
        threads = len(os.sched_getaffinity(0))
    case = CASES[1]
    dims = case.dims
    w = gen_layer_weights(dims, case.case_id)
    _, meta, _, x = gen_activations(dims, case.case_id, seqs, case.seq_len)
    t0 = time.perf_counter()
    orc.prefill(dims, w, meta, x)
    dt = time.perf_counter() - t0
    tokens = seqs * case.seq_len
    return {"value": round(tokens / dt, 1), "unit": "tokens/s", "cores": int(threads),
            "kind": "oracle",
            "sample": f"{seqs} of the {case.batch} sequences of the prefill workload "
                      f"({case.seq_len} tokens + {dims.n_meta} meta tokens each, fp64 numpy), "
                      f"{dt:.1f} s"}


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (this layer is built and measured on a single "
              f"MI355X; requested --gpus {args.gpus})", file=sys.stderr)
        sys.exit(2)
    import torch
    import hybrid_attention_ssm_proj_amd as hy
    from synth import CASES, gen_layer_weights

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    dev = "cuda:0"
    torch.cuda.set_device(0)
    ceilings = measure_ceilings(hy, torch, dev)
    case = CASES[1]
    dims = case.dims
    B, L = case.batch, case.seq_len
    log(f"[bench] prefill workload {case.name}: B={B} L={L} M={dims.n_meta}")
    w = gen_layer_weights(dims, case.case_id)
    layer = hy.HymbaLayer(dims, w.torch, device=dev)
    gen = torch.Generator(device=dev)
    gen.manual_seed(1001)
    meta = torch.randn(dims.n_meta, dims.d_model, generator=gen, device=dev).to(torch.bfloat16)
    x = torch.randn(B, L, dims.d_model, generator=gen, device=dev).to(torch.bfloat16)
    y = torch.empty(B, L, dims.d_model, dtype=torch.bfloat16, device=dev)
    y_meta = torch.empty(dims.n_meta, dims.d_model, dtype=torch.bfloat16, device=dev)
    h = torch.empty(B, dims.d_inner, dims.d_state, dtype=torch.float32, device=dev)
    pos = torch.empty(B, dtype=torch.int32, device=dev)
    state = hy.make_state(h, pos)
    stream = torch.cuda.current_stream()

    def step():
        layer.prefill(meta, x, state_out=state, y=y, y_meta=y_meta, stream=stream)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    # 1) stage breakdown: every launch bracketed by HIP events (not the timed pass)
    stages = stage_pass(hy, torch, step, max(3, args.steps // 2), -1)
    work = stage_work(dims, B, L)
    dominant = max((n for n in stages if n in work),
                   key=lambda n: stages[n]["avg_ms"] * stages[n]["per_step"])
    dom_idx = hy.STAGES.index(dominant)

    # 2) timed pass: K steps between synchronisations, only the dominant kernel's
    #    launches bracketed by events (on the stream it runs on)
    for i in range(len(hy.STAGES)):
        hy.hymba_timer_read(i)
    hy.hymba_timer_enable(1 << dom_idx)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    hy.hymba_timer_enable(0)
    dom_ms, dom_n = hy.hymba_timer_read(dom_idx)
    ms_per_step = elapsed * 1e3 / args.steps
    tokens = B * L
    value = tokens / (elapsed / args.steps)
    log(f"[bench] prefill {ms_per_step:.3f} ms/step, {value / 1e6:.3f} M tokens/s")

    stage_report = {}
    for name, rec in stages.items():
        entry = {"avg_ms": round(rec["avg_ms"], 4), "launches_per_step": rec["per_step"]}
        if name in work:
            bound, wk = work[name]
            entry.update(roofline_entry(bound, wk / rec["per_step"], rec["avg_ms"]))
        if name == "scan":
            # exponentials rows * Di * N against the v_exp_f32 rate measured on this chip
            exps = B * L * dims.d_inner * dims.d_state
            rate = exps / (rec["avg_ms"] * 1e-3)
            entry["exp"] = {"achieved": round(rate / 1e12, 3), "peak": EXP_TPS["value"],
                            "unit": "Texp/s",
                            "frac": round(rate / 1e12 / EXP_TPS["value"], 4)}
        stage_report[name] = entry
    bound, wk = work[dominant]
    per_launch = wk / stages[dominant]["per_step"]
    roof = roofline_entry(bound, per_launch, dom_ms / dom_n)
    roof["kernel"] = dominant
    roof["avg_launch_ms"] = round(dom_ms / dom_n, 4)
    roof["work_per_launch"] = per_launch
    roof["traffic"] = traffic_for(dominant)
    if bound == "mfma" and ceilings.get("mfma_bf16_layer_data_tflops"):
        # context: the MFMA rate this chip sustains on operands with the layer's value
        # distributions (probe kind 3), beside the published peak the fraction uses
        md = ceilings["mfma_bf16_layer_data_tflops"]
        roof["measured_ceiling"] = {"value": md, "unit": "TFLOP/s",
                                    "frac": round(roof["achieved"] / md, 4),
                                    "probe": "MFMA loop on the layer's operand distributions"}
    log("[bench] stages: " + ", ".join(f"{k} {v['avg_ms']:.3f} ms x{v['launches_per_step']}"
                                       for k, v in stage_report.items()))

    # The same workload from a meta-prefix cache: the meta rows' K/V, post-meta SSM state
    # and y_meta built once per weight set (outside the timed region), then every step
    # runs the layer over X only.  Reported beside the headline, which recomputes the
    # meta rows every step.
    cache_t, cache = layer.build_meta_cache(meta, stream=stream)

    def step_cached():
        layer.prefill_cached(cache, x, state_out=state, y=y, stream=stream)

    for _ in range(args.warmup):
        step_cached()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step_cached()
    torch.cuda.synchronize()
    el_c = time.perf_counter() - t0
    cached = {"value": round(tokens / (el_c / args.steps), 1), "unit": "tokens/s",
              "ms_per_step": round(el_c * 1e3 / args.steps, 4),
              "workload": "same prefill from a meta-prefix cache built once per weight set"}
    log(f"[bench] prefill from the meta cache {cached['ms_per_step']:.3f} ms/step, "
        f"{cached['value'] / 1e6:.3f} M tokens/s")
    del cache_t

    if args.copy_calibration > 0:
        n = args.copy_calibration
        src = torch.empty(n, dtype=torch.uint8, device=dev)
        dst = torch.empty(n, dtype=torch.uint8, device=dev)
        torch.cuda.synchronize()
        hy.hymba_op_copy(src, dst, n, stream=stream)
        torch.cuda.synchronize()
        log(f"[bench] copy calibration: {n} bytes")
        del src, dst

    decode = None
    if not args.no_decode:
        decode = bench_decode(hy, torch, dev, args)

    stack = None
    if not args.no_stack:
        stack = bench_stack(hy, torch, dev)

    pair = long_ctx = None
    if not args.no_long:
        pair = bench_pair(hy, torch, dev, args)
        long_ctx = bench_long(hy, torch, dev, args)

    head_ssm = group_norm = block = None
    if not args.no_head_ssm:
        head_ssm = bench_head_ssm(hy, torch, dev, args, stages)
        group_norm = bench_group_norm(hy, torch, dev, args, stages)
        block = bench_block(hy, torch, dev, args, ms_per_step)

    cpu = None
    if not args.no_cpu_baseline:
        log("[bench] timing the CPU oracle sample")
        cpu = cpu_baseline(args.cpu_seqs)

    out = {
        "metric": METRIC, "value": round(value, 1), "unit": "tokens/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "hymba hybrid-head layer prefill, bf16, B=8, L=2048, 128 meta "
                               "tokens, d=2048, 16x128 q / 4 kv heads, full causal, Di=4096, N=16",
                   "global_batch": B, "seq_len": L, "n_meta": dims.n_meta},
        "roofline": roof,
        "cpu_baseline": cpu,
        "decode": decode,
        "prefill_meta_cached": cached,
        "stack": stack,
        "layer_pair": pair,
        "long_context": long_ctx,
        "head_ssm": head_ssm,
        "group_norm": group_norm,
        "block": block,
        "stages": stage_report,
        "ceilings_measured": ceilings,
    }
    print(json.dumps(out), flush=True)


def prefill_variant(hy, torch, dev, args, dims, seed):
    """Prefill of the prefill workload with layer `dims`: (ms per step, stage times)."""
    from synth import CASES, gen_layer_weights
    case = CASES[1]
    B, L, M = case.batch, case.seq_len, dims.n_meta
    w = gen_layer_weights(dims, case.case_id)
    layer = hy.HymbaLayer(dims, w.torch, device=dev)
    gen = torch.Generator(device=dev)
    gen.manual_seed(seed)
    meta = torch.randn(M, dims.d_model, generator=gen, device=dev).to(torch.bfloat16)
    x = torch.randn(B, L, dims.d_model, generator=gen, device=dev).to(torch.bfloat16)
    y = torch.empty(B, L, dims.d_model, dtype=torch.bfloat16, device=dev)
    y_meta = torch.empty(M, dims.d_model, dtype=torch.bfloat16, device=dev)
    h = torch.empty(B, dims.d_inner, dims.d_state, dtype=torch.float32, device=dev)
    pos = torch.empty(B, dtype=torch.int32, device=dev)
    state = hy.make_state(h, pos)
    stream = torch.cuda.current_stream()

    def step():
        layer.prefill(meta, x, state_out=state, y=y, y_meta=y_meta, stream=stream)

    for _ in range(args.warmup):
        step()
    stages = stage_pass(hy, torch, step, max(3, args.steps // 2), -1)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    ms = (time.perf_counter() - t0) / args.steps * 1e3
    del layer
    torch.cuda.empty_cache()
    return ms, stages


def _scan_entry(dims, B, L, rec):
    """The sequence launch of the scan: its time, its algorithmic HBM bytes (x, G, y bf16
    per (row, channel); delta bf16, B and C fp32 per row; h once) and exponentials
    (rows x Di x N) against the v_exp_f32 rate of this chip."""
    Di, N, R = dims.d_inner, dims.d_state, dims.dt_rank
    rows = B * L
    nbytes = rows * (Di * 6 + 2 * R + 8 * N) + B * Di * N * 4
    exps = rows * Di * N
    ms = rec["avg_ms"]
    out = roofline_entry("hbm", nbytes, ms)
    out["avg_ms"] = round(ms, 4)
    out["exp"] = {"achieved": round(exps / (ms * 1e-3) / 1e12, 3), "peak": EXP_TPS["value"],
                  "unit": "Texp/s",
                  "frac": round(exps / (ms * 1e-3) / 1e12 / EXP_TPS["value"], 4)}
    return out


def _layer_io(torch, dims, B, L, seed, dev):
    gen = torch.Generator(device=dev)
    gen.manual_seed(seed)
    meta = torch.randn(dims.n_meta, dims.d_model, generator=gen, device=dev).to(torch.bfloat16)
    x = torch.randn(B, L, dims.d_model, generator=gen, device=dev).to(torch.bfloat16)
    return meta, x


def bench_pair(hy, torch, dev, args):
    """The layer-pair workload: two sliding-window layers (window 1024) over B=4, L=8192
    with 128 meta tokens; the first is a producer keeping every position of its K/V, the
    second a consumer reading them (cross-layer KV sharing).  Layer 2 takes layer 1's y
    and y_meta.  tokens/s counts B*L per pair; stage times are per layer."""
    from synth import CASES
    case = CASES[2]
    p_dims = case.dims
    c_dims = p_dims.replace(kv_share=1)
    B, L, M = case.batch, case.seq_len, p_dims.n_meta
    log(f"[bench] layer pair {case.name}: B={B} L={L} W={p_dims.window}")
    l1 = hy.HymbaLayer(p_dims, device_weights(torch, p_dims, 2001, dev), device=dev)
    l2 = hy.HymbaLayer(c_dims, device_weights(torch, c_dims, 2002, dev), device=dev)
    meta, x = _layer_io(torch, p_dims, B, L, 2003, dev)
    Hkv, dh = p_dims.n_kv_heads, p_dims.head_dim
    kv = {n: torch.empty(shape, dtype=torch.bfloat16, device=dev) for n, shape in (
        ("k_meta", (Hkv, M, dh)), ("v_meta", (Hkv, M, dh)), ("k", (B, Hkv, L, dh)),
        ("v", (B, Hkv, L, dh)))}
    kvs = hy.make_kv(kv["k_meta"], kv["v_meta"], kv["k"], kv["v"])
    y1 = torch.empty(B, L, p_dims.d_model, dtype=torch.bfloat16, device=dev)
    y2 = torch.empty_like(y1)
    ym1 = torch.empty(M, p_dims.d_model, dtype=torch.bfloat16, device=dev)
    ym2 = torch.empty_like(ym1)
    stream = torch.cuda.current_stream()

    def step():
        l1.prefill(meta, x, kv_out=kvs, y=y1, y_meta=ym1, stream=stream)
        l2.prefill(ym1, y1, kv_in=kvs, y=y2, y_meta=ym2, stream=stream)

    for _ in range(max(1, args.warmup)):
        step()
    stages = stage_pass(hy, torch, step, 3, -1)
    steps = max(3, args.steps // 4)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        step()
    torch.cuda.synchronize()
    ms = (time.perf_counter() - t0) / steps * 1e3
    scan = _scan_entry(p_dims, B, L, {"avg_ms": stages["scan"]["avg_ms"]})
    del l1, l2, kv, y1, y2
    torch.cuda.empty_cache()
    log(f"[bench] layer pair: {ms:.3f} ms per pair, {B * L / ms / 1e3:.3f} M tokens/s; "
        f"scan {scan['avg_ms']:.3f} ms per layer")
    return {"workload": "two layers, bf16, B=4, L=8192, 128 meta tokens, window 1024; the "
                        "second reuses the first's K/V; d=2048, 16x128 q / 4 kv heads, "
                        "Di=4096, N=16",
            "value": round(B * L / ms * 1e3, 1), "unit": "tokens/s", "ms_per_pair": round(ms, 4),
            "scan_per_layer": scan,
            "stages_ms_per_layer": {k: round(v["avg_ms"] * v["per_step"] / 2, 4)
                                    for k, v in stages.items()}}


def bench_long(hy, torch, dev, args):
    """The long-context workload: one layer, B=1, L=32768 after 128 meta tokens, window
    1024, state 128.  The scan runs in time chunks chosen by the library; the same
    layer with one chunk (the plain serial scan) is timed beside it."""
    from synth import CASES
    case = CASES[3]
    dims = case.dims
    B, L, M = case.batch, case.seq_len, dims.n_meta
    log(f"[bench] long context {case.name}: B={B} L={L} N={dims.d_state}")
    w = device_weights(torch, dims, 3001, dev)
    meta, x = _layer_io(torch, dims, B, L, 3002, dev)
    y = torch.empty(B, L, dims.d_model, dtype=torch.bfloat16, device=dev)
    ym = torch.empty(M, dims.d_model, dtype=torch.bfloat16, device=dev)
    h = torch.empty(B, dims.d_inner, dims.d_state, device=dev)
    pos = torch.empty(B, dtype=torch.int32, device=dev)
    state = hy.make_state(h, pos)
    stream = torch.cuda.current_stream()
    out = {"workload": "one layer, bf16, B=1, L=32768, 128 meta tokens, window 1024, d=2048, "
                       "16x128 q / 4 kv heads, Di=4096, N=128"}
    for name, chunk in (("chunked", 0), ("one_chunk", L)):
        layer = hy.HymbaLayer(dims.replace(scan_chunk=chunk), w, device=dev)

        def step():
            layer.prefill(meta, x, state_out=state, y=y, y_meta=ym, stream=stream)

        step()
        stages = stage_pass(hy, torch, step, 2, -1)
        if name == "chunked":
            steps = max(3, args.steps // 4)
            torch.cuda.synchronize()
            t0 = time.perf_counter()
            for _ in range(steps):
                step()
            torch.cuda.synchronize()
            ms = (time.perf_counter() - t0) / steps * 1e3
            out.update(value=round(B * L / ms * 1e3, 1), unit="tokens/s", ms_per_step=round(ms, 4),
                       scan=_scan_entry(dims, B, L, stages["scan"]),
                       stages_ms={k: round(v["avg_ms"] * v["per_step"], 4)
                                  for k, v in stages.items()})
        else:
            out["one_chunk_scan_ms"] = round(stages["scan"]["avg_ms"], 4)
        del layer
        torch.cuda.empty_cache()
    log(f"[bench] long context: {out['ms_per_step']:.3f} ms/step, "
        f"{out['value'] / 1e6:.3f} M tokens/s; scan {out['scan']['avg_ms']:.3f} ms "
        f"(one chunk: {out['one_chunk_scan_ms']:.3f} ms)")
    return out


def bench_block(hy, torch, dev, args, layer_ms):
    """The prefill workload through the block wrapper: pre-norm, the layer, residual, FFN
    (intermediate 5632, SiLU), residual.  Reports the step, the FFN's two GEMMs against
    the bf16 MFMA peak, and the block's cost over the bare layer."""
    from synth import CASES, gen_block_weights, gen_layer_weights
    case = CASES[1]
    dims, inter = case.dims, 5632
    B, L, M = case.batch, case.seq_len, dims.n_meta
    log(f"[bench] block wrapper: intermediate={inter}")
    w = gen_layer_weights(dims, case.case_id)
    bw = gen_block_weights(dims, case.case_id, inter)
    blk = hy.HymbaBlock(dims, w.torch, bw.torch, device=dev)
    gen = torch.Generator(device=dev)
    gen.manual_seed(1007)
    meta = torch.randn(M, dims.d_model, generator=gen, device=dev).to(torch.bfloat16)
    x = torch.randn(B, L, dims.d_model, generator=gen, device=dev).to(torch.bfloat16)
    y = torch.empty(B, L, dims.d_model, dtype=torch.bfloat16, device=dev)
    y_meta = torch.empty(M, dims.d_model, dtype=torch.bfloat16, device=dev)
    stream = torch.cuda.current_stream()

    def step():
        blk.prefill(meta, x, y=y, y_meta=y_meta, stream=stream)

    for _ in range(args.warmup):
        step()
    stages = stage_pass(hy, torch, step, max(3, args.steps // 2), 1 << hy.STAGES.index("block"))
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    ms = (time.perf_counter() - t0) / args.steps * 1e3
    rows = M + B * L
    ffn_flop = 2 * 2 * rows * dims.d_model * inter
    blk_ms = stages["block"]["avg_ms"] * stages["block"]["per_step"]
    del blk
    torch.cuda.empty_cache()
    log(f"[bench] block wrapper: prefill {ms:.3f} ms ({B * L / ms / 1e3:.3f} M tok/s), "
        f"wrapper kernels {blk_ms:.3f} ms per step")
    out = {"workload": "the prefill workload through the block wrapper (pre-norm, residual, "
                       "FFN with intermediate 5632 and SiLU)",
           "prefill_ms": round(ms, 4), "prefill_tokens_per_s": round(B * L / ms * 1e3, 1),
           "layer_prefill_ms": round(layer_ms, 4),
           "wrapper_ms_per_step": round(blk_ms, 4),
           "ffn_flop_per_step": ffn_flop,
           "ffn_and_norms_tflops": round(ffn_flop / (blk_ms * 1e-3) / 1e12, 1)}
    if not args.no_decode:
        dec = bench_decode(hy, torch, dev, args, block_inter=inter)
        out["decode_us_per_step"] = dec["us_per_step"]
        out["decode_tokens_per_s"] = dec["value"]
        out["decode_hbm_frac_of_peak"] = dec["hbm_frac_of_peak"]
        out["decode_block_us"] = dec["stage_us"].get("block", {}).get("us")
    return out


def bench_group_norm(hy, torch, dev, args, default_stages):
    """The prefill workload with the group-normalisation fusion (groups of 128 channels):
    the branch norms can no longer be folded into out_proj as per-row factors, so F is
    normalised in place by one pass (reads and writes F once)."""
    from synth import CASES
    case = CASES[1]
    dims = case.dims.replace(norm_group=128)
    B, L = case.batch, case.seq_len
    log(f"[bench] group-norm variant: norm_group={dims.norm_group}")
    ms, stages = prefill_variant(hy, torch, dev, args, dims, 1006)
    rows = dims.n_meta + B * L
    f_bytes = 2 * rows * dims.f_width * 2
    norm_ms = stages["norm"]["avg_ms"]
    achieved = f_bytes / (norm_ms * 1e-3) / 1e9
    log(f"[bench] group-norm variant: prefill {ms:.3f} ms ({B * L / ms / 1e3:.3f} M tok/s), "
        f"norm pass {norm_ms:.3f} ms ({achieved:.0f} GB/s)")
    return {"workload": "the prefill workload with group normalisation of each branch in "
                        "groups of 128 channels",
            "prefill_ms": round(ms, 4), "prefill_tokens_per_s": round(B * L / ms * 1e3, 1),
            "norm_ms": round(norm_ms, 4),
            "default_norm_ms": round(default_stages["norm"]["avg_ms"], 4),
            "norm_roofline": {"bound": "hbm", "achieved": round(achieved, 1),
                              "peak": PEAK_HBM_GBS, "unit": "GB/s",
                              "frac": round(achieved / PEAK_HBM_GBS, 4),
                              "bytes_per_launch": f_bytes},
            "stages_ms": {k: round(v["avg_ms"], 4) for k, v in stages.items()}}


def bench_head_ssm(hy, torch, dev, args, mamba_stages):
    """The same prefill and decode workloads with the Mamba-2 SSM head (64 heads of 64
    channels, scalar A and dt per head): the scan runs in the chunked matrix form on MFMA.
    Reports step times, the scan's time against the Mamba head's, and the scan's HBM
    roofline (it reads x, G and [u | B | C] per token of every sequence, the meta prefix
    included, and writes y once per row and the final state)."""
    from synth import CASES, gen_layer_weights
    case = CASES[1]
    dims = case.dims.replace(ssm_heads=64, dt_rank=0)
    B, L, M = case.batch, case.seq_len, dims.n_meta
    log(f"[bench] head-SSM variant: ssm_heads={dims.ssm_heads}, prefill B={B} L={L}")
    w = gen_layer_weights(dims, case.case_id)
    layer = hy.HymbaLayer(dims, w.torch, device=dev)
    gen = torch.Generator(device=dev)
    gen.manual_seed(1005)
    meta = torch.randn(M, dims.d_model, generator=gen, device=dev).to(torch.bfloat16)
    x = torch.randn(B, L, dims.d_model, generator=gen, device=dev).to(torch.bfloat16)
    y = torch.empty(B, L, dims.d_model, dtype=torch.bfloat16, device=dev)
    y_meta = torch.empty(M, dims.d_model, dtype=torch.bfloat16, device=dev)
    h = torch.empty(B, dims.d_inner, dims.d_state, dtype=torch.float32, device=dev)
    pos = torch.empty(B, dtype=torch.int32, device=dev)
    state = hy.make_state(h, pos)
    stream = torch.cuda.current_stream()

    def step():
        layer.prefill(meta, x, state_out=state, y=y, y_meta=y_meta, stream=stream)

    for _ in range(args.warmup):
        step()
    stages = stage_pass(hy, torch, step, max(3, args.steps // 2), -1)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    ms = (time.perf_counter() - t0) / args.steps * 1e3
    T, Di, N, H = M + L, dims.d_inner, dims.d_state, dims.ssm_heads
    scan_bytes = B * T * (2 * Di * 2 + (H + 2 * N) * 4) + (M + B * L) * Di * 2 + B * Di * N * 4
    scan_ms = stages["scan"]["avg_ms"]
    achieved = scan_bytes / (scan_ms * 1e-3) / 1e9
    del layer
    torch.cuda.empty_cache()
    dec = None if args.no_decode else bench_decode(hy, torch, dev, args, dims=CASES[4].dims.replace(
        ssm_heads=64, dt_rank=0))
    out = {"workload": f"the prefill workload with the Mamba-2 SSM head: {H} heads of "
                       f"{Di // H} channels, one dt and A per head, N={N}",
           "prefill_ms": round(ms, 4), "prefill_tokens_per_s": round(B * L / ms * 1e3, 1),
           "scan_ms": round(scan_ms, 4),
           "mamba_head_scan_ms": round(mamba_stages["scan"]["avg_ms"], 4),
           "scan_roofline": {"bound": "hbm", "achieved": round(achieved, 1),
                             "peak": PEAK_HBM_GBS, "unit": "GB/s",
                             "frac": round(achieved / PEAK_HBM_GBS, 4),
                             "bytes_per_launch": scan_bytes},
           "stages_ms": {k: round(v["avg_ms"], 4) for k, v in stages.items()}}
    if dec is not None:
        out["decode_us_per_step"] = dec["us_per_step"]
        out["decode_tokens_per_s"] = dec["value"]
    log(f"[bench] head-SSM variant: prefill {ms:.3f} ms ({B * L / ms / 1e3:.3f} M tok/s), "
        f"scan {scan_ms:.3f} ms (Mamba head {mamba_stages['scan']['avg_ms']:.3f} ms), "
        f"{achieved:.0f} GB/s" + (f"; decode {dec['us_per_step']} us/step" if dec else ""))
    return out


def device_weights(torch, dims, seed, dev):
    """Synthetic weights of one layer drawn on the device (the distributions of the
    seeded CPU generator: W ~ N(0, 0.02), dt_bias ~ U[-4, -2], A = -exp(U[0, 2]),
    D ~ N(0, 1), beta = 1), for stacks too large to draw on the host quickly."""
    g = torch.Generator(device=dev)
    g.manual_seed(seed)
    bf = torch.bfloat16
    n = lambda *sh, std=0.02: (torch.randn(*sh, generator=g, device=dev) * std)
    u = lambda lo, hi, *sh: torch.rand(*sh, generator=g, device=dev) * (hi - lo) + lo
    Di, N, R = dims.d_inner, dims.d_state, dims.dt_rank
    return {"w_in": n(dims.n_in, dims.d_model).to(bf), "w_x": n(R + 2 * N, Di).to(bf),
            "w_dt": n(Di, R).to(bf), "w_out": n(dims.d_model, dims.f_width).to(bf),
            "dt_bias": u(-4, -2, Di), "A": -torch.exp(u(0, 2, Di, N)),
            "D": n(Di, std=1.0), "beta_attn": torch.ones(dims.q_width, device=dev),
            "beta_ssm": torch.ones(Di, device=dev)}


def bench_stack(hy, torch, dev, n_layers=16, B=1, L=8192, W=1024, dsteps=16, steps=3):
    """The partial sliding-window schedule with KV-sharing pairs (global attention at the
    first, middle and last layers) against an all-global stack of the same depth: prefill
    tokens/s, decode tokens/s and the K/V bytes kept for decode."""
    from hybrid_attention_ssm_proj_amd.stack import HymbaStack
    from synth import CASES
    dims = CASES[1].dims
    gen = torch.Generator(device=dev)
    gen.manual_seed(7)
    meta = torch.randn(dims.n_meta, dims.d_model, generator=gen, device=dev).to(torch.bfloat16)
    x = torch.randn(B, L + dsteps, dims.d_model, generator=gen, device=dev).to(torch.bfloat16)
    xp = x[:, :L].contiguous()
    res = {}
    for name, win in (("partial_swa", W), ("all_global", 0)):
        st = HymbaStack(dims, n_layers, lambda l, ld: device_weights(torch, ld, 1000 + l, dev),
                        win, device=dev)
        st.alloc(B, L, L + 2 * dsteps)
        st.prefill(meta, xp)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(steps):
            st.prefill(meta, xp)
        torch.cuda.synchronize()
        tp = (time.perf_counter() - t0) / steps
        t0 = time.perf_counter()
        for s in range(dsteps):
            st.decode(x[:, L + s].contiguous())
        torch.cuda.synchronize()
        td = (time.perf_counter() - t0) / dsteps
        # the same steps replayed from a HIP graph of one whole-stack decode step (the
        # caches have room for 2 * dsteps positions past the prompt)
        xs = torch.empty_like(x[:, L])
        g, _ = st.capture_decode(xs)
        t0 = time.perf_counter()
        for s in range(dsteps):
            xs.copy_(x[:, L + s])
            g.replay()
        torch.cuda.synchronize()
        tg = (time.perf_counter() - t0) / dsteps
        del g
        res[name] = {"prefill_ms": round(tp * 1e3, 3), "prefill_tokens_per_s": round(B * L / tp, 1),
                     "decode_us_per_step": round(td * 1e6, 1),
                     "decode_tokens_per_s": round(B / td, 1),
                     "decode_graph_us_per_step": round(tg * 1e6, 1),
                     "decode_cache_bytes": st.decode_cache_bytes(B, L + dsteps),
                     "global_layers": [l for l, sc in enumerate(st.sched) if sc[0] == 0],
                     "consumers": [l for l, sc in enumerate(st.sched) if sc[1] == 1]}
        log(f"[bench] stack {name}: prefill {tp * 1e3:.2f} ms ({B * L / tp / 1e6:.3f} M tok/s), "
            f"decode {td * 1e6:.1f} us/step (graph {tg * 1e6:.1f}), "
            f"cache {res[name]['decode_cache_bytes'] / 1e6:.1f} MB")
        del st
        torch.cuda.empty_cache()
    a, g = res["partial_swa"], res["all_global"]
    res["ratios"] = {"prefill_speedup": round(g["prefill_ms"] / a["prefill_ms"], 3),
                     "decode_speedup": round(g["decode_us_per_step"] / a["decode_us_per_step"], 3),
                     "decode_graph_speedup": round(g["decode_graph_us_per_step"] /
                                                   a["decode_graph_us_per_step"], 3),
                     "cache_reduction": round(g["decode_cache_bytes"] / a["decode_cache_bytes"], 3)}
    res["workload"] = (f"{n_layers} layers of the prefill layer shape, B={B}, L={L}, window {W}, "
                       f"then {dsteps} decode steps; layer l+1 takes layer l's y and y_meta")
    return res


def bench_decode(hy, torch, dev, args, dims=None, block_inter=0):
    """The decode workload (config 4) on the layer, or (block_inter > 0) on the layer
    inside its block wrapper with that FFN intermediate size."""
    from synth import CASES, gen_block_weights, gen_layer_weights
    case = CASES[4]
    dims = dims or case.dims
    B, S, prior = case.batch, case.ring_slots, case.prior_tokens
    log(f"[bench] decode workload {case.name}: B={B} ring={S} prior={prior}"
        f"{' ssm_heads=%d' % dims.ssm_heads if dims.ssm_heads else ''}"
        f"{' block intermediate=%d' % block_inter if block_inter else ''}")
    w = gen_layer_weights(dims, case.case_id)
    if block_inter:
        bw = gen_block_weights(dims, case.case_id, block_inter)
        layer = hy.HymbaBlock(dims, w.torch, bw.torch, device=dev)
    else:
        layer = hy.HymbaLayer(dims, w.torch, device=dev)
    gen = torch.Generator(device=dev)
    gen.manual_seed(1004)
    Hkv, M, dh = dims.n_kv_heads, dims.n_meta, dims.head_dim
    kv = {n: torch.zeros(shape, dtype=torch.bfloat16, device=dev) for n, shape in (
        ("k_meta", (Hkv, M, dh)), ("v_meta", (Hkv, M, dh)), ("k", (B, Hkv, S, dh)),
        ("v", (B, Hkv, S, dh)))}
    h = torch.zeros(B, dims.d_inner, dims.d_state, dtype=torch.float32, device=dev)
    pos = torch.zeros(B, dtype=torch.int32, device=dev)
    kvs = hy.make_kv(kv["k_meta"], kv["v_meta"], kv["k"], kv["v"])
    sts = hy.make_state(h, pos)
    # state: the library's own prefill over `prior` N(0,1) tokens per sequence, in
    # batch slices (fills the ring with the last 1024 positions and h, pos = prior).
    meta = torch.randn(M, dims.d_model, generator=gen, device=dev).to(torch.bfloat16)
    slice_b = 16
    for b0 in range(0, B, slice_b):
        xs = torch.randn(slice_b, prior, dims.d_model, generator=gen, device=dev).to(torch.bfloat16)
        sub_kv = hy.make_kv(kv["k_meta"], kv["v_meta"], kv["k"][b0:b0 + slice_b],
                            kv["v"][b0:b0 + slice_b])
        sub_st = hy.make_state(h[b0:b0 + slice_b], pos[b0:b0 + slice_b])
        layer.prefill(meta, xs, kv_out=sub_kv, state_out=sub_st)
        del xs
    torch.cuda.synchronize()
    layer._ws = None
    torch.cuda.empty_cache()
    steps = args.decode_steps
    xin = torch.randn(steps + 4, B, dims.d_model, generator=gen, device=dev).to(torch.bfloat16)
    yout = torch.empty(B, dims.d_model, dtype=torch.bfloat16, device=dev)
    stream = torch.cuda.current_stream()
    for s in range(4):  # warm-up steps advance the state like any other step
        layer.decode(xin[steps + s], kvs, sts, y=yout, stream=stream)
    torch.cuda.synchronize()
    # breakdown on a copy of the state so the timed span starts from the same place
    saved = {k: v.clone() for k, v in kv.items()}, h.clone(), pos.clone()
    n_break = min(32, steps)
    it = iter(range(n_break))
    st_rec = stage_pass(hy, torch, lambda: layer.decode(xin[next(it)], kvs, sts, y=yout,
                                                         stream=stream), n_break, -1)
    for k, v in saved[0].items():
        kv[k].copy_(v)
    h.copy_(saved[1])
    pos.copy_(saved[2])
    del saved
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for s in range(steps):
        layer.decode(xin[s], kvs, sts, y=yout, stream=stream)
    torch.cuda.synchronize()
    span = time.perf_counter() - t0
    # the same steps replayed from a HIP graph of 8 consecutive decode steps (inputs
    # xin[0..7], outputs into yout): the kernels without host launch gaps; every replay
    # advances the ring, the positions and the SSM state like eager steps
    g_steps = 8
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        cs = torch.cuda.current_stream()
        for s in range(g_steps):
            layer.decode(xin[s], kvs, sts, y=yout, stream=cs)
    torch.cuda.synchronize()
    reps = max(1, steps // g_steps)
    t0 = time.perf_counter()
    for _ in range(reps):
        graph.replay()
    torch.cuda.synchronize()
    g_us = (time.perf_counter() - t0) / (reps * g_steps) * 1e6
    del graph
    st = {name: {"us": round(r["avg_ms"] * 1e3, 2), "launches_per_step": r["per_step"]}
          for name, r in st_rec.items()}
    # algorithmic bytes per step: weights, ring K/V read, meta K/V, state read + write
    wbytes = 2 * (dims.n_in * dims.d_model + dims.n_xproj * dims.d_inner +
                  dims.d_inner * dims.dt_rank + dims.d_model * dims.f_width +
                  2 * dims.d_model * block_inter)
    ring_bytes = B * dims.n_kv_heads * min(S, dims.window) * dims.head_dim * 2 * 2
    meta_bytes = dims.n_kv_heads * M * dh * 2 * 2
    h_bytes = B * dims.d_inner * dims.d_state * 4 * 2
    step_bytes = wbytes + ring_bytes + meta_bytes + h_bytes
    us = span / steps * 1e6
    tps = B * steps / span
    log(f"[bench] decode {us:.1f} us/step, {tps / 1e6:.3f} M tokens/s "
        f"(HIP graph of {g_steps} steps: {g_us:.1f} us/step)")
    return {"value": round(tps, 1), "unit": "tokens/s", "us_per_step": round(us, 2),
            "steps": steps, "batch": B,
            "graph": {"us_per_step": round(g_us, 2), "tokens_per_s": round(B / g_us * 1e6, 1),
                      "steps_per_graph": g_steps, "replays": reps},
            "workload": "decode, bf16, B=128, 1 token per sequence after 4096 prior tokens, "
                        "window 1024 ring + 128 meta entries, same layer shape" +
                        (f", inside the block wrapper (FFN {block_inter})" if block_inter else ""),
            "hbm_bytes_per_step": step_bytes,
            "hbm_frac_of_peak": round(step_bytes / (span / steps) / 1e9 / PEAK_HBM_GBS, 4),
            "stage_us": st}


if __name__ == "__main__":
    main()
