#!/usr/bin/env python3
"""Phi-3-mini-shape f16 prefill benchmark on one MI355X.

One step = one full prefill forward (embedding, 32 decoder layers, final norm,
lm_head) over a batch of synthetic ids, ids -> fp32 logits at every position,
through the C ABI.  Weights (seeded N(0, 0.02), float16) and ids are resident
in HBM before the timed region.  Printed as one JSON line:

  value         prefill tokens/s (batch * seq * steps / wall time of the
                timed steps, bracketed by device synchronisation)
  roofline      the dominant kernel (fused gate/up GEMM + SiLU*up): its
                launches inside forwards run right after the timed steps,
                timed by HIP events that the library attaches to each of its
                dispatches on the forward's stream (the kernel's own run
                time, as a kernel trace measures it); algorithmic flops 2 * T * 2I * H per
                launch against the f16 MFMA peak; HBM traffic per launch from
                the committed counter summary (null if the kernel changed)
  decode        K16/V8 decode attention per call at the two Phi-4 shapes,
                algorithmic bytes per call against HBM bandwidth; HBM
                traffic per call from the committed counter summary (null
                if the kernel changed)
  cpu_baseline  the fp64 oracle on the host, on the first positions of the
                same ids (a bounded sample), with the parity of those rows
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

MFMA_F16_PEAK_TFLOPS = 2500.0  # MI355X dense f16 MFMA
HBM_PEAK_GBS = 8000.0           # MI355X HBM3E


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def measured_traffic(profile: str, source: str, key: str = "traffic_bytes_per_launch"):
    """HBM-side bytes per launch (the `key` line) from a committed counter
    summary, or None when the kernel source has changed since the counters
    were taken."""
    import hashlib
    try:
        text = open(os.path.join(ROOT, "profiles", profile)).read()
        fields = dict(l.split(": ", 1) for l in text.splitlines() if l.startswith(("traffic_bytes", "kernel_source")))
        digest = hashlib.sha256(open(os.path.join(ROOT, source), "rb").read()).hexdigest()
        if fields.get("kernel_source_sha256", "").strip() != digest:
            return None
        return int(fields[key])
    except (OSError, KeyError, ValueError):
        return None


def prefill_flops(cfg, batch, seq) -> float:
    n_lin = sum(n * k for n, k in cfg.linear_shapes().values()) * cfg.n_layers + cfg.vocab * cfg.hidden
    attn = cfg.n_layers * batch * 4 * cfg.n_heads * cfg.head_dim * seq * (seq + 1) / 2
    return 2.0 * n_lin * batch * seq + attn


def profile_forwards(model, ids, logits, workspace, stream, n):
    """Per-stage device time over n forwards, from HIP events that the library
    attaches to each of its kernel dispatches on the forward's stream."""
    model.profile_enable(True)
    for _ in range(n):
        model.prefill_logits(ids, logits, workspace, stream)
    prof = model.profile_read()
    model.profile_enable(False)
    return prof


def decode_bytes(wl) -> int:
    """Algorithmic bytes of one decode-attention call: every cached key (2 B)
    and value (1 B) element once, plus q, out, scales, block table, lengths."""
    D = wl.head_dim
    kv = wl.batch * wl.ctx * wl.n_kv_heads * D * 3
    return kv + wl.batch * wl.n_q_heads * D * 2 * 2 + wl.n_kv_heads * 4 + wl.n_pages * 4 + wl.batch * 4


def time_decode(phi, torch, np, synth, wl, reps=200):
    d = synth.decode_inputs(wl)
    t = lambda x: torch.from_numpy(np.ascontiguousarray(x)).cuda()
    q, vs, bt, cl = t(d.q), t(d.v_scale), t(d.block_table), t(d.ctx_lens)
    pool_bytes = d.k_pool.nbytes + d.v_pool.nbytes
    # rotate distinct copies so that each call streams its cache from HBM, not the 256 MB MALL
    copies = max(2, -(-1024 * 2 ** 20 // pool_bytes))
    kp0, vp0 = t(d.k_pool), t(d.v_pool)
    pools = [(kp0, vp0)] + [(kp0.clone(), vp0.clone()) for _ in range(copies - 1)]
    out = torch.empty((wl.batch, wl.n_q_heads, wl.head_dim), dtype=torch.float16, device="cuda")
    ws = torch.empty(phi.attn_decode_k16v8_workspace_bytes(wl.batch, wl.n_q_heads, wl.n_kv_heads, wl.head_dim,
                                                           wl.ctx), dtype=torch.uint8, device="cuda")
    stream = torch.cuda.current_stream()
    sm = 1 / np.sqrt(wl.head_dim)
    for i in range(10):
        kp, vp = pools[i % copies]
        phi.attn_decode_k16v8(q, kp, vp, vs, bt, cl, wl.ctx, sm, out=out, workspace=ws, stream=stream)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record(stream)
    for i in range(reps):
        kp, vp = pools[i % copies]
        phi.attn_decode_k16v8(q, kp, vp, vs, bt, cl, wl.ctx, sm, out=out, workspace=ws, stream=stream)
    e1.record(stream)
    torch.cuda.synchronize()
    us = e0.elapsed_time(e1) * 1e3 / reps
    nbytes = decode_bytes(wl)
    gbs = nbytes / (us * 1e-6) / 1e9
    return {"workload": wl.name, "us_per_call": round(us, 2), "bytes_per_call": nbytes,
            "roofline": {"bound": "hbm", "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                         "frac": round(gbs / HBM_PEAK_GBS, 4),
                         "traffic": measured_traffic("decode_k16v8_traffic.md", "logits_parity_amd/csrc/decode.hpp",
                                                     f"traffic_bytes_per_call_{wl.name}")},
            "cache_copies_rotated": copies}


def cpu_baseline(cfg, ws, ids_np, gpu_logits, positions):
    """The fp64 oracle as it stands on the first `positions` ids of the same
    input; causal prefix invariance makes those rows comparable to the GPU's."""
    import numpy as np
    from oracle import parity, prefill
    threads = os.cpu_count()
    try:
        from threadpoolctl import threadpool_info
        info = [p for p in threadpool_info() if p.get("internal_api") in ("openblas", "mkl", "blis")]
        if info:
            threads = max(p["num_threads"] for p in info)
    except Exception:
        pass
    sample = ids_np[:, :positions]
    t0 = time.perf_counter()
    ref = prefill.prefill_logits(cfg, ws, sample)
    dt = time.perf_counter() - t0
    s = parity.summary(gpu_logits[:, :positions].reshape(-1, cfg.vocab), ref.reshape(-1, cfg.vocab))
    base = {"value": round(sample.size / dt, 3), "unit": "tokens/s", "cores": threads, "kind": "oracle",
            "sample": f"fp64 numpy oracle, all {cfg.n_layers} layers + lm_head on the first {positions} "
                      f"positions of the same ids ({sample.size} tokens), {dt:.1f} s wall"}
    par = {"positions": int(sample.size), "min_cos": s["min_cos"], "mean_cos": s["mean_cos"],
           "argmax_gated": s["gated"], "argmax_gated_agree": s["gated_agree"]}
    return base, par


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="mini_f16_1x512")
    ap.add_argument("--cpu-positions", type=int, default=384)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-decode", action="store_true")
    ap.add_argument("--copy-probe-mb", type=int, default=0,
                    help="also run one plain device copy of this many MiB (counter calibration)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (got --gpus {args.gpus}); the path has no multi-GPU mode",
              file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import logits_parity_amd as phi
    import synth
    from logits_parity_amd.weights import to_device

    phi.lib()
    wl = synth.PREFILL_WORKLOADS[args.workload]
    cfg = wl.cfg
    log(f"bench: generating {cfg.name} weights")
    ws = synth.WeightSet(cfg)
    dev = to_device(ws, cfg.n_layers, "cuda")
    model = phi.phi_load_fused(cfg, dev)
    ids_np = synth.token_ids(cfg, wl.batch, wl.seq)
    ids = torch.from_numpy(ids_np).cuda()
    logits = torch.empty((wl.batch, wl.seq, cfg.vocab), dtype=torch.float32, device="cuda")
    workspace = torch.empty(model.workspace_bytes(wl.batch, wl.seq), dtype=torch.uint8, device="cuda")
    stream = torch.cuda.current_stream()

    if args.copy_probe_mb:
        src = torch.empty(args.copy_probe_mb << 20, dtype=torch.uint8, device="cuda").fill_(1)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    log(f"bench: warmup {args.warmup}")
    for _ in range(args.warmup):
        model.prefill_logits(ids, logits, workspace, stream)
    torch.cuda.synchronize()
    log(f"bench: timing {args.steps} steps")
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    e0.record(stream)
    for _ in range(args.steps):
        model.prefill_logits(ids, logits, workspace, stream)
    e1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_step = wall * 1e3 / args.steps
    tokens = wl.batch * wl.seq
    value = tokens * args.steps / wall
    flops = prefill_flops(cfg, wl.batch, wl.seq)
    gpu_logits = logits.cpu().numpy()
    finite = bool(np.isfinite(gpu_logits).all())

    log("bench: per-stage device time inside forwards")
    n_prof = min(args.steps, 10)
    prof = profile_forwards(model, ids, logits, workspace, stream, n_prof)
    gu_ms, gu_n = prof["gate_up"]
    avg_s = gu_ms / 1e3 / gu_n
    kflops = 2.0 * tokens * 2 * cfg.intermediate * cfg.hidden
    ach = kflops / avg_s / 1e12
    traffic = None
    if args.workload == "mini_f16_1x512":
        traffic = measured_traffic("gate_up_gemm_mini_f16_1x512_traffic.md", "logits_parity_amd/csrc/gemm.hpp")
    roof = {"bound": "mfma", "achieved": round(ach, 1), "peak": MFMA_F16_PEAK_TFLOPS, "unit": "TFLOP/s",
            "frac": round(ach / MFMA_F16_PEAK_TFLOPS, 4), "traffic": traffic,
            "kernel": "phi_gemm_mfma_kernel<..., EPI_SILU> (fused gate/up GEMM + SiLU*up)",
            "avg_launch_us": round(avg_s * 1e6, 2), "flops_per_launch": kflops,
            "launches_timed": gu_n}
    stages = {k: round(v[0] / n_prof, 4) for k, v in prof.items()}

    out = {"metric": "Phi-3-mini-shape f16 prefill tokens/s, % MFMA peak; logit cosine vs oracle",
           "value": round(value, 1), "unit": "tokens/s", "n_gpus": 1, "steps": args.steps,
           "warmup": args.warmup, "ms_per_step": round(ms_step, 4), "higher_is_better": True,
           "scaling": "weak", "vs_baseline": None, "dtype": "f32" if cfg.wtype == "f32" else "f16",
           "data": "synthetic",
           "config": {"workload": wl.name, "batch": wl.batch, "seq_len": wl.seq, "layers": cfg.n_layers,
                      "hidden": cfg.hidden, "heads": cfg.n_heads, "head_dim": cfg.head_dim,
                      "intermediate": cfg.intermediate, "vocab": cfg.vocab,
                      "weights": {"f32": "random N(0,0.02) float32, seed 1", "f16": "random N(0,0.02) float16, seed 1",
                                  "i8": "int8 per-row codes + float16 scales of random N(0,0.02) float16, seed 1"}[
                          cfg.wtype],
                      "ids": "uniform, seed 2"},
           "roofline": roof,
           "model_mfma_frac": round(flops / (wall / args.steps) / 1e12 / MFMA_F16_PEAK_TFLOPS, 4),
           "event_ms_per_step": round(e0.elapsed_time(e1) / args.steps, 4),
           "stage_ms_per_step": stages,
           "logits_finite": finite}

    if not args.no_decode:
        log("bench: decode")
        out["decode"] = [time_decode(phi, torch, np, synth, w) for w in synth.DECODE_WORKLOADS.values()]

    if not args.no_cpu_baseline:
        log(f"bench: cpu baseline on {args.cpu_positions} positions")
        base, par = cpu_baseline(cfg, ws, ids_np, gpu_logits, args.cpu_positions)
        out["cpu_baseline"] = base
        out["parity_sample"] = par
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
