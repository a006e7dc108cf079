#!/usr/bin/env python3
"""Phi-3-mini-shape f16 prefill benchmark on one MI355X.

One step = one full prefill forward (embedding, every decoder layer, final
norm, lm_head) over a batch of synthetic ids, ids -> fp32 logits at every
position, through the C ABI.  Weights (seeded N(0, 0.02)) and ids are
resident in HBM before the timed region.  Printed as one JSON line whose
headline is the Phi-3-mini f16 1 x 512 prefill:

  value         prefill tokens/s (batch * seq * steps / wall time of the
                timed steps, bracketed by device synchronisation)
  step_ms       median, p10 and p90 of the timed steps, from HIP events
                recorded between the steps on the forward's stream
  roofline      the dominant kernel (fused gate/up GEMM + SiLU*up): its
                launches inside forwards run right after the timed steps,
                timed by HIP events that the library attaches to each of its
                dispatches on the forward's stream (the kernel's own run
                time, as a kernel trace measures it); algorithmic flops
                2 * T * 2I * H per launch against the f16 MFMA peak; HBM
                traffic per launch from the committed counter summary (null
                if the kernel changed since the counters were taken)
  workloads     the same measurements for the other prefill configurations:
                1 x 4096 f16, 4 x 1024 with int8 weights, and the tiny fp32
                model (1 x 16)
  decode        K16/V8 decode attention per call at the two Phi-4 shapes,
                algorithmic bytes per call against HBM bandwidth; HBM
                traffic per call from the committed counter summary (null
                if the kernel changed)
  cpu_baseline  the fp64 oracle on the host over all 512 positions of the
                headline input, timed, with the parity of those rows; the
                same leg checks the other workloads' logits at every
                position against the stored oracle results
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
FP32_VECTOR_PEAK_TFLOPS = 157.3  # MI355X fp32 vector ALU
HBM_PEAK_GBS = 8000.0           # MI355X HBM3E
HEADLINE = "mini_f16_1x512"
EXTRA = ("mini_f16_1x4096", "mini_w8_4x1024", "tiny_f32_1x16")
GEMM_SRC = "logits_parity_amd/csrc/gemm.hpp"


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


def pct(xs, q):
    import numpy as np
    return round(float(np.percentile(np.asarray(xs), q)), 4)


def profile_forwards(model, ids, logits, workspace, stream, n):
    """Per-stage device time over n forwards, from HIP events that the library
    attaches to each of its kernel dispatches on the forward's stream."""
    model.profile_enable(True)
    for _ in range(n):
        model.prefill_logits(ids, logits, workspace, stream)
    prof = model.profile_read()
    model.profile_enable(False)
    return prof


def run_prefill(phi, torch, np, synth, wl, dev_weights, steps, warmup):
    """Warm-up, then exactly `steps` timed forwards (value, wall clock) with
    an event between consecutive steps (per-step distribution), then
    per-stage event timing over further forwards."""
    cfg = wl.cfg
    model = phi.phi_load_fused(cfg, dev_weights)
    ids_np = synth.token_ids(cfg, wl.batch, wl.seq)
    ids = torch.from_numpy(ids_np).cuda()
    logits = torch.empty((wl.batch, wl.seq, cfg.vocab), dtype=torch.float32, device="cuda")
    workspace = torch.empty(model.workspace_bytes(wl.batch, wl.seq), dtype=torch.uint8, device="cuda")
    stream = torch.cuda.current_stream()
    log(f"bench: {wl.name}: warmup {warmup}")
    for _ in range(warmup):
        model.prefill_logits(ids, logits, workspace, stream)
    torch.cuda.synchronize()
    log(f"bench: {wl.name}: timing {steps} steps")
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(steps + 1)]
    t0 = time.perf_counter()
    ev[0].record(stream)
    for i in range(steps):
        model.prefill_logits(ids, logits, workspace, stream)
        ev[i + 1].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    step_ms = [ev[i].elapsed_time(ev[i + 1]) for i in range(steps)]
    tokens = wl.batch * wl.seq
    flops = prefill_flops(cfg, wl.batch, wl.seq)
    gpu_logits = logits.cpu().numpy()

    n_prof = min(steps, 10)
    prof = profile_forwards(model, ids, logits, workspace, stream, n_prof)
    gu_ms, gu_n = prof["gate_up"]
    avg_s = gu_ms / 1e3 / gu_n
    kflops = 2.0 * tokens * 2 * cfg.intermediate * cfg.hidden
    ach = kflops / avg_s / 1e12
    if cfg.wtype == "f32":
        bound, peak, kernel = "alu", FP32_VECTOR_PEAK_TFLOPS, "phi_gemm_simt_f32_kernel<..., EPI_SILU> (fp32 gate/up)"
    else:
        bound, peak = "mfma", MFMA_F16_PEAK_TFLOPS
        kernel = "phi_gemm_mfma_kernel<..., EPI_SILU> (fused gate/up GEMM + SiLU*up)"
    traffic = measured_traffic(f"gate_up_gemm_{wl.name}_traffic.md", GEMM_SRC)
    roof = {"bound": bound, "achieved": round(ach, 1), "peak": peak, "unit": "TFLOP/s",
            "frac": round(ach / peak, 4), "traffic": traffic, "kernel": kernel,
            "avg_launch_us": round(avg_s * 1e6, 2), "flops_per_launch": kflops, "launches_timed": gu_n}
    res = {"workload": wl.name, "value": round(tokens * steps / wall, 1), "unit": "tokens/s", "steps": steps,
           "warmup": warmup, "ms_per_step": round(wall * 1e3 / steps, 4),
           "step_ms": {"median": pct(step_ms, 50), "p10": pct(step_ms, 10), "p90": pct(step_ms, 90)},
           "dtype": "f32" if cfg.wtype == "f32" else "f16",
           "weight_dtype": {"f32": "f32", "f16": "f16", "i8": "int8 per-row codes + f16 row scales"}[cfg.wtype],
           "config": {"workload": wl.name, "batch": wl.batch, "seq_len": wl.seq, "layers": cfg.n_layers,
                      "hidden": cfg.hidden, "heads": cfg.n_heads, "head_dim": cfg.head_dim,
                      "intermediate": cfg.intermediate, "vocab": cfg.vocab,
                      "weights": {"f32": "random N(0,0.02) float32, seed 1",
                                  "f16": "random N(0,0.02) float16, seed 1",
                                  "i8": "int8 per-row codes + float16 scales of random N(0,0.02) float16, seed 1"}[
                          cfg.wtype],
                      "ids": "uniform, seed 2"},
           "roofline": roof,
           "model_frac": round(flops / (wall / steps) / 1e12 / peak, 4),
           "stage_ms_per_step": {k: round(v[0] / n_prof, 4) for k, v in prof.items()},
           "logits_finite": bool(np.isfinite(gpu_logits).all())}
    del model, workspace, logits
    return res, ids_np, gpu_logits


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
    call = lambda i: phi.attn_decode_k16v8(q, *pools[i % copies], vs, bt, cl, wl.ctx, sm, out=out, workspace=ws,
                                           stream=stream)
    for i in range(10):
        call(i)
    # back-to-back calls between two events: the mean per call
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record(stream)
    for i in range(reps):
        call(i)
    e1.record(stream)
    torch.cuda.synchronize()
    us = e0.elapsed_time(e1) * 1e3 / reps
    # the distribution: an event before and after every call
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(2 * reps)]
    for i in range(reps):
        ev[2 * i].record(stream)
        call(i)
        ev[2 * i + 1].record(stream)
    torch.cuda.synchronize()
    per = [ev[2 * i].elapsed_time(ev[2 * i + 1]) * 1e3 for i in range(reps)]
    nbytes = decode_bytes(wl)
    gbs = nbytes / (us * 1e-6) / 1e9
    return {"workload": wl.name, "us_per_call": round(us, 2),
            "us_per_call_dist": {"median": pct(per, 50), "p10": pct(per, 10), "p90": pct(per, 90), "reps": reps},
            "bytes_per_call": nbytes,
            "roofline": {"bound": "hbm", "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                         "frac": round(gbs / HBM_PEAK_GBS, 4),
                         "traffic": measured_traffic("decode_k16v8_traffic.md", "logits_parity_amd/csrc/decode.hpp",
                                                     f"traffic_bytes_per_call_{wl.name}")},
            "cache_copies_rotated": copies}


# ---------------------------------------------------------------- cpu_baseline leg (the only oracle use)
def _oracle_threads() -> int:
    threads = os.cpu_count()
    try:
        from threadpoolctl import threadpool_info
        info = [p for p in threadpool_info() if p.get("internal_api") in ("openblas", "mkl", "blis")]
        if info:
            threads = max(p["num_threads"] for p in info)
    except Exception:
        pass
    return threads


def cpu_baseline(cfg, ws, ids_np, gpu_logits, positions):
    """The fp64 oracle as it stands on the first `positions` ids of the same
    input; causal prefix invariance makes those rows comparable to the GPU's."""
    from oracle import parity, prefill
    sample = ids_np[:, :positions]
    t0 = time.perf_counter()
    ref = prefill.prefill_logits(cfg, ws, sample)
    dt = time.perf_counter() - t0
    s = parity.summary(gpu_logits[:, :positions].reshape(-1, cfg.vocab), ref.reshape(-1, cfg.vocab))
    base = {"value": round(sample.size / dt, 3), "unit": "tokens/s", "cores": _oracle_threads(), "kind": "oracle",
            "sample": f"fp64 numpy oracle, all {cfg.n_layers} layers + lm_head on the first {positions} "
                      f"positions of the same ids ({sample.size} tokens), {dt:.1f} s wall"}
    par = {"positions": int(sample.size), "min_cos": s["min_cos"], "mean_cos": s["mean_cos"],
           "argmax_gated": s["gated"], "argmax_gated_agree": s["gated_agree"], "against": "live oracle"}
    return base, par


def stored_parity(wl, ws, ids_np, gpu_logits):
    """Logits at every position against the stored oracle results: each
    reference row is the oracle's lm_head step applied to its stored final
    hidden state; argmax where the stored top-2 gap exceeds 1e-3."""
    import hashlib

    import numpy as np

    from oracle import parity, prefill
    path = os.path.join(ROOT, "tests", "golden", wl.name + ".npz")
    if not os.path.exists(path):
        return {"status": "no stored oracle results"}
    g = np.load(path)
    ids_ok = hashlib.sha256(np.ascontiguousarray(ids_np, dtype=np.int32).tobytes()).hexdigest() == str(g["ids_sha256"])
    if not ids_ok or ws.digest() != str(g["weights_sha256"]):
        return {"status": "inputs differ from the stored oracle's"}
    if "hidden" not in g.files:
        return {"status": "stored results hold no hidden state"}
    flat = gpu_logits.reshape(-1, wl.cfg.vocab)
    hidden = g["hidden"]
    cos = np.empty(len(flat))
    for r0 in range(0, len(flat), 512):
        ref = prefill.logits_from_hidden(hidden[r0:r0 + 512], ws.lm_head)
        cos[r0:r0 + 512] = parity.row_cosines(flat[r0:r0 + 512], ref)
    gated = g["gap"] > 1e-3
    agree = np.argmax(flat, axis=1) == g["argmax"]
    return {"positions": int(len(flat)), "min_cos": float(cos.min()), "mean_cos": float(cos.mean()),
            "argmax_gated": int(gated.sum()), "argmax_gated_agree": int((gated & agree).sum()),
            "against": "stored oracle (int8 weights: the oracle on the same int8 weights)"}


# ---------------------------------------------------------------- main
def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default=HEADLINE, help="the headline prefill workload")
    ap.add_argument("--no-extra", action="store_true", help="only the headline workload")
    ap.add_argument("--cpu-positions", type=int, default=512)
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
    if args.copy_probe_mb:
        src = torch.empty(args.copy_probe_mb << 20, dtype=torch.uint8, device="cuda").fill_(1)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    names = [args.workload] + ([] if args.no_extra else [w for w in EXTRA if w != args.workload])
    weights, results, kept = {}, {}, {}
    for name in names:
        wl = synth.PREFILL_WORKLOADS[name]
        cfg = wl.cfg
        if cfg.name not in weights:
            log(f"bench: generating {cfg.name} weights")
            ws = synth.WeightSet(cfg)
            weights[cfg.name] = (ws, to_device(ws, cfg.n_layers, "cuda"))
        ws, dev = weights[cfg.name]
        res, ids_np, gpu_logits = run_prefill(phi, torch, np, synth, wl, dev, args.steps, args.warmup)
        results[name] = res
        kept[name] = (wl, ws, ids_np, gpu_logits)
        # weights no later workload uses leave the GPU
        if all(synth.PREFILL_WORKLOADS[n].cfg.name != cfg.name for n in names[names.index(name) + 1:]):
            weights[cfg.name] = (ws, None)
            del dev
            torch.cuda.empty_cache()

    head = results[args.workload]
    out = {"metric": "Phi-3-mini-shape f16 prefill tokens/s, % MFMA peak; logit cosine vs oracle",
           "value": head["value"], "unit": "tokens/s", "n_gpus": 1, "steps": args.steps,
           "warmup": args.warmup, "ms_per_step": head["ms_per_step"], "higher_is_better": True,
           "scaling": "weak", "vs_baseline": None, "dtype": head["dtype"], "weight_dtype": head["weight_dtype"],
           "data": "synthetic", "config": head["config"], "step_ms": head["step_ms"],
           "roofline": head["roofline"], "model_mfma_frac": head["model_frac"],
           "stage_ms_per_step": head["stage_ms_per_step"], "logits_finite": head["logits_finite"]}

    if not args.no_decode:
        log("bench: decode")
        out["decode"] = [time_decode(phi, torch, np, synth, w) for w in synth.DECODE_WORKLOADS.values()]

    if not args.no_cpu_baseline:
        wl, ws, ids_np, gpu_logits = kept[args.workload]
        pos = min(args.cpu_positions, wl.seq)
        log(f"bench: cpu baseline on {pos} positions")
        base, par = cpu_baseline(wl.cfg, ws, ids_np, gpu_logits, pos)
        out["cpu_baseline"] = base
        out["parity_sample"] = par
        for name in names[1:]:
            wl, ws, ids_np, gpu_logits = kept[name]
            log(f"bench: parity of {name}")
            if wl.seq * wl.batch <= 64:
                results[name]["parity"] = cpu_baseline(wl.cfg, ws, ids_np, gpu_logits, wl.seq)[1]
            else:
                results[name]["parity"] = stored_parity(wl, ws, ids_np, gpu_logits)
    out["workloads"] = [results[n] for n in names[1:]]
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
