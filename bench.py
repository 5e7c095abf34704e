#!/usr/bin/env python3
"""Benchmark of the GQA decoder forward pass on one MI355X.

One step = one pass of the whole hot path over one batch of synthetic input: the prefill
of the workload's prompt (batch x prompt_len), then its greedy decode steps, each
consuming the previous step's argmax on the device. Inputs (weights, ids) are resident
in HBM before the timed region. Prints ONE JSON line:

  value        whole-job tokens/s: (batch*prompt_len + batch*decode_steps) / step time
  roofline     the dominant kernel (largest time per step) against its roof, from HIP
               events around that kernel's own launches (ember_time_kernel, same stream
               and arguments as in the step)
  cpu_baseline the oracle timed on this host's cores on a bounded sample
  sampler_us   the sampler of one decode step (temperature / top-k / top-p draw over the
               vocabulary), timed after the greedy steps; not part of `value`

Usage: python bench.py [--steps K] [--warmup W] [--workload qwen05b] [--precision exact]
"""
import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_HBM_GBS = 8000.0          # MI355X HBM3E, published
PEAK_BF16_TFLOPS = 2500.0      # MI355X dense bf16 MFMA, published
PEAK_FP32_TFLOPS = 157.3
METRIC = "prefill & decode tokens/s at 1 GPU + % of HBM / bf16-MFMA roofline"


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=3)
    ap.add_argument("--warmup", type=int, default=1)
    ap.add_argument("--workload", default="qwen05b",
                    choices=["tiny", "qwen05b", "llama1b", "encoder", "longctx", "qwen05b-q8"])
    ap.add_argument("--precision", default="exact", choices=["exact", "fast"])
    ap.add_argument("--kv", default=None, choices=[None, "f32", "bf16"])
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--timing-iters", type=int, default=100)
    ap.add_argument("--calibrate-copy", type=int, default=0, metavar="BYTES",
                    help="only run one plain device copy of BYTES (counter calibration)")
    return ap.parse_args()


def weight_bytes(m):
    """Stored bytes per weight: bf16 2, f32 4, q8_0 34 per 32 (an f16 scale per 32 int8)."""
    return {"bf16": 2.0, "f32": 4.0, "q8_0": 34.0 / 32.0}[m.weight_dtype]


def kernel_work(m, kind, phase, M, S, kv_bytes):
    """Algorithmic bytes (decode, HBM-bound) or FLOPs (prefill projections, MFMA-bound)
    of one launch of `kind`: weights read once at their stored dtype, activations f32 in
    and out, K/V at the cache dtype; no implementation scratch (split partials)."""
    from gqa_decoder_transformer_amd import binding as B
    es = weight_bytes(m)
    H, FF, V = m.hidden, m.ffn, m.vocab
    qn = (m.heads + 2 * m.kv_heads) * m.head_dim
    qd = m.q_dim
    if phase == 0:
        if kind == B.K_LM_HEAD:
            return "hbm", V * H * es + H * 4 + V * 4 * M
        if kind == B.K_QKV:
            return "hbm", qn * H * es + M * (2 * H * 4 + qn * 4) + (qn * 4 if m.qkv_bias else 0)
        if kind == B.K_O:
            return "hbm", H * qd * es + M * (qd * 4 + 2 * H * 4)
        if kind == B.K_GATE_UP:
            return "hbm", 2 * FF * H * es + M * (2 * H * 4 + FF * 4)
        if kind == B.K_DOWN:
            return "hbm", H * FF * es + M * (FF * 4 + 2 * H * 4)
        if kind == B.K_ATTN:
            return "hbm", M * (2 * S * m.kv_heads * m.head_dim * kv_bytes + qn * 4 + qd * 4)
    else:
        if kind == B.K_LM_HEAD:
            return "mfma", 2.0 * M * V * H
        if kind == B.K_QKV:
            return "mfma", 2.0 * M * qn * H
        if kind == B.K_O:
            return "mfma", 2.0 * M * H * qd
        if kind == B.K_GATE_UP:
            return "mfma", 2.0 * M * 2 * FF * H
        if kind == B.K_DOWN:
            return "mfma", 2.0 * M * H * FF
        if kind == B.K_ATTN:
            return "mfma", None   # set by the caller (causal pairs)
    raise ValueError(kind)


def cpu_baseline(w, ck, prompt):
    """The oracle as it stands (f32 NumPy, BLAS threads as configured) on a bounded
    sample: the full prompt of row 0, then up to 16 greedy decode steps."""
    import numpy as np
    import oracle as O
    try:
        from threadpoolctl import threadpool_info
        cores = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        cores = len(os.sched_getaffinity(0))
    om = O.OracleModel(w.model, ck)
    T = prompt.shape[1]
    t0 = time.perf_counter()
    if w.decode_steps == 0:
        om.forward_sequence(prompt[0], 0, None, all_positions=True)
        dt = time.perf_counter() - t0
        return {"value": T / dt, "unit": "tokens/s", "cores": cores, "kind": "oracle",
                "sample": f"row 0 of the batch: {T} tokens, bidirectional, f32 NumPy"}
    n = min(16, w.decode_steps)
    O.generate(om, prompt[0], n, max_seq=T + n)
    dt = time.perf_counter() - t0
    return {"value": (T + n) / dt, "unit": "tokens/s", "cores": cores, "kind": "oracle",
            "sample": f"row 0: prefill {T} tokens + {n} greedy decode steps, f32 NumPy"}


def measured_traffic(workload, precision, kernel):
    """HBM bytes per launch of `kernel` from the hardware-counter record in profiles/
    (rocprofv3 FETCH_SIZE + WRITE_SIZE, scaled by a copy of known size), or None when
    there is no record or the kernel's source changed since it was taken."""
    from gqa_decoder_transformer_amd import profiling
    path = os.path.join(ROOT, "profiles", "pmc_traffic.json")
    if not os.path.exists(path):
        return None
    with open(path) as fh:
        recs = json.load(fh)
    for r in recs:
        if (r["name"], r["workload"], r["precision"]) != (kernel, workload, precision):
            continue
        src = os.path.join(ROOT, r["source"])
        if os.path.exists(src) and profiling.source_sha256(src) == r["source_sha256"]:
            return r["bytes_per_launch"]
    return None


def calibrate_copy(nbytes):
    """One plain device-to-device copy of `nbytes` (reference for the memory counters)."""
    import torch
    src = torch.ones(nbytes, dtype=torch.uint8, device="cuda:0")
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"calibrate_copy_bytes": nbytes}), flush=True)


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (got --gpus {args.gpus}): the library has no "
              "multi-GPU path", file=sys.stderr)
        sys.exit(2)
    if args.calibrate_copy:
        calibrate_copy(args.calibrate_copy)
        return
    import numpy as np
    import torch
    import workloads as W
    from gqa_decoder_transformer_amd import binding as B

    w = W.get(args.workload)
    m = w.model
    prec = B.EXACT if args.precision == "exact" else B.FAST
    # multi-token passes on bf16 MFMA: bf16 weights, or q8_0 dequantised to bf16 in FAST
    mfma_path = m.weight_dtype in ("bf16", "q8_0")
    kv = {"f32": B.F32, "bf16": B.BF16, None: None}[args.kv]
    ck = W.weights_for(w)
    prompt = W.make_ids(w)
    Bn, T, N = w.batch, w.prompt_len, w.decode_steps
    max_tokens = Bn * T if Bn * T <= 16384 else T
    cfg = B.make_config(m, precision=prec, kv_dtype=kv, max_batch=Bn, max_seq=w.max_pos,
                        max_tokens=max_tokens)
    dev = torch.device("cuda:0")
    s = torch.cuda.Stream(device=dev)
    with torch.cuda.stream(s):
        eng = B.Engine(cfg, ck, device="cuda:0", stream=s)
        ids = torch.empty((Bn,) if m.causal else (Bn, T), dtype=torch.int32, device=dev)

        def step(ev):
            ev[0].record(s)
            eng.prefill(prompt, next_ids=ids)
            ev[1].record(s)
            for k in range(N):
                eng.decode_step(ids, T + k, ids)
            ev[2].record(s)

        for _ in range(args.warmup):
            step([torch.cuda.Event(enable_timing=True) for _ in range(3)])
        torch.cuda.synchronize()
        evs = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(args.steps)]
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for e in evs:
            step(e)
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
        eng.sync()
        pre_ms = [e[0].elapsed_time(e[1]) for e in evs]
        dec_ms = [e[1].elapsed_time(e[2]) for e in evs]
        step_ms = [e[0].elapsed_time(e[2]) for e in evs]

        # ---- per-kernel live timings (HIP events on the same stream)
        kv_bytes = 4 if cfg.kv_dtype == B.F32 else 2
        S_mean = T + (N + 1) / 2.0
        kernels = {}
        phases = ([0] if N > 0 else []) + [1]
        for phase in phases:
            for kind, name in enumerate(["lm_head", "qkv", "attn", "o", "gate_up", "down"]):
                if m.head != "tied_lm" and kind == B.K_LM_HEAD:
                    continue
                if phase == 1 and kind == B.K_LM_HEAD:
                    continue
                if phase == 0:   # re-establish a decode state at the last position
                    pass
                us = eng.time_kernel(kind, phase, args.timing_iters)
                launches = (1 if kind == B.K_LM_HEAD else m.layers) * (N if phase == 0 else
                                                                          -(-Bn * T // max_tokens))
                bound, work = kernel_work(m, kind, phase, Bn if phase == 0 else max_tokens,
                                          S_mean if phase == 0 else T, kv_bytes)
                if phase == 1 and kind == B.K_ATTN:
                    rows = max_tokens // T
                    pairs = T * (T + 1) / 2 if m.causal else T * T
                    work = 4.0 * m.head_dim * m.heads * pairs * rows
                kernels[f"{'decode' if phase == 0 else 'prefill'}.{name}"] = {
                    "avg_us": us, "launches_per_step": launches,
                    "ms_per_step": us * launches / 1000.0, "bound": bound, "work_per_launch": work}
        # one whole layer (every kernel, back to back, cycling the layers) beside the sum of
        # its kernels timed one kind at a time
        layer_us = {}
        for phase in phases:
            tag = "decode" if phase == 0 else "prefill"
            layer_us[tag] = eng.time_kernel(B.K_LAYER, phase, args.timing_iters)
            layer_us[tag + "_kernel_sum"] = sum(
                v["avg_us"] for k, v in kernels.items()
                if k.startswith(tag + ".") and not k.endswith("lm_head"))
        # the sampler of one decode step (outside the timed steps, which are greedy): one
        # draw per row over the vocabulary, at two settings
        sampler_us = {}
        if N > 0 and m.head == "tied_lm":
            U = torch.from_numpy(W.make_uniforms(5, w.max_pos, Bn)).to(dev)
            for tag, (t_, k_, p_) in {"t1.0": (1.0, 0, 1.0),
                                      "t0.8_k50_p0.9": (0.8, 50, 0.9)}.items():
                eng.set_sampler(t_, k_, p_, U)
                sampler_us[tag] = eng.time_kernel(B.K_SAMPLE, 0, args.timing_iters)
            eng.set_sampler()
    for k, v in kernels.items():
        if v["bound"] == "hbm":
            v["achieved"] = v["work_per_launch"] / (v["avg_us"] * 1e-6) / 1e9
            v["peak"], v["unit"] = PEAK_HBM_GBS, "GB/s"
        else:
            v["achieved"] = v["work_per_launch"] / (v["avg_us"] * 1e-6) / 1e12
            peak = PEAK_BF16_TFLOPS if mfma_path else PEAK_FP32_TFLOPS
            v["peak"], v["unit"] = peak, "TFLOP/s"
        v["frac"] = v["achieved"] / v["peak"]
    dom_name = max(kernels, key=lambda k: kernels[k]["ms_per_step"])
    dom = kernels[dom_name]

    ms = float(np.mean(step_ms))
    tokens = Bn * T + Bn * N
    value = tokens / (ms / 1000.0)
    # decode step as a whole against HBM: weights once + KV read/write + logits, per step
    es = weight_bytes(m)
    n_params = m.vocab * m.hidden + m.layers * (m.hidden * (m.q_dim + 2 * m.kv_dim) +
                                               m.hidden * m.q_dim + 3 * m.hidden * m.ffn)
    extra = {}
    if N > 0:
        dec_step_ms = float(np.mean(dec_ms)) / N
        kv_step = Bn * m.layers * 2 * m.kv_heads * m.head_dim * kv_bytes * (S_mean + 1)
        step_bytes = n_params * es + kv_step + Bn * m.vocab * 4
        extra["decode_tok_s"] = Bn * N / (float(np.mean(dec_ms)) / 1000.0)
        extra["decode_ms_per_token_step"] = dec_step_ms
        extra["decode_step_hbm_frac"] = step_bytes / (dec_step_ms * 1e-3) / 1e9 / PEAK_HBM_GBS
    pre = float(np.mean(pre_ms))
    extra["prefill_tok_s"] = Bn * T / (pre / 1000.0)
    extra["prefill_ms"] = pre
    if mfma_path:
        flops = 2.0 * Bn * T * (n_params - m.vocab * m.hidden)
        pairs = T * (T + 1) / 2 if m.causal else T * T
        flops += 4.0 * m.head_dim * m.heads * m.layers * pairs * Bn
        if m.head == "tied_lm":
            flops += 2.0 * Bn * m.vocab * m.hidden
        extra["prefill_mfma_frac"] = flops / (pre * 1e-3) / 1e12 / PEAK_BF16_TFLOPS

    line = {
        "metric": METRIC, "value": value, "unit": "tokens/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": ms,
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "f32" if prec == B.EXACT else "bf16", "data": "synthetic",
        "config": {"workload": w.description, "batch": Bn, "prompt_len": T, "decode_steps": N,
                   "precision": args.precision,
                   "kv_dtype": "f32" if cfg.kv_dtype == B.F32 else "bf16",
                   "weights": f"random-init N(0,0.02) {m.weight_dtype}, seed {w.weight_seed}"},
        "wall_s": wall,
        "roofline": {"bound": dom["bound"], "kernel": dom_name,
                     "achieved": dom["achieved"], "peak": dom["peak"], "unit": dom["unit"],
                     "frac": dom["frac"],
                     "traffic": measured_traffic(args.workload, args.precision, dom_name),
                     "avg_us": dom["avg_us"], "work_per_launch": dom["work_per_launch"]},
        "kernels": {k: {kk: (round(vv, 4) if isinstance(vv, float) else vv)
                        for kk, vv in v.items()} for k, v in kernels.items()},
        "layer_us": {k: round(v, 3) for k, v in layer_us.items()},
        "sampler_us": {k: round(v, 3) for k, v in sampler_us.items()},
        **extra,
    }
    eng.close()
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(w, ck, prompt)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
