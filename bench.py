#!/usr/bin/env python3
"""Benchmark of the GQA decoder forward pass on one MI355X.

One step = one pass of the whole hot path over one batch of synthetic input: the prefill
of the workload's prompt (batch x prompt_len), then its greedy decode steps, each
consuming the previous step's argmax on the device. Inputs (weights, ids) are resident
in HBM before the timed region. The default workload is the largest: the long-context
batched decode (Llama-3.2-1B shape, 64 rows x 8192 prompt tokens, 128 greedy steps),
EXACT precision with an f32 KV cache. Prints ONE JSON line:

  value        whole-job tokens/s: (batch*prompt_len + batch*decode_steps) / step time
  roofline     the dominant kernel (largest time per step) against its roof, from HIP
               events around that kernel's own launches (ember_time_kernel, same stream
               and arguments as in the step), also against the measured achievable peak
  peaks        achievable peaks measured here: a streaming copy, a streaming read and an
               MFMA-only loop (HBM-bound kernels, which mostly read, are also reported
               against the read)
  extra        the spec measurements on the Llama-3.2-1B shape (batch-1 decode
               EXACT with f32 KV; the 2048-token prefill EXACT and FAST) and the
               long-context decode with a bf16 KV cache (FAST)
  cpu_baseline the oracle timed on this host's cores on a bounded sample (prefill and
               decode rates apart, combined in the workload's proportions)

Usage: python bench.py [--steps K] [--warmup W] [--workload longctx] [--precision exact]
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
KINDS = ["lm_head", "qkv", "attn", "o", "gate_up", "down"]


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=3)
    ap.add_argument("--warmup", type=int, default=1)
    ap.add_argument("--workload", default="longctx",
                    choices=["tiny", "qwen05b", "llama1b", "encoder", "longctx", "qwen05b-q8"])
    ap.add_argument("--precision", default="exact", choices=["exact", "fast"])
    ap.add_argument("--kv", default=None, choices=[None, "f32", "bf16"])
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-extra", action="store_true",
                    help="skip the extra measurements (1B batch-1 decode and prefill, bf16 KV)")
    ap.add_argument("--timing-iters", type=int, default=100)
    ap.add_argument("--calibrate-copy", type=int, default=0, metavar="BYTES",
                    help="only run one plain device copy of BYTES (counter calibration)")
    return ap.parse_args()


def progress(msg):
    """One progress line on stderr (the JSON result is the only line on stdout)."""
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def weight_bytes(m):
    """Stored bytes per weight: bf16 2, f32 4, q8_0 34 per 32 (an f16 scale per 32 int8)."""
    return {"bf16": 2.0, "f32": 4.0, "q8_0": 34.0 / 32.0}[m.weight_dtype]


def matrix_params(m):
    return m.layers * (m.hidden * (m.q_dim + 2 * m.kv_dim) + m.hidden * m.q_dim + 3 * m.hidden * m.ffn)


def kernel_work(m, kind, phase, M, S, kv_bytes, rows=1, T=1):
    """Algorithmic bytes (decode, HBM-bound) or FLOPs (multi-token passes, MFMA-bound) of
    one launch of `kind`: weights read once at their stored dtype, activations f32 in and
    out, K/V at the cache dtype, no implementation scratch (split partials); FLOPs
    2 M N K per GEMM and 4 HD NH per attention pair (causal T(T+1)/2, else T^2, per row)."""
    es = weight_bytes(m)
    H, FF, V = m.hidden, m.ffn, m.vocab
    qn = (m.heads + 2 * m.kv_heads) * m.head_dim
    qd = m.q_dim
    name = KINDS[kind]
    if phase == 0 and M == 1 or (phase == 0 and name == "attn"):
        if name == "lm_head":
            return "hbm", V * H * es + H * 4 + V * 4 * M
        if name == "qkv":
            return "hbm", qn * H * es + M * (2 * H * 4 + qn * 4) + (qn * 4 if m.qkv_bias else 0)
        if name == "o":
            return "hbm", H * qd * es + M * (qd * 4 + 2 * H * 4)
        if name == "gate_up":
            return "hbm", 2 * FF * H * es + M * (2 * H * 4 + FF * 4)
        if name == "down":
            return "hbm", H * FF * es + M * (FF * 4 + 2 * H * 4)
        if name == "attn":
            return "hbm", M * (2 * S * m.kv_heads * m.head_dim * kv_bytes + qn * 4 + qd * 4)
    if phase == 0:
        # batched decode projections: weights streamed once for M rows (HBM-bound at M=64)
        w = {"lm_head": V * H, "qkv": qn * H, "o": H * qd, "gate_up": 2 * FF * H, "down": H * FF}[name]
        return "hbm", w * es + M * 4 * ({"lm_head": H + V, "qkv": 2 * H + qn, "o": qd + 2 * H,
                                         "gate_up": 2 * H + FF, "down": FF + 2 * H}[name])
    if name == "attn":
        pairs = T * (T + 1) / 2 if m.causal else T * T
        return "mfma", 4.0 * m.head_dim * m.heads * pairs * rows
    n = {"lm_head": V * H, "qkv": qn * H, "o": H * qd, "gate_up": 2 * FF * H, "down": H * FF}[name]
    return "mfma", 2.0 * M * n


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


def measure_peaks(s):
    """Achievable peaks on this GPU: streaming copy GB/s (read + write) and streaming read
    GB/s over a 2 GiB buffer, dense bf16 MFMA TFLOP/s (library measurement kernels)."""
    import torch
    from gqa_decoder_transformer_amd import binding as B
    buf = torch.empty(2 << 30, dtype=torch.uint8, device="cuda:0")
    copy = B.ember_measure_peak(B.PEAK_COPY, buf.data_ptr(), buf.numel(), 20, s.cuda_stream)
    read = B.ember_measure_peak(B.PEAK_READ, buf.data_ptr(), buf.numel(), 20, s.cuda_stream)
    mfma = B.ember_measure_peak(B.PEAK_MFMA, buf.data_ptr(), buf.numel(), 5, s.cuda_stream)
    del buf
    return {"copy_gbs": copy, "read_gbs": read, "mfma_bf16_tflops": mfma}


class Run:
    """One engine on one workload: the timed steps (prefill + greedy decode), and the
    per-kernel timings of the last prefill pass and the last decode step."""

    def __init__(self, w, prec, kv, s):
        from gqa_decoder_transformer_amd import binding as B
        import workloads as W
        import torch
        self.w, self.m, self.s = w, w.model, s
        self.B = B
        self.prec = prec
        self.ck = W.weights_for(w)
        self.prompt = W.make_ids(w)
        Bn, T = w.batch, w.prompt_len
        self.max_tokens = Bn * T if Bn * T <= 16384 else T
        self.cfg = B.make_config(self.m, precision=prec, kv_dtype=kv, max_batch=Bn,
                                 max_seq=w.max_pos, max_tokens=self.max_tokens)
        self.kv_bytes = 4 if self.cfg.kv_dtype == B.F32 else 2
        with torch.cuda.stream(s):
            self.eng = B.Engine(self.cfg, self.ck, device="cuda:0", stream=s)
            self.ids = torch.empty((Bn,) if self.m.causal else (Bn, T), dtype=torch.int32,
                                   device="cuda:0")
        progress(f"engine ready: {w.name}, precision {'exact' if prec == B.EXACT else 'fast'}")

    def step(self, ev, decode=True, prefill=True):
        w = self.w
        ev[0].record(self.s)
        if prefill:
            self.eng.prefill(self.prompt, next_ids=self.ids)
        ev[1].record(self.s)
        if decode:
            for k in range(w.decode_steps):
                self.eng.decode_step(self.ids, w.prompt_len + k, self.ids)
        ev[2].record(self.s)

    def timed(self, steps, warmup, decode=True, prefill=True):
        """Mean prefill ms, decode ms (all steps) and step ms over `steps` timed steps."""
        import numpy as np
        import torch
        with torch.cuda.stream(self.s):
            for i in range(warmup):
                self.step([torch.cuda.Event(enable_timing=True) for _ in range(3)], decode, prefill)
                torch.cuda.synchronize()
                progress(f"warm-up step {i + 1}/{warmup} done")
            evs = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(steps)]
            t0 = time.perf_counter()
            for i, e in enumerate(evs):
                self.step(e, decode, prefill)
                if len(evs) <= 3 or i == len(evs) - 1:
                    progress(f"timed step {i + 1}/{len(evs)} enqueued")
            torch.cuda.synchronize()
            progress("timed steps done")
            wall = time.perf_counter() - t0
            self.eng.sync()
        pre = float(np.mean([e[0].elapsed_time(e[1]) for e in evs]))
        dec = float(np.mean([e[1].elapsed_time(e[2]) for e in evs]))
        tot = float(np.mean([e[0].elapsed_time(e[2]) for e in evs]))
        return pre, dec, tot, wall

    def kernels(self, iters):
        """Per-kernel average durations (HIP events on the engine's stream) with their
        algorithmic work and roofline fractions."""
        B, m, w = self.B, self.m, self.w
        Bn, T, N = w.batch, w.prompt_len, w.decode_steps
        S_mean = T + (N + 1) / 2.0
        mfma_path = m.weight_dtype in ("bf16", "q8_0")
        out = {}
        for phase in ([0] if N > 0 else []) + [1]:
            for kind, name in enumerate(KINDS):
                if kind == B.K_LM_HEAD and (m.head != "tied_lm" or phase == 1):
                    continue
                us = self.eng.time_kernel(kind, phase, iters)
                progress(f"kernel {'decode' if phase == 0 else 'prefill'}.{name}: {us:.2f} us")
                passes = -(-Bn * T // self.max_tokens)
                launches = (1 if kind == B.K_LM_HEAD else m.layers) * (N if phase == 0 else passes)
                rows = self.max_tokens // T if phase == 1 else 1
                bound, work = kernel_work(m, kind, phase, Bn if phase == 0 else self.max_tokens,
                                          S_mean, self.kv_bytes, rows=rows, T=T)
                v = {"avg_us": us, "launches_per_step": launches,
                     "ms_per_step": us * launches / 1000.0, "bound": bound, "work_per_launch": work}
                if bound == "hbm":
                    v["achieved"] = work / (us * 1e-6) / 1e9
                    v["peak"], v["unit"] = PEAK_HBM_GBS, "GB/s"
                else:
                    v["achieved"] = work / (us * 1e-6) / 1e12
                    v["peak"] = PEAK_BF16_TFLOPS if mfma_path else PEAK_FP32_TFLOPS
                    v["unit"] = "TFLOP/s"
                v["frac"] = v["achieved"] / v["peak"]
                out[f"{'decode' if phase == 0 else 'prefill'}.{name}"] = v
        layer_us = {}
        for phase in ([0] if N > 0 else []) + [1]:
            tag = "decode" if phase == 0 else "prefill"
            layer_us[tag] = self.eng.time_kernel(B.K_LAYER, phase, max(4, iters // 10))
            layer_us[tag + "_kernel_sum"] = sum(v["avg_us"] for k, v in out.items()
                                                if k.startswith(tag + ".") and not k.endswith("lm_head"))
        return out, layer_us

    def sampler_us(self, iters):
        """The sampler of one decode step (one draw per row over the vocabulary, after the
        greedy steps; not part of `value`) at two settings."""
        import torch
        import workloads as W
        w = self.w
        if w.decode_steps == 0 or self.m.head != "tied_lm":
            return {}
        U = torch.from_numpy(W.make_uniforms(5, w.max_pos, w.batch)).to("cuda:0")
        out = {}
        for tag, (t_, k_, p_) in {"t1.0": (1.0, 0, 1.0), "t0.8_k50_p0.9": (0.8, 50, 0.9)}.items():
            self.eng.set_sampler(t_, k_, p_, U)
            out[tag] = self.eng.time_kernel(self.B.K_SAMPLE, 0, iters)
        self.eng.set_sampler()
        return out

    def decode_bytes_per_step(self):
        """Algorithmic HBM bytes of one decode step: every weight once, the KV cache read
        at the mean length and written at the new position, the logits written f32."""
        m, w = self.m, self.w
        S_mean = w.prompt_len + (w.decode_steps + 1) / 2.0
        kv = w.batch * m.layers * 2 * m.kv_heads * m.head_dim * self.kv_bytes * (S_mean + 1)
        return (matrix_params(m) + m.vocab * m.hidden) * weight_bytes(m) + kv + w.batch * m.vocab * 4

    def prefill_flops(self):
        m, w = self.m, self.w
        T, Bn = w.prompt_len, w.batch
        flops = 2.0 * Bn * T * matrix_params(m)
        pairs = T * (T + 1) / 2 if m.causal else T * T
        flops += 4.0 * m.head_dim * m.heads * m.layers * pairs * Bn
        if m.head == "tied_lm":
            flops += 2.0 * Bn * m.vocab * m.hidden
        return flops

    def close(self):
        import torch
        self.eng.close()
        del self.eng
        torch.cuda.synchronize()
        torch.cuda.empty_cache()


def precision_label(prec, B):
    return ("f32 (decode: f32 FMA on widened bf16 weights; multi-token passes: bf16 MFMA on "
            "hi+lo activation planes, attention scores from three planes)"
            if prec == B.EXACT else "bf16 (bf16 MFMA inputs and KV cache, f32 accumulation)")


def extra_1b(s, peaks):
    """The spec measurements on the Llama-3.2-1B shape: batch-1 decode (EXACT, f32
    KV: 256 steps after the 2048-token prefill) against HBM, and the 2048-token prefill
    (EXACT and FAST) against bf16 MFMA."""
    import workloads as W
    from gqa_decoder_transformer_amd import binding as B
    w = W.get("llama1b")
    out = {"workload": w.description}
    for prec, tag in ((B.EXACT, "exact"), (B.FAST, "fast")):
        r = Run(w, prec, None, s)
        pre, dec, _, _ = r.timed(5, 1, decode=(prec == B.EXACT))
        flops = r.prefill_flops()
        e = {"prefill_ms": pre, "prefill_tok_s": w.prompt_len / (pre / 1e3),
             "prefill_mfma_frac": flops / (pre * 1e-3) / 1e12 / PEAK_BF16_TFLOPS,
             "prefill_mfma_frac_measured_peak": flops / (pre * 1e-3) / 1e12 / peaks["mfma_bf16_tflops"],
             "dtype": precision_label(prec, B)}
        if prec == B.EXACT:
            ms_tok = dec / w.decode_steps
            by = r.decode_bytes_per_step()
            e.update({"decode_ms_per_token": ms_tok, "decode_tok_s": 1e3 / ms_tok,
                      "kv_dtype": "f32", "decode_bytes_per_token": by,
                      "decode_hbm_frac": by / (ms_tok * 1e-3) / 1e9 / PEAK_HBM_GBS,
                      "decode_hbm_frac_measured_peak": by / (ms_tok * 1e-3) / 1e9 / peaks["read_gbs"]})
        out[tag] = e
        r.close()
    return out


def extra_longctx_bf16kv(s, peaks):
    """The long-context batched decode with a bf16 KV cache (FAST precision): prefill once
    (untimed), then the 128 decode steps timed twice."""
    import workloads as W
    from gqa_decoder_transformer_amd import binding as B
    w = W.get("longctx")
    r = Run(w, B.FAST, B.BF16, s)
    r.timed(1, 0, decode=False)
    _, dec, _, _ = r.timed(2, 1, prefill=False)
    ms = dec / w.decode_steps
    by = r.decode_bytes_per_step()
    r.close()
    return {"workload": w.description + " (decode only)", "kv_dtype": "bf16",
            "dtype": precision_label(B.FAST, B), "decode_ms_per_step": ms,
            "decode_tok_s": w.batch / (ms * 1e-3), "decode_bytes_per_step": by,
            "decode_hbm_frac": by / (ms * 1e-3) / 1e9 / PEAK_HBM_GBS,
            "decode_hbm_frac_measured_peak": by / (ms * 1e-3) / 1e9 / peaks["read_gbs"]}


def cpu_baseline(w, ck, prompt):
    """The oracle as it stands (f32 NumPy, BLAS threads as configured) on a bounded sample
    of row 0: a prefill of up to 4096 prompt tokens, then up to 16 greedy decode steps.
    The prefill and decode rates are reported apart and combined into the workload's
    tokens/s (its prefill and decode token counts at those rates)."""
    import oracle as O
    try:
        from threadpoolctl import threadpool_info
        cores = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        cores = len(os.sched_getaffinity(0))
    om = O.OracleModel(w.model, ck)
    Bn, T, N = w.batch, w.prompt_len, w.decode_steps
    t = min(T, 4096)
    if N == 0:
        t0 = time.perf_counter()
        om.forward_sequence(prompt[0][:t], 0, None, all_positions=True)
        pre = t / (time.perf_counter() - t0)
        return {"value": pre, "unit": "tokens/s", "cores": cores, "kind": "oracle",
                "prefill_tok_s": pre,
                "sample": f"row 0, its first {t} tokens, bidirectional, f32 NumPy"}
    n = min(16, N)
    cache = O.KVCache(w.model, t + n)
    t0 = time.perf_counter()
    lg = om.forward_sequence(prompt[0][:t], 0, cache)
    t1 = time.perf_counter()
    tok = int(O.greedy_argmax(lg))
    for k in range(n):
        tok = int(O.greedy_argmax(om.forward_token(tok, t + k, cache)))
    t2 = time.perf_counter()
    pre, dec = t / (t1 - t0), n / (t2 - t1)
    value = (Bn * T + Bn * N) / (Bn * T / pre + Bn * N / dec)
    return {"value": value, "unit": "tokens/s", "cores": cores, "kind": "oracle",
            "prefill_tok_s": pre, "decode_tok_s": dec,
            "sample": (f"row 0: prefill of its first {t} prompt tokens, then {n} greedy decode "
                       f"steps at positions {t}..{t + n - 1}, f32 NumPy; value = the workload's "
                       f"{Bn}x{T} prefill and {Bn}x{N} decode tokens at those two rates")}


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU (got --gpus {args.gpus}): the forward pass runs on one "
              "device and has no multi-GPU path", file=sys.stderr)
        sys.exit(2)
    if args.calibrate_copy:
        calibrate_copy(args.calibrate_copy)
        return
    import torch
    import workloads as W
    from gqa_decoder_transformer_amd import binding as B

    w = W.get(args.workload)
    m = w.model
    prec = B.EXACT if args.precision == "exact" else B.FAST
    kv = {"f32": B.F32, "bf16": B.BF16, None: None}[args.kv]
    s = torch.cuda.Stream(device=torch.device("cuda:0"))
    peaks = measure_peaks(s)
    progress(f"peaks {peaks}")

    r = Run(w, prec, kv, s)
    pre, dec, ms, wall = r.timed(args.steps, args.warmup)
    kernels, layer_us = r.kernels(args.timing_iters)
    sampler_us = r.sampler_us(max(4, args.timing_iters // 10))
    Bn, T, N = w.batch, w.prompt_len, w.decode_steps
    tokens = Bn * T + Bn * N
    value = tokens / (ms / 1000.0)
    mfma_path = m.weight_dtype in ("bf16", "q8_0")
    for v in kernels.values():
        meas = peaks["read_gbs"] if v["bound"] == "hbm" else (
            peaks["mfma_bf16_tflops"] if mfma_path else None)
        v["frac_measured_peak"] = v["achieved"] / meas if meas else None
    dom_name = max(kernels, key=lambda k: kernels[k]["ms_per_step"])
    dom = kernels[dom_name]
    extra = {"prefill_ms": pre, "prefill_tok_s": Bn * T / (pre / 1000.0)}
    if mfma_path:
        f = r.prefill_flops() / (pre * 1e-3) / 1e12
        extra["prefill_mfma_frac"] = f / PEAK_BF16_TFLOPS
        extra["prefill_mfma_frac_measured_peak"] = f / peaks["mfma_bf16_tflops"]
    if N > 0:
        ms_step = dec / N
        by = r.decode_bytes_per_step()
        extra["decode_tok_s"] = Bn * N / (dec / 1000.0)
        extra["decode_ms_per_step"] = ms_step
        extra["decode_bytes_per_step"] = by
        extra["decode_step_hbm_frac"] = by / (ms_step * 1e-3) / 1e9 / PEAK_HBM_GBS
        extra["decode_step_hbm_frac_measured_peak"] = by / (ms_step * 1e-3) / 1e9 / peaks["read_gbs"]
    r.close()

    line = {
        "metric": METRIC, "value": value, "unit": "tokens/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": ms,
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": precision_label(prec, B), "data": "synthetic",
        "config": {"workload": w.description, "batch": Bn, "prompt_len": T, "decode_steps": N,
                   "precision": args.precision,
                   "kv_dtype": "f32" if r.cfg.kv_dtype == B.F32 else "bf16",
                   "weights": f"random-init N(0,0.02) {m.weight_dtype}, seed {w.weight_seed}"},
        "wall_s": wall,
        "roofline": {"bound": dom["bound"], "kernel": dom_name,
                     "achieved": dom["achieved"], "peak": dom["peak"], "unit": dom["unit"],
                     "frac": dom["frac"], "frac_measured_peak": dom["frac_measured_peak"],
                     "traffic": measured_traffic(args.workload, args.precision, dom_name),
                     "avg_us": dom["avg_us"], "work_per_launch": dom["work_per_launch"]},
        "peaks": peaks,
        **extra,
        "kernels": {k: {kk: (round(vv, 4) if isinstance(vv, float) else vv)
                        for kk, vv in v.items()} for k, v in kernels.items()},
        "layer_us": {k: round(v, 3) for k, v in layer_us.items()},
        "sampler_us": {k: round(v, 3) for k, v in sampler_us.items()},
    }
    if not args.no_extra and args.workload == "longctx":
        line["extra"] = {"llama1b": extra_1b(s, peaks),
                         "longctx_bf16kv": extra_longctx_bf16kv(s, peaks)}
    if not args.no_cpu_baseline:
        progress("cpu baseline (oracle on the host cores)")
        line["cpu_baseline"] = cpu_baseline(w, r.ck, r.prompt)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
