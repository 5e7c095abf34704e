"""Brute-force form of the forward pass: scalar Python loops over Python floats (f64).

TEST INFRASTRUCTURE ONLY -- see the package docstring. Meant for tiny shapes only.

Written in the style of the Falcon-H1 Rust reference ("Falcon-H1-0.5B-Rust src/lib.rs":
``fn linear`` row-by-column loops, ``fn norm``, ``fn rope`` with the angle computed per
pair, and the per-query attention loops over ``j in 0..=t`` of ``Model::logits``), but for
the GQA decoder of the other pages (no Mamba branch, no multipliers). It shares no code
with the vectorised forms. The llama3 frequency scaling is written in its wavelength form
(unscaled when ``2*pi/freq < orig/high``, divided by ``factor`` when above ``orig/low``,
otherwise a linear blend in ``orig/wavelength``), which is algebraically the
``lerp(1/factor, 1, clip(z, 0, 1))`` form of "LowLlamaBasic reference.py".
"""
from __future__ import annotations

import math

import numpy as np


def _widen(tag, arr):
    if tag == "bf16":
        out = []
        for b in np.asarray(arr, dtype=np.uint16).reshape(-1).tolist():
            # sign, 8-bit exponent, 7-bit mantissa, decoded from the bit fields
            s = -1.0 if b & 0x8000 else 1.0
            e = (b >> 7) & 0xFF
            m = b & 0x7F
            if e == 0:
                out.append(s * m * 2.0 ** (-126 - 7))
            elif e == 0xFF:
                out.append(s * math.inf if m == 0 else math.nan)
            else:
                out.append(s * (1.0 + m / 128.0) * 2.0 ** (e - 127))
        return np.array(out, dtype=np.float64).reshape(np.asarray(arr).shape).tolist()
    return np.asarray(arr, dtype=np.float64).tolist()


def _linear(x, w):
    rows = len(w)
    cols = len(w[0])
    y = [0.0] * rows
    for i in range(rows):
        acc = 0.0
        for j in range(cols):
            acc += w[i][j] * x[j]
        y[i] = acc
    return y


def _norm(x, weight, eps):
    ss = 0.0
    for v in x:
        ss += v * v
    rms = math.sqrt(ss / len(x) + eps)
    return [a / rms * b for a, b in zip(x, weight)]


def _freqs(head_dim, theta, llama3):
    out = []
    for i in range(head_dim // 2):
        f = 1.0 / math.pow(theta, 2.0 * i / head_dim)
        if llama3 is not None:
            factor, low, high, orig = llama3
            wavelen = 2.0 * math.pi / f
            if wavelen < orig / high:
                pass
            elif wavelen > orig / low:
                f = f / factor
            else:
                smooth = (orig / wavelen - low) / (high - low)
                f = (1.0 - smooth) * f / factor + smooth * f
        out.append(f)
    return out


def _rope(x, pos, freqs):
    half = len(x) // 2
    y = list(x)
    for i in range(half):
        ang = pos * freqs[i]
        c, s = math.cos(ang), math.sin(ang)
        a, b = x[i], x[i + half]
        y[i] = a * c - b * s
        y[i + half] = b * c + a * s
    return y


def forward_all(cfg, checkpoint, ids, mask=None):
    """Head output at every position of one row ``ids`` (list of ints), full prefix, no
    cache. ``mask[t][j]`` (optional) marks key ``j`` admissible for query ``t``."""
    W = {name: _widen(tag, arr) for name, (tag, arr) in checkpoint.items()}
    n = len(ids)
    HD = cfg.head_dim
    freqs = _freqs(HD, cfg.rope_theta, cfg.llama3)
    x = [list(W["model.embed_tokens.weight"][i]) for i in ids]
    for layer in range(cfg.layers):
        p = f"model.layers.{layer}."
        a = [_norm(x[t], W[p + "input_layernorm.weight"], cfg.rms_eps) for t in range(n)]
        q, k, v = [], [], []
        for t in range(n):
            qt = _linear(a[t], W[p + "self_attn.q_proj.weight"])
            kt = _linear(a[t], W[p + "self_attn.k_proj.weight"])
            vt = _linear(a[t], W[p + "self_attn.v_proj.weight"])
            if cfg.qkv_bias:
                qt = [u + b for u, b in zip(qt, W[p + "self_attn.q_proj.bias"])]
                kt = [u + b for u, b in zip(kt, W[p + "self_attn.k_proj.bias"])]
                vt = [u + b for u, b in zip(vt, W[p + "self_attn.v_proj.bias"])]
            for h in range(cfg.heads):
                seg = qt[h * HD:(h + 1) * HD]
                if cfg.qk_norm:
                    seg = _norm(seg, W[p + "self_attn.q_norm.weight"], cfg.rms_eps)
                qt[h * HD:(h + 1) * HD] = _rope(seg, t, freqs)
            for h in range(cfg.kv_heads):
                seg = kt[h * HD:(h + 1) * HD]
                if cfg.qk_norm:
                    seg = _norm(seg, W[p + "self_attn.k_norm.weight"], cfg.rms_eps)
                kt[h * HD:(h + 1) * HD] = _rope(seg, t, freqs)
            q.append(qt)
            k.append(kt)
            v.append(vt)
        for t in range(n):
            y = [0.0] * (cfg.heads * HD)
            for h in range(cfg.heads):
                kv = h // (cfg.heads // cfg.kv_heads)
                keys = [j for j in range(n) if (j <= t or not cfg.causal)
                        and (mask is None or mask[t][j])]
                if not keys:  # fully masked row: uniform over the row's keys
                    keys_all = list(range(n))
                    wts = [1.0 / len(keys_all)] * len(keys_all)
                    keys = keys_all
                else:
                    scores = []
                    for j in keys:
                        d = 0.0
                        for e in range(HD):
                            d += q[t][h * HD + e] * k[j][kv * HD + e]
                        scores.append(d / math.sqrt(HD))
                    mx = max(scores)
                    ex = [math.exp(z - mx) for z in scores]
                    den = sum(ex)
                    wts = [e / den for e in ex]
                for wj, j in zip(wts, keys):
                    for e in range(HD):
                        y[h * HD + e] += wj * v[j][kv * HD + e]
            o = _linear(y, W[p + "self_attn.o_proj.weight"])
            for i in range(cfg.hidden):
                x[t][i] += o[i]
        for t in range(n):
            a2 = _norm(x[t], W[p + "post_attention_layernorm.weight"], cfg.rms_eps)
            g = _linear(a2, W[p + "mlp.gate_proj.weight"])
            u = _linear(a2, W[p + "mlp.up_proj.weight"])
            z = [gi / (1.0 + math.exp(-gi)) * ui for gi, ui in zip(g, u)]
            d = _linear(z, W[p + "mlp.down_proj.weight"])
            for i in range(cfg.hidden):
                x[t][i] += d[i]
    out = []
    for t in range(n):
        h = _norm(x[t], W["model.norm.weight"], cfg.rms_eps)
        if cfg.head == "tied_lm":
            out.append(_linear(h, W["model.embed_tokens.weight"]))
        else:
            lg = _linear(h, W["token_cls_head.weight"])
            out.append([a + b for a, b in zip(lg, W["token_cls_head.bias"])])
    return np.array(out, dtype=np.float64)


def argmax_first(row):
    """Lowest index of the maximum, by a scalar scan."""
    best, bi = -math.inf, 0
    for i, val in enumerate(row):
        if val > best:
            best, bi = val, i
    return bi
