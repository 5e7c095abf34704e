"""Seeded synthetic inputs: random-init weights and random prompt ids.

This module is shared by the oracle and the GPU path and holds none of the forward
pass's arithmetic: it only draws numbers and stores them in the checkpoint formats the
pages load (bf16 bit patterns or f32, under HuggingFace tensor names).

Recipe (all draws from ``numpy.random.default_rng(seed)``, PCG64):

* weights: seed = the workload's ``weight_seed``; tensors are drawn in a fixed order --
  embedding, then per layer the order in which ember's NumPy reference reads them
  (q, q-bias, k, k-bias, v, v-bias, o, gate, up, down), then the classification head
  weight and bias, then (when configured) the sensitivity head's weight and bias; each
  draw is ``standard_normal(shape, float32) * 0.02``.
* every RMSNorm weight (input, post-attention, final, per-head q/k) is 1.0 and is not
  drawn, as the Falcon-H1 Rust reference's ``synthetic_weights`` fills norm weights with 1.
* bf16 models: each f32 draw is rounded once to bf16 (round to nearest, ties to even);
  those bf16 values *are* the model.
* q8_0 models: every matrix is quantised to q8_0 blocks (``quantize_q8_0``: per 32
  values d = f16(max|x| / 127), q = rint(x / d)); the dequantised values are the model.
  Norm weights and biases stay f32.
* prompt ids: seed = the workload's ``ids_seed``,
  ``integers(0, vocab, size=(batch, prompt_len), dtype=int32)``.
* sampler draws: ``random((n_pos, ld), dtype=float32)``, values in [0, 1).
* sampler logits (inputs of the sampling stage alone): per row a spread
  s = ``uniform(1, 4)``, ``standard_normal(vocab, float32) * s``, and 16 distinct
  tokens raised by ``uniform(2, 10) * s`` (a peaked head over a broad tail, as an LM's
  next-token logits); with ``ties`` the values are rounded to multiples of 1/4, so many
  tokens share a value.
"""
from __future__ import annotations

from collections import OrderedDict
from typing import Dict, Tuple

import numpy as np

from .configs import ModelConfig, Workload

# A checkpoint: HF tensor name -> (dtype tag, array). dtype tag "bf16" means the array is
# uint16 bit patterns; "f32" means float32 values.
Checkpoint = "OrderedDict[str, Tuple[str, np.ndarray]]"

INIT_STD = 0.02


def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """Round float32 values to bfloat16 (nearest, ties to even) and return the bit patterns.

    Used only to store the seeded draws in bf16, the checkpoint format; inputs are finite.
    """
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32)
    bias = ((u >> np.uint32(16)) & np.uint32(1)) + np.uint32(0x7FFF)
    return ((u + bias) >> np.uint32(16)).astype(np.uint16)


def tensor_shapes(m: ModelConfig) -> "OrderedDict[str, Tuple[int, ...]]":
    """Names and shapes of every tensor of the model, in draw order."""
    s: "OrderedDict[str, Tuple[int, ...]]" = OrderedDict()
    s["model.embed_tokens.weight"] = (m.vocab, m.hidden)
    for i in range(m.layers):
        p = f"model.layers.{i}."
        s[p + "input_layernorm.weight"] = (m.hidden,)
        s[p + "self_attn.q_proj.weight"] = (m.q_dim, m.hidden)
        if m.qkv_bias:
            s[p + "self_attn.q_proj.bias"] = (m.q_dim,)
        s[p + "self_attn.k_proj.weight"] = (m.kv_dim, m.hidden)
        if m.qkv_bias:
            s[p + "self_attn.k_proj.bias"] = (m.kv_dim,)
        s[p + "self_attn.v_proj.weight"] = (m.kv_dim, m.hidden)
        if m.qkv_bias:
            s[p + "self_attn.v_proj.bias"] = (m.kv_dim,)
        s[p + "self_attn.o_proj.weight"] = (m.hidden, m.q_dim)
        if m.qk_norm:
            s[p + "self_attn.q_norm.weight"] = (m.head_dim,)
            s[p + "self_attn.k_norm.weight"] = (m.head_dim,)
        s[p + "post_attention_layernorm.weight"] = (m.hidden,)
        s[p + "mlp.gate_proj.weight"] = (m.ffn, m.hidden)
        s[p + "mlp.up_proj.weight"] = (m.ffn, m.hidden)
        s[p + "mlp.down_proj.weight"] = (m.hidden, m.ffn)
    s["model.norm.weight"] = (m.hidden,)
    if m.head == "cls":
        s["token_cls_head.weight"] = (m.n_classes, m.hidden)
        s["token_cls_head.bias"] = (m.n_classes,)
    if m.sens_head:
        s["sensitivity_head.weight"] = (1, m.hidden)
        s["sensitivity_head.bias"] = (1,)
    return s


def is_norm_weight(name: str) -> bool:
    return name.endswith("layernorm.weight") or name.endswith("norm.weight")


def make_weights(m: ModelConfig, seed: int) -> "OrderedDict[str, Tuple[str, np.ndarray]]":
    rng = np.random.default_rng(seed)
    out: "OrderedDict[str, Tuple[str, np.ndarray]]" = OrderedDict()
    for name, shape in tensor_shapes(m).items():
        if is_norm_weight(name):
            a = np.ones(shape, dtype=np.float32)
        else:
            a = rng.standard_normal(shape, dtype=np.float32)
            a *= np.float32(INIT_STD)
        if m.weight_dtype == "bf16":
            out[name] = ("bf16", f32_to_bf16_bits(a))
        elif m.weight_dtype == "f32":
            out[name] = ("f32", a)
        elif m.weight_dtype == "q8_0":
            out[name] = ("q8_0", quantize_q8_0(a)) if a.ndim == 2 else ("f32", a)
        else:
            raise ValueError(f"unknown weight dtype {m.weight_dtype}")
    return out


def quantize_q8_0(a: np.ndarray) -> np.ndarray:
    """f32 [n, k] -> q8_0 rows [n, k / 32 * 34] uint8 (the stored form of a q8_0 model).

    Per block of 32 values along the row: d = f16(max|x| / 127), q = clip(rint(x / d),
    -127, 127) (q = 0 when d = 0); stored as d's two bytes, little-endian, then the 32 q
    bytes. Only makes test and benchmark inputs: the dequantised values q * d *are* the
    model."""
    a = np.ascontiguousarray(a, dtype=np.float32)
    n, k = a.shape
    if k % 32:
        raise ValueError("q8_0 rows need a multiple of 32 values")
    blk = a.reshape(n, k // 32, 32)
    d16 = (np.abs(blk).max(-1) / np.float32(127.0)).astype(np.float16)
    d = d16.astype(np.float32)[..., None]
    with np.errstate(divide="ignore", invalid="ignore"):
        q = np.where(d > 0, np.rint(blk / np.where(d > 0, d, 1.0)), 0.0)
    q = np.clip(q, -127, 127).astype(np.int8)
    out = np.empty((n, k // 32, 34), np.uint8)
    out[..., :2] = d16.view(np.uint8).reshape(n, k // 32, 2)      # little-endian f16
    out[..., 2:] = q.view(np.uint8)
    return out.reshape(n, k // 32 * 34)


def make_ids(w: Workload, batch: int | None = None, prompt_len: int | None = None) -> np.ndarray:
    rng = np.random.default_rng(w.ids_seed)
    b = w.batch if batch is None else batch
    t = w.prompt_len if prompt_len is None else prompt_len
    return rng.integers(0, w.model.vocab, size=(b, t), dtype=np.int32)


_cache: Dict[Tuple, object] = {}


def weights_for(w: Workload):
    """Weights of a workload, memoised per process (the large shapes take seconds)."""
    key = (w.model, w.weight_seed)
    if key not in _cache:
        _cache[key] = make_weights(w.model, w.weight_seed)
    return _cache[key]


def make_uniforms(seed: int, n_pos: int, ld: int) -> np.ndarray:
    """Draws of the sampler, [n_pos, ld] float32 in [0, 1)."""
    return np.random.default_rng(seed).random((n_pos, ld), dtype=np.float32)


def make_logits(seed: int, rows: int, vocab: int, ties: bool = False) -> np.ndarray:
    """LM-like next-token logits [rows, vocab] float32 (recipe in the module docstring)."""
    rng = np.random.default_rng(seed)
    out = np.empty((rows, vocab), np.float32)
    for r in range(rows):
        s = np.float32(rng.uniform(1.0, 4.0))
        z = rng.standard_normal(vocab, dtype=np.float32) * s
        head = rng.choice(vocab, size=min(16, vocab), replace=False)
        z[head] += rng.uniform(2.0, 10.0, size=head.size).astype(np.float32) * s
        if ties:
            z = np.round(z * 4.0) / 4.0
        out[r] = z.astype(np.float32)
    return out
