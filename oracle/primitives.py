"""Oracle primitives: the per-step math of the decoder forward pass, written out plainly.

TEST INFRASTRUCTURE ONLY -- see the package docstring. Every function states the passage
of the pages it follows. Arrays carry their own dtype: float32 reproduces the pages'
f32 arithmetic, float64 is the shadow used to measure rounding error.
"""
from __future__ import annotations

import numpy as np

NEG_INF = -np.inf


# --------------------------------------------------------------------------- weights

def widen_bf16(bits: np.ndarray) -> np.ndarray:
    """bf16 -> f32 widening: the 16 stored bits become the high half of an f32 word.

    Exact for every bit pattern. Follows "ember scripts/reference_forward.py",
    ``load_safetensors`` (the BF16 branch: uint16 -> uint32, shift left 16, view as f32).
    """
    u = np.asarray(bits, dtype=np.uint16).astype(np.uint32)
    return (u << np.uint32(16)).view(np.float32)


def f16_to_f32(bits: np.ndarray) -> np.ndarray:
    """IEEE binary16 bit patterns -> f32 values (exact: every f16 value is an f32 value).

    Sign bit 15, exponent bits 14..10 (bias 15), fraction bits 9..0: exponent 0 is zero or
    subnormal (fraction * 2^-24), 1..30 normal ((1024 + fraction) * 2^(exponent - 25)),
    31 infinity (fraction 0) or NaN."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.int64)
    sign = np.where(b >> 15, -1.0, 1.0)
    e = (b >> 10) & 0x1F
    f = (b & 0x3FF).astype(np.float64)
    mag = np.where(e == 0, f * 2.0 ** -24, (1024.0 + f) * np.exp2((e - 25).astype(np.float64)))
    mag = np.where(e == 31, np.where(f == 0, np.inf, np.nan), mag)
    return (sign * mag).astype(np.float32)


Q8_BLOCK = 32          # values per q8_0 block
Q8_BLOCK_BYTES = 34    # 2-byte scale + 32 int8


def dequant_q8_0(raw: np.ndarray, k: int) -> np.ndarray:
    """q8_0 rows -> f32 [n, k] ("ember internals", section
    "GGUF format and quantization", subsection "q8_0 block quantization", its
    decompression loop): each block of 34 bytes is a
    little-endian f16 scale d followed by 32 signed int8 values q, and block value j is
    q_j * d in f32. Blocks run along the row (the inner dimension, a multiple of 32).
    The product of an int8 and an f16 value is exact in f32."""
    raw = np.asarray(raw, dtype=np.uint8)
    if k % Q8_BLOCK:
        raise ValueError("q8_0 rows need a multiple of 32 values")
    n = raw.shape[0]
    blocks = raw.reshape(n, k // Q8_BLOCK, Q8_BLOCK_BYTES)
    d_bits = blocks[..., 0].astype(np.uint16) | (blocks[..., 1].astype(np.uint16) << np.uint16(8))
    d = f16_to_f32(d_bits)[..., None]
    q = blocks[..., 2:].view(np.int8).astype(np.float32)
    return (q * d).astype(np.float32).reshape(n, k)


def decode_tensor(dtype_tag: str, arr: np.ndarray) -> np.ndarray:
    """A stored tensor as f32 values: BF16 is widened, F32 passes through, q8_0 rows
    ([n, k / 32 * 34] bytes) are dequantised; anything else is an error ("ember
    scripts/reference_forward.py", ``load_safetensors``, final branch)."""
    if dtype_tag == "bf16":
        return widen_bf16(arr)
    if dtype_tag == "f32":
        return np.asarray(arr, dtype=np.float32)
    if dtype_tag == "q8_0":
        return dequant_q8_0(arr, arr.shape[1] // Q8_BLOCK_BYTES * Q8_BLOCK)
    raise ValueError(f"unsupported dtype {dtype_tag}")


# --------------------------------------------------------------------------- norms

def rmsnorm(x: np.ndarray, w: np.ndarray, eps: float) -> np.ndarray:
    """RMSNorm over the last axis: ``x / sqrt(mean(x^2) + eps) * w``.

    The operation order is the one of "ember scripts/reference_forward.py" (``rmsnorm``);
    "LowLlamaBasic reference.py" (``rms_norm``), "PII-Tracer serving/reference_forward.py"
    (``rms_norm``) and the ember internals page ("RMS norm") state the same formula.
    """
    ms = np.mean(x * x, axis=-1, keepdims=True)
    return x / np.sqrt(ms + x.dtype.type(eps)) * w


# --------------------------------------------------------------------------- RoPE

def rope_inv_freq(head_dim: int, theta: float, llama3=None) -> np.ndarray:
    """Rotary frequencies in float64, one per rotated pair ``(i, i + head_dim/2)``.

    ``freq_i = 1 / theta^(2i / head_dim)`` ("ember scripts/reference_forward.py",
    ``inv_freq`` in ``main``). With ``llama3 = (factor, low, high, orig)`` each frequency is
    multiplied by ``lerp(1/factor, 1, clip(z, 0, 1))``, ``z = (orig*freq/(2*pi) - low) /
    (high - low)`` ("LowLlamaBasic reference.py", ``rotary_cos_sin``). Evaluated in f64.
    """
    half = head_dim // 2
    freq = 1.0 / (float(theta) ** (2.0 * np.arange(half, dtype=np.float64) / head_dim))
    if llama3 is not None:
        factor, low, high, orig = (float(v) for v in llama3)
        z = (orig * freq / (2.0 * np.pi) - low) / (high - low)
        wgt = np.clip(z, 0.0, 1.0)
        start = 1.0 / factor
        freq = freq * (start + wgt * (1.0 - start))
    return freq


def rope_tables(n_pos: int, head_dim: int, theta: float, llama3=None,
                dtype=np.float32):
    """cos/sin tables ``[n_pos, head_dim/2]`` for positions ``0..n_pos-1``.

    Angles ``pos * freq`` and their cos/sin are computed in f64 and rounded once to
    ``dtype``: the tables are precomputed so the hot path does no trigonometry (ember
    internals page, "rotary position embeddings"); f64 angles follow the NumPy reference.
    """
    inv = rope_inv_freq(head_dim, theta, llama3)
    ang = np.arange(n_pos, dtype=np.float64)[:, None] * inv[None, :]
    return np.cos(ang).astype(dtype), np.sin(ang).astype(dtype)


def apply_rope(x: np.ndarray, cos: np.ndarray, sin: np.ndarray) -> np.ndarray:
    """Rotate-half RoPE over the last axis: elements ``i`` and ``i + half`` form a pair.

    ``out[i] = x[i] cos - x[i+half] sin``, ``out[i+half] = x[i+half] cos + x[i] sin``
    ("ember scripts/reference_forward.py", ``rope``; "LowLlamaBasic reference.py",
    ``rotate``; "PII-Tracer serving/reference_forward.py", ``apply_rope``). ``cos``/``sin``
    broadcast against ``x[..., :half]``.
    """
    half = x.shape[-1] // 2
    x0 = x[..., :half]
    x1 = x[..., half:]
    return np.concatenate([x0 * cos - x1 * sin, x1 * cos + x0 * sin], axis=-1)


# --------------------------------------------------------------------------- softmax

def softmax(s: np.ndarray) -> np.ndarray:
    """Max-subtracted softmax over the last axis with the fully-masked-row fallback.

    ``exp(s - max) / sum`` ("ember scripts/reference_forward.py", the score softmax in
    ``forward``); a row whose maximum is -inf (every entry masked) becomes uniform
    (ember internals page, sampler step "softmax", and "edge cases": fully masked rows).
    """
    m = np.max(s, axis=-1, keepdims=True)
    dead = np.isneginf(m)
    with np.errstate(invalid="ignore", divide="ignore"):
        e = np.exp(s - np.where(dead, 0, m).astype(s.dtype))
        p = e / np.sum(e, axis=-1, keepdims=True)
    n = s.shape[-1]
    return np.where(dead, s.dtype.type(1.0 / n) if n else s.dtype.type(0), p).astype(s.dtype)


# --------------------------------------------------------------------------- attention

def attention(q: np.ndarray, k: np.ndarray, v: np.ndarray, q_pos: np.ndarray,
              k_pos: np.ndarray, causal: bool, mask: np.ndarray | None = None,
              q_block: int = 1024) -> np.ndarray:
    """Grouped-query scaled dot-product attention.

    q ``[T, NH, HD]``, k/v ``[S, NKV, HD]``; query head ``h`` reads kv head
    ``h // (NH/NKV)`` (ember internals page, "grouped-query attention"; NumPy reference,
    ``kh = h // GROUP``). Scores are ``q.k * (1/sqrt(HD))`` (scale applied as a multiply in
    the array dtype); key ``s`` is admissible for query ``t`` iff ``k_pos[s] <= q_pos[t]``
    when ``causal`` ("LowLlamaBasic reference.py", ``self_attn``: the strictly upper
    triangle is -inf), and always when not ("PII-Tracer serving/reference_forward.py":
    no mask). ``mask`` (bool ``[T, S]``, True = admissible) further restricts keys; it
    exists so tests can reach the fully-masked-row fallback of ``softmax``. The output is
    ``softmax(scores) @ v`` per head, ``[T, NH, HD]``.

    The block arithmetic runs on torch CPU tensors (multithreaded elementwise ops; the
    steps are the ones above, with the fallback of ``softmax``), the query heads that share
    a kv head batched together, and queries in blocks of ``q_block`` rows to bound memory.
    In the causal case without an explicit mask every query of a block admits key
    position 0..its own position, so keys after the block's last query position are
    inadmissible for all of its rows and contribute exactly zero; they are dropped from
    that block's product.
    """
    import torch
    T, NH, HD = q.shape
    S, NKV, _ = k.shape
    if NH % NKV:
        raise ValueError("query heads must be a multiple of kv heads")
    group = NH // NKV
    dt = torch.float64 if q.dtype == np.float64 else torch.float32
    scale = torch.tensor(q.dtype.type(1.0 / np.sqrt(HD)), dtype=dt)
    out = np.zeros((T, NH, HD), dtype=q.dtype)
    q_pos = np.asarray(q_pos)
    k_pos = np.asarray(k_pos)
    tq = torch.from_numpy(np.ascontiguousarray(q))
    tk = torch.from_numpy(np.ascontiguousarray(k))
    tv = torch.from_numpy(np.ascontiguousarray(v))
    for t0 in range(0, T, q_block):
        t1 = min(T, t0 + q_block)
        qp = q_pos[t0:t1]
        s_hi = S
        if causal and mask is None and S and k_pos[0] <= qp.min() and np.all(np.diff(k_pos) > 0):
            s_hi = int(np.searchsorted(k_pos, qp.max(), side="right"))
        allowed = np.ones((t1 - t0, s_hi), dtype=bool)
        if causal:
            allowed &= k_pos[None, :s_hi] <= qp[:, None]
        if mask is not None:
            allowed &= mask[t0:t1, :s_hi]
        ta = torch.from_numpy(allowed)
        for kh in range(NKV):
            hs = slice(kh * group, (kh + 1) * group)
            qb = tq[t0:t1, hs, :].permute(1, 0, 2)                  # [G, tb, HD]
            sc = torch.matmul(qb, tk[:s_hi, kh, :].T) * scale       # [G, tb, s_hi]
            sc = torch.where(ta, sc, torch.tensor(float("-inf"), dtype=dt))
            p = _softmax_t(sc)
            out[t0:t1, hs, :] = torch.matmul(p, tv[:s_hi, kh, :]).permute(1, 0, 2).numpy()
    return out


def _softmax_t(s):
    """``softmax`` on a torch tensor (same max-subtracted form and fallback)."""
    import torch
    m = torch.amax(s, dim=-1, keepdim=True) if s.shape[-1] else torch.zeros(s.shape[:-1] + (1,), dtype=s.dtype)
    dead = torch.isneginf(m)
    e = torch.exp(s - torch.where(dead, torch.zeros_like(m), m))
    p = e / torch.sum(e, dim=-1, keepdim=True)
    n = s.shape[-1]
    return torch.where(dead, torch.full_like(p, 1.0 / n if n else 0.0), p)


# --------------------------------------------------------------------------- MLP

def silu(z: np.ndarray) -> np.ndarray:
    """``z / (1 + exp(-z))`` ("LowLlamaBasic reference.py", ``silu``; NumPy reference)."""
    with np.errstate(over="ignore"):
        return z / (z.dtype.type(1.0) + np.exp(-z))


def swiglu(gate: np.ndarray, up: np.ndarray) -> np.ndarray:
    """``silu(gate) * up`` (ember internals page, "SwiGLU mlp"; NumPy reference ``act``)."""
    return silu(gate) * up


# --------------------------------------------------------------------------- argmax

def greedy_argmax(logits: np.ndarray) -> np.ndarray:
    """Greedy token choice: the lowest index of the maximum logit along the last axis.

    ``np.argmax`` as in the NumPy reference's decode loop (first maximum wins; the Rust
    ``max_by`` variants of the other pages would take the last). NaN is an error.
    """
    if np.isnan(logits).any():
        raise FloatingPointError("non-finite (NaN) logits")
    return np.argmax(logits, axis=-1)
