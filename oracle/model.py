"""Oracle model: the decoder (and bidirectional encoder) forward pass in two forms.

TEST INFRASTRUCTURE ONLY -- see the package docstring.

* ``forward_sequence`` -- the full-sequence form: every position of a row in one pass of
  ``[T, H]`` matrix products and a masked ``[T, S]`` score matrix per head
  ("LowLlamaBasic reference.py", ``predict``; "PII-Tracer serving/reference_forward.py",
  ``forward``). With a ``KVCache`` it also stores k/v at explicit positions and attends
  over everything stored before, so it doubles as the prefill.
* ``forward_token`` -- the incremental form of "ember scripts/reference_forward.py"
  (``forward(tok, pos)``): one token, matrix-vector products, per-head loops, k/v
  appended to the cache at the explicit position ``pos`` (the fix of the ember internals
  page's KV-cache bug: "pos = cursor + token_index").

Both read the same widened weights; tests check that they agree (cached decode equals
full-prefix recompute).
"""
from __future__ import annotations

import numpy as np

from .primitives import (apply_rope, attention, decode_tensor, greedy_argmax, rmsnorm,
                         rope_tables, softmax, swiglu)

MAX_TOKENS = 16384  # sequence cap of the Falcon-H1 Rust reference (``Model::logits``)


class KVCache:
    """Per-layer K/V storage ``[max_seq, NKV, HD]`` written at explicit positions.

    One contiguous block per layer holding every kv head and position, kv heads only
    (ember internals page, "kv cache" layout and GQA: the cache stores n_kv_heads).
    """

    def __init__(self, cfg, max_seq: int, dtype=np.float32):
        self.max_seq = max_seq
        self.k = [np.zeros((max_seq, cfg.kv_heads, cfg.head_dim), dtype) for _ in range(cfg.layers)]
        self.v = [np.zeros((max_seq, cfg.kv_heads, cfg.head_dim), dtype) for _ in range(cfg.layers)]
        self.length = 0   # positions 0..length-1 hold data

    def write(self, layer: int, positions: np.ndarray, k: np.ndarray, v: np.ndarray):
        if positions.max() >= self.max_seq:
            raise ValueError("KV cache capacity exceeded")
        self.k[layer][positions] = k
        self.v[layer][positions] = v

    def view(self, layer: int, n: int):
        return self.k[layer][:n], self.v[layer][:n], np.arange(n)


class OracleModel:
    def __init__(self, cfg, checkpoint, dtype=np.float32):
        """``checkpoint``: HF tensor name -> (dtype tag, array), as the seeded generator
        stores it. Every tensor is widened to f32 ("ember scripts/reference_forward.py",
        ``load_safetensors``), then held in ``dtype``."""
        self.cfg = cfg
        self.dtype = np.dtype(dtype)
        self.w = {}
        for name, (tag, arr) in checkpoint.items():
            a = decode_tensor(tag, arr)
            self.w[name] = a if a.dtype == self.dtype else a.astype(self.dtype)
        self._cos = np.zeros((0, cfg.head_dim // 2), self.dtype)
        self._sin = self._cos

    # -- helpers ---------------------------------------------------------------------
    def tables(self, positions: np.ndarray):
        need = int(positions.max()) + 1
        if need > self._cos.shape[0]:
            n = max(need, 2 * self._cos.shape[0])
            c = self.cfg
            self._cos, self._sin = rope_tables(n, c.head_dim, c.rope_theta, c.llama3,
                                               dtype=self.dtype)
        return self._cos[positions], self._sin[positions]

    def _check_ids(self, ids):
        ids = np.asarray(ids)
        if ids.size == 0:
            raise ValueError("input_ids must not be empty")
        if ids.shape[-1] > MAX_TOKENS:
            raise ValueError("sequence too long")
        if (ids < 0).any() or (ids >= self.cfg.vocab).any():
            raise ValueError("token outside vocabulary")
        return ids

    def head(self, h: np.ndarray) -> np.ndarray:
        """Final RMSNorm, then the tied LM head ``E . h`` ("ember scripts/
        reference_forward.py", end of ``forward``) or, for the encoder, the token
        classification head ``Wc h + bc`` ("PII-Tracer serving/reference_forward.py")."""
        c, w = self.cfg, self.w
        h = rmsnorm(h, w["model.norm.weight"], c.rms_eps)
        if c.head == "tied_lm":
            return h @ w["model.embed_tokens.weight"].T
        return h @ w["token_cls_head.weight"].T + w["token_cls_head.bias"]

    # -- full-sequence form ------------------------------------------------------------
    def layer_sequence(self, li: int, x: np.ndarray, positions: np.ndarray,
                       cache: KVCache | None) -> np.ndarray:
        """One decoder block over ``T`` tokens of one row, ``x [T, H]``."""
        c, w = self.cfg, self.w
        p = f"model.layers.{li}."
        T = x.shape[0]
        xb = rmsnorm(x, w[p + "input_layernorm.weight"], c.rms_eps)
        q = xb @ w[p + "self_attn.q_proj.weight"].T
        k = xb @ w[p + "self_attn.k_proj.weight"].T
        v = xb @ w[p + "self_attn.v_proj.weight"].T
        if c.qkv_bias:
            q = q + w[p + "self_attn.q_proj.bias"]
            k = k + w[p + "self_attn.k_proj.bias"]
            v = v + w[p + "self_attn.v_proj.bias"]
        q = q.reshape(T, c.heads, c.head_dim)
        k = k.reshape(T, c.kv_heads, c.head_dim)
        v = v.reshape(T, c.kv_heads, c.head_dim)
        if c.qk_norm:  # per-head RMSNorm before RoPE (PII-Tracer ``forward``)
            q = rmsnorm(q, w[p + "self_attn.q_norm.weight"], c.rms_eps)
            k = rmsnorm(k, w[p + "self_attn.k_norm.weight"], c.rms_eps)
        cos, sin = self.tables(positions)
        q = apply_rope(q, cos[:, None, :], sin[:, None, :])
        k = apply_rope(k, cos[:, None, :], sin[:, None, :])
        if cache is not None:
            cache.write(li, positions, k, v)
            kk, vv, kpos = cache.view(li, int(positions.max()) + 1)
        else:
            kk, vv, kpos = k, v, positions
        att = attention(q, kk, vv, positions, kpos, c.causal)
        x = x + att.reshape(T, c.q_dim) @ w[p + "self_attn.o_proj.weight"].T
        xb = rmsnorm(x, w[p + "post_attention_layernorm.weight"], c.rms_eps)
        act = swiglu(xb @ w[p + "mlp.gate_proj.weight"].T, xb @ w[p + "mlp.up_proj.weight"].T)
        return x + act @ w[p + "mlp.down_proj.weight"].T

    def forward_sequence(self, ids, start_pos: int = 0, cache: KVCache | None = None,
                         all_positions: bool = False, progress=None) -> np.ndarray:
        """Forward of one row of ``T`` tokens at positions ``start_pos..start_pos+T-1``.

        Returns the head output at the last position (``[out_dim]``) or, with
        ``all_positions``, at every position (``[T, out_dim]``). ``progress(layer)`` is
        called after each layer when given (long runs report that they are alive).
        """
        ids = self._check_ids(ids)
        T = ids.shape[0]
        positions = np.arange(start_pos, start_pos + T)
        x = self.w["model.embed_tokens.weight"][ids].astype(self.dtype, copy=True)
        for li in range(self.cfg.layers):
            x = self.layer_sequence(li, x, positions, cache)
            if progress is not None:
                progress(li)
        if cache is not None:
            cache.length = max(cache.length, start_pos + T)
        return self.head(x if all_positions else x[-1])

    def forward_with_activations(self, ids, start_pos: int = 0, cache: KVCache | None = None):
        """The forward pass of one row that also keeps the hidden state after every block
        at the last position (ember internals, "ForwardModel trait",
        ``forward_with_activations``, and "probing pipeline": ``activations[layer][d]``).
        Returns ``(acts [layers, H], head output at the last position)``; the states are
        the residual stream before the final norm."""
        ids = self._check_ids(ids)
        T = ids.shape[0]
        positions = np.arange(start_pos, start_pos + T)
        x = self.w["model.embed_tokens.weight"][ids].astype(self.dtype, copy=True)
        acts = []
        for li in range(self.cfg.layers):
            x = self.layer_sequence(li, x, positions, cache)
            acts.append(x[-1].copy())
        if cache is not None:
            cache.length = max(cache.length, start_pos + T)
        return np.stack(acts), self.head(x[-1])

    def sensitivity(self, ids) -> float:
        """The encoder's sequence score ("PII-Tracer serving/reference_forward.py",
        ``forward``, sensitivity head): the final-normed hidden states averaged over the
        row's tokens, then ``. sensitivity_head.weight + sensitivity_head.bias``."""
        ids = self._check_ids(ids)
        positions = np.arange(ids.shape[0])
        x = self.w["model.embed_tokens.weight"][ids].astype(self.dtype, copy=True)
        for li in range(self.cfg.layers):
            x = self.layer_sequence(li, x, positions, None)
        h = rmsnorm(x, self.w["model.norm.weight"], self.cfg.rms_eps)
        s = h.mean(0) @ self.w["sensitivity_head.weight"].T + self.w["sensitivity_head.bias"]
        return float(s[0])

    def encode(self, ids) -> np.ndarray:
        """Bidirectional encoder over a batch ``[B, T]`` -> per-token head ``[B, T, C]``."""
        ids = np.atleast_2d(ids)
        return np.stack([self.forward_sequence(r, 0, None, all_positions=True) for r in ids])

    # -- incremental (cached) form -----------------------------------------------------
    def forward_token(self, tok: int, pos: int, cache: KVCache) -> np.ndarray:
        """One token at position ``pos`` against the cache, as in the NumPy reference's
        ``forward(tok, pos)``: matrix-vector products, RoPE per head, k/v stored at
        ``pos``, then a per-head softmax over cached positions ``0..pos``."""
        c, w = self.cfg, self.w
        if not c.causal:
            raise ValueError("the cached form is defined for causal models only")
        self._check_ids([tok])
        HD, G = c.head_dim, c.group
        x = w["model.embed_tokens.weight"][tok].astype(self.dtype, copy=True)
        cos, sin = self.tables(np.array([pos]))
        cos, sin = cos[0], sin[0]
        scale = self.dtype.type(1.0 / np.sqrt(HD))
        for li in range(c.layers):
            p = f"model.layers.{li}."
            xb = rmsnorm(x, w[p + "input_layernorm.weight"], c.rms_eps)
            q = w[p + "self_attn.q_proj.weight"] @ xb
            k = w[p + "self_attn.k_proj.weight"] @ xb
            v = w[p + "self_attn.v_proj.weight"] @ xb
            if c.qkv_bias:
                q = q + w[p + "self_attn.q_proj.bias"]
                k = k + w[p + "self_attn.k_proj.bias"]
                v = v + w[p + "self_attn.v_proj.bias"]
            for h in range(c.heads):
                seg = q[h * HD:(h + 1) * HD]
                if c.qk_norm:
                    seg = rmsnorm(seg, w[p + "self_attn.q_norm.weight"], c.rms_eps)
                q[h * HD:(h + 1) * HD] = apply_rope(seg, cos, sin)
            for h in range(c.kv_heads):
                seg = k[h * HD:(h + 1) * HD]
                if c.qk_norm:
                    seg = rmsnorm(seg, w[p + "self_attn.k_norm.weight"], c.rms_eps)
                k[h * HD:(h + 1) * HD] = apply_rope(seg, cos, sin)
            cache.write(li, np.array([pos]), k.reshape(1, c.kv_heads, HD),
                        v.reshape(1, c.kv_heads, HD))
            kc, vc, _ = cache.view(li, pos + 1)
            att = np.zeros(c.q_dim, self.dtype)
            for h in range(c.heads):
                kh = h // G
                sc = (kc[:, kh, :] @ q[h * HD:(h + 1) * HD]) * scale
                att[h * HD:(h + 1) * HD] = softmax(sc) @ vc[:, kh, :]
            x = x + w[p + "self_attn.o_proj.weight"] @ att
            xb = rmsnorm(x, w[p + "post_attention_layernorm.weight"], c.rms_eps)
            act = swiglu(w[p + "mlp.gate_proj.weight"] @ xb, w[p + "mlp.up_proj.weight"] @ xb)
            x = x + w[p + "mlp.down_proj.weight"] @ act
        cache.length = max(cache.length, pos + 1)
        return self.head(x)


def generate(model: OracleModel, prompt, n_steps: int, max_seq: int | None = None,
             progress=None, pick=None, return_cache: bool = False):
    """Prefill once, then ``n_steps`` steps, one cached forward each (the NumPy
    reference's generation loop; ember internals page: one prefill and one cached step per
    new token). End-of-sequence ids are not special: the step count is fixed.

    ``pick(k, logits) -> id`` chooses the token after step ``k`` (``k = 0``: the prefill);
    by default the greedy argmax. Returns ``(ids, logits)`` with ``logits[k]`` the head
    output after step ``k`` (``k = 0`` is the prefill's last position) and ``ids[k]`` the
    token picked from it: ``n_steps + 1`` of each, of which ``ids[0..n_steps-1]`` are fed
    back. With ``return_cache`` the ``KVCache`` after the last step is returned third.
    """
    if pick is None:
        def pick(k, lg):
            return int(greedy_argmax(lg))
    prompt = np.asarray(prompt)
    T = prompt.shape[0]
    cache = KVCache(model.cfg, max_seq or (T + n_steps), model.dtype)
    logits = [model.forward_sequence(prompt, 0, cache, progress=progress)]
    ids = [int(pick(0, logits[0]))]
    for k in range(n_steps):
        logits.append(model.forward_token(ids[-1], T + k, cache))
        ids.append(int(pick(k + 1, logits[-1])))
    if return_cache:
        return np.array(ids, dtype=np.int64), np.stack(logits), cache
    return np.array(ids, dtype=np.int64), np.stack(logits)


def recompute_logits(model: OracleModel, prompt, fed_ids) -> np.ndarray:
    """Full-prefix recompute (no cache): logits at the last prompt position and after
    each fed id, from one full-sequence pass over ``prompt + fed_ids`` -- the form of
    "LowLlamaBasic reference.py" and of the Rust reference's ``generate``."""
    seq = np.concatenate([np.asarray(prompt), np.asarray(fed_ids, dtype=np.asarray(prompt).dtype)])
    full = model.forward_sequence(seq, 0, None, all_positions=True)
    return full[len(prompt) - 1:]
