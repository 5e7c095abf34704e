"""Thin ctypes binding of ``libember.so`` (include/ember.h).

Argument marshalling only: every step of the forward pass runs in the HIP library.
PyTorch supplies device memory (workspace, KV cache, outputs) and the HIP stream.
Importing this module fails loudly when the library has not been built.
"""
from __future__ import annotations

import ctypes
import os
from typing import Dict, Iterable, Optional, Tuple

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libember.so")

EMBER_OK = 0
STATUS_NAMES = {0: "OK", 1: "E_ARG", 2: "E_CONFIG", 3: "E_TENSOR_MISSING", 4: "E_TENSOR_SHAPE",
                5: "E_DTYPE", 6: "E_TOKEN", 7: "E_CAPACITY", 8: "E_STATE", 9: "E_DEVICE",
                10: "E_NONFINITE"}
F32, BF16, Q8_0 = 0, 1, 2
EXACT, FAST = 0, 1
HEAD_TIED_LM, HEAD_CLS = 0, 1

EXPORTED = ["ember_workspace_bytes", "ember_kv_cache_bytes", "ember_load_weights",
            "ember_cache_bind", "ember_prefill", "ember_decode_step", "ember_logits",
            "ember_sync", "ember_cache_free", "ember_free", "ember_last_error",
            "ember_rope_table", "ember_time_kernel", "ember_set_sampler", "ember_sample",
            "ember_forward_with_activations", "ember_sensitivity", "ember_prefill_rows",
            "ember_decode_step_rows", "ember_measure_peak", "ember_sample_noalloc"]
K_LM_HEAD, K_QKV, K_ATTN, K_O, K_GATE_UP, K_DOWN, K_LAYER, K_SAMPLE = range(8)


class EmberConfig(ctypes.Structure):
    _fields_ = [("rope_theta", ctypes.c_double),
                ("llama3_factor", ctypes.c_double),
                ("llama3_low_freq_factor", ctypes.c_double),
                ("llama3_high_freq_factor", ctypes.c_double),
                ("llama3_original_max_pos", ctypes.c_double),
                ("rms_eps", ctypes.c_float),
                ("vocab", ctypes.c_int32), ("hidden", ctypes.c_int32), ("layers", ctypes.c_int32),
                ("heads", ctypes.c_int32), ("kv_heads", ctypes.c_int32),
                ("head_dim", ctypes.c_int32), ("ffn", ctypes.c_int32),
                ("rope_llama3", ctypes.c_int32), ("qkv_bias", ctypes.c_int32),
                ("qk_norm", ctypes.c_int32), ("causal", ctypes.c_int32),
                ("head_kind", ctypes.c_int32), ("n_classes", ctypes.c_int32),
                ("weight_dtype", ctypes.c_int32), ("kv_dtype", ctypes.c_int32),
                ("precision", ctypes.c_int32), ("max_batch", ctypes.c_int32),
                ("max_seq", ctypes.c_int32), ("max_tokens", ctypes.c_int32),
                ("sens_head", ctypes.c_int32)]


class EmberTensor(ctypes.Structure):
    _fields_ = [("name", ctypes.c_char_p), ("data", ctypes.c_void_p),
                ("shape", ctypes.c_int64 * 4), ("ndim", ctypes.c_int32),
                ("dtype", ctypes.c_int32)]


class EmberSampler(ctypes.Structure):
    _fields_ = [("temperature", ctypes.c_float), ("top_k", ctypes.c_int32),
                ("top_p", ctypes.c_float), ("d_uniform", ctypes.c_void_p),
                ("n_pos", ctypes.c_int32), ("ld", ctypes.c_int32),
                ("seed", ctypes.c_uint64)]


class EmberError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"{STATUS_NAMES.get(status, status)}: {message}")
        self.status = status
        self.message = message


def _load():
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is missing: build it with __graft_entry__.build() "
                          "(hipcc --offload-arch=gfx950); there is no fallback path")
    # torch's bundled HIP runtime carries the same soname as the system one; loading torch
    # first makes the library bind to that runtime, so the process holds one HIP runtime
    # (a second, separately loaded runtime finds no device)
    import torch  # noqa: F401
    lib = ctypes.CDLL(LIB_PATH)
    P = ctypes.c_void_p
    cfgp = ctypes.POINTER(EmberConfig)
    sig = {
        "ember_workspace_bytes": (ctypes.c_size_t, [cfgp]),
        "ember_kv_cache_bytes": (ctypes.c_size_t, [cfgp]),
        "ember_load_weights": (ctypes.c_int, [cfgp, ctypes.POINTER(EmberTensor), ctypes.c_int32,
                                              P, ctypes.c_size_t, P, ctypes.POINTER(P)]),
        "ember_cache_bind": (ctypes.c_int, [P, P, ctypes.c_size_t, ctypes.POINTER(P)]),
        "ember_prefill": (ctypes.c_int, [P, P, P, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32,
                                         P, P, P]),
        "ember_decode_step": (ctypes.c_int, [P, P, P, ctypes.c_int32, ctypes.c_int32, P, P]),
        "ember_logits": (ctypes.c_int, [P, P, ctypes.c_int32, P]),
        "ember_sync": (ctypes.c_int, [P, P]),
        "ember_cache_free": (None, [P]),
        "ember_free": (None, [P]),
        "ember_last_error": (ctypes.c_char_p, []),
        "ember_rope_table": (ctypes.c_int, [cfgp, ctypes.c_int32, P, P]),
        "ember_time_kernel": (ctypes.c_int, [P, P, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32,
                                             P, ctypes.POINTER(ctypes.c_float)]),
        "ember_set_sampler": (ctypes.c_int, [P, ctypes.POINTER(EmberSampler)]),
        "ember_sample": (ctypes.c_int, [P, P, ctypes.c_int32, ctypes.c_int64, ctypes.c_int32, P, P]),
        "ember_forward_with_activations": (ctypes.c_int, [P, P, P, ctypes.c_int32, ctypes.c_int32,
                                                          ctypes.c_int32, P, P, P]),
        "ember_sensitivity": (ctypes.c_int, [P, P, P]),
        "ember_prefill_rows": (ctypes.c_int, [P, P, P, P, P, ctypes.c_int32, P, P]),
        "ember_decode_step_rows": (ctypes.c_int, [P, P, P, ctypes.c_int32, P, P, P]),
        "ember_measure_peak": (ctypes.c_int, [ctypes.c_int32, P, ctypes.c_size_t, ctypes.c_int32,
                                              P, ctypes.POINTER(ctypes.c_float)]),
        "ember_sample_noalloc": (ctypes.c_int, [P, P, ctypes.c_int32, ctypes.c_int64, ctypes.c_int32,
                                                P, P]),
    }
    for name, (res, args) in sig.items():
        f = getattr(lib, name)
        f.restype = res
        f.argtypes = args
    return lib


LIB = _load()


def _check(status: int):
    if status != EMBER_OK:
        raise EmberError(status, LIB.ember_last_error().decode())


# ------------------------------------------------------------------ same-name wrappers

def ember_workspace_bytes(cfg: EmberConfig) -> int:
    return LIB.ember_workspace_bytes(ctypes.byref(cfg))


def ember_kv_cache_bytes(cfg: EmberConfig) -> int:
    return LIB.ember_kv_cache_bytes(ctypes.byref(cfg))


def ember_load_weights(cfg: EmberConfig, tensors, d_workspace: int, workspace_bytes: int,
                       stream: int) -> int:
    arr = (EmberTensor * len(tensors))(*tensors)
    out = ctypes.c_void_p()
    _check(LIB.ember_load_weights(ctypes.byref(cfg), arr, len(tensors), d_workspace,
                                  workspace_bytes, stream, ctypes.byref(out)))
    return out.value


def ember_cache_bind(model: int, d_kv: int, kv_bytes: int) -> int:
    out = ctypes.c_void_p()
    _check(LIB.ember_cache_bind(model, d_kv, kv_bytes, ctypes.byref(out)))
    return out.value


def ember_prefill(model: int, cache: int, h_ids: np.ndarray, start_pos: int,
                  d_all_logits: int, d_next: int, stream: int):
    ids = np.ascontiguousarray(h_ids, dtype=np.int32)
    if ids.ndim != 2:
        raise ValueError("ids must be [batch, n_tokens]")
    _check(LIB.ember_prefill(model, cache, ids.ctypes.data, ids.shape[0], ids.shape[1],
                             start_pos, d_all_logits, d_next, stream))


def ember_forward_with_activations(model: int, cache: int, h_ids: np.ndarray, start_pos: int,
                                   d_acts: int, d_next: int, stream: int):
    ids = np.ascontiguousarray(h_ids, dtype=np.int32)
    if ids.ndim != 2:
        raise ValueError("ids must be [batch, n_tokens]")
    _check(LIB.ember_forward_with_activations(model, cache, ids.ctypes.data, ids.shape[0],
                                              ids.shape[1], start_pos, d_acts, d_next, stream))


def ember_prefill_rows(model: int, cache: int, rows, starts, d_next: int, stream: int):
    """rows: a list of 1-D int32 id arrays (one per batch row); starts: their positions."""
    ids = np.ascontiguousarray(np.concatenate([np.asarray(r, np.int32) for r in rows]), np.int32)
    lens = np.ascontiguousarray([len(r) for r in rows], np.int32)
    st = np.ascontiguousarray(starts, np.int32)
    if st.shape != lens.shape:
        raise ValueError("one start position per row")
    _check(LIB.ember_prefill_rows(model, cache, ids.ctypes.data, lens.ctypes.data, st.ctypes.data,
                                  len(rows), d_next, stream))


def ember_decode_step_rows(model: int, cache: int, d_ids: int, batch: int, positions,
                           d_next: int, stream: int):
    pos = np.ascontiguousarray(positions, np.int32)
    if pos.shape != (batch,):
        raise ValueError("one position per row")
    _check(LIB.ember_decode_step_rows(model, cache, d_ids, batch, pos.ctypes.data, d_next, stream))


def ember_sensitivity(model: int, d_out: int, stream: int):
    _check(LIB.ember_sensitivity(model, d_out, stream))


def ember_decode_step(model: int, cache: int, d_ids: int, batch: int, pos: int, d_next: int,
                      stream: int):
    _check(LIB.ember_decode_step(model, cache, d_ids, batch, pos, d_next, stream))


def ember_logits(model: int, d_out: int, dtype: int, stream: int):
    _check(LIB.ember_logits(model, d_out, dtype, stream))


def ember_sync(model: int, stream: int):
    _check(LIB.ember_sync(model, stream))


def ember_cache_free(cache: int):
    LIB.ember_cache_free(cache)


def ember_free(model: int):
    LIB.ember_free(model)


def ember_last_error() -> str:
    return LIB.ember_last_error().decode()


def ember_rope_table(cfg: EmberConfig, n_pos: int) -> Tuple[np.ndarray, np.ndarray]:
    half = cfg.head_dim // 2
    cos = np.zeros((n_pos, half), np.float32)
    sin = np.zeros((n_pos, half), np.float32)
    _check(LIB.ember_rope_table(ctypes.byref(cfg), n_pos, cos.ctypes.data, sin.ctypes.data))
    return cos, sin


def ember_time_kernel(model: int, cache: int, kernel: int, phase: int, iters: int,
                      stream: int) -> float:
    out = ctypes.c_float()
    _check(LIB.ember_time_kernel(model, cache, kernel, phase, iters, stream, ctypes.byref(out)))
    return out.value


def ember_set_sampler(model: int, sampler: Optional[EmberSampler]):
    _check(LIB.ember_set_sampler(model, ctypes.byref(sampler) if sampler is not None else None))


def ember_sample(model: int, d_logits: int, rows: int, ld_logits: int, pos: int, d_next: int,
                 stream: int):
    _check(LIB.ember_sample(model, d_logits, rows, ld_logits, pos, d_next, stream))


PEAK_COPY, PEAK_MFMA, PEAK_READ = 0, 1, 2


def ember_measure_peak(kind: int, d_buf: int, nbytes: int, iters: int, stream: int) -> float:
    out = ctypes.c_float()
    _check(LIB.ember_measure_peak(kind, d_buf, nbytes, iters, stream, ctypes.byref(out)))
    return out.value


NOALLOC_MAX_ROWS = 16


def ember_sample_noalloc(model: int, d_logits: int, rows: int, ld_logits: int, pos: int,
                         d_next: int, stream: int):
    _check(LIB.ember_sample_noalloc(model, d_logits, rows, ld_logits, pos, d_next, stream))


# ------------------------------------------------------------------ marshalling helpers

def make_config(model, *, precision: int = EXACT, kv_dtype: Optional[int] = None,
                max_batch: int = 1, max_seq: int = 256, max_tokens: Optional[int] = None
                ) -> EmberConfig:
    """An ``EmberConfig`` from a model description with the attribute names of
    ``workloads.ModelConfig`` (vocab, hidden, layers, heads, kv_heads, head_dim, ffn,
    rms_eps, rope_theta, llama3, qkv_bias, qk_norm, causal, head, n_classes,
    weight_dtype)."""
    c = EmberConfig()
    c.vocab, c.hidden, c.layers = model.vocab, model.hidden, model.layers
    c.heads, c.kv_heads, c.head_dim, c.ffn = model.heads, model.kv_heads, model.head_dim, model.ffn
    c.rms_eps = model.rms_eps
    c.rope_theta = model.rope_theta
    if model.llama3 is not None:
        c.rope_llama3 = 1
        (c.llama3_factor, c.llama3_low_freq_factor, c.llama3_high_freq_factor,
         c.llama3_original_max_pos) = model.llama3
    c.qkv_bias, c.qk_norm, c.causal = int(model.qkv_bias), int(model.qk_norm), int(model.causal)
    c.head_kind = HEAD_CLS if model.head == "cls" else HEAD_TIED_LM
    c.n_classes = model.n_classes
    c.weight_dtype = {"bf16": BF16, "f32": F32, "q8_0": Q8_0}[model.weight_dtype]
    if kv_dtype is None:
        kv_dtype = F32 if precision == EXACT else BF16
    c.kv_dtype = kv_dtype
    c.precision = precision
    c.max_batch, c.max_seq = max_batch, max_seq
    c.max_tokens = max_tokens if max_tokens is not None else max(max_batch, 1)
    c.sens_head = int(getattr(model, "sens_head", False))
    return c


class Engine:
    """Owns (through torch) the workspace, KV cache and weight staging of one model and
    forwards calls to the C ABI."""

    def __init__(self, cfg: EmberConfig, checkpoint: Dict[str, Tuple[str, np.ndarray]],
                 device: str = "cuda", stream=None, poison: bool = False):
        """poison: fill the workspace and the KV cache with 0xFF bytes (NaN as f32 and
        bf16) before use, so that a read of memory the library has not written shows up
        as NaN in the results."""
        import torch
        self.torch = torch
        self.cfg = cfg
        self.device = torch.device(device)
        self.stream = stream if stream is not None else torch.cuda.current_stream(self.device)
        self.sp = self.stream.cuda_stream
        ws_bytes = ember_workspace_bytes(cfg)
        if ws_bytes == 0:
            # surface the validation message
            _check(LIB.ember_load_weights(ctypes.byref(cfg), None, 0, None, 0, None,
                                          ctypes.byref(ctypes.c_void_p())))
        self.workspace = torch.empty(ws_bytes, dtype=torch.uint8, device=self.device)
        if poison:
            self.workspace.fill_(255)
        staged = []
        tensors = []
        for name, (tag, arr) in checkpoint.items():
            if tag == "bf16":
                t = torch.from_numpy(np.ascontiguousarray(arr).view(np.int16)).to(self.device)
                dt = BF16
            elif tag == "f32":
                t = torch.from_numpy(np.ascontiguousarray(arr, dtype=np.float32)).to(self.device)
                dt = F32
            elif tag == "q8_0":
                # rows of 34-byte blocks; the tensor's shape is the logical [N, K]
                t = torch.from_numpy(np.ascontiguousarray(arr, dtype=np.uint8)).to(self.device)
                dt = Q8_0
            else:
                raise ValueError(f"unsupported dtype tag {tag}")
            staged.append(t)
            dims = list(arr.shape)
            if tag == "q8_0":
                dims = [arr.shape[0], arr.shape[1] // 34 * 32]
            shape = (ctypes.c_int64 * 4)(*(dims + [0] * (4 - arr.ndim)))
            tensors.append(EmberTensor(name.encode(), t.data_ptr(), shape, arr.ndim, dt))
        with torch.cuda.stream(self.stream):
            self.model = ember_load_weights(cfg, tensors, self.workspace.data_ptr(), ws_bytes, self.sp)
        del staged
        kv_bytes = ember_kv_cache_bytes(cfg)
        self.kv = torch.empty(kv_bytes, dtype=torch.uint8, device=self.device)
        if poison:
            self.kv.fill_(255)
        self.cache = ember_cache_bind(self.model, self.kv.data_ptr(), kv_bytes)
        self.out_dim = cfg.n_classes if cfg.head_kind == HEAD_CLS else cfg.vocab

    # -- calls ----------------------------------------------------------------------
    def prefill(self, ids: np.ndarray, start_pos: int = 0, all_logits: bool = False,
                next_ids=None):
        torch = self.torch
        ids = np.atleast_2d(np.asarray(ids, dtype=np.int32))
        B, T = ids.shape
        out = None
        if all_logits:
            out = torch.empty((B, T, self.out_dim), dtype=torch.float32, device=self.device)
        if next_ids is None:
            shape = (B, T) if self.cfg.head_kind == HEAD_CLS else (B,)
            next_ids = torch.empty(shape, dtype=torch.int32, device=self.device)
        ember_prefill(self.model, self.cache, ids, start_pos, out.data_ptr() if out is not None else 0,
                      next_ids.data_ptr(), self.sp)
        return next_ids, out

    def forward_with_activations(self, ids: np.ndarray, start_pos: int = 0, next_ids=None):
        """Prefill that also returns the hidden state after every block at each row's last
        position: (activations [B, layers, H] f32, next ids)."""
        torch = self.torch
        ids = np.atleast_2d(np.asarray(ids, dtype=np.int32))
        B = ids.shape[0]
        acts = torch.empty((B, self.cfg.layers, self.cfg.hidden), dtype=torch.float32,
                           device=self.device)
        if next_ids is None:
            shape = (B, ids.shape[1]) if self.cfg.head_kind == HEAD_CLS else (B,)
            next_ids = torch.empty(shape, dtype=torch.int32, device=self.device)
        ember_forward_with_activations(self.model, self.cache, ids, start_pos, acts.data_ptr(),
                                       next_ids.data_ptr(), self.sp)
        return acts, next_ids

    def prefill_rows(self, rows, starts=None, next_ids=None):
        """Ragged prefill: rows is a list of 1-D id arrays, starts their start positions."""
        torch = self.torch
        starts = [0] * len(rows) if starts is None else list(starts)
        if next_ids is None:
            n = sum(len(r) for r in rows) if self.cfg.head_kind == HEAD_CLS else len(rows)
            next_ids = torch.empty(n, dtype=torch.int32, device=self.device)
        ember_prefill_rows(self.model, self.cache, rows, starts, next_ids.data_ptr(), self.sp)
        return next_ids

    def decode_step_rows(self, d_ids, positions, d_next=None):
        if d_next is None:
            d_next = d_ids
        ember_decode_step_rows(self.model, self.cache, d_ids.data_ptr(), d_ids.numel(), positions,
                               d_next.data_ptr(), self.sp)
        return d_next

    def sensitivity(self, rows: int):
        """The mean-pooled sequence scores of the last prefill, [rows] f32."""
        out = self.torch.empty(rows, dtype=self.torch.float32, device=self.device)
        ember_sensitivity(self.model, out.data_ptr(), self.sp)
        return out

    def decode_step(self, d_ids, pos: int, d_next=None):
        if d_next is None:
            d_next = d_ids
        ember_decode_step(self.model, self.cache, d_ids.data_ptr(), d_ids.numel(), pos,
                          d_next.data_ptr(), self.sp)
        return d_next

    def logits(self, rows: int, dtype: int = F32):
        torch = self.torch
        tdt = torch.float32 if dtype == F32 else torch.bfloat16
        out = torch.empty((rows, self.out_dim), dtype=tdt, device=self.device)
        ember_logits(self.model, out.data_ptr(), dtype, self.sp)
        return out

    def sync(self):
        ember_sync(self.model, self.sp)

    def set_sampler(self, temperature: float = 0.0, top_k: int = 0, top_p: float = 1.0,
                    uniform=None, seed=None):
        """uniform: device f32 tensor [n_pos, ld] of draws in [0, 1), kept referenced here
        while the sampler is set; or seed (with uniform None): draws generated on the
        device (Philox4x32-10). temperature 0 returns to greedy argmax."""
        if temperature == 0.0 and uniform is None and seed is None:
            self._uniform = None
            ember_set_sampler(self.model, None)
            return
        if uniform is None:
            if seed is None:
                raise ValueError("draws need a uniform tensor or a seed")
            s = EmberSampler(temperature, top_k, top_p, None, 0, 0, int(seed))
            ember_set_sampler(self.model, s)
            self._uniform = None
            return
        if uniform.dim() != 2 or not uniform.is_contiguous():
            raise ValueError("uniform must be a contiguous [n_pos, ld] device tensor")
        if uniform.dtype != self.torch.float32:
            raise ValueError("uniform must be float32")
        s = EmberSampler(temperature, top_k, top_p, uniform.data_ptr(), uniform.shape[0],
                         uniform.shape[1], 0)
        ember_set_sampler(self.model, s)
        self._uniform = uniform

    def sample(self, d_logits, pos: int, d_next=None):
        """Next ids of the rows of device logits [rows, V] f32 with the current sampler."""
        if d_logits.dtype != self.torch.float32 or d_logits.dim() != 2 or d_logits.stride(1) != 1:
            raise ValueError("logits must be a [rows, V] float32 tensor with unit column stride")
        rows = d_logits.shape[0]
        if d_next is None:
            d_next = self.torch.empty(rows, dtype=self.torch.int32, device=self.device)
        ember_sample(self.model, d_logits.data_ptr(), rows, d_logits.stride(0), pos,
                     d_next.data_ptr(), self.sp)
        return d_next

    def time_kernel(self, kernel: int, phase: int, iters: int = 20) -> float:
        return ember_time_kernel(self.model, self.cache, kernel, phase, iters, self.sp)

    def close(self):
        if getattr(self, "cache", None):
            ember_cache_free(self.cache)
            self.cache = None
        if getattr(self, "model", None):
            ember_free(self.model)
            self.model = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass
