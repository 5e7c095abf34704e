"""The C-ABI library on the host: it loads, exports every symbol include/ember.h declares,
validates configs without touching a device, and builds the same RoPE tables as the
oracle (host-only entry points; no compute call needs a GPU here)."""
import ctypes
import os
import re

import numpy as np
import pytest

import oracle as O
from gqa_decoder_transformer_amd import binding as B
from workloads import WORKLOADS

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared():
    text = open(os.path.join(ROOT, "include", "ember.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(ember_[a-z_]+)\s*\(", text)))


def test_header_declares_the_binding_surface():
    assert _declared() == sorted(B.EXPORTED)


def test_library_exports_every_declared_symbol():
    lib = ctypes.CDLL(B.LIB_PATH)
    for name in _declared():
        assert hasattr(lib, name), name


def _cfg(name="qwen05b", **kw):
    w = WORKLOADS[name]
    return B.make_config(w.model, max_batch=w.batch, max_seq=w.max_pos,
                         max_tokens=w.batch * w.prompt_len, **kw)


@pytest.mark.parametrize("name", list(WORKLOADS))
def test_every_workload_config_validates_and_sizes(name):
    c = _cfg(name)
    ws = B.ember_workspace_bytes(c)
    assert ws > 0
    # the workspace holds at least the weights in their stored dtype
    m = WORKLOADS[name].model
    es = {"bf16": 2, "f32": 4, "q8_0": 34 / 32}[m.weight_dtype]
    params = m.vocab * m.hidden + m.layers * (m.hidden * (m.q_dim + 2 * m.kv_dim) +
                                             m.hidden * m.q_dim + 3 * m.hidden * m.ffn)
    assert ws >= params * es
    kv = B.ember_kv_cache_bytes(c)
    assert kv == 2 * m.layers * c.max_batch * m.kv_heads * c.max_seq * m.head_dim * 4


def test_q8_configs_need_the_lm_head_and_whole_blocks():
    c = _cfg("qwen05b-q8")
    assert B.ember_workspace_bytes(c) > 0
    c.head_kind, c.n_classes = B.HEAD_CLS, 2
    assert B.ember_workspace_bytes(c) == 0          # q8_0 with a classification head
    c = _cfg("qwen05b-q8")
    c.hidden = 880                                   # a multiple of 8 but not of 32
    assert B.ember_workspace_bytes(c) == 0


@pytest.mark.parametrize("field,value", [("heads", 0), ("kv_heads", 3), ("head_dim", 7),
                                         ("vocab", 0), ("ffn", 100), ("weight_dtype", 7),
                                         ("kv_dtype", 2), ("max_seq", 0)])
def test_invalid_configs_are_rejected(field, value):
    c = _cfg()
    setattr(c, field, value)
    assert B.ember_workspace_bytes(c) == 0
    assert B.ember_kv_cache_bytes(c) == 0


def test_exact_mode_rejects_bf16_kv():
    assert B.ember_workspace_bytes(_cfg(precision=B.EXACT, kv_dtype=B.BF16)) == 0
    assert B.ember_workspace_bytes(_cfg(precision=B.FAST, kv_dtype=B.BF16)) > 0


def test_load_weights_reports_config_errors_without_a_device():
    c = _cfg()
    c.heads = 5
    with pytest.raises(B.EmberError) as e:
        B.ember_load_weights(c, [], 1, 1 << 20, 0)
    assert e.value.status == 2 and "GQA" in e.value.message


@pytest.mark.parametrize("name", ["tiny", "qwen05b", "llama1b", "encoder"])
def test_host_rope_table_equals_oracle_table(name):
    m = WORKLOADS[name].model
    c = _cfg(name)
    n = 8320 if name == "llama1b" else c.max_seq
    cos, sin = B.ember_rope_table(c, n)
    oc, os_ = O.rope_tables(n, m.head_dim, m.rope_theta, m.llama3, dtype=np.float32)
    # f64 angles rounded once to f32 on both sides; libm vs NumPy may differ by one f64
    # ulp before rounding, which can flip an f32 rounding only at an exact tie
    assert np.abs(cos.view(np.int32) - oc.view(np.int32)).max() <= 1
    assert np.abs(sin.view(np.int32) - os_.view(np.int32)).max() <= 1
    assert (cos != oc).mean() < 1e-4 and (sin != os_).mean() < 1e-4


def test_one_hip_runtime_in_process():
    """The library must bind to the HIP runtime torch already holds (both carry the soname
    libamdhip64.so.7); two runtimes in one process leave the library without a device.
    Checked in a fresh interpreter that imports the binding before anything else."""
    import subprocess
    import sys
    code = ("from gqa_decoder_transformer_amd import binding\n"
            "import torch\n"
            "maps = open('/proc/self/maps').read().split('\\n')\n"
            "libs = sorted({l.split()[-1] for l in maps if 'libamdhip64' in l})\n"
            "print(len(libs)); print(libs)\n")
    out = subprocess.run([sys.executable, "-c", code], cwd=ROOT, capture_output=True, text=True,
                         timeout=300)
    assert out.returncode == 0, out.stderr
    assert out.stdout.split("\n")[0] == "1", out.stdout
