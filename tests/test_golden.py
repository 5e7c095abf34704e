"""Figures the "ember internals" page works out for KV-cache sizes (tests/golden/
kv_cache_sizes.txt, each case citing its section), against the oracle's cache and the
C-ABI library's sizing (host-only calls, no device)."""
import os

import numpy as np

import oracle as O
from gqa_decoder_transformer_amd import binding as B
from workloads import configs as C

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden", "kv_cache_sizes.txt")


def _cases():
    cases, cur = {}, None
    for line in open(GOLDEN):
        line = line.split("#", 1)[0].strip()
        if not line:
            continue
        key, val = line.split(None, 1)
        if key == "case":
            cur = cases.setdefault(val, {})
        else:
            cur[key] = int(val)
    return cases


def _model(g, kv_heads=None):
    kv = g["kv_heads"] if kv_heads is None else kv_heads
    return C.shrink_model(C.LLAMA1B, name="golden", layers=g["layers"], heads=g["heads"],
                          kv_heads=kv, head_dim=g["head_dim"], hidden=g["heads"] * g["head_dim"],
                          ffn=4 * g["heads"] * g["head_dim"])


def _library_bytes(model, max_seq):
    cfg = B.make_config(model, precision=B.EXACT, max_batch=1, max_seq=max_seq, max_tokens=64)
    return B.ember_kv_cache_bytes(cfg)


def _oracle_bytes(model, max_seq):
    cache = O.KVCache(model, max_seq)
    return sum(a.nbytes for a in cache.k) + sum(a.nbytes for a in cache.v), sum(a.nbytes for a in cache.k)


def test_gpt2_small_cache_at_2048_positions():
    g = _cases()["gpt2_small_2048"]
    m = _model(g)
    assert g["elem_bytes"] == np.dtype(np.float32).itemsize
    total, one_side = _oracle_bytes(m, g["max_seq"])
    assert total == g["kv_bytes"]
    assert one_side == g["one_side_mib"] * 2 ** 20
    assert _library_bytes(m, g["max_seq"]) == g["kv_bytes"]


def test_grouped_query_cache_saving():
    g = _cases()["llama32_1b_gqa"]
    S = 128
    gqa, mha = _model(g), _model(g, kv_heads=g["heads"])
    for grouped, full in ((_library_bytes(gqa, S), _library_bytes(mha, S)),
                          (_oracle_bytes(gqa, S)[0], _oracle_bytes(mha, S)[0])):
        assert grouped > 0
        assert 100 * (full - grouped) == g["saving_percent"] * full
