"""Pins of the oracle's primitives against closed forms, invariants and library routines.

Each test is chosen so that a plausible mistake (a dropped term, a wrong sign or index,
a transposed operand, the other RoPE pairing, the other tie rule) fails it.
"""
import math

import numpy as np
import pytest
import scipy.special
import torch

import oracle as O
from oracle import brute


# ----------------------------------------------------------------------------- widening

def test_widen_bf16_every_bit_pattern_matches_torch_and_field_decode():
    bits = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    ours = O.widen_bf16(bits)
    lib = torch.from_numpy(bits.view(np.int16).copy()).view(torch.bfloat16).float().numpy()
    nan = np.isnan(lib)
    assert np.array_equal(np.isnan(ours), nan)
    assert np.array_equal(ours[~nan].view(np.uint32), lib[~nan].view(np.uint32))
    # an independent decode of the sign / exponent / mantissa fields (incl. subnormals)
    fields = np.array(brute._widen("bf16", bits), dtype=np.float64)
    assert np.array_equal(np.isnan(fields), nan)
    assert np.array_equal(ours[~nan].astype(np.float64), fields[~nan])


def test_decode_tensor_passes_f32_and_rejects_other_dtypes():
    a = np.random.default_rng(0).standard_normal(17).astype(np.float32)
    assert np.array_equal(O.decode_tensor("f32", a).view(np.uint32), a.view(np.uint32))
    for tag in ("f16", "i8", "q4_0"):
        with pytest.raises(ValueError):
            O.decode_tensor(tag, a)


# ----------------------------------------------------------------------------- RMSNorm

@pytest.mark.parametrize("c", [0.02, -3.0, 1e-3])
def test_rmsnorm_constant_vector_closed_form(c):
    n, eps = 96, 1e-5
    w = np.linspace(0.5, 1.5, n)
    y = O.rmsnorm(np.full(n, c, np.float64), w, eps)
    assert np.allclose(y, c / math.sqrt(c * c + eps) * w, rtol=1e-14, atol=0)


def test_rmsnorm_unit_mean_square_and_matches_torch():
    rng = np.random.default_rng(1)
    x = rng.standard_normal((5, 64)) * 0.3
    y = O.rmsnorm(x, np.ones(64), 0.0)
    assert np.allclose((y * y).mean(-1), 1.0, rtol=1e-13)
    w = rng.standard_normal(64)
    lib = torch.nn.functional.rms_norm(torch.from_numpy(x), (64,), torch.from_numpy(w), eps=1e-6)
    assert np.allclose(O.rmsnorm(x, w, 1e-6), lib.numpy(), rtol=1e-12, atol=1e-14)


# ----------------------------------------------------------------------------- RoPE

LLAMA3 = (32.0, 1.0, 4.0, 8192.0)


@pytest.mark.parametrize("hd,theta,l3", [(8, 1e4, None), (64, 1e6, None), (64, 5e5, LLAMA3),
                                         (128, 1e6, None)])
def test_rope_preserves_norms_at_every_position(hd, theta, l3):
    n = 8320
    cos, sin = O.rope_tables(n, hd, theta, l3, dtype=np.float64)
    x = np.random.default_rng(2).standard_normal((n, hd))
    y = O.apply_rope(x, cos, sin)
    h = hd // 2
    pair_in = x[:, :h] ** 2 + x[:, h:] ** 2
    pair_out = y[:, :h] ** 2 + y[:, h:] ** 2
    assert np.allclose(pair_in, pair_out, rtol=1e-12)


def test_rope_position_zero_is_identity():
    cos, sin = O.rope_tables(1, 64, 5e5, LLAMA3)
    x = np.random.default_rng(3).standard_normal(64).astype(np.float32)
    assert np.array_equal(O.apply_rope(x, cos[0], sin[0]), x)


def test_rope_pairs_i_with_i_plus_half_not_adjacent():
    hd, pos = 16, 7
    cos, sin = O.rope_tables(pos + 1, hd, 1e4, dtype=np.float64)
    e1 = np.zeros(hd)
    e1[1] = 1.0
    y = O.apply_rope(e1, cos[pos], sin[pos])
    f1 = 1e4 ** (-2.0 / hd)
    expect = np.zeros(hd)
    expect[1] = math.cos(pos * f1)
    expect[1 + hd // 2] = math.sin(pos * f1)   # the interleaved convention would fill [0]
    assert np.allclose(y, expect, atol=1e-15)


def test_rope_equals_complex_multiplication():
    hd, n, theta = 64, 300, 1e6
    rng = np.random.default_rng(4)
    x = rng.standard_normal((n, hd))
    cos, sin = O.rope_tables(n, hd, theta, dtype=np.float64)
    y = O.apply_rope(x, cos, sin)
    h = hd // 2
    freqs = theta ** (-np.arange(0, hd, 2) / hd)
    z = (x[:, :h] + 1j * x[:, h:]) * np.exp(1j * np.arange(n)[:, None] * freqs[None, :])
    assert np.allclose(y[:, :h], z.real, atol=1e-12) and np.allclose(y[:, h:], z.imag, atol=1e-12)


def test_rope_relative_position_property():
    hd = 64
    cos, sin = O.rope_tables(2000, hd, 5e5, LLAMA3, dtype=np.float64)
    rng = np.random.default_rng(5)
    q, k = rng.standard_normal(hd), rng.standard_normal(hd)
    for m, n in [(10, 3), (1999, 1000), (512, 512)]:
        lhs = O.apply_rope(q, cos[m], sin[m]) @ O.apply_rope(k, cos[n], sin[n])
        rhs = O.apply_rope(q, cos[m - n], sin[m - n]) @ k
        assert abs(lhs - rhs) < 1e-10


def test_llama3_scaling_piecewise_at_llama_1b_constants():
    base = O.rope_inv_freq(64, 5e5, None)
    scaled = O.rope_inv_freq(64, 5e5, LLAMA3)
    ratio = scaled / base
    # wavelength 2*pi/freq below orig/high = 2048 -> unscaled; above orig/low = 8192 -> /32
    assert np.allclose(ratio[:15], 1.0, rtol=0, atol=1e-15)
    assert np.allclose(ratio[18:], 1 / 32, rtol=1e-15)
    z = (ratio[15:18] - 1 / 32) / (1 - 1 / 32)       # blend weight of the middle band
    assert np.allclose(z, [0.593, 0.281, 0.075], atol=1e-3)
    # the wavelength form written independently in the brute-force module agrees
    assert np.allclose(scaled, brute._freqs(64, 5e5, LLAMA3), rtol=1e-14, atol=0)
    # factor 1 means no scaling at all
    assert np.allclose(O.rope_inv_freq(64, 5e5, (1.0, 1.0, 4.0, 8192.0)), base, rtol=1e-15)


def test_rope_tables_are_f64_angles_rounded_once():
    cos, sin = O.rope_tables(5000, 64, 5e5, LLAMA3, dtype=np.float32)
    c64, s64 = O.rope_tables(5000, 64, 5e5, LLAMA3, dtype=np.float64)
    assert cos.dtype == np.float32
    assert np.array_equal(cos, c64.astype(np.float32)) and np.array_equal(sin, s64.astype(np.float32))
    # angles in f32 (the other pages' choice) differ at large positions: the tables must not
    ang32 = np.arange(5000, dtype=np.float32)[:, None] * O.rope_inv_freq(64, 5e5, LLAMA3).astype(np.float32)
    assert not np.array_equal(cos, np.cos(ang32))


# ----------------------------------------------------------------------------- softmax

def test_softmax_matches_scipy_sums_to_one_and_is_shift_invariant():
    rng = np.random.default_rng(6)
    s = rng.standard_normal((7, 300)) * 5
    p = O.softmax(s)
    assert np.allclose(p, scipy.special.softmax(s, axis=-1), rtol=1e-13, atol=1e-300)
    assert np.allclose(p.sum(-1), 1.0, rtol=1e-14)
    assert np.allclose(O.softmax(s + 1234.5), p, rtol=1e-9)
    s32 = s.astype(np.float32)
    assert np.allclose(O.softmax(s32).sum(-1), 1.0, atol=300 * 2 ** -24)


def test_softmax_masked_entries_and_fully_masked_row():
    s = np.array([[1.0, -np.inf, 2.0, -np.inf], [-np.inf] * 4])
    p = O.softmax(s)
    assert p[0, 1] == 0 and p[0, 3] == 0
    assert np.allclose(p[0, [0, 2]], scipy.special.softmax([1.0, 2.0]))
    assert np.array_equal(p[1], np.full(4, 0.25))
    assert not np.isnan(p).any()


# ----------------------------------------------------------------------------- attention

def _qkv(T, S, NH, NKV, HD, seed):
    rng = np.random.default_rng(seed)
    return rng.standard_normal((T, NH, HD)), rng.standard_normal((S, NKV, HD)), rng.standard_normal((S, NKV, HD))


@pytest.mark.parametrize("causal", [True, False])
@pytest.mark.parametrize("NH,NKV,HD", [(4, 2, 8), (14, 2, 64), (16, 8, 128), (6, 6, 16)])
def test_attention_matches_torch_sdpa_with_gqa(causal, NH, NKV, HD):
    T = 37
    q, k, v = _qkv(T, T, NH, NKV, HD, 7)
    pos = np.arange(T)
    ours = O.attention(q, k, v, pos, pos, causal, q_block=16)
    tq = torch.from_numpy(q).permute(1, 0, 2)[None]
    tk = torch.from_numpy(k).permute(1, 0, 2)[None]
    tv = torch.from_numpy(v).permute(1, 0, 2)[None]
    lib = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, is_causal=causal,
                                                           enable_gqa=True)
    assert np.allclose(ours, lib[0].permute(1, 0, 2).numpy(), rtol=1e-11, atol=1e-12)


def test_attention_with_cached_prefix_matches_sdpa_with_explicit_mask():
    # 5 new queries at positions 20..24 over 25 cached keys (prefix + themselves)
    NH, NKV, HD, S = 8, 2, 16, 25
    q, k, v = _qkv(5, S, NH, NKV, HD, 8)
    qpos, kpos = np.arange(20, 25), np.arange(S)
    ours = O.attention(q, k, v, qpos, kpos, True)
    allowed = torch.from_numpy(kpos[None, :] <= qpos[:, None])
    lib = torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(q).permute(1, 0, 2)[None], torch.from_numpy(k).permute(1, 0, 2)[None],
        torch.from_numpy(v).permute(1, 0, 2)[None], attn_mask=allowed, enable_gqa=True)
    assert np.allclose(ours, lib[0].permute(1, 0, 2).numpy(), rtol=1e-11, atol=1e-12)


def test_gqa_equals_mha_with_repeat_interleaved_kv():
    NH, NKV, HD, T = 12, 3, 16, 20
    q, k, v = _qkv(T, T, NH, NKV, HD, 9)
    pos = np.arange(T)
    g = O.attention(q, k, v, pos, pos, True)
    m = O.attention(q, np.repeat(k, NH // NKV, axis=1), np.repeat(v, NH // NKV, axis=1), pos, pos, True)
    assert np.allclose(g, m, rtol=1e-14, atol=1e-15)


def test_attention_single_key_and_zero_query():
    q, k, v = _qkv(1, 1, 4, 2, 8, 10)
    out = O.attention(q, k, v, np.array([0]), np.array([0]), True)
    assert np.allclose(out[0], np.repeat(v, 2, axis=1)[0], rtol=1e-15)
    T = 9
    q, k, v = _qkv(T, T, 4, 2, 8, 11)
    out = O.attention(np.zeros_like(q), k, v, np.arange(T), np.arange(T), True)
    for t in range(T):   # q = 0: uniform weights over the admissible keys 0..t
        assert np.allclose(out[t], np.repeat(v[:t + 1].mean(0), 2, axis=0), rtol=1e-13)


def test_attention_brute_force_loops_tiny():
    NH, NKV, HD, T = 4, 2, 8, 6
    q, k, v = _qkv(T, T, NH, NKV, HD, 12)
    ours = O.attention(q, k, v, np.arange(T), np.arange(T), True)
    for t in range(T):
        for h in range(NH):
            kh = h // (NH // NKV)
            sc = [sum(q[t, h, e] * k[j, kh, e] for e in range(HD)) / math.sqrt(HD) for j in range(t + 1)]
            mx = max(sc)
            ex = [math.exp(s - mx) for s in sc]
            y = [sum(ex[j] / sum(ex) * v[j, kh, e] for j in range(t + 1)) for e in range(HD)]
            assert np.allclose(ours[t, h], y, rtol=1e-12, atol=1e-14)


def test_attention_fully_masked_row_gives_uniform_weights_and_no_nan():
    T = 5
    q, k, v = _qkv(T, T, 2, 1, 8, 13)
    mask = np.ones((T, T), bool)
    mask[2, :] = False
    out = O.attention(q, k, v, np.arange(T), np.arange(T), False, mask=mask)
    assert not np.isnan(out).any()
    assert np.allclose(out[2, 0], v[:, 0].mean(0))


def test_attention_query_blocking_does_not_change_results():
    q, k, v = _qkv(70, 70, 4, 2, 16, 14)
    pos = np.arange(70)
    for causal in (True, False):
        a = O.attention(q, k, v, pos, pos, causal, q_block=512)
        b = O.attention(q, k, v, pos, pos, causal, q_block=7)
        assert np.allclose(a, b, rtol=1e-14, atol=1e-15)


# ----------------------------------------------------------------------------- MLP, argmax

def test_silu_and_swiglu():
    z = np.linspace(-30, 30, 1001)
    assert np.allclose(O.silu(z), torch.nn.functional.silu(torch.from_numpy(z)).numpy(), rtol=1e-14)
    assert O.silu(np.array([0.0]))[0] == 0.0
    u = np.linspace(-1, 1, 1001)
    assert np.allclose(O.swiglu(z, u), z * scipy.special.expit(z) * u, rtol=1e-13)


def test_greedy_argmax_lowest_index_on_ties_zero_signs_and_inf():
    assert O.greedy_argmax(np.array([1.0, 3.0, 3.0, 2.0])) == 1
    assert O.greedy_argmax(np.array([-0.0, 0.0, -1.0])) == 0
    assert O.greedy_argmax(np.array([0.0, -0.0, -1.0])) == 0
    assert O.greedy_argmax(np.array([-np.inf, -np.inf, -5.0])) == 2
    assert O.greedy_argmax(np.array([np.inf, 1.0, np.inf])) == 0
    with pytest.raises(FloatingPointError):
        O.greedy_argmax(np.array([1.0, np.nan]))
    rng = np.random.default_rng(15)
    for _ in range(50):
        row = rng.integers(0, 4, 40).astype(np.float32)
        assert O.greedy_argmax(row) == brute.argmax_first(row.tolist())
