"""Pins of the oracle's q8_0 dequantisation ("ember internals", section "GGUF format and
quantization", subsection "q8_0 block quantization"): the f16 scale decode against
numpy's float16 over every bit pattern, hand-built blocks with values worked out by hand
(byte order, sign of the int8 values, subnormal and large scales, block order along the
row), and the seeded quantiser's round trip."""
import numpy as np

import oracle as O
import workloads as W


def test_f16_decode_matches_numpy_float16_for_every_pattern():
    bits = np.arange(65536, dtype=np.uint16)
    got = O.f16_to_f32(bits)
    ref = bits.view(np.float16).astype(np.float32)
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan].view(np.uint32), ref[~nan].view(np.uint32))   # signed zeros too


def _block(d_lo, d_hi, q):
    q = np.asarray(q + [0] * (32 - len(q)), np.int8)
    return np.concatenate([np.array([d_lo, d_hi], np.uint8), q.view(np.uint8)])


def test_hand_built_blocks():
    # d = 0x3C00 = 1.0 (stored little-endian: 0x00, 0x3C); q as signed bytes
    row = _block(0x00, 0x3C, [1, -1, 127, -128, 0, 2])
    v = O.dequant_q8_0(row[None], 32)[0]
    assert v[:6].tolist() == [1.0, -1.0, 127.0, -128.0, 0.0, 2.0] and not v[6:].any()
    # d = 0x3800 = 0.5; 0xB800 = -0.5 flips every sign
    assert O.dequant_q8_0(_block(0x00, 0x38, [3, -5])[None], 32)[0][:2].tolist() == [1.5, -2.5]
    assert O.dequant_q8_0(_block(0x00, 0xB8, [3, -5])[None], 32)[0][:2].tolist() == [-1.5, 2.5]
    # byte order: (0x3C, 0x00) is 0x003C = 60 * 2^-24 (a subnormal), not 1.0
    assert O.dequant_q8_0(_block(0x3C, 0x00, [1])[None], 32)[0][0] == np.float32(60 * 2.0 ** -24)
    # the largest finite scale, 0x7BFF = 65504, times -128
    assert O.dequant_q8_0(_block(0xFF, 0x7B, [-128])[None], 32)[0][0] == np.float32(-8384512.0)


def test_blocks_run_along_the_row():
    # two rows of two blocks: row r, block b has scale 2^(r + b) and q_j = j - 16
    rows = []
    for r in range(2):
        blocks = []
        for b in range(2):
            e = 15 + r + b                                # f16 exponent field for 2^(r+b)
            bits = e << 10
            blocks.append(_block(bits & 0xFF, bits >> 8, [j - 16 for j in range(32)]))
        rows.append(np.concatenate(blocks))
    v = O.dequant_q8_0(np.stack(rows), 64)
    for r in range(2):
        for b in range(2):
            for j in range(32):
                assert v[r, 32 * b + j] == (j - 16) * 2.0 ** (r + b)


def test_quantiser_round_trip_is_within_half_a_step():
    a = np.random.default_rng(1).standard_normal((5, 96)).astype(np.float32) * 0.02
    a[2, 32:64] = 0.0                                     # an all-zero block: d = 0, q = 0
    raw = W.quantize_q8_0(a)
    assert raw.shape == (5, 3 * 34)
    v = O.dequant_q8_0(raw, 96)
    d = O.f16_to_f32((raw.reshape(5, 3, 34)[..., 0].astype(np.uint16)
                      | (raw.reshape(5, 3, 34)[..., 1].astype(np.uint16) << 8)))
    step = np.repeat(d, 32, axis=1)
    assert np.all(np.abs(v - a) <= step * 0.5 + 1e-12)
    assert not v[2, 32:64].any()
    # a block's largest magnitude maps to +-127 (d = f16(amax / 127) is within 2^-11 of it)
    q = raw.reshape(5, 3, 34)[..., 2:].view(np.int8)
    assert np.all(np.abs(q[:, [0, 2]]).max(-1) >= 126)


def test_q8_model_checkpoint_decodes_to_its_dequantised_weights():
    m = W.configs.shrink_model(W.get("qwen05b-q8").model, vocab=64, hidden=64, layers=1,
                               heads=2, kv_heads=1, head_dim=32, ffn=64)
    ck = W.make_weights(m, 3)
    tags = {n: t for n, (t, _) in ck.items()}
    assert tags["model.embed_tokens.weight"] == "q8_0"
    assert tags["model.layers.0.mlp.down_proj.weight"] == "q8_0"
    assert tags["model.layers.0.input_layernorm.weight"] == "f32"
    assert tags["model.layers.0.self_attn.q_proj.bias"] == "f32"
    om = O.OracleModel(m, ck)
    assert om.w["model.layers.0.mlp.down_proj.weight"].shape == (64, 64)
