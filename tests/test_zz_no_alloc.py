"""The no-allocation draw (ember_sample_noalloc: the sampler's per-row scratch in a fixed
device array of the library) against ember_sample (the same kernels with their scratch in
the model's workspace), through the C ABI: identical token ids (integer results, compared
exactly) on two calls in a row, the second with fewer rows, another row stride and another
draw row, at three sampler settings (plain draw, top-k + top-p, greedy)."""
import numpy as np
import pytest

import workloads as W
from tests.gpu_util import say
from tests.small_models import LLAMA_SMALL

pytestmark = pytest.mark.gpu

WIDE_VOCAB = W.shrink_model(LLAMA_SMALL, name="llama-vocab152k", vocab=151936)


@pytest.mark.parametrize("setting", [(1.0, 0, 1.0), (0.8, 50, 0.9), (0.0, 0, 1.0)],
                         ids=["plain", "topk50-topp0.9", "greedy"])
def test_no_alloc_draw_equals_workspace_draw(setting):
    import torch
    from gqa_decoder_transformer_amd import binding as B
    m = WIDE_VOCAB
    R = B.NOALLOC_MAX_ROWS
    cfg = B.make_config(m, precision=B.EXACT, max_batch=R, max_seq=8, max_tokens=R)
    eng = B.Engine(cfg, W.make_weights(m, 81), poison=True)
    U = torch.from_numpy(W.make_uniforms(82, 8, R)).to(eng.device)
    t, k, p = setting
    if t > 0:
        eng.set_sampler(t, k, p, U)
    dev = eng.device
    # call 1: all R rows, unit stride; call 2: 5 rows, padded stride, another draw row
    lg1 = torch.from_numpy(W.make_logits(83, R, m.vocab, ties=True)).to(dev)
    lg2 = torch.from_numpy(W.make_logits(84, 5, m.vocab + 64)).to(dev)[:, :m.vocab]
    for call, (lg, pos) in enumerate(((lg1, 3), (lg2, 6))):
        rows = lg.shape[0]
        a = torch.full((rows,), -1, dtype=torch.int32, device=dev)
        b = torch.full((rows,), -2, dtype=torch.int32, device=dev)
        B.ember_sample(eng.model, lg.data_ptr(), rows, lg.stride(0), pos, a.data_ptr(), eng.sp)
        B.ember_sample_noalloc(eng.model, lg.data_ptr(), rows, lg.stride(0), pos, b.data_ptr(),
                               eng.sp)
        eng.sync()
        a, b = a.cpu().numpy(), b.cpu().numpy()
        say(f"no-alloc draw {setting} call {call}: {rows} rows, ids {b[:4].tolist()}...")
        assert ((a >= 0) & (a < m.vocab)).all()
        assert np.array_equal(a, b), (a, b)
    big = torch.zeros((R + 1, m.vocab), dtype=torch.float32, device=dev)
    out = torch.zeros(R + 1, dtype=torch.int32, device=dev)
    with pytest.raises(B.EmberError) as e:
        B.ember_sample_noalloc(eng.model, big.data_ptr(), R + 1, m.vocab, 0, out.data_ptr(), eng.sp)
    assert e.value.status == 7                     # beyond the array's rows: nothing enqueued
    eng.sync()
    eng.close()
