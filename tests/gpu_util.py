"""Helpers of the GPU parity tests: run the HIP path through the C ABI and compare it
with the oracle under the tolerance tiers (EXACT: f32 logits within 1e-4 relative
max-abs; FAST: bf16 logits within 2e-2) and the near-tie rule for greedy ids."""
import sys

import numpy as np

TOL_EXACT = 1e-4
TOL_FAST = 2e-2


def say(msg):
    print(f"[gpu-step] {msg}", flush=True)
    sys.stdout.flush()


def rel_maxabs(g, o):
    """Per row: max_i |g_i - o_i| / max_i |o_i| (rows along the last axis)."""
    g = np.asarray(g, np.float64)
    o = np.asarray(o, np.float64)
    return np.abs(g - o).max(-1) / np.abs(o).max(-1)


def check_greedy(gpu_ids, or_ids, or_logits, tol):
    """Free-running greedy ids must equal the oracle's. A divergence is accepted only at
    a step where the GPU's token is within 2*eps of the oracle's maximum logit
    (eps = tol * max|logit|): several tokens are then legitimate greedy choices. Returns
    the step of such a divergence (later steps are not comparable) or None."""
    for k in range(len(or_ids)):
        if int(gpu_ids[k]) != int(or_ids[k]):
            lg = or_logits[k]
            eps = tol * np.abs(lg).max()
            gap = lg.max() - lg[int(gpu_ids[k])]
            assert gap <= 2 * eps, (f"step {k}: GPU chose {gpu_ids[k]}, oracle {or_ids[k]}, "
                                    f"gap {gap:.3g} > 2 eps {2 * eps:.3g}")
            say(f"near-tie divergence at step {k} (gap {gap:.3g} <= 2 eps {2 * eps:.3g})")
            return k
    return None


def gpu_decode(eng, first, start, n_steps, feed=None, logits_dtype=0, rows=None):
    """``n_steps`` decode steps at positions ``start..`` after a prefill whose next ids are
    the device tensor ``first`` [B]. With ``feed`` ([n_steps, B] ids) the steps are
    teacher-forced, otherwise each consumes the previous argmax. Returns (ids [n_steps, B],
    logits [n_steps, R, V]) for the batch rows ``rows`` (all when None); ids[k] is the
    argmax written by step k."""
    import torch
    B = first.shape[0]
    sel = None if rows is None else torch.as_tensor(list(rows), device=eng.device)
    ids, logs = [], []
    prev = first
    for k in range(n_steps):
        if feed is not None:
            cur = torch.from_numpy(np.ascontiguousarray(feed[k], dtype=np.int32)).to(eng.device)
        else:
            cur = prev.clone()
        out = torch.empty_like(cur)
        eng.decode_step(cur, start + k, out)
        ids.append(out)
        lg = eng.logits(B, logits_dtype)
        logs.append((lg if sel is None else lg.index_select(0, sel)).float().cpu())
        prev = out
    eng.sync()
    return torch.stack(ids).cpu().numpy(), torch.stack(logs).numpy()


def check_teacher_forced_ids(gpu_ids, or_logits, tol):
    """Teacher-forced steps (the GPU fed the oracle's ids): the GPU's argmax must equal the
    oracle's wherever the oracle's top-2 gap exceeds 2*eps (eps = tol * max|logit|); at a
    closer pair either is a legitimate greedy choice, but only a token within 2*eps of the
    maximum. Returns the number of near-tie steps where they differ."""
    near = 0
    for k in range(len(gpu_ids)):
        lg = np.asarray(or_logits[k], np.float64)
        eps = tol * np.abs(lg).max()
        g = int(gpu_ids[k])
        gap = lg.max() - lg[g]
        assert gap <= 2 * eps, f"step {k}: GPU id {g} is {gap:.3g} below the oracle's maximum (2 eps {2 * eps:.3g})"
        near += int(g != int(np.argmax(lg)))
    return near


def gpu_generate(eng, prompt, n_steps, feed=None, logits_dtype=0):
    """Prefill ``prompt [B, T]`` then ``n_steps`` decode steps on the GPU. With ``feed``
    ([n_steps, B] ids) the steps are teacher-forced; otherwise each step consumes the
    previous step's argmax. Returns (ids [n_steps + 1, B], logits [n_steps + 1, B, V])
    where ids[k] is the argmax the GPU wrote after step k (k = 0: the prefill)."""
    import torch
    B, T = prompt.shape
    nxt, _ = eng.prefill(prompt)
    ids = [nxt.clone()]
    logs = [eng.logits(B, logits_dtype)]
    for k in range(n_steps):
        if feed is not None:
            cur = torch.from_numpy(np.ascontiguousarray(feed[k], dtype=np.int32)).to(eng.device)
        else:
            cur = ids[-1].clone()
        out = torch.empty_like(cur)
        eng.decode_step(cur, T + k, out)
        ids.append(out)
        logs.append(eng.logits(B, logits_dtype))
    eng.sync()
    ids = torch.stack(ids).cpu().numpy()
    logs = torch.stack(logs).float().cpu().numpy()
    return ids, logs
