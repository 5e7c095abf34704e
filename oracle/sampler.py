"""Sampling after the LM head -- TEST INFRASTRUCTURE (see the package docstring).

The five stages of the "ember internals" page, section "sampler", in its order and in
f32 (the page's types): temperature scaling, top-k masking, top-p (nucleus) masking
against a temporary softmax, the final softmax with its uniform fallback for a fully
masked row, and an inverse-CDF categorical draw with its argmax fallback for rounding.
The uniform draw r in [0, 1) is an input (the caller's seeded generator supplies it).

Readings of what the page leaves open:
* temperature 0 is the greedy argmax of the decode loop (lowest index of the maximum,
  "ember scripts/reference_forward.py"); the page sends t = 0 straight to an argmax and
  the step must reduce to greedy decoding.
* top-k is off for k = 0 or k >= V (the page says so); ties with the k-th largest value
  survive (its mask is "strictly below the threshold").
* top-p is applied for 0 < p < 1 and off otherwise. ``nucleus_cutoff`` is named but not
  printed: the temporary probabilities are sorted in decreasing order, the shortest
  prefix whose running f32 sum exceeds p is taken, and its last probability is the
  cutoff (the smallest probability of the smallest set whose cumulative probability
  exceeds p); when no prefix exceeds p the cutoff is the smallest probability.
* sums over a row are sequential f32 sums in index order (the page's iterator sum and
  running cumulative sum).
* the draw's rounding fallback keeps the last of equal maxima (the page's max_by).
"""
import numpy as np

F32 = np.float32


def apply_temperature(logits: np.ndarray, temperature: float) -> np.ndarray:
    """Stage 1: logits / t for t > 0 (t = 0 is handled by ``sample`` as greedy)."""
    z = np.asarray(logits, F32).copy()
    if temperature > 0.0:
        z = (z / F32(temperature)).astype(F32)
    return z


def top_k_mask(logits: np.ndarray, k: int) -> np.ndarray:
    """Stage 2: every logit strictly below the k-th largest becomes -inf."""
    z = np.asarray(logits, F32).copy()
    V = z.shape[0]
    if k <= 0 or k >= V:
        return z
    threshold = np.sort(z)[::-1][k - 1]
    z[z < threshold] = -np.inf
    return z


def softmax(logits: np.ndarray) -> np.ndarray:
    """Stage 4 (and the temporary softmax of stage 3): max-subtracted exponentials over
    their sequential f32 sum; a row with no finite logit gives the uniform distribution."""
    z = np.asarray(logits, F32)
    V = z.shape[0]
    m = F32(-np.inf)
    for x in z:                                   # fold with max, as the page does
        m = max(m, x)
    if m == -np.inf:
        return np.full(V, F32(1.0) / F32(V), F32)
    e = np.exp((z - m).astype(F32)).astype(F32)
    s = np.cumsum(e, dtype=F32)[-1]               # sequential f32 sum
    return (e / s).astype(F32)


def nucleus_cutoff(probs: np.ndarray, p: float) -> np.float32:
    """The last probability of the shortest decreasing-order prefix whose running sum
    exceeds p (the smallest probability when none does)."""
    desc = np.sort(np.asarray(probs, F32))[::-1]
    cum = np.cumsum(desc, dtype=F32)
    over = np.nonzero(cum > F32(p))[0]
    return desc[over[0]] if over.size else desc[-1]


def top_p_mask(logits: np.ndarray, p: float) -> np.ndarray:
    """Stage 3: tokens whose temporary probability is below the nucleus cutoff -> -inf."""
    z = np.asarray(logits, F32).copy()
    if not (0.0 < p < 1.0):
        return z
    soft = softmax(z)
    cutoff = nucleus_cutoff(soft, p)
    z[soft < cutoff] = -np.inf
    return z


def categorical(dist: np.ndarray, r: float) -> int:
    """Stage 5: the first index whose running f32 sum exceeds r; the last of the maxima
    when rounding leaves the total at or below r."""
    d = np.asarray(dist, F32)
    cum = np.cumsum(d, dtype=F32)
    hit = np.nonzero(F32(r) < cum)[0]
    if hit.size:
        return int(hit[0])
    mx = d.max()
    return int(np.nonzero(d == mx)[0][-1])


def sample(logits: np.ndarray, temperature: float, top_k: int, top_p: float, r: float) -> int:
    """One token from one row of logits through the five stages."""
    z = np.asarray(logits, F32)
    if temperature <= 0.0:
        return int(np.argmax(z))                  # greedy: lowest index of the maximum
    z = apply_temperature(z, temperature)
    z = top_k_mask(z, top_k)
    z = top_p_mask(z, top_p)
    return categorical(softmax(z), r)


def sample_rows(logits: np.ndarray, temperature: float, top_k: int, top_p: float,
                r: np.ndarray) -> np.ndarray:
    """``sample`` for every row of a [R, V] array with draws r[R]."""
    return np.array([sample(logits[i], temperature, top_k, top_p, float(r[i]))
                     for i in range(logits.shape[0])], np.int32)


def final_distribution(logits: np.ndarray, temperature: float, top_k: int,
                       top_p: float) -> np.ndarray:
    """The distribution stage 5 draws from (t > 0), for validity checks of a draw."""
    z = apply_temperature(logits, temperature)
    return softmax(top_p_mask(top_k_mask(z, top_k), top_p))
