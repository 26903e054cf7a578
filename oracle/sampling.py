"""fp64 top-k / top-p sampling of one logits row with a given uniform draw.

TEST INFRASTRUCTURE ONLY (see the package docstring).  numpy only.

The sampling step after the LM head turns a row of logits into one token id ("Kernels,
Fusion & CUDA Graphs", Fix 1 table: sampling; "The serving engine's kernel stack").
The pages name the step, not a rule; this is the usual top-k / nucleus rule, written out
plainly (the readings are listed with the design notes):

  order   the indices by logit, largest first, the lower index first on equal logits
          (NaN ranks as -inf);
  top-k   keep the first k of that order;
  weight  w_j = exp((z_j - z_max) / T) over the kept candidates, in that order;
  nucleus keep the shortest prefix m whose running weight reaches top_p of the total;
  draw    the first candidate j <= m whose running weight exceeds u * W_m, u in [0, 1)
          (u is an input: the random number is drawn by the caller).

top_k = 1 is greedy sampling.  `sample` returns the token id and, for tests, the
distance of u * W_m and of top_p * W from the running weights that decided the result
(relative to W_m), so that a test can tell a robust decision from one that rounding in
another precision may move to a neighbouring candidate.
"""

from __future__ import annotations

from typing import NamedTuple

import numpy as np


class Sample(NamedTuple):
    token: int
    order: np.ndarray      # candidate indices, ranked
    probs: np.ndarray      # nucleus probabilities of the ranked candidates (0 past the nucleus)
    margin: float          # smallest relative distance of a deciding comparison


def _rank(z: np.ndarray) -> np.ndarray:
    zz = np.where(np.isnan(z), -np.inf, z)
    # numpy's lexsort sorts by the last key first: value descending, then index ascending
    return np.lexsort((np.arange(zz.size), -zz))


def sample(logits, temperature: float, top_k: int, top_p: float, u: float) -> Sample:
    z = np.asarray(logits, dtype=np.float64).ravel()
    if not (temperature > 0) or not (0 < top_p <= 1) or top_k < 1 or not (0 <= u < 1):
        raise ValueError("need temperature > 0, 0 < top_p <= 1, top_k >= 1, 0 <= u < 1")
    order = _rank(z)[: min(top_k, z.size)]
    zk = np.where(np.isnan(z[order]), -np.inf, z[order])
    zmax = zk[0]
    w = np.where(zk == -np.inf, 0.0, np.exp((zk - zmax) / temperature)) if np.isfinite(zmax) else np.zeros(zk.size)
    cum = np.cumsum(w)
    total = cum[-1]
    # nucleus: the first running weight that reaches top_p of the total
    reach = np.nonzero(cum >= top_p * total)[0]
    m = int(reach[0]) if reach.size else zk.size - 1
    wm = cum[m]
    target = u * wm
    above = np.nonzero(cum[: m + 1] > target)[0]
    j = int(above[0]) if above.size else m
    scale = wm if wm > 0 else 1.0
    margins = [abs(cum[j] - target) / scale]
    if j > 0:
        margins.append(abs(target - cum[j - 1]) / scale)
    margins.append(abs(cum[m] - top_p * total) / scale)
    if m > 0:
        margins.append(abs(top_p * total - cum[m - 1]) / scale)
    probs = np.zeros(zk.size)
    if wm > 0:
        probs[: m + 1] = w[: m + 1] / wm
    return Sample(int(order[j]), order, probs, float(min(margins)))
