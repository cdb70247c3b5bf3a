"""Oracle for the generator's token sampling (fp64, NumPy, CPU).

TEST INFRASTRUCTURE ONLY -- see the package docstring. Never called by the library.

Source: "PersonaPlex native LM audit" (Clockless Inkling, personaplex-research page),
section 7 "One exact generator step" and the note after it: generation samples text
with temperature 0.7 over the top 25 logits and audio with temperature 0.8 over the top
250. The page does not spell out the sampling procedure; the reading used here (and by
the library) is the plain one:

  1. order the candidates by logit, largest first (equal logits: lower index first) and
     keep the first top_k;
  2. weights w_i = exp((l_i - l_0) / temperature) over those candidates, l_0 the largest;
  3. with a uniform draw u in [0, 1), return the first candidate whose running sum
     w_0 + ... + w_i exceeds u * (w_0 + ... + w_{k-1}) (inverse of the categorical CDF).

top_k <= 1 or temperature <= 0 is plain argmax (lowest index on ties). The random
numbers are inputs: the caller supplies u, so both implementations consume the same
draws. Logits arrive as float32 values and are widened exactly; every step after that
is fp64 -- the same precision the library uses for this decision.
"""

import numpy as np


def top_k_order(logits, top_k):
    """Indices of the top_k largest logits, largest first, equal values by lower index."""
    l = np.asarray(logits, np.float64)
    idx = np.arange(l.shape[0])
    order = np.lexsort((idx, -l))          # primary key -l (ascending), then index
    return order[:max(1, min(int(top_k), l.shape[0]))]


def sample_top_k(logits, temperature, top_k, u):
    """One draw from the temperature-scaled softmax over the top_k logits (see above)."""
    l = np.asarray(logits, np.float64)
    if int(top_k) <= 1 or float(temperature) <= 0.0:
        return int(np.argmax(l))           # first maximum
    order = top_k_order(l, top_k)
    w = np.exp((l[order] - l[order[0]]) / np.float64(np.float32(temperature)))
    c = np.cumsum(w)                       # running sums, left to right
    r = np.float64(u) * c[-1]
    i = int(np.searchsorted(c, r, side="right"))   # first i with c[i] > r
    return int(order[min(i, len(order) - 1)])
