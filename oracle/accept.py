"""Greedy draft acceptance -- TEST INFRASTRUCTURE ONLY (same rule as the
rest of ``oracle``: only tests/, the smoke check and the bench's CPU leg may
use it).

What a speculative round does after its verify pass, read from the pages:
- the crit README, section "Inference", bullet on generating several
  tokens per round: speculative decoding proposes a continuation, verifies
  it and keeps the accepted tokens; its section "Core" lists greedy draft
  acceptance under the sampling part;
- the crit-hub engine card "mtp7-device-confidence", section "Design", rows
  "Decode" (the verify pass runs over the drafts made, inside the round's
  device graph) and "Exactness" (the output equals plain greedy decoding,
  bit for bit);
- the crit landing page, its Eval list: drafting is checked against plain
  greedy decoding.

Reading (the pages give no formula):
- the verify pass has N columns: column 0 holds the last accepted token,
  columns 1..N-1 the N-1 drafts d_1..d_{N-1};
- column j's target token t_j is the greedy choice of the head's logits
  for that column: the index of the largest logit, the first one on ties,
  with a NaN logit counting as larger than any number (so the first NaN
  wins; +0 and -0 are equal);
- draft d_j is accepted when it equals t_{j-1} and every earlier draft was
  accepted; the round emits t_0..t_a for a accepted drafts.
"""
from __future__ import annotations

import math
from typing import Sequence, Tuple

import numpy as np


def greedy_token(logits: Sequence[float]) -> int:
    """Index of the largest value; first on ties; the first NaN beats all."""
    best = 0
    bv = float(logits[0])
    if math.isnan(bv):
        return 0
    for i in range(1, len(logits)):
        v = float(logits[i])
        if math.isnan(v):
            return i
        if v > bv:
            best, bv = i, v
    return best


def greedy_accept(logits: np.ndarray, drafts: Sequence[int]) -> Tuple[np.ndarray, int]:
    """(t[0..N-1], a) for logits [N][V] and drafts d_1..d_{N-1}."""
    N = logits.shape[0]
    if len(drafts) != N - 1:
        raise ValueError("need N - 1 drafts")
    tokens = np.array([greedy_token(logits[n]) for n in range(N)], dtype=np.int64)
    a = 0
    while a < N - 1 and int(drafts[a]) == int(tokens[a]):
        a += 1
    return tokens, a
