"""Pins of the greedy-acceptance oracle (CPU only): the greedy choice
against numpy's argmax (a library routine with the same tie and NaN rule),
hand cases, and the pages' exactness property -- a speculative round
emits exactly what plain greedy decoding emits -- on a toy model."""
import numpy as np
import pytest

from oracle.accept import greedy_accept, greedy_token


def test_greedy_token_hand_cases():
    assert greedy_token([1.0, 3.0, 3.0, 2.0]) == 1          # first of a tie
    assert greedy_token([-5.0]) == 0
    assert greedy_token([float("nan"), 5.0, float("nan")]) == 0
    assert greedy_token([1.0, float("nan"), 9.0, float("nan")]) == 1
    assert greedy_token([-0.0, 0.0]) == 0 and greedy_token([0.0, -0.0]) == 0
    assert greedy_token([-np.inf, -1e30]) == 1
    assert greedy_token([np.inf, np.inf]) == 0


@pytest.mark.parametrize("seed", range(6))
def test_greedy_token_matches_numpy_argmax(seed):
    rng = np.random.default_rng(seed)
    v = rng.standard_normal(3000).astype(np.float32)
    # plant ties at the maximum and, for some seeds, NaNs and signed zeros
    top = v.max() + 1.0
    v[rng.integers(0, 3000, 3)] = top
    if seed % 2:
        v[rng.integers(0, 3000, 2)] = np.nan
    if seed % 3 == 0:
        v[:] = -np.abs(v)
        v[rng.integers(0, 3000, 4)] = 0.0
        v[rng.integers(0, 3000, 4)] = -0.0
    assert greedy_token(v) == int(np.argmax(v))


def test_accept_counts_the_matching_prefix():
    logits = np.zeros((4, 6))
    for n, t in enumerate([2, 5, 1, 3]):
        logits[n, t] = 1.0
    t, a = greedy_accept(logits, [2, 5, 1])
    assert list(t) == [2, 5, 1, 3] and a == 3
    t, a = greedy_accept(logits, [2, 4, 1])
    assert list(t) == [2, 5, 1, 3] and a == 1           # the second draft fails; the third is not kept
    assert greedy_accept(logits, [0, 5, 1])[1] == 0
    assert greedy_accept(logits[:1], [])[1] == 0        # N = 1: no drafts


@pytest.mark.parametrize("seed", range(20))
def test_round_equals_plain_greedy_on_a_toy_model(seed):
    # A toy model whose next-token logits depend on the current token only.
    # Plain greedy decoding from t0 gives g1, g2, ...; a round over drafts
    # d_1..d_{N-1} sees at column j the logits after (t0, d_1..d_j), and must
    # emit a prefix of g1, g2, ... whose length is 1 + the drafts that match.
    rng = np.random.default_rng(seed)
    V = 7
    table = rng.standard_normal((V, V))
    table[rng.integers(0, V), :] = table[rng.integers(0, V), :]  # a duplicate row: ties between tokens
    t0 = int(rng.integers(0, V))
    greedy = [t0]
    for _ in range(9):
        greedy.append(int(np.argmax(table[greedy[-1]])))
    N = int(rng.integers(1, 9))
    drafts = []
    for j in range(1, N):
        drafts.append(greedy[j] if rng.random() < 0.7 else int(rng.integers(0, V)))
    ctx = [t0] + drafts
    logits = np.stack([table[ctx[j]] for j in range(N)])
    tokens, a = greedy_accept(logits, drafts)
    emitted = list(tokens[:a + 1])
    assert emitted == greedy[1:a + 2]
    matches = 0
    while matches < N - 1 and drafts[matches] == greedy[matches + 1]:
        matches += 1
    assert a == matches
