"""Selection readings that the near-threshold band would hide, checked
exactly on the GPU through the C ABI.

The inputs make every pooled statistic and every pooled score exact in
float32 and float64 alike: each block's query rows and key rows are one
small-integer vector repeated (so the block mean is that vector), d = 64
(scale 1/8, a power of two) and the score is an integer over 8.  The GPU
and the oracle then see the same score values, and the lists must agree bit
for bit with no band exemption:

* a row whose pooled scores are all negative keeps only its arg-max blocks
  (the threshold is the max itself: every arg-max lies exactly on it;
  FlashPrefill summary 2(b), with the reading for a non-positive max);
* alpha * max exactly equal to some scores keeps them (>= at the threshold);
* top-k with equal scores straddling the k-th place keeps the lower block
  indices (PISA explainer, documented density call; ties to the lower J).
"""

import numpy as np
import pytest

import oracle
from gpu_helpers import TOL_OUT, run_gpu, say

pytestmark = pytest.mark.gpu

D = 64
BLOCK = 64


def _blocks_to_tokens(vecs: np.ndarray, N: int) -> np.ndarray:
    """[M, d] per-block vectors -> [N, d] token rows (every row of block J is vecs[J])."""
    return np.repeat(vecs, BLOCK, axis=0)[:N].astype(np.float32)


def _inputs(M: int, q_blocks: np.ndarray, k_blocks: np.ndarray, seed: int, Hq=1):
    N = M * BLOCK
    rng = np.random.default_rng(seed)
    q = np.stack([_blocks_to_tokens(q_blocks, N)] * Hq)[None]
    k = _blocks_to_tokens(k_blocks, N)[None, None]
    v = rng.integers(-4, 5, size=(1, 1, N, D)).astype(np.float32)   # bf16-exact values
    return q, k, v


def _score_table(M: int, rows_pattern):
    """Key and query block vectors giving s_IJ = pattern[type(I)][J] / 8
    exactly: query block I is the unit vector e_{type(I)}, key block J
    carries pattern[t][J] in coordinate t."""
    T = len(rows_pattern)
    kb = np.zeros((M, D), np.float32)
    for t, pat in enumerate(rows_pattern):
        kb[:, t] = np.asarray(pat, np.float32)
    qb = np.zeros((M, D), np.float32)
    for I in range(M):
        qb[I, I % T] = 1.0
    return qb, kb


def _check_exact(q, k, v, *, causal, approx, mode, alpha=0.5, density=0.15):
    ref = oracle.forward(q, k, v, block=BLOCK, causal=causal, approx=approx, mode=mode, alpha=alpha,
                         density=density)
    g = run_gpu(q, k, v, dtype="bf16", block=BLOCK, causal=causal, approx=approx, mode=mode, alpha=alpha,
                density=density)
    diff = g["mask"] != ref["mask"]
    assert not diff.any(), f"{int(diff.sum())} blocks differ (no band), first at {np.argwhere(diff)[:5].tolist()}"
    err = np.abs(g["out"] - ref["out"]).max()
    say(f"  lists identical ({int(ref['mask'].sum())} blocks), output max-abs {err:.3e}")
    assert err <= TOL_OUT["bf16"]
    return ref


M = 20   # k = ceil(0.15 * 20) = 3 in density mode (non-causal)

# pooled scores x 8, one pattern per query-block type (I % 4)
PATTERNS = [
    # four equal maxima, k = 3: the first three (J = 0, 1, 2); alpha: all four
    [5, 5, 5, 5] + [1] * 16,
    # one top score, then four tied at the cut (J = 3, 8, 12, 19): keep J = 3, 8
    [0, 0, 0, 3, 0, 0, 9, 0, 3, 0, 0, 0, 3, 0, 0, 0, 0, 0, 0, 3],
    # every score negative, the maximum -1 tied at J = 4 and 15
    [-3, -7, -2, -5, -1, -9, -4, -6, -2, -8, -3, -5, -7, -2, -6, -1, -4, -9, -3, -8],
    # max 8, alpha 0.5 -> threshold exactly 4: the 4s are kept, 3s dropped
    [8, 4, 3, 4, 0, 3, 4, 1, 2, 3, 4, 0, -4, 3, 4, 1, 0, 2, 3, 4],
]


@pytest.mark.parametrize("mode", ["alpha", "density"])
@pytest.mark.parametrize("causal", [False, True])
def test_exact_ties_and_nonpositive_max(mode, causal):
    say("exact selection", mode, "causal" if causal else "full")
    qb, kb = _score_table(M, PATTERNS)
    q, k, v = _inputs(M, qb, kb, seed=3, Hq=2)
    ref = _check_exact(q, k, v, causal=causal, approx=not causal, mode=mode)
    s = ref["scores"][0, 0]
    sel = ref["mask"][0, 0]
    if not causal:
        # the readings themselves, on the rows built for them
        if mode == "density":
            assert list(np.nonzero(sel[0])[0]) == [0, 1, 2]          # equal maxima: lower J
            assert list(np.nonzero(sel[1])[0]) == [3, 6, 8]          # tie at the cut: lower J
        else:
            assert list(np.nonzero(sel[2])[0]) == [4, 15]            # non-positive max: arg-max set
            kept = np.nonzero(sel[3])[0]
            assert np.all(s[3, kept] >= 0.5 * s[3].max()) and (s[3, kept] == 0.5 * s[3].max()).sum() == 6
    assert np.all(ref["mask"].sum(-1) >= 1)


def test_exact_all_rows_negative_grouped_heads():
    """Every row of both query heads (one KV head) has only negative pooled
    scores: each keeps exactly its arg-max set, with the tail on."""
    say("exact selection, all rows non-positive")
    rng = np.random.default_rng(11)
    Mn = 24
    kb = np.zeros((Mn, D), np.float32)
    kb[:, :8] = rng.integers(1, 4, size=(Mn, 8))          # positive key coordinates
    qb = np.zeros((Mn, D), np.float32)
    qb[:, :8] = -rng.integers(0, 3, size=(Mn, 8))         # non-positive query coordinates
    qb[:, 0] -= 1.0                                        # every score strictly negative
    q, k, v = _inputs(Mn, qb, kb, seed=12, Hq=2)
    ref = _check_exact(q, k, v, causal=False, approx=True, mode="alpha", alpha=0.5)
    s = ref["scores"]
    assert np.all(s < 0)
    m = s.max(-1, keepdims=True)
    assert np.array_equal(ref["mask"], s == m)
