"""Pins of the CPU oracle against facts that do not come from the oracle itself:
library routines (dense softmax attention, matmul), closed forms, invariants,
the pages' own parameters, and a scalar brute force.  CPU only."""

import json
import math
import os

import numpy as np
import pytest
import torch
from hypothesis import given, settings, strategies as st

import oracle
from brute_force import brute_forward
from synth import random_qkv

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def _dense_sdpa(q, k, v, causal, scale=None):
    """Dense softmax attention from torch's CPU routine, float64, K/V heads
    repeated for grouped queries."""
    G = q.shape[1] // k.shape[1]
    qt = torch.from_numpy(np.asarray(q, np.float64))
    kt = torch.from_numpy(np.asarray(k, np.float64)).repeat_interleave(G, dim=1)
    vt = torch.from_numpy(np.asarray(v, np.float64)).repeat_interleave(G, dim=1)
    return torch.nn.functional.scaled_dot_product_attention(
        qt, kt, vt, is_causal=causal, scale=scale).numpy()


CASES = [
    # B, Hq, Hkv, N, d, block
    (1, 2, 2, 256, 16, 64),
    (2, 4, 2, 200, 8, 64),     # GQA + ragged last block (200 = 3*64 + 8)
    (1, 3, 1, 130, 12, 32),    # 3 Q heads per KV head, last block of 2 tokens
    (1, 2, 2, 97, 8, 128),     # a single partial block
]


# ---------------------------------------------------------------- P1: density 1

@pytest.mark.parametrize("case", CASES)
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("approx", [False, True])
def test_density_one_is_dense_attention(case, causal, approx):
    B, Hq, Hkv, N, d, block = case
    q, k, v = random_qkv(B, Hq, Hkv, N, d, seed=1, block=block)
    r = oracle.forward(q, k, v, block=block, causal=causal, approx=approx, mode="density",
                       density=1.0)
    ref = _dense_sdpa(q, k, v, causal)
    assert np.all(r["mask"] == oracle.eligible_mask(r["mask"].shape[-1], causal))
    np.testing.assert_allclose(r["out"], ref, atol=1e-12, rtol=0)


# ------------------------------------------- P2: online recurrence == full softmax

def _online(z, vals, mult, block, dtype):
    """Running max / sum recurrence of the tutorial's section 2, over the logits
    in chunks of ``block``; pseudo-keys carry a multiplicity in the sum."""
    m = -np.inf
    l = dtype(0)
    o = np.zeros(vals.shape[1], dtype)
    for s in range(0, len(z), block):
        zb = z[s:s + block].astype(dtype)
        mb = max(m, zb.max())
        c = np.exp(dtype(m - mb)) if np.isfinite(m) else dtype(0)
        p = np.exp(zb - mb).astype(dtype)
        l = l * c + (p * mult[s:s + block].astype(dtype)).sum(dtype=dtype)
        o = o * c + (p[:, None] * vals[s:s + block].astype(dtype)).sum(axis=0, dtype=dtype)
        m = mb
    return o / l


def test_online_softmax_matches_closed_form_page_row():
    g = _golden("online_softmax_row.json")
    n, blk = g["row_length"], g["block"]
    rng = np.random.default_rng(7)
    d = 4
    q = rng.standard_normal((1, 1, 1, d))
    k = rng.standard_normal((1, 1, n, d)) * 3.0
    v = rng.standard_normal((1, 1, n, d))
    # one query token; put it in a query block of its own by using N=n keys and
    # a selection mask that keeps every key block
    M = -(-n // blk)
    sel = np.ones((1, 1, 1, M), bool)
    out = oracle.attend_block(q[0, 0], 0, k[0, 0], v[0, 0], None, None, sel[0, 0, 0],
                              np.ones(M, bool), block=blk, scale=1.0, causal=False, approx=False)
    z = (k[0, 0] @ q[0, 0, 0])
    o64 = _online(z, v[0, 0], np.ones(n), blk, np.float64)
    o32 = _online(z.astype(np.float32), v[0, 0].astype(np.float32), np.ones(n), blk, np.float32)
    np.testing.assert_allclose(o64, out[0], atol=1e-14, rtol=0)
    # float32 recurrence: error of the size the page reports, far below 1e-6
    assert np.abs(o32 - out[0]).max() < 1e-6
    assert n % blk != 0   # the page's row has a ragged last chunk (2000 = 15*128 + 80)


@pytest.mark.parametrize("causal", [False, True])
def test_online_recurrence_with_tail_matches_oracle(causal):
    """The GPU kernel folds exact keys and tail pseudo-keys into one running
    max/sum; that recurrence must reproduce the oracle's closed form."""
    B, Hq, Hkv, N, d, block = 1, 2, 1, 320, 16, 64
    q, k, v = (x.astype(np.float64) for x in random_qkv(B, Hq, Hkv, N, d, seed=3, block=block))
    r = oracle.forward(q, k, v, block=block, causal=causal, approx=True, mode="alpha", alpha=0.6)
    M = r["mask"].shape[-1]
    scale = 1 / math.sqrt(d)
    for h in range(Hq):
        for I in range(M):
            elig = oracle.eligible_mask(M, causal)[I]
            sel = r["mask"][0, h, I]
            tail = [J for J in range(M) if elig[J] and not sel[J]]
            for i in range(I * block, min(N, (I + 1) * block), 17):
                keys = [j for J in range(M) if sel[J]
                        for j in range(J * block, min(N, (J + 1) * block)) if not causal or j <= i]
                z = np.concatenate([scale * k[0, 0, keys] @ q[0, h, i],
                                    scale * r["k_bar"][0, 0, tail] @ q[0, h, i]])
                vals = np.concatenate([v[0, 0, keys], r["v_sum"][0, 0, tail]])
                mult = np.concatenate([np.ones(len(keys)), r["n"][tail]])
                o = _online(z, vals, mult, 64, np.float64)
                np.testing.assert_allclose(o, r["out"][0, h, i], atol=1e-13, rtol=0)


# ------------------------------------ P3: identical keys in a block -> tail is exact

@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("case", CASES[:3])
def test_tail_exact_for_identical_keys(case, causal):
    B, Hq, Hkv, N, d, block = case
    q, _, v = random_qkv(B, Hq, Hkv, N, d, seed=5, block=block)
    rng = np.random.default_rng(11)
    M = -(-N // block)
    centres = rng.standard_normal((B, Hkv, M, d))
    k = np.repeat(centres, block, axis=2)[:, :, :N]
    # an arbitrary selection with at least one block per row
    sel = rng.random((B, Hq, M, M)) < 0.3
    sel &= oracle.eligible_mask(M, causal)
    sel[..., 0] = True
    if causal:
        sel |= np.eye(M, dtype=bool)    # causal + tail keeps the diagonal exact
    r = oracle.forward(q, k, v, block=block, causal=causal, approx=True, mode="alpha", sel=sel)
    np.testing.assert_allclose(r["out"], _dense_sdpa(q, k, v, causal), atol=1e-12, rtol=0)
    # without the tail the same selection must differ from dense attention
    r0 = oracle.forward(q, k, v, block=block, causal=causal, approx=False, mode="alpha", sel=sel)
    assert np.abs(r0["out"] - _dense_sdpa(q, k, v, causal)).max() > 1e-3


# ------------------------------------------------------------------ P4: AM-GM

def test_tail_weight_never_exceeds_block_mass():
    """n_J * exp(scale q.kbar_J) <= sum_j exp(scale q.k_j): the pooled key is a
    lower bound on the block's softmax mass (FlashPrefill summary 2(a), GM<=AM)."""
    q, k, _ = random_qkv(1, 2, 2, 192, 16, seed=2, block=64, noise=1.0)
    scale = 0.25
    kbar = oracle.pool_mean(k, 64)
    n = oracle.block_sizes(192, 64)
    for h in range(2):
        za = scale * q[0, h] @ kbar[0, h].T                      # [N, M]
        zt = scale * q[0, h] @ k[0, h].T                          # [N, N]
        mass = np.stack([np.exp(zt[:, s:e]).sum(1) for s, e in oracle.block_bounds(192, 64)], 1)
        assert np.all(n * np.exp(za) <= mass * (1 + 1e-12))


# ------------------------------------------------------- P5: 2D-reduction identity

@pytest.mark.parametrize("case", CASES)
def test_pooled_score_is_mean_of_token_scores(case):
    """FlashPrefill summary 2(a): scoring pooled vectors equals reducing the
    token-level score tile; s_IJ = scale * mean_{i in I, j in J} q_i.k_j."""
    B, Hq, Hkv, N, d, block = case
    q, k, _ = random_qkv(B, Hq, Hkv, N, d, seed=4, block=block)
    scale = 0.37
    s = oracle.block_scores(oracle.pool_mean(q, block), oracle.pool_mean(k, block), scale)
    G = Hq // Hkv
    kt = torch.from_numpy(k.astype(np.float64)).repeat_interleave(G, dim=1)
    full = scale * torch.matmul(torch.from_numpy(q.astype(np.float64)), kt.transpose(-1, -2))
    bnd = oracle.block_bounds(N, block)
    red = np.array([[[[full[b, h, si:ei, sj:ej].mean().item() for (sj, ej) in bnd]
                      for (si, ei) in bnd] for h in range(Hq)] for b in range(B)])
    np.testing.assert_allclose(s, red, atol=1e-12, rtol=0)


# --------------------------------------------------------- P6: selection invariants

def test_threshold_half_of_max_page_cases():
    g = _golden("threshold_half_of_max.json")
    for c in g["cases"]:
        s = np.array(c["scores"])[None, :]
        sel = oracle.select_alpha(s, np.ones((1, len(s[0])), bool), g["alpha"])
        assert list(np.nonzero(sel[0])[0]) == c["kept"]


def test_topk_count_page_defaults():
    g = _golden("pisa_call_defaults.json")
    for c in g["derived_counts"]:
        assert oracle.topk_count(c["blocks_per_row"], g["density"]) == c["k"]
    assert oracle.topk_count(50, 1.0) == 50
    assert oracle.topk_count(50, 1e-6) == 1


@settings(max_examples=60, deadline=None)
@given(st.integers(1, 40), st.floats(0.05, 1.0), st.booleans(), st.integers(0, 10_000))
def test_alpha_selection_invariants(M, alpha, causal, seed):
    rng = np.random.default_rng(seed)
    s = rng.standard_normal((M, M)) + rng.choice([0.0, 1.0])
    elig = oracle.eligible_mask(M, causal)
    sel = oracle.select_alpha(s, elig, alpha)
    for I in range(M):
        row = np.where(elig[I], s[I], -np.inf)
        arg = np.argmax(row)
        assert sel[I, arg]                                   # argmax always kept
        assert not np.any(sel[I] & ~elig[I])                 # eligible only
        kept, drop = s[I][sel[I]], s[I][elig[I] & ~sel[I]]
        if len(drop):
            assert kept.min() > drop.max()                   # a threshold split
        if row.max() > 0:
            assert np.all(kept >= alpha * row.max())
        else:
            assert np.all(kept == row.max())                 # non-positive max: argmax set
    # alpha = 1 keeps exactly the arg-max set; smaller alpha keeps a superset
    one = oracle.select_alpha(s, elig, 1.0)
    for I in range(M):
        row = np.where(elig[I], s[I], -np.inf)
        assert np.array_equal(np.nonzero(one[I])[0], np.nonzero(row == row.max())[0])
    assert np.all(oracle.select_alpha(s, elig, alpha * 0.5) >= sel) or np.all(s.max(1) <= 0)


@settings(max_examples=60, deadline=None)
@given(st.integers(1, 40), st.floats(0.01, 1.0), st.booleans(), st.integers(0, 10_000))
def test_density_selection_invariants(M, density, causal, seed):
    rng = np.random.default_rng(seed)
    s = np.round(rng.standard_normal((M, M)), 1)     # coarse values -> many ties
    elig = oracle.eligible_mask(M, causal)
    sel = oracle.select_density(s, elig, density)
    for I in range(M):
        e = np.nonzero(elig[I])[0]
        k = oracle.topk_count(len(e), density)
        assert sel[I].sum() == k
        kept = np.nonzero(sel[I])[0]
        drop = np.array([J for J in e if not sel[I, J]])
        if len(drop):
            assert s[I, kept].min() >= s[I, drop].max()
            # ties at the cut go to the lower block index
            cut = s[I, kept].min()
            tied_drop = drop[s[I, drop] == cut]
            tied_kept = kept[s[I, kept] == cut]
            if len(tied_drop):
                assert tied_kept.max() < tied_drop.min()


@pytest.mark.parametrize("mode", ["alpha", "density"])
def test_selection_invariant_to_positive_query_scale(mode):
    q, k, v = random_qkv(1, 2, 2, 512, 16, seed=9, block=64)
    a = oracle.forward(q, k, v, block=64, causal=False, approx=True, mode=mode, alpha=0.5,
                       density=0.3, rows=[])
    b = oracle.forward(q * 3.5, k, v, block=64, causal=False, approx=True, mode=mode,
                       alpha=0.5, density=0.3, rows=[])
    assert np.array_equal(a["mask"], b["mask"])


def test_mask_to_lists_ascending():
    rng = np.random.default_rng(0)
    sel = rng.random((2, 3, 9, 9)) < 0.4
    idx, cnt = oracle.mask_to_lists(sel)
    for pos in np.ndindex(2, 3, 9):
        c = cnt[pos]
        assert list(idx[pos][:c]) == list(np.nonzero(sel[pos])[0])
        assert np.all(idx[pos][c:] == -1)


# ------------------------------------------------------------- P7: brute force

BRUTE = [
    # B, Hq, Hkv, N, d, block, causal, approx, mode
    (1, 2, 2, 256, 4, 64, False, True, "alpha"),
    (1, 2, 1, 200, 4, 64, True, False, "alpha"),
    (1, 2, 2, 150, 3, 32, True, True, "density"),
    (2, 2, 1, 96, 5, 32, False, False, "density"),
    (1, 4, 2, 70, 3, 16, False, True, "density"),
]


@pytest.mark.parametrize("case", BRUTE)
def test_brute_force_agrees(case):
    B, Hq, Hkv, N, d, block, causal, approx, mode = case
    q, k, v = random_qkv(B, Hq, Hkv, N, d, seed=12, block=block, noise=0.5)
    r = oracle.forward(q, k, v, block=block, causal=causal, approx=approx, mode=mode,
                       alpha=0.5, density=0.3)
    bm, bo = brute_forward(q.astype(float).tolist(), k.astype(float).tolist(),
                           v.astype(float).tolist(), block=block, causal=causal, approx=approx,
                           mode=mode, alpha=0.5, density=0.3)
    idx, cnt = oracle.mask_to_lists(r["mask"])
    for b in range(B):
        for h in range(Hq):
            for I in range(len(bm[b][h])):
                assert list(idx[b, h, I, :cnt[b, h, I]]) == bm[b][h][I]
    np.testing.assert_allclose(r["out"], np.array(bo), atol=1e-12, rtol=0)


# ------------------------------------------- P8: permutation and GQA invariances

def test_permutation_inside_block_changes_nothing():
    q, k, v = random_qkv(1, 2, 2, 256, 8, seed=21, block=64)
    rng = np.random.default_rng(3)
    perm = np.concatenate([rng.permutation(64) + s for s in range(0, 256, 64)])
    a = oracle.forward(q, k, v, block=64, causal=False, approx=True, mode="alpha", alpha=0.4)
    b = oracle.forward(q, k[:, :, perm], v[:, :, perm], block=64, causal=False, approx=True,
                       mode="alpha", alpha=0.4)
    assert np.array_equal(a["mask"], b["mask"])
    np.testing.assert_allclose(a["out"], b["out"], atol=1e-12, rtol=0)


@pytest.mark.parametrize("causal,approx,mode", [(False, True, "density"), (True, False, "alpha"),
                                                (True, True, "alpha")])
def test_gqa_equals_repeated_heads(causal, approx, mode):
    q, k, v = random_qkv(1, 4, 2, 192, 8, seed=8, block=64)
    a = oracle.forward(q, k, v, block=64, causal=causal, approx=approx, mode=mode)
    kr, vr = np.repeat(k, 2, axis=1), np.repeat(v, 2, axis=1)
    b = oracle.forward(q, kr, vr, block=64, causal=causal, approx=approx, mode=mode)
    assert np.array_equal(a["mask"], b["mask"])
    np.testing.assert_allclose(a["out"], b["out"], atol=1e-13, rtol=0)


# --------------------------------------------------- hand-derived closed forms

def _tiny_case():
    """N=4, block 2, d=1, scale 1.  Keys: block 0 = (ln 2, ln 2), block 1 =
    (ln 3, -ln 3) so kbar_1 = 0; every query is 1; values 1, 3, 5, 7.
    Pooled scores: s_I0 = ln 2, s_I1 = 0 -> alpha=0.5 keeps block 0 only."""
    q = np.ones((1, 1, 4, 1))
    k = np.array([math.log(2), math.log(2), math.log(3), -math.log(3)]).reshape(1, 1, 4, 1)
    v = np.array([1.0, 3.0, 5.0, 7.0]).reshape(1, 1, 4, 1)
    return q, k, v


def test_closed_form_tiny_with_tail():
    # exact: exp(ln2)*(1+3) = 8 over weight 4; tail: pseudo-key 0 -> exp(0)=1,
    # weight n=2, value sum 12.  o = (8 + 12) / (4 + 2) = 10/3.
    q, k, v = _tiny_case()
    r = oracle.forward(q, k, v, block=2, causal=False, approx=True, mode="alpha", alpha=0.5,
                       scale=1.0)
    assert r["mask"][0, 0].tolist() == [[True, False], [True, False]]
    np.testing.assert_allclose(r["out"][0, 0, :, 0], [10 / 3] * 4, rtol=0, atol=1e-15)


def test_closed_form_tiny_without_tail_and_dense():
    q, k, v = _tiny_case()
    r = oracle.forward(q, k, v, block=2, causal=False, approx=False, mode="alpha", alpha=0.5,
                       scale=1.0)
    np.testing.assert_allclose(r["out"][0, 0, :, 0], [2.0] * 4, rtol=0, atol=1e-15)   # (2+6)/4
    # dense: weights 2,2,3,1/3 -> (2 + 6 + 15 + 7/3) / (2+2+3+1/3) = (76/3)/(22/3) = 38/11
    rd = oracle.forward(q, k, v, block=2, causal=False, approx=True, mode="density",
                        density=1.0, scale=1.0)
    np.testing.assert_allclose(rd["out"][0, 0, :, 0], [38 / 11] * 4, rtol=0, atol=1e-14)


def test_closed_form_causal_diagonal():
    # causal, no tail, alpha 0.5: query block 1 sees blocks 0 (s=ln2) and 1
    # (s=0): keeps block 0 only.  Query block 0 keeps block 0; token 0 sees
    # only key 0 -> o=1; token 1 sees keys 0,1 (equal weights) -> o=2.
    q, k, v = _tiny_case()
    r = oracle.forward(q, k, v, block=2, causal=True, approx=False, mode="alpha", alpha=0.5,
                       scale=1.0)
    np.testing.assert_allclose(r["out"][0, 0, :, 0], [1.0, 2.0, 2.0, 2.0], rtol=0, atol=1e-15)


def test_band_marks_only_close_pairs():
    # density 0.5 of 4 blocks -> k=2: scores 1.0, 0.5, 0.5+1e-7, -1: the 2nd and
    # 3rd are within 1e-5 of their midpoint; alpha 0.5 of max 1.0 -> t=0.5
    s = np.tile(np.array([1.0, 0.5, 0.5 + 1e-7, -1.0]), (4, 1))     # [M, M], M = 4
    t = oracle.thresholds(s, causal=False, mode="density", density=0.5)
    assert oracle.band_mask(s, t, False).tolist() == [[False, True, True, False]] * 4
    t = oracle.thresholds(s, causal=False, mode="alpha", alpha=0.5)
    assert oracle.band_mask(s, t, False).tolist() == [[False, True, True, False]] * 4
    t = oracle.thresholds(s, causal=False, mode="alpha", alpha=0.9)
    assert not oracle.band_mask(s, t, False).any()
    t = oracle.thresholds(s, causal=False, mode="density", density=1.0)
    assert not oracle.band_mask(s, t, False).any()
