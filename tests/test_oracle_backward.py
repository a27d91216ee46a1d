"""Pins of the oracle's gradients (``oracle.backward``) against things other
than themselves: central finite differences of the oracle's forward (with the
selection held fixed, the forward is a smooth function of q, k, v), and
torch's autograd of dense softmax attention for density 1.  CPU only."""

import numpy as np
import pytest
import torch

import oracle
from synth import random_qkv

CASES = [
    # B, Hq, Hkv, N, d, block, causal, approx
    (1, 2, 1, 40, 8, 16, False, True),    # GQA, ragged last block (40 = 2*16 + 8), tail on
    (1, 2, 2, 48, 8, 16, True, True),     # causal + tail (forced diagonal)
    (2, 2, 1, 37, 4, 8, True, False),     # causal, no tail, several ragged blocks
    (1, 1, 1, 64, 8, 16, False, False),
]


def _selection(q, k, v, block, causal, approx):
    r = oracle.forward(q, k, v, block=block, causal=causal, approx=approx, mode="density",
                       density=0.4)
    return r["mask"]


def _loss(q, k, v, dout, sel, block, causal, approx):
    r = oracle.forward(q, k, v, block=block, causal=causal, approx=approx, mode="density",
                       density=0.4, sel=sel)
    return float((dout * r["out"]).sum())


@pytest.mark.parametrize("case", CASES)
def test_gradients_match_finite_differences(case):
    B, Hq, Hkv, N, d, block, causal, approx = case
    q, k, v = random_qkv(B, Hq, Hkv, N, d, seed=21, block=block)
    q, k, v = (np.asarray(x, np.float64) for x in (q, k, v))
    rng = np.random.default_rng(5)
    dout = rng.standard_normal(q.shape)
    sel = _selection(q, k, v, block, causal, approx)
    if approx:
        # the case must exercise pooled pseudo-keys
        assert (~sel & oracle.eligible_mask(sel.shape[-1], causal)).any()
    g = oracle.backward(q, k, v, dout, sel, block=block, causal=causal, approx=approx)
    h = 1e-6
    for name, x in (("dq", q), ("dk", k), ("dv", v)):
        flat = x.reshape(-1)
        picks = rng.choice(flat.size, size=min(flat.size, 48), replace=False)
        for p in picks:
            keep = flat[p]
            flat[p] = keep + h
            lp = _loss(q, k, v, dout, sel, block, causal, approx)
            flat[p] = keep - h
            lm = _loss(q, k, v, dout, sel, block, causal, approx)
            flat[p] = keep
            fd = (lp - lm) / (2 * h)
            an = g[name].reshape(-1)[p]
            assert abs(fd - an) <= 1e-6 * (1 + abs(fd)), (name, p, fd, an)


@pytest.mark.parametrize("causal", [False, True])
def test_density_one_gradients_equal_dense_autograd(causal):
    """Every eligible block exact: the gradients of dense softmax attention
    (torch autograd, float64, key/value heads repeated for the query heads)."""
    B, Hq, Hkv, N, d, block = 1, 4, 2, 90, 8, 32
    q, k, v = random_qkv(B, Hq, Hkv, N, d, seed=22, block=block)
    q, k, v = (np.asarray(x, np.float64) for x in (q, k, v))
    dout = np.random.default_rng(6).standard_normal(q.shape)
    M = -(-N // block)
    sel = np.broadcast_to(oracle.eligible_mask(M, causal), (B, Hq, M, M)).copy()
    g = oracle.backward(q, k, v, dout, sel, block=block, causal=causal, approx=True)

    G = Hq // Hkv
    qt = torch.from_numpy(q).requires_grad_()
    kt = torch.from_numpy(k).requires_grad_()
    vt = torch.from_numpy(v).requires_grad_()
    out = torch.nn.functional.scaled_dot_product_attention(
        qt, kt.repeat_interleave(G, 1), vt.repeat_interleave(G, 1), is_causal=causal)
    out.backward(torch.from_numpy(dout))
    np.testing.assert_allclose(g["dq"], qt.grad.numpy(), atol=1e-11, rtol=0)
    np.testing.assert_allclose(g["dk"], kt.grad.numpy(), atol=1e-11, rtol=0)
    np.testing.assert_allclose(g["dv"], vt.grad.numpy(), atol=1e-11, rtol=0)


def test_tail_only_gradient_spreads_evenly_over_block_tokens():
    """A key block reached only through its pooled key gets the same dk and
    dv on every one of its tokens (the mean spreads the gradient evenly)."""
    B, Hq, Hkv, N, d, block = 1, 1, 1, 48, 4, 16
    q, k, v = random_qkv(B, Hq, Hkv, N, d, seed=23, block=block)
    q, k, v = (np.asarray(x, np.float64) for x in (q, k, v))
    dout = np.random.default_rng(7).standard_normal(q.shape)
    sel = np.zeros((1, 1, 3, 3), bool)
    sel[..., 0] = True                      # every query block attends block 0 exactly
    g = oracle.backward(q, k, v, dout, sel, block=block, causal=False, approx=True)
    for J in (1, 2):
        rows = slice(J * block, (J + 1) * block)
        assert np.allclose(g["dk"][0, 0, rows], g["dk"][0, 0, J * block])
        assert np.allclose(g["dv"][0, 0, rows], g["dv"][0, 0, J * block])
    assert not np.allclose(g["dk"][0, 0, 0], g["dk"][0, 0, 1])


@pytest.mark.parametrize("causal", [False, True])
def test_lse_at_density_one_is_dense_logsumexp(causal):
    """The forward's log-denominator at density 1 is torch's logsumexp of the
    dense scaled scores (causally masked)."""
    B, Hq, Hkv, N, d, block = 1, 2, 1, 70, 8, 16
    q, k, v = random_qkv(B, Hq, Hkv, N, d, seed=24, block=block)
    r = oracle.forward(q, k, v, block=block, causal=causal, approx=True, mode="density", density=1.0)
    qt = torch.from_numpy(np.asarray(q, np.float64))
    kt = torch.from_numpy(np.asarray(k, np.float64)).repeat_interleave(2, 1)
    z = qt @ kt.transpose(-1, -2) / np.sqrt(d)
    if causal:
        z = z.masked_fill(torch.triu(torch.ones(N, N, dtype=torch.bool), 1), float("-inf"))
    np.testing.assert_allclose(r["lse"], torch.logsumexp(z, -1).numpy(), atol=1e-12, rtol=0)


def test_lse_with_tail_counts_block_multiplicity():
    """Identical keys inside every block: the tail is exact, so the
    log-denominator equals the dense one for any selection."""
    B, Hq, Hkv, N, d, block = 1, 1, 1, 48, 4, 16
    q, k, v = random_qkv(B, Hq, Hkv, N, d, seed=25, block=block)
    k = np.repeat(np.asarray(k, np.float64)[:, :, ::block], block, axis=2)[:, :, :N]
    sel = np.zeros((1, 1, 3, 3), bool)
    sel[..., 1] = True
    r = oracle.forward(q, k, v, block=block, causal=False, approx=True, mode="density", sel=sel)
    z = np.asarray(q, np.float64)[0, 0] @ k[0, 0].T / np.sqrt(d)
    ref = np.log(np.exp(z).sum(-1))
    np.testing.assert_allclose(r["lse"][0, 0], ref, atol=1e-12, rtol=0)


@pytest.mark.parametrize("causal,approx", [(True, True), (False, True), (True, False)])
def test_gradient_identities(causal, approx):
    """Two identities of softmax attention that hold for any selection: the
    value gradients of a KV head's tokens sum to the sum of dO over the query
    heads reading it (every row's weights, pooled blocks with their
    multiplicity included, sum to one), and the key gradients sum to zero
    (every row of dS sums to zero).  A dropped 1/n_J spread or a lost tail
    term breaks both."""
    B, Hq, Hkv, N, d, block = 1, 4, 2, 200, 8, 16
    q, k, v = random_qkv(B, Hq, Hkv, N, d, seed=26, block=block)
    q, k, v = (np.asarray(x, np.float64) for x in (q, k, v))
    dout = np.random.default_rng(8).standard_normal(q.shape)
    sel = _selection(q, k, v, block, causal, approx)
    g = oracle.backward(q, k, v, dout, sel, block=block, causal=causal, approx=approx)
    G = Hq // Hkv
    for gg in range(Hkv):
        np.testing.assert_allclose(g["dv"][0, gg].sum(0), dout[0, gg * G:(gg + 1) * G].sum((0, 1)),
                                   atol=1e-12, rtol=0)
        np.testing.assert_allclose(g["dk"][0, gg].sum(0), 0.0, atol=1e-12)
