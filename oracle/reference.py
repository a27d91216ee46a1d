"""Oracle steps, one function per step of the method (float64 numpy).

TEST INFRASTRUCTURE ONLY: see the package docstring.

Notation: tokens are cut into M = ceil(N/b) contiguous blocks of b tokens; the
last block may hold fewer (n_J tokens).  Q is [B,Hq,N,d], K and V are
[B,Hkv,N,d]; Q head h reads KV head g(h) = floor(h / (Hq/Hkv)).
"""

from __future__ import annotations

import math
from typing import Dict, List, Optional, Sequence, Tuple

import numpy as np


# --------------------------------------------------------------------------
# step 1: partition into contiguous token blocks
#   PISA explainer, section "what PISA changes" (tokens are grouped into
#   contiguous blocks) and the O(N log N) section (M = N/B blocks).
# --------------------------------------------------------------------------

def block_bounds(N: int, block: int) -> List[Tuple[int, int]]:
    """[start, stop) of every block; the last block is cut at N."""
    M = -(-N // block)
    return [(J * block, min(N, (J + 1) * block)) for J in range(M)]


def block_sizes(N: int, block: int) -> np.ndarray:
    """n_J, the number of real tokens in block J (float64)."""
    return np.array([e - s for s, e in block_bounds(N, block)], dtype=np.float64)


def kv_group(h: int, Hq: int, Hkv: int) -> int:
    """KV head read by Q head h: consecutive Q heads share one KV head."""
    return h // (Hq // Hkv)


# --------------------------------------------------------------------------
# step 2: block representatives
#   PISA explainer, "how candidate blocks are narrowed": per block a Q and K
#   representative and a V *sum*; routing table: unselected blocks are
#   approximated with the block-mean key and the value sum.
#   FlashPrefill summary, section 2(a) "block approximation": keys are
#   average-pooled per block.
# --------------------------------------------------------------------------

def pool_mean(x: np.ndarray, block: int) -> np.ndarray:
    """Mean over the real tokens of each block: [..., N, d] -> [..., M, d]."""
    N = x.shape[-2]
    out = [np.asarray(x[..., s:e, :], dtype=np.float64).mean(axis=-2)
           for s, e in block_bounds(N, block)]
    return np.stack(out, axis=-2)


def pool_sum(x: np.ndarray, block: int) -> np.ndarray:
    """Sum over the tokens of each block: [..., N, d] -> [..., M, d]."""
    N = x.shape[-2]
    out = [np.asarray(x[..., s:e, :], dtype=np.float64).sum(axis=-2)
           for s, e in block_bounds(N, block)]
    return np.stack(out, axis=-2)


# --------------------------------------------------------------------------
# step 3: pooled block scores
#   PISA explainer, "how candidate blocks are narrowed" (score per query
#   block); FlashPrefill summary 2(a)/2(b): Score_{I,J} from pooled vectors.
#   Reading: Score is the scaled pooled logit scale * qbar_I . kbar_J.
# --------------------------------------------------------------------------

def block_scores(q_bar: np.ndarray, k_bar: np.ndarray, scale: float) -> np.ndarray:
    """s[b,h,I,J] = scale * qbar[b,h,I] . kbar[b,g(h),J]  ->  [B,Hq,M,M] float64."""
    B, Hq, M, d = q_bar.shape
    Hkv = k_bar.shape[1]
    s = np.empty((B, Hq, M, M), dtype=np.float64)
    for b in range(B):
        for h in range(Hq):
            g = kv_group(h, Hq, Hkv)
            s[b, h] = scale * (q_bar[b, h].astype(np.float64) @ k_bar[b, g].astype(np.float64).T)
    return s


def eligible_mask(M: int, causal: bool) -> np.ndarray:
    """E[I,J]: key block J may be attended by query block I (J <= I if causal)."""
    if causal:
        return np.tril(np.ones((M, M), dtype=bool))
    return np.ones((M, M), dtype=bool)


# --------------------------------------------------------------------------
# step 4: block selection
# --------------------------------------------------------------------------

def select_alpha(s: np.ndarray, elig: np.ndarray, alpha: float) -> np.ndarray:
    """Max-based dynamic threshold, FlashPrefill summary 2(b):
    thresh_I = alpha * max_J Score_{I,J}; keep J with Score_{I,J} >= thresh_I.

    Row maxima that are not positive would put alpha*max above the max; then
    the threshold is the max itself (only the arg-max blocks are kept).
    """
    sm = np.where(elig, s, -np.inf)
    m = sm.max(axis=-1, keepdims=True)
    t = np.where(m > 0, alpha * m, m)
    return elig & (s >= t)


def topk_count(n_elig: int, density: float) -> int:
    """Exact blocks kept per query block at a density (PISA explainer: the
    density argument of the documented call ties to the exact-path share).

    k = ceil(density * |E_I|) evaluated in float64 with a 1e-9 guard against
    representation error (0.15*100 -> 15, not 16), clamped to [1, |E_I|].
    """
    k = math.ceil(float(density) * n_elig - 1e-9)
    return int(min(n_elig, max(1, k)))


def select_density(s: np.ndarray, elig: np.ndarray, density: float) -> np.ndarray:
    """Top-k of the eligible scores of each query-block row, k from
    ``topk_count``; higher score first, equal scores -> lower block index."""
    sel = np.zeros(s.shape, dtype=bool)
    lead = s.shape[:-2]
    M = s.shape[-1]
    for idx in np.ndindex(*lead):
        for I in range(M):
            cand = np.nonzero(elig[I])[0]
            k = topk_count(len(cand), density)
            order = np.lexsort((cand, -s[idx + (I,)][cand]))   # primary: -score, then J
            sel[idx + (I, cand[order[:k]])] = True
    return sel


def select(s: np.ndarray, *, causal: bool, approx: bool, mode: str,
           alpha: float = 0.5, density: float = 0.15) -> np.ndarray:
    """Selected-block mask [.., M, M].  With causal attention and the tail on,
    the diagonal block is always exact: its pooled key would mix in keys later
    than the query token."""
    M = s.shape[-1]
    elig = eligible_mask(M, causal)
    if mode == "alpha":
        sel = select_alpha(s, elig, alpha)
    elif mode == "density":
        sel = select_density(s, elig, density)
    else:
        raise ValueError(mode)
    if causal and approx:
        sel = sel | np.eye(M, dtype=bool)
    return sel


def thresholds(s: np.ndarray, *, causal: bool, mode: str, alpha: float = 0.5,
               density: float = 0.15) -> np.ndarray:
    """The per-row threshold t_I separating kept from dropped blocks ([.., M]).

    alpha mode: alpha * max (or the max when it is not positive).  density
    mode: the midpoint between the k-th and (k+1)-th largest eligible scores,
    so that only a close pair straddling the cut is near it; -inf when every
    eligible block is kept."""
    M = s.shape[-1]
    elig = eligible_mask(M, causal)
    sm = np.where(elig, s, -np.inf)
    if mode == "alpha":
        m = sm.max(axis=-1)
        return np.where(m > 0, alpha * m, m)
    t = np.empty(s.shape[:-1])
    for idx in np.ndindex(*s.shape[:-1]):
        row = np.sort(sm[idx][np.isfinite(sm[idx])])[::-1]
        k = topk_count(len(row), density)
        t[idx] = 0.5 * (row[k - 1] + row[k]) if k < len(row) else -np.inf
    return t


def band_mask(s: np.ndarray, t: np.ndarray, causal: bool, rel: float = 1e-5) -> np.ndarray:
    """Eligible (I,J) whose score lies within ``rel`` of the threshold.  When
    |t| is tiny next to the row's scores, the band is rel * max_J |s_IJ|."""
    M = s.shape[-1]
    elig = eligible_mask(M, causal)
    amax = np.where(elig, np.abs(s), 0.0).max(axis=-1)
    with np.errstate(invalid="ignore"):
        width = np.where(np.abs(t) < 1e-3 * amax, rel * amax, rel * np.abs(t))
        near = np.abs(s - t[..., None]) <= width[..., None]
    return elig & np.isfinite(t)[..., None] & near


def mask_to_lists(sel: np.ndarray) -> Tuple[np.ndarray, np.ndarray]:
    """Ascending selected-block lists: idx [.., M, M] int32 (first cnt valid,
    rest -1) and cnt [.., M] int32."""
    M = sel.shape[-1]
    cnt = sel.sum(axis=-1).astype(np.int32)
    idx = np.full(sel.shape, -1, dtype=np.int32)
    for pos in np.ndindex(*sel.shape[:-1]):
        j = np.nonzero(sel[pos])[0]
        idx[pos + (slice(0, len(j)),)] = j
    return idx, cnt


# --------------------------------------------------------------------------
# step 5: attention over exact blocks plus the 0th-order tail
#   FlashAttention tutorial section 2 (online softmax): the running max / sum
#   recurrence produces exactly the full softmax; this oracle evaluates the
#   full (closed-form) softmax directly.
#   PISA explainer, routing table and "why softmax survives": selected blocks
#   use their original K/V tokens; each unselected block J enters the *same*
#   normaliser as one pseudo-key kbar_J of multiplicity n_J carrying the value
#   sum SigmaV_J, i.e. weight n_J*exp(q.kbar_J) in the denominator and
#   exp(q.kbar_J)*SigmaV_J in the numerator.
# --------------------------------------------------------------------------

def attend_block(q_rows: np.ndarray, row0: int, k: np.ndarray, v: np.ndarray,
                 k_bar: Optional[np.ndarray], v_sum: Optional[np.ndarray],
                 sel_row: np.ndarray, elig_row: np.ndarray, *, block: int, scale: float,
                 causal: bool, approx: bool, with_lse: bool = False):
    """Output rows for one (batch, head, query block).

    q_rows [nI, d] are the block's query tokens (token index row0 + r);
    k, v [N, d] the KV head; k_bar, v_sum [M, d] its pooled key / value sum.
    Returns [nI, d] float64 (and, with ``with_lse``, the natural log of each
    row's denominator, [nI]).
    """
    N = k.shape[0]
    nI = q_rows.shape[0]
    qf = np.asarray(q_rows, dtype=np.float64)
    bounds = block_bounds(N, block)
    S = [J for J in range(len(bounds)) if sel_row[J]]
    keys = np.concatenate([np.arange(*bounds[J]) for J in S]) if S else np.zeros(0, int)

    z = scale * (qf @ np.asarray(k[keys], dtype=np.float64).T)           # [nI, |X|]
    if causal:
        tok = row0 + np.arange(nI)
        z = np.where(keys[None, :] <= tok[:, None], z, -np.inf)

    if approx:
        T = [J for J in range(len(bounds)) if elig_row[J] and not sel_row[J]]
        n = np.array([bounds[J][1] - bounds[J][0] for J in T], dtype=np.float64)
        zt = scale * (qf @ np.asarray(k_bar[T], dtype=np.float64).T) if T else np.zeros((nI, 0))
        vt = np.asarray(v_sum[T], dtype=np.float64) if T else np.zeros((0, qf.shape[1]))
    else:
        n = np.zeros(0)
        zt = np.zeros((nI, 0))
        vt = np.zeros((0, qf.shape[1]))

    m = np.maximum(z.max(axis=1, initial=-np.inf), zt.max(axis=1, initial=-np.inf))
    m = np.where(np.isfinite(m), m, 0.0)
    e = np.exp(z - m[:, None])
    et = np.exp(zt - m[:, None])
    num = e @ np.asarray(v[keys], dtype=np.float64) + et @ vt
    den = e.sum(axis=1) + et @ n
    out = np.zeros_like(num)
    ok = den > 0
    out[ok] = num[ok] / den[ok, None]
    if with_lse:
        with np.errstate(divide="ignore"):
            return out, m + np.log(den)
    return out


# --------------------------------------------------------------------------
# the whole path
# --------------------------------------------------------------------------

def forward(q: np.ndarray, k: np.ndarray, v: np.ndarray, *, block: int, causal: bool,
            approx: bool, mode: str, alpha: float = 0.5, density: float = 0.15,
            scale: Optional[float] = None,
            rows: Optional[Sequence[Tuple[int, int, int]]] = None,
            sel: Optional[np.ndarray] = None) -> Dict[str, np.ndarray]:
    """Run pool -> score -> select -> attend.

    q [B,Hq,N,d], k/v [B,Hkv,N,d].  ``rows``: optional list of (b, h, I)
    query blocks to attend (default: all); outputs of other rows stay NaN.
    ``sel``: optional selection mask [B,Hq,M,M] to use instead of the
    oracle's own (e.g. density 1 / dense lists).

    Returns a dict with q_bar, k_bar, v_sum, n, scores, mask, thresholds, out
    and lse (natural log of each query row's softmax denominator).
    """
    B, Hq, N, d = q.shape
    Hkv = k.shape[1]
    if Hq % Hkv:
        raise ValueError("Hq must be a multiple of Hkv")
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    M = -(-N // block)
    q_bar = pool_mean(q, block)
    k_bar = pool_mean(k, block)
    v_sum = pool_sum(v, block) if approx else None
    s = block_scores(q_bar, k_bar, scale)
    mask = select(s, causal=causal, approx=approx, mode=mode, alpha=alpha,
                  density=density) if sel is None else sel
    t = thresholds(s, causal=causal, mode=mode, alpha=alpha, density=density)
    elig = eligible_mask(M, causal)
    out = np.full((B, Hq, N, d), np.nan)
    lse = np.full((B, Hq, N), np.nan)
    todo = rows if rows is not None else [(b, h, I) for b in range(B) for h in range(Hq)
                                          for I in range(M)]
    bounds = block_bounds(N, block)
    for (b, h, I) in todo:
        g = kv_group(h, Hq, Hkv)
        r0, r1 = bounds[I]
        out[b, h, r0:r1], lse[b, h, r0:r1] = attend_block(
            q[b, h, r0:r1], r0, k[b, g], v[b, g],
            k_bar[b, g], None if v_sum is None else v_sum[b, g],
            mask[b, h, I], elig[I], block=block, scale=scale, causal=causal, approx=approx,
            with_lse=True)
    return dict(q_bar=q_bar, k_bar=k_bar, v_sum=v_sum, n=block_sizes(N, block), scores=s,
                mask=mask, thresholds=t, out=out, lse=lse)


# --------------------------------------------------------------------------
# gradients of the attention step (the training path of the 0th-order form)
#   PISA explainer, "minimal documented usage": the simplified 0th-order
#   variant is the one meant for training, so gradients flow through the
#   exact blocks and through the pooled pseudo-keys of the tail.  The block
#   selection is piecewise constant in the inputs and passes no gradient;
#   the selection mask is an input here.
#
#   With P_ia the softmax weight of key a (exact token j: exp(z_ij)/den;
#   pooled block J: n_J exp(z_iJ)/den) and u_a its value (v_j, or the block
#   mean SigmaV_J / n_J), o_i = sum_a P_ia u_a and, for a loss with gradient
#   dO at o:
#     dz_ia = P_ia (dO_i . u_a - dO_i . o_i)
#     dq_i  = scale sum_a dz_ia key_a            (key: k_j or kbar_J)
#     dk_j += scale dz_ij q_i,  dv_j += P_ij dO_i            (exact keys)
#     dkbar_J = scale sum_i dz_iJ q_i, du_J = sum_i P_iJ dO_i  (pooled)
#   and the block means hand dkbar_J / n_J and du_J / n_J to every token of
#   block J.
# --------------------------------------------------------------------------

def attend_block_grad(q_rows: np.ndarray, row0: int, dout_rows: np.ndarray, k: np.ndarray,
                      v: np.ndarray, sel_row: np.ndarray, elig_row: np.ndarray, *, block: int,
                      scale: float, causal: bool, approx: bool):
    """Gradients from one (batch, head, query block): returns (dq_rows
    [nI, d], dk [N, d], dv [N, d]) with dk, dv of the KV head (exact keys
    and the tokens under each pooled block), float64."""
    N, d = k.shape
    nI = q_rows.shape[0]
    qf = np.asarray(q_rows, dtype=np.float64)
    go = np.asarray(dout_rows, dtype=np.float64)
    kf = np.asarray(k, dtype=np.float64)
    vf = np.asarray(v, dtype=np.float64)
    bounds = block_bounds(N, block)
    S = [J for J in range(len(bounds)) if sel_row[J]]
    keys = np.concatenate([np.arange(*bounds[J]) for J in S]) if S else np.zeros(0, int)
    T = [J for J in range(len(bounds)) if approx and elig_row[J] and not sel_row[J]]
    n = np.array([bounds[J][1] - bounds[J][0] for J in T], dtype=np.float64)
    kbar = np.stack([kf[slice(*bounds[J])].mean(axis=0) for J in T]) if T else np.zeros((0, d))
    ubar = np.stack([vf[slice(*bounds[J])].mean(axis=0) for J in T]) if T else np.zeros((0, d))

    z = scale * (qf @ kf[keys].T)
    if causal:
        tok = row0 + np.arange(nI)
        z = np.where(keys[None, :] <= tok[:, None], z, -np.inf)
    zt = scale * (qf @ kbar.T) + np.log(n)[None, :] if T else np.zeros((nI, 0))
    m = np.maximum(z.max(axis=1, initial=-np.inf), zt.max(axis=1, initial=-np.inf))
    m = np.where(np.isfinite(m), m, 0.0)
    e = np.exp(z - m[:, None])
    et = np.exp(zt - m[:, None])
    den = e.sum(axis=1) + et.sum(axis=1)
    den = np.where(den > 0, den, 1.0)
    P = e / den[:, None]                  # exact weights
    Pt = et / den[:, None]                # pooled weights (multiplicity included)
    o = P @ vf[keys] + Pt @ ubar
    Dlt = (go * o).sum(axis=1)
    dz = P * (go @ vf[keys].T - Dlt[:, None])
    dzt = Pt * (go @ ubar.T - Dlt[:, None])

    dq = scale * (dz @ kf[keys] + dzt @ kbar)
    dk = np.zeros((N, d))
    dv = np.zeros((N, d))
    np.add.at(dk, keys, scale * (dz.T @ qf))
    np.add.at(dv, keys, P.T @ go)
    dkbar = scale * (dzt.T @ qf)
    dubar = Pt.T @ go
    for t, J in enumerate(T):
        s0, s1 = bounds[J]
        dk[s0:s1] += dkbar[t] / n[t]
        dv[s0:s1] += dubar[t] / n[t]
    return dq, dk, dv


def backward(q: np.ndarray, k: np.ndarray, v: np.ndarray, dout: np.ndarray, sel: np.ndarray, *,
             block: int, causal: bool, approx: bool,
             scale: Optional[float] = None) -> Dict[str, np.ndarray]:
    """Gradients (dq [B,Hq,N,d], dk, dv [B,Hkv,N,d], float64) of
    sum(dout * forward(...)["out"]) for the fixed selection mask ``sel``
    [B,Hq,M,M].  Query heads of one KV group add into its dk, dv."""
    B, Hq, N, d = q.shape
    Hkv = k.shape[1]
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    M = -(-N // block)
    elig = eligible_mask(M, causal)
    bounds = block_bounds(N, block)
    dq = np.zeros((B, Hq, N, d))
    dk = np.zeros((B, Hkv, N, d))
    dv = np.zeros((B, Hkv, N, d))
    for b in range(B):
        for h in range(Hq):
            g = kv_group(h, Hq, Hkv)
            for I in range(M):
                r0, r1 = bounds[I]
                gq, gk, gv = attend_block_grad(q[b, h, r0:r1], r0, dout[b, h, r0:r1], k[b, g], v[b, g],
                                               sel[b, h, I], elig[I], block=block, scale=scale,
                                               causal=causal, approx=approx)
                dq[b, h, r0:r1] = gq
                dk[b, g] += gk
                dv[b, g] += gv
    return dict(dq=dq, dk=dk, dv=dv)
