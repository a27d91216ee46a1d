"""Helpers for the GPU parity tests: upload seeded inputs, run the HIP path
through the C ABI, bring results back, and compare with the oracle."""

from __future__ import annotations

import sys

import numpy as np

import block_sparse_attention_08_amd as bsa
import oracle

# max-abs output tolerances (float32 and bfloat16 inputs)
TOL_OUT = {"f32": 1e-4, "bf16": 2e-2}
# pooled statistics: float32 sums of at most 128 exactly representable values
TOL_POOL_REL = 2e-6


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def to_dev(x: np.ndarray, dtype: str):
    import torch
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32))
    t = t.to(torch.bfloat16) if dtype == "bf16" else t   # values are bf16-exact: no rounding
    return t.cuda().contiguous()


def to_host(t) -> np.ndarray:
    import torch
    return t.detach().to(torch.float32).cpu().numpy() if t.is_floating_point() else t.cpu().numpy()


def lists_to_mask(idx: np.ndarray, cnt: np.ndarray) -> np.ndarray:
    M = idx.shape[-1]
    mask = np.zeros(idx.shape, dtype=bool)
    for pos in np.ndindex(*cnt.shape):
        c = int(cnt[pos])
        assert 1 <= c <= M, (pos, c)
        row = idx[pos][:c]
        assert np.all(np.diff(row) > 0), ("not strictly ascending", pos, row)
        assert row.min() >= 0 and row.max() < M, (pos, row)
        mask[pos + (row,)] = True
    return mask


def run_gpu(q, k, v, *, dtype, block, causal, approx, mode, alpha=0.5, density=0.15,
            scale=None, sel_mask=None):
    """Run pool -> select -> fwd on the GPU.  With ``sel_mask`` (oracle mask),
    those lists replace the GPU's own for the fwd stage."""
    import torch
    B, Hq, N, d = q.shape
    Hkv = k.shape[1]
    desc = bsa.make_desc(B, Hq, Hkv, N, d, block=block, dtype=dtype,
                         alpha=alpha if mode == "alpha" else None,
                         density=density if mode == "density" else None,
                         causal=causal, approx=approx, scale=scale)
    qd, kd, vd = to_dev(q, dtype), to_dev(k, dtype), to_dev(v, dtype)
    ws = bsa.Workspace(desc)
    out = torch.empty_like(qd)
    bsa.block_pool(desc, qd, kd, vd, ws.q_bar, ws.k_bar, ws.v_sum, ws.tail)
    bsa.select(desc, ws.q_bar, ws.k_bar, ws.blk_idx, ws.blk_cnt)
    if sel_mask is not None:
        idx, cnt = oracle.mask_to_lists(sel_mask)
        fidx = torch.from_numpy(idx).cuda()
        fcnt = torch.from_numpy(cnt).cuda()
    else:
        fidx, fcnt = ws.blk_idx, ws.blk_cnt
    bsa.fwd(desc, qd, kd, vd, ws.k_bar, ws.v_sum, ws.tail, fidx, fcnt, out)
    torch.cuda.synchronize()
    res = dict(q_bar=to_host(ws.q_bar), k_bar=to_host(ws.k_bar),
               v_sum=None if ws.v_sum is None else to_host(ws.v_sum),
               idx=to_host(ws.blk_idx), cnt=to_host(ws.blk_cnt), out=to_host(out))
    res["mask"] = lists_to_mask(res["idx"], res["cnt"])
    return res


def compare_masks(gpu_mask, ref, causal):
    """Masks must agree outside the near-threshold band; returns
    (#band blocks, #band blocks where they differ, rows that differ)."""
    band = oracle.band_mask(ref["scores"], ref["thresholds"], causal)
    diff = gpu_mask != ref["mask"]
    bad = diff & ~band
    assert not bad.any(), f"{int(bad.sum())} mask mismatches outside the band, first at " \
                          f"{np.argwhere(bad)[:5].tolist()}"
    rows = diff.any(axis=-1)
    return int(band.sum()), int(diff.sum()), rows


def assert_pool(gpu, ref, approx):
    for name in ("q_bar", "k_bar") + (("v_sum",) if approx else ()):
        g, r = gpu[name], ref[name]
        err = np.abs(g - r)
        lim = TOL_POOL_REL * (np.abs(r) + 1.0) * (128 if name == "v_sum" else 1)
        assert np.all(err <= lim), f"{name}: max err {err.max():.3e}"
