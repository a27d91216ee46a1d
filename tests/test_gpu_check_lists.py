"""sparse_attn_check_lists (through the C ABI): lists written by
sparse_attn_select pass; corrupted caller lists are reported with the flag
of each violation, the number of bad rows and the lowest bad row; the
Python fwd(check=True) refuses them before launching the attention."""

import numpy as np
import pytest

import oracle
from gpu_helpers import say, to_dev
from synth import random_qkv

pytestmark = pytest.mark.gpu


def _setup(causal, approx, N=1000, block=64, Hq=2):
    import torch
    import block_sparse_attention_08_amd as bsa
    q, k, v = random_qkv(1, Hq, 1, N, 64, seed=21, block=block, dtype="bf16")
    desc = bsa.make_desc(1, Hq, 1, N, 64, block=block, dtype="bf16", alpha=0.5, causal=causal, approx=approx)
    qd, kd, vd = (to_dev(x, "bf16") for x in (q, k, v))
    ws = bsa.Workspace(desc)
    bsa.block_pool(desc, qd, kd, vd, ws.q_bar, ws.k_bar, ws.v_sum, ws.tail)
    bsa.select(desc, ws.q_bar, ws.k_bar, ws.blk_idx, ws.blk_cnt)
    torch.cuda.synchronize()
    return desc, (qd, kd, vd), ws


@pytest.mark.parametrize("causal,approx", [(False, True), (True, False), (True, True)])
def test_selected_lists_pass(causal, approx):
    import block_sparse_attention_08_amd as bsa
    desc, _, ws = _setup(causal, approx)
    r = bsa.check_lists(desc, ws.blk_idx, ws.blk_cnt)
    say("select's lists", causal, approx, r)
    assert r["ok"] and r["bad_rows"] == 0 and r["first_bad_row"] is None


def _corrupt(idx, cnt, M, kind, row):
    """Apply one corruption to row `row` (b=0, h, I) of host copies."""
    b, h, I = row
    c = int(cnt[b, h, I])
    if kind == "range_high":
        idx[b, h, I, c - 1] = M + 5
    elif kind == "range_negative":
        idx[b, h, I, 0] = -3
    elif kind == "duplicate":
        assert c >= 2
        idx[b, h, I, 1] = idx[b, h, I, 0]
    elif kind == "count_zero":
        cnt[b, h, I] = 0
    elif kind == "count_too_big":
        cnt[b, h, I] = M + 7
    elif kind == "ineligible":
        idx[b, h, I, :2] = [I, I + 1]
        cnt[b, h, I] = 2
    elif kind == "no_diagonal":
        idx[b, h, I, :2] = [0, 1]
        cnt[b, h, I] = 2
    else:
        raise ValueError(kind)


CASES = [  # (kind, causal, approx, expected flag)
    ("range_high", False, True, "range"),
    ("range_negative", False, True, "range"),
    ("duplicate", False, False, "order"),
    ("count_zero", False, True, "count"),
    ("count_too_big", False, True, "count"),
    ("ineligible", True, False, "ineligible"),
    ("no_diagonal", True, True, "no_diagonal"),
]


@pytest.mark.parametrize("kind,causal,approx,flag", CASES, ids=[c[0] for c in CASES])
def test_corrupted_lists_are_reported(kind, causal, approx, flag):
    import torch
    import block_sparse_attention_08_amd as bsa
    say("corrupted lists", kind)
    desc, (qd, kd, vd), ws = _setup(causal, approx)
    M = ws.blk_cnt.shape[-1]
    # dense lists (every eligible block) so every row has room to corrupt
    sel = np.broadcast_to(oracle.eligible_mask(M, causal), tuple(ws.blk_cnt.shape) + (M,))
    idx, cnt = oracle.mask_to_lists(sel)
    rows = [(0, 1, M - 3), (0, 0, M - 1)]
    for row in rows:
        _corrupt(idx, cnt, M, kind, row)
    idx_d, cnt_d = torch.from_numpy(idx).cuda(), torch.from_numpy(cnt).cuda()
    r = bsa.check_lists(desc, idx_d, cnt_d)
    say("  ", r)
    assert not r["ok"]
    assert flag in r["flags"]
    assert r["bad_rows"] == 2
    assert r["first_bad_row"] == min((h * M + I) for (_, h, I) in rows)
    out = torch.full_like(qd, float("nan"))
    with pytest.raises(ValueError, match="invalid block lists"):
        bsa.fwd(desc, qd, kd, vd, ws.k_bar, ws.v_sum, ws.tail, idx_d, cnt_d, out, check=True)
    torch.cuda.synchronize()
    assert bool(torch.isnan(out).all()), "the attention ran on refused lists"
