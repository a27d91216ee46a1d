"""Parity at the workloads' full sizes, in the launch configuration the bench
times (pool -> select -> fwd over every head at once), through the C ABI.

Selection is compared for every head and query block (bit-exact outside the
1e-5 near-threshold band); pooled statistics on sampled heads.  The output
tensor starts as NaN and must come back finite everywhere (every row
written).  Outputs are compared with the oracle's, computed on the oracle's
own selection, for one whole query head plus a seeded sample of query
blocks of the other heads (the tiny float32 workload in full); query blocks
whose GPU selection differs from the oracle's inside the band are skipped
and counted.  The 256K workload's dense comparison (every causal block
listed, up to 2048 blocks = 4096 key tiles per row) is checked on its last
query blocks."""

import functools

import numpy as np
import pytest

import oracle
from gpu_helpers import TOL_OUT, TOL_POOL_REL, say, to_host
from synth import CONFIGS, get_config, make_inputs

pytestmark = pytest.mark.gpu


@functools.lru_cache(maxsize=1)
def _inputs(name):
    return make_inputs(get_config(name), seed=0)


def _run_full(wl, q, k, v):
    import torch
    import block_sparse_attention_08_amd as bsa
    dt = torch.bfloat16 if wl.dtype == "bf16" else torch.float32
    qd, kd, vd = (torch.from_numpy(x).to(dt).cuda() for x in (q, k, v))
    desc = bsa.make_desc(wl.B, wl.Hq, wl.Hkv, wl.N, wl.d, block=wl.block, dtype=wl.dtype,
                         alpha=wl.alpha if wl.select == "alpha" else None,
                         density=wl.density if wl.select == "density" else None,
                         causal=wl.causal, approx=wl.approx)
    ws = bsa.Workspace(desc)
    out = torch.full_like(qd, float("nan"))
    bsa.block_pool(desc, qd, kd, vd, ws.q_bar, ws.k_bar, ws.v_sum, ws.tail)
    bsa.select(desc, ws.q_bar, ws.k_bar, ws.blk_idx, ws.blk_cnt)
    bsa.fwd(desc, qd, kd, vd, ws.k_bar, ws.v_sum, ws.tail, ws.blk_idx, ws.blk_cnt, out)
    torch.cuda.synchronize()
    n_bad = int((~torch.isfinite(out)).sum())
    assert n_bad == 0, f"{n_bad} output elements not written or not finite"
    cnt = to_host(ws.blk_cnt)
    idx = to_host(ws.blk_idx)
    mask = np.zeros(idx.shape, dtype=bool)
    for pos in np.ndindex(*cnt.shape):
        c = int(cnt[pos])
        assert 1 <= c <= wl.M, (pos, c)
        row = idx[pos][:c]
        assert np.all(np.diff(row) > 0) and row[0] >= 0 and row[-1] < wl.M, (pos, row[:8])
        mask[pos + (row,)] = True
    return dict(mask=mask, out=out, q_bar=ws.q_bar, k_bar=ws.k_bar, v_sum=ws.v_sum)


# the 256K workload last, so the dense test after it reuses its cached inputs
_ORDER = [c for c in CONFIGS if c.name != "llm_prefill_256k"] + [get_config("llm_prefill_256k")]


@pytest.mark.parametrize("wl", _ORDER, ids=[c.name for c in _ORDER])
def test_full_size_workload(wl):
    say(f"workload {wl.name}: generating inputs")
    q, k, v = _inputs(wl.name)
    say("  running the HIP path")
    g = _run_full(wl, q, k, v)
    rng = np.random.default_rng(1234)
    M = wl.M
    if wl.name == "dit_tiny_f32":
        rows = None
    else:
        # one whole query head (every query block), plus sampled blocks of others
        h_all = int(rng.integers(wl.Hq))
        picks = {(0, h_all, I) for I in range(M)} | {(0, 0, 0), (0, wl.Hq - 1, M - 1)}
        while len(picks) < M + 8:
            picks.add((0, int(rng.integers(wl.Hq)), int(rng.integers(M))))
        rows = sorted(picks)
        say(f"  whole head {h_all} ({M} query blocks) + {len(picks) - M} sampled blocks")
    say("  oracle: pool, score, select (all heads), attend (checked rows)")
    ref = oracle.forward(q, k, v, block=wl.block, causal=wl.causal, approx=wl.approx,
                         mode=wl.select, alpha=wl.alpha, density=wl.density, rows=rows)

    # selection, every head
    band = oracle.band_mask(ref["scores"], ref["thresholds"], wl.causal)
    diff = g["mask"] != ref["mask"]
    bad = diff & ~band
    assert not bad.any(), f"{int(bad.sum())} mask mismatches outside the band"
    row_diff = diff.any(-1)
    say(f"  band blocks {int(band.sum())}, differing in band {int(diff.sum())}, "
        f"selected {int(ref['mask'].sum())} of {int(oracle.eligible_mask(M, wl.causal).sum()) * wl.Hq}")

    # pooled statistics on two heads
    for h in (0, wl.Hq - 1):
        gq = to_host(g["q_bar"][0, h])
        assert np.all(np.abs(gq - ref["q_bar"][0, h]) <= TOL_POOL_REL * (np.abs(ref["q_bar"][0, h]) + 1))
    for hk in (0, wl.Hkv - 1):
        gk = to_host(g["k_bar"][0, hk])
        assert np.all(np.abs(gk - ref["k_bar"][0, hk]) <= TOL_POOL_REL * (np.abs(ref["k_bar"][0, hk]) + 1))

    # outputs
    check = [(b, h, I) for b in range(wl.B) for h in range(wl.Hq) for I in range(M)] \
        if rows is None else rows
    worst = 0.0
    compared = 0
    bounds = oracle.block_bounds(wl.N, wl.block)
    for (b, h, I) in check:
        if row_diff[b, h, I]:
            continue
        s, e = bounds[I]
        go = to_host(g["out"][b, h, s:e])
        worst = max(worst, float(np.abs(go - ref["out"][b, h, s:e]).max()))
        compared += 1
    say(f"  outputs: {compared} of {len(check)} query blocks compared "
        f"({len(check) - compared} skipped: selection differs in the band), max-abs err {worst:.3e}")
    assert compared >= len(check) - max(1, len(check) // 100)
    assert worst <= TOL_OUT[wl.dtype]


def test_dense_lists_at_256k():
    """The 256K prefill with every causal block listed (the bench's dense
    comparison): rows of up to 2048 blocks, 4096 key tiles of the online
    softmax (FlashAttention tutorial, section 2).  The last query blocks of
    two heads against the oracle on the same dense selection; every output
    element written."""
    import torch
    import block_sparse_attention_08_amd as bsa
    wl = get_config("llm_prefill_256k")
    say("dense lists at 256K: generating inputs")
    q, k, v = _inputs(wl.name)
    M = wl.M
    desc = bsa.make_desc(wl.B, wl.Hq, wl.Hkv, wl.N, wl.d, block=wl.block, dtype=wl.dtype, alpha=wl.alpha,
                         causal=True, approx=False)
    qd, kd, vd = (torch.from_numpy(x).to(torch.bfloat16).cuda() for x in (q, k, v))
    idx = torch.arange(M, dtype=torch.int32, device="cuda").expand(wl.B, wl.Hq, M, M).contiguous()
    cnt = torch.arange(1, M + 1, dtype=torch.int32, device="cuda").expand(wl.B, wl.Hq, M).contiguous()
    out = torch.full_like(qd, float("nan"))
    say("  running the dense forward")
    bsa.fwd(desc, qd, kd, vd, None, None, None, idx, cnt, out)
    torch.cuda.synchronize()
    assert bool(torch.isfinite(out).all()), "dense output has unwritten or non-finite elements"
    rows = [(0, h, I) for h in (0, wl.Hq - 1) for I in (M - 2, M - 1)]
    sel = np.broadcast_to(oracle.eligible_mask(M, True), (wl.B, wl.Hq, M, M))
    say("  oracle on the last query blocks of heads 0 and 7")
    ref = oracle.forward(q, k, v, block=wl.block, causal=True, approx=False, mode="alpha", alpha=wl.alpha,
                         rows=rows, sel=sel)
    worst = 0.0
    for (b, h, I) in rows:
        s, e = I * wl.block, (I + 1) * wl.block
        go = to_host(out[b, h, s:e])
        worst = max(worst, float(np.abs(go - ref["out"][b, h, s:e]).max()))
    say(f"  dense rows of 2047-2048 blocks: max-abs err {worst:.3e}")
    assert worst <= TOL_OUT["bf16"]


@pytest.mark.parametrize("causal,mode,Hq,Hkv", [(False, "density", 2, 2), (True, "alpha", 4, 2)],
                         ids=["topk_full", "alpha_causal_gqa"])
def test_tail_at_2048_blocks(causal, mode, Hq, Hkv):
    """The largest row the library takes with 64-row blocks: N = 131072, M =
    2048 (`kMaxBlocks`), with the 0th-order tail, the clustered generator.
    Non-causal top-k at density 0.05 (k = 103, the 32-pass radix select over
    2048 keys per row; 1945 pooled rows, 61 tail tiles per query block), and
    causal alpha = 0.5 with grouped queries (the diagonal forced exact, the
    tail over the earlier blocks).  Lists on every row bit-exact outside the
    band; outputs of 16 sampled query blocks against the oracle on its own
    selection; every output element written."""
    import torch
    import block_sparse_attention_08_amd as bsa
    from synth import random_qkv
    B, N, d, block, density, alpha = 1, 131072, 128, 64, 0.05, 0.5
    H = Hq
    M = N // block
    say(f"2048 blocks of 64 rows, {mode}, causal={causal}, tail: generating inputs")
    q, k, v = random_qkv(B, Hq, Hkv, N, d, seed=31, block=block, dtype="bf16", kind="cluster", noise=0.5)
    desc = bsa.make_desc(B, Hq, Hkv, N, d, block=block, dtype="bf16",
                         density=density if mode == "density" else None,
                         alpha=alpha if mode == "alpha" else None, causal=causal, approx=True)
    qd, kd, vd = (torch.from_numpy(x).to(torch.bfloat16).cuda() for x in (q, k, v))
    ws = bsa.Workspace(desc)
    out = torch.full_like(qd, float("nan"))
    bsa.block_pool(desc, qd, kd, vd, ws.q_bar, ws.k_bar, ws.v_sum, ws.tail)
    bsa.select(desc, ws.q_bar, ws.k_bar, ws.blk_idx, ws.blk_cnt)
    bsa.fwd(desc, qd, kd, vd, ws.k_bar, ws.v_sum, ws.tail, ws.blk_idx, ws.blk_cnt, out)
    torch.cuda.synchronize()
    assert bool(torch.isfinite(out).all()), "output has unwritten or non-finite elements"
    cnt, idx = to_host(ws.blk_cnt), to_host(ws.blk_idx)
    if mode == "density":
        kk = int(np.ceil(density * M - 1e-9))
        assert np.all(cnt == kk), (int(cnt.min()), int(cnt.max()), kk)
    mask = np.zeros((B, H, M, M), dtype=bool)
    for pos in np.ndindex(*cnt.shape):
        mask[pos + (idx[pos][:int(cnt[pos])],)] = True
    rng = np.random.default_rng(7)
    rows = sorted({(0, int(rng.integers(H)), int(rng.integers(M))) for _ in range(14)} | {(0, 0, 0), (0, H - 1, M - 1)})
    say(f"  oracle: selection on every row, attention on {len(rows)} query blocks")
    ref = oracle.forward(q, k, v, block=block, causal=causal, approx=True, mode=mode, density=density,
                         alpha=alpha, rows=rows)
    band = oracle.band_mask(ref["scores"], ref["thresholds"], causal)
    diff = mask != ref["mask"]
    assert not (diff & ~band).any(), f"{int((diff & ~band).sum())} mask mismatches outside the band"
    row_diff = diff.any(-1)
    worst, compared = 0.0, 0
    for (b, h, I) in rows:
        if row_diff[b, h, I]:
            continue
        s, e = I * block, (I + 1) * block
        worst = max(worst, float(np.abs(to_host(out[b, h, s:e]) - ref["out"][b, h, s:e]).max()))
        compared += 1
    say(f"  band blocks {int(band.sum())}; {compared} of {len(rows)} query blocks compared, max-abs {worst:.3e}")
    assert compared >= len(rows) - 1
    assert worst <= TOL_OUT["bf16"]
