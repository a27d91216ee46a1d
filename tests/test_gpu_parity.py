"""GPU parity of the HIP path (through the C ABI) against the CPU oracle.

Each stage is checked on its own -- pooled statistics, selected-block lists
(bit-exact outside the 1e-5 near-threshold band), and the attention output
with the oracle's own lists fed to the kernel (max-abs 1e-4 for float32,
2e-2 for bfloat16) -- and then end to end.  Shapes span several tiles and a
ragged last block; edge cases cover single partial blocks, grouped queries,
alpha=1, density=1 (dense), causal with the tail, caller-supplied lists,
determinism and stream ordering."""

import numpy as np
import pytest

import oracle
from gpu_helpers import TOL_OUT, assert_pool, compare_masks, lists_to_mask, run_gpu, say, to_dev, to_host
from synth import random_qkv

pytestmark = pytest.mark.gpu

# (B, Hq, Hkv, N, d, block, dtype, causal, approx, mode)
CASES = [
    (1, 2, 2, 1000, 128, 64, "bf16", False, True, "density"),   # ragged: 15*64 + 40
    (1, 2, 2, 1000, 128, 64, "bf16", False, True, "alpha"),
    (1, 4, 2, 1300, 128, 128, "bf16", True, False, "alpha"),    # GQA, causal, 10*128 + 20
    (2, 2, 1, 700, 64, 64, "bf16", True, True, "alpha"),         # causal + tail (forced diagonal)
    (1, 4, 2, 2600, 128, 128, "bf16", True, True, "alpha"),     # causal + tail, 128-row blocks, GQA
    (1, 2, 2, 900, 64, 128, "bf16", False, False, "density"),
    # 64-row blocks with >= 384 blocks per row take the pipelined two-wave kernel
    (1, 2, 2, 24616, 128, 64, "bf16", False, True, "density"),   # M = 385, ragged 384*64 + 40
    (1, 2, 1, 24600, 64, 64, "bf16", True, True, "alpha"),       # d = 64, causal + tail, GQA
    (1, 2, 2, 640, 64, 64, "f32", False, True, "alpha"),
    (1, 2, 1, 555, 128, 128, "f32", True, False, "density"),
    (1, 3, 3, 777, 128, 64, "f32", True, True, "density"),
    (1, 2, 1, 1500, 64, 128, "bf16", True, True, "alpha"),      # d = 64, 128-row blocks, causal + tail, GQA, 11*128 + 92
    (1, 2, 2, 700, 64, 128, "f32", False, True, "alpha"),       # f32, 128-row blocks, tail, 5*128 + 60
    (1, 2, 1, 4100, 128, 64, "f32", True, True, "alpha"),       # f32, 65 blocks (64*64 + 4), causal + tail, GQA
]


def _ids(c):
    return "B{}_H{}x{}_N{}_d{}_b{}_{}_{}_{}_{}".format(
        c[0], c[1], c[2], c[3], c[4], c[5], c[6], "causal" if c[7] else "full",
        "tail" if c[8] else "notail", c[9])


def _inputs(c, seed=0, kind="cluster"):
    B, Hq, Hkv, N, d, block, dtype, causal, approx, mode = c
    return random_qkv(B, Hq, Hkv, N, d, seed=seed, block=block, dtype=dtype, kind=kind, noise=0.5)


@pytest.mark.parametrize("case", CASES, ids=_ids)
def test_stages_against_oracle(case):
    B, Hq, Hkv, N, d, block, dtype, causal, approx, mode = case
    say("case", _ids(case))
    q, k, v = _inputs(case)
    ref = oracle.forward(q, k, v, block=block, causal=causal, approx=approx, mode=mode,
                         alpha=0.5, density=0.2)
    # stage 3 on the oracle's own lists (no GPU selection involved)
    g = run_gpu(q, k, v, dtype=dtype, block=block, causal=causal, approx=approx, mode=mode,
                alpha=0.5, density=0.2, sel_mask=ref["mask"])
    assert_pool(g, ref, approx)
    band, ndiff, _ = compare_masks(g["mask"], ref, causal)
    err = np.abs(g["out"] - ref["out"]).max()
    say(f"  band={band} diff_in_band={ndiff} fwd max-abs err={err:.3e}")
    assert err <= TOL_OUT[dtype]


@pytest.mark.parametrize("case", CASES, ids=_ids)
def test_end_to_end(case):
    B, Hq, Hkv, N, d, block, dtype, causal, approx, mode = case
    say("case", _ids(case))
    q, k, v = _inputs(case, seed=1)
    ref = oracle.forward(q, k, v, block=block, causal=causal, approx=approx, mode=mode,
                         alpha=0.5, density=0.2)
    g = run_gpu(q, k, v, dtype=dtype, block=block, causal=causal, approx=approx, mode=mode,
                alpha=0.5, density=0.2)
    _, _, rows = compare_masks(g["mask"], ref, causal)
    # compare outputs of query blocks whose selection agrees
    ok = ~rows
    M = ok.shape[-1]
    bounds = oracle.block_bounds(N, block)
    worst = 0.0
    for b_, h, I in np.argwhere(ok):
        s, e = bounds[I]
        worst = max(worst, float(np.abs(g["out"][b_, h, s:e] - ref["out"][b_, h, s:e]).max()))
    say(f"  rows compared {int(ok.sum())}/{ok.size}, max-abs err {worst:.3e}")
    assert ok.sum() >= 0.9 * ok.size
    assert worst <= TOL_OUT[dtype]


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("causal", [False, True])
def test_density_one_is_dense(dtype, causal):
    """density=1 keeps every eligible block: dense softmax attention."""
    import torch
    say("dense", dtype, causal)
    q, k, v = random_qkv(1, 2, 1, 600, 128, seed=4, block=64, dtype=dtype)
    g = run_gpu(q, k, v, dtype=dtype, block=64, causal=causal, approx=True, mode="density",
                density=1.0)
    G = 2
    ref = torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(q).double(), torch.from_numpy(k).double().repeat_interleave(G, 1),
        torch.from_numpy(v).double().repeat_interleave(G, 1), is_causal=causal).numpy()
    assert np.array_equal(g["mask"], np.broadcast_to(oracle.eligible_mask(10, causal), g["mask"].shape))
    assert np.abs(g["out"] - ref).max() <= TOL_OUT[dtype]


@pytest.mark.parametrize("N,block", [(1, 64), (37, 64), (64, 64), (100, 128), (129, 128)])
def test_tiny_and_single_block(N, block):
    say("tiny", N, block)
    for dtype in ("bf16", "f32"):
        q, k, v = random_qkv(1, 2, 2, N, 64, seed=5, block=block, dtype=dtype)
        for causal, approx, mode in ((False, True, "alpha"), (True, True, "density"),
                                     (True, False, "alpha")):
            ref = oracle.forward(q, k, v, block=block, causal=causal, approx=approx, mode=mode)
            g = run_gpu(q, k, v, dtype=dtype, block=block, causal=causal, approx=approx, mode=mode)
            compare_masks(g["mask"], ref, causal)
            assert np.abs(g["out"] - ref["out"]).max() <= TOL_OUT[dtype]


def test_alpha_one_keeps_argmax_only():
    say("alpha=1")
    q, k, v = random_qkv(1, 2, 2, 1024, 128, seed=6, block=64, dtype="bf16")
    ref = oracle.forward(q, k, v, block=64, causal=False, approx=True, mode="alpha", alpha=1.0)
    g = run_gpu(q, k, v, dtype="bf16", block=64, causal=False, approx=True, mode="alpha", alpha=1.0)
    compare_masks(g["mask"], ref, False)
    assert np.all(g["cnt"] >= 1)
    assert np.abs(g["out"] - ref["out"]).max() <= TOL_OUT["bf16"]


def test_caller_lists_dense_causal():
    """fwd with caller-built lists holding every causal block equals dense causal attention."""
    import torch
    import block_sparse_attention_08_amd as bsa
    say("caller lists")
    N, block = 1000, 128
    q, k, v = random_qkv(1, 4, 2, N, 128, seed=7, block=block, dtype="bf16")
    M = -(-N // block)
    desc = bsa.make_desc(1, 4, 2, N, 128, block=block, dtype="bf16", alpha=0.5, causal=True,
                         approx=False)
    idx = np.full((1, 4, M, M), -1, np.int32)
    for I in range(M):
        idx[..., I, :I + 1] = np.arange(I + 1)
    cnt = np.broadcast_to(np.arange(1, M + 1, dtype=np.int32), (1, 4, M)).copy()
    qd, kd, vd = to_dev(q, "bf16"), to_dev(k, "bf16"), to_dev(v, "bf16")
    out = torch.empty_like(qd)
    bsa.fwd(desc, qd, kd, vd, None, None, None, torch.from_numpy(idx).cuda(), torch.from_numpy(cnt).cuda(), out)
    ref = torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(q).double(), torch.from_numpy(k).double().repeat_interleave(2, 1),
        torch.from_numpy(v).double().repeat_interleave(2, 1), is_causal=True).numpy()
    assert np.abs(to_host(out) - ref).max() <= TOL_OUT["bf16"]


def test_deterministic_and_stream_ordered():
    """Two runs on a side stream give bit-identical lists and outputs, ordered
    with torch work on that stream."""
    import torch
    import block_sparse_attention_08_amd as bsa
    say("determinism")
    q, k, v = random_qkv(1, 4, 4, 2048, 128, seed=8, block=64, dtype="bf16")
    qd, kd, vd = to_dev(q, "bf16"), to_dev(k, "bf16"), to_dev(v, "bf16")
    s = torch.cuda.Stream()
    outs = []
    with torch.cuda.stream(s):
        for _ in range(2):
            qq = qd * 1.0          # torch kernel on the side stream feeding the library
            o, idx, cnt = bsa.block_sparse_attention(qq, kd, vd, block_size=64, density=0.15,
                                                     return_selection=True)
            outs.append((o.clone(), idx.clone(), cnt.clone()))
    s.synchronize()
    o0, i0, c0 = outs[0]
    o1, i1, c1 = outs[1]
    assert torch.equal(c0, c1)
    for pos in np.ndindex(*c0.shape):
        c = int(c0[pos])
        assert torch.equal(i0[pos][:c], i1[pos][:c])
    assert torch.equal(o0, o1)


@pytest.mark.parametrize("N,dtype,causal", [(8192 + 17, "bf16", False), (24616, "bf16", False),
                                             (1000, "f32", False), (777, "f32", True)])
def test_lse_of_each_forward_kernel(N, dtype, causal):
    """fwd_lse through each forward kernel that serves 64-row blocks (the
    16-row bf16 kernel at M = 129, the pipelined one at M = 385, the float32
    one): out and lse against the oracle on its own lists."""
    import torch
    import block_sparse_attention_08_amd as bsa
    q, k, v = random_qkv(1, 2, 2, N, 128, seed=12, block=64, dtype=dtype, kind="cluster", noise=0.5)
    ref = oracle.forward(q, k, v, block=64, causal=causal, approx=True, mode="density", density=0.2)
    desc = bsa.make_desc(1, 2, 2, N, 128, block=64, dtype=dtype, density=0.2, approx=True, causal=causal)
    qd, kd, vd = (to_dev(x, dtype) for x in (q, k, v))
    ws = bsa.Workspace(desc)
    bsa.block_pool(desc, qd, kd, vd, ws.q_bar, ws.k_bar, ws.v_sum, ws.tail)
    idx, cnt = oracle.mask_to_lists(ref["mask"])
    out = torch.empty_like(qd)
    lse = torch.empty((1, 2, N), dtype=torch.float32, device="cuda")
    bsa.fwd_lse(desc, qd, kd, vd, ws.k_bar, ws.v_sum, ws.tail, torch.from_numpy(idx).cuda(),
                torch.from_numpy(cnt).cuda(), out, lse)
    torch.cuda.synchronize()
    err_o = np.abs(to_host(out) - ref["out"]).max()
    err_l = np.abs(to_host(lse) - ref["lse"]).max()
    say(f"  N={N} {dtype}: out err {err_o:.3e}, lse err {err_l:.3e}")
    assert err_o <= TOL_OUT[dtype]
    assert err_l <= (2e-3 if dtype == "bf16" else 1e-5) * (1 + np.abs(ref["lse"]).max())


def test_wrapper_rejects_mismatched_workspace_and_out():
    """The Python wrapper refuses a workspace built for another shape and an
    out tensor unlike q (the library itself only sees raw pointers)."""
    import torch
    import block_sparse_attention_08_amd as bsa
    q, k, v = random_qkv(1, 2, 2, 256, 64, seed=9, block=64, dtype="bf16")
    qd, kd, vd = (to_dev(x, "bf16") for x in (q, k, v))
    other = bsa.Workspace(bsa.make_desc(1, 2, 2, 512, 64, block=64, dtype="bf16", density=0.2))
    with pytest.raises(ValueError):
        bsa.block_sparse_attention(qd, kd, vd, density=0.2, workspace=other)
    with pytest.raises(ValueError):
        bsa.block_sparse_attention(qd, kd, vd, density=0.2,
                                   out=torch.empty((1, 2, 256, 32), dtype=torch.bfloat16, device="cuda"))
    ws = bsa.Workspace(bsa.make_desc(1, 2, 2, 256, 64, block=64, dtype="bf16", density=0.2))
    # a workspace carries its descriptor: any argument that contradicts it
    # (rule, threshold, block, causal, tail, scale) is refused, not ignored
    for kw in (dict(density=0.3), dict(alpha=0.5), dict(density=0.2, causal=True),
               dict(density=0.2, approx=False), dict(density=0.2, block_size=128),
               dict(density=0.2, scale=0.5)):
        with pytest.raises(ValueError, match="another problem"):
            bsa.block_sparse_attention(qd, kd, vd, workspace=ws, **kw)
    out = torch.empty_like(qd)
    o = bsa.block_sparse_attention(qd, kd, vd, density=0.2, workspace=ws, out=out)
    # without a rule argument the workspace's rule is used
    o2 = bsa.block_sparse_attention(qd, kd, vd, workspace=ws)
    torch.cuda.synchronize()
    assert torch.equal(o, o2)
    torch.cuda.synchronize()
    assert o.data_ptr() == out.data_ptr()
    gpu_mask = lists_to_mask(to_host(ws.blk_idx), to_host(ws.blk_cnt))
    assert (gpu_mask.sum(-1) == oracle.topk_count(4, 0.2)).all()
    ref = oracle.forward(q, k, v, block=64, causal=False, approx=True, mode="density", density=0.2,
                         sel=gpu_mask)
    assert np.abs(to_host(o) - ref["out"]).max() <= TOL_OUT["bf16"]


@pytest.mark.parametrize("N,block,causal,mode", [(4096 + 17, 64, False, "density"), (4096 + 100, 128, True, "alpha")])
def test_graph_capture_replays_match_eager(N, block, causal, mode):
    """pool -> select -> fwd captured in a HIP graph (torch.cuda.CUDAGraph):
    three replays, with eager work on the buffers in between, each give the
    eager run's lists and outputs bit for bit (the library records no memset
    or allocation, so the captured launches are the whole computation)."""
    import torch
    import block_sparse_attention_08_amd as bsa
    q, k, v = random_qkv(1, 4, 2, N, 128, seed=13, block=block, dtype="bf16", kind="cluster", noise=0.5)
    qd, kd, vd = (to_dev(x, "bf16") for x in (q, k, v))
    desc = bsa.make_desc(1, 4, 2, N, 128, block=block, dtype="bf16", alpha=0.5 if mode == "alpha" else None,
                         density=0.2 if mode == "density" else None, causal=causal, approx=True)
    ws = bsa.Workspace(desc)
    out = torch.empty_like(qd)

    def layer():
        bsa.block_pool(desc, qd, kd, vd, ws.q_bar, ws.k_bar, ws.v_sum, ws.tail)
        bsa.select(desc, ws.q_bar, ws.k_bar, ws.blk_idx, ws.blk_cnt)
        bsa.fwd(desc, qd, kd, vd, ws.k_bar, ws.v_sum, ws.tail, ws.blk_idx, ws.blk_cnt, out)

    layer()
    torch.cuda.synchronize()
    ref_out, ref_cnt, ref_idx = out.clone(), ws.blk_cnt.clone(), ws.blk_idx.clone()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        layer()
    torch.cuda.current_stream().wait_stream(side)
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        layer()
    cnt_h = to_host(ref_cnt)
    for rep in range(3):
        out.zero_()
        ws.blk_cnt.zero_()
        ws.k_bar.zero_()
        graph.replay()
        torch.cuda.synchronize()
        say(f"  replay {rep}")
        assert torch.equal(out, ref_out), rep
        assert torch.equal(ws.blk_cnt, ref_cnt), rep
        idx, ridx = to_host(ws.blk_idx), to_host(ref_idx)
        for pos in np.ndindex(*cnt_h.shape):
            c = int(cnt_h[pos])
            assert np.array_equal(idx[pos][:c], ridx[pos][:c]), (rep, pos)
