"""GPU parity of the gradients (sparse_attn_fwd_lse + sparse_attn_bwd, through
the C ABI) against the oracle's float64 gradients, for the oracle's own
selection fed to both sides.

Tolerance: the kernels round P and dS to bfloat16 (relative 2^-9) before the
products and accumulate in float32, and the tail uses bf16 block means; the
errors stay near 1% of the largest gradient entry.  A gradient entry is
accepted within 2e-2 * max|ref| (per tensor) -- an error of that size is
well below what a wrong term (a missing 1/n_J, a dropped tail, a sign)
produces, since each of those changes entries by tens of percent of the
largest one."""

import numpy as np
import pytest

import oracle
from gpu_helpers import say, to_dev, to_host
from synth import random_qkv

pytestmark = pytest.mark.gpu

REL = 2e-2

# (B, Hq, Hkv, N, d, block, causal, approx, mode)
CASES = [
    (1, 2, 2, 1000, 128, 64, False, True, "density"),    # ragged 15*64 + 40, tail
    (1, 4, 2, 1300, 128, 128, True, False, "alpha"),     # GQA, causal, ragged
    (1, 2, 1, 700, 64, 64, True, True, "alpha"),         # d = 64, causal + tail, GQA
    (1, 2, 2, 2600, 128, 128, True, True, "alpha"),      # 128-row blocks, causal + tail
    (2, 2, 2, 640, 128, 64, False, False, "density"),
    (1, 2, 2, 300, 64, 128, False, True, "density"),     # d = 64, 128-row blocks, tail
    (2, 4, 2, 700, 128, 128, True, True, "alpha"),       # batch 2, GQA, 128-row blocks (two-group dq pass)
    (1, 4, 2, 1400, 64, 128, True, True, "alpha"),       # d = 64 two-group dq pass, causal + tail, GQA, 10*128 + 120
]


def _ids(c):
    return "B{}_H{}x{}_N{}_d{}_b{}_{}_{}_{}".format(
        c[0], c[1], c[2], c[3], c[4], c[5], "causal" if c[6] else "full", "tail" if c[7] else "notail", c[8])


def run_train(q, k, v, dout, *, block, causal, approx, mode, sel, alpha=0.5, density=0.2):
    import torch
    import block_sparse_attention_08_amd as bsa
    B, Hq, N, d = q.shape
    Hkv = k.shape[1]
    desc = bsa.make_desc(B, Hq, Hkv, N, d, block=block, dtype="bf16",
                         alpha=alpha if mode == "alpha" else None,
                         density=density if mode == "density" else None, causal=causal, approx=approx)
    qd, kd, vd, gd = (to_dev(x, "bf16") for x in (q, k, v, dout))
    ws = bsa.Workspace(desc)
    bws = bsa.BwdWorkspace(desc)
    bsa.block_pool(desc, qd, kd, vd, ws.q_bar, ws.k_bar, ws.v_sum, ws.tail)
    idx, cnt = oracle.mask_to_lists(sel)
    idx_d, cnt_d = torch.from_numpy(idx).cuda(), torch.from_numpy(cnt).cuda()
    out = torch.empty_like(qd)
    bsa.fwd_lse(desc, qd, kd, vd, ws.k_bar, ws.v_sum, ws.tail, idx_d, cnt_d, out, bws.lse)
    dq, dk, dv = torch.empty_like(qd), torch.empty_like(kd), torch.empty_like(vd)
    bsa.bwd(desc, qd, kd, vd, ws.tail, idx_d, cnt_d, out, gd, bws, dq, dk, dv)
    torch.cuda.synchronize()
    return dict(out=to_host(out), lse=to_host(bws.lse), dq=to_host(dq), dk=to_host(dk), dv=to_host(dv))


@pytest.mark.parametrize("case", CASES, ids=_ids)
def test_gradients_against_oracle(case):
    B, Hq, Hkv, N, d, block, causal, approx, mode = case
    say("case", _ids(case))
    q, k, v = random_qkv(B, Hq, Hkv, N, d, seed=31, block=block, dtype="bf16", kind="cluster", noise=0.5)
    dout = random_qkv(B, Hq, Hq, N, d, seed=32, block=block, dtype="bf16")[0]
    ref = oracle.forward(q, k, v, block=block, causal=causal, approx=approx, mode=mode, alpha=0.5,
                         density=0.2)
    if approx:
        assert (~ref["mask"] & oracle.eligible_mask(ref["mask"].shape[-1], causal)).any()
    g = run_train(q, k, v, dout, block=block, causal=causal, approx=approx, mode=mode, sel=ref["mask"])
    assert np.abs(g["out"] - ref["out"]).max() <= 2e-2
    assert np.abs(g["lse"] - ref["lse"]).max() <= 2e-3 * (1 + np.abs(ref["lse"]).max())
    gr = oracle.backward(q, k, v, dout, ref["mask"], block=block, causal=causal, approx=approx)
    for name in ("dq", "dk", "dv"):
        err = np.abs(g[name] - gr[name]).max()
        top = np.abs(gr[name]).max()
        say(f"  {name}: max-abs err {err:.3e}, max |ref| {top:.3e}, ratio {err / top:.2e}")
        assert err <= REL * top, name


def test_dense_lists_match_torch_autograd():
    """Every causal block listed (dense causal attention): the gradients equal
    torch's float64 autograd of dense attention on the same bf16 inputs."""
    import torch
    B, Hq, Hkv, N, d, block = 1, 4, 2, 900, 128, 128
    say("dense causal vs autograd")
    q, k, v = random_qkv(B, Hq, Hkv, N, d, seed=33, block=block, dtype="bf16")
    dout = random_qkv(B, Hq, Hq, N, d, seed=34, block=block, dtype="bf16")[0]
    M = -(-N // block)
    sel = np.broadcast_to(oracle.eligible_mask(M, True), (B, Hq, M, M)).copy()
    g = run_train(q, k, v, dout, block=block, causal=True, approx=False, mode="alpha", sel=sel)
    qt = torch.from_numpy(np.asarray(q, np.float64)).requires_grad_()
    kt = torch.from_numpy(np.asarray(k, np.float64)).requires_grad_()
    vt = torch.from_numpy(np.asarray(v, np.float64)).requires_grad_()
    o = torch.nn.functional.scaled_dot_product_attention(
        qt, kt.repeat_interleave(2, 1), vt.repeat_interleave(2, 1), is_causal=True)
    o.backward(torch.from_numpy(np.asarray(dout, np.float64)))
    for name, ref in (("dq", qt.grad), ("dk", kt.grad), ("dv", vt.grad)):
        r = ref.numpy()
        err = np.abs(g[name] - r).max()
        say(f"  {name}: max-abs err {err:.3e}, max |ref| {np.abs(r).max():.3e}")
        assert err <= REL * np.abs(r).max(), name
