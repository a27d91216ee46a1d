"""The kernels write their outputs and nothing else.

Each output tensor (out; dq, dk, dv) is a view into a larger buffer whose
guard region after the tensor holds a sentinel value.  After a call through
the C ABI the guard must be untouched and every output element must be
finite.  Shapes have a ragged last block and several heads, so the last
wave of the last block of the last head has rows past the end of the
sequence: the store paths that move whole rows (staged through LDS) must
stop at the sequence end.  One case per forward kernel: the 16-row bf16
kernel (64-row blocks, M < 384), the 32-row kernel with 128-row blocks and
with 64-row blocks (M >= 384), and the float32 kernel."""

import numpy as np
import pytest

from gpu_helpers import say, to_dev
from synth import random_qkv

pytestmark = pytest.mark.gpu

GUARD = 4096          # elements after each output
SENTINEL = -7.5       # exact in bf16 and f32, never produced by a softmax average here


def _guarded(shape, dtype):
    """(view, buffer): a contiguous view of `shape` at the start of a buffer
    with GUARD extra elements, all filled with NaN (view) / SENTINEL (guard)."""
    import torch
    n = int(np.prod(shape))
    buf = torch.full((n + GUARD,), SENTINEL, dtype=dtype, device="cuda")
    buf[:n] = float("nan")
    return buf[:n].view(shape), buf


def _check(name, view, buf):
    import torch
    n = view.numel()
    guard_ok = bool(torch.all(buf[n:] == SENTINEL).item())
    finite = bool(torch.isfinite(view).all().item())
    say(f"  {name}: guard intact {guard_ok}, all finite {finite}")
    assert guard_ok, f"{name}: a kernel wrote past the end of the tensor"
    assert finite, f"{name}: unwritten or non-finite elements"


# (B, Hq, Hkv, N, d, block, dtype, causal, approx, mode)
FWD_CASES = [
    (2, 3, 3, 1000, 128, 64, "bf16", False, True, "density"),      # 16-row kernel, 15*64 + 40
    (1, 4, 2, 1300, 128, 128, "bf16", True, False, "alpha"),       # 32-row kernel, 10*128 + 20
    (1, 2, 2, 24616, 128, 64, "bf16", False, True, "density"),     # 32-row kernel, 64-row blocks, M = 385
    (1, 3, 3, 777, 128, 64, "f32", True, True, "density"),
]


@pytest.mark.parametrize("case", FWD_CASES, ids=lambda c: f"N{c[3]}_b{c[5]}_{c[6]}")
def test_forward_writes_only_its_output(case):
    import torch
    import block_sparse_attention_08_amd as bsa
    B, Hq, Hkv, N, d, block, dtype, causal, approx, mode = case
    q, k, v = random_qkv(B, Hq, Hkv, N, d, seed=21, block=block, dtype=dtype, kind="cluster", noise=0.5)
    desc = bsa.make_desc(B, Hq, Hkv, N, d, block=block, dtype=dtype,
                         alpha=0.5 if mode == "alpha" else None,
                         density=0.2 if mode == "density" else None, causal=causal, approx=approx)
    qd, kd, vd = (to_dev(x, dtype) for x in (q, k, v))
    ws = bsa.Workspace(desc)
    bsa.block_pool(desc, qd, kd, vd, ws.q_bar, ws.k_bar, ws.v_sum, ws.tail)
    bsa.select(desc, ws.q_bar, ws.k_bar, ws.blk_idx, ws.blk_cnt)
    out, obuf = _guarded(tuple(qd.shape), qd.dtype)
    bsa.fwd(desc, qd, kd, vd, ws.k_bar, ws.v_sum, ws.tail, ws.blk_idx, ws.blk_cnt, out)
    torch.cuda.synchronize()
    _check("out", out, obuf)


# (B, Hq, Hkv, N, d, block, causal, approx, mode)
BWD_CASES = [
    (2, 2, 2, 1000, 128, 64, False, True, "density"),
    (1, 4, 2, 1300, 128, 128, True, True, "alpha"),
]


@pytest.mark.parametrize("case", BWD_CASES, ids=lambda c: f"N{c[3]}_b{c[5]}")
def test_backward_writes_only_its_gradients(case):
    import torch
    import block_sparse_attention_08_amd as bsa
    B, Hq, Hkv, N, d, block, causal, approx, mode = case
    q, k, v = random_qkv(B, Hq, Hkv, N, d, seed=22, block=block, dtype="bf16", kind="cluster", noise=0.5)
    desc = bsa.make_desc(B, Hq, Hkv, N, d, block=block, dtype="bf16",
                         alpha=0.5 if mode == "alpha" else None,
                         density=0.2 if mode == "density" else None, causal=causal, approx=approx)
    qd, kd, vd = (to_dev(x, "bf16") for x in (q, k, v))
    g = torch.Generator(device="cuda")
    g.manual_seed(5)
    dout = torch.randn(qd.shape, device="cuda", generator=g).to(torch.bfloat16)
    ws = bsa.Workspace(desc)
    bws = bsa.BwdWorkspace(desc)
    bsa.block_pool(desc, qd, kd, vd, ws.q_bar, ws.k_bar, ws.v_sum, ws.tail)
    bsa.select(desc, ws.q_bar, ws.k_bar, ws.blk_idx, ws.blk_cnt)
    out = torch.empty_like(qd)
    bsa.fwd_lse(desc, qd, kd, vd, ws.k_bar, ws.v_sum, ws.tail, ws.blk_idx, ws.blk_cnt, out, bws.lse)
    dq, qbuf = _guarded(tuple(qd.shape), torch.bfloat16)
    dk, kbuf = _guarded(tuple(kd.shape), torch.bfloat16)
    dv, vbuf = _guarded(tuple(vd.shape), torch.bfloat16)
    bsa.bwd(desc, qd, kd, vd, ws.tail, ws.blk_idx, ws.blk_cnt, out, dout, bws, dq, dk, dv)
    torch.cuda.synchronize()
    _check("dq", dq, qbuf)
    _check("dk", dk, kbuf)
    _check("dv", dv, vbuf)
