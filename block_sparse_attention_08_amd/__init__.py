"""Block-sparse attention with pooled block routing for AMD MI355X (gfx950).

Python face of the C ABI in ``include/sparse_attn.h``.  Every step of the
computation runs in the HIP kernels of ``libsparse_attn.so``; this module only
checks tensors, marshals pointers and passes torch's current HIP stream.
torch supplies device memory and streams.

    out = block_sparse_attention(q, k, v, block_size=64, density=0.15)
    out = block_sparse_attention(q, k, v, block_size=128, alpha=0.5, causal=True,
                                 approx=False)

q: [B, Hq, N, d], k/v: [B, Hkv, N, d], contiguous, bfloat16 or float32, on
the GPU.  The three stages are also exposed one by one (``block_pool``,
``select``, ``fwd``) with caller-owned buffers from ``Workspace``; ``route``
runs the first two in one launch.
"""

from __future__ import annotations

import math
from typing import Optional

from . import _lib
from ._lib import SA_DTYPE_BF16, SA_DTYPE_F32, SA_SELECT_ALPHA, SA_SELECT_DENSITY, SaDesc, SparseAttnError

__all__ = [
    "Workspace", "block_pool", "block_sparse_attention", "buffer_sizes", "fwd", "make_desc",
    "route", "select", "SparseAttnError", "abi_version", "fwd_lse", "bwd_buffer_sizes",
    "BwdWorkspace", "bwd", "bwd_noalloc", "bwd_noalloc_scratch", "check_lists",
]


def abi_version() -> int:
    return int(_lib.lib().sparse_attn_abi_version())


def make_desc(B: int, Hq: int, Hkv: int, N: int, d: int, *, block: int, dtype: str,
              alpha: Optional[float] = None, density: Optional[float] = None,
              causal: bool = False, approx: bool = True, scale: Optional[float] = None) -> SaDesc:
    """Descriptor for one problem; exactly one of ``alpha`` / ``density``."""
    if (alpha is None) == (density is None):
        raise ValueError("give exactly one of alpha (threshold) or density (top-k)")
    if dtype not in ("bf16", "f32"):
        raise ValueError(f"dtype must be 'bf16' or 'f32', not {dtype!r}")
    return SaDesc(
        batch=B, heads_q=Hq, heads_kv=Hkv, seq_len=N, head_dim=d, block=block,
        dtype=SA_DTYPE_BF16 if dtype == "bf16" else SA_DTYPE_F32,
        select_mode=SA_SELECT_ALPHA if alpha is not None else SA_SELECT_DENSITY,
        alpha=float(alpha or 0.0), density=float(density or 0.0),
        scale=float(scale) if scale is not None else 0.0,
        causal=int(bool(causal)), approx=int(bool(approx)))


def buffer_sizes(desc: SaDesc) -> dict:
    """Bytes of each intermediate buffer (host-only call)."""
    s = _lib.SaSizes()
    _lib.check(_lib.lib().sparse_attn_buffer_sizes(desc, s), "sparse_attn_buffer_sizes")
    return {n: int(getattr(s, n)) for n, _ in s._fields_}


def _stream(stream):
    import torch
    if stream is None:
        stream = torch.cuda.current_stream()
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)


def _ptr(t):
    return None if t is None else t.data_ptr()


def _m(desc: SaDesc) -> int:
    return -(-desc.seq_len // desc.block)


class Workspace:
    """Caller-owned intermediates for one descriptor: pooled Q/K (float32),
    V sums (float32, when the tail is on), the bf16 tail operands (block
    means of K and V, bf16 inputs with the tail on), block lists and counts
    (int32)."""

    def __init__(self, desc: SaDesc, device="cuda"):
        import torch
        sizes = buffer_sizes(desc)
        B, Hq, Hkv, d, M = desc.batch, desc.heads_q, desc.heads_kv, desc.head_dim, _m(desc)
        f32, i32 = torch.float32, torch.int32
        self.desc = desc
        self.q_bar = torch.empty((B, Hq, M, d), dtype=f32, device=device)
        self.k_bar = torch.empty((B, Hkv, M, d), dtype=f32, device=device)
        self.v_sum = torch.empty((B, Hkv, M, d), dtype=f32, device=device) if desc.approx else None
        self.tail = (torch.empty((2, B, Hkv, M, d), dtype=torch.bfloat16, device=device)
                     if sizes["tail"] else None)
        self.blk_idx = torch.empty((B, Hq, M, M), dtype=i32, device=device)
        self.blk_cnt = torch.empty((B, Hq, M), dtype=i32, device=device)
        assert self.q_bar.numel() * 4 == sizes["q_bar"] and self.blk_idx.numel() * 4 == sizes["blk_idx"]


def block_pool(desc, q, k, v, q_bar, k_bar, v_sum, tail=None, stream=None) -> None:
    """Stage 1: block means of q and k, block sums of v (v_sum when approx),
    and the bf16 tail operands (bf16 inputs with approx)."""
    st = _lib.lib().sparse_attn_block_pool(desc, _ptr(q), _ptr(k), _ptr(v), _ptr(q_bar),
                                           _ptr(k_bar), _ptr(v_sum), _ptr(tail), _stream(stream))
    _lib.check(st, "sparse_attn_block_pool")


def select(desc, q_bar, k_bar, blk_idx, blk_cnt, stream=None) -> None:
    """Stage 2: pooled scores, threshold / top-k selection, ascending block lists."""
    st = _lib.lib().sparse_attn_select(desc, _ptr(q_bar), _ptr(k_bar), _ptr(blk_idx),
                                       _ptr(blk_cnt), _stream(stream))
    _lib.check(st, "sparse_attn_select")


def route(desc, q, k, v, q_bar, k_bar, v_sum, tail, blk_idx, blk_cnt, stream=None) -> None:
    """Stages 1 + 2 in one cooperative launch (fused routing): writes what
    ``block_pool`` then ``select`` write."""
    st = _lib.lib().sparse_attn_route(desc, _ptr(q), _ptr(k), _ptr(v), _ptr(q_bar), _ptr(k_bar),
                                      _ptr(v_sum), _ptr(tail), _ptr(blk_idx), _ptr(blk_cnt),
                                      _stream(stream))
    _lib.check(st, "sparse_attn_route")


def check_lists(desc, blk_idx, blk_cnt, stream=None) -> dict:
    """Validate block lists on the device (``sparse_attn_check_lists``) and
    wait for the result: ``{"ok", "flags" (names of the violations), "bad_rows",
    "first_bad_row"}``."""
    import torch
    res = torch.empty(4, dtype=torch.int32, device=blk_idx.device)
    st = _lib.lib().sparse_attn_check_lists(desc, _ptr(blk_idx), _ptr(blk_cnt), _ptr(res), _stream(stream))
    _lib.check(st, "sparse_attn_check_lists")
    if stream is None:
        torch.cuda.current_stream(blk_idx.device).synchronize()
    else:
        stream.synchronize()
    flags, bad, first = (int(x) & 0xFFFFFFFF for x in res[:3].cpu().tolist())
    return {"ok": flags == 0, "flags": [n for b, n in _lib.LIST_FLAGS.items() if flags & b],
            "bad_rows": bad, "first_bad_row": None if bad == 0 else first}


def fwd(desc, q, k, v, k_bar, v_sum, tail, blk_idx, blk_cnt, out, stream=None, check=False) -> None:
    """Stage 3: attention over the listed blocks (+ 0th-order tail when
    approx: k_bar/v_sum for float32 inputs, tail for bf16 inputs).  With
    ``check`` the lists are validated on the device first (``check_lists``,
    which waits for the stream) and a bad list raises ValueError before the
    attention is launched."""
    if check:
        r = check_lists(desc, blk_idx, blk_cnt, stream)
        if not r["ok"]:
            raise ValueError(f"invalid block lists: {r['flags']} in {r['bad_rows']} rows "
                             f"(first row {r['first_bad_row']})")
    st = _lib.lib().sparse_attn_fwd(desc, _ptr(q), _ptr(k), _ptr(v), _ptr(k_bar), _ptr(v_sum),
                                    _ptr(tail), _ptr(blk_idx), _ptr(blk_cnt), _ptr(out),
                                    _stream(stream))
    _lib.check(st, "sparse_attn_fwd")


def fwd_lse(desc, q, k, v, k_bar, v_sum, tail, blk_idx, blk_cnt, out, lse, stream=None) -> None:
    """Stage 3 that also writes ``lse`` [B, Hq, N] float32 (log of each row's
    softmax denominator), for the backward."""
    st = _lib.lib().sparse_attn_fwd_lse(desc, _ptr(q), _ptr(k), _ptr(v), _ptr(k_bar), _ptr(v_sum),
                                        _ptr(tail), _ptr(blk_idx), _ptr(blk_cnt), _ptr(out), _ptr(lse),
                                        _stream(stream))
    _lib.check(st, "sparse_attn_fwd_lse")


def bwd_buffer_sizes(desc: SaDesc) -> dict:
    """Bytes of each backward buffer (host-only call)."""
    s = _lib.SaBwdSizes()
    _lib.check(_lib.lib().sparse_attn_bwd_buffer_sizes(desc, s), "sparse_attn_bwd_buffer_sizes")
    return {n: int(getattr(s, n)) for n, _ in s._fields_}


class BwdWorkspace:
    """Caller-owned buffers of the backward: lse (from ``fwd_lse``) and the
    scratch of ``bwd``."""

    def __init__(self, desc: SaDesc, device="cuda"):
        import torch
        sz = bwd_buffer_sizes(desc)
        B, Hq, Hkv, N, d, M = desc.batch, desc.heads_q, desc.heads_kv, desc.seq_len, desc.head_dim, _m(desc)
        f32, i32 = torch.float32, torch.int32
        W = -(-M // 32)
        self.lse = torch.empty((B, Hq, N), dtype=f32, device=device)
        self.delta = torch.empty(sz["delta"] // 4, dtype=f32, device=device)
        self.sel_bits = torch.empty((B, Hq, M, W), dtype=i32, device=device)
        self.col_idx = torch.empty(sz["col_idx"] // 4, dtype=i32, device=device)
        self.col_cnt = torch.empty((B, Hkv, M), dtype=i32, device=device)
        self.dk_bar = torch.empty(sz["dk_bar"] // 4, dtype=f32, device=device) if sz["dk_bar"] else None
        self.dv_bar = torch.empty(sz["dv_bar"] // 4, dtype=f32, device=device) if sz["dv_bar"] else None
        assert self.sel_bits.numel() * 4 == sz["sel_bits"] and self.lse.numel() * 4 == sz["lse"]


def bwd(desc, q, k, v, tail, blk_idx, blk_cnt, out, dout, bws: BwdWorkspace, dq, dk, dv,
        stream=None) -> None:
    """Gradients dq, dk, dv (bf16) of sum(dout * out) for the lists the
    forward used; ``out`` and ``bws.lse`` come from ``fwd_lse``."""
    st = _lib.lib().sparse_attn_bwd(desc, _ptr(q), _ptr(k), _ptr(v), _ptr(tail), _ptr(blk_idx),
                                    _ptr(blk_cnt), _ptr(out), _ptr(bws.lse), _ptr(dout), _ptr(bws.delta),
                                    _ptr(bws.sel_bits), _ptr(bws.col_idx), _ptr(bws.col_cnt),
                                    _ptr(bws.dk_bar), _ptr(bws.dv_bar), _ptr(dq), _ptr(dk), _ptr(dv),
                                    _stream(stream))
    _lib.check(st, "sparse_attn_bwd")


def bwd_noalloc_scratch(desc: SaDesc) -> tuple:
    """(bytes of scratch ``bwd_noalloc`` needs for ``desc``, bytes the
    library's fixed scratch array holds); host-only call."""
    import ctypes
    need, cap = ctypes.c_size_t(0), ctypes.c_size_t(0)
    _lib.check(_lib.lib().sparse_attn_bwd_noalloc_scratch(desc, ctypes.byref(need), ctypes.byref(cap)),
               "sparse_attn_bwd_noalloc_scratch")
    return int(need.value), int(cap.value)


def bwd_noalloc(desc, q, k, v, tail, blk_idx, blk_cnt, out, lse, dout, dq, dk, dv, stream=None) -> None:
    """``bwd`` without caller scratch: the library's fixed per-device scratch
    array stands in for the ``BwdWorkspace`` buffers (for callers that cannot
    allocate).  Calls that overlap on one device race on that array."""
    st = _lib.lib().sparse_attn_bwd_noalloc(desc, _ptr(q), _ptr(k), _ptr(v), _ptr(tail), _ptr(blk_idx),
                                            _ptr(blk_cnt), _ptr(out), _ptr(lse), _ptr(dout), _ptr(dq),
                                            _ptr(dk), _ptr(dv), _stream(stream))
    _lib.check(st, "sparse_attn_bwd_noalloc")


def _check_tensors(q, k, v):
    import torch
    for name, t in (("q", q), ("k", k), ("v", v)):
        if not t.is_cuda:
            raise ValueError(f"{name} must be a GPU tensor")
        if not t.is_contiguous():
            raise ValueError(f"{name} must be contiguous [B, H, N, d]")
        if t.dim() != 4:
            raise ValueError(f"{name} must be 4-D [B, H, N, d]")
    if not (q.dtype == k.dtype == v.dtype) or q.dtype not in (torch.bfloat16, torch.float32):
        raise ValueError("q, k, v must share dtype bfloat16 or float32")
    if k.shape != v.shape or q.shape[0] != k.shape[0] or q.shape[2:] != k.shape[2:]:
        raise ValueError(f"shape mismatch: q {tuple(q.shape)}, k {tuple(k.shape)}, v {tuple(v.shape)}")


def block_sparse_attention(q, k, v, *, block_size: int = 64, alpha: Optional[float] = None,
                           density: Optional[float] = None, causal: bool = False,
                           approx: bool = True, scale: Optional[float] = None,
                           return_selection: bool = False, workspace: Optional[Workspace] = None,
                           out=None):
    """Pool -> select -> attend.  Returns ``out`` (dtype of q), or
    ``(out, blk_idx, blk_cnt)`` with ``return_selection``."""
    import torch
    _check_tensors(q, k, v)
    B, Hq, N, d = q.shape
    Hkv = k.shape[1]
    dt = "bf16" if q.dtype == torch.bfloat16 else "f32"
    if workspace is not None and alpha is None and density is None:
        # the selection rule is the one the workspace was built for
        wd = workspace.desc
        alpha, density = (wd.alpha, None) if wd.select_mode == SA_SELECT_ALPHA else (None, wd.density)
    desc = make_desc(B, Hq, Hkv, N, d, block=block_size, dtype=dt, alpha=alpha, density=density,
                     causal=causal, approx=approx, scale=scale)
    if workspace is None:
        buffer_sizes(desc)   # validates before any allocation
        workspace = Workspace(desc, device=q.device)
    ws = workspace
    if ws.q_bar.device != q.device:
        raise ValueError("workspace is on another device")
    bad = [name for name, _ in SaDesc._fields_ if getattr(ws.desc, name) != getattr(desc, name)]
    if bad:
        raise ValueError(f"workspace was built for another problem (differs in {', '.join(bad)})")
    if out is None:
        out = torch.empty_like(q)
    elif (out.shape != q.shape or out.dtype != q.dtype or out.device != q.device
          or not out.is_contiguous()):
        raise ValueError("out must be a contiguous tensor of q's shape, dtype and device")
    block_pool(desc, q, k, v, ws.q_bar, ws.k_bar, ws.v_sum, ws.tail)
    select(desc, ws.q_bar, ws.k_bar, ws.blk_idx, ws.blk_cnt)
    fwd(desc, q, k, v, ws.k_bar, ws.v_sum, ws.tail, ws.blk_idx, ws.blk_cnt, out)
    if return_selection:
        return out, ws.blk_idx, ws.blk_cnt
    return out


def default_scale(d: int) -> float:
    return 1.0 / math.sqrt(d)
