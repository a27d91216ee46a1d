"""Host logic of bench.py (no GPU): the work counts the bench line divides
by, the LDS operand bytes it reports, and the source hash that decides
whether a committed counter summary still describes the kernel."""

import os
import shutil

import numpy as np
import pytest

import bench


def test_work_units_dense_causal_is_the_triangle():
    # N = 100 in blocks of 64 (the last one 36 tokens), every causal block
    # listed: the allowed pairs are the N (N + 1) / 2 of the causal triangle
    N, block, M = 100, 64, 2
    cnt = np.array([[[1, 2]]], dtype=np.int32)
    idx = np.array([[[[0, -1], [0, 1]]]], dtype=np.int32)
    ex, tl = bench.work_units(idx, cnt, N, block, causal=True, approx=True)
    assert ex == N * (N + 1) // 2
    assert tl == 0


def test_work_units_tail_pairs():
    # query block 1 lists only itself: its 36 rows see their own causal
    # triangle exactly and block 0 through one pooled key each
    N, block = 100, 64
    cnt = np.array([[[1, 1]]], dtype=np.int32)
    idx = np.array([[[[0, -1], [1, -1]]]], dtype=np.int32)
    ex, tl = bench.work_units(idx, cnt, N, block, causal=True, approx=True)
    assert ex == 64 * 65 // 2 + 36 * 37 // 2
    assert tl == 36 * 1
    ex2, tl2 = bench.work_units(idx, cnt, N, block, causal=True, approx=False)
    assert (ex2, tl2) == (ex, 0)


def test_lds_operand_bytes_counts_tiles_per_wave():
    d = 128
    cnt = np.array([[[2, 1]]], dtype=np.int64)   # M = 2, non-causal
    # 16-row kernel: 64-key tiles, 4 waves; tails: 0 and 1 blocks -> 0 and 1 tiles
    w16 = bench.lds_operand_bytes(cnt, 64, d, False, True, "attn_w16_kernel")
    assert w16 == (2 + 0 + 1 + 1) * 4 * 2 * 64 * d * 2
    # pipelined kernel, 128-row blocks: two 64-key tiles per listed block
    gen = bench.lds_operand_bytes(cnt, 128, d, False, False, "attn_bf16_kernel")
    assert gen == (2 * 2 + 2 * 1) * 4 * 2 * 64 * d * 2
    assert bench.lds_operand_bytes(cnt, 64, d, False, True, "attn_f32_kernel") is None


def test_code_only_drops_comments_and_blank_lines():
    src = "int a; // one\n\n/* two\n three */ int b;\n  // four\nint c;  \n"
    assert bench._code_only(src) == "int a;\n int b;\nint c;"


def test_kernel_hash_ignores_comment_edits(tmp_path, monkeypatch):
    pkg = tmp_path / "block_sparse_attention_08_amd" / "csrc"
    shutil.copytree(os.path.join(bench.ROOT, "block_sparse_attention_08_amd", "csrc"), pkg)
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    before = bench.kernel_hash("attn_w16_kernel")
    f = pkg / "attn_bf16_w16.hip"
    f.write_text(f.read_text() + "\n// a comment added at the end\n")
    assert bench.kernel_hash("attn_w16_kernel") == before
    f.write_text(f.read_text() + "\nstatic int sa_unused_probe_value = 1;\n")
    assert bench.kernel_hash("attn_w16_kernel") != before


def test_read_traffic_needs_the_dispatched_kernel():
    assert bench.read_traffic("dit_image_8k", "attn_bf16_kernel") is None
    assert bench.read_traffic("no_such_workload", "attn_w16_kernel") is None
