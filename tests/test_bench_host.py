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


class _FakeDev:
    """Host stand-in for the device tensors the CPU-baseline parity reads
    (indexing, .cpu(), .float(), .numpy())."""

    def __init__(self, a):
        self.a = np.asarray(a)

    def __getitem__(self, key):
        return _FakeDev(self.a[key])

    def cpu(self):
        return self

    def float(self):
        return _FakeDev(self.a.astype(np.float32))

    def numpy(self):
        return self.a


def test_cpu_baseline_reports_stages_and_checks_parity():
    """The CPU-baseline leg on the 1K-token workload: every stage timed, the
    affinity core count reported, and the parity check flags a planted
    wrong list entry and a planted wrong output (the oracle's own lists and
    outputs pass)."""
    import oracle
    from synth import get_config, make_inputs
    wl = get_config("dit_tiny_f32")
    q, k, v = make_inputs(wl, 0)
    ref = oracle.forward(q, k, v, block=wl.block, causal=wl.causal, approx=wl.approx, mode=wl.select,
                         alpha=wl.alpha, density=wl.density)
    idx, cnt = oracle.mask_to_lists(ref["mask"])
    out = ref["out"].astype(np.float32)
    r = bench.cpu_baseline(wl, 0, 0.0, gpu=(_FakeDev(idx), _FakeDev(cnt), _FakeDev(out)))
    assert r["cores"] == len(os.sched_getaffinity(0)) and r["kind"] == "oracle"
    assert set(r["stage_s"]) == {"pool_s", "score_s", "select_s", "attend_s"}
    p = r["parity"]
    G = wl.Hq // wl.Hkv          # a zero budget still runs one whole KV group
    assert p["heads"] == G and p["mismatch_out_of_band"] == 0 and p["blocks_skipped"] == 0
    assert p["blocks_compared"] == G * wl.M and p["max_abs_err"] < 1e-6
    # the lists of every head are compared, not only the timed group's
    assert p["lists_all_heads"]["heads"] == wl.Hq and p["lists_all_heads"]["mismatch_out_of_band"] == 0
    # plant one wrong list entry (a block the oracle did not keep) and one
    # wrong output value in another row
    bad_idx, bad_cnt = idx.copy(), cnt.copy()
    row = (0, 0, 3)
    drop = np.nonzero(~ref["mask"][row])[0][0]
    c = int(bad_cnt[row])
    bad_idx[row + (slice(0, c + 1),)] = np.sort(np.append(idx[row][:c], drop))
    bad_cnt[row] += 1
    bad_out = out.copy()
    bad_out[0, 0, 5, 7] += 0.5
    r = bench.cpu_baseline(wl, 0, 0.0, gpu=(_FakeDev(bad_idx), _FakeDev(bad_cnt), _FakeDev(bad_out)))
    p = r["parity"]
    assert p["mismatch_out_of_band"] == 1 and p["blocks_skipped"] == 1
    assert abs(p["max_abs_err"] - 0.5) < 1e-3
    assert p["lists_all_heads"]["mismatch_out_of_band"] == 1
    # a wrong entry in a head outside the timed group shows only in the
    # all-heads list check
    assert wl.Hq > G
    bad_idx, bad_cnt = idx.copy(), cnt.copy()
    row = (0, wl.Hq - 1, 2)
    drop = np.nonzero(~ref["mask"][row])[0][0]
    c = int(bad_cnt[row])
    bad_idx[row + (slice(0, c + 1),)] = np.sort(np.append(idx[row][:c], drop))
    bad_cnt[row] += 1
    r = bench.cpu_baseline(wl, 0, 0.0, gpu=(_FakeDev(bad_idx), _FakeDev(bad_cnt), _FakeDev(out)))
    p = r["parity"]
    assert p["mismatch_out_of_band"] == 0 and p["lists_all_heads"]["mismatch_out_of_band"] == 1
