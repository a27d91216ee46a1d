"""Benchmark of the block-sparse attention layer on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]

One step = one layer: block pooling, scoring + selection, and attention over
all heads of the workload, with inputs already resident in HBM.  Default
workload: llm_prefill_256k (bf16, B=1, 8 heads, N=262144, d=128, block 128,
causal, alpha=0.5 threshold, no tail), the top of the 8K-256K range the
metric is quoted over.  Prints one JSON line.

Beside the timed steps: the dense comparison (the same attention kernel with
every eligible block listed, timed on its own launches; its speed-up and its
output difference from the sparse run), and the oracle on whole KV groups,
timed step by step on the host cores and checked against the timed run's
lists and outputs.

Stage times come from HIP events recorded on the stream the library launches
on (torch's current stream) around every stage of every timed step.  The
effective throughput counts algorithmic work only: 4*d flops per allowed
exact (query, key) pair and per (query, tail block) pair, from the selection
the run produced.  The CPU baseline times the oracle on a bounded sample of
the same workload (whole heads; heads are independent).
"""

from __future__ import annotations

import argparse
import hashlib
import json
import os
import re
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0      # MI355X dense bf16 matrix peak
PEAK_F32_ALU_TFLOPS = 157.3    # MI355X fp32 vector peak (256 CUs x 2.4 GHz x 256 flop/clk)
PEAK_HBM_GBS = 8000.0          # MI355X HBM3E
METRIC = "block-sparse attn fwd ms/layer + effective TFLOP/s (MFMA %) at N=8K–256K"
# sources each attention kernel is built from (a counter summary is used only
# while their hash matches the one it was taken on)
KERNEL_SOURCES = {
    "attn_w16_kernel": ["attn_bf16_w16.hip", "attn_common.h", "device_common.h", "launch.h"],
    "attn_bf16_kernel": ["attn_bf16.hip", "attn_common.h", "device_common.h", "launch.h"],
    "attn_f32_kernel": ["attn_f32.hip", "device_common.h", "launch.h"],
}


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=100)
    p.add_argument("--warmup", type=int, default=10)
    p.add_argument("--workload", default="llm_prefill_256k")
    p.add_argument("--seed", type=int, default=0)
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--no-peaks", action="store_true",
                   help="skip the achievable-rate kernels (streaming read, MFMA loop)")
    p.add_argument("--cpu-budget-s", type=float, default=12.0,
                   help="CPU seconds the oracle sample may take (whole KV groups, at least one)")
    p.add_argument("--calib-copy-mib", type=int, default=0,
                   help="also run one device copy of this size (counter calibration runs)")
    p.add_argument("--dense", action="store_true",
                   help="attend every eligible block (caller lists) in the timed steps")
    p.add_argument("--no-dense-compare", action="store_true",
                   help="skip the in-run dense comparison (every eligible block listed, same kernel)")
    p.add_argument("--dense-steps", type=int, default=3,
                   help="timed launches of the dense comparison")
    p.add_argument("--backward", action="store_true",
                   help="also run the gradients (fwd_lse + bwd) each step and report them")
    p.add_argument("--no-graph", action="store_true",
                   help="skip the HIP-graph replay of the step (reported beside the eager figures)")
    p.add_argument("--fused-route", action="store_true",
                   help="pool + select in one cooperative launch (sparse_attn_route)")
    return p.parse_args()


def work_units(idx, cnt, N, block, causal, approx):
    """Allowed exact (i, j) pairs and (i, tail block) pairs of a selection."""
    B, Hq, M = cnt.shape
    n = np.array([min(block, N - J * block) for J in range(M)], dtype=np.int64)
    exact = 0
    tail = 0
    for b in range(B):
        for h in range(Hq):
            for I in range(M):
                c = int(cnt[b, h, I])
                sel = idx[b, h, I, :c]
                nI = int(n[I])
                off = sel[sel != I] if causal else sel
                exact += nI * int(n[off].sum())
                if causal and (sel == I).any():
                    exact += nI * (nI + 1) // 2
                if approx:
                    n_elig = I + 1 if causal else M
                    tail += nI * (n_elig - c)
    return exact, tail


def lds_operand_bytes(cnt, block, d, causal, approx, kernel):
    """Bytes the attention kernel's waves read from LDS as product operands in
    one launch: every wave of a workgroup reads the whole K tile and the whole
    V tile (T keys x d, bf16) of every tile the workgroup visits -- the listed
    blocks (block / T tiles each) and the tail tiles (T pooled rows each).
    None for kernels without LDS operand tiles."""
    if kernel == "attn_w16_kernel":
        nw, t = 4, 64
    elif kernel == "attn_bf16_kernel":
        nw, t = block // 32, block // 2
    else:
        return None
    M = cnt.shape[-1]
    jend = np.arange(1, M + 1) if causal else np.full(M, M)
    rest = (jend - cnt.astype(np.int64)) if approx else np.zeros_like(cnt, dtype=np.int64)
    tiles = (block // t) * cnt.astype(np.int64) + (rest + t - 1) // t
    return float(tiles.sum()) * nw * 2 * t * d * 2


def _code_only(text):
    """Source text without comments and blank lines: what the compiler sees
    of it (no string literal in these sources holds a comment marker)."""
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    text = re.sub(r"//[^\n]*", "", text)
    return "\n".join(line.rstrip() for line in text.splitlines() if line.strip())


def kernel_hash(kernel=None):
    """Hash of the code (comments dropped) of the sources of `kernel` (a key
    of KERNEL_SOURCES), or of every library source when None: a summary of
    counters stays valid across edits of comments only."""
    csrc = os.path.join(ROOT, "block_sparse_attention_08_amd", "csrc")
    files = KERNEL_SOURCES[kernel] if kernel else sorted(os.listdir(csrc))
    h = hashlib.sha256()
    for f in files:
        with open(os.path.join(csrc, f), encoding="utf-8") as fh:
            h.update(_code_only(fh.read()).encode())
    return h.hexdigest()[:16]


def read_traffic(workload, kernel):
    """HBM bytes per launch of `kernel` from the committed counter summary, if
    it covers that kernel and was taken on its current sources (else None)."""
    path = os.path.join(ROOT, "profiles", f"traffic_attn_{workload}.txt")
    if not os.path.exists(path):
        return None
    kv = {}
    for line in open(path):
        if "=" in line and not line.startswith("#"):
            a, b = line.split("=", 1)
            kv[a.strip()] = b.strip()
    if kv.get("kernel", "").split("<")[0] != kernel or kv.get("kernel_sources_sha") != kernel_hash(kernel):
        return None
    try:
        return float(kv["hbm_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def achievable_peaks(dev, read_mib=2048, reps=5, mfma_iters=20000, lds_iters=20000):
    """Rates the machine reaches with the measurement kernels of
    libsa_peaks.so: a streaming read of a buffer 8x the last-level cache,
    loops of independent bf16 matrix-core products (on one operand pair, and
    on changing data: the chip holds a lower clock for the latter) and a loop
    of 16-byte LDS reads, timed with events on the launch stream.  Returns
    HBM GB/s, MFMA TFLOP/s (one pair), MFMA TFLOP/s (changing data) and LDS
    GB/s per compute unit."""
    import ctypes
    import torch
    from block_sparse_attention_08_amd import _lib
    h = _lib.peaks_lib()
    st = torch.cuda.current_stream()
    buf = torch.zeros(read_mib << 20, dtype=torch.uint8, device=dev)
    sink = torch.zeros(256, dtype=torch.int32, device=dev)
    got = ctypes.c_size_t(0)
    flops = ctypes.c_double(0.0)

    def timed(fn):
        assert fn() == 0
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(st)
        for _ in range(reps):
            assert fn() == 0
        e1.record(st)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) * 1e-3 / reps

    t_read = timed(lambda: h.sa_peak_read(buf.data_ptr(), buf.numel(), sink.data_ptr(),
                                          st.cuda_stream, ctypes.byref(got)))
    t_mfma = timed(lambda: h.sa_peak_mfma_bf16(mfma_iters, sink.data_ptr(), st.cuda_stream,
                                               ctypes.byref(flops)))
    dflops = ctypes.c_double(0.0)
    t_data = timed(lambda: h.sa_peak_mfma_bf16_data(max(1, mfma_iters // 2), sink.data_ptr(), st.cuda_stream,
                                                    ctypes.byref(dflops)))
    lds = ctypes.c_double(0.0)
    t_lds = timed(lambda: h.sa_peak_lds_read(lds_iters, sink.data_ptr(), st.cuda_stream, ctypes.byref(lds)))
    cus = torch.cuda.get_device_properties(dev).multi_processor_count
    del buf
    return (got.value / t_read / 1e9, flops.value / t_mfma / 1e12, dflops.value / t_data / 1e12,
            lds.value / t_lds / 1e9 / cus)


def _cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(wl, seed, budget_s, gpu=None):
    """Time the oracle (as it stands, float64 numpy) on whole KV groups of
    the workload, in KV-group order, until about `budget_s` of oracle time is
    spent (at least one group; further passes when the workload takes less).
    Each step of the method is timed on its own: pooling, block scores,
    selection (mask and thresholds), attention of every query block.

    With `gpu` = (blk_idx, blk_cnt, out) device tensors of the timed GPU run,
    the first pass over each group is also a parity check of that run: the
    GPU's lists against the oracle's (bit-exact outside the 1e-5 band around
    the threshold; band blocks counted) and the GPU's outputs against the
    oracle's on every query block whose selection agrees (max-abs).  The
    lists of the groups the timed passes did not reach are then checked too
    (pooling, scores and selection only, untimed: cheap next to attention),
    so the selection is compared on every head."""
    import oracle
    from synth import make_group
    try:
        from threadpoolctl import threadpool_info
        blas_threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:
        blas_threads = None
    G = wl.Hq // wl.Hkv
    M = wl.M
    scale = 1.0 / np.sqrt(wl.d)
    bounds = oracle.block_bounds(wl.N, wl.block)

    def list_diff(gidx, gcnt, heads, sel, sc, thr):
        """(GPU mask != oracle mask, oracle band) over the query heads `heads`."""
        gc = gcnt[0, heads].cpu().numpy()
        gi = gidx[0, heads].cpu().numpy()
        gmask = np.zeros((1, len(heads), M, M), bool)
        for hl in range(len(heads)):
            for I in range(M):
                gmask[0, hl, I, gi[hl, I, :gc[hl, I]]] = True
        return gmask != sel, oracle.band_mask(sc, thr, wl.causal)

    elig = oracle.eligible_mask(M, wl.causal)
    t_stage = {"pool_s": 0.0, "score_s": 0.0, "select_s": 0.0, "attend_s": 0.0}
    flops = 0.0
    groups = 0
    par = {"heads": 0, "band_blocks": 0, "band_differ": 0, "mismatch_out_of_band": 0,
           "blocks_compared": 0, "blocks_skipped": 0, "max_abs_err": 0.0}
    checked = set()
    while sum(t_stage.values()) < budget_s or groups == 0:
        g = groups % wl.Hkv
        q, k, v = make_group(wl, seed, 0, g)
        qb4, kb4 = q[None], k[None, None]
        t0 = time.perf_counter()
        q_bar = oracle.pool_mean(qb4, wl.block)
        k_bar = oracle.pool_mean(kb4, wl.block)
        v_sum = oracle.pool_sum(v[None, None], wl.block) if wl.approx else None
        t1 = time.perf_counter()
        sc = oracle.block_scores(q_bar, k_bar, scale)
        t2 = time.perf_counter()
        sel = oracle.select(sc, causal=wl.causal, approx=wl.approx, mode=wl.select, alpha=wl.alpha,
                            density=wl.density)
        thr = oracle.thresholds(sc, causal=wl.causal, mode=wl.select, alpha=wl.alpha, density=wl.density)
        t3 = time.perf_counter()
        out = np.empty((G, wl.N, wl.d))
        for hl in range(G):
            for I in range(M):
                r0, r1 = bounds[I]
                out[hl, r0:r1] = oracle.attend_block(
                    q[hl, r0:r1], r0, k, v, k_bar[0, 0], None if v_sum is None else v_sum[0, 0],
                    sel[0, hl, I], elig[I], block=wl.block, scale=scale, causal=wl.causal, approx=wl.approx)
        t4 = time.perf_counter()
        t_stage["pool_s"] += t1 - t0
        t_stage["score_s"] += t2 - t1
        t_stage["select_s"] += t3 - t2
        t_stage["attend_s"] += t4 - t3
        idx, cnt = oracle.mask_to_lists(sel)
        ex, tl = work_units(idx, cnt, wl.N, wl.block, wl.causal, wl.approx)
        flops += 4.0 * wl.d * (ex + tl)
        if gpu is not None and g not in checked:
            checked.add(g)
            gidx, gcnt, gout = gpu
            heads = list(range(g * G, (g + 1) * G))
            diff, band = list_diff(gidx, gcnt, heads, sel, sc, thr)
            par["heads"] += G
            par["band_blocks"] += int(band.sum())
            par["band_differ"] += int((diff & band).sum())
            par["mismatch_out_of_band"] += int((diff & ~band).sum())
            rows_ok = ~diff.any(-1)[0]
            go = gout[0, heads].float().cpu().numpy()
            for hl in range(G):
                for I in range(M):
                    if not rows_ok[hl, I]:
                        par["blocks_skipped"] += 1
                        continue
                    r0, r1 = bounds[I]
                    e = float(np.abs(go[hl, r0:r1] - out[hl, r0:r1]).max())
                    par["max_abs_err"] = max(par["max_abs_err"], e)
                    par["blocks_compared"] += 1
        groups += 1
    spent = sum(t_stage.values())
    if gpu is not None:
        # the selection of every head: the groups the timed passes reached,
        # then the rest (pooling, scores and selection only, not timed)
        allm = {"heads": par["heads"], "band_blocks": par["band_blocks"], "band_differ": par["band_differ"],
                "mismatch_out_of_band": par["mismatch_out_of_band"]}
        for g in range(wl.Hkv):
            if g in checked:
                continue
            q, k, _ = make_group(wl, seed, 0, g)
            q_bar = oracle.pool_mean(q[None], wl.block)
            k_bar = oracle.pool_mean(k[None, None], wl.block)
            sc = oracle.block_scores(q_bar, k_bar, scale)
            sel = oracle.select(sc, causal=wl.causal, approx=wl.approx, mode=wl.select, alpha=wl.alpha,
                                density=wl.density)
            thr = oracle.thresholds(sc, causal=wl.causal, mode=wl.select, alpha=wl.alpha, density=wl.density)
            diff, band = list_diff(gpu[0], gpu[1], list(range(g * G, (g + 1) * G)), sel, sc, thr)
            allm["heads"] += G
            allm["band_blocks"] += int(band.sum())
            allm["band_differ"] += int((diff & band).sum())
            allm["mismatch_out_of_band"] += int((diff & ~band).sum())
        par["lists_all_heads"] = allm
    if groups >= wl.Hkv:
        what = (f"all {wl.Hq} query heads, {groups / wl.Hkv:.2f} passes over the workload"
                if groups % wl.Hkv else f"all {wl.Hq} query heads x {groups // wl.Hkv} passes")
    else:
        what = f"{groups * G} of {wl.Hq} query heads (KV groups 0..{groups - 1})"
    res = {
        "value": flops / spent / 1e12, "unit": "TFLOP/s (effective)",
        "cores": len(os.sched_getaffinity(0)), "kind": "oracle",
        "sample": f"{what}, full sequence, every query block: float64 numpy oracle, "
                  f"pool+score+select+attend, {spent:.1f} s",
        "cpu_model": _cpu_model(), "blas_threads": blas_threads,
        "stage_s": {k_: round(v_, 3) for k_, v_ in t_stage.items()},
        "fraction_of_layer": round(groups / wl.Hkv, 4),
    }
    if gpu is not None:
        res["parity"] = par
    return res


def dense_compare(args, wl, desc, ws, qd, kd, vd, out, ms_step, ms_fwd, sparse_flops):
    """The same attention kernel on caller lists holding every eligible
    block (dense attention, causal if the workload is), timed with events on
    the launch stream over its own launches after one warmup launch; the
    routing stages are the sparse run's.  Returns its times, the speed-up of
    the sparse layer and the difference between the two outputs."""
    import torch
    import block_sparse_attention_08_amd as bsa
    M = wl.M
    dev = qd.device
    idx = torch.arange(M, dtype=torch.int32, device=dev).expand(wl.B, wl.Hq, M, M).contiguous()
    if wl.causal:
        cnt = torch.arange(1, M + 1, dtype=torch.int32, device=dev).expand(wl.B, wl.Hq, M).contiguous()
    else:
        cnt = torch.full((wl.B, wl.Hq, M), M, dtype=torch.int32, device=dev)
    dout = torch.empty_like(out)
    bsa.fwd(desc, qd, kd, vd, ws.k_bar, ws.v_sum, ws.tail, idx, cnt, dout)
    torch.cuda.synchronize()
    st = torch.cuda.current_stream()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(st)
    for _ in range(args.dense_steps):
        bsa.fwd(desc, qd, kd, vd, ws.k_bar, ws.v_sum, ws.tail, idx, cnt, dout)
    e1.record(st)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / args.dense_steps
    ex, tl = work_units(idx.cpu().numpy(), cnt.cpu().numpy(), wl.N, wl.block, wl.causal, False)
    dflops = 4.0 * wl.d * (ex + tl)
    diff = (out.float() - dout.float()).abs()
    ms_layer = ms_step - ms_fwd + ms
    res = {
        "fwd_ms": round(ms, 3), "layer_ms": round(ms_layer, 3),
        "speedup_layer": round(ms_layer / ms_step, 2), "speedup_fwd": round(ms / ms_fwd, 2),
        "algorithmic_gflop": round(dflops / 1e9, 1),
        "TFLOPs": round(dflops / (ms * 1e-3) / 1e12, 1),
        "frac_of_bf16_peak": round(dflops / (ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4),
        "sparse_flop_share": round(sparse_flops / dflops, 5),
        "max_abs_diff_sparse_vs_dense": round(float(diff.max()), 5),
        "mean_abs_diff_sparse_vs_dense": round(float(diff.mean()), 6),
        "launches": args.dense_steps,
    }
    del idx, cnt, dout, diff
    torch.cuda.empty_cache()
    return res


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only: the library has no multi-GPU path "
              f"(--gpus {args.gpus} requested)", file=sys.stderr)
        sys.exit(2)
    import torch

    import block_sparse_attention_08_amd as bsa
    from synth import get_config, make_inputs

    wl = get_config(args.workload)
    dev = torch.device("cuda", 0)
    torch.cuda.set_device(dev)
    q, k, v = make_inputs(wl, args.seed)
    tdt = torch.bfloat16 if wl.dtype == "bf16" else torch.float32
    qd = torch.from_numpy(q).to(tdt).to(dev)
    kd = torch.from_numpy(k).to(tdt).to(dev)
    vd = torch.from_numpy(v).to(tdt).to(dev)
    del q, k, v
    desc = bsa.make_desc(wl.B, wl.Hq, wl.Hkv, wl.N, wl.d, block=wl.block, dtype=wl.dtype,
                         alpha=wl.alpha if wl.select == "alpha" else None,
                         density=wl.density if wl.select == "density" else None,
                         causal=wl.causal, approx=wl.approx)
    ws = bsa.Workspace(desc, device=dev)
    out = torch.empty_like(qd)
    if args.backward:
        if wl.dtype != "bf16":
            print("--backward needs a bf16 workload", file=sys.stderr)
            sys.exit(2)
        bws = bsa.BwdWorkspace(desc, device=dev)
        gen = torch.Generator(device=dev).manual_seed(args.seed + 1)
        dout = torch.randn(qd.shape, generator=gen, device=dev, dtype=torch.float32).to(torch.bfloat16)
        dq, dk, dv = torch.empty_like(qd), torch.empty_like(kd), torch.empty_like(vd)
    M = wl.M
    dense_idx = dense_cnt = None
    if args.dense:
        idx = np.zeros((wl.B, wl.Hq, M, M), np.int32)
        idx[...] = np.arange(M, dtype=np.int32)
        cnt = np.full((wl.B, wl.Hq, M), M, np.int32)
        if wl.causal:
            cnt[...] = np.arange(1, M + 1, dtype=np.int32)
        dense_idx, dense_cnt = torch.from_numpy(idx).to(dev), torch.from_numpy(cnt).to(dev)

    def step(ev=None):
        if ev:
            ev[0].record()
        if args.fused_route:
            bsa.route(desc, qd, kd, vd, ws.q_bar, ws.k_bar, ws.v_sum, ws.tail, ws.blk_idx, ws.blk_cnt)
            if ev:
                ev[1].record()
                ev[2].record()
        else:
            bsa.block_pool(desc, qd, kd, vd, ws.q_bar, ws.k_bar, ws.v_sum, ws.tail)
            if ev:
                ev[1].record()
            bsa.select(desc, ws.q_bar, ws.k_bar, ws.blk_idx, ws.blk_cnt)
            if ev:
                ev[2].record()
        if args.dense:
            bsa.fwd(desc, qd, kd, vd, ws.k_bar, ws.v_sum, ws.tail, dense_idx, dense_cnt, out)
        elif args.backward:
            bsa.fwd_lse(desc, qd, kd, vd, ws.k_bar, ws.v_sum, ws.tail, ws.blk_idx, ws.blk_cnt, out, bws.lse)
        else:
            bsa.fwd(desc, qd, kd, vd, ws.k_bar, ws.v_sum, ws.tail, ws.blk_idx, ws.blk_cnt, out)
        if ev:
            ev[3].record()
        if args.backward:
            bsa.bwd(desc, qd, kd, vd, ws.tail, ws.blk_idx, ws.blk_cnt, out, dout, bws, dq, dk, dv)
            if ev:
                ev[4].record()

    if args.calib_copy_mib:
        n = args.calib_copy_mib * (1 << 20) // 4
        a = torch.ones(n, dtype=torch.float32, device=dev)
        b_ = torch.empty_like(a)
        b_.copy_(a)
        torch.cuda.synchronize()
        del a, b_

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    print(f"[bench] {wl.name}: warmup {args.warmup} done", file=sys.stderr, flush=True)

    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(5)] for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(evs[i])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_pool = np.mean([e[0].elapsed_time(e[1]) for e in evs])
    ms_sel = np.mean([e[1].elapsed_time(e[2]) for e in evs])
    ms_fwd = np.mean([e[2].elapsed_time(e[3]) for e in evs])
    ms_step = wall * 1e3 / args.steps
    print(f"[bench] timed {args.steps} steps: {ms_step:.3f} ms/step", file=sys.stderr, flush=True)

    # The same step captured once in a HIP graph and replayed K times (the
    # launch gaps between the stages go away); reported beside the eager
    # figures, which stay the bench line.
    graph_ms = None
    if not (args.no_graph or args.fused_route or args.backward or args.dense):
        graph = torch.cuda.CUDAGraph()
        side = torch.cuda.Stream(device=dev)
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            step()
        torch.cuda.current_stream().wait_stream(side)
        with torch.cuda.graph(graph):
            step()
        graph.replay()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(args.steps):
            graph.replay()
        torch.cuda.synchronize()
        graph_ms = (time.perf_counter() - t0) * 1e3 / args.steps
        print(f"[bench] graph replay: {graph_ms:.3f} ms/step", file=sys.stderr, flush=True)

    # algorithmic work of this selection
    if args.dense:
        idx_h, cnt_h = dense_idx.cpu().numpy(), dense_cnt.cpu().numpy()
    else:
        idx_h, cnt_h = ws.blk_idx.cpu().numpy(), ws.blk_cnt.cpu().numpy()
    ex, tl = work_units(idx_h, cnt_h, wl.N, wl.block, wl.causal, wl.approx and not args.dense)
    flops = 4.0 * wl.d * (ex + tl)
    elt = 2 if wl.dtype == "bf16" else 4
    n_pool_heads = wl.Hq + wl.Hkv * (2 if wl.approx else 1)
    pool_bytes = wl.B * n_pool_heads * (wl.N * wl.d * elt + M * wl.d * 4)
    if wl.approx and wl.dtype == "bf16":
        pool_bytes += 2 * wl.B * wl.Hkv * M * wl.d * 2      # bf16 tail operands
    n_elig = wl.B * wl.Hq * (M * (M + 1) // 2 if wl.causal else M * M)
    sel_flops = 2.0 * wl.d * n_elig
    sel_bytes = wl.B * (wl.Hq + wl.Hkv) * M * wl.d * 4 + 4 * (int(cnt_h.sum()) + cnt_h.size)
    eff_tflops_fwd = flops / (ms_fwd * 1e-3) / 1e12
    peak = PEAK_BF16_TFLOPS if wl.dtype == "bf16" else PEAK_F32_ALU_TFLOPS
    # the library's dispatch: 64-row blocks with fewer than 384 blocks per row
    # run the 16-row-per-wave kernel, every other bf16 case the pipelined one
    attn_kernel = ("attn_f32_kernel" if wl.dtype != "bf16" else
                   "attn_w16_kernel" if wl.block == 64 and M < 384 else "attn_bf16_kernel")
    traffic = read_traffic(wl.name, attn_kernel) if not args.dense else None
    eligible_blocks = n_elig
    result = {
        "metric": METRIC,
        "value": round(flops / (ms_step * 1e-3) / 1e12, 3),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": wl.dtype,
        "data": "synthetic",
        "config": {"workload": wl.name + ("+dense" if args.dense else ""), "B": wl.B,
                   "heads_q": wl.Hq, "heads_kv": wl.Hkv, "seq_len": wl.N, "head_dim": wl.d,
                   "block": wl.block, "causal": wl.causal,
                   "selection": (f"alpha={wl.alpha}" if wl.select == "alpha"
                                 else f"density={wl.density}") if not args.dense else "all",
                   "tail": bool(wl.approx and not args.dense), "parallelism": "single-gpu",
                   "routing": "fused" if args.fused_route else "pool+select"},
        "roofline": {
            "bound": "mfma" if wl.dtype == "bf16" else "alu",
            "kernel": attn_kernel,
            "achieved": round(eff_tflops_fwd, 2), "peak": peak, "unit": "TFLOP/s",
            "frac": round(eff_tflops_fwd / peak, 4),
            "traffic": traffic,
        },
        "stages": {
            "pool_ms": round(ms_pool, 4), "select_ms": round(ms_sel, 4), "fwd_ms": round(ms_fwd, 4),
            "pool_GBps": round(pool_bytes / (ms_pool * 1e-3) / 1e9, 1),
            "pool_hbm_frac": round(pool_bytes / (ms_pool * 1e-3) / 1e9 / PEAK_HBM_GBS, 4),
            "select_TFLOPs": round(sel_flops / (ms_sel * 1e-3) / 1e12, 2),
            "select_hbm_frac": round(sel_bytes / (ms_sel * 1e-3) / 1e9 / PEAK_HBM_GBS, 4),
            "pool_select_hbm_frac": round((pool_bytes + sel_bytes) / ((ms_pool + ms_sel) * 1e-3)
                                          / 1e9 / PEAK_HBM_GBS, 4),
            "exact_pairs": int(ex), "tail_pairs": int(tl), "algorithmic_gflop": round(flops / 1e9, 3),
            "selected_blocks": int(cnt_h.sum()), "eligible_blocks": int(eligible_blocks),
            "realised_density": round(float(cnt_h.sum()) / eligible_blocks, 5),
            "dense_equiv_tflops": round(4.0 * wl.d * wl.B * wl.Hq * wl.N * wl.N
                                        * (0.5 if wl.causal else 1.0) / (ms_step * 1e-3) / 1e12, 2),
        },
    }
    if graph_ms is not None:
        result["graph"] = {
            "ms_per_step": round(graph_ms, 4), "value": round(flops / (graph_ms * 1e-3) / 1e12, 3),
            "note": "the same step captured in a HIP graph and replayed; value, ms_per_step and the "
                    "stages above come from the eager steps"}
    if args.backward:
        ms_bwd = np.mean([e[3].elapsed_time(e[4]) for e in evs])
        bflops = 10.0 * wl.d * (ex + tl)      # S, dP, dV, dK, dQ: 2d each per pair
        result["backward"] = {
            "bwd_ms": round(ms_bwd, 4), "algorithmic_gflop": round(bflops / 1e9, 3),
            "TFLOPs": round(bflops / (ms_bwd * 1e-3) / 1e12, 2),
            "frac_of_bf16_peak": round(bflops / (ms_bwd * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4),
            "note": "step = pool + select + fwd_lse + bwd; value/ms_per_step include the backward"}
    if not args.no_peaks:
        print("[bench] measuring achievable HBM read, bf16 MFMA and LDS read rates", file=sys.stderr, flush=True)
        hbm, mfma, mfma_data, lds = achievable_peaks(dev)
        pool_gbps = pool_bytes / (ms_pool * 1e-3) / 1e9
        lds_bytes = (lds_operand_bytes(cnt_h, wl.block, wl.d, wl.causal, wl.approx and not args.dense,
                                       attn_kernel) if wl.dtype == "bf16" else None)
        cus = torch.cuda.get_device_properties(dev).multi_processor_count
        fwd_lds = lds_bytes / (ms_fwd * 1e-3) / 1e9 / cus if lds_bytes else None
        result["achievable"] = {
            "hbm_read_GBps": round(hbm, 1), "mfma_bf16_TFLOPs": round(mfma, 1),
            "lds_read_GBps_per_CU": round(lds, 1),
            "fwd_lds_operand_GBps_per_CU": round(fwd_lds, 1) if fwd_lds else None,
            "fwd_frac_of_achievable_lds": round(fwd_lds / lds, 4) if fwd_lds else None,
            "pool_frac_of_achievable_hbm": round(pool_gbps / hbm, 4),
            "pool_select_frac_of_achievable_hbm": round(
                (pool_bytes + sel_bytes) / ((ms_pool + ms_sel) * 1e-3) / 1e9 / hbm, 4),
            "fwd_frac_of_achievable_mfma": (round(eff_tflops_fwd / mfma, 4)
                                            if wl.dtype == "bf16" else None),
            "mfma_bf16_data_TFLOPs": round(mfma_data, 1),
            "fwd_frac_of_data_mfma": (round(eff_tflops_fwd / mfma_data, 4)
                                      if wl.dtype == "bf16" else None),
        }
    if not (args.dense or args.no_dense_compare or args.backward):
        print("[bench] dense comparison: every eligible block listed", file=sys.stderr, flush=True)
        result["dense_compare"] = dense_compare(args, wl, desc, ws, qd, kd, vd, out, ms_step, ms_fwd, flops)
    if not args.no_cpu_baseline:
        print("[bench] timing the CPU oracle sample", file=sys.stderr, flush=True)
        gpu = None if (args.dense or args.backward) else (ws.blk_idx, ws.blk_cnt, out)
        result["cpu_baseline"] = cpu_baseline(wl, args.seed, args.cpu_budget_s, gpu=gpu)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
