#!/usr/bin/env python3
"""Benchmark of the MSA hot path on one MI355X.

One step = one whole hot path: msa_prefill on the 32K-token prefill workload
(batch 1, 64 query / 8 KV heads, head dim 128, blocks of 128, top_k 16:
pooling, index top-k, query->block inversion, KV-outer attention over every
kept block, partial merge) followed by one msa_decode on the decode workload (16 sequences over
262144-token caches, same heads).  Inputs are seeded synthetic tensors
already resident in HBM.  Prints one JSON line.

    python bench.py [--gpus 1] [--steps 20] [--warmup 5] [--no-cpu-baseline]
"""
import argparse
import hashlib
import json
import os
import subprocess
import sys
import tempfile
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 MFMA
PEAK_HBM_GBS = 8000.0       # MI355X HBM3E
D_HEAD = 128
CPU_SAMPLE_ROWS = 6144      # oracle rows timed on the host (about 15-20 s, one thread)


def _prefill_counts(w):
    """Algorithmic work of one prefill: attended keys summed over queries
    (per query head) and the (query row, kept block) pairs, own block
    included."""
    import numpy as np
    t = np.arange(w.seq_len, dtype=np.int64)
    own = t // w.block_size
    kept = np.minimum(w.top_k - 1, own)
    keys = kept * w.block_size + (t % w.block_size) + 1
    per_head_keys = int(keys.sum()) * w.batch
    pairs = int((kept + 1).sum()) * w.batch * w.n_q_heads
    rows_merged = int((own > 0).sum()) * w.batch * w.n_q_heads   # rows with partials to merge
    return per_head_keys, pairs, rows_merged


def _decode_bytes(w):
    B, Hq, G, D, bs, k = w.batch, w.n_q_heads, w.n_kv_heads, w.head_dim, w.block_size, w.top_k
    nb = -(-w.seq_len // bs)
    q = B * Hq * D * 2
    q_idx = B * G * w.idx_dim
    summaries = B * G * nb * w.idx_dim
    kv = B * G * min(k, nb) * bs * D * 2 * 2
    out = B * Hq * D * 2
    return q + q_idx + summaries + kv + out


def kernel_source_hash():
    """Hash of the main-branch kernel source; counter summaries are valid only
    for the source they were taken on."""
    h = hashlib.sha256()
    with open(os.path.join(ROOT, "block_sparse_attention_33_amd", "csrc", "main_branch.hip"), "rb") as f:
        h.update(f.read())
    return h.hexdigest()[:16]


def _measured_traffic():
    """HBM bytes per launch of the attention kernel from the committed
    rocprofv3 FETCH_SIZE / WRITE_SIZE summary (already scaled by the copy
    kernel calibration), if it was taken on the current kernel source."""
    path = os.path.join(ROOT, "profiles", "attend_prefill_32k_traffic.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f)
    if rec.get("kernel_source_sha256_16") != kernel_source_hash():
        return None
    return rec.get("bytes_per_launch")


def pmc_run():
    """Workload for counter runs under rocprofv3 --pmc: two 32K prefills, the
    32K training forward and two backward calls, two decodes of the decode
    workload, then a 1 GiB device copy whose bytes are known (the
    calibration of the FETCH_SIZE / WRITE_SIZE counters)."""
    import torch
    import block_sparse_attention_33_amd as msa
    from synth import decode_inputs, get_workload, grad_output, prefill_inputs
    dev = torch.device("cuda:0")
    w = get_workload("prefill_32k")
    inp = prefill_inputs(w, seed=0, device=dev)
    ws = torch.empty(msa.msa_workspace_bytes(
        msa.MSA_OP_PREFILL, msa.make_dims(w.batch, w.seq_len, w.n_q_heads, w.n_kv_heads, w.block_size,
                                           w.top_k))[1], dtype=torch.uint8, device=dev)
    for _ in range(2):
        msa.msa_prefill(inp["q"], inp["k"], inp["v"], inp["q_idx"], inp["k_idx"], w.block_size, w.top_k,
                        workspace=ws)
    out, sel, lse = msa.msa_prefill_lse(inp["q"], inp["k"], inp["v"], inp["q_idx"], inp["k_idx"], w.block_size,
                                        w.top_k, workspace=ws)
    del ws
    dout = grad_output(w, seed=0, device=dev)
    for _ in range(2):
        msa.msa_prefill_backward(inp["q"], inp["k"], inp["v"], out, dout, lse, sel, w.block_size)
    torch.cuda.synchronize()
    del inp, out, sel, lse, dout
    wd = get_workload("decode_b16_256k")
    din = decode_inputs(wd, seed=0, device=dev)
    bk = msa.msa_pool_block_keys(din["k_idx_cache"], wd.block_size)
    del din["k_idx_cache"]
    for _ in range(2):
        msa.msa_decode(din["q"], din["q_idx"], din["k_cache"], din["v_cache"], bk, wd.block_size, wd.top_k)
    del din, bk
    src = torch.ones(2**30 // 4, dtype=torch.float32, device=dev)
    dst = torch.empty_like(src)
    dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"pmc_run": "done", "copy_bytes_each_way": 2**30,
                      "kernel_source_sha256_16": kernel_source_hash()}))


def pmc_summary(fetch_csv, write_csv, commands):
    """Per-dispatch HBM traffic of the MSA kernels from two rocprofv3 --pmc
    runs of --pmc-run (FETCH_SIZE, then WRITE_SIZE; KiB per dispatch), each
    scaled by what the counter reads for the 1 GiB copy at the end of the
    run.  Writes the record that the benchmark line's roofline.traffic reads."""
    import csv
    import re

    def per_kernel(path, counter):
        got = {}
        with open(path, newline="") as f:
            for row in csv.DictReader(f):
                if row["Counter_Name"] != counter:
                    continue
                name = row["Kernel_Name"]
                m = re.search(r"msa::\(anonymous namespace\)::(\w+(?:<\d+>)?)", name)
                key = m.group(1) if m else ("copy" if "copyBuffer" in name else None)
                if key:
                    got.setdefault(key, []).append(float(row["Counter_Value"]))
        return got

    fk, wk = per_kernel(fetch_csv, "FETCH_SIZE"), per_kernel(write_csv, "WRITE_SIZE")
    copy_kib = 2**30 / 1024.0
    fscale, wscale = copy_kib / fk["copy"][-1], copy_kib / wk["copy"][-1]
    rec = {
        "kernel": "attend_kernel<128>",
        "workload": "prefill_32k (batch 1, seq 32768, 64q/8kv heads, head_dim 128, block 128, top_k 16); "
                    "decode_b16_256k (16 x 262144-token caches, same heads)",
        "kernel_source_sha256_16": kernel_source_hash(),
        "commands": commands,
        "calibration": {"kernel": "__amd_rocclr_copyBuffer, 1 GiB device copy",
                        "fetch_kib_read": fk["copy"][-1], "write_kib_read": wk["copy"][-1],
                        "bytes_each_way": 2**30, "fetch_scale": round(fscale, 5), "write_scale": round(wscale, 5)},
        "note": "FETCH_SIZE counts L2 misses sent to the fabric (memory-side cache hits included); "
                "values are per dispatch, scaled by the copy-kernel factors",
    }
    for k in sorted(set(fk) & set(wk)):
        if k == "copy":
            continue
        fb = sum(fk[k]) / len(fk[k]) * 1024 * fscale
        wb = sum(wk[k]) / len(wk[k]) * 1024 * wscale
        rec[k] = {"dispatches": len(fk[k]), "fetch_kib_per_dispatch": fk[k], "write_kib_per_dispatch": wk[k],
                  "fetch_bytes": round(fb), "write_bytes": round(wb), "bytes": round(fb + wb)}
    rec["bytes_per_launch"] = rec["attend_kernel<128>"]["bytes"]
    out = os.path.join(ROOT, "profiles", "attend_prefill_32k_traffic.json")
    with open(out, "w") as f:
        json.dump(rec, f, indent=1)
    print(json.dumps({"written": out, "attend_bytes_per_launch": rec["bytes_per_launch"]}))


def cpu_baseline_worker(npz_path):
    """Runs in a child process with one BLAS/OpenMP thread: the oracle on the
    sampled rows.  Prints a JSON line with the time."""
    import numpy as np
    if hasattr(os, "sched_setaffinity"):
        os.sched_setaffinity(0, {min(os.sched_getaffinity(0))})
    from oracle import msa_oracle as O
    d = np.load(npz_path)
    rows = d["rows"]
    bs, top_k = int(d["bs"]), int(d["top_k"])
    t0 = time.perf_counter()
    summ = O.pool_block_keys(d["k_idx"], bs)
    sel = O.select_blocks(d["q_idx"], summ, bs, top_k, rows)
    O.attention_rows(d["q_rows"], d["k"], d["v"], sel, rows, bs)
    dt = time.perf_counter() - t0
    print(json.dumps({"seconds": dt, "rows": int(len(rows))}))


def cpu_baseline(inp, w, n_rows):
    import numpy as np
    import torch
    from synth import sample_rows
    rows = sample_rows(w.seq_len, n_rows, 12345)
    rt = torch.as_tensor(rows, device=inp["q"].device)
    with tempfile.TemporaryDirectory() as td:
        path = os.path.join(td, "cpu_baseline.npz")
        np.savez(path, rows=rows, bs=w.block_size, top_k=w.top_k,
                 q_rows=inp["q"][:, rt].float().cpu().numpy(), k=inp["k"].float().cpu().numpy(),
                 v=inp["v"].float().cpu().numpy(), q_idx=inp["q_idx"].cpu().numpy(),
                 k_idx=inp["k_idx"].cpu().numpy())
        env = dict(os.environ, OMP_NUM_THREADS="1", OPENBLAS_NUM_THREADS="1", MKL_NUM_THREADS="1",
                   NUMEXPR_NUM_THREADS="1", HIP_VISIBLE_DEVICES="", CUDA_VISIBLE_DEVICES="")
        res = subprocess.run([sys.executable, os.path.abspath(__file__), "--cpu-baseline-worker", path],
                             env=env, capture_output=True, text=True, timeout=600)
    if res.returncode != 0:
        raise RuntimeError(f"cpu baseline worker failed:\n{res.stderr}")
    rec = json.loads(res.stdout.strip().splitlines()[-1])
    return {
        "value": rec["rows"] / rec["seconds"],
        "unit": "tokens/s",
        "cores": 1,
        "kind": "oracle",
        "sample": (f"{rec['rows']} seeded query positions of the 32K prefill (all 8 groups, 64 heads): "
                   f"pooling of all blocks + selection + attention, {rec['seconds']:.1f} s, one thread"),
    }


def block_keys_prefill_shape(pin, w):
    """An int8 tensor shaped like the prefill's block summaries [B, G, nb, 64]."""
    import torch
    B, G, S, di = pin["k_idx"].shape
    return torch.empty((B, G, -(-S // w.block_size), di), dtype=torch.int8, device=pin["k_idx"].device)


def _chunk_ws_bytes(msa, dims, count):
    import ctypes
    from block_sparse_attention_33_amd import _lib
    hi = ctypes.c_size_t(0)
    rc = _lib.load().msa_prefill_chunk_workspace_bytes(ctypes.byref(dims), count, None, ctypes.byref(hi))
    if rc != 0:
        raise RuntimeError(f"msa_prefill_chunk_workspace_bytes: {rc}")
    return hi.value


def train_only(steps, warmup):
    """The 32K prefill for training alone: forward with log-sum-exp, then the
    backward, each timed over `steps` calls (for profiler runs)."""
    import torch
    import block_sparse_attention_33_amd as msa
    from synth import get_workload, grad_output, prefill_inputs

    dev = torch.device("cuda:0")
    w = get_workload("prefill_32k")
    pin = prefill_inputs(w, seed=0, device=dev)
    dout = grad_output(w, seed=0, device=dev)
    dims = msa.make_dims(w.batch, w.seq_len, w.n_q_heads, w.n_kv_heads, w.block_size, w.top_k)
    pws = torch.empty(msa.msa_workspace_bytes(msa.MSA_OP_PREFILL, dims)[1], dtype=torch.uint8, device=dev)
    bws = torch.empty(msa.msa_workspace_bytes(msa.MSA_OP_BACKWARD, dims)[1], dtype=torch.uint8, device=dev)

    def fwd():
        return msa.msa_prefill_lse(pin["q"], pin["k"], pin["v"], pin["q_idx"], pin["k_idx"], w.block_size, w.top_k,
                                   workspace=pws)

    out, sel, lse = fwd()

    def bwd():
        return msa.msa_prefill_backward(pin["q"], pin["k"], pin["v"], out, dout, lse, sel, w.block_size,
                                        workspace=bws)

    res = {}
    for name, fn in (("forward_lse", fwd), ("backward", bwd)):
        for _ in range(warmup):
            fn()
        torch.cuda.synchronize()
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
        for a, b in ev:
            a.record()
            fn()
            b.record()
        torch.cuda.synchronize()
        res[name] = sorted(a.elapsed_time(b) for a, b in ev)[steps // 2]
    per_head_keys, _, _ = _prefill_counts(w)
    flop = 2.5 * 4.0 * w.head_dim * w.n_q_heads * per_head_keys
    print(json.dumps({"workload": "prefill_32k training", "forward_lse_ms": round(res["forward_lse"], 4),
                      "backward_ms": round(res["backward"], 4),
                      "backward_tflops_alg": round(flop / (res["backward"] * 1e-3) / 1e12, 2)}), flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--core-only", action="store_true",
                    help="time the step only: no chunked, short-sequence or generation-step extras")
    ap.add_argument("--train-only", action="store_true",
                    help="time only the training forward (with log-sum-exp) and backward of the 32K prefill")
    ap.add_argument("--cpu-baseline-worker", default=None, help=argparse.SUPPRESS)
    ap.add_argument("--pmc-run", action="store_true",
                    help="run the counter-collection workload instead of the benchmark")
    ap.add_argument("--pmc-summary", nargs=2, metavar=("FETCH_CSV", "WRITE_CSV"),
                    help="write the traffic record from the two counter runs' CSV files")
    ap.add_argument("--pmc-commands", nargs="*", default=[], help=argparse.SUPPRESS)
    args = ap.parse_args()
    if args.pmc_summary:
        pmc_summary(args.pmc_summary[0], args.pmc_summary[1], args.pmc_commands)
        return 0
    if args.cpu_baseline_worker:
        cpu_baseline_worker(args.cpu_baseline_worker)
        return 0
    if args.pmc_run:
        pmc_run()
        return 0
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported "
              "(the MSA path here runs on a single MI355X).", file=sys.stderr)
        return 2
    if args.train_only:
        train_only(args.steps, args.warmup)
        return 0

    import torch
    import block_sparse_attention_33_amd as msa
    from synth import decode_inputs, get_workload, prefill_inputs

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    wp = get_workload("prefill_32k")
    wd = get_workload("decode_b16_256k")
    print(f"[bench] generating inputs", file=sys.stderr, flush=True)
    pin = prefill_inputs(wp, seed=0, device=dev)
    din = decode_inputs(wd, seed=0, device=dev)
    block_keys = msa.msa_pool_block_keys(din["k_idx_cache"], wd.block_size)
    # generation step (append + decode) at the same shape: the caches hold
    # L - 1 tokens and each step appends token L - 1
    L = wd.seq_len
    gen_keys, gen_sums = msa.msa_decode_init(din["k_idx_cache"], L - 1, wd.block_size)
    k_new = din["k_cache"][:, :, L - 1].contiguous()
    v_new = din["v_cache"][:, :, L - 1].contiguous()
    k_idx_new = din["k_idx_cache"][:, :, L - 1].contiguous()
    del din["k_idx_cache"]
    out = torch.empty_like(pin["q"])
    dout = torch.empty_like(din["q"])
    pdims = msa.make_dims(wp.batch, wp.seq_len, wp.n_q_heads, wp.n_kv_heads, wp.block_size, wp.top_k)
    ddims = msa.make_dims(wd.batch, wd.seq_len, wd.n_q_heads, wd.n_kv_heads, wd.block_size, wd.top_k)
    pws = torch.empty(msa.msa_workspace_bytes(msa.MSA_OP_PREFILL, pdims)[1], dtype=torch.uint8, device=dev)
    dws = torch.empty(msa.msa_workspace_bytes(msa.MSA_OP_DECODE, ddims)[1], dtype=torch.uint8, device=dev)

    def prefill():
        msa.msa_prefill(pin["q"], pin["k"], pin["v"], pin["q_idx"], pin["k_idx"], wp.block_size, wp.top_k,
                        out=out, workspace=pws)

    def decode():
        msa.msa_decode(din["q"], din["q_idx"], din["k_cache"], din["v_cache"], block_keys, wd.block_size,
                       wd.top_k, out=dout, workspace=dws)

    print(f"[bench] warmup {args.warmup}", file=sys.stderr, flush=True)
    for _ in range(args.warmup):
        prefill()
        decode()
    torch.cuda.synchronize()

    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True),
           torch.cuda.Event(enable_timing=True)) for _ in range(args.steps)]
    # Timed region: the library's kernel timing is on for the prefill (its
    # kernels are long; the per-kernel events cost microseconds) and off for
    # the ~0.1 ms decode call, whose kernel breakdown comes from a separate
    # pass below.
    msa.profile_read()              # drop anything recorded before
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        ev[i][0].record()
        msa.profile_enable(True)
        prefill()
        msa.profile_enable(False)
        ev[i][1].record()
        decode()
        ev[i][2].record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    kt = msa.profile_read()
    pre_ms = sorted(a.elapsed_time(b) for a, b, _ in ev)
    dec_ms = sorted(b.elapsed_time(c) for _, b, c in ev)
    pre_med = pre_ms[len(pre_ms) // 2]
    dec_med = dec_ms[len(dec_ms) // 2]
    ms_per_step = wall * 1e3 / args.steps
    # decode kernel breakdown (instrumented, outside the timed region)
    msa.profile_enable(True)
    for _ in range(args.steps):
        decode()
    torch.cuda.synchronize()
    msa.profile_enable(False)
    dkt = msa.profile_read()

    # further measurements outside the timed step (left out by --core-only,
    # e.g. under a profiler, so that each kernel's launches are those of the
    # step alone)
    gen_med = ch_ms = dwarm_med = None
    short_ms, short_flop = {}, None
    train_ms, bkt = {}, {}
    other_cfg = {}
    if not args.core_only:
        # generation step: append token L - 1 to the caches, refresh its block's
        # summary, decode (outside the timed region; same events)
        def gen_step():
            msa.msa_decode_step(din["q"], din["q_idx"], k_new, v_new, k_idx_new, din["k_cache"], din["v_cache"],
                                gen_sums, gen_keys, L, wd.block_size, wd.top_k, out=dout, workspace=dws)

        for _ in range(3):
            gen_step()
        torch.cuda.synchronize()
        gev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(args.steps)]
        for a, b in gev:
            a.record()
            gen_step()
            b.record()
        torch.cuda.synchronize()
        gen_us = sorted(a.elapsed_time(b) * 1e3 for a, b in gev)
        gen_med = gen_us[len(gen_us) // 2]
        # chunked prefill of the same 32K workload: four chunks of 8192 queries
        # against the cache (the K/V tensors serve as caches of capacity S)
        bounds = [0, 8192, 16384, 24576, wp.seq_len]
        cq = [pin["q"][:, a:b].contiguous() for a, b in zip(bounds[:-1], bounds[1:])]
        cqi = [pin["q_idx"][:, :, a:b].contiguous() for a, b in zip(bounds[:-1], bounds[1:])]
        couts = [torch.empty_like(x) for x in cq]
        ckeys = torch.empty_like(block_keys_prefill_shape(pin, wp))
        cws = torch.empty(_chunk_ws_bytes(msa, pdims, 8192), dtype=torch.uint8, device=dev)

        def chunked():
            for i, a in enumerate(bounds[:-1]):
                msa.msa_prefill_chunk(cq[i], cqi[i], pin["k"], pin["v"], pin["k_idx"], ckeys, a, wp.block_size,
                                      wp.top_k, out=couts[i], workspace=cws)

        chunked()
        torch.cuda.synchronize()
        cev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(5)]
        for a, b in cev:
            a.record()
            chunked()
            b.record()
        torch.cuda.synchronize()
        ch_ms = sorted(a.elapsed_time(b) for a, b in cev)[2]
        del cq, cqi, couts, cws

        # short sequence, top_k covering every block (4096 tokens, top_k 32 =
        # nb): msa_prefill takes the dense causal kernel; the chunked entry point
        # runs the sparse path on the same data
        ws_ = get_workload("prefill_32k", top_k=32)
        Ss = 4096
        sin = prefill_inputs(ws_, seed=1, device=dev, seq_len=Ss)
        sout = torch.empty_like(sin["q"])
        skeys = torch.empty((1, ws_.n_kv_heads, Ss // ws_.block_size, 64), dtype=torch.int8, device=dev)
        sdims = msa.make_dims(1, Ss, ws_.n_q_heads, ws_.n_kv_heads, ws_.block_size, ws_.top_k)
        sws = torch.empty(_chunk_ws_bytes(msa, sdims, Ss), dtype=torch.uint8, device=dev)
        short_runs = {
            "dense": lambda: msa.msa_prefill(sin["q"], sin["k"], sin["v"], sin["q_idx"], sin["k_idx"], ws_.block_size,
                                             ws_.top_k, out=sout),
            "sparse_path": lambda: msa.msa_prefill_chunk(sin["q"], sin["q_idx"], sin["k"], sin["v"], sin["k_idx"], skeys,
                                                         0, ws_.block_size, ws_.top_k, out=sout, workspace=sws),
        }
        short_ms = {}
        for name_, fn in short_runs.items():
            fn()
            torch.cuda.synchronize()
            sev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(5)]
            for a, b in sev:
                a.record()
                fn()
                b.record()
            torch.cuda.synchronize()
            short_ms[name_] = sorted(a.elapsed_time(b) for a, b in sev)[2]
        short_flop = 4.0 * D_HEAD * ws_.n_q_heads * Ss * (Ss + 1) / 2
        del sin, sout, sws

        # training step of the same 32K prefill: the forward with its
        # log-sum-exp, then the backward (dq, dk, dv; selection fixed)
        from synth import grad_output
        bout, bsel, blse = msa.msa_prefill_lse(pin["q"], pin["k"], pin["v"], pin["q_idx"], pin["k_idx"],
                                               wp.block_size, wp.top_k, workspace=pws)
        bdout = grad_output(wp, seed=0, device=dev)
        bws = torch.empty(msa.msa_workspace_bytes(msa.MSA_OP_BACKWARD, pdims)[1], dtype=torch.uint8, device=dev)
        train_runs = {
            "forward_lse": lambda: msa.msa_prefill_lse(pin["q"], pin["k"], pin["v"], pin["q_idx"], pin["k_idx"],
                                                       wp.block_size, wp.top_k, workspace=pws),
            "backward": lambda: msa.msa_prefill_backward(pin["q"], pin["k"], pin["v"], bout, bdout, blse, bsel,
                                                         wp.block_size, workspace=bws),
        }
        for name_, fn in train_runs.items():
            fn()
            torch.cuda.synchronize()
            msa.profile_read()
            msa.profile_enable(name_ == "backward")
            tev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(5)]
            for a, b in tev:
                a.record()
                fn()
                b.record()
            torch.cuda.synchronize()
            msa.profile_enable(False)
            train_ms[name_] = sorted(a.elapsed_time(b) for a, b in tev)[2]
            if name_ == "backward":
                bkt = msa.profile_read()
        del bout, bsel, blse, bdout, bws

        # the other prefill workloads, timed the same way (median of a few
        # calls after one warm-up; the 2K one is launch-bound)
        for name_, reps in (("tiny_2k", 10), ("structured_128k", 5), ("prefill_1m", 3)):
            wc = get_workload(name_)
            cin = prefill_inputs(wc, seed=0, device=dev)
            cdims = msa.make_dims(wc.batch, wc.seq_len, wc.n_q_heads, wc.n_kv_heads, wc.block_size, wc.top_k)
            cws = torch.empty(msa.msa_workspace_bytes(msa.MSA_OP_PREFILL, cdims)[1], dtype=torch.uint8, device=dev)
            cout = torch.empty_like(cin["q"])

            def fn():
                msa.msa_prefill(cin["q"], cin["k"], cin["v"], cin["q_idx"], cin["k_idx"], wc.block_size, wc.top_k,
                                out=cout, workspace=cws)

            fn()
            torch.cuda.synchronize()
            pev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(reps)]
            for a, b in pev:
                a.record()
                fn()
                b.record()
            torch.cuda.synchronize()
            cms = sorted(a.elapsed_time(b) for a, b in pev)[reps // 2]
            cflop = 4.0 * wc.head_dim * wc.n_q_heads * _prefill_counts(wc)[0]
            other_cfg[name_] = {"seq_len": wc.seq_len, "n_q_heads": wc.n_q_heads, "n_kv_heads": wc.n_kv_heads,
                                "block_size": wc.block_size, "top_k": wc.top_k, "calls": reps,
                                "ms": round(cms, 4), "tokens_per_s": round(wc.batch * wc.seq_len / (cms * 1e-3), 1),
                                "tflops_alg": round(cflop / (cms * 1e-3) / 1e12, 2),
                                "frac_bf16_peak": round(cflop / (cms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4)}
            print(f"[bench] {name_}: {cms:.3f} ms", file=sys.stderr, flush=True)
            if name_ == "prefill_1m":
                # its backward too: the full workspace (about 276 GB) does not
                # fit beside the tensors, so it runs in query passes in what
                # the binding allocates by default (80 % of the free memory)
                cws = None
                torch.cuda.empty_cache()
                tout, tsel, tlse = msa.msa_prefill_lse(cin["q"], cin["k"], cin["v"], cin["q_idx"], cin["k_idx"],
                                                       wc.block_size, wc.top_k)
                tdout = grad_output(wc, seed=0, device=dev)
                cout = None
                torch.cuda.empty_cache()

                def bfn():
                    return msa.msa_prefill_backward(cin["q"], cin["k"], cin["v"], tout, tdout, tlse, tsel,
                                                    wc.block_size, workspace=tws)

                tlo, thi = msa.msa_workspace_bytes(msa.MSA_OP_BACKWARD, cdims)
                tws = torch.empty(max(tlo, min(thi, int(torch.cuda.mem_get_info(dev)[0] * 0.8) - (20 << 30))),
                                  dtype=torch.uint8, device=dev)
                bfn()
                torch.cuda.synchronize()
                msa.profile_read()
                msa.profile_enable(True)
                bev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(2)]
                for a, b in bev:
                    a.record()
                    bfn()
                    b.record()
                torch.cuda.synchronize()
                msa.profile_enable(False)
                bk1 = msa.profile_read()
                bms = max(a.elapsed_time(b) for a, b in bev)
                other_cfg[name_]["backward"] = {
                    "workspace_gib": round(tws.numel() / 2**30, 1), "passes": bk1["bwd_kv"][0] // 2,
                    "ms": round(bms, 2), "tflops_alg": round(2.5 * cflop / (bms * 1e-3) / 1e12, 2),
                    "bwd_kv_ms": round(bk1["bwd_kv"][1] / 2, 2)}
                print(f"[bench] {name_} backward: {bms:.1f} ms", file=sys.stderr, flush=True)
                del tout, tsel, tlse, tdout, tws
            cin = cout = cws = None
            torch.cuda.empty_cache()

        # the plain decode timed the same way (back to back, so the kept blocks
        # may still sit in the memory-side cache, unlike in the step above where
        # a prefill runs in between)
        for a, b in gev:
            a.record()
            decode()
            b.record()
        torch.cuda.synchronize()
        dwarm_us = sorted(a.elapsed_time(b) * 1e3 for a, b in gev)
        dwarm_med = dwarm_us[len(dwarm_us) // 2]

    per_head_keys, pairs, rows_merged = _prefill_counts(wp)
    D = wp.head_dim
    flop_alg = 4.0 * D * wp.n_q_heads * per_head_keys
    tokens = wp.batch * wp.seq_len
    # dominant kernel: the attention kernel (all selected blocks of every
    # query); per step it may run in several launches (passes)
    n_att, att_ms = kt.get("attend", (0, 0.0))
    att_ms_step = att_ms / args.steps
    att_launch_ms = att_ms / max(1, n_att)
    launches_per_step = max(1, n_att // args.steps)
    att_tflops = flop_alg / (att_ms_step * 1e-3) / 1e12 if att_ms_step > 0 else None
    # bytes the KV-outer design moves: per (query row, kept block) pair a
    # gathered Q row (256 B) and a bf16 partial + fp32 (max, sum) (264 B)
    att_design_bytes = pairs * (2 * D + 2 * D + 8)
    n_mrg, mrg_ms = kt.get("merge", (0, 0.0))
    mrg_ms_step = mrg_ms / args.steps
    mrg_design_bytes = (pairs - (tokens * wp.n_q_heads - rows_merged)) * (2 * D + 8) + rows_merged * 2 * D
    dbytes = _decode_bytes(wd)
    traffic = _measured_traffic()

    kernels = {k: {"launches": n, "avg_ms": round(ms / max(1, n), 4)}
               for k, (n, ms) in sorted(list(kt.items()) + list(dkt.items()))}
    rec = {
        "metric": "MSA prefill tokens/s + TFLOP/s (% bf16 MFMA peak); decode tokens/s, HBM GB/s",
        "value": round(tokens / (pre_med * 1e-3), 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "prefill_32k + decode_b16_256k", "batch": wp.batch, "seq_len": wp.seq_len,
                   "n_q_heads": wp.n_q_heads, "n_kv_heads": wp.n_kv_heads, "head_dim": D,
                   "block_size": wp.block_size, "top_k": wp.top_k, "decode_batch": wd.batch,
                   "decode_cache_len": wd.seq_len, "parallelism": "none (1 GPU)"},
        "prefill": {
            "ms": round(pre_med, 4),
            "tokens_per_s": round(tokens / (pre_med * 1e-3), 1),
            "tflops_alg": round(flop_alg / (pre_med * 1e-3) / 1e12, 2),
            "frac_bf16_peak": round(flop_alg / (pre_med * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4),
            "flop_alg": flop_alg,
        },
        "decode": {
            "us": round(dec_med * 1e3, 2),
            "tokens_per_s": round(wd.batch / (dec_med * 1e-3), 1),
            "hbm_gbs_alg": round(dbytes / (dec_med * 1e-3) / 1e9, 1),
            "frac_hbm_peak": round(dbytes / (dec_med * 1e-3) / 1e9 / PEAK_HBM_GBS, 4),
            "bytes_alg": dbytes,
        },
        "prefill_chunked": None if ch_ms is None else {
            "what": "the same 32K prefill as four chunks of 8192 queries against the cache",
            "ms": round(ch_ms, 4),
            "tokens_per_s": round(tokens / (ch_ms * 1e-3), 1),
            "tflops_alg": round(flop_alg / (ch_ms * 1e-3) / 1e12, 2),
        },
        "prefill_short_dense": None if not short_ms else {
            "what": "4096 tokens, top_k 32 = every block: dense causal kernel vs the sparse path on the same data",
            "dense_ms": round(short_ms["dense"], 4),
            "sparse_path_ms": round(short_ms["sparse_path"], 4),
            "dense_tflops": round(short_flop / (short_ms["dense"] * 1e-3) / 1e12, 2),
            "dense_frac_bf16_peak": round(short_flop / (short_ms["dense"] * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4),
        },
        "training": None if not train_ms else {
            "what": "the 32K prefill for training: forward with log-sum-exp, and the main-branch backward "
                    "(dq, dk, dv; selection fixed)",
            "forward_lse_ms": round(train_ms["forward_lse"], 4),
            "backward_ms": round(train_ms["backward"], 4),
            "backward_tflops_alg": round(2.5 * flop_alg / (train_ms["backward"] * 1e-3) / 1e12, 2),
            "backward_frac_bf16_peak": round(2.5 * flop_alg / (train_ms["backward"] * 1e-3) / 1e12 / PEAK_BF16_TFLOPS,
                                             4),
            "backward_flop_alg": 2.5 * flop_alg,
            "bwd_kv_tflops_alg": round(2.5 * flop_alg / (bkt["bwd_kv"][1] / bkt["bwd_kv"][0] * 1e-3) / 1e12, 2)
            if "bwd_kv" in bkt else None,
            "kernels": {k: {"launches": n, "avg_ms": round(ms / max(1, n), 4)} for k, (n, ms) in sorted(bkt.items())},
        },
        "prefill_other_workloads": other_cfg or None,
        "decode_step": None if gen_med is None else {
            "what": "append one token per sequence (K/V rows, running index-key sum, block summary) + decode",
            "us": round(gen_med, 2),
            "tokens_per_s": round(wd.batch / (gen_med * 1e-6), 1),
            "frac_hbm_peak": round(dbytes / (gen_med * 1e-6) / 1e9 / PEAK_HBM_GBS, 4),
            "timing": "back-to-back calls",
            "decode_only_back_to_back_us": round(dwarm_med, 2),
        },
        "roofline": {
            "kernel": "attend (KV-outer block attention, all kept blocks)",
            "bound": "mfma",
            "achieved": round(att_tflops, 2) if att_tflops else None,
            "peak": PEAK_BF16_TFLOPS,
            "unit": "TFLOP/s",
            "frac": round(att_tflops / PEAK_BF16_TFLOPS, 4) if att_tflops else None,
            "traffic": traffic,
            "avg_launch_ms": round(att_launch_ms, 4),
            "launches_per_step": launches_per_step,
            "flop_per_launch": flop_alg / launches_per_step,
            "design_bytes_per_step": att_design_bytes,
            "design_hbm_gbs": round(att_design_bytes / (att_ms_step * 1e-3) / 1e9, 1) if att_ms_step else None,
            # the same kernel against the HBM roof, with the bytes the KV-outer
            # design moves (gathered Q rows and partials) and with the
            # measured bytes: the design is bound by this traffic, the
            # algorithm (each tensor once) by the MFMA roof above
            "design_frac_hbm_peak": round(att_design_bytes / (att_ms_step * 1e-3) / 1e9 / PEAK_HBM_GBS, 4)
            if att_ms_step else None,
            "measured_frac_hbm_peak": round(traffic / (att_launch_ms * 1e-3) / 1e9 / PEAK_HBM_GBS, 4)
            if (traffic and att_launch_ms) else None,
        },
        "merge_kernel": {
            "ms": round(mrg_ms_step, 4),
            "design_bytes": mrg_design_bytes,
            "hbm_gbs": round(mrg_design_bytes / (mrg_ms_step * 1e-3) / 1e9, 1) if mrg_ms_step else None,
        },
        "kernels": kernels,
    }
    if not args.no_cpu_baseline:
        print(f"[bench] cpu baseline ({CPU_SAMPLE_ROWS} rows)", file=sys.stderr, flush=True)
        rec["cpu_baseline"] = cpu_baseline(pin, wp, CPU_SAMPLE_ROWS)
    else:
        rec["cpu_baseline"] = None
    print(json.dumps(rec), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
